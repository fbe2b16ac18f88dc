"""QSA (Qwen Sparse Attention) decode step for AMD Instinct MI355X (gfx950).

The hot path -- incremental pooled-key cache, indexer scoring, block top-k and
gathered GQA attention -- is hand-written HIP in libqsa.so behind the C ABI of
include/qsa.h; ``qsa`` is its ctypes binding.
"""
from .qsa import *  # noqa: F401,F403
from .qsa import LayerBuffers, QSAError, batch_workspace, chunk_workspace, lib, make_desc, workspace  # noqa: F401

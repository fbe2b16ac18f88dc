"""ctypes binding of libqsa.so (include/qsa.h).  Argument marshalling only:
every step of the decode path runs in the library's HIP kernels.

Functions carry the C names.  Tensors are torch CUDA tensors (device memory
and streams are all torch is used for); the default stream is torch's current
stream.  A non-OK status raises QSAError with the library's message.  If the
library is not built, importing works but every call raises -- there is no
other implementation to fall back to.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqsa.so")

QSA_OK, QSA_ERR_ARG, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE, QSA_ERR_HIP = 0, -1, -2, -3, -4
QSA_F32, QSA_F16 = 0, 1

# Entry points declared in include/qsa.h (checked by the ABI test).
EXPORTS = ("qsa_workspace_bytes", "qsa_state_invalidate", "qsa_state_truncate",
           "qsa_cache_update", "qsa_index_score", "qsa_topk_blocks", "qsa_gather_attend",
           "qsa_decode_step", "qsa_decode_step_static", "qsa_decode_score", "qsa_batch_workspace_bytes", "qsa_decode_step_batch",
           "qsa_chunk_workspace_bytes", "qsa_chunk_step", "qsa_chunk_step_grouped",
           "qsa_multi_workspace_bytes",
           "qsa_decode_step_multi", "qsa_ablation_workspace_bytes", "qsa_topk_cells",
           "qsa_attend_masked", "qsa_q8_0_quantize", "qsa_gather_attend_q8_0",
           "qsa_status_string", "qsa_last_error")
QSA_MAX_BATCH = 8
QSA_MAX_CHUNK = 4096
QSA_MAX_MULTI = 4
QSA_DECODE_STATUS_OFFSET = 8        # byte offset of the decode step's status word in its workspace
QSA_PATH_HIST, QSA_PATH_FULL = 1, 2


class QSAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class qsa_layer_desc(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("idx_dtype", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("top_k_tokens", ctypes.c_int32),
                ("attn_scale", ctypes.c_float)]


class qsa_layer_cache(ctypes.Structure):
    _fields_ = [("idx_k", ctypes.c_void_p), ("summary", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int32)]


class qsa_kv_q8_0(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("capacity", ctypes.c_int32)]


class qsa_seq_state(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_valid_blocks", ctypes.c_int32)]


class qsa_seq_io(ctypes.Structure):
    _fields_ = [("idx_k_row", ctypes.c_void_p), ("k_row", ctypes.c_void_p),
                ("v_row", ctypes.c_void_p), ("q_idx", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("out", ctypes.c_void_p), ("sel_out", ctypes.c_void_p),
                ("scores_out", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded libqsa.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D, C, S = ctypes.POINTER(qsa_layer_desc), ctypes.POINTER(qsa_layer_cache), ctypes.POINTER(qsa_seq_state)
        L.qsa_workspace_bytes.restype = sz
        L.qsa_workspace_bytes.argtypes = [D, i32]
        L.qsa_state_invalidate.restype = None
        L.qsa_state_invalidate.argtypes = [S, i32]
        L.qsa_state_truncate.restype = None
        L.qsa_state_truncate.argtypes = [S, i32]
        L.qsa_cache_update.argtypes = [D, C, P, i32, i32, P]
        L.qsa_index_score.argtypes = [D, C, i32, P, P, P, P]
        L.qsa_topk_blocks.argtypes = [P, i32, i32, P, P, sz, P]
        L.qsa_gather_attend.argtypes = [D, C, i32, P, i32, P, P, P, sz, P]
        L.qsa_decode_step.argtypes = [D, C, S, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.qsa_decode_score.argtypes = [D, C, S, P, P, P, P, P, sz, P]
        L.qsa_decode_step_static.argtypes = [D, C, S, P, P, P, P, P, P, P, P, P, P, P]
        L.qsa_batch_workspace_bytes.restype = sz
        L.qsa_batch_workspace_bytes.argtypes = [D, i32, ctypes.POINTER(i32)]
        L.qsa_decode_step_batch.argtypes = [D, i32, C, S, ctypes.POINTER(qsa_seq_io), P, P, sz, P]
        L.qsa_chunk_workspace_bytes.restype = sz
        L.qsa_chunk_workspace_bytes.argtypes = [D, i32, i32]
        L.qsa_chunk_step.argtypes = [D, C, S, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.qsa_chunk_step_grouped.argtypes = [D, C, S, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.qsa_multi_workspace_bytes.restype = sz
        L.qsa_multi_workspace_bytes.argtypes = [D, i32, i32]
        L.qsa_decode_step_multi.argtypes = [D, C, S, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.qsa_ablation_workspace_bytes.restype = sz
        L.qsa_ablation_workspace_bytes.argtypes = [D, i32]
        L.qsa_topk_cells.argtypes = [P, i32, i32, P, P, sz, P]
        L.qsa_attend_masked.argtypes = [D, C, i32, P, i32, P, P, P, sz, P]
        L.qsa_q8_0_quantize.argtypes = [P, ctypes.c_int64, P, P, P]
        L.qsa_gather_attend_q8_0.argtypes = [D, ctypes.POINTER(qsa_kv_q8_0), i32, P, i32, P, P, P, sz, P]
        for f in ("qsa_cache_update", "qsa_index_score", "qsa_topk_blocks", "qsa_gather_attend",
                  "qsa_decode_step", "qsa_decode_step_static", "qsa_decode_score", "qsa_decode_step_batch", "qsa_chunk_step", "qsa_chunk_step_grouped",
                  "qsa_decode_step_multi", "qsa_topk_cells", "qsa_attend_masked",
                  "qsa_q8_0_quantize", "qsa_gather_attend_q8_0"):
            getattr(L, f).restype = ctypes.c_int
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_status_string.argtypes = [ctypes.c_int]
        L.qsa_last_error.restype = ctypes.c_char_p
        L.qsa_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status):
    if status != QSA_OK:
        raise QSAError(status, lib().qsa_last_error().decode() or lib().qsa_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ws(ws):
    return (None, 0) if ws is None else (ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size())


# ------------------------------------------------------------------ helpers
def make_desc(idx_heads, idx_dim, idx_dtype, q_heads, kv_heads, head_dim, top_k_tokens,
              rms_eps=1e-6, rope_theta=1e4, attn_scale=0.0, block=4):
    return qsa_layer_desc(block, idx_heads, idx_dim, idx_dtype, rms_eps, rope_theta,
                          q_heads, kv_heads, head_dim, top_k_tokens, attn_scale)


class LayerBuffers:
    """Device buffers of one sequence x one layer (torch tensors) and the
    qsa_layer_cache struct pointing at them."""

    def __init__(self, desc, capacity, device="cuda"):
        dt = torch.float16 if desc.idx_dtype == QSA_F16 else torch.float32
        self.capacity = int(capacity)
        self.idx_k = torch.empty((capacity, desc.idx_heads, desc.idx_dim), dtype=dt, device=device)
        self.summary = torch.empty((capacity // 4, desc.idx_heads, desc.idx_dim), dtype=dt, device=device)
        self.k = torch.empty((capacity, desc.kv_heads, desc.head_dim), dtype=torch.float16, device=device)
        self.v = torch.empty_like(self.k)
        self.cache = qsa_layer_cache(self.idx_k.data_ptr(), self.summary.data_ptr(),
                                     self.k.data_ptr(), self.v.data_ptr(), self.capacity)


def workspace(desc, capacity, device="cuda"):
    n = lib().qsa_workspace_bytes(ctypes.byref(desc), int(capacity))
    if n == 0:
        raise QSAError(QSA_ERR_UNSUPPORTED, "qsa_workspace_bytes rejected the descriptor")
    return torch.empty(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------- entry points
def qsa_workspace_bytes(desc, capacity):
    return lib().qsa_workspace_bytes(ctypes.byref(desc), int(capacity))


def qsa_state_invalidate(state, pos):
    lib().qsa_state_invalidate(ctypes.byref(state), int(pos))


def qsa_state_truncate(state, pos):
    lib().qsa_state_truncate(ctypes.byref(state), int(pos))


def qsa_cache_update(desc, cache, gamma, blk_begin, blk_end, stream=None):
    _check(lib().qsa_cache_update(ctypes.byref(desc), ctypes.byref(cache), _ptr(gamma),
                                  int(blk_begin), int(blk_end), _stream(stream)))


def qsa_index_score(desc, cache, n_blocks, q_idx, w, scores, stream=None):
    _check(lib().qsa_index_score(ctypes.byref(desc), ctypes.byref(cache), int(n_blocks),
                                 _ptr(q_idx), _ptr(w), _ptr(scores), _stream(stream)))


def qsa_topk_blocks(scores, n_blocks, k_blocks, sel, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_topk_blocks(_ptr(scores), int(n_blocks), int(k_blocks), _ptr(sel), p, n,
                                 _stream(stream)))


def qsa_gather_attend(desc, cache, n_tokens, sel, n_sel_blocks, q, out, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_gather_attend(ctypes.byref(desc), ctypes.byref(cache), int(n_tokens), _ptr(sel),
                                   int(n_sel_blocks), _ptr(q), _ptr(out), p, n, _stream(stream)))


def qsa_decode_step(desc, cache, state, idx_k_row, k_row, v_row, gamma, q_idx, w, q, out,
                    sel_out=None, scores_out=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_decode_step(ctypes.byref(desc), ctypes.byref(cache), ctypes.byref(state),
                                 _ptr(idx_k_row), _ptr(k_row), _ptr(v_row), _ptr(gamma), _ptr(q_idx),
                                 _ptr(w), _ptr(q), _ptr(out), _ptr(sel_out), _ptr(scores_out),
                                 p, n, _stream(stream)))


def qsa_decode_step_static(desc, cache, state, idx_k_row, k_row, v_row, gamma, q_idx, w, q, out,
                           sel_out=None, scores_out=None, stream=None):
    _check(lib().qsa_decode_step_static(ctypes.byref(desc), ctypes.byref(cache), ctypes.byref(state),
                                        _ptr(idx_k_row), _ptr(k_row), _ptr(v_row), _ptr(gamma),
                                        _ptr(q_idx), _ptr(w), _ptr(q), _ptr(out), _ptr(sel_out),
                                        _ptr(scores_out), _stream(stream)))


def qsa_decode_score(desc, cache, state, gamma, q_idx, w, scores_out=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_decode_score(ctypes.byref(desc), ctypes.byref(cache), ctypes.byref(state),
                                  _ptr(gamma), _ptr(q_idx), _ptr(w), _ptr(scores_out), p, n,
                                  _stream(stream)))


def qsa_batch_workspace_bytes(desc, capacities):
    caps = (ctypes.c_int32 * len(capacities))(*[int(c) for c in capacities])
    return lib().qsa_batch_workspace_bytes(ctypes.byref(desc), len(capacities), caps)


def batch_workspace(desc, capacities, device="cuda"):
    n = qsa_batch_workspace_bytes(desc, capacities)
    if n == 0:
        raise QSAError(QSA_ERR_UNSUPPORTED, "qsa_batch_workspace_bytes rejected the arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def qsa_decode_step_batch(desc, caches, states, io, gamma, ws, stream=None):
    """caches: list of qsa_layer_cache; states: list of qsa_seq_state (updated in
    place); io: list of dicts with keys idx_k_row, k_row, v_row, q_idx, w, q, out
    and optional sel_out (torch tensors)."""
    n = len(caches)
    c_arr = (qsa_layer_cache * n)(*caches)
    s_arr = (qsa_seq_state * n)(*[qsa_seq_state(s.n_tokens, s.n_valid_blocks) for s in states])
    io_arr = (qsa_seq_io * n)(*[qsa_seq_io(*[None if x.get(k) is None else x[k].data_ptr()
                                              for k in ("idx_k_row", "k_row", "v_row", "q_idx", "w",
                                                        "q", "out", "sel_out", "scores_out")])
                                  for x in io])
    p, nbytes = _ws(ws)
    _check(lib().qsa_decode_step_batch(ctypes.byref(desc), n, c_arr, s_arr, io_arr, _ptr(gamma), p,
                                       nbytes, _stream(stream)))
    for i, st in enumerate(states):
        st.n_tokens, st.n_valid_blocks = s_arr[i].n_tokens, s_arr[i].n_valid_blocks


def qsa_chunk_workspace_bytes(desc, capacity, n_q):
    return lib().qsa_chunk_workspace_bytes(ctypes.byref(desc), int(capacity), int(n_q))


def chunk_workspace(desc, capacity, n_q, device="cuda"):
    n = qsa_chunk_workspace_bytes(desc, capacity, n_q)
    if n == 0:
        raise QSAError(QSA_ERR_UNSUPPORTED, "qsa_chunk_workspace_bytes rejected the arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def qsa_chunk_step(desc, cache, state, n_q, idx_k_rows, k_rows, v_rows, gamma, q_idx, w, q, out,
                   sel_out=None, scores_out=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_chunk_step(ctypes.byref(desc), ctypes.byref(cache), ctypes.byref(state), int(n_q),
                                _ptr(idx_k_rows), _ptr(k_rows), _ptr(v_rows), _ptr(gamma), _ptr(q_idx),
                                _ptr(w), _ptr(q), _ptr(out), _ptr(sel_out), _ptr(scores_out),
                                p, n, _stream(stream)))


def qsa_chunk_step_grouped(desc, cache, state, n_q, idx_k_rows, k_rows, v_rows, gamma, q_idx, w, q, out,
                           sel_out=None, scores_out=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_chunk_step_grouped(ctypes.byref(desc), ctypes.byref(cache), ctypes.byref(state),
                                        int(n_q), _ptr(idx_k_rows), _ptr(k_rows), _ptr(v_rows), _ptr(gamma),
                                        _ptr(q_idx), _ptr(w), _ptr(q), _ptr(out), _ptr(sel_out),
                                        _ptr(scores_out), p, n, _stream(stream)))


def qsa_multi_workspace_bytes(desc, capacity, n_q):
    return lib().qsa_multi_workspace_bytes(ctypes.byref(desc), int(capacity), int(n_q))


def multi_workspace(desc, capacity, n_q, device="cuda"):
    n = qsa_multi_workspace_bytes(desc, capacity, n_q)
    if n == 0:
        raise QSAError(QSA_ERR_UNSUPPORTED, "qsa_multi_workspace_bytes rejected the arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def qsa_decode_step_multi(desc, cache, state, n_q, idx_k_rows, k_rows, v_rows, gamma, q_idx, w, q,
                          out, sel_out=None, scores_out=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_decode_step_multi(ctypes.byref(desc), ctypes.byref(cache), ctypes.byref(state),
                                       int(n_q), _ptr(idx_k_rows), _ptr(k_rows), _ptr(v_rows),
                                       _ptr(gamma), _ptr(q_idx), _ptr(w), _ptr(q), _ptr(out),
                                       _ptr(sel_out), _ptr(scores_out), p, n, _stream(stream)))


def qsa_ablation_workspace_bytes(desc, capacity):
    return lib().qsa_ablation_workspace_bytes(ctypes.byref(desc), int(capacity))


def ablation_workspace(desc, capacity, device="cuda"):
    n = qsa_ablation_workspace_bytes(desc, capacity)
    if n == 0:
        raise QSAError(QSA_ERR_UNSUPPORTED, "qsa_ablation_workspace_bytes rejected the arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def qsa_topk_cells(block_scores, n_tokens, top_k_tokens, cells, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_topk_cells(_ptr(block_scores), int(n_tokens), int(top_k_tokens), _ptr(cells),
                                p, n, _stream(stream)))


def qsa_attend_masked(desc, cache, n_tokens, sel, n_sel_blocks, q, out, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_attend_masked(ctypes.byref(desc), ctypes.byref(cache), int(n_tokens), _ptr(sel),
                                   int(n_sel_blocks), _ptr(q), _ptr(out), p, n, _stream(stream)))


# ------------------------------------------------------------------ q8_0 K/V
def kv_q8_0(k_codes, k_scales, v_codes, v_scales):
    """qsa_kv_q8_0 over torch tensors: codes int8 [cap, Hkv, Dh], scales
    (binary16 bits, any 2-byte dtype) [cap, Hkv, Dh/32]."""
    return qsa_kv_q8_0(k_codes.data_ptr(), k_scales.data_ptr(), v_codes.data_ptr(),
                       v_scales.data_ptr(), int(k_codes.shape[0]))


def qsa_q8_0_quantize(x, codes, scales, n_values=None, stream=None):
    n = x.numel() if n_values is None else n_values
    _check(lib().qsa_q8_0_quantize(_ptr(x), int(n), _ptr(codes), _ptr(scales), _stream(stream)))


def qsa_gather_attend_q8_0(desc, kv, n_tokens, sel, n_sel_blocks, q, out, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().qsa_gather_attend_q8_0(ctypes.byref(desc), ctypes.byref(kv), int(n_tokens), _ptr(sel),
                                        int(n_sel_blocks), _ptr(q), _ptr(out), p, n, _stream(stream)))

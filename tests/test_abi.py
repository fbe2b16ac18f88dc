"""The C ABI on the CPU: every symbol declared in include/*.h is exported,
argument errors are reported before anything is launched, and the host-only
state calls behave as documented.  No call here reaches a kernel launch."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"\b(qsa_[a-z_0-9]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    import sparse_attention_decode_cache_amd as qsa
    L = qsa.lib()
    declared = _declared()
    assert declared == set(qsa.EXPORTS), declared ^ set(qsa.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def _objs():
    import sparse_attention_decode_cache_amd as qsa
    d = qsa.make_desc(4, 128, qsa.QSA_F16, 16, 2, 256, 2048)
    c = qsa.qsa_layer_cache(0x1000, 0x2000, 0x3000, 0x4000, 4096)
    return qsa, d, c


def test_workspace_bytes():
    qsa, d, _ = _objs()
    n = qsa.qsa_workspace_bytes(d, 255248)
    assert n > 255248 // 4 * 12 and n % 256 == 0
    assert qsa.qsa_workspace_bytes(d, 4095) == 0          # capacity not a multiple of 4
    bad = qsa.make_desc(4, 128, qsa.QSA_F32, 16, 2, 256, 2048)   # 2 KB indexer rows
    assert qsa.qsa_workspace_bytes(bad, 4096) == 0


@pytest.mark.parametrize("field,value,status", [
    ("block", 8, -2), ("idx_heads", 2, -2), ("idx_dim", 96, -2), ("head_dim", 512, -2),
    ("q_heads", 12, -2), ("q_heads", 32, -2), ("top_k_tokens", 2046, -2), ("top_k_tokens", 0, -2),
    ("idx_dtype", 7, -2), ("rope_theta", 0.0, -1)])
def test_descriptor_errors(field, value, status):
    qsa, d, c = _objs()
    setattr(d, field, value)
    st = qsa.qsa_seq_state(10, 0)
    rc = qsa.lib().qsa_decode_step(ctypes.byref(d), ctypes.byref(c), ctypes.byref(st), *[ctypes.c_void_p(16)] * 8,
                                   None, None, None, 0, None)
    assert rc == status
    assert (st.n_tokens, st.n_valid_blocks) == (10, 0)     # state untouched on error
    assert qsa.lib().qsa_last_error()


def test_argument_errors_before_launch():
    qsa, d, c = _objs()
    L = qsa.lib()
    P = ctypes.c_void_p
    D, C = ctypes.byref(d), ctypes.byref(c)
    # null / bad ranges
    assert L.qsa_cache_update(D, C, None, 0, 4, None) == -1
    assert L.qsa_cache_update(D, C, P(16), 3, 2, None) == -1
    assert L.qsa_cache_update(D, C, P(16), 0, 1025, None) == -1
    assert L.qsa_index_score(D, C, 1025, P(16), P(16), P(16), None) == -1
    assert L.qsa_index_score(D, C, 10, None, P(16), P(16), None) == -1
    assert L.qsa_topk_blocks(P(16), -1, 5, P(16), None, 0, None) == -1
    assert L.qsa_topk_blocks(P(16), 100, 0, P(16), None, 0, None) == -1
    assert L.qsa_topk_blocks(P(16), 100, 5, P(16), None, 0, None) == -3          # no workspace
    assert L.qsa_topk_blocks(P(16), 100, 5, P(16), P(256), 16, None) == -3        # too small
    assert L.qsa_topk_blocks(P(16), 100, 5, P(16), P(255 + 256), 1 << 20, None) == -3   # misaligned
    assert L.qsa_gather_attend(D, C, 0, P(16), 0, P(16), P(16), P(256), 1 << 30, None) == -1
    assert L.qsa_gather_attend(D, C, 4097, P(16), 0, P(16), P(16), P(256), 1 << 30, None) == -1
    assert L.qsa_gather_attend(D, C, 4096, P(16), 513, P(16), P(16), P(256), 1 << 30, None) == -1
    assert L.qsa_gather_attend(D, C, 4096, None, 5, P(16), P(16), P(256), 1 << 30, None) == -1
    assert L.qsa_gather_attend(D, C, 4096, P(16), 5, P(16), P(16), P(256), 64, None) == -3
    assert L.qsa_gather_attend(D, C, 4096, P(16), 0, P(16), P(16), P(256), 1 << 30, None) == -1   # no cell
    assert b"no cell" in L.qsa_last_error()
    assert L.qsa_gather_attend(D, C, 4096, P(16), 5, P(8), P(16), P(256), 1 << 30, None) == -1    # q misaligned
    assert L.qsa_gather_attend(D, C, 4096, P(16), 5, P(16), P(8), P(256), 1 << 30, None) == -1    # out misaligned
    assert b"aligned" in L.qsa_last_error()
    # decode step: position at capacity, null rows, small workspace
    st = qsa.qsa_seq_state(4096, 1024)
    args = [P(16)] * 8
    assert L.qsa_decode_step(D, C, ctypes.byref(st), *args, None, None, P(256), 1 << 30, None) == -1
    st = qsa.qsa_seq_state(100, 25)
    assert L.qsa_decode_step(D, C, ctypes.byref(st), None, *args[1:], None, None, P(256), 1 << 30, None) == -1
    assert L.qsa_decode_step(D, C, ctypes.byref(st), *args, None, None, P(256), 100, None) == -3
    assert (st.n_tokens, st.n_valid_blocks) == (100, 25)
    c2 = qsa.qsa_layer_cache(0x1000, 0x2000, 0x3000, 0x4000, 4094)               # capacity % 4
    assert L.qsa_decode_step(D, ctypes.byref(c2), ctypes.byref(st), *args, None, None, P(256), 1 << 30, None) == -1
    assert L.qsa_status_string(-3) == b"workspace missing or too small"


def test_batch_argument_errors_before_launch():
    qsa, d, c = _objs()
    L = qsa.lib()
    P = ctypes.c_void_p
    D = ctypes.byref(d)
    caps = (ctypes.c_int32 * 3)(4096, 8192, 400)
    one = qsa.qsa_batch_workspace_bytes(d, [4096])
    assert one == qsa.qsa_workspace_bytes(d, 4096)
    assert qsa.qsa_batch_workspace_bytes(d, [4096, 8192, 400]) > one
    assert L.qsa_batch_workspace_bytes(D, 0, caps) == 0
    assert L.qsa_batch_workspace_bytes(D, 9, caps) == 0
    assert qsa.qsa_batch_workspace_bytes(d, [4096, 4094]) == 0          # capacity % 4
    cs = (qsa.qsa_layer_cache * 2)(c, c)
    sts = (qsa.qsa_seq_state * 2)(qsa.qsa_seq_state(100, 25), qsa.qsa_seq_state(4096, 1024))
    io = (qsa.qsa_seq_io * 2)(qsa.qsa_seq_io(*[16] * 7, None), qsa.qsa_seq_io(*[16] * 7, None))
    assert L.qsa_decode_step_batch(D, 0, cs, sts, io, P(16), P(256), 1 << 30, None) == -1
    assert L.qsa_decode_step_batch(D, 9, cs, sts, io, P(16), P(256), 1 << 30, None) == -1
    assert L.qsa_decode_step_batch(D, 2, cs, sts, io, None, P(256), 1 << 30, None) == -1
    # sequence 1 sits at its capacity
    assert L.qsa_decode_step_batch(D, 2, cs, sts, io, P(16), P(256), 1 << 30, None) == -1
    assert b"sequence 1" in L.qsa_last_error()
    sts[1] = qsa.qsa_seq_state(200, 50)
    io[0].q = 8                                                          # q must be 16-byte aligned
    assert L.qsa_decode_step_batch(D, 2, cs, sts, io, P(16), P(256), 1 << 30, None) == -1
    io[0].q = 16
    assert L.qsa_decode_step_batch(D, 2, cs, sts, io, P(16), P(256), 100, None) == -3
    assert [(x.n_tokens, x.n_valid_blocks) for x in sts] == [(100, 25), (200, 50)]


def test_state_invalidate_and_truncate():
    import sparse_attention_decode_cache_amd as qsa
    st = qsa.qsa_seq_state(1000, 250)
    qsa.qsa_state_invalidate(st, 999)
    assert (st.n_tokens, st.n_valid_blocks) == (1000, 249)
    qsa.qsa_state_invalidate(st, 2000)
    assert (st.n_tokens, st.n_valid_blocks) == (1000, 249)
    qsa.qsa_state_invalidate(st, 13)
    assert (st.n_tokens, st.n_valid_blocks) == (1000, 3)
    st = qsa.qsa_seq_state(1000, 250)
    qsa.qsa_state_truncate(st, 601)
    assert (st.n_tokens, st.n_valid_blocks) == (601, 150)
    qsa.qsa_state_truncate(st, -5)
    assert (st.n_tokens, st.n_valid_blocks) == (0, 0)


def test_chunk_argument_errors_before_launch():
    qsa, d, c = _objs()
    L = qsa.lib()
    P = ctypes.c_void_p
    D = ctypes.byref(d)
    one = qsa.qsa_chunk_workspace_bytes(d, 4096, 64)
    assert one > 0 and qsa.qsa_chunk_workspace_bytes(d, 4096, 1024) > one
    assert qsa.qsa_chunk_workspace_bytes(d, 4096, 0) == 0
    assert qsa.qsa_chunk_workspace_bytes(d, 4096, qsa.QSA_MAX_CHUNK + 1) == 0
    assert qsa.qsa_chunk_workspace_bytes(d, 4094, 16) == 0

    def call(st, n_q, q=16, ws_bytes=1 << 40, gamma=16):
        return L.qsa_chunk_step(D, ctypes.byref(c), ctypes.byref(st), n_q, P(16), P(16), P(16),
                                P(gamma) if gamma else None, P(16), P(16), P(q), P(16), None, None,
                                P(256), ws_bytes, None)

    st = qsa.qsa_seq_state(4000, 1000)
    assert call(st, 0) == -1
    assert call(st, qsa.QSA_MAX_CHUNK + 1) == -1
    assert call(st, 97) == -1                       # 4000 + 97 > capacity 4096
    assert b"outside" in L.qsa_last_error()
    assert call(st, 16, q=8) == -1                  # q must be 16-byte aligned
    assert call(st, 16, gamma=0) == -1
    assert call(st, 16, ws_bytes=100) == -3
    assert (st.n_tokens, st.n_valid_blocks) == (4000, 1000)


def test_multi_argument_errors_before_launch():
    qsa, d, c = _objs()
    L = qsa.lib()
    P = ctypes.c_void_p
    D = ctypes.byref(d)
    one = qsa.qsa_multi_workspace_bytes(d, 4096, 1)
    assert one == qsa.qsa_workspace_bytes(d, 4096)
    assert qsa.qsa_multi_workspace_bytes(d, 4096, 4) == 4 * one
    assert qsa.qsa_multi_workspace_bytes(d, 4096, 0) == 0
    assert qsa.qsa_multi_workspace_bytes(d, 4096, qsa.QSA_MAX_MULTI + 1) == 0
    assert qsa.qsa_multi_workspace_bytes(d, 4094, 2) == 0
    # a chunk of at most QSA_MAX_MULTI tokens runs the multi-query path
    assert qsa.qsa_chunk_workspace_bytes(d, 4096, 3) >= qsa.qsa_multi_workspace_bytes(d, 4096, 3)

    def call(st, n_q, q=16, ws_bytes=1 << 40, rows=16):
        return L.qsa_decode_step_multi(D, ctypes.byref(c), ctypes.byref(st), n_q, P(rows), P(16),
                                       P(16), P(16), P(16), P(16), P(q), P(16), None, None, P(256),
                                       ws_bytes, None)

    st = qsa.qsa_seq_state(4093, 1023)
    assert call(st, 0) == -1
    assert call(st, qsa.QSA_MAX_MULTI + 1) == -1
    assert call(st, 4) == -1                        # 4093 + 4 > capacity 4096
    assert b"outside" in L.qsa_last_error()
    assert call(st, 3, q=8) == -1                   # q must be 16-byte aligned
    assert call(st, 3, rows=0) == -1                # null rows
    assert call(st, 3, ws_bytes=100) == -3
    assert (st.n_tokens, st.n_valid_blocks) == (4093, 1023)


def test_ablation_argument_errors_before_launch():
    qsa, d, c = _objs()
    L = qsa.lib()
    P = ctypes.c_void_p
    D, C = ctypes.byref(d), ctypes.byref(c)
    need = qsa.qsa_ablation_workspace_bytes(d, 4096)
    assert need > 0 and need % 256 == 0
    assert qsa.qsa_ablation_workspace_bytes(d, 4094) == 0
    # cell-level top-k
    assert L.qsa_topk_cells(P(16), 0, 2048, P(16), P(256), need, None) == -1
    assert L.qsa_topk_cells(P(16), 4096, 2046, P(16), P(256), need, None) == -1
    assert L.qsa_topk_cells(None, 4096, 2048, P(16), P(256), need, None) == -1
    assert L.qsa_topk_cells(P(16), 4 * (1 << 17) + 4, 2048, P(16), P(256), 1 << 40, None) == -1
    assert L.qsa_topk_cells(P(16), 4096, 2048, P(16), P(256), 64, None) == -3
    # masked attention
    assert L.qsa_attend_masked(D, C, 0, P(16), 0, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_attend_masked(D, C, 4097, P(16), 0, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_attend_masked(D, C, 4096, None, 5, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_attend_masked(D, C, 4096, P(16), 1025, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_attend_masked(D, C, 4096, P(16), 5, P(8), P(16), P(256), need, None) == -1
    assert L.qsa_attend_masked(D, C, 4096, P(16), 5, P(16), P(16), P(256), need - 256, None) == -3
    assert L.qsa_attend_masked(D, C, 4096, None, 0, P(16), P(16), P(256), need, None) == -1   # no cell


def test_q8_0_argument_errors_before_launch():
    qsa, d, c = _objs()
    L = qsa.lib()
    P = ctypes.c_void_p
    D = ctypes.byref(d)
    # quantise: n a non-negative multiple of 32, aligned pointers; 0 values is a no-op
    assert L.qsa_q8_0_quantize(P(16), 31, P(16), P(16), None) == -1
    assert L.qsa_q8_0_quantize(P(16), -32, P(16), P(16), None) == -1
    assert L.qsa_q8_0_quantize(None, 64, P(16), P(16), None) == -1
    assert L.qsa_q8_0_quantize(P(8), 64, P(16), P(16), None) == -1
    assert L.qsa_q8_0_quantize(P(16), 64, P(16), P(17), None) == -1
    assert L.qsa_q8_0_quantize(None, 0, None, None, None) == 0
    # attention over the q8_0 planes
    kv = qsa.qsa_kv_q8_0(0x1000, 0x2000, 0x3000, 0x4000, 4096)
    K = ctypes.byref(kv)
    need = qsa.qsa_workspace_bytes(d, 4096)
    assert L.qsa_gather_attend_q8_0(D, K, 4096, P(16), 5, P(16), P(16), P(256), need - 256, None) == -3
    assert L.qsa_gather_attend_q8_0(D, K, 0, P(16), 0, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_gather_attend_q8_0(D, K, 4097, P(16), 1, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_gather_attend_q8_0(D, K, 4096, P(16), 513, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_gather_attend_q8_0(D, K, 4096, None, 5, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_gather_attend_q8_0(D, K, 4096, P(16), 0, P(16), P(16), P(256), need, None) == -1
    assert L.qsa_gather_attend_q8_0(D, K, 4096, P(16), 5, P(8), P(16), P(256), need, None) == -1
    assert L.qsa_gather_attend_q8_0(D, None, 4096, P(16), 5, P(16), P(16), P(256), need, None) == -1
    for bad in (qsa.qsa_kv_q8_0(0x1000, 0x2000, 0x3000, 0x4008, 4096),
                qsa.qsa_kv_q8_0(0, 0x2000, 0x3000, 0x4000, 4096),
                qsa.qsa_kv_q8_0(0x1000, 0x2000, 0x3000, 0x4000, 4094)):
        assert L.qsa_gather_attend_q8_0(D, ctypes.byref(bad), 4096, P(16), 5, P(16), P(16), P(256),
                                        need, None) == -1
    bad_desc = qsa.make_desc(4, 128, qsa.QSA_F16, 16, 2, 96, 2048)
    assert L.qsa_gather_attend_q8_0(ctypes.byref(bad_desc), K, 4096, P(16), 5, P(16), P(16), P(256),
                                    need, None) < 0


def test_static_workspace_too_small_is_an_error_before_launch():
    """qsa_decode_step_static rejects, before touching the device, a cache
    whose workspace exceeds its static one (many KV heads, large top-k)."""
    import sparse_attention_decode_cache_amd as qsa
    L = qsa.lib()
    d = qsa.make_desc(4, 128, qsa.QSA_F16, 256, 32, 256, 16380)
    c = qsa.qsa_layer_cache(0x1000, 0x2000, 0x3000, 0x4000, 1 << 20)
    assert qsa.qsa_workspace_bytes(d, 1 << 20) > L_STATIC_BYTES
    st = qsa.qsa_seq_state(10, 0)
    rc = L.qsa_decode_step_static(ctypes.byref(d), ctypes.byref(c), ctypes.byref(st),
                                  *[ctypes.c_void_p(16)] * 8, None, None, None)
    assert rc == -3
    assert b"static" in L.qsa_last_error()
    assert (st.n_tokens, st.n_valid_blocks) == (10, 0)


L_STATIC_BYTES = 16 << 20      # QSA_STATIC_SCRATCH_BYTES in include/qsa.h

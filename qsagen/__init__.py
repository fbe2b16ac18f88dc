"""Seeded synthetic inputs for the QSA decode-step tests and benchmark.

This module serves both the GPU path (device fills) and the CPU oracle (host
fills); it holds none of the attention method's arithmetic.  The host and
device fills produce identical bits for the same (seed, tensor id, element
index), so the oracle can regenerate any row without copying the GPU's
buffers back.  See ``csrc/qsagen_core.h`` for the definitions.

Element indexing: a cache tensor of rows [position][...] uses one stream per
(kind, sequence, layer); element (t, j) has index t * row_len + j, so the row
appended at step s is simply row n0 + s of the same stream.  Per-step query
tensors use one stream per (kind, sequence, layer, step).
"""
import ctypes
import os
import subprocess
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HOST_LIB = os.path.join(HERE, "libqsagen_host.so")
DEV_LIB = os.path.join(HERE, "libqsagen_dev.so")

KIND_RAW, KIND_K, KIND_V, KIND_QIDX, KIND_W, KIND_Q, KIND_GAMMA = 1, 2, 3, 4, 5, 6, 7
BASE_SEED = 0x51534100

HIP_FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def tensor_id(kind, layer=0, step=0, seq=0):
    """Distinct 64-bit id per (kind, sequence, layer, step)."""
    return (int(kind) << 56) | (int(seq) << 40) | (int(layer) << 24) | int(step)


def build(verbose=False):
    """Compile the host fill library (gcc) and the device fill library (hipcc, gfx950)."""
    src_h = os.path.join(CSRC, "qsagen_host.c")
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-o", HOST_LIB + ".tmp", src_h]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(HOST_LIB + ".tmp", HOST_LIB)
    src_d = os.path.join(CSRC, "qsagen_dev.hip")
    cmd = ["hipcc", *HIP_FLAGS, "-o", DEV_LIB + ".tmp", src_d]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(DEV_LIB + ".tmp", DEV_LIB)


_host = None
_dev = None


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build()
        L = ctypes.CDLL(HOST_LIB)
        u64, P = ctypes.c_uint64, ctypes.c_void_p
        L.qsagen_host_normal_f32.argtypes = [P, u64, u64, u64]
        L.qsagen_host_unit_f32.argtypes = [P, u64, u64, u64, ctypes.c_float]
        L.qsagen_host_normal_rows_f32.argtypes = [P, P, u64, u64, u64]
        L.qsagen_host_stream.restype = u64
        L.qsagen_host_stream.argtypes = [u64, u64]
        L.qsagen_host_mix.restype = u64
        L.qsagen_host_mix.argtypes = [u64]
        _host = L
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(DEV_LIB)
        u64, P = ctypes.c_uint64, ctypes.c_void_p
        L.qsagen_dev_normal_f16.argtypes = [P, u64, u64, u64, P]
        L.qsagen_dev_normal_f32.argtypes = [P, u64, u64, u64, P]
        L.qsagen_dev_unit_f32.argtypes = [P, u64, u64, u64, ctypes.c_float, P]
        for f in (L.qsagen_dev_normal_f16, L.qsagen_dev_normal_f32, L.qsagen_dev_unit_f32):
            f.restype = ctypes.c_int
        _dev = L
    return _dev


def mix(x):
    return int(host_lib().qsagen_host_mix(int(x) & (2**64 - 1)))


def stream_of(seed, tid):
    return int(host_lib().qsagen_host_stream(int(seed) & (2**64 - 1), int(tid) & (2**64 - 1)))


# ---------------------------------------------------------------- host fills
def host_normal(shape, seed, tid, e0=0, dtype=np.float32):
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    host_lib().qsagen_host_normal_f32(out.ctypes.data_as(ctypes.c_void_p), n,
                                      stream_of(seed, tid), int(e0))
    return out.reshape(shape).astype(dtype)


def host_unit(shape, seed, tid, e0=0, offset=0.0):
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    host_lib().qsagen_host_unit_f32(out.ctypes.data_as(ctypes.c_void_p), n,
                                    stream_of(seed, tid), int(e0), float(offset))
    return out.reshape(shape)


def host_rows(rows, row_shape, seed, tid, dtype=np.float32):
    """Rows `rows` (positions) of a [positions, *row_shape] normal tensor."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    row_len = int(np.prod(row_shape))
    out = np.empty((rows.shape[0], row_len), np.float32)
    host_lib().qsagen_host_normal_rows_f32(out.ctypes.data_as(ctypes.c_void_p),
                                           rows.ctypes.data_as(ctypes.c_void_p),
                                           rows.shape[0], row_len, stream_of(seed, tid))
    return out.reshape((rows.shape[0],) + tuple(row_shape)).astype(dtype)


# -------------------------------------------------------------- device fills
def _stream_handle(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dev_normal_(t, seed, tid, e0=0, stream=None):
    """Fill a contiguous torch float16/float32 CUDA tensor in place."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    st = stream_of(seed, tid)
    if t.dtype == torch.float16:
        rc = dev_lib().qsagen_dev_normal_f16(t.data_ptr(), t.numel(), st, int(e0), _stream_handle(stream))
    elif t.dtype == torch.float32:
        rc = dev_lib().qsagen_dev_normal_f32(t.data_ptr(), t.numel(), st, int(e0), _stream_handle(stream))
    else:
        raise TypeError(t.dtype)
    if rc != 0:
        raise RuntimeError(f"qsagen device fill failed ({rc})")
    return t


def dev_unit_(t, seed, tid, e0=0, offset=0.0, stream=None):
    import torch
    assert t.is_cuda and t.is_contiguous() and t.dtype == torch.float32
    rc = dev_lib().qsagen_dev_unit_f32(t.data_ptr(), t.numel(), stream_of(seed, tid), int(e0),
                                       float(offset), _stream_handle(stream))
    if rc != 0:
        raise RuntimeError(f"qsagen device fill failed ({rc})")
    return t

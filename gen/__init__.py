"""Seeded synthetic inputs for the five workloads.

A module of its own: it holds none of the method's arithmetic and is the only
code that both the oracle side and the HIP side consume (they consume its
arrays; neither calls the other).  Generation runs in C (``gen/csrc/sg_gen.c``)
with counter-based SplitMix64 streams, so results do not depend on the thread
count.

Workloads (sizes from the method's own settings):
  1  n=4 workers, dense fp32 M=2^20, 1% nonzeros per worker drawn Zipf(1.1)
     without replacement, N(0,1) values; P=4.
  2  embedding rows: table 1,000,000 x 64 fp32, n=8, 4096 distinct Zipf(1.05)
     rows per worker, N(0, sigma=0.01) values; P=8.
  3  DGC-style: n=8 dense 4096 x 11008 fp32, N(0,1) x per-row lognormal(0,1)
     scale, 0.7 inter-worker correlation; top 5%; P=8.
  4  skewed: n=16, M=2^28, 1% per worker, 60% of each worker's nonzeros uniform
     in [0, M/8), the rest uniform in [M/8, M); N(0,1) values; P=16.
  5  dense reduce-scatter: n=8 buffers of 2^26 fp32 N(0,1), 256 KiB slices,
     p_skip=0.5, DropReduce rescale.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "sg_gen.c")
_LIB = os.path.join(_HERE, "libsggen.so")

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        L.gen_normal_f32.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_double, _f32p]
        L.gen_normal_f32.restype = None
        L.gen_normal_nonzero_f32.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_double, _f32p]
        L.gen_normal_nonzero_f32.restype = None
        L.gen_uniform_distinct.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_uint64, _u32p]
        L.gen_uniform_distinct.restype = C.c_int
        L.gen_zipf_distinct.argtypes = [C.c_uint64, C.c_uint64, C.c_double, C.c_uint64, _u32p]
        L.gen_zipf_distinct.restype = C.c_int
        L.gen_rowscaled_dense.argtypes = [C.c_uint64, C.c_uint32, C.c_uint64, C.c_uint64, C.c_double, _f32p]
        L.gen_rowscaled_dense.restype = None
        L.gen_f32_to_bf16.argtypes = [_f32p, C.c_uint64, _u16p]
        L.gen_f32_to_bf16.restype = None
        L.gen_num_threads.restype = C.c_int
        _lib = L
    return _lib


def stream_seed(workload: int, stream: int) -> int:
    return ((workload & 0xFFFFFFFF) << 32) | (stream & 0xFFFFFFFF)


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------

def normal(seed: int, count: int, sigma: float = 1.0, first: int = 0, nonzero: bool = False) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    if count:
        f = lib().gen_normal_nonzero_f32 if nonzero else lib().gen_normal_f32
        f(seed, first, count, sigma, out)
    return out


def uniform_distinct(seed: int, lo: int, hi: int, count: int) -> np.ndarray:
    out = np.empty(max(count, 1), dtype=np.uint32)
    if count and lib().gen_uniform_distinct(seed, lo, hi, count, out) != 0:
        raise ValueError("cannot draw %d distinct values from [%d, %d)" % (count, lo, hi))
    return out[:count]


def zipf_distinct(seed: int, R: int, s: float, count: int) -> np.ndarray:
    out = np.empty(max(count, 1), dtype=np.uint32)
    if count and lib().gen_zipf_distinct(seed, R, s, count, out) != 0:
        raise ValueError("cannot draw %d distinct Zipf ranks from %d" % (count, R))
    return out[:count]


def to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns (uint16) of a float32 array."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    if a.size:
        lib().gen_f32_to_bf16(a.reshape(-1), a.size, out.reshape(-1))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def coo_from_lists(lists, vals):
    """Concatenate per-worker sorted index lists into (idx, in_off, val)."""
    in_off = np.zeros(len(lists) + 1, dtype=np.uint64)
    for w, l in enumerate(lists):
        in_off[w + 1] = in_off[w] + len(l)
    idx = np.concatenate(lists).astype(np.uint32) if lists else np.zeros(0, np.uint32)
    val = np.concatenate(vals) if vals else None
    return idx, in_off, val


def coo_zipf(workload: int, n: int, R: int, count: int, s: float, D: int = 1, sigma: float = 1.0,
             nonzero: bool = False):
    """n workers, each `count` distinct Zipf(s) indices over [0, R), sorted,
    with N(0, sigma) values ([count] if D == 1 else [count, D])."""
    lists, vals = [], []
    for w in range(n):
        lists.append(zipf_distinct(stream_seed(workload, w), R, s, count))
        v = normal(stream_seed(workload, 100 + w), count * D, sigma, nonzero=nonzero)
        vals.append(v if D == 1 else v.reshape(count, D))
    return coo_from_lists(lists, vals)


def coo_skewed(workload: int, n: int, M: int, count: int, head_frac: float, head_range: int):
    """n workers, each `count` distinct indices: floor(head_frac*count) uniform
    without replacement in [0, head_range), the rest uniform without replacement
    in [head_range, M).  N(0,1) values."""
    h = int(head_frac * count)
    t = count - h
    lists, vals = [], []
    for w in range(n):
        a = uniform_distinct(stream_seed(workload, 2 * w), 0, head_range, h)
        b = uniform_distinct(stream_seed(workload, 2 * w + 1), head_range, M, t)
        lists.append(np.concatenate([a, b]))
        vals.append(normal(stream_seed(workload, 100 + w), count))
    return coo_from_lists(lists, vals)


def dense_from_coo(n: int, M: int, idx: np.ndarray, in_off: np.ndarray, val: np.ndarray) -> np.ndarray:
    dense = np.zeros((n, M), dtype=np.float32)
    for w in range(n):
        b, e = int(in_off[w]), int(in_off[w + 1])
        dense[w, idx[b:e]] = val[b:e]
    return dense


def dense_rowscaled(workload: int, n: int, rows: int, cols: int, rho: float = 0.7) -> np.ndarray:
    out = np.empty((n, rows * cols), dtype=np.float32)
    if out.size:
        lib().gen_rowscaled_dense(stream_seed(workload, 0), n, rows, cols, rho, out.reshape(-1))
    return out


def dense_normal(workload: int, n: int, M: int) -> np.ndarray:
    return normal(stream_seed(workload, 0), n * M).reshape(n, M)


# --------------------------------------------------------------------------
# the five workloads (full size by default; tests use the `scale` knobs)
# --------------------------------------------------------------------------

CFG1 = dict(n=4, M=1 << 20, density_div=100, s=1.1, P=4, seed=1)
CFG2 = dict(n=8, rows=1_000_000, D=64, count=4096, s=1.05, sigma=0.01, P=8, seed=2)
CFG3 = dict(n=8, rows=4096, cols=11008, density_div=20, rho=0.7, P=8, seed=3)
CFG4 = dict(n=16, M=1 << 28, density_div=100, head_frac=0.6, P=16, seed=4)
CFG5 = dict(n=8, M=1 << 26, slice_bytes=256 * 1024, p=0.5, mode=1, seed=5)


def config1(n=4, M=1 << 20):
    """Dense fp32 per worker holding floor(M/100) Zipf(1.1) nonzeros; returns
    dense [n, M] plus the COO it was built from (k = nnz per worker)."""
    c = M // 100
    idx, in_off, val = coo_zipf(1, n, M, c, 1.1, nonzero=True)
    dense = dense_from_coo(n, M, idx, in_off, val)
    return dict(dense=dense, idx=idx, in_off=in_off, val=val, n=n, M=M, k=c, P=4, seed=1)


def config2(n=8, rows=1_000_000, D=64, count=4096):
    idx, in_off, val = coo_zipf(2, n, rows, count, 1.05, D=D, sigma=0.01)
    return dict(idx=idx, in_off=in_off, val=val, n=n, M=rows, D=D, P=8, seed=2)


def config3(n=8, rows=4096, cols=11008):
    dense = dense_rowscaled(3, n, rows, cols, 0.7)
    M = rows * cols
    return dict(dense=dense, n=n, M=M, k=M // 20, P=8, seed=3)


def config4(n=16, M=1 << 28):
    c = M // 100
    idx, in_off, val = coo_skewed(4, n, M, c, 0.6, M // 8)
    return dict(idx=idx, in_off=in_off, val=val, n=n, M=M, P=16, seed=4)


def config5(n=8, M=1 << 26):
    return dict(bufs=dense_normal(5, n, M), n=n, M=M, slice_elems=(256 * 1024) // 4, p=0.5, mode=1, seed=5)

"""CPU oracle for the sparse gradient synchronization hot path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``sparse_gradient_synchronization_amd``) never imports, links or calls
it, and the two share no code: this wrapper drives ``oracle/sg_oracle.c``, a
plain single-threaded C file built with gcc (``-O2 -ffp-contract=off``).

Each function cites, in its docstring, the passage of the pages it follows
(titles and sections are spelled out in ``sg_oracle.c``).  Floating-point sums
are returned in float64.

Parity unpinned: whether MurmurHash2 (32-bit, 4 little-endian index bytes,
mod P) is the hash the Zen authors ran.  The page names only "MurmurHash 2.0".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sg_oracle.c")
_LIB = os.path.join(_HERE, "libsgoracle.so")

F32, BF16 = 0, 1

_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(dtype=np.uint64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (single-threaded, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
             "-Wall", "-Wno-unused-function", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _StatsOut(C.Structure):
    _fields_ = [
        ("union_size", C.c_uint64), ("sum_nnz", C.c_uint64), ("max_nnz", C.c_uint64),
        ("nnz", C.c_void_p), ("inter", C.c_void_p), ("overlap", C.c_void_p),
        ("overlap_mean", C.c_double), ("overlap_min", C.c_double), ("overlap_max", C.c_double),
        ("gamma_n", C.c_double),
        ("contig_counts", C.c_void_p), ("skew_contig", C.c_void_p),
        ("class_size", C.c_void_p), ("hashed_counts", C.c_void_p), ("skew_hashed", C.c_void_p),
        ("push_imbalance", C.c_double), ("pull_imbalance", C.c_double),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        L.orc_murmur2.restype = C.c_uint32
        L.orc_murmur2.argtypes = [C.c_char_p, C.c_uint64, C.c_uint32]
        L.orc_h0.restype = C.c_uint32
        L.orc_h0.argtypes = [C.c_uint32, C.c_uint32, C.c_uint32]
        L.orc_h0_array.restype = None
        L.orc_h0_array.argtypes = [_u32p, C.c_uint64, C.c_uint32, C.c_uint32, _u32p]
        L.orc_splitmix64_next.restype = C.c_uint64
        L.orc_splitmix64_next.argtypes = [C.POINTER(C.c_uint64)]
        L.orc_splitmix64_at.restype = C.c_uint64
        L.orc_splitmix64_at.argtypes = [C.c_uint64, C.c_uint64]
        L.orc_topk_to_coo.restype = C.c_int
        L.orc_topk_to_coo.argtypes = [C.c_void_p, C.c_int, C.c_uint32, C.c_uint64, C.c_uint64,
                                      _u32p, C.c_void_p]
        L.orc_hash_partition.restype = C.c_int
        L.orc_hash_partition.argtypes = [_u32p, C.c_void_p, C.c_int, C.c_uint32, _u64p, C.c_uint32,
                                         C.c_uint32, C.c_uint32, _u32p, C.c_void_p, _u64p]
        L.orc_aggregate.restype = C.c_int
        L.orc_aggregate.argtypes = [_u32p, C.c_void_p, C.c_int, C.c_uint32, _u64p, C.c_uint32,
                                    C.c_uint32, C.c_uint64, _u32p, _f64p, _f64p, _u64p]
        L.orc_classmap.restype = C.c_int
        L.orc_classmap.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, _u64p, _u32p]
        L.orc_encode.restype = C.c_int
        L.orc_encode.argtypes = [_u32p, _u64p, C.c_uint32, C.c_uint64, C.c_uint32, _u32p, _u64p]
        L.orc_decode.restype = C.c_int
        L.orc_decode.argtypes = [_u32p, C.c_uint32, C.c_uint64, C.c_uint32, _u32p, _u64p]
        L.orc_scatter_dense.restype = C.c_int
        L.orc_scatter_dense.argtypes = [_u32p, _f32p, C.c_uint32, _u64p, C.c_uint32, C.c_uint64, _f32p]
        L.orc_format_sizes.restype = C.c_int
        L.orc_format_sizes.argtypes = [_u32p, _u64p, C.c_uint32, C.c_uint64, C.c_uint32, C.c_uint32, _u64p]
        L.orc_skip_mask_static.restype = C.c_int
        L.orc_skip_mask_static.argtypes = [C.c_uint32, C.c_uint64, C.c_uint32, _u8p]
        L.orc_skip_mask_random.restype = C.c_int
        L.orc_skip_mask_random.argtypes = [C.c_uint32, C.c_uint64, C.c_uint32, C.c_uint64, _u8p]
        L.orc_dropout_reduce_scatter.restype = C.c_int
        L.orc_dropout_reduce_scatter.argtypes = [C.c_void_p, C.c_int, C.c_uint32, C.c_uint64, C.c_double, C.c_uint64,
                                                 C.c_int, _f64p, _f64p, C.c_void_p]
        L.orc_selective_reduce_scatter.restype = C.c_int
        L.orc_selective_reduce_scatter.argtypes = [C.c_void_p, C.c_int, C.c_uint32, C.c_uint64, C.c_uint32, _u64p,
                                                   _f64p, C.c_uint64, C.c_uint64, C.c_int, _f64p, _f64p]
        L.orc_allgather.restype = C.c_int
        L.orc_allgather.argtypes = [_f64p, C.c_void_p, C.c_int, C.c_uint32, C.c_uint64, C.c_void_p, _f64p]
        L.orc_hierarchical_hash.restype = C.c_int
        L.orc_hierarchical_hash.argtypes = [_u32p, C.c_void_p, C.c_int, C.c_uint32, _u64p, C.c_uint32, C.c_uint32,
                                            C.c_uint32, C.c_uint32, C.c_uint64, C.c_uint64, _u32p, C.c_void_p, _u64p,
                                            _u32p, _u64p]
        L.orc_dgc_sample_pos.restype = C.c_uint64
        L.orc_dgc_sample_pos.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64]
        L.orc_dgc_rank.restype = C.c_uint64
        L.orc_dgc_rank.argtypes = [C.c_double, C.c_uint64]
        L.orc_dgc_select.restype = C.c_int
        L.orc_dgc_select.argtypes = [_f32p, _f32p, C.c_uint32, C.c_uint64, C.c_double, C.c_uint64, _u32p, _f32p,
                                     C.c_uint64, _u64p, C.POINTER(C.c_uint32)]
        L.orc_skip_threshold.restype = C.c_uint32
        L.orc_skip_threshold.argtypes = [C.c_double]
        L.orc_skip_mask.restype = C.c_int
        L.orc_skip_mask.argtypes = [C.c_uint32, C.c_uint64, C.c_double, C.c_uint64, _u8p]
        L.orc_skip_reduce_scatter.restype = C.c_int
        L.orc_skip_reduce_scatter.argtypes = [C.c_void_p, C.c_int, C.c_uint32, C.c_uint64, C.c_uint64,
                                              C.c_double, C.c_uint64, C.c_void_p, C.c_int,
                                              _f64p, _f64p, C.c_void_p]
        L.orc_ring_replay.restype = C.c_int
        L.orc_ring_replay.argtypes = [C.c_void_p, C.c_int, C.c_uint32, C.c_uint64, C.c_uint64,
                                      _u8p, _f64p]
        L.orc_stats.restype = C.c_int
        L.orc_stats.argtypes = [_u32p, _u64p, C.c_uint32, C.c_uint64, C.c_uint32, C.c_int, C.c_uint32,
                                C.POINTER(_StatsOut)]
        _lib = L
    return _lib


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with status %d" % (what, rc))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError("values must be float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


# --------------------------------------------------------------------------
# hash and random numbers
# --------------------------------------------------------------------------

def murmur2(data: bytes, seed: int) -> int:
    """MurmurHash2 (32-bit) of a byte string: the hash family that the Zen page
    (section 4, Implementation) names as "MurmurHash 2.0"."""
    return int(lib().orc_murmur2(data, len(data), seed & 0xFFFFFFFF))


def h0(idx, seed: int, P: int):
    """First-level partition hash of Zen section 3.2 (Technique #3): the
    MurmurHash2 of the index's 4 little-endian bytes, mod P."""
    if np.isscalar(idx):
        return int(lib().orc_h0(int(idx), seed, P))
    a = np.ascontiguousarray(idx, dtype=np.uint32)
    out = np.empty_like(a)
    lib().orc_h0_array(a, a.size, seed, P, out)
    return out


def splitmix64_outputs(seed: int, count: int):
    """The first `count` outputs of SplitMix64 started at `seed`."""
    s = C.c_uint64(seed & 0xFFFFFFFFFFFFFFFF)
    return [int(lib().orc_splitmix64_next(C.byref(s))) for _ in range(count)]


def splitmix64_at(seed: int, ctr: int) -> int:
    return int(lib().orc_splitmix64_at(seed & 0xFFFFFFFFFFFFFFFF, ctr))


# --------------------------------------------------------------------------
# the six operations
# --------------------------------------------------------------------------

def topk_to_coo(dense: np.ndarray, k: int):
    """Per-worker exact top-k by |value| into COO, ascending index order, ties
    toward the lower index (Skip section 2; Zen section 4, DGC top-5%).
    dense: [n, M] float32 or uint16 (bf16 bits).  Returns idx [n, k] uint32 and
    val [n, k] of the input dtype (bit copies)."""
    dense = np.ascontiguousarray(dense)
    n, M = dense.shape
    idx = np.zeros((n, k), dtype=np.uint32)
    val = np.zeros((n, k), dtype=dense.dtype)
    _check(lib().orc_topk_to_coo(_ptr(dense), _dtype_code(dense), n, M, k, idx.reshape(-1), _ptr(val)),
           "topk_to_coo")
    return idx, val


def dgc_sample_pos(M: int, S: int, j: int) -> int:
    return int(lib().orc_dgc_sample_pos(M, S, j))


def dgc_rank(density: float, Ns: int) -> int:
    return int(lib().orc_dgc_rank(density, Ns))


def dgc_select(grad: np.ndarray, resid: np.ndarray, density: float, S: int, cap: int | None = None):
    """One DGC iteration with a sampled global threshold and residuals (Zen
    section 4; Skip section 2).  grad, resid: [n, M] float32 (resid is not
    modified; the new residual is returned).  Returns (idx [n, cap] uint32,
    val [n, cap] float32, count [n] uint64, new_resid [n, M], thr_key)."""
    grad = np.ascontiguousarray(grad, dtype=np.float32)
    r = np.array(resid, dtype=np.float32, copy=True, order="C")
    n, M = grad.shape
    cap = M if cap is None else cap
    idx = np.zeros((n, max(cap, 1)), dtype=np.uint32)
    val = np.zeros((n, max(cap, 1)), dtype=np.float32)
    cnt = np.zeros(n, dtype=np.uint64)
    thr = C.c_uint32(0)
    _check(lib().orc_dgc_select(grad.reshape(-1), r.reshape(-1), n, M, density, S, idx.reshape(-1), val.reshape(-1),
                                max(cap, 1) if cap else 0, cnt, C.byref(thr)), "dgc_select")
    return idx[:, :cap], val[:, :cap], cnt, r, int(thr.value)


def hash_partition(idx: np.ndarray, val, in_off: np.ndarray, P: int, seed: int):
    """Stable grouping of each worker's entries by h0 (Zen section 3.1 Problem 1,
    section 3.2 Technique #3).  val: None, [total] or [total, D].
    Returns out_idx, out_val, part_off [n, P+1] (absolute)."""
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    in_off = np.ascontiguousarray(in_off, dtype=np.uint64)
    n = in_off.size - 1
    if val is None:
        D, vptr, code, out_val = 0, None, F32, None
    else:
        val = np.ascontiguousarray(val)
        D = 1 if val.ndim == 1 else val.shape[1]
        code = _dtype_code(val)
        out_val = np.empty_like(val)
        vptr = _ptr(val)
    out_idx = np.empty_like(idx)
    part_off = np.zeros((n, P + 1), dtype=np.uint64)
    _check(lib().orc_hash_partition(idx, vptr, code, D, in_off, n, P, seed, out_idx,
                                    None if out_val is None else _ptr(out_val), part_off.reshape(-1)),
           "hash_partition")
    return out_idx, out_val, part_off


def hierarchical_hash(idx: np.ndarray, val, in_off: np.ndarray, P: int, seed: int, k: int, r1: int, r2: int):
    """Algorithm 1 of the Zen page (section 3.2), run sequentially.  val: None,
    [total] or [total, D].  Returns out_idx, out_val, part_off [n, P+1],
    slot_of [total] and counts [n, 2] (serial writes, lost entries)."""
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    in_off = np.ascontiguousarray(in_off, dtype=np.uint64)
    n = in_off.size - 1
    total = idx.size
    D = 0 if val is None else (1 if val.ndim == 1 else val.shape[1])
    out_idx = np.zeros(max(total, 1), dtype=np.uint32)
    slot_of = np.zeros(max(total, 1), dtype=np.uint32)
    part_off = np.zeros(n * (P + 1), dtype=np.uint64)
    counts = np.zeros(max(2 * n, 1), dtype=np.uint64)
    if val is None:
        out_val, vp, dt = None, None, F32
    else:
        v = np.ascontiguousarray(val)
        out_val = np.zeros_like(v) if total else np.zeros((1,) + v.shape[1:], v.dtype)
        vp, dt = _ptr(v), _dtype_code(v)
    _check(lib().orc_hierarchical_hash(idx if total else np.zeros(1, np.uint32), vp, dt, D, in_off, n, P, seed, k, r1,
                                       r2, out_idx, None if out_val is None else _ptr(out_val), part_off, slot_of,
                                       counts), "hierarchical_hash")
    return (out_idx[:total], None if out_val is None else out_val[:total], part_off.reshape(n, P + 1),
            slot_of[:total], counts[: 2 * n].reshape(n, 2))


def aggregate(idx: np.ndarray, val, part_off: np.ndarray, M: int):
    """Per-partition union-sum in float64 (Zen section 3.1, server-side
    aggregation; section 3.2, equal to the dense AllReduce result).
    part_off: [n, P+1].  Returns agg_idx, agg_val (float64), agg_abs (float64,
    sum of |x| of the same terms), agg_off [P+1]."""
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    part_off = np.ascontiguousarray(part_off, dtype=np.uint64)
    n, P1 = part_off.shape
    P = P1 - 1
    if val is None:
        D, vptr, code = 0, None, F32
    else:
        val = np.ascontiguousarray(val)
        D = 1 if val.ndim == 1 else val.shape[1]
        code = _dtype_code(val)
        vptr = _ptr(val)
    cap = max(1, idx.size)
    Dv = max(D, 1)
    agg_idx = np.zeros(cap, dtype=np.uint32)
    agg_val = np.zeros(cap * Dv, dtype=np.float64)
    agg_abs = np.zeros(cap * Dv, dtype=np.float64)
    agg_off = np.zeros(P + 1, dtype=np.uint64)
    _check(lib().orc_aggregate(idx, vptr, code, D, part_off.reshape(-1), n, P, M, agg_idx, agg_val,
                               agg_abs, agg_off), "aggregate")
    u = int(agg_off[P])
    agg_val = agg_val[: u * Dv]
    agg_abs = agg_abs[: u * Dv]
    if D > 1:
        agg_val = agg_val.reshape(u, D)
        agg_abs = agg_abs.reshape(u, D)
    return agg_idx[:u].copy(), agg_val.copy(), agg_abs.copy(), agg_off


def classmap(M: int, P: int, seed: int):
    """Class sizes |C_p| and each index's rank inside its class C_p (Zen
    section 3.3.2: the per-server index sets, fixed offline by h0)."""
    size = np.zeros(P, dtype=np.uint64)
    rank = np.zeros(max(M, 1), dtype=np.uint32)
    _check(lib().orc_classmap(M, P, seed, size, rank), "classmap")
    return size, rank[:M]


def encode(agg_idx: np.ndarray, agg_off: np.ndarray, M: int, seed: int):
    """Hash bitmap of Zen section 3.3.2 (Fig. 10).  Returns bitmap (uint32
    words) and word_off [P+1]."""
    agg_idx = np.ascontiguousarray(agg_idx, dtype=np.uint32)
    if agg_idx.size == 0:
        agg_idx = np.zeros(1, dtype=np.uint32)
    agg_off = np.ascontiguousarray(agg_off, dtype=np.uint64)
    P = agg_off.size - 1
    bitmap = np.zeros(M // 32 + P + 1, dtype=np.uint32)
    word_off = np.zeros(P + 1, dtype=np.uint64)
    _check(lib().orc_encode(agg_idx, agg_off, P, M, seed, bitmap, word_off), "encode")
    return bitmap[: int(word_off[P])].copy(), word_off


def decode(bitmap: np.ndarray, P: int, M: int, seed: int):
    """Hash-bitmap decode (Zen section 3.3.2): bits back to global indices."""
    bitmap = np.ascontiguousarray(bitmap, dtype=np.uint32)
    if bitmap.size == 0:
        bitmap = np.zeros(1, dtype=np.uint32)
    out = np.zeros(max(M, 1), dtype=np.uint32)
    off = np.zeros(P + 1, dtype=np.uint64)
    _check(lib().orc_decode(bitmap, P, M, seed, out, off), "decode")
    return out[: int(off[P])].copy(), off


def scatter_dense(idx: np.ndarray, val: np.ndarray, off: np.ndarray, M: int, D: int = 1):
    """Pull-side scatter (Zen sections 3.1, 3.3.2): dense [M] (or [M, D])
    zero except the aggregated indices, which take their values."""
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    val = np.ascontiguousarray(val, dtype=np.float32).reshape(-1)
    off = np.ascontiguousarray(off, dtype=np.uint64)
    if idx.size == 0:
        idx = np.zeros(1, dtype=np.uint32)
    if val.size == 0:
        val = np.zeros(1, dtype=np.float32)
    P = off.size - 1
    out = np.zeros(max(M * max(D, 1), 1), dtype=np.float32)
    _check(lib().orc_scatter_dense(idx, val, D, off, P, M, out), "scatter_dense")
    out = out[: M * max(D, 1)]
    return out if D <= 1 else out.reshape(M, D)


FORMAT_NAMES = ("dense", "coo", "block", "bitmap", "hash_bitmap", "union", "nonempty_blocks")


def format_sizes(agg_idx: np.ndarray, agg_off: np.ndarray, M: int, D: int, seed: int) -> dict:
    """Bytes of an aggregate under the formats of Zen sections 3.3.1-3.3.2
    (dense, COO, 256-gradient tensor blocks, contiguous-range bitmap, hash
    bitmap), plus |I| and the number of non-empty blocks."""
    agg_idx = np.ascontiguousarray(agg_idx, dtype=np.uint32)
    if agg_idx.size == 0:
        agg_idx = np.zeros(1, dtype=np.uint32)
    agg_off = np.ascontiguousarray(agg_off, dtype=np.uint64)
    out = np.zeros(7, dtype=np.uint64)
    _check(lib().orc_format_sizes(agg_idx, agg_off, agg_off.size - 1, M, D, seed, out), "format_sizes")
    return {k: int(v) for k, v in zip(FORMAT_NAMES, out)}


def skip_threshold(p: float) -> int:
    return int(lib().orc_skip_threshold(p))


def num_slices(n: int, M: int, slice_elems: int) -> int:
    maxchunk = (M + n - 1) // n
    return (maxchunk + slice_elems - 1) // slice_elems if maxchunk else 0


def skip_mask(n: int, S: int, p: float, seed: int) -> np.ndarray:
    """Seeded inclusion mask [n chunks, n ring positions, S slices] (Skip
    section 4.3, Random SkipReduce with a shared seed)."""
    m = np.zeros(max(1, n * n * S), dtype=np.uint8)
    _check(lib().orc_skip_mask(n, S, p, seed, m), "skip_mask")
    return m[: n * n * S].reshape(n, n, S)


def skip_reduce_scatter(bufs: np.ndarray, slice_elems: int, p: float, seed: int, include=None,
                        mode: int = 1):
    """Ring reduce-scatter with slice skipping (CMU ring aggregation phase; Skip
    sections 4.1-4.3).  bufs: [n, M] float32 or uint16 (bf16).  Returns
    out (float64 [M]), out_abs (float64 [M]), count (uint8 [n, S])."""
    bufs = np.ascontiguousarray(bufs)
    n, M = bufs.shape
    S = num_slices(n, M, slice_elems)
    out = np.zeros(max(M, 1), dtype=np.float64)
    out_abs = np.zeros(max(M, 1), dtype=np.float64)
    count = np.zeros(max(1, n * S), dtype=np.uint8)
    inc_ptr = None
    if include is not None:
        include = np.ascontiguousarray(include, dtype=np.uint8)
        assert include.size == n * n * S
        inc_ptr = _ptr(include)
    _check(lib().orc_skip_reduce_scatter(_ptr(bufs), _dtype_code(bufs), n, M, slice_elems, p, seed, inc_ptr,
                                         mode, out, out_abs, _ptr(count)), "skip_reduce_scatter")
    return out[:M], out_abs[:M], count[: n * S].reshape(n, S)


def skip_mask_static(n: int, S: int, k: int) -> np.ndarray:
    """Static SkipReduce(k) mask (Skip section 4.2, Algorithm 2): t >= k kept."""
    m = np.zeros(max(1, n * n * S), dtype=np.uint8)
    _check(lib().orc_skip_mask_static(n, S, k, m), "skip_mask_static")
    return m[: n * n * S].reshape(n, n, S)


def skip_mask_random(n: int, S: int, k: int, seed: int) -> np.ndarray:
    """Random SkipReduce mask (Skip section 4.3): the static mask rotated by a
    shared random offset."""
    m = np.zeros(max(1, n * n * S), dtype=np.uint8)
    _check(lib().orc_skip_mask_random(n, S, k, seed, m), "skip_mask_random")
    return m[: n * n * S].reshape(n, n, S)


def dropout_reduce_scatter(bufs: np.ndarray, p: float, seed: int, mode: int = 1):
    """AllReduce_Dropout (Skip section 4.2, Algorithm 1): per-element skipping.
    Returns out, out_abs (float64 [M]) and count (uint8 [M])."""
    bufs = np.ascontiguousarray(bufs)
    n, M = bufs.shape
    out = np.zeros(max(M, 1), dtype=np.float64)
    out_abs = np.zeros(max(M, 1), dtype=np.float64)
    count = np.zeros(max(M, 1), dtype=np.uint8)
    _check(lib().orc_dropout_reduce_scatter(_ptr(bufs), _dtype_code(bufs), n, M, p, seed, mode, out, out_abs,
                                            _ptr(count)), "dropout_reduce_scatter")
    return out[:M], out_abs[:M], count[:M]


def selective_reduce_scatter(bufs: np.ndarray, bucket_off, p, seed: int, slice_elems: int, mode: int = 1):
    """Selective SkipReduce (Skip section 4.4): a skip rate per bucket."""
    bufs = np.ascontiguousarray(bufs)
    n, M = bufs.shape
    bo = np.ascontiguousarray(bucket_off, dtype=np.uint64)
    pr = np.ascontiguousarray(p, dtype=np.float64)
    out = np.zeros(max(M, 1), dtype=np.float64)
    out_abs = np.zeros(max(M, 1), dtype=np.float64)
    _check(lib().orc_selective_reduce_scatter(_ptr(bufs), _dtype_code(bufs), n, M, pr.size, bo, pr, seed, slice_elems,
                                              mode, out, out_abs), "selective_reduce_scatter")
    return out[:M], out_abs[:M]


def allgather(reduced: np.ndarray, bufs: np.ndarray, ag_include=None) -> np.ndarray:
    """The ring's AllGather of a reduced tensor (CMU broadcast phase), with an
    optional delivery mask [n chunks, n positions]; returns [n, M] float64."""
    bufs = np.ascontiguousarray(bufs)
    n, M = bufs.shape
    red = np.ascontiguousarray(reduced, dtype=np.float64)
    out = np.zeros(max(n * M, 1), dtype=np.float64)
    inc = None if ag_include is None else np.ascontiguousarray(ag_include, dtype=np.uint8)
    _check(lib().orc_allgather(red if red.size else np.zeros(1), _ptr(bufs), _dtype_code(bufs), n, M,
                               None if inc is None else _ptr(inc), out), "allgather")
    return out[: n * M].reshape(n, M)


def ring_replay(bufs: np.ndarray, slice_elems: int, include: np.ndarray) -> np.ndarray:
    """Step-by-step replay of the ring with the send/receive slice indices of
    Skip Algorithms 1-2 (no rescale).  Test use only."""
    bufs = np.ascontiguousarray(bufs)
    n, M = bufs.shape
    include = np.ascontiguousarray(include, dtype=np.uint8).reshape(-1)
    if include.size == 0:
        include = np.zeros(1, dtype=np.uint8)
    out = np.zeros(max(M, 1), dtype=np.float64)
    _check(lib().orc_ring_replay(_ptr(bufs), _dtype_code(bufs), n, M, slice_elems, include, out), "ring_replay")
    return out[:M]


def stats(idx: np.ndarray, in_off: np.ndarray, M: int, P: int, hashed: bool = False, seed: int = 0):
    """Defs. 3, 4, 5 (Zen section 2.1) and Def. 8 (section 3.1) from exact
    counts.  Returns a dict of numpy arrays and floats."""
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    if idx.size == 0:
        idx = np.zeros(1, dtype=np.uint32)
    in_off = np.ascontiguousarray(in_off, dtype=np.uint64)
    n = in_off.size - 1
    arr = dict(
        nnz=np.zeros(n, np.uint64), inter=np.zeros(n * n, np.uint64), overlap=np.zeros(n * n, np.float64),
        contig_counts=np.zeros((n + 1) * P, np.uint64), skew_contig=np.zeros(n + 1, np.float64),
        class_size=np.zeros(P, np.uint64), hashed_counts=np.zeros((n + 1) * P, np.uint64),
        skew_hashed=np.zeros(n + 1, np.float64))
    o = _StatsOut()
    for k, a in arr.items():
        setattr(o, k, a.ctypes.data)
    _check(lib().orc_stats(idx, in_off, n, M, P, 1 if hashed else 0, seed, C.byref(o)), "stats")
    res = {k: v for k, v in arr.items()}
    res["inter"] = res["inter"].reshape(n, n)
    res["overlap"] = res["overlap"].reshape(n, n)
    res["contig_counts"] = res["contig_counts"].reshape(n + 1, P)
    res["hashed_counts"] = res["hashed_counts"].reshape(n + 1, P)
    for k in ("union_size", "sum_nnz", "max_nnz"):
        res[k] = int(getattr(o, k))
    for k in ("overlap_mean", "overlap_min", "overlap_max", "gamma_n", "push_imbalance", "pull_imbalance"):
        res[k] = float(getattr(o, k))
    return res

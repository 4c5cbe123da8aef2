"""Python binding of libsg (include/sg.h): sparse gradient synchronization
compute on one AMD MI355X (gfx950).

Argument marshalling only.  Every step runs in the HIP kernels of libsg.so;
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if libsg.so is missing or no GPU is present, the calls raise.

The functions carry the names of the C entry points.  Tensors must be CUDA
(ROCm) tensors on the current device; outputs and workspaces are allocated
with torch on the input's device; calls are queued on
``torch.cuda.current_stream()``.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsg.so")

SG_F32, SG_BF16 = 0, 1
SG_RESCALE_NONE, SG_RESCALE_DROP = 0, 1

_STATUS = {0: "SG_OK", -1: "SG_EINVAL", -2: "SG_ECAPACITY", -3: "SG_EUNSORTED", -4: "SG_EHIP",
           -5: "SG_EUNSUPPORTED", -6: "SG_ERANGE", -7: "SG_EDEVICE"}


class SgError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, _STATUS.get(status, "?"), status))


class StatsOut(C.Structure):
    _fields_ = [
        ("union_size", C.c_uint64), ("sum_nnz", C.c_uint64), ("max_nnz", C.c_uint64),
        ("nnz", C.c_void_p), ("inter", C.c_void_p), ("overlap", C.c_void_p),
        ("overlap_mean", C.c_double), ("overlap_min", C.c_double), ("overlap_max", C.c_double),
        ("gamma_n", C.c_double),
        ("contig_counts", C.c_void_p), ("skew_contig", C.c_void_p),
        ("class_size", C.c_void_p), ("hashed_counts", C.c_void_p), ("skew_hashed", C.c_void_p),
        ("push_imbalance", C.c_double), ("pull_imbalance", C.c_double),
    ]


_u32, _u64, _sz, _vp, _int, _dbl = C.c_uint32, C.c_uint64, C.c_size_t, C.c_void_p, C.c_int, C.c_double

# C signatures of include/sg.h
SIGNATURES = {
    "sg_strerror": (C.c_char_p, [_int]),
    "sg_device_error": (_int, [_vp]),
    "sg_probe_set": (_int, [_int, _vp, _vp]),
    "sg_validate_workspace_bytes": (_sz, []),
    "sg_validate_coo": (_int, [_vp, _vp, _u32, _u64, _u64, _vp, _sz, _vp]),
    "sg_topk_workspace_bytes": (_sz, [_u32, _u64, _u64, _int]),
    "sg_topk_to_coo": (_int, [_vp, _int, _u32, _u64, _u64, _vp, _vp, _vp, _sz, _vp]),
    "sg_hierarchical_hash_workspace_bytes": (_sz, [_u32, _u32, _u64, _u64]),
    "sg_hierarchical_hash": (_int, [_vp, _vp, _int, _u32, _vp, _u32, _u64, _u32, _u32, _u32, _u64, _u64, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _sz, _vp]),
    "sg_dgc_rank": (_u64, [_dbl, _u64]),
    "sg_dgc_workspace_bytes": (_sz, [_u32, _u64, _u64]),
    "sg_dgc_select": (_int, [_vp, _vp, _u32, _u64, _dbl, _u64, _vp, _vp, _u64, _vp, _vp, _vp, _sz, _vp]),
    "sg_partition_workspace_bytes": (_sz, [_u32, _u64, _u32]),
    "sg_hash_partition": (_int, [_vp, _vp, _int, _u32, _vp, _u32, _u64, _u32, _u32, _vp, _vp, _vp, _vp, _sz,
                                 _vp]),
    "sg_hash_partition_noalloc": (_int, [_vp, _vp, _int, _u32, _vp, _u32, _u64, _u32, _u32, _vp, _vp, _vp, _vp]),
    "sg_aggregate_workspace_bytes": (_sz, [_u32, _u32, _u64, _u64, _u32]),
    "sg_aggregate": (_int, [_vp, _vp, _int, _u32, _vp, _u32, _u32, _u64, _u64, _vp, _vp, _u64, _vp, _vp, _sz,
                            _vp]),
    "sg_classmap_bytes": (_sz, [_u64, _u32]),
    "sg_classmap_build": (_int, [_u64, _u32, _u32, _vp, _sz, _vp]),
    "sg_encode_max_words": (_u64, [_u64, _u32]),
    "sg_encode_workspace_bytes": (_sz, [_u64, _u32]),
    "sg_encode": (_int, [_vp, _vp, _u64, _u64, _u32, _vp, _sz, _vp, _u64, _vp, _vp, _sz, _vp]),
    "sg_skip_num_slices": (_u64, [_u32, _u64, _u64, _int]),
    "sg_skip_reduce_scatter": (_int, [_vp, _int, _u32, _u64, _u64, _dbl, _u64, _vp, _int, _vp, _vp, _vp]),
    "sg_skip_random_offset": (_u32, [_u32, _u64]),
    "sg_skip_reduce_k": (_int, [_vp, _int, _u32, _u64, _u64, _u32, _int, _u64, _int, _vp, _vp, _vp]),
    "sg_selective_reduce_scatter": (_int, [_vp, _int, _u32, _u64, _u32, _vp, _vp, _u64, _u64, _int, _vp, _vp]),
    "sg_dropout_reduce_scatter": (_int, [_vp, _int, _u32, _u64, _dbl, _u64, _int, _vp, _vp, _vp]),
    "sg_allgather": (_int, [_vp, _vp, _int, _u32, _u64, _vp, _vp, _vp]),
    "sg_stats_workspace_bytes": (_sz, [_u32, _u64, _u64, _u32]),
    "sg_decode_workspace_bytes": (_sz, [_u64, _u32]),
    "sg_decode": (_int, [_vp, _u64, _vp, _sz, _u64, _u32, _vp, _u64, _vp, _vp, _sz, _vp]),
    "sg_scatter_dense_workspace_bytes": (_sz, [_u64, _u32]),
    "sg_scatter_dense": (_int, [_vp, _vp, _u32, _vp, _u32, _u64, _u64, _vp, _vp, _sz, _vp]),
    "sg_format_sizes_workspace_bytes": (_sz, [_u64]),
    "sg_format_sizes": (_int, [_vp, _vp, _u64, _u64, _u32, _u32, _vp, _sz, _vp, _vp, _sz, _vp]),
    "sg_stats": (_int, [_vp, _vp, _u32, _u64, _u64, _u32, _vp, _sz, C.POINTER(StatsOut), _vp, _sz, _vp]),
    "sg_stats_block_bytes": (_sz, [_u32, _u32]),
    "sg_stats_async": (_int, [_vp, _vp, _u32, _u64, _u64, _u32, _vp, _sz, _vp, _sz, _vp, _sz, _vp]),
    "sg_stats_collect": (_int, [_vp, _u32, _u64, _u64, _u32, _int, C.POINTER(StatsOut)]),
}

_lib = None


def lib():
    """The loaded libsg.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsg.so is not built (run __graft_entry__.build() or "
                               "python -m sparse_gradient_synchronization_amd.build)")
        L = C.CDLL(LIB_PATH)
        missing = [name for name in SIGNATURES if not hasattr(L, name)]
        if missing:
            raise RuntimeError("libsg.so at %s does not export %s: it is stale, rebuild it "
                               "(python -m sparse_gradient_synchronization_amd.build)" % (LIB_PATH, ", ".join(missing)))
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(SIGNATURES)


def _check(rc: int, what: str):
    if rc != 0:
        raise SgError(rc, what)


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SG_F32
    if t.dtype == torch.bfloat16:
        return SG_BF16
    raise TypeError("values must be float32 or bfloat16, got %s" % t.dtype)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _contig(t):
    return None if t is None else t.contiguous()


# --------------------------------------------------------------------------
# the entry points
# --------------------------------------------------------------------------

def sg_topk_to_coo(dense: torch.Tensor, k: int, workspace: torch.Tensor | None = None):
    """dense [n, M] float32/bfloat16 -> (idx [n, k] int32 holding uint32 indices, val [n, k])."""
    _need_cuda(dense)
    dense = dense.contiguous()
    n, M = dense.shape
    dt = _dtype_code(dense)
    idx = torch.empty((n, k), dtype=torch.int32, device=dense.device)
    val = torch.empty((n, k), dtype=dense.dtype, device=dense.device)
    need = lib().sg_topk_workspace_bytes(n, M, k, dt)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, dense.device)
    _check(lib().sg_topk_to_coo(_p(dense), dt, n, M, k, _p(idx), _p(val), _p(ws), ws.numel(), _stream()),
           "sg_topk_to_coo")
    return idx, val


def sg_hash_partition(idx: torch.Tensor, val, in_off: torch.Tensor, P: int, seed: int,
                      workspace: torch.Tensor | None = None):
    """idx [total] int32, val None / [total] / [total, D], in_off [n+1] int64 ->
    (out_idx, out_val, part_off [n, P+1] int64)."""
    _need_cuda(idx, val, in_off)
    idx, val, in_off = _contig(idx), _contig(val), _contig(in_off)
    n = in_off.numel() - 1
    total = idx.numel()
    if val is None:
        D, dt, out_val = 0, SG_F32, None
    else:
        D = 1 if val.dim() == 1 else val.shape[1]
        dt = _dtype_code(val)
        out_val = torch.empty_like(val)
    out_idx = torch.empty_like(idx)
    part_off = torch.empty((n, P + 1), dtype=torch.int64, device=idx.device)
    need = lib().sg_partition_workspace_bytes(n, total, P)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, idx.device)
    _check(lib().sg_hash_partition(_p(idx), _p(val), dt, D, _p(in_off), n, total, P, seed, _p(out_idx),
                                   _p(out_val), _p(part_off), _p(ws), ws.numel(), _stream()),
           "sg_hash_partition")
    return out_idx, out_val, part_off


def sg_hash_partition_noalloc(idx: torch.Tensor, val, in_off: torch.Tensor, P: int, seed: int, out=None):
    """sg_hash_partition through the entry point that allocates nothing (its
    scratch is the library's fixed per-GPU array).  out: optional (out_idx,
    out_val, part_off) to write into; else they are allocated here, by the
    caller's side of the boundary."""
    _need_cuda(idx, val, in_off)
    idx, val, in_off = _contig(idx), _contig(val), _contig(in_off)
    n = in_off.numel() - 1
    total = idx.numel()
    if val is None:
        D, dt = 0, SG_F32
    else:
        D = 1 if val.dim() == 1 else val.shape[1]
        dt = _dtype_code(val)
    if out is None:
        out = (torch.empty_like(idx), None if val is None else torch.empty_like(val),
               torch.empty((n, P + 1), dtype=torch.int64, device=idx.device))
    out_idx, out_val, part_off = out
    _check(lib().sg_hash_partition_noalloc(_p(idx), _p(val), dt, D, _p(in_off), n, total, P, seed, _p(out_idx),
                                           _p(out_val), _p(part_off), _stream()), "sg_hash_partition_noalloc")
    return out_idx, out_val, part_off


def sg_aggregate(idx: torch.Tensor, val, part_off: torch.Tensor, M: int, workspace: torch.Tensor | None = None,
                 capacity: int | None = None):
    """Partitioned COO -> (agg_idx [capacity] int32, agg_val [capacity(, D)] float32, agg_off [P+1] int64).
    The valid length is agg_off[P] (read after synchronizing)."""
    _need_cuda(idx, val, part_off)
    idx, val, part_off = _contig(idx), _contig(val), _contig(part_off)
    n, P1 = part_off.shape
    P = P1 - 1
    total = idx.numel()
    cap = total if capacity is None else capacity
    if val is None:
        D, dt, agg_val = 0, SG_F32, None
    else:
        D = 1 if val.dim() == 1 else val.shape[1]
        dt = _dtype_code(val)
        agg_val = torch.empty((max(cap, 1),) if D == 1 else (max(cap, 1), D), dtype=torch.float32,
                              device=idx.device)
    agg_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=idx.device)
    agg_off = torch.empty(P + 1, dtype=torch.int64, device=idx.device)
    need = lib().sg_aggregate_workspace_bytes(n, P, M, total, D)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, idx.device)
    _check(lib().sg_aggregate(_p(idx), _p(val), dt, D, _p(part_off), n, P, M, total, _p(agg_idx), _p(agg_val),
                              cap, _p(agg_off), _p(ws), ws.numel(), _stream()), "sg_aggregate")
    return agg_idx, agg_val, agg_off


def sg_classmap_build(M: int, P: int, seed: int, device=None):
    """Class map of h0 over [0, M) (opaque uint8 tensor)."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    nbytes = lib().sg_classmap_bytes(M, P)
    cmap = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _check(lib().sg_classmap_build(M, P, seed, _p(cmap), cmap.numel(), _stream()), "sg_classmap_build")
    return cmap


def sg_encode(agg_idx: torch.Tensor, agg_off: torch.Tensor, M: int, cmap: torch.Tensor,
              workspace: torch.Tensor | None = None):
    """-> (bitmap [max_words] int32 holding uint32 words, word_off [P+1] int64)."""
    _need_cuda(agg_idx, agg_off, cmap)
    P = agg_off.numel() - 1
    words = lib().sg_encode_max_words(M, P)
    bitmap = torch.empty(max(words, 1), dtype=torch.int32, device=agg_idx.device)
    word_off = torch.empty(P + 1, dtype=torch.int64, device=agg_idx.device)
    need = lib().sg_encode_workspace_bytes(M, P)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, agg_idx.device)
    _check(lib().sg_encode(_p(agg_idx.contiguous()), _p(agg_off.contiguous()), agg_idx.numel(), M, P, _p(cmap),
                           cmap.numel(), _p(bitmap), words,
                           _p(word_off), _p(ws), ws.numel(), _stream()), "sg_encode")
    return bitmap, word_off


def sg_decode(bitmap: torch.Tensor, M: int, P: int, cmap: torch.Tensor, capacity: int | None = None,
              workspace: torch.Tensor | None = None):
    """Hash bitmap -> (indices [capacity] int32 holding uint32, off [P+1] int64);
    class p's indices are idx[off[p]:off[p+1]], ascending."""
    _need_cuda(bitmap, cmap)
    cap = int(capacity) if capacity is not None else int(M)
    out = torch.empty(max(cap, 1), dtype=torch.int32, device=bitmap.device)
    off = torch.empty(P + 1, dtype=torch.int64, device=bitmap.device)
    need = lib().sg_decode_workspace_bytes(M, P)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, bitmap.device)
    bm = bitmap.contiguous()
    _check(lib().sg_decode(_p(bm), bm.numel(), _p(cmap), cmap.numel(), M, P, _p(out), cap, _p(off), _p(ws),
                           ws.numel(), _stream()), "sg_decode")
    return out, off


def sg_scatter_dense(idx: torch.Tensor, val, off: torch.Tensor, M: int, D: int = 1, out: torch.Tensor | None = None):
    """Dense [M] (or [M, D]) fp32: zero except idx[off[0]:off[P]] <- val."""
    _need_cuda(idx, off)
    P = off.numel() - 1
    dense = out if out is not None else torch.empty((M, D) if D > 1 else (max(M, 1),), dtype=torch.float32,
                                                        device=idx.device)
    v = None if val is None else _contig(val.float())
    ws = _ws(lib().sg_scatter_dense_workspace_bytes(M, P), idx.device)
    _check(lib().sg_scatter_dense(_p(idx.contiguous()), _p(v), D, _p(off.contiguous()), P, idx.numel(), M,
                                  _p(dense), _p(ws), ws.numel(), _stream()), "sg_scatter_dense")
    return dense


FORMAT_NAMES = ("dense", "coo", "block", "bitmap", "hash_bitmap", "union", "nonempty_blocks")


def sg_format_sizes(agg_idx: torch.Tensor, agg_off: torch.Tensor, M: int, D: int, cmap: torch.Tensor) -> dict:
    """Bytes of the aggregate as dense, COO, 256-gradient blocks, contiguous
    bitmaps and hash bitmaps (and |I|, the non-empty blocks)."""
    _need_cuda(agg_idx, agg_off, cmap)
    P = agg_off.numel() - 1
    need = lib().sg_format_sizes_workspace_bytes(M)
    ws = _ws(need, agg_idx.device)
    out = (C.c_uint64 * 7)()
    _check(lib().sg_format_sizes(_p(agg_idx.contiguous()), _p(agg_off.contiguous()), agg_idx.numel(), M, P, D,
                                 _p(cmap), cmap.numel(), C.cast(out, C.c_void_p), _p(ws), ws.numel(), _stream()),
           "sg_format_sizes")
    return {k: int(v) for k, v in zip(FORMAT_NAMES, out)}


def sg_skip_num_slices(n: int, M: int, slice_bytes: int, dtype=torch.float32) -> int:
    return int(lib().sg_skip_num_slices(n, M, slice_bytes, SG_BF16 if dtype == torch.bfloat16 else SG_F32))


def sg_skip_reduce_scatter(bufs: torch.Tensor, slice_bytes: int, p_skip: float, seed: int, include=None,
                           mode: int = SG_RESCALE_DROP, want_count: bool = True, out=None):
    """bufs [n, M] float32/bfloat16 -> (out [M] float32, count [n, S] uint8 or None)."""
    _need_cuda(bufs, include)
    bufs = bufs.contiguous()
    n, M = bufs.shape
    dt = _dtype_code(bufs)
    S = lib().sg_skip_num_slices(n, M, slice_bytes, dt)
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=bufs.device)
    count = torch.empty((n, S), dtype=torch.uint8, device=bufs.device) if want_count else None
    if include is not None:
        include = include.contiguous().to(torch.uint8)
        if include.numel() != n * n * S:
            raise ValueError("include must have n*n*S = %d entries" % (n * n * S))
    _check(lib().sg_skip_reduce_scatter(_p(bufs), dt, n, M, slice_bytes, float(p_skip), seed & (2**64 - 1),
                                        _p(include), mode, _p(out), _p(count), _stream()),
           "sg_skip_reduce_scatter")
    return out, count


def sg_skip_random_offset(n: int, seed: int) -> int:
    return int(lib().sg_skip_random_offset(n, seed & (2**64 - 1)))


def sg_skip_reduce_k(bufs: torch.Tensor, slice_bytes: int, k: int, random_offset: bool = False, seed: int = 0,
                     mode: int = SG_RESCALE_DROP, want_count: bool = True, out=None):
    """SkipReduce(k), static or with a random offset: bufs [n, M] ->
    (out [M] float32, count [n, S] uint8 or None)."""
    _need_cuda(bufs)
    bufs = bufs.contiguous()
    n, M = bufs.shape
    dt = _dtype_code(bufs)
    S = lib().sg_skip_num_slices(n, M, slice_bytes, dt)
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=bufs.device)
    count = torch.empty((n, S), dtype=torch.uint8, device=bufs.device) if want_count else None
    _check(lib().sg_skip_reduce_k(_p(bufs), dt, n, M, slice_bytes, k, 1 if random_offset else 0,
                                  seed & (2**64 - 1), mode, _p(out), _p(count), _stream()), "sg_skip_reduce_k")
    return out, count


def sg_selective_reduce_scatter(bufs: torch.Tensor, bucket_off, p_skip, slice_bytes: int, seed: int,
                                mode: int = SG_RESCALE_DROP, out=None):
    """Selective SkipReduce: bucket_off (nb+1 offsets) and p_skip (nb rates)
    are host sequences.  Returns out [M] float32 (elements outside every
    bucket are zero when out is allocated here)."""
    import numpy as np
    _need_cuda(bufs)
    bufs = bufs.contiguous()
    n, M = bufs.shape
    dt = _dtype_code(bufs)
    bo = np.ascontiguousarray(bucket_off, dtype=np.uint64)
    pr = np.ascontiguousarray(p_skip, dtype=np.float64)
    if bo.size != pr.size + 1:
        raise ValueError("bucket_off must have one more entry than p_skip")
    if out is None:
        out = torch.zeros(M, dtype=torch.float32, device=bufs.device)
    _check(lib().sg_selective_reduce_scatter(_p(bufs), dt, n, M, pr.size, C.c_void_p(bo.ctypes.data),
                                             C.c_void_p(pr.ctypes.data), slice_bytes, seed & (2**64 - 1), mode,
                                             _p(out), _stream()), "sg_selective_reduce_scatter")
    return out


def sg_dropout_reduce_scatter(bufs: torch.Tensor, p_skip: float, seed: int, mode: int = SG_RESCALE_DROP,
                              want_count: bool = True, out=None):
    """AllReduce_Dropout: bufs [n, M] -> (out [M] float32, count [M] uint8 or None)."""
    _need_cuda(bufs)
    bufs = bufs.contiguous()
    n, M = bufs.shape
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=bufs.device)
    count = torch.empty(M, dtype=torch.uint8, device=bufs.device) if want_count else None
    _check(lib().sg_dropout_reduce_scatter(_p(bufs), _dtype_code(bufs), n, M, float(p_skip), seed & (2**64 - 1),
                                           mode, _p(out), _p(count), _stream()), "sg_dropout_reduce_scatter")
    return out, count


def sg_allgather(reduced: torch.Tensor, bufs: torch.Tensor, ag_include=None, out=None):
    """reduced [M] float32, bufs [n, M] -> out [n, M] float32, every rank's
    tensor after the all-gather phase; ag_include [n, n] uint8 or None."""
    _need_cuda(reduced, bufs, ag_include)
    reduced, bufs = reduced.contiguous(), bufs.contiguous()
    n, M = bufs.shape
    if reduced.dtype != torch.float32 or reduced.numel() != M:
        raise ValueError("reduced must be float32 [M]")
    if ag_include is not None:
        ag_include = ag_include.contiguous().to(torch.uint8)
        if ag_include.numel() != n * n:
            raise ValueError("ag_include must have n*n entries")
    if out is None:
        out = torch.empty((n, M), dtype=torch.float32, device=bufs.device)
    _check(lib().sg_allgather(_p(reduced), _p(bufs), _dtype_code(bufs), n, M, _p(ag_include), _p(out), _stream()),
           "sg_allgather")
    return out


def sg_hierarchical_hash(idx: torch.Tensor, val, in_off: torch.Tensor, P: int, seed: int, k: int, r1: int, r2: int,
                         want_slots: bool = False, workspace: torch.Tensor | None = None):
    """Algorithm 1 of the Zen page (hierarchical hashing).  Returns out_idx,
    out_val (or None), part_off [n, P+1] int64, slot_of (or None) and
    counts [n, 2] int64 (serial writes, lost entries)."""
    _need_cuda(idx, in_off, val)
    idx, in_off = idx.contiguous(), in_off.contiguous()
    n = in_off.numel() - 1
    total = idx.numel()
    dev = idx.device
    D = 0 if val is None else (1 if val.dim() == 1 else val.shape[1])
    dt = SG_F32 if val is None else _dtype_code(val)
    if val is not None:
        val = val.contiguous()
    out_idx = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
    out_val = None if val is None else torch.empty((max(total, 1),) + tuple(val.shape[1:]), dtype=val.dtype,
                                                   device=dev)
    part_off = torch.empty((n, P + 1), dtype=torch.int64, device=dev)
    slot_of = torch.empty(max(total, 1), dtype=torch.int32, device=dev) if want_slots else None
    counts = torch.empty((n, 2), dtype=torch.int64, device=dev)
    need = lib().sg_hierarchical_hash_workspace_bytes(n, P, r1, r2)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, dev)
    _check(lib().sg_hierarchical_hash(_p(idx), _p(val), dt, D, _p(in_off), n, total, P, seed, k, r1, r2, _p(out_idx),
                                      _p(out_val), _p(part_off), _p(slot_of), _p(counts), _p(ws), ws.numel(),
                                      _stream()), "sg_hierarchical_hash")
    return (out_idx[:total], None if out_val is None else out_val[:total], part_off,
            None if slot_of is None else slot_of[:total], counts)


def sg_dgc_select(grad: torch.Tensor, resid: torch.Tensor, density: float, S: int, cap: int,
                  workspace: torch.Tensor | None = None):
    """One DGC iteration (sampled global threshold, residuals) for grad and
    resid [n, M] float32; resid is updated in place.  Returns (idx [n, cap]
    int32 (uint32 bits), val [n, cap] float32, count [n] int64, thr_key
    [1] int32)."""
    _need_cuda(grad, resid)
    if grad.dtype != torch.float32 or resid.dtype != torch.float32 or grad.shape != resid.shape:
        raise ValueError("grad and resid must be float32 tensors of one shape [n, M]")
    if not resid.is_contiguous():
        raise ValueError("resid must be contiguous (it is updated in place)")
    grad = grad.contiguous()
    n, M = grad.shape
    dev = grad.device
    idx = torch.empty((n, max(cap, 1)), dtype=torch.int32, device=dev)
    val = torch.empty((n, max(cap, 1)), dtype=torch.float32, device=dev)
    cnt = torch.empty(n, dtype=torch.int64, device=dev)
    thr = torch.empty(1, dtype=torch.int32, device=dev)
    need = lib().sg_dgc_workspace_bytes(n, M, S)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, dev)
    _check(lib().sg_dgc_select(_p(grad), _p(resid), n, M, float(density), S, _p(idx), _p(val), cap, _p(cnt),
                               _p(thr), _p(ws), ws.numel(), _stream()), "sg_dgc_select")
    return idx[:, :cap], val[:, :cap], cnt, thr


def _stats_out(n, P):
    import numpy as np
    arr = dict(
        nnz=np.zeros(n, np.uint64), inter=np.zeros(n * n, np.uint64), overlap=np.zeros(n * n, np.float64),
        contig_counts=np.zeros((n + 1) * P, np.uint64), skew_contig=np.zeros(n + 1, np.float64),
        class_size=np.zeros(P, np.uint64), hashed_counts=np.zeros((n + 1) * P, np.uint64),
        skew_hashed=np.zeros(n + 1, np.float64))
    o = StatsOut()
    for k, a in arr.items():
        setattr(o, k, a.ctypes.data)
    return arr, o


def sg_stats(idx: torch.Tensor, in_off: torch.Tensor, M: int, P: int, cmap=None,
             workspace: torch.Tensor | None = None):
    """Defs. 3-5 and 8 of the Zen page from exact counts.  Returns a dict."""
    _need_cuda(idx, in_off, cmap)
    idx, in_off = idx.contiguous(), in_off.contiguous()
    n = in_off.numel() - 1
    total = idx.numel()
    arr, o = _stats_out(n, P)
    need = lib().sg_stats_workspace_bytes(n, M, total, P)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, idx.device)
    _check(lib().sg_stats(_p(idx), _p(in_off), n, M, total, P, _p(cmap), 0 if cmap is None else cmap.numel(),
                          C.byref(o), _p(ws), ws.numel(),
                          _stream()), "sg_stats")
    return _stats_result(arr, o, n, P)


def sg_stats_async(idx: torch.Tensor, in_off: torch.Tensor, M: int, P: int, cmap=None,
                   workspace: torch.Tensor | None = None, block: torch.Tensor | None = None):
    """Queues the statistics passes and the copy of the raw counts into a
    pinned host block; returns (block, args) for sg_stats_collect, to be
    called after the current stream has passed this point."""
    _need_cuda(idx, in_off, cmap)
    idx, in_off = idx.contiguous(), in_off.contiguous()
    n = in_off.numel() - 1
    total = idx.numel()
    nb = lib().sg_stats_block_bytes(n, P)
    if block is None or block.numel() < nb:
        block = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    need = lib().sg_stats_workspace_bytes(n, M, total, P)
    ws = workspace if workspace is not None and workspace.numel() >= need else _ws(need, idx.device)
    _check(lib().sg_stats_async(_p(idx), _p(in_off), n, M, total, P, _p(cmap), 0 if cmap is None else cmap.numel(),
                                _p(block), block.numel(), _p(ws), ws.numel(), _stream()), "sg_stats_async")
    return block, (n, M, total, P, 0 if cmap is None else 1)


def sg_stats_collect(block: torch.Tensor, args) -> dict:
    """The statistics from a block filled by sg_stats_async (host only)."""
    n, M, total, P, hashed = args
    arr, o = _stats_out(n, P)
    _check(lib().sg_stats_collect(_p(block), n, M, total, P, hashed, C.byref(o)), "sg_stats_collect")
    return _stats_result(arr, o, n, P)


def _stats_result(arr, o, n, P):
    res = dict(arr)
    res["inter"] = res["inter"].reshape(n, n)
    res["overlap"] = res["overlap"].reshape(n, n)
    res["contig_counts"] = res["contig_counts"].reshape(n + 1, P)
    res["hashed_counts"] = res["hashed_counts"].reshape(n + 1, P)
    for k in ("union_size", "sum_nnz", "max_nnz"):
        res[k] = int(getattr(o, k))
    for k in ("overlap_mean", "overlap_min", "overlap_max", "gamma_n", "push_imbalance", "pull_imbalance"):
        res[k] = float(getattr(o, k))
    return res


def sg_validate_coo(idx: torch.Tensor, in_off: torch.Tensor, M: int) -> int:
    """Returns the status code (0 = valid)."""
    _need_cuda(idx, in_off)
    ws = _ws(lib().sg_validate_workspace_bytes(), idx.device)
    n = in_off.numel() - 1
    return int(lib().sg_validate_coo(_p(idx.contiguous()), _p(in_off.contiguous()), n, M, idx.numel(), _p(ws),
                                     ws.numel(), _stream()))


def sg_device_error() -> int:
    return int(lib().sg_device_error(_stream()))

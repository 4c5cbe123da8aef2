"""GPU parity of whole chains at the workloads' full sizes: every stage's
output compared with the oracle's, the GPU chain feeding each GPU stage with
the previous GPU stage's output and the oracle chain feeding the oracle.

- DGC-style workload (n=8 dense 4096 x 11008 fp32 gradients, top 5%, P=8):
  top-k -> hash partition -> union-sum -> hash-bitmap encode -> decode, plus
  the statistics of the top-k sets (Zen sections 3.1, 3.2, 3.3.2 and 2.1).
- workload 1 (n=4, M=2^20, 1% Zipf nonzeros, P=4): the same chain from the
  dense tensors.
- workload 2 (embedding rows 1,000,000 x 64, n=8, P=8): partition, union-sum of
  64-wide rows, encode and statistics.

Indices, offsets, bitmaps and statistics are bit-exact; fp32 sums are within
|d| <= 1e-6 * sum|x| + 1e-30 of the oracle's float64 sums.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import assert_sum_close, host_bits, host_u32, host_u64, need_gpu, to_dev_u32, to_dev_u64, to_dev_vals

pytestmark = pytest.mark.gpu

STAT_INT = ("nnz", "inter", "contig_counts", "class_size", "hashed_counts")
STAT_FLOAT = ("overlap", "skew_contig", "skew_hashed")
STAT_SCALAR = ("union_size", "sum_nnz", "max_nnz", "overlap_mean", "overlap_min", "overlap_max", "gamma_n",
               "push_imbalance", "pull_imbalance")


def _stats_equal(got, ref):
    for k in STAT_INT + STAT_FLOAT:
        assert np.array_equal(np.asarray(got[k]), np.asarray(ref[k])), k
    for k in STAT_SCALAR:
        assert got[k] == ref[k], (k, got[k], ref[k])


def _sparse_chain(g_idx, g_val, g_in_off, r_idx, r_val, in_off, M, P, seed, D=1):
    """Partition -> aggregate -> encode -> decode on both sides, compared stage
    by stage; statistics of the input sets.  g_*: device tensors (the GPU
    chain), r_*: host arrays (the oracle chain).  Returns the union size."""
    # A2: stable grouping by h0
    pi, pv, po = sg.sg_hash_partition(g_idx, g_val, g_in_off, P, seed)
    roi, rov, rpo = oracle.hash_partition(r_idx, r_val, in_off, P, seed)
    torch.cuda.synchronize()
    assert np.array_equal(host_u64(po), rpo.reshape(-1).reshape(rpo.shape)), "part_off"
    assert np.array_equal(host_u32(pi), roi), "partitioned indices"
    assert np.array_equal(host_bits(pv).reshape(-1), rov.reshape(-1).view(np.uint32)), "partitioned values"
    # A3: union-sum per partition
    ai, av, ao = sg.sg_aggregate(pi, pv, po, M)
    rai, rav, raa, rao = oracle.aggregate(roi, rov, rpo, M)
    torch.cuda.synchronize()
    gao = host_u64(ao)
    assert np.array_equal(gao, rao), "agg_off"
    u = int(rao[-1])
    assert np.array_equal(host_u32(ai)[:u], rai), "union indices"
    gv = av.cpu().numpy()[:u]
    assert_sum_close(gv.reshape(-1), rav.reshape(-1), raa.reshape(-1), 1e-6, "union sums")
    # A4: hash bitmap; then the Pull side decodes it back to the union
    cmap = sg.sg_classmap_build(M, P, seed)
    bm, wo = sg.sg_encode(ai, ao, M, cmap)
    rb, rwo = oracle.encode(rai, rao, M, seed)
    torch.cuda.synchronize()
    assert np.array_equal(host_u64(wo), rwo), "word_off"
    assert np.array_equal(host_u32(bm)[: int(rwo[-1])], rb), "bitmap"
    di, do = sg.sg_decode(bm, M, P, cmap, capacity=max(u, 1))
    torch.cuda.synchronize()
    assert np.array_equal(host_u64(do), rao), "decoded offsets"
    assert np.array_equal(host_u32(di)[:u], rai), "decoded indices"
    # A6: Defs. 3-5 and 8 of the input index sets, hashed skew included
    got = sg.sg_stats(g_idx, g_in_off, M, P, cmap=cmap)
    ref = oracle.stats(r_idx, in_off, M, P, hashed=True, seed=seed)
    _stats_equal(got, ref)
    assert got["union_size"] == u  # the union the aggregate built
    assert sg.sg_device_error() == 0
    return u


def test_chain_dgc_top5_full():
    need_gpu()
    c = gen.config3()
    n, M, k, P, seed = c["n"], c["M"], c["k"], c["P"], c["seed"]
    # A1: per-worker exact top-k
    gi, gv = sg.sg_topk_to_coo(to_dev_vals(c["dense"]), k)
    ri, rv = oracle.topk_to_coo(c["dense"], k)
    torch.cuda.synchronize()
    assert np.array_equal(host_u32(gi), ri), "top-k indices"
    assert np.array_equal(host_bits(gv), rv.view(np.uint32)), "top-k values"
    in_off = np.arange(n + 1, dtype=np.uint64) * np.uint64(k)
    u = _sparse_chain(gi.reshape(-1), gv.reshape(-1), to_dev_u64(in_off), ri.reshape(-1), rv.reshape(-1), in_off,
                      M, P, seed)
    # the correlated workers overlap: the union is far below n*k
    assert n * k // 8 < u < n * k // 2


def test_chain_config1_full():
    need_gpu()
    c = gen.config1()
    n, M, k, P, seed = c["n"], c["M"], c["k"], c["P"], c["seed"]
    gi, gv = sg.sg_topk_to_coo(to_dev_vals(c["dense"]), k)
    ri, rv = oracle.topk_to_coo(c["dense"], k)
    torch.cuda.synchronize()
    assert np.array_equal(host_u32(gi), ri)
    assert np.array_equal(host_bits(gv), rv.view(np.uint32))
    in_off = np.arange(n + 1, dtype=np.uint64) * np.uint64(k)
    _sparse_chain(gi.reshape(-1), gv.reshape(-1), to_dev_u64(in_off), ri.reshape(-1), rv.reshape(-1), in_off, M, P,
                  seed)


def test_chain_config2_full():
    need_gpu()
    c = gen.config2()
    M, P, seed = c["M"], c["P"], c["seed"]
    _sparse_chain(to_dev_u32(c["idx"]), to_dev_vals(c["val"]), to_dev_u64(c["in_off"]), c["idx"], c["val"],
                  c["in_off"], M, P, seed)

"""GPU parity of sg_stats against the oracle: every count bit-exact and every
ratio (Defs. 3, 4, 5 and 8 of the Zen page) equal as a double."""
import numpy as np
import pytest

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import need_gpu, to_dev_u32, to_dev_u64

pytestmark = pytest.mark.gpu

INT_KEYS = ("nnz", "inter", "contig_counts")
HASH_INT_KEYS = ("class_size", "hashed_counts")
FLOAT_KEYS = ("overlap", "skew_contig")
SCALARS = ("union_size", "sum_nnz", "max_nnz", "overlap_mean", "overlap_min", "overlap_max", "gamma_n")


def _check(idx, in_off, M, P, seed=None):
    need_gpu()
    cmap = None if seed is None else sg.sg_classmap_build(M, P, seed)
    got = sg.sg_stats(to_dev_u32(idx if idx.size else np.zeros(1, np.uint32))[: idx.size], to_dev_u64(in_off), M, P,
                      cmap=cmap)
    ref = oracle.stats(idx, in_off, M, P, hashed=seed is not None, seed=seed or 0)
    for k in INT_KEYS + FLOAT_KEYS:
        assert np.array_equal(got[k], ref[k]), k
    for k in SCALARS:
        assert got[k] == ref[k], (k, got[k], ref[k])
    if seed is not None:
        for k in HASH_INT_KEYS:
            assert np.array_equal(got[k], ref[k]), k
        assert np.array_equal(got["skew_hashed"], ref["skew_hashed"])
        assert got["push_imbalance"] == ref["push_imbalance"]
        assert got["pull_imbalance"] == ref["pull_imbalance"]
    assert sg.sg_device_error() == 0
    return got


# (n, P) spans the counting passes: the dense pass (n <= 16, P <= 16, lists
# not too sparse for M: 3000 entries per worker over 120000 keys are), the
# merge engine (more workers, or more classes with a class map) and the
# window pass (n <= 16 and more parts without a class map)
@pytest.mark.parametrize("n,P", [(1, 1), (2, 2), (4, 4), (7, 3), (16, 16), (64, 8), (17, 5), (5, 200), (9, 17)])
def test_stats_zipf(n, P):
    idx, in_off, _ = gen.coo_zipf(500 + n, n, 120000, 3000, 1.1)
    _check(idx, in_off, 120000, P, seed=13)
    _check(idx, in_off, 120000, P)


# lists too sparse for the dense pass (3000 entries per worker over 2^24
# keys): the window pass (n <= 16, P <= 16)
@pytest.mark.parametrize("n,P", [(3, 4), (8, 8), (16, 16), (11, 1)])
def test_stats_window_sparse(n, P):
    M = 1 << 24
    idx, in_off, _ = gen.coo_zipf(700 + n, n, M, 3000, 1.1)
    _check(idx, in_off, M, P, seed=29)
    _check(idx, in_off, M, P)


# the dense pass at its edges: M not a multiple of 32 with the last key
# present, runs of consecutive keys longer than a 32-key word and than a
# wave, an empty worker between others, part boundaries inside words, n and
# P at and below the compile-time bounds
@pytest.mark.parametrize("n,P", [(16, 16), (9, 7), (2, 16)])
def test_stats_dense_edges(n, P):
    M = 100003
    rng = np.random.default_rng(40 + n)
    lists = []
    for w in range(n):
        if w == n // 2 and n > 2:
            lists.append(np.zeros(0, np.uint32))
            continue
        runs = [np.arange(s, min(s + ln, M), dtype=np.uint32)
                for s, ln in zip(rng.integers(0, M, 40), rng.integers(1, 200, 40))]
        runs.append(np.array([0, M - 1], np.uint32))
        lists.append(np.unique(np.concatenate(runs + [rng.integers(0, M, 2000).astype(np.uint32)])))
    idx, in_off, _ = gen.coo_from_lists(lists, [a.astype(np.float32) for a in lists])
    _check(idx, in_off, M, P, seed=5)
    _check(idx, in_off, M, P)


def test_stats_identical_disjoint_empty():
    a = np.arange(0, 5000, 2, dtype=np.uint32)
    b = np.arange(1, 5000, 2, dtype=np.uint32)
    idx, in_off, _ = gen.coo_from_lists([a, a, b, np.zeros(0, np.uint32)], [a, a, b, a[:0]])
    g = _check(idx, in_off, 5000, 4, seed=2)
    assert g["inter"][0, 1] == a.size and g["inter"][0, 2] == 0


def test_stats_config1_full():
    c = gen.config1()
    _check(c["idx"], c["in_off"], c["M"], c["P"], seed=c["seed"])


def test_stats_config4_full():
    c = gen.config4()
    g = _check(c["idx"], c["in_off"], c["M"], c["P"], seed=c["seed"])
    # skewed before hashing, balanced after (Zen section 2.1 C3 and Theorem 2)
    assert g["skew_contig"][:16].min() > 4.5 and g["skew_hashed"].max() < 1.05


@pytest.mark.parametrize("n,P", [(4, 4), (16, 16), (64, 8), (9, 17)])
def test_stats_async_matches_blocking(n, P):
    """sg_stats_async + sg_stats_collect give what sg_stats gives, twice in a
    row into the same block and workspace, with and without a class map."""
    need_gpu()
    import torch
    idx, in_off, _ = gen.coo_zipf(900 + n, n, 120000, 3000, 1.1)
    d_idx, d_off = to_dev_u32(idx), to_dev_u64(in_off)
    for seed in (None, 13):
        cmap = None if seed is None else sg.sg_classmap_build(120000, P, seed)
        ref = sg.sg_stats(d_idx, d_off, 120000, P, cmap=cmap)
        block = None
        for _ in range(2):
            block, args = sg.sg_stats_async(d_idx, d_off, 120000, P, cmap=cmap, block=block)
            torch.cuda.synchronize()
            got = sg.sg_stats_collect(block, args)
            for k, v in ref.items():
                assert np.array_equal(np.asarray(got[k]), np.asarray(v)), k

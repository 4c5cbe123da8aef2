"""Host evaluation of the statistics (sg_stats_collect, no GPU): a block of
raw counts assembled from the oracle's exact counts gives back the oracle's
ratios (Zen page, section 2.1 Defs. 3-5) as the same doubles."""
import numpy as np
import pytest

import gen
import oracle
import sparse_gradient_synchronization_amd as sg


def _block(ref, in_off, n, P):
    # layout of the block: pair counts (a <= b, row-major), union, union per
    # contiguous part, union per hash class, per-worker contiguous counts,
    # per-worker class counts, worker offsets, class sizes, map header
    pairs = [ref["inter"][a, b] for a in range(n) for b in range(a, n)]
    words = (pairs + [ref["union_size"]] + list(ref["contig_counts"][n]) + [0] * P
             + list(ref["contig_counts"][:n].reshape(-1)) + [0] * (n * P) + list(in_off) + [0] * P + [0] * 4)
    blk = np.array(words, dtype=np.uint64)
    assert blk.nbytes == sg.lib().sg_stats_block_bytes(n, P)
    return blk


@pytest.mark.parametrize("n,P", [(1, 1), (3, 2), (7, 5), (16, 16), (33, 7)])
def test_collect_matches_oracle(n, P):
    import torch
    M = 50000
    idx, in_off, _ = gen.coo_zipf(70 + n, n, M, 900, 1.2)
    ref = oracle.stats(idx, in_off, M, P)
    blk = torch.from_numpy(_block(ref, in_off, n, P).view(np.uint8))
    got = sg.sg_stats_collect(blk, (n, M, int(in_off[-1]), P, 0))
    for k in ("nnz", "inter", "contig_counts", "overlap", "skew_contig"):
        assert np.array_equal(got[k], ref[k]), k
    for k in ("union_size", "sum_nnz", "max_nnz", "overlap_mean", "overlap_min", "overlap_max", "gamma_n"):
        assert got[k] == ref[k], k


def test_collect_rejects_bad_arguments():
    import torch
    L = sg.lib()
    assert L.sg_stats_block_bytes(0, 4) == 0 and L.sg_stats_block_bytes(4, 0) == 0
    assert L.sg_stats_block_bytes(65, 4) == 0 and L.sg_stats_block_bytes(4, 257) == 0
    blk = torch.zeros(L.sg_stats_block_bytes(4, 4), dtype=torch.uint8)
    with pytest.raises(RuntimeError):
        sg.sg_stats_collect(blk, (0, 100, 0, 4, 0))
    with pytest.raises(RuntimeError):
        sg.sg_stats_collect(blk, (4, 0, 0, 4, 0))
    # a class map header that does not match (M, P) is refused
    with pytest.raises(RuntimeError):
        sg.sg_stats_collect(blk, (4, 100, 0, 4, 1))

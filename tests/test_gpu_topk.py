"""GPU parity of sg_topk_to_coo against the oracle: bit-exact indices and
values (integer work on bit patterns), including ties, signed zeros, bf16,
ragged tails, a band the sample misses, and the full workloads 1 and 3."""
import numpy as np
import pytest

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import host_bits, host_u32, need_gpu, to_dev_vals

pytestmark = pytest.mark.gpu


def _check(dense, k, bf16=False):
    need_gpu()
    idx, val = sg.sg_topk_to_coo(to_dev_vals(dense, bf16), k)
    ri, rv = oracle.topk_to_coo(dense, k)
    gi = host_u32(idx)
    assert gi.shape == ri.shape
    bad = np.flatnonzero((gi != ri).any(1)) if k else []
    assert len(bad) == 0, "worker %s differs" % bad
    assert np.array_equal(host_bits(val).view(np.uint8), rv.view(np.uint8))
    assert sg.sg_device_error() == 0


@pytest.mark.parametrize("M", [1, 5, 100, 1024, 2048, 4096, 4097, 5000, 12288, 16383, 16384, 16385, 100003, 1 << 18])
def test_topk_shapes(M):
    dense = gen.dense_normal(200 + M % 97, 3, M)
    for k in sorted({1, max(1, M // 20), M // 2, M - 1, M} - {0}):
        _check(dense, k)


@pytest.mark.parametrize("bf16", [False, True])
def test_topk_ties_and_zeros(bf16):
    rng = np.random.default_rng(4)
    M = 50000
    vals = rng.integers(-4, 5, size=(4, M)).astype(np.float32)
    vals[1] = 1.0  # all equal
    vals[2, ::3] = -0.0
    dense = gen.to_bf16(vals) if bf16 else vals
    for k in (1, 7, 1000, 12345, M):
        _check(dense, k, bf16)


def test_topk_bf16_normal():
    dense = gen.to_bf16(gen.dense_normal(7, 4, 300000))
    _check(dense, 15000, True)


def test_topk_sample_miss_forces_refilter():
    M = 1 << 20
    dense = gen.dense_normal(9, 2, M)
    S = 16384
    pos = ((2 * np.arange(S) + 1) * M) // (2 * S)
    dense[:, pos] = 1e-3  # every sampled element is tiny
    _check(dense, M // 20)


def test_topk_sparse_k_equals_nnz_config1():
    c = gen.config1()
    _check(c["dense"], c["k"])
    # the result is the nonzero extraction
    need_gpu()
    idx, _ = sg.sg_topk_to_coo(to_dev_vals(c["dense"]), c["k"])
    gi = host_u32(idx)
    for w in range(c["n"]):
        b, e = int(c["in_off"][w]), int(c["in_off"][w + 1])
        assert np.array_equal(gi[w], c["idx"][b:e])


def test_topk_config3_full():
    c = gen.config3()
    _check(c["dense"], c["k"])

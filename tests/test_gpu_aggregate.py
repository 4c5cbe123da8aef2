"""GPU parity of sg_aggregate against the oracle: bit-exact union indices and
partition offsets; fp32 sums within |d| <= 1e-6 sum|x| + 1e-30 (1e-3 for bf16
inputs) of the oracle's float64 sums."""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import assert_sum_close, host_u32, host_u64, need_gpu, to_dev_u32, to_dev_u64, to_dev_vals

pytestmark = pytest.mark.gpu


def _check(idx, in_off, val, M, P, seed, bf16=False):
    need_gpu()
    oi, ov, po = oracle.hash_partition(idx, val, in_off, P, seed)
    d_val = None if val is None else to_dev_vals(ov, bf16)
    ai, av, ao = sg.sg_aggregate(to_dev_u32(oi), d_val, to_dev_u64(po), M)
    torch.cuda.synchronize()
    rvals = None if val is None else (gen.bf16_to_f32(ov) if bf16 else ov)
    ri, rv, ra, rao = oracle.aggregate(oi, rvals, po, M)
    gao = host_u64(ao)
    assert np.array_equal(gao, rao)
    u = int(rao[-1])
    assert np.array_equal(host_u32(ai)[:u], ri)
    if val is not None:
        gv = av.cpu().numpy()[:u]
        assert_sum_close(gv, rv, ra, 1e-3 if bf16 else 1e-6, "aggregate")
    assert sg.sg_device_error() == 0


@pytest.mark.parametrize("n,P", [(1, 1), (2, 3), (4, 4), (8, 8), (16, 16), (5, 256), (64, 7)])
def test_aggregate_zipf(n, P):
    idx, in_off, val = gen.coo_zipf(300 + n, n, 200000, 6000, 1.1)
    _check(idx, in_off, val, 200000, P, 9)


@pytest.mark.parametrize("D", [0, 3, 64])
def test_aggregate_rows(D):
    idx, in_off, val = gen.coo_zipf(310 + D, 6, 40000, 2500, 1.05, D=max(D, 1), sigma=0.01)
    _check(idx, in_off, None if D == 0 else val, 40000, 8, 4)


def test_aggregate_bf16():
    idx, in_off, val = gen.coo_zipf(320, 8, 100000, 5000, 1.1)
    _check(idx, in_off, gen.to_bf16(val), 100000, 8, 3, bf16=True)


@pytest.mark.parametrize("D", [2, 3, 64])
def test_aggregate_rows_bf16(D):
    idx, in_off, val = gen.coo_zipf(330 + D, 5, 40000, 2000, 1.05, D=D)
    _check(idx, in_off, gen.to_bf16(val), 40000, 4, 6, bf16=True)


def test_aggregate_rows_in_windows():
    # rows whose buckets are denser than a window: their contributor lists
    # are recorded window by window
    n, M, D = 16, 1 << 16, 5
    lists = [np.arange(0, 3000, dtype=np.uint32) for _ in range(n)]
    vals = [gen.normal(500 + w, 3000 * D).reshape(3000, D) for w in range(n)]
    idx, in_off, val = gen.coo_from_lists(lists, vals)
    _check(idx, in_off, val, M, 1, 1)
    _check(idx, in_off, val, M, 3, 1)


def test_aggregate_identical_and_oversized_buckets():
    # every worker holds the same dense block of keys: one bucket far larger
    # than an LDS tile, consumed in windows
    n, M = 16, 1 << 20
    lists = [np.arange(0, 3000, dtype=np.uint32) for _ in range(n)]
    vals = [gen.normal(400 + w, 3000) for w in range(n)]
    idx, in_off, val = gen.coo_from_lists(lists, vals)
    _check(idx, in_off, val, M, 1, 1)
    _check(idx, in_off, val, M, 4, 1)


def test_aggregate_empty_workers_and_partitions():
    lists = [np.array([], np.uint32), np.array([3, 5, 100], np.uint32), np.array([], np.uint32),
             np.array([5, 99999], np.uint32)]
    vals = [gen.normal(1, len(l)) for l in lists]
    idx, in_off, val = gen.coo_from_lists(lists, vals)
    _check(idx, in_off, val, 100000, 16, 2)
    _check(np.zeros(0, np.uint32), np.zeros(3, np.uint64), np.zeros(0, np.float32), 1000, 4, 2)


def test_aggregate_config1_full():
    c = gen.config1()
    _check(c["idx"], c["in_off"], c["val"], c["M"], c["P"], c["seed"])


def test_aggregate_config2_full():
    c = gen.config2()
    _check(c["idx"], c["in_off"], c["val"], c["M"], c["P"], c["seed"])


def test_aggregate_config4_full():
    c = gen.config4()
    _check(c["idx"], c["in_off"], c["val"], c["M"], c["P"], c["seed"])

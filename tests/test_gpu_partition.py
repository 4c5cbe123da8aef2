"""GPU parity of sg_hash_partition against the oracle: bit-exact indices,
values and offsets."""
import numpy as np
import pytest

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import host_bits, host_u32, host_u64, need_gpu, to_dev_u32, to_dev_u64, to_dev_vals

pytestmark = pytest.mark.gpu


def _check(idx, in_off, val, P, seed, bf16=False):
    need_gpu()
    d_val = None if val is None else to_dev_vals(val, bf16)
    oi, ov, po = sg.sg_hash_partition(to_dev_u32(idx), d_val, to_dev_u64(in_off), P, seed)
    ri, rv, rpo = oracle.hash_partition(idx, val, in_off, P, seed)
    assert np.array_equal(host_u64(po), rpo)
    assert np.array_equal(host_u32(oi), ri)
    if val is not None:
        assert np.array_equal(host_bits(ov).reshape(rv.shape).view(np.uint8), rv.view(np.uint8))
    assert sg.sg_device_error() == 0


@pytest.mark.parametrize("P", [1, 2, 3, 8, 16, 100, 256])
def test_partition_scalar_values(P):
    idx, in_off, val = gen.coo_zipf(70 + P, 5, 300000, 9000, 1.05)
    _check(idx, in_off, val, P, 11)


@pytest.mark.parametrize("D", [0, 2, 3, 64])
def test_partition_rows(D):
    idx, in_off, val = gen.coo_zipf(80 + D, 4, 50000, 3000, 1.05, D=max(D, 1))
    _check(idx, in_off, None if D == 0 else val, 8, 2)


def test_partition_bf16():
    idx, in_off, val = gen.coo_zipf(90, 3, 100000, 7000, 1.1)
    _check(idx, in_off, gen.to_bf16(val), 8, 5, bf16=True)
    idx, in_off, val = gen.coo_zipf(91, 3, 100000, 700, 1.1, D=3)
    _check(idx, in_off, gen.to_bf16(val), 5, 5, bf16=True)


def test_partition_empty_and_ragged_workers():
    lists = [np.array([], np.uint32), np.arange(0, 20000, 3, dtype=np.uint32), np.array([], np.uint32),
             np.array([7], np.uint32), np.arange(5, 100000, 7, dtype=np.uint32)[:4097]]
    vals = [gen.normal(1, len(l)) for l in lists]
    idx, in_off, val = gen.coo_from_lists(lists, vals)
    _check(idx, in_off, val, 16, 3)
    # no entries at all
    _check(np.zeros(0, np.uint32), np.zeros(4, np.uint64), np.zeros(0, np.float32), 4, 3)


def test_partition_config2_full():
    c = gen.config2()
    _check(c["idx"], c["in_off"], c["val"], c["P"], c["seed"])


def test_partition_config4_full():
    c = gen.config4()
    _check(c["idx"], c["in_off"], c["val"], c["P"], c["seed"])

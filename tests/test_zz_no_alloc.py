"""sg_hash_partition_noalloc (the partition entry point that allocates
nothing, its scratch a fixed per-GPU array of the library) against
sg_hash_partition with a caller workspace: bit-exact outputs, for two calls
in a row on the same GPU, the second with a smaller input (the array keeps
the first call's contents), for scalar values, rows and indices only; and the
size limit refused before any launch."""
import numpy as np
import pytest
import torch

import gen
import sparse_gradient_synchronization_amd as sg
from gpu_util import host_bits, host_u32, host_u64, need_gpu, to_dev_u32, to_dev_u64, to_dev_vals

pytestmark = pytest.mark.gpu


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert x.shape == y.shape
        assert np.array_equal(host_bits(x) if x.is_floating_point() else x.cpu().numpy(),
                              host_bits(y) if y.is_floating_point() else y.cpu().numpy())


def _both(idx, in_off, val, P, seed):
    d_idx, d_off = to_dev_u32(idx), to_dev_u64(in_off)
    d_val = None if val is None else to_dev_vals(val)
    ref = sg.sg_hash_partition(d_idx, d_val, d_off, P, seed)
    got = sg.sg_hash_partition_noalloc(d_idx, d_val, d_off, P, seed)
    torch.cuda.synchronize()
    _same(got, ref)
    assert sg.sg_device_error() == 0
    return got


@pytest.mark.parametrize("D", [1, 0, 64])
def test_noalloc_matches_workspace_entry_twice(D):
    need_gpu()
    big = gen.coo_zipf(950 + D, 8, 400000, 30000 if D != 64 else 3000, 1.05, D=max(D, 1))
    small = gen.coo_zipf(960 + D, 3, 50000, 2000 if D != 64 else 500, 1.1, D=max(D, 1))
    for idx, in_off, val in (big, small):
        _both(idx, in_off, None if D == 0 else val, 8, 3)


def test_noalloc_full_dgc_sized_partition_then_small():
    need_gpu()
    n, k, M = 8, 2254438, 4096 * 11008
    lists = [np.sort(gen.uniform_distinct(gen.stream_seed(97, w), 0, M, k)) for w in range(n)]
    vals = [gen.normal(970 + w, k) for w in range(n)]
    idx, in_off, val = gen.coo_from_lists(lists, vals)
    _both(idx, in_off, val, 8, 3)
    idx, in_off, val = gen.coo_zipf(971, 2, 1000, 100, 1.1)
    _both(idx, in_off, val, 5, 7)


def test_noalloc_refuses_oversized_input():
    need_gpu()
    # 2^20 entries over 256 partitions need 256 * 520 tiles of counts (fits);
    # rows of 2^23 entries need 32 MiB of sources (does not)
    idx = torch.zeros(1 << 23, dtype=torch.int32, device="cuda")
    val = torch.zeros((1 << 23, 2), dtype=torch.float32, device="cuda")
    off = torch.tensor([0, 1 << 23], dtype=torch.int64, device="cuda")
    with pytest.raises(sg.SgError) as e:
        sg.sg_hash_partition_noalloc(idx, val, off, 4, 1)
    assert e.value.status == -2

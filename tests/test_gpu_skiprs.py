"""GPU parity of sg_skip_reduce_scatter against the oracle (fp64 sums).

Tolerance (the method's acceptance bar): |out - exact| <= 1e-6 (n/c) sum|x|
+ 1e-30 for fp32 inputs, 1e-3 for bf16 inputs; counts bit-exact."""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import assert_sum_close, host_u32, need_gpu, to_dev_vals

pytestmark = pytest.mark.gpu


def _run(bufs_np, slice_elems, p, seed, mode, include=None, bf16=False):
    need_gpu()
    n, M = bufs_np.shape
    esz = 2 if bf16 else 4
    bufs = to_dev_vals(bufs_np, bf16)
    inc_t = None if include is None else torch.from_numpy(np.ascontiguousarray(include)).cuda()
    out, cnt = sg.sg_skip_reduce_scatter(bufs, slice_elems * esz, p, seed, include=inc_t, mode=mode)
    torch.cuda.synchronize()
    ref, ref_abs, ref_cnt = oracle.skip_reduce_scatter(bufs_np, slice_elems, p, seed, include=include, mode=mode)
    assert np.array_equal(cnt.cpu().numpy(), ref_cnt)
    assert_sum_close(out.cpu().numpy(), ref, ref_abs, 1e-3 if bf16 else 1e-6, "skip_rs")
    assert sg.sg_device_error() == 0


@pytest.mark.parametrize("n,M,sl", [(1, 1000, 64), (2, 4096 * 2, 1024), (3, 12345, 100), (8, 8 * 4096 * 3, 4096),
                                    (8, 8 * 65536 + 8 * 12, 65536 // 4), (5, 777, 1), (64, 64 * 40, 8)])
@pytest.mark.parametrize("p", [0.0, 0.5, 1.0])
def test_skip_rs_shapes(n, M, sl, p):
    bufs = gen.dense_normal(50 + n, n, M)
    _run(bufs, sl, p, 1234 + n, 1)
    _run(bufs, sl, p, 99, 0)


@pytest.mark.parametrize("n,M,sl", [(4, 4 * 8192, 2048), (3, 1001, 10)])
def test_skip_rs_bf16(n, M, sl):
    bufs = gen.to_bf16(gen.dense_normal(60, n, M))
    _run(bufs, sl, 0.5, 7, 1, bf16=True)


def test_skip_rs_explicit_masks():
    n, M, sl = 8, 8 * 4096, 512
    bufs = gen.dense_normal(61, n, M)
    S = oracle.num_slices(n, M, sl)
    rng = np.random.default_rng(3)
    for k in range(n):  # static SkipReduce(k)
        inc = np.zeros((n, n, S), np.uint8)
        inc[:, k:, :] = 1
        _run(bufs, sl, 0.0, 0, 0, include=inc)
    inc = (rng.random((n, n, S)) < 0.3).astype(np.uint8)  # includes c = 0 slices
    _run(bufs, sl, 0.0, 0, 1, include=inc)
    dead = np.ones((n, n, S), np.uint8)
    for j in range(n):
        dead[j, (5 - j) % n, :] = 0
    _run(bufs, sl, 0.0, 0, 1, include=dead)


def test_skip_rs_full_config5():
    need_gpu()
    c = gen.config5()
    _run(c["bufs"], c["slice_elems"], c["p"], c["seed"], c["mode"])

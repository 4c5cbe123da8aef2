"""GPU parity of sg_dgc_select (DGC with a sampled global threshold and
residual accumulation) against the oracle.  Every output is decided on or
copied from fp32 values both sides compute with one IEEE addition, so all of
them are compared bit for bit: the threshold key, the counts, the selected
indices and values, and the new residual."""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import host_bits, host_u32, need_gpu

pytestmark = pytest.mark.gpu


def _run(grad, resid, density, S, cap):
    need_gpu()
    g = torch.from_numpy(np.ascontiguousarray(grad)).cuda()
    r = torch.from_numpy(np.ascontiguousarray(resid)).cuda()
    idx, val, cnt, thr = sg.sg_dgc_select(g, r, density, S, cap)
    torch.cuda.synchronize()
    ri, rv, rc, rr, rthr = oracle.dgc_select(grad, resid, density, S, cap=cap)
    assert int(host_u32(thr)[0]) == rthr
    gc = cnt.cpu().numpy().astype(np.uint64)
    assert np.array_equal(gc, rc)
    gi, gv = host_u32(idx), host_bits(val)
    for w in range(grad.shape[0]):
        c = min(int(rc[w]), cap)
        assert np.array_equal(gi[w, :c], ri[w, :c]), w
        assert np.array_equal(gv[w, :c], rv[w, :c].view(np.uint32)), w
    assert np.array_equal(host_bits(r), rr.view(np.uint32))
    assert sg.sg_device_error() == 0
    return rr


@pytest.mark.parametrize("n,M,S,density", [(1, 1000, 100, 0.05), (3, 4096, 4096, 0.1), (2, 3 * 65536 + 5, 1000, 0.05),
                                           (8, 1 << 18, 16384, 0.05), (5, 1023, 7, 0.5), (4, 64, 64, 1.0),
                                           (4, 5000, 300, 0.0)])
def test_dgc_shapes(n, M, S, density):
    rng = np.random.default_rng(M + n)
    grad = (rng.standard_normal((n, M)) * np.exp(rng.standard_normal((n, 1)))).astype(np.float32)
    resid = (rng.standard_normal((n, M)) * 0.05).astype(np.float32)
    _run(grad, resid, density, S, M)


def test_dgc_capacity_truncates_but_counts():
    rng = np.random.default_rng(3)
    n, M = 3, 20000
    grad = rng.standard_normal((n, M)).astype(np.float32)
    _run(grad, np.zeros_like(grad), 0.2, 2000, 100)   # about 4000 selected per worker, 100 kept
    _run(grad, np.zeros_like(grad), 0.2, 2000, 0)     # counts only


def test_dgc_iterations_carry_the_residual():
    rng = np.random.default_rng(9)
    n, M, S = 4, 50000, 4096
    resid = np.zeros((n, M), np.float32)
    for it in range(4):
        grad = rng.standard_normal((n, M)).astype(np.float32)
        resid = _run(grad, resid, 0.05, S, M)


def test_dgc_full_workload():
    # the dgc-top5 gradients (n=8, 4096 x 11008 each), one iteration from a
    # zero residual, 16384 samples per worker, density 5%
    c = gen.config3()
    grad = c["dense"]
    _run(grad, np.zeros_like(grad), 0.05, 16384, c["k"] + c["k"] // 4)

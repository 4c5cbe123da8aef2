"""GPU parity of sg_classmap_build + sg_encode against the oracle: the hash
bitmap and word offsets bit-exact, plus the Fig. 10 walk-through replayed on
the GPU."""
import json
import os

import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_gradient_synchronization_amd as sg
from gpu_util import host_u32, host_u64, need_gpu, to_dev_u32, to_dev_u64

pytestmark = pytest.mark.gpu


def _agg_of(keys, P, seed):
    keys = np.unique(np.asarray(keys, dtype=np.uint32))
    h = oracle.h0(keys, seed, P)
    order = np.argsort(h, kind="stable")
    off = np.concatenate([[0], np.cumsum(np.bincount(h, minlength=P))]).astype(np.uint64)
    return keys[order], off


def _check(agg_idx, agg_off, M, seed):
    need_gpu()
    P = agg_off.size - 1
    cmap = sg.sg_classmap_build(M, P, seed)
    bm, wo = sg.sg_encode(to_dev_u32(agg_idx if agg_idx.size else np.zeros(1, np.uint32)), to_dev_u64(agg_off), M,
                          cmap)
    torch.cuda.synchronize()
    rb, rwo = oracle.encode(agg_idx, agg_off, M, seed)
    assert np.array_equal(host_u64(wo), rwo)
    assert np.array_equal(host_u32(bm)[: int(rwo[-1])], rb)
    assert sg.sg_device_error() == 0


@pytest.mark.parametrize("M", [1, 31, 32, 33, 4095, 4096, 4097, 100003, 1 << 20])
@pytest.mark.parametrize("P", [1, 3, 16])
def test_encode_random_sets(M, P):
    rng = np.random.default_rng(M * 7 + P)
    keys = np.flatnonzero(rng.random(M) < 0.2)
    a, o = _agg_of(keys, P, 5)
    _check(a, o, M, 5)


@pytest.mark.parametrize("P", [2, 8, 17, 64, 100, 256])
def test_encode_partition_counts(P):
    rng = np.random.default_rng(P)
    M = 300001
    keys = np.flatnonzero(rng.random(M) < 0.5)
    a, o = _agg_of(keys, P, 77)
    _check(a, o, M, 77)


def test_encode_empty_and_full():
    M, P = 70000, 16
    a, o = _agg_of(np.zeros(0, np.uint32), P, 3)
    _check(a, o, M, 3)
    a, o = _agg_of(np.arange(M), P, 3)
    _check(a, o, M, 3)


def test_encode_fig10_on_gpu():
    with open(os.path.join(os.path.dirname(__file__), "golden", "zen_fig10.json")) as f:
        g = json.load(f)
    need_gpu()
    nz = np.array([i - 1 for i in g["page_nonzero_indices_1based"]], np.uint32)
    off = np.array([0, 2, 2, 2], np.uint64)
    cmap = sg.sg_classmap_build(g["G"], g["servers"], g["seed"])
    bm, wo = sg.sg_encode(to_dev_u32(nz), to_dev_u64(off), g["G"], cmap)
    w0 = int(host_u32(bm)[int(host_u64(wo)[0])])
    assert [b for b in range(32) if w0 >> b & 1] == [b - 1 for b in g["page_set_bits_1based"]]


def test_encode_config4_full():
    c = gen.config4()
    oi, ov, po = oracle.hash_partition(c["idx"], None, c["in_off"], c["P"], c["seed"])
    ai, _, _, ao = oracle.aggregate(oi, None, po, c["M"])
    _check(ai, ao, c["M"], c["seed"])


def test_encode_config1_full():
    c = gen.config1()
    oi, ov, po = oracle.hash_partition(c["idx"], None, c["in_off"], c["P"], c["seed"])
    ai, _, _, ao = oracle.aggregate(oi, None, po, c["M"])
    _check(ai, ao, c["M"], c["seed"])


# The group encode (2 <= P <= 16 with at least 2048 groups of windows): sizes
# just past that threshold with a ragged last window, sparse and dense
# stretches (a window of all keys takes many rounds of 64 per partition),
# classes with no aggregated key at all.
_GROUP_M = {2: 2048 * 4096 + 12345, 3: 2048 * 4096 + 5, 4: 2048 * 4096 + 1, 5: 2048 * 4096 + 777,
            8: 2048 * 4096 + 4095, 9: 4 * 2048 * 4096 + 4097, 13: 4 * 2048 * 4096 + 999, 16: 4 * 2048 * 4096 + 31}


@pytest.mark.parametrize("P", sorted(_GROUP_M))
def test_encode_group_path(P):
    M = _GROUP_M[P]
    rng = np.random.default_rng(1000 + P)
    dens = np.where(np.arange(M) < M // 16, 0.6, 0.03)
    keys = np.flatnonzero(rng.random(M) < dens)
    dense_run = np.arange(M // 2, M // 2 + 3 * 4096 + 17) # every key of a few windows
    keys = np.union1d(keys, dense_run)
    a, o = _agg_of(keys, P, 40 + P)
    _check(a, o, M, 40 + P)


def test_encode_group_path_empty_classes():
    M, P, seed = 4 * 2048 * 4096 + 100, 16, 9
    rng = np.random.default_rng(3)
    keys = np.flatnonzero(rng.random(M) < 0.1).astype(np.uint32)
    keys = keys[oracle.h0(keys, seed, P) % 3 == 0] # classes 1, 2, 4, 5, ... have nothing
    a, o = _agg_of(keys, P, seed)
    _check(a, o, M, seed)

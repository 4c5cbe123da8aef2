"""Pins of the CPU oracle against things other than itself.

Each test checks an oracle function against a value the pages or the
mathematics fix: a published check value, brute force on tiny inputs written
with different primitives (numpy sorts, Python sets, fsum), closed forms, or
invariants.  A plausible mistake in the oracle (a dropped term, a wrong sign or
index, a transposed operand) fails at least one of these.  No GPU needed.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# hash and random numbers: published check values
# --------------------------------------------------------------------------

def test_murmur2_verification_value():
    g = _golden("hash_check_values.json")["murmur2_32"]
    key = bytearray(256)
    blob = b""
    for i in range(256):
        key[i] = i
        blob += struct.pack("<I", oracle.murmur2(bytes(key[:i]), 256 - i))
    assert oracle.murmur2(blob, 0) == int(g["verification"], 16)


def test_splitmix64_published_outputs():
    g = _golden("hash_check_values.json")["splitmix64"]
    assert oracle.splitmix64_outputs(0, 3) == [int(x, 16) for x in g["seed_0_first3"]]
    assert oracle.splitmix64_outputs(1234567, 5) == g["seed_1234567_first5"]
    # the counter form used by the skip mask is the same stream
    for c in range(5):
        assert oracle.splitmix64_at(1234567, c) == g["seed_1234567_first5"][c]


def test_splitmix64_counter_form_is_the_stream():
    # output number c of the stream started at seed, against stepping the
    # stream c + 1 times
    rng = np.random.default_rng(1)
    for seed in [0, 1, 2**63 + 5] + [int(x) for x in rng.integers(0, 2**63, size=3, dtype=np.uint64)]:
        outs = oracle.splitmix64_outputs(seed, 300)
        for c in (0, 1, 2, 17, 150, 299):
            assert oracle.splitmix64_at(seed, c) == outs[c]


def test_h0_is_murmur2_of_le_bytes_mod_P():
    rng = np.random.default_rng(0)
    xs = rng.integers(0, 2**32, size=200, dtype=np.uint64).astype(np.uint32)
    for P in (1, 3, 16, 255):
        got = oracle.h0(xs, 7, P)
        for x, g in zip(xs, got):
            assert g == oracle.murmur2(struct.pack("<I", int(x)), 7) % P


def test_h0_balance_matches_theorem2_scale():
    # Zen section 3.2, Theorem 2: with a universal hash the heaviest of n
    # partitions exceeds the mean by a factor 1 + Theta(sqrt(n ln n / N)).
    N, P = 1 << 20, 16
    parts = oracle.h0(np.arange(N, dtype=np.uint32), 4, P)
    counts = np.bincount(parts, minlength=P)
    imb = counts.max() * P / N
    assert 1.0 <= imb < 1.0 + 4.0 * math.sqrt(P * math.log(P) / N)


# --------------------------------------------------------------------------
# A1 top-k
# --------------------------------------------------------------------------

def _topk_brute(row, k, bf16):
    bits = row.view(np.uint16 if bf16 else np.uint32).astype(np.uint64)
    mag = bits & (0x7FFF if bf16 else 0x7FFFFFFF)
    order = np.lexsort((np.arange(row.size), -mag.astype(np.int64)))  # by -|x|, then index
    return np.sort(order[:k])


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M,k", [(1, 1), (7, 0), (7, 3), (7, 7), (100, 37), (257, 256)])
def test_topk_brute_force_with_ties(M, k, bf16):
    rng = np.random.default_rng(M * 31 + k)
    n = 3
    # few distinct magnitudes so ties (and +0/-0) are common
    vals = rng.integers(-3, 4, size=(n, M)).astype(np.float32)
    vals[vals == 0] = np.where(rng.random((vals == 0).sum()) < 0.5, 0.0, -0.0)
    dense = gen.to_bf16(vals) if bf16 else vals
    idx, val = oracle.topk_to_coo(dense, k)
    for w in range(n):
        exp = _topk_brute(dense[w], k, bf16)
        assert np.array_equal(idx[w], exp.astype(np.uint32))
        assert np.array_equal(val[w].view(np.uint8), dense[w][exp].view(np.uint8))


def test_topk_selection_invariant_random():
    rng = np.random.default_rng(5)
    dense = rng.standard_normal((2, 5000)).astype(np.float32)
    k = 321
    idx, val = oracle.topk_to_coo(dense, k)
    for w in range(2):
        sel = np.zeros(5000, bool)
        sel[idx[w]] = True
        assert np.all(np.diff(idx[w].astype(np.int64)) > 0)
        assert np.abs(dense[w][sel]).min() >= np.abs(dense[w][~sel]).max()
        assert np.array_equal(val[w], dense[w][idx[w]])


def test_topk_k_equals_nnz_is_nonzero_extraction():
    c = gen.config1(n=2, M=1 << 14)
    idx, _ = oracle.topk_to_coo(c["dense"], c["k"])
    for w in range(2):
        assert np.array_equal(idx[w], np.flatnonzero(c["dense"][w]).astype(np.uint32))


# --------------------------------------------------------------------------
# A2 hash partition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("P", [1, 3, 16])
@pytest.mark.parametrize("D", [0, 1, 3])
def test_partition_is_stable_grouping_by_h0(P, D):
    c = gen.coo_zipf(9, 3, 5000, 300, 1.1, D=max(D, 1))
    idx, in_off, val = c
    if D == 0:
        val = None
    oi, ov, po = oracle.hash_partition(idx, val, in_off, P, 11)
    h = oracle.h0(idx, 11, P)
    for w in range(3):
        b, e = int(in_off[w]), int(in_off[w + 1])
        order = b + np.argsort(h[b:e], kind="stable")
        assert np.array_equal(oi[b:e], idx[order])
        if D:
            assert np.array_equal(ov[b:e], val[order])
        counts = np.bincount(h[b:e], minlength=P)
        assert np.array_equal(np.diff(po[w].astype(np.int64)), counts)
        assert po[w, 0] == b and po[w, P] == e


def test_partition_same_index_same_server():
    idx = np.array([5, 9, 100, 5, 100, 7], dtype=np.uint32)
    in_off = np.array([0, 3, 6], dtype=np.uint64)
    oi, _, po = oracle.hash_partition(idx, None, in_off, 4, 3)
    where = {}
    for w in range(2):
        for p in range(4):
            for x in oi[int(po[w, p]):int(po[w, p + 1])]:
                assert where.setdefault(int(x), p) == p


# --------------------------------------------------------------------------
# A3 aggregate
# --------------------------------------------------------------------------

def _agg_brute(idx, val, part_off, D):
    n, P1 = part_off.shape
    sums, abss, owner = {}, {}, {}
    for w in range(n):
        for p in range(P1 - 1):
            for i in range(int(part_off[w, p]), int(part_off[w, p + 1])):
                x = int(idx[i])
                v = val[i] if D > 1 else [val[i]]
                sums.setdefault(x, [[] for _ in range(max(D, 1))])
                for d in range(max(D, 1)):
                    sums[x][d].append(float(v[d]))
                owner[x] = p
    return sums, owner


@pytest.mark.parametrize("D", [1, 4])
def test_aggregate_brute_force(D):
    idx, in_off, val = gen.coo_zipf(13, 5, 400, 60, 0.8, D=D)
    oi, ov, po = oracle.hash_partition(idx, val, in_off, 3, 2)
    ai, av, aa, ao = oracle.aggregate(oi, ov, po, 400)
    sums, owner = _agg_brute(oi, ov, po, D)
    assert ai.size == len(sums)
    for p in range(3):
        keys = sorted(k for k, q in owner.items() if q == p)
        assert list(ai[int(ao[p]):int(ao[p + 1])]) == keys
    for j, x in enumerate(ai):
        for d in range(D):
            terms = sums[int(x)][d]
            exact = math.fsum(terms)
            got = av[j, d] if D > 1 else av[j]
            absum = aa[j, d] if D > 1 else aa[j]
            assert abs(got - exact) <= len(terms) * 2.0**-52 * sum(abs(t) for t in terms)
            assert abs(absum - math.fsum(abs(t) for t in terms)) <= 1e-12 * absum + 1e-300


def test_aggregate_union_bounds_and_extremes():
    # disjoint supports: |I| = sum, values unchanged
    a = np.array([1, 5, 9], np.uint32)
    b = np.array([2, 6, 10], np.uint32)
    idx = np.concatenate([a, b])
    val = np.arange(6, dtype=np.float32) + 1
    in_off = np.array([0, 3, 6], np.uint64)
    oi, ov, po = oracle.hash_partition(idx, val, in_off, 2, 1)
    ai, av, _, _ = oracle.aggregate(oi, ov, po, 16)
    assert ai.size == 6
    m = dict(zip(idx.tolist(), val.tolist()))
    assert all(av[j] == m[int(x)] for j, x in enumerate(ai))
    # identical supports: |I| = |I_w|, values add
    idx = np.concatenate([a, a, a])
    val = np.ones(9, np.float32)
    in_off = np.array([0, 3, 6, 9], np.uint64)
    oi, ov, po = oracle.hash_partition(idx, val, in_off, 2, 1)
    ai, av, _, _ = oracle.aggregate(oi, ov, po, 16)
    assert ai.size == 3 and np.all(av == 3.0)
    # a cancelling index stays in the aggregate (membership, not value)
    idx = np.array([4, 4], np.uint32)
    val = np.array([2.5, -2.5], np.float32)
    oi, ov, po = oracle.hash_partition(idx, val, np.array([0, 1, 2], np.uint64), 1, 0)
    ai, av, _, _ = oracle.aggregate(oi, ov, po, 8)
    assert list(ai) == [4] and av[0] == 0.0
    # general bounds
    idx, in_off, val = gen.coo_zipf(3, 6, 3000, 400, 1.0)
    oi, ov, po = oracle.hash_partition(idx, val, in_off, 4, 3)
    ai, _, _, ao = oracle.aggregate(oi, ov, po, 3000)
    nnz = np.diff(in_off.astype(np.int64))
    assert nnz.max() <= ai.size <= nnz.sum() and ao[-1] == ai.size


def test_aggregate_dense_allreduce_equivalence():
    # Zen section 3.2: the sparse aggregate equals the dense AllReduce
    n, M = 4, 2000
    idx, in_off, val = gen.coo_zipf(21, n, M, 150, 1.2)
    dense = gen.dense_from_coo(n, M, idx, in_off, val).astype(np.float64).sum(0)
    oi, ov, po = oracle.hash_partition(idx, val, in_off, 5, 9)
    ai, av, _, _ = oracle.aggregate(oi, ov, po, M)
    out = np.zeros(M)
    out[ai] = av
    assert np.allclose(out, dense, rtol=0, atol=1e-12)


def _skewed_expectations(n, M, c):
    h = int(0.6 * c)
    t = c - h
    Rh, Rt = M // 8, M - M // 8
    Uh = Rh * (1 - (1 - h / Rh) ** n)
    Ut = Rt * (1 - (1 - t / Rt) ** n)
    return h, t, Rh, Rt, Uh, Ut


def test_config4_union_closed_form_scaled():
    # Each region is sampled uniformly without replacement, so an index is in
    # a worker's set with probability c_region / R_region, independently over
    # workers: E|I| = sum over regions of R (1 - (1 - c/R)^n).
    n, M = 16, 1 << 22
    d = gen.config4(n=n, M=M)
    oi, ov, po = oracle.hash_partition(d["idx"], d["val"], d["in_off"], 16, 4)
    ai, _, _, _ = oracle.aggregate(oi, ov, po, M)
    h, t, Rh, Rt, Uh, Ut = _skewed_expectations(n, M, M // 100)
    ph, pt = 1 - (1 - h / Rh) ** n, 1 - (1 - t / Rt) ** n
    sd = math.sqrt(Rh * ph * (1 - ph) + Rt * pt * (1 - pt))
    assert abs(ai.size - (Uh + Ut)) < 6 * sd
    # the full-size value of the same formula, as the survey states it
    _, _, _, _, Uh4, Ut4 = _skewed_expectations(16, 1 << 28, (1 << 28) // 100)
    assert abs((Uh4 + Ut4) - 34_884_067.5) < 1.0


# --------------------------------------------------------------------------
# A4 encode / decode
# --------------------------------------------------------------------------

def test_encode_fig10_walkthrough():
    g = _golden("zen_fig10.json")
    G, P, seed = g["G"], g["servers"], g["seed"]
    nz = np.array([i - 1 for i in g["page_nonzero_indices_1based"]], np.uint32)
    # server 0 holds exactly these two indices
    agg_off = np.array([0, 2, 2, 2], np.uint64)
    bitmap, word_off = oracle.encode(nz, agg_off, G, seed)
    bits0 = [b for b in range(32) if bitmap[int(word_off[0])] >> b & 1]
    assert bits0 == [b - 1 for b in g["page_set_bits_1based"]]
    dec, off = oracle.decode(bitmap, P, G, seed)
    assert list(dec[int(off[0]):int(off[1])]) == list(nz)


@pytest.mark.parametrize("M,P", [(1, 1), (31, 2), (1000, 7), (1 << 15, 16)])
def test_encode_popcount_size_and_roundtrip(M, P):
    rng = np.random.default_rng(M + P)
    keys = np.flatnonzero(rng.random(M) < 0.3).astype(np.uint32)
    h = oracle.h0(keys, 5, P)
    order = np.argsort(h, kind="stable")
    agg_idx = keys[order]
    agg_off = np.concatenate([[0], np.cumsum(np.bincount(h, minlength=P))]).astype(np.uint64)
    bitmap, word_off = oracle.encode(agg_idx, agg_off, M, 5)
    csize, rank = oracle.classmap(M, P, 5)
    assert csize.sum() == M
    assert np.array_equal(np.diff(word_off.astype(np.int64)), (csize.astype(np.int64) + 31) // 32)
    assert M / 32 <= word_off[P] <= M / 32 + P
    for p in range(P):
        words = bitmap[int(word_off[p]):int(word_off[p + 1])]
        pc = sum(bin(int(x)).count("1") for x in words)
        assert pc == agg_off[p + 1] - agg_off[p]
        # padding bits beyond |C_p| are zero
        if csize[p] % 32:
            assert int(words[-1]) >> int(csize[p] % 32) == 0
    dec, off = oracle.decode(bitmap, P, M, 5)
    assert np.array_equal(dec, agg_idx) and np.array_equal(off, agg_off)
    # rank is the position inside the ascending class list
    for p in range(P):
        members = np.flatnonzero(oracle.h0(np.arange(M, dtype=np.uint32), 5, P) == p)
        assert np.array_equal(rank[members], np.arange(members.size, dtype=np.uint32))


# --------------------------------------------------------------------------
# A5 skip reduce-scatter
# --------------------------------------------------------------------------

def _rs_brute(bufs, slice_elems, include, mode):
    n, M = bufs.shape
    b = bufs.astype(np.float64)
    out = np.zeros(M)
    S = include.shape[2]
    for j in range(n):
        cb, ce = (M * j) // n, (M * (j + 1)) // n
        for q in range(S):
            sb, se = cb + q * slice_elems, min(cb + (q + 1) * slice_elems, ce)
            if sb >= se:
                continue
            ranks = [(j + t) % n for t in range(n) if include[j, t, q]]
            c = len(ranks)
            if c == 0:
                continue
            s = np.zeros(se - sb)
            for r in ranks:  # ring order
                s = s + b[r, sb:se]
            out[sb:se] = s * (n / c if mode == 1 else 1.0)
    return out


@pytest.mark.parametrize("n,M,sl", [(1, 10, 3), (2, 9, 2), (4, 64, 4), (5, 103, 7), (8, 1000, 32)])
def test_skip_rs_brute_force(n, M, sl):
    rng = np.random.default_rng(n * 1000 + M)
    bufs = rng.standard_normal((n, M)).astype(np.float32)
    for p, mode in ((0.0, 1), (0.5, 1), (0.5, 0), (0.9, 1)):
        out, out_abs, cnt = oracle.skip_reduce_scatter(bufs, sl, p, 77, mode=mode)
        S = oracle.num_slices(n, M, sl)
        inc = oracle.skip_mask(n, S, p, 77)
        assert np.all(inc[:, 0, :] == 1)
        assert np.array_equal(cnt, inc.sum(1).astype(np.uint8))
        assert np.allclose(out, _rs_brute(bufs, sl, inc, mode), rtol=1e-13, atol=1e-13)
        assert np.all(out_abs >= np.abs(out) - 1e-12)


def test_skip_rs_p0_is_full_sum():
    bufs = gen.dense_normal(99, 6, 5000)
    out, _, cnt = oracle.skip_reduce_scatter(bufs, 100, 0.0, 1)
    assert np.all(cnt == 6)
    exact = np.array([math.fsum(col) for col in bufs.astype(np.float64).T])
    assert np.allclose(out, exact, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_skip_rs_closed_form_equals_ring_replay(n):
    # Skip Algorithms 1-2 replayed with explicit send/recv buffers gives the
    # same arithmetic as the closed form (mode 0: no rescale), bit for bit.
    rng = np.random.default_rng(n)
    M, sl = 37 * n + 3, 5
    bufs = rng.standard_normal((n, M)).astype(np.float32)
    S = oracle.num_slices(n, M, sl)
    for trial in range(3):
        inc = (rng.random((n, n, S)) < 0.6).astype(np.uint8)
        if trial == 0:
            inc[:] = 1
        out, _, _ = oracle.skip_reduce_scatter(bufs, sl, 0.0, 0, include=inc, mode=0)
        rep = oracle.ring_replay(bufs, sl, inc)
        assert np.array_equal(out, rep)


def test_static_skipreduce_skips_k_over_n():
    # Skip Algorithm 2 runs the reduce-scatter loop from s = k: chunk j keeps
    # only ring positions t >= k, i.e. k/N of the contributions are skipped.
    n, M, sl = 8, 8 * 64, 16
    S = oracle.num_slices(n, M, sl)
    bufs = gen.dense_normal(7, n, M)
    for k in range(n):
        inc = np.zeros((n, n, S), np.uint8)
        inc[:, k:, :] = 1
        out, _, cnt = oracle.skip_reduce_scatter(bufs, sl, 0.0, 0, include=inc, mode=0)
        assert cnt.sum() == (n - k) * n * S
        assert 1 - cnt.sum() / (n * n * S) == pytest.approx(k / n)
        rep = oracle.ring_replay(bufs, sl, inc)
        assert np.array_equal(out, rep)


def test_seeded_mask_rate():
    n, S, p = 8, 128, 0.5
    inc = oracle.skip_mask(n, S, p, 5)
    draws = inc[:, 1:, :]
    rate = 1 - draws.mean()
    sd = math.sqrt(p * (1 - p) / draws.size)
    assert abs(rate - p) < 5 * sd
    assert oracle.skip_threshold(0.5) == 1 << 23 and oracle.skip_threshold(1.0) == 1 << 24
    assert oracle.skip_threshold(0.0) == 0


def test_dead_rank_mask():
    n, M, sl = 4, 400, 10
    S = oracle.num_slices(n, M, sl)
    bufs = gen.dense_normal(8, n, M)
    dead = 2
    inc = np.ones((n, n, S), np.uint8)
    for j in range(n):
        inc[j, (dead - j) % n, :] = 0
    out, _, _ = oracle.skip_reduce_scatter(bufs, sl, 0.0, 0, include=inc, mode=1)
    others = np.delete(bufs.astype(np.float64), dead, axis=0).sum(0) * n / (n - 1)
    assert np.allclose(out, others, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# A6 stats
# --------------------------------------------------------------------------

def test_stats_brute_force():
    idx, in_off, _ = gen.coo_zipf(31, 5, 700, 90, 0.9)
    M, P = 700, 6
    st = oracle.stats(idx, in_off, M, P, hashed=True, seed=3)
    sets = [set(idx[int(in_off[w]):int(in_off[w + 1])].tolist()) for w in range(5)]
    U = set().union(*sets)
    assert st["union_size"] == len(U)
    for a in range(5):
        for b in range(5):
            assert st["inter"][a, b] == len(sets[a] & sets[b])
            assert st["overlap"][a, b] == len(sets[a] & sets[b]) / min(len(sets[a]), len(sets[b]))
    assert st["gamma_n"] == 5 * len(U) / sum(len(s) for s in sets)
    bounds = [(M * i) // P for i in range(P + 1)]
    for w, s in enumerate(sets + [U]):
        cnt = [sum(1 for x in s if bounds[i] <= x < bounds[i + 1]) for i in range(P)]
        assert list(st["contig_counts"][w]) == cnt
        sk = max((cnt[i] / (bounds[i + 1] - bounds[i])) / (len(s) / M) for i in range(P))
        assert st["skew_contig"][w] == pytest.approx(sk, rel=1e-14)
    cls = oracle.h0(np.arange(M, dtype=np.uint32), 3, P)
    for w, s in enumerate(sets + [U]):
        hc = np.bincount(oracle.h0(np.array(sorted(s), np.uint32), 3, P), minlength=P)
        assert np.array_equal(st["hashed_counts"][w], hc)
    g = np.bincount(cls, minlength=P)
    push = max(P * st["hashed_counts"][w, i] / len(sets[w]) for w in range(5) for i in range(P))
    pull = max(P * st["hashed_counts"][5, i] / len(U) for i in range(P))
    assert st["push_imbalance"] == pytest.approx(push, rel=1e-14)
    assert st["pull_imbalance"] == pytest.approx(pull, rel=1e-14)
    assert np.array_equal(st["class_size"], g)


def test_stats_identical_disjoint_and_gamma_bounds():
    a = np.arange(0, 50, 2, dtype=np.uint32)
    b = np.arange(1, 50, 2, dtype=np.uint32)
    st = oracle.stats(np.concatenate([a, a, a]), np.array([0, 25, 50, 75], np.uint64), 64, 4)
    assert st["overlap_min"] == st["overlap_max"] == 1.0 and st["gamma_n"] == 1.0
    st = oracle.stats(np.concatenate([a, b]), np.array([0, 25, 50], np.uint64), 64, 4)
    assert st["overlap_max"] == 0.0 and st["gamma_n"] == 2.0
    idx, in_off, _ = gen.coo_zipf(5, 8, 5000, 500, 1.1)
    st = oracle.stats(idx, in_off, 5000, 8)
    # Zen section 2.1: densification stays below n when supports overlap
    assert 1.0 <= st["gamma_n"] < 8.0 and st["overlap_max"] > 0


def test_config4_stats_closed_forms_scaled():
    n, M, P = 16, 1 << 22, 16
    d = gen.config4(n=n, M=M)
    st = oracle.stats(d["idx"], d["in_off"], M, P, hashed=True, seed=4)
    c = M // 100
    h, t, Rh, Rt, Uh, Ut = _skewed_expectations(n, M, c)
    # overlap of two independent uniform samples: E|I_a & I_b| = h^2/Rh + t^2/Rt
    assert st["overlap_mean"] == pytest.approx((h * h / Rh + t * t / Rt) / c, rel=0.02)
    assert st["gamma_n"] == pytest.approx((Uh + Ut) / c, rel=0.002)
    # contiguous skew: parts 0 and 1 split the head, each ~h/2 of c entries
    assert np.all(np.abs(st["skew_contig"][:n] - 16 * (h / 2) / c) < 0.2)
    assert st["skew_contig"][n] == pytest.approx(16 * (Uh / 2) / (Uh + Ut), rel=0.02)
    # after hashing: Theorem 2 scale, close to 1
    bound = 1 + 6 * math.sqrt(P * math.log(P) / c)
    assert np.all(st["skew_hashed"] < bound) and st["push_imbalance"] < bound
    assert st["pull_imbalance"] < 1 + 6 * math.sqrt(P * math.log(P) / st["union_size"])


# --------------------------------------------------------------------------
# NEXT-1: Pull-side scatter to dense and encoded-size accounting
# --------------------------------------------------------------------------

def test_scatter_dense_places_values_and_zeros_elsewhere():
    rng = np.random.default_rng(5)
    M, P = 5000, 4
    idx = np.sort(rng.choice(M, size=700, replace=False)).astype(np.uint32)
    val = rng.standard_normal(700).astype(np.float32)
    off = np.array([0, 100, 400, 400, 700], dtype=np.uint64)
    dense = oracle.scatter_dense(idx, val, off, M)
    assert dense.dtype == np.float32 and dense.shape == (M,)
    assert np.array_equal(dense[idx].view(np.uint32), val.view(np.uint32))  # bit copies
    rest = np.ones(M, bool)
    rest[idx] = False
    assert not np.any(dense[rest])
    rows = rng.standard_normal((700, 3)).astype(np.float32)
    dense3 = oracle.scatter_dense(idx, rows, off, M, D=3)
    assert np.array_equal(dense3[idx], rows) and not np.any(dense3[rest])


def test_scatter_of_aggregate_is_the_dense_allreduce():
    # Zen section 3.2: the synchronized result equals the dense AllReduce; after
    # Pull a worker's dense gradient is the sum of all workers' gradients
    c = gen.config1(n=4, M=1 << 14)
    n, M, P, seed = c["n"], c["M"], c["P"], c["seed"]
    oi, ov, po = oracle.hash_partition(c["idx"], c["val"], c["in_off"], P, seed)
    ai, av, aa, ao = oracle.aggregate(oi, ov, po, M)
    dense = oracle.scatter_dense(ai, av, ao, M)
    want = c["dense"].astype(np.float64).sum(axis=0)
    tol = 1e-6 * np.abs(c["dense"].astype(np.float64)).sum(axis=0) + 1e-30
    assert np.all(np.abs(dense.astype(np.float64) - want) <= tol)


def test_format_sizes_against_page_examples():
    g = _golden("zen_formats.json")
    # density after aggregation: dense / values-only and dense / COO traffic
    ex = g["coo_after_aggregation"]
    M = 100_000
    U = int(round(ex["density"] * M))
    idx = np.arange(U, dtype=np.uint32) * (M // U)
    s = oracle.format_sizes(np.sort(idx), np.array([0, U], np.uint64), M, 1, 7)
    assert s["coo"] == U * 8 and s["dense"] == M * 4
    assert round(s["dense"] / (U * 4), 1) == ex["values_only_reduction"]
    assert round(s["dense"] / s["coo"], 1) == ex["coo_reduction"]
    # contiguous bitmap: |G| = 15 over 3 servers
    ex = g["contiguous_bitmap_example"]
    s = oracle.format_sizes(np.zeros(0, np.uint32), np.zeros(ex["servers"] + 1, np.uint64), ex["G"], 1, 1)
    assert s["bitmap"] == 4 * ex["words_per_server"] * ex["servers"]
    # the hash bitmap of 15 indices over 3 classes: one word per non-empty class
    assert s["hash_bitmap"] <= 4 * ex["servers"]


def test_format_sizes_bitmaps_total_G_over_32():
    # Zen sections 3.3.1-3.3.2: the bitmaps a worker receives add up to about
    # |G|/32 words whatever the number of servers; the page's 856 MB table
    g = _golden("zen_formats.json")["deepfm_bitmap"]
    M = g["table_MB"] * 1_000_000 // 4
    for P in (1, 8):
        s = oracle.format_sizes(np.zeros(0, np.uint32), np.zeros(P + 1, np.uint64), M, 1, 2)
        for fmt in ("bitmap", "hash_bitmap"):
            assert M / 8 <= s[fmt] <= M / 8 + 4 * P
            assert round(s[fmt] / 1e6) == g["bitmap_MB"]


def test_format_sizes_brute_force_blocks_and_classes():
    rng = np.random.default_rng(11)
    for M, P, D in ((1000, 3, 1), (70_000, 8, 4), (256 * 40 + 13, 5, 2)):
        U = M // 7
        idx = np.sort(rng.choice(M, size=U, replace=False)).astype(np.uint32)
        part = oracle.h0(idx, 9, P)
        order = np.argsort(part, kind="stable")
        idx = idx[order]
        off = np.zeros(P + 1, np.uint64)
        off[1:] = np.cumsum(np.bincount(part, minlength=P))
        s = oracle.format_sizes(idx, off, M, D, 9)
        blocks = np.unique(idx // 256).size
        assert s["nonempty_blocks"] == blocks
        assert s["block"] == blocks * (256 * 4 * D + 4)
        csize = np.bincount(oracle.h0(np.arange(M, dtype=np.uint32), 9, P), minlength=P)
        assert s["hash_bitmap"] == 4 * int(np.sum((csize + 31) // 32)) + U * 4 * D
        bounds = [(M * i) // P for i in range(P + 1)]
        assert s["bitmap"] == 4 * sum((bounds[i + 1] - bounds[i] + 31) // 32 for i in range(P)) + U * 4 * D
        assert s["coo"] == U * (4 + 4 * D) and s["union"] == U
    # full density: every block is used
    M = 256 * 9 + 1
    s = oracle.format_sizes(np.arange(M, dtype=np.uint32), np.array([0, M], np.uint64), M, 1, 3)
    assert s["nonempty_blocks"] == 10


# --------------------------------------------------------------------------
# NEXT-2: the SkipReduce family
# --------------------------------------------------------------------------

def _replay_alg2_shifted(bufs, k, off):
    """Skip Algorithm 2 with explicit per-rank buffers, the reduce-scatter loop
    from step k and the slice indices shifted by `off` (Random SkipReduce,
    section 4.3).  One slice per chunk.  Returns the reduced chunks, each from
    the rank that ends holding it."""
    n, M = bufs.shape
    x = bufs.astype(np.float64).copy()
    cb = [(M * j) // n for j in range(n + 1)]
    for s in range(k, n - 1):
        msgs = [x[r, cb[(r - s + off) % n]:cb[(r - s + off) % n + 1]].copy() for r in range(n)]
        for r in range(n):
            c = (r - s - 1 + off) % n
            x[r, cb[c]:cb[c + 1]] += msgs[(r - 1) % n]
    out = np.zeros(M)
    for r in range(n):  # after the last step (N-2) rank r received chunk (r - (N-2) - 1 + off)
        c = (r - (n - 2) - 1 + off) % n
        out[cb[c]:cb[c + 1]] = x[r, cb[c]:cb[c + 1]]
    return out


@pytest.mark.parametrize("n", [2, 3, 5, 8])
def test_static_and_random_skipreduce_masks_replay_algorithm2(n):
    rng = np.random.default_rng(40 + n)
    M = 11 * n + 2
    bufs = rng.standard_normal((n, M)).astype(np.float32)
    sl = M  # one slice per chunk
    for k in range(n):
        st = oracle.skip_mask_static(n, 1, k)
        assert st[:, :k].sum() == 0 and st[:, k:].all()
        out, _, cnt = oracle.skip_reduce_scatter(bufs, sl, 0.0, 0, include=st, mode=0)
        assert np.allclose(out, _replay_alg2_shifted(bufs, k, 0), rtol=1e-12, atol=1e-12)
        for seed in (1, 2, 3, 99):
            off = oracle.splitmix64_at(seed, 0) % n
            rm = oracle.skip_mask_random(n, 1, k, seed)
            assert np.array_equal(rm, np.roll(st, -off, axis=1))  # the static mask rotated
            out, _, _ = oracle.skip_reduce_scatter(bufs, sl, 0.0, 0, include=rm, mode=0)
            assert np.allclose(out, _replay_alg2_shifted(bufs, k, off), rtol=1e-12, atol=1e-12)


def test_random_skipreduce_offsets_are_uniform():
    n, trials = 8, 4000
    offs = np.array([oracle.skip_mask_random(n, 1, 1, s)[0, :, 0].argmin() for s in range(trials)])
    counts = np.bincount((n - offs) % n, minlength=n)
    exp = trials / n
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 30  # 7 degrees of freedom


def _replay_alg1(bufs, p, seed):
    """Skip Algorithm 1 (AllReduce_Dropout) with explicit per-rank buffers:
    ReduceOrSkip per element, drawing SplitMix64 output (t-1)*M + e for the
    element e received at ring position t."""
    n, M = bufs.shape
    thr = oracle.skip_threshold(p)
    x = bufs.astype(np.float64).copy()
    cb = [(M * j) // n for j in range(n + 1)]
    for s in range(n - 1):
        msgs = [x[r, cb[(r - s) % n]:cb[(r - s) % n + 1]].copy() for r in range(n)]
        for r in range(n):
            c = (r - s - 1) % n
            t = (r - c) % n
            y = msgs[(r - 1) % n]
            for i, e in enumerate(range(cb[c], cb[c + 1])):
                skip = (oracle.splitmix64_at(seed, (t - 1) * M + e) >> 40) < thr
                x[r, e] = y[i] if skip else x[r, e] + y[i]
    out = np.zeros(M)
    for r in range(n):
        c = (r + 1) % n
        out[cb[c]:cb[c + 1]] = x[r, cb[c]:cb[c + 1]]
    return out


@pytest.mark.parametrize("n,p", [(2, 0.5), (4, 0.3), (5, 0.9)])
def test_dropout_reduce_scatter_replays_algorithm1(n, p):
    rng = np.random.default_rng(n)
    M = 7 * n + 3
    bufs = rng.standard_normal((n, M)).astype(np.float32)
    out, _, cnt = oracle.dropout_reduce_scatter(bufs, p, 17, mode=0)
    assert np.allclose(out, _replay_alg1(bufs, p, 17), rtol=1e-12, atol=1e-12)
    assert cnt.min() >= 1 and cnt.max() <= n


def test_dropout_reduce_scatter_limits_and_rate():
    n, M = 8, 50000
    bufs = gen.dense_normal(9, n, M)
    full = bufs.astype(np.float64).sum(0)
    out, _, cnt = oracle.dropout_reduce_scatter(bufs, 0.0, 3, mode=1)
    assert np.allclose(out, full, rtol=1e-12, atol=1e-12) and np.all(cnt == n)
    out, _, cnt = oracle.dropout_reduce_scatter(bufs, 1.0, 3, mode=1)
    own = np.concatenate([bufs[j, (M * j) // n:(M * (j + 1)) // n] for j in range(n)]).astype(np.float64)
    assert np.all(cnt == 1) and np.allclose(out, own * n, rtol=1e-12, atol=1e-12)
    _, _, cnt = oracle.dropout_reduce_scatter(bufs, 0.25, 4, mode=1)
    mean = cnt.mean()  # 1 + Binomial(n-1, 0.75)
    assert abs(mean - (1 + (n - 1) * 0.75)) < 5 * math.sqrt((n - 1) * 0.75 * 0.25 / M)


def test_selective_reduce_scatter_is_per_bucket_skipreduce():
    n, M, sl = 4, 3001, 32
    bufs = gen.dense_normal(10, n, M)
    # one bucket: plain seeded SkipReduce
    a, _ = oracle.selective_reduce_scatter(bufs, [0, M], [0.5], 7, sl)
    b, _, _ = oracle.skip_reduce_scatter(bufs, sl, 0.5, 7, mode=1)
    assert np.array_equal(a, b)
    # buckets: each one a tensor of its own, with its own rate and seed + b
    bo = [0, 1000, 1000, 2500, M]
    ps = [0.0, 0.9, 0.5, 0.25]
    out, _ = oracle.selective_reduce_scatter(bufs, bo, ps, 7, sl)
    for b_, (lo, hi) in enumerate(zip(bo[:-1], bo[1:])):
        if hi == lo:
            continue
        want, _, _ = oracle.skip_reduce_scatter(np.ascontiguousarray(bufs[:, lo:hi]), sl, ps[b_], 7 + b_, mode=1)
        assert np.array_equal(out[lo:hi], want)
    assert np.allclose(out[:1000], bufs[:, :1000].astype(np.float64).sum(0), rtol=1e-12, atol=1e-12)


def test_allgather_copies_the_reduced_chunks():
    n, M = 5, 103
    rng = np.random.default_rng(3)
    bufs = rng.standard_normal((n, M)).astype(np.float32)
    red = rng.standard_normal(M)
    out = oracle.allgather(red, bufs)
    assert np.array_equal(out, np.tile(red, (n, 1)))
    # the ring's broadcast phase replayed: holder j-1 sends, position u receives at step u
    inc = (rng.random((n, n)) < 0.6).astype(np.uint8)
    out = oracle.allgather(red, bufs, inc)
    cb = [(M * j) // n for j in range(n + 1)]
    for j in range(n):
        for u in range(n):
            r = (j + u) % n
            got = u == n - 1 or inc[j, u]
            want = red[cb[j]:cb[j + 1]] if got else bufs[r, cb[j]:cb[j + 1]].astype(np.float64)
            assert np.array_equal(out[r, cb[j]:cb[j + 1]], want)


# ---------------------------------------------------------------------------
# DGC with a sampled global threshold and residuals (Zen section 4; Skip
# section 2): pins written from the definition with numpy, not the oracle
# ---------------------------------------------------------------------------

def _dgc_reference(grad, resid, density, S):
    """The definition in numpy float32: accumulate, sample, pool, threshold,
    select, update the residual."""
    n, M = grad.shape
    a = (resid.astype(np.float32) + grad.astype(np.float32)).astype(np.float32)
    keys = a.view(np.uint32) & np.uint32(0x7FFFFFFF)
    S = min(S, M)
    if S >= M:
        pos = np.arange(M)
    else:
        pos = np.array([((2 * j + 1) * M) // (2 * S) for j in range(S)], dtype=np.int64)
    pool = np.sort(keys[:, pos].reshape(-1))[::-1]
    ks = math.ceil(density * float(n * S))
    ks = min(max(ks, 1), n * S)
    thr = int(pool[ks - 1])
    sel = keys >= thr
    new_resid = np.where(sel, np.float32(0.0), a).astype(np.float32)
    return a, sel, thr, new_resid


@pytest.mark.parametrize("n,M,S,density", [(3, 1000, 1000, 0.05), (2, 777, 777, 0.3), (4, 5000, 5000, 0.01)])
def test_dgc_full_sample_is_exact_global_topk(n, M, S, density):
    rng = np.random.default_rng(n * 7 + M)
    g = rng.standard_normal((n, M)).astype(np.float32)
    r = (rng.standard_normal((n, M)) * 0.1).astype(np.float32)
    idx, val, cnt, new_r, thr = oracle.dgc_select(g, r, density, S)
    a, sel, thr_ref, r_ref = _dgc_reference(g, r, density, S)
    assert thr == thr_ref
    # with every element sampled, the threshold is the ks-th largest of all
    # n*M magnitudes: exactly ks are selected when magnitudes are distinct
    keys = (a.view(np.uint32) & np.uint32(0x7FFFFFFF)).reshape(-1)
    if np.unique(keys).size == keys.size:
        assert int(cnt.sum()) == min(max(math.ceil(density * float(n * M)), 1), n * M)
    for w in range(n):
        want = np.flatnonzero(sel[w])
        assert int(cnt[w]) == want.size
        assert np.array_equal(idx[w, : want.size], want)
        assert np.array_equal(val[w, : want.size].view(np.uint32), a[w, want].view(np.uint32))
    assert np.array_equal(new_r.view(np.uint32), r_ref.view(np.uint32))


@pytest.mark.parametrize("S", [1, 7, 64, 1000])
def test_dgc_sampled_threshold_is_the_pooled_order_statistic(S):
    rng = np.random.default_rng(S)
    n, M = 4, 3001
    g = (rng.standard_normal((n, M)) * np.exp(rng.standard_normal((n, 1)))).astype(np.float32)
    r = np.zeros((n, M), np.float32)
    for density in (0.0, 0.05, 0.5, 1.0, 2.0):
        idx, val, cnt, new_r, thr = oracle.dgc_select(g, r, density, S)
        a, sel, thr_ref, r_ref = _dgc_reference(g, r, density, S)
        assert thr == thr_ref, density
        assert np.array_equal(cnt, sel.sum(axis=1).astype(np.uint64))
        assert np.array_equal(new_r.view(np.uint32), r_ref.view(np.uint32))
    # density 0 keeps only magnitudes at or above the largest sample; density
    # >= 1 takes the smallest sample as the threshold
    _, _, _, _, thr_hi = oracle.dgc_select(g, r, 0.0, S)
    _, _, _, _, thr_lo = oracle.dgc_select(g, r, 1.0, S)
    pos = [oracle.dgc_sample_pos(M, min(S, M), j) for j in range(min(S, M))]
    smp = (g[:, pos].view(np.uint32) & np.uint32(0x7FFFFFFF))
    assert thr_hi == int(smp.max()) and thr_lo == int(smp.min())


def test_dgc_residuals_conserve_the_gradient():
    # after one gradient and then zero gradients, every nonzero element
    # leaves through exactly one emission carrying its accumulated value (a
    # threshold of 0 also re-takes elements already at 0, adding nothing),
    # and the residual drains: once most samples are 0 the threshold is 0
    rng = np.random.default_rng(11)
    n, M = 3, 4096
    g0 = rng.standard_normal((n, M)).astype(np.float32)
    r = np.zeros((n, M), np.float32)
    nonzero_emits = np.zeros((n, M), dtype=np.int64)
    total = np.zeros((n, M), dtype=np.float64)
    g = g0
    for it in range(200):
        idx, val, cnt, r, thr = oracle.dgc_select(g, r, 0.05, 512)
        for w in range(n):
            c = int(cnt[w])
            nonzero_emits[w, idx[w, :c]] += val[w, :c] != 0
            total[w, idx[w, :c]] += val[w, :c].astype(np.float64)
        g = np.zeros_like(g0)
        if not r.any():
            break
    assert not r.any(), "the residual did not drain"
    assert nonzero_emits.max() <= 1
    assert np.array_equal(total, g0.astype(np.float64))


def test_dgc_selected_fraction_tracks_density():
    # a strided sample of N(0,1) values puts the threshold near the
    # (1 - density) quantile: the selected fraction is close to the density
    rng = np.random.default_rng(5)
    n, M = 4, 1 << 16
    g = rng.standard_normal((n, M)).astype(np.float32)
    _, _, cnt, _, _ = oracle.dgc_select(g, np.zeros_like(g), 0.05, 4096, cap=0)
    frac = cnt.sum() / (n * M)
    assert abs(frac - 0.05) < 0.005, frac


def test_dgc_sample_positions_and_rank():
    assert [oracle.dgc_sample_pos(10, 4, j) for j in range(4)] == [1, 3, 6, 8]
    assert [oracle.dgc_sample_pos(5, 9, j) for j in range(5)] == [0, 1, 2, 3, 4]
    assert oracle.dgc_rank(0.05, 100) == 5 and oracle.dgc_rank(0.051, 100) == 6
    assert oracle.dgc_rank(0.0, 100) == 1 and oracle.dgc_rank(3.0, 100) == 100


# ---------------------------------------------------------------------------
# Algorithm 1 (Zen section 3.2): hierarchical hash memory
# ---------------------------------------------------------------------------

def _alg1_python(idx, in_off, P, seed, k, r1, r2):
    """Algorithm 1 written again in plain Python (sequential, input order),
    with the hashes from MurmurHash2 (pinned by its published check value)."""
    n = len(in_off) - 1
    out, slots, counts = [], [], []
    for w in range(n):
        R = r1 + r2
        x = [[0] * R for _ in range(P)]
        c = [r1] * P
        serial = lost = 0
        for e in range(int(in_off[w]), int(in_off[w + 1])):
            i_ = int(idx[e])
            b = struct.pack("<I", i_)
            p = oracle.murmur2(b, seed) % P
            placed = False
            for i in range(1, k + 1):
                q = oracle.murmur2(b, seed + i) % r1
                if x[p][q] == 0:
                    x[p][q] = e - int(in_off[w]) + 1
                    placed = True
                    break
            if not placed:
                serial += 1
                q = c[p]
                c[p] += 1
                if q < R:
                    x[p][q] = e - int(in_off[w]) + 1
                else:
                    lost += 1
        for p in range(P):
            for q in range(R):
                if x[p][q]:
                    out.append(int(idx[int(in_off[w]) + x[p][q] - 1]))
                    slots.append(q)
        counts.append((serial, lost))
    return out, slots, counts


@pytest.mark.parametrize("k,r1,r2", [(1, 16, 64), (2, 8, 8), (4, 40, 4), (3, 5, 0)])
def test_alg1_matches_a_plain_python_replay(k, r1, r2):
    rng = np.random.default_rng(k * 100 + r1)
    lists = [np.sort(rng.choice(5000, size=s, replace=False)).astype(np.uint32) for s in (60, 0, 37)]
    idx, in_off, val = gen.coo_from_lists(lists, [l.astype(np.float32) for l in lists])
    oi, ov, po, so, cnt = oracle.hierarchical_hash(idx, val, in_off, 4, 21, k, r1, r2)
    want, wslots, wcnt = _alg1_python(idx, in_off, 4, 21, k, r1, r2)
    # a worker's output starts at its input offset; lost entries leave a gap
    got = np.concatenate([oi[int(po[w, 0]):int(po[w, -1])] for w in range(po.shape[0])])
    gslots = np.concatenate([so[int(po[w, 0]):int(po[w, -1])] for w in range(po.shape[0])])
    gval = np.concatenate([ov[int(po[w, 0]):int(po[w, -1])] for w in range(po.shape[0])])
    assert list(got) == want and list(gslots) == wslots
    assert [tuple(int(v) for v in r) for r in cnt] == wcnt
    assert np.array_equal(gval, got.astype(np.float32))  # values follow their index


def test_alg1_membership_is_the_hash_partition():
    # with room in the serial memory nothing is lost, and every partition
    # holds exactly the entries that the stable grouping by h0 puts there
    idx, in_off, val = gen.coo_zipf(77, 5, 300000, 4000, 1.1)
    P, seed = 8, 3
    oi, ov, po, so, cnt = oracle.hierarchical_hash(idx, val, in_off, P, seed, 2, 600, 600)
    assert cnt[:, 1].sum() == 0
    hi, hv, hpo = oracle.hash_partition(idx, val, in_off, P, seed)
    assert np.array_equal(po, hpo)
    for w in range(5):
        for p in range(P):
            a, b = int(po[w, p]), int(po[w, p + 1])
            order = np.argsort(oi[a:b], kind="stable")
            assert np.array_equal(oi[a:b][order], hi[a:b])
            assert np.array_equal(ov[a:b][order], hv[a:b])


def test_alg1_losses_and_rehash_collision_rate():
    rng = np.random.default_rng(1)
    lst = np.sort(rng.choice(1 << 22, size=40000, replace=False)).astype(np.uint32)
    idx, in_off, val = gen.coo_from_lists([lst], [lst.astype(np.float32)])
    P = 16
    # no serial memory, one hash: whatever collides is lost, and the rest
    # is kept
    oi, _, po, so, cnt = oracle.hierarchical_hash(idx, val, in_off, P, 9, 1, 40000 // P, 0)
    assert int(cnt[0, 1]) == int(cnt[0, 0]) and int(po[0, -1]) == 40000 - int(cnt[0, 1])
    # parallel memory four times the nonzeros and four hashes: under 1% of
    # the entries reach the serial memory (the page reports < 1% with four
    # hash functions)
    _, _, _, _, cnt4 = oracle.hierarchical_hash(idx, val, in_off, P, 9, 4, 4 * 40000 // P, 4000)
    assert cnt4[0, 1] == 0 and cnt4[0, 0] < 0.01 * 40000
    # more hash functions never put more entries into the serial memory here
    serial = [int(oracle.hierarchical_hash(idx, val, in_off, P, 9, kk, 2 * 40000 // P, 40000)[4][0, 0])
              for kk in (1, 2, 3, 4)]
    assert serial == sorted(serial, reverse=True), serial

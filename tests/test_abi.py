"""The C ABI of libsg without a GPU: the library loads, exports every function
include/sg.h declares with the arity the Python binding marshals, its pure
host functions (sizes, slice counts) follow their documented formulas, and
every host-checkable bad argument is refused with the documented status before
any launch.  No call here reaches the device: each one either returns from its
host checks or is a size query.
"""
import ctypes as C
import os
import re
import subprocess

import pytest

import sparse_gradient_synchronization_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sg.h")

SG_OK, SG_EINVAL, SG_ECAPACITY, SG_EUNSORTED, SG_EHIP, SG_EUNSUPPORTED, SG_ERANGE, SG_EDEVICE = 0, -1, -2, -3, -4, -5, -6, -7


def _header_prototypes():
    """{name: number of parameters} for every function prototype in sg.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"typedef\s+(enum|struct)\s+\w+\s*\{.*?\}\s*\w+\s*;", " ", text, flags=re.S)
    protos = {}
    for m in re.finditer(r"([A-Za-z_][\w\s\*]*?)\b(sg_\w+)\s*\(([^)]*)\)\s*;", text):
        params = m.group(3).strip()
        nparams = 0 if params in ("", "void") else params.count(",") + 1
        protos[m.group(2)] = nparams
    return protos


@pytest.fixture(scope="module")
def L():
    return sg.lib()


F = C.c_void_p(0x10000)  # a non-null pointer that no host check dereferences
N = None


def test_header_parses():
    protos = _header_prototypes()
    for name in ("sg_topk_to_coo", "sg_hash_partition", "sg_aggregate", "sg_classmap_build", "sg_encode",
                 "sg_skip_reduce_scatter", "sg_stats", "sg_validate_coo", "sg_probe_set"):
        assert name in protos


def test_every_declared_symbol_is_exported(L):
    protos = _header_prototypes()
    missing = [name for name in protos if not hasattr(L, name)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH], capture_output=True, text=True, check=True).stdout
    dynsyms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(protos) <= dynsyms, sorted(set(protos) - dynsyms)


def test_binding_matches_header_arity():
    protos = _header_prototypes()
    assert set(sg.SIGNATURES) == set(protos)
    for name, nparams in protos.items():
        assert len(sg.SIGNATURES[name][1]) == nparams, name


def test_no_undeclared_sg_exports():
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip() and line.split()[-1].startswith("sg_")}
    assert exported == set(_header_prototypes())


def test_strerror_total(L):
    for code in range(-10, 3):
        s = L.sg_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert L.sg_strerror(SG_OK) == b"ok"
    assert L.sg_strerror(99) == b"unknown status"


def test_skip_num_slices_formula(L):
    # S = ceil(ceil(M / n) / slice_elems)
    for n in (1, 2, 3, 8, 64):
        for M in (1, 7, 1000, 1 << 20, (1 << 26) + 5):
            for sb, esz, dt in ((4, 4, 0), (256 * 1024, 4, 0), (6, 2, 1), (1 << 18, 2, 1)):
                e = sb // esz
                want = -(-(-(-M // n)) // e)
                assert L.sg_skip_num_slices(n, M, sb, dt) == want


def test_encode_words_cover_every_class(L):
    # the bitmap of class p takes ceil(|C_p| / 32) words; the total never
    # exceeds M/32 + P + 1 whatever the class sizes are
    for M in (1, 31, 32, 33, 1000, 1 << 20):
        for P in (1, 2, 7, 16, 256):
            assert L.sg_encode_max_words(M, P) * 32 >= M + 31 * P
    # one 8-byte cursor per (key window, partition), windows of at most 4096 keys
    assert L.sg_encode_workspace_bytes(1 << 20, 8) >= 8 * 8 * ((1 << 20) // 4096 + 1)


def test_workspace_sizes_monotone(L):
    a = L.sg_topk_workspace_bytes(8, 1 << 20, 1 << 14, 0)
    b = L.sg_topk_workspace_bytes(8, 1 << 22, 1 << 16, 0)
    assert 0 < a <= b
    assert L.sg_partition_workspace_bytes(4, 1000, 8) <= L.sg_partition_workspace_bytes(4, 100000, 8)
    assert L.sg_aggregate_workspace_bytes(4, 8, 1 << 20, 1000, 1) <= L.sg_aggregate_workspace_bytes(4, 8, 1 << 20, 100000, 1)
    assert L.sg_stats_workspace_bytes(4, 1 << 20, 1000, 8) > 0
    assert L.sg_classmap_bytes(1 << 20, 8) >= (1 << 20) // 8  # at least a few bits of class id per key
    assert L.sg_validate_workspace_bytes() >= 16


def test_topk_host_checks(L):
    ws = L.sg_topk_workspace_bytes(4, 1024, 10, 0)
    assert L.sg_topk_to_coo(N, 0, 4, 1024, 10, F, F, F, ws, N) == SG_EINVAL      # null input
    assert L.sg_topk_to_coo(F, 0, 4, 1024, 1025, F, F, F, ws, N) == SG_EINVAL    # k > M
    assert L.sg_topk_to_coo(F, 0, 0, 1024, 10, F, F, F, ws, N) == SG_EINVAL      # n = 0
    assert L.sg_topk_to_coo(F, 7, 4, 1024, 10, F, F, F, ws, N) == SG_EINVAL      # dtype
    assert L.sg_topk_to_coo(F, 0, 4, 1 << 32, 10, F, F, F, 1 << 40, N) == SG_EINVAL  # M >= 2^32
    assert L.sg_topk_to_coo(F, 0, 4, 1024, 10, F, F, F, ws - 1, N) == SG_ECAPACITY


def test_partition_host_checks(L):
    ws = L.sg_partition_workspace_bytes(4, 100, 8)
    assert L.sg_hash_partition(F, F, 0, 1, F, 4, 100, 0, 1, F, F, F, F, ws, N) == SG_EINVAL     # P = 0
    assert L.sg_hash_partition(F, F, 0, 1, F, 4, 100, 257, 1, F, F, F, F, 1 << 30, N) == SG_EINVAL  # P > 256
    assert L.sg_hash_partition(F, N, 0, 1, F, 4, 100, 8, 1, F, F, F, F, ws, N) == SG_EINVAL     # D > 0, no values
    assert L.sg_hash_partition(F, F, 0, 1, N, 4, 100, 8, 1, F, F, F, F, ws, N) == SG_EINVAL     # no offsets
    assert L.sg_hash_partition(F, F, 0, 1, F, 4, 100, 8, 1, F, F, F, F, ws - 1, N) == SG_ECAPACITY


def test_partition_noalloc_host_checks(L):
    f = L.sg_hash_partition_noalloc
    assert f(F, F, 0, 1, F, 4, 100, 0, 1, F, F, F, N) == SG_EINVAL      # P = 0
    assert f(F, F, 0, 1, F, 4, 100, 257, 1, F, F, F, N) == SG_EINVAL    # P > 256
    assert f(F, N, 0, 1, F, 4, 100, 8, 1, F, F, F, N) == SG_EINVAL      # D > 0, no values
    assert f(F, F, 0, 1, N, 4, 100, 8, 1, F, F, F, N) == SG_EINVAL      # no offsets
    assert f(F, F, 0, 1, F, 4, 1 << 32, 8, 1, F, F, F, N) == SG_EUNSUPPORTED
    # beyond the fixed scratch: counts of 2^31 entries over 256 partitions,
    # or the sources of 2^23 rows
    assert f(F, F, 0, 1, F, 1, 1 << 31, 256, 1, F, F, F, N) == SG_ECAPACITY
    assert f(F, F, 0, 2, F, 1, 1 << 23, 4, 1, F, F, F, N) == SG_ECAPACITY


def test_aggregate_host_checks(L):
    ws = L.sg_aggregate_workspace_bytes(4, 8, 1 << 20, 100, 1)
    assert L.sg_aggregate(F, F, 0, 1, F, 65, 8, 1 << 20, 100, F, F, 100, F, F, 1 << 30, N) == SG_EINVAL  # n > 64
    assert L.sg_aggregate(F, F, 0, 1, F, 4, 0, 1 << 20, 100, F, F, 100, F, F, 1 << 30, N) == SG_EINVAL   # P = 0
    assert L.sg_aggregate(F, F, 0, 1, F, 4, 8, 1 << 20, 100, F, F, 99, F, F, ws, N) == SG_ECAPACITY     # capacity < total
    assert L.sg_aggregate(F, F, 0, 1, F, 4, 8, 1 << 20, 100, F, F, 100, F, F, ws - 1, N) == SG_ECAPACITY
    assert L.sg_aggregate(F, F, 0, 1, N, 4, 8, 1 << 20, 100, F, F, 100, F, F, ws, N) == SG_EINVAL      # no offsets


def test_encode_host_checks(L):
    M, P = 1 << 20, 8
    cb, mw = L.sg_classmap_bytes(M, P), L.sg_encode_max_words(M, P)
    assert L.sg_classmap_build(M, P, 1, F, cb - 1, N) == SG_ECAPACITY
    assert L.sg_classmap_build(M, 0, 1, F, cb, N) == SG_EINVAL
    assert L.sg_classmap_build(1 << 32, P, 1, F, 1 << 40, N) == SG_EINVAL
    ew = L.sg_encode_workspace_bytes(M, P)
    assert L.sg_encode(F, F, 100, M, P, F, cb, F, mw - 1, F, F, ew, N) == SG_ECAPACITY
    assert L.sg_encode(F, F, 100, M, P, F, cb - 1, F, mw, F, F, ew, N) == SG_ECAPACITY
    assert L.sg_encode(F, F, 100, M, P, F, cb, F, mw, F, F, ew - 1, N) == SG_ECAPACITY
    assert L.sg_encode(F, F, 100, M, P, N, cb, F, mw, F, F, ew, N) == SG_EINVAL
    assert L.sg_encode(F, F, 100, M, P, F, cb, F, mw, F, N, ew, N) == SG_EINVAL
    assert L.sg_encode(F, F, 100, M, 257, F, 1 << 40, F, 1 << 40, F, F, 1 << 40, N) == SG_EINVAL


def test_skip_rs_host_checks(L):
    assert L.sg_skip_reduce_scatter(F, 0, 4, 1024, 64, 1.5, 1, N, 0, F, N, N) == SG_EINVAL   # p > 1
    assert L.sg_skip_reduce_scatter(F, 0, 4, 1024, 64, -0.1, 1, N, 0, F, N, N) == SG_EINVAL  # p < 0
    assert L.sg_skip_reduce_scatter(F, 0, 4, 1024, 66, 0.5, 1, N, 0, F, N, N) == SG_EINVAL   # slice % 4
    assert L.sg_skip_reduce_scatter(F, 0, 65, 1024, 64, 0.5, 1, N, 0, F, N, N) == SG_EINVAL  # n > 64
    assert L.sg_skip_reduce_scatter(F, 0, 4, 1024, 64, 0.5, 1, N, 5, F, N, N) == SG_EINVAL   # mode
    assert L.sg_skip_reduce_scatter(F, 0, 4, 1024, 64, 0.5, 1, N, 0, N, N, N) == SG_EINVAL   # no output
    assert L.sg_skip_reduce_scatter(F, 0, 4, 1024, 0, 0.5, 1, N, 0, F, N, N) == SG_EINVAL    # slice 0


def test_stats_host_checks(L):
    n, P = 4, 8
    ws = L.sg_stats_workspace_bytes(n, 1 << 20, 100, P)
    out = sg.StatsOut()
    assert L.sg_stats(F, F, n, 1 << 20, 100, P, N, 0, None, F, ws, N) == SG_EINVAL          # no output struct
    assert L.sg_stats(F, F, n, 1 << 20, 100, P, N, 0, C.byref(out), F, ws, N) == SG_EINVAL  # no host arrays
    keep = []
    for field, count, ctype in (("nnz", n, C.c_uint64), ("inter", n * n, C.c_uint64), ("overlap", n * n, C.c_double),
                                ("contig_counts", (n + 1) * P, C.c_uint64), ("skew_contig", n + 1, C.c_double)):
        arr = (ctype * count)()
        keep.append(arr)
        setattr(out, field, C.cast(arr, C.c_void_p))
    assert L.sg_stats(F, F, 65, 1 << 20, 100, P, N, 0, C.byref(out), F, 1 << 30, N) == SG_EINVAL  # n > 64
    assert L.sg_stats(F, F, n, 1 << 20, 100, P, F, 1 << 30, C.byref(out), F, ws, N) == SG_EINVAL  # class map, no hashed arrays
    assert L.sg_stats(F, F, n, 1 << 20, 100, P, N, 0, C.byref(out), F, ws - 1, N) == SG_ECAPACITY


def test_probe_and_validate_host_checks(L):
    assert L.sg_probe_set(99, N, N) == SG_EINVAL
    assert L.sg_probe_set(1, N, N) == SG_EINVAL
    assert L.sg_probe_set(0, N, N) == SG_OK
    assert L.sg_validate_coo(F, N, 4, 100, 100, F, 256, N) == SG_EINVAL
    assert L.sg_validate_coo(F, F, 4, 100, 100, F, L.sg_validate_workspace_bytes() - 1, N) == SG_ECAPACITY


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 16)
    with pytest.raises((ValueError, RuntimeError)):
        sg.sg_topk_to_coo(x, 2)


def test_pull_side_host_checks(L):
    M, P = 1 << 20, 8
    cb = L.sg_classmap_bytes(M, P)
    dw = L.sg_decode_workspace_bytes(M, P)
    assert dw > 0
    assert L.sg_decode(F, 100, F, cb, M, P, F, 10, F, F, dw - 1, N) == SG_ECAPACITY
    assert L.sg_decode(F, 100, F, cb - 1, M, P, F, 10, F, F, dw, N) == SG_ECAPACITY
    assert L.sg_decode(N, 100, F, cb, M, P, F, 10, F, F, dw, N) == SG_EINVAL
    assert L.sg_decode(F, 100, F, cb, M, 0, F, 10, F, F, dw, N) == SG_EINVAL
    sw = L.sg_scatter_dense_workspace_bytes(M, P)
    assert sw > 0 and L.sg_scatter_dense_workspace_bytes(M, 257) == 0
    assert L.sg_scatter_dense(F, F, 1, F, P, 10, 0, F, F, sw, N) == SG_EINVAL            # M = 0
    assert L.sg_scatter_dense(F, F, 1, N, P, 10, M, F, F, sw, N) == SG_EINVAL            # no offsets
    assert L.sg_scatter_dense(F, F, 1, F, P, 10, M, C.c_void_p(0x10004), F, sw, N) == SG_EINVAL  # misaligned dense
    assert L.sg_scatter_dense(F, F, 1, F, P, 10, M, F, N, sw, N) == SG_EINVAL            # no workspace
    assert L.sg_scatter_dense(F, F, 1, F, P, 10, M, F, F, sw - 1, N) == SG_ECAPACITY     # workspace too small
    assert L.sg_scatter_dense(F, F, 1, F, 257, 10, M, F, F, sw, N) == SG_EINVAL          # P > 256
    fw = L.sg_format_sizes_workspace_bytes(M)
    out = (C.c_uint64 * 7)()
    assert L.sg_format_sizes(F, F, 10, M, P, 1, F, cb, C.cast(out, C.c_void_p), F, fw - 1, N) == SG_ECAPACITY
    assert L.sg_format_sizes(F, F, 10, M, P, 1, F, cb, None, F, fw, N) == SG_EINVAL
    assert L.sg_format_sizes(F, F, 10, M, P, 1, F, cb - 1, C.cast(out, C.c_void_p), F, fw, N) == SG_ECAPACITY


def test_skip_family_host_checks(L):
    # SkipReduce(k): k > n refused; the other checks are those of the seeded call
    assert L.sg_skip_reduce_k(F, 0, 4, 1024, 64, 5, 0, 1, 0, F, N, N) == SG_EINVAL     # k > n
    assert L.sg_skip_reduce_k(F, 0, 4, 1024, 66, 2, 0, 1, 0, F, N, N) == SG_EINVAL     # slice % 4
    assert L.sg_skip_reduce_k(F, 0, 0, 1024, 64, 0, 0, 1, 0, F, N, N) == SG_EINVAL     # n = 0
    assert L.sg_skip_reduce_k(N, 0, 4, 1024, 64, 2, 1, 1, 0, F, N, N) == SG_EINVAL     # no input
    assert L.sg_skip_reduce_k(F, 0, 4, 0, 64, 2, 1, 1, 0, F, N, N) == SG_OK            # M = 0: nothing to do
    # selective: offsets must be non-decreasing and within M, rates within [0, 1]
    off = (C.c_uint64 * 3)(0, 512, 1024)
    bad_off = (C.c_uint64 * 3)(0, 600, 512)
    big_off = (C.c_uint64 * 3)(0, 512, 1025)
    rates = (C.c_double * 2)(0.5, 0.25)
    bad_rates = (C.c_double * 2)(0.5, 1.25)
    vp = lambda a: C.cast(a, C.c_void_p)  # noqa: E731
    assert L.sg_selective_reduce_scatter(F, 0, 4, 1024, 2, vp(bad_off), vp(rates), 64, 1, 0, F, N) == SG_EINVAL
    assert L.sg_selective_reduce_scatter(F, 0, 4, 1024, 2, vp(big_off), vp(rates), 64, 1, 0, F, N) == SG_EINVAL
    assert L.sg_selective_reduce_scatter(F, 0, 4, 1024, 2, vp(off), vp(bad_rates), 64, 1, 0, F, N) == SG_EINVAL
    assert L.sg_selective_reduce_scatter(F, 0, 4, 1024, 0, vp(off), vp(rates), 64, 1, 0, F, N) == SG_EINVAL
    assert L.sg_selective_reduce_scatter(F, 0, 4, 1024, 2, N, vp(rates), 64, 1, 0, F, N) == SG_EINVAL
    # dropout and all-gather
    assert L.sg_dropout_reduce_scatter(F, 0, 4, 1024, 1.5, 1, 0, F, N, N) == SG_EINVAL
    assert L.sg_dropout_reduce_scatter(F, 0, 65, 1024, 0.5, 1, 0, F, N, N) == SG_EINVAL
    assert L.sg_dropout_reduce_scatter(F, 0, 4, 1024, 0.5, 1, 3, F, N, N) == SG_EINVAL
    assert L.sg_dropout_reduce_scatter(F, 0, 4, 1024, 0.5, 1, 0, N, N, N) == SG_EINVAL
    assert L.sg_allgather(N, F, 0, 4, 1024, N, F, N) == SG_EINVAL
    assert L.sg_allgather(F, N, 0, 4, 1024, F, F, N) == SG_EINVAL   # a delivery mask needs the local buffers
    assert L.sg_allgather(F, F, 2, 4, 1024, N, F, N) == SG_EINVAL   # dtype


def test_random_offset_matches_the_oracle_mask(L):
    # Random SkipReduce: the library's shared offset, applied to the static
    # mask, gives the oracle's mask for the same seed
    import numpy as np
    import oracle
    for n in (1, 2, 3, 8, 13, 64):
        for seed in (0, 1, 5, 12345, 2**63 + 7):
            off = L.sg_skip_random_offset(n, seed)
            assert 0 <= off < n
            S = 3
            for k in (0, n // 2, n):
                want = oracle.skip_mask_random(n, S, k, seed)
                t = np.arange(n)
                got = np.broadcast_to((((t + off) % n) >= k)[None, :, None], (n, n, S)).astype(np.uint8)
                assert np.array_equal(got, want)

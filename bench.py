#!/usr/bin/env python3
"""Benchmark of the sparse gradient synchronization hot path on one MI355X.

One step = one pass of every stage of the path over one batch of synthetic
input already resident in HBM.  The headline workload "dgc-top5": n=8
workers, dense fp32 gradients of 4096 x 11008 each (per-row lognormal scale,
0.7 inter-worker correlation),
    A1 top-5% per worker into COO            sg_topk_to_coo
    A2 hash partition into 8                  sg_hash_partition
    A3 per-partition union-sum                sg_aggregate
    A4 hash-bitmap encode                     sg_encode
    A6 overlap / densification / skew stats   sg_stats_async (queued)
    A5 the dense counterpart on the same gradients: ring reduce-scatter
       arithmetic, 256 KiB slices skipped w.p. 0.5, DropReduce rescale
                                              sg_skip_reduce_scatter
    A6 the statistics evaluated on the host   sg_stats_collect

The other workloads run the stages that apply to them, each measured the
same way and reported under "configs":
    cfg1  n=4, dense M=2^20 with 1% Zipf(1.1) nonzeros: A1 (k = nnz), A2-A4, A6
    cfg2  embedding rows 1,000,000 x 64, n=8, 4096 Zipf(1.05) rows: A2-A4, A6
    cfg4  n=16, M=2^28, 1% per worker, 60% in the first M/8: A2-A4, A6
    cfg5  n=8 buffers of 2^26 fp32, 256 KiB slices, p=0.5: A5

Metric: aggregated input nonzeros per second (the COO entries that enter
aggregation, divided by the step time; elements per second for cfg5), plus
the HBM roofline of the step's dominant kernel timed with HIP events on the
stream it runs on, and every stage's and kernel's fraction of HBM peak from
its algorithmic bytes.

After the timed steps the outputs of the last step are compared with the
oracle's outputs for the same inputs (bit-exact indices, offsets, bitmaps,
counts and statistics; fp32 sums within 1e-6 * sum|x| + 1e-30), and the
oracle's step is timed single-threaded on the host ("cpu_baseline").  A
parity failure is reported in the line and makes the exit status 3.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import ctypes as C
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak

METRIC = "aggregated input nonzeros/sec + achieved HBM GB/s (% of MI355X peak), 1 GPU"
WORKLOADS = ("dgc-top5", "cfg1", "cfg2", "cfg4", "cfg5")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Two raw HIP events (the probe hook of libsg records them around one
    kernel inside a multi-kernel call)."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        self.start = C.c_void_p()
        self.stop = C.c_void_p()
        assert self.hip.hipEventCreate(C.byref(self.start)) == 0
        assert self.hip.hipEventCreate(C.byref(self.stop)) == 0

    def elapsed_ms(self):
        assert self.hip.hipEventSynchronize(self.stop) == 0
        ms = C.c_float()
        assert self.hip.hipEventElapsedTime(C.byref(ms), self.start, self.stop) == 0
        return float(ms.value)

    def __del__(self):
        try:
            self.hip.hipEventDestroy(self.start)
            self.hip.hipEventDestroy(self.stop)
        except Exception:
            pass


def build_workload(name, torch, sg, gen):
    """Inputs on the GPU, preallocated outputs/workspaces, and the stage list."""
    L = sg.lib()
    dev = torch.device("cuda", 0)
    u32 = lambda a: torch.from_numpy(a.view("int32")).to(dev)  # noqa: E731
    u64 = lambda a: torch.from_numpy(a.view("int64")).to(dev)  # noqa: E731
    W = {"name": name}
    out = {}  # device outputs of the last step, for the parity check
    W["out"] = out
    stages = []
    nbytes = {}

    def vp(t):
        return None if t is None else C.c_void_p(t.data_ptr())

    stream = lambda: C.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731

    def chk(rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with status %d" % (what, rc))

    import numpy as np

    if name in ("dgc-top5", "cfg1"):
        c = gen.config3() if name == "dgc-top5" else gen.config1()
        W["host"] = c
        n, M, k, P, seed = c["n"], c["M"], c["k"], c["P"], c["seed"]
        dense = torch.from_numpy(c["dense"]).to(dev)
        W.update(n=n, M=M, k=k, P=P)
        idx = torch.empty(n * k, dtype=torch.int32, device=dev)
        val = torch.empty(n * k, dtype=torch.float32, device=dev)
        ws_t = torch.empty(L.sg_topk_workspace_bytes(n, M, k, 0), dtype=torch.uint8, device=dev)
        in_off_np = np.arange(n + 1, dtype=np.uint64) * np.uint64(k)
        in_off = u64(in_off_np)
        total = n * k

        def topk():
            chk(L.sg_topk_to_coo(vp(dense), 0, n, M, k, vp(idx), vp(val), vp(ws_t), ws_t.numel(), stream()),
                "sg_topk_to_coo")
        stages.append(("topk_to_coo", topk))
        nbytes["topk_to_coo"] = n * M * 4 + n * k * 8
        src_idx, src_val, D = idx, val, 1
        out.update(topk_idx=idx, topk_val=val)
        W["in_off_host"] = in_off_np
    elif name in ("cfg2", "cfg4"):
        c = gen.config2() if name == "cfg2" else gen.config4()
        W["host"] = c
        W["in_off_host"] = c["in_off"]
        n, M, P, seed = c["n"], c["M"], c["P"], c["seed"]
        D = c.get("D", 1)
        src_idx = u32(c["idx"])
        src_val = torch.from_numpy(c["val"]).to(dev)
        in_off = u64(c["in_off"])
        total = int(c["in_off"][-1])
        W.update(n=n, M=M, P=P, D=D, total=total)
    elif name == "cfg5":
        c = gen.config5()
        W["host"] = c
        n, M = c["n"], c["M"]
        W.update(n=n, M=M, slice_bytes=c["slice_elems"] * 4, p_skip=c["p"])
        total = None
    else:
        raise SystemExit("unknown workload %s" % name)

    if name != "cfg5":
        pidx = torch.empty(total, dtype=torch.int32, device=dev)
        pval = torch.empty_like(src_val)
        part_off = torch.empty((n, P + 1), dtype=torch.int64, device=dev)
        ws_p = torch.empty(L.sg_partition_workspace_bytes(n, total, P), dtype=torch.uint8, device=dev)
        agg_idx = torch.empty(total, dtype=torch.int32, device=dev)
        agg_val = torch.empty((total, D) if D > 1 else (total,), dtype=torch.float32, device=dev)
        agg_off = torch.empty(P + 1, dtype=torch.int64, device=dev)
        ws_a = torch.empty(L.sg_aggregate_workspace_bytes(n, P, M, total, D), dtype=torch.uint8, device=dev)
        cmap = sg.sg_classmap_build(M, P, seed)
        words = L.sg_encode_max_words(M, P)
        bitmap = torch.empty(words, dtype=torch.int32, device=dev)
        word_off = torch.empty(P + 1, dtype=torch.int64, device=dev)
        ws_e = torch.empty(L.sg_encode_workspace_bytes(M, P), dtype=torch.uint8, device=dev)
        ws_s = torch.empty(L.sg_stats_workspace_bytes(n, M, total, P), dtype=torch.uint8, device=dev)
        st_arr = dict(
            nnz=np.zeros(n, np.uint64), inter=np.zeros(n * n, np.uint64), overlap=np.zeros(n * n, np.float64),
            contig_counts=np.zeros((n + 1) * P, np.uint64), skew_contig=np.zeros(n + 1, np.float64),
            class_size=np.zeros(P, np.uint64), hashed_counts=np.zeros((n + 1) * P, np.uint64),
            skew_hashed=np.zeros(n + 1, np.float64))
        so = sg.StatsOut()
        for key, a in st_arr.items():
            setattr(so, key, a.ctypes.data)
        W["stats_out"] = so
        W["stats_arrays"] = st_arr  # keeps the host arrays alive

        def part():
            chk(L.sg_hash_partition(vp(src_idx), vp(src_val), 0, D, vp(in_off), n, total, P, seed, vp(pidx), vp(pval),
                                    vp(part_off), vp(ws_p), ws_p.numel(), stream()), "sg_hash_partition")

        def agg():
            chk(L.sg_aggregate(vp(pidx), vp(pval), 0, D, vp(part_off), n, P, M, total, vp(agg_idx), vp(agg_val),
                               total, vp(agg_off), vp(ws_a), ws_a.numel(), stream()), "sg_aggregate")

        def enc():
            chk(L.sg_encode(vp(agg_idx), vp(agg_off), total, M, P, vp(cmap), cmap.numel(), vp(bitmap), words,
                            vp(word_off), vp(ws_e), ws_e.numel(), stream()), "sg_encode")

        # statistics in two halves: the passes and the copy of the raw counts
        # are queued, the skip reduce-scatter is queued behind them, and the
        # host evaluates the definitions once the copy is done
        st_block = torch.empty(L.sg_stats_block_bytes(n, P), dtype=torch.uint8, pin_memory=True)
        st_done = torch.cuda.Event()

        def stats():
            chk(L.sg_stats_async(vp(src_idx), vp(in_off), n, M, total, P, vp(cmap), cmap.numel(), vp(st_block),
                                 st_block.numel(), vp(ws_s), ws_s.numel(), stream()), "sg_stats_async")
            st_done.record()

        def stats_collect():
            st_done.synchronize()
            chk(L.sg_stats_collect(vp(st_block), n, M, total, P, 1, C.byref(so)), "sg_stats_collect")

        stages += [("hash_partition", part), ("aggregate", agg), ("encode", enc), ("stats", stats)]
        W["stats_collect"] = stats_collect
        W.update(seed=seed)
        out.update(pidx=pidx, pval=pval, part_off=part_off, agg_idx=agg_idx, agg_val=agg_val, agg_off=agg_off,
                   bitmap=bitmap, word_off=word_off)

        # the Pull side after the step (timed on its own, not part of the step)
        dec_idx = torch.empty(total, dtype=torch.int32, device=dev)
        dec_off = torch.empty(P + 1, dtype=torch.int64, device=dev)
        ws_d = torch.empty(max(L.sg_decode_workspace_bytes(M, P), 1), dtype=torch.uint8, device=dev)
        pull_dense = torch.empty((M, D) if D > 1 else (M,), dtype=torch.float32, device=dev)
        ws_f = torch.empty(L.sg_format_sizes_workspace_bytes(M), dtype=torch.uint8, device=dev)

        def dec():
            chk(L.sg_decode(vp(bitmap), words, vp(cmap), cmap.numel(), M, P, vp(dec_idx), total, vp(dec_off), vp(ws_d),
                            ws_d.numel(), stream()), "sg_decode")

        ws_sc = torch.empty(L.sg_scatter_dense_workspace_bytes(M, P), dtype=torch.uint8, device=dev)

        def scat():
            chk(L.sg_scatter_dense(vp(agg_idx), vp(agg_val), D, vp(agg_off), P, total, M, vp(pull_dense), vp(ws_sc),
                                   ws_sc.numel(), stream()), "sg_scatter_dense")

        def fmt():
            out = (C.c_uint64 * 7)()
            chk(L.sg_format_sizes(vp(agg_idx), vp(agg_off), total, M, P, D, vp(cmap), cmap.numel(),
                                  C.cast(out, C.c_void_p), vp(ws_f), ws_f.numel(), stream()), "sg_format_sizes")
            return dict(zip(sg.FORMAT_NAMES, (int(v) for v in out)))
        W["pull"] = [("decode", dec), ("scatter_dense", scat)]
        W["format_sizes"] = fmt
        esz = 4 * D
        nbytes["hash_partition"] = 2 * total * (4 + esz)
        W["agg_off"] = agg_off
        W["word_off"] = word_off
        W["bytes_agg"] = lambda U: total * (4 + esz) + U * (4 + 4 * D)  # noqa: E731
        W["bytes_enc"] = lambda U, words_: U * 4 + words_ * 4  # noqa: E731
        W["nnz"] = total

    if name in ("dgc-top5", "cfg5"):
        bufs = dense if name == "dgc-top5" else torch.from_numpy(c["bufs"]).to(dev)
        W["bufs"] = bufs
        if name == "dgc-top5":
            W["dense"] = dense
        slice_bytes = 256 * 1024
        S = L.sg_skip_num_slices(n, M, slice_bytes, 0)
        rs_out = torch.empty(M, dtype=torch.float32, device=dev)
        rs_cnt = torch.empty((n, S), dtype=torch.uint8, device=dev)
        rs_seed = 5

        def rs():
            chk(L.sg_skip_reduce_scatter(vp(bufs), 0, n, M, slice_bytes, 0.5, rs_seed, None, 1, vp(rs_out),
                                         vp(rs_cnt), stream()), "sg_skip_reduce_scatter")
        stages.append(("skip_reduce_scatter", rs))
        W["rs_cnt"] = rs_cnt
        out.update(rs_out=rs_out, rs_cnt=rs_cnt)
        W["rs_seed"] = rs_seed
        W["rs_geom"] = (n, M, slice_bytes // 4, S)
        W.update(slice_bytes=slice_bytes, p_skip=0.5)
        if name == "cfg5":
            W["elements"] = n * M
    if "stats_collect" in W:  # the host half of the statistics, after everything else is queued
        stages.append(("stats_collect", W["stats_collect"]))
    W["stages"] = stages
    W["nbytes"] = nbytes
    return W


def rs_bytes(W):
    """Bytes the skip reduce-scatter must move: the kept slices (read once)
    plus the output (written once)."""
    import numpy as np
    n, M, se, S = W["rs_geom"]
    cnt = W["rs_cnt"].cpu().numpy().astype(np.int64)
    tot = 0
    for j in range(n):
        cb, ce = (M * j) // n, (M * (j + 1)) // n
        lens = np.clip(ce - (cb + np.arange(S) * se), 0, se)
        tot += int((cnt[j] * lens).sum()) * 4
    return tot + M * 4


PROBES = {  # stage -> (probe id, kernel name, source files the kernel is built from)
    "dgc_select": (13, "dgc_filter_kernel", ["sg_dgc.hip", "sg_topk.hip"]),
    "hierarchical_hash": (14, "hh_insert_kernel", ["sg_hhash.hip"]),
    "skip_reduce_k": (5, "skip_rs_kernel", ["sg_skiprs.hip"]),
    "dropout_reduce_scatter": (11, "dropout_rs_kernel", ["sg_skiprs.hip"]),
    "allgather": (12, "allgather_kernel", ["sg_skiprs.hip"]),
    "topk_to_coo": (1, "topk_filter_pipe_kernel", ["sg_topk.hip"]),
    "hash_partition": (2, "part_scatter_kernel", ["sg_partition.hip"]),
    "aggregate": (3, "un_write_kernel", ["sg_union.hip", "sg_merge.hip", "sg_aggregate.hip"]),
    "encode": (4, "enc_kernel", ["sg_encode.hip"]),
    "decode": (9, "dec_emit_kernel", ["sg_decode.hip"]),
    "scatter_dense": (10, "scatter_window_kernel", ["sg_decode.hip"]),  # scatter_rows_kernel for rows (D > 1)
    "skip_reduce_scatter": (5, "skip_rs_kernel", ["sg_skiprs.hip"]),
}
COMMON_SOURCES = ["sg_device.h", "sg_host.h"]


def encode_kernel_name(W):
    """The encode kernel the library picks for the workload: a wave per group
    of class-map windows (enc_group_kernel, then enc_fix_kernel) for 2..16
    classes and at least 2048 groups, else a block per window (enc_kernel)."""
    P, M = W["P"], W["M"]
    if P < 2 or P > 16:
        return "enc_kernel"
    windows = -(-M // 4096)
    G = 4 if P > 8 else 1
    return "enc_group_kernel" if -(-windows // G) >= 2048 else "enc_kernel"


def decode_kernel_name(W):
    """The decode emit kernel the library picks: a wave per group of windows
    (dec_group_kernel; 4 windows for 9..16 classes, else 1) for 2..16 classes
    and at least 2048 groups, else a block per window (dec_emit_kernel)."""
    P, M = W["P"], W["M"]
    if P < 2 or P > 16:
        return "dec_emit_kernel"
    windows = -(-M // 4096)
    G = 4 if P > 8 else 1
    return "dec_group_kernel" if -(-windows // G) >= 2048 else "dec_emit_kernel"


HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_source_digest(stage):
    """sha256 over the sources of the probed kernel of a stage: a recorded
    HBM traffic figure is valid only for the source it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in PROBES[stage][2] + COMMON_SOURCES:
        with open(os.path.join(HERE, "sparse_gradient_synchronization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(stage, workload, kernel=None):
    """HBM bytes per launch of the probed kernel, from the rocprofv3 counter
    summary under profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the same counter reads for a plain copy of known size).  None when no
    summary exists for this kernel and workload, or when the kernel's source
    has changed since the counters were taken."""
    path = os.path.join(HERE, "profiles", "traffic_%s_%s.txt" % (kernel or PROBES[stage][1], workload))
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != kernel_source_digest(stage):
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, nbytes):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters of a profile run (FETCH_SIZE / WRITE_SIZE of this copy against
    nbytes read and nbytes written)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 3 copies of %d bytes" % nbytes)
    del src, dst


def concurrent_step(stages, torch):
    """The step with its independent rows overlapped on their own streams
    (default priority): the statistics and the skip reduce-scatter once the
    aggregate is queued (they then overlap the encode and each other: the
    statistics are latency-bound, the reduce-scatter bandwidth-bound; the
    reduce-scatter started earlier competes with the top-k filter for
    bandwidth and delays top-k's small kernels, and the statistics started
    after top-k slow the partition and the merge a little more than they
    gain); everything else runs in order on the current stream.  The streams
    join at the end of the step, and the host half of the statistics runs
    last.  A workload without an aggregate starts them with the step, and
    one without a top-k starts the statistics with the step (their input
    lists are there from the start).  Measured on dgc-top5, the statistics
    after the top-k and the reduce-scatter after the top-k or the partition
    were all slower (1.22-1.29 vs 1.217 ms).  None when the step has
    nothing to overlap."""
    fns = dict(stages)
    side_names = [nm for nm in ("skip_reduce_scatter", "stats") if nm in fns]
    if not side_names or len(fns) - len(side_names) - ("stats_collect" in fns) < 1:
        return None
    side = {nm: torch.cuda.Stream() for nm in side_names}
    after = {"stats": "aggregate", "skip_reduce_scatter": "aggregate"}
    if "topk_to_coo" not in fns:
        # the statistics read the step's input lists: with no top-k before
        # them they start with the step (workload 4: 1.69 -> 1.57 ms)
        after["stats"] = None
    evs = {nm: torch.cuda.Event() for nm in side_names}

    def launch(nm):
        evs[nm].record(torch.cuda.current_stream())
        s = side[nm]
        s.wait_event(evs[nm])
        with torch.cuda.stream(s):
            fns[nm]()

    def run():
        main = torch.cuda.current_stream()
        for nm in side_names:
            if after[nm] is None or after[nm] not in fns:
                launch(nm)
        for nm, f in stages:
            if nm in side or nm == "stats_collect":
                continue
            f()
            for nm2 in side_names:
                if after[nm2] == nm:
                    launch(nm2)
        for s in side.values():
            main.wait_stream(s)
        if "stats_collect" in fns:
            fns["stats_collect"]()
    return run


def copy_bandwidth(torch, nbytes=2 << 30, reps=5):
    """The box's achievable HBM bandwidth: a plain device-to-device copy of
    nbytes, read + write bytes over the median time of reps copies."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst
    t = sorted(ms)[len(ms) // 2]
    return {"bytes_copied": nbytes, "median_ms": t, "GBps": 2 * nbytes / (t * 1e-3) / 1e9}


def cold_steps(torch, step, steps, flush_bytes=1 << 30):
    """Each step timed alone with HIP events after a 1 GiB scratch write has
    pushed its working set out of the caches; returns the median in ms."""
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    ms = []
    for _ in range(steps):
        scratch.fill_(0.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    del scratch
    return sorted(ms)[len(ms) // 2]


def pull_side(W, L, torch, steps):
    """Decode of the step's hash bitmap and the scatter of its aggregate into
    a dense tensor, each timed alone (whole call with torch events, probed
    kernel with HIP events), plus the aggregate's encoded sizes."""
    out = {}
    for nm, f in W["pull"]:
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        evs = [HipEvents() for _ in range(steps)]
        a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for s in range(steps):
            L.sg_probe_set(PROBES[nm][0], evs[s].start, evs[s].stop)
            a[s].record()
            f()
            b[s].record()
        torch.cuda.synchronize()
        L.sg_probe_set(0, None, None)
        kms = sum(e.elapsed_ms() for e in evs) / steps
        nbytes = algorithmic_bytes(W, nm)
        gbps = nbytes / (kms * 1e-3) / 1e9
        ms = sum(a[s].elapsed_time(b[s]) for s in range(steps)) / steps
        kname = PROBES[nm][1]
        if nm == "scatter_dense" and W.get("D", 1) > 1:
            kname = "scatter_rows_kernel"
        elif nm == "decode":
            kname = decode_kernel_name(W)
        out[nm] = {"ms": ms, "kernel": kname, "kernel_ms": kms, "kernel_algorithmic_bytes": nbytes,
                   "kernel_GBps": gbps, "kernel_frac": gbps / HBM_PEAK_GBS}
        if nm == "scatter_dense":  # the whole call: the dense tensor written, the aggregate read
            U = int(W["agg_off"][-1].item())
            call_bytes = W["M"] * 4 * W.get("D", 1) + U * (4 + 4 * W.get("D", 1))
            out[nm]["call_algorithmic_bytes"] = call_bytes
            out[nm]["call_GBps"] = call_bytes / (ms * 1e-3) / 1e9
    out["format_sizes_bytes"] = W["format_sizes"]()
    return out


def time_call(L, torch, f, steps, probe=None):
    """Average time of a call (torch events on the current stream) and of
    its probed kernel (HIP events the library records around it)."""
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    evs = [HipEvents() for _ in range(steps)] if probe else []
    a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for s in range(steps):
        if probe and L.sg_probe_set(PROBES[probe][0], evs[s].start, evs[s].stop) != 0:
            raise RuntimeError("sg_probe_set refused probe %s" % probe)
        a[s].record()
        f()
        b[s].record()
    torch.cuda.synchronize()
    L.sg_probe_set(0, None, None)
    ms = sum(a[s].elapsed_time(b[s]) for s in range(steps)) / steps
    kms = sum(e.elapsed_ms() for e in evs) / steps if probe else None
    return ms, kms


def next_rows(name, W, L, torch, sg, steps):
    """The rows built after the hot path, each timed alone on this
    workload's buffers: DGC's sampled threshold with residuals (dgc-top5),
    the rest of the SkipReduce family (cfg5)."""
    out = {}

    def entry(nm, ms, kms, nbytes, what):
        e = {"ms": ms, "kernel": PROBES[nm][1] if nm in PROBES else None, "kernel_ms": kms,
             "kernel_algorithmic_bytes": nbytes, "bytes_are": what}
        if kms and nbytes:
            e["kernel_GBps"] = nbytes / (kms * 1e-3) / 1e9
            e["kernel_frac"] = e["kernel_GBps"] / HBM_PEAK_GBS
        return e

    if name == "dgc-top5":
        dense = W["dense"]
        n, M, k = W["n"], W["M"], W["k"]
        resid = torch.zeros_like(dense)
        ws = torch.empty(L.sg_dgc_workspace_bytes(n, M, 16384), dtype=torch.uint8, device=dense.device)
        box = {}

        def dgc():
            box["r"] = sg.sg_dgc_select(dense, resid, 0.05, 16384, k + k // 4, workspace=ws)
        ms, kms = time_call(L, torch, dgc, steps, "dgc_select")
        cnt = box["r"][2].cpu().tolist()
        # the filter reads the gradient and the residual and writes the residual
        out["dgc_select"] = entry("dgc_select", ms, kms, 12 * n * M, "grad and resid read, resid written")
        out["dgc_select"].update(samples_per_worker=16384, density=0.05, selected_per_worker=cnt,
                                 note="iterations carry the residual from call to call")
    if name == "cfg5":
        bufs = W["bufs"]
        n, M = W["n"], W["M"]
        slice_bytes = W["slice_bytes"]
        rs_out = torch.empty(M, dtype=torch.float32, device=bufs.device)
        S = L.sg_skip_num_slices(n, M, slice_bytes, 0)
        cnt = torch.empty((n, S), dtype=torch.uint8, device=bufs.device)
        kk = n // 2

        def sk():
            sg.sg_skip_reduce_k(bufs, slice_bytes, kk, True, 5, want_count=False, out=rs_out)
        ms, kms = time_call(L, torch, sk, steps, "skip_reduce_k")
        kept = (n - kk) * n * M // n * 4  # every slice keeps n - k contributions
        out["skip_reduce_k"] = entry("skip_reduce_k", ms, kms, kept + 4 * M, "kept slices read, output written")
        out["skip_reduce_k"].update(k=kk, random_offset=True)

        def dr():
            sg.sg_dropout_reduce_scatter(bufs, 0.5, 5, want_count=False, out=rs_out)
        ms, kms = time_call(L, torch, dr, steps, "dropout_reduce_scatter")
        out["dropout_reduce_scatter"] = entry("dropout_reduce_scatter", ms, kms, 4 * n * M + 4 * M,
                                              "every contribution read (a dropped element shares its line), "
                                              "output written")
        out["dropout_reduce_scatter"]["p"] = 0.5
        offs = [0, M // 4, M // 2, 3 * M // 4, M]
        rates = [0.0, 0.25, 0.5, 0.75]

        def se():
            sg.sg_selective_reduce_scatter(bufs, offs, rates, slice_bytes, 5, out=rs_out)
        ms, _ = time_call(L, torch, se, steps)
        out["selective_reduce_scatter"] = {"ms": ms, "bucket_off": offs, "p_skip": rates}
        red = torch.randn(M, dtype=torch.float32, device=bufs.device)
        ag = torch.empty((n, M), dtype=torch.float32, device=bufs.device)

        def al():
            sg.sg_allgather(red, bufs, None, out=ag)
        ms, kms = time_call(L, torch, al, steps, "allgather")
        out["allgather"] = entry("allgather", ms, kms, 4 * M + 4 * n * M, "reduced tensor read, n copies written")
    if name == "cfg4":
        out["alg1_study"] = alg1_study(L, torch, sg, steps)
    return out


def batched_mode(name, L, torch, sg, steps):
    """Batched mode of the two latency-bound workloads, labelled as such (one
    step of one instance leaves the GPU mostly idle): B independent
    instances of the workload's first stage in one launch, since a call
    takes any number of workers.  Workload 1: top-k of B x 4 dense gradients
    (instance b's four workers draw their Zipf(1.1) nonzeros from seed
    namespace 1000 + b); workload 2: the hash partition of B x 8 workers'
    64-wide rows (namespace 2000 + b).  Two instances are checked against the
    same call on that instance alone (bit-exact)."""
    import numpy as np
    import gen
    dev = torch.device("cuda", 0)
    res = {"label": "batched mode: B independent instances of the first stage in one launch"}
    if name == "cfg1":
        B, n, M = 64, 4, 1 << 20
        k = M // 100
        dense_h = np.empty((B * n, M), dtype=np.float32)
        for b in range(B):
            idx, off, val = gen.coo_zipf(1000 + b, n, M, k, 1.1, nonzero=True)
            dense_h[b * n:(b + 1) * n] = gen.dense_from_coo(n, M, idx, off, val)
        dense = torch.from_numpy(dense_h).to(dev)
        del dense_h
        box = {}
        ws = torch.empty(L.sg_topk_workspace_bytes(B * n, M, k, 0), dtype=torch.uint8, device=dev)

        def run():
            box["r"] = sg.sg_topk_to_coo(dense, k, workspace=ws)
        ms, _ = time_call(L, torch, run, steps)
        bi, bv = box["r"]
        same = True
        for b in (0, B - 1):
            si, sv = sg.sg_topk_to_coo(dense[b * n:(b + 1) * n].contiguous(), k)
            same = same and torch.equal(si, bi[b * n:(b + 1) * n]) and torch.equal(sv, bv[b * n:(b + 1) * n])
        nbytes = B * n * M * 4 + B * n * k * 8
        res.update({"stage": "topk_to_coo", "B": B, "workers": B * n, "ms": ms, "us_per_instance": ms * 1e3 / B,
                    "algorithmic_bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "matches_single_instance": bool(same)})
    elif name == "cfg2":
        B, n, R, cnt, D, P, seed = 32, 8, 1_000_000, 4096, 64, 8, 2
        idxs, vals = [], []
        for b in range(B):
            idx, off, val = gen.coo_zipf(2000 + b, n, R, cnt, 1.05, D=D, sigma=0.01)
            idxs.append(idx)
            vals.append(val)
        idx = torch.from_numpy(np.concatenate(idxs).view(np.int32)).to(dev)
        val = torch.from_numpy(np.concatenate(vals)).to(dev)
        in_off = torch.arange(B * n + 1, dtype=torch.int64, device=dev) * cnt
        box = {}

        def run():
            box["r"] = sg.sg_hash_partition(idx, val, in_off, P, seed)
        ms, _ = time_call(L, torch, run, steps)
        pi, pv, po = box["r"]
        same = True
        e = n * cnt
        for b in (0, B - 1):
            si, sv, so = sg.sg_hash_partition(idx[b * e:(b + 1) * e].contiguous(), val[b * e:(b + 1) * e].contiguous(),
                                              torch.arange(n + 1, dtype=torch.int64, device=dev) * cnt, P, seed)
            same = (same and torch.equal(si, pi[b * e:(b + 1) * e]) and torch.equal(sv, pv[b * e:(b + 1) * e])
                    and torch.equal(so + b * e, po[b * n:(b + 1) * n]))
        nbytes = 2 * B * n * cnt * (4 + D * 4)
        res.update({"stage": "hash_partition", "B": B, "workers": B * n, "ms": ms, "us_per_instance": ms * 1e3 / B,
                    "algorithmic_bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "matches_single_instance": bool(same)})
    return res


def alg1_study(L, torch, sg, steps):
    """Algorithm 1's parameter study on a synthetic 214M-element tensor (one
    worker, 1% density, uniform distinct indices, 16 partitions): the time of
    sg_hierarchical_hash for parallel memories of 1, 2 and 4 times the
    nonzeros and k = 1..4 rehash functions, serial memory equal to the
    nonzeros; beside it sg_hash_partition on the same entries."""
    import numpy as np
    import gen
    M, P, seed = 214_000_000, 16, 6
    nnz = M // 100
    idx_np = np.sort(gen.uniform_distinct(gen.stream_seed(6, 1), 0, M, nnz)).astype(np.uint32)
    dev = torch.device("cuda", 0)
    idx = torch.from_numpy(idx_np.view(np.int32)).to(dev)
    val = torch.from_numpy(gen.normal(gen.stream_seed(6, 2), nnz)).to(dev)
    in_off = torch.tensor([0, nnz], dtype=torch.int64, device=dev)
    res = {"M": M, "nnz": nnz, "P": P, "r2": nnz, "runs": []}
    ws = torch.empty(L.sg_hierarchical_hash_workspace_bytes(1, P, 4 * nnz // P, nnz), dtype=torch.uint8, device=dev)
    for alpha in (1, 2, 4):
        r1 = alpha * nnz // P
        for k in (1, 2, 3, 4):
            box = {}

            def run():
                box["r"] = sg.sg_hierarchical_hash(idx, val, in_off, P, seed, k, r1, nnz, workspace=ws)
            ms, kms = time_call(L, torch, run, steps, "hierarchical_hash")
            cnt = box["r"][4].cpu().tolist()[0]
            res["runs"].append({"alpha": alpha, "r1": r1, "k": k, "ms": ms, "insert_kernel_ms": kms,
                                "serial_writes": cnt[0], "lost": cnt[1]})
    wsp = torch.empty(L.sg_partition_workspace_bytes(1, nnz, P), dtype=torch.uint8, device=dev)

    def a2():
        sg.sg_hash_partition(idx, val, in_off, P, seed, workspace=wsp)
    res["hash_partition_ms"], _ = time_call(L, torch, a2, steps)
    return res


def union_size(W):
    return int(W["agg_off"][-1].item())


def stage_bytes(W, stage):
    """Algorithmic bytes of a whole stage call: what the method itself must
    read and write (inputs once, outputs once; workspaces excluded)."""
    n = W.get("n")
    D = W.get("D", 1)
    if stage == "topk_to_coo":
        return n * W["M"] * 4 + n * W["k"] * 8
    if stage == "hash_partition":
        return W["nbytes"]["hash_partition"]
    if stage == "aggregate":
        return W["bytes_agg"](union_size(W))
    if stage == "encode":
        return W["bytes_enc"](union_size(W), int(W["word_off"][-1].item()))
    if stage == "skip_reduce_scatter":
        return rs_bytes(W)
    if stage == "stats":  # report-only: the index lists read once
        return W["nnz"] * 4
    return None


def algorithmic_bytes(W, stage):
    """Algorithmic bytes per launch of the primary probed kernel of a stage
    (and of the Pull-side kernels)."""
    if stage == "topk_to_coo":
        return W["n"] * W["M"] * 4  # the dense read; slots are workspace
    if stage in ("hash_partition", "aggregate", "encode", "skip_reduce_scatter"):
        return stage_bytes(W, stage)
    if stage == "decode":  # the bitmap words read, the indices written
        return int(W["word_off"][-1].item()) * 4 + union_size(W) * 4
    if stage == "scatter_dense":
        D = W.get("D", 1)
        if D == 1:  # the window pass: the aggregate read, every dense element written once
            return W["M"] * 4 + union_size(W) * 8
        return union_size(W) * (4 + 8 * D)  # rows: the aggregate read, its rows written in place
    raise KeyError(stage)


# every probed hot-path kernel: (stage, probe id, kernel, algorithmic bytes per launch)
KERNELS = [
    ("topk_to_coo", 1, "topk_filter_pipe_kernel", lambda W: W["n"] * W["M"] * 4),
    ("topk_to_coo", 8, "topk_write_kernel", lambda W: 2 * W["n"] * W["k"] * 8),
    ("hash_partition", 7, "part_hist_kernel", lambda W: W["nnz"] * 4),
    ("hash_partition", 2, "part_scatter_kernel", lambda W: W["nbytes"]["hash_partition"]),
    ("aggregate", 6, "mg_bnd_kernel", lambda W: W["nnz"] * 4),
    ("aggregate", 15, "un_count_kernel", lambda W: W["nnz"] * 4),
    ("aggregate", 3, "un_write_kernel", lambda W: stage_bytes(W, "aggregate")),
    ("encode", 4, "enc_kernel", lambda W: stage_bytes(W, "encode")),
    ("skip_reduce_scatter", 5, "skip_rs_kernel", lambda W: rs_bytes(W)),
]


def host_cpu():
    """The host's CPU model and core counts (the oracle baseline's machine)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def oracle_step(name, W):
    """The oracle on one full step of the workload (every stage the GPU step
    runs, full size, single-threaded C), on the same host inputs.  Returns its
    outputs and its wall time."""
    import numpy as np
    import oracle
    c = W["host"]
    ref = {}
    t0 = time.perf_counter()
    if name in ("dgc-top5", "cfg1"):
        idx, val = oracle.topk_to_coo(c["dense"], W["k"])
        ref["topk"] = (idx, val)
        src_idx, src_val = idx.reshape(-1), val.reshape(-1)
    elif name in ("cfg2", "cfg4"):
        src_idx, src_val = c["idx"], c["val"]
    if name != "cfg5":
        M, P, seed, in_off = W["M"], W["P"], W["seed"], W["in_off_host"]
        oi, ov, po = oracle.hash_partition(src_idx, src_val, in_off, P, seed)
        ai, av, aa, ao = oracle.aggregate(oi, ov, po, M)
        bm, wo = oracle.encode(ai, ao, M, seed)
        st = oracle.stats(src_idx, in_off, M, P, hashed=True, seed=seed)
        ref.update(part=(oi, ov, po), agg=(ai, av, aa, ao), enc=(bm, wo), stats=st)
    if name in ("dgc-top5", "cfg5"):
        bufs = c["dense"] if name == "dgc-top5" else c["bufs"]
        ref["rs"] = oracle.skip_reduce_scatter(bufs, W["slice_bytes"] // 4, W["p_skip"], W["rs_seed"], mode=1)
    return ref, time.perf_counter() - t0


def compare_outputs(W, ref):
    """The GPU step's outputs against the oracle's: bit-exact where the result
    is integer or a bit copy, within |d| <= 1e-6 * sum|x| + 1e-30 for fp32
    sums.  Returns {check: bool} plus the largest error / bound ratio."""
    import numpy as np
    o = W["out"]
    ok = {}
    worst = 0.0

    def u32(t):
        return t.cpu().numpy().view(np.uint32)

    def within(got, exact, abs_sum):
        nonlocal worst
        got = np.asarray(got, dtype=np.float64).reshape(-1)
        bound = 1e-6 * np.asarray(abs_sum, dtype=np.float64).reshape(-1) + 1e-30
        r = np.abs(got - np.asarray(exact).reshape(-1)) / bound
        worst = max(worst, float(r.max()) if r.size else 0.0)
        return bool(np.all(r <= 1.0))

    if "topk" in ref:
        ri, rv = ref["topk"]
        ok["topk_indices"] = bool(np.array_equal(u32(o["topk_idx"]).reshape(-1), ri.reshape(-1)))
        ok["topk_values"] = bool(np.array_equal(u32(o["topk_val"]).reshape(-1), rv.reshape(-1).view(np.uint32)))
    if "part" in ref:
        oi, ov, po = ref["part"]
        ok["partition_offsets"] = bool(np.array_equal(o["part_off"].cpu().numpy().view(np.uint64), po))
        ok["partition_indices"] = bool(np.array_equal(u32(o["pidx"]), oi))
        ok["partition_values"] = bool(np.array_equal(u32(o["pval"]).reshape(-1), ov.reshape(-1).view(np.uint32)))
        ai, av, aa, ao = ref["agg"]
        gao = o["agg_off"].cpu().numpy().view(np.uint64)
        ok["aggregate_offsets"] = bool(np.array_equal(gao, ao))
        u = int(ao[-1])
        ok["aggregate_indices"] = bool(np.array_equal(u32(o["agg_idx"])[:u], ai))
        ok["aggregate_sums"] = within(o["agg_val"].cpu().numpy()[:u], av, aa)
        bm, wo = ref["enc"]
        ok["encode_word_offsets"] = bool(np.array_equal(o["word_off"].cpu().numpy().view(np.uint64), wo))
        ok["encode_bitmap"] = bool(np.array_equal(u32(o["bitmap"])[: int(wo[-1])], bm))
        st, got = ref["stats"], W["stats_arrays"]
        so = W["stats_out"]
        same = all(np.array_equal(got[k], np.asarray(st[k]).reshape(-1)) for k in got)
        for k in ("union_size", "sum_nnz", "max_nnz", "overlap_mean", "overlap_min", "overlap_max", "gamma_n",
                  "push_imbalance", "pull_imbalance"):
            same = same and getattr(so, k) == st[k]
        ok["stats"] = bool(same)
    if "rs" in ref:
        out, oabs, cnt = ref["rs"]
        ok["skip_rs_counts"] = bool(np.array_equal(o["rs_cnt"].cpu().numpy(), cnt))
        ok["skip_rs_sums"] = within(o["rs_out"].cpu().numpy(), out, oabs)
    return ok, worst


def measure_workload(name, args, torch, sg, gen, headline):
    """Build one workload, time its step, time every probed kernel, compare
    the outputs with the oracle and time the oracle.  Returns the workload's
    record (the JSON line's fields for the headline workload)."""
    log("building workload", name)
    W = build_workload(name, torch, sg, gen)
    stages = W["stages"]
    L = sg.lib()
    steps = args.steps
    evs = [HipEvents() for _ in range(steps)]   # one probe pair per timed step
    starts = [[torch.cuda.Event(enable_timing=True) for _ in stages] for _ in range(steps)]
    stops = [[torch.cuda.Event(enable_timing=True) for _ in stages] for _ in range(steps)]

    def step(s=None):
        for i, (nm, f) in enumerate(stages):
            if s is not None:
                starts[s][i].record()
            f()
            if s is not None:
                stops[s][i].record()

    overlapped = concurrent_step(stages, torch)
    run_step = overlapped or step

    for _ in range(max(args.warmup, 1)):
        run_step()
    torch.cuda.synchronize()

    # every probed kernel of the workload, each timed over `steps` sequential
    # steps with HIP events the library records around it
    kernels = {}
    have = {nm for nm, _ in stages}
    rows = W.get("D", 1) > 1
    for stg, pid, kname, fbytes in KERNELS:
        if stg not in have or (rows and kname == "un_count_kernel"):
            continue
        if rows and kname == "un_write_kernel":
            kname = "mg_merge_kernel"  # rows (D >= 2) take the merge engine
        if kname == "enc_kernel":
            kname = encode_kernel_name(W)
        for s in range(steps):
            L.sg_probe_set(pid, evs[s].start, evs[s].stop)
            step()
        torch.cuda.synchronize()
        L.sg_probe_set(0, None, None)
        kms = sum(e.elapsed_ms() for e in evs) / steps
        nb = fbytes(W)
        kernels[kname] = {"stage": stg, "avg_ms": kms, "algorithmic_bytes": nb,
                          "GBps": nb / (kms * 1e-3) / 1e9, "frac": nb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    prim = {nm: PROBES[nm][1] for nm in have if nm in PROBES}
    if rows and "aggregate" in prim:
        prim["aggregate"] = "mg_merge_kernel"
    if "encode" in prim:
        prim["encode"] = encode_kernel_name(W)
    dom = args.probe or max(prim, key=lambda nm: kernels[prim[nm]]["avg_ms"])
    log("kernels (ms):", {k: round(v["avg_ms"], 4) for k, v in kernels.items()}, "dominant stage:", dom)

    # timed region: K steps bracketed by synchronize; the dominant kernel of
    # every step is bracketed by its own pair of HIP events on its stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        L.sg_probe_set(PROBES[dom][0], evs[s].start, evs[s].stop)
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    L.sg_probe_set(0, None, None)
    # per-stage times from a second, untimed pass with the stages one after
    # another on one stream: an event recorded between two stages costs the
    # queue a few microseconds, so the timed steps carry none but the probe
    # pair
    for s in range(steps):
        step(s)
    torch.cuda.synchronize()
    if sg.sg_device_error() != 0:
        raise SystemExit("a kernel recorded a violated precondition")

    ms_per_step = (t1 - t0) * 1000.0 / steps
    per = [e.elapsed_ms() for e in evs]
    dom_avg = sum(per) / len(per)
    dom_bytes = algorithmic_bytes(W, dom)
    achieved = dom_bytes / (dom_avg * 1e-3) / 1e9
    stages_ms = {nm: sum(starts[s][i].elapsed_time(stops[s][i]) for s in range(steps)) / steps
                 for i, (nm, _) in enumerate(stages)}
    stages_out = {}
    for nm, ms in stages_ms.items():
        e = {"ms": round(ms, 4)}
        nb = stage_bytes(W, nm)
        if nb is not None and ms > 0:
            e.update(algorithmic_bytes=nb, GBps=nb / (ms * 1e-3) / 1e9, frac=nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
            if nm == "stats":
                e["note"] = "report-only: the index lists read once"
        stages_out[nm] = e

    if name == "cfg5":
        units, unit = W["elements"], "elements/s"
    elif "k" in W:
        units, unit = W["n"] * W["k"], "nonzeros/s"
    else:
        units, unit = W["nnz"], "nonzeros/s"
    value = units / (ms_per_step * 1e-3)

    step_bytes = sum(stage_bytes(W, nm) or 0 for nm in stages_ms if nm != "stats")
    cfg = {"workload": name}
    for key in ("n", "M", "k", "P", "D", "total", "slice_bytes", "p_skip"):
        if key in W:
            cfg[key] = W[key]
    if "agg_off" in W:
        cfg["union_size"] = union_size(W)
    rec = {
        "value": value,
        "unit": unit,
        "ms_per_step": ms_per_step,
        "config": cfg,
        "stages": stages_out,
        "kernels": kernels,
        "overlap": ("skip reduce-scatter and statistics on their own streams once the aggregate is queued, "
                    "overlapped with the encode and each other; stage times from a sequential pass")
        if overlapped else None,
        "step_algorithmic_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(dom, name, prim[dom]),
            "kernel": prim[dom], "stage": dom, "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_ms": dom_avg,
        },
        "cpu_baseline": None,
        "parity": None,
    }
    if name in ("cfg1", "cfg2"):
        # working sets below 256 MB fit the caches: the hot figure above, and
        # each step alone after a cache-flushing write
        rec["cold_ms_per_step"] = cold_steps(torch, run_step, steps)
        rec["cold_value"] = units / (rec["cold_ms_per_step"] * 1e-3)
        rec["batched"] = batched_mode(name, L, torch, sg, steps)
    if headline and "pull" in W:
        rec["pull_side"] = pull_side(W, L, torch, steps)
    nr = next_rows(name, W, L, torch, sg, steps)
    if nr:
        rec["next_rows"] = nr
    if not args.no_cpu_baseline:
        log("oracle step (single-threaded) on", name)
        ref, secs = oracle_step(name, W)
        ok, worst = compare_outputs(W, ref)
        rec["parity"] = {"ok": all(ok.values()), "checks": ok, "max_err_over_bound": worst,
                         "against": "oracle outputs for the same inputs, full size"}
        cb = {"value": units / secs, "unit": unit, "cores": 1, "kind": "oracle",
              "sample": "one full step of the workload (every stage the GPU step runs, full size), "
                        "single-threaded C oracle",
              "seconds": round(secs, 3)}
        cb.update(host_cpu())
        rec["cpu_baseline"] = cb
        log("parity", name, "ok" if rec["parity"]["ok"] else "FAILED %s" % ok)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=("all",) + WORKLOADS,
                    help="one workload only (default: all five, dgc-top5 as the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (parity and baseline)")
    ap.add_argument("--probe", default=None, help="stage whose kernel is timed for the roofline (default: slowest)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run a plain device copy of BYTES (for scaling HBM counters under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the n workers are simulated resident on it); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gen
    import sparse_gradient_synchronization_amd as sg

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
    names = WORKLOADS if args.workload == "all" else (args.workload,)
    recs = {}
    for nm in names:
        recs[nm] = measure_workload(nm, args, torch, sg, gen, headline=nm == names[0])
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    head = recs[names[0]]
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generators, shapes and distributions of the workload)",
    }
    res.update({k: v for k, v in head.items() if k not in res})
    res["hbm_copy"] = copy_bandwidth(torch)
    if len(names) > 1:
        res["configs"] = {nm: recs[nm] for nm in names[1:]}
    bad = [nm for nm, r in recs.items() if r["parity"] is not None and not r["parity"]["ok"]]
    print(json.dumps(res), flush=True)
    if bad:
        log("parity FAILED on", bad)
        sys.exit(3)


if __name__ == "__main__":
    main()

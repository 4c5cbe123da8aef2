// sg_union.hip -- the union-sum of A3 for scalar values and bare indices
// (D <= 1): per partition, the union of the n workers' sorted runs with the
// values of each index summed (the server side of Push in the Zen OSDI'25
// digest, section 3.1; equal to the dense AllReduce, section 3.2).
//
// The key space of every partition is cut into tiles of 2^tb keys; the
// merge engine's boundary pass (sg_merge.hip) records where each tile starts
// in each run.  Tiles are taken in (partition, key) order, which is the
// output order, and dealt to blocks as contiguous ranges of equal work (the
// tile's entries plus a fixed cost), from a scan of the per-tile work.  Two
// passes, a block of 256 threads per range, no atomics on global memory:
//   count  a tile's keys OR-ed into an LDS presence bitmap of its span (up
//          to 2^17 keys); the popcounts summed over the block's tiles give
//          its union size, and a scan of those gives every block its output
//          offset.
//   write  a tile's entries in windows of at most 2048 (a window takes up to
//          8 g entries of every run, g = 256 / n rounded to a power of two,
//          and ends at the smallest last-loaded key of a run it cut short,
//          so every key is whole inside one window): the presence bitmap and
//          its prefix popcounts give each entry the rank of its key; values
//          are added into an LDS slot per rank, one wave after the other in
//          the order of the runs they hold, so every sum is taken in worker
//          order; keys and sums are written once, in order, at the block's
//          offset, with consecutive threads on consecutive addresses.
// A window gives run w the g threads [w g, (w+1) g): thread s of the group
// reads entries s, s + g, s + 2g, ... of the run's part of the window, so an
// entry's address is its run's position plus a constant.
#include "sg_host.h"

namespace sg {

constexpr int UN_THREADS = 256;              // threads per block
constexpr int UN_WAVES = UN_THREADS / SG_WAVE;
constexpr int UN_PER = 8;                    // slots per thread
constexpr int UN_CAP = UN_PER * UN_THREADS;  // entries of a window
#ifndef SG_UN_TARGET
#define SG_UN_TARGET 1536
#endif
constexpr int UN_TARGET = SG_UN_TARGET;      // mean entries per tile aimed at
#ifndef SG_UN_SPAN_LOG_MAX
#define SG_UN_SPAN_LOG_MAX 17
#endif
constexpr int UN_SPAN_LOG_MAX = SG_UN_SPAN_LOG_MAX; // a tile spans at most 2^17 keys (WPT = 16)
#ifndef SG_UN_FIXED
#define SG_UN_FIXED 512
#endif
constexpr uint32_t UN_FIXED = SG_UN_FIXED;   // a tile's fixed cost, in entries, for the balance of blocks

// Value modes: VM_NONE (indices only), VM_F32, VM_BF16 (widened to fp32 where
// the values are added, so the loaded registers are not touched before).
constexpr int VM_NONE = 0, VM_F32 = 1, VM_BF16 = 2;

template <int VM>
__device__ __forceinline__ float un_value(uint32_t b)
{
    return __uint_as_float(VM == VM_BF16 ? b << 16 : b);
}

// Threads per run: 256 / (n rounded up to a power of two), as a log.
__device__ __forceinline__ uint32_t un_glog(uint32_t n)
{
    uint32_t l = 0;
    while ((1u << l) < n) ++l;
    return 8 - l; // n <= 64
}

// Run bookkeeping of a block, in LDS: run w's next position (absolute),
// remaining entries of the tile, and the window's take.
struct UnRuns {
    uint32_t pos[64];
    uint32_t rem[64];
    uint32_t take[64];
    uint32_t drop[64];
    uint32_t kmax;   // the window's last key (cut windows)
    uint32_t more;   // entries left in the tile after the window
    uint32_t cut;    // some run continues after the window
};

// Wave 0 (threads below n hold runs): the raw run range of tile t (lanes
// past n repeat run n-1, tiles past the last repeat the last), issued
// without waiting; un_runs_put clamps it into LDS once it is needed.
struct URaw {
    uint64_t a, e; // the run's absolute range
    uint32_t x, y; // the tile's part, relative to the run
};

__device__ __forceinline__ URaw un_runs_issue(const MergeParams& p, uint32_t t)
{
    const uint32_t w = threadIdx.x & (SG_WAVE - 1);
    const uint32_t T = p.G * p.NT;
    const uint32_t tt = t < T ? t : T - 1;
    const uint32_t ww = w < p.n ? w : p.n - 1;
    const uint32_t g = tt / p.NT, b = tt % p.NT;
    URaw r;
    r.a = p.off[(uint64_t)ww * p.stride + g];
    r.e = p.off[(uint64_t)ww * p.stride + g + 1];
    const uint32_t* row = p.bnd + ((uint64_t)g * p.n + ww) * (p.NT + 1);
    r.x = row[b];
    r.y = row[b + 1];
    return r;
}

__device__ __forceinline__ void un_runs_put(const MergeParams& p, const URaw& r, UnRuns& R)
{
    const uint32_t w = threadIdx.x;
    uint64_t a = r.a > p.total ? p.total : r.a, e = r.e > p.total ? p.total : r.e;
    if (e < a) e = a;
    const uint64_t len = e - a;
    uint64_t x = r.x > len ? len : r.x, y = r.y > len ? len : r.y;
    if (y < x) y = x;
    if (w < p.n) {
        R.pos[w] = (uint32_t)(a + x);
        R.rem[w] = (uint32_t)(y - x);
    }
}

// Wave 0: the tile's run parts into LDS (loads and waits).
__device__ __forceinline__ void un_runs_load(const MergeParams& p, uint32_t t, UnRuns& R)
{
    if (threadIdx.x >= SG_WAVE) return;
    const URaw r = un_runs_issue(p, t);
    un_runs_put(p, r, R);
}

// Wave 0: the next window's take of every run (at most 8 g entries), whether
// a run continues after it; the cut key starts at "none".
__device__ __forceinline__ void un_runs_window(uint32_t n, uint32_t glog, UnRuns& R)
{
    const uint32_t w = threadIdx.x;
    if (w >= SG_WAVE) return;
    const uint32_t cap = (uint32_t)UN_PER << glog;
    const uint32_t rem = w < n ? R.rem[w] : 0u;
    const uint32_t take = rem < cap ? rem : cap;
    if (w < n) {
        R.take[w] = take;
        R.drop[w] = 0u;
    }
    const bool cut = ballot(take < rem) != 0;
    if (w == 0) {
        R.cut = cut ? 1u : 0u;
        R.kmax = 0xffffffffu;
    }
}

// Every thread: its run's window entries into registers, slot i holding entry
// i g + s of the run's part (s = the thread's place in its group).  Returns
// the slots that hold an entry.  The loaded registers are not touched here,
// so the loads stay in flight together until their first use; slots past
// the run's take load the run's first window entry (or the last entry of
// the input).
template <int VM>
__device__ __forceinline__ uint32_t un_window_load(const MergeParams& p, const UnRuns& R, uint32_t glog,
                                                   uint32_t (&key)[UN_PER], uint32_t (&vb)[UN_PER])
{
    const uint32_t w = threadIdx.x >> glog, s = threadIdx.x & ((1u << glog) - 1u);
    const uint32_t take = w < p.n ? R.take[w] : 0u;
    const uint32_t base = w < p.n ? R.pos[w] : 0u;
    const uint32_t last = p.total > 0 ? (uint32_t)(p.total - 1) : 0u;
    uint32_t valid = 0;
#pragma unroll
    for (int i = 0; i < UN_PER; ++i) {
        const uint32_t e = ((uint32_t)i << glog) + s;
        uint32_t pos = base + (e < take ? e : 0u);
        pos = pos < last ? pos : last;
        key[i] = p.idx[pos];
        if (VM == VM_F32) vb[i] = static_cast<const uint32_t*>(p.val)[pos];
        if (VM == VM_BF16) vb[i] = static_cast<const uint16_t*>(p.val)[pos];
        valid |= (e < take ? 1u : 0u) << i;
    }
    return valid;
}

// Wave 0, once the window's entries are accounted for: advance every run by
// the entries it used, and whether the tile has entries left.
__device__ __forceinline__ void un_runs_advance(uint32_t n, UnRuns& R)
{
    const uint32_t w = threadIdx.x;
    if (w >= SG_WAVE) return;
    uint32_t rem = 0;
    if (w < n) {
        const uint32_t used = R.take[w] - R.drop[w];
        R.pos[w] += used;
        rem = R.rem[w] - used;
        R.rem[w] = rem;
    }
    const bool more = ballot(rem > 0) != 0;
    if (w == 0) R.more = more ? 1u : 0u;
}

// ---------------------------------------------------------------------------
// the balance: work of every tile, its scan, the first tile of every block
// ---------------------------------------------------------------------------

// work of tile t = its entries + UN_FIXED; exclusive prefix inside scan
// blocks of MG_SCAN_BLOCK tiles (MG_SCAN_PER consecutive tiles per thread,
// the loads of 8 runs in flight together)
__global__ __launch_bounds__(1024) void un_work_scan_kernel(MergeParams p)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    const uint32_t T = p.G * p.NT;
    const uint64_t t0 = (uint64_t)blockIdx.x * MG_SCAN_BLOCK + (uint64_t)threadIdx.x * MG_SCAN_PER;
    uint32_t c[MG_SCAN_PER];
    uint64_t sum = 0;
#pragma unroll
    for (int j = 0; j < MG_SCAN_PER; ++j) {
        c[j] = 0;
        const uint64_t t = t0 + j;
        if (t >= T) continue;
        const uint32_t g = (uint32_t)(t / p.NT), b = (uint32_t)(t % p.NT);
        const uint32_t* rows = p.bnd + (uint64_t)g * p.n * (p.NT + 1) + b;
        uint32_t E = 0;
        for (uint32_t w0 = 0; w0 < p.n; w0 += 8) {
            uint32_t x[8], y[8];
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u) {
                const uint32_t* row = rows + (uint64_t)(w0 + u < p.n ? w0 + u : 0u) * (p.NT + 1);
                x[u] = row[0];
                y[u] = row[1];
            }
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u)
                if (w0 + u < p.n && y[u] > x[u]) E += y[u] - x[u];
        }
        c[j] = E + UN_FIXED;
        sum += c[j];
    }
    uint64_t tot;
    uint64_t ex = block_excl_scan64<1024>(sum, scan_lds, &tot);
#pragma unroll
    for (int j = 0; j < MG_SCAN_PER; ++j) {
        if (t0 + j < T) p.wcum[t0 + j] = ex;
        ex += c[j];
    }
    if (threadIdx.x == 0) p.wblk[blockIdx.x] = tot;
}

// exclusive prefix of the scan blocks' totals (in place) and the total
__global__ __launch_bounds__(1024) void un_work_top_kernel(MergeParams p)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    uint64_t carry = 0;
    for (uint32_t base = 0; base < p.nscan; base += 1024) {
        const uint32_t i = base + threadIdx.x;
        const uint64_t v = i < p.nscan ? p.wblk[i] : 0ull;
        uint64_t tot;
        const uint64_t ex = block_excl_scan64<1024>(v, scan_lds, &tot);
        if (i < p.nscan) p.wblk[i] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) *p.wtotal = carry;
}

// Block k of W takes the tiles whose cumulative work starts in
// [k*C/W, (k+1)*C/W): wstart[k] is its first tile, wstart[W] = T.  The
// thread of tile t writes wstart[k] for k(t-1) < k <= k(t), with
// k(t) = floor(cum[t]*W/C), so every k is written once.
__global__ __launch_bounds__(256) void un_starts_kernel(MergeParams p)
{
    const uint32_t T = p.G * p.NT, W = p.nwaves;
    const uint64_t C = *p.wtotal;
    for (uint32_t t = blockIdx.x * 256 + threadIdx.x; t < T; t += gridDim.x * 256) {
        const uint64_t cum = p.wcum[t] + p.wblk[t / MG_SCAN_BLOCK];
        const uint64_t kt = C ? cum * W / C : 0;
        int64_t kp = -1;
        if (t > 0) {
            const uint64_t cp = p.wcum[t - 1] + p.wblk[(t - 1) / MG_SCAN_BLOCK];
            kp = (int64_t)(C ? cp * W / C : 0);
        }
        for (int64_t k = kp + 1; k <= (int64_t)kt && k < (int64_t)W; ++k) p.wstart[k] = t;
        if (t == T - 1)
            for (uint64_t k = kt + 1; k <= W; ++k) p.wstart[k] = T;
    }
}

// exclusive prefix of the blocks' union sizes (in place); wave_tot[W] = |I|
// and agg_off[G]
__global__ __launch_bounds__(1024) void un_tot_scan_kernel(MergeParams p)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    uint64_t carry = 0;
    for (uint32_t base = 0; base < p.nwaves; base += 1024) {
        const uint32_t i = base + threadIdx.x;
        const uint64_t v = i < p.nwaves ? p.wave_tot[i] : 0ull;
        uint64_t tot;
        const uint64_t ex = block_excl_scan64<1024>(v, scan_lds, &tot);
        if (i < p.nwaves) p.wave_tot[i] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        p.wave_tot[p.nwaves] = carry;
        p.agg_off[p.G] = carry;
    }
}

// ---------------------------------------------------------------------------
// the two passes
// ---------------------------------------------------------------------------

// LDS of the count pass: the bitmap of a tile's span, WPT words per thread,
// and the run parts of the tile being counted and of the next one.
template <int WPT>
struct UnCountSmem {
    uint32_t bits[WPT * UN_THREADS];
    UnRuns R[2];
    uint32_t red[UN_WAVES];
};

// One tile of the count pass.  Tile t's first window is in flight in kc
// (its runs in Rc); wave 0's raw ranges of tile t+1 are in flight in rr.
// Before counting tile t the block puts tile t+1's runs in Rn and issues
// its first window into kn, and wave 0 issues the ranges of tile t+2.
template <int WPT>
__device__ __forceinline__ void un_count_tile(const MergeParams& p, UnCountSmem<WPT>& sm, uint32_t t, uint32_t te,
                                              uint32_t glog, UnRuns& Rc, UnRuns& Rn, uint32_t& vc,
                                              uint32_t (&kc)[UN_PER], uint32_t& vn, uint32_t (&kn)[UN_PER],
                                              URaw& rr, uint64_t& total)
{
    constexpr int NCH = WPT / 4;
    const uint32_t tid = threadIdx.x, lane = lane_id(), wid = tid / SG_WAVE;
    const uint32_t n = p.n, span = 1u << p.tb;
    const bool next = t + 1 < te; // uniform
    if (next && tid < SG_WAVE) {
        un_runs_put(p, rr, Rn);
        un_runs_window(n, glog, Rn);
        rr = un_runs_issue(p, t + 2);
    }
    __syncthreads();
    uint32_t vb[UN_PER];
    if (next) vn = un_window_load<VM_NONE>(p, Rn, glog, kn, vb);
    const uint32_t klo = (t % p.NT) << p.tb;
    uint32_t valid = vc;
    while (true) {
        bool bad = false;
#pragma unroll
        for (int i = 0; i < UN_PER; ++i) {
            const uint32_t o = kc[i] - klo;
            const bool has = (valid >> i) & 1u;
            bad |= has && o >= span; // outside the tile: cannot happen for valid input
            if (has && o < span) atomicOr(&sm.bits[o >> 5], 1u << (o & 31u));
        }
        if (ballot(bad) && lane == 0) report_error(kDevErrIndexRange);
        __syncthreads(); // every thread is done reading Rc for this window
        un_runs_advance(n, Rc); // wave 0
        __syncthreads();
        if (!Rc.more) break;
        // a tile of more than one window: its later windows one at a time
        un_runs_window(n, glog, Rc);
        __syncthreads();
        valid = un_window_load<VM_NONE>(p, Rc, glog, kc, vb);
    }
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        uint4* w4 = reinterpret_cast<uint4*>(&sm.bits[4 * (q * UN_THREADS + tid)]);
        const uint4 v = *w4;
        c += (uint32_t)(__popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w));
        *w4 = make_uint4(0u, 0u, 0u, 0u);
    }
    const uint32_t ws = wave_sum(c);
    if (lane == 0) sm.red[wid] = ws;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < UN_WAVES; ++i) total += sm.red[i];
}

// Union size of each block's tiles (keys only).  The next tile's first
// window is loading while a tile is counted.
template <int WPT>
__global__ __launch_bounds__(UN_THREADS) void un_count_kernel(MergeParams p)
{
    static_assert(WPT % 4 == 0, "the bitmap is read as 16-byte chunks");
    __shared__ __align__(16) UnCountSmem<WPT> sm;
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < (uint32_t)(WPT * UN_THREADS); i += UN_THREADS) sm.bits[i] = 0u;
    const uint32_t n = p.n, glog = un_glog(n);
    const uint32_t k = blockIdx.x;
    const uint32_t ts = p.wstart[k], te = p.wstart[k + 1];
    uint64_t total = 0;
    if (ts < te) { // uniform
        URaw rr = {0ull, 0ull, 0u, 0u};
        if (tid < SG_WAVE) {
            un_runs_load(p, ts, sm.R[0]);
            un_runs_window(n, glog, sm.R[0]);
            rr = un_runs_issue(p, ts + 1);
        }
        __syncthreads();
        uint32_t ka[UN_PER], kb[UN_PER], vb[UN_PER], va = 0, vbb = 0;
        va = un_window_load<VM_NONE>(p, sm.R[0], glog, ka, vb);
        for (uint32_t t = ts; t < te; t += 2) {
            un_count_tile<WPT>(p, sm, t, te, glog, sm.R[0], sm.R[1], va, ka, vbb, kb, rr, total);
            if (t + 1 >= te) break;
            un_count_tile<WPT>(p, sm, t + 1, te, glog, sm.R[1], sm.R[0], vbb, kb, va, ka, rr, total);
        }
    }
    if (tid == 0) p.wave_tot[k] = total;
}

// LDS of the write pass.
template <int WPT>
struct UnWriteSmem {
    uint32_t bits[WPT * UN_THREADS];  // presence bitmap of the tile's span
    uint16_t wpre[WPT * UN_THREADS];  // distinct keys before each bitmap word
    float acc[UN_CAP];                // sums by rank
    uint32_t keys[UN_CAP];            // keys by rank
    uint32_t tot[(WPT >= 4 ? WPT / 4 : 1)][UN_WAVES]; // popcounts of a chunk round per wave
    UnRuns R;
};

// Keys (and sums) of each block's tiles at the block's offset.
template <int WPT, int VM>
__global__ __launch_bounds__(UN_THREADS) void un_write_kernel(MergeParams p)
{
    constexpr bool VALS = VM != VM_NONE;
    constexpr int NCH = WPT >= 4 ? WPT / 4 : 1;
    static_assert(WPT >= 4, "the write pass reads the bitmap as 16-byte chunks");
    __shared__ __align__(16) UnWriteSmem<WPT> sm;
    const uint32_t tid = threadIdx.x, lane = lane_id(), wid = tid / SG_WAVE;
    for (uint32_t i = tid; i < (uint32_t)(WPT * UN_THREADS); i += UN_THREADS) sm.bits[i] = 0u;
    for (uint32_t i = tid; i < (uint32_t)UN_CAP; i += UN_THREADS) sm.acc[i] = 0.0f;
    const uint32_t n = p.n, glog = un_glog(n);
    const uint32_t gmask = (1u << glog) - 1u;
    const uint32_t my_w = tid >> glog, my_s = tid & gmask;
    const uint32_t k = blockIdx.x;
    const uint32_t ts = p.wstart[k], te = p.wstart[k + 1];
    uint64_t out = p.wave_tot[k];
    const uint64_t out_end = p.wave_tot[k + 1];
    if (out_end < out || out_end > p.capacity) { // cannot happen: the union is no larger than the input
        if (tid == 0) report_error(kDevErrPartition);
        return; // uniform
    }
    const uint32_t span = 1u << p.tb;
    for (uint32_t t = ts; t < te; ++t) {
        if (t % p.NT == 0 && tid == 0) p.agg_off[t / p.NT] = out;
        un_runs_load(p, t, sm.R);
        const uint32_t klo = (t % p.NT) << p.tb;
        while (true) {
            un_runs_window(n, glog, sm.R);
            __syncthreads();
            uint32_t key[UN_PER], vb[UN_PER];
            uint32_t valid = un_window_load<VM>(p, sm.R, glog, key, vb);
            if (sm.R.cut) { // uniform: some run continues after the window
                // the window ends at the smallest last-loaded key of such a
                // run; later keys go back to their runs.  The last loaded
                // entry of run w is entry take_w - 1 of its part: slot
                // (take_w - 1) / g of thread w g + (take_w - 1) % g.
                if (my_w < n) {
                    const uint32_t tk = sm.R.take[my_w];
                    if (tk > 0 && tk < sm.R.rem[my_w] && ((tk - 1) & gmask) == my_s) {
                        uint32_t lk = 0;
#pragma unroll
                        for (int i = 0; i < UN_PER; ++i)
                            if ((uint32_t)i == ((tk - 1) >> glog)) lk = key[i];
                        atomicMin(&sm.R.kmax, lk);
                    }
                }
                __syncthreads();
                const uint32_t kmax = sm.R.kmax;
                uint32_t gone = 0;
#pragma unroll
                for (int i = 0; i < UN_PER; ++i) gone |= (key[i] > kmax ? 1u : 0u) << i;
                gone &= valid;
                valid &= ~gone;
                if (gone) atomicAdd(&sm.R.drop[my_w], (uint32_t)__popc(gone));
            }
            // presence bitmap of the window's keys
            uint32_t off[UN_PER];
            uint32_t inr = 0; // slots whose key lies in the tile
#pragma unroll
            for (int i = 0; i < UN_PER; ++i) {
                off[i] = key[i] - klo;
                inr |= (off[i] < span ? 1u : 0u) << i;
            }
            if (ballot((valid & ~inr) != 0u) && lane == 0) report_error(kDevErrIndexRange); // cannot happen
            valid &= inr;
#pragma unroll
            for (int i = 0; i < UN_PER; ++i)
                if ((valid >> i) & 1u) atomicOr(&sm.bits[off[i] >> 5], 1u << (off[i] & 31u));
            __syncthreads();
            un_runs_advance(n, sm.R); // wave 0; read after the next barrier
            // prefix popcounts of the bitmap words: 16-byte chunk q * 256 +
            // tid per thread and round; a wave scan per round, the waves'
            // round totals through LDS
            uint32_t c[NCH][4], inc[NCH];
#pragma unroll
            for (int q = 0; q < NCH; ++q) {
                const uint4 bw = *reinterpret_cast<const uint4*>(&sm.bits[4 * (q * UN_THREADS + tid)]);
                c[q][0] = __popc(bw.x);
                c[q][1] = __popc(bw.y);
                c[q][2] = __popc(bw.z);
                c[q][3] = __popc(bw.w);
                inc[q] = wave_incl_scan(c[q][0] + c[q][1] + c[q][2] + c[q][3]);
                if (lane == SG_WAVE - 1) sm.tot[q][wid] = inc[q];
            }
            __syncthreads();
            uint32_t U = 0;
#pragma unroll
            for (int q = 0; q < NCH; ++q) {
                uint32_t before = U; // everything of earlier rounds, then earlier waves of this round
#pragma unroll
                for (int v = 0; v < UN_WAVES; ++v) {
                    const uint32_t x = sm.tot[q][v];
                    if ((uint32_t)v < wid) before += x;
                    U += x;
                }
                const uint32_t e0 = before + inc[q] - (c[q][0] + c[q][1] + c[q][2] + c[q][3]);
                const uint32_t e1 = e0 + c[q][0], e2 = e1 + c[q][1], e3 = e2 + c[q][2];
                *reinterpret_cast<uint2*>(&sm.wpre[4 * (q * UN_THREADS + tid)]) =
                    make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
            }
            __syncthreads();
            // ranks; keys by rank; the sums, one wave after the other (the
            // waves hold the runs in order, so each sum is in worker order)
            uint32_t rk[UN_PER];
#pragma unroll
            for (int i = 0; i < UN_PER; ++i) {
                rk[i] = 0;
                if ((valid >> i) & 1u) {
                    const uint32_t wd = off[i] >> 5;
                    rk[i] = (uint32_t)sm.wpre[wd] + (uint32_t)__popc(sm.bits[wd] & ((1u << (off[i] & 31u)) - 1u));
                    sm.keys[rk[i]] = key[i]; // every holder of a key writes the same value
                }
            }
            if (VALS) {
#pragma unroll
                for (int v = 0; v < UN_WAVES; ++v) {
                    if ((uint32_t)v == wid) {
#pragma unroll
                        for (int i = 0; i < UN_PER; ++i)
                            if ((valid >> i) & 1u) atomicAdd(&sm.acc[rk[i]], un_value<VM>(vb[i]));
                    }
                    __syncthreads();
                }
            } else {
                __syncthreads();
            }
            // the block's slot holds the keys its count pass found (a run
            // that broke the input's order could make the passes disagree;
            // nothing is written past the slot)
            const uint64_t room = out_end - out;
            const uint32_t lim = room < U ? (uint32_t)room : U;
            for (uint32_t q = tid; q < U; q += UN_THREADS) {
                if (q < lim) {
                    p.agg_idx[out + q] = sm.keys[q];
                    if (VALS) p.agg_val[out + q] = sm.acc[q];
                }
                if (VALS) sm.acc[q] = 0.0f;
            }
#pragma unroll
            for (int q = 0; q < NCH; ++q)
                *reinterpret_cast<uint4*>(&sm.bits[4 * (q * UN_THREADS + tid)]) = make_uint4(0u, 0u, 0u, 0u);
            out += lim;
            const bool more = sm.R.more != 0;
            __syncthreads();
            if (!more) break;
        }
    }
    if (out != out_end && tid == 0) report_error(kDevErrPartition); // the two passes disagree: cannot happen
}

} // namespace sg

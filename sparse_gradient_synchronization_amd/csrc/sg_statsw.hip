// sg_statsw.hip -- the statistics pass of A6 over key windows, for up to 16
// workers and 16 hash classes (the common case; sg_stats falls back to the
// merge engine otherwise).
//
// Zen OSDI'25 digest, section 2.1 (Defs. 3-5) needs, from the workers' index
// sets, the size of their union, every pairwise intersection, and the union's
// count per contiguous part and per hash class; section 3.1 (Def. 8) the same
// per class.  None of it needs values or an ordered output, so the key space
// is cut into windows of 2048 keys, one bitmap word per lane of a wave (the
// code allows 2^SW_TB keys, SW_WPL words per lane; small windows keep the
// densest window, which one wave handles alone, short):
//
//   bits    the entries of each worker that fall in the window are loaded 64
//           at a time (slots of one worker's consecutive entries, found from
//           the boundary table of the merge engine) and set one bit each in
//           that worker's bitmap of the window (LDS);
//   counts  lane j reads its words (j, j+64, ...) of every worker's bitmap;
//           a union word is
//           their OR; |I_a & I_b| accumulates popcount(W_a & W_b) for every
//           pair in registers; the union's hash classes come from the class
//           map's bit planes of the same 32 keys (a class mask is an AND of
//           planes or their complements), its contiguous parts from the keys'
//           positions.
//
// Each wave takes a contiguous range of windows of about equal work and
// writes one partial row of counts at its end; a last pass sums the rows.
// The next window's boundaries and first slots are loaded before the current
// window is counted.
#include "sg_host.h"

namespace sg {

constexpr int SW_WAVES = 4;
constexpr int SW_THREADS = SW_WAVES * SG_WAVE;
constexpr int SW_SLOTS = 8;              // slots (64 entries of one worker) per round
constexpr uint32_t SW_TB = 11;           // windows of 2^11 keys: 64 words, one per lane
constexpr int SW_WPL = (1 << SW_TB) / 32 / SG_WAVE;
constexpr int SW_MAXN = 16;              // workers
constexpr int SW_MAXP = 16;              // hash classes (contiguous parts: any P <= 256)
constexpr uint32_t SW_FIXED = 3;         // work of a window beyond its rounds, in rounds
constexpr uint32_t SW_MAX_WAVES = 16384; // persistent waves, at most

struct SwParams {
    MergeParams m;          // runs (G = 1), boundary table, tb = SW_TB
    const uint32_t* planes; // class map bit planes [chunk][stride], or null
    uint32_t nbits, stride;
    uint32_t* wstart;       // [W+1] first window of each wave
    uint64_t* wtotal;       // [1] total work
    uint32_t* work;         // [NT] work of each window
    uint64_t* wcum;         // [NT] exclusive prefix of the work inside its scan block
    uint64_t* wblk;         // [nscan] scan block prefix
    uint64_t* rows;         // [W][st_row] partial rows
};

// A window's layout, one value per lane w < n (lanes >= n: empty runs).
struct SwLay {
    uint64_t src;  // absolute position of worker w's first entry in the window
    uint32_t cnt;  // worker w's entries in the window
    uint32_t ps;   // slots of workers before w
    uint32_t NS;   // slots of the window (uniform)
};

struct SwBnd {
    uint64_t a, e; // the worker's list
    uint32_t x, y; // the window's boundaries inside it
};

// The boundary loads of window t (unconditional, clamped addresses; nothing
// is computed from them until sw_finish, so they stay in flight).
__device__ __forceinline__ void sw_issue(const MergeParams& p, uint32_t t, uint32_t lane, SwBnd& r)
{
    const uint32_t tc = t < p.NT ? t : p.NT - 1;
    const uint32_t w = lane < p.n ? lane : p.n - 1;
    r.a = p.off[w];
    r.e = p.off[w + 1];
    const uint32_t* row = p.bnd + (uint64_t)w * (p.NT + 1);
    r.x = row[tc];
    r.y = row[tc + 1];
}

__device__ __forceinline__ SwLay sw_finish(const MergeParams& p, uint32_t t, uint32_t lane, const SwBnd& r)
{
    uint64_t a = r.a, e = r.e;
    if (a > p.total) a = p.total;
    if (e > p.total) e = p.total;
    if (e < a) e = a;
    const uint64_t len = e - a;
    uint64_t x = r.x, y = r.y;
    if (x > len) x = len;
    if (y > len) y = len;
    if (y < x) y = x;
    SwLay L;
    L.cnt = (lane < p.n && t < p.NT) ? (uint32_t)(y - x) : 0u;
    L.src = a + x;
    const uint32_t cs = (L.cnt + SG_WAVE - 1) / SG_WAVE;
    const uint32_t incl = wave_incl_scan(cs);
    L.ps = incl - cs;
    L.NS = (uint32_t)__builtin_amdgcn_readlane((int)incl, SG_WAVE - 1);
    return L;
}

__device__ __forceinline__ uint64_t sw_readlane64(uint64_t v, int l)
{
    return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l) |
           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l) << 32);
}

// Keys of round r of a window: slot s of the round is slot q = r*SW_SLOTS + s
// of the window, entries 64*j .. 64*j+63 of worker w (the last worker whose
// first slot is at or before q; j = q - ps_w).  run[s] = w (uniform), cnt[s]
// the valid lanes (0 past the window's end, where entry 0 is read: the caller
// launches only with total > 0).  All loads are issued before any is used.
__device__ __forceinline__ void sw_load(const MergeParams& p, const SwLay& L, uint32_t r, uint32_t lane,
                                        uint32_t (&key)[SW_SLOTS], uint32_t (&run)[SW_SLOTS],
                                        uint32_t (&cnt)[SW_SLOTS])
{
    uint64_t pos[SW_SLOTS];
#pragma unroll
    for (int s = 0; s < SW_SLOTS; ++s) {
        const uint32_t q = r * (uint32_t)SW_SLOTS + (uint32_t)s;
        const uint64_t m = ballot(lane < p.n && L.ps <= q);
        const uint32_t w = 63u - (uint32_t)__builtin_clzll(m | 1ull);
        const uint32_t j = q - (uint32_t)__builtin_amdgcn_readlane((int)L.ps, (int)w);
        const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)L.cnt, (int)w);
        const uint64_t src = sw_readlane64(L.src, (int)w);
        const bool live = q < L.NS;
        const uint32_t left = live ? c - j * SG_WAVE : 0u;
        cnt[s] = left < (uint32_t)SG_WAVE ? left : (uint32_t)SG_WAVE;
        run[s] = w;
        const uint32_t l = lane < cnt[s] ? lane : (cnt[s] ? cnt[s] - 1 : 0u);
        pos[s] = live ? src + (uint64_t)j * SG_WAVE + l : 0ull;
    }
#pragma unroll
    for (int s = 0; s < SW_SLOTS; ++s) key[s] = p.idx[pos[s]];
}

// Work of a window (its rounds of slots plus a fixed cost: a window's set-up
// and counts cost about three rounds), for the balance of waves.
__global__ __launch_bounds__(256) void sw_weight_kernel(SwParams sp)
{
    const MergeParams& p = sp.m;
    for (uint32_t t = blockIdx.x * 256 + threadIdx.x; t < p.NT; t += gridDim.x * 256) {
        uint32_t NS = 0;
        for (uint32_t w = 0; w < p.n; ++w) {
            uint64_t s, e;
            run_range(p, 0, w, s, e);
            const uint64_t len = e - s;
            const uint32_t* row = p.bnd + (uint64_t)w * (p.NT + 1);
            uint64_t x = row[t], y = row[t + 1];
            if (x > len) x = len;
            if (y > len) y = len;
            NS += y > x ? (uint32_t)((y - x + SG_WAVE - 1) / SG_WAVE) : 0u;
        }
        sp.work[t] = (NS + SW_SLOTS - 1) / SW_SLOTS + SW_FIXED;
    }
}

// exclusive prefix of the window work inside scan blocks of MG_SCAN_BLOCK windows
__global__ __launch_bounds__(1024) void sw_scan_local_kernel(SwParams sp)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    const uint32_t T = sp.m.NT;
    const uint64_t t0 = (uint64_t)blockIdx.x * MG_SCAN_BLOCK + (uint64_t)threadIdx.x * MG_SCAN_PER;
    uint32_t c[MG_SCAN_PER];
    uint64_t sum = 0;
#pragma unroll
    for (int j = 0; j < MG_SCAN_PER; ++j) {
        c[j] = t0 + j < T ? sp.work[t0 + j] : 0u;
        sum += c[j];
    }
    uint64_t tot;
    uint64_t ex = block_excl_scan64<1024>(sum, scan_lds, &tot);
#pragma unroll
    for (int j = 0; j < MG_SCAN_PER; ++j) {
        if (t0 + j < T) sp.wcum[t0 + j] = ex;
        ex += c[j];
    }
    if (threadIdx.x == 0) sp.wblk[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void sw_scan_top_kernel(SwParams sp, uint32_t nscan)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    uint64_t carry = 0;
    for (uint32_t base = 0; base < nscan; base += 1024) {
        const uint32_t i = base + threadIdx.x;
        const uint64_t v = i < nscan ? sp.wblk[i] : 0ull;
        uint64_t tot;
        const uint64_t ex = block_excl_scan64<1024>(v, scan_lds, &tot);
        if (i < nscan) sp.wblk[i] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) *sp.wtotal = carry;
}

// Wave k of W takes the windows whose cumulative work starts in
// [k*C/W, (k+1)*C/W): wstart[k] is its first window, wstart[W] = NT.  The
// thread of window t writes wstart[k] for k(t-1) < k <= k(t), with
// k(t) = floor(cum[t]*W/C), so every k is written once.
__global__ __launch_bounds__(256) void sw_starts_kernel(SwParams sp, uint32_t W)
{
    const uint32_t T = sp.m.NT;
    const uint64_t C = *sp.wtotal;
    for (uint32_t t = blockIdx.x * 256 + threadIdx.x; t < T; t += gridDim.x * 256) {
        const uint64_t cum = sp.wcum[t] + sp.wblk[t / MG_SCAN_BLOCK];
        const uint64_t kt = C ? cum * W / C : 0;
        int64_t kp = -1;
        if (t > 0) {
            const uint64_t cp = sp.wcum[t - 1] + sp.wblk[(t - 1) / MG_SCAN_BLOCK];
            kp = (int64_t)(C ? cp * W / C : 0);
        }
        for (int64_t k = kp + 1; k <= (int64_t)kt && k < (int64_t)W; ++k) sp.wstart[k] = t;
        if (t == T - 1)
            for (uint64_t k = kt + 1; k <= W; ++k) sp.wstart[k] = T;
    }
}

template <int N>
struct SwSmem {
    uint32_t bw[N][SW_WPL * SG_WAVE]; // worker bitmaps of the window
    uint32_t part[256];            // union count per contiguous part
};

// The class map's bit planes of the lane's words of window t (HASHED:
// 1 <= nbits <= 4; addresses clamped).
__device__ __forceinline__ void sw_planes(const SwParams& sp, uint32_t t, uint32_t lane, uint32_t (&pl)[SW_WPL][4])
{
    const uint64_t nc = ((uint64_t)sp.m.M + 31) / 32;
#pragma unroll
    for (int i = 0; i < SW_WPL; ++i) {
        uint64_t c = ((uint64_t)t << (SW_TB - 5)) + (uint64_t)i * SG_WAVE + lane;
        if (c > nc) c = nc;
        if (sp.stride == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(sp.planes + c * 4);
            pl[i][0] = v.x;
            pl[i][1] = v.y;
            pl[i][2] = v.z;
            pl[i][3] = v.w;
        } else {
#pragma unroll
            for (uint32_t b = 0; b < 4; ++b) pl[i][b] = sp.planes[c * sp.stride + (b < sp.nbits ? b : sp.nbits - 1)];
        }
    }
}

// The statistics pass.  N (8 or 16) bounds the workers at compile time, so
// the pair counters stay in registers; words of workers >= n are zero.
// HASHED: count the union per hash class from the class map (2 <= P <= 16).
template <int N, bool HASHED>
__global__ __launch_bounds__(SW_THREADS) void sw_stats_kernel(SwParams sp)
{
    __shared__ SwSmem<N> smem[SW_WAVES];
    const MergeParams& p = sp.m;
    const uint32_t wid = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x / SG_WAVE));
    const uint32_t lane = lane_id();
    SwSmem<N>& sm = smem[wid];
    const uint32_t k = blockIdx.x * SW_WAVES + wid;
    const uint32_t T = p.NT;
    const uint32_t t1 = sp.wstart[k + 1] < T ? sp.wstart[k + 1] : T;
    const uint32_t t0 = sp.wstart[k] < t1 ? sp.wstart[k] : t1;
    constexpr int NP = N * (N - 1) / 2;

    uint32_t pacc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) pacc[i] = 0;
    uint32_t hacc[SW_MAXP];
#pragma unroll
    for (int i = 0; i < SW_MAXP; ++i) hacc[i] = 0;
    uint32_t uacc = 0;
    for (uint32_t i = lane; i < p.Ps; i += SG_WAVE) sm.part[i] = 0;
#pragma unroll
    for (int a = 0; a < N; ++a)
#pragma unroll
        for (int i = 0; i < SW_WPL; ++i) sm.bw[a][i * SG_WAVE + lane] = 0;
    wave_sync();

    if (t0 < t1) {
        SwBnd bn;
        sw_issue(p, t0, lane, bn);
        SwLay Lc = sw_finish(p, t0, lane, bn);
        sw_issue(p, t0 + 1 < t1 ? t0 + 1 : T, lane, bn);
        uint32_t key[SW_SLOTS], run[SW_SLOTS], cnt[SW_SLOTS];
        uint32_t nkey[SW_SLOTS], nrun[SW_SLOTS], ncnt[SW_SLOTS];
        sw_load(p, Lc, 0, lane, key, run, cnt);
        SwLay Ln = Lc;
        uint32_t pl4[SW_WPL][4];
        uint32_t t = t0, r = 0;
        while (true) {
            const uint32_t R = (Lc.NS + SW_SLOTS - 1) / SW_SLOTS;
            const uint32_t klo = t << SW_TB;
            if (r == 0) { // a window starts: lay out the next one, fetch the one after
                Ln = sw_finish(p, t + 1 < t1 ? t + 1 : T, lane, bn);
                sw_issue(p, t + 2 < t1 ? t + 2 : T, lane, bn);
                if (HASHED) sw_planes(sp, t, lane, pl4); // used at the window's end
            }
            const bool last = r + 1 >= R;
            const uint32_t tn = last ? t + 1 : t, rn = last ? 0u : r + 1;
            const bool more = tn < t1;
            if (more) {
                SwLay Lv; // by value: a reference to either would put both in memory
                Lv.src = last ? Ln.src : Lc.src;
                Lv.cnt = last ? Ln.cnt : Lc.cnt;
                Lv.ps = last ? Ln.ps : Lc.ps;
                Lv.NS = last ? Ln.NS : Lc.NS;
                sw_load(p, Lv, rn, lane, nkey, nrun, ncnt);
            }
            // the slots of this round: one bit per entry in its worker's bitmap
            bool stray = false;
#pragma unroll
            for (int s = 0; s < SW_SLOTS; ++s) {
                const uint32_t o = key[s] - klo;
                const bool in = lane < cnt[s] && key[s] >= klo && o < (1u << SW_TB);
                stray |= lane < cnt[s] && !in;
                if (in) atomicOr(&sm.bw[run[s]][o >> 5], 1u << (o & 31u));
            }
            if (stray) report_error(kDevErrIndexRange);
            if (last) {
                wave_sync();
                // counts of the window: lane l, words l + 64 i (keys klo + 32 word ..)
                uint32_t usum = 0;
                const uint32_t pf = contig_part(klo, p.M, p.Ps, p.inv_m);
                const uint64_t wl = (uint64_t)klo + (1u << SW_TB) - 1;
                const uint32_t pl = contig_part(wl < p.M ? wl : p.M - 1, p.M, p.Ps, p.inv_m);
#pragma unroll
                for (int i = 0; i < SW_WPL; ++i) {
                    const uint32_t wi = (uint32_t)i * SG_WAVE + lane;
                    uint32_t Wd[N];
                    uint32_t U = 0;
#pragma unroll
                    for (int a = 0; a < N; ++a) {
                        Wd[a] = sm.bw[a][wi];
                        U |= Wd[a];
                    }
#pragma unroll
                    for (int a = 0; a < N; ++a) sm.bw[a][wi] = 0;
                    usum += __popc(U);
                    int pi = 0;
#pragma unroll
                    for (int a = 0; a < N; ++a)
#pragma unroll
                        for (int b = a + 1; b < N; ++b) pacc[pi++] += __popc(Wd[a] & Wd[b]);
                    if (pf != pl) { // the window crosses a part boundary: part by key
                        const uint64_t kw = (uint64_t)klo + 32u * wi;
                        uint32_t rest = U;
                        while (rest) {
                            const uint32_t bit = __builtin_ctz(rest);
                            rest &= rest - 1;
                            atomicAdd(&sm.part[contig_part(kw + bit, p.M, p.Ps, p.inv_m)], 1u);
                        }
                    }
                    // hash classes of the union, from the class map's planes
                    if (HASHED) {
#pragma unroll
                        for (int c = 0; c < SW_MAXP; ++c) {
                            uint32_t m = U;
#pragma unroll
                            for (uint32_t b = 0; b < 4; ++b)
                                if (b < sp.nbits) m &= ((c >> b) & 1) ? pl4[i][b] : ~pl4[i][b];
                            hacc[c] += (uint32_t)c < p.Ps ? __popc(m) : 0u;
                        }
                    }
                }
                uacc += usum;
                if (pf == pl) { // the whole window lies in one part: one add
                    const uint32_t c = wave_sum(usum);
                    if (lane == 0 && c) atomicAdd(&sm.part[pf], c);
                }
                wave_sync();
            }
            if (!more) break;
            if (last) {
                Lc.src = Ln.src;
                Lc.cnt = Ln.cnt;
                Lc.ps = Ln.ps;
                Lc.NS = Ln.NS;
            }
            t = tn;
            r = rn;
            static_assert(SW_SLOTS == 8, "the copy below is written out for 8 slots");
#define SW_MOVE(q) do { key[q] = nkey[q]; run[q] = nrun[q]; cnt[q] = ncnt[q]; } while (0)
            SW_MOVE(0); SW_MOVE(1); SW_MOVE(2); SW_MOVE(3); SW_MOVE(4); SW_MOVE(5); SW_MOVE(6); SW_MOVE(7);
#undef SW_MOVE
        }
    }

    // this wave's partial row: pairs (a <= b; the diagonal is left 0, the
    // host takes it from the list lengths), union, contiguous parts, classes
    wave_sync();
    uint64_t* row = sp.rows + (uint64_t)k * p.st_row;
    {
        int pi = 0;
        uint32_t ri = 0;
#pragma unroll
        for (uint32_t a = 0; a < (uint32_t)N; ++a) {
#pragma unroll
            for (uint32_t b = a; b < (uint32_t)N; ++b) {
                uint32_t v = 0;
                if (b > a) {
#pragma unroll
                    for (int q = 0; q < NP; ++q)
                        if (q == pi) v = pacc[q];
                    ++pi;
                }
                const uint32_t s = wave_sum(v);
                if (a < p.n && b < p.n) {
                    if (lane == 0) row[ri] = s;
                    ++ri;
                }
            }
        }
    }
    const uint32_t us = wave_sum(uacc);
    if (lane == 0) row[p.npairs] = us;
    for (uint32_t i = lane; i < p.Ps; i += SG_WAVE) row[p.npairs + 1 + i] = sm.part[i];
#pragma unroll
    for (int i = 0; i < SW_MAXP; ++i) {
        const uint32_t s = wave_sum(hacc[i]);
        if ((uint32_t)i < p.Ps && lane == 0) row[p.npairs + 1 + p.Ps + i] = HASHED ? s : 0u;
    }
}

} // namespace sg

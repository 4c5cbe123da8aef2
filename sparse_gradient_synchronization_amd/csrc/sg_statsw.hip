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
// Tiles are taken the way the union engine takes them (sg_union.hip): wave
// k of NW takes windows k, k + NW, ..., the next window's run ranges are
// loaded while the current one is counted, and a window's entries are the
// workers' parts laid end to end (no lane is idle on a sparse worker).  Each
// wave writes one partial row of counts at its end; a last pass sums the
// rows.
#include "sg_host.h"

namespace sg {

constexpr int SW_WAVES = 4;
constexpr int SW_THREADS = SW_WAVES * SG_WAVE;
constexpr uint32_t SW_TB = 11;           // windows of 2^11 keys: 64 words, one per lane
constexpr int SW_MAXN = 16;              // workers
constexpr int SW_MAXP = 16;              // hash classes (contiguous parts: any P <= 256)
constexpr uint32_t SW_MAX_WAVES = 16384; // persistent waves, at most
constexpr uint32_t SW_FLUSH = 1024;      // windows between flushes of the 16-bit pair counters
static_assert((1u << SW_TB) == 32u * SG_WAVE, "one bitmap word per lane");

struct SwParams {
    MergeParams m;          // runs (G = 1), boundary table, tb = SW_TB
    const uint32_t* planes; // class map bit planes [chunk][stride], or null
    uint32_t nbits, stride;
    uint64_t* rows;         // [W][st_row] partial rows
};

template <int N, int S>
struct SwSmem {
    uint32_t bw[N][SG_WAVE];   // worker bitmaps of the window
    uint32_t part[256];        // union count per contiguous part
    uint32_t pairs[N * (N - 1) / 2 + 1]; // flushed pair counts
    UnTables<S, true> tb;      // window tables, the parts' workers, the next window's parts
};

// The class map's bit planes of the lane's 32 keys of window t (1 <= nbits
// <= 4; the chunk clamped to the map).
__device__ __forceinline__ void sw_planes(const SwParams& sp, uint32_t t, uint32_t lane, uint32_t (&pl)[4])
{
    const uint64_t nc = ((uint64_t)sp.m.M + 31) / 32;
    uint64_t c = ((uint64_t)t << (SW_TB - 5)) + lane;
    if (c > nc) c = nc;
    if (sp.stride == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(sp.planes + c * 4);
        pl[0] = v.x;
        pl[1] = v.y;
        pl[2] = v.z;
        pl[3] = v.w;
    } else {
#pragma unroll
        for (uint32_t b = 0; b < 4; ++b) pl[b] = sp.planes[c * sp.stride + (b < sp.nbits ? b : sp.nbits - 1)];
    }
}

// The statistics pass.  N (8 or 16) bounds the workers at compile time, so
// the pair counters stay in registers (two 16-bit counters to a register,
// flushed to LDS every SW_FLUSH windows: a lane adds at most 32 per window);
// words of workers >= n are zero.  HASHED: count the union per hash class
// from the class map (2 <= P <= 16).
template <int N, bool HASHED>
__global__ __launch_bounds__(SW_THREADS) void sw_stats_kernel(SwParams sp)
{
    constexpr int S = N <= 8 ? 16 : 8; // entry slots per lane of a window round
    constexpr int NP = N * (N - 1) / 2;
    constexpr int NQ = (NP + 1) / 2;
    __shared__ __align__(16) SwSmem<N, S> smem[SW_WAVES];
    const MergeParams& p = sp.m;
    const uint32_t wid = uniform(threadIdx.x / SG_WAVE), lane = lane_id();
    SwSmem<N, S>& sm = smem[wid];
    const uint32_t k = blockIdx.x * SW_WAVES + wid;
    const uint32_t T = p.NT, NW = gridDim.x * SW_WAVES;
    constexpr uint32_t span = 1u << SW_TB;

    uint32_t pk[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) pk[i] = 0;
    uint32_t hacc[SW_MAXP];
#pragma unroll
    for (int i = 0; i < SW_MAXP; ++i) hacc[i] = 0;
    uint32_t uacc = 0;
    for (uint32_t i = lane; i < p.Ps; i += SG_WAVE) sm.part[i] = 0;
    for (uint32_t i = lane; i <= (uint32_t)NP; i += SG_WAVE) sm.pairs[i] = 0;
#pragma unroll
    for (int a = 0; a < N; ++a) sm.bw[a][lane] = 0;
    auto flush = [&]() {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const uint32_t sq = wave_sum((pk[q >> 1] >> (16 * (q & 1))) & 0xffffu);
            if (lane == 0) sm.pairs[q] += sq;
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) pk[i] = 0;
    };

    uint32_t t = k, done = 0;
    if (t < T) {
        un_stash<false>(p, sm.tb, un_raw_issue<false>(p, t));
        for (; t < T; t += NW) { // uniform
            wave_sync();
            uint32_t pos = sm.tb.npos[lane], rem = sm.tb.nrem[lane];
            wave_sync();
            const URaw nxt = un_raw_issue<false>(p, t + NW < T ? t + NW : t); // unconditional: no register merge
            uint32_t pl4[4] = {0u, 0u, 0u, 0u};
            if (HASHED) sw_planes(sp, t, lane, pl4); // used at the window's end
            const uint32_t klo = t << SW_TB;
            uint32_t rtot = wave_sum(rem);
            if (rtot == 0) { // uniform: an empty window adds nothing
                un_stash<false>(p, sm.tb, nxt);
                if (HASHED) un_hold(pl4);
                continue;
            }
            bool stray = false;
            do {
                uint32_t take, kr, key[S], vb[S], part[S];
                uint64_t sbs[S];
                const uint32_t E = un_window<S, VM_NONE>(p, sm.tb, pos, rem, rtot, take, kr, key, vb, part, sbs);
                un_hold(key);
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    const uint32_t o = key[i] - klo;
                    const bool has = lane + (uint32_t)i * SG_WAVE < E;
                    stray |= has && o >= span; // outside the window: cannot happen for valid input
                    if (has && o < span) {
                        const uint32_t a = sm.tb.wk[part[i]];
                        atomicOr(&sm.bw[a < (uint32_t)N ? a : N - 1][o >> 5], 1u << (o & 31u));
                    }
                }
                un_stash<false>(p, sm.tb, nxt);
                pos += take;
                rem -= take;
                rtot -= E;
            } while (rtot > 0);
            if (ballot(stray) && lane == 0) report_error(kDevErrIndexRange);
            wave_sync();
            // counts of the window: lane l, word l (keys klo + 32 l ..)
            const uint32_t pf = contig_part(klo, p.M, p.Ps, p.inv_m);
            const uint64_t wl = (uint64_t)klo + span - 1;
            const uint32_t plast = contig_part(wl < p.M ? wl : p.M - 1, p.M, p.Ps, p.inv_m);
            uint32_t Wd[N];
            uint32_t U = 0;
#pragma unroll
            for (int a = 0; a < N; ++a) {
                Wd[a] = sm.bw[a][lane];
                U |= Wd[a];
            }
#pragma unroll
            for (int a = 0; a < N; ++a) sm.bw[a][lane] = 0;
            const uint32_t usum = (uint32_t)__popc(U);
            int pi = 0;
#pragma unroll
            for (int a = 0; a < N; ++a)
#pragma unroll
                for (int b = a + 1; b < N; ++b, ++pi) pk[pi >> 1] += (uint32_t)__popc(Wd[a] & Wd[b]) << (16 * (pi & 1));
            if (pf != plast) { // the window crosses a part boundary: part by key
                const uint64_t kw = (uint64_t)klo + 32u * lane;
                uint32_t rest = U;
                while (rest) {
                    const uint32_t bit = __builtin_ctz(rest);
                    rest &= rest - 1;
                    atomicAdd(&sm.part[contig_part(kw + bit, p.M, p.Ps, p.inv_m)], 1u);
                }
            } else { // the whole window lies in one part: one add
                const uint32_t c = wave_sum(usum);
                if (lane == 0 && c) atomicAdd(&sm.part[pf], c);
            }
            // hash classes of the union, from the class map's planes
            if (HASHED) {
#pragma unroll
                for (int c = 0; c < SW_MAXP; ++c) {
                    uint32_t m = U;
#pragma unroll
                    for (uint32_t b = 0; b < 4; ++b)
                        if (b < sp.nbits) m &= ((c >> b) & 1) ? pl4[b] : ~pl4[b];
                    hacc[c] += (uint32_t)c < p.Ps ? (uint32_t)__popc(m) : 0u;
                }
            }
            uacc += usum;
            if (++done == SW_FLUSH) { // uniform
                flush();
                done = 0;
            }
        }
    }
    flush();

    // this wave's partial row: pairs (a <= b; the diagonal is left 0, the
    // host takes it from the list lengths), union, contiguous parts, classes
    wave_sync();
    uint64_t* row = sp.rows + (uint64_t)k * p.st_row;
    {
        int pi = 0;
        uint32_t ri = 0;
        for (uint32_t a = 0; a < p.n; ++a) {
            for (uint32_t b = a; b < p.n; ++b) {
                const uint32_t v = b > a ? sm.pairs[pi++] : 0u;
                if (lane == 0) row[ri] = v;
                ++ri;
            }
            pi += N - p.n; // the pairs (a, b) with b >= n
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

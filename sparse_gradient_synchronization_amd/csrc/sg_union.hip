// sg_union.hip -- the union-sum of A3 for scalar values and bare indices
// (D <= 1): per partition, the union of the n workers' sorted runs with the
// values of each index summed (the server side of Push in the Zen OSDI'25
// digest, section 3.1; equal to the dense AllReduce, section 3.2).
//
// The key space of every partition is cut into tiles of 2^tb keys (a few
// hundred entries on average); the merge engine's boundary pass
// (sg_merge.hip) records where each tile starts in each run.  A wave owns a
// whole tile at a time, with no block barrier and no global atomic: the waves
// of the grid take tiles t = k, k + NW, k + 2 NW, ... (k the wave's number,
// NW the waves of the grid), and the run ranges of a wave's next tile are
// loaded while it works on the current one.  Two passes:
//   count  the tile's keys OR-ed into an LDS presence bitmap of its span; the
//          popcount is the tile's union size.  A scan of the sizes gives
//          every tile its output offset (and every partition its start).
//   write  the tile's entries again, with their values: the bitmap and its
//          prefix popcounts give each entry the rank of its key, the keys go
//          to an LDS slot per rank and the values are added there, in worker
//          order (below); keys and sums are then written once, in order, at
//          the tile's offset, with consecutive lanes on consecutive
//          addresses.
// A window holds at most 64 S entries (S = 8 slots per lane in both passes;
// 16 in the count pass was slower on sparse spans): the run parts of the tile laid end to end, lane
// l taking entries l, l + 64, l + 128, ... of the window, so every load
// instruction reads 256 consecutive bytes (split only where one run's part
// ends and the next begins).  A tile with more entries is taken in several
// windows, each run giving a share in proportion to what it has left; in the
// write pass such a window ends at the smallest last-loaded key of the runs
// it cut short (later entries go back to their runs), so every key is whole
// inside one window.
//
// Both passes are bound by instruction issue, not by memory: the code keeps
// the instructions per entry few (part lookup by mbcnt over part-end marks,
// invalid slots folded into an out-of-span offset, bitmap word and prefix
// read together).  LDS float atomics are avoided: they cost far more than
// the plain read-add-write rounds used instead.
#include "sg_host.h"

namespace sg {

constexpr int UN_WPB = 4;                    // waves per block (each on tiles of its own)
constexpr int UN_THREADS = UN_WPB * SG_WAVE; // threads per block
constexpr int UN_SC = 8;                     // entry slots per lane, count pass
constexpr int UN_SW = 8;                     // entry slots per lane, write pass
constexpr int UN_CAP = UN_SW * SG_WAVE;      // entries of a write window (distinct keys of a window, at most)
#ifndef SG_UN_TARGET
#define SG_UN_TARGET 320
#endif
constexpr int UN_TARGET = SG_UN_TARGET;      // mean entries per tile aimed at
constexpr int UN_SPAN_LOG_MAX = 16;          // a tile spans at most 2^16 keys (32 bitmap words per lane)
static_assert(UN_CAP >= 2 * SG_WAVE, "a window must hold one entry of each of up to 64 runs and more");
static_assert(UN_CAP < 65536, "ranks inside a window fit in the bitmap prefix words");

// Value modes: VM_NONE (indices only), VM_F32, VM_BF16 (widened to fp32 where
// the values are added, so the loaded registers are not touched before).
constexpr int VM_NONE = 0, VM_F32 = 1, VM_BF16 = 2;

template <int VM>
__device__ __forceinline__ float un_value(uint32_t b)
{
    return __uint_as_float(VM == VM_BF16 ? b << 16 : b);
}

// Window tables and the next tile's parts, shared by both passes (WK: with
// the run of every part, for callers that need it).
template <int S, bool WK = false>
struct UnTables {
    uint32_t sb[2 * S];        // bit j set where entry j + 1 of the window begins a part
    uint32_t base[SG_WAVE];    // k-th non-empty part: its first position minus its window start
    uint32_t drop[SG_WAVE];    // entries of the k-th part returned by a cut window
    uint32_t npos[SG_WAVE];    // the next tile: lane w's part, its position
    uint32_t nrem[SG_WAVE];    // and length
    uint32_t wk[WK ? SG_WAVE : 1]; // k-th non-empty part: its run (worker)
    uint64_t nout, nend;       // the next tile's output slot (write pass)
};

// LDS of a wave in the count pass: the presence bitmap of the tile's span.
template <int WPL>
struct UnCountWave {
    uint32_t bits[WPL * SG_WAVE];
    UnTables<UN_SC> tb;
};

// LDS of a wave in the write pass: bitmap word w with the distinct keys
// before it (read together when an entry is ranked), keys and sums by rank.
template <int WPL>
struct UnWriteWave {
    uint2 bw[WPL * SG_WAVE];
    uint32_t keys[UN_CAP];
    float acc[UN_CAP];
    UnTables<UN_SW> tb;
};

// The raw run ranges of tile t in the lanes below n (lanes past n repeat run
// n-1) and the tile's output slot (write pass), issued without waiting;
// un_raw_put clamps the ranges once they are needed.
struct URaw {
    uint64_t a, e;  // the run's absolute range
    uint32_t x, y;  // the tile's part, relative to the run
    uint64_t out;   // the tile's output offset inside its scan block, then the block's
    uint64_t blk;
    uint32_t cnt;   // the tile's union size
};

template <bool WRITE>
__device__ __forceinline__ URaw un_raw_issue(const MergeParams& p, uint32_t t)
{
    const uint32_t w = lane_id();
    const uint32_t ww = w < p.n ? w : p.n - 1;
    const uint32_t g = t / p.NT, b = t % p.NT;
    URaw r;
    r.a = p.off[(uint64_t)ww * p.stride + g];
    r.e = p.off[(uint64_t)ww * p.stride + g + 1];
    const uint32_t* row = p.bnd + ((uint64_t)g * p.n + ww) * (p.NT + 1);
    r.x = row[b];
    r.y = row[b + 1];
    r.out = r.blk = 0;
    r.cnt = 0;
    if (WRITE) { // every lane (one request): a load under a branch would be copied, and waited for, at once
        r.out = p.tile_out[t];
        r.blk = p.blk_sum[t / MG_SCAN_BLOCK];
        r.cnt = p.tile_cnt[t];
    }
    return r;
}

// Marks loaded registers as used here, so their wait is taken on every path:
// a load whose first use sits under a branch some paths skip stays pending
// on those paths, and the register's next write then waits for every
// vector memory operation in flight (prefetches and stores included).
template <int N>
__device__ __forceinline__ void un_hold(uint32_t (&r)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

// lane w < n: the part's absolute start and length (empty in the other lanes)
__device__ __forceinline__ void un_raw_put(const MergeParams& p, const URaw& r, uint32_t& pos, uint32_t& rem)
{
    uint64_t a = r.a > p.total ? p.total : r.a, e = r.e > p.total ? p.total : r.e;
    if (e < a) e = a;
    const uint64_t len = e - a;
    uint64_t x = r.x > len ? len : r.x, y = r.y > len ? len : r.y;
    if (y < x) y = x;
    const bool mine = lane_id() < p.n;
    pos = mine ? (uint32_t)(a + x) : 0u;
    rem = mine ? (uint32_t)(y - x) : 0u;
}

// The next tile's parts and output slot, from the prefetched registers into
// LDS.  The compiler waits for those loads here; a window calls this once
// its own loads (issued after the prefetch) have been used, so the wait
// costs nothing.  Kept in registers until the next tile, they would be
// copied between registers at the top of the tile loop, and a copy of a
// pending load waits for every vector memory operation in flight, the
// tile's output stores included (loads and stores share one counter).
template <bool WRITE, int S, bool WK>
__device__ __forceinline__ void un_stash(const MergeParams& p, UnTables<S, WK>& tb, const URaw& nxt)
{
    // every vector memory operation issued before the window's loads is
    // done once those loads are (they complete in order), so this wait is
    // free here and leaves nothing pending for the compiler to wait for later
    wait_vmem();
    // a copy marked as changed here, so nothing computed from it is moved
    // ahead of this point
    URaw r = nxt;
    asm volatile("" : "+v"(r.a), "+v"(r.e), "+v"(r.x), "+v"(r.y));
    if (WRITE) asm volatile("" : "+v"(r.out), "+v"(r.blk), "+v"(r.cnt));
    uint32_t pos, rem;
    un_raw_put(p, r, pos, rem);
    const uint32_t lane = lane_id();
    tb.npos[lane] = pos;
    tb.nrem[lane] = rem;
    if (WRITE && lane == 0) {
        tb.nout = r.out + r.blk;
        tb.nend = r.out + r.blk + r.cnt;
    }
}

// One window of a tile.  In: the run parts left (lane w < n: position `pos`,
// `rem` entries; rtot = their sum > 0, wave-uniform).  Takes `take` entries
// of every part (all of them when they fit, else a share), lays them end to
// end and loads entry j = l + 64 i into slot i of lane l: keys, and values
// unless VM is VM_NONE.  Returns the window's entry count E (slots with
// j >= E hold no entry).  part[i] is the entry's part (its place among the
// non-empty parts, in worker order; `kr` is the lane's own), sbs[i] the
// slot's part-end marks.  The loaded registers are not touched here, so the
// loads stay in flight together until their first use.
template <int S, int VM, bool WK>
__device__ __forceinline__ uint32_t un_window(const MergeParams& p, UnTables<S, WK>& tb, uint32_t pos, uint32_t rem,
                                              uint32_t rtot, uint32_t& take, uint32_t& kr, uint32_t (&key)[S],
                                              uint32_t (&vb)[S], uint32_t (&part)[S], uint64_t (&sbs)[S])
{
    constexpr uint32_t CAP = (uint32_t)S * SG_WAVE;
    const uint32_t lane = lane_id();
    take = rem;
    if (rtot > CAP) { // uniform: a share in proportion, at least one entry of every part
        const uint32_t share = 1u + (uint32_t)(((uint64_t)(CAP - p.n) * rem) / rtot);
        take = rem == 0 ? 0u : (share < rem ? share : rem);
    }
    const uint32_t inc = wave_incl_scan(take);
    const uint32_t E = lane_value(inc, SG_WAVE - 1);
    const uint32_t pre = inc - take;
    kr = count_below(ballot(take > 0));
    if (lane < 2u * S) tb.sb[lane] = 0u;
    tb.drop[lane] = 0u;
    wave_sync();
    if (take > 0) {
        if (pre > 0) atomicOr(&tb.sb[(pre - 1) >> 5], 1u << ((pre - 1) & 31u)); // the entry before the part
        tb.base[kr] = pos - pre;
        if (WK) tb.wk[kr] = lane;
    }
    wave_sync();
    const uint32_t last = (uint32_t)(p.total - 1); // total > 0 here
    uint32_t pc = 0; // marks in earlier slots
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const uint2 sw = *reinterpret_cast<const uint2*>(&tb.sb[2 * i]);
        const uint32_t lo = uniform(sw.x), hi = uniform(sw.y);
        const uint32_t j = lane + (uint32_t)i * SG_WAVE;
        // the part of entry j: the marks before it (mbcnt counts the set
        // bits of the lanes below this one)
        part[i] = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, pc));
        sbs[i] = (uint64_t)lo | ((uint64_t)hi << 32);
        pc += (uint32_t)(__popc(lo) + __popc(hi));
        uint32_t q = tb.base[part[i]] + j;
        q = q < last ? q : last;
        key[i] = p.idx[q];
        if (VM == VM_F32) vb[i] = static_cast<const uint32_t*>(p.val)[q];
        if (VM == VM_BF16) vb[i] = static_cast<const uint16_t*>(p.val)[q];
    }
    return E;
}

// Bitmap word w (keys 32 w .. 32 w + 31 of the span) belongs to lane w / WPL,
// which takes its WPL words in order for the prefix popcounts; it is stored
// at (w % WPL) * 64 + w / WPL, so the lanes read their q-th words from 64
// consecutive places (no LDS bank conflict).
template <int WPL>
__device__ __forceinline__ uint32_t un_phys(uint32_t w)
{
    constexpr uint32_t L = WPL == 1 ? 0 : WPL == 2 ? 1 : WPL == 4 ? 2 : WPL == 8 ? 3 : WPL == 16 ? 4 : 5;
    return WPL == 1 ? w : ((w & (WPL - 1)) << 6) | (w >> L);
}

// The lane's WPL bitmap words of the count pass: their popcount; cleared.
template <int WPL>
__device__ __forceinline__ uint32_t un_count_words(uint32_t* bits)
{
    const uint32_t lane = lane_id();
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < WPL; ++q) {
        c += (uint32_t)__popc(bits[q * SG_WAVE + lane]);
        bits[q * SG_WAVE + lane] = 0u;
    }
    return c;
}

// ---------------------------------------------------------------------------
// the two passes
// ---------------------------------------------------------------------------

// Union size of every tile (keys only) into tile_cnt.
template <int WPL>
__global__ __launch_bounds__(UN_THREADS) void un_count_kernel(MergeParams p)
{
    constexpr int S = UN_SC;
    __shared__ __align__(16) UnCountWave<WPL> smw[UN_WPB];
    const uint32_t wid = uniform(threadIdx.x / SG_WAVE), lane = lane_id();
    UnCountWave<WPL>& sm = smw[wid];
    const uint32_t T = p.G * p.NT, NW = gridDim.x * UN_WPB;
    const uint32_t span = 1u << p.tb;
    uint32_t t = blockIdx.x * UN_WPB + wid;
    if (t >= T) return; // uniform
    for (uint32_t q = lane; q < (uint32_t)(WPL * SG_WAVE); q += SG_WAVE) sm.bits[q] = 0u;
    un_stash<false>(p, sm.tb, un_raw_issue<false>(p, t));
    for (; t < T; t += NW) { // uniform
        wave_sync();
        uint32_t pos = sm.tb.npos[lane], rem = sm.tb.nrem[lane];
        wave_sync();
        const URaw nxt = un_raw_issue<false>(p, t + NW < T ? t + NW : t); // unconditional: no register merge
        const uint32_t klo = (t % p.NT) << p.tb;
        uint32_t rtot = wave_sum(rem);
        bool bad = false;
        if (rtot == 0) { // uniform: an empty tile
            un_stash<false>(p, sm.tb, nxt);
        } else {
            do {
                uint32_t take, kr, key[S], vb[S], part[S];
                uint64_t sbs[S];
                const uint32_t E = un_window<S, VM_NONE>(p, sm.tb, pos, rem, rtot, take, kr, key, vb, part, sbs);
                un_hold(key);
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    const uint32_t o = key[i] - klo;
                    const bool has = lane + (uint32_t)i * SG_WAVE < E;
                    bad |= has && o >= span; // outside the tile: cannot happen for valid input
                    if (has && o < span) atomicOr(&sm.bits[un_phys<WPL>(o >> 5)], 1u << (o & 31u));
                }
                un_stash<false>(p, sm.tb, nxt);
                pos += take;
                rem -= take;
                rtot -= E;
            } while (rtot > 0);
        }
        if (ballot(bad) && lane == 0) report_error(kDevErrIndexRange);
        wave_sync();
        const uint32_t U = wave_sum(un_count_words<WPL>(sm.bits));
        if (lane == 0) p.tile_cnt[t] = U;
    }
}

// The lane's WPL bitmap words of the write pass: their popcount, then the
// exclusive prefix (from `below`) into the words' prefix halves.
template <int WPL>
__device__ __forceinline__ uint32_t un_words_count(const uint2* bw)
{
    const uint32_t lane = lane_id();
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < WPL; ++q) c += (uint32_t)__popc(bw[q * SG_WAVE + lane].x);
    return c;
}

template <int WPL>
__device__ __forceinline__ void un_words_prefix(uint2* bw, uint32_t below)
{
    const uint32_t lane = lane_id();
    uint32_t e = below;
#pragma unroll
    for (int q = 0; q < WPL; ++q) {
        const uint32_t x = bw[q * SG_WAVE + lane].x;
        bw[q * SG_WAVE + lane].y = e;
        e += (uint32_t)__popc(x);
    }
}

template <int WPL>
__device__ __forceinline__ void un_words_clear(uint2* bw)
{
    const uint32_t lane = lane_id();
#pragma unroll
    for (int q = 0; q < WPL; ++q) bw[q * SG_WAVE + lane] = make_uint2(0u, 0u);
}

// Keys (and sums) of every tile at its offset.
template <int WPL, int VM>
__global__ __launch_bounds__(UN_THREADS) void un_write_kernel(MergeParams p)
{
    constexpr int S = UN_SW;
    constexpr bool VALS = VM != VM_NONE;
    constexpr uint32_t NONE = 0xffffffffu; // the offset of a slot with no entry (never inside a span)
    __shared__ __align__(16) UnWriteWave<WPL> smw[UN_WPB];
    const uint32_t wid = uniform(threadIdx.x / SG_WAVE), lane = lane_id();
    UnWriteWave<WPL>& sm = smw[wid];
    const uint32_t T = p.G * p.NT, NW = gridDim.x * UN_WPB;
    const uint32_t span = 1u << p.tb;
    uint32_t t = blockIdx.x * UN_WPB + wid;
    if (t >= T) return; // uniform
    un_words_clear<WPL>(sm.bw);
    for (uint32_t q = lane; q < (uint32_t)UN_CAP; q += SG_WAVE) sm.acc[q] = 0.0f;
    un_stash<true>(p, sm.tb, un_raw_issue<true>(p, t));
    for (; t < T; t += NW) { // uniform
        wave_sync();
        uint32_t pos = sm.tb.npos[lane], rem = sm.tb.nrem[lane];
        uint64_t out = uniform64(sm.tb.nout), out_end = uniform64(sm.tb.nend);
        wave_sync();
        const URaw nxt = un_raw_issue<true>(p, t + NW < T ? t + NW : t); // unconditional: no register merge
        if (out_end > p.capacity || out_end < out) { // cannot happen: the union is no larger than the input
            if (lane == 0) report_error(kDevErrPartition);
            out_end = out = p.capacity;
        }
        if (t % p.NT == 0 && lane == 0) p.agg_off[t / p.NT] = out;
        const uint32_t klo = (t % p.NT) << p.tb;
        uint32_t rtot = wave_sum(rem);
        if (rtot == 0) { // uniform: an empty tile
            un_stash<true>(p, sm.tb, nxt);
        } else {
            do {
                uint32_t take, kr, key[S], vb[S], part[S];
                uint64_t sbs[S];
                const uint32_t E = un_window<S, VM>(p, sm.tb, pos, rem, rtot, take, kr, key, vb, part, sbs);
                un_hold(key);
                // the key's offset in the tile's span; NONE for an empty slot
                uint32_t off[S];
                bool bad = false;
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    const bool has = lane + (uint32_t)i * SG_WAVE < E;
                    const uint32_t o = key[i] - klo;
                    bad |= has && o >= span; // outside the tile: cannot happen for valid input
                    off[i] = has ? o : NONE;
                }
                if (ballot(bad) && lane == 0) report_error(kDevErrIndexRange);
                uint32_t used = take;
                if (rtot > (uint32_t)UN_CAP) { // uniform: a cut window
                    // it ends at the smallest last-loaded key of a part it
                    // cut short; that part's later keys, and every later key
                    // of the other cut parts, go back to their runs
                    const bool cut = take < rem;
                    uint32_t lk = 0xffffffffu;
                    if (cut) lk = p.idx[pos + take - 1];
                    const uint32_t kmax = wave_min(lk);
#pragma unroll
                    for (int i = 0; i < S; ++i) {
                        if (off[i] != NONE && key[i] > kmax) {
                            atomicAdd(&sm.tb.drop[part[i]], 1u);
                            off[i] = NONE;
                        }
                    }
                    wave_sync();
                    if (take > 0) used = take - sm.tb.drop[kr];
                    // the part whose last loaded key is kmax keeps that entry,
                    // so a window always uses one; only input changed while
                    // it is read could break that: report it and take the
                    // whole window, so the loop still ends
                    if (wave_sum(used) == 0) { // uniform
                        if (lane == 0) report_error(kDevErrUnsorted);
                        used = take;
                    }
                }
                pos += used;
                rem -= used;
                // presence bitmap of the window's keys
#pragma unroll
                for (int i = 0; i < S; ++i)
                    if (off[i] < span) atomicOr(&sm.bw[un_phys<WPL>(off[i] >> 5)].x, 1u << (off[i] & 31u));
                wave_sync();
                // prefix popcounts of the words
                const uint32_t c = un_words_count<WPL>(sm.bw);
                const uint32_t inc = wave_incl_scan(c);
                const uint32_t U = lane_value(inc, SG_WAVE - 1);
                un_words_prefix<WPL>(sm.bw, inc - c);
                wave_sync();
                // ranks; keys by rank
                uint32_t rk[S];
#pragma unroll
                for (int i = 0; i < S; ++i) {
                    rk[i] = 0;
                    if (off[i] < span) {
                        const uint2 d = sm.bw[un_phys<WPL>(off[i] >> 5)];
                        rk[i] = d.y + (uint32_t)__popc(d.x & ((1u << (off[i] & 31u)) - 1u));
                        sm.keys[rk[i]] = key[i]; // every holder of a key writes the same value
                    }
                }
                // the sums, slot by slot and, inside a slot, part by part:
                // a part's keys are distinct, so a plain read-add-write of
                // one part's lanes has no race, and the parts come in
                // worker order, so every sum is taken in worker order
                if (VALS) {
                    un_hold(vb);
                    uint32_t pcb = 0; // marks in earlier slots: the part of the slot's first entry
#pragma unroll
                    for (int i = 0; i < S; ++i) {
                        const uint64_t sw = sbs[i];
                        if ((uint32_t)i * SG_WAVE < E) { // uniform
                            const uint64_t inner = sw & ~(1ull << 63); // part ends before the slot's last lane
                            if (inner == 0) { // one part: every lane at once
                                if (off[i] < span) sm.acc[rk[i]] += un_value<VM>(vb[i]);
                            } else {
                                const uint32_t nr = 1u + popc64(inner);
                                for (uint32_t r = 0; r < nr; ++r) { // uniform
                                    if (off[i] < span && part[i] == pcb + r) sm.acc[rk[i]] += un_value<VM>(vb[i]);
                                }
                            }
                        }
                        pcb += popc64(sw);
                    }
                }
                un_stash<true>(p, sm.tb, nxt);
                wave_sync();
                // the tile's slot holds the keys its count found (a run that
                // broke the input's order could make the passes disagree;
                // nothing is written past the slot)
                const uint64_t room = out_end - out;
                const uint32_t lim = room < U ? (uint32_t)room : U;
                uint32_t* const oi = p.agg_idx + out;
                float* const ov = p.agg_val + out;
#pragma unroll
                for (int m = 0; m < S; ++m) {
                    const uint32_t q = lane + (uint32_t)m * SG_WAVE;
                    if ((uint32_t)m * SG_WAVE < U) { // uniform
                        if (q < lim) {
                            oi[q] = sm.keys[q];
                            if (VALS) ov[q] = sm.acc[q];
                        }
                        if (VALS && q < U) sm.acc[q] = 0.0f;
                    }
                }
                un_words_clear<WPL>(sm.bw);
                out += lim;
                rtot = wave_sum(rem);
                wave_sync();
            } while (rtot > 0);
        }
        if (out != out_end && lane == 0) report_error(kDevErrPartition); // the two passes disagree: cannot happen
    }
}

} // namespace sg

// sg_topk.hip -- A1: exact per-worker top-k by magnitude into COO.
//
// What is computed: DGC-style top-k sparsification (Zen OSDI'25 digest,
// section 4: the top 5% of each gradient; SkipReduce MICRO'25 digest,
// section 2: top-k keeps the largest magnitudes), exact, with ties taken
// lowest index first and the output in ascending index order.
//
// How, on gfx950: the dense gradient is read from HBM once.
//   1. sample:  16K strided magnitudes per worker; two order statistics of
//               the sample (radix select in LDS) give a band [lo, hi] that
//               holds the k-th largest key with very high probability.
//   2. filter:  one streaming pass; one wave per 1024-element tile compacts
//               the entries with key >= lo in index order (wave ballots, no
//               atomics, no barriers) into the tile's own slot, and the
//               candidate keys (lo <= key <= hi) into a second slot.
//   3. totals:  per worker, the number of sure entries (key > hi) and of
//               candidates; if the band missed, the worker is re-filtered with
//               the band [0, max] (exact, slower).
//   4. select:  MSD radix select (11-bit digits) over the candidate keys only
//               gives the exact threshold key T and how many entries equal to
//               T are taken.
//   5. write:   per tile counts above/equal T, a per-worker scan, and an
//               ordered compaction of the tile slots into idx[w][*], val[w][*].
// Keys are magnitude bit patterns (sign cleared), which order like |x|.
#include "sg_host.h"

namespace sg {

constexpr int TK_THREADS = 256;
constexpr int TK_TILE = 1024;      // elements per filter tile (one wave)
constexpr int TK_SAMPLES = 16384;
constexpr int TK_DIGIT_BITS = 11;
constexpr int TK_BINS = 1 << TK_DIGIT_BITS;
constexpr int TK_GROUP = 64;       // tiles per wave in the select and write passes (one per lane)
constexpr int TK_HIST_TPW = 64;    // tiles per wave in the histogram pass (one tile group)
constexpr int TK_WRITE_WAVES = 16; // waves per tile group in the write pass

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SelState {
    uint32_t lo, hi;       // band
    uint32_t redo;         // 1: band missed, worker re-filtered with [0, max]
    uint32_t sure, cand;   // counts of key > hi and lo <= key <= hi
    uint32_t R;            // rank still to find among candidates (1-based)
    uint32_t prefix;       // fixed high bits of (T - lo)
    uint32_t top;          // bits >= top of (T - lo) are fixed
    uint32_t T, need;      // threshold key; entries equal to T to take
    uint32_t pad[6];
};

struct TopkParams {
    const void* dense;
    uint32_t* out_idx;
    void* out_val;
    SelState* st;          // [n]
    uint32_t* tcnt;        // [n*NT] entries with key >= lo
    uint32_t* ccnt;        // [n*NT] candidates
    uint16_t* slot_idx;    // [n*NT*TILE] position of a slot entry in its tile
    uint32_t* slot_val;    // [n*NT*TILE] value bits (bf16 in the low half)
    uint32_t* slot_key;    // [n*NT*TILE] candidate keys
    uint32_t* hist;        // [n][TK_BINS]
    uint32_t* samples;     // [n][TK_SAMPLES]
    uint32_t* gtx;         // [n*NT] entries > T of a tile
    uint32_t* eqx;         // [n*NT] entries == T of a tile
    uint32_t* ggt;         // [n*NG] per tile group: entries > T, then their exclusive prefix
    uint32_t* geq;         // [n*NG] per tile group: entries == T, then their exclusive prefix
    uint64_t M, k;
    uint32_t n, NT, NG;
    uint32_t keymax;       // 0x7fffffff (fp32) or 0x7fff (bf16)
    int bf16;
};

__device__ __forceinline__ uint32_t key_of_bits(uint32_t bits, int bf16)
{
    return bf16 ? (bits & 0x7fffu) : (bits & 0x7fffffffu);
}

__device__ __forceinline__ uint32_t load_bits(const TopkParams& p, uint64_t i)
{
    return p.bf16 ? (uint32_t) static_cast<const uint16_t*>(p.dense)[i] : static_cast<const uint32_t*>(p.dense)[i];
}

// --------------------------------------------------------------------------
// 1. band from a strided sample
// --------------------------------------------------------------------------
// Strided sample of each worker's magnitudes, gathered by many blocks (one
// 4-byte load per sample: spread over the chip, not one CU per worker).
__global__ __launch_bounds__(256) void topk_gather_kernel(TopkParams p)
{
    const uint32_t w = blockIdx.y;
    const uint64_t M = p.M;
    const uint32_t S = M < (uint64_t)TK_SAMPLES ? (uint32_t)M : (uint32_t)TK_SAMPLES;
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i >= S) return;
    // (2i + 1) M < 2^15 * 2^32: the product fits 64 bits
    const uint64_t pos = (S == M) ? i : ((2ull * i + 1) * M) / (2ull * S);
    p.samples[(uint64_t)w * TK_SAMPLES + i] = key_of_bits(load_bits(p, (uint64_t)w * M + pos), p.bf16);
}

// LDS histogram increment by a whole wave (every lane calls it): the lanes
// that share the first active lane's digit add their count with one atomic,
// the others one each.  A sample of mostly equal keys (a gradient that is
// mostly zero) would otherwise queue every lane on one LDS address.
__device__ __forceinline__ void hist_add_wave(uint32_t* h, bool act, uint32_t d)
{
    const uint64_t am = ballot(act);
    if (am == 0) return;
    const uint32_t leader = (uint32_t)__builtin_ctzll(am);
    const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, (int)leader);
    const uint64_t same = ballot(act && d == dl);
    if (lane_id() == leader) atomicAdd(&h[dl], popc64(same));
    if (act && d != dl) atomicAdd(&h[d], 1u);
}

// Two order statistics of the sample (the band's ends) by MSD radix select in
// LDS: 11-bit digits, both ranks at once, one block per worker.  Two digits
// suffice: the band only has to hold the k-th key, so its low end is the
// first order statistic with the undecided low bits cleared and its high end
// the second with them set (a band wider by at most 2^10 units of the key).
__global__ __launch_bounds__(1024) void topk_sample_kernel(TopkParams p)
{
    __shared__ uint32_t s[TK_SAMPLES];
    __shared__ uint32_t hist[2][TK_BINS];
    __shared__ uint32_t scan_lds[1024 / SG_WAVE + 1];
    __shared__ uint32_t pick[2][2];
    const uint32_t w = blockIdx.x;
    const uint64_t M = p.M;
    const uint32_t S = M < (uint64_t)TK_SAMPLES ? (uint32_t)M : (uint32_t)TK_SAMPLES;
    {
        constexpr uint32_t SPT = TK_SAMPLES / 1024; // every load in flight before the first store
        uint32_t v[SPT];
#pragma unroll
        for (uint32_t j = 0; j < SPT; ++j) {
            const uint32_t i = j * 1024 + threadIdx.x;
            v[j] = p.samples[(uint64_t)w * TK_SAMPLES + (i < S ? i : 0u)];
        }
#pragma unroll
        for (uint32_t j = 0; j < SPT; ++j)
            if (j * 1024 + threadIdx.x < S) s[j * 1024 + threadIdx.x] = v[j];
    }
    // the worker's histogram row of the selection passes starts at zero
    for (uint32_t i = threadIdx.x; i < TK_BINS; i += 1024) p.hist[(uint64_t)w * TK_BINS + i] = 0;
    // target ranks, 1-based from the smallest; 0 = not needed
    uint32_t R[2];
    bool none_hi = false, none_lo = false;
    if (S == M) {
        R[0] = R[1] = (uint32_t)(M - p.k) + 1;
    } else {
        const double r = (double)p.k * (double)S / (double)M; // expected descending rank
        const double q = (double)p.k / (double)M;
        const double delta = 4.0 * sqrt(r * (1.0 - q)) + 8.0;
        const double rhi = floor(r - delta), rlo = ceil(r + delta);
        none_hi = rhi < 0.0;
        none_lo = rlo >= (double)S;
        // descending rank d is ascending index S-1-d, 1-based rank S-d
        R[0] = none_lo ? 1u : S - (uint32_t)rlo;
        R[1] = none_hi ? S : S - (uint32_t)rhi;
    }
    uint32_t prefix[2] = {0u, 0u};
    uint32_t top = p.bf16 ? 15u : 31u;
    __syncthreads();
    for (int pass = 0; pass < 2 && top > 0; ++pass) {
        const uint32_t shift = top > (uint32_t)TK_DIGIT_BITS ? top - TK_DIGIT_BITS : 0u;
        const uint32_t width = top - shift;
        // both ranks under one prefix (always in the first pass, and in the
        // second when they share a top digit): one histogram serves both
        const bool same = prefix[0] == prefix[1]; // uniform
        for (uint32_t i = threadIdx.x; i < 2 * TK_BINS; i += 1024) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (uint32_t i0 = 0; i0 < S; i0 += 1024) { // uniform: the waves' ballots below
            const uint32_t i = i0 + threadIdx.x;
            const bool valid = i < S;
            const uint32_t key = valid ? s[i] : 0u;
            const uint32_t d = (key >> shift) & ((1u << width) - 1u);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (t == 1 && same) continue;
                hist_add_wave(hist[t], valid && (top >= 32 ? 0u : (key >> top)) == (top >= 32 ? 0u : (prefix[t] >> top)),
                              d);
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t* ht = hist[same ? 0 : t];
            const uint32_t d0 = 2 * threadIdx.x;
            const uint32_t c0 = ht[d0], c1 = ht[d0 + 1];
            uint32_t tot;
            const uint32_t ex = block_excl_scan<1024>(c0 + c1, scan_lds, &tot);
            if (ex < R[t] && R[t] <= ex + c0) {
                pick[t][0] = d0;
                pick[t][1] = ex;
            } else if (ex + c0 < R[t] && R[t] <= ex + c0 + c1) {
                pick[t][0] = d0 + 1;
                pick[t][1] = ex + c0;
            }
            __syncthreads();
            prefix[t] |= pick[t][0] << shift;
            R[t] -= pick[t][1];
            __syncthreads();
        }
        top = shift;
    }
    if (threadIdx.x == 0) {
        SelState st;
        for (int i = 0; i < 6; ++i) st.pad[i] = 0;
        // A sampled low end of 0 (many zero keys, as in a sparse tensor with
        // k near its nonzero count) would make every zero a candidate; the
        // band starts at the smallest positive key instead.  If the k-th key
        // is in fact 0 the band misses and the worker is filtered again with
        // the full band, which stays exact.
        st.lo = none_lo ? 0u : (prefix[0] == 0u ? 1u : prefix[0]);
        st.hi = none_hi ? p.keymax : (prefix[1] | ((1u << top) - 1u)); // top <= 9: the bits not decided
        st.redo = 0;
        st.sure = st.cand = 0;
        st.R = 0;
        st.prefix = 0;
        st.top = 0;
        st.T = 0;
        st.need = 0;
        p.st[w] = st;
    }
}

// --------------------------------------------------------------------------
// 2. filter: one pass over the dense data
// --------------------------------------------------------------------------
// One wave owns one tile of TK_TILE elements; there is no LDS and no barrier,
// so every wave streams independently.  Element e of a tile, for iteration i,
// lane l and vector element v:
//   e = i * (64 * EPV) + l * EPV + v          (EPV = 16 bytes / element size)
// which is ascending in (i, l, v): the compacted slots keep index order.
// A lane's count of selected elements (0..EPV) is prefix-summed over the wave
// bit plane by bit plane, one ballot per plane.
template <int EPV>
__device__ __forceinline__ void wave_count_scan(uint32_t c, uint64_t lt, uint32_t& excl, uint32_t& total)
{
    constexpr int CB = EPV == 4 ? 3 : 4; // bits of a count in [0, EPV]
    excl = 0;
    total = 0;
#pragma unroll
    for (int b = 0; b < CB; ++b) {
        const uint64_t m = ballot((c >> b) & 1u);
        excl += popc64(m & lt) << b;
        total += popc64(m) << b;
    }
}

template <int EPV, bool VEC>
__device__ __forceinline__ void filter_tile(const TopkParams& p, uint32_t w, uint32_t t, uint32_t lo, uint32_t hi)
{
    constexpr int ITERS = TK_TILE / (SG_WAVE * EPV);
    const uint32_t lane = lane_id();
    const uint64_t lt = lanemask_lt();
    const uint64_t tile0 = (uint64_t)t * TK_TILE;
    const uint32_t len = (p.M - tile0) < (uint64_t)TK_TILE ? (uint32_t)(p.M - tile0) : (uint32_t)TK_TILE;
    const uint64_t gbase = (uint64_t)w * p.M + tile0;
    const uint64_t g = (uint64_t)w * p.NT + t;
    const uint64_t slot = g * TK_TILE;

    uint32_t bits[ITERS][EPV];
    const bool full = VEC && len == TK_TILE;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const uint32_t e0 = i * (SG_WAVE * EPV) + lane * EPV;
        if (full) {
            // 16 bytes per lane; the dense data is read once, so the load
            // does not keep it in the caches
            const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                static_cast<const char*>(p.dense) + (gbase + e0) * (EPV == 4 ? 4u : 2u)));
            if constexpr (EPV == 4) {
                bits[i][0] = x.x;
                bits[i][1] = x.y;
                bits[i][2] = x.z;
                bits[i][3] = x.w;
            } else {
                uint32_t q[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int v = 0; v < EPV; ++v) bits[i][v] = (q[v / 2] >> (16 * (v % 2))) & 0xffffu;
            }
        } else {
#pragma unroll
            for (int v = 0; v < EPV; ++v)
                bits[i][v] = (e0 + v < len) ? load_bits(p, gbase + e0 + v) : 0u;
        }
    }
    uint32_t run_ge = 0, run_ca = 0;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const uint32_t e0 = i * (SG_WAVE * EPV) + lane * EPV;
        uint32_t fge = 0, fca = 0;
#pragma unroll
        for (int v = 0; v < EPV; ++v) {
            const uint32_t key = key_of_bits(bits[i][v], p.bf16);
            const bool ge = (e0 + v < len) && key >= lo;
            fge |= (uint32_t)ge << v;
            fca |= (uint32_t)(ge && key <= hi) << v;
        }
        uint32_t x, tot;
        wave_count_scan<EPV>((uint32_t)__popc(fge), lt, x, tot);
        if (fge) {
            uint32_t pos = run_ge + x;
#pragma unroll
            for (int v = 0; v < EPV; ++v) {
                if ((fge >> v) & 1u) {
                    p.slot_idx[slot + pos] = (uint16_t)(e0 + v);
                    p.slot_val[slot + pos] = bits[i][v];
                    ++pos;
                }
            }
        }
        run_ge += tot;
        if (ballot(fca != 0)) { // candidates are rare: the band is narrow
            wave_count_scan<EPV>((uint32_t)__popc(fca), lt, x, tot);
            uint32_t pos = run_ca + x;
#pragma unroll
            for (int v = 0; v < EPV; ++v) {
                if ((fca >> v) & 1u) {
                    p.slot_key[slot + pos] = key_of_bits(bits[i][v], p.bf16);
                    ++pos;
                }
            }
            run_ca += tot;
        }
    }
    if (lane == 0) {
        p.tcnt[g] = run_ge;
        p.ccnt[g] = run_ca;
    }
}

// A full tile whose 16-byte vectors are already in registers: the same
// selection and slot order as filter_tile.  The tile's slot bases are scalar
// and stores take 32-bit byte offsets; each lane stores its selected
// elements one per round, so a round's store carries every lane that still
// has one.
template <int EPV>
__device__ __forceinline__ void filter_full_tile(const TopkParams& p, uint32_t w, uint32_t t, uint32_t lo, uint32_t hi,
                                                 const u32x4 (&x)[TK_TILE / (SG_WAVE * EPV)], uint16_t* lidx,
                                                 uint32_t* lval)
{
    constexpr int ITERS = TK_TILE / (SG_WAVE * EPV);
    constexpr int CB = EPV == 4 ? 3 : 4; // bits of a per-lane count in [0, EPV]
    const uint32_t lane = lane_id();
    const uint64_t g = (uint64_t)w * p.NT + t;
    char* const sidx = reinterpret_cast<char*>(p.slot_idx + g * TK_TILE);
    char* const sval = reinterpret_cast<char*>(p.slot_val + g * TK_TILE);
    char* const skey = reinterpret_cast<char*>(p.slot_key + g * TK_TILE);
    uint32_t run_ge = 0, run_ca = 0;
    // the lane's selected elements of every iteration first, their counts
    // two to a register (16-bit fields: a wave total is at most 64 EPV), and
    // one DPP scan per register places them all
    auto unpack = [&](int i, uint32_t (&bits)[EPV]) {
        if constexpr (EPV == 4) {
            bits[0] = x[i].x;
            bits[1] = x[i].y;
            bits[2] = x[i].z;
            bits[3] = x[i].w;
        } else {
            const uint32_t q[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
            for (int v = 0; v < EPV; ++v) bits[v] = (q[v / 2] >> (16 * (v % 2))) & 0xffffu;
        }
    };
    constexpr int NPK = (ITERS + 1) / 2;
    uint32_t fge[ITERS], fca[ITERS], pk[NPK];
#pragma unroll
    for (int h = 0; h < NPK; ++h) pk[h] = 0;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        uint32_t bits[EPV];
        unpack(i, bits);
        fge[i] = 0;
        fca[i] = 0;
#pragma unroll
        for (int v = 0; v < EPV; ++v) {
            const uint32_t key = key_of_bits(bits[v], p.bf16);
            fge[i] |= (uint32_t)(key >= lo) << v;
            fca[i] |= (uint32_t)(key >= lo && key <= hi) << v;
        }
        pk[i / 2] |= (uint32_t)__popc(fge[i]) << (16 * (i % 2));
    }
    uint32_t ex[NPK], tot[NPK];
#pragma unroll
    for (int h = 0; h < NPK; ++h) {
        const uint32_t inc = wave_incl_scan(pk[h]);
        tot[h] = (uint32_t)__builtin_amdgcn_readlane((int)inc, SG_WAVE - 1);
        ex[h] = inc - pk[h];
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        uint32_t bits[EPV];
        unpack(i, bits);
        const uint32_t e0 = i * (SG_WAVE * EPV) + lane * EPV; // in the tile
        uint32_t pos = run_ge + ((ex[i / 2] >> (16 * (i % 2))) & 0xffffu);
        run_ge += (tot[i / 2] >> (16 * (i % 2))) & 0xffffu;
        for (uint32_t f = fge[i]; ballot(f != 0);) { // into the wave's LDS copy of the tile's slots
            if (f) {
                const uint32_t v = (uint32_t)__builtin_ctz(f);
                uint32_t b = bits[0];
#pragma unroll
                for (int u = 1; u < EPV; ++u) b = v == (uint32_t)u ? bits[u] : b;
                lidx[pos] = (uint16_t)(e0 + v);
                lval[pos] = b;
                ++pos;
                f &= f - 1u;
            }
        }
        if (ballot(fca[i] != 0)) { // candidates are rare: the band is narrow
            const uint32_t cc = (uint32_t)__popc(fca[i]);
            uint32_t cpos = run_ca;
#pragma unroll
            for (int b = 0; b < CB; ++b) {
                const uint64_t m = ballot((cc >> b) & 1u);
                cpos += count_below(m) << b;
                run_ca += popc64(m) << b;
            }
            for (uint32_t f = fca[i]; ballot(f != 0);) {
                if (f) {
                    const uint32_t v = (uint32_t)__builtin_ctz(f);
                    uint32_t b = bits[0];
#pragma unroll
                    for (int u = 1; u < EPV; ++u) b = v == (uint32_t)u ? bits[u] : b;
                    *reinterpret_cast<uint32_t*>(skey + cpos * 4u) = key_of_bits(b, p.bf16);
                    ++cpos;
                    f &= f - 1u;
                }
            }
        }
    }
    // the selected slots out with contiguous stores
    wave_sync();
    for (uint32_t j = lane; j < run_ge; j += SG_WAVE) {
        *reinterpret_cast<uint16_t*>(sidx + j * 2u) = lidx[j];
        *reinterpret_cast<uint32_t*>(sval + j * 4u) = lval[j];
    }
    wave_sync(); // the LDS copy is reused by the wave's next tile
    if (lane == 0) {
        p.tcnt[g] = run_ge;
        p.ccnt[g] = run_ca;
    }
}

template <int EPV>
__device__ __forceinline__ void load_full_tile(const TopkParams& p, uint32_t w, uint32_t t,
                                               u32x4 (&x)[TK_TILE / (SG_WAVE * EPV)])
{
    constexpr int ITERS = TK_TILE / (SG_WAVE * EPV);
    // 16 bytes per lane; the dense data is read once, so the load does not
    // keep it in the caches
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(p.dense) +
                                                      ((uint64_t)w * p.M + (uint64_t)t * TK_TILE) * (EPV == 4 ? 4u : 2u));
#pragma unroll
    for (int i = 0; i < ITERS; ++i) x[i] = __builtin_nontemporal_load(src + i * SG_WAVE + lane_id());
}

// A wave's walk over the tiles g = w * NT + t, g0, g0 + stride, ...: (w, t)
// advanced without a division per step.
struct TileWalk {
    uint32_t w, t, dw, dt, NT, n;
    __device__ bool valid() const { return w < n; }
    __device__ void next()
    {
        t += dt;
        w += dw;
        if (t >= NT) {
            t -= NT;
            ++w;
        }
    }
};

// The main pass over 16-byte aligned rows with M >= TK_TILE: while a wave
// works on one tile, the loads of its next tile are in flight (two register
// buffers used in turn).  Every step issues the same loads (a tile that is
// not full, or past the end, reads the full tile 0 of worker 0 instead and
// ignores it), so the waits before each tile's use count only the loads
// issued after it.  Tiles at the end of a row shorter than TK_TILE go
// through filter_tile.
template <int EPV>
__device__ __forceinline__ void prefetch_tile(const TopkParams& p, const TileWalk& c, uint32_t full_tiles,
                                              uint32_t& lo, uint32_t& hi, u32x4 (&x)[TK_TILE / (SG_WAVE * EPV)])
{
    const uint32_t w = c.valid() ? c.w : 0u;
    const uint2 band = *reinterpret_cast<const uint2*>(&p.st[w].lo);
    lo = band.x;
    hi = band.y;
    const bool full = c.valid() && c.t < full_tiles;
    load_full_tile<EPV>(p, full ? c.w : 0u, full ? c.t : 0u, x);
}

template <int EPV>
__device__ __forceinline__ void filter_step(const TopkParams& p, const TileWalk& c, uint32_t full_tiles, uint32_t lo,
                                            uint32_t hi, const u32x4 (&x)[TK_TILE / (SG_WAVE * EPV)], uint16_t* lidx,
                                            uint32_t* lval)
{
    if (c.t < full_tiles) filter_full_tile<EPV>(p, c.w, c.t, lo, hi, x, lidx, lval);
    else filter_tile<EPV, false>(p, c.w, c.t, lo, hi);
}

template <int EPV>
__global__ __launch_bounds__(TK_THREADS) void topk_filter_pipe_kernel(TopkParams p)
{
    constexpr int ITERS = TK_TILE / (SG_WAVE * EPV);
    // per wave, an LDS copy of a tile's selected slots
    __shared__ uint16_t sl_idx[TK_THREADS / SG_WAVE][TK_TILE];
    __shared__ uint32_t sl_val[TK_THREADS / SG_WAVE][TK_TILE];
    uint16_t* const lidx = sl_idx[threadIdx.x / SG_WAVE];
    uint32_t* const lval = sl_val[threadIdx.x / SG_WAVE];
    const uint32_t full_tiles = (uint32_t)(p.M / TK_TILE); // tiles t < full_tiles of a row are full
    const uint32_t g0 = blockIdx.x * (TK_THREADS / SG_WAVE) + uniform(threadIdx.x / SG_WAVE);
    const uint32_t stride = gridDim.x * (TK_THREADS / SG_WAVE);
    TileWalk cur = {g0 / p.NT, g0 % p.NT, stride / p.NT, stride % p.NT, p.NT, p.n};
    u32x4 a[ITERS], b[ITERS];
    uint32_t lo_a, hi_a, lo_b, hi_b;
    prefetch_tile<EPV>(p, cur, full_tiles, lo_a, hi_a, a);
    while (cur.valid()) {
        TileWalk nx = cur;
        nx.next();
        prefetch_tile<EPV>(p, nx, full_tiles, lo_b, hi_b, b);
        filter_step<EPV>(p, cur, full_tiles, lo_a, hi_a, a, lidx, lval);
        cur = nx;
        if (!cur.valid()) break;
        nx.next();
        prefetch_tile<EPV>(p, nx, full_tiles, lo_a, hi_a, a);
        filter_step<EPV>(p, cur, full_tiles, lo_b, hi_b, b, lidx, lval);
        cur = nx;
    }
}

// REDO: process only the workers whose band missed (st.redo == 1); the whole
// launch returns at once when there are none.
template <int EPV, bool VEC, bool REDO>
__global__ __launch_bounds__(TK_THREADS) void topk_filter_kernel(TopkParams p)
{
    if (REDO) {
        bool any = false;
        for (uint32_t w = lane_id(); w < p.n; w += SG_WAVE) any |= p.st[w].redo != 0;
        if (!ballot(any)) return;
    }
    const uint64_t ntiles = (uint64_t)p.n * p.NT;
    const uint64_t stride = (uint64_t)gridDim.x * (TK_THREADS / SG_WAVE);
    for (uint64_t g = (uint64_t)blockIdx.x * (TK_THREADS / SG_WAVE) + threadIdx.x / SG_WAVE; g < ntiles;
         g += stride) {
        const uint32_t w = (uint32_t)(g / p.NT), t = (uint32_t)(g % p.NT);
        const SelState& st = p.st[w];
        if (REDO && st.redo == 0) continue;
        filter_tile<EPV, VEC>(p, w, t, st.lo, st.hi);
    }
}

// --------------------------------------------------------------------------
// 3. totals per worker; a missed band schedules a re-filter with [0, max]
// --------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void topk_totals_kernel(TopkParams p, int second)
{
    __shared__ uint32_t red[2][16];
    const uint32_t w = blockIdx.x;
    uint32_t sure = 0, cand = 0;
    const uint32_t* const tc = p.tcnt + (uint64_t)w * p.NT;
    const uint32_t* const cc = p.ccnt + (uint64_t)w * p.NT;
    for (uint32_t t0 = threadIdx.x; t0 < p.NT; t0 += 8 * 1024) { // eight tiles' loads in flight
        uint32_t a[8], c[8];
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) {
            const uint32_t t = t0 + u * 1024;
            a[u] = t < p.NT ? tc[t] : 0u;
            c[u] = t < p.NT ? cc[t] : 0u;
        }
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) {
            sure += a[u] - c[u];
            cand += c[u];
        }
    }
    sure = wave_sum(sure);
    cand = wave_sum(cand);
    if (lane_id() == 0) {
        red[0][threadIdx.x / SG_WAVE] = sure;
        red[1][threadIdx.x / SG_WAVE] = cand;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t S = 0, Cn = 0;
        for (int i = 0; i < 16; ++i) {
            S += red[0][i];
            Cn += red[1][i];
        }
        SelState& st = p.st[w];
        if (second && !st.redo) return; // this worker's first result stands
        st.sure = S;
        st.cand = Cn;
        const uint64_t k = p.k;
        const bool ok = (uint64_t)S < k && k <= (uint64_t)S + Cn;
        if (!ok) {
            if (!second) {
                st.redo = 1;
                st.lo = 0;
                st.hi = p.keymax;
            } else {
                report_error(kDevErrPartition); // cannot happen with the full band
            }
            st.R = 0;
        } else {
            st.redo = second ? 2u : 0u;
            st.R = (uint32_t)(k - S);
            uint32_t span = st.hi - st.lo;
            uint32_t nb = 0;
            while (nb < 32 && (span >> nb) != 0) ++nb;
            st.top = nb; // bits >= top of (T - lo) are known (zero)
            st.prefix = 0;
            st.T = st.lo;   // final when nb == 0 (the band is one key)
            st.need = st.R;
        }
    }
}

// --------------------------------------------------------------------------
// 4. radix select among the candidates
// --------------------------------------------------------------------------
__device__ __forceinline__ void digit_window(uint32_t top, uint32_t& shift, uint32_t& width)
{
    shift = top > (uint32_t)TK_DIGIT_BITS ? top - TK_DIGIT_BITS : 0u;
    width = top - shift;
}

// digit of a candidate key for the current pass, or TK_BINS when its
// higher digits differ from the prefix chosen so far
__device__ __forceinline__ uint32_t cand_digit(const SelState& st, uint32_t key, uint32_t shift, uint32_t width)
{
    const uint32_t r = key - st.lo;
    const uint32_t hi_part = st.top >= 32 ? 0u : (r >> st.top);
    const uint32_t pre_part = st.top >= 32 ? 0u : (st.prefix >> st.top);
    return hi_part != pre_part ? (uint32_t)TK_BINS : (r >> shift) & ((1u << width) - 1u);
}

// Histogram of the current digit over the candidates.  A wave takes groups
// of 64 tiles (the tile counts in one load, one lane per tile) and loads the
// first 128 candidates of 16 tiles at a time, so the loads overlap (a tile
// with more candidates loads the rest afterwards).
__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(TopkParams p)
{
    __shared__ uint32_t h[TK_BINS];
    constexpr uint32_t UPG = TK_GROUP / TK_HIST_TPW; // waves per tile group
    const uint32_t units = p.NG * UPG;               // waves per worker
    const uint32_t bpw = (units + (TK_THREADS / SG_WAVE) - 1) / (TK_THREADS / SG_WAVE);
    const uint32_t w = blockIdx.x / bpw, bi = blockIdx.x % bpw;
    const SelState st = p.st[w];
    if (st.R == 0 || st.top == 0) return;
    uint32_t shift, width;
    digit_window(st.top, shift, width);
    for (uint32_t i = threadIdx.x; i < TK_BINS; i += TK_THREADS) h[i] = 0;
    __syncthreads();
    const uint32_t wid = uniform(threadIdx.x / SG_WAVE), lane = lane_id();
    const uint32_t unit = bi * (TK_THREADS / SG_WAVE) + wid;
    if (unit < units) {
        const uint32_t grp = unit / UPG, jb = (unit % UPG) * TK_HIST_TPW;
        const uint64_t g0 = (uint64_t)w * p.NT + (uint64_t)grp * TK_GROUP;
        const uint32_t c = grp * TK_GROUP + lane < p.NT ? p.ccnt[g0 + lane] : 0u;
        for (uint32_t j0 = jb; j0 < jb + TK_HIST_TPW; j0 += 16) {
            uint32_t kk[16], k2[16], cj[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                cj[u] = (uint32_t)__builtin_amdgcn_readlane((int)c, (int)(j0 + u));
                const uint32_t* sk = p.slot_key + (g0 + j0 + u) * TK_TILE;
                kk[u] = lane < cj[u] ? sk[lane] : 0u;
                k2[u] = SG_WAVE + lane < cj[u] ? sk[SG_WAVE + lane] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (lane < cj[u]) {
                    const uint32_t d = cand_digit(st, kk[u], shift, width);
                    if (d < (uint32_t)TK_BINS) atomicAdd(&h[d], 1u);
                }
                if (SG_WAVE + lane < cj[u]) {
                    const uint32_t d = cand_digit(st, k2[u], shift, width);
                    if (d < (uint32_t)TK_BINS) atomicAdd(&h[d], 1u);
                }
                for (uint32_t i = 2 * SG_WAVE + lane; i < cj[u]; i += SG_WAVE) { // tiles with more than 128 candidates
                    const uint32_t d = cand_digit(st, p.slot_key[(g0 + j0 + u) * TK_TILE + i], shift, width);
                    if (d < (uint32_t)TK_BINS) atomicAdd(&h[d], 1u);
                }
            }
        }
    }
    __syncthreads();
    uint32_t* gh = p.hist + (uint64_t)w * TK_BINS;
    for (uint32_t i = threadIdx.x; i < (1u << width); i += TK_THREADS)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

// One block per worker: pick the digit holding rank R, then clear the
// histogram for the next pass.
__global__ __launch_bounds__(TK_THREADS) void topk_pick_kernel(TopkParams p)
{
    __shared__ uint32_t h[TK_BINS];
    __shared__ uint32_t scan_lds[TK_THREADS / SG_WAVE + 1];
    const uint32_t w = blockIdx.x;
    SelState st = p.st[w];
    uint32_t* gh = p.hist + (uint64_t)w * TK_BINS;
    if (st.R == 0 || st.top == 0) return;
    uint32_t shift, width;
    digit_window(st.top, shift, width);
    const uint32_t nbins = 1u << width;
    for (uint32_t i = threadIdx.x; i < TK_BINS; i += TK_THREADS) {
        h[i] = i < nbins ? gh[i] : 0u;
        gh[i] = 0u;
    }
    __syncthreads();
    // counts from the top digit down: thread j owns digits [j*8, j*8+8) of the
    // reversed order
    constexpr int PER = TK_BINS / TK_THREADS;
    uint32_t loc[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        uint32_t d = nbins - 1u - (threadIdx.x * PER + i); // reversed digit
        loc[i] = (threadIdx.x * PER + i < nbins) ? h[d] : 0u;
        sum += loc[i];
    }
    uint32_t tot;
    uint32_t ex = block_excl_scan<TK_THREADS>(sum, scan_lds, &tot);
    __shared__ uint32_t pick_d, pick_above;
    uint32_t run = ex;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        uint32_t rd = threadIdx.x * PER + i;
        if (rd < nbins && run < st.R && st.R <= run + loc[i]) {
            pick_d = nbins - 1u - rd;
            pick_above = run;
        }
        run += loc[i];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        SelState& g = p.st[w];
        if (tot < st.R) { // cannot happen: candidates were counted
            report_error(kDevErrPartition);
            g.R = 0;
            return;
        }
        g.prefix = st.prefix | (pick_d << shift);
        g.R = st.R - pick_above;
        g.top = shift;
        if (shift == 0) {
            g.T = st.lo + g.prefix;
            g.need = g.R;
        }
    }
}

// Small inputs (a worker's tiles in at most TK_SMALL_GROUPS groups of 64):
// every digit pass of the selection in one block per worker, then the tile
// counts and the group scan, instead of a histogram and a pick launch per
// digit and two more launches.  The worker's candidates are gathered into
// LDS once (up to TK_SMALL_CAP of them; more are read from the slots in
// every pass).
constexpr uint32_t TK_SMALL_GROUPS = 32;
constexpr uint32_t TK_SMALL_TILES = TK_SMALL_GROUPS * TK_GROUP;
constexpr uint32_t TK_SMALL_CAP = 24576;
__global__ __launch_bounds__(1024) void topk_select_small_kernel(TopkParams p)
{
    __shared__ uint32_t h[TK_BINS];
    __shared__ uint32_t cand[TK_SMALL_CAP];
    __shared__ uint32_t toff[TK_SMALL_TILES + 1];
    __shared__ uint32_t scan_lds[1024 / SG_WAVE + 1];
    __shared__ uint32_t pick_d, pick_above;
    __shared__ uint32_t sgt[TK_SMALL_GROUPS], seq[TK_SMALL_GROUPS];
    const uint32_t w = blockIdx.x;
    const uint32_t wid = uniform(threadIdx.x / SG_WAVE), lane = lane_id();
    const uint64_t t0 = (uint64_t)w * p.NT; // the worker's first tile
    SelState st = p.st[w];
    // the tiles' candidate offsets (two tiles per thread)
    uint32_t cc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const uint32_t t = threadIdx.x * 2 + u;
        cc[u] = t < p.NT ? p.ccnt[t0 + t] : 0u;
    }
    uint32_t C;
    const uint32_t ex = block_excl_scan<1024>(cc[0] + cc[1], scan_lds, &C);
    if (threadIdx.x * 2 < TK_SMALL_TILES) toff[threadIdx.x * 2] = ex;
    if (threadIdx.x * 2 + 1 < TK_SMALL_TILES) toff[threadIdx.x * 2 + 1] = ex + cc[0];
    if (threadIdx.x == 0) toff[p.NT] = C;
    const bool staged = C <= TK_SMALL_CAP; // uniform
    __syncthreads();
    if (staged) { // gather: a wave per tile group, 16 tiles' loads at a time
        for (uint32_t grp = wid; grp < p.NG; grp += 1024 / SG_WAVE) {
            const uint32_t tg = grp * TK_GROUP;
            const uint32_t c = tg + lane < p.NT ? p.ccnt[t0 + tg + lane] : 0u;
            for (uint32_t j0 = 0; j0 < (uint32_t)TK_GROUP; j0 += 16) {
                uint32_t kk[16], k2[16], cj[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    cj[u] = (uint32_t)__builtin_amdgcn_readlane((int)c, (int)(j0 + u));
                    const uint32_t* sk = p.slot_key + (t0 + tg + j0 + u) * TK_TILE;
                    kk[u] = lane < cj[u] ? sk[lane] : 0u;
                    k2[u] = SG_WAVE + lane < cj[u] ? sk[SG_WAVE + lane] : 0u;
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    if (cj[u] == 0) continue;
                    uint32_t* dst = cand + toff[tg + j0 + u];
                    if (lane < cj[u]) dst[lane] = kk[u];
                    if (SG_WAVE + lane < cj[u]) dst[SG_WAVE + lane] = k2[u];
                    for (uint32_t i = 2 * SG_WAVE + lane; i < cj[u]; i += SG_WAVE)
                        dst[i] = p.slot_key[(t0 + tg + j0 + u) * TK_TILE + i];
                }
            }
        }
        __syncthreads();
    }
    // the digit passes
    bool fail = false;
    while (st.R != 0 && st.top != 0) { // uniform: st is the same in every thread
        uint32_t shift, width;
        digit_window(st.top, shift, width);
        for (uint32_t i = threadIdx.x; i < TK_BINS; i += 1024) h[i] = 0;
        __syncthreads();
        if (staged) {
            for (uint32_t i = threadIdx.x; i < C; i += 1024) {
                const uint32_t d = cand_digit(st, cand[i], shift, width);
                if (d < (uint32_t)TK_BINS) atomicAdd(&h[d], 1u);
            }
        } else {
            for (uint32_t grp = wid; grp < p.NG; grp += 1024 / SG_WAVE) {
                const uint32_t tg = grp * TK_GROUP;
                const uint32_t c = tg + lane < p.NT ? p.ccnt[t0 + tg + lane] : 0u;
                for (uint32_t j0 = 0; j0 < (uint32_t)TK_GROUP; j0 += 16) {
                    uint32_t kk[16], k2[16], cj[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        cj[u] = (uint32_t)__builtin_amdgcn_readlane((int)c, (int)(j0 + u));
                        const uint32_t* sk = p.slot_key + (t0 + tg + j0 + u) * TK_TILE;
                        kk[u] = lane < cj[u] ? sk[lane] : 0u;
                        k2[u] = SG_WAVE + lane < cj[u] ? sk[SG_WAVE + lane] : 0u;
                    }
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        if (lane < cj[u]) {
                            const uint32_t d = cand_digit(st, kk[u], shift, width);
                            if (d < (uint32_t)TK_BINS) atomicAdd(&h[d], 1u);
                        }
                        if (SG_WAVE + lane < cj[u]) {
                            const uint32_t d = cand_digit(st, k2[u], shift, width);
                            if (d < (uint32_t)TK_BINS) atomicAdd(&h[d], 1u);
                        }
                        for (uint32_t i = 2 * SG_WAVE + lane; i < cj[u]; i += SG_WAVE) { // tiles with more than 128 candidates
                            const uint32_t d = cand_digit(st, p.slot_key[(t0 + tg + j0 + u) * TK_TILE + i], shift, width);
                            if (d < (uint32_t)TK_BINS) atomicAdd(&h[d], 1u);
                        }
                    }
                }
            }
        }
        __syncthreads();
        // the digit holding rank R, counted from the top digit down: thread j
        // owns digits [2j, 2j+2) of the reversed order
        const uint32_t nbins = 1u << width;
        constexpr int PER = TK_BINS / 1024;
        uint32_t loc[PER], sum = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t rd = threadIdx.x * PER + i;
            loc[i] = rd < nbins ? h[nbins - 1u - rd] : 0u;
            sum += loc[i];
        }
        uint32_t tot;
        uint32_t run = block_excl_scan<1024>(sum, scan_lds, &tot);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t rd = threadIdx.x * PER + i;
            if (rd < nbins && run < st.R && st.R <= run + loc[i]) {
                pick_d = nbins - 1u - rd;
                pick_above = run;
            }
            run += loc[i];
        }
        __syncthreads();
        if (tot < st.R) { // cannot happen: candidates were counted
            fail = true;
            break;
        }
        st.prefix |= pick_d << shift;
        st.R -= pick_above;
        st.top = shift;
        if (shift == 0) {
            st.T = st.lo + st.prefix;
            st.need = st.R;
        }
        __syncthreads(); // h and the pick are reused by the next digit
    }
    if (threadIdx.x == 0) {
        SelState& g = p.st[w];
        if (fail) {
            report_error(kDevErrPartition);
            g.R = 0;
        } else {
            g.prefix = st.prefix;
            g.R = st.R;
            g.top = st.top;
            g.T = st.T;
            g.need = st.need;
        }
    }
    // then, as the tile-count and scan passes do: per tile the entries above
    // T and equal to T, per group their sums, and the groups' exclusive
    // prefixes.  A wave per group, a lane per tile.
    const uint32_t T = st.T;
    for (uint32_t grp = wid; grp < p.NG; grp += 1024 / SG_WAVE) {
        const uint32_t t = grp * TK_GROUP + lane;
        const bool valid = t < p.NT;
        uint32_t my_gt = 0, my_eq = 0;
        if (valid) {
            const uint32_t c = p.ccnt[t0 + t];
            my_gt = p.tcnt[t0 + t] - c;
            if (staged) {
                for (uint32_t i = toff[t]; i < toff[t] + c; ++i) {
                    my_gt += cand[i] > T;
                    my_eq += cand[i] == T;
                }
            } else {
                const uint32_t* sk = p.slot_key + (t0 + t) * TK_TILE;
                for (uint32_t i = 0; i < c; ++i) {
                    const uint32_t key = sk[i];
                    my_gt += key > T;
                    my_eq += key == T;
                }
            }
            p.gtx[t0 + t] = my_gt;
            p.eqx[t0 + t] = my_eq;
        }
        const uint32_t sg = wave_sum(my_gt), se = wave_sum(my_eq);
        if (lane == 0) {
            sgt[grp] = sg;
            seq[grp] = se;
        }
    }
    __syncthreads();
    if (wid == 0) { // at most TK_SMALL_GROUPS < 64 groups: one wave scan each
        const uint32_t a = lane < p.NG ? sgt[lane] : 0u, b = lane < p.NG ? seq[lane] : 0u;
        const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
        if (lane < p.NG) {
            p.ggt[(uint64_t)w * p.NG + lane] = ia - a;
            p.geq[(uint64_t)w * p.NG + lane] = ib - b;
        }
    }
}

// --------------------------------------------------------------------------
// 5. counts per tile, per-worker scan, ordered write
// --------------------------------------------------------------------------
// One wave per group of 64 tiles: per tile, entries above T (the sure ones
// and the candidates above T) and equal to T; per group, their sums.
__global__ __launch_bounds__(TK_THREADS) void topk_tilecount_kernel(TopkParams p)
{
    const uint64_t gw = (uint64_t)blockIdx.x * (TK_THREADS / SG_WAVE) + threadIdx.x / SG_WAVE;
    if (gw >= (uint64_t)p.n * p.NG) return;
    const uint32_t lane = lane_id();
    const uint32_t w = (uint32_t)(gw / p.NG), grp = (uint32_t)(gw % p.NG);
    const uint32_t T = p.st[w].T;
    const uint64_t g0 = (uint64_t)w * p.NT + (uint64_t)grp * TK_GROUP;
    const bool valid = grp * TK_GROUP + lane < p.NT;
    const uint32_t c = valid ? p.ccnt[g0 + lane] : 0u;
    uint32_t my_gt = valid ? p.tcnt[g0 + lane] - c : 0u, my_eq = 0;
    for (uint32_t j0 = 0; j0 < (uint32_t)TK_GROUP; j0 += 8) {
        uint32_t kk[8], k2[8], cj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            cj[u] = (uint32_t)__builtin_amdgcn_readlane((int)c, (int)(j0 + u));
            const uint32_t* sk = p.slot_key + (g0 + j0 + u) * TK_TILE;
            kk[u] = lane < cj[u] ? sk[lane] : 0u;
            k2[u] = SG_WAVE + lane < cj[u] ? sk[SG_WAVE + lane] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            uint32_t gt = popc64(ballot(lane < cj[u] && kk[u] > T)) + popc64(ballot(SG_WAVE + lane < cj[u] && k2[u] > T));
            uint32_t eq = popc64(ballot(lane < cj[u] && kk[u] == T)) + popc64(ballot(SG_WAVE + lane < cj[u] && k2[u] == T));
            for (uint32_t i0 = 2 * SG_WAVE; i0 < cj[u]; i0 += SG_WAVE) { // tiles with more than 128 candidates
                const uint32_t i = i0 + lane;
                const uint32_t key = i < cj[u] ? p.slot_key[(g0 + j0 + u) * TK_TILE + i] : 0u;
                gt += popc64(ballot(i < cj[u] && key > T));
                eq += popc64(ballot(i < cj[u] && key == T));
            }
            if (lane == j0 + u) {
                my_gt += gt;
                my_eq = eq;
            }
        }
    }
    if (valid) {
        p.gtx[g0 + lane] = my_gt;
        p.eqx[g0 + lane] = my_eq;
    }
    const uint32_t sg = wave_sum(my_gt), se = wave_sum(my_eq);
    if (lane == 0) {
        p.ggt[gw] = sg;
        p.geq[gw] = se;
    }
}

// Per-worker exclusive scans of the group sums (in place); each thread takes
// 8 consecutive groups per round.
__global__ __launch_bounds__(1024) void topk_scan_kernel(TopkParams p)
{
    constexpr uint32_t PT = 8;
    __shared__ uint32_t scan_lds[1024 / SG_WAVE + 1];
    const uint32_t w = blockIdx.x;
    uint32_t carry_gt = 0, carry_eq = 0;
    for (uint32_t base = 0; base < p.NG; base += 1024 * PT) {
        const uint32_t t0 = base + threadIdx.x * PT;
        const uint64_t g0 = (uint64_t)w * p.NG + t0;
        uint32_t a[PT], b[PT], sa = 0, sb = 0;
#pragma unroll
        for (uint32_t j = 0; j < PT; ++j) {
            const bool in = t0 + j < p.NG;
            a[j] = in ? p.ggt[g0 + j] : 0u;
            b[j] = in ? p.geq[g0 + j] : 0u;
            sa += a[j];
            sb += b[j];
        }
        uint32_t ta, tb;
        uint32_t xa = block_excl_scan<1024>(sa, scan_lds, &ta);
        __syncthreads();
        uint32_t xb = block_excl_scan<1024>(sb, scan_lds, &tb);
        xa += carry_gt;
        xb += carry_eq;
#pragma unroll
        for (uint32_t j = 0; j < PT; ++j) {
            if (t0 + j < p.NG) {
                p.ggt[g0 + j] = xa;
                p.geq[g0 + j] = xb;
            }
            xa += a[j];
            xb += b[j];
        }
        carry_gt += ta;
        carry_eq += tb;
        __syncthreads();
    }
}

// Ordered compaction of one chunk of up to 64 slot entries: entries above T,
// and entries equal to T while fewer than `need` equal ones precede them.
// oidx / oval are the worker's output rows.
template <bool BF16>
__device__ __forceinline__ void write_chunk(uint32_t* oidx, void* oval, uint64_t k, uint32_t valid_n, uint32_t bits,
                                            uint32_t ix, uint32_t T, uint32_t need, uint64_t& pos, uint32_t& eqr)
{
    const bool valid = lane_id() < valid_n;
    const uint32_t key = key_of_bits(bits, BF16);
    const bool eq = valid && key == T;
    const uint64_t meq = ballot(eq);
    const uint32_t my_eq = eqr + count_below(meq);
    const bool sel = valid && (key > T || (eq && my_eq < need));
    const uint64_t ms = ballot(sel);
    if (sel) {
        const uint64_t o = pos + count_below(ms);
        if (o < k) {
            oidx[o] = ix;
            if (BF16) static_cast<uint16_t*>(oval)[o] = (uint16_t)bits;
            else static_cast<uint32_t*>(oval)[o] = bits;
        }
    }
    pos += popc64(ms);
    eqr += popc64(meq);
}

// One load round of the ordered write: chunks b0 .. b0 + B - 1 of the wave's
// chunk numbering (all B loads issued, then the chunks written in order).
struct WriteWave {
    uint32_t nch, cst, cnt, xg, xe, C, grp, T, need;
    uint64_t g0;
    uint32_t* oidx;
    void* oval;
};

template <bool BF16, int B>
__device__ __forceinline__ void write_round(const TopkParams& p, const WriteWave& v, uint32_t b0, uint32_t& cur_tile,
                                            uint32_t& eqr, uint64_t& pos)
{
    const uint32_t lane = lane_id();
    uint32_t vb[B], vi[B], tj[B], ch[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const uint32_t q = b0 + u;
        const uint64_t has = ballot(v.nch > 0 && v.cst <= q);
        tj[u] = has ? 63u - (uint32_t)__builtin_clzll(has) : 0u; // the last tile starting at or before chunk q
        const uint32_t first = lane_value(v.cst, tj[u]);
        const uint32_t cj = lane_value(v.cnt, tj[u]);
        ch[u] = q < v.C ? (q - first) * SG_WAVE : cj; // entry offset of the chunk in its tile
        const uint32_t i = ch[u] + lane;
        const uint64_t sb = (v.g0 + tj[u]) * TK_TILE;
        vb[u] = q < v.C && i < cj ? p.slot_val[sb + i] : 0u;
        vi[u] = q < v.C && i < cj ? (uint32_t)p.slot_idx[sb + i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
        if (b0 + u >= v.C) break;
        if (tj[u] != cur_tile) {
            cur_tile = tj[u];
            eqr = lane_value(v.xe, cur_tile);
            pos = (uint64_t)lane_value(v.xg, cur_tile) + (eqr < v.need ? eqr : v.need);
        }
        const uint32_t cj = lane_value(v.cnt, tj[u]);
        const uint32_t tile0 = (v.grp * TK_GROUP + tj[u]) * TK_TILE; // first index of the tile
        write_chunk<BF16>(v.oidx, v.oval, p.k, cj - ch[u], vb[u], tile0 + vi[u], v.T, v.need, pos, eqr);
    }
}

// TK_WRITE_WAVES waves per group of 64 tiles; wave j writes the tiles j,
// j + TK_WRITE_WAVES, ... of it, so the tiles of a dense row (one chunk per
// 64 entries, up to 16 per tile) are spread over several waves.  The tiles'
// output offsets come from the group prefix and a wave scan over the group.
// The wave's slot chunks are numbered across its tiles and loaded up to 8 at
// a time (rounds of 2 or 4 when fewer remain, as for most waves), so dense
// tiles cost no more load rounds than their size demands.
template <bool BF16>
__global__ __launch_bounds__(TK_THREADS) void topk_write_kernel(TopkParams p)
{
    const uint64_t gq = (uint64_t)blockIdx.x * (TK_THREADS / SG_WAVE) + uniform(threadIdx.x / SG_WAVE);
    if (gq >= (uint64_t)p.n * p.NG * TK_WRITE_WAVES) return;
    const uint64_t gw = gq / TK_WRITE_WAVES;
    const uint32_t part = (uint32_t)(gq % TK_WRITE_WAVES);
    const uint32_t lane = lane_id();
    const uint32_t w = (uint32_t)(gw / p.NG);
    WriteWave v;
    v.grp = (uint32_t)(gw % p.NG);
    v.T = p.st[w].T;
    v.need = p.st[w].need;
    v.g0 = (uint64_t)w * p.NT + (uint64_t)v.grp * TK_GROUP;
    const bool valid = v.grp * TK_GROUP + lane < p.NT;
    v.cnt = valid ? p.tcnt[v.g0 + lane] : 0u;
    const uint32_t gt = valid ? p.gtx[v.g0 + lane] : 0u, eq = valid ? p.eqx[v.g0 + lane] : 0u;
    v.xg = p.ggt[gw] + wave_incl_scan(gt) - gt;
    v.xe = p.geq[gw] + wave_incl_scan(eq) - eq;
    // chunks of this wave's tiles, numbered in tile order
    const bool mine = lane % TK_WRITE_WAVES == part;
    v.nch = mine ? (v.cnt + SG_WAVE - 1) / SG_WAVE : 0u;
    const uint32_t cinc = wave_incl_scan(v.nch);
    v.cst = cinc - v.nch;
    v.C = lane_value(cinc, SG_WAVE - 1);
    v.oidx = p.out_idx + (uint64_t)w * p.k;
    v.oval = static_cast<char*>(p.out_val) + (uint64_t)w * p.k * (BF16 ? 2u : 4u);
    uint32_t cur_tile = 0xffffffffu, eqr = 0;
    uint64_t pos = 0;
    for (uint32_t b0 = 0; b0 < v.C;) {
        const uint32_t left = v.C - b0;
        if (left <= 2) {
            write_round<BF16, 2>(p, v, b0, cur_tile, eqr, pos);
            b0 += 2;
        } else if (left <= 4) {
            write_round<BF16, 4>(p, v, b0, cur_tile, eqr, pos);
            b0 += 4;
        } else {
            write_round<BF16, 8>(p, v, b0, cur_tile, eqr, pos);
            b0 += 8;
        }
    }
}

} // namespace sg

using namespace sg;

static uint64_t topk_carve(Carver& c, uint32_t n, uint64_t M, TopkParams* p)
{
    const uint64_t NT = ceil_div(M, TK_TILE);
    const uint64_t nt = (uint64_t)n * NT;
    p->st = c.take<SelState>(n);
    p->tcnt = c.take<uint32_t>(nt);
    p->ccnt = c.take<uint32_t>(nt);
    p->gtx = c.take<uint32_t>(nt);
    p->eqx = c.take<uint32_t>(nt);
    const uint64_t ng = (uint64_t)n * ceil_div(NT, TK_GROUP);
    p->ggt = c.take<uint32_t>(ng);
    p->geq = c.take<uint32_t>(ng);
    p->hist = c.take<uint32_t>((uint64_t)n * TK_BINS);
    p->samples = c.take<uint32_t>((uint64_t)n * TK_SAMPLES);
    p->slot_idx = c.take<uint16_t>(nt * TK_TILE);
    p->slot_val = c.take<uint32_t>(nt * TK_TILE);
    p->slot_key = c.take<uint32_t>(nt * TK_TILE);
    return c.bytes();
}

extern "C" size_t sg_topk_workspace_bytes(uint32_t n, uint64_t M, uint64_t k, sg_dtype dt)
{
    (void)k;
    (void)dt;
    TopkParams p;
    Carver c(nullptr);
    return topk_carve(c, n, M, &p);
}

extern "C" int sg_topk_to_coo(const void* d_dense, sg_dtype dt, uint32_t n, uint64_t M, uint64_t k,
                              uint32_t* d_idx, void* d_val, void* d_ws, size_t ws_bytes, void* stream)
{
    if (n == 0 || M == 0 || M >= (1ull << 32) || k > M || (dt != SG_F32 && dt != SG_BF16)) return SG_EINVAL;
    if (k == 0) return SG_OK;
    if (!d_dense || !d_idx || !d_val || !d_ws) return SG_EINVAL;
    if (ws_bytes < sg_topk_workspace_bytes(n, M, k, dt)) return SG_ECAPACITY;
    if ((uintptr_t)d_dense % 16) return SG_EINVAL;
    if ((uint64_t)n * ceil_div(M, TK_TILE) >= (1ull << 31)) return SG_EUNSUPPORTED; // tiles and tile groups index grids

    TopkParams p;
    Carver c(d_ws);
    topk_carve(c, n, M, &p);
    p.dense = d_dense;
    p.out_idx = d_idx;
    p.out_val = d_val;
    p.M = M;
    p.k = k;
    p.n = n;
    p.NT = (uint32_t)ceil_div(M, TK_TILE);
    p.NG = (uint32_t)ceil_div(p.NT, TK_GROUP);
    p.bf16 = dt == SG_BF16;
    p.keymax = p.bf16 ? 0x7fffu : 0x7fffffffu;
    // a full 16-byte vector must start on a 16-byte boundary in every row
    const bool rows_aligned = (M * (p.bf16 ? 2 : 4)) % 16 == 0;
    hipStream_t st = as_stream(stream);

    topk_gather_kernel<<<dim3(TK_SAMPLES / 256, n), 256, 0, st>>>(p);
    SG_TRY_LAUNCH();
    topk_sample_kernel<<<n, 1024, 0, st>>>(p);
    SG_TRY_LAUNCH();
    const uint64_t ntiles = (uint64_t)n * p.NT;
    const uint64_t fblocks = ceil_div(ntiles, TK_THREADS / SG_WAVE);
    const unsigned fgrid = (unsigned)(fblocks < 16384 ? fblocks : 16384);
    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 0) {
            probe_begin(SG_PROBE_TOPK_FILTER, st);
            if (p.bf16) {
                if (rows_aligned && M >= TK_TILE) topk_filter_pipe_kernel<8><<<fgrid, TK_THREADS, 0, st>>>(p);
                else topk_filter_kernel<8, false, false><<<fgrid, TK_THREADS, 0, st>>>(p);
            } else {
                if (rows_aligned && M >= TK_TILE) topk_filter_pipe_kernel<4><<<fgrid, TK_THREADS, 0, st>>>(p);
                else topk_filter_kernel<4, false, false><<<fgrid, TK_THREADS, 0, st>>>(p);
            }
            SG_TRY_LAUNCH();
            probe_end(SG_PROBE_TOPK_FILTER, st);
        } else {
            // the re-filter of a missed band (rare): a smaller grid, so the
            // usual launch, which finds nothing to do, ends at once
            const unsigned rgrid = fgrid < 2048u ? fgrid : 2048u;
            if (p.bf16) {
                if (rows_aligned) topk_filter_kernel<8, true, true><<<rgrid, TK_THREADS, 0, st>>>(p);
                else topk_filter_kernel<8, false, true><<<rgrid, TK_THREADS, 0, st>>>(p);
            } else {
                if (rows_aligned) topk_filter_kernel<4, true, true><<<rgrid, TK_THREADS, 0, st>>>(p);
                else topk_filter_kernel<4, false, true><<<rgrid, TK_THREADS, 0, st>>>(p);
            }
            SG_TRY_LAUNCH();
        }
        topk_totals_kernel<<<n, 1024, 0, st>>>(p, pass);
        SG_TRY_LAUNCH();
    }
    if (p.NG <= TK_SMALL_GROUPS) {
        topk_select_small_kernel<<<n, 1024, 0, st>>>(p);
        SG_TRY_LAUNCH();
    } else {
        const unsigned hgrid = n * (unsigned)ceil_div((uint64_t)p.NG * (TK_GROUP / TK_HIST_TPW), TK_THREADS / SG_WAVE);
        for (int pass = 0; pass < 3; ++pass) {
            topk_hist_kernel<<<hgrid, TK_THREADS, 0, st>>>(p);
            SG_TRY_LAUNCH();
            topk_pick_kernel<<<n, TK_THREADS, 0, st>>>(p);
            SG_TRY_LAUNCH();
        }
    }
    const unsigned wgridw = (unsigned)ceil_div((uint64_t)n * p.NG * TK_WRITE_WAVES, TK_THREADS / SG_WAVE);
    if (p.NG > TK_SMALL_GROUPS) { // the small-input selection also counted the tiles
        topk_tilecount_kernel<<<(unsigned)ceil_div((uint64_t)n * p.NG, TK_THREADS / SG_WAVE), TK_THREADS, 0, st>>>(p);
        SG_TRY_LAUNCH();
        topk_scan_kernel<<<n, 1024, 0, st>>>(p);
        SG_TRY_LAUNCH();
    }
    probe_begin(SG_PROBE_TOPK_WRITE, st);
    if (p.bf16) topk_write_kernel<true><<<wgridw, TK_THREADS, 0, st>>>(p);
    else topk_write_kernel<false><<<wgridw, TK_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_TOPK_WRITE, st);
    return SG_OK;
}

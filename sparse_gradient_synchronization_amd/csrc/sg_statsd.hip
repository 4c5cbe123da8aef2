// sg_statsd.hip -- the dense statistics pass of A6, for up to 16 workers and
// 16 parts when the index sets are not too sparse for their key space.
//
// Zen OSDI'25 digest, section 2.1 (Defs. 3-5) and section 3.1 (Def. 8) need
// the union of the workers' index sets, every pairwise intersection, the
// union's count per contiguous part and per hash class, and each worker's
// count per part and per class.  Here every worker's set becomes a bitmap of
// the whole key space in HBM (n * ceil(M/32) words); the pass that builds the
// bitmaps also counts each worker's entries per class, and one streaming
// pass over the bitmaps takes every other count:
//
//   build  a block takes 4096 consecutive list entries.  Each list ascends,
//          so a worker's entries in the block span a range of words; their
//          bits are OR-ed into an LDS copy of that range (8192 words at a
//          time), whose nonzero words are written out with plain stores
//          inside and atomic ORs at its two ends (the neighbouring blocks may
//          have entries in those words).  The same
//          pass counts each worker's entries per hash class (LDS counters,
//          added to the result at the block's end).
//   count  a wave takes a contiguous range of words, 64 at a time (lane l:
//          word i0 + l).  The union word is the OR of the n workers' words;
//          |I_a & I_b| accumulates popcount(W_a & W_b); the union's classes
//          come from the class map's bit planes of the same 32 keys; the
//          union's and each worker's counts go to the contiguous part of the
//          words' keys (64 words usually lie in one part: one wave sum when
//          the part changes; a step across a part boundary counts per key).
//          Each wave writes one partial row; a last pass sums the rows.
//
// Cost: zeroing and one read of the bitmaps, one read of the lists and the
// planes; the sparse passes (windows, merge) cost a few instructions per
// entry and several dependent loads per window instead.
#include "sg_host.h"

namespace sg {

constexpr uint32_t DN_MAXN = 16;          // workers
constexpr uint32_t DN_MAXP = 16;          // parts and hash classes
constexpr uint32_t DN_MAX_WAVES = 2048;   // waves (partial rows) of the count pass, at most
constexpr uint32_t DN_CHUNK = 4096;       // list entries per chunk of the build, at most (16 per thread)
constexpr uint32_t DN_BUILD_BLOCKS = 1024; // build blocks (they stride over the chunks), at most
constexpr uint32_t DN_SPAN = 8192;        // LDS words of a build block's window of keys
constexpr uint32_t DN_WINDOWS = 64;       // windows of a worker's run in a build block, at most

struct DnParams {
    const uint32_t* idx;
    const uint64_t* in_off;
    uint64_t total, M, words; // words = ceil(M / 32)
    uint32_t n, P;
    double inv_m;
    uint32_t* bm;             // [n][words] worker bitmaps
    const uint32_t* planes;   // class map bit planes [chunk][stride] (null: no classes)
    uint32_t nbits, stride;
    const uint32_t* seed_at;  // class map seed (device)
    int classes;              // a class map is given: count each worker's entries per class
    Divider div;
    uint64_t* whashed;        // [n*P] per-worker class counts, accumulated
    uint64_t* rows;           // [W][st_row] partial rows
    uint32_t st_row;          // npairs + 1 + 2P + nP
    uint32_t npairs;
    uint64_t wpw;             // words per wave (a multiple of 64)
};

// A block takes chunks of 256 U consecutive list entries (all loads of a
// chunk at once; blocks stride over the chunks, so the class counts are
// added to the result once per block) and,
// for each worker's part of them (a sorted run of keys), ORs their bits into
// an LDS copy of the words the run spans (DN_SPAN words at a time), then
// writes the nonzero words out: plain stores inside the span (no other entry
// falls there), atomic ORs at its two ends (the neighbouring chunks may have
// entries in the same words).  A run spanning more than DN_WINDOWS windows,
// or not ascending, ORs its bits into the bitmap one entry at a time.
// U entries per thread: 16 for large lists; fewer (chunks of 256 U entries)
// when the lists are short, so that a small input still spreads over many
// blocks instead of zeroing and scanning a wide LDS span in a few.
template <uint32_t U>
__global__ __launch_bounds__(256) void dn_build_kernel(DnParams d)
{
    constexpr uint32_t CHUNK = 256 * U;
    __shared__ uint64_t off[DN_MAXN + 1];
    __shared__ uint32_t hh[DN_MAXN * DN_MAXP];
    __shared__ uint32_t span[DN_SPAN];
    const bool classes = d.classes != 0;
    if (threadIdx.x == 0) { // clamped, non-decreasing list offsets
        uint64_t prev = 0;
        for (uint32_t w = 0; w <= d.n; ++w) {
            uint64_t v = d.in_off[w];
            if (v > d.total) v = d.total;
            if (v < prev) v = prev;
            off[w] = v;
            prev = v;
        }
    }
    for (uint32_t i = threadIdx.x; i < DN_MAXN * DN_MAXP; i += 256) hh[i] = 0;
    __syncthreads();
    const uint32_t hseed = classes ? d.seed_at[0] : 0u;
    for (uint64_t c0 = (uint64_t)blockIdx.x * CHUNK; c0 < d.total; c0 += (uint64_t)gridDim.x * CHUNK) {
        const uint32_t len_c = (uint32_t)(d.total - c0 < CHUNK ? d.total - c0 : CHUNK);
        const uint32_t* const src = d.idx + c0;
        uint32_t key[U]; // entry r = j * 256 + threadIdx.x of the chunk
#pragma unroll
        for (uint32_t j = 0; j < U; ++j) {
            const uint32_t r = j * 256 + threadIdx.x;
            key[j] = src[r < len_c ? r : len_c - 1];
        }
        for (uint32_t w = 0; w < d.n; ++w) { // the workers whose lists meet the chunk (uniform)
            const uint64_t ea = off[w] > c0 ? off[w] : c0, eb = off[w + 1] < c0 + len_c ? off[w + 1] : c0 + len_c;
            if (ea >= eb) continue;
            const uint32_t ra = (uint32_t)(ea - c0), rb = (uint32_t)(eb - c0); // the run: entries [ra, rb)
            const uint32_t ka = src[ra], kb = src[rb - 1];
            const uint32_t wa = ka >> 5, wb = kb >> 5;
            uint32_t* const row = d.bm + (uint64_t)w * d.words;
            uint32_t mine = 0; // bit j: entry j * 256 + threadIdx.x is in the run
#pragma unroll
            for (uint32_t j = 0; j < U; ++j) mine |= (uint32_t)(j * 256 + threadIdx.x - ra < rb - ra) << j;
            // the run's words in windows of DN_SPAN; a run that does not ascend,
            // or spans more than DN_WINDOWS windows, goes one entry at a time
            const bool staged = ka <= kb && kb < d.M && wb - wa < DN_WINDOWS * DN_SPAN;
            const uint32_t S = staged ? wb - wa + 1 : 0u;
            if (!staged) {
#pragma unroll
                for (uint32_t j = 0; j < U; ++j)
                    if (((mine >> j) & 1u) && key[j] < d.M) atomicOr(&row[key[j] >> 5], 1u << (key[j] & 31u));
            }
            for (uint32_t base = 0; base < S; base += DN_SPAN) {
                const uint32_t len = S - base < DN_SPAN ? S - base : DN_SPAN;
                for (uint32_t i = threadIdx.x; i < len; i += 256) span[i] = 0;
                __syncthreads();
#pragma unroll
                for (uint32_t j = 0; j < U; ++j) {
                    const uint32_t o = (key[j] >> 5) - wa - base; // wraps for words below the window
                    if (((mine >> j) & 1u) && o < len) atomicOr(&span[o], 1u << (key[j] & 31u));
                }
                __syncthreads();
                for (uint32_t i0 = threadIdx.x; i0 < len; i0 += 4 * 256) { // four LDS reads in flight
                    uint32_t v[4];
#pragma unroll
                    for (uint32_t u = 0; u < 4; ++u) v[u] = i0 + u * 256 < len ? span[i0 + u * 256] : 0u;
#pragma unroll
                    for (uint32_t u = 0; u < 4; ++u) {
                        const uint32_t i = i0 + u * 256;
                        if (!v[u]) continue; // the bitmap starts zeroed (and words past the window read 0)
                        if (base + i == 0 || base + i == S - 1) atomicOr(&row[wa + base + i], v[u]);
                        else row[wa + base + i] = v[u];
                    }
                }
                __syncthreads(); // the span is reused
            }
            // range check and class counts, once per entry
#pragma unroll
            for (uint32_t j = 0; j < U; ++j) {
                if (!((mine >> j) & 1u)) continue;
                if (key[j] >= d.M) report_error(kDevErrIndexRange);
                else if (classes) atomicAdd(&hh[w * d.P + h0(key[j], hseed, d.div)], 1u);
            }
        }
    }
    if (!classes) return;
    __syncthreads(); // every class count of the block is in
    for (uint32_t i = threadIdx.x; i < d.n * d.P; i += 256)
        if (hh[i]) atomicAdd((unsigned long long*)&d.whashed[i], (unsigned long long)hh[i]);
}

// The count pass.  N (8 or 16) bounds the workers at compile time, so the
// pair counters stay in registers; words of workers >= n are zero.
template <int N, bool HASHED>
__global__ __launch_bounds__(256) void dn_count_kernel(DnParams d)
{
    constexpr int NP = N * (N - 1) / 2;
    __shared__ uint32_t lpart[4][DN_MAXP];          // union per contiguous part
    __shared__ uint32_t lwork[4][DN_MAXN * DN_MAXP]; // worker a, part q at a * P + q
    const uint32_t wid = uniform(threadIdx.x / SG_WAVE), lane = lane_id();
    const uint32_t k = blockIdx.x * 4 + wid;
    uint32_t* const upart = lpart[wid];
    uint32_t* const wpart = lwork[wid];
    for (uint32_t i = lane; i < DN_MAXP; i += SG_WAVE) upart[i] = 0;
    for (uint32_t i = lane; i < DN_MAXN * DN_MAXP; i += SG_WAVE) wpart[i] = 0;
    wave_sync();

    uint32_t pacc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) pacc[i] = 0;
    uint32_t hacc[DN_MAXP];
#pragma unroll
    for (int i = 0; i < (int)DN_MAXP; ++i) hacc[i] = 0;
    uint32_t uacc = 0;
    // running counts of the current contiguous part
    uint32_t cur = 0xffffffffu, cu = 0, cw[N];
#pragma unroll
    for (int a = 0; a < N; ++a) cw[a] = 0;
    auto flush = [&]() {
        if (cur == 0xffffffffu) return;
        const uint32_t s = wave_sum(cu);
        if (lane == 0 && s) atomicAdd(&upart[cur], s);
#pragma unroll
        for (int a = 0; a < N; ++a) {
            const uint32_t t = wave_sum(cw[a]); // 0 for workers >= n
            if (lane == 0 && t) atomicAdd(&wpart[a * d.P + cur], t);
            cw[a] = 0;
        }
        cu = 0;
    };

    const uint64_t ib = (uint64_t)k * d.wpw;
    const uint64_t ie = ib + d.wpw < d.words ? ib + d.wpw : d.words;
    for (uint64_t i0 = ib; i0 < ie; i0 += SG_WAVE) {
        const uint64_t i = i0 + lane;
        const bool live = i < ie;
        const uint64_t ic = live ? i : ib;
        uint32_t Wd[N];
        uint32_t U = 0;
#pragma unroll
        for (int a = 0; a < N; ++a) {
            Wd[a] = (uint32_t)a < d.n ? d.bm[(uint64_t)a * d.words + ic] : 0u;
            if (!live) Wd[a] = 0u;
            U |= Wd[a];
        }
        uacc += __popc(U);
        {
            int pi = 0;
#pragma unroll
            for (int a = 0; a < N; ++a)
#pragma unroll
                for (int b = a + 1; b < N; ++b) pacc[pi++] += __popc(Wd[a] & Wd[b]);
        }
        if (HASHED) { // 1 <= nbits <= 4
            uint32_t pl[4];
            if (d.stride == 4) {
                const uint4 q = *reinterpret_cast<const uint4*>(d.planes + ic * 4);
                pl[0] = q.x;
                pl[1] = q.y;
                pl[2] = q.z;
                pl[3] = q.w;
            } else {
#pragma unroll
                for (uint32_t b = 0; b < 4; ++b) pl[b] = d.planes[ic * d.stride + (b < d.nbits ? b : d.nbits - 1)];
            }
#pragma unroll
            for (int c = 0; c < (int)DN_MAXP; ++c) {
                uint32_t m = U;
#pragma unroll
                for (uint32_t b = 0; b < 4; ++b)
                    if (b < d.nbits) m &= ((c >> b) & 1) ? pl[b] : ~pl[b];
                hacc[c] += (uint32_t)c < d.P ? __popc(m) : 0u;
            }
        }
        // the contiguous parts of this step's keys [32 i0, 32 min(i0 + 64, ie)) clipped to M
        const uint64_t klast = (i0 + SG_WAVE < ie ? i0 + SG_WAVE : ie) * 32;
        const uint32_t pf = contig_part(i0 * 32, d.M, d.P, d.inv_m);
        const uint32_t pl_ = contig_part((klast < d.M ? klast : d.M) - 1, d.M, d.P, d.inv_m);
        if (pf == pl_) {
            if (pf != cur) {
                flush();
                cur = pf;
            }
            cu += __popc(U);
#pragma unroll
            for (int a = 0; a < N; ++a) cw[a] += __popc(Wd[a]);
        } else { // across a part boundary: part by key
            const uint64_t kw = i * 32;
            for (uint32_t rest = U; rest; rest &= rest - 1)
                atomicAdd(&upart[contig_part(kw + __builtin_ctz(rest), d.M, d.P, d.inv_m)], 1u);
            for (int a = 0; a < N; ++a)
                for (uint32_t rest = Wd[a]; rest; rest &= rest - 1)
                    atomicAdd(&wpart[a * d.P + contig_part(kw + __builtin_ctz(rest), d.M, d.P, d.inv_m)], 1u);
        }
    }
    flush();
    wave_sync();

    // this wave's partial row: pairs (a <= b; the diagonal is left 0, the
    // host takes it from the list lengths), union, union per contiguous part,
    // union per class, each worker's count per contiguous part
    uint64_t* row = d.rows + (uint64_t)k * d.st_row;
    // pair (a, b), a <= b < n, sits at a*n - a(a-1)/2 + (b - a)
    for (uint32_t a = lane; a < d.n; a += SG_WAVE) row[a * d.n - a * (a - 1) / 2] = 0;
    {
        int pi = 0;
#pragma unroll
        for (uint32_t a = 0; a < (uint32_t)N; ++a) {
#pragma unroll
            for (uint32_t b = a + 1; b < (uint32_t)N; ++b) {
                const uint32_t s = wave_sum(pacc[pi++]);
                if (b < d.n && lane == 0) row[a * d.n - a * (a - 1) / 2 + (b - a)] = s;
            }
        }
    }
    const uint32_t us = wave_sum(uacc);
    if (lane == 0) row[d.npairs] = us;
    for (uint32_t i = lane; i < d.P; i += SG_WAVE) row[d.npairs + 1 + i] = upart[i];
#pragma unroll
    for (int i = 0; i < (int)DN_MAXP; ++i) {
        const uint32_t s = wave_sum(hacc[i]);
        if ((uint32_t)i < d.P && lane == 0) row[d.npairs + 1 + d.P + i] = HASHED ? s : 0u;
    }
    for (uint32_t i = lane; i < d.n * d.P; i += SG_WAVE) row[d.npairs + 1 + 2 * d.P + i] = wpart[i];
}

} // namespace sg

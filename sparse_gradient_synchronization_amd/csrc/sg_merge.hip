// sg_merge.hip -- the n-way sorted-run union engine behind A3 (aggregate)
// and A6 (statistics).
//
// Input: G groups of n sorted runs each (aggregate: group = partition p, run
// (w, p) = worker w's partition-p entries from the hash partition; statistics:
// one group whose runs are the workers' index lists).  Output per group: the
// union of its runs in ascending order, each index with its values summed in
// worker order (aggregate), or exact union / pairwise-intersection counts
// (statistics).
//
// Design for gfx950:
//   tiles  the key space of every group is cut into fixed tiles of 2^tb keys
//          (tb chosen from the mean density so a tile holds a few hundred
//          entries); tile t = g * NT + b.
//   bnd    one streaming pass over the run entries records, per run, where
//          each tile begins (plain stores, no atomics, no search).
//   merge  a wave merges one tile at a time with no block barrier: it loads
//          the tile's entries of all n runs (at most MG_WCAP at once; a
//          denser tile is consumed in windows that end at the smallest
//          last-loaded key of a cut run), sets one bit per key in an LDS
//          bitmap of the tile's span, and prefix popcounts give every key its
//          rank among the distinct keys.  A 64-bit mask per rank records the
//          workers holding it; the entries are then laid out by (rank,
//          worker), so each rank's contributions are summed in worker order
//          (the order of a ring) by one lane, deterministically.  Aggregate
//          output goes to a staging area at the tile's input offset (a tile
//          never has more distinct keys than entries), so tiles are
//          independent.  Waves are persistent: tiles with many entries are
//          dealt out first, the rest come from 64 queues of contiguous tiles
//          with a ticket counter each.
//   place  a scan of the tiles' distinct counts and a copy of every tile's
//          staged entries to its final offset.
#include "sg_host.h"

namespace sg {

constexpr int MG_WAVES = 4;                          // waves per block
constexpr int MG_THREADS = MG_WAVES * SG_WAVE;
constexpr int MG_WCAP = 256;                         // entries of a window
constexpr int MG_PER = MG_WCAP / SG_WAVE;            // entries per lane
constexpr int MG_SPAN_LOG = 13;                      // a tile spans at most 2^13 keys
constexpr int MG_WORDS = (1 << MG_SPAN_LOG) / 32;    // bitmap words of a span
constexpr int MG_WPL = MG_WORDS / SG_WAVE;           // bitmap words per lane
constexpr int MG_TARGET = 128;                       // mean entries per tile aimed at
constexpr int MG_CHUNK = 4096;                       // run entries per bnd block
constexpr int MG_HEAVY = 2 * MG_WCAP;                // a tile with more entries is scheduled first
constexpr int MG_CHUNK_TILES = 4;                    // tiles per work ticket
constexpr int MG_NQ = 64;                            // work queues (contiguous tile ranges)
constexpr int MG_QSTRIDE = 64;                       // words between queue counters (separate lines)
constexpr int MG_SCAN_PER = 8;                       // tiles per thread in the tile scan
constexpr int MG_SCAN_BLOCK = 1024 * MG_SCAN_PER;    // tiles per scan block
static_assert(MG_WCAP >= 64, "a window must hold one entry of each of up to 64 runs");
static_assert(MG_WORDS >= MG_WCAP, "ranks reuse the bitmap words");

enum MergeMode { MODE_AGG = 0, MODE_STATS = 1 };

struct MergeParams {
    // runs: run (g, w) = [off[w*stride + g], off[w*stride + g + 1])
    const uint32_t* idx;
    const uint64_t* off;
    uint32_t stride;
    uint32_t G, n;
    uint64_t total;
    uint64_t M;
    uint32_t tb;            // tile width 2^tb keys
    uint32_t NT;            // tiles per group
    // values (aggregate)
    const void* val;
    uint32_t D;
    int bf16;
    uint32_t* agg_idx;
    float* agg_val;
    uint64_t* agg_off;      // [G+1]
    uint64_t capacity;
    // workspace
    uint32_t* chunk_start;  // [n*G + 1] bnd blocks per run (position order)
    uint4* chunk_rec;       // [nchunks_max] bnd block c: {run (position order) or ~0, first entry in the run, run length, run start}
    uint32_t nchunks_max;   // bnd blocks launched
    uint32_t* bnd;          // [(g*n + w) * (NT+1) + b]
    uint32_t* tile_cnt;     // [G*NT] distinct keys of a tile
    uint64_t* tile_sb;      // [G*NT] staging offset of a tile
    uint64_t* tile_out;     // [G*NT] exclusive prefix inside its scan block
    uint64_t* blk_sum;      // [nscan] scan block totals, then their exclusive prefix
    uint32_t nscan;
    uint32_t* stage_idx;    // [total]
    float* stage_val;       // [total] (D <= 1)
    // rows (D >= 2): sums are formed after the merge, one output row per wave
    uint32_t* stage_src;    // [total] contributors' entry positions, by (staged key, worker), tile-relative layout
    uint32_t* stage_first;  // [total] a staged key's first contributor, relative to its tile's staging base
    uint32_t* tile_ent;     // [G*NT] entries of a tile
    uint2* row_rng;         // [total] output row o: its contributors are stage_src[x .. y)
    uint32_t* queue;        // [nqsets * MG_NQ * MG_QSTRIDE]: queue[0] heavy tiles listed; queue[(s * MG_NQ + q) * MG_QSTRIDE + 1]
                            // chunk tickets of queue q in set s (one set per pass over the tiles)
    uint32_t nqsets;        // counter sets in queue
    // union engine (sg_union.hip): waves take contiguous tile ranges of equal work
    uint32_t* work;         // [G*NT] work of a tile
    uint64_t* wcum;         // [G*NT] exclusive prefix of the work inside its scan block
    uint64_t* wblk;         // [nscan] scan block totals, then their exclusive prefix
    uint64_t* wtotal;       // [1] total work
    uint32_t* wstart;       // [nwaves+1] first tile of wave k
    uint64_t* wave_tot;     // [nwaves+1] union size of wave k's tiles, then its exclusive prefix
    uint32_t nwaves;
    uint32_t* heavy;        // [G*NT] tiles with more than MG_HEAVY entries
    // statistics
    uint64_t* st_part;      // [grid][st_row] per-block partial counts
    uint32_t st_row;        // words per partial row: npairs + 1 + 2*Ps
    uint32_t npairs;
    uint32_t Ps;            // parts for skew
    double inv_m;           // 1 / M
    uint32_t seed;
    const uint32_t* seed_at; // when set, the seed is read here on the device (a class map header)
    int hashed;
    Divider div;
};

__device__ __forceinline__ void run_range(const MergeParams& p, uint32_t g, uint32_t w, uint64_t& s, uint64_t& e)
{
    uint64_t a = p.off[(uint64_t)w * p.stride + g], b = p.off[(uint64_t)w * p.stride + g + 1];
    if (a > p.total) a = p.total;
    if (b > p.total) b = p.total;
    if (b < a) b = a;
    s = a;
    e = b;
}

// runs in position order: r' = w*G + g
__global__ __launch_bounds__(512) void mg_plan_kernel(MergeParams p)
{
    __shared__ uint32_t scan_lds[512 / SG_WAVE + 1];
    const uint32_t R = p.n * p.G;
    uint32_t carry = 0;
    for (uint32_t base = 0; base < R; base += 512) {
        const uint32_t r = base + threadIdx.x;
        uint32_t c = 0;
        if (r < R) {
            uint64_t s, e;
            run_range(p, r % p.G, r / p.G, s, e);
            c = (uint32_t)ceil_div_dev(e - s, MG_CHUNK);
        }
        uint32_t tot;
        uint32_t ex = block_excl_scan<512>(c, scan_lds, &tot);
        if (r < R) p.chunk_start[r] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) p.chunk_start[R] = carry;
    const uint32_t qwords = (p.nqsets > 1 ? p.nqsets : 1u) * (uint32_t)(MG_NQ * MG_QSTRIDE);
    for (uint32_t i = threadIdx.x; i < qwords; i += 512) p.queue[i] = 0;
    __syncthreads();
    // block -> run table of the boundary pass
    for (uint32_t r = threadIdx.x / SG_WAVE; r < R; r += 512 / SG_WAVE) { // one wave per run
        const uint32_t c0 = p.chunk_start[r], c1 = p.chunk_start[r + 1];
        uint64_t s, e;
        run_range(p, r % p.G, r / p.G, s, e);
        for (uint32_t c = c0 + lane_id(); c < c1; c += SG_WAVE)
            p.chunk_rec[c] = make_uint4(r, (c - c0) * MG_CHUNK, (uint32_t)(e - s), (uint32_t)s);
    }
    for (uint32_t c = p.chunk_start[R] + threadIdx.x; c < p.nchunks_max; c += 512)
        p.chunk_rec[c] = make_uint4(0xffffffffu, 0u, 0u, 0u);
}

__device__ __forceinline__ uint32_t tile_of(const MergeParams& p, uint32_t key)
{
    uint64_t b = (uint64_t)key >> p.tb;
    if (b >= p.NT) {
        report_error(kDevErrIndexRange);
        b = p.NT - 1;
    }
    return (uint32_t)b;
}

// bnd[run][b] = first position (relative to the run) whose key is >= b * 2^tb;
// bnd[run][NT] = the run's length.  A block takes a 4096-entry chunk; thread
// t looks at entries t, t + 512, ... of it (coalesced loads), each with the
// entry before it, and writes the tile starts that fall between the two.
// All loads are issued and waited for before the first store.
__global__ __launch_bounds__(512) void mg_bnd_kernel(MergeParams p)
{
    constexpr int E = MG_CHUNK / 512;
    // the rows of empty runs (which have no chunk) are all zero; block r
    // looks after run r (the grid has at least one block per run)
    for (uint32_t r = blockIdx.x; r < p.n * p.G; r += gridDim.x) {
        uint64_t s, e;
        run_range(p, r / p.n, r % p.n, s, e); // row r = g * n + w
        if (s == e)
            for (uint32_t x = threadIdx.x; x <= p.NT; x += 512) p.bnd[(uint64_t)r * (p.NT + 1) + x] = 0;
    }
    for (uint32_t c = blockIdx.x; c < p.nchunks_max; c += gridDim.x) {
    const uint4 rec = p.chunk_rec[c];
    if (rec.x == 0xffffffffu) continue;
    const uint32_t rp = rec.x, g = rp % p.G, w = rp / p.G;
    const uint64_t s = rec.w, len = rec.z;
    uint32_t* row = p.bnd + ((uint64_t)g * p.n + w) * (p.NT + 1);
    uint32_t key[E], prev[E];
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const uint64_t j = (uint64_t)rec.y + (uint64_t)u * 512 + threadIdx.x;
        const uint64_t jc = j < len ? j : len - 1; // len > 0: the run has this chunk
        key[u] = p.idx[s + jc];
        prev[u] = p.idx[s + (jc > 0 ? jc - 1 : 0)];
    }
    wait_vmem();
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const uint64_t j = (uint64_t)rec.y + (uint64_t)u * 512 + threadIdx.x;
        if (j >= len) break;
        const uint32_t b = tile_of(p, key[u]);
        const uint32_t x0 = j > 0 ? tile_of(p, prev[u]) + 1 : 0u;
        for (uint32_t x = x0; x <= b; ++x) row[x] = (uint32_t)j;
        if (j == len - 1)
            for (uint64_t x = (uint64_t)b + 1; x <= p.NT; ++x) row[x] = (uint32_t)len;
    }
    }
}

// Tiles with more than MG_HEAVY entries, listed so the merge starts them
// first (longest first keeps the last waves short).  A tile's entry count is
// the sum over its runs of bnd[b + 1] - bnd[b]; the loads of 8 runs are
// issued together (rows past the last run read run 0's row and are not
// counted).  The count only orders the work, so a row is not checked here
// against its run's length (the merge does that).  Appends to the list are
// gathered per block (one device-scope atomic per block and round: a single
// counter hit by every wave of the chip serializes).
__global__ __launch_bounds__(256) void mg_heavy_kernel(MergeParams p)
{
    __shared__ uint32_t wcnt[256 / SG_WAVE], wofs[256 / SG_WAVE + 1];
    const uint32_t T = p.G * p.NT;
    const uint32_t wid = uniform(threadIdx.x / SG_WAVE);
    for (uint32_t t0 = blockIdx.x * 256; t0 < T; t0 += gridDim.x * 256) { // uniform per block
        const uint32_t t = t0 + threadIdx.x;
        const bool valid = t < T;
        const uint32_t tc = valid ? t : T - 1;
        const uint32_t g = tc / p.NT, b = tc % p.NT;
        uint32_t E = 0;
        const uint32_t* rows = p.bnd + (uint64_t)g * p.n * (p.NT + 1) + b;
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
        const bool hv = valid && E > (uint32_t)MG_HEAVY;
        const uint64_t m = ballot(hv);
        if (lane_id() == 0) wcnt[wid] = (uint32_t)popc64(m);
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t sum = 0;
            for (uint32_t i = 0; i < 256 / SG_WAVE; ++i) {
                wofs[i] = sum;
                sum += wcnt[i];
            }
            wofs[256 / SG_WAVE] = sum ? atomicAdd(&p.queue[0], sum) : 0u;
        }
        __syncthreads();
        if (hv) p.heavy[wofs[256 / SG_WAVE] + wofs[wid] + count_below(m)] = t;
        __syncthreads(); // wcnt and wofs are reused
    }
}

// Contiguous part of `key` among P parts [floor(iM/P), floor((i+1)M/P)):
// the largest i with i*M < (key+1)*P, i.e. floor(((key+1)P - 1) / M).  The
// quotient is estimated in double (x < 2^40, so it is off by at most one)
// and corrected with exact integer products.
__device__ __forceinline__ uint32_t contig_part(uint64_t key, uint64_t M, uint32_t P, double inv_m)
{
    const uint64_t x = (key + 1) * P - 1;
    uint64_t q = (uint64_t)((double)x * inv_m);
    if (q * M > x) --q;
    else if ((q + 1) * M <= x) ++q;
    return q < P ? (uint32_t)q : P - 1;
}

// Counts of a wave's keys per part into LDS counters h.  Keys in ascending
// order have non-decreasing contiguous parts: when the first and the last
// agree (the usual case), one add counts them all.
__device__ __forceinline__ void count_sorted_parts(uint32_t* h, uint32_t part, bool has)
{
    const uint64_t act = ballot(has);
    if (!act) return;
    const uint32_t fl = (uint32_t)__builtin_ctzll(act), ll = 63u - (uint32_t)__builtin_clzll(act);
    const uint32_t pf = (uint32_t)__builtin_amdgcn_readlane((int)part, (int)fl);
    const uint32_t pl = (uint32_t)__builtin_amdgcn_readlane((int)part, (int)ll);
    if (pf == pl) {
        if (lane_id() == fl) atomicAdd(&h[pf], popc64(act));
    } else if (has) {
        atomicAdd(&h[part], 1u);
    }
}

// Counts of a wave's keys per part for parts in any order: one ballot per
// part when there are few, else one LDS atomic per key.
__device__ __forceinline__ void count_parts(uint32_t* h, uint32_t part, bool has, uint32_t P)
{
    if (P <= 16) {
        for (uint32_t b = 0; b < P; ++b) {
            const uint32_t c = popc64(ballot(has && part == b));
            if (c && lane_id() == 0) atomicAdd(&h[b], c);
        }
    } else if (has) {
        atomicAdd(&h[part], 1u);
    }
}

// the lanes' (a, b) worker pair of pair index pi, a <= b, row-major
__device__ __forceinline__ void pair_of(uint32_t pi, uint32_t n, uint32_t& a, uint32_t& b)
{
    uint32_t x = 0, rem = pi;
    while (rem >= n - x) {
        rem -= n - x;
        ++x;
    }
    a = x;
    b = x + rem;
}

struct alignas(16) WaveSmem {
    uint32_t bits[MG_WORDS];         // presence bitmap of the window's keys; then keys by rank
    uint16_t wpre[MG_WORDS];         // distinct keys before a bitmap word; then first slot of a rank
    unsigned long long mask[MG_WCAP]; // workers holding a rank
    uint32_t slot[MG_WCAP];          // by (rank, worker): value bits (D == 1) or entry position (rows)
    uint32_t wofs[65];               // window offset of run w
    uint32_t untaken[64];            // loaded entries of run w beyond the window's cut
    uint32_t cut[64];                // run w continues after the window
    uint64_t src[64];                // absolute position of run w's first loaded entry
    unsigned long long vm[64];       // statistics: per worker, which of 64 ranks it holds
};

template <int MODE>
struct BlockSmem {
    WaveSmem wv[MG_WAVES];
    uint32_t part[MODE == MODE_STATS ? 512 : 1];  // statistics: union counts per contiguous / hashed part
    uint32_t pairs[MODE == MODE_STATS ? 2080 : 1];  // a block's pair counts stay below 2^32 (total does)
};

// A tile's part of each run, held by lane w < n (positions relative to the
// run; below 2^32 since total is).
struct TileRuns {
    uint64_t rs;    // absolute start of run (g, w)
    uint32_t cur;   // next entry
    uint32_t end;   // end of the tile's part
    uint32_t base;  // aggregate staging: the run's entries before this tile, earlier groups included
};

// Loads of a tile's run ranges (independent of each other: one round trip).
__device__ __forceinline__ TileRuns tile_runs(const MergeParams& p, uint32_t t, uint32_t lane)
{
    TileRuns r = {0ull, 0u, 0u, 0u};
    if (lane < p.n && t < p.G * p.NT) {
        const uint32_t g = t / p.NT, b = t % p.NT;
        uint64_t s, e;
        run_range(p, g, lane, s, e);
        const uint64_t len = e - s;
        const uint32_t* row = p.bnd + ((uint64_t)g * p.n + lane) * (p.NT + 1);
        uint64_t x = row[b], y = row[b + 1];
        if (x > len) x = len;
        if (y > len) y = len;
        if (y < x) y = x;
        r.rs = s;
        r.cur = (uint32_t)x;
        r.end = (uint32_t)y;
        r.base = (uint32_t)(s - p.off[(uint64_t)lane * p.stride] + x);
    }
    return r;
}

// Layout of the next window of a tile (E = the tile's remaining entries): all
// of them when they fit, else at most MG_WCAP, shared among the runs by water
// filling (an even share first, then the rest to the runs that still have
// entries).
__device__ __forceinline__ uint32_t begin_window(WaveSmem& sm, const TileRuns& r, uint32_t n, uint32_t lane,
                                                 uint32_t E, uint32_t& take, bool& windowed)
{
    const uint32_t rem = r.end - r.cur;
    windowed = E > (uint32_t)MG_WCAP;
    if (!windowed) {
        take = rem;
    } else {
        const uint32_t nz = wave_sum(rem > 0 ? 1u : 0u);
        const uint32_t q1 = (uint32_t)MG_WCAP / nz;
        take = rem < q1 ? rem : q1;
        const uint32_t left = (uint32_t)MG_WCAP - wave_sum(take);
        const uint32_t nb = wave_sum(rem > take ? 1u : 0u);
        if (left > 0 && nb > 0) {
            const uint32_t q2 = left / nb, more = rem - take;
            take += more < q2 ? more : q2;
        }
    }
    const uint32_t incl = wave_incl_scan(take);
    const uint32_t L = (uint32_t)__builtin_amdgcn_readlane((int)incl, SG_WAVE - 1);
    if (lane < n) {
        sm.wofs[lane] = incl - take;
        sm.src[lane] = r.rs + r.cur;
        sm.cut[lane] = take > 0 && r.cur + take < r.end; // the run continues after this window
    }
    if (lane == 0) sm.wofs[n] = L;
    wave_sync();
    return L;
}

// Issue the window's loads into registers: lane l holds window entries
// l*MG_PER .. l*MG_PER + MG_PER - 1 (one run search per lane).
template <int MODE>
__device__ __forceinline__ void load_window(const MergeParams& p, const WaveSmem& sm, uint32_t L, uint32_t n,
                                            uint32_t lane, uint32_t (&key)[MG_PER], uint32_t (&wk)[MG_PER],
                                            uint32_t (&vb)[MG_PER])
{
    const uint32_t lp0 = lane * MG_PER;
    uint32_t lo = 0;
    if (lp0 < L) {
        uint32_t hi = n;
        while (lo + 1 < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (sm.wofs[mid] <= lp0) lo = mid;
            else hi = mid;
        }
    }
#pragma unroll
    for (int i = 0; i < MG_PER; ++i) {
        const uint32_t lp = lp0 + i;
        key[i] = 0;
        wk[i] = 0xffffffffu;
        vb[i] = 0;
        if (lp < L) {
            while (sm.wofs[lo + 1] <= lp) ++lo; // wofs[n] = L > lp ends it
            const uint64_t pos = sm.src[lo] + (lp - sm.wofs[lo]);
            key[i] = p.idx[pos];
            wk[i] = lo;
            if (MODE == MODE_AGG) {
                if (p.D == 1)
                    vb[i] = p.bf16 ? ((uint32_t) static_cast<const uint16_t*>(p.val)[pos] << 16)
                                   : static_cast<const uint32_t*>(p.val)[pos];
                else
                    vb[i] = (uint32_t)pos;
            }
        }
    }
}

// Once the loads are in (windowed tiles only): the window ends at the
// smallest last-loaded key of a run that continues; entries above it go back
// to their runs (counted per run in sm.untaken and dropped here).
__device__ __forceinline__ void finish_window(WaveSmem& sm, uint32_t n, uint32_t lane, const uint32_t (&key)[MG_PER],
                                              uint32_t (&wk)[MG_PER])
{
    uint32_t cutk = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < MG_PER; ++i) {
        const uint32_t lp = lane * MG_PER + i;
        if (wk[i] != 0xffffffffu && sm.cut[wk[i]] && lp + 1 == sm.wofs[wk[i] + 1])
            cutk = key[i] < cutk ? key[i] : cutk;
    }
    const uint32_t kmax = wave_min(cutk);
    if (lane < n) sm.untaken[lane] = 0;
    wave_sync();
#pragma unroll
    for (int i = 0; i < MG_PER; ++i) {
        if (wk[i] != 0xffffffffu && key[i] > kmax) {
            atomicAdd(&sm.untaken[wk[i]], 1u);
            wk[i] = 0xffffffffu;
        }
    }
    wave_sync();
}

// Work of a wave.  Heavy tiles first, dealt out statically (wave w takes
// heavy tiles w, w + W, ...: the longest work starts first).  Then the tiles
// are split into MG_NQ contiguous queues, each with its own ticket counter
// (no single hot address); a wave starts at queue w mod MG_NQ, takes chunks
// of MG_CHUNK_TILES tiles, and when its queue runs dry finds an open one with
// one lane-parallel probe of all counters.
struct WaveWork {
    uint32_t hnext;  // next heavy list index
    uint32_t q;      // current queue
    uint32_t next, end;
    bool heavy_phase;
};

__device__ __forceinline__ uint32_t queue_first(uint32_t q, uint32_t T)
{
    return (uint32_t)(((uint64_t)q * T) / MG_NQ);
}

// Next tile of the wave, or T when none is left.  `set` picks the ticket
// counters (each pass over the tiles has its own; the heavy list is shared).
__device__ __forceinline__ uint32_t acquire_tile(const MergeParams& p, uint32_t T, uint32_t W, WaveWork& k,
                                                 bool& from_heavy, uint32_t set = 0)
{
    uint32_t* const ctr = p.queue + (uint64_t)set * MG_NQ * MG_QSTRIDE + 1;
    if (k.heavy_phase) {
        if (k.hnext < p.queue[0]) {
            const uint32_t t = p.heavy[k.hnext];
            k.hnext += W;
            from_heavy = true;
            return t;
        }
        k.heavy_phase = false;
    }
    from_heavy = false;
    if (k.next < k.end) return k.next++;
    while (true) {
        uint32_t c = 0;
        if (lane_id() == 0) c = atomicAdd(&ctr[k.q * MG_QSTRIDE], 1u);
        c = (uint32_t)__builtin_amdgcn_readfirstlane((int)c);
        const uint64_t first = (uint64_t)queue_first(k.q, T) + (uint64_t)c * MG_CHUNK_TILES;
        const uint32_t qend = queue_first(k.q + 1, T);
        if (first < qend) {
            k.next = (uint32_t)first;
            k.end = (uint32_t)(first + MG_CHUNK_TILES < qend ? first + MG_CHUNK_TILES : qend);
            return k.next++;
        }
        // this queue is empty: probe the others (plain loads, one per lane)
        const uint32_t j = lane_id();
        bool open = false;
        uint32_t qq = 0;
        if (j + 1 < (uint32_t)MG_NQ) {
            qq = (k.q + 1 + j) % MG_NQ;
            const uint32_t v = __atomic_load_n(&ctr[qq * MG_QSTRIDE], __ATOMIC_RELAXED);
            open = (uint64_t)queue_first(qq, T) + (uint64_t)v * MG_CHUNK_TILES < queue_first(qq + 1, T);
        }
        const uint64_t m = ballot(open);
        if (!m) return T;
        k.q = (k.q + 1 + (uint32_t)__builtin_ctzll(m)) % MG_NQ;
    }
}

// Persistent waves take tiles from the work queue.  Inside a tile the next
// window's entries are loaded before the current window is merged.
template <int MODE>
__global__ __launch_bounds__(MG_THREADS) void mg_merge_kernel(MergeParams p)
{
    __shared__ BlockSmem<MODE> bs;
    const uint32_t wid = threadIdx.x / SG_WAVE, lane = lane_id();
    WaveSmem& sm = bs.wv[wid];
    const uint32_t n = p.n;
    const uint32_t T = p.G * p.NT;
    const uint64_t span = 1ull << p.tb;
    uint64_t union_cnt = 0;
    const uint32_t hseed = (MODE == MODE_STATS && p.seed_at) ? p.seed_at[0] : p.seed;
    if (MODE == MODE_STATS) {
        for (uint32_t i = threadIdx.x; i < 2 * p.Ps; i += MG_THREADS) bs.part[i] = 0;
        for (uint32_t i = threadIdx.x; i < p.npairs; i += MG_THREADS) bs.pairs[i] = 0;
        __syncthreads();
    }
    const uint32_t W = gridDim.x * MG_WAVES;
    const uint32_t gwave = blockIdx.x * MG_WAVES + wid;
    // statistics: the lane's first four worker pairs
    uint32_t pair_a[4] = {0, 0, 0, 0}, pair_b[4] = {0, 0, 0, 0};
    if (MODE == MODE_STATS)
        for (int j = 0; j < 4; ++j)
            if (lane + 64u * j < p.npairs) pair_of(lane + 64u * j, n, pair_a[j], pair_b[j]);
    WaveWork work = {gwave, gwave % MG_NQ, 0u, 0u, true};
    bool from_heavy = false;
    uint32_t key[MG_PER], wk[MG_PER], vb[MG_PER];

    while (true) {
        const uint32_t t = acquire_tile(p, T, W, work, from_heavy);
        if (t >= T) break;
        TileRuns cr = tile_runs(p, t, lane);
        uint32_t E = wave_sum(cr.end - cr.cur);
        if (!from_heavy && E > (uint32_t)MG_HEAVY) continue; // merged in the heavy phase
        const uint32_t csbase = MODE == MODE_AGG ? wave_sum(cr.base) : 0u;
        const uint64_t klo = (uint64_t)(t % p.NT) << p.tb;
        uint32_t produced = 0;
        uint32_t consumed = 0; // entries of the tile merged in earlier windows
        if (E == 0) {
            if (MODE == MODE_AGG && lane == 0) {
                p.tile_cnt[t] = 0;
                p.tile_sb[t] = csbase;
            }
            continue;
        }
        uint32_t take = 0;
        bool windowed = false;
        uint32_t L = begin_window(sm, cr, n, lane, E, take, windowed);
        load_window<MODE>(p, sm, L, n, lane, key, wk, vb);
        while (true) {
            if (windowed) {
                finish_window(sm, n, lane, key, wk);
                if (lane < n) cr.cur += take - sm.untaken[lane];
            } else {
                cr.cur += take;
            }
            uint32_t ck[MG_PER], cw[MG_PER], cv[MG_PER];
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                ck[i] = key[i];
                cw[i] = wk[i];
                cv[i] = vb[i];
            }
            // issue the tile's next window before merging this one
            E = wave_sum(cr.end - cr.cur);
            const bool tile_done = E == 0;
            if (!tile_done) {
                L = begin_window(sm, cr, n, lane, E, take, windowed);
                load_window<MODE>(p, sm, L, n, lane, key, wk, vb);
            }

            // merge the current window
            // a lane's words as one 16-byte access (consecutive lanes,
            // consecutive addresses: no bank conflicts)
            static_assert(MG_WPL == 4 && MG_WCAP / SG_WAVE == 4, "four words and four ranks per lane");
            *reinterpret_cast<uint4*>(&sm.bits[lane * MG_WPL]) = make_uint4(0u, 0u, 0u, 0u);
            wave_sync();
            uint32_t off[MG_PER];
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                off[i] = 0;
                if (cw[i] == 0xffffffffu) continue;
                const uint64_t o = (uint64_t)ck[i] - klo;
                if (ck[i] < klo || o >= span) { // outside the tile: cannot happen for valid input
                    report_error(kDevErrIndexRange);
                    cw[i] = 0xffffffffu; // consumed, not counted
                    continue;
                }
                off[i] = (uint32_t)o;
                atomicOr(&sm.bits[off[i] >> 5], 1u << (off[i] & 31u));
            }
            wave_sync();
            // prefix popcounts over the bitmap -> ranks
            uint32_t U;
            {
                const uint4 bw = *reinterpret_cast<const uint4*>(&sm.bits[lane * MG_WPL]);
                const uint32_t c[4] = {(uint32_t)__popc(bw.x), (uint32_t)__popc(bw.y), (uint32_t)__popc(bw.z),
                                       (uint32_t)__popc(bw.w)};
                const uint32_t sum = c[0] + c[1] + c[2] + c[3];
                const uint32_t inc = wave_incl_scan(sum);
                U = (uint32_t)__builtin_amdgcn_readlane((int)inc, SG_WAVE - 1);
                const uint32_t e0 = inc - sum, e1 = e0 + c[0], e2 = e1 + c[1], e3 = e2 + c[2];
                *reinterpret_cast<uint2*>(&sm.wpre[lane * MG_WPL]) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
            }
            wave_sync();
            uint32_t rk[MG_PER];
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                rk[i] = 0;
                if (cw[i] != 0xffffffffu)
                    rk[i] = sm.wpre[off[i] >> 5] + __popc(sm.bits[off[i] >> 5] & ((1u << (off[i] & 31u)) - 1u));
            }
            for (uint32_t r = lane; r < U; r += SG_WAVE) sm.mask[r] = 0ull;
            wave_sync();
            // keys by rank (every holder writes the same key), holders by rank
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                if (cw[i] == 0xffffffffu) continue;
                sm.bits[rk[i]] = ck[i];
                atomicOr(&sm.mask[rk[i]], 1ull << cw[i]);
            }
            wave_sync();
            if (MODE == MODE_AGG) {
                uint32_t slots; // entries of this window
                // first slot of each rank: exclusive prefix of the holder counts
                {
                    constexpr int RPL = MG_WCAP / SG_WAVE;
                    // the lane's four masks in two 16-byte reads (masks of ranks >= U are stale)
                    const ulonglong2 m01 = *reinterpret_cast<const ulonglong2*>(&sm.mask[lane * RPL]);
                    const ulonglong2 m23 = *reinterpret_cast<const ulonglong2*>(&sm.mask[lane * RPL + 2]);
                    const uint64_t mv[4] = {m01.x, m01.y, m23.x, m23.y};
                    uint32_t c[RPL], sum = 0;
#pragma unroll
                    for (int j = 0; j < RPL; ++j) {
                        c[j] = lane * RPL + j < U ? popc64(mv[j]) : 0u;
                        sum += c[j];
                    }
                    const uint32_t inc = wave_incl_scan(sum);
                    slots = (uint32_t)__builtin_amdgcn_readlane((int)inc, SG_WAVE - 1);
                    const uint32_t e0 = inc - sum, e1 = e0 + c[0], e2 = e1 + c[1], e3 = e2 + c[2];
                    *reinterpret_cast<uint2*>(&sm.wpre[lane * RPL]) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
                }
                wave_sync();
#pragma unroll
                for (int i = 0; i < MG_PER; ++i) {
                    if (cw[i] == 0xffffffffu) continue;
                    const uint32_t s = sm.wpre[rk[i]] + popc64(sm.mask[rk[i]] & ((1ull << cw[i]) - 1ull));
                    sm.slot[s] = cv[i];
                }
                wave_sync();
                const uint64_t ob = (uint64_t)csbase + produced;
                if (p.D == 1) {
                    for (uint32_t r = lane; r < U; r += SG_WAVE) {
                        const uint32_t s0 = sm.wpre[r], c = popc64(sm.mask[r]);
                        float acc = 0.0f;
                        for (uint32_t j = 0; j < c; ++j) acc += __uint_as_float(sm.slot[s0 + j]);
                        if (ob + r >= p.total) break; // only for inconsistent offsets
                        p.stage_idx[ob + r] = sm.bits[r];
                        p.stage_val[ob + r] = acc;
                    }
                } else if (p.D > 1) {
                    // rows: each staged key's contributors in worker order; the
                    // sums are formed by mg_rows_kernel
                    for (uint32_t q = lane; q < slots; q += SG_WAVE) p.stage_src[csbase + consumed + q] = sm.slot[q];
                    for (uint32_t r = lane; r < U && ob + r < p.total; r += SG_WAVE) {
                        p.stage_idx[ob + r] = sm.bits[r];
                        p.stage_first[ob + r] = consumed + sm.wpre[r];
                    }
                    consumed += slots;
                    if (tile_done && lane == 0) p.tile_ent[t] = consumed;
                } else {
                    for (uint32_t r = lane; r < U && ob + r < p.total; r += SG_WAVE) p.stage_idx[ob + r] = sm.bits[r];
                }
                if (tile_done && lane == 0) {
                    p.tile_cnt[t] = produced + U;
                    p.tile_sb[t] = csbase;
                }
            } else {
                // statistics: union part counts and pairwise intersections
                for (uint32_t q0 = 0; q0 < U; q0 += SG_WAVE) {
                    const uint32_t q = q0 + lane;
                    const bool has = q < U;
                    unsigned long long m = 0;
                    uint32_t k = 0;
                    if (has) {
                        k = sm.bits[q];
                        m = sm.mask[q];
                    }
                    count_sorted_parts(bs.part, has ? contig_part(k, p.M, p.Ps, p.inv_m) : 0u, has);
                    if (p.hashed) count_parts(bs.part + p.Ps, has ? h0(k, hseed, p.div) : 0u, has, p.Ps);
                    for (uint32_t a = 0; a < n; ++a) {
                        const uint64_t v = ballot((m >> a) & 1ull);
                        if (lane == 0) sm.vm[a] = v;
                    }
                    wave_sync();
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (lane + 64u * j >= p.npairs) break;
                        const uint32_t c = popc64(sm.vm[pair_a[j]] & sm.vm[pair_b[j]]);
                        if (c) atomicAdd(&bs.pairs[lane + 64u * j], c);
                    }
                    for (uint32_t pi = lane + 256; pi < p.npairs; pi += SG_WAVE) { // n > 22
                        uint32_t a, bb;
                        pair_of(pi, n, a, bb);
                        const uint32_t c = popc64(sm.vm[a] & sm.vm[bb]);
                        if (c) atomicAdd(&bs.pairs[pi], c);
                    }
                    wave_sync();
                }
                union_cnt += U;
            }
            produced += U;
            wave_sync();
            if (tile_done) break;
        }
    }
    if (MODE == MODE_STATS) {
        __syncthreads();
        uint64_t* row = p.st_part + (uint64_t)blockIdx.x * p.st_row;
        for (uint32_t i = threadIdx.x; i < p.npairs; i += MG_THREADS) row[i] = bs.pairs[i];
        for (uint32_t i = threadIdx.x; i < 2 * p.Ps; i += MG_THREADS) row[p.npairs + 1 + i] = bs.part[i];
        // union count: per-wave totals summed in LDS
        __syncthreads();
        if (lane == 0) bs.wv[wid].src[0] = union_cnt;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t u = 0;
            for (int i = 0; i < MG_WAVES; ++i) u += bs.wv[i].src[0];
            row[p.npairs] = u;
        }
    }
}

// statistics: sum the blocks' partial rows, one block per word
__global__ __launch_bounds__(256) void mg_stats_reduce_kernel(MergeParams p, uint32_t rows, uint64_t* out)
{
    __shared__ uint64_t red[256 / SG_WAVE];
    const uint32_t i = blockIdx.x;
    uint64_t s = 0;
    for (uint32_t r = threadIdx.x; r < rows; r += 256) s += p.st_part[(uint64_t)r * p.st_row + i];
#pragma unroll
    for (int d = SG_WAVE / 2; d > 0; d >>= 1) s += __shfl_xor(s, d, SG_WAVE);
    if (lane_id() == 0) red[threadIdx.x / SG_WAVE] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int w = 0; w < 256 / SG_WAVE; ++w) t += red[w];
        out[i] = t;
    }
}

// aggregate placement: exclusive prefix of tile counts inside each scan block
__global__ __launch_bounds__(1024) void mg_scan_local_kernel(MergeParams p)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    const uint32_t T = p.G * p.NT;
    const uint64_t t0 = (uint64_t)blockIdx.x * MG_SCAN_BLOCK + (uint64_t)threadIdx.x * MG_SCAN_PER;
    uint32_t c[MG_SCAN_PER];
    uint64_t sum = 0;
#pragma unroll
    for (int j = 0; j < MG_SCAN_PER; ++j) {
        c[j] = t0 + j < T ? p.tile_cnt[t0 + j] : 0u;
        sum += c[j];
    }
    uint64_t tot;
    uint64_t ex = block_excl_scan64<1024>(sum, scan_lds, &tot);
#pragma unroll
    for (int j = 0; j < MG_SCAN_PER; ++j) {
        if (t0 + j < T) p.tile_out[t0 + j] = ex;
        ex += c[j];
    }
    if (threadIdx.x == 0) p.blk_sum[blockIdx.x] = tot;
}

// exclusive prefix of the scan blocks' totals (in place); agg_off[G]
__global__ __launch_bounds__(1024) void mg_scan_top_kernel(MergeParams p)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    uint64_t carry = 0;
    for (uint32_t base = 0; base < p.nscan; base += 1024) {
        const uint32_t i = base + threadIdx.x;
        const uint64_t v = i < p.nscan ? p.blk_sum[i] : 0ull;
        uint64_t tot;
        const uint64_t ex = block_excl_scan64<1024>(v, scan_lds, &tot);
        if (i < p.nscan) p.blk_sum[i] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) p.agg_off[p.G] = carry;
}

// A wave places MG_PLACE_TILES consecutive tiles: their counts and offsets
// in one load (lane j holds tile t0 + j), then their staged keys (and
// values) in chunks of 64 entries numbered across the tiles, MG_PLACE_CHUNKS
// chunks per round with all loads of a round in flight before it is waited
// for once and written out.
constexpr int MG_PLACE_TILES = 16;
constexpr int MG_PLACE_CHUNKS = 16;

__global__ __launch_bounds__(256) void mg_place_kernel(MergeParams p)
{
    const uint32_t T = p.G * p.NT;
    const uint32_t lane = lane_id();
    const uint32_t stride = gridDim.x * 4 * MG_PLACE_TILES;
    for (uint32_t t0 = (blockIdx.x * 4 + uniform(threadIdx.x / SG_WAVE)) * MG_PLACE_TILES; t0 < T; t0 += stride) {
        const uint32_t t = t0 + lane;
        uint32_t c = 0;
        uint64_t sb = 0, ob = 0;
        if (lane < (uint32_t)MG_PLACE_TILES && t < T) {
            c = p.tile_cnt[t];
            sb = p.tile_sb[t];
            ob = p.tile_out[t] + p.blk_sum[t / MG_SCAN_BLOCK];
            if (t % p.NT == 0) p.agg_off[t / p.NT] = ob;
            if (ob + c > p.capacity || sb + c > p.total) { // cannot happen: a tile has no more keys than entries
                report_error(kDevErrPartition);
                c = 0;
            }
        }
        if (p.D <= 1) {
            const uint32_t nch = (c + SG_WAVE - 1) / SG_WAVE;
            const uint32_t cinc = wave_incl_scan(nch);
            const uint32_t cst = cinc - nch;
            const uint32_t C = lane_value(cinc, SG_WAVE - 1);
            for (uint32_t b0 = 0; b0 < C; b0 += MG_PLACE_CHUNKS) {
                uint32_t vi[MG_PLACE_CHUNKS], vv[MG_PLACE_CHUNKS], ci[MG_PLACE_CHUNKS], tj[MG_PLACE_CHUNKS];
#pragma unroll
                for (int u = 0; u < MG_PLACE_CHUNKS; ++u) {
                    const uint32_t q = b0 + u;
                    // the last tile whose chunks start at or before chunk q
                    // (for q >= C: the last tile with entries)
                    const uint64_t has = ballot(nch > 0 && cst <= q);
                    tj[u] = has ? 63u - (uint32_t)__builtin_clzll(has) : 0u;
                    const uint32_t cj = lane_value(c, tj[u]);
                    const uint32_t i = (q - lane_value(cst, tj[u])) * SG_WAVE + lane;
                    ci[u] = q < C && i < cj ? i : 0xffffffffu;
                    const uint64_t src = lane_value64(sb, tj[u]) + (ci[u] != 0xffffffffu ? i : 0u);
                    vi[u] = p.stage_idx[src];
                    vv[u] = p.D == 1 ? __float_as_uint(p.stage_val[src]) : 0u;
                }
                wait_vmem();
#pragma unroll
                for (int u = 0; u < MG_PLACE_CHUNKS; ++u) {
                    if (ci[u] == 0xffffffffu) continue;
                    const uint64_t o = lane_value64(ob, tj[u]) + ci[u];
                    p.agg_idx[o] = vi[u];
                    if (p.D == 1) p.agg_val[o] = __uint_as_float(vv[u]);
                }
            }
        } else {
            // rows: the key, and where the row's contributors are listed
            for (uint32_t j = 0; j < (uint32_t)MG_PLACE_TILES && t0 + j < T; ++j) {
                const uint32_t cj = lane_value(c, j);
                const uint64_t sbj = lane_value64(sb, j), obj = lane_value64(ob, j);
                const uint32_t ent = cj ? uniform(p.tile_ent[t0 + j]) : 0u;
                for (uint32_t i = lane; i < cj; i += SG_WAVE) {
                    p.agg_idx[obj + i] = p.stage_idx[sbj + i];
                    const uint32_t f0 = p.stage_first[sbj + i], f1 = i + 1 < cj ? p.stage_first[sbj + i + 1] : ent;
                    p.row_rng[obj + i] = make_uint2((uint32_t)(sbj + f0), (uint32_t)(sbj + (f1 > f0 ? f1 : f0)));
                }
            }
        }
    }
}

// Rows (D >= 2): one wave per output row.  The row's contributors (at most
// one per worker) are listed in stage_src in worker order; their rows are
// read 16 at a time and summed in that order, lanes across the columns.
constexpr int MG_ROW_BATCH = 16;

__global__ __launch_bounds__(256) void mg_rows_kernel(MergeParams p)
{
    const uint64_t U = p.agg_off[p.G] < p.capacity ? p.agg_off[p.G] : p.capacity;
    const uint32_t lane = lane_id();
    for (uint64_t o = (uint64_t)blockIdx.x * 4 + uniform(threadIdx.x / SG_WAVE); o < U; o += (uint64_t)gridDim.x * 4) {
        const uint2 rng = p.row_rng[o];
        const uint32_t x = uniform(rng.x), y = uniform(rng.y);
        const uint32_t cnt = y > x ? y - x : 0u;
        if (cnt > 64u || y > p.total) { // cannot happen: one contributor per worker
            if (lane == 0) report_error(kDevErrPartition);
            continue;
        }
        const uint32_t my = lane < cnt ? p.stage_src[x + lane] : 0u;
        for (uint32_t c0 = 0; c0 < p.D; c0 += SG_WAVE) {
            const uint32_t col = c0 + lane;
            const uint32_t cc = col < p.D ? col : p.D - 1;
            float acc = 0.0f;
            for (uint32_t j0 = 0; j0 < cnt; j0 += MG_ROW_BATCH) {
                float v[MG_ROW_BATCH];
#pragma unroll
                for (int j = 0; j < MG_ROW_BATCH; ++j) {
                    v[j] = 0.0f;
                    if (j0 + j < cnt) { // uniform
                        const uint64_t vi = (uint64_t)__builtin_amdgcn_readlane((int)my, (int)(j0 + j)) * p.D + cc;
                        v[j] = p.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.val)[vi])
                                      : static_cast<const float*>(p.val)[vi];
                    }
                }
#pragma unroll
                for (int j = 0; j < MG_ROW_BATCH; ++j)
                    if (j0 + j < cnt) acc += v[j];
            }
            if (col < p.D) p.agg_val[o * p.D + col] = acc;
        }
    }
}

} // namespace sg

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
//   bnd    one streaming pass over the run entries records, per run, where
//          each key bucket of width 2^bs begins (plain stores, no atomics);
//   tiles  per group, consecutive buckets are grouped into tiles of about
//          2048 entries (at most 4096, and at most 2^20 keys wide; a denser
//          bucket is split into key sub-ranges), from the bucket totals;
//   union  persistent blocks take tiles in order through an atomic ticket
//          and hold a tile's entries in registers (8 per thread).  A
//          two-level presence bitmap over the tile's key span (one bit per
//          32-key group, then one word per non-empty group) gives every key
//          its rank among the tile's distinct keys by prefix popcounts, with
//          no sorting and no merge chains.  Values are summed into the rank
//          slots one worker after another, so every sum is taken in worker
//          order (deterministic, the order of a ring).  Output offsets come
//          from a decoupled look-back over the tiles' unique counts (bounded
//          spin).  A tile with more than 4096 entries (a key sub-range denser
//          than its neighbours) is consumed in windows of 4096/n entries per
//          run, each window ending at the smallest last-loaded key of a cut
//          run, which guarantees progress.
#include "sg_host.h"

namespace sg {

constexpr int MG_THREADS = 512;
constexpr int MG_CAP = 4096;        // entries of a tile (window) held at once, in registers
constexpr int MG_TARGET = 2048;     // target entries per tile
constexpr int MG_PER = MG_CAP / MG_THREADS;
constexpr int MG_SPAN_LOG = 20;     // a tile spans at most 2^20 keys
constexpr int MG_CWORDS = (1 << MG_SPAN_LOG) >> 10; // coarse bitmap words: one bit per 32 keys
constexpr int MG_CHUNK = 4096;      // run entries per bnd block
constexpr uint64_t MG_FLAG_AGG = 1ull << 62;
constexpr uint64_t MG_FLAG_INC = 2ull << 62;
constexpr uint64_t MG_VAL_MASK = (1ull << 62) - 1;

enum MergeMode { MODE_AGG = 0, MODE_STATS = 1 };

struct MergeParams {
    // runs: run (g, w) = [off[w*stride + g], off[w*stride + g + 1])
    const uint32_t* idx;
    const uint64_t* off;
    uint32_t stride;
    uint32_t G, n;
    uint64_t total;
    uint64_t M;
    uint32_t bs;            // bucket width 2^bs
    uint32_t NB;            // buckets
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
    uint32_t* bnd;          // [(g*n + w) * (NB+1) + b]
    uint64_t* tile_key;     // [G * tcap] first key of tile j of group g (j <= ntiles[g]: sentinel)
    uint32_t* ntiles;       // [G]
    uint32_t* tile_prefix;  // [G+1]
    uint32_t* tile_pos;     // [rows * n] start (relative to the run) of run w in tile row r
    uint32_t* tile_group;   // [max_tiles] group of global tile t (tile row = t + group)
    uint64_t* tile_lo;      // [max_tiles] first key of tile t
    uint64_t* tile_hi;      // [max_tiles] end key of tile t
    uint64_t* status;       // [max_tiles] look-back words
    uint32_t* ticket;       // [1]
    uint32_t tcap;          // tile slots per group
    uint32_t max_tiles;     // bound on the total number of tiles
    uint32_t max_rows;      // max_tiles + G (one sentinel row per group)
    // statistics
    uint64_t* st_inter;     // [n*n]
    uint64_t* st_union;     // [1]
    uint64_t* st_ucontig;   // [Ps]
    uint64_t* st_uhashed;   // [Ps]
    uint32_t Ps;            // parts for skew
    uint32_t seed;
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
__global__ __launch_bounds__(MG_THREADS) void mg_plan_kernel(MergeParams p)
{
    __shared__ uint32_t scan_lds[MG_THREADS / SG_WAVE + 1];
    const uint32_t R = p.n * p.G;
    uint32_t carry = 0;
    for (uint32_t base = 0; base < R; base += MG_THREADS) {
        const uint32_t r = base + threadIdx.x;
        uint32_t c = 0;
        if (r < R) {
            uint64_t s, e;
            run_range(p, r % p.G, r / p.G, s, e);
            c = (uint32_t)ceil_div_dev(e - s, MG_CHUNK);
        }
        uint32_t tot;
        uint32_t ex = block_excl_scan<MG_THREADS>(c, scan_lds, &tot);
        if (r < R) p.chunk_start[r] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) p.chunk_start[R] = carry;
}

__device__ __forceinline__ uint32_t bucket_of(const MergeParams& p, uint32_t key)
{
    uint64_t b = p.bs >= 32 ? 0ull : ((uint64_t)key >> p.bs);
    if (b >= p.NB) {
        report_error(kDevErrIndexRange);
        b = p.NB - 1;
    }
    return (uint32_t)b;
}

// bnd[run][b] = first position (relative to the run) whose key is >= b * 2^bs
__global__ __launch_bounds__(MG_THREADS) void mg_bnd_kernel(MergeParams p)
{
    const uint32_t R = p.n * p.G;
    const uint32_t c = blockIdx.x;
    if (c >= p.chunk_start[R]) return;
    uint32_t lo = 0, hi = R;
    while (lo + 1 < hi) {
        uint32_t mid = (lo + hi) >> 1;
        if (p.chunk_start[mid] <= c) lo = mid;
        else hi = mid;
    }
    const uint32_t rp = lo, g = rp % p.G, w = rp / p.G;
    uint64_t s, e;
    run_range(p, g, w, s, e);
    const uint64_t len = e - s;
    const uint64_t j0 = (uint64_t)(c - p.chunk_start[rp]) * MG_CHUNK;
    uint32_t* row = p.bnd + ((uint64_t)g * p.n + w) * (p.NB + 1);
    for (uint64_t j = j0 + threadIdx.x; j < j0 + MG_CHUNK && j < len; j += MG_THREADS) {
        const uint32_t b = bucket_of(p, p.idx[s + j]);
        int64_t pb = -1;
        if (j > 0) {
            const uint32_t kp = p.idx[s + j - 1];
            pb = bucket_of(p, kp);
        }
        for (int64_t x = pb + 1; x <= (int64_t)b; ++x) row[x] = (uint32_t)j;
        if (j == len - 1)
            for (uint64_t x = (uint64_t)b + 1; x <= p.NB; ++x) row[x] = (uint32_t)len;
    }
}

// rows of empty runs are all zero
__global__ void mg_bnd_empty_kernel(MergeParams p)
{
    const uint64_t cnt = (uint64_t)p.n * p.G * (p.NB + 1);
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < cnt; i += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t row = i / (p.NB + 1);
        const uint32_t g = (uint32_t)(row / p.n), w = (uint32_t)(row % p.n);
        uint64_t s, e;
        run_range(p, g, w, s, e);
        if (s == e) p.bnd[i] = 0;
    }
}

__device__ __forceinline__ uint32_t bnd_at(const MergeParams& p, uint32_t g, uint32_t w, uint32_t b, uint64_t len)
{
    uint32_t v = p.bnd[((uint64_t)g * p.n + w) * (p.NB + 1) + b];
    return (uint64_t)v > len ? (uint32_t)len : v;
}

// One block per group: bucket totals, their prefix, and tiles.  Consecutive
// buckets are grouped into tiles of about MG_TARGET entries; a bucket holding
// more than MG_TARGET entries is split into 2^s equal key sub-ranges (dense
// regions are dense inside the bucket too), so tiles stay near the target.
__device__ __forceinline__ uint32_t split_log2(uint32_t tot, uint32_t bs)
{
    uint32_t need = (tot + MG_TARGET - 1) / MG_TARGET, s = 0;
    while ((1u << s) < need && s < bs && s < 16) ++s;
    return s;
}

__global__ __launch_bounds__(1024) void mg_tiles_kernel(MergeParams p)
{
    __shared__ uint32_t scan_lds[1024 / SG_WAVE + 1];
    __shared__ uint32_t prev_pre[1024], prev_tot[1024];
    __shared__ uint32_t carry_lds[4];
    const uint32_t g = blockIdx.x;
    uint64_t* keys = p.tile_key + (uint64_t)g * p.tcap;
    uint32_t carry_pre = 0, carry_tiles = 0;
    uint32_t last_pre = 0, last_tot = 0;
    for (uint32_t base = 0; base < p.NB; base += 1024) {
        const uint32_t b = base + threadIdx.x;
        uint32_t tot = 0;
        if (b < p.NB) {
            for (uint32_t w = 0; w < p.n; ++w) {
                uint64_t s, e;
                run_range(p, g, w, s, e);
                const uint64_t len = e - s;
                uint32_t x = bnd_at(p, g, w, b, len), y = bnd_at(p, g, w, b + 1, len);
                tot += y > x ? y - x : 0u;
            }
        }
        uint32_t all;
        uint32_t pre = carry_pre + block_excl_scan<1024>(tot, scan_lds, &all);
        prev_pre[threadIdx.x] = pre;
        prev_tot[threadIdx.x] = tot;
        __syncthreads();
        uint32_t ppre = threadIdx.x ? prev_pre[threadIdx.x - 1] : last_pre;
        uint32_t ptot = threadIdx.x ? prev_tot[threadIdx.x - 1] : last_tot;
        uint32_t cnt = 0, sl = 0;
        if (b < p.NB) {
            const uint32_t span_buckets = p.bs >= MG_SPAN_LOG ? 1u : (1u << (MG_SPAN_LOG - p.bs));
            const bool flag = (b == 0) || (pre / MG_TARGET != ppre / MG_TARGET) || tot > MG_TARGET ||
                              ptot > MG_TARGET || (b % span_buckets) == 0;
            if (flag) {
                sl = tot > MG_TARGET ? split_log2(tot, p.bs) : 0u;
                cnt = 1u << sl;
            }
        }
        uint32_t nf;
        __syncthreads();
        uint32_t pos = carry_tiles + block_excl_scan<1024>(cnt, scan_lds, &nf);
        const uint64_t bw = 1ull << p.bs;
        for (uint32_t i = 0; i < cnt; ++i)
            if (pos + i < p.tcap) keys[pos + i] = ((uint64_t)b << p.bs) + (uint64_t)i * (bw >> sl);
        if (threadIdx.x == 1023) {
            carry_lds[0] = pre;
            carry_lds[1] = tot;
        }
        __syncthreads();
        last_pre = carry_lds[0];
        last_tot = carry_lds[1];
        carry_pre += all;
        carry_tiles += nf;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        uint32_t nt = carry_tiles < p.tcap ? carry_tiles : p.tcap - 1;
        if (nt != carry_tiles) report_error(kDevErrPartition);
        p.ntiles[g] = nt;
        keys[nt] = (uint64_t)p.NB << p.bs;
    }
}

__global__ __launch_bounds__(MG_THREADS) void mg_tile_prefix_kernel(MergeParams p)
{
    __shared__ uint32_t scan_lds[MG_THREADS / SG_WAVE + 1];
    uint32_t carry = 0;
    for (uint32_t base = 0; base < p.G; base += MG_THREADS) {
        const uint32_t g = base + threadIdx.x;
        uint32_t c = g < p.G ? p.ntiles[g] : 0u, tot;
        uint32_t ex = block_excl_scan<MG_THREADS>(c, scan_lds, &tot);
        if (g < p.G) p.tile_prefix[g] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        p.tile_prefix[p.G] = carry;
        p.ticket[0] = 0;
    }
}

// lower bound of `target` in the ascending keys a[lo, hi), by one wave:
// 64 probes per round cut the range 65-fold, then one load finishes.
__device__ uint64_t wave_lower_bound(const uint32_t* a, uint64_t lo, uint64_t hi, uint64_t target)
{
    const uint32_t lane = lane_id();
    while (hi - lo > SG_WAVE) {
        const uint64_t len = hi - lo;
        const uint64_t pos = lo + ((uint64_t)(lane + 1) * len) / 65;
        const uint32_t c = popc64(ballot((uint64_t)a[pos] < target));
        const uint64_t nlo = c == 0 ? lo : lo + ((uint64_t)c * len) / 65 + 1;
        const uint64_t nhi = c == SG_WAVE ? hi : lo + ((uint64_t)(c + 1) * len) / 65;
        lo = nlo;
        hi = nhi;
    }
    const uint64_t pos = lo + lane;
    const bool less = pos < hi && (uint64_t)a[pos] < target;
    return lo + popc64(ballot(less));
}

// Row r of tile_pos: for every run, where the tile starting at tile_key
// begins (bucket boundaries come from bnd; split points are searched inside
// their bucket).  Rows are global: row = tile_prefix[g] + g + j.
__global__ __launch_bounds__(MG_THREADS) void mg_refine_kernel(MergeParams p)
{
    const uint32_t rows = p.tile_prefix[p.G] + p.G;
    const uint32_t wid = threadIdx.x / SG_WAVE;
    for (uint32_t r = blockIdx.x; r < rows; r += gridDim.x) {
        // group of row r: largest g with tile_prefix[g] + g <= r
        uint32_t lo = 0, hi = p.G;
        while (lo + 1 < hi) {
            uint32_t mid = (lo + hi) >> 1;
            if (p.tile_prefix[mid] + mid <= r) lo = mid;
            else hi = mid;
        }
        const uint32_t g = lo, j = r - (p.tile_prefix[g] + g);
        const uint64_t key = p.tile_key[(uint64_t)g * p.tcap + j];
        if (threadIdx.x == 0 && j < p.ntiles[g]) {
            const uint32_t t = r - g;
            p.tile_group[t] = g;
            p.tile_lo[t] = key;
            p.tile_hi[t] = p.tile_key[(uint64_t)g * p.tcap + j + 1];
        }
        const uint32_t b = (uint32_t)(key >> p.bs);
        const bool aligned = (key & ((1ull << p.bs) - 1ull)) == 0;
        for (uint32_t w = wid; w < p.n; w += MG_THREADS / SG_WAVE) {
            uint64_t s, e;
            run_range(p, g, w, s, e);
            const uint64_t len = e - s;
            uint32_t v;
            if (aligned || b >= p.NB) {
                v = bnd_at(p, g, w, b < p.NB ? b : p.NB, len);
            } else {
                const uint32_t x = bnd_at(p, g, w, b, len), y = bnd_at(p, g, w, b + 1, len);
                v = (uint32_t)(wave_lower_bound(p.idx + s, x, y > x ? y : x, key));
            }
            if (lane_id() == 0) p.tile_pos[(uint64_t)r * p.n + w] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// the merge kernel
// ---------------------------------------------------------------------------
// decoupled look-back by wave 0: exclusive prefix of tile `t`
__device__ uint64_t look_back(const MergeParams& p, uint32_t t)
{
    uint64_t sum = 0;
    int64_t j = (int64_t)t - 1;
    while (j >= 0) {
        const int64_t x = j - (int64_t)lane_id();
        uint64_t s = MG_FLAG_INC; // before tile 0: inclusive 0
        if (x >= 0) {
            uint32_t spins = 0;
            s = load_agent(p.status + x);
            while ((s >> 62) == 0) {
                __builtin_amdgcn_s_sleep(2);
                s = load_agent(p.status + x);
                if (++spins > (1u << 22)) {
                    report_error(kDevErrSpin);
                    s = MG_FLAG_INC;
                    break;
                }
            }
        }
        const uint64_t inc = ballot((s >> 62) == 2);
        const uint32_t first = inc ? (uint32_t)__builtin_ctzll(inc) : 64u;
        uint64_t v = (lane_id() <= first) ? (s & MG_VAL_MASK) : 0ull;
        for (int d = SG_WAVE / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, SG_WAVE);
        sum += v;
        if (inc) break;
        j -= SG_WAVE;
    }
    return sum;
}

// Contiguous part of `key` among P parts [floor(iM/P), floor((i+1)M/P)):
// the largest i with i*M < (key+1)*P, i.e. floor(((key+1)P - 1) / M).
__device__ __forceinline__ uint32_t contig_part(uint64_t key, uint64_t M, uint32_t P)
{
    const uint64_t part = ((key + 1) * P - 1) / (M ? M : 1);
    return part < P ? (uint32_t)part : P - 1;
}

template <int MODE>
struct UnionSmem {
    uint32_t coarse[MG_CWORDS];  // bit per 32-key group of the tile span
    uint16_t cpre[MG_CWORDS];    // non-empty groups before a coarse word
    uint32_t fine[MG_CAP];       // bits of the non-empty groups; then the distinct keys by rank
    uint16_t fpre[MG_CAP];       // distinct keys before a fine word
    union {
        float acc[MG_CAP];       // sums by rank (scalar values)
        uint32_t ekey[MG_CAP];   // entry keys by load position (rows)
        unsigned long long mask[MODE == MODE_STATS ? MG_CAP : 1]; // statistics: workers holding a key
    };
    uint32_t wofs[65];           // load offset of worker w's window
    uint32_t take[64], taken[64];
    uint32_t cur[64], end[64];
    uint64_t src0[64];
    uint32_t scan[MG_THREADS / SG_WAVE + 1];
    uint32_t bcast[4];
    uint64_t bcast64[2];
    unsigned long long vmask[MODE == MODE_STATS ? MG_THREADS / SG_WAVE : 1][64];
    uint32_t ucontig[MODE == MODE_STATS ? 256 : 1], uhashed[MODE == MODE_STATS ? 256 : 1];
};

template <int MODE>
__global__ __launch_bounds__(MG_THREADS) void mg_merge_kernel(MergeParams p)
{
    __shared__ UnionSmem<MODE> sm;
    const uint32_t n = p.n;
    const uint32_t tid = threadIdx.x, wid = tid / SG_WAVE;
    const uint32_t total_tiles = p.tile_prefix[p.G];
    // statistics: each lane owns up to 4 worker pairs (a <= b), pair index
    // pi = lane + 64*i; further pairs (n > 22) go straight to global atomics
    uint32_t pair_acc[4] = {0, 0, 0, 0};
    const uint32_t npairs = n * (n + 1) / 2;
    uint64_t union_cnt = 0;
    if (MODE == MODE_STATS)
        for (uint32_t i = tid; i < 256; i += MG_THREADS) sm.ucontig[i] = sm.uhashed[i] = 0;

    while (true) {
        if (tid == 0) sm.bcast[0] = atomicAdd(p.ticket, 1u);
        __syncthreads();
        const uint32_t t = sm.bcast[0];
        if (t >= total_tiles) break;
        const uint32_t g = p.tile_group[t];
        const uint64_t klo = p.tile_lo[t], khi = p.tile_hi[t];
        const uint32_t row = t + g;
        const uint32_t jfirst = p.tile_prefix[g] == t; // first tile of its group
        if (tid < n) {
            uint64_t s, e;
            run_range(p, g, tid, s, e);
            const uint64_t len = e - s;
            uint32_t x = p.tile_pos[(uint64_t)row * n + tid], y = p.tile_pos[(uint64_t)(row + 1) * n + tid];
            if (x > len) x = (uint32_t)len;
            if (y > len) y = (uint32_t)len;
            if (y < x) y = x;
            sm.src0[tid] = s;
            sm.cur[tid] = x;
            sm.end[tid] = y;
        }
        __syncthreads();
        uint32_t E = 0;
        for (uint32_t w = 0; w < n; ++w) E += sm.end[w] - sm.cur[w];
        const bool single = E <= (uint32_t)MG_CAP;
        uint64_t span = khi > klo ? khi - klo : 0;
        if (span > (1ull << MG_SPAN_LOG)) { // the tiler never builds one; keep LDS indices in range
            report_error(kDevErrPartition);
            span = 1ull << MG_SPAN_LOG;
        }
        const uint32_t win = MG_CAP / n;

        uint64_t X = 0;
        if (MODE == MODE_AGG && !single) {
            if (tid < SG_WAVE) {
                uint64_t x = t == 0 ? 0ull : look_back(p, t);
                if (tid == 0) sm.bcast64[0] = x;
            }
            __syncthreads();
            X = sm.bcast64[0];
        }
        uint64_t produced = 0;

        while (true) {
            // window of each worker
            if (tid == 0) {
                uint32_t acc = 0;
                for (uint32_t w = 0; w < n; ++w) {
                    const uint32_t rem = sm.end[w] - sm.cur[w];
                    const uint32_t a = single ? rem : (rem < win ? rem : win);
                    sm.wofs[w] = acc;
                    sm.take[w] = a;
                    acc += a;
                }
                sm.wofs[n] = acc;
                sm.bcast[1] = 0xffffffffu; // cut key
            }
            if (tid < 64) sm.taken[tid] = 0;
            for (uint32_t i = tid; i < MG_CWORDS; i += MG_THREADS) sm.coarse[i] = 0;
            for (uint32_t i = tid; i < MG_CAP; i += MG_THREADS) {
                sm.fine[i] = 0;
                if (MODE == MODE_AGG) sm.acc[i] = 0.0f;
                else sm.mask[i] = 0ull;
            }
            __syncthreads();
            const uint32_t L = sm.wofs[n];
            if (L == 0 && !single) break; // a single tile runs once, even when empty
            // smallest last-loaded key of a run whose window does not reach its end
            if (!single && tid < n) {
                const uint32_t a = sm.take[tid];
                if (a > 0 && sm.cur[tid] + a < sm.end[tid])
                    atomicMin(&sm.bcast[1], p.idx[sm.src0[tid] + sm.cur[tid] + a - 1]);
            }
            // entries into registers
            uint32_t key[MG_PER], wk[MG_PER];
            float val[MG_PER];
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                const uint32_t lp = tid + i * MG_THREADS;
                key[i] = 0xffffffffu;
                wk[i] = 0xffffffffu;
                val[i] = 0.0f;
                if (lp < L) {
                    uint32_t lo = 0, hi = n;
                    while (lo + 1 < hi) {
                        const uint32_t mid = (lo + hi) >> 1;
                        if (sm.wofs[mid] <= lp) lo = mid;
                        else hi = mid;
                    }
                    const uint64_t pos = sm.src0[lo] + sm.cur[lo] + (lp - sm.wofs[lo]);
                    key[i] = p.idx[pos];
                    wk[i] = lo;
                    if (MODE == MODE_AGG && p.D == 1)
                        val[i] = p.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.val)[pos])
                                        : static_cast<const float*>(p.val)[pos];
                }
            }
            __syncthreads();
            const uint32_t kmax = sm.bcast[1];
            // take entries up to the cut; coarse presence
            uint32_t off[MG_PER];
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                const bool tk = wk[i] != 0xffffffffu && key[i] <= kmax;
                if (!tk) wk[i] = 0xffffffffu;
                off[i] = 0;
                if (tk) {
                    atomicAdd(&sm.taken[wk[i]], 1u);
                    const uint64_t o = (uint64_t)key[i] - klo;
                    if (o < span) {
                        off[i] = (uint32_t)o;
                        const uint32_t grp = (uint32_t)(o >> 5);
                        atomicOr(&sm.coarse[grp >> 5], 1u << (grp & 31u));
                    } else {
                        wk[i] = 0xffffffffu; // outside the tile: cannot happen for valid input
                        report_error(kDevErrIndexRange);
                    }
                }
            }
            __syncthreads();
            // prefix over coarse words -> index of each non-empty group
            {
                constexpr int CW = MG_CWORDS / MG_THREADS;
                uint32_t c[CW], sum = 0;
#pragma unroll
                for (int j = 0; j < CW; ++j) {
                    c[j] = __popc(sm.coarse[tid * CW + j]);
                    sum += c[j];
                }
                uint32_t F;
                uint32_t ex = block_excl_scan<MG_THREADS>(sum, sm.scan, &F);
#pragma unroll
                for (int j = 0; j < CW; ++j) {
                    sm.cpre[tid * CW + j] = (uint16_t)ex;
                    ex += c[j];
                }
            }
            __syncthreads();
            uint32_t ci[MG_PER];
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                ci[i] = 0;
                if (wk[i] != 0xffffffffu) {
                    const uint32_t grp = off[i] >> 5, cw = grp >> 5, cb = grp & 31u;
                    ci[i] = sm.cpre[cw] + __popc(sm.coarse[cw] & ((1u << cb) - 1u));
                    atomicOr(&sm.fine[ci[i]], 1u << (off[i] & 31u));
                }
            }
            __syncthreads();
            // prefix over fine words -> rank of each distinct key
            uint32_t U;
            {
                uint32_t c[MG_PER], sum = 0;
#pragma unroll
                for (int j = 0; j < MG_PER; ++j) {
                    c[j] = __popc(sm.fine[tid * MG_PER + j]);
                    sum += c[j];
                }
                uint32_t ex = block_excl_scan<MG_THREADS>(sum, sm.scan, &U);
#pragma unroll
                for (int j = 0; j < MG_PER; ++j) {
                    sm.fpre[tid * MG_PER + j] = (uint16_t)ex;
                    ex += c[j];
                }
            }
            // the unique count is known: let successors use it right away
            if (MODE == MODE_AGG && single && tid == 0)
                store_agent(p.status + t, (t == 0 ? MG_FLAG_INC : MG_FLAG_AGG) | U);
            __syncthreads();
            uint32_t rk[MG_PER];
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                rk[i] = 0;
                if (wk[i] != 0xffffffffu)
                    rk[i] = sm.fpre[ci[i]] + __popc(sm.fine[ci[i]] & ((1u << (off[i] & 31u)) - 1u));
            }
            __syncthreads();
            // distinct keys by rank (every holder of a key writes the same value)
#pragma unroll
            for (int i = 0; i < MG_PER; ++i) {
                if (wk[i] == 0xffffffffu) continue;
                sm.fine[rk[i]] = key[i];
                if (MODE == MODE_STATS) atomicOr(&sm.mask[rk[i]], 1ull << wk[i]);
                if (MODE == MODE_AGG && p.D > 1) sm.ekey[tid + i * MG_THREADS] = key[i];
            }
            __syncthreads();
            if (MODE == MODE_AGG && p.D == 1) {
                // sums in worker order: worker w's entries have distinct keys,
                // so one worker at a time needs no atomics
                for (uint32_t w = 0; w < n; ++w) {
                    if (sm.taken[w] == 0) continue;
#pragma unroll
                    for (int i = 0; i < MG_PER; ++i)
                        if (wk[i] == w) sm.acc[rk[i]] += val[i];
                    __syncthreads();
                }
            }

            if (MODE == MODE_AGG) {
                if (single) {
                    if (tid < SG_WAVE) {
                        uint64_t x = t == 0 ? 0ull : look_back(p, t);
                        if (tid == 0) {
                            if (t != 0) store_agent(p.status + t, MG_FLAG_INC | (x + U));
                            sm.bcast64[0] = x;
                        }
                    }
                    __syncthreads();
                    X = sm.bcast64[0];
                }
                const uint64_t ob = X + produced;
                if (p.D <= 1) {
                    for (uint32_t q = tid; q < U; q += MG_THREADS) {
                        const uint64_t dst = ob + q;
                        if (dst >= p.capacity) continue;
                        p.agg_idx[dst] = sm.fine[q];
                        if (p.D == 1) p.agg_val[dst] = sm.acc[q];
                    }
                } else {
                    // rows: one wave per distinct key, lanes across the row;
                    // each worker's entry is found by binary search in its window
                    for (uint32_t q = wid; q < U; q += MG_THREADS / SG_WAVE) {
                        const uint32_t k = sm.fine[q];
                        const uint64_t dst = ob + q;
                        if (dst >= p.capacity) continue;
                        if (lane_id() == 0) p.agg_idx[dst] = k;
                        for (uint32_t c0 = 0; c0 < p.D; c0 += SG_WAVE) {
                            const uint32_t c = c0 + lane_id();
                            float acc = 0.0f;
                            for (uint32_t w = 0; w < n; ++w) {
                                uint32_t lo = sm.wofs[w], hi = sm.wofs[w] + sm.taken[w];
                                while (lo < hi) {
                                    const uint32_t mid = (lo + hi) >> 1;
                                    if (sm.ekey[mid] < k) lo = mid + 1;
                                    else hi = mid;
                                }
                                if (lo < sm.wofs[w] + sm.taken[w] && sm.ekey[lo] == k && c < p.D) {
                                    const uint64_t pos = sm.src0[w] + sm.cur[w] + (lo - sm.wofs[w]);
                                    const uint64_t vi = pos * p.D + c;
                                    acc += p.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.val)[vi])
                                                  : static_cast<const float*>(p.val)[vi];
                                }
                            }
                            if (c < p.D) p.agg_val[dst * p.D + c] = acc;
                        }
                    }
                }
            } else {
                // statistics: pairwise intersections from per-key worker masks
                for (uint32_t q0 = wid * SG_WAVE; q0 < U; q0 += MG_THREADS) {
                    const uint32_t q = q0 + lane_id();
                    unsigned long long m = 0;
                    if (q < U) {
                        const uint32_t k = sm.fine[q];
                        m = sm.mask[q];
                        atomicAdd(&sm.ucontig[contig_part(k, p.M, p.Ps)], 1u);
                        if (p.hashed) atomicAdd(&sm.uhashed[h0(k, p.seed, p.div)], 1u);
                    }
                    for (uint32_t a = 0; a < n; ++a) {
                        const uint64_t v = ballot((m >> a) & 1ull);
                        if (lane_id() == 0) sm.vmask[wid][a] = v;
                    }
                    for (uint32_t i = 0, pi = lane_id(); pi < npairs; ++i, pi += SG_WAVE) {
                        uint32_t a = 0, rem = pi;
                        while (rem >= n - a) {
                            rem -= n - a;
                            ++a;
                        }
                        const uint32_t b = a + rem;
                        const uint32_t c = popc64(sm.vmask[wid][a] & sm.vmask[wid][b]);
                        if (i < 4) pair_acc[i] += c;
                        else if (c) atomicAdd((unsigned long long*)&p.st_inter[a * n + b], (unsigned long long)c);
                    }
                }
                union_cnt += U;
            }
            produced += U;
            __syncthreads();
            if (tid < n) sm.cur[tid] += sm.taken[tid];
            __syncthreads();
            if (single) break;
        }
        if (MODE == MODE_AGG && tid == 0) {
            if (!single) store_agent(p.status + t, MG_FLAG_INC | (X + produced));
            if (t == total_tiles - 1) p.agg_off[p.G] = X + produced;
            if (jfirst) p.agg_off[g] = X;
        }
        __syncthreads();
    }
    if (MODE == MODE_STATS) {
        __syncthreads();
        for (uint32_t i = 0, pi = lane_id(); i < 4 && pi < npairs; ++i, pi += SG_WAVE) {
            if (!pair_acc[i]) continue;
            uint32_t a = 0, rem = pi;
            while (rem >= n - a) {
                rem -= n - a;
                ++a;
            }
            const uint32_t b = a + rem;
            atomicAdd((unsigned long long*)&p.st_inter[a * n + b], (unsigned long long)pair_acc[i]);
        }
        for (uint32_t i = tid; i < p.Ps; i += MG_THREADS) {
            if (sm.ucontig[i]) atomicAdd((unsigned long long*)&p.st_ucontig[i], (unsigned long long)sm.ucontig[i]);
            if (p.hashed && sm.uhashed[i])
                atomicAdd((unsigned long long*)&p.st_uhashed[i], (unsigned long long)sm.uhashed[i]);
        }
        if (tid == 0 && union_cnt) atomicAdd((unsigned long long*)p.st_union, (unsigned long long)union_cnt);
    }
}

} // namespace sg

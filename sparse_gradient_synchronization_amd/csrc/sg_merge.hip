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
//          2048 entries (never more than 4096 unless one bucket alone is
//          larger), from the bucket totals;
//   merge  persistent blocks take tiles in order through an atomic ticket,
//          load the n sub-runs of a tile into LDS, merge them pairwise
//          (merge path, ties to the lower worker, so equal keys end up in
//          worker order), mark segment heads, and sum each segment's values
//          in worker order.  Output offsets come from a decoupled look-back
//          over the tiles' unique counts (bounded spin).  A tile larger than
//          LDS is consumed in windows of 4096/n entries per run; each window
//          ends at the smallest last-loaded key of a cut run, which
//          guarantees progress.
#include "sg_host.h"

namespace sg {

constexpr int MG_THREADS = 256;
constexpr int MG_CAP = 4096;       // entries per LDS tile
constexpr int MG_TARGET = 2048;    // target entries per tile
constexpr int MG_CHUNK = 4096;     // run entries per bnd block
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
            const bool flag = (b == 0) || (pre / MG_TARGET != ppre / MG_TARGET) || tot > MG_TARGET || ptot > MG_TARGET;
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
struct MergeSmem {
    uint32_t keys[2][MG_CAP];
    uint16_t lidx[2][MG_CAP]; // load position of the entry (into vals / source map)
    float vals[MG_CAP];
    uint16_t hpos[MG_CAP];    // sorted position of unique u
    uint32_t lofs[65];        // list offsets (merge tree)
    uint32_t wofs[65];        // load offsets per worker
    uint64_t src0[64];        // absolute position of the first loaded entry of worker w
    uint32_t cur[64], end[64], take[64];
    uint32_t scan[MG_THREADS / SG_WAVE + 1];
    uint32_t bcast[8];
    uint64_t bcast64[2];
    uint64_t vmask[MG_THREADS / SG_WAVE][64]; // statistics: per-wave worker bit vectors
};

__device__ __forceinline__ uint32_t merge_path(const uint32_t* A, uint32_t la, const uint32_t* B, uint32_t lb,
                                               uint32_t d)
{
    uint32_t lo = d > lb ? d - lb : 0u, hi = d < la ? d : la;
    while (lo < hi) {
        uint32_t mid = (lo + hi) >> 1;
        if (A[mid] <= B[d - 1 - mid]) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Merge the nl sorted lists held in keys[in] (offsets lofs[0..nl]) pairwise
// until one remains.  Returns the buffer index holding the result.
__device__ int merge_tree(MergeSmem& sm, uint32_t nl, uint32_t E)
{
    int in = 0;
    while (nl > 1) {
        const uint32_t per = (E + MG_THREADS - 1) / MG_THREADS;
        const uint32_t o0 = threadIdx.x * per;
        const uint32_t o1 = o0 + per < E ? o0 + per : E;
        const uint32_t* K = sm.keys[in];
        const uint16_t* L = sm.lidx[in];
        uint32_t* KO = sm.keys[in ^ 1];
        uint16_t* LO = sm.lidx[in ^ 1];
        uint32_t o = o0;
        uint32_t q = 0; // pair index containing o
        while (o < o1) {
            while (q + 1 < (nl + 1) / 2 && sm.lofs[2 * (q + 1)] <= o) ++q;
            const uint32_t ps = sm.lofs[2 * q];
            const uint32_t mid = sm.lofs[2 * q + 1 < nl ? 2 * q + 1 : nl];
            const uint32_t pe = sm.lofs[2 * q + 2 < nl ? 2 * q + 2 : nl];
            const uint32_t la = mid - ps, lb = pe - mid;
            const uint32_t stop = o1 < pe ? o1 : pe;
            uint32_t i = merge_path(K + ps, la, K + mid, lb, o - ps);
            uint32_t j = (o - ps) - i;
            for (; o < stop; ++o) {
                bool takeA = (j >= lb) || (i < la && K[ps + i] <= K[mid + j]);
                if (takeA) {
                    KO[o] = K[ps + i];
                    LO[o] = L[ps + i];
                    ++i;
                } else {
                    KO[o] = K[mid + j];
                    LO[o] = L[mid + j];
                    ++j;
                }
            }
        }
        __syncthreads();
        // rebuild offsets: new list k starts where old list 2k started
        const uint32_t nn = (nl + 1) / 2;
        uint32_t newoff = 0;
        if (threadIdx.x <= nn) newoff = (2 * threadIdx.x < nl) ? sm.lofs[2 * threadIdx.x] : E;
        __syncthreads();
        if (threadIdx.x <= nn) sm.lofs[threadIdx.x] = newoff;
        __syncthreads();
        nl = nn;
        in ^= 1;
    }
    return in;
}

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

__device__ __forceinline__ uint32_t contig_part(uint64_t key, uint64_t M, uint32_t P)
{
    uint64_t part = (uint64_t)(((unsigned __int128)key * P) / (M ? M : 1));
    if (part >= P) part = P - 1;
    // exact boundaries floor(i M / P)
    while (part + 1 < P && key >= (uint64_t)(((unsigned __int128)M * (part + 1)) / P)) ++part;
    while (part > 0 && key < (uint64_t)(((unsigned __int128)M * part) / P)) --part;
    return (uint32_t)part;
}

template <int MODE>
__global__ __launch_bounds__(MG_THREADS) void mg_merge_kernel(MergeParams p)
{
    __shared__ MergeSmem sm;
    __shared__ uint32_t inter_lds[MODE == MODE_STATS ? 64 * 64 : 1];
    __shared__ uint32_t ucontig[MODE == MODE_STATS ? 256 : 1], uhashed[MODE == MODE_STATS ? 256 : 1];
    __shared__ uint64_t union_lds;
    const uint32_t n = p.n;
    const uint32_t total_tiles = p.tile_prefix[p.G];

    if (MODE == MODE_STATS) {
        for (uint32_t i = threadIdx.x; i < 64 * 64; i += MG_THREADS) inter_lds[i] = 0;
        for (uint32_t i = threadIdx.x; i < 256; i += MG_THREADS) ucontig[i] = uhashed[i] = 0;
        if (threadIdx.x == 0) union_lds = 0;
    }

    while (true) {
        if (threadIdx.x == 0) sm.bcast[0] = atomicAdd(p.ticket, 1u);
        __syncthreads();
        const uint32_t t = sm.bcast[0];
        if (t >= total_tiles) break;
        // group and tile index
        uint32_t lo = 0, hi = p.G;
        while (lo + 1 < hi) {
            uint32_t mid = (lo + hi) >> 1;
            if (p.tile_prefix[mid] <= t) lo = mid;
            else hi = mid;
        }
        const uint32_t g = lo, jt = t - p.tile_prefix[g];
        const uint32_t row = p.tile_prefix[g] + g + jt;
        const uint64_t klo = p.tile_key[(uint64_t)g * p.tcap + jt];
        const uint64_t khi = p.tile_key[(uint64_t)g * p.tcap + jt + 1];
        if (threadIdx.x < n) {
            uint64_t s, e;
            run_range(p, g, threadIdx.x, s, e);
            const uint64_t len = e - s;
            uint32_t x = p.tile_pos[(uint64_t)row * n + threadIdx.x], y = p.tile_pos[(uint64_t)(row + 1) * n + threadIdx.x];
            if (x > len) x = (uint32_t)len;
            if (y > len) y = (uint32_t)len;
            if (y < x) y = x;
            sm.src0[threadIdx.x] = s;
            sm.cur[threadIdx.x] = x;
            sm.end[threadIdx.x] = y;
        }
        __syncthreads();
        uint32_t E = 0;
        for (uint32_t w = 0; w < n; ++w) E += sm.end[w] - sm.cur[w];
        const bool single = E <= (uint32_t)MG_CAP;
        const uint32_t win = MG_CAP / n;

        uint64_t X = 0;
        bool early = false; // unique count published before the windows run
        if (MODE == MODE_AGG && !single) {
            uint32_t U0 = 0;
            const uint64_t span = khi > klo ? khi - klo : 0;
            early = span <= (uint64_t)MG_CAP * 32;
            if (early) {
                // count the tile's distinct keys with a presence bitmap over
                // [klo, khi) so successors need not wait for the whole tile
                uint32_t* bm = sm.keys[1];
                const uint32_t nwords = (uint32_t)((span + 31) / 32);
                for (uint32_t i = threadIdx.x; i < nwords; i += MG_THREADS) bm[i] = 0u;
                __syncthreads();
                for (uint32_t w = 0; w < n; ++w) {
                    const uint64_t gs = sm.src0[w] + sm.cur[w];
                    const uint32_t cnt = sm.end[w] - sm.cur[w];
                    for (uint32_t i = threadIdx.x; i < cnt; i += MG_THREADS) {
                        const uint64_t off = (uint64_t)p.idx[gs + i] - klo;
                        if (off < span) atomicOr(&bm[off >> 5], 1u << (off & 31u));
                    }
                }
                __syncthreads();
                uint32_t c = 0;
                for (uint32_t i = threadIdx.x; i < nwords; i += MG_THREADS) c += __popc(bm[i]);
                block_excl_scan<MG_THREADS>(c, sm.scan, &U0);
            }
            if (threadIdx.x < SG_WAVE) {
                if (early && threadIdx.x == 0) store_agent(p.status + t, (t == 0 ? MG_FLAG_INC : MG_FLAG_AGG) | U0);
                uint64_t x = t == 0 ? 0ull : look_back(p, t);
                if (threadIdx.x == 0) {
                    if (early && t != 0) store_agent(p.status + t, MG_FLAG_INC | (x + U0));
                    sm.bcast64[0] = x;
                }
            }
            __syncthreads();
            X = sm.bcast64[0];
        }
        uint64_t produced = 0;

        while (true) {
            // windows per worker
            if (threadIdx.x == 0) {
                uint32_t acc = 0;
                for (uint32_t w = 0; w < n; ++w) {
                    uint32_t rem = sm.end[w] - sm.cur[w];
                    uint32_t a = single ? rem : (rem < win ? rem : win);
                    sm.wofs[w] = acc;
                    sm.take[w] = a;
                    acc += a;
                }
                sm.wofs[n] = acc;
            }
            __syncthreads();
            const uint32_t L = sm.wofs[n];
            if (L == 0 && !single) break; // a single tile runs once, even when empty
            // load windows (keys; values for scalar aggregate)
            for (uint32_t w = 0; w < n; ++w) {
                const uint32_t a = sm.take[w], base = sm.wofs[w];
                const uint64_t gs = sm.src0[w] + sm.cur[w];
                for (uint32_t i = threadIdx.x; i < a; i += MG_THREADS) {
                    sm.keys[0][base + i] = p.idx[gs + i];
                    sm.lidx[0][base + i] = (uint16_t)(base + i);
                    if (MODE == MODE_AGG && p.D == 1)
                        sm.vals[base + i] = p.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.val)[gs + i])
                                                   : static_cast<const float*>(p.val)[gs + i];
                }
            }
            __syncthreads();
            // cut: keys <= kmax are complete in every window
            if (threadIdx.x == 0) {
                uint32_t kmax = 0xffffffffu;
                bool cut = false;
                for (uint32_t w = 0; w < n; ++w) {
                    const uint32_t a = sm.take[w];
                    if (a > 0 && sm.cur[w] + a < sm.end[w]) {
                        uint32_t last = sm.keys[0][sm.wofs[w] + a - 1];
                        if (!cut || last < kmax) kmax = last;
                        cut = true;
                    }
                }
                sm.bcast[1] = kmax;
                sm.bcast[2] = cut ? 1u : 0u;
            }
            __syncthreads();
            const bool cut = sm.bcast[2] != 0;
            if (cut) {
                // per worker: entries <= kmax (a prefix of the window)
                const uint32_t kmax = sm.bcast[1];
                if (threadIdx.x < n) {
                    const uint32_t w = threadIdx.x, a = sm.take[w], base = sm.wofs[w];
                    uint32_t l = 0, h = a;
                    while (l < h) {
                        uint32_t m = (l + h) >> 1;
                        if (sm.keys[0][base + m] <= kmax) l = m + 1;
                        else h = m;
                    }
                    sm.take[w] = l;
                }
                __syncthreads();
                // compact the taken prefixes to the front, keeping worker order
                if (threadIdx.x == 0) {
                    uint32_t acc = 0;
                    for (uint32_t w = 0; w < n; ++w) {
                        sm.lofs[w] = acc; // new offsets (temporarily in lofs)
                        acc += sm.take[w];
                    }
                    sm.lofs[n] = acc;
                }
                __syncthreads();
                for (uint32_t w = 0; w < n; ++w) {
                    const uint32_t a = sm.take[w], from = sm.wofs[w], to = sm.lofs[w];
                    for (uint32_t i = threadIdx.x; i < a; i += MG_THREADS) {
                        sm.keys[1][to + i] = sm.keys[0][from + i];
                        sm.lidx[1][to + i] = sm.lidx[0][from + i];
                    }
                }
                __syncthreads();
                const uint32_t E2 = sm.lofs[n];
                for (uint32_t i = threadIdx.x; i < E2; i += MG_THREADS) {
                    sm.keys[0][i] = sm.keys[1][i];
                    sm.lidx[0][i] = sm.lidx[1][i];
                }
                __syncthreads();
            } else {
                if (threadIdx.x <= n) sm.lofs[threadIdx.x] = sm.wofs[threadIdx.x];
                __syncthreads();
            }
            const uint32_t E2 = sm.lofs[n];
            // merge
            const int fin = merge_tree(sm, n, E2);
            const uint32_t* K = sm.keys[fin];
            const uint16_t* LI = sm.lidx[fin];
            // heads and unique ranks
            const uint32_t per = (E2 + MG_THREADS - 1) / MG_THREADS;
            const uint32_t o0 = threadIdx.x * per, o1 = o0 + per < E2 ? o0 + per : E2;
            uint32_t hc = 0;
            for (uint32_t o = o0; o < o1; ++o) hc += (o == 0 || K[o] != K[o - 1]);
            uint32_t U;
            uint32_t u = block_excl_scan<MG_THREADS>(hc, sm.scan, &U);
            for (uint32_t o = o0; o < o1; ++o)
                if (o == 0 || K[o] != K[o - 1]) sm.hpos[u++] = (uint16_t)o;
            __syncthreads();

            if (MODE == MODE_AGG) {
                if (single) {
                    if (threadIdx.x < SG_WAVE) {
                        if (threadIdx.x == 0) store_agent(p.status + t, (t == 0 ? MG_FLAG_INC : MG_FLAG_AGG) | U);
                        uint64_t x = t == 0 ? 0ull : look_back(p, t);
                        if (threadIdx.x == 0) {
                            if (t != 0) store_agent(p.status + t, MG_FLAG_INC | (x + U));
                            sm.bcast64[0] = x;
                        }
                    }
                    __syncthreads();
                    X = sm.bcast64[0];
                }
                const uint64_t ob = X + produced;
                if (p.D <= 1) {
                    for (uint32_t q = threadIdx.x; q < U; q += MG_THREADS) {
                        const uint32_t o = sm.hpos[q];
                        const uint32_t key = K[o];
                        const uint64_t dst = ob + q;
                        if (dst >= p.capacity) continue;
                        p.agg_idx[dst] = key;
                        if (p.D == 1) {
                            float acc = 0.0f;
                            for (uint32_t z = o; z < E2 && K[z] == key; ++z) acc += sm.vals[LI[z]];
                            p.agg_val[dst] = acc;
                        }
                    }
                } else {
                    // rows: one wave per unique, lanes across the row
                    const uint32_t wid = threadIdx.x / SG_WAVE;
                    for (uint32_t q = wid; q < U; q += MG_THREADS / SG_WAVE) {
                        const uint32_t o = sm.hpos[q];
                        const uint32_t key = K[o];
                        const uint64_t dst = ob + q;
                        if (dst >= p.capacity) continue;
                        if (lane_id() == 0) p.agg_idx[dst] = key;
                        for (uint32_t c0 = 0; c0 < p.D; c0 += SG_WAVE) {
                            const uint32_t c = c0 + lane_id();
                            float acc = 0.0f;
                            for (uint32_t z = o; z < E2 && K[z] == key; ++z) {
                                const uint32_t li = LI[z];
                                uint32_t w = 0;
                                while (w + 1 < n && sm.wofs[w + 1] <= li) ++w;
                                const uint64_t pos = sm.src0[w] + sm.cur[w] + (li - sm.wofs[w]);
                                if (c < p.D) {
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
                // statistics: union size, pairwise intersections, per-part counts
                const uint32_t wid = threadIdx.x / SG_WAVE;
                for (uint32_t q0 = wid * SG_WAVE; q0 < U; q0 += MG_THREADS) {
                    const uint32_t q = q0 + lane_id();
                    uint64_t m = 0;
                    uint32_t key = 0;
                    if (q < U) {
                        const uint32_t o = sm.hpos[q];
                        key = K[o];
                        for (uint32_t z = o; z < E2 && K[z] == key; ++z) {
                            const uint32_t li = LI[z];
                            uint32_t w = 0;
                            while (w + 1 < n && sm.wofs[w + 1] <= li) ++w;
                            m |= 1ull << w;
                        }
                        atomicAdd(&ucontig[contig_part(key, p.M, p.Ps)], 1u);
                        if (p.hashed) atomicAdd(&uhashed[h0(key, p.seed, p.div)], 1u);
                    }
                    for (uint32_t a = 0; a < n; ++a) {
                        const uint64_t v = ballot((m >> a) & 1ull);
                        if (lane_id() == 0) sm.vmask[wid][a] = v;
                    }
                    // lanes take pairs (a, b), a <= b
                    const uint32_t npairs = n * (n + 1) / 2;
                    for (uint32_t pi = lane_id(); pi < npairs; pi += SG_WAVE) {
                        uint32_t a = 0, rem = pi;
                        while (rem >= n - a) {
                            rem -= n - a;
                            ++a;
                        }
                        const uint32_t b = a + rem;
                        const uint32_t c = popc64(sm.vmask[wid][a] & sm.vmask[wid][b]);
                        if (c) atomicAdd(&inter_lds[a * 64 + b], c);
                    }
                }
                if (threadIdx.x == 0) union_lds += U;
            }
            produced += U;
            // advance (after every wave is done reading the cursors)
            __syncthreads();
            if (threadIdx.x < n) sm.cur[threadIdx.x] += sm.take[threadIdx.x];
            __syncthreads();
            if (single) break;
        }
        if (MODE == MODE_AGG) {
            if (!single && !early && threadIdx.x == 0) store_agent(p.status + t, MG_FLAG_INC | (X + produced));
            if (t == total_tiles - 1 && threadIdx.x == 0) p.agg_off[p.G] = X + produced;
            if (jt == 0 && threadIdx.x == 0) p.agg_off[g] = X;
        }
        __syncthreads();
    }
    if (MODE == MODE_STATS) {
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < n * n; i += MG_THREADS) {
            const uint32_t a = i / n, b = i % n;
            if (a <= b && inter_lds[a * 64 + b]) atomicAdd((unsigned long long*)&p.st_inter[a * n + b], (unsigned long long)inter_lds[a * 64 + b]);
        }
        for (uint32_t i = threadIdx.x; i < p.Ps; i += MG_THREADS) {
            if (ucontig[i]) atomicAdd((unsigned long long*)&p.st_ucontig[i], (unsigned long long)ucontig[i]);
            if (p.hashed && uhashed[i]) atomicAdd((unsigned long long*)&p.st_uhashed[i], (unsigned long long)uhashed[i]);
        }
        if (threadIdx.x == 0 && union_lds) atomicAdd((unsigned long long*)p.st_union, (unsigned long long)union_lds);
    }
}

} // namespace sg

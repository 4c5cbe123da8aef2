// sg_partition.hip -- A2: hash partition of n workers' COO entries.
//
// Zen (OSDI'25) digest, section 3.1 Problem 1 and section 3.2 Technique #3:
// one partition hash h0 shared by all workers sends every index to the same
// server.  Zen realises it with slot memory, rehashing and an atomic serial
// area (Algorithm 1) because its extraction then runs nonzero() over the slot
// memory.  Here the same membership comes from a stable multi-split with no
// slot memory and no collisions: per 2048-entry tile a histogram of h0, one
// scan of the per-(tile, partition) counts, and a scatter that ranks entries
// inside the tile with wave64 ballots, stages them partition-sorted in LDS and
// writes each partition's run with consecutive lanes on consecutive
// addresses.  Reads: idx twice (histogram, scatter) and values once; writes:
// idx and values once.
#include "sg_host.h"

namespace sg {

constexpr int PT_THREADS = 256;
constexpr int PT_TILE = 2048; // entries per tile (2048: twice the blocks per CU of 4096, whose LDS staging allowed three)
constexpr int PT_WAVES = PT_THREADS / SG_WAVE;
constexpr int PT_STRIPS = PT_TILE / PT_THREADS; // 64-entry strips per wave

struct PartParams {
    const uint32_t* idx;
    const void* val;
    const uint64_t* in_off;
    uint32_t* out_idx;
    void* out_val;
    uint64_t* part_off;
    uint32_t* tile_start; // [n+1] first global tile of worker w
    uint32_t* counts;     // [max_tiles][P] counts, then destination offsets
    uint32_t* src_of;     // [total] rows (D >= 2): the input entry each output entry comes from
    uint64_t total;
    uint32_t n, P, seed, D, esz, nbits;
    uint32_t row_w4; // rows can be copied as 4-byte words
    uint32_t max_tiles;
    Divider div;
};

__device__ __forceinline__ void worker_range(const PartParams& p, uint32_t w, uint64_t& b, uint64_t& e)
{
    uint64_t x = p.in_off[w], y = p.in_off[w + 1];
    if (x > p.total) x = p.total;
    if (y > p.total) y = p.total;
    if (y < x) y = x;
    b = x;
    e = y;
}

// tile_start[w] = sum over workers before w of ceil(len/TILE)
__global__ void part_plan_kernel(PartParams p)
{
    __shared__ uint32_t scan_lds[PT_WAVES + 1];
    uint32_t carry = 0;
    bool bad = false;
    for (uint32_t base = 0; base < p.n; base += PT_THREADS) {
        uint32_t w = base + threadIdx.x;
        uint32_t tiles = 0;
        if (w < p.n) {
            uint64_t b, e;
            worker_range(p, w, b, e);
            tiles = (uint32_t)ceil_div_dev(e - b, PT_TILE);
            if (p.in_off[w] > p.in_off[w + 1] || p.in_off[w + 1] > p.total) bad = true;
        }
        uint32_t tot;
        uint32_t ex = block_excl_scan<PT_THREADS>(tiles, scan_lds, &tot);
        if (w < p.n) p.tile_start[w] = carry + ex;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        p.tile_start[p.n] = carry;
        if (p.in_off[0] != 0 || p.in_off[p.n] != p.total) bad = true;
    }
    if (bad) report_error(kDevErrBadOffsets);
}

// worker of global tile t (tile_start is non-decreasing)
__device__ __forceinline__ uint32_t tile_worker(const PartParams& p, uint32_t t)
{
    uint32_t lo = 0, hi = p.n;
    while (lo + 1 < hi) {
        uint32_t mid = (lo + hi) >> 1;
        if (p.tile_start[mid] <= t) lo = mid;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ bool tile_bounds(const PartParams& p, uint32_t t, uint32_t& w, uint64_t& e0,
                                            uint64_t& e1)
{
    if (t >= p.tile_start[p.n]) return false;
    w = tile_worker(p, t);
    uint64_t b, e;
    worker_range(p, w, b, e);
    e0 = b + (uint64_t)(t - p.tile_start[w]) * PT_TILE;
    e1 = e0 + PT_TILE < e ? e0 + PT_TILE : e;
    return e0 < e1;
}

__global__ __launch_bounds__(PT_THREADS) void part_hist_kernel(PartParams p)
{
    __shared__ uint32_t hist[256];
    const uint32_t t = blockIdx.x;
    uint32_t w;
    uint64_t e0, e1;
    for (uint32_t i = threadIdx.x; i < p.P; i += PT_THREADS) hist[i] = 0;
    __syncthreads();
    bool live = tile_bounds(p, t, w, e0, e1);
    if (live) {
        // every load first (clamped to the tile), then the counts
        const uint32_t len = (uint32_t)(e1 - e0);
        uint32_t key[PT_STRIPS];
#pragma unroll
        for (int s = 0; s < PT_STRIPS; ++s) {
            const uint32_t le = s * PT_THREADS + threadIdx.x;
            key[s] = p.idx[e0 + (le < len ? le : len - 1)];
        }
#pragma unroll
        for (int s = 0; s < PT_STRIPS; ++s)
            if (s * PT_THREADS + threadIdx.x < len) atomicAdd(&hist[h0(key[s], p.seed, p.div)], 1u);
    }
    __syncthreads();
    if (t < p.max_tiles)
        for (uint32_t i = threadIdx.x; i < p.P; i += PT_THREADS) p.counts[(uint64_t)t * p.P + i] = live ? hist[i] : 0u;
}

// One block per worker: for each partition q, exclusive scan of counts over
// the worker's tiles, offset by the start of partition q inside the worker.
// The block's 1024 threads are P partitions x S tile segments: each thread
// sums its segment, the S segment sums of a partition are scanned, and each
// thread writes its segment's running offsets.
constexpr int PS_THREADS = 1024;
__global__ __launch_bounds__(PS_THREADS) void part_scan_kernel(PartParams p)
{
    __shared__ uint32_t seg[PS_THREADS];
    __shared__ uint32_t part_tot[256], part_base[256];
    __shared__ uint32_t scan_lds[PS_THREADS / SG_WAVE + 1];
    const uint32_t w = blockIdx.x;
    const uint32_t t0 = p.tile_start[w], t1 = p.tile_start[w + 1], nt = t1 - t0;
    uint64_t b, e;
    worker_range(p, w, b, e);
    const uint32_t S = PS_THREADS / p.P; // segments per partition (>= 4)
    const uint32_t q = threadIdx.x % p.P, sgi = threadIdx.x / p.P;
    const bool act = sgi < S;
    const uint32_t per = (nt + S - 1) / S;
    const uint32_t a0 = t0 + sgi * per, a1 = (a0 + per < t1) ? a0 + per : t1;
    uint32_t sum = 0;
    if (act)
        for (uint32_t t = a0; t < a1; ++t) sum += p.counts[(uint64_t)t * p.P + q];
    seg[threadIdx.x] = act ? sum : 0u;
    __syncthreads();
    // per partition: exclusive scan over its S segments (thread q walks them)
    if (threadIdx.x < p.P) {
        uint32_t run = 0;
        for (uint32_t k = 0; k < S; ++k) {
            const uint32_t v = seg[k * p.P + threadIdx.x];
            seg[k * p.P + threadIdx.x] = run;
            run += v;
        }
        part_tot[threadIdx.x] = run;
    }
    __syncthreads();
    uint32_t all;
    const uint32_t ex = block_excl_scan<PS_THREADS>(threadIdx.x < p.P ? part_tot[threadIdx.x] : 0u, scan_lds, &all);
    if (threadIdx.x < p.P) {
        part_base[threadIdx.x] = (uint32_t)b + ex;
        p.part_off[(uint64_t)w * (p.P + 1) + threadIdx.x] = (uint32_t)b + ex;
    }
    if (threadIdx.x == 0) p.part_off[(uint64_t)w * (p.P + 1) + p.P] = e;
    __syncthreads();
    if (act) {
        uint32_t run = part_base[q] + seg[threadIdx.x];
        for (uint32_t t = a0; t < a1; ++t) {
            const uint32_t c = p.counts[(uint64_t)t * p.P + q];
            p.counts[(uint64_t)t * p.P + q] = run;
            run += c;
        }
    }
}

template <bool STAGE_VALS, typename VT>
__global__ __launch_bounds__(PT_THREADS) void part_scatter_kernel(PartParams p)
{
    __shared__ uint32_t keys_s[PT_TILE];
    __shared__ VT vals_s[STAGE_VALS ? PT_TILE : 1];
    __shared__ uint8_t part_s[PT_TILE];
    __shared__ uint16_t rank_s[STAGE_VALS ? 1 : PT_TILE]; // rows: input order -> staging position
    __shared__ uint32_t wave_cnt[PT_WAVES][256];
    __shared__ uint32_t lps[256];   // staging start of partition q
    __shared__ uint32_t dbase[256]; // global destination of the tile's run of q
    __shared__ uint32_t scan_lds[PT_WAVES + 1];

    const uint32_t t = blockIdx.x;
    uint32_t w;
    uint64_t e0, e1;
    if (!tile_bounds(p, t, w, e0, e1)) return; // uniform per block
    const uint32_t len = (uint32_t)(e1 - e0);
    const uint32_t wid = threadIdx.x / SG_WAVE, lane = lane_id();

    for (uint32_t i = threadIdx.x; i < PT_WAVES * 256; i += PT_THREADS) (&wave_cnt[0][0])[i] = 0;
    __syncthreads();

    // 1. stable ranks inside each wave's quarter of the tile
    uint32_t key_r[PT_STRIPS];
    uint8_t part_r[PT_STRIPS];
    uint16_t rank_r[PT_STRIPS];
    VT val_r[STAGE_VALS ? PT_STRIPS : 1];
    // every strip's loads first (unconditional, clamped to the tile), so
    // they are in flight together
#pragma unroll
    for (int s = 0; s < PT_STRIPS; ++s) {
        const uint32_t le = wid * (PT_TILE / PT_WAVES) + s * SG_WAVE + lane;
        const uint64_t src = e0 + (le < len ? le : len - 1);
        key_r[s] = p.idx[src];
        if (STAGE_VALS) val_r[s] = static_cast<const VT*>(p.val)[src];
    }
#pragma unroll
    for (int s = 0; s < PT_STRIPS; ++s) {
        const uint32_t le = wid * (PT_TILE / PT_WAVES) + s * SG_WAVE + lane;
        const bool valid = le < len;
        const uint32_t key = key_r[s];
        uint32_t q = valid ? h0(key, p.seed, p.div) : 0u;
        uint64_t peers = ballot(valid);
        for (uint32_t bit = 0; bit < p.nbits; ++bit) {
            uint64_t m = ballot(valid && ((q >> bit) & 1u));
            peers &= ((q >> bit) & 1u) ? m : ~m;
        }
        uint32_t below = popc64(peers & lanemask_lt());
        uint32_t base = valid ? wave_cnt[wid][q] : 0u;
        if (valid && below == 0) wave_cnt[wid][q] = base + popc64(peers);
        part_r[s] = (uint8_t)q;
        rank_r[s] = (uint16_t)(base + below);
    }
    for (uint32_t i = threadIdx.x; i < p.P; i += PT_THREADS) dbase[i] = p.counts[(uint64_t)t * p.P + i];
    __syncthreads();

    // 2. per-partition wave prefixes and staging starts
    uint32_t tile_cnt = 0;
    if (threadIdx.x < p.P) {
        uint32_t acc = 0;
        for (int v = 0; v < PT_WAVES; ++v) {
            uint32_t c = wave_cnt[v][threadIdx.x];
            wave_cnt[v][threadIdx.x] = acc;
            acc += c;
        }
        tile_cnt = acc;
    }
    uint32_t all;
    uint32_t ex = block_excl_scan<PT_THREADS>(tile_cnt, scan_lds, &all);
    if (threadIdx.x < p.P) lps[threadIdx.x] = ex;
    __syncthreads();

    // 3. stage partition-sorted
#pragma unroll
    for (int s = 0; s < PT_STRIPS; ++s) {
        const uint32_t le = wid * (PT_TILE / PT_WAVES) + s * SG_WAVE + lane;
        if (le < len) {
            uint32_t q = part_r[s];
            uint32_t sp = lps[q] + wave_cnt[wid][q] + rank_r[s];
            keys_s[sp] = key_r[s];
            part_s[sp] = (uint8_t)q;
            if (STAGE_VALS) vals_s[sp] = val_r[s];
            if (!STAGE_VALS) rank_s[le] = (uint16_t)sp;
        }
    }
    __syncthreads();

    // 4. write each partition's run: consecutive lanes, consecutive addresses
    //    (four staged entries per thread read before any is written)
    for (uint32_t i0 = threadIdx.x; i0 < len; i0 += 4 * PT_THREADS) {
        uint32_t dst[4], kv[4];
        VT vv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t i = i0 + u * PT_THREADS;
            const uint32_t ic = i < len ? i : 0u;
            const uint32_t q = part_s[ic];
            dst[u] = i < len ? dbase[q] + (i - lps[q]) : 0xffffffffu;
            kv[u] = keys_s[ic];
            if (STAGE_VALS) vv[u] = vals_s[ic];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (dst[u] >= p.total) continue; // past the tile, or inconsistent offsets
            p.out_idx[dst[u]] = kv[u];
            if (STAGE_VALS) static_cast<VT*>(p.out_val)[dst[u]] = vv[u];
        }
    }

    // 5. rows (D >= 2): the source of every output entry, for part_rows_kernel
    if (!STAGE_VALS && p.D > 1) {
        for (uint32_t le = threadIdx.x; le < len; le += PT_THREADS) {
            const uint32_t sp = rank_s[le];
            const uint32_t q = part_s[sp];
            const uint64_t dst = (uint64_t)dbase[q] + (sp - lps[q]);
            if (dst < p.total) p.src_of[dst] = (uint32_t)(e0 + le);
        }
    }
}

// Rows (D >= 2): output row r is input row src_of[r].  One thread per word
// of the output (4 bytes, or 2 when a row is not a whole number of 4-byte
// words); consecutive threads, consecutive addresses.
template <typename W>
__global__ __launch_bounds__(256) void part_rows_kernel(PartParams p)
{
    const uint32_t wpr = p.D * p.esz / (uint32_t)sizeof(W); // words per row
    const uint64_t words = p.total * wpr;
    const W* src = static_cast<const W*>(p.val);
    W* out = static_cast<W*>(p.out_val);
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < words; i += (uint64_t)gridDim.x * 256) {
        const uint64_t r = i / wpr;
        const uint32_t k = (uint32_t)(i - r * wpr);
        const uint32_t from = p.src_of[r];
        if (from >= p.total) { // cannot happen: every output entry has a source
            report_error(kDevErrPartition);
            continue;
        }
        out[i] = src[(uint64_t)from * wpr + k];
    }
}

} // namespace sg

using namespace sg;

static uint32_t part_max_tiles(uint32_t n, uint64_t total) { return (uint32_t)(ceil_div(total, PT_TILE) + n); }

// rows: whether the source of every output entry is recorded (D >= 2)
static uint64_t part_carve(Carver& c, uint32_t n, uint64_t total, uint32_t P, bool rows, uint32_t** tile_start,
                           uint32_t** counts, uint32_t** src_of)
{
    *tile_start = c.take<uint32_t>((uint64_t)n + 1);
    *counts = c.take<uint32_t>((uint64_t)part_max_tiles(n, total) * P);
    *src_of = c.take<uint32_t>(rows ? total : 0);
    return c.bytes();
}

static int part_check(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D, const uint64_t* d_in_off,
                      uint32_t n, uint64_t total, uint32_t P, const uint32_t* d_out_idx, const void* d_out_val,
                      const uint64_t* d_part_off)
{
    if (n == 0 || P == 0 || P > 256 || D > 65536 || (dt != SG_F32 && dt != SG_BF16)) return SG_EINVAL;
    if (total >= (1ull << 32)) return SG_EUNSUPPORTED;
    if (!d_in_off || !d_part_off) return SG_EINVAL;
    if (total > 0 && (!d_idx || !d_out_idx)) return SG_EINVAL;
    if (D > 0 && total > 0 && (!d_val || !d_out_val)) return SG_EINVAL;
    return SG_OK;
}

// The launches, with the workspace already carved into p.
static int part_run(PartParams& p, const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D,
                    const uint64_t* d_in_off, uint32_t n, uint64_t total, uint32_t P, uint32_t seed,
                    uint32_t* d_out_idx, void* d_out_val, uint64_t* d_part_off, hipStream_t st);

extern "C" size_t sg_partition_workspace_bytes(uint32_t n, uint64_t total, uint32_t P)
{
    Carver c(nullptr);
    uint32_t *a, *b, *d;
    return part_carve(c, n, total, P, true, &a, &b, &d);
}

extern "C" int sg_hash_partition(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D,
                                 const uint64_t* d_in_off, uint32_t n, uint64_t total, uint32_t P, uint32_t seed,
                                 uint32_t* d_out_idx, void* d_out_val, uint64_t* d_part_off, void* d_ws,
                                 size_t ws_bytes, void* stream)
{
    const int rc = part_check(d_idx, d_val, dt, D, d_in_off, n, total, P, d_out_idx, d_out_val, d_part_off);
    if (rc != SG_OK) return rc;
    if (!d_ws) return SG_EINVAL;
    if (ws_bytes < sg_partition_workspace_bytes(n, total, P)) return SG_ECAPACITY;
    PartParams p;
    Carver c(d_ws);
    part_carve(c, n, total, P, true, &p.tile_start, &p.counts, &p.src_of);
    return part_run(p, d_idx, d_val, dt, D, d_in_off, n, total, P, seed, d_out_idx, d_out_val, d_part_off,
                    as_stream(stream));
}

// ---------------------------------------------------------------------------
// The same partition with no workspace argument and no allocation: the
// per-tile counts (and, for rows, the output entries' sources) live in a
// fixed device array of the library, `scratch`, one per GPU for the life of
// the process.  Its device address is looked up once per device with the
// device current (the host-side name of a __device__ array is not a device
// address) and kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SG_PARTITION_SCRATCH_BYTES];

static constexpr int PT_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[PT_MAX_DEVICES] = {};

static int scratch_of_current_device(void** out)
{
    int dev = 0;
    SG_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= PT_MAX_DEVICES) return SG_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        SG_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return SG_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SG_OK;
}

extern "C" int sg_hash_partition_noalloc(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D,
                                         const uint64_t* d_in_off, uint32_t n, uint64_t total, uint32_t P,
                                         uint32_t seed, uint32_t* d_out_idx, void* d_out_val, uint64_t* d_part_off,
                                         void* stream)
{
    const int rc = part_check(d_idx, d_val, dt, D, d_in_off, n, total, P, d_out_idx, d_out_val, d_part_off);
    if (rc != SG_OK) return rc;
    uint32_t *a, *b, *d;
    Carver sz(nullptr);
    if (part_carve(sz, n, total, P, D > 1, &a, &b, &d) > SG_PARTITION_SCRATCH_BYTES) return SG_ECAPACITY;
    void* base = nullptr;
    const int src = scratch_of_current_device(&base);
    if (src != SG_OK) return src;
    // every word the kernels read is written first by the same call (tile
    // starts by the plan kernel, all counts by the histogram kernel, the
    // sources by the scatter), so nothing is cleared
    PartParams p;
    Carver c(base);
    part_carve(c, n, total, P, D > 1, &p.tile_start, &p.counts, &p.src_of);
    return part_run(p, d_idx, d_val, dt, D, d_in_off, n, total, P, seed, d_out_idx, d_out_val, d_part_off,
                    as_stream(stream));
}

static int part_run(PartParams& p, const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D,
                    const uint64_t* d_in_off, uint32_t n, uint64_t total, uint32_t P, uint32_t seed,
                    uint32_t* d_out_idx, void* d_out_val, uint64_t* d_part_off, hipStream_t st)
{
    p.idx = d_idx;
    p.val = d_val;
    p.in_off = d_in_off;
    p.out_idx = d_out_idx;
    p.out_val = d_out_val;
    p.part_off = d_part_off;
    p.total = total;
    p.n = n;
    p.P = P;
    p.seed = seed;
    p.D = D;
    p.esz = dt == SG_BF16 ? 2 : 4;
    p.nbits = 0;
    while ((1u << p.nbits) < P) ++p.nbits;
    p.max_tiles = part_max_tiles(n, total);
    p.div = make_divider(P);
    p.row_w4 = ((uint64_t)D * p.esz % 4 == 0) && ((uintptr_t)d_val % 4 == 0) && ((uintptr_t)d_out_val % 4 == 0);

    part_plan_kernel<<<1, PT_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_PARTITION_HIST, st);
    part_hist_kernel<<<p.max_tiles, PT_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_PARTITION_HIST, st);
    part_scan_kernel<<<n, PS_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_PARTITION_SCATTER, st);
    if (D == 0) part_scatter_kernel<false, uint32_t><<<p.max_tiles, PT_THREADS, 0, st>>>(p);
    else if (D == 1 && dt == SG_F32) part_scatter_kernel<true, uint32_t><<<p.max_tiles, PT_THREADS, 0, st>>>(p);
    else if (D == 1) part_scatter_kernel<true, uint16_t><<<p.max_tiles, PT_THREADS, 0, st>>>(p);
    else part_scatter_kernel<false, uint32_t><<<p.max_tiles, PT_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_PARTITION_SCATTER, st);
    if (D > 1 && total > 0) {
        const uint64_t words = total * D * p.esz / (p.row_w4 ? 4 : 2);
        const unsigned grid = (unsigned)(ceil_div(words, 256) < 65536 ? ceil_div(words, 256) : 65536);
        if (p.row_w4) part_rows_kernel<uint32_t><<<grid, 256, 0, st>>>(p);
        else part_rows_kernel<uint16_t><<<grid, 256, 0, st>>>(p);
        SG_TRY_LAUNCH();
    }
    return SG_OK;
}

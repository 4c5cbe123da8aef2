// sg_stats.hip -- A6: sparsity statistics of n workers' index sets, from
// exact integer counts (Zen OSDI'25 digest, section 2.1 Defs. 3-5; section
// 3.1 Def. 8).
//
// The union and every pairwise intersection come, for up to 16 workers and
// 16 parts when the lists hold at least one entry per 2 * 32 keys of the
// key space per worker on average (or the bitmaps take at most 64 MB), from
// the dense pass of sg_statsd.hip
// (per-worker bitmaps of the whole key space, which also give each worker's
// counts per part and per class); otherwise, for up to 16 workers and 16
// hash classes, from the window pass of sg_statsw.hip (per-worker bitmaps of
// 2048-key windows); otherwise from the merge engine run over the workers'
// lists (one group): per union index the set of workers holding it is a
// 64-bit mask; per 64 indices a wave turns the masks into one ballot word per
// worker and adds popcount(V_a & V_b) for each pair.  Every pass writes
// partial rows of counts and a last pass sums the rows.  Outside the dense
// pass each worker's counts per contiguous part come from binary searches in
// its ascending list, its counts per hash class from one pass over the
// entries.  The host then evaluates the definitions in double with fixed
// expressions.
#include "sg_host.h"

namespace sg {

// The counts and everything else the host needs after the passes sit in one
// block of u64, copied to the host at once: row, wcontig, whashed, then the
// tail written by st_pack_kernel.
struct StatsCounts {
    uint64_t* row;      // [npairs + 1 + 2*Ps]: pair counts (a <= b, row-major), union, union per part
    uint64_t* wcontig;  // [n*Ps]
    uint64_t* whashed;  // [n*Ps]
    uint64_t* tail;     // [n + 1 + Ps + 4]: worker offsets, class sizes, map magic, P, M, seed
    uint64_t words;     // of the whole block
};

__global__ void st_pack_kernel(const uint64_t* __restrict__ in_off, uint32_t n, const uint64_t* __restrict__ class_size,
                               const CmapHeader* __restrict__ hdr, uint32_t P, uint64_t* __restrict__ tail)
{
    for (uint32_t i = threadIdx.x; i <= n; i += blockDim.x) tail[i] = in_off[i];
    for (uint32_t i = threadIdx.x; i < P; i += blockDim.x) tail[n + 1 + i] = class_size ? class_size[i] : 0ull;
    if (threadIdx.x == 0) {
        uint64_t* h = tail + n + 1 + P;
        h[0] = hdr ? hdr->magic : 0ull;
        h[1] = hdr ? hdr->P : 0ull;
        h[2] = hdr ? hdr->M : 0ull;
        h[3] = hdr ? hdr->seed : 0ull;
    }
}

// Per-worker counts per contiguous part: a worker's list is ascending, so the
// entries of part q = [floor(qM/P), floor((q+1)M/P)) lie between the lower
// bounds of the two ends.  One wave per (worker, part) finds both by 64-ary
// search: each round the lanes probe 64 evenly spaced positions of the
// remaining range of each bound (both bounds' probes in the same round).
__global__ __launch_bounds__(256) void st_contig_kernel(MergeParams p, StatsCounts c)
{
    const uint32_t i = blockIdx.x * 4 + uniform(threadIdx.x / SG_WAVE);
    if (i >= p.n * p.Ps) return;
    const uint32_t lane = lane_id();
    const uint32_t w = i / p.Ps, q = i % p.Ps;
    uint64_t s, e;
    run_range(p, 0, w, s, e);
    const uint64_t key[2] = {p.M * q / p.Ps, p.M * (q + 1) / p.Ps}; // M < 2^32, P <= 256
    uint64_t lo[2] = {0, 0}, hi[2] = {e - s, e - s}; // the bound lies in [lo, hi]
    while (hi[0] > lo[0] || hi[1] > lo[1]) {
        uint64_t step[2], pos[2];
        bool lt[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // probes lo + l*step for l < 64 and < hi; a[pos] < key is true on a prefix
            step[h] = (hi[h] - lo[h] + SG_WAVE - 1) / SG_WAVE;
            pos[h] = lo[h] + (uint64_t)lane * step[h];
            const bool in = hi[h] > lo[h] && pos[h] < hi[h];
            lt[h] = in && (uint64_t)p.idx[s + pos[h]] < key[h];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (hi[h] <= lo[h]) continue;
            const uint32_t cnt = popc64(ballot(lt[h])); // probes below the key
            if (cnt == 0) {
                hi[h] = lo[h];
            } else {
                const uint64_t last = lo[h] + (uint64_t)(cnt - 1) * step[h]; // a[last] < key
                const uint64_t nxt = lo[h] + (uint64_t)cnt * step[h];
                lo[h] = last + 1;
                if (nxt < hi[h]) hi[h] = nxt; // a[nxt] >= key when it is a probe
            }
        }
    }
    if (lane == 0) c.wcontig[i] = lo[1] - lo[0];
}

// Per-worker counts per hash class: one block per 4096-entry chunk of a
// worker (chunk plan of the merge engine, G = 1); all of a thread's loads in
// flight at once, then one LDS atomic per key; the block's counts are added
// to the worker's after each chunk.
__global__ __launch_bounds__(MG_THREADS) void st_entries_kernel(MergeParams p, StatsCounts c)
{
    constexpr int U = MG_CHUNK / MG_THREADS;
    __shared__ uint32_t hh[256];
    const uint32_t hseed = p.seed_at ? p.seed_at[0] : p.seed;
    for (uint32_t i = threadIdx.x; i < p.Ps; i += MG_THREADS) hh[i] = 0;
    __syncthreads();
    for (uint32_t ch = blockIdx.x; ch < p.nchunks_max; ch += gridDim.x) {
        const uint4 rec = p.chunk_rec[ch];
        if (rec.x == 0xffffffffu) continue;
        const uint32_t w = rec.x; // one group: the run is the worker
        const uint64_t s = rec.w, len = rec.z, j0 = rec.y;
        uint32_t key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t j = j0 + (uint64_t)u * MG_THREADS + threadIdx.x;
            key[u] = p.idx[s + (j < len ? j : len - 1)];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j0 + (uint64_t)u * MG_THREADS + threadIdx.x < len) atomicAdd(&hh[h0(key[u], hseed, p.div)], 1u);
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < p.Ps; i += MG_THREADS) {
            if (hh[i]) atomicAdd((unsigned long long*)&c.whashed[(uint64_t)w * p.Ps + i], (unsigned long long)hh[i]);
            hh[i] = 0;
        }
        __syncthreads();
    }
}

} // namespace sg

using namespace sg;

// The window pass serves up to SW_MAXN workers and, with a class map, up to
// SW_MAXP classes.
static bool stats_windowed(uint32_t n, uint32_t P, bool hashed)
{
    return n <= (uint32_t)SW_MAXN && (!hashed || P <= (uint32_t)SW_MAXP);
}

// The dense pass: few enough workers and parts, and bitmaps of the key space
// no more than 16 times the entries (n * ceil(M/32) words <= 16 * total).
static bool stats_dense(uint32_t n, uint64_t M, uint64_t total, uint32_t P)
{
    // the dense pass zeroes, writes and reads n bitmaps of the key space; the
    // window pass reads the lists once (with a few instructions per entry):
    // the bitmaps must be small next to the lists for the dense pass to win
    // (measured: 0.6 bitmap words per entry, dense 2x faster; 3.1 words per
    // entry, windows 1.4x faster), unless the bitmaps are small anyway (up to
    // 64 MB: a few microseconds of traffic, fewer steps than the windows)
    const uint64_t words = (uint64_t)n * ceil_div(M, 32);
    return total > 0 && n <= DN_MAXN && P <= DN_MAXP && (words <= 2ull * total || words <= (16ull << 20));
}

static void stats_setup(MergeParams* p, uint32_t n, uint64_t M, uint64_t total, uint32_t P, bool windowed)
{
    *p = MergeParams();
    p->n = n;
    p->G = 1;
    p->stride = 1;
    p->M = M;
    p->total = total;
    p->Ps = P;
    p->inv_m = 1.0 / (double)M;
    p->npairs = n * (n + 1) / 2;
    p->st_row = p->npairs + 1 + 2 * P;
    if (windowed) {
        p->tb = SW_TB;
        const uint64_t nt = (M + (1ull << SW_TB) - 1) >> SW_TB;
        p->NT = (uint32_t)(nt ? nt : 1);
    } else {
        choose_tiles(1, M, total, &p->tb, &p->NT);
    }
}

static uint64_t stats_carve(Carver& c, MergeParams* p, uint32_t P, StatsCounts* k, SwParams* sw, DnParams* dn)
{
    const uint32_t n = p->n;
    if (dn) { // the dense pass: bitmaps, partial rows (with each worker's counts per part)
        dn->words = ceil_div(p->M, 32);
        dn->st_row = p->st_row + n * P;
        dn->bm = c.take<uint32_t>((uint64_t)n * dn->words);
        dn->rows = c.take<uint64_t>((uint64_t)DN_MAX_WAVES * dn->st_row);
    } else if (sw) { // the window pass: the boundary plan of the merge engine, the balance, partial rows
        const uint64_t R = n;
        p->nscan = (uint32_t)ceil_div(p->NT, MG_SCAN_BLOCK);
        p->chunk_start = c.take<uint32_t>(R + 1);
        p->nchunks_max = (uint32_t)(ceil_div(p->total, MG_CHUNK) + R);
        p->chunk_rec = c.take<uint4>(p->nchunks_max);
        p->bnd = c.take<uint32_t>(R * (p->NT + 1));
        p->nqsets = 1;
        p->queue = c.take<uint32_t>((uint64_t)MG_NQ * MG_QSTRIDE);
        sw->rows = c.take<uint64_t>((uint64_t)SW_MAX_WAVES * p->st_row);
    } else {
        merge_carve(c, p, MODE_STATS);
    }
    k->words = (uint64_t)p->st_row + 2ull * n * P + n + 1 + P + 4;
    k->row = c.take<uint64_t>(k->words);
    k->wcontig = k->row ? k->row + p->st_row : nullptr;
    k->whashed = k->wcontig ? k->wcontig + (uint64_t)n * P : nullptr;
    k->tail = k->whashed ? k->whashed + (uint64_t)n * P : nullptr;
    return c.bytes();
}

extern "C" size_t sg_stats_workspace_bytes(uint32_t n, uint64_t M, uint64_t total, uint32_t P)
{
    if (n == 0 || P == 0) return 256;
    // enough for any pass the call can take (the class map is not known here)
    size_t best = 0;
    for (int mode = 0; mode < 3; ++mode) { // merge, window, dense
        if (mode == 1 && !stats_windowed(n, P, false)) continue;
        if (mode == 2 && !stats_dense(n, M, total, P)) continue;
        MergeParams p;
        stats_setup(&p, n, M, total, P, mode == 1);
        Carver c(nullptr);
        StatsCounts k;
        SwParams sw;
        DnParams dn;
        const size_t b = stats_carve(c, &p, P, &k, mode == 1 ? &sw : nullptr, mode == 2 ? &dn : nullptr);
        if (b > best) best = b;
    }
    return best;
}

// The window pass: boundaries, balance, counts, the sum of the partial rows.
static int stats_window_run(MergeParams& p, SwParams& sw, hipStream_t st, uint64_t* out)
{
    const int ix = p.n <= 8 ? 0 : 1;
    const bool hashed = sw.planes != nullptr;
    int resident = 0;
    const void* kern = ix == 0 ? (const void*)sw_stats_kernel<8, true> : (const void*)sw_stats_kernel<16, true>;
    if (resident_blocks(kern, SW_THREADS, (int)(SW_MAX_WAVES / SW_WAVES), &resident) != SG_OK) return SG_EHIP;
    const uint64_t T = p.NT;
    const uint64_t wblocks = ceil_div(T, SW_WAVES);
    uint64_t grid = wblocks < (uint64_t)resident ? wblocks : (uint64_t)resident;
    if (grid == 0) grid = 1;
    const uint32_t W = (uint32_t)grid * SW_WAVES;
    mg_plan_kernel<<<1, 512, 0, st>>>(p);
    SG_TRY_LAUNCH();
    mg_bnd_kernel<<<p.nchunks_max < 65536 ? p.nchunks_max : 65536, 512, 0, st>>>(p);
    SG_TRY_LAUNCH();
    sw.m = p;
    if (ix == 0) {
        if (hashed) sw_stats_kernel<8, true><<<(unsigned)grid, SW_THREADS, 0, st>>>(sw);
        else sw_stats_kernel<8, false><<<(unsigned)grid, SW_THREADS, 0, st>>>(sw);
    } else {
        if (hashed) sw_stats_kernel<16, true><<<(unsigned)grid, SW_THREADS, 0, st>>>(sw);
        else sw_stats_kernel<16, false><<<(unsigned)grid, SW_THREADS, 0, st>>>(sw);
    }
    SG_TRY_LAUNCH();
    MergeParams q = p;
    q.st_part = sw.rows;
    mg_stats_reduce_kernel<<<p.st_row, 256, 0, st>>>(q, W, out);
    SG_TRY_LAUNCH();
    return SG_OK;
}

// The dense pass: zeroed bitmaps, their build (with each worker's counts per
// class), the count pass, the sum of the partial rows into `out` (the row and
// then each worker's counts per contiguous part).
static int stats_dense_run(MergeParams& p, DnParams& d, hipStream_t st, uint64_t* out)
{
    int rc = fill_u32(d.bm, (uint64_t)d.n * d.words, 0, st);
    if (rc) return rc;
    // entries per thread: the largest of 16, 8, 4, 2, 1 that still makes
    // 512 chunks (short lists), 16 otherwise
    uint32_t u = 16;
    while (u > 1 && ceil_div(d.total, 256ull * u) < 512) u >>= 1;
    const uint64_t chunks = ceil_div(d.total, 256ull * u);
    const unsigned bgrid = (unsigned)(chunks < DN_BUILD_BLOCKS ? chunks : DN_BUILD_BLOCKS);
    switch (u) {
    case 16: dn_build_kernel<16><<<bgrid, 256, 0, st>>>(d); break;
    case 8: dn_build_kernel<8><<<bgrid, 256, 0, st>>>(d); break;
    case 4: dn_build_kernel<4><<<bgrid, 256, 0, st>>>(d); break;
    case 2: dn_build_kernel<2><<<bgrid, 256, 0, st>>>(d); break;
    default: dn_build_kernel<1><<<bgrid, 256, 0, st>>>(d); break;
    }
    SG_TRY_LAUNCH();
    uint64_t W = ceil_div(d.words, SG_WAVE);
    if (W > DN_MAX_WAVES) W = DN_MAX_WAVES;
    d.wpw = ceil_div(ceil_div(d.words, W), SG_WAVE) * SG_WAVE;
    const unsigned grid = (unsigned)ceil_div(ceil_div(d.words, d.wpw), 4);
    const bool hashed = d.planes != nullptr;
    if (d.n <= 8) {
        if (hashed) dn_count_kernel<8, true><<<grid, 256, 0, st>>>(d);
        else dn_count_kernel<8, false><<<grid, 256, 0, st>>>(d);
    } else {
        if (hashed) dn_count_kernel<16, true><<<grid, 256, 0, st>>>(d);
        else dn_count_kernel<16, false><<<grid, 256, 0, st>>>(d);
    }
    SG_TRY_LAUNCH();
    MergeParams q = p;
    q.st_part = d.rows;
    q.st_row = d.st_row;
    mg_stats_reduce_kernel<<<d.st_row, 256, 0, st>>>(q, grid * 4, out);
    SG_TRY_LAUNCH();
    return SG_OK;
}

// Def. 5 on one set J: max over parts of (c_i M) / (g_i |J|); 0 if J is empty.
static double skew_of(const uint64_t* c, const uint64_t* g, uint32_t P, uint64_t M, uint64_t J)
{
    double best = 0.0;
    if (J == 0) return 0.0;
    for (uint32_t i = 0; i < P; ++i) {
        if (g[i] == 0) continue;
        const double s = ((double)c[i] * (double)M) / ((double)g[i] * (double)J);
        if (s > best) best = s;
    }
    return best;
}

// The block of raw counts the host evaluates: see StatsCounts.
static uint64_t stats_block_words(uint32_t n, uint32_t P)
{
    return (uint64_t)n * (n + 1) / 2 + 1 + 2ull * P + 2ull * n * P + n + 1 + P + 4;
}

static int stats_check_out(const sg_stats_out* o, bool hashed)
{
    if (!o || !o->nnz || !o->inter || !o->overlap || !o->contig_counts || !o->skew_contig) return SG_EINVAL;
    if (hashed && (!o->class_size || !o->hashed_counts || !o->skew_hashed)) return SG_EINVAL;
    return SG_OK;
}

// Validation and every pass on `stream`; on return *d_block is the device
// block of raw counts (stats_block_words long), complete once the stream
// passes this point.
static int stats_enqueue(const uint32_t* d_idx, const uint64_t* d_in_off, uint32_t n, uint64_t M, uint64_t total,
                         uint32_t P, const void* d_cmap, size_t cmap_bytes, void* d_ws, size_t ws_bytes, hipStream_t st,
                         const uint64_t** d_block)
{
    if (n == 0 || n > 64 || P == 0 || P > 256 || !d_in_off || !d_ws) return SG_EINVAL;
    if (M == 0 || M >= (1ull << 32) || total >= (1ull << 32)) return SG_EUNSUPPORTED;
    if (total > 0 && !d_idx) return SG_EINVAL;
    if (ws_bytes < sg_stats_workspace_bytes(n, M, total, P)) return SG_ECAPACITY;

    // The class map's header (seed, and its magic, P and M, checked after the
    // passes) and class sizes are read on the device: no copy before the
    // kernels.  Its layout follows from (M, P) alone, so a wrong map cannot
    // send a read out of the cmap_bytes checked here.
    CmapPtrs cm{};
    if (d_cmap) {
        const CmapLayout L = cmap_layout(M, P);
        if (cmap_bytes < L.bytes) return SG_ECAPACITY;
        cm = cmap_ptrs(const_cast<void*>(d_cmap), L);
    }

    const bool dense = stats_dense(n, M, total, P);
    const bool windowed = !dense && total > 0 && stats_windowed(n, P, d_cmap != nullptr);
    MergeParams p;
    stats_setup(&p, n, M, total, P, windowed);
    Carver c(d_ws);
    StatsCounts k;
    SwParams sw;
    DnParams dn;
    stats_carve(c, &p, P, &k, windowed ? &sw : nullptr, dense ? &dn : nullptr);
    p.idx = d_idx;
    p.off = d_in_off;
    p.seed = 0;
    p.seed_at = d_cmap ? &cm.hdr->seed : nullptr;
    p.hashed = d_cmap != nullptr;
    p.div = make_divider(P);
    // per-worker part counters are accumulated with atomics: zero them
    int rc = fill_u64(k.wcontig, 2ull * n * P, 0, st); // wcontig and whashed are adjacent
    if (rc) return rc;
    if (dense) {
        dn.idx = d_idx;
        dn.in_off = d_in_off;
        dn.total = total;
        dn.M = M;
        dn.n = n;
        dn.P = P;
        dn.inv_m = p.inv_m;
        dn.planes = nullptr;
        dn.nbits = 0;
        dn.stride = 0;
        if (d_cmap && P >= 2) { // P = 1: every key is in class 0 (the union's count, below)
            const CmapLayout L = cmap_layout(M, P);
            dn.planes = cmap_ptrs(const_cast<void*>(d_cmap), L).planes;
            dn.nbits = L.nbits;
            dn.stride = L.stride;
        }
        dn.seed_at = p.seed_at;
        dn.classes = d_cmap != nullptr;
        dn.div = p.div;
        dn.whashed = k.whashed;
        dn.npairs = p.npairs;
        rc = stats_dense_run(p, dn, st, k.row);
    } else if (windowed) {
        sw.planes = nullptr;
        sw.nbits = 0;
        sw.stride = 0;
        if (d_cmap && P >= 2) { // P = 1: every key is in class 0 (the union's count, below)
            const CmapLayout L = cmap_layout(M, P);
            sw.planes = cmap_ptrs(const_cast<void*>(d_cmap), L).planes;
            sw.nbits = L.nbits;
            sw.stride = L.stride;
        }
        rc = stats_window_run(p, sw, st, k.row);
    } else {
        rc = merge_run(p, MODE_STATS, st, k.row);
    }
    if (rc) return rc;
    if (!dense) {
        st_contig_kernel<<<(unsigned)ceil_div((uint64_t)n * P, 4), 256, 0, st>>>(p, k);
        SG_TRY_LAUNCH();
    }
    if (!dense && d_cmap && total > 0) {
        st_entries_kernel<<<p.nchunks_max < 65536 ? p.nchunks_max : 65536, MG_THREADS, 0, st>>>(p, k);
        SG_TRY_LAUNCH();
    }

    st_pack_kernel<<<1, 256, 0, st>>>(d_in_off, n, d_cmap ? cm.class_size : nullptr, d_cmap ? cm.hdr : nullptr, P,
                                      k.tail);
    SG_TRY_LAUNCH();

    *d_block = k.row;
    return SG_OK;
}

// The definitions evaluated on the host from a block of raw counts.
static int stats_collect(const uint64_t* blk, uint32_t n, uint64_t M, uint64_t total, uint32_t P, bool hashed,
                         sg_stats_out* o)
{
    const bool windowed = total > 0 && stats_windowed(n, P, hashed);
    const uint32_t npairs = n * (n + 1) / 2;
    const uint32_t st_row = npairs + 1 + 2 * P;
    std::vector<uint64_t> rowv(blk, blk + st_row);
    uint64_t* row = rowv.data();
    const uint64_t* wc = blk + st_row;
    const uint64_t* wh = wc + (size_t)n * P;
    const uint64_t* off = wh + (size_t)n * P;
    const uint64_t* class_size = off + n + 1;
    const uint64_t* hdr = class_size + P;
    if (hashed && (hdr[0] != CM_MAGIC || hdr[1] != P || hdr[2] != M)) return SG_EINVAL;
    std::vector<uint64_t> inter((size_t)n * n, 0);
    for (uint32_t a = 0, pi = 0; a < n; ++a)
        for (uint32_t b = a; b < n; ++b, ++pi) inter[(size_t)a * n + b] = row[pi];
    const uint64_t uni = row[npairs];
    if (windowed && hashed && P == 1) row[npairs + 1 + P] = uni; // one class holds every key
    const uint64_t* uc = &row[npairs + 1];
    const uint64_t* uh = &row[npairs + 1 + P];

    // exact counts
    o->sum_nnz = 0;
    o->max_nnz = 0;
    for (uint32_t a = 0; a < n; ++a) {
        uint64_t x = off[a] > total ? total : off[a], y = off[a + 1] > total ? total : off[a + 1];
        o->nnz[a] = y > x ? y - x : 0;
        o->sum_nnz += o->nnz[a];
        if (o->nnz[a] > o->max_nnz) o->max_nnz = o->nnz[a];
    }
    o->union_size = uni;
    if (windowed) // the window pass leaves the diagonal to the list lengths: |I_a & I_a| = |I_a|
        for (uint32_t a = 0; a < n; ++a) inter[(size_t)a * n + a] = o->nnz[a];
    for (uint32_t a = 0; a < n; ++a)
        for (uint32_t b = 0; b < n; ++b) o->inter[(uint64_t)a * n + b] = a <= b ? inter[(size_t)a * n + b] : inter[(size_t)b * n + a];
    // Def. 3 over all pairs
    uint64_t npo = 0; // pairs a < b seen
    double sum_ov = 0.0;
    o->overlap_min = 0.0;
    o->overlap_max = 0.0;
    for (uint32_t a = 0; a < n; ++a)
        for (uint32_t b = 0; b < n; ++b) {
            const uint64_t mn = o->nnz[a] < o->nnz[b] ? o->nnz[a] : o->nnz[b];
            const double ov = mn ? (double)o->inter[(uint64_t)a * n + b] / (double)mn : 0.0;
            o->overlap[(uint64_t)a * n + b] = ov;
            if (a < b) {
                if (npo == 0 || ov < o->overlap_min) o->overlap_min = ov;
                if (npo == 0 || ov > o->overlap_max) o->overlap_max = ov;
                sum_ov += ov;
                ++npo;
            }
        }
    o->overlap_mean = npo ? sum_ov / (double)npo : 0.0;
    // Def. 4
    o->gamma_n = o->sum_nnz ? ((double)n * (double)o->union_size) / (double)o->sum_nnz : 0.0;
    // Def. 5, contiguous parts
    std::vector<uint64_t> g(P);
    for (uint32_t i = 0; i < P; ++i)
        g[i] = (uint64_t)(((unsigned __int128)M * (i + 1)) / P) - (uint64_t)(((unsigned __int128)M * i) / P);
    for (uint32_t a = 0; a < n; ++a) {
        for (uint32_t i = 0; i < P; ++i) o->contig_counts[(uint64_t)a * P + i] = wc[(size_t)a * P + i];
        o->skew_contig[a] = skew_of(&wc[(size_t)a * P], g.data(), P, M, o->nnz[a]);
    }
    for (uint32_t i = 0; i < P; ++i) o->contig_counts[(uint64_t)n * P + i] = uc[i];
    o->skew_contig[n] = skew_of(uc, g.data(), P, M, o->union_size);
    // hash classes and Def. 8
    o->push_imbalance = 0.0;
    o->pull_imbalance = 0.0;
    if (hashed) {
        for (uint32_t i = 0; i < P; ++i) o->class_size[i] = class_size[i];
        for (uint32_t a = 0; a < n; ++a) {
            for (uint32_t i = 0; i < P; ++i) o->hashed_counts[(uint64_t)a * P + i] = wh[(size_t)a * P + i];
            o->skew_hashed[a] = skew_of(&wh[(size_t)a * P], class_size, P, M, o->nnz[a]);
        }
        for (uint32_t i = 0; i < P; ++i) o->hashed_counts[(uint64_t)n * P + i] = uh[i];
        o->skew_hashed[n] = skew_of(uh, class_size, P, M, o->union_size);
        for (uint32_t a = 0; a < n; ++a) {
            if (o->nnz[a] == 0) continue;
            for (uint32_t i = 0; i < P; ++i) {
                const double v = ((double)P * (double)wh[(size_t)a * P + i]) / (double)o->nnz[a];
                if (v > o->push_imbalance) o->push_imbalance = v;
            }
        }
        if (o->union_size)
            for (uint32_t i = 0; i < P; ++i) {
                const double v = ((double)P * (double)uh[i]) / (double)o->union_size;
                if (v > o->pull_imbalance) o->pull_imbalance = v;
            }
    }
    return SG_OK;
}

extern "C" size_t sg_stats_block_bytes(uint32_t n, uint32_t P)
{
    if (n == 0 || n > 64 || P == 0 || P > 256) return 0;
    return (size_t)(8 * stats_block_words(n, P));
}

extern "C" int sg_stats(const uint32_t* d_idx, const uint64_t* d_in_off, uint32_t n, uint64_t M, uint64_t total,
                        uint32_t P, const void* d_cmap, size_t cmap_bytes, sg_stats_out* o, void* d_ws,
                        size_t ws_bytes, void* stream)
{
    int rc = stats_check_out(o, d_cmap != nullptr);
    if (rc) return rc;
    hipStream_t st = as_stream(stream);
    const uint64_t* d_block = nullptr;
    rc = stats_enqueue(d_idx, d_in_off, n, M, total, P, d_cmap, cmap_bytes, d_ws, ws_bytes, st, &d_block);
    if (rc) return rc;
    const uint64_t words = stats_block_words(n, P);
    std::vector<uint64_t> blk(words);
    {
        HostStage hs;
        rc = host_stage(8ull * words, &hs);
        if (rc) return rc;
        SG_TRY(hipMemcpyAsync(hs.ptr, d_block, 8ull * words, hipMemcpyDeviceToHost, st));
        SG_TRY(hipStreamSynchronize(st));
        std::memcpy(blk.data(), hs.ptr, 8ull * words);
    }
    return stats_collect(blk.data(), n, M, total, P, d_cmap != nullptr, o);
}

extern "C" int sg_stats_async(const uint32_t* d_idx, const uint64_t* d_in_off, uint32_t n, uint64_t M, uint64_t total,
                              uint32_t P, const void* d_cmap, size_t cmap_bytes, void* h_block, size_t block_bytes,
                              void* d_ws, size_t ws_bytes, void* stream)
{
    if (!h_block) return SG_EINVAL;
    if (block_bytes < sg_stats_block_bytes(n, P)) return SG_ECAPACITY;
    hipStream_t st = as_stream(stream);
    const uint64_t* d_block = nullptr;
    const int rc = stats_enqueue(d_idx, d_in_off, n, M, total, P, d_cmap, cmap_bytes, d_ws, ws_bytes, st, &d_block);
    if (rc) return rc;
    SG_TRY(hipMemcpyAsync(h_block, d_block, sg_stats_block_bytes(n, P), hipMemcpyDeviceToHost, st));
    return SG_OK;
}

extern "C" int sg_stats_collect(const void* h_block, uint32_t n, uint64_t M, uint64_t total, uint32_t P, int hashed,
                                sg_stats_out* o)
{
    if (!h_block || n == 0 || n > 64 || P == 0 || P > 256) return SG_EINVAL;
    if (M == 0 || M >= (1ull << 32) || total >= (1ull << 32)) return SG_EUNSUPPORTED;
    const int rc = stats_check_out(o, hashed != 0);
    if (rc) return rc;
    return stats_collect(static_cast<const uint64_t*>(h_block), n, M, total, P, hashed != 0, o);
}

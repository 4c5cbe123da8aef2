// sg_aggregate.hip -- A3 entry point: per-partition union-sum of n workers'
// partitioned COO tensors (the server side of Push in Zen OSDI'25 digest,
// section 3.1; equal to the dense AllReduce of the same gradients, section
// 3.2).  The work is done by the merge engine in sg_merge.hip.
#include "sg_host.h"

namespace sg {

constexpr uint32_t MG_STATS_MAX_GRID = 2048; // persistent blocks of the statistics pass, at most

// Tile width 2^tb so that a (group, tile) holds MG_TARGET to 2*MG_TARGET
// entries on average, within [2^5, 2^MG_SPAN_LOG] keys.
static void choose_tiles(uint32_t G, uint64_t M, uint64_t total, uint32_t* tb, uint32_t* NT)
{
    uint32_t b = MG_SPAN_LOG;
    if (total > 0) {
        const double want = (double)MG_TARGET * (double)G * (double)M / (double)total;
        b = 0;
        while (b < 63 && (double)(1ull << (b + 1)) <= want) ++b;
        ++b; // 2^b > want
        if (b < 5) b = 5;
        if (b > MG_SPAN_LOG) b = MG_SPAN_LOG;
    }
    *tb = b;
    uint64_t nt = (M + (1ull << b) - 1) >> b;
    *NT = (uint32_t)(nt ? nt : 1);
}

static uint64_t merge_carve(Carver& c, MergeParams* p, int mode)
{
    const uint64_t R = (uint64_t)p->n * p->G;
    const uint64_t T = (uint64_t)p->G * p->NT;
    p->nscan = (uint32_t)ceil_div(T, MG_SCAN_BLOCK);
    p->chunk_start = c.take<uint32_t>(R + 1);
    p->nchunks_max = (uint32_t)(ceil_div(p->total, MG_CHUNK) + R);
    p->chunk_rec = c.take<uint4>(p->nchunks_max);
    p->bnd = c.take<uint32_t>(R * (p->NT + 1));
    p->nqsets = 1;
    p->queue = c.take<uint32_t>((uint64_t)MG_NQ * MG_QSTRIDE);
    p->heavy = c.take<uint32_t>(T);
    if (mode == MODE_AGG) {
        p->tile_cnt = c.take<uint32_t>(T);
        p->tile_sb = c.take<uint64_t>(T);
        p->tile_out = c.take<uint64_t>(T);
        p->blk_sum = c.take<uint64_t>(p->nscan);
        p->stage_idx = c.take<uint32_t>(p->total);
        if (p->D > 1) {
            p->stage_val = nullptr;
            p->stage_src = c.take<uint32_t>(p->total);
            p->stage_first = c.take<uint32_t>(p->total);
            p->tile_ent = c.take<uint32_t>(T);
            p->row_rng = c.take<uint2>(p->total);
        } else {
            p->stage_val = c.take<float>(p->total);
        }
    } else {
        p->st_part = c.take<uint64_t>((uint64_t)MG_STATS_MAX_GRID * p->st_row);
    }
    return c.bytes();
}

// Scalar values and bare indices (D <= 1): tiles of 2^tb keys holding about
// UN_TARGET entries on average (2^tb the power of two nearest to the span
// that holds that many), within [2^5, 2^UN_SPAN_LOG_MAX] keys.
constexpr uint64_t UN_MIN_TILES = 2048;

static void union_tiles(uint32_t G, uint64_t M, uint64_t total, uint32_t* tb, uint32_t* NT)
{
    uint32_t b = UN_SPAN_LOG_MAX;
    if (total > 0) {
        const double want = (double)UN_TARGET * (double)G * (double)M / (double)total;
        b = 0;
        while (b < 63 && (double)(1ull << (b + 1)) <= want) ++b; // 2^b <= want < 2^(b+1)
        if (want >= 1.4142135623730951 * (double)(1ull << b)) ++b;
        if (b < 5) b = 5;
        if (b > UN_SPAN_LOG_MAX) b = UN_SPAN_LOG_MAX;
        // small inputs: enough tiles for every SIMD of the chip to take one
        // or two, rather than a few long tiles
        while (b > 5 && (uint64_t)G * ((M + (1ull << b) - 1) >> b) < UN_MIN_TILES) --b;
    }
    *tb = b;
    uint64_t nt = (M + (1ull << b) - 1) >> b;
    *NT = (uint32_t)(nt ? nt : 1);
}

// bitmap words per lane of the union passes for tiles of 2^tb keys (64 lanes
// of 32-bit words; spans below 2^11 keys leave words unused)
static int union_wpl(uint32_t tb) { return tb <= 11 ? 1 : 1 << (tb - 11); }

static uint64_t union_carve(Carver& c, MergeParams* p)
{
    const uint64_t R = (uint64_t)p->n * p->G;
    const uint64_t T = (uint64_t)p->G * p->NT;
    p->nscan = (uint32_t)ceil_div(T, MG_SCAN_BLOCK);
    p->chunk_start = c.take<uint32_t>(R + 1);
    p->nchunks_max = (uint32_t)(ceil_div(p->total, MG_CHUNK) + R);
    p->chunk_rec = c.take<uint4>(p->nchunks_max);
    p->bnd = c.take<uint32_t>(R * (p->NT + 1));
    p->nqsets = 1;
    p->queue = c.take<uint32_t>((uint64_t)MG_NQ * MG_QSTRIDE); // zeroed by the plan kernel, unused
    p->tile_cnt = c.take<uint32_t>(T);
    p->tile_out = c.take<uint64_t>(T);
    p->blk_sum = c.take<uint64_t>(p->nscan);
    return c.bytes();
}

// blocks of a union pass: as many as can be resident, no more than the tiles
// need (UN_WPB tiles per block at once)
static int union_blocks(const void* kernel, uint64_t T, unsigned* blocks)
{
    int resident = 0;
    if (resident_blocks(kernel, UN_THREADS, 1 << 30, &resident) != SG_OK) return SG_EHIP;
    uint64_t b = ceil_div(T, UN_WPB);
    if (b > (uint64_t)resident) b = (uint64_t)resident;
    *blocks = (unsigned)(b ? b : 1);
    return SG_OK;
}

template <int WPL>
static int union_launch(MergeParams& p, hipStream_t st)
{
    const uint64_t T = (uint64_t)p.G * p.NT;
    const void* wk = p.D == 0  ? (const void*)un_write_kernel<WPL, VM_NONE>
                     : p.bf16 ? (const void*)un_write_kernel<WPL, VM_BF16>
                              : (const void*)un_write_kernel<WPL, VM_F32>;
    unsigned cb = 0, wb = 0;
    if (union_blocks((const void*)un_count_kernel<WPL>, T, &cb) != SG_OK) return SG_EHIP;
    if (union_blocks(wk, T, &wb) != SG_OK) return SG_EHIP;
    probe_begin(SG_PROBE_AGGREGATE_COUNT, st);
    un_count_kernel<WPL><<<cb, UN_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_AGGREGATE_COUNT, st);
    mg_scan_local_kernel<<<p.nscan, 1024, 0, st>>>(p);
    SG_TRY_LAUNCH();
    mg_scan_top_kernel<<<1, 1024, 0, st>>>(p); // agg_off[G]
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_AGGREGATE_MERGE, st);
    if (p.D == 0) un_write_kernel<WPL, VM_NONE><<<wb, UN_THREADS, 0, st>>>(p);
    else if (p.bf16) un_write_kernel<WPL, VM_BF16><<<wb, UN_THREADS, 0, st>>>(p);
    else un_write_kernel<WPL, VM_F32><<<wb, UN_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_AGGREGATE_MERGE, st);
    return SG_OK;
}

// Plan and boundaries of the merge engine, then the count pass, the scan of
// the tiles' union sizes and the write pass.
static int union_run(MergeParams& p, hipStream_t st)
{
    if (p.total == 0) return fill_u64(p.agg_off, (uint64_t)p.G + 1, 0ull, st);
    mg_plan_kernel<<<1, 512, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_AGGREGATE_BND, st);
    mg_bnd_kernel<<<p.nchunks_max < 65536 ? p.nchunks_max : 65536, 512, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_AGGREGATE_BND, st);
    switch (union_wpl(p.tb)) {
    case 1: return union_launch<1>(p, st);
    case 2: return union_launch<2>(p, st);
    case 4: return union_launch<4>(p, st);
    case 8: return union_launch<8>(p, st);
    case 16: return union_launch<16>(p, st);
    default: return union_launch<32>(p, st);
    }
}

// Queue the engine: plan, boundaries, merge (and, for the aggregate, the
// scan and placement).  `stats_out` receives the reduced statistics row.
static int merge_run(MergeParams& p, int mode, hipStream_t st, uint64_t* stats_out)
{
    const uint64_t R = (uint64_t)p.n * p.G;
    const uint64_t T = (uint64_t)p.G * p.NT;
    mg_plan_kernel<<<1, 512, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_AGGREGATE_BND, st);
    mg_bnd_kernel<<<p.nchunks_max < 65536 ? p.nchunks_max : 65536, 512, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_AGGREGATE_BND, st);
    mg_heavy_kernel<<<(unsigned)(ceil_div(T, 256) < 1024 ? ceil_div(T, 256) : 1024), 256, 0, st>>>(p);
    SG_TRY_LAUNCH();
    // persistent blocks: as many as can be resident at once
    int resident = 0;
    if (mode == MODE_AGG) {
        if (resident_blocks((const void*)mg_merge_kernel<MODE_AGG>, MG_THREADS, 1 << 30, &resident) != SG_OK)
            return SG_EHIP;
    } else if (resident_blocks((const void*)mg_merge_kernel<MODE_STATS>, MG_THREADS, 1 << 30, &resident) != SG_OK) {
        return SG_EHIP;
    }
    const uint64_t wblocks = ceil_div(T, MG_WAVES);
    uint64_t grid = wblocks < (uint64_t)resident ? wblocks : (uint64_t)resident;
    if (mode == MODE_STATS && grid > MG_STATS_MAX_GRID) grid = MG_STATS_MAX_GRID;
    if (grid == 0) grid = 1;
    if (mode == MODE_AGG) {
        probe_begin(SG_PROBE_AGGREGATE_MERGE, st);
        mg_merge_kernel<MODE_AGG><<<(unsigned)grid, MG_THREADS, 0, st>>>(p);
        SG_TRY_LAUNCH();
        probe_end(SG_PROBE_AGGREGATE_MERGE, st);
        mg_scan_local_kernel<<<p.nscan, 1024, 0, st>>>(p);
        SG_TRY_LAUNCH();
        mg_scan_top_kernel<<<1, 1024, 0, st>>>(p);
        SG_TRY_LAUNCH();
        const uint64_t pwaves = ceil_div(T, MG_PLACE_TILES);
        const uint64_t pblocks = ceil_div(pwaves, 4) < 65536 ? ceil_div(pwaves, 4) : 65536;
        mg_place_kernel<<<(unsigned)pblocks, 256, 0, st>>>(p);
        SG_TRY_LAUNCH();
        if (p.D > 1 && p.total > 0) {
            const uint64_t rblocks = ceil_div(p.total, 4) < 65536 ? ceil_div(p.total, 4) : 65536;
            mg_rows_kernel<<<(unsigned)rblocks, 256, 0, st>>>(p);
            SG_TRY_LAUNCH();
        }
        return SG_OK;
    }
    mg_merge_kernel<MODE_STATS><<<(unsigned)grid, MG_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    mg_stats_reduce_kernel<<<p.st_row, 256, 0, st>>>(p, (uint32_t)grid, stats_out);
    SG_TRY_LAUNCH();
    return SG_OK;
}

} // namespace sg

using namespace sg;

static void agg_setup(MergeParams* p, uint32_t n, uint32_t P, uint64_t M, uint64_t total, uint32_t D)
{
    *p = MergeParams();
    p->n = n;
    p->G = P;
    p->stride = P + 1;
    p->M = M;
    p->total = total;
    p->D = D;
    if (D <= 1) union_tiles(P, M, total, &p->tb, &p->NT);
    else choose_tiles(P, M, total, &p->tb, &p->NT);
}

extern "C" size_t sg_aggregate_workspace_bytes(uint32_t n, uint32_t P, uint64_t M, uint64_t total, uint32_t D)
{
    if (n == 0 || P == 0) return 256;
    MergeParams p;
    agg_setup(&p, n, P, M, total, D);
    Carver c(nullptr);
    return D <= 1 ? union_carve(c, &p) : merge_carve(c, &p, MODE_AGG);
}

extern "C" int sg_aggregate(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D,
                            const uint64_t* d_part_off, uint32_t n, uint32_t P, uint64_t M, uint64_t total,
                            uint32_t* d_agg_idx, float* d_agg_val, uint64_t capacity, uint64_t* d_agg_off,
                            void* d_ws, size_t ws_bytes, void* stream)
{
    if (n == 0 || n > 64 || P == 0 || P > 256 || D > 65536 || (dt != SG_F32 && dt != SG_BF16)) return SG_EINVAL;
    if (M == 0 || M >= (1ull << 32) || total >= (1ull << 32)) return SG_EUNSUPPORTED;
    if (!d_part_off || !d_agg_off || !d_ws) return SG_EINVAL;
    if (total > 0 && (!d_idx || !d_agg_idx)) return SG_EINVAL;
    if (D > 0 && total > 0 && (!d_val || !d_agg_val)) return SG_EINVAL;
    if (capacity < total) return SG_ECAPACITY;
    if (ws_bytes < sg_aggregate_workspace_bytes(n, P, M, total, D)) return SG_ECAPACITY;

    MergeParams p;
    agg_setup(&p, n, P, M, total, D);
    Carver c(d_ws);
    if (D <= 1) union_carve(c, &p);
    else merge_carve(c, &p, MODE_AGG);
    p.idx = d_idx;
    p.off = d_part_off;
    p.val = d_val;
    p.bf16 = dt == SG_BF16;
    p.agg_idx = d_agg_idx;
    p.agg_val = d_agg_val;
    p.agg_off = d_agg_off;
    p.capacity = capacity;
    p.div = make_divider(P);
    if (D <= 1) return union_run(p, as_stream(stream));
    return merge_run(p, MODE_AGG, as_stream(stream), nullptr);
}

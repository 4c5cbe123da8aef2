// sg_aggregate.hip -- A3 entry point: per-partition union-sum of n workers'
// partitioned COO tensors (the server side of Push in Zen OSDI'25 digest,
// section 3.1; equal to the dense AllReduce of the same gradients, section
// 3.2).  The work is done by the merge engine in sg_merge.hip.
#include "sg_host.h"

namespace sg {

// Bucket width 2^bs so that a (group, bucket) holds about MG_TARGET/2 entries
// on average, with the boundary table n*G*(NB+1) words kept under 16M entries.
static void choose_buckets(uint32_t n, uint32_t G, uint64_t M, uint64_t total, uint32_t* bs, uint32_t* NB)
{
    const double want = total > 0 ? (double)(MG_TARGET / 2) * (double)M * (double)G / (double)total : (double)M;
    uint32_t b = 0;
    while (b < MG_SPAN_LOG && (double)(1ull << (b + 1)) <= want) ++b;
    for (;;) {
        uint64_t nb = (M + (1ull << b) - 1) >> b;
        if (nb == 0) nb = 1;
        // a bucket never spans more keys than a tile may
        if ((uint64_t)n * G * (nb + 1) <= (16ull << 20) || b >= MG_SPAN_LOG) {
            *bs = b;
            *NB = (uint32_t)nb;
            return;
        }
        ++b;
    }
}

static void merge_sizes(MergeParams* p)
{
    const uint64_t splits = 4 * ceil_div(p->total, MG_TARGET);
    p->tcap = (uint32_t)(p->NB + splits + 2);
    p->max_tiles = (uint32_t)((uint64_t)p->G * p->NB + splits + p->G);
    p->max_rows = p->max_tiles + p->G;
}

static uint64_t merge_carve(Carver& c, MergeParams* p)
{
    merge_sizes(p);
    const uint64_t R = (uint64_t)p->n * p->G;
    p->chunk_start = c.take<uint32_t>(R + 1);
    p->bnd = c.take<uint32_t>(R * (p->NB + 1));
    p->tile_key = c.take<uint64_t>((uint64_t)p->G * p->tcap);
    p->ntiles = c.take<uint32_t>(p->G);
    p->tile_prefix = c.take<uint32_t>((uint64_t)p->G + 1);
    p->tile_pos = c.take<uint32_t>((uint64_t)p->max_rows * p->n);
    p->tile_group = c.take<uint32_t>(p->max_tiles);
    p->tile_lo = c.take<uint64_t>(p->max_tiles);
    p->tile_hi = c.take<uint64_t>(p->max_tiles);
    p->status = c.take<uint64_t>(p->max_tiles);
    p->ticket = c.take<uint32_t>(1);
    return c.bytes();
}

// Queue the engine: plan, boundaries, tiles, merge.
static int merge_run(MergeParams& p, int mode, hipStream_t st)
{
    const uint64_t R = (uint64_t)p.n * p.G;
    merge_sizes(&p);
    mg_plan_kernel<<<1, MG_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    const uint64_t nchunks = ceil_div(p.total, MG_CHUNK) + R;
    probe_begin(SG_PROBE_AGGREGATE_BND, st);
    mg_bnd_kernel<<<(unsigned)nchunks, MG_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_AGGREGATE_BND, st);
    const uint64_t cells = R * (p.NB + 1);
    mg_bnd_empty_kernel<<<(unsigned)(ceil_div(cells, 256) < 2048 ? ceil_div(cells, 256) : 2048), 256, 0, st>>>(p);
    SG_TRY_LAUNCH();
    mg_tiles_kernel<<<p.G, 1024, 0, st>>>(p);
    SG_TRY_LAUNCH();
    mg_tile_prefix_kernel<<<1, MG_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    mg_refine_kernel<<<p.max_rows < 4096u ? p.max_rows : 4096u, MG_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    if (mode == MODE_AGG) {
        int rc = fill_u64(p.status, p.max_tiles, 0, st);
        if (rc) return rc;
    }
    // persistent grid: as many blocks as can be resident at once
    static int resident[2] = {0, 0};
    if (!resident[mode]) {
        int dev = 0, cus = 0, per = 0;
        SG_TRY(hipGetDevice(&dev));
        SG_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
        if (mode == MODE_AGG)
            SG_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, mg_merge_kernel<MODE_AGG>, MG_THREADS, 0));
        else
            SG_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, mg_merge_kernel<MODE_STATS>, MG_THREADS, 0));
        resident[mode] = (per > 0 ? per : 1) * (cus > 0 ? cus : 1);
    }
    const unsigned grid = p.max_tiles < (uint32_t)resident[mode] ? p.max_tiles : (unsigned)resident[mode];
    probe_begin((mode == MODE_AGG ? SG_PROBE_AGGREGATE_MERGE : -1), st);
    if (mode == MODE_AGG) mg_merge_kernel<MODE_AGG><<<grid, MG_THREADS, 0, st>>>(p);
    else mg_merge_kernel<MODE_STATS><<<grid, MG_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end((mode == MODE_AGG ? SG_PROBE_AGGREGATE_MERGE : -1), st);
    return SG_OK;
}

} // namespace sg

using namespace sg;

static void agg_setup(MergeParams* p, uint32_t n, uint32_t P, uint64_t M, uint64_t total)
{
    *p = MergeParams();
    p->n = n;
    p->G = P;
    p->stride = P + 1;
    p->M = M;
    p->total = total;
    choose_buckets(n, P, M, total, &p->bs, &p->NB);
}

extern "C" size_t sg_aggregate_workspace_bytes(uint32_t n, uint32_t P, uint64_t M, uint64_t total, uint32_t D)
{
    (void)D;
    if (n == 0 || P == 0) return 256;
    MergeParams p;
    agg_setup(&p, n, P, M, total);
    Carver c(nullptr);
    return merge_carve(c, &p);
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
    agg_setup(&p, n, P, M, total);
    Carver c(d_ws);
    merge_carve(c, &p);
    p.idx = d_idx;
    p.off = d_part_off;
    p.val = d_val;
    p.D = D;
    p.bf16 = dt == SG_BF16;
    p.agg_idx = d_agg_idx;
    p.agg_val = d_agg_val;
    p.agg_off = d_agg_off;
    p.capacity = capacity;
    p.div = make_divider(P);
    return merge_run(p, MODE_AGG, as_stream(stream));
}

// sg_dgc.hip -- DGC-style top-k with a sampled global threshold and residual
// accumulation, for n workers resident on one GPU.
//
// Zen OSDI'25 digest, section 4 (Implementation): DGC adapted to tensor
// parallelism -- each device samples its gradient locally, the samples of all
// devices are gathered, one global top-k threshold is computed from them and
// applied locally by every device.  SkipReduce MICRO'25 digest, section 2:
// gradients that are not selected accumulate locally into the next
// iterations' gradients until they are large enough to be selected.
//
// One call is one iteration for all n workers:
//   sample  a = resid + grad at S strided positions per worker; the pool of
//           n*S magnitude keys (fp32 bits without the sign);
//   select  the ceil(density * n*S)-th largest key of the pool, by MSD radix
//           select (11-bit digits: a chip-wide histogram pass, then a one-block
//           pick, three times);
//   filter  one streaming pass over grad and resid: a = resid + grad, the new
//           residual (0 where |a| >= threshold, a elsewhere) written back in
//           place, and the selected (index, a) compacted per 1024-element tile
//           in index order (one wave per tile, ballots, no atomics);
//   write   the top-k write path: per-tile counts, per-worker scan, ordered
//           copy of the tiles' entries into idx[w][*], val[w][*].
#include "sg_host.h"

namespace sg {

constexpr int DG_HIST_BLOCKS = 512;

struct DgcState {
    uint32_t rank;    // rank (1-based, from the largest) still to find among keys with the prefix
    uint32_t prefix;  // fixed high bits of the threshold key
    uint32_t thr;     // the threshold key once found
    uint32_t pad;
};

struct DgcParams {
    const float* grad;
    float* resid;
    uint32_t* samples;  // [n*S]
    uint32_t* hist;     // [TK_BINS]
    DgcState* ds;
    uint32_t* thr_out;  // caller's threshold word, or null
    uint64_t* count;    // [n]
    TopkParams t;       // tiles, slots and the ordered write of the top-k path
    uint64_t M, S, Ns;
    uint32_t n, ks;
};

// Sample j of worker w: position floor((2j + 1) M / (2S)) (every position
// when S == M), key of a = resid + grad there.
__global__ __launch_bounds__(256) void dgc_sample_kernel(DgcParams p)
{
    const bool fits = p.M <= ~0ull / (2 * p.S); // (2j + 1) M fits 64 bits
    for (uint64_t q = (uint64_t)blockIdx.x * 256 + threadIdx.x; q < p.Ns; q += (uint64_t)gridDim.x * 256) {
        const uint32_t w = (uint32_t)(q / p.S);
        const uint64_t j = q % p.S;
        const uint64_t pos = p.S >= p.M ? j
                             : fits   ? ((2 * j + 1) * p.M) / (2 * p.S)
                                      : (uint64_t)(((unsigned __int128)(2 * j + 1) * p.M) / (2 * p.S));
        const uint64_t e = (uint64_t)w * p.M + pos;
        const float a = p.resid[e] + p.grad[e];
        p.samples[q] = __float_as_uint(a) & 0x7fffffffu;
    }
}

// Digit d (0: bits 30..20, 1: 19..9, 2: 8..0) of a key, and the shift of the
// bits above it.
__device__ __forceinline__ uint32_t dg_shift(int d) { return d == 0 ? 20u : (d == 1 ? 9u : 0u); }
__device__ __forceinline__ uint32_t dg_mask(int d) { return d == 2 ? 0x1ffu : 0x7ffu; }

// Histogram of digit d over the pooled keys whose higher digits equal the
// prefix found so far (LDS per block, one global add per non-empty bin).
__global__ __launch_bounds__(256) void dgc_hist_kernel(DgcParams p, int d)
{
    __shared__ uint32_t h[TK_BINS];
    for (uint32_t i = threadIdx.x; i < (uint32_t)TK_BINS; i += 256) h[i] = 0;
    __syncthreads();
    const uint32_t sh = dg_shift(d), mk = dg_mask(d);
    const uint32_t hs = sh + (d == 0 ? 11u : (d == 1 ? 11u : 9u)); // bits at and above hs are the prefix
    const uint32_t prefix = d == 0 ? 0u : p.ds->prefix;
    for (uint64_t q = (uint64_t)blockIdx.x * 256 + threadIdx.x; q < p.Ns; q += (uint64_t)gridDim.x * 256) {
        const uint32_t key = p.samples[q];
        if (d == 0 || (key >> hs) == (prefix >> hs)) atomicAdd(&h[(key >> sh) & mk], 1u);
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < (uint32_t)TK_BINS; i += 256)
        if (h[i]) atomicAdd(&p.hist[i], h[i]);
}

// The bin of the sought rank, counted from the top bin down, by one wave:
// lane l sums 32 bins from the top, a wave scan finds the lane, the lane
// walks its bins.  Updates the prefix and the rank; clears the histogram.
__global__ __launch_bounds__(SG_WAVE) void dgc_pick_kernel(DgcParams p, int d)
{
    const uint32_t lane = lane_id();
    const uint32_t nb = d == 2 ? 512u : 2048u;
    const uint32_t per = nb / SG_WAVE;
    uint32_t rank = d == 0 ? p.ks : p.ds->rank;
    uint32_t prefix = d == 0 ? 0u : p.ds->prefix;
    // lane l: bins [nb - per*(l+1), nb - per*l), top first
    uint32_t s = 0;
    for (uint32_t i = 0; i < per; ++i) s += p.hist[nb - 1 - (lane * per + i)];
    const uint32_t inc = wave_incl_scan(s);
    const uint64_t reach = ballot(inc >= rank);
    const uint32_t L = reach ? (uint32_t)__builtin_ctzll(reach) : SG_WAVE - 1;
    if (lane == L) {
        uint32_t before = inc - s;
        uint32_t bin = nb - 1 - lane * per;
        for (uint32_t i = 0; i < per; ++i) {
            const uint32_t b = nb - 1 - (lane * per + i);
            const uint32_t c = p.hist[b];
            bin = b;
            if (before + c >= rank) break;
            before += c;
        }
        rank -= before;
        prefix |= bin << dg_shift(d);
        p.ds->rank = rank;
        p.ds->prefix = prefix;
        if (d == 2) {
            p.ds->thr = prefix;
            if (p.thr_out) *p.thr_out = prefix;
            for (uint32_t w = 0; w < p.n; ++w) { // the write path selects key >= T
                p.t.st[w].T = prefix;
                p.t.st[w].need = 0xffffffffu;
            }
        }
    }
    // clear the histogram for the next digit
    for (uint32_t i = lane; i < (uint32_t)TK_BINS; i += SG_WAVE) p.hist[i] = 0;
}

// One 1024-element tile of worker w: new residual in place, selected entries
// compacted into the tile's slot in index order.
template <bool VEC>
__device__ __forceinline__ void dgc_tile(const DgcParams& p, uint32_t w, uint32_t t, uint32_t thr)
{
    constexpr int EPV = 4;
    constexpr int ITERS = TK_TILE / (SG_WAVE * EPV);
    const uint32_t lane = lane_id();
    const uint64_t lt = lanemask_lt();
    const uint64_t tile0 = (uint64_t)t * TK_TILE;
    const uint32_t len = (p.M - tile0) < (uint64_t)TK_TILE ? (uint32_t)(p.M - tile0) : (uint32_t)TK_TILE;
    const uint64_t gbase = (uint64_t)w * p.M + tile0;
    const uint64_t g = (uint64_t)w * p.t.NT + t;
    const uint64_t slot = g * TK_TILE;
    const bool full = VEC && len == TK_TILE;
    float a[ITERS][EPV];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const uint32_t e0 = i * (SG_WAVE * EPV) + lane * EPV;
        if (full) {
            // the gradient is read once: keep it out of the caches
            const u32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.grad + gbase + e0));
            const float4 rv = *reinterpret_cast<const float4*>(p.resid + gbase + e0);
            a[i][0] = rv.x + __uint_as_float(gv.x);
            a[i][1] = rv.y + __uint_as_float(gv.y);
            a[i][2] = rv.z + __uint_as_float(gv.z);
            a[i][3] = rv.w + __uint_as_float(gv.w);
        } else {
#pragma unroll
            for (int v = 0; v < EPV; ++v)
                a[i][v] = (e0 + v < len) ? p.resid[gbase + e0 + v] + p.grad[gbase + e0 + v] : 0.0f;
        }
    }
    uint32_t run = 0;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const uint32_t e0 = i * (SG_WAVE * EPV) + lane * EPV;
        uint32_t f = 0;
        float nr[EPV];
#pragma unroll
        for (int v = 0; v < EPV; ++v) {
            const bool sel = (e0 + v < len) && (__float_as_uint(a[i][v]) & 0x7fffffffu) >= thr;
            f |= (uint32_t)sel << v;
            nr[v] = sel ? 0.0f : a[i][v];
        }
        if (full) {
            *reinterpret_cast<float4*>(p.resid + gbase + e0) = make_float4(nr[0], nr[1], nr[2], nr[3]);
        } else {
#pragma unroll
            for (int v = 0; v < EPV; ++v)
                if (e0 + v < len) p.resid[gbase + e0 + v] = nr[v];
        }
        uint32_t x, tot;
        wave_count_scan<EPV>((uint32_t)__popc(f), lt, x, tot);
        if (f) {
            uint32_t pos = run + x;
#pragma unroll
            for (int v = 0; v < EPV; ++v) {
                if ((f >> v) & 1u) {
                    p.t.slot_idx[slot + pos] = (uint16_t)(e0 + v);
                    p.t.slot_val[slot + pos] = __float_as_uint(a[i][v]);
                    ++pos;
                }
            }
        }
        run += tot;
    }
    if (lane == 0) {
        p.t.tcnt[g] = run;
        p.t.ccnt[g] = 0;
    }
}

template <bool VEC>
__global__ __launch_bounds__(TK_THREADS) void dgc_filter_kernel(DgcParams p)
{
    const uint32_t thr = p.ds->thr;
    const uint64_t ntiles = (uint64_t)p.n * p.t.NT;
    const uint64_t stride = (uint64_t)gridDim.x * (TK_THREADS / SG_WAVE);
    for (uint64_t g = (uint64_t)blockIdx.x * (TK_THREADS / SG_WAVE) + threadIdx.x / SG_WAVE; g < ntiles;
         g += stride)
        dgc_tile<VEC>(p, (uint32_t)(g / p.t.NT), (uint32_t)(g % p.t.NT), thr);
}

// selected entries per worker: the sum of its tile counts
__global__ __launch_bounds__(1024) void dgc_count_kernel(DgcParams p)
{
    __shared__ uint64_t red[1024 / SG_WAVE];
    const uint32_t w = blockIdx.x;
    uint64_t s = 0;
    const uint32_t* const tc = p.t.tcnt + (uint64_t)w * p.t.NT;
    for (uint32_t t0 = threadIdx.x; t0 < p.t.NT; t0 += 8 * 1024) { // eight tiles' loads in flight
        uint32_t a[8];
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) a[u] = t0 + u * 1024 < p.t.NT ? tc[t0 + u * 1024] : 0u;
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) s += a[u];
    }
#pragma unroll
    for (int o = SG_WAVE / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, SG_WAVE);
    if (lane_id() == 0) red[threadIdx.x / SG_WAVE] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t c = 0;
        for (int i = 0; i < 1024 / SG_WAVE; ++i) c += red[i];
        p.count[w] = c;
    }
}

} // namespace sg

using namespace sg;

static uint64_t dgc_carve(Carver& c, uint32_t n, uint64_t M, uint64_t S, DgcParams* p)
{
    const uint64_t NT = ceil_div(M, TK_TILE);
    const uint64_t nt = (uint64_t)n * NT;
    const uint64_t ng = (uint64_t)n * ceil_div(NT, TK_GROUP);
    p->t.st = c.take<SelState>(n);
    p->t.tcnt = c.take<uint32_t>(nt);
    p->t.ccnt = c.take<uint32_t>(nt);
    p->t.gtx = c.take<uint32_t>(nt);
    p->t.eqx = c.take<uint32_t>(nt);
    p->t.ggt = c.take<uint32_t>(ng);
    p->t.geq = c.take<uint32_t>(ng);
    p->t.slot_idx = c.take<uint16_t>(nt * TK_TILE);
    p->t.slot_val = c.take<uint32_t>(nt * TK_TILE);
    p->samples = c.take<uint32_t>((uint64_t)n * S);
    p->hist = c.take<uint32_t>(TK_BINS);
    p->ds = c.take<DgcState>(1);
    return c.bytes();
}

extern "C" size_t sg_dgc_workspace_bytes(uint32_t n, uint64_t M, uint64_t S)
{
    if (S > M) S = M;
    DgcParams p;
    Carver c(nullptr);
    return dgc_carve(c, n, M, S, &p);
}

extern "C" uint64_t sg_dgc_rank(double density, uint64_t Ns)
{
    const double x = ceil(density * (double)Ns);
    if (!(x >= 1.0)) return 1;
    if (x >= (double)Ns) return Ns;
    return (uint64_t)x;
}

extern "C" int sg_dgc_select(const float* d_grad, float* d_resid, uint32_t n, uint64_t M, double density,
                             uint64_t S, uint32_t* d_idx, float* d_val, uint64_t cap, uint64_t* d_count,
                             uint32_t* d_thr, void* d_ws, size_t ws_bytes, void* stream)
{
    if (n == 0 || n > 64 || M == 0 || M >= (1ull << 32) || S == 0) return SG_EINVAL;
    if (!(density >= 0.0)) return SG_EINVAL;
    if (!d_grad || !d_resid || !d_count || !d_ws) return SG_EINVAL;
    if (cap > 0 && (!d_idx || !d_val)) return SG_EINVAL;
    if (S > M) S = M;
    if ((uint64_t)n * S >= (1ull << 32)) return SG_EUNSUPPORTED;
    if (ws_bytes < sg_dgc_workspace_bytes(n, M, S)) return SG_ECAPACITY;

    DgcParams p;
    Carver c(d_ws);
    dgc_carve(c, n, M, S, &p);
    p.grad = d_grad;
    p.resid = d_resid;
    p.thr_out = d_thr;
    p.count = d_count;
    p.M = M;
    p.S = S;
    p.Ns = (uint64_t)n * S;
    p.n = n;
    p.ks = (uint32_t)sg_dgc_rank(density, p.Ns);
    p.t.dense = nullptr;
    p.t.out_idx = d_idx;
    p.t.out_val = d_val;
    p.t.slot_key = nullptr; // no candidate keys: every slot entry is at or above the threshold
    p.t.M = M;
    p.t.k = cap;
    p.t.n = n;
    p.t.NT = (uint32_t)ceil_div(M, TK_TILE);
    p.t.NG = (uint32_t)ceil_div(p.t.NT, TK_GROUP);
    p.t.bf16 = 0;
    p.t.keymax = 0x7fffffffu;
    const bool vec = ((uintptr_t)d_grad % 16 == 0) && ((uintptr_t)d_resid % 16 == 0) && (M % 4 == 0);
    hipStream_t st = as_stream(stream);

    int rc = fill_u32(p.hist, TK_BINS, 0, st);
    if (rc) return rc;
    const uint64_t sblocks = ceil_div(p.Ns, 256);
    dgc_sample_kernel<<<(unsigned)(sblocks < 4096 ? sblocks : 4096), 256, 0, st>>>(p);
    SG_TRY_LAUNCH();
    const uint64_t hb = ceil_div(p.Ns, 256 * 8);
    const unsigned hgrid = (unsigned)(hb < DG_HIST_BLOCKS ? (hb ? hb : 1) : DG_HIST_BLOCKS);
    for (int d = 0; d < 3; ++d) {
        dgc_hist_kernel<<<hgrid, 256, 0, st>>>(p, d);
        SG_TRY_LAUNCH();
        dgc_pick_kernel<<<1, SG_WAVE, 0, st>>>(p, d);
        SG_TRY_LAUNCH();
    }
    const uint64_t ntiles = (uint64_t)n * p.t.NT;
    const uint64_t fblocks = ceil_div(ntiles, TK_THREADS / SG_WAVE);
    const unsigned fgrid = (unsigned)(fblocks < 16384 ? fblocks : 16384);
    probe_begin(SG_PROBE_DGC_FILTER, st);
    if (vec) dgc_filter_kernel<true><<<fgrid, TK_THREADS, 0, st>>>(p);
    else dgc_filter_kernel<false><<<fgrid, TK_THREADS, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_DGC_FILTER, st);
    dgc_count_kernel<<<n, 1024, 0, st>>>(p);
    SG_TRY_LAUNCH();
    if (cap == 0) return SG_OK;
    const unsigned wgridw = (unsigned)ceil_div((uint64_t)n * p.t.NG * TK_WRITE_WAVES, TK_THREADS / SG_WAVE);
    topk_tilecount_kernel<<<(unsigned)ceil_div((uint64_t)n * p.t.NG, TK_THREADS / SG_WAVE), TK_THREADS, 0, st>>>(p.t);
    SG_TRY_LAUNCH();
    topk_scan_kernel<<<n, 1024, 0, st>>>(p.t);
    SG_TRY_LAUNCH();
    if (p.t.bf16) topk_write_kernel<true><<<wgridw, TK_THREADS, 0, st>>>(p.t);
    else topk_write_kernel<false><<<wgridw, TK_THREADS, 0, st>>>(p.t);
    SG_TRY_LAUNCH();
    return SG_OK;
}

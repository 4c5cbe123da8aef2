// sg_skiprs.hip -- A5: ring reduce-scatter arithmetic with SkipReduce-style
// slice skipping, for n worker buffers resident on one GPU.
//
// The ring's reduce-scatter phase (CMU 15-442/642 notes, "Ring AllReduce",
// aggregation phase): chunk j starts at rank j and is passed around the ring;
// the rank at ring position t adds its own copy of the chunk before
// forwarding.  SkipReduce (MICRO'25 digest, section 4.2, Algorithms 1-2) lets
// a rank skip that add for a slice, forwarding what it received; Random
// SkipReduce (section 4.3) draws the skips from a seed shared by all ranks;
// DropReduce (section 4.1) rescales by n/c instead of treating skipped data
// as zero.  On one GPU the n-1 sequential ring steps collapse into one pass:
// every output element is the ring-ordered sum of the kept contributions, so
// each kept input byte is read once, each output byte written once, and a
// skipped slice is never read.  The path is HBM-bound: no LDS, 16-byte
// vector loads, several contributors' loads in flight per thread.
#include "sg_host.h"

namespace sg {

constexpr int RS_THREADS = 256;
constexpr int RS_VEC_PER_THREAD = 4; // 16-byte vectors per thread per contributor

struct RsParams {
    const void* bufs;
    float* out;
    uint8_t* count;
    const uint8_t* include;
    uint64_t M;
    uint64_t stride;    // elements between two ranks' buffers (M, or more for a bucket)
    uint64_t slice_elems;
    uint64_t S;         // slices per chunk
    uint64_t tiles_per_slice;
    uint64_t nblocks;   // n * S * tiles_per_slice
    uint64_t seed;
    uint32_t n;
    uint32_t thr24;     // floor(p * 2^24)
    int drop;
    int kind;           // RS_BERNOULLI or RS_STEPS (used when include == NULL)
    uint32_t k;         // RS_STEPS: chain positions below k are not reduced
    uint32_t off;       // RS_STEPS: shift of the chain (0 = static SkipReduce)
};

enum { RS_BERNOULLI = 0, RS_STEPS = 1 };

template <typename T>
struct VecTraits;
template <>
struct VecTraits<float> {
    static constexpr int EPV = 4; // elements per 16-byte vector
};
template <>
struct VecTraits<uint16_t> {
    static constexpr int EPV = 8;
};

__device__ __forceinline__ void load_vec(const float* p, float (&v)[8])
{
    float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x;
    v[1] = x.y;
    v[2] = x.z;
    v[3] = x.w;
}

__device__ __forceinline__ void load_vec(const uint16_t* p, float (&v)[8])
{
    uint4 x = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ float load_one(const float* p) { return *p; }
__device__ __forceinline__ float load_one(const uint16_t* p) { return bf16_to_f32(*p); }

// Inclusion mask of (j, q) over ring positions t (bit t), computed by every
// wave on its own (n <= 64 lanes, one SplitMix64 draw per lane).
__device__ __forceinline__ uint64_t rs_mask(const RsParams& p, uint32_t j, uint64_t q)
{
    const uint32_t t = lane_id();
    bool inc = false;
    if (t < p.n) {
        if (p.include) {
            inc = p.include[((uint64_t)j * p.n + t) * p.S + q] != 0;
        } else if (p.kind == RS_STEPS) {
            inc = (t + p.off) % p.n >= p.k;
        } else if (t == 0) {
            inc = true;
        } else {
            uint64_t ctr = ((uint64_t)j * (p.n - 1) + (t - 1)) * p.S + q;
            inc = (uint32_t)(splitmix64_at(p.seed, ctr) >> 40) >= p.thr24;
        }
    }
    return ballot(inc);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(RS_THREADS) void skip_rs_kernel(RsParams p)
{
    constexpr int EPV = VecTraits<T>::EPV;
    constexpr int TILE = RS_THREADS * RS_VEC_PER_THREAD * (VEC ? EPV : 1);
    const T* __restrict__ bufs = static_cast<const T*>(p.bufs);

    for (uint64_t b = blockIdx.x; b < p.nblocks; b += gridDim.x) {
        const uint64_t tile = b % p.tiles_per_slice;
        const uint64_t q = (b / p.tiles_per_slice) % p.S;
        const uint32_t j = (uint32_t)(b / (p.tiles_per_slice * p.S));
        const uint64_t cb = (uint64_t)(((unsigned __int128)p.M * j) / p.n);
        const uint64_t ce = (uint64_t)(((unsigned __int128)p.M * (j + 1)) / p.n);

        const uint64_t mask = rs_mask(p, j, q);
        const uint32_t c = popc64(mask);
        if (tile == 0 && threadIdx.x == 0 && p.count) p.count[(uint64_t)j * p.S + q] = (uint8_t)c;

        uint64_t s0 = cb + q * p.slice_elems;
        uint64_t s1 = s0 + p.slice_elems;
        if (s1 > ce) s1 = ce;
        uint64_t e0 = s0 + tile * (uint64_t)TILE;
        uint64_t e1 = e0 + TILE;
        if (e1 > s1) e1 = s1;
        if (e0 >= e1) continue;

        const float scale = (p.drop && c > 0) ? (float)p.n / (float)c : 1.0f;

        if (VEC) {
            // vector v of this thread covers elements e0 + (threadIdx.x + v*RS_THREADS)*EPV
            float acc[RS_VEC_PER_THREAD][EPV];
#pragma unroll
            for (int v = 0; v < RS_VEC_PER_THREAD; ++v)
#pragma unroll
                for (int i = 0; i < EPV; ++i) acc[v][i] = 0.0f;
            uint64_t m = mask;
            while (m) {
                // up to two kept contributors per round keep 8 vectors in flight
                uint32_t t0 = __builtin_ctzll(m);
                m &= m - 1;
                int have1 = m != 0;
                uint32_t t1 = have1 ? __builtin_ctzll(m) : t0;
                if (have1) m &= m - 1;
                const T* src0 = bufs + (uint64_t)((j + t0) % p.n) * p.stride;
                const T* src1 = bufs + (uint64_t)((j + t1) % p.n) * p.stride;
                float x0[RS_VEC_PER_THREAD][8], x1[RS_VEC_PER_THREAD][8];
#pragma unroll
                for (int v = 0; v < RS_VEC_PER_THREAD; ++v) {
                    uint64_t e = e0 + ((uint64_t)threadIdx.x + (uint64_t)v * RS_THREADS) * EPV;
                    if (e < e1) {
                        load_vec(src0 + e, x0[v]);
                        if (have1) load_vec(src1 + e, x1[v]);
                    }
                }
#pragma unroll
                for (int v = 0; v < RS_VEC_PER_THREAD; ++v) {
#pragma unroll
                    for (int i = 0; i < EPV; ++i) {
                        acc[v][i] += x0[v][i];
                        if (have1) acc[v][i] += x1[v][i];
                    }
                }
            }
#pragma unroll
            for (int v = 0; v < RS_VEC_PER_THREAD; ++v) {
                uint64_t e = e0 + ((uint64_t)threadIdx.x + (uint64_t)v * RS_THREADS) * EPV;
                if (e < e1) {
                    float r[EPV];
#pragma unroll
                    for (int i = 0; i < EPV; ++i) r[i] = c ? acc[v][i] * scale : 0.0f;
#pragma unroll
                    for (int h = 0; h < EPV; h += 4)
                        *reinterpret_cast<float4*>(p.out + e + h) = make_float4(r[h], r[h + 1], r[h + 2], r[h + 3]);
                }
            }
        } else {
            for (uint64_t e = e0 + threadIdx.x; e < e1; e += RS_THREADS) {
                float acc = 0.0f;
                uint64_t m = mask;
                while (m) {
                    uint32_t t = __builtin_ctzll(m);
                    m &= m - 1;
                    acc += load_one(bufs + (uint64_t)((j + t) % p.n) * p.stride + e);
                }
                p.out[e] = c ? acc * scale : 0.0f;
            }
        }
    }
}


// ---------------------------------------------------------------------------
// AllReduce_Dropout (SkipReduce digest, section 4.2, Algorithm 1): the
// ReduceOrSkip decision is taken per element.  Element e at ring position
// t >= 1 is dropped when the top 24 bits of SplitMix64 output number
// (t-1)*M + e fall below floor(p * 2^24); the origin (t = 0) is always kept.
// Every contribution's cache lines are read (a dropped element shares its
// line with kept ones); the draws are the ALU cost.
// ---------------------------------------------------------------------------
struct DropParams {
    const void* bufs;
    float* out;
    uint8_t* count;
    uint64_t M;
    uint64_t chunk;     // M / n when the vector path is taken
    uint64_t ngroups;   // element groups of EPV (vector path) or elements
    uint64_t seed;
    uint32_t n;
    uint32_t thr24;
    int drop;
};

// Chunk of element e: the largest j with floor(jM/n) <= e.
__device__ __forceinline__ uint32_t chunk_of(uint64_t e, uint64_t M, uint32_t n)
{
    return (uint32_t)(((e + 1) * n - 1) / M);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(RS_THREADS) void dropout_rs_kernel(DropParams p)
{
    constexpr int EPV = VEC ? VecTraits<T>::EPV : 1;
    const T* __restrict__ bufs = static_cast<const T*>(p.bufs);
    for (uint64_t g = (uint64_t)blockIdx.x * RS_THREADS + threadIdx.x; g < p.ngroups;
         g += (uint64_t)gridDim.x * RS_THREADS) {
        const uint64_t e0 = g * EPV;
        const uint32_t j = VEC ? (uint32_t)(e0 / p.chunk) : chunk_of(e0, p.M, p.n);
        float acc[EPV];
        uint32_t c[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            acc[i] = 0.0f;
            c[i] = 0;
        }
        uint32_t r = j;
        for (uint32_t t = 0; t < p.n; ++t) {
            float x[8];
            if (VEC) load_vec(bufs + (uint64_t)r * p.M + e0, x);
            else x[0] = load_one(bufs + (uint64_t)r * p.M + e0);
#pragma unroll
            for (int i = 0; i < EPV; ++i) {
                bool keep = true;
                if (t > 0)
                    keep = (uint32_t)(splitmix64_at(p.seed, (uint64_t)(t - 1) * p.M + e0 + i) >> 40) >= p.thr24;
                if (keep) {
                    acc[i] += x[i];
                    ++c[i];
                }
            }
            r = r + 1 == p.n ? 0 : r + 1;
        }
        float res[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            const float scale = (p.drop && c[i] > 0) ? (float)p.n / (float)c[i] : 1.0f;
            res[i] = c[i] ? acc[i] * scale : 0.0f;
        }
        if (VEC) {
#pragma unroll
            for (int h = 0; h < EPV; h += 4)
                *reinterpret_cast<float4*>(p.out + e0 + h) = make_float4(res[h], res[h + 1], res[h + 2], res[h + 3]);
        } else {
            p.out[e0] = res[0];
        }
        if (p.count) {
#pragma unroll
            for (int i = 0; i < EPV; ++i) p.count[e0 + i] = (uint8_t)c[i];
        }
    }
}

// ---------------------------------------------------------------------------
// The ring's all-gather phase (CMU notes, broadcast phase): the holder of
// reduced chunk j passes it on; ring position u = 0..n-2 of chunk j (rank
// (j+u) mod n) receives it at step u, position n-1 holds it already.  With a
// delivery mask, a rank whose delivery is skipped keeps its own values of the
// chunk.  One thread covers EPV elements of every rank: the reduced values are
// read once and written n times.
// ---------------------------------------------------------------------------
struct AgParams {
    const float* reduced;
    const void* bufs;
    const uint8_t* ag_include;  // [n][n] (chunk j, position u), or NULL
    float* out;                 // [n][M]
    uint64_t M;
    uint64_t chunk;
    uint64_t ngroups;
    uint32_t n;
};

template <typename T, bool VEC>
__global__ __launch_bounds__(RS_THREADS) void allgather_kernel(AgParams p)
{
    constexpr int EPV = VEC ? 4 : 1;  // fp32 output vectors of 16 bytes
    const T* __restrict__ bufs = static_cast<const T*>(p.bufs);
    for (uint64_t g = (uint64_t)blockIdx.x * RS_THREADS + threadIdx.x; g < p.ngroups;
         g += (uint64_t)gridDim.x * RS_THREADS) {
        const uint64_t e0 = g * EPV;
        const uint32_t j = VEC ? (uint32_t)(e0 / p.chunk) : chunk_of(e0, p.M, p.n);
        float red[4];
        if (VEC) {
            float4 v = *reinterpret_cast<const float4*>(p.reduced + e0);
            red[0] = v.x;
            red[1] = v.y;
            red[2] = v.z;
            red[3] = v.w;
        } else {
            red[0] = p.reduced[e0];
        }
        for (uint32_t u = 0; u < p.n; ++u) {
            const uint32_t r = (j + u) % p.n;
            const bool got = u == p.n - 1 || !p.ag_include || p.ag_include[(uint64_t)j * p.n + u] != 0;
            float v[4];
#pragma unroll
            for (int i = 0; i < EPV; ++i) v[i] = red[i];
            if (!got) {
#pragma unroll
                for (int i = 0; i < EPV; ++i) v[i] = load_one(bufs + (uint64_t)r * p.M + e0 + i);
            }
            float* o = p.out + (uint64_t)r * p.M + e0;
            if (VEC) *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
            else o[0] = v[0];
        }
    }
}

} // namespace sg

using namespace sg;

static uint32_t skip_threshold(double p)
{
    if (!(p > 0.0)) return 0;
    if (p >= 1.0) return 1u << 24;
    return (uint32_t)floor(p * 16777216.0);
}

static uint64_t grid_for(uint64_t blocks) { return blocks < 65536 ? (blocks ? blocks : 1) : 65536; }

extern "C" uint64_t sg_skip_num_slices(uint32_t n, uint64_t M, uint64_t slice_bytes, sg_dtype dt)
{
    uint64_t esz = dt == SG_BF16 ? 2 : 4;
    if (n == 0 || slice_bytes < esz) return 0;
    uint64_t se = slice_bytes / esz;
    uint64_t maxchunk = ceil_div(M, n);
    return maxchunk ? ceil_div(maxchunk, se) : 0;
}

// Checks shared by the slice-granular entry points.
static int rs_check(sg_dtype dt, uint32_t n, uint64_t M, uint64_t slice_bytes, sg_rescale mode)
{
    if (n == 0 || n > 64 || (dt != SG_F32 && dt != SG_BF16)) return SG_EINVAL;
    if (mode != SG_RESCALE_NONE && mode != SG_RESCALE_DROP) return SG_EINVAL;
    const uint64_t esz = dt == SG_BF16 ? 2 : 4;
    if (slice_bytes == 0 || slice_bytes % esz) return SG_EINVAL;
    if (M >= (1ull << 40)) return SG_EUNSUPPORTED;
    return SG_OK;
}

// Launch of the reduce-scatter kernel over one tensor of M elements whose
// rank buffers are `stride` elements apart.
static int rs_launch(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, uint64_t stride, uint64_t slice_bytes,
                     int kind, double p_skip, uint32_t k, uint32_t off, uint64_t seed, const uint8_t* d_include,
                     sg_rescale mode, float* d_out, uint8_t* d_count, hipStream_t st)
{
    const uint64_t esz = dt == SG_BF16 ? 2 : 4;
    RsParams p;
    p.bufs = d_bufs;
    p.out = d_out;
    p.count = d_count;
    p.include = d_include;
    p.M = M;
    p.stride = stride;
    p.slice_elems = slice_bytes / esz;
    p.S = sg_skip_num_slices(n, M, slice_bytes, dt);
    p.seed = seed;
    p.n = n;
    p.thr24 = skip_threshold(p_skip);
    p.drop = mode == SG_RESCALE_DROP;
    p.kind = kind;
    p.k = k;
    p.off = off;

    const int epv = dt == SG_BF16 ? 8 : 4;
    const bool aligned = ((uintptr_t)d_bufs % 16 == 0) && ((uintptr_t)d_out % 16 == 0) && ((stride * esz) % 16 == 0);
    const bool vec = aligned && (M % ((uint64_t)epv * n) == 0) && (p.slice_elems % epv == 0);
    const uint64_t tile = (uint64_t)RS_THREADS * RS_VEC_PER_THREAD * (vec ? epv : 1);
    const uint64_t chunk_max = ceil_div(M, n);
    const uint64_t per_slice = p.slice_elems < chunk_max ? p.slice_elems : chunk_max;
    p.tiles_per_slice = ceil_div(per_slice, tile);
    if (p.tiles_per_slice == 0) p.tiles_per_slice = 1;
    p.nblocks = (uint64_t)n * p.S * p.tiles_per_slice;
    const uint64_t grid = grid_for(p.nblocks);
    probe_begin(SG_PROBE_SKIP_RS, st);
    if (dt == SG_F32) {
        if (vec) skip_rs_kernel<float, true><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
        else skip_rs_kernel<float, false><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
    } else {
        if (vec) skip_rs_kernel<uint16_t, true><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
        else skip_rs_kernel<uint16_t, false><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
    }
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_SKIP_RS, st);
    return SG_OK;
}

extern "C" int sg_skip_reduce_scatter(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, uint64_t slice_bytes,
                                      double p_skip, uint64_t seed, const uint8_t* d_include, sg_rescale mode,
                                      float* d_out, uint8_t* d_count, void* stream)
{
    int rc = rs_check(dt, n, M, slice_bytes, mode);
    if (rc) return rc;
    if (!(p_skip >= 0.0 && p_skip <= 1.0)) return SG_EINVAL;
    if (M == 0) return SG_OK;
    if (!d_bufs || !d_out) return SG_EINVAL;
    return rs_launch(d_bufs, dt, n, M, M, slice_bytes, RS_BERNOULLI, p_skip, 0, 0, seed, d_include, mode, d_out,
                     d_count, as_stream(stream));
}

extern "C" uint32_t sg_skip_random_offset(uint32_t n, uint64_t seed)
{
    return n ? (uint32_t)(splitmix64_at(seed, 0) % n) : 0;
}

extern "C" int sg_skip_reduce_k(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, uint64_t slice_bytes,
                                uint32_t k, int random_offset, uint64_t seed, sg_rescale mode, float* d_out,
                                uint8_t* d_count, void* stream)
{
    int rc = rs_check(dt, n, M, slice_bytes, mode);
    if (rc) return rc;
    if (k > n) return SG_EINVAL;
    if (M == 0) return SG_OK;
    if (!d_bufs || !d_out) return SG_EINVAL;
    const uint32_t off = random_offset ? sg_skip_random_offset(n, seed) : 0;
    return rs_launch(d_bufs, dt, n, M, M, slice_bytes, RS_STEPS, 0.0, k, off, seed, nullptr, mode, d_out, d_count,
                     as_stream(stream));
}

extern "C" int sg_selective_reduce_scatter(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, uint32_t nb,
                                           const uint64_t* h_bucket_off, const double* h_p_skip,
                                           uint64_t slice_bytes, uint64_t seed, sg_rescale mode, float* d_out,
                                           void* stream)
{
    int rc = rs_check(dt, n, M, slice_bytes, mode);
    if (rc) return rc;
    if (nb == 0 || !h_bucket_off || !h_p_skip) return SG_EINVAL;
    if (M > 0 && (!d_bufs || !d_out)) return SG_EINVAL;
    if (h_bucket_off[0] > M) return SG_EINVAL;
    for (uint32_t b = 0; b < nb; ++b) {
        if (h_bucket_off[b + 1] < h_bucket_off[b] || h_bucket_off[b + 1] > M) return SG_EINVAL;
        if (!(h_p_skip[b] >= 0.0 && h_p_skip[b] <= 1.0)) return SG_EINVAL;
    }
    const uint64_t esz = dt == SG_BF16 ? 2 : 4;
    hipStream_t st = as_stream(stream);
    for (uint32_t b = 0; b < nb; ++b) {
        const uint64_t lo = h_bucket_off[b], Mb = h_bucket_off[b + 1] - lo;
        if (Mb == 0) continue;
        rc = rs_launch(static_cast<const char*>(d_bufs) + lo * esz, dt, n, Mb, M, slice_bytes, RS_BERNOULLI,
                       h_p_skip[b], 0, 0, seed + b, nullptr, mode, d_out + lo, nullptr, st);
        if (rc) return rc;
    }
    return SG_OK;
}

extern "C" int sg_dropout_reduce_scatter(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, double p_skip,
                                         uint64_t seed, sg_rescale mode, float* d_out, uint8_t* d_count,
                                         void* stream)
{
    if (n == 0 || n > 64 || (dt != SG_F32 && dt != SG_BF16)) return SG_EINVAL;
    if (mode != SG_RESCALE_NONE && mode != SG_RESCALE_DROP) return SG_EINVAL;
    if (!(p_skip >= 0.0 && p_skip <= 1.0)) return SG_EINVAL;
    if (M >= (1ull << 40)) return SG_EUNSUPPORTED;
    if (M == 0) return SG_OK;
    if (!d_bufs || !d_out) return SG_EINVAL;
    DropParams p;
    p.bufs = d_bufs;
    p.out = d_out;
    p.count = d_count;
    p.M = M;
    p.seed = seed;
    p.n = n;
    p.thr24 = skip_threshold(p_skip);
    p.drop = mode == SG_RESCALE_DROP;
    const uint64_t esz = dt == SG_BF16 ? 2 : 4;
    const int epv = dt == SG_BF16 ? 8 : 4;
    const bool vec = ((uintptr_t)d_bufs % 16 == 0) && ((uintptr_t)d_out % 16 == 0) && ((M * esz) % 16 == 0) &&
                     (M % ((uint64_t)epv * n) == 0);
    p.chunk = M / n;
    p.ngroups = vec ? M / epv : M;
    const uint64_t grid = grid_for(ceil_div(p.ngroups, RS_THREADS));
    hipStream_t st = as_stream(stream);
    probe_begin(SG_PROBE_DROPOUT_RS, st);
    if (dt == SG_F32) {
        if (vec) dropout_rs_kernel<float, true><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
        else dropout_rs_kernel<float, false><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
    } else {
        if (vec) dropout_rs_kernel<uint16_t, true><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
        else dropout_rs_kernel<uint16_t, false><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
    }
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_DROPOUT_RS, st);
    return SG_OK;
}

extern "C" int sg_allgather(const float* d_reduced, const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M,
                            const uint8_t* d_ag_include, float* d_out, void* stream)
{
    if (n == 0 || n > 64 || (dt != SG_F32 && dt != SG_BF16)) return SG_EINVAL;
    if (M >= (1ull << 40)) return SG_EUNSUPPORTED;
    if (M == 0) return SG_OK;
    if (!d_reduced || !d_out) return SG_EINVAL;
    if (d_ag_include && !d_bufs) return SG_EINVAL;
    AgParams p;
    p.reduced = d_reduced;
    p.bufs = d_bufs;
    p.ag_include = d_ag_include;
    p.out = d_out;
    p.M = M;
    p.n = n;
    const bool vec = ((uintptr_t)d_reduced % 16 == 0) && ((uintptr_t)d_out % 16 == 0) && (M % (4ull * n) == 0);
    p.chunk = M / n;
    p.ngroups = vec ? M / 4 : M;
    const uint64_t grid = grid_for(ceil_div(p.ngroups, RS_THREADS));
    hipStream_t st = as_stream(stream);
    probe_begin(SG_PROBE_ALLGATHER, st);
    if (dt == SG_F32) {
        if (vec) allgather_kernel<float, true><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
        else allgather_kernel<float, false><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
    } else {
        if (vec) allgather_kernel<uint16_t, true><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
        else allgather_kernel<uint16_t, false><<<(unsigned)grid, RS_THREADS, 0, st>>>(p);
    }
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_ALLGATHER, st);
    return SG_OK;
}

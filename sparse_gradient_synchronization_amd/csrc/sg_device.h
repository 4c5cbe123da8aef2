// sg_device.h -- device-side helpers shared by the gfx950 kernels of libsg.
// Wave64 primitives, the h0 partition hash, the counter-based RNG of the
// skip mask, and small block-level scans.  Everything here is written for
// CDNA4 (64-wide wavefronts); there is no warp-32 path.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SG_WAVE 64

namespace sg {

// ---------------------------------------------------------------------------
// error reporting from device code
// ---------------------------------------------------------------------------
// A single word per device; the host reads and clears it with
// sg_device_error().  Kernels never trap: a violated precondition records a
// code here and the kernel keeps every access in bounds.
extern __device__ int g_device_error;

// codes recorded in g_device_error
constexpr int kDevErrBadOffsets = 1;
constexpr int kDevErrIndexRange = 2;
constexpr int kDevErrUnsorted = 3;
constexpr int kDevErrSpin = 4;
constexpr int kDevErrCmap = 5;
constexpr int kDevErrPartition = 6;

__host__ __device__ __forceinline__ uint64_t ceil_div_dev(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ void report_error(int code)
{
    atomicCAS(&g_device_error, 0, code);
}

// ---------------------------------------------------------------------------
// wave primitives
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }
__device__ __forceinline__ uint32_t popc64(uint64_t x) { return (uint32_t)__popcll(x); }
// set bits of m in the lanes below this one (two mbcnt instructions)
__device__ __forceinline__ uint32_t count_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
// Waits until every vector memory operation of the wave is done (the GFX9
// s_waitcnt with vmcnt = 0 and the other counters left at their maxima).
// The vector memory counter covers stores as well as loads, so once a store
// is issued the compiler can no longer wait for an earlier load alone: a
// kernel that loads a batch and then stores waits for the batch here, before
// its first store, and needs no wait after.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// a value every lane holds alike, moved to a scalar register
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    return ((uint64_t)uniform((uint32_t)(v >> 32)) << 32) | uniform((uint32_t)v);
}

// v of lane l (l wave-uniform), in scalar registers
__device__ __forceinline__ uint32_t lane_value(uint32_t v, uint32_t l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)l);
}

__device__ __forceinline__ uint64_t lane_value64(uint64_t v, uint32_t l)
{
    return ((uint64_t)lane_value((uint32_t)(v >> 32), l) << 32) | lane_value((uint32_t)v, l);
}

// Cross-lane moves by DPP (data-parallel primitives of the GFX9 ISA family):
// a lane reads another lane's register inside the VALU, without the LDS
// round trip of ds_bpermute.  Lanes whose source is outside its row, or whose
// row is masked off, receive `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_move(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// inclusive scan over the 64 lanes of a wave: log steps inside each row of
// 16 lanes, then row 0's total into row 1 (and row 2's into row 3), then the
// first half's total into the second half
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v)
{
    v += dpp_move<kDppRowShr1>(0u, v);
    v += dpp_move<kDppRowShr2>(0u, v);
    v += dpp_move<kDppRowShr4>(0u, v);
    v += dpp_move<kDppRowShr8>(0u, v);
    v += dpp_move<kDppRowBcast15, 0xa>(0u, v);
    v += dpp_move<kDppRowBcast31, 0xc>(0u, v);
    return v;
}

__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t v)
{
#pragma unroll
    for (int d = 1; d < SG_WAVE; d <<= 1) {
        uint64_t t = __shfl_up(v, d, SG_WAVE);
        if ((int)lane_id() >= d) v += t;
    }
    return v;
}

// sum over the wave, the same in every lane
__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), SG_WAVE - 1);
}

// minimum over the wave, the same in every lane
__device__ __forceinline__ uint32_t wave_min(uint32_t v)
{
    constexpr uint32_t top = 0xffffffffu;
    uint32_t t;
    t = dpp_move<kDppRowShr1>(top, v); v = t < v ? t : v;
    t = dpp_move<kDppRowShr2>(top, v); v = t < v ? t : v;
    t = dpp_move<kDppRowShr4>(top, v); v = t < v ? t : v;
    t = dpp_move<kDppRowShr8>(top, v); v = t < v ? t : v;
    t = dpp_move<kDppRowBcast15, 0xa>(top, v); v = t < v ? t : v;
    t = dpp_move<kDppRowBcast31, 0xc>(top, v); v = t < v ? t : v;
    return (uint32_t)__builtin_amdgcn_readlane((int)v, SG_WAVE - 1);
}

// maximum over the wave, the same in every lane
__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    uint32_t t;
    t = dpp_move<kDppRowShr1>(0u, v); v = t > v ? t : v;
    t = dpp_move<kDppRowShr2>(0u, v); v = t > v ? t : v;
    t = dpp_move<kDppRowShr4>(0u, v); v = t > v ? t : v;
    t = dpp_move<kDppRowShr8>(0u, v); v = t > v ? t : v;
    t = dpp_move<kDppRowBcast15, 0xa>(0u, v); v = t > v ? t : v;
    t = dpp_move<kDppRowBcast31, 0xc>(0u, v); v = t > v ? t : v;
    return (uint32_t)__builtin_amdgcn_readlane((int)v, SG_WAVE - 1);
}

// Exclusive scan over the threads of a block of NT threads (NT a multiple of
// 64, at most 1024).  `lds` must hold NT/64 + 1 words.  Returns the exclusive
// prefix; *total receives the block total.  Contains two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* lds, uint32_t* total)
{
    constexpr int NW = NT / SG_WAVE;
    const uint32_t wid = threadIdx.x / SG_WAVE;
    uint32_t inc = wave_incl_scan(v);
    if (lane_id() == SG_WAVE - 1) lds[wid] = inc;
    __syncthreads();
    if (threadIdx.x < SG_WAVE) {
        uint32_t w = threadIdx.x < NW ? lds[threadIdx.x] : 0u;
        uint32_t wi = wave_incl_scan(w);
        if (threadIdx.x < NW) lds[threadIdx.x] = wi - w;
        if (threadIdx.x == NW - 1) lds[NW] = wi;
    }
    __syncthreads();
    uint32_t res = lds[wid] + inc - v;
    *total = lds[NW];
    return res;
}

template <int NT>
__device__ __forceinline__ uint64_t block_excl_scan64(uint64_t v, uint64_t* lds, uint64_t* total)
{
    constexpr int NW = NT / SG_WAVE;
    const uint32_t wid = threadIdx.x / SG_WAVE;
    uint64_t inc = wave_incl_scan64(v);
    if (lane_id() == SG_WAVE - 1) lds[wid] = inc;
    __syncthreads();
    if (threadIdx.x < SG_WAVE) {
        uint64_t w = threadIdx.x < NW ? lds[threadIdx.x] : 0ull;
        uint64_t wi = wave_incl_scan64(w);
        if (threadIdx.x < NW) lds[threadIdx.x] = wi - w;
        if (threadIdx.x == NW - 1) lds[NW] = wi;
    }
    __syncthreads();
    uint64_t res = lds[wid] + inc - v;
    *total = lds[NW];
    return res;
}

// ---------------------------------------------------------------------------
// h0: MurmurHash2 (32-bit) of the index as four little-endian bytes, mod P.
// The Zen page (section 4, Implementation) names MurmurHash 2.0, seeded per
// hash function; this is the 4-byte-key case of Appleby's published algorithm
// (one block, no tail).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t murmur2_u32(uint32_t key, uint32_t seed)
{
    const uint32_t m = 0x5bd1e995u;
    uint32_t k = key * m;
    k ^= k >> 24;
    k *= m;
    uint32_t h = (seed ^ 4u) * m;
    h ^= k;
    h ^= h >> 13;
    h *= m;
    h ^= h >> 15;
    return h;
}

// Division by a runtime-invariant P through a precomputed reciprocal
// (Granlund-Montgomery round-up method): q = mulhi(h, mul) >> shift, exact for
// all 32-bit h.  Built on the host by make_divider().
struct Divider {
    uint32_t P;
    uint32_t mul;
    uint32_t shift;
    uint32_t pow2; // 1 when P is a power of two (then mul/shift unused)
};

__device__ __forceinline__ uint32_t mod_p(uint32_t h, const Divider& d)
{
    if (d.pow2) return h & (d.P - 1u);
    uint32_t q = __umulhi(h, d.mul);
    q = (q + ((h - q) >> 1)) >> d.shift;
    return h - q * d.P;
}

__device__ __forceinline__ uint32_t h0(uint32_t idx, uint32_t seed, const Divider& d)
{
    return mod_p(murmur2_u32(idx, seed), d);
}

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014), counter form: output number
// ctr (0-based) of the stream that starts at `seed`.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t ctr)
{
    uint64_t z = seed + (ctr + 1ull) * 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// ---------------------------------------------------------------------------
// agent-scope atomics used by the ordered (look-back) scans
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t load_agent(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// LDS written by some lanes of a wave and read by others: a wave executes its
// LDS operations in order; this keeps the compiler from moving them.  The
// fences name LDS only: a fence on every address space would also wait for
// the wave's outstanding global loads and stores (vmcnt 0), which takes the
// latency of prefetched loads and of written output onto every such point.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

} // namespace sg

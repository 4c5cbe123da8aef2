// sg_encode.hip -- A4: hash-bitmap encoding of the aggregate's indices
// (Zen OSDI'25 digest, section 3.3.2 and the Fig. 10 walk-through).
//
// Server p's index set is the class C_p = { i : h0(i) = p }, ascending,
// fixed offline; its bitmap has bit b set when C_p[b] is in the server's
// aggregate.  The bit of an aggregated index i of partition p is its rank in
// C_p: (class-p keys before i's window) + (class-p keys before i inside the
// window).
//
// Class map (built once per (M, P, seed), like the page's offline C_p):
//   - bit-sliced class ids: per 32-key chunk, ceil(log2 P) plane words, so
//     the class-p members of a chunk are an AND of planes (or complements);
//   - per window of W keys, the number of class-p keys before it (cpre);
//   - class sizes and word offsets.
// Encode streams the key space once, all partitions together: per window a
// block forms the class masks of its chunks and their prefix counts in LDS,
// each wave walks its partitions' aggregated keys (a cursor per partition,
// sorted input) and sets bits in an LDS copy of the block's bitmap segments,
// and the segments are written out at the end.  Words shared with a
// neighbouring block are merged with atomicOr after the preparation kernel
// has zeroed them; all other words are plain stores.
#include "sg_host.h"

namespace sg {

constexpr uint32_t CM_MAGIC = 0x53474d31u; // "SGM1"
constexpr int EN_THREADS = 256;
constexpr int EN_SEG_WORDS = 512; // a window's bitmap words: at most W/32 + P <= 128 + 256

struct CmapLayout {
    uint64_t M;
    uint32_t P, nbits, stride, NCW, W;
    uint64_t NW, NC;
    uint64_t off_class_size, off_word_off, off_cpre, off_planes, bytes;
};

struct CmapHeader {
    uint32_t magic, P;
    uint64_t M;
    uint32_t seed, nbits, stride, NCW, W, pad;
    uint64_t NW, NC;
};

static CmapLayout cmap_layout(uint64_t M, uint32_t P)
{
    CmapLayout L;
    L.M = M;
    L.P = P;
    L.nbits = 0;
    while ((1u << L.nbits) < P) ++L.nbits;
    L.stride = L.nbits == 0 ? 0 : (L.nbits == 1 ? 1 : (L.nbits == 2 ? 2 : (L.nbits <= 4 ? 4 : 8)));
    // chunks per window: a power of two in [8, 128] with NCW * P <= 2048
    L.NCW = 128;
    while (L.NCW > 8 && L.NCW * P > 2048) L.NCW >>= 1;
    L.W = 32 * L.NCW;
    L.NW = ceil_div(M, L.W);
    L.NC = ceil_div(M, 32);
    uint64_t off = align_up(sizeof(CmapHeader), 256);
    L.off_class_size = off;
    off = align_up(off + 8ull * P, 256);
    L.off_word_off = off;
    off = align_up(off + 8ull * (P + 1), 256);
    L.off_cpre = off;
    off = align_up(off + 4ull * (L.NW + 1) * P, 256);
    L.off_planes = off;
    off = align_up(off + 4ull * L.stride * (L.NC + 1), 256);
    L.bytes = off;
    return L;
}

struct CmapPtrs {
    CmapHeader* hdr;
    uint64_t* class_size;
    uint64_t* word_off;
    uint32_t* cpre;   // [(NW+1)][P]
    uint32_t* planes; // [NC][stride]
};

__host__ __device__ inline CmapPtrs cmap_ptrs(void* base, const CmapLayout& L)
{
    char* b = static_cast<char*>(base);
    CmapPtrs q;
    q.hdr = reinterpret_cast<CmapHeader*>(b);
    q.class_size = reinterpret_cast<uint64_t*>(b + L.off_class_size);
    q.word_off = reinterpret_cast<uint64_t*>(b + L.off_word_off);
    q.cpre = reinterpret_cast<uint32_t*>(b + L.off_cpre);
    q.planes = reinterpret_cast<uint32_t*>(b + L.off_planes);
    return q;
}

// ---------------------------------------------------------------------------
// class map build (setup)
// ---------------------------------------------------------------------------
// one block per window, one thread per 32-key chunk: plane words, and the
// window's class counts (written to cpre, scanned in place afterwards)
__global__ __launch_bounds__(128) void cm_planes_kernel(CmapLayout L, CmapPtrs q, uint32_t seed, Divider div)
{
    __shared__ uint32_t cnt[256];
    const uint64_t win = blockIdx.x;
    for (uint32_t i = threadIdx.x; i < L.P; i += 128) cnt[i] = 0;
    __syncthreads();
    if (threadIdx.x < L.NCW) {
        const uint64_t c = win * L.NCW + threadIdx.x;
        if (c < L.NC) {
            uint32_t planes[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (uint32_t i = 0; i < 32; ++i) {
                const uint64_t key = c * 32 + i;
                if (key >= L.M) break;
                const uint32_t cls = h0((uint32_t)key, seed, div);
                for (uint32_t b = 0; b < L.nbits; ++b) planes[b] |= ((cls >> b) & 1u) << i;
                atomicAdd(&cnt[cls], 1u);
            }
            for (uint32_t b = 0; b < L.stride; ++b) q.planes[c * L.stride + b] = planes[b];
        }
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < L.P; i += 128) q.cpre[win * L.P + i] = cnt[i];
}

// per class: exclusive scan of window counts -> cpre; sizes; word offsets
__global__ __launch_bounds__(256) void cm_scan_kernel(CmapLayout L, CmapPtrs q, uint32_t seed)
{
    const uint32_t p = threadIdx.x;
    __shared__ uint64_t sizes[256];
    if (p < L.P) {
        uint32_t run = 0;
        for (uint64_t w = 0; w < L.NW; ++w) {
            uint32_t c = q.cpre[w * L.P + p];
            q.cpre[w * L.P + p] = run;
            run += c;
        }
        q.cpre[L.NW * L.P + p] = run;
        q.class_size[p] = run;
        sizes[p] = run;
    }
    __syncthreads();
    if (p == 0) {
        uint64_t acc = 0;
        for (uint32_t i = 0; i < L.P; ++i) {
            q.word_off[i] = acc;
            acc += (sizes[i] + 31) / 32;
        }
        q.word_off[L.P] = acc;
        CmapHeader h;
        h.magic = CM_MAGIC;
        h.P = L.P;
        h.M = L.M;
        h.seed = seed;
        h.nbits = L.nbits;
        h.stride = L.stride;
        h.NCW = L.NCW;
        h.W = L.W;
        h.pad = 0;
        h.NW = L.NW;
        h.NC = L.NC;
        *q.hdr = h;
    }
}

// ---------------------------------------------------------------------------
// encode
// ---------------------------------------------------------------------------
struct EncParams {
    CmapLayout L;
    CmapPtrs q;
    const uint32_t* agg_idx;
    const uint64_t* agg_off;
    uint64_t agg_cap;  // entries d_agg_idx holds
    uint32_t* bitmap;
    uint64_t bitmap_words;
    uint64_t* word_off_out;
    uint64_t* cur;     // [(NW+1) * P] first aggregated entry of partition p at or after window w's first key
    uint32_t* side;    // group encode: [groups][P][2] a group's bits in its first and last word when shared
};

// class-p mask of one chunk from its planes (valid = keys of the chunk below M)
__device__ __forceinline__ uint32_t class_mask(const uint32_t* pl, uint32_t nbits, uint32_t p, uint32_t valid)
{
    uint32_t m = valid;
    for (uint32_t b = 0; b < nbits; ++b) m &= ((p >> b) & 1u) ? pl[b] : ~pl[b];
    return m;
}

__device__ __forceinline__ uint32_t chunk_valid(const CmapLayout& L, uint64_t c)
{
    if (c >= L.NC) return 0u;
    const uint64_t left = L.M - c * 32;
    return left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
}

// partition offsets clamped to the aggregate's capacity (into LDS)
__device__ __forceinline__ void load_agg_offsets(const EncParams& e, uint64_t* offs)
{
    const uint32_t P = e.L.P;
    for (uint32_t i = threadIdx.x; i <= P; i += blockDim.x) {
        uint64_t v = e.agg_off[i];
        offs[i] = v > e.agg_cap ? e.agg_cap : v;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Window cursors of sorted partitions (encode and the dense scatter): for key
// windows of 2^wsh keys, cur[w P + p] is the first entry of partition p
// (entries [offs[p], offs[p+1]) of idx, ascending keys) whose key is at or
// after window w's first key, for w in [0, NW]; cur[NW P + p] = offs[p+1].
// ---------------------------------------------------------------------------
// cursors that entry i (key, after prev in its partition p; first: no entry
// before it) sets: it is the first of p in windows (win(prev), win(key)], and
// the last entry also closes the windows after its own
__device__ __forceinline__ void window_cursors_of(uint64_t* cur, uint32_t P, uint32_t NW, uint32_t wsh, uint32_t p,
                                                  uint64_t i, uint32_t key, uint32_t prev, bool first, bool last,
                                                  uint64_t pe)
{
    uint32_t win = key >> wsh;
    if (win >= NW) win = NW - 1;
    uint32_t w = 0;
    if (!first) {
        const uint32_t pw = prev >> wsh;
        w = (pw < NW ? pw : NW - 1) + 1;
    }
    for (; w <= win; ++w) cur[(uint64_t)w * P + p] = i;
    if (last)
        for (w = win + 1; w <= NW; ++w) cur[(uint64_t)w * P + p] = pe;
}

// Chunks of WC_CV * WC_CR * 256 entries: thread t takes WC_CR runs of WC_CV
// consecutive entries, run r at c0 + r WC_CV 256 + t WC_CV, so that one load
// instruction reads 256 contiguous entries of a wave (one 16-byte load per
// lane when VEC: idx 16-byte aligned).
constexpr int WC_CV = 4;
constexpr int WC_CR = 2;
constexpr uint32_t WC_CHUNK = WC_CV * WC_CR * 256;

// The block's share of the pass (256 threads, every thread calls it; offs in
// LDS).  Returns true when a partition's keys do not ascend (the cursors are
// then not those of the definition).  Also fills the cursors of empty
// partitions.
template <bool VEC>
__device__ bool window_cursor_pass(const uint32_t* idx, uint64_t capacity, const uint64_t* offs, uint32_t P,
                                   uint32_t NW, uint32_t wsh, uint64_t* cur)
{
    __shared__ uint32_t lastk[2][256 / SG_WAVE][WC_CR]; // lane 63's last key per wave and run, by chunk parity
    const uint64_t first = offs[0], nagg = offs[P];
    const uint32_t lane = lane_id(), wv = threadIdx.x / SG_WAVE;
    bool bad = false;
    uint32_t par = 0;
    // chunks start at multiples of WC_CV (aligned runs); entries before
    // `first` are not the caller's
    for (uint64_t c0 = (first & ~(uint64_t)(WC_CV - 1)) + blockIdx.x * (uint64_t)WC_CHUNK; c0 < nagg;
         c0 += (uint64_t)gridDim.x * WC_CHUNK, par ^= 1u) {
        uint32_t key[WC_CR][WC_CV];
#pragma unroll
        for (int r = 0; r < WC_CR; ++r) {
            const uint64_t g0 = c0 + (uint64_t)r * WC_CV * 256 + threadIdx.x * WC_CV;
            if (VEC && g0 + WC_CV <= capacity) {
                const uint4 v = *reinterpret_cast<const uint4*>(idx + g0);
                key[r][0] = v.x;
                key[r][1] = v.y;
                key[r][2] = v.z;
                key[r][3] = v.w;
            } else {
#pragma unroll
                for (int c = 0; c < WC_CV; ++c) key[r][c] = idx[g0 + c < capacity ? g0 + c : capacity - 1];
            }
        }
        const uint32_t pk0 = threadIdx.x == 0 && c0 > 0 ? idx[c0 - 1] : 0u; // the entry before the chunk
        uint32_t up[WC_CR];
#pragma unroll
        for (int r = 0; r < WC_CR; ++r) {
            up[r] = (uint32_t)__shfl_up((int)key[r][WC_CV - 1], 1, SG_WAVE);
            if (lane == SG_WAVE - 1) lastk[par][wv][r] = key[r][WC_CV - 1];
        }
        __syncthreads();
        uint32_t p = 0, hi = P;
        uint64_t ps = 0, pe = 0;
#pragma unroll
        for (int r = 0; r < WC_CR; ++r) {
            const uint64_t g0 = c0 + (uint64_t)r * WC_CV * 256 + threadIdx.x * WC_CV;
            if (g0 >= nagg) break;
            // the key before the run: the next lane down's last key; lane 0
            // takes the wave before's (the last wave's of the run before for
            // wave 0, the chunk's predecessor for run 0)
            uint32_t before = up[r];
            if (lane == 0)
                before = wv > 0 ? lastk[par][wv - 1][r] : (r > 0 ? lastk[par][256 / SG_WAVE - 1][r - 1] : pk0);
            if (r == 0) {
                const uint64_t gs = g0 > first ? g0 : first; // largest p with offs[p] <= gs
                while (p + 1 < hi) {
                    const uint32_t mid = (p + hi) >> 1;
                    if (offs[mid] <= gs) p = mid;
                    else hi = mid;
                }
                ps = offs[p];
                pe = offs[p + 1];
            }
            if (g0 > ps && g0 >= first && g0 + WC_CV < pe) {
                // the usual case: the run inside p, neither its first nor its
                // last entry; only a change of window sets cursors
#pragma unroll
                for (int c = 0; c < WC_CV; ++c) {
                    const uint32_t prev = c == 0 ? before : key[r][c - 1];
                    bad = bad || key[r][c] <= prev;
                    if (((key[r][c] ^ prev) >> wsh) != 0u || (key[r][c] >> wsh) >= NW)
                        window_cursors_of(cur, P, NW, wsh, p, g0 + c, key[r][c], prev, false, false, pe);
                }
            } else {
#pragma unroll
                for (int c = 0; c < WC_CV; ++c) {
                    const uint64_t i = g0 + c;
                    if (i >= nagg) break;
                    if (i < first) continue;
                    const uint32_t prev = c == 0 ? before : key[r][c - 1];
                    while (i >= pe) { // into the next non-empty partition
                        ++p;
                        ps = offs[p];
                        pe = offs[p + 1];
                    }
                    if (i > ps && key[r][c] <= prev) bad = true;
                    window_cursors_of(cur, P, NW, wsh, p, i, key[r][c], prev, i == ps, i == pe - 1, pe);
                }
            }
        }
    }
    // cursors of empty partitions
    const uint64_t nthreads = (uint64_t)gridDim.x * 256;
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < ((uint64_t)NW + 1) * P; i += nthreads) {
        const uint32_t p = (uint32_t)(i % P);
        if (offs[p + 1] == offs[p]) cur[i] = offs[p];
    }
    return bad;
}

// Window cursors (the pass above, at the class map's window size), the
// cursors of empty partitions, and the bitmap words that two neighbouring
// groups of gw windows share zeroed (the encode kernels merge them with
// atomicOr).
template <bool VEC>
__global__ __launch_bounds__(256) void enc_prep_kernel(EncParams e, uint32_t gw)
{
    __shared__ uint64_t offs[257];
    load_agg_offsets(e, offs);
    const uint32_t P = e.L.P;
    const uint64_t NW = e.L.NW;
    window_cursor_pass<VEC>(e.agg_idx, e.agg_cap, offs, P, (uint32_t)NW, (uint32_t)__builtin_ctzll(e.L.W), e.cur);
    const uint32_t tid32 = blockIdx.x * 256 + threadIdx.x, nth32 = gridDim.x * 256;
    for (uint32_t i = tid32; gw != 0 && i < (uint32_t)(NW * P); i += nth32) {
        const uint32_t w = i / P;
        const uint32_t p = i % P;
        if (gw == 0 || w == 0 || w % gw != 0) continue; // only words shared by two groups of gw windows
        const uint32_t a = e.q.cpre[(uint64_t)w * P + p];
        if ((a & 31u) == 0 || a >= e.q.class_size[p]) continue;
        const uint64_t gw = e.q.word_off[p] + (a >> 5);
        if (gw < e.bitmap_words) e.bitmap[gw] = 0u;
    }
}

// A block per window of W keys (blocks loop over windows), all partitions
// together: class masks of
// the window's chunks and their per-class prefix counts in LDS; every
// aggregated key of the window (loaded in one round, its range known from the
// cursors) sets the bit of its rank in an LDS copy of the window's bitmap
// words; the words are then written out.
// six waves per SIMD (80 registers, a few spilled) keep more windows in
// flight than the five the unconstrained allocation allows
__global__ __launch_bounds__(EN_THREADS) __attribute__((amdgpu_waves_per_eu(6))) void enc_kernel(EncParams e)
{
    constexpr int KB = 4; // keys per thread per load round
    // partition-major [P][NCW] (NCW*P <= 2048): a thread's 8 chunks of one
    // partition are 16-byte accesses, consecutive threads on consecutive
    // addresses
    __shared__ __align__(16) uint32_t masks[2048];
    __shared__ __align__(16) uint16_t pre[2048];
    __shared__ uint32_t seg[EN_SEG_WORDS];
    __shared__ uint32_t segofs[257], kof[257], a_bits[256], b_bits[256];
    __shared__ uint64_t kbeg[256];
    __shared__ uint32_t scan_lds[EN_THREADS / SG_WAVE + 1];

    const CmapLayout& L = e.L;
    const uint32_t P = L.P, NCW = L.NCW;
    const uint32_t lane = lane_id();
    for (uint64_t win = blockIdx.x; win < L.NW; win += gridDim.x) {
    const uint64_t wstart = win * L.W;

    if (win == 0)
        for (uint32_t i = threadIdx.x; i <= P; i += EN_THREADS) e.word_off_out[i] = e.q.word_off[i];
    if (win == 0 && threadIdx.x == 0) {
        const CmapHeader h = *e.q.hdr;
        if (h.magic != CM_MAGIC || h.P != P || h.M != L.M) report_error(kDevErrCmap);
    }

    // every independent load first: the chunk's bit planes, the partition's
    // offsets, cursors and class prefixes
    uint32_t pl[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t valid = 0;
    if (threadIdx.x < NCW) {
        const uint64_t c = win * NCW + threadIdx.x;
        valid = chunk_valid(L, c);
        if (valid)
            for (uint32_t b = 0; b < L.nbits; ++b) pl[b] = e.q.planes[c * L.stride + b];
    }
    // key ranges and bitmap word ranges of the window per partition
    uint32_t kc = 0, nw = 0;
    if (threadIdx.x < P) {
        const uint32_t p = threadIdx.x;
        uint64_t s = e.agg_off[p], en = e.agg_off[p + 1];
        s = s > e.agg_cap ? e.agg_cap : s;
        en = en > e.agg_cap ? e.agg_cap : (en < s ? s : en);
        uint64_t a = e.cur[win * P + p], b = e.cur[(win + 1) * P + p];
        a = a < s ? s : (a > en ? en : a);
        b = b < a ? a : (b > en ? en : b);
        if (b - a > L.W) b = a + L.W; // at most W keys fall in a window (valid input)
        kbeg[p] = a;
        kc = (uint32_t)(b - a);
        const uint32_t ca = e.q.cpre[win * P + p], cb = e.q.cpre[(win + 1) * P + p];
        a_bits[p] = ca;
        b_bits[p] = cb;
        nw = cb > ca ? ((cb - 1) >> 5) - (ca >> 5) + 1 : 0u;
    }
    uint32_t K, nseg;
    const uint32_t ko = block_excl_scan<EN_THREADS>(kc, scan_lds, &K);
    __syncthreads();
    const uint32_t so = block_excl_scan<EN_THREADS>(nw, scan_lds, &nseg);
    if (threadIdx.x < P) {
        kof[threadIdx.x] = ko;
        segofs[threadIdx.x] = so;
    }
    if (threadIdx.x == 0) {
        kof[P] = K;
        segofs[P] = nseg;
    }
    for (uint32_t i = threadIdx.x; i < EN_SEG_WORDS; i += EN_THREADS) seg[i] = 0u;
    __syncthreads();
    if (nseg > EN_SEG_WORDS) { // cannot happen: at most W/32 + P words
        if (threadIdx.x == 0) report_error(kDevErrCmap);
        __syncthreads();
        continue;
    }
    // issue the first round of key loads before building the masks
    uint32_t key[KB], kp[KB];
    auto load_round = [&](uint32_t j0) {
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const uint32_t j = j0 + u * EN_THREADS + threadIdx.x;
            kp[u] = 0xffffffffu;
            key[u] = 0;
            if (j < K) {
                uint32_t lo = 0, hi = P; // largest p with kof[p] <= j
                while (lo + 1 < hi) {
                    const uint32_t mid = (lo + hi) >> 1;
                    if (kof[mid] <= j) lo = mid;
                    else hi = mid;
                }
                kp[u] = lo;
                key[u] = e.agg_idx[kbeg[lo] + (j - kof[lo])];
            }
        }
    };
    load_round(0);

    // a) class masks of the window's chunks (NCW <= 128 < EN_THREADS); up to
    //    16 classes by splitting: each level splits every mask by one plane
    if (threadIdx.x < NCW) {
        uint32_t* mrow = masks + threadIdx.x; // class k at mrow[k * NCW]
        if (L.nbits <= 4) {
            uint32_t m[16];
            m[0] = valid;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if ((uint32_t)b < L.nbits) {
#pragma unroll
                    for (int k = (1 << b) - 1; k >= 0; --k) { // class id bit b set: m & plane_b
                        m[k + (1 << b)] = m[k] & pl[b];
                        m[k] &= ~pl[b];
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if ((uint32_t)k < P) mrow[k * NCW] = m[k];
        } else {
            for (uint32_t p = 0; p < P; ++p) mrow[p * NCW] = class_mask(pl, L.nbits, p, valid);
        }
    }
    __syncthreads();
    // b) per-partition prefix over the chunks of the window: the NCW*P counts
    //    as P segments of NCW (partition-major), 8 per thread, then a
    //    segmented scan over the NCW/8 <= 16 threads of a segment (inside one
    //    DPP row)
    {
        const uint32_t e0 = threadIdx.x * 8;
        uint32_t c[8], run = 0;
        const bool act = e0 < NCW * P;
        const uint4 ma = act ? *reinterpret_cast<const uint4*>(&masks[e0]) : make_uint4(0u, 0u, 0u, 0u);
        const uint4 mb = act ? *reinterpret_cast<const uint4*>(&masks[e0 + 4]) : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t mw[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w}; // 8 chunks of one partition
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            c[j] = __popc(mw[j]);
            run += c[j];
        }
        const uint32_t sg = NCW / 8; // threads per segment: a power of two, at most 16
        const uint32_t inrow = lane & 15u;
        uint32_t inc = run, x;
        x = dpp_move<kDppRowShr1>(0u, inc);
        if (sg > 1 && (inrow & (sg - 1)) >= 1) inc += x;
        x = dpp_move<kDppRowShr2>(0u, inc);
        if (sg > 2 && (inrow & (sg - 1)) >= 2) inc += x;
        x = dpp_move<kDppRowShr4>(0u, inc);
        if (sg > 4 && (inrow & (sg - 1)) >= 4) inc += x;
        x = dpp_move<kDppRowShr8>(0u, inc);
        if (sg > 8 && (inrow & (sg - 1)) >= 8) inc += x;
        if (act) {
            uint32_t ex[8];
            ex[0] = inc - run;
#pragma unroll
            for (int j = 1; j < 8; ++j) ex[j] = ex[j - 1] + c[j - 1];
            *reinterpret_cast<uint4*>(&pre[e0]) = make_uint4(ex[0] | (ex[1] << 16), ex[2] | (ex[3] << 16),
                                                            ex[4] | (ex[5] << 16), ex[6] | (ex[7] << 16));
        }
    }
    __syncthreads();
    // c) the bit of every aggregated key: its rank in its class
    for (uint32_t j0 = 0; j0 < K; j0 += KB * EN_THREADS) {
        if (j0 > 0) load_round(j0);
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            if (kp[u] == 0xffffffffu) continue;
            const uint32_t p = kp[u];
            const uint64_t o = (uint64_t)key[u] - wstart;
            if (key[u] < wstart || o >= L.W) { // not in this window: cannot happen for valid input
                report_error(kDevErrPartition);
                continue;
            }
            const uint32_t t = (uint32_t)(o >> 5), bit = (uint32_t)(o & 31u);
            const uint32_t mk = masks[p * NCW + t];
            if (!((mk >> bit) & 1u)) report_error(kDevErrPartition);
            const uint32_t r = a_bits[p] + pre[p * NCW + t] + __popc(mk & ((1u << bit) - 1u));
            const uint32_t lw = (r >> 5) - (a_bits[p] >> 5);
            if (lw < segofs[p + 1] - segofs[p]) atomicOr(&seg[segofs[p] + lw], 1u << (r & 31u));
        }
    }
    __syncthreads();
    // d) write the window's words: plain stores for words inside the window,
    //    atomicOr for the words shared with a neighbour (pre-zeroed)
    for (uint32_t i = threadIdx.x; i < nseg; i += EN_THREADS) {
        uint32_t lo = 0, hi = P; // partition of segment word i
        while (lo + 1 < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (segofs[mid] <= i) lo = mid;
            else hi = mid;
        }
        const uint32_t p = lo;
        const uint32_t a = a_bits[p], b = b_bits[p];
        const uint32_t qw = (a >> 5) + (i - segofs[p]);
        const uint64_t csize = e.q.class_size[p];
        const bool excl = (uint64_t)qw * 32 >= a && ((uint64_t)(qw + 1) * 32 <= b || (uint64_t)b == csize);
        const uint64_t gw = e.q.word_off[p] + qw;
        if (gw >= e.bitmap_words) continue;
        const uint32_t v = seg[i];
        if (excl) e.bitmap[gw] = v;
        else if (v) atomicOr(&e.bitmap[gw], v);
    }
    __syncthreads(); // LDS is reused by the block's next window
    }
}


// ---------------------------------------------------------------------------
// Group encode, 2 <= P <= 16 and at least 2048 groups: a wave per group of
// G consecutive windows (G = 4 for 9..16 classes, else 1), no block barrier.
// Loads run a window ahead (planes, cursors, the first rounds of keys).  Per
// window the wave
//   a) splits the planes of the window's 128 chunks (two per lane) into the
//      class masks of both chunks (one AND per mask and plane level), counts
//      every class in them as 16-bit fields packed two classes to a register
//      and scans those registers over the lanes: each chunk's LDS record holds
//      its planes and its per-class count of the window's keys before it;
//   b) takes the window's aggregated keys in rounds of 64 per partition: a
//      round's keys are laid end to end in LDS with their class, and each
//      lane then takes a run of them (the lanes of one step far apart, so
//      their bits rarely share a word): a key's bit is its rank in its class
//      (the class's bits before the window, the chunk's prefix, the class
//      members before it in the chunk), OR-ed into an LDS copy of the group's
//      bitmap words.
// After the group the words go out class by class, each class's bits of the
// group one contiguous run written with consecutive lanes on consecutive
// words (for 16 classes and G = 4 about 32 words, 128 bytes).  The first and
// last word of a run may hold bits of a neighbouring group: those go to a
// side buffer, and enc_fix_kernel writes each such word once, as the OR of
// every group's part (no global atomics, nothing zeroed beforehand).
// ---------------------------------------------------------------------------
constexpr int EG_WAVES = 4; // waves per block, each on a group of its own
constexpr uint32_t EG_NCW = 128; // chunks of a class-map window (P <= 16)

template <int NB>
struct EgShape {
    static constexpr int NCLS = 1 << NB;                            // class ids the planes can hold
    static constexpr int STRIDE = NB == 1 ? 1 : (NB == 2 ? 2 : 4);  // plane words per chunk in the class map
    static constexpr int NPK = NCLS / 2;                            // prefix words per chunk: two 16-bit counts
    static constexpr int REC = STRIDE + NPK;                        // LDS words per chunk record
    static constexpr uint32_t G = NB == 4 ? 4 : 1;                  // windows per group (measured best)
    static constexpr uint32_t SEG = G * EG_NCW + 2 * NCLS;          // bitmap words of a group, at most
};

// plane words of chunk c (c <= NC: the class map holds NC + 1 chunks)
template <int NB>
__device__ __forceinline__ void eg_load_planes(const uint32_t* planes, uint64_t c, uint32_t (&pl)[4])
{
    using S = EgShape<NB>;
    if (S::STRIDE == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(planes + c * 4);
        pl[0] = v.x; pl[1] = v.y; pl[2] = v.z; pl[3] = v.w;
    } else if (S::STRIDE == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(planes + c * 2);
        pl[0] = v.x; pl[1] = v.y; pl[2] = 0u; pl[3] = 0u;
    } else {
        pl[0] = planes[c]; pl[1] = 0u; pl[2] = 0u; pl[3] = 0u;
    }
}

// class masks of one chunk: m[k] = the chunk's keys of class k
template <int NB>
__device__ __forceinline__ void eg_masks(const uint32_t (&pl)[4], uint32_t valid, uint32_t (&m)[1 << NB])
{
    m[0] = valid;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int k = (1 << b) - 1; k >= 0; --k) { // class id bit b set: m & plane_b
            m[k + (1 << b)] = m[k] & pl[b];
            m[k] &= ~pl[b];
        }
    }
}

// rounds 0 .. KR-1 of every partition's keys of a window whose entries start
// at tlo[p] (LDS; partitions past P hold entry 0 and are never used)
template <int NB, int KR>
__device__ __forceinline__ void eg_first_loads(const uint32_t* keys, uint64_t last, const uint64_t* tlo,
                                               uint32_t (&kreg)[1 << NB][KR])
{
#pragma unroll
    for (int p = 0; p < (1 << NB); ++p)
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const uint64_t i = tlo[p] + (uint64_t)r * SG_WAVE + lane_id();
            kreg[p][r] = keys[i < last ? i : last];
        }
}

// RR rounds of a window's keys: entries 64 r0 .. 64 (r0 + RR) - 1 of every
// partition's range (key[p][q] in lane l: entry 64 (r0 + q) + l of partition
// p; cnt in lane p: the window's count of partition p).  The keys are first
// laid end to end in LDS, each as its window offset and its class
// (o | p << 16; offset 0xffff: outside the window), then every lane takes
// whole staged keys, four at a time with all their LDS reads issued
// together: the bit of a key is its rank in its class (the class's bits
// before the window, tab[p].x, plus the chunk's prefix and the class members
// before it inside the chunk), OR-ed into the group's LDS words.  A key
// outside the window, not of its class, or with a bit outside its class's
// words sets `bad`.
template <int NB, int RR>
__device__ __forceinline__ void eg_rounds(const uint4* tab, const uint32_t* rec, uint32_t* seg, uint32_t* stage,
                                          uint32_t wstart, uint32_t r0, const uint32_t (&key)[1 << NB][RR],
                                          uint32_t cnt, bool cl, bool& bad)
{
    using S = EgShape<NB>;
    constexpr uint32_t W = EG_NCW * 32u;
    constexpr uint32_t SKIP = 0xffffffffu;
    const uint32_t lane = lane_id();
    const uint32_t rem = cl && cnt > r0 * SG_WAVE ? cnt - r0 * SG_WAVE : 0u;
    const uint32_t c = rem < RR * SG_WAVE ? rem : RR * SG_WAVE;
    const uint32_t incl = wave_incl_scan(c);
    const uint32_t off = incl - c;
    const uint32_t K = lane_value(incl, SG_WAVE - 1);
#pragma unroll
    for (int p = 0; p < (1 << NB); ++p) {
        const uint32_t cp = lane_value(c, p), op = lane_value(off, p);
#pragma unroll
        for (int q = 0; q < RR; ++q) {
            const uint32_t o = key[p][q] - wstart;
            if (q * SG_WAVE + lane < cp) stage[op + q * SG_WAVE + lane] = (o < W ? o : 0xffffu) | ((uint32_t)p << 16);
        }
    }
    wave_sync();
    // lane l takes staged keys l Kq .. l Kq + Kq - 1 (Kq odd): the lanes of
    // one step hold keys Kq apart, so their bits rarely share an LDS word
    // (same-word atomics serialize), and the stage reads hit distinct banks
    const uint32_t Kq = ((K + SG_WAVE - 1) / SG_WAVE) | 1u;
    for (uint32_t i0 = 0; i0 < Kq; i0 += 4) {
        uint32_t u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t j = lane * Kq + i0 + q;
            const bool in = i0 + q < Kq && j < K;
            u[q] = stage[in ? j : 0];
            u[q] = in ? u[q] : SKIP;
        }
        uint4 t[4], pv[4];
        uint32_t pre[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t o = u[q] & 0xffffu, p = (u[q] >> 16) & 0xffu;
            const uint32_t ch = o < W ? (o >> 5) : 0u;
            const uint32_t* rp = rec + ch * S::REC;
            t[q] = tab[p < (1u << NB) ? p : 0u]; // x: base bit, y: first word, z: words
            if (S::STRIDE == 4) pv[q] = *reinterpret_cast<const uint4*>(rp);
            else if (S::STRIDE == 2) pv[q] = make_uint4(rp[0], rp[1], 0u, 0u);
            else pv[q] = make_uint4(rp[0], 0u, 0u, 0u);
            pre[q] = reinterpret_cast<const uint16_t*>(rp + S::STRIDE)[p < (1u << NB) ? p : 0u];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (u[q] == SKIP) continue;
            const uint32_t o = u[q] & 0xffffu, p = u[q] >> 16;
            const uint32_t pl[4] = {pv[q].x, pv[q].y, pv[q].z, pv[q].w};
            // the class-p members of the chunk: plane b where p has bit b, else its complement
            uint32_t m = 0xffffffffu;
#pragma unroll
            for (int b = 0; b < NB; ++b) m &= pl[b] ^ (((p >> b) & 1u) - 1u);
            const uint32_t bit = o & 31u;
            const uint32_t pos = t[q].x + pre[q] + __popc(m & ((1u << bit) - 1u));
            if (o >= W || !((m >> bit) & 1u) || (pos >> 5) - t[q].y >= t[q].z) {
                bad = true;
                continue;
            }
            atomicOr(&seg[pos >> 5], 1u << (pos & 31u));
        }
    }
    wave_sync(); // the stage is read before the next round writes it
}

template <int NB, int KR>
__global__ __launch_bounds__(EG_WAVES * SG_WAVE) void enc_group_kernel(EncParams e, uint64_t NG)
{
    using S = EgShape<NB>;
    constexpr int NCLS = S::NCLS;
    constexpr uint32_t W = EG_NCW * 32u;
    __shared__ __align__(16) uint32_t rec_all[EG_WAVES][EG_NCW * S::REC];
    __shared__ __align__(16) uint32_t seg_all[EG_WAVES][S::SEG];
    __shared__ __align__(16) uint32_t stage_all[EG_WAVES][NCLS * SG_WAVE * KR];
    __shared__ __align__(16) uint4 tab_all[EG_WAVES][NCLS];
    __shared__ uint64_t tlo_all[EG_WAVES][2][NCLS];
    const uint32_t wv = threadIdx.x / SG_WAVE, lane = lane_id();
    uint32_t* rec = rec_all[wv];
    uint32_t* seg = seg_all[wv];
    uint32_t* stage = stage_all[wv];
    uint4* tab = tab_all[wv];
    const uint64_t g = (uint64_t)blockIdx.x * EG_WAVES + wv;
    if (g >= NG) return; // the whole wave: nothing below waits for other waves
    const CmapLayout& L = e.L;
    const uint32_t P = L.P;
    const uint64_t NW = L.NW;
    const uint64_t w0 = g * S::G;
    const uint64_t w1 = w0 + S::G < NW ? w0 + S::G : NW;
    const uint64_t cap = e.agg_cap;
    const bool cl = lane < P; // lane p holds class p's values
    const uint32_t pc = cl ? lane : 0u;

    if (g == 0) {
        if (lane <= P) e.word_off_out[lane] = e.q.word_off[lane];
        if (lane == 0) {
            const CmapHeader h = *e.q.hdr;
            if (h.magic != CM_MAGIC || h.P != P || h.M != L.M) report_error(kDevErrCmap);
        }
    }

    // the class's bits [A, B) of the group, its words, the partition's entries
    uint32_t A = e.q.cpre[w0 * P + pc], B = e.q.cpre[w1 * P + pc];
    uint64_t s = e.agg_off[pc], en = e.agg_off[pc + 1];
    uint64_t lo = e.cur[w0 * P + pc], hi = e.cur[(w0 + 1) * P + pc];
    if (!cl) { // lanes past P: an empty class
        A = B = 0;
        s = en = lo = hi = 0;
    }
    s = s > cap ? cap : s;
    en = en > cap ? cap : (en < s ? s : en);
    lo = lo < s ? s : (lo > en ? en : lo);
    hi = hi < lo ? lo : (hi > en ? en : hi);
    const uint32_t nw = B > A ? ((B - 1u) >> 5) - (A >> 5) + 1u : 0u;
    const uint32_t nincl = wave_incl_scan(nw);
    const uint32_t so = nincl - nw;
    const uint32_t nseg = lane_value(nincl, SG_WAVE - 1);
    if (nseg > S::SEG) { // cannot happen with a valid class map
        if (lane == 0) report_error(kDevErrCmap);
        return;
    }
    uint32_t cw = A; // the class's bits before the window
    const uint32_t segbase = 32u * so - 32u * (A >> 5);

    // Loads run a window ahead: window w's planes, cursors and first key
    // rounds are issued while window w - 1 is worked on.  The window loop is
    // unrolled with two register sets used in turn, so no loaded register
    // is copied (a copy would wait for the load at once).
    uint32_t pl[2][8];
    uint32_t kreg[2][NCLS][KR];
    uint64_t hin[2];
    uint32_t cwn[2];
    // every load below is unconditional (clamped indices, a one-word stand-in
    // for an empty aggregate), so the compiler waits for each where it is
    // used and not at a branch
    const uint32_t* keys = cap > 0 ? e.agg_idx : reinterpret_cast<const uint32_t*>(e.q.word_off);
    const uint64_t klast = cap > 0 ? cap - 1 : 0;
    auto issue = [&](int set, uint64_t w, uint64_t* tl) {
        w = w < NW ? w : NW - 1;
        const uint64_t ca = w * EG_NCW + 2 * lane, cb = ca + 1;
        uint32_t pa[4], pb[4];
        eg_load_planes<NB>(e.q.planes, ca < L.NC ? ca : L.NC, pa);
        eg_load_planes<NB>(e.q.planes, cb < L.NC ? cb : L.NC, pb);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            pl[set][b] = pa[b];
            pl[set][4 + b] = pb[b];
        }
        eg_first_loads<NB, KR>(keys, klast, tl, kreg[set]);
        hin[set] = e.cur[((w + 2 <= NW ? w + 2 : NW)) * P + pc];
        cwn[set] = e.q.cpre[(w + 1) * P + pc];
    };
    for (uint32_t i = lane * 4; i < nseg; i += SG_WAVE * 4)
        *reinterpret_cast<uint4*>(&seg[i]) = make_uint4(0u, 0u, 0u, 0u);
    if (lane < (uint32_t)NCLS) tlo_all[wv][0][lane] = lo;
    wave_sync();
    issue(0, w0, tlo_all[wv][0]);

    bool bad = false;
#pragma unroll
    for (uint32_t wi = 0; wi < S::G; ++wi) {
        const uint64_t w = w0 + wi;
        if (w >= w1) break;
        const int cs = wi & 1, ns = cs ^ 1;
        const uint32_t wstart = (uint32_t)(w * W);
        const uint64_t* tlo = tlo_all[wv][cs];
        const uint32_t cnt = (uint32_t)(hi - lo > W ? W : hi - lo); // at most W keys fall in a window (valid input)
        // the next window's loads (its keys start where this window's end)
        if (wi + 1 < S::G) { // (past the group's last window: loads of a window not used)
            if (lane < (uint32_t)NCLS) tlo_all[wv][ns][lane] = hi;
            wave_sync();
            issue(ns, w + 1, tlo_all[wv][ns]);
        }
        // a) class counts of the lane's two chunks, 16-bit fields two classes
        //    to a register; their exclusive scan over the lanes
        const uint64_t ca = w * EG_NCW + 2 * lane, cb = ca + 1;
        uint32_t pa[4], pb[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            pa[b] = pl[cs][b];
            pb[b] = pl[cs][4 + b];
        }
        uint32_t cpa[S::NPK], tot[S::NPK];
        {
            uint32_t m[NCLS];
            eg_masks<NB>(pa, chunk_valid(L, ca), m);
#pragma unroll
            for (int i = 0; i < S::NPK; ++i) cpa[i] = __popc(m[2 * i]) | (__popc(m[2 * i + 1]) << 16);
            eg_masks<NB>(pb, chunk_valid(L, cb), m);
#pragma unroll
            for (int i = 0; i < S::NPK; ++i) tot[i] = cpa[i] + (__popc(m[2 * i]) | (__popc(m[2 * i + 1]) << 16));
        }
        if (lane < (uint32_t)NCLS) tab[lane] = make_uint4(segbase + cw, so, nw, 0u);
        {
            uint32_t* ra = rec + (2 * lane) * S::REC;
            uint32_t* rb = ra + S::REC;
            uint32_t va[S::REC], vb[S::REC];
#pragma unroll
            for (int b = 0; b < S::STRIDE; ++b) {
                va[b] = pa[b];
                vb[b] = pb[b];
            }
#pragma unroll
            for (int i = 0; i < S::NPK; ++i) {
                const uint32_t ex = wave_incl_scan(tot[i]) - tot[i];
                va[S::STRIDE + i] = ex;
                vb[S::STRIDE + i] = ex + cpa[i];
            }
            if (S::REC % 4 == 0) {
#pragma unroll
                for (int q = 0; q < S::REC; q += 4) {
                    *reinterpret_cast<uint4*>(ra + q) = make_uint4(va[q], va[q + 1], va[q + 2], va[q + 3]);
                    *reinterpret_cast<uint4*>(rb + q) = make_uint4(vb[q], vb[q + 1], vb[q + 2], vb[q + 3]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < S::REC; ++q) {
                    ra[q] = va[q];
                    rb[q] = vb[q];
                }
            }
        }
        wave_sync();
        // b) the keys, 64 entries of every partition per round: the rounds
        //    loaded ahead, then any further rounds (dense windows)
        const uint32_t maxcnt = wave_max(cl ? cnt : 0u);
        eg_rounds<NB, KR>(tab, rec, seg, stage, wstart, 0, kreg[cs], cnt, cl, bad);
        for (uint32_t r = KR; r * SG_WAVE < maxcnt; ++r) {
            uint32_t kr[NCLS][1];
#pragma unroll
            for (int p = 0; p < NCLS; ++p) {
                const uint64_t i = tlo[p] + r * SG_WAVE + lane;
                kr[p][0] = keys[i < klast ? i : klast];
            }
            eg_rounds<NB, 1>(tab, rec, seg, stage, wstart, r, kr, cnt, cl, bad);
        }
        // next window
        lo = hi;
        hi = hin[cs] < lo ? lo : (hin[cs] > en ? en : hin[cs]);
        cw = cwn[cs];
    }
    if (bad) report_error(kDevErrPartition);
    wave_sync();
    // the group's words, class by class
    uint64_t csz = 0, wbv = 0;
    if (cl) {
        csz = e.q.class_size[pc];
        wbv = e.q.word_off[pc] + (A >> 5);
    }
#pragma unroll
    for (int p = 0; p < NCLS; ++p) {
        if ((uint32_t)p >= P) continue;
        const uint32_t nwp = lane_value(nw, p), sop = lane_value(so, p);
        const uint32_t Ap = lane_value(A, p), Bp = lane_value(B, p);
        const uint64_t csize = lane_value64(csz, p), wbase = lane_value64(wbv, p);
        for (uint32_t j = lane; j < nwp; j += SG_WAVE) {
            const uint32_t val = seg[sop + j];
            // a word is shared when it also holds bits of the group before
            // (its first) or after (its last, unless the class ends there)
            const bool first = j == 0 && (Ap & 31u) != 0u;
            const bool last = j == nwp - 1 && (Bp & 31u) != 0u && (uint64_t)Bp < csize;
            uint32_t* sd = e.side + (g * P + p) * 2;
            if (first) sd[0] = val;
            if (last) sd[1] = val;
            const uint64_t gw = wbase + j;
            if (!first && !last && gw < e.bitmap_words) e.bitmap[gw] = val;
        }
    }
}

// The words the group encode shares between groups: the word X holding a
// group's first bit A when A is not at a word start.  The last group with
// bits in X (its bits run past X, or the class ends in X) writes it: its own
// first-word bits OR the last-word bits of the groups before it that reach
// into X.  A thread per (group, class).
__global__ __launch_bounds__(256) void enc_fix_kernel(EncParams e, uint64_t NG, uint32_t G)
{
    const uint64_t t = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    const uint32_t P = e.L.P;
    if (t >= NG * P) return;
    const uint64_t g = t / P;
    const uint32_t p = (uint32_t)(t % P);
    const uint64_t NW = e.L.NW;
    auto start = [&](uint64_t h) -> uint32_t { // class-p bits before group h
        const uint64_t w = h * G < NW ? h * G : NW;
        return e.q.cpre[w * P + p];
    };
    const uint32_t A = start(g), B = start(g + 1);
    const uint64_t csize = e.q.class_size[p];
    if (B <= A || (A & 31u) == 0u) return;
    const uint32_t X = A >> 5;
    if (!((uint64_t)B >= 32ull * (X + 1) || (uint64_t)B == csize)) return; // a later group writes X
    uint32_t v = e.side[(g * P + p) * 2];
    for (uint64_t h = g; h-- > 0;) {
        const uint32_t a = start(h), b = start(h + 1);
        if (b <= 32u * X) break; // no bits in X
        if (b <= a) continue;    // no bits at all
        v |= e.side[(h * P + p) * 2 + 1];
        if ((a >> 5) < X || (a & 31u) == 0u) break; // it starts at or before X's first bit
    }
    const uint64_t gw = e.q.word_off[p] + X;
    if (gw < e.bitmap_words) e.bitmap[gw] = v;
}

// windows per group of the group encode for this layout (0: the block-per-
// window encode, for P = 1, P > 16 or fewer windows than fill the chip)
static uint32_t enc_group_windows(const CmapLayout& L)
{
    if (L.P < 2 || L.P > 16 || L.NCW != EG_NCW) return 0;
    const uint32_t G = L.nbits == 4 ? EgShape<4>::G : (L.nbits == 3 ? EgShape<3>::G : 1u);
    if (ceil_div(L.NW, G) < 2048) return 0;
    return G;
}

} // namespace sg

using namespace sg;

extern "C" size_t sg_classmap_bytes(uint64_t M, uint32_t P)
{
    if (P == 0 || P > 256) return 0;
    return cmap_layout(M, P).bytes;
}

extern "C" int sg_classmap_build(uint64_t M, uint32_t P, uint32_t seed, void* d_cmap, size_t cmap_bytes,
                                 void* stream)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32) || !d_cmap) return SG_EINVAL;
    const CmapLayout L = cmap_layout(M, P);
    if (cmap_bytes < L.bytes) return SG_ECAPACITY;
    hipStream_t st = as_stream(stream);
    CmapPtrs q = cmap_ptrs(d_cmap, L);
    cm_planes_kernel<<<(unsigned)L.NW, 128, 0, st>>>(L, q, seed, make_divider(P));
    SG_TRY_LAUNCH();
    cm_scan_kernel<<<1, 256, 0, st>>>(L, q, seed);
    SG_TRY_LAUNCH();
    return SG_OK;
}

extern "C" uint64_t sg_encode_max_words(uint64_t M, uint32_t P) { return M / 32 + P + 1; }

// Workspace: the window cursors, (NW + 1) * P words of 8 bytes.
extern "C" size_t sg_encode_workspace_bytes(uint64_t M, uint32_t P)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32)) return 0;
    const CmapLayout L = cmap_layout(M, P);
    const uint64_t cur = align_up(8ull * (L.NW + 1) * P, 256);
    const uint32_t G = enc_group_windows(L);
    return (size_t)(cur + (G ? 8ull * ceil_div(L.NW, G) * P : 0));
}

extern "C" int sg_encode(const uint32_t* d_agg_idx, const uint64_t* d_agg_off, uint64_t agg_capacity, uint64_t M,
                         uint32_t P, const void* d_cmap, size_t cmap_bytes, uint32_t* d_bitmap, uint64_t bitmap_words, uint64_t* d_word_off,
                         void* d_ws, size_t ws_bytes, void* stream)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32)) return SG_EINVAL;
    if (!d_agg_off || !d_cmap || !d_bitmap || !d_word_off || !d_agg_idx || !d_ws) return SG_EINVAL;
    if (ws_bytes < sg_encode_workspace_bytes(M, P)) return SG_ECAPACITY;
    if (bitmap_words < sg_encode_max_words(M, P)) return SG_ECAPACITY;
    if (cmap_bytes < sg_classmap_bytes(M, P)) return SG_ECAPACITY;
    EncParams e;
    e.L = cmap_layout(M, P);
    e.q = cmap_ptrs(const_cast<void*>(d_cmap), e.L);
    e.agg_idx = d_agg_idx;
    e.agg_off = d_agg_off;
    e.agg_cap = agg_capacity;
    e.bitmap = d_bitmap;
    e.bitmap_words = bitmap_words;
    e.word_off_out = d_word_off;
    e.cur = static_cast<uint64_t*>(d_ws);
    e.side = reinterpret_cast<uint32_t*>(static_cast<char*>(d_ws) + align_up(8ull * (e.L.NW + 1) * P, 256));
    // a window's words never exceed W/32 + P
    if (e.L.W / 32 + P + 2 > (uint64_t)EN_SEG_WORDS) return SG_EUNSUPPORTED;
    hipStream_t st = as_stream(stream);
    // a chunk of entries per block where they allow, and enough blocks for
    // the per-window work
    uint64_t pblocks = ceil_div(agg_capacity, (uint64_t)WC_CHUNK);
    const uint64_t fill = ceil_div((e.L.NW + 1) * P, 1024);
    pblocks = pblocks > fill ? pblocks : fill;
    pblocks = pblocks < 4096 ? (pblocks ? pblocks : 1) : 4096;
    // 2 <= P <= 16 and enough windows: a wave per group of windows, the
    // shared words merged by a fix-up pass; otherwise a block per window, the
    // shared words zeroed here and merged with atomicOr
    const uint32_t nb = e.L.nbits;
    const uint32_t G = enc_group_windows(e.L);
    const bool group = G != 0;
    if ((uintptr_t)d_agg_idx % 16 == 0)
        enc_prep_kernel<true><<<(unsigned)pblocks, 256, 0, st>>>(e, group ? 0u : 1u);
    else
        enc_prep_kernel<false><<<(unsigned)pblocks, 256, 0, st>>>(e, group ? 0u : 1u);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_ENCODE, st);
    if (group) {
        const uint64_t NG = ceil_div(e.L.NW, G);
        const unsigned blocks = (unsigned)ceil_div(NG, (uint64_t)EG_WAVES);
        // two rounds of 64 keys per partition loaded ahead when the entries
        // (an upper bound on the union) average more than 80 per partition
        // and window
        const bool kr2 = agg_capacity > 80ull * e.L.NW * P;
        switch (nb * 2 + (kr2 ? 1 : 0)) {
        case 2: enc_group_kernel<1, 1><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        case 3: enc_group_kernel<1, 2><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        case 4: enc_group_kernel<2, 1><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        case 5: enc_group_kernel<2, 2><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        case 6: enc_group_kernel<3, 1><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        case 7: enc_group_kernel<3, 2><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        case 8: enc_group_kernel<4, 1><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        default: enc_group_kernel<4, 2><<<blocks, EG_WAVES * SG_WAVE, 0, st>>>(e, NG); break;
        }
        SG_TRY_LAUNCH();
        enc_fix_kernel<<<(unsigned)ceil_div(NG * P, 256), 256, 0, st>>>(e, NG, G);
    } else {
        enc_kernel<<<(unsigned)e.L.NW, EN_THREADS, 0, st>>>(e);
    }
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_ENCODE, st);
    return SG_OK;
}

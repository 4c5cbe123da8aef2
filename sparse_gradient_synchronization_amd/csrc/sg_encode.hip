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
// windows share zeroed (the encode kernel merges them with atomicOr).
template <bool VEC>
__global__ __launch_bounds__(256) void enc_prep_kernel(EncParams e)
{
    __shared__ uint64_t offs[257];
    load_agg_offsets(e, offs);
    const uint32_t P = e.L.P;
    const uint64_t NW = e.L.NW;
    window_cursor_pass<VEC>(e.agg_idx, e.agg_cap, offs, P, (uint32_t)NW, (uint32_t)__builtin_ctzll(e.L.W), e.cur);
    const uint32_t tid32 = blockIdx.x * 256 + threadIdx.x, nth32 = gridDim.x * 256;
    for (uint32_t i = tid32; i < (uint32_t)(NW * P); i += nth32) {
        const uint32_t w = i / P;
        const uint32_t p = i % P;
        if (w == 0) continue;
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
    return (size_t)(8ull * (L.NW + 1) * P);
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
    // a window's words never exceed W/32 + P
    if (e.L.W / 32 + P + 2 > (uint64_t)EN_SEG_WORDS) return SG_EUNSUPPORTED;
    hipStream_t st = as_stream(stream);
    // a chunk of entries per block where they allow, and enough blocks for
    // the per-window work
    uint64_t pblocks = ceil_div(agg_capacity, (uint64_t)WC_CHUNK);
    const uint64_t fill = ceil_div((e.L.NW + 1) * P, 1024);
    pblocks = pblocks > fill ? pblocks : fill;
    pblocks = pblocks < 4096 ? (pblocks ? pblocks : 1) : 4096;
    if ((uintptr_t)d_agg_idx % 16 == 0)
        enc_prep_kernel<true><<<(unsigned)pblocks, 256, 0, st>>>(e);
    else
        enc_prep_kernel<false><<<(unsigned)pblocks, 256, 0, st>>>(e);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_ENCODE, st);
    enc_kernel<<<(unsigned)e.L.NW, EN_THREADS, 0, st>>>(e);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_ENCODE, st);
    return SG_OK;
}

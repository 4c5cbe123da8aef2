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
// neighbouring block are merged with atomicOr after a pre-zeroing pass; all
// other words are plain stores.
#include "sg_host.h"

namespace sg {

constexpr uint32_t CM_MAGIC = 0x53474d31u; // "SGM1"
constexpr int EN_THREADS = 256;
constexpr int EN_SEG_WORDS = 4096;

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
    L.NCW = 2048 / P;
    if (L.NCW > 128) L.NCW = 128;
    if (L.NCW == 0) L.NCW = 1;
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
    uint64_t agg_cap; // entries d_agg_idx holds
    uint32_t* bitmap;
    uint64_t bitmap_words;
    uint64_t* word_off_out;
    uint32_t SR;      // windows per block
    uint32_t nblocks;
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

// zero the words that two neighbouring blocks share (they are merged with
// atomicOr by the encode kernel)
__global__ void enc_zero_kernel(EncParams e)
{
    const uint32_t P = e.L.P;
    const uint64_t cnt = (uint64_t)e.nblocks * P;
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < cnt; i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t blk = (uint32_t)(i / P), p = (uint32_t)(i % P);
        if (blk == 0) continue;
        const uint64_t w0 = (uint64_t)blk * e.SR;
        if (w0 > e.L.NW) continue;
        const uint32_t a = e.q.cpre[w0 * P + p];
        if ((a & 31u) == 0 || a >= e.q.class_size[p]) continue;
        const uint64_t gw = e.q.word_off[p] + (a >> 5);
        if (gw < e.bitmap_words) e.bitmap[gw] = 0u;
    }
}

__global__ __launch_bounds__(EN_THREADS) void enc_kernel(EncParams e)
{
    __shared__ uint32_t masks[128 * 16 > 2048 ? 2048 : 2048]; // [NCW][P], NCW*P <= 2048
    __shared__ uint16_t pre[2048];                              // [NCW][P]
    __shared__ uint32_t seg[EN_SEG_WORDS];
    __shared__ uint32_t segofs[257];
    __shared__ uint32_t a_bits[256], base_bits[256], wtot[256];
    __shared__ uint64_t cursor[256], cend[256];
    __shared__ uint32_t scan_lds[EN_THREADS / SG_WAVE + 1];

    const CmapLayout& L = e.L;
    const uint32_t P = L.P, NCW = L.NCW;
    const uint32_t blk = blockIdx.x;
    const uint64_t w0 = (uint64_t)blk * e.SR;
    uint64_t w1 = w0 + e.SR;
    if (w1 > L.NW) w1 = L.NW;
    if (w0 >= w1) return;
    const uint32_t wid = threadIdx.x / SG_WAVE, lane = lane_id();

    if (blk == 0)
        for (uint32_t i = threadIdx.x; i <= P; i += EN_THREADS) e.word_off_out[i] = e.q.word_off[i];
    if (blk == 0 && threadIdx.x == 0) {
        const CmapHeader h = *e.q.hdr;
        if (h.magic != CM_MAGIC || h.P != P || h.M != L.M) report_error(kDevErrCmap);
    }

    // segment layout and cursors
    uint32_t nw = 0;
    if (threadIdx.x < P) {
        const uint32_t p = threadIdx.x;
        const uint32_t a = e.q.cpre[w0 * P + p], b = e.q.cpre[w1 * P + p];
        a_bits[p] = a;
        base_bits[p] = a;
        nw = b > a ? ((b - 1) >> 5) - (a >> 5) + 1 : 0u;
        // first aggregated key of partition p at or after the block's first key
        uint64_t lo0 = e.agg_off[p], hi0 = e.agg_off[p + 1];
        if (hi0 > e.agg_cap) hi0 = e.agg_cap;
        if (lo0 > hi0) lo0 = hi0;
        const uint64_t key0 = w0 * L.W;
        uint64_t lo = lo0, hi = hi0;
        while (lo < hi) {
            const uint64_t mid = (lo + hi) >> 1;
            if ((uint64_t)e.agg_idx[mid] < key0) lo = mid + 1;
            else hi = mid;
        }
        cursor[p] = lo;
        cend[p] = hi0;
    }
    uint32_t tot;
    const uint32_t so = block_excl_scan<EN_THREADS>(nw, scan_lds, &tot);
    if (threadIdx.x < P) segofs[threadIdx.x] = so;
    if (threadIdx.x == 0) segofs[P] = tot;
    for (uint32_t i = threadIdx.x; i < EN_SEG_WORDS; i += EN_THREADS) seg[i] = 0u;
    __syncthreads();
    if (tot > EN_SEG_WORDS) { // cannot happen with the host's choice of SR
        if (threadIdx.x == 0) report_error(kDevErrCmap);
        return;
    }

    for (uint64_t win = w0; win < w1; ++win) {
        const uint64_t wstart = win * L.W;
        // a) class masks of the window's chunks
        for (uint32_t t = threadIdx.x; t < NCW; t += EN_THREADS) {
            const uint64_t c = win * NCW + t;
            const uint32_t valid = chunk_valid(L, c);
            uint32_t pl[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (valid)
                for (uint32_t b = 0; b < L.nbits; ++b) pl[b] = e.q.planes[c * L.stride + b];
            for (uint32_t p = 0; p < P; ++p) masks[t * P + p] = class_mask(pl, L.nbits, p, valid);
        }
        __syncthreads();
        // b) per-partition prefix over the chunks of the window
        if (threadIdx.x < P) {
            const uint32_t p = threadIdx.x;
            uint32_t run = 0;
            for (uint32_t t = 0; t < NCW; ++t) {
                pre[t * P + p] = (uint16_t)run;
                run += __popc(masks[t * P + p]);
            }
            wtot[p] = run;
        }
        __syncthreads();
        // c) aggregated keys of each partition inside the window
        for (uint32_t p = wid; p < P; p += EN_THREADS / SG_WAVE) {
            uint64_t cur = cursor[p];
            const uint64_t end = cend[p];
            const uint64_t wend = wstart + L.W;
            const uint32_t seg_lo = a_bits[p] >> 5;
            const uint32_t bb = base_bits[p];
            while (cur < end) {
                const uint64_t i = cur + lane;
                const uint32_t key = i < end ? e.agg_idx[i] : 0xffffffffu;
                const bool in = i < end && (uint64_t)key < wend && (uint64_t)key >= wstart;
                const uint64_t m = ballot(in);
                if (in) {
                    const uint32_t o = (uint32_t)(key - wstart);
                    const uint32_t t = o >> 5, bit = o & 31u;
                    const uint32_t mk = masks[t * P + p];
                    if (!((mk >> bit) & 1u)) report_error(kDevErrPartition);
                    const uint32_t r = bb + pre[t * P + p] + __popc(mk & ((1u << bit) - 1u));
                    const uint32_t lw = (r >> 5) - seg_lo;
                    if (lw < segofs[p + 1] - segofs[p]) atomicOr(&seg[segofs[p] + lw], 1u << (r & 31u));
                }
                const uint32_t took = popc64(m);
                cur += took;
                if (took < SG_WAVE) break;
            }
            if (lane == 0) cursor[p] = cur;
        }
        __syncthreads();
        if (threadIdx.x < P) base_bits[threadIdx.x] += wtot[threadIdx.x];
        __syncthreads();
    }

    // write the segments
    for (uint32_t p = 0; p < P; ++p) {
        const uint32_t a = a_bits[p], b = base_bits[p];
        if (b <= a) continue;
        const uint32_t q0 = a >> 5, nwp = segofs[p + 1] - segofs[p];
        const uint64_t csize = e.q.class_size[p];
        const uint64_t wbase = e.q.word_off[p];
        for (uint32_t lw = threadIdx.x; lw < nwp; lw += EN_THREADS) {
            const uint32_t qw = q0 + lw;
            const bool excl = (uint64_t)qw * 32 >= a && ((uint64_t)(qw + 1) * 32 <= b || (uint64_t)b == csize);
            const uint64_t gw = wbase + qw;
            if (gw >= e.bitmap_words) continue;
            const uint32_t v = seg[segofs[p] + lw];
            if (excl) e.bitmap[gw] = v;
            else if (v) atomicOr(&e.bitmap[gw], v);
        }
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

// The encode pass keeps all its scratch in LDS.
extern "C" size_t sg_encode_workspace_bytes(uint64_t M, uint32_t P)
{
    (void)M;
    (void)P;
    return 0;
}

extern "C" int sg_encode(const uint32_t* d_agg_idx, const uint64_t* d_agg_off, uint64_t agg_capacity, uint64_t M,
                         uint32_t P, const void* d_cmap, size_t cmap_bytes, uint32_t* d_bitmap, uint64_t bitmap_words, uint64_t* d_word_off,
                         void* d_ws, size_t ws_bytes, void* stream)
{
    (void)d_ws;
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32)) return SG_EINVAL;
    if (!d_agg_off || !d_cmap || !d_bitmap || !d_word_off || !d_agg_idx) return SG_EINVAL;
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
    // windows per block: enough blocks to fill the chip, and the block's
    // bitmap segments must fit in LDS
    uint64_t sr = e.L.NW / 2048;
    if (sr < 1) sr = 1;
    const uint64_t srmax = ((uint64_t)(EN_SEG_WORDS - 2 * P - 2) * 32) / e.L.W;
    if (sr > srmax) sr = srmax;
    if (sr > 64) sr = 64;
    if (sr < 1) return SG_EUNSUPPORTED;
    e.SR = (uint32_t)sr;
    e.nblocks = (uint32_t)ceil_div(e.L.NW, sr);
    hipStream_t st = as_stream(stream);
    const uint64_t zc = (uint64_t)e.nblocks * P;
    enc_zero_kernel<<<(unsigned)(ceil_div(zc, 256) < 1024 ? ceil_div(zc, 256) : 1024), 256, 0, st>>>(e);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_ENCODE, st);
    enc_kernel<<<e.nblocks, EN_THREADS, 0, st>>>(e);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_ENCODE, st);
    return SG_OK;
}

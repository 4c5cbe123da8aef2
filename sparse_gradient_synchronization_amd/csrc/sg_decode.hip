// sg_decode.hip -- the Pull side after A4 (Zen OSDI'25 digest, section
// 3.3.2, hash_bitmap_decode; section 3.1, every worker holds the aggregate
// after Pull): hash bitmap back to indices, the scatter of aggregated values
// into a dense tensor, and the encoded size of an aggregate under the formats
// of section 3.3.1.
//
// Decode, on gfx950: the class map's key windows again.
//   ranks  the output position of a set bit is the number of set bits before
//          it in the whole encoded bitmap (classes in order, each ascending):
//          an exclusive prefix over the words' bit counts (block sums, their
//          scan, then the per-word prefix);
//   emit   a block per window forms the class masks of its chunks and their
//          per-class prefix counts (as encode does) and loads the window's
//          bitmap words.  Per (chunk, class) pair, the class's members in the
//          chunk are the set bits of its mask, and their bitmap bits are one
//          run of that many bits; the k-th set bit of the run is the k-th
//          member, written at the run's rank plus the set bits before it;
//   group  for 2..16 classes and enough windows, a wave per group of
//          consecutive windows does the emit with no block barrier, each
//          class's bits of the group loaded once as one contiguous run
//          (dec_group_kernel below).
#include "sg_host.h"

namespace sg {

struct DecParams {
    CmapLayout L;
    CmapPtrs q;
    const uint32_t* bitmap;
    uint64_t bitmap_words;
    uint32_t* out_idx;
    uint64_t capacity;
    uint64_t* out_off; // [P+1]
    uint32_t* wpre;    // [words + 1] set bits of the encoded words before each word
    uint32_t* bsum;    // [NB] set bits per block of DS_WPB words, then their exclusive prefix
    uint32_t NB;
};

// Ranks of set bits: the output position of a set bit is the number of set
// bits before it in the whole encoded bitmap (classes in order, each
// ascending), so an exclusive prefix over the words gives every window's
// output offsets.  Padding bits past a class's size are not counted.
constexpr int DS_ROUNDS = 4;                  // 16-byte loads per thread
constexpr int DS_WPB = DS_ROUNDS * 4 * 256;   // words per block: round r, thread t holds 4 words at r 1024 + 4 t

// the encoded words the buffer holds
__device__ __forceinline__ uint64_t dec_words(const DecParams& d)
{
    const uint64_t n = d.q.word_off[d.L.P];
    return n < d.bitmap_words ? n : d.bitmap_words;
}

// words g0 .. g0+3 (g0 a multiple of 4; zero past nwords), the bits past each
// class's size cleared; wo, cs: word offsets and class sizes in LDS.  VEC:
// the bitmap is 16-byte aligned.
template <bool VEC>
__device__ __forceinline__ void dec_load_words(const DecParams& d, const uint64_t* wo, const uint64_t* cs, uint64_t g0,
                                               uint64_t nwords, uint32_t (&v)[4])
{
    if (VEC && g0 + 4 <= nwords) {
        const uint4 x = *reinterpret_cast<const uint4*>(d.bitmap + g0);
        v[0] = x.x, v[1] = x.y, v[2] = x.z, v[3] = x.w;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = g0 + c < nwords ? d.bitmap[g0 + c] : 0u;
    }
    if (g0 >= nwords) return;
    const uint32_t P = d.L.P;
    uint32_t p = 0, hi = P; // largest p with wo[p] <= g0: the class of word g0
    while (p + 1 < hi) {
        const uint32_t mid = (p + hi) >> 1;
        if (wo[mid] <= g0) p = mid;
        else hi = mid;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint64_t gw = g0 + c;
        if (gw >= nwords) break;
        while (p + 1 < P && gw >= wo[p + 1]) ++p;
        const uint32_t r = (uint32_t)(cs[p] & 31u);
        if (gw + 1 == wo[p + 1] && r != 0u) v[c] &= (1u << r) - 1u;
    }
}

__device__ __forceinline__ void dec_load_class_table(const DecParams& d, uint64_t* wo, uint64_t* cs)
{
    for (uint32_t p = threadIdx.x; p <= d.L.P; p += blockDim.x) {
        wo[p] = d.q.word_off[p];
        if (p < d.L.P) cs[p] = d.q.class_size[p];
    }
    __syncthreads();
}

// set bits per block of DS_WPB words
template <bool VEC>
__global__ __launch_bounds__(256) void dec_wsum_kernel(DecParams d)
{
    __shared__ uint64_t wo[257], cs[256];
    __shared__ uint32_t scan_lds[256 / SG_WAVE + 1];
    dec_load_class_table(d, wo, cs);
    const uint64_t nwords = dec_words(d);
    uint32_t sum = 0;
#pragma unroll
    for (int r = 0; r < DS_ROUNDS; ++r) {
        uint32_t v[4];
        dec_load_words<VEC>(d, wo, cs, (uint64_t)blockIdx.x * DS_WPB + r * 1024 + threadIdx.x * 4, nwords, v);
        sum += __popc(v[0]) + __popc(v[1]) + __popc(v[2]) + __popc(v[3]);
    }
    uint32_t tot;
    block_excl_scan<256>(sum, scan_lds, &tot);
    if (threadIdx.x == 0) d.bsum[blockIdx.x] = tot;
}

// one block: exclusive prefix of the block sums, in place
__global__ __launch_bounds__(1024) void dec_bscan_kernel(DecParams d)
{
    constexpr uint32_t PT = 8;
    __shared__ uint32_t scan_lds[1024 / SG_WAVE + 1];
    uint32_t carry = 0; // the encoded bits number below 2^32
    for (uint32_t base = 0; base < d.NB; base += 1024 * PT) {
        const uint32_t b0 = base + threadIdx.x * PT;
        uint32_t c[PT], sum = 0;
#pragma unroll
        for (uint32_t j = 0; j < PT; ++j) {
            c[j] = b0 + j < d.NB ? d.bsum[b0 + j] : 0u;
            sum += c[j];
        }
        uint32_t tot;
        uint32_t ex = block_excl_scan<1024>(sum, scan_lds, &tot);
#pragma unroll
        for (uint32_t j = 0; j < PT; ++j) {
            if (b0 + j < d.NB) d.bsum[b0 + j] = carry + ex;
            ex += c[j];
        }
        carry += tot;
        __syncthreads();
    }
}

// per word, the set bits of the words before it; the entry past the last
// word holds the total.  One block scan serves the four rounds: the
// thread's per-round counts (at most 128) packed in 16-bit fields, whose
// block totals (at most 32768) do not carry into each other.
template <bool VEC>
__global__ __launch_bounds__(256) void dec_wpre_kernel(DecParams d)
{
    __shared__ uint64_t wo[257], cs[256];
    __shared__ uint64_t scan_lds[256 / SG_WAVE + 1];
    dec_load_class_table(d, wo, cs);
    const uint64_t nwords = dec_words(d);
    const uint64_t b0 = (uint64_t)blockIdx.x * DS_WPB;
    uint32_t v[DS_ROUNDS][4];
    uint64_t packed = 0;
#pragma unroll
    for (int r = 0; r < DS_ROUNDS; ++r) {
        dec_load_words<VEC>(d, wo, cs, b0 + r * 1024 + threadIdx.x * 4, nwords, v[r]);
        const uint64_t sr = __popc(v[r][0]) + __popc(v[r][1]) + __popc(v[r][2]) + __popc(v[r][3]);
        packed |= sr << (16 * r);
    }
    uint64_t tot;
    const uint64_t ex = block_excl_scan64<256>(packed, scan_lds, &tot);
    uint32_t before = d.bsum[blockIdx.x]; // set bits of the rounds before
#pragma unroll
    for (int r = 0; r < DS_ROUNDS; ++r) {
        const uint64_t g0 = b0 + r * 1024 + threadIdx.x * 4;
        uint32_t run = before + (uint32_t)((ex >> (16 * r)) & 0xffffu);
        uint32_t pre[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pre[c] = run;
            run += __popc(v[r][c]);
            if (g0 + c + 1 == nwords) d.wpre[nwords] = run;
        }
        if (g0 + 4 <= nwords) {
            *reinterpret_cast<uint4*>(d.wpre + g0) = make_uint4(pre[0], pre[1], pre[2], pre[3]);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (g0 + c < nwords) d.wpre[g0 + c] = pre[c];
        }
        before += (uint32_t)((tot >> (16 * r)) & 0xffffu);
    }
    if (nwords == 0 && blockIdx.x == 0 && threadIdx.x == 0) d.wpre[0] = 0;
}

constexpr int DC_THREADS = 256;
constexpr int DC_WORDS = 512; // a window's bitmap words: at most W/32 + P <= 128 + 256

__global__ __launch_bounds__(DC_THREADS) void dec_emit_kernel(DecParams d)
{
    // partition-major [P][NCW]: a thread's 8 chunks of one class are 16-byte
    // accesses, consecutive threads on consecutive addresses
    __shared__ __align__(16) uint32_t masks[2048];
    __shared__ uint32_t segofs[257], a_bits[256], b_bits[256], cls_first[256];
    __shared__ uint64_t obase[256];
    __shared__ uint32_t wex[DC_WORDS], segw[DC_WORDS];
    __shared__ uint32_t scan_lds[DC_THREADS / SG_WAVE + 1];
    const CmapLayout& L = d.L;
    const uint32_t P = L.P, NCW = L.NCW;
    const uint64_t win = blockIdx.x;
    const uint32_t lane = lane_id();

    uint32_t pl[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t valid = 0;
    if (threadIdx.x < NCW) {
        const uint64_t c = win * NCW + threadIdx.x;
        valid = c < L.NC ? (L.M - c * 32 >= 32 ? 0xffffffffu : ((1u << (L.M - c * 32)) - 1u)) : 0u;
        if (valid)
            for (uint32_t b = 0; b < L.nbits; ++b) pl[b] = d.q.planes[c * L.stride + b];
    }
    uint32_t nw = 0;
    if (threadIdx.x < P) {
        const uint32_t p = threadIdx.x;
        const uint32_t ca = d.q.cpre[win * P + p], cb = d.q.cpre[(win + 1) * P + p];
        a_bits[p] = ca;
        b_bits[p] = cb;
        // output position of the class's first bit in the window: the set
        // bits before it (words before its word, and its word's lower bits)
        if (cb > ca) {
            const uint64_t nwords = dec_words(d);
            const uint64_t gw0 = d.q.word_off[p] + (ca >> 5);
            const uint32_t v0 = gw0 < nwords ? d.bitmap[gw0] : 0u;
            obase[p] = (uint64_t)d.wpre[gw0 < nwords ? gw0 : nwords] + __popc(v0 & ((1u << (ca & 31u)) - 1u));
        }
        nw = cb > ca ? ((cb - 1) >> 5) - (ca >> 5) + 1 : 0u;
    }
    if (win == 0) { // the classes' offsets
        const uint64_t nwords = dec_words(d);
        for (uint32_t p = threadIdx.x; p <= P; p += DC_THREADS) {
            const uint64_t w = d.q.word_off[p];
            d.out_off[p] = d.wpre[w < nwords ? w : nwords];
        }
    }
    uint32_t nseg;
    const uint32_t so = block_excl_scan<DC_THREADS>(nw, scan_lds, &nseg);
    if (threadIdx.x < P) segofs[threadIdx.x] = so;
    if (threadIdx.x == 0) segofs[P] = nseg;
    // class masks of the window's chunks by plane splitting (as in encode)
    if (threadIdx.x < NCW) {
        uint32_t* mrow = masks + threadIdx.x; // class k at mrow[k * NCW]
        uint32_t m[16];
        if (L.nbits <= 4) {
            m[0] = valid;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if ((uint32_t)b < L.nbits) {
#pragma unroll
                    for (int k = (1 << b) - 1; k >= 0; --k) {
                        m[k + (1 << b)] = m[k] & pl[b];
                        m[k] &= ~pl[b];
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if ((uint32_t)k < P) mrow[k * NCW] = m[k];
        } else {
            for (uint32_t p = 0; p < P; ++p) {
                uint32_t v = valid;
                for (uint32_t b = 0; b < L.nbits; ++b) v &= ((p >> b) & 1u) ? pl[b] : ~pl[b];
                mrow[p * NCW] = v;
            }
        }
    }
    __syncthreads();
    if (nseg > DC_WORDS) { // cannot happen: at most W/32 + P words
        if (threadIdx.x == 0) report_error(kDevErrCmap);
        return;
    }
    // per-class prefix over the window's chunks: P segments of NCW, 8
    // per thread, segmented scan inside a DPP row (NCW/8 <= 16 threads);
    // the thread keeps its 8 (chunk, class) masks, counts and prefixes
    const uint32_t e0 = threadIdx.x * 8;
    const bool act = e0 < NCW * P;
    uint32_t mw[8], c[8], ex[8];
    {
        uint32_t run = 0;
        const uint4 ma = act ? *reinterpret_cast<const uint4*>(&masks[e0]) : make_uint4(0u, 0u, 0u, 0u);
        const uint4 mb = act ? *reinterpret_cast<const uint4*>(&masks[e0 + 4]) : make_uint4(0u, 0u, 0u, 0u);
        mw[0] = ma.x, mw[1] = ma.y, mw[2] = ma.z, mw[3] = ma.w;
        mw[4] = mb.x, mw[5] = mb.y, mw[6] = mb.z, mw[7] = mb.w; // 8 chunks of one class
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            c[j] = __popc(mw[j]);
            run += c[j];
        }
        const uint32_t sg = NCW / 8;
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
        ex[0] = inc - run;
#pragma unroll
        for (int j = 1; j < 8; ++j) ex[j] = ex[j - 1] + c[j - 1];
    }
    // the window's words (class-major), masked to the class ranges
    uint32_t wv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t i = threadIdx.x * 2 + h;
        wv[h] = 0;
        if (i < nseg) {
            uint32_t lo = 0, hi = P; // class of word i
            while (lo + 1 < hi) {
                const uint32_t mid = (lo + hi) >> 1;
                if (segofs[mid] <= i) lo = mid;
                else hi = mid;
            }
            const uint32_t p = lo, a = a_bits[p], b = b_bits[p];
            const uint32_t qw = (a >> 5) + (i - segofs[p]);
            const uint64_t gw = d.q.word_off[p] + qw;
            uint32_t v = gw < d.bitmap_words ? d.bitmap[gw] : 0u;
            const uint32_t lo_b = qw * 32 < a ? a - qw * 32 : 0u;
            const uint32_t hi_b = (qw + 1) * 32 > b ? b - qw * 32 : 32u;
            uint32_t m = ~((1u << lo_b) - 1u);
            if (hi_b < 32) m &= (1u << hi_b) - 1u;
            wv[h] = v & m;
        }
    }
    // the words into LDS, and the exclusive prefix of their set bits
    uint32_t sum = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t i = threadIdx.x * 2 + h;
        if (i < nseg) segw[i] = wv[h];
        sum += __popc(wv[h]);
    }
    uint32_t tot;
    const uint32_t wx = block_excl_scan<DC_THREADS>(sum, scan_lds, &tot);
    if (threadIdx.x * 2 < DC_WORDS) wex[threadIdx.x * 2] = wx;
    if (threadIdx.x * 2 + 1 < DC_WORDS) wex[threadIdx.x * 2 + 1] = wx + __popc(wv[0]);
    __syncthreads();
    if (threadIdx.x < P) cls_first[threadIdx.x] = segofs[threadIdx.x] < nseg ? wex[segofs[threadIdx.x]] : tot;
    __syncthreads();
    // every set bit back to its key, by (chunk, class) pair: the class-p
    // members of chunk ch are the set bits of its mask, with window
    // ranks ex, ex + 1, ...; their bitmap bits are the run of c bits at
    // a + ex, and the k-th set bit of the run is the member at the k-th
    // set bit of the mask
    if (act) {
        const uint32_t p = e0 / NCW, ch0 = e0 % NCW;
        const uint32_t a = a_bits[p], so2 = segofs[p], a5 = a >> 5;
        const uint64_t base = obase[p];
        const uint32_t first = cls_first[p];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (c[j] == 0) continue;
            const uint32_t g = a + ex[j];
            const uint32_t k = so2 + (g >> 5) - a5, bit = g & 31u;
            const uint32_t w0 = segw[k];
            uint32_t run = w0 >> bit;
            if (bit + c[j] > 32) run |= segw[k + 1] << (32 - bit); // bit > 0 here
            if (c[j] < 32) run &= (1u << c[j]) - 1u;
            if (run == 0) continue;
            uint32_t f = wex[k] + __popc(w0 & ((1u << bit) - 1u)); // rank among the window's set bits
            const uint32_t kbase = (uint32_t)(win * L.W) + (ch0 + j) * 32;
            uint32_t m = mw[j]; // the members not yet passed, in key order
            while (run) {
                const uint32_t z = __ffs(run) - 1u; // members to pass over
                run = (run >> z) >> 1;
                for (uint32_t i = 0; i < z; ++i) m &= m - 1u;
                const uint64_t o = base + (f - first);
                if (o < d.capacity) d.out_idx[o] = kbase + (__ffs(m) - 1u);
                m &= m - 1u;
                ++f;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Group decode, 2 <= P <= 16 and enough groups to fill the chip: a wave per
// group of G consecutive windows, no block barrier (the mirror image of the
// group encode).  A class's bits of the group are one contiguous run of its
// bitmap, so the wave first loads every class's run (all classes' loads in
// flight together), masked to the class's bits of the group, into LDS with
// the set bits before each word of the run; the output position of the
// class's first bit of the group is the ranks pass's prefix of its word plus
// the set bits below it in that word.  Per window (its planes and class
// offsets loaded a window ahead, in two register sets used in turn) the
// lane's two chunks are split into class masks and counted per class, as
// 16-bit fields two classes to a register, scanned over the lanes; the
// class-p members of a chunk then own the run of class-p bits at the
// window's class offset plus the chunk's prefix, and each set bit of that
// run is written as the key of the matching member.
// ---------------------------------------------------------------------------
constexpr int DG_WAVES = 4; // waves per block, each on a group of its own

// windows per group for class ids of nbits bits (measured best: 4 for 9..16
// classes, where a window's class runs are short; 1 below)
constexpr int dg_group(uint32_t nbits) { return nbits >= 4 ? 4 : 1; }

template <int NB, int G>
struct DgShape {
    static constexpr int NCLS = 1 << NB;
    static constexpr int NPK = NCLS / 2;                         // prefix registers: two 16-bit counts each
    static constexpr uint32_t SEG = G * EG_NCW + 2 * NCLS;       // words of a group's class runs, at most
};

template <int NB, int G>
__global__ __launch_bounds__(DG_WAVES * SG_WAVE) void dec_group_kernel(DecParams d, uint64_t NG)
{
    using S = DgShape<NB, G>;
    constexpr int NCLS = S::NCLS;
    constexpr uint32_t W = EG_NCW * 32u;
    // the runs, and per word the run's set bits before it; two words of
    // slack past the longest runs: a member run read at a class's end
    // touches at most the word after it, and is masked to nothing there
    __shared__ __align__(16) uint32_t seg_all[DG_WAVES][S::SEG + 2];
    __shared__ __align__(16) uint32_t sx_all[DG_WAVES][S::SEG + 2];
    const uint32_t wv = threadIdx.x / SG_WAVE, lane = lane_id();
    uint32_t* seg = seg_all[wv];
    uint32_t* sx = sx_all[wv];
    const uint64_t g = (uint64_t)blockIdx.x * DG_WAVES + wv;
    if (g >= NG) return; // the whole wave: nothing below waits for other waves
    const CmapLayout& L = d.L;
    const uint32_t P = L.P;
    const uint64_t NW = L.NW;
    const uint64_t w0 = g * G;
    const uint64_t w1 = w0 + G < NW ? w0 + G : NW;
    const bool cl = lane < P; // lane p holds class p's values
    const uint32_t pc = cl ? lane : 0u;
    const uint64_t nwords = dec_words(d);
    // every global load is unconditional (clamped index; a one-word stand-in
    // when the buffer holds no words, whose value is never used), so the
    // compiler waits for each where it is used and not at a branch
    const uint32_t* bm = nwords ? d.bitmap : reinterpret_cast<const uint32_t*>(d.q.word_off);
    const uint64_t blast = nwords ? nwords - 1 : 0;

    uint32_t pl[2][8];
    uint32_t cwn[2];
    auto issue = [&](int set, uint64_t w) {
        w = w < NW ? w : NW - 1;
        const uint64_t ca = w * EG_NCW + 2 * lane, cb = ca + 1;
        uint32_t pa[4], pb[4];
        eg_load_planes<NB>(d.q.planes, ca < L.NC ? ca : L.NC, pa);
        eg_load_planes<NB>(d.q.planes, cb < L.NC ? cb : L.NC, pb);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            pl[set][b] = pa[b];
            pl[set][4 + b] = pb[b];
        }
        cwn[set] = d.q.cpre[(w + 1) * P + pc];
    };
    issue(0, w0);

    if (g == 0 && lane <= P) { // the classes' output offsets
        const uint64_t wo = d.q.word_off[lane];
        d.out_off[lane] = d.wpre[wo < nwords ? wo : nwords];
    }
    // the class's bits [A, B) of the group, its words, their place in LDS
    uint32_t A = d.q.cpre[w0 * P + pc], B = d.q.cpre[w1 * P + pc];
    const uint64_t wof = d.q.word_off[pc];
    if (!cl) A = B = 0; // lanes past P: an empty class
    const uint32_t nw = B > A ? ((B - 1u) >> 5) - (A >> 5) + 1u : 0u;
    const uint32_t nincl = wave_incl_scan(nw);
    const uint32_t so = nincl - nw;
    const uint32_t nseg = lane_value(nincl, SG_WAVE - 1);
    if (nseg > S::SEG) { // cannot happen with a valid class map
        if (lane == 0) report_error(kDevErrCmap);
        return;
    }
    const uint64_t wb = wof + (A >> 5); // the class's first word of the group
    // first round of every class's run (64 words; a run is about 32 G / P
    // words long, a longer one takes further rounds below)
    uint32_t v[NCLS];
#pragma unroll
    for (int p = 0; p < NCLS; ++p) {
        const uint64_t gw = lane_value64(wb, p) + lane;
        v[p] = bm[gw < blast ? gw : blast];
    }
    // output position of the class's first bit of the group
    uint32_t ob;
    {
        const uint32_t f0 = bm[wb < blast ? wb : blast];
        const uint32_t pre = d.wpre[wb < nwords ? wb : nwords];
        ob = pre + (uint32_t)__popc((wb < nwords ? f0 : 0u) & ((1u << (A & 31u)) - 1u));
    }
    // a class's word j holds class bits [32 q, 32 q + 32), q = A / 32 + j:
    // keep those in [A, B); words past the buffer's end read as zero
    auto keep = [&](uint32_t x, uint32_t j, uint32_t nwp, uint32_t Ap, uint32_t Bp, uint64_t wbp) -> uint32_t {
        const uint32_t base = ((Ap >> 5) + j) << 5;
        const uint32_t lo = Ap > base ? Ap - base : 0u;
        const uint32_t rest = Bp - base;
        uint32_t m = ~((1u << lo) - 1u);
        if (rest < 32u) m &= (1u << rest) - 1u;
        return j < nwp && wbp + j < nwords ? x & m : 0u;
    };
#pragma unroll
    for (int p = 0; p < NCLS; ++p) {
        if ((uint32_t)p >= P) continue; // uniform (a constant trip count: the loop unrolls)
        const uint32_t nwp = lane_value(nw, p), sop = lane_value(so, p);
        const uint32_t Ap = lane_value(A, p), Bp = lane_value(B, p);
        const uint64_t wbp = lane_value64(wb, p);
        const uint32_t x = keep(v[p], lane, nwp, Ap, Bp, wbp);
        const uint32_t c = (uint32_t)__popc(x);
        const uint32_t inc = wave_incl_scan(c);
        if (lane < nwp) {
            seg[sop + lane] = x;
            sx[sop + lane] = inc - c;
        }
    }
    // further rounds of long runs (a class holding most of the group's keys)
    if (wave_max(nw) > (uint32_t)SG_WAVE) {
        wave_sync();
        for (uint32_t p = 0; p < P; ++p) {
            const uint32_t nwp = lane_value(nw, p), sop = lane_value(so, p);
            const uint32_t Ap = lane_value(A, p), Bp = lane_value(B, p);
            const uint64_t wbp = lane_value64(wb, p);
            for (uint32_t j0 = SG_WAVE; j0 < nwp; j0 += SG_WAVE) { // uniform
                const uint32_t carry = sx[sop + j0 - 1] + (uint32_t)__popc(seg[sop + j0 - 1]);
                const uint32_t j = j0 + lane;
                const uint64_t gw = wbp + j;
                const uint32_t x = keep(bm[gw < blast ? gw : blast], j, nwp, Ap, Bp, wbp);
                const uint32_t c = (uint32_t)__popc(x);
                const uint32_t inc = wave_incl_scan(c);
                if (j < nwp) {
                    seg[sop + j] = x;
                    sx[sop + j] = carry + inc - c;
                }
                wave_sync();
            }
        }
    }
    wave_sync();

    // output positions are ranks of encoded bits, below M < 2^32
    const uint32_t cap = d.capacity < 0xffffffffull ? (uint32_t)d.capacity : 0xffffffffu;
    uint32_t cw = A; // the class's bits before the window
#pragma unroll
    for (uint32_t wi = 0; wi < (uint32_t)G; ++wi) {
        const uint64_t w = w0 + wi;
        if (w >= w1) break;
        const int cs = wi & 1, ns = cs ^ 1;
        if (wi + 1 < (uint32_t)G) issue(ns, w + 1); // (past the group's last window: loads not used)
        const uint64_t ca = w * EG_NCW + 2 * lane, cb = ca + 1;
        uint32_t pa[4], pb[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            pa[b] = pl[cs][b];
            pb[b] = pl[cs][4 + b];
        }
        const uint32_t va = chunk_valid(L, ca), vb = chunk_valid(L, cb);
        // class counts of the lane's two chunks, and their exclusive scan
        uint32_t cpa[S::NPK], ex[S::NPK];
        {
            uint32_t m[NCLS];
            eg_masks<NB>(pa, va, m);
#pragma unroll
            for (int i = 0; i < S::NPK; ++i) cpa[i] = __popc(m[2 * i]) | (__popc(m[2 * i + 1]) << 16);
            eg_masks<NB>(pb, vb, m);
#pragma unroll
            for (int i = 0; i < S::NPK; ++i) {
                const uint32_t tot = cpa[i] + (__popc(m[2 * i]) | (__popc(m[2 * i + 1]) << 16));
                ex[i] = wave_incl_scan(tot) - tot;
            }
        }
        // the window's first class bit, from the start of the class's run
        const uint32_t rb = cw - (A & ~31u);
#pragma unroll
        for (int p = 0; p < NCLS; ++p) {
            if ((uint32_t)p >= P) continue; // uniform (a constant trip count: the loop unrolls)
            const uint32_t rbp = lane_value(rb, p), sop = lane_value(so, p), obp = lane_value(ob, p);
            const uint32_t sh = 16u * (p & 1);
            const uint32_t ea = (ex[p >> 1] >> sh) & 0xffffu;
            const uint32_t na = (cpa[p >> 1] >> sh) & 0xffffu;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // the chunk's class-p members: plane b where p has bit b, else its complement
                uint32_t m = h ? vb : va;
#pragma unroll
                for (int b = 0; b < NB; ++b) m &= (h ? pb[b] : pa[b]) ^ (((p >> b) & 1u) - 1u);
                const uint32_t c = (uint32_t)__popc(m);
                const uint32_t gb = rbp + ea + (h ? na : 0u);
                const uint32_t k = sop + (gb >> 5), bit = gb & 31u;
                const uint32_t lo = seg[k], hi = seg[k + 1];
                uint32_t run = (uint32_t)(((((uint64_t)hi) << 32) | lo) >> bit);
                if (c < 32u) run &= (1u << c) - 1u;
                if (run == 0u) continue;
                // the k-th set bit of the run is the k-th member, at the run's
                // output position plus the set bits before it
                uint32_t o = obp + sx[k] + (uint32_t)__popc(lo & ((1u << bit) - 1u));
                const uint32_t kb = (uint32_t)(w * W) + (2 * lane + h) * 32u;
                while (run) {
                    const uint32_t z = __builtin_ctz(run); // members to pass over
                    run = (run >> z) >> 1;
                    for (uint32_t i = 0; i < z; ++i) m &= m - 1u;
                    if (o < cap) d.out_idx[o] = kb + __builtin_ctz(m);
                    m &= m - 1u;
                    ++o;
                }
            }
        }
        cw = cwn[cs];
    }
}

// windows per group of the group decode for this layout (0: the block-per-
// window decode, for P = 1, P > 16 or fewer groups than fill the chip)
static uint32_t dec_group_windows(const CmapLayout& L)
{
    if (L.P < 2 || L.P > 16 || L.NCW != EG_NCW) return 0;
    const uint32_t G = (uint32_t)dg_group(L.nbits);
    if (ceil_div(L.NW, G) < 2048) return 0;
    return G;
}

// Pull-side scatter: dense [M][D] zero except entries [off[0], off[P]).
//
// Scalar values (D == 1) go through key windows of SC_W keys, since an
// aggregate's partitions each hold ascending keys:
//   cursors  one streaming pass over the entries: for each (window,
//            partition), the first entry of the partition at or after the
//            window's first key; a partition whose keys do not ascend marks
//            its pass block's flag word;
//   window   a block per window zeroes an LDS copy of the window, drops the
//            window's entries of every partition into it and writes the
//            window out with 16-byte stores: every dense element is written
//            once, by coalesced stores;
//   fix      if any flag word is set, the plain per-entry scatter over the
//            windows' output (values at distinct keys are written again,
//            so the result is the same whatever the cursors were).
// Rows (D > 1) zero the tensor, then a thread per 16 bytes (or value) of
// every row copies it.
constexpr int SC_W = 4096;          // keys per window
constexpr int SC_CUR_BLOCKS = 4096; // blocks of the cursor pass, one flag word each
constexpr int SC_FIX_BLOCKS = 128;  // blocks of the per-entry pass
constexpr int SC_KB = 8;            // entries per thread per load round of the window kernel

struct ScatterParams {
    const uint32_t* idx;
    const float* val;
    const uint64_t* off;
    uint32_t P, D;
    uint64_t capacity, M;
    float* dense;
    uint64_t NW;   // windows of SC_W keys over [0, M)
    uint64_t* cur; // [NW+1][P] first entry of partition p at or after key w SC_W
    uint32_t* bad; // [SC_CUR_BLOCKS] nonzero: the cursors cannot be trusted
    uint32_t nbad; // flag words written: the blocks of the cursor pass
};

// offsets clamped to the entries held; false if they do not ascend
__device__ __forceinline__ bool scatter_offsets(const ScatterParams& s, uint64_t* offs)
{
    for (uint32_t p = threadIdx.x; p <= s.P; p += blockDim.x) offs[p] = s.off[p] < s.capacity ? s.off[p] : s.capacity;
    __syncthreads();
    bool ok = true;
    for (uint32_t p = threadIdx.x; p < s.P; p += blockDim.x) ok = ok && offs[p] <= offs[p + 1];
    return __syncthreads_and(ok) != 0;
}

template <bool VEC>
__global__ __launch_bounds__(256) void scatter_cursor_kernel(ScatterParams s)
{
    __shared__ uint64_t offs[257];
    bool bad = !scatter_offsets(s, offs);
    if (!bad)
        bad = window_cursor_pass<VEC>(s.idx, s.capacity, offs, s.P, (uint32_t)s.NW,
                                      (uint32_t)__builtin_ctz((uint32_t)SC_W), s.cur);
    const int any = __syncthreads_or(bad);
    if (threadIdx.x == 0) s.bad[blockIdx.x] = any ? 1u : 0u;
}

// position of the entry j of the window among the partitions' runs: the
// largest p with pre[p] <= j
__device__ __forceinline__ uint32_t scatter_run_of(const uint32_t* pre, uint32_t P, uint32_t j)
{
    uint32_t lo = 0, hi = P;
    while (lo + 1 < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (pre[mid] <= j) lo = mid;
        else hi = mid;
    }
    return lo;
}

// NT: the window's stores bypass the caches (a dense tensor larger than the
// last-level cache)
template <bool NT>
__global__ __launch_bounds__(256) void scatter_window_kernel(ScatterParams s)
{
    __shared__ __align__(16) float buf[SC_W];
    __shared__ uint64_t beg[256];
    __shared__ uint32_t pre[257];
    __shared__ uint32_t scan_lds[256 / SG_WAVE + 1];
    const uint32_t P = s.P, t = threadIdx.x;
    // windows in launch order: the XCDs write neighbouring windows together
    // (measured faster than giving each XCD a contiguous run of windows)
    const uint64_t w = blockIdx.x, k0 = w * SC_W;
    uint32_t n = 0;
    if (t < P) {
        // cursors clamped to the partition's entries (they are only read
        // inside them, whatever the cursor pass found)
        const uint64_t lo = s.off[t] < s.capacity ? s.off[t] : s.capacity;
        uint64_t hi = s.off[t + 1] < s.capacity ? s.off[t + 1] : s.capacity;
        if (hi < lo) hi = lo;
        uint64_t b = s.cur[w * P + t], e = s.cur[(w + 1) * P + t];
        b = b < lo ? lo : (b > hi ? hi : b);
        e = e < lo ? lo : (e > hi ? hi : e);
        beg[t] = b;
        if (e > b) {
            // an ascending partition holds at most SC_W keys of a window below M
            n = e - b <= (uint64_t)SC_W ? (uint32_t)(e - b) : (uint32_t)SC_W;
            if (e - b > (uint64_t)SC_W) s.bad[0] = 1u;
        }
    }
    float4* b4 = reinterpret_cast<float4*>(buf);
#pragma unroll
    for (int j = 0; j < SC_W / 4 / 256; ++j) b4[j * 256 + t] = make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t tot;
    const uint32_t ex = block_excl_scan<256>(n, scan_lds, &tot);
    if (t < P) pre[t] = ex;
    __syncthreads();
    for (uint32_t j0 = 0; j0 < tot; j0 += 256 * SC_KB) {
        uint32_t x[SC_KB];
        float v[SC_KB];
#pragma unroll
        for (int r = 0; r < SC_KB; ++r) {
            const uint32_t j = j0 + r * 256 + t;
            x[r] = 0xffffffffu;
            v[r] = 0.f;
            if (j < tot) {
                const uint32_t p = scatter_run_of(pre, P, j);
                const uint64_t i = beg[p] + (j - pre[p]);
                x[r] = s.idx[i];
                v[r] = s.val[i];
            }
        }
#pragma unroll
        for (int r = 0; r < SC_KB; ++r) {
            if (j0 + r * 256 + t >= tot) continue;
            if (x[r] >= s.M) {
                report_error(kDevErrIndexRange);
                continue;
            }
            const uint64_t o = (uint64_t)x[r] - k0;
            if (o < (uint64_t)SC_W) buf[o] = v[r];
        }
    }
    __syncthreads();
    float4* d4 = reinterpret_cast<float4*>(s.dense + k0);
    if (w + 1 < s.NW) { // a whole window below M
        if (NT) {
            typedef float v4f __attribute__((ext_vector_type(4)));
            const v4f* bv = reinterpret_cast<const v4f*>(buf);
            v4f* dv = reinterpret_cast<v4f*>(s.dense + k0);
#pragma unroll
            for (int j = 0; j < SC_W / 4 / 256; ++j) __builtin_nontemporal_store(bv[j * 256 + t], &dv[j * 256 + t]);
        } else {
#pragma unroll
            for (int j = 0; j < SC_W / 4 / 256; ++j) d4[j * 256 + t] = b4[j * 256 + t];
        }
    } else { // the last window: keys [k0, M), 1 to SC_W of them
        const uint32_t lim = (uint32_t)(s.M - k0);
        for (uint32_t j = t; j < lim / 4; j += 256) d4[j] = b4[j];
        for (uint32_t j = (lim / 4) * 4 + t; j < lim; j += 256) s.dense[k0 + j] = buf[j];
    }
}

// the plain scatter: every entry's value to its key (for D == 1 only when a
// flag word of the cursor pass is set; D == 0 checks the keys only)
__global__ __launch_bounds__(256) void scatter_kernel(ScatterParams s)
{
    if (s.bad) {
        uint32_t any = 0;
        for (uint32_t j = threadIdx.x; j < s.nbad; j += 256) any |= s.bad[j];
        if (!__syncthreads_or(any != 0u)) return;
    }
    uint64_t b = s.off[0], e = s.off[s.P];
    if (e > s.capacity) e = s.capacity;
    if (b > e) b = e;
    for (uint64_t i = b + blockIdx.x * 256ull + threadIdx.x; i < e; i += (uint64_t)gridDim.x * 256) {
        const uint32_t x = s.idx[i];
        if (x >= s.M) {
            report_error(kDevErrIndexRange);
            continue;
        }
        if (s.D == 1) s.dense[x] = s.val[i];
    }
}

// rows of D > 1: a thread per 16 bytes of a row (VEC: D a multiple of 4 and
// the values 16-byte aligned) or per value, the grid over every thread of
// the entries held, so each thread makes one index load, one value load and
// one store (a wave per row walking many rows waits on each row in turn)
template <bool VEC>
__global__ __launch_bounds__(256) void scatter_rows_kernel(ScatterParams s)
{
    uint64_t b = s.off[0], e = s.off[s.P];
    if (e > s.capacity) e = s.capacity;
    if (b > e) b = e;
    const uint32_t per = VEC ? s.D / 4 : s.D; // threads per row
    const uint64_t n = (e - b) * per;
    const bool narrow = n <= 0xffffffffull; // 32-bit division
    for (uint64_t t = blockIdx.x * 256ull + threadIdx.x; t < n; t += (uint64_t)gridDim.x * 256) {
        const uint64_t r = narrow ? (uint64_t)((uint32_t)t / per) : t / per;
        const uint32_t c = (uint32_t)(t - r * per);
        const uint64_t i = b + r;
        const uint32_t x = s.idx[i];
        if (x >= s.M) {
            if (c == 0) report_error(kDevErrIndexRange);
            continue;
        }
        if (VEC)
            reinterpret_cast<float4*>(s.dense + (uint64_t)x * s.D)[c] =
                reinterpret_cast<const float4*>(s.val + i * s.D)[c];
        else
            s.dense[(uint64_t)x * s.D + c] = s.val[i * s.D + c];
    }
}

__global__ __launch_bounds__(256) void scatter_zero_kernel(ScatterParams s)
{
    const uint64_t words = s.M * (s.D ? s.D : 1);
    const uint64_t n4 = words / 4;
    float4* d4 = reinterpret_cast<float4*>(s.dense);
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < n4; i += (uint64_t)gridDim.x * 256)
        d4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (uint64_t i = n4 * 4 + blockIdx.x * 256ull + threadIdx.x; i < words; i += (uint64_t)gridDim.x * 256)
        s.dense[i] = 0.f;
}

// non-empty 256-gradient blocks of an aggregate: one bit per block
__global__ __launch_bounds__(256) void blocks_mark_kernel(const uint32_t* idx, const uint64_t* off, uint32_t P,
                                                          uint64_t capacity, uint64_t M, uint32_t* used)
{
    uint64_t b = off[0], e = off[P];
    if (e > capacity) e = capacity;
    if (b > e) b = e;
    for (uint64_t i = b + blockIdx.x * 256ull + threadIdx.x; i < e; i += (uint64_t)gridDim.x * 256) {
        const uint32_t x = idx[i];
        if (x >= M) {
            report_error(kDevErrIndexRange);
            continue;
        }
        const uint32_t blk = x >> 8;
        atomicOr(&used[blk >> 5], 1u << (blk & 31u));
    }
}

__global__ __launch_bounds__(256) void blocks_count_kernel(const uint32_t* used, uint64_t words, unsigned long long* out)
{
    uint32_t c = 0;
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < words; i += (uint64_t)gridDim.x * 256) c += __popc(used[i]);
    c = wave_sum(c);
    if (lane_id() == 0 && c) atomicAdd(out, (unsigned long long)c);
}

} // namespace sg

using namespace sg;

extern "C" size_t sg_decode_workspace_bytes(uint64_t M, uint32_t P)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32)) return 0;
    const uint64_t maxw = sg_encode_max_words(M, P);
    Carver c(nullptr);
    c.take<uint32_t>(maxw + 1);
    c.take<uint32_t>(ceil_div(maxw, DS_WPB));
    return (size_t)c.bytes();
}

extern "C" int sg_decode(const uint32_t* d_bitmap, uint64_t bitmap_words, const void* d_cmap, size_t cmap_bytes,
                         uint64_t M, uint32_t P, uint32_t* d_out_idx, uint64_t capacity, uint64_t* d_out_off,
                         void* d_ws, size_t ws_bytes, void* stream)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32)) return SG_EINVAL;
    if (!d_bitmap || !d_cmap || !d_out_idx || !d_out_off || !d_ws) return SG_EINVAL;
    if (cmap_bytes < sg_classmap_bytes(M, P)) return SG_ECAPACITY;
    if (ws_bytes < sg_decode_workspace_bytes(M, P)) return SG_ECAPACITY;
    DecParams d;
    d.L = cmap_layout(M, P);
    if (d.L.W / 32 + P + 2 > (uint64_t)DC_WORDS) return SG_EUNSUPPORTED;
    d.q = cmap_ptrs(const_cast<void*>(d_cmap), d.L);
    d.bitmap = d_bitmap;
    d.bitmap_words = bitmap_words;
    d.out_idx = d_out_idx;
    d.capacity = capacity;
    d.out_off = d_out_off;
    const uint64_t maxw = sg_encode_max_words(M, P);
    const uint64_t words = bitmap_words < maxw ? bitmap_words : maxw; // the scan covers at most these
    d.bitmap_words = words;
    d.NB = (uint32_t)ceil_div(words ? words : 1, DS_WPB);
    Carver c(d_ws);
    d.wpre = c.take<uint32_t>(maxw + 1);
    d.bsum = c.take<uint32_t>(ceil_div(maxw, DS_WPB));
    hipStream_t st = as_stream(stream);
    const bool vec = (uintptr_t)d_bitmap % 16 == 0;
    if (vec) dec_wsum_kernel<true><<<d.NB, 256, 0, st>>>(d);
    else dec_wsum_kernel<false><<<d.NB, 256, 0, st>>>(d);
    SG_TRY_LAUNCH();
    dec_bscan_kernel<<<1, 1024, 0, st>>>(d);
    SG_TRY_LAUNCH();
    if (vec) dec_wpre_kernel<true><<<d.NB, 256, 0, st>>>(d);
    else dec_wpre_kernel<false><<<d.NB, 256, 0, st>>>(d);
    SG_TRY_LAUNCH();
    probe_begin(SG_PROBE_DECODE, st);
    const uint32_t G = dec_group_windows(d.L);
    if (G) {
        const uint64_t NG = ceil_div(d.L.NW, G);
        const unsigned blocks = (unsigned)ceil_div(NG, DG_WAVES);
        switch (d.L.nbits) {
        case 1: dec_group_kernel<1, dg_group(1)><<<blocks, DG_WAVES * SG_WAVE, 0, st>>>(d, NG); break;
        case 2: dec_group_kernel<2, dg_group(2)><<<blocks, DG_WAVES * SG_WAVE, 0, st>>>(d, NG); break;
        case 3: dec_group_kernel<3, dg_group(3)><<<blocks, DG_WAVES * SG_WAVE, 0, st>>>(d, NG); break;
        default: dec_group_kernel<4, dg_group(4)><<<blocks, DG_WAVES * SG_WAVE, 0, st>>>(d, NG); break;
        }
    } else {
        dec_emit_kernel<<<(unsigned)d.L.NW, DC_THREADS, 0, st>>>(d);
    }
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_DECODE, st);
    return SG_OK;
}

extern "C" size_t sg_scatter_dense_workspace_bytes(uint64_t M, uint32_t P)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32)) return 0;
    Carver c(nullptr);
    c.take<uint32_t>(SC_CUR_BLOCKS);
    c.take<uint64_t>((ceil_div(M, SC_W) + 1) * P);
    return (size_t)c.bytes();
}

extern "C" int sg_scatter_dense(const uint32_t* d_idx, const float* d_val, uint32_t D, const uint64_t* d_off,
                                uint32_t P, uint64_t capacity, uint64_t M, float* d_dense, void* d_ws, size_t ws_bytes,
                                void* stream)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32) || D > 65536 || !d_off || !d_dense || !d_ws) return SG_EINVAL;
    if (capacity > 0 && (!d_idx || (D > 0 && !d_val))) return SG_EINVAL;
    if ((uintptr_t)d_dense % 16) return SG_EINVAL;
    if (ws_bytes < sg_scatter_dense_workspace_bytes(M, P)) return SG_ECAPACITY;
    ScatterParams s;
    s.idx = d_idx;
    s.val = d_val;
    s.off = d_off;
    s.P = P;
    s.D = D;
    s.capacity = capacity;
    s.M = M;
    s.dense = d_dense;
    s.NW = ceil_div(M, SC_W);
    Carver c(d_ws);
    s.bad = c.take<uint32_t>(SC_CUR_BLOCKS);
    s.cur = c.take<uint64_t>((s.NW + 1) * P);
    hipStream_t st = as_stream(stream);
    if (D == 1 && capacity > 0) {
        // a chunk per block where the entries allow, and enough blocks for
        // the cursors of empty partitions (every block writes its flag word)
        uint64_t cb = ceil_div(capacity, (uint64_t)WC_CHUNK);
        const uint64_t fill = ceil_div((s.NW + 1) * P, 4096);
        cb = cb > fill ? cb : fill;
        s.nbad = (uint32_t)(cb < SC_CUR_BLOCKS ? cb : SC_CUR_BLOCKS);
        if ((uintptr_t)d_idx % 16 == 0)
            scatter_cursor_kernel<true><<<s.nbad, 256, 0, st>>>(s);
        else
            scatter_cursor_kernel<false><<<s.nbad, 256, 0, st>>>(s);
        SG_TRY_LAUNCH();
        probe_begin(SG_PROBE_SCATTER, st);
        if (M * 4 > (256ull << 20)) // beyond the 256 MB last-level cache
            scatter_window_kernel<true><<<(unsigned)s.NW, 256, 0, st>>>(s);
        else
            scatter_window_kernel<false><<<(unsigned)s.NW, 256, 0, st>>>(s);
        SG_TRY_LAUNCH();
        probe_end(SG_PROBE_SCATTER, st);
        // the per-entry pass, needed only after a flag: a small grid
        const uint64_t fb = ceil_div(capacity, 256);
        scatter_kernel<<<(unsigned)(fb < SC_FIX_BLOCKS ? fb : SC_FIX_BLOCKS), 256, 0, st>>>(s);
        SG_TRY_LAUNCH();
        return SG_OK;
    }
    const uint64_t words = M * (D ? D : 1);
    s.bad = nullptr;
    s.nbad = 0;
    scatter_zero_kernel<<<(unsigned)(ceil_div(words / 4 + 1, 256) < 8192 ? ceil_div(words / 4 + 1, 256) : 8192), 256, 0, st>>>(s);
    SG_TRY_LAUNCH();
    if (capacity > 0) {
        probe_begin(SG_PROBE_SCATTER, st);
        if (D > 1) {
            const bool vec = D % 4 == 0 && (uintptr_t)d_val % 16 == 0;
            const uint64_t nb = ceil_div(capacity * (vec ? D / 4 : D), 256);
            const unsigned blocks = (unsigned)(nb < 65536 ? nb : 65536);
            if (vec) scatter_rows_kernel<true><<<blocks, 256, 0, st>>>(s);
            else scatter_rows_kernel<false><<<blocks, 256, 0, st>>>(s);
        } else {
            scatter_kernel<<<(unsigned)(ceil_div(capacity, 256) < 8192 ? ceil_div(capacity, 256) : 8192), 256, 0, st>>>(s);
        }
        SG_TRY_LAUNCH();
        probe_end(SG_PROBE_SCATTER, st);
    }
    return SG_OK;
}

extern "C" size_t sg_format_sizes_workspace_bytes(uint64_t M)
{
    return (size_t)(align_up(4ull * ceil_div(ceil_div(M, 256), 32), 256) + 256);
}

extern "C" int sg_format_sizes(const uint32_t* d_agg_idx, const uint64_t* d_agg_off, uint64_t capacity, uint64_t M,
                               uint32_t P, uint32_t D, const void* d_cmap, size_t cmap_bytes, uint64_t* h_out,
                               void* d_ws, size_t ws_bytes, void* stream)
{
    if (P == 0 || P > 256 || M == 0 || M >= (1ull << 32) || !d_agg_off || !d_cmap || !h_out || !d_ws) return SG_EINVAL;
    if (capacity > 0 && !d_agg_idx) return SG_EINVAL;
    if (cmap_bytes < sg_classmap_bytes(M, P)) return SG_ECAPACITY;
    if (ws_bytes < sg_format_sizes_workspace_bytes(M)) return SG_ECAPACITY;
    hipStream_t st = as_stream(stream);
    const CmapLayout L = cmap_layout(M, P);
    CmapPtrs q = cmap_ptrs(const_cast<void*>(d_cmap), L);
    Carver c(d_ws);
    const uint64_t words = ceil_div(ceil_div(M, 256), 32);
    uint32_t* used = c.take<uint32_t>(words);
    unsigned long long* cnt = c.take<unsigned long long>(1);
    int rc = fill_u32(used, words, 0, st);
    if (rc) return rc;
    rc = fill_u64(reinterpret_cast<uint64_t*>(cnt), 1, 0, st);
    if (rc) return rc;
    if (capacity > 0) {
        blocks_mark_kernel<<<(unsigned)(ceil_div(capacity, 256) < 4096 ? ceil_div(capacity, 256) : 4096), 256, 0, st>>>(
            d_agg_idx, d_agg_off, P, capacity, M, used);
        SG_TRY_LAUNCH();
    }
    blocks_count_kernel<<<(unsigned)(ceil_div(words, 256) < 1024 ? (ceil_div(words, 256) ? ceil_div(words, 256) : 1) : 1024), 256, 0, st>>>(
        used, words, cnt);
    SG_TRY_LAUNCH();
    uint64_t off0 = 0, offP = 0, nblocks = 0, hash_words = 0;
    CmapHeader h;
    SG_TRY(hipMemcpyAsync(&off0, d_agg_off, 8, hipMemcpyDeviceToHost, st));
    SG_TRY(hipMemcpyAsync(&offP, d_agg_off + P, 8, hipMemcpyDeviceToHost, st));
    SG_TRY(hipMemcpyAsync(&nblocks, cnt, 8, hipMemcpyDeviceToHost, st));
    SG_TRY(hipMemcpyAsync(&hash_words, q.word_off + P, 8, hipMemcpyDeviceToHost, st));
    SG_TRY(hipMemcpyAsync(&h, q.hdr, sizeof(h), hipMemcpyDeviceToHost, st));
    SG_TRY(hipStreamSynchronize(st));
    if (h.magic != CM_MAGIC || h.P != P || h.M != M) return SG_EINVAL;
    if (offP > capacity) offP = capacity;
    const uint64_t U = offP > off0 ? offP - off0 : 0;
    uint64_t bitmap_words = 0;
    for (uint32_t p = 0; p < P; ++p) {
        const uint64_t lo = (uint64_t)(((unsigned __int128)M * p) / P), hi = (uint64_t)(((unsigned __int128)M * (p + 1)) / P);
        bitmap_words += (hi - lo + 31) / 32;
    }
    h_out[0] = M * 4ull * D;
    h_out[1] = U * (4ull + 4ull * D);
    h_out[2] = nblocks * (256ull * 4ull * D + 4ull);
    h_out[3] = bitmap_words * 4ull + U * 4ull * D;
    h_out[4] = hash_words * 4ull + U * 4ull * D;
    h_out[5] = U;
    h_out[6] = nblocks;
    return SG_OK;
}

/*
 * sg_oracle.c -- plain, slow, single-threaded CPU oracle for the sparse
 * gradient synchronization hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Only the test suite, the smoke check of the package entry
 * and the CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or constant generator with the HIP library.
 *
 * Sources (the pages this follows; each function names its passage):
 *   [Zen]  "Zen: Empowering Distributed Training with Sparsity-driven Data
 *          Synchronization" (OSDI'25), digest page.
 *   [Skip] "SkipReduce: (Interconnection) Network Sparsity to Accelerate
 *          Distributed Machine Learning" (MICRO'25), digest page.
 *   [Ring] CMU 15-442/642 "Machine Learning Systems: Distributed Training and
 *          Parallelization -- Data Parallelism and Zero Redundancy
 *          Optimization", section "Ring AllReduce", aggregation phase.
 *
 * Floating point: every sum is formed in IEEE double (fp64) from inputs that
 * are converted exactly (fp32 and bf16 both embed exactly in double).  The
 * file is compiled with -ffp-contract=off so no fused multiply-add changes a
 * rounding.  Integer work (indices, partitions, counts, bitmaps) is exact.
 *
 * Pins: see tests/test_oracle_pins.py.  Every function below is pinned by at
 * least one check that does not re-run this code (brute force, a published
 * check value, a closed form or an invariant).  The one documented "parity
 * unpinned" item is which hash the Zen authors actually ran: the page cites
 * "MurmurHash 2.0" and nothing more, so h0 below is the reading that
 * MurmurHash2 (32-bit) of the index's 4 little-endian bytes, then mod P, is
 * that hash.
 */
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ENOMEM -2
#define ORC_EINCONSISTENT -3

#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------------------ */
/* Hash and random-number definitions                                        */
/* ------------------------------------------------------------------------ */

/* MurmurHash2, 32-bit variant, written from Austin Appleby's public
 * description (2008): multiply constant 0x5bd1e995, shift 24, 4-byte blocks
 * read little-endian, a 1-3 byte tail, and a final three-step avalanche.
 * [Zen] section 4 (Implementation) names MurmurHash 2.0 with per-function
 * seeds as the hash family. */
uint32_t orc_murmur2(const uint8_t* data, uint64_t len, uint32_t seed)
{
    const uint32_t m = 0x5bd1e995u;
    uint32_t h = seed ^ (uint32_t)len;
    while (len >= 4) {
        uint32_t k = (uint32_t)data[0] | ((uint32_t)data[1] << 8) |
                     ((uint32_t)data[2] << 16) | ((uint32_t)data[3] << 24);
        k *= m;
        k ^= k >> 24;
        k *= m;
        h *= m;
        h ^= k;
        data += 4;
        len -= 4;
    }
    if (len == 3) h ^= (uint32_t)data[2] << 16;
    if (len >= 2) h ^= (uint32_t)data[1] << 8;
    if (len >= 1) {
        h ^= (uint32_t)data[0];
        h *= m;
    }
    h ^= h >> 13;
    h *= m;
    h ^= h >> 15;
    return h;
}

/* h0: the first-level partition hash of [Zen] section 3.2 (Technique #3 and
 * Algorithm 1, the line that picks the partition): the same function on every
 * worker, so an index always reaches the same server. */
uint32_t orc_h0(uint32_t idx, uint32_t seed, uint32_t P)
{
    uint8_t b[4];
    b[0] = (uint8_t)(idx & 0xff);
    b[1] = (uint8_t)((idx >> 8) & 0xff);
    b[2] = (uint8_t)((idx >> 16) & 0xff);
    b[3] = (uint8_t)((idx >> 24) & 0xff);
    return orc_murmur2(b, 4, seed) % P;
}

/* h0 over an array, for tests that need many hashes at once. */
void orc_h0_array(const uint32_t* idx, uint64_t count, uint32_t seed, uint32_t P, uint32_t* out)
{
    uint64_t i;
    for (i = 0; i < count; ++i) out[i] = orc_h0(idx[i], seed, P);
}

/* SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): the state advances by the
 * golden-ratio increment and each output is the state passed through the
 * published two-multiply mixer. */
uint64_t orc_splitmix64_next(uint64_t* state)
{
    uint64_t z;
    *state += 0x9e3779b97f4a7c15ull;
    z = *state;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

/* The ctr-th output (0-based) of a SplitMix64 stream that starts at `seed`:
 * advance the state ctr+1 times, mix once. */
uint64_t orc_splitmix64_at(uint64_t seed, uint64_t ctr)
{
    /* the state advances by the same constant per output, so after ctr + 1
       outputs it is seed + (ctr + 1) * gamma (mod 2^64) */
    uint64_t s = seed + ctr * 0x9e3779b97f4a7c15ull;
    return orc_splitmix64_next(&s);
}

/* ------------------------------------------------------------------------ */
/* Small helpers                                                             */
/* ------------------------------------------------------------------------ */

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double f32_to_double(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double load_val(const void* base, int dtype, uint64_t i)
{
    if (dtype == ORC_BF16) return bf16_to_double(((const uint16_t*)base)[i]);
    return f32_to_double(((const uint32_t*)base)[i]);
}

/* Magnitude key of an element: the bit pattern with the sign bit cleared.
 * For IEEE floats of one sign, the bit pattern orders like the value, so
 * comparing these keys compares |x|. */
static uint32_t mag_key(const void* base, int dtype, uint64_t i)
{
    if (dtype == ORC_BF16) return (uint32_t)(((const uint16_t*)base)[i] & 0x7fffu);
    return ((const uint32_t*)base)[i] & 0x7fffffffu;
}

/* ------------------------------------------------------------------------ */
/* A1: top-k of a dense gradient into COO                                    */
/* ------------------------------------------------------------------------ */

/* Quickselect on distinct 64-bit keys: afterwards a[r] holds the value of rank
 * r (0-based, ascending).  Plain Lomuto partition with a middle pivot. */
static void quickselect_u64(uint64_t* a, uint64_t n, uint64_t r)
{
    uint64_t lo = 0, hi = n - 1;
    while (lo < hi) {
        uint64_t mid = lo + (hi - lo) / 2;
        uint64_t pivot = a[mid], t, store, i;
        a[mid] = a[hi];
        a[hi] = pivot;
        store = lo;
        for (i = lo; i < hi; ++i) {
            if (a[i] < pivot) {
                t = a[i];
                a[i] = a[store];
                a[store] = t;
                ++store;
            }
        }
        a[hi] = a[store];
        a[store] = pivot;
        if (store == r) return;
        if (r < store) hi = store - 1;
        else lo = store + 1;
    }
}

/* Per worker, the k entries of largest |g|, emitted in ascending index order
 * with the original signed value copied bit for bit.
 * [Skip] section 2 (top-k sparsification keeps the largest-magnitude
 * gradients) and [Zen] section 4 (DGC keeps the top 5%).
 * Reading: equal magnitudes (including +0 and -0) are broken toward the lower
 * index; this is encoded in the 64-bit key (magnitude, then complemented
 * index), which makes every key distinct, so "the k largest keys" is a unique
 * set. */
int orc_topk_to_coo(const void* dense, int dtype, uint32_t n, uint64_t M, uint64_t k,
                    uint32_t* out_idx, void* out_val)
{
    uint64_t* keys;
    uint32_t w;
    if (k > M || M > 0xffffffffull) return ORC_EINVAL;
    if (k == 0 || n == 0) return ORC_OK;
    keys = (uint64_t*)malloc(M * sizeof(uint64_t));
    if (!keys) return ORC_ENOMEM;
    for (w = 0; w < n; ++w) {
        uint64_t i, thr, o = 0;
        const uint64_t base = (uint64_t)w * M;
        for (i = 0; i < M; ++i)
            keys[i] = ((uint64_t)mag_key(dense, dtype, base + i) << 32) |
                      (uint64_t)(0xffffffffu - (uint32_t)i);
        /* the k-th largest key has ascending rank M - k */
        quickselect_u64(keys, M, M - k);
        thr = keys[M - k];
        for (i = 0; i < M; ++i) {
            uint64_t key = ((uint64_t)mag_key(dense, dtype, base + i) << 32) |
                           (uint64_t)(0xffffffffu - (uint32_t)i);
            if (key >= thr) {
                out_idx[(uint64_t)w * k + o] = (uint32_t)i;
                if (dtype == ORC_BF16)
                    ((uint16_t*)out_val)[(uint64_t)w * k + o] = ((const uint16_t*)dense)[base + i];
                else
                    ((uint32_t*)out_val)[(uint64_t)w * k + o] = ((const uint32_t*)dense)[base + i];
                ++o;
            }
        }
        if (o != k) {
            free(keys);
            return ORC_EINCONSISTENT;
        }
    }
    free(keys);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* DGC with a sampled global threshold and residual accumulation             */
/* ------------------------------------------------------------------------ */

/* Descending order of 32-bit keys, for qsort. */
static int cmp_u32_desc(const void* x, const void* y)
{
    uint32_t a = *(const uint32_t*)x, b = *(const uint32_t*)y;
    return a < b ? 1 : (a > b ? -1 : 0);
}

/* Position of sample j of S in a worker's M elements: the midpoint of the
 * j-th of S equal strides, floor((2j + 1) M / (2S)); every position when
 * S >= M. */
uint64_t orc_dgc_sample_pos(uint64_t M, uint64_t S, uint64_t j)
{
    if (S >= M) return j;
    return (uint64_t)(((unsigned __int128)(2 * j + 1) * M) / (2 * S));
}

/* Rank of the threshold among the pooled samples: ks = ceil(density * Ns)
 * evaluated in double, clamped to [1, Ns]. */
uint64_t orc_dgc_rank(double density, uint64_t Ns)
{
    double x = ceil(density * (double)Ns);
    if (!(x >= 1.0)) return 1;
    if (x >= (double)Ns) return Ns;
    return (uint64_t)x;
}

/* One iteration of DGC-style top-k with a sampled global threshold and
 * residual accumulation, for n workers at once.
 *   [Zen] section 4 (Implementation): DGC adapted to tensor parallelism --
 *   every device samples its gradient locally, the samples of all devices are
 *   gathered, one global top-k threshold is computed from them, and every
 *   device applies it locally to select its top-k values.
 *   [Skip] section 2: gradients that are not selected are accumulated
 *   locally into later iterations' gradients until their accumulated
 *   magnitude is large enough to be selected (residuals).
 * Steps, in the pages' order:
 *   1. accumulate: a[w][i] = resid[w][i] + grad[w][i], one fp32 addition;
 *   2. sample: worker w contributes |a[w][pos_j]| for the S positions of
 *      orc_dgc_sample_pos (S clamped to M);
 *   3. gather: the n*S samples form one pool;
 *   4. threshold: thr = the ks-th largest pooled magnitude, ks = orc_dgc_rank;
 *   5. select: every (w, i) with |a[w][i]| >= thr, in ascending i, emitted as
 *      (i, a[w][i]) into out_idx[w][*], out_val[w][*] (at most cap per worker;
 *      count[w] is the number selected, which may exceed cap);
 *   6. residual: resid[w][i] = 0 where selected, a[w][i] elsewhere.
 * Magnitudes are compared as fp32 bit patterns with the sign cleared (they
 * order like |a|); inputs are finite.  thr_key (optional) receives the
 * threshold's bit pattern. */
int orc_dgc_select(const float* grad, float* resid, uint32_t n, uint64_t M, double density, uint64_t S,
                   uint32_t* out_idx, float* out_val, uint64_t cap, uint64_t* count, uint32_t* thr_key)
{
    uint32_t w;
    uint64_t i, j, Ns, ks;
    uint32_t* pool;
    uint32_t thr;
    if (n == 0 || M == 0 || S == 0) return ORC_EINVAL;
    if (S > M) S = M;
    Ns = (uint64_t)n * S;
    pool = (uint32_t*)malloc(Ns * sizeof(uint32_t));
    if (!pool) return ORC_ENOMEM;
    for (w = 0; w < n; ++w)
        for (j = 0; j < S; ++j) {
            uint64_t e = (uint64_t)w * M + orc_dgc_sample_pos(M, S, j);
            float a = resid[e] + grad[e];
            uint32_t bits;
            memcpy(&bits, &a, 4);
            pool[(uint64_t)w * S + j] = bits & 0x7fffffffu;
        }
    qsort(pool, Ns, sizeof(uint32_t), cmp_u32_desc);
    ks = orc_dgc_rank(density, Ns);
    thr = pool[ks - 1];
    free(pool);
    if (thr_key) *thr_key = thr;
    for (w = 0; w < n; ++w) {
        uint64_t c = 0;
        for (i = 0; i < M; ++i) {
            uint64_t e = (uint64_t)w * M + i;
            float a = resid[e] + grad[e];
            uint32_t bits;
            memcpy(&bits, &a, 4);
            if ((bits & 0x7fffffffu) >= thr) {
                if (c < cap) {
                    out_idx[(uint64_t)w * cap + c] = (uint32_t)i;
                    out_val[(uint64_t)w * cap + c] = a;
                }
                ++c;
                resid[e] = 0.0f;
            } else {
                resid[e] = a;
            }
        }
        count[w] = c;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* A2: hash partition                                                        */
/* ------------------------------------------------------------------------ */

/* Each worker's COO entries grouped by p = h0(idx), partition 0 first, the
 * entries of one partition kept in input order.
 * [Zen] section 3.1 (Problem 1: a map f from indices to [n] that is the same
 * for all workers) and section 3.2 (Technique #3, Algorithm 1's first-level
 * hash).  Reading: order inside a partition does not change the aggregate
 * ([Zen] Technique #1 says so), so the contract fixes the stable order, which
 * makes outputs comparable byte for byte.
 * D is the row width (values per index); D == 0 means indices only.
 * part_off is [n][P+1], absolute offsets into the output. */
int orc_hash_partition(const uint32_t* idx, const void* val, int dtype, uint32_t D,
                       const uint64_t* in_off, uint32_t n, uint32_t P, uint32_t seed,
                       uint32_t* out_idx, void* out_val, uint64_t* part_off)
{
    uint32_t w, p;
    const size_t esz = (dtype == ORC_BF16) ? 2 : 4;
    if (P == 0) return ORC_EINVAL;
    for (w = 0; w < n; ++w) {
        uint64_t o = in_off[w];
        uint64_t b = in_off[w], e = in_off[w + 1], i;
        if (e < b) return ORC_EINVAL;
        for (p = 0; p < P; ++p) {
            part_off[(uint64_t)w * (P + 1) + p] = o;
            for (i = b; i < e; ++i) {
                if (orc_h0(idx[i], seed, P) != p) continue;
                out_idx[o] = idx[i];
                if (D > 0)
                    memcpy((char*)out_val + o * D * esz, (const char*)val + i * D * esz, D * esz);
                ++o;
            }
        }
        part_off[(uint64_t)w * (P + 1) + P] = o;
        if (o != e) return ORC_EINCONSISTENT;
    }
    return ORC_OK;
}

/* Algorithm 1 of [Zen] section 3.2 (hierarchical hashing with the four
 * techniques), run sequentially, worker by worker, entries in input order.
 * Partition memory x[p] has r1 parallel slots and r2 serial slots (Technique
 * #1); entry e with index idx goes to partition p = h0(idx) (Technique #3)
 * and tries the slots h_i(idx) for i = 1..k in turn (Technique #2), taking
 * the first empty one; after k occupied slots it takes the next serial slot
 * r1 + c_p (the atomic counter of lines 9-10, starting at r1), and is lost
 * (counted in overflow) when the serial slots are used up.  Technique #4's
 * read-after-write check concerns concurrent writers only; sequentially
 * every write sticks.  Extraction (lines 19-23) reads each partition's slots
 * in slot order.
 * Readings: indices are 0-based, and a slot holds (entry position + 1), 0
 * meaning empty, so the extraction gathers both the index and its values;
 * h_i(idx) = MurmurHash2(idx as 4 LE bytes, seed + i) mod r1 (the text maps
 * h_i to [r1]).
 * Outputs as orc_hash_partition (out_idx, out_val, part_off [n][P+1]
 * absolute), slot_of[out position] = the slot that held the entry;
 * counts[w*2] = serial writes, counts[w*2+1] = entries lost. */
int orc_hierarchical_hash(const uint32_t* idx, const void* val, int dtype, uint32_t D, const uint64_t* in_off,
                          uint32_t n, uint32_t P, uint32_t seed, uint32_t k, uint64_t r1, uint64_t r2,
                          uint32_t* out_idx, void* out_val, uint64_t* part_off, uint32_t* slot_of,
                          uint64_t* counts)
{
    uint32_t w, p, i;
    uint64_t e, q;
    const uint64_t R = r1 + r2;
    size_t esz = dtype == ORC_BF16 ? 2 : 4;
    uint32_t* x;
    uint64_t* c;
    if (P == 0 || r1 == 0 || k == 0) return ORC_EINVAL;
    x = (uint32_t*)malloc((size_t)P * R * sizeof(uint32_t));
    c = (uint64_t*)malloc((size_t)P * sizeof(uint64_t));
    if (!x || !c) {
        free(x);
        free(c);
        return ORC_ENOMEM;
    }
    for (w = 0; w < n; ++w) {
        uint64_t o = in_off[w];
        memset(x, 0, (size_t)P * R * sizeof(uint32_t));
        for (p = 0; p < P; ++p) c[p] = r1;
        counts[2 * w] = 0;
        counts[2 * w + 1] = 0;
        for (e = in_off[w]; e < in_off[w + 1]; ++e) {
            uint32_t id = idx[e];
            int placed = 0;
            p = orc_h0(id, seed, P);
            for (i = 1; i <= k && !placed; ++i) {
                uint8_t b[4];
                b[0] = (uint8_t)id;
                b[1] = (uint8_t)(id >> 8);
                b[2] = (uint8_t)(id >> 16);
                b[3] = (uint8_t)(id >> 24);
                q = orc_murmur2(b, 4, seed + i) % r1;
                if (x[(uint64_t)p * R + q] == 0) {
                    x[(uint64_t)p * R + q] = (uint32_t)(e - in_off[w] + 1);
                    placed = 1;
                }
            }
            if (!placed) {
                counts[2 * w] += 1;
                q = c[p]++;
                if (q < R) x[(uint64_t)p * R + q] = (uint32_t)(e - in_off[w] + 1);
                else counts[2 * w + 1] += 1;
            }
        }
        for (p = 0; p < P; ++p) {
            part_off[(uint64_t)w * (P + 1) + p] = o;
            for (q = 0; q < R; ++q) {
                uint32_t s = x[(uint64_t)p * R + q];
                uint64_t src;
                if (!s) continue;
                src = in_off[w] + s - 1;
                out_idx[o] = idx[src];
                if (D > 0 && val)
                    memcpy((char*)out_val + o * D * esz, (const char*)val + src * D * esz, D * esz);
                if (slot_of) slot_of[o] = (uint32_t)q;
                ++o;
            }
        }
        part_off[(uint64_t)w * (P + 1) + P] = o;
    }
    free(x);
    free(c);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* A3: per-partition union-sum                                               */
/* ------------------------------------------------------------------------ */

/* For each partition p, the union of all workers' indices in that partition,
 * ascending, each with its values summed over the workers that hold it.
 * [Zen] section 3.1 (each server aggregates the partition it receives) and
 * section 3.2 ("no accuracy impact": the sparse aggregate equals the dense
 * AllReduce of the same gradients).  Written as that plain definition: a dense
 * scatter-add over [0, M) in double, then the touched indices in order.
 * Reading: membership means "some worker sent the index", not "the sum is
 * non-zero"; an index whose values cancel to 0 stays in the aggregate.
 * Outputs: agg_idx[cap], agg_val[cap*D] (double), agg_abs[cap*D] (double, the
 * sum of |x| of the same terms, used for the tolerance), agg_off[P+1].
 * Returns ORC_EINCONSISTENT if one index arrives in two partitions. */
int orc_aggregate(const uint32_t* idx, const void* val, int dtype, uint32_t D,
                  const uint64_t* part_off, uint32_t n, uint32_t P, uint64_t M,
                  uint32_t* agg_idx, double* agg_val, double* agg_abs, uint64_t* agg_off)
{
    double *acc = NULL, *accabs = NULL;
    uint32_t* owner = NULL; /* partition + 1 of a touched index, 0 if untouched */
    uint64_t* cnt = NULL;
    uint32_t w, p;
    uint64_t i, d;
    const uint32_t Dv = D ? D : 1;
    int rc = ORC_OK;
    if (P == 0 || M > 0xffffffffull) return ORC_EINVAL;
    acc = (double*)calloc(M * Dv, sizeof(double));
    accabs = (double*)calloc(M * Dv, sizeof(double));
    owner = (uint32_t*)calloc(M, sizeof(uint32_t));
    cnt = (uint64_t*)calloc(P + 1, sizeof(uint64_t));
    if (!acc || !accabs || !owner || !cnt) {
        rc = ORC_ENOMEM;
        goto done;
    }
    for (w = 0; w < n; ++w) {
        for (p = 0; p < P; ++p) {
            uint64_t b = part_off[(uint64_t)w * (P + 1) + p];
            uint64_t e = part_off[(uint64_t)w * (P + 1) + p + 1];
            for (i = b; i < e; ++i) {
                uint32_t x = idx[i];
                if (x >= M) {
                    rc = ORC_EINVAL;
                    goto done;
                }
                if (owner[x] != 0 && owner[x] != p + 1) {
                    rc = ORC_EINCONSISTENT;
                    goto done;
                }
                owner[x] = p + 1;
                for (d = 0; d < D; ++d) {
                    double v = load_val(val, dtype, i * D + d);
                    acc[(uint64_t)x * Dv + d] += v;
                    accabs[(uint64_t)x * Dv + d] += fabs(v);
                }
            }
        }
    }
    for (i = 0; i < M; ++i)
        if (owner[i]) cnt[owner[i]]++;
    agg_off[0] = 0;
    for (p = 0; p < P; ++p) agg_off[p + 1] = agg_off[p] + cnt[p + 1];
    for (p = 0; p < P; ++p) cnt[p + 1] = agg_off[p];
    for (i = 0; i < M; ++i) {
        uint64_t o;
        if (!owner[i]) continue;
        o = cnt[owner[i]]++;
        agg_idx[o] = (uint32_t)i;
        for (d = 0; d < D; ++d) {
            agg_val[o * Dv + d] = acc[i * Dv + d];
            agg_abs[o * Dv + d] = accabs[i * Dv + d];
        }
    }
done:
    free(acc);
    free(accabs);
    free(owner);
    free(cnt);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* A4: hash-bitmap encode (and decode, used by the pins)                     */
/* ------------------------------------------------------------------------ */

/* Class lists C_p = { idx in [0, M) : h0(idx) = p } in ascending order, as
 * [Zen] section 3.3.2 defines them (computed once, offline, and the same for
 * servers and workers).  Outputs: class_size[P], rank[M] = position of idx
 * inside its class. */
int orc_classmap(uint64_t M, uint32_t P, uint32_t seed, uint64_t* class_size, uint32_t* rank)
{
    uint64_t i;
    if (P == 0 || M > 0xffffffffull) return ORC_EINVAL;
    memset(class_size, 0, P * sizeof(uint64_t));
    for (i = 0; i < M; ++i) {
        uint32_t p = orc_h0((uint32_t)i, seed, P);
        rank[i] = (uint32_t)class_size[p]++;
    }
    return ORC_OK;
}

/* Hash bitmap of [Zen] section 3.3.2 (the Fig. 10 walk-through): server p's
 * bitmap has one bit per member of C_p, set when that member is in the
 * server's aggregated index set.  Readings (the text fixes none of these): bit
 * b lives in 32-bit word b/32 at bit b%32 (least significant first); bit
 * positions are 0-based; each class's bitmap is padded with zero bits to a
 * whole word and the classes are concatenated in order p = 0..P-1, starting at
 * word_off[p] = sum over q < p of ceil(|C_q|/32).  Values need no re-encoding:
 * the aggregate lists a partition's indices in ascending order, which is the
 * order of C_p. */
int orc_encode(const uint32_t* agg_idx, const uint64_t* agg_off, uint32_t P, uint64_t M,
               uint32_t seed, uint32_t* bitmap, uint64_t* word_off)
{
    uint64_t* csize;
    uint32_t* rank;
    uint32_t p;
    uint64_t i;
    int rc;
    if (P == 0 || M > 0xffffffffull) return ORC_EINVAL;
    csize = (uint64_t*)malloc(P * sizeof(uint64_t));
    rank = (uint32_t*)malloc((M ? M : 1) * sizeof(uint32_t));
    if (!csize || !rank) {
        free(csize);
        free(rank);
        return ORC_ENOMEM;
    }
    rc = orc_classmap(M, P, seed, csize, rank);
    if (rc) goto done;
    word_off[0] = 0;
    for (p = 0; p < P; ++p) word_off[p + 1] = word_off[p] + (csize[p] + 31) / 32;
    memset(bitmap, 0, word_off[P] * sizeof(uint32_t));
    for (p = 0; p < P; ++p) {
        for (i = agg_off[p]; i < agg_off[p + 1]; ++i) {
            uint32_t x = agg_idx[i];
            uint64_t b;
            if (x >= M || orc_h0(x, seed, P) != p) {
                rc = ORC_EINCONSISTENT;
                goto done;
            }
            b = rank[x];
            bitmap[word_off[p] + b / 32] |= 1u << (b % 32);
        }
    }
done:
    free(csize);
    free(rank);
    return rc;
}

/* Inverse of orc_encode: bit positions back to global indices through C_p
 * ([Zen] section 3.3.2, hash_bitmap_decode).  out_off[P+1] is filled; out_idx
 * must hold M entries. */
int orc_decode(const uint32_t* bitmap, uint32_t P, uint64_t M, uint32_t seed,
               uint32_t* out_idx, uint64_t* out_off)
{
    uint64_t *csize, *woff, *fill;
    uint32_t** members;
    uint32_t p;
    uint64_t i, o = 0;
    int rc = ORC_OK;
    if (P == 0 || M > 0xffffffffull) return ORC_EINVAL;
    csize = (uint64_t*)calloc(P, sizeof(uint64_t));
    woff = (uint64_t*)calloc(P + 1, sizeof(uint64_t));
    fill = (uint64_t*)calloc(P, sizeof(uint64_t));
    members = (uint32_t**)calloc(P, sizeof(uint32_t*));
    if (!csize || !woff || !fill || !members) {
        rc = ORC_ENOMEM;
        goto done;
    }
    for (i = 0; i < M; ++i) csize[orc_h0((uint32_t)i, seed, P)]++;
    for (p = 0; p < P; ++p) {
        members[p] = (uint32_t*)malloc((csize[p] ? csize[p] : 1) * sizeof(uint32_t));
        if (!members[p]) {
            rc = ORC_ENOMEM;
            goto done;
        }
        woff[p + 1] = woff[p] + (csize[p] + 31) / 32;
    }
    for (i = 0; i < M; ++i) {
        p = orc_h0((uint32_t)i, seed, P);
        members[p][fill[p]++] = (uint32_t)i;
    }
    for (p = 0; p < P; ++p) {
        uint64_t b;
        out_off[p] = o;
        for (b = 0; b < csize[p]; ++b)
            if (bitmap[woff[p] + b / 32] & (1u << (b % 32))) out_idx[o++] = members[p][b];
    }
    out_off[P] = o;
done:
    if (members)
        for (p = 0; p < P; ++p) free(members[p]);
    free(members);
    free(csize);
    free(woff);
    free(fill);
    return rc;
}

/* Pull-side scatter ([Zen] section 3.1: after Pull every worker holds the
 * aggregated gradient; section 3.3.2: the decoded indices select where the
 * received values go).  The dense [M][D] tensor is zero except at the
 * aggregated indices, which receive their aggregated values, copied as they
 * are.  Entries [off[0], off[P]) of idx/val are scattered. */
int orc_scatter_dense(const uint32_t* idx, const float* val, uint32_t D, const uint64_t* off, uint32_t P,
                      uint64_t M, float* dense)
{
    uint64_t i, c;
    if (P == 0) return ORC_EINVAL;
    memset(dense, 0, M * (D ? D : 1) * sizeof(float));
    for (i = off[0]; i < off[P]; ++i) {
        if (idx[i] >= M) return ORC_EINCONSISTENT;
        for (c = 0; c < D; ++c) dense[(uint64_t)idx[i] * D + c] = val[i * D + c];
    }
    return ORC_OK;
}

/* Encoded size of an aggregate under the sparse formats of [Zen] section
 * 3.3.1 and the hash bitmap of section 3.3.2, in bytes, with 4-byte indices
 * and D fp32 values per index:
 *   dense        M * 4D
 *   coo          |I| * (4 + 4D)
 *   block        tensor blocks of 256 gradients (OmniReduce): every block of
 *                [0, M) holding an aggregated index sends its 256 * D values
 *                and a 4-byte block id
 *   bitmap       each of the P servers owns the contiguous range
 *                [floor(iM/P), floor((i+1)M/P)) and sends a bitmap of it,
 *                ceil(len_i / 32) words, plus the values
 *   hash_bitmap  server p's bitmap covers its class C_p, ceil(|C_p| / 32)
 *                words, plus the values
 * Reading: the block format is taken over the whole aggregated tensor (what
 * one worker receives in Pull), the last block of [0, M) counting as a full
 * block of 256.  out[0..5] = dense, coo, block, bitmap, hash_bitmap, |I|;
 * out[6] = the number of non-empty blocks. */
int orc_format_sizes(const uint32_t* agg_idx, const uint64_t* agg_off, uint32_t P, uint64_t M, uint32_t D,
                     uint32_t seed, uint64_t* out)
{
    uint64_t i, U, nb, nblocks = 0, bitmap_words = 0, hash_words = 0;
    uint8_t* used;
    uint64_t* csize;
    uint32_t p;
    if (P == 0 || M > 0xffffffffull) return ORC_EINVAL;
    nb = (M + 255) / 256;
    used = (uint8_t*)calloc(nb ? nb : 1, 1);
    csize = (uint64_t*)calloc(P, sizeof(uint64_t));
    if (!used || !csize) {
        free(used);
        free(csize);
        return ORC_ENOMEM;
    }
    U = agg_off[P] - agg_off[0];
    for (i = agg_off[0]; i < agg_off[P]; ++i) {
        if (agg_idx[i] >= M) {
            free(used);
            free(csize);
            return ORC_EINCONSISTENT;
        }
        used[agg_idx[i] / 256] = 1;
    }
    for (i = 0; i < nb; ++i) nblocks += used[i];
    for (p = 0; p < P; ++p) {
        uint64_t lo = (uint64_t)(((unsigned __int128)M * p) / P), hi = (uint64_t)(((unsigned __int128)M * (p + 1)) / P);
        bitmap_words += (hi - lo + 31) / 32;
    }
    for (i = 0; i < M; ++i) csize[orc_h0((uint32_t)i, seed, P)]++;
    for (p = 0; p < P; ++p) hash_words += (csize[p] + 31) / 32;
    out[0] = M * 4ull * D;
    out[1] = U * (4ull + 4ull * D);
    out[2] = nblocks * (256ull * 4ull * D + 4ull);
    out[3] = bitmap_words * 4ull + U * 4ull * D;
    out[4] = hash_words * 4ull + U * 4ull * D;
    out[5] = U;
    out[6] = nblocks;
    free(used);
    free(csize);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* A5: ring reduce-scatter arithmetic with slice skipping                    */
/* ------------------------------------------------------------------------ */

/* Chunk j of the n ring chunks: [floor(jM/n), floor((j+1)M/n)). */
static uint64_t chunk_begin(uint64_t M, uint32_t n, uint32_t j)
{
    return (uint64_t)(((unsigned __int128)M * j) / n);
}

/* Skip decision for contributor t of chunk j, slice q (seeded mode).
 * [Skip] section 4.3 (Random SkipReduce: every rank draws the same random
 * numbers from a seed shared by all ranks).  Reading: one Bernoulli(p) draw per
 * (chunk, ring position t >= 1, slice), taken as the top 24 bits of the
 * SplitMix64 output number (j*(n-1) + t-1)*S + q of the stream seeded by
 * `seed`; the draw skips when those bits fall below floor(p * 2^24). */
static int seeded_skip(uint64_t seed, uint32_t n, uint64_t S, uint32_t j, uint32_t t, uint64_t q,
                       uint32_t thr24)
{
    uint64_t ctr = ((uint64_t)j * (n - 1) + (t - 1)) * S + q;
    uint64_t u = orc_splitmix64_at(seed, ctr) >> 40;
    return u < thr24;
}

/* Threshold of the seeded draw: floor(p * 2^24), clamped to [0, 2^24]. */
uint32_t orc_skip_threshold(double p)
{
    double t;
    if (!(p > 0.0)) return 0;
    if (p >= 1.0) return 1u << 24;
    t = floor(p * 16777216.0);
    return (uint32_t)t;
}

/* Inclusion mask [n chunks][n ring positions][S slices] (1 = included).
 * Seeded mode: position 0 (the chunk's origin rank, which only sends) is
 * always included; positions 1..n-1 are skipped per seeded_skip. */
int orc_skip_mask(uint32_t n, uint64_t S, double p, uint64_t seed, uint8_t* include)
{
    uint32_t j, t;
    uint64_t q;
    uint32_t thr = orc_skip_threshold(p);
    for (j = 0; j < n; ++j)
        for (t = 0; t < n; ++t)
            for (q = 0; q < S; ++q) {
                uint8_t inc = 1;
                if (t > 0 && seeded_skip(seed, n, S, j, t, q, thr)) inc = 0;
                include[((uint64_t)j * n + t) * S + q] = inc;
            }
    return ORC_OK;
}

/* Ring reduce-scatter of n equal-role buffers bufs[n][M] into out[M], with
 * per-slice skipping.  Chunk j starts at rank j and travels j -> j+1 -> ... ;
 * the rank at ring position t = 1..n-1 adds its own slice of chunk j to the
 * partial it received ([Ring] aggregation phase; [Skip] section 4.2 Algorithm
 * 1's ReduceOrSkip, where a skipped rank forwards what it received unchanged,
 * and Algorithm 2, where SkipReduce drops whole ring steps).  Position 0 sends
 * its slice unreduced.  For each slice the included contributions are summed
 * in ring order; c = number included.  Rescale mode 1 multiplies by n/c (the
 * DropReduce divisor change of [Skip] section 4.1 and the DropReduce
 * discussion); mode 0 leaves the sum as is (plain SkipReduce treats a skipped
 * gradient as zero).  c = 0 gives +0.
 * Outputs are double; out_abs[M] holds (scale) * sum |x| of the included
 * terms, for the tolerance; count[n][S] (optional) holds c.
 * include (optional, [n][n][S]) overrides the seeded mask. */
int orc_skip_reduce_scatter(const void* bufs, int dtype, uint32_t n, uint64_t M, uint64_t slice_elems,
                            double p, uint64_t seed, const uint8_t* include, int mode,
                            double* out, double* out_abs, uint8_t* count);

/* Static SkipReduce(k) ([Skip] section 4.2, Algorithm 2): the
 * reduce-scatter loop starts at step k, so the first k ring positions of
 * every chunk (its origin included) never enter the sum: include[j][t][q] is
 * 1 exactly for t >= k. */
int orc_skip_mask_static(uint32_t n, uint64_t S, uint32_t k, uint8_t* include)
{
    uint32_t j, t;
    uint64_t q;
    if (n == 0) return ORC_EINVAL;
    for (j = 0; j < n; ++j)
        for (t = 0; t < n; ++t)
            for (q = 0; q < S; ++q) include[((uint64_t)j * n + t) * S + q] = t >= k;
    return ORC_OK;
}

/* Random SkipReduce ([Skip] section 4.3): Algorithm 2's slice indices are
 * shifted by a random offset that every rank draws alike, once per call.
 * Reading: off = (SplitMix64 output 0 of the stream at `seed`) mod n; the
 * chain of chunk j then starts at rank j - off, so the rank at position t
 * (rank j + t) holds chain position (t + off) mod n, and is kept exactly when
 * that position is at least k. */
int orc_skip_mask_random(uint32_t n, uint64_t S, uint32_t k, uint64_t seed, uint8_t* include)
{
    uint32_t j, t, off;
    uint64_t q;
    if (n == 0) return ORC_EINVAL;
    off = (uint32_t)(orc_splitmix64_at(seed, 0) % n);
    for (j = 0; j < n; ++j)
        for (t = 0; t < n; ++t)
            for (q = 0; q < S; ++q) include[((uint64_t)j * n + t) * S + q] = (t + off) % n >= k;
    return ORC_OK;
}

/* AllReduce_Dropout ([Skip] section 4.2, Algorithm 1, ReduceOrSkip): each
 * element of a received chunk is reduced or skipped on its own.  Reading:
 * element e (its index in [0, M)) at ring position t >= 1 is skipped when the
 * top 24 bits of SplitMix64 output number (t-1)*M + e of the stream at `seed`
 * are below floor(p * 2^24); position 0, the origin's data, is always kept.
 * out[e] = sum of the kept contributions (times n/c for DROP; 0 if c = 0);
 * count[e] = c when count is not NULL. */
int orc_dropout_reduce_scatter(const void* bufs, int dtype, uint32_t n, uint64_t M, double p, uint64_t seed,
                               int mode, double* out, double* out_abs, uint8_t* count)
{
    uint32_t j, t;
    uint64_t e;
    uint32_t thr = orc_skip_threshold(p);
    if (n == 0) return ORC_EINVAL;
    for (j = 0; j < n; ++j) {
        uint64_t cb = chunk_begin(M, n, j), ce = chunk_begin(M, n, j + 1);
        for (e = cb; e < ce; ++e) {
            double acc = 0.0, accabs = 0.0, scale;
            uint32_t c = 0;
            for (t = 0; t < n; ++t) {
                double v;
                if (t > 0 && (uint32_t)(orc_splitmix64_at(seed, (uint64_t)(t - 1) * M + e) >> 40) < thr) continue;
                v = load_val(bufs, dtype, (uint64_t)((j + t) % n) * M + e);
                acc += v;
                accabs += fabs(v);
                ++c;
            }
            scale = (mode == 1 && c > 0) ? (double)n / (double)c : 1.0;
            out[e] = acc * scale;
            out_abs[e] = accabs * scale;
            if (count) count[e] = (uint8_t)c;
        }
    }
    return ORC_OK;
}

/* Selective SkipReduce ([Skip] section 4.4): gradients travel in buckets,
 * each reduced by an AllReduce of its own, so each bucket can have its own
 * skip rate.  Bucket b is [bucket_off[b], bucket_off[b+1]) of every rank's
 * buffer, reduce-scattered as a tensor of its own (its own n chunks and
 * slices) with skip rate p[b] and the seed seed + b. */
int orc_selective_reduce_scatter(const void* bufs, int dtype, uint32_t n, uint64_t M, uint32_t nb,
                                 const uint64_t* bucket_off, const double* p, uint64_t seed, uint64_t slice_elems,
                                 int mode, double* out, double* out_abs)
{
    uint32_t b, r;
    size_t esz = dtype == 1 ? 2 : 4;
    if (n == 0 || slice_elems == 0) return ORC_EINVAL;
    for (b = 0; b < nb; ++b) {
        uint64_t lo = bucket_off[b], hi = bucket_off[b + 1], Mb;
        void* tmp;
        uint8_t* cnt;
        int rc;
        if (hi < lo || hi > M) return ORC_EINVAL;
        Mb = hi - lo;
        if (Mb == 0) continue;
        tmp = malloc((size_t)n * Mb * esz);
        cnt = (uint8_t*)malloc((size_t)n * ((Mb + n - 1) / n / slice_elems + 2));
        if (!tmp || !cnt) {
            free(tmp);
            free(cnt);
            return ORC_ENOMEM;
        }
        for (r = 0; r < n; ++r)
            memcpy((char*)tmp + (size_t)r * Mb * esz, (const char*)bufs + ((size_t)r * M + lo) * esz, Mb * esz);
        rc = orc_skip_reduce_scatter(tmp, dtype, n, Mb, slice_elems, p[b], seed + b, NULL, mode, out + lo,
                                     out_abs + lo, cnt);
        free(tmp);
        free(cnt);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* AllGather phase of the ring ([Ring] broadcast phase; [Skip] Algorithms 1
 * and 2 end with it unchanged): the holder of chunk j (ring position n-1,
 * rank j-1) passes the reduced chunk on, and position u (rank (j+u) mod n,
 * u = 0..n-2) receives it at step u.  ag_include[j][u] (NULL: all) says
 * whether that delivery happens.  Reading of AllGather skipping: a rank whose
 * delivery is skipped keeps its own local values of the chunk, and the chunk
 * still reaches the ranks after it.  out[r][e] for every rank r. */
int orc_allgather(const double* reduced, const void* bufs, int dtype, uint32_t n, uint64_t M,
                  const uint8_t* ag_include, double* out)
{
    uint32_t j, u;
    uint64_t e;
    if (n == 0) return ORC_EINVAL;
    for (j = 0; j < n; ++j) {
        uint64_t cb = chunk_begin(M, n, j), ce = chunk_begin(M, n, j + 1);
        for (u = 0; u < n; ++u) {
            uint32_t r = (j + u) % n;
            int got = u == n - 1 || !ag_include || ag_include[(uint64_t)j * n + u];
            for (e = cb; e < ce; ++e) out[(uint64_t)r * M + e] = got ? reduced[e] : load_val(bufs, dtype, (uint64_t)r * M + e);
        }
    }
    return ORC_OK;
}

int orc_skip_reduce_scatter(const void* bufs, int dtype, uint32_t n, uint64_t M, uint64_t slice_elems,
                            double p, uint64_t seed, const uint8_t* include, int mode,
                            double* out, double* out_abs, uint8_t* count)
{
    uint64_t maxchunk, S, q, e;
    uint32_t j, t;
    uint8_t* mask = NULL;
    const uint8_t* m;
    if (n == 0 || slice_elems == 0) return ORC_EINVAL;
    maxchunk = (M + n - 1) / n;
    S = maxchunk ? (maxchunk + slice_elems - 1) / slice_elems : 0;
    if (!include) {
        mask = (uint8_t*)malloc((size_t)n * n * (S ? S : 1));
        if (!mask) return ORC_ENOMEM;
        orc_skip_mask(n, S, p, seed, mask);
        m = mask;
    } else {
        m = include;
    }
    for (j = 0; j < n; ++j) {
        uint64_t cb = chunk_begin(M, n, j), ce = chunk_begin(M, n, j + 1);
        for (q = 0; q < S; ++q) {
            uint64_t sb = cb + q * slice_elems, se = sb + slice_elems;
            uint32_t c = 0;
            double scale;
            for (t = 0; t < n; ++t) c += m[((uint64_t)j * n + t) * S + q] ? 1 : 0;
            if (count) count[(uint64_t)j * S + q] = (uint8_t)c;
            scale = (mode == 1 && c > 0) ? (double)n / (double)c : 1.0;
            if (se > ce) se = ce;
            for (e = sb; e < se; ++e) {
                double acc = 0.0, accabs = 0.0;
                for (t = 0; t < n; ++t) {
                    uint32_t r = (j + t) % n;
                    double v;
                    if (!m[((uint64_t)j * n + t) * S + q]) continue;
                    v = load_val(bufs, dtype, (uint64_t)r * M + e);
                    acc += v;
                    accabs += fabs(v);
                }
                out[e] = (c > 0) ? acc * scale : 0.0;
                out_abs[e] = (c > 0) ? accabs * scale : 0.0;
            }
        }
    }
    free(mask);
    return ORC_OK;
}

/* The same reduce-scatter replayed step by step with explicit per-rank
 * buffers and the slice indices of [Skip] Algorithms 1-2: at step s every rank
 * r sends its chunk (r - s) mod n to r+1 and the receiver either adds its own
 * copy of chunk (r - s - 1) mod n (ReduceOrSkip with no skip) or keeps the
 * received data (skip).  A contributor excluded at position t = 0 sends zeros
 * (nothing of its own).  Only the test suite uses this, to check that the
 * closed form above is the ring's arithmetic.  Rescaling is not applied here;
 * out[M] receives the raw sums, in double. */
int orc_ring_replay(const void* bufs, int dtype, uint32_t n, uint64_t M, uint64_t slice_elems,
                    const uint8_t* include, double* out)
{
    double* x; /* x[r][e]: rank r's working copy */
    uint64_t maxchunk, S, e;
    uint32_t r, s;
    if (n == 0 || slice_elems == 0) return ORC_EINVAL;
    maxchunk = (M + n - 1) / n;
    S = maxchunk ? (maxchunk + slice_elems - 1) / slice_elems : 0;
    x = (double*)malloc((size_t)n * (M ? M : 1) * sizeof(double));
    if (!x) return ORC_ENOMEM;
    for (r = 0; r < n; ++r)
        for (e = 0; e < M; ++e) x[(uint64_t)r * M + e] = load_val(bufs, dtype, (uint64_t)r * M + e);
    /* Position 0 of chunk j is rank j: if excluded it contributes nothing. */
    for (r = 0; r < n; ++r) {
        uint64_t cb = chunk_begin(M, n, r), ce = chunk_begin(M, n, r + 1);
        for (e = cb; e < ce; ++e) {
            uint64_t q = (e - cb) / slice_elems;
            if (!include[((uint64_t)r * n + 0) * S + q]) x[(uint64_t)r * M + e] = 0.0;
        }
    }
    for (s = 0; s + 1 < n; ++s) {
        /* messages of this step, taken before any receiver updates */
        double* msg = (double*)malloc((size_t)n * (maxchunk ? maxchunk : 1) * sizeof(double));
        if (!msg) {
            free(x);
            return ORC_ENOMEM;
        }
        for (r = 0; r < n; ++r) {
            uint32_t cs = (uint32_t)((r + n - (s % n)) % n); /* chunk sent by r */
            uint64_t cb = chunk_begin(M, n, cs), ce = chunk_begin(M, n, cs + 1);
            for (e = cb; e < ce; ++e) msg[(uint64_t)r * maxchunk + (e - cb)] = x[(uint64_t)r * M + e];
        }
        for (r = 0; r < n; ++r) {
            uint32_t from = (r + n - 1) % n;
            uint32_t cr = (uint32_t)((r + 2 * n - s - 1) % n); /* chunk received by r */
            uint32_t t = (r + n - cr) % n;                     /* r's ring position for chunk cr */
            uint64_t cb = chunk_begin(M, n, cr), ce = chunk_begin(M, n, cr + 1);
            for (e = cb; e < ce; ++e) {
                uint64_t q = (e - cb) / slice_elems;
                double y = msg[(uint64_t)from * maxchunk + (e - cb)];
                if (include[((uint64_t)cr * n + t) * S + q])
                    x[(uint64_t)r * M + e] = x[(uint64_t)r * M + e] + y;
                else
                    x[(uint64_t)r * M + e] = y;
            }
        }
        free(msg);
    }
    /* chunk j ends on rank (j - 1) mod n */
    for (r = 0; r < n; ++r) {
        uint32_t j = (r + 1) % n;
        uint64_t cb = chunk_begin(M, n, j), ce = chunk_begin(M, n, j + 1);
        for (e = cb; e < ce; ++e) out[e] = x[(uint64_t)r * M + e];
    }
    free(x);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* A6: sparsity statistics                                                   */
/* ------------------------------------------------------------------------ */

/* Output record of orc_stats; arrays are caller-owned. */
typedef struct {
    uint64_t union_size, sum_nnz, max_nnz;
    uint64_t* nnz;           /* [n] */
    uint64_t* inter;         /* [n*n]  |I_a intersect I_b| */
    double* overlap;         /* [n*n]  Def. 3 */
    double overlap_mean, overlap_min, overlap_max; /* over pairs a < b */
    double gamma_n;          /* Def. 4 */
    uint64_t* contig_counts; /* [(n+1)*P] worker w (row w) and the union (row n) per contiguous part */
    double* skew_contig;     /* [n+1] Def. 5 on contiguous parts */
    uint64_t* class_size;    /* [P] |C_i| (hashed parts), filled when hashed != 0 */
    uint64_t* hashed_counts; /* [(n+1)*P] per hash class */
    double* skew_hashed;     /* [n+1] Def. 5 evaluated on the hash classes */
    double push_imbalance, pull_imbalance; /* Def. 8 with f = h0 */
} orc_stats_out;

/* Def. 5 on one set J: max over parts i of (c_i * M) / (g_i * |J|); 0 if J is
 * empty; parts with g_i = 0 are skipped. */
static double skew_of(const uint64_t* c, const uint64_t* g, uint32_t P, uint64_t M, uint64_t J)
{
    double best = 0.0;
    uint32_t i;
    if (J == 0) return 0.0;
    for (i = 0; i < P; ++i) {
        double s;
        if (g[i] == 0) continue;
        s = ((double)c[i] * (double)M) / ((double)g[i] * (double)J);
        if (s > best) best = s;
    }
    return best;
}

/* Sparsity statistics of n workers' index sets (each strictly ascending).
 * Def. 3 (overlap ratio), Def. 4 (densification ratio), Def. 5 (n-partition
 * skew ratio) of [Zen] section 2.1, and Def. 8 (push and pull imbalance) of
 * [Zen] section 3.1.  Readings: for n > 2 the overlap ratio is reported for
 * every pair (Fig. 2a plots a distribution over pairs); gamma_n uses the
 * workers' mean density as d_G (gamma = n |I| / sum |I_w|); skew uses P
 * contiguous parts [floor(iM/P), floor((i+1)M/P)); "skew after hashing" is
 * Def. 5 evaluated on the hash classes C_i; an empty set gives 0. */
int orc_stats(const uint32_t* idx, const uint64_t* in_off, uint32_t n, uint64_t M, uint32_t P,
              int hashed, uint32_t seed, orc_stats_out* o)
{
    uint32_t a, b, i;
    uint8_t* seen = NULL;
    uint64_t* g = NULL;
    uint64_t e, npairs = 0;
    double sum_ov = 0.0;
    if (P == 0 || M > 0xffffffffull) return ORC_EINVAL;
    seen = (uint8_t*)calloc(M ? M : 1, 1);
    g = (uint64_t*)calloc(P, sizeof(uint64_t));
    if (!seen || !g) {
        free(seen);
        free(g);
        return ORC_ENOMEM;
    }
    o->sum_nnz = 0;
    o->max_nnz = 0;
    for (a = 0; a < n; ++a) {
        o->nnz[a] = in_off[a + 1] - in_off[a];
        o->sum_nnz += o->nnz[a];
        if (o->nnz[a] > o->max_nnz) o->max_nnz = o->nnz[a];
    }
    /* union */
    o->union_size = 0;
    for (a = 0; a < n; ++a)
        for (e = in_off[a]; e < in_off[a + 1]; ++e)
            if (idx[e] < M && !seen[idx[e]]) {
                seen[idx[e]] = 1;
                o->union_size++;
            }
    /* pairwise intersections by merging the two sorted lists */
    for (a = 0; a < n; ++a)
        for (b = 0; b < n; ++b) {
            uint64_t x = in_off[a], y = in_off[b], c = 0;
            while (x < in_off[a + 1] && y < in_off[b + 1]) {
                if (idx[x] < idx[y]) ++x;
                else if (idx[x] > idx[y]) ++y;
                else {
                    ++c;
                    ++x;
                    ++y;
                }
            }
            o->inter[(uint64_t)a * n + b] = c;
        }
    o->overlap_min = 0.0;
    o->overlap_max = 0.0;
    for (a = 0; a < n; ++a)
        for (b = 0; b < n; ++b) {
            uint64_t mn = o->nnz[a] < o->nnz[b] ? o->nnz[a] : o->nnz[b];
            double ov = mn ? (double)o->inter[(uint64_t)a * n + b] / (double)mn : 0.0;
            o->overlap[(uint64_t)a * n + b] = ov;
            if (a < b) {
                if (npairs == 0 || ov < o->overlap_min) o->overlap_min = ov;
                if (npairs == 0 || ov > o->overlap_max) o->overlap_max = ov;
                sum_ov += ov;
                ++npairs;
            }
        }
    o->overlap_mean = npairs ? sum_ov / (double)npairs : 0.0;
    o->gamma_n = o->sum_nnz ? ((double)n * (double)o->union_size) / (double)o->sum_nnz : 0.0;
    /* contiguous parts */
    memset(o->contig_counts, 0, (size_t)(n + 1) * P * sizeof(uint64_t));
    for (a = 0; a < n; ++a)
        for (e = in_off[a]; e < in_off[a + 1]; ++e) {
            uint32_t part = (uint32_t)(((unsigned __int128)idx[e] * P) / (M ? M : 1));
            /* idx in [floor(iM/P), floor((i+1)M/P)) <=> part i; correct the
             * integer estimate against the exact boundaries */
            while (part + 1 < P && idx[e] >= chunk_begin(M, P, part + 1)) ++part;
            while (part > 0 && idx[e] < chunk_begin(M, P, part)) --part;
            o->contig_counts[(uint64_t)a * P + part]++;
        }
    for (e = 0; e < M; ++e) {
        uint32_t part;
        if (!seen[e]) continue;
        part = (uint32_t)(((unsigned __int128)e * P) / (M ? M : 1));
        while (part + 1 < P && e >= chunk_begin(M, P, part + 1)) ++part;
        while (part > 0 && e < chunk_begin(M, P, part)) --part;
        o->contig_counts[(uint64_t)n * P + part]++;
    }
    for (i = 0; i < P; ++i) g[i] = chunk_begin(M, P, i + 1) - chunk_begin(M, P, i);
    for (a = 0; a < n; ++a) o->skew_contig[a] = skew_of(o->contig_counts + (uint64_t)a * P, g, P, M, o->nnz[a]);
    o->skew_contig[n] = skew_of(o->contig_counts + (uint64_t)n * P, g, P, M, o->union_size);
    /* hash classes */
    o->push_imbalance = 0.0;
    o->pull_imbalance = 0.0;
    if (hashed) {
        memset(o->class_size, 0, P * sizeof(uint64_t));
        memset(o->hashed_counts, 0, (size_t)(n + 1) * P * sizeof(uint64_t));
        for (e = 0; e < M; ++e) o->class_size[orc_h0((uint32_t)e, seed, P)]++;
        for (a = 0; a < n; ++a)
            for (e = in_off[a]; e < in_off[a + 1]; ++e)
                o->hashed_counts[(uint64_t)a * P + orc_h0(idx[e], seed, P)]++;
        for (e = 0; e < M; ++e)
            if (seen[e]) o->hashed_counts[(uint64_t)n * P + orc_h0((uint32_t)e, seed, P)]++;
        for (a = 0; a < n; ++a)
            o->skew_hashed[a] = skew_of(o->hashed_counts + (uint64_t)a * P, o->class_size, P, M, o->nnz[a]);
        o->skew_hashed[n] = skew_of(o->hashed_counts + (uint64_t)n * P, o->class_size, P, M, o->union_size);
        /* Def. 8: push = max over (w, j) of P |I_w^j| / |I_w|; pull = max
         * over j of P |I'_j| / |I| */
        for (a = 0; a < n; ++a) {
            if (o->nnz[a] == 0) continue;
            for (i = 0; i < P; ++i) {
                double v = ((double)P * (double)o->hashed_counts[(uint64_t)a * P + i]) / (double)o->nnz[a];
                if (v > o->push_imbalance) o->push_imbalance = v;
            }
        }
        if (o->union_size)
            for (i = 0; i < P; ++i) {
                double v = ((double)P * (double)o->hashed_counts[(uint64_t)n * P + i]) / (double)o->union_size;
                if (v > o->pull_imbalance) o->pull_imbalance = v;
            }
    }
    free(seen);
    free(g);
    return ORC_OK;
}

/*
 * sg_gen.c -- seeded synthetic inputs for the sparse gradient
 * synchronization workloads.  Input generation only: nothing here computes any
 * step of the method.  Both the oracle and the HIP library are fed from these
 * arrays; neither side calls into this file.
 *
 * Random numbers: counter-based SplitMix64 (Steele, Lea, Flood, OOPSLA 2014).
 * Value number c (0-based) of a stream with seed s is mix(s + (c+1) * gamma),
 * so every element can be produced independently and the output does not
 * depend on the thread count.  A stream's seed is (workload id << 32) | stream.
 *
 * Distributions:
 *   uniform [0,1)   top 53 bits of one draw times 2^-53
 *   normal N(0,1)   Box-Muller on draws 2c and 2c+1: sqrt(-2 ln(1-u1)) cos(2 pi u2),
 *                   formed in double, rounded once to float
 *   Zipf(s) on [1,R] inverse CDF over a double table of r^-s; index = r - 1
 *   "distinct"      successive sampling: redraw until the value is new, then sort
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <omp.h>

#define GAMMA 0x9e3779b97f4a7c15ull

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint64_t c) { return mix64(seed + (c + 1) * GAMMA); }

static inline double unif(uint64_t seed, uint64_t c) { return (double)(draw(seed, c) >> 11) * (1.0 / 9007199254740992.0); }

static inline double normal(uint64_t seed, uint64_t c)
{
    double u1 = unif(seed, 2 * c), u2 = unif(seed, 2 * c + 1);
    return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586476925 * u2);
}

/* out[i] = sigma * N(0,1) for counters first .. first+count-1 */
void gen_normal_f32(uint64_t seed, uint64_t first, uint64_t count, double sigma, float* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (int64_t)count; ++i) out[i] = (float)(sigma * normal(seed, first + (uint64_t)i));
}

/* Same, but a value that rounds to zero is replaced by +2^-20 so every
 * listed nonzero really is nonzero. */
void gen_normal_nonzero_f32(uint64_t seed, uint64_t first, uint64_t count, double sigma, float* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (int64_t)count; ++i) {
        float v = (float)(sigma * normal(seed, first + (uint64_t)i));
        if (v == 0.0f) v = 9.5367431640625e-07f;
        out[i] = v;
    }
}

/* count distinct values uniform in [lo, hi), sorted ascending.  Returns 0, or
 * -1 if count exceeds the range or memory runs out. */
int gen_uniform_distinct(uint64_t seed, uint64_t lo, uint64_t hi, uint64_t count, uint32_t* out)
{
    uint64_t range = hi - lo, got = 0, c = 0, i, o = 0;
    uint8_t* bits;
    if (hi < lo || count > range) return -1;
    bits = (uint8_t*)calloc((range + 7) / 8 + 1, 1);
    if (!bits) return -1;
    while (got < count) {
        uint64_t r = (uint64_t)(((unsigned __int128)draw(seed, c++) * range) >> 64);
        if (!(bits[r >> 3] & (1u << (r & 7)))) {
            bits[r >> 3] |= (uint8_t)(1u << (r & 7));
            ++got;
        }
    }
    for (i = 0; i < range; i += 8) {
        uint8_t byte = bits[i >> 3];
        uint64_t j;
        if (!byte) continue;
        for (j = 0; j < 8 && i + j < range; ++j)
            if (byte & (1u << j)) out[o++] = (uint32_t)(lo + i + j);
    }
    free(bits);
    return 0;
}

/* Zipf(s) CDF over ranks 1..R: cdf[r-1] = sum_{j<=r} j^-s / H. */
static double* zipf_cdf(uint64_t R, double s)
{
    double* cdf = (double*)malloc(R * sizeof(double));
    double acc = 0.0;
    uint64_t r;
    if (!cdf) return NULL;
    for (r = 0; r < R; ++r) {
        acc += pow((double)(r + 1), -s);
        cdf[r] = acc;
    }
    for (r = 0; r < R; ++r) cdf[r] /= acc;
    cdf[R - 1] = 1.0;
    return cdf;
}

/* count distinct Zipf(s) ranks over [1, R], returned as 0-based indices
 * (rank - 1) sorted ascending, so the hottest index is 0. */
int gen_zipf_distinct(uint64_t seed, uint64_t R, double s, uint64_t count, uint32_t* out)
{
    double* cdf;
    uint8_t* bits;
    uint64_t got = 0, c = 0, i, o = 0;
    if (count > R || R == 0) return -1;
    cdf = zipf_cdf(R, s);
    bits = (uint8_t*)calloc((R + 7) / 8 + 1, 1);
    if (!cdf || !bits) {
        free(cdf);
        free(bits);
        return -1;
    }
    while (got < count) {
        double u = unif(seed, c++);
        uint64_t lo = 0, hi = R - 1;
        while (lo < hi) { /* first r with cdf[r] > u */
            uint64_t mid = lo + (hi - lo) / 2;
            if (cdf[mid] > u) hi = mid;
            else lo = mid + 1;
        }
        if (!(bits[lo >> 3] & (1u << (lo & 7)))) {
            bits[lo >> 3] |= (uint8_t)(1u << (lo & 7));
            ++got;
        }
    }
    for (i = 0; i < R; i += 8) {
        uint8_t byte = bits[i >> 3];
        uint64_t j;
        if (!byte) continue;
        for (j = 0; j < 8 && i + j < R; ++j)
            if (byte & (1u << j)) out[o++] = (uint32_t)(i + j);
    }
    free(cdf);
    free(bits);
    return 0;
}

/* Dense per-row-scaled correlated gradients, n workers of rows x cols:
 * g_w[r][c] = sigma_r * (sqrt(rho) z0[r][c] + sqrt(1-rho) z_{w+1}[r][c]),
 * sigma_r = exp(N(0,1)) shared by all workers; z0 and z_{w+1} are independent
 * N(0,1) fields (streams seed_base+0 and seed_base+w+1), so two workers'
 * entries have correlation rho.  Row scales use stream seed_base + 1000. */
void gen_rowscaled_dense(uint64_t seed_base, uint32_t n, uint64_t rows, uint64_t cols, double rho, float* out)
{
    const double a = sqrt(rho), b = sqrt(1.0 - rho);
    int64_t r;
#pragma omp parallel for schedule(dynamic, 16)
    for (r = 0; r < (int64_t)rows; ++r) {
        double sig = exp(normal(seed_base + 1000, (uint64_t)r));
        uint64_t c;
        uint32_t w;
        for (c = 0; c < cols; ++c) {
            uint64_t e = (uint64_t)r * cols + c;
            double z0 = normal(seed_base + 0, e);
            for (w = 0; w < n; ++w) {
                double z = normal(seed_base + 1 + w, e);
                out[(uint64_t)w * rows * cols + e] = (float)(sig * (a * z0 + b * z));
            }
        }
    }
}

/* bf16 of a float array, round to nearest even (inputs are finite). */
void gen_f32_to_bf16(const float* in, uint64_t count, uint16_t* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (int64_t)count; ++i) {
        uint32_t u;
        memcpy(&u, &in[i], 4);
        u += 0x7fffu + ((u >> 16) & 1u);
        out[i] = (uint16_t)(u >> 16);
    }
}

int gen_num_threads(void) { return omp_get_max_threads(); }

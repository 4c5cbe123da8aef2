/*
 * sg.h -- C ABI of libsg: the on-device compute of sparsity-driven gradient
 * synchronization on one AMD MI355X (gfx950).
 *
 * The n workers of the method are simulated resident on one GPU: every
 * worker's buffers live in this GPU's HBM and there is no communication.  The
 * library implements the compute a worker or server performs:
 *
 *   sg_topk_to_coo          top-k sparsification of dense gradients into COO
 *   sg_dgc_select           DGC-style top-k: sampled global threshold and
 *                           residual accumulation
 *   sg_hash_partition       data-independent hash partition of COO indices
 *   sg_hierarchical_hash    the same partition by Algorithm 1's slot memory
 *   sg_aggregate            per-partition union-sum of n workers' COO tensors
 *   sg_classmap_build,
 *   sg_encode               hash-bitmap encoding of the aggregate's indices
 *   sg_skip_reduce_scatter  ring reduce-scatter arithmetic with seeded slice
 *                           skipping (SkipReduce / DropReduce)
 *   sg_skip_reduce_k,
 *   sg_selective_reduce_scatter,
 *   sg_dropout_reduce_scatter,
 *   sg_allgather            the rest of the SkipReduce family: static and
 *                           random-offset step skipping, per-bucket rates,
 *                           per-element dropout, and the all-gather phase
 *   sg_stats                overlap, densification and skew ratios
 *   sg_decode,
 *   sg_scatter_dense,
 *   sg_format_sizes         the Pull side: hash bitmap back to indices, the
 *                           aggregate scattered into a dense tensor, and the
 *                           aggregate's size under the sparse formats
 *
 * Sources: "Zen: Empowering Distributed Training with Sparsity-driven Data
 * Synchronization" (OSDI'25) digest page [Zen]; "SkipReduce: (Interconnection)
 * Network Sparsity to Accelerate Distributed Machine Learning" (MICRO'25)
 * digest page [Skip]; CMU 15-442/642 lecture notes on data parallelism, "Ring
 * AllReduce" aggregation phase [Ring].
 *
 * Conventions for every call:
 *   - Pointers named d_* are device memory on the current HIP device, owned by
 *     the caller.  The library never allocates, frees or synchronizes, except
 *     sg_stats and sg_device_error, which return host values and therefore
 *     block on `stream`.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is queued on it in order; sizes that only the device knows (for
 *     example agg_off[P]) are read by the caller after synchronizing.
 *   - Indices are 0-based uint32; dense sizes M must be below 2^32.
 *   - Each worker's COO index list is strictly ascending and every index is
 *     below M (the sets I_i of [Zen] section 3.1).  sg_validate_coo checks
 *     this.  Kernels keep every memory access in bounds whatever the input,
 *     but results on invalid input are unspecified; a violation they notice is
 *     recorded and returned by sg_device_error.
 *   - Return value: SG_OK (0) or a negative sg_status.  Host-checkable
 *     problems (null pointers, sizes, workspace) fail before any launch.
 *   - Workspace: each call that needs scratch memory takes d_ws of at least
 *     the size its *_workspace_bytes function returns for the same arguments.
 *     Its contents on entry do not matter.
 *   - Calls are not re-entrant on one workspace: two calls that overlap in
 *     time must use different workspaces.
 */
#ifndef SG_H
#define SG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sg_status {
    SG_OK = 0,
    SG_EINVAL = -1,       /* bad argument: null pointer, size out of range, unsupported shape */
    SG_ECAPACITY = -2,    /* an output or workspace buffer is smaller than required */
    SG_EUNSORTED = -3,    /* sg_validate_coo: a worker's indices are not strictly ascending */
    SG_EHIP = -4,         /* a HIP launch or copy failed */
    SG_EUNSUPPORTED = -5, /* parameters outside what this build implements (stated per call) */
    SG_ERANGE = -6,       /* sg_validate_coo: an index is >= M, or offsets are inconsistent */
    SG_EDEVICE = -7       /* a kernel noticed a violated precondition (see sg_device_error) */
} sg_status;

typedef enum sg_dtype {
    SG_F32 = 0,  /* IEEE binary32 */
    SG_BF16 = 1  /* bfloat16, accumulated in fp32 */
} sg_dtype;

typedef enum sg_rescale {
    SG_RESCALE_NONE = 0, /* SkipReduce proper: a skipped contribution counts as zero ([Skip] section 4.1) */
    SG_RESCALE_DROP = 1  /* DropReduce: the sum is multiplied by n/c, c = contributions kept ([Skip] section 4.1 and its DropReduce study) */
} sg_rescale;

/* Text for a status code.  Never NULL. */
const char* sg_strerror(int status);

/* Returns SG_OK, or SG_EDEVICE if any kernel of this library recorded a
 * violated precondition on the current device since the last call; clears the
 * record.  Synchronizes `stream`. */
int sg_device_error(void* stream);

/* Measurement hook (process-wide, not thread-safe).  While set, the calls of
 * this library record the HIP events `start_event` and `stop_event`
 * (hipEvent_t passed as void*) on their stream right before and right after
 * launching the kernel named by kernel_id, so a caller can time one kernel
 * inside a multi-kernel call.  kernel_id SG_PROBE_NONE clears the hook. */
typedef enum sg_probe_kernel {
    SG_PROBE_NONE = 0,
    SG_PROBE_TOPK_FILTER = 1,        /* top-k: the streaming pass over the dense data (first pass) */
    SG_PROBE_PARTITION_SCATTER = 2,  /* hash partition: the scatter pass */
    SG_PROBE_AGGREGATE_MERGE = 3,    /* aggregate: the merge pass */
    SG_PROBE_ENCODE = 4,             /* encode: the streaming pass over the key space */
    SG_PROBE_SKIP_RS = 5,            /* skip reduce-scatter: its single kernel */
    SG_PROBE_AGGREGATE_BND = 6,      /* aggregate: the bucket-boundary pass */
    SG_PROBE_PARTITION_HIST = 7,     /* hash partition: the histogram pass */
    SG_PROBE_TOPK_WRITE = 8,         /* top-k: the ordered write */
    SG_PROBE_DECODE = 9,             /* decode: the pass that emits the indices */
    SG_PROBE_SCATTER = 10,           /* scatter to dense: the scatter pass */
    SG_PROBE_DROPOUT_RS = 11,        /* per-element dropout reduce-scatter: its single kernel */
    SG_PROBE_ALLGATHER = 12,         /* all-gather: its single kernel */
    SG_PROBE_DGC_FILTER = 13,        /* DGC select: the streaming pass over gradient and residual */
    SG_PROBE_HHASH_INSERT = 14,      /* hierarchical hash: the insertion into the slot memory */
    SG_PROBE_AGGREGATE_COUNT = 15    /* aggregate: the pass counting each tile's union (scalar values) */
} sg_probe_kernel;
int sg_probe_set(int kernel_id, void* start_event, void* stop_event);

/* Checks that every worker's index list is strictly ascending and below M and
 * that in_off is non-decreasing with in_off[0] = 0 and in_off[n] = total.
 * Returns SG_OK, SG_EUNSORTED or SG_ERANGE.  d_ws: sg_validate_workspace_bytes().
 * Synchronizes `stream`. */
size_t sg_validate_workspace_bytes(void);
int sg_validate_coo(const uint32_t* d_idx, const uint64_t* d_in_off, uint32_t n, uint64_t M, uint64_t total,
                    void* d_ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A1. Top-k sparsification into COO.
 * [Skip] section 2 (top-k keeps the largest-magnitude gradients; unselected
 * ones stay local) and [Zen] section 4 (DGC selects the top 5% per tensor).
 * For each worker w: the k entries of largest |dense[w][i]|, written in
 * ascending index order to idx[w][0..k) with the signed value copied bit for
 * bit to val[w][0..k) (same dtype as the input).  Equal magnitudes (+0 and -0
 * included) are taken lowest index first.  NaN payloads order above +Inf
 * (they are compared as bit patterns); finite inputs are the contract.
 *   d_dense  [n][M] of dt, row-major (worker-major)
 *   d_idx    [n][k] uint32 out;   d_val [n][k] of dt out
 * Limits: 1 <= n, 1 <= M < 2^32, k <= M (else SG_EINVAL); n * ceil(M / 1024)
 * < 2^31 (else SG_EUNSUPPORTED).  k == 0 writes nothing.
 * Workspace (sg_topk_workspace_bytes): sized for the worst case, in which
 * the sampled magnitude band misses the k-th key and every element becomes a
 * candidate: three slot arrays of n*M 32-bit words (about 12 * n * M bytes,
 * 4.03 GiB for n = 8, M = 4096 * 11008) plus per-tile counts; the usual case
 * touches a few percent of it.
 * ------------------------------------------------------------------------ */
size_t sg_topk_workspace_bytes(uint32_t n, uint64_t M, uint64_t k, sg_dtype dt);
int sg_topk_to_coo(const void* d_dense, sg_dtype dt, uint32_t n, uint64_t M, uint64_t k, uint32_t* d_idx,
                   void* d_val, void* d_ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * DGC-style top-k with a sampled global threshold and residuals (one
 * iteration for all n workers).
 * [Zen] section 4 (Implementation): DGC adapted to tensor parallelism --
 * every device samples locally, the samples are gathered, one global top-k
 * threshold is computed from them and applied locally.  [Skip] section 2:
 * unselected gradients accumulate locally into later iterations.
 *   1. a[w][i] = d_resid[w][i] + d_grad[w][i] (one fp32 addition);
 *   2. S samples per worker (S clamped to M) at positions
 *      floor((2j+1) M / (2S)), j < S; their magnitudes are pooled (n*S);
 *   3. threshold = the ks-th largest pooled magnitude,
 *      ks = sg_dgc_rank(density, n*S) = ceil(density * n*S) in double,
 *      clamped to [1, n*S];
 *   4. entries with |a| >= threshold are selected: written in ascending index
 *      order as (i, a) to d_idx[w][*], d_val[w][*] (row stride cap; at most
 *      cap per worker); d_count[w] = the number selected (may exceed cap);
 *   5. d_resid[w][i] becomes 0 where selected, a elsewhere (in place).
 * Magnitudes are compared as fp32 bit patterns without the sign; inputs are
 * finite.  d_thr (optional) receives the threshold's bit pattern.
 *   d_grad, d_resid [n][M] fp32 (d_resid in/out)
 *   d_idx [n][cap] uint32, d_val [n][cap] fp32 out (may be NULL if cap == 0)
 *   d_count [n] uint64 out; d_thr [1] uint32 out or NULL
 * Limits: 1 <= n <= 64, 1 <= M < 2^32, S >= 1, n*S < 2^32, density >= 0.
 * ------------------------------------------------------------------------ */
uint64_t sg_dgc_rank(double density, uint64_t Ns);
size_t sg_dgc_workspace_bytes(uint32_t n, uint64_t M, uint64_t S);
int sg_dgc_select(const float* d_grad, float* d_resid, uint32_t n, uint64_t M, double density, uint64_t S,
                  uint32_t* d_idx, float* d_val, uint64_t cap, uint64_t* d_count, uint32_t* d_thr, void* d_ws,
                  size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A2. Hash partition.
 * [Zen] section 3.1 (Problem 1: one map f from indices to [P] shared by all
 * workers) and section 3.2 (Technique #3 / Algorithm 1: the first-level hash
 * h0 picks the partition).  h0(i) = MurmurHash2-32(4 little-endian bytes of
 * i, seed) mod P.  Each worker's entries are grouped by partition 0..P-1 and
 * kept in input order inside a partition (order inside a partition does not
 * change the aggregate, [Zen] Technique #1; the stable order makes results
 * reproducible and keeps every (worker, partition) run ascending).
 *   d_idx      [total] uint32, worker w's entries at [in_off[w], in_off[w+1])
 *   d_val      [total][D] of dt, or NULL when D == 0 (indices only)
 *   d_in_off   [n+1] uint64, in_off[0] = 0, in_off[n] = total
 *   d_out_idx  [total] out;  d_out_val [total][D] out (NULL when D == 0)
 *   d_part_off [n][P+1] uint64 out, absolute offsets: run (w,p) is
 *              [part_off[w][p], part_off[w][p+1]); part_off[w][P] = in_off[w+1]
 * Limits: 1 <= P <= 256, n >= 1, total < 2^32, D <= 65536.
 * ------------------------------------------------------------------------ */
size_t sg_partition_workspace_bytes(uint32_t n, uint64_t total, uint32_t P);
int sg_hash_partition(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D, const uint64_t* d_in_off,
                      uint32_t n, uint64_t total, uint32_t P, uint32_t seed, uint32_t* d_out_idx, void* d_out_val,
                      uint64_t* d_part_off, void* d_ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the hash
 * partition above with no workspace argument.  Same arguments, results,
 * limits and errors as sg_hash_partition, minus d_ws / ws_bytes.
 * Its scratch (the per-tile partition counts, and for rows the source of
 * every output entry) is a fixed device array of the library,
 * SG_PARTITION_SCRATCH_BYTES (16 MiB) per GPU, held until the process ends;
 * the call itself allocates nothing.  It needs 4 * (n + 1) +
 * 4 * P * (ceil(total / 2048) + n) bytes, plus 4 * total when D >= 2 (each
 * part rounded up to 256 bytes, plus 256); larger inputs return SG_ECAPACITY
 * before any launch (for P = 16 that is over 5 * 10^8 scalar entries, for
 * P = 256 about 3.3 * 10^7; rows with D >= 2 up to about 4 * 10^6).
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (two streams, or two host threads) race and give wrong results; order
 * them on one stream.  The array keeps the last call's contents; a call
 * writes every word it reads before reading it, so nothing is cleared.
 * The stream must belong to the current device (the array is looked up on
 * the current device).
 * ------------------------------------------------------------------------ */
#define SG_PARTITION_SCRATCH_BYTES (16u << 20)
int sg_hash_partition_noalloc(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D,
                              const uint64_t* d_in_off, uint32_t n, uint64_t total, uint32_t P, uint32_t seed,
                              uint32_t* d_out_idx, void* d_out_val, uint64_t* d_part_off, void* stream);

/* ------------------------------------------------------------------------
 * Algorithm 1 of [Zen] section 3.2 (hierarchical hashing), a comparison
 * variant of sg_hash_partition with the same partition membership.
 * Per worker, partition p has a slot memory of r1 parallel and r2 serial
 * slots (Technique #1).  Entry e goes to p = h0(idx) (Technique #3, the same
 * h0 as sg_hash_partition), then tries slots h_i(idx) = MurmurHash2(idx as 4
 * LE bytes, seed + i) mod r1 for i = 1..k (Technique #2), taking one with a
 * compare-and-swap from empty (Technique #4: no write is lost to a concurrent
 * writer); after k occupied slots it takes the next serial slot from the
 * partition's atomic counter (starting at r1), and is lost when the r2 serial
 * slots are used up.  Extraction reads each partition's slots in slot order.
 * Which entry wins a contested slot depends on thread timing, so the order
 * inside a partition (and which entries go serial) is not fixed; the set of
 * entries of each partition is, when nothing is lost.
 *   inputs as sg_hash_partition (d_idx, d_val rows of D values of dt, d_in_off)
 *   d_out_idx, d_out_val out: worker w's partitions from d_in_off[w] on, in
 *             partition order, slot order inside a partition (lost entries
 *             leave the worker's tail unwritten)
 *   d_part_off [n][P+1] out (absolute; [w][P] - [w][0] = entries kept)
 *   d_slot_of [total] out (the slot each written entry came from) or NULL
 *   d_counts [n][2] out: serial writes, lost entries
 * Limits: 1 <= P <= 65536, 1 <= k <= 64, r1 >= 1, r1 + r2 < 2^32,
 * r1 + total < 2^32.
 * ------------------------------------------------------------------------ */
size_t sg_hierarchical_hash_workspace_bytes(uint32_t n, uint32_t P, uint64_t r1, uint64_t r2);
int sg_hierarchical_hash(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D, const uint64_t* d_in_off,
                         uint32_t n, uint64_t total, uint32_t P, uint32_t seed, uint32_t k, uint64_t r1, uint64_t r2,
                         uint32_t* d_out_idx, void* d_out_val, uint64_t* d_part_off, uint32_t* d_slot_of,
                         uint64_t* d_counts, void* d_ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A3. Per-partition union-sum (the server side of Push).
 * [Zen] section 3.1 (server p aggregates the partition-p tensors of all
 * workers) and section 3.2 (the result equals the dense AllReduce).  For each
 * partition p: the union of the n runs (w,p) in ascending index order, each
 * index with its D values summed in fp32 over the workers holding it, in
 * worker order.  Membership: an index sent by any worker is in the aggregate,
 * even if its sum is zero.
 *   inputs as produced by sg_hash_partition (each run strictly ascending,
 *   runs of one partition hold only indices of that partition)
 *   d_agg_idx  [capacity] uint32 out
 *   d_agg_val  [capacity][D] fp32 out (NULL when D == 0)
 *   d_agg_off  [P+1] uint64 out: partition p is [agg_off[p], agg_off[p+1])
 * capacity must be >= total (the worst case, all indices distinct).
 * Limits: 1 <= n <= 64, 1 <= P <= 256, M < 2^32, total < 2^32.
 * ------------------------------------------------------------------------ */
size_t sg_aggregate_workspace_bytes(uint32_t n, uint32_t P, uint64_t M, uint64_t total, uint32_t D);
int sg_aggregate(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D, const uint64_t* d_part_off,
                 uint32_t n, uint32_t P, uint64_t M, uint64_t total, uint32_t* d_agg_idx, float* d_agg_val,
                 uint64_t capacity, uint64_t* d_agg_off, void* d_ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A4. Hash-bitmap encode.
 * [Zen] section 3.3.2 (hash bitmap, Fig. 10): the index set of server p is
 * the class C_p = { i in [0,M) : h0(i) = p } in ascending order, fixed offline;
 * the server's bitmap has bit b set iff C_p[b] is in its aggregate.  Layout:
 * bit b of class p is bit (b % 32) of word word_off[p] + b/32; classes are
 * concatenated p = 0..P-1, each padded with zero bits to whole words, so
 * word_off[p] = sum_{q<p} ceil(|C_q| / 32) and the total is about M/32 words.
 * Values need no re-encoding: the aggregate is already in C_p order.
 *
 * sg_classmap_build fills an opaque class map (setup, done once per (M, P,
 * seed), like the offline computation of the page).  sg_encode reads it;
 * cmap_bytes is the size of the caller's class-map buffer.
 *   d_agg_idx, d_agg_off  as produced by sg_aggregate (indices of partition p
 *                         ascending and with h0 = p); agg_capacity is the
 *                         number of entries d_agg_idx holds (offsets beyond it
 *                         are clamped)
 *   d_bitmap   [bitmap_words] uint32 out, bitmap_words >= sg_encode_max_words(M, P)
 *   d_word_off [P+1] uint64 out
 *   d_ws       sg_encode_workspace_bytes(M, P) bytes: per key window of the
 *              class map and partition, where the partition's aggregated
 *              entries of that window begin; for 2 <= P <= 16 over a large
 *              key space also two words per (group of windows, class): the
 *              group's bits in bitmap words it shares with its neighbours,
 *              merged by a second kernel (no global atomics)
 * Limits: 1 <= P <= 256, 1 <= M < 2^32.
 * ------------------------------------------------------------------------ */
size_t sg_classmap_bytes(uint64_t M, uint32_t P);
int sg_classmap_build(uint64_t M, uint32_t P, uint32_t seed, void* d_cmap, size_t cmap_bytes, void* stream);
uint64_t sg_encode_max_words(uint64_t M, uint32_t P);
size_t sg_encode_workspace_bytes(uint64_t M, uint32_t P);
int sg_encode(const uint32_t* d_agg_idx, const uint64_t* d_agg_off, uint64_t agg_capacity, uint64_t M, uint32_t P,
              const void* d_cmap, size_t cmap_bytes, uint32_t* d_bitmap, uint64_t bitmap_words, uint64_t* d_word_off, void* d_ws,
              size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Pull side of A4 (after the aggregate and its encoding).
 * [Zen] section 3.3.2 (hash_bitmap_decode: the set bits of server p's bitmap
 * are ranks in C_p, and C_p[rank] is the global index); section 3.1 (after
 * Pull every worker holds the aggregate); section 3.3.1 (the sparse formats
 * the hash bitmap is compared with).
 *
 * sg_decode: bitmap and layout as written by sg_encode for the same (M, P,
 * class map).  Outputs, per class p in order, the indices C_p[b] of the set
 * bits b in ascending order:
 *   d_out_idx  [capacity] uint32 out (capacity >= the number of set bits;
 *              the aggregate's size is enough; extra indices are dropped)
 *   d_out_off  [P+1] uint64 out: class p is [out_off[p], out_off[p+1])
 *   d_ws       sg_decode_workspace_bytes(M, P) bytes
 * Limits: 1 <= P <= 256, 1 <= M < 2^32.
 *
 * sg_scatter_dense: d_dense [M][D] fp32 out (16-byte aligned) becomes zero
 * except at the entries [off[0], off[P]) of (d_idx, d_val [][D]), whose
 * values are copied to their index (for an aggregate: off = agg_off).
 * capacity is the number of entries d_idx holds (offsets are clamped to it).
 * D == 0 only zeroes.  Indices must be distinct and below M (an index >= M is
 * skipped and recorded for sg_device_error).  Entries in ascending key order
 * within each partition [off[p], off[p+1]) (as sg_aggregate writes them) take
 * the fast path for D == 1: every dense element written once by 16-byte
 * stores; other orders give the same result through a per-entry pass.
 *   d_ws  sg_scatter_dense_workspace_bytes(M, P) bytes: a flag word per
 *         block of the cursor pass, and per (key window of 4096, partition)
 *         the partition's first entry in the window
 * Limits: 1 <= P <= 256, 1 <= M < 2^32, D <= 65536.
 *
 * sg_format_sizes: bytes of an aggregate (d_agg_idx, d_agg_off as produced
 * by sg_aggregate) with D fp32 values per index and 4-byte indices, written
 * to h_out[7] (host):
 *   [0] dense        M * 4D
 *   [1] coo          |I| * (4 + 4D)
 *   [2] block        256-gradient tensor blocks over [0, M) holding an
 *                    aggregated index, each 256 * 4D + a 4-byte block id
 *   [3] bitmap       P contiguous ranges [floor(iM/P), floor((i+1)M/P)),
 *                    ceil(len/32) words each, plus the values
 *   [4] hash_bitmap  sum over classes of ceil(|C_p|/32) words, plus the values
 *   [5] |I|, [6] the number of non-empty blocks
 * Blocks on `stream`.  d_ws: sg_format_sizes_workspace_bytes(M).
 * ------------------------------------------------------------------------ */
size_t sg_decode_workspace_bytes(uint64_t M, uint32_t P);
int sg_decode(const uint32_t* d_bitmap, uint64_t bitmap_words, const void* d_cmap, size_t cmap_bytes, uint64_t M,
              uint32_t P, uint32_t* d_out_idx, uint64_t capacity, uint64_t* d_out_off, void* d_ws, size_t ws_bytes,
              void* stream);
size_t sg_scatter_dense_workspace_bytes(uint64_t M, uint32_t P);
int sg_scatter_dense(const uint32_t* d_idx, const float* d_val, uint32_t D, const uint64_t* d_off, uint32_t P,
                     uint64_t capacity, uint64_t M, float* d_dense, void* d_ws, size_t ws_bytes, void* stream);
size_t sg_format_sizes_workspace_bytes(uint64_t M);
int sg_format_sizes(const uint32_t* d_agg_idx, const uint64_t* d_agg_off, uint64_t capacity, uint64_t M, uint32_t P,
                    uint32_t D, const void* d_cmap, size_t cmap_bytes, uint64_t* h_out, void* d_ws, size_t ws_bytes,
                    void* stream);

/* ------------------------------------------------------------------------
 * A5. Ring reduce-scatter arithmetic with slice skipping.
 * [Ring] aggregation phase (n-1 steps; chunk j starts at rank j, each rank
 * adds its own copy and forwards; rank (j-1) mod n ends with the full chunk);
 * [Skip] section 4.2 Algorithms 1-2 (ReduceOrSkip: a skipping rank forwards
 * what it received without adding; SkipReduce drops whole ring steps),
 * section 4.3 (Random SkipReduce: ranks draw identical random numbers from a
 * shared seed), section 4.1 (skip vs drop).
 * Chunk j = [floor(jM/n), floor((j+1)M/n)), cut into slices of slice_bytes
 * (slice q of chunk j starts q*slice_elems after the chunk start; the last one
 * may be short).  S = ceil(ceil(M/n) / slice_elems) slices per chunk.  Ring
 * position t = 0..n-1 of chunk j is rank (j+t) mod n.
 * Seeded mode (d_include == NULL): position 0 is always kept; position t >= 1
 * of (j, q) is skipped iff the top 24 bits of SplitMix64 output number
 * (j*(n-1) + t-1)*S + q of the stream started at `seed` are below
 * floor(p_skip * 2^24).
 * Explicit mode: d_include [n][n][S] uint8 (nonzero = kept) for (j, t, q).
 * Kept contributions are summed in fp32 in ring order t = 0, 1, ...; c = the
 * number kept; SG_RESCALE_DROP multiplies by fp32(n)/fp32(c); c == 0 gives +0.
 * Skipped slices are never read.
 *   d_bufs  [n][M] of dt (bf16 is widened to fp32 before adding)
 *   d_out   [M] fp32 out: chunk j in place at its own offsets
 *   d_count [n][S] uint8 out (c per (j, q)), or NULL
 * Limits: 1 <= n <= 64, 1 <= M < 2^40, slice_bytes a positive multiple of the
 * element size, 0 <= p_skip <= 1.
 * ------------------------------------------------------------------------ */
uint64_t sg_skip_num_slices(uint32_t n, uint64_t M, uint64_t slice_bytes, sg_dtype dt);
int sg_skip_reduce_scatter(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, uint64_t slice_bytes,
                           double p_skip, uint64_t seed, const uint8_t* d_include, sg_rescale mode, float* d_out,
                           uint8_t* d_count, void* stream);

/* ------------------------------------------------------------------------
 * The rest of the SkipReduce family, on the same ring arithmetic as
 * sg_skip_reduce_scatter (same chunks, slices, ring order, fp32 sums, rescale
 * modes and limits unless stated).
 *
 * sg_skip_reduce_k: SkipReduce(k) of [Skip] section 4.2, Algorithm 2: the
 * reduce-scatter loop starts at step k, so the first k positions of each
 * chunk's chain contribute nothing.  With random_offset == 0 (static
 * SkipReduce) position t of chunk j is kept iff t >= k.  With random_offset
 * != 0 (Random SkipReduce, [Skip] section 4.3: the slice indices are shifted
 * by one random offset shared by every rank) the chain is rotated by
 * off = sg_skip_random_offset(n, seed) = (SplitMix64 output 0 of `seed`) mod n
 * and position t is kept iff (t + off) mod n >= k.  Every slice then has
 * c = n - k; k == n gives +0 everywhere.  d_count as in sg_skip_reduce_scatter.
 * Limits: 0 <= k <= n.
 *
 * sg_selective_reduce_scatter: Selective SkipReduce ([Skip] section 4.4):
 * buckets of gradients with a skip rate each.  Bucket b covers elements
 * [h_bucket_off[b], h_bucket_off[b+1]) of every rank's buffer (host array of
 * nb+1 non-decreasing offsets <= M; elements outside every bucket are left
 * untouched in d_out) and is reduce-scattered as a tensor of its own (its own
 * n chunks and slices) in seeded mode with rate h_p_skip[b] and seed seed + b.
 * One launch per non-empty bucket.
 *
 * sg_dropout_reduce_scatter: AllReduce_Dropout ([Skip] section 4.2,
 * Algorithm 1, ReduceOrSkip per element).  Element e of chunk j at ring
 * position t >= 1 is skipped iff the top 24 bits of SplitMix64 output number
 * (t-1)*M + e of the stream at `seed` are below floor(p_skip * 2^24);
 * position 0 is always kept.  Sums, c and the rescale are per element.
 *   d_count [M] uint8 out (c per element), or NULL.
 *
 * sg_allgather: the all-gather phase that follows the reduce-scatter ([Ring]
 * broadcast phase; [Skip] Algorithms 1-2 end with it).  Rank (j-1) mod n holds
 * reduced chunk j; ring position u = 0..n-2 of chunk j (rank (j+u) mod n)
 * receives it.  d_ag_include [n][n] uint8 (chunk j, position u; NULL = every
 * delivery happens) skips deliveries: a rank whose delivery is skipped keeps
 * its own values of the chunk from d_bufs; position n-1 always has it.
 *   d_reduced [M] fp32 (for example the output of a reduce-scatter call)
 *   d_bufs    [n][M] of dt (read only for skipped deliveries; may be NULL
 *             when d_ag_include is NULL)
 *   d_out     [n][M] fp32 out: every rank's tensor after the phase
 * ------------------------------------------------------------------------ */
uint32_t sg_skip_random_offset(uint32_t n, uint64_t seed);
int sg_skip_reduce_k(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, uint64_t slice_bytes, uint32_t k,
                     int random_offset, uint64_t seed, sg_rescale mode, float* d_out, uint8_t* d_count, void* stream);
int sg_selective_reduce_scatter(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, uint32_t nb,
                                const uint64_t* h_bucket_off, const double* h_p_skip, uint64_t slice_bytes,
                                uint64_t seed, sg_rescale mode, float* d_out, void* stream);
int sg_dropout_reduce_scatter(const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M, double p_skip, uint64_t seed,
                              sg_rescale mode, float* d_out, uint8_t* d_count, void* stream);
int sg_allgather(const float* d_reduced, const void* d_bufs, sg_dtype dt, uint32_t n, uint64_t M,
                 const uint8_t* d_ag_include, float* d_out, void* stream);

/* ------------------------------------------------------------------------
 * A6. Sparsity statistics.
 * [Zen] section 2.1: Def. 3 overlap ratio |I_a & I_b| / min(|I_a|, |I_b|);
 * Def. 4 densification ratio gamma_n = d_n / d_G; Def. 5 n-partition skew
 * ratio max_i d_{G_i} / d_G; section 3.1 Def. 8 push and pull imbalance.
 * Readings: overlap is reported for every pair; gamma_n = n |I| / sum |I_w|
 * (d_G = the workers' mean density); skew uses P contiguous parts
 * G_i = [floor(iM/P), floor((i+1)M/P)) and, with a class map, the hash classes
 * C_i (skew "after hashing"); push/pull imbalance use f = h0 with P servers.
 * Every value is computed from exact counts with these double expressions:
 *   overlap[a][b] = (double)inter / (double)min(nnz_a, nnz_b), 0 if the min is 0
 *   overlap_mean  = (sum over a<b in lexicographic order) / (double)npairs
 *   gamma_n       = ((double)n * (double)|I|) / (double)sum_nnz, 0 if sum is 0
 *   skew(J)       = max_i ((double)c_i * (double)M) / ((double)g_i * (double)|J|)
 *   push          = max_{w,i} ((double)P * (double)|I_w^i|) / (double)nnz_w
 *   pull          = max_i ((double)P * (double)|I'_i|) / (double)|I|
 * Inputs: n workers' COO index lists (d_idx, d_in_off as in sg_hash_partition).
 * d_cmap: a class map for (M, P) from sg_classmap_build, or NULL (then the
 * hashed fields are left untouched).  Blocks on `stream`.
 * Limits: 1 <= n <= 64, 1 <= P <= 256, total < 2^32.
 * ------------------------------------------------------------------------ */
typedef struct sg_stats_out {
    uint64_t union_size, sum_nnz, max_nnz;
    uint64_t* nnz;           /* [n]        caller-provided host array */
    uint64_t* inter;         /* [n*n]      |I_a & I_b| */
    double* overlap;         /* [n*n] */
    double overlap_mean, overlap_min, overlap_max; /* over pairs a < b */
    double gamma_n;
    uint64_t* contig_counts; /* [(n+1)*P]  row w: worker w, row n: the union */
    double* skew_contig;     /* [n+1] */
    uint64_t* class_size;    /* [P]        |C_i| (with a class map) */
    uint64_t* hashed_counts; /* [(n+1)*P] */
    double* skew_hashed;     /* [n+1] */
    double push_imbalance, pull_imbalance;
} sg_stats_out;

/* Workspace of sg_stats / sg_stats_async for these sizes.  With n <= 16,
 * P <= 16 and n * ceil(M/32) <= 16 * total it holds one bitmap of the key
 * space per worker (n * ceil(M/32) * 4 bytes) for the dense counting pass. */
size_t sg_stats_workspace_bytes(uint32_t n, uint64_t M, uint64_t total, uint32_t P);
int sg_stats(const uint32_t* d_idx, const uint64_t* d_in_off, uint32_t n, uint64_t M, uint64_t total, uint32_t P,
             const void* d_cmap, size_t cmap_bytes, sg_stats_out* h_out, void* d_ws, size_t ws_bytes, void* stream);

/* The same statistics in two halves, so a caller can queue more work before
 * it waits.  sg_stats_async validates like sg_stats, queues the passes on
 * `stream` and a copy of the raw counts into h_block (host memory of at
 * least sg_stats_block_bytes(n, P) bytes, owned by the caller; pinned memory
 * keeps the copy asynchronous) and returns without waiting.  Once the stream
 * has passed that point (an event or a synchronize of the caller's),
 * sg_stats_collect evaluates the definitions above from h_block into h_out;
 * n, M, total and P are those of the sg_stats_async call and hashed is 1 iff
 * it had a class map (a block whose class map header does not match (M, P)
 * gives SG_EINVAL).  The workspace and h_block must not be reused before
 * that point.  sg_stats_block_bytes returns 0 for n or P out of range. */
size_t sg_stats_block_bytes(uint32_t n, uint32_t P);
int sg_stats_async(const uint32_t* d_idx, const uint64_t* d_in_off, uint32_t n, uint64_t M, uint64_t total,
                   uint32_t P, const void* d_cmap, size_t cmap_bytes, void* h_block, size_t block_bytes, void* d_ws,
                   size_t ws_bytes, void* stream);
int sg_stats_collect(const void* h_block, uint32_t n, uint64_t M, uint64_t total, uint32_t P, int hashed,
                     sg_stats_out* h_out);

#ifdef __cplusplus
}
#endif
#endif /* SG_H */

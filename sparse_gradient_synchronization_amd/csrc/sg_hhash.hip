// sg_hhash.hip -- Algorithm 1 of Zen (OSDI'25 digest, section 3.2):
// hierarchical hashing into a per-partition slot memory, as a comparison
// variant of the histogram/scan/scatter partition of sg_partition.hip.
//
// Technique #1: the memory of partition p has r1 parallel slots and r2 serial
// slots.  Technique #3: the partition is p = h0(idx), the same function on
// every worker.  Technique #2: an entry tries the slots h_1(idx) .. h_k(idx)
// of its partition's parallel memory.  Technique #4: a write must not be lost
// to a concurrent writer of the same slot -- here the check and the write are
// one compare-and-swap (the atomic form of "write if empty, notice if
// another thread won").  After k occupied slots the entry takes the next
// serial slot from the partition's atomic counter (starting at r1); past
// r1 + r2 it is lost and counted.  The partitions are then extracted in slot
// order.
//
// A slot holds (entry position within the worker + 1), 0 meaning empty, so
// the extraction gathers the index and its values.  h_i(idx) is MurmurHash2
// of the index's 4 bytes with seed + i, mod r1.
//
// Kernels: insert (one thread per entry), then per 1024-slot tile a count,
// a per-worker scan of the tiles in slot order, and an ordered write.
#include "sg_host.h"

namespace sg {

constexpr int HH_TILE = 1024;

struct HhParams {
    const uint32_t* idx;
    const void* val;
    const uint64_t* in_off;
    uint32_t* x;          // [n][P][R] slot memory
    uint32_t* ctr;        // [n][P] serial counters
    uint32_t* tcnt;       // [ntiles] occupied slots of a tile
    uint64_t* tpre;       // [ntiles] exclusive prefix inside the worker
    uint32_t* out_idx;
    void* out_val;
    uint64_t* part_off;   // [n][P+1]
    uint32_t* slot_of;    // [total] or null
    uint64_t* counts;     // [n][2]: serial writes, lost entries
    uint64_t total, R, r1;
    uint32_t n, P, D, k, seed, TPP; // TPP: tiles per partition
    int bf16;
    Divider divP, divR1;
};

// one thread per entry of worker blockIdx.y
__global__ __launch_bounds__(256) void hh_insert_kernel(HhParams p)
{
    const uint32_t w = blockIdx.y;
    uint64_t s = p.in_off[w], e = p.in_off[w + 1];
    if (s > p.total) s = p.total;
    if (e > p.total) e = p.total;
    uint32_t serial = 0, lost = 0;
    for (uint64_t q = s + (uint64_t)blockIdx.x * 256 + threadIdx.x; q < e; q += (uint64_t)gridDim.x * 256) {
        const uint32_t id = p.idx[q];
        const uint32_t mark = (uint32_t)(q - s) + 1u;
        const uint32_t part = h0(id, p.seed, p.divP);
        uint32_t* mem = p.x + ((uint64_t)w * p.P + part) * p.R;
        bool placed = false;
        for (uint32_t i = 1; i <= p.k && !placed; ++i) {
            const uint32_t slot = mod_p(murmur2_u32(id, p.seed + i), p.divR1);
            placed = atomicCAS(&mem[slot], 0u, mark) == 0u;
        }
        if (!placed) {
            ++serial;
            const uint32_t slot = atomicAdd(&p.ctr[(uint64_t)w * p.P + part], 1u);
            if ((uint64_t)slot < p.R) mem[slot] = mark;
            else ++lost;
        }
    }
    // per wave, one add of its serial writes and losses
    const uint32_t sw = wave_sum(serial), lw = wave_sum(lost);
    if (lane_id() == 0) {
        if (sw) atomicAdd((unsigned long long*)&p.counts[2 * w], (unsigned long long)sw);
        if (lw) atomicAdd((unsigned long long*)&p.counts[2 * w + 1], (unsigned long long)lw);
    }
}

// tile t = ((w*P + p)*TPP + j): slots [j*HH_TILE, min(R, (j+1)*HH_TILE)) of
// partition p of worker w; one wave per tile
__device__ __forceinline__ void hh_tile(const HhParams& p, uint64_t t, uint32_t& w, uint32_t& part,
                                        uint64_t& s0, uint32_t& len)
{
    const uint64_t wp = t / p.TPP;
    const uint32_t j = (uint32_t)(t % p.TPP);
    w = (uint32_t)(wp / p.P);
    part = (uint32_t)(wp % p.P);
    s0 = (uint64_t)j * HH_TILE;
    const uint64_t left = p.R - s0;
    len = left < (uint64_t)HH_TILE ? (uint32_t)left : (uint32_t)HH_TILE;
}

__global__ __launch_bounds__(256) void hh_count_kernel(HhParams p, uint64_t ntiles)
{
    const uint64_t t = (uint64_t)blockIdx.x * 4 + threadIdx.x / SG_WAVE;
    if (t >= ntiles) return;
    uint32_t w, part, len;
    uint64_t s0;
    hh_tile(p, t, w, part, s0, len);
    const uint32_t* mem = p.x + ((uint64_t)w * p.P + part) * p.R + s0;
    uint32_t c = 0;
    for (uint32_t i = lane_id(); i < len; i += SG_WAVE) c += mem[i] != 0u;
    c = wave_sum(c);
    if (lane_id() == 0) p.tcnt[t] = c;
}

// per worker: exclusive prefix of its tiles (slot order), partition offsets
__global__ __launch_bounds__(1024) void hh_scan_kernel(HhParams p)
{
    __shared__ uint64_t scan_lds[1024 / SG_WAVE + 1];
    const uint32_t w = blockIdx.x;
    const uint64_t nt = (uint64_t)p.P * p.TPP;
    const uint64_t t0 = (uint64_t)w * nt;
    uint64_t base = p.in_off[w];
    if (base > p.total) base = p.total;
    uint64_t carry = 0;
    for (uint64_t b = 0; b < nt; b += 1024) {
        const uint64_t t = b + threadIdx.x;
        const uint64_t v = t < nt ? p.tcnt[t0 + t] : 0ull;
        uint64_t tot;
        const uint64_t ex = block_excl_scan64<1024>(v, scan_lds, &tot);
        if (t < nt) {
            p.tpre[t0 + t] = base + carry + ex;
            if (t % p.TPP == 0) p.part_off[(uint64_t)w * (p.P + 1) + t / p.TPP] = base + carry + ex;
        }
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) p.part_off[(uint64_t)w * (p.P + 1) + p.P] = base + carry;
}

// ordered write of a tile's occupied slots
__global__ __launch_bounds__(256) void hh_write_kernel(HhParams p, uint64_t ntiles)
{
    const uint64_t t = (uint64_t)blockIdx.x * 4 + threadIdx.x / SG_WAVE;
    if (t >= ntiles) return;
    uint32_t w, part, len;
    uint64_t s0;
    hh_tile(p, t, w, part, s0, len);
    const uint32_t* mem = p.x + ((uint64_t)w * p.P + part) * p.R + s0;
    const uint64_t ws = p.in_off[w];
    uint64_t pos = p.tpre[t];
    const uint32_t lane = lane_id();
    for (uint32_t i0 = 0; i0 < len; i0 += SG_WAVE) {
        const uint32_t i = i0 + lane;
        const uint32_t m = i < len ? mem[i] : 0u;
        const uint64_t occ = ballot(m != 0u);
        if (m) {
            const uint64_t o = pos + popc64(occ & lanemask_lt());
            const uint64_t src = ws + m - 1;
            if (o < p.total && src < p.total) {
                p.out_idx[o] = p.idx[src];
                if (p.slot_of) p.slot_of[o] = (uint32_t)(s0 + i);
                if (p.D > 0) {
                    if (p.bf16) {
                        const uint16_t* v = static_cast<const uint16_t*>(p.val) + src * p.D;
                        uint16_t* d = static_cast<uint16_t*>(p.out_val) + o * p.D;
                        for (uint32_t c = 0; c < p.D; ++c) d[c] = v[c];
                    } else {
                        const uint32_t* v = static_cast<const uint32_t*>(p.val) + src * p.D;
                        uint32_t* d = static_cast<uint32_t*>(p.out_val) + o * p.D;
                        for (uint32_t c = 0; c < p.D; ++c) d[c] = v[c];
                    }
                }
            } else {
                report_error(kDevErrPartition);
            }
        }
        pos += popc64(occ);
    }
}

} // namespace sg

using namespace sg;

static uint64_t hh_carve(Carver& c, uint32_t n, uint32_t P, uint64_t R, HhParams* p)
{
    const uint64_t TPP = ceil_div(R, HH_TILE);
    p->x = c.take<uint32_t>((uint64_t)n * P * R);
    p->ctr = c.take<uint32_t>((uint64_t)n * P);
    p->tcnt = c.take<uint32_t>((uint64_t)n * P * TPP);
    p->tpre = c.take<uint64_t>((uint64_t)n * P * TPP);
    return c.bytes();
}

extern "C" size_t sg_hierarchical_hash_workspace_bytes(uint32_t n, uint32_t P, uint64_t r1, uint64_t r2)
{
    HhParams p;
    Carver c(nullptr);
    return hh_carve(c, n, P, r1 + r2, &p);
}

extern "C" int sg_hierarchical_hash(const uint32_t* d_idx, const void* d_val, sg_dtype dt, uint32_t D,
                                    const uint64_t* d_in_off, uint32_t n, uint64_t total, uint32_t P, uint32_t seed,
                                    uint32_t k, uint64_t r1, uint64_t r2, uint32_t* d_out_idx, void* d_out_val,
                                    uint64_t* d_part_off, uint32_t* d_slot_of, uint64_t* d_counts, void* d_ws,
                                    size_t ws_bytes, void* stream)
{
    if (n == 0 || n > 65535 || P == 0 || P > 65536 || k == 0 || k > 64 || r1 == 0) return SG_EINVAL;
    if (dt != SG_F32 && dt != SG_BF16) return SG_EINVAL;
    // slots and the serial counters (r1 + at most `total` increments) stay below 2^32
    if (r1 + r2 >= (1ull << 32) || total >= (1ull << 32) || r1 + total >= (1ull << 32)) return SG_EUNSUPPORTED;
    if (!d_in_off || !d_part_off || !d_counts || !d_ws) return SG_EINVAL;
    if (total > 0 && (!d_idx || !d_out_idx)) return SG_EINVAL;
    if (D > 0 && total > 0 && (!d_val || !d_out_val)) return SG_EINVAL;
    if (ws_bytes < sg_hierarchical_hash_workspace_bytes(n, P, r1, r2)) return SG_ECAPACITY;

    HhParams p;
    Carver c(d_ws);
    const uint64_t R = r1 + r2;
    hh_carve(c, n, P, R, &p);
    p.idx = d_idx;
    p.val = d_val;
    p.in_off = d_in_off;
    p.out_idx = d_out_idx;
    p.out_val = d_out_val;
    p.part_off = d_part_off;
    p.slot_of = d_slot_of;
    p.counts = d_counts;
    p.total = total;
    p.R = R;
    p.r1 = r1;
    p.n = n;
    p.P = P;
    p.D = D;
    p.k = k;
    p.seed = seed;
    p.TPP = (uint32_t)ceil_div(R, HH_TILE);
    p.bf16 = dt == SG_BF16;
    p.divP = make_divider(P);
    p.divR1 = make_divider((uint32_t)r1);
    hipStream_t st = as_stream(stream);

    int rc = fill_u32(p.x, (uint64_t)n * P * R, 0u, st);
    if (rc) return rc;
    rc = fill_u32(p.ctr, (uint64_t)n * P, (uint32_t)r1, st);
    if (rc) return rc;
    rc = fill_u64(d_counts, 2ull * n, 0ull, st);
    if (rc) return rc;
    // entries per worker are not known on the host: a fixed grid per worker,
    // grid-striding over its entries
    const uint64_t per = n ? ceil_div(total, n) : 0;
    uint64_t bx = ceil_div(per ? per : 1, 256);
    if (bx > 2048) bx = 2048;
    probe_begin(SG_PROBE_HHASH_INSERT, st);
    hh_insert_kernel<<<dim3((unsigned)bx, n), 256, 0, st>>>(p);
    SG_TRY_LAUNCH();
    probe_end(SG_PROBE_HHASH_INSERT, st);
    const uint64_t ntiles = (uint64_t)n * P * p.TPP;
    hh_count_kernel<<<(unsigned)ceil_div(ntiles, 4), 256, 0, st>>>(p, ntiles);
    SG_TRY_LAUNCH();
    hh_scan_kernel<<<n, 1024, 0, st>>>(p);
    SG_TRY_LAUNCH();
    hh_write_kernel<<<(unsigned)ceil_div(ntiles, 4), 256, 0, st>>>(p, ntiles);
    SG_TRY_LAUNCH();
    return SG_OK;
}

// sg_common.hip -- status text, the device error record, fill kernels and
// the COO validation entry point of libsg.
#include "sg_host.h"

namespace sg {

__device__ int g_device_error = 0;
Probe g_probe = {0, nullptr, nullptr};

__global__ void fill_u32_kernel(uint32_t* d, uint64_t count, uint32_t v)
{
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < count;
         i += (uint64_t)gridDim.x * blockDim.x)
        d[i] = v;
}

__global__ void fill_u64_kernel(uint64_t* d, uint64_t count, uint64_t v)
{
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < count;
         i += (uint64_t)gridDim.x * blockDim.x)
        d[i] = v;
}

int fill_u32(uint32_t* d, uint64_t count, uint32_t v, hipStream_t st)
{
    if (count == 0) return SG_OK;
    uint64_t blocks = ceil_div(count, 256);
    if (blocks > 4096) blocks = 4096;
    fill_u32_kernel<<<(unsigned)blocks, 256, 0, st>>>(d, count, v);
    SG_TRY_LAUNCH();
    return SG_OK;
}

int fill_u64(uint64_t* d, uint64_t count, uint64_t v, hipStream_t st)
{
    if (count == 0) return SG_OK;
    uint64_t blocks = ceil_div(count, 256);
    if (blocks > 4096) blocks = 4096;
    fill_u64_kernel<<<(unsigned)blocks, 256, 0, st>>>(d, count, v);
    SG_TRY_LAUNCH();
    return SG_OK;
}

// Blocks of `kernel` (launched with `threads` threads) that fit on the
// current device at once, at most `cap`: the grid of a persistent kernel.
// Cached per (device, kernel) under a lock, so concurrent callers on several
// host threads and several devices each see their own device's figure.
static std::mutex g_resident_mu;
static std::map<std::pair<int, const void*>, int> g_resident;

int resident_blocks(const void* kernel, int threads, int cap, int* out)
{
    int dev = 0;
    SG_TRY(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_resident_mu);
    auto it = g_resident.find({dev, kernel});
    if (it == g_resident.end()) {
        int cus = 0, per = 0;
        SG_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
        SG_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0));
        it = g_resident.emplace(std::make_pair(dev, kernel), (per > 0 ? per : 1) * (cus > 0 ? cus : 1)).first;
    }
    *out = it->second < cap ? it->second : cap;
    return SG_OK;
}

static std::mutex g_stage_mu;
static void* g_stage = nullptr;
static size_t g_stage_cap = 0;

int host_stage(size_t bytes, HostStage* out)
{
    out->lock = std::unique_lock<std::mutex>(g_stage_mu);
    if (bytes > g_stage_cap) {
        // earlier users synchronized their copies before releasing the lock
        if (g_stage) SG_TRY(hipHostFree(g_stage));
        g_stage = nullptr;
        g_stage_cap = 0;
        const size_t cap = align_up(bytes < 65536 ? 65536 : bytes, 4096);
        SG_TRY(hipHostMalloc(&g_stage, cap, hipHostMallocDefault));
        g_stage_cap = cap;
    }
    out->ptr = g_stage;
    return SG_OK;
}

// flags[0]: offsets bad, flags[1]: index >= M, flags[2]: not strictly ascending
__global__ void validate_kernel(const uint32_t* __restrict__ idx, const uint64_t* __restrict__ in_off, uint32_t n,
                                uint64_t M, uint64_t total, uint32_t* flags)
{
    const uint64_t tid = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x;
    if (tid <= n) {
        uint64_t o = in_off[tid];
        if (tid == 0 && o != 0) flags[0] = 1;
        if (tid == n && o != total) flags[0] = 1;
        if (tid > 0 && in_off[tid - 1] > o) flags[0] = 1;
    }
    for (uint64_t pos = tid; pos < total; pos += (uint64_t)gridDim.x * blockDim.x) {
        // worker of pos: last w with in_off[w] <= pos
        uint32_t lo = 0, hi = n; // search in [0, n)
        while (lo + 1 < hi) {
            uint32_t mid = (lo + hi) >> 1;
            if (in_off[mid] <= pos) lo = mid;
            else hi = mid;
        }
        uint64_t start = in_off[lo];
        uint32_t x = idx[pos];
        if ((uint64_t)x >= M) flags[1] = 1;
        if (pos > start && pos >= 1 && idx[pos - 1] >= x) flags[2] = 1;
    }
}

} // namespace sg

using namespace sg;

extern "C" const char* sg_strerror(int status)
{
    switch (status) {
    case SG_OK: return "ok";
    case SG_EINVAL: return "invalid argument";
    case SG_ECAPACITY: return "output or workspace buffer too small";
    case SG_EUNSORTED: return "indices of a worker are not strictly ascending";
    case SG_EHIP: return "HIP runtime error";
    case SG_EUNSUPPORTED: return "parameters outside what this build implements";
    case SG_ERANGE: return "index out of range or inconsistent offsets";
    case SG_EDEVICE: return "a kernel recorded a violated precondition";
    default: return "unknown status";
    }
}

extern "C" int sg_device_error(void* stream)
{
    int v = 0, zero = 0;
    hipStream_t st = as_stream(stream);
    SG_TRY(hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_device_error), sizeof(int), 0, hipMemcpyDeviceToHost, st));
    SG_TRY(hipMemcpyToSymbolAsync(HIP_SYMBOL(g_device_error), &zero, sizeof(int), 0, hipMemcpyHostToDevice, st));
    SG_TRY(hipStreamSynchronize(st));
    return v ? SG_EDEVICE : SG_OK;
}

extern "C" int sg_probe_set(int kernel_id, void* start_event, void* stop_event)
{
    if (kernel_id < 0 || kernel_id > SG_PROBE_AGGREGATE_COUNT) return SG_EINVAL; // the last id of sg_probe_kernel
    if (kernel_id != SG_PROBE_NONE && (!start_event || !stop_event)) return SG_EINVAL;
    g_probe.id = kernel_id;
    g_probe.start = reinterpret_cast<hipEvent_t>(start_event);
    g_probe.stop = reinterpret_cast<hipEvent_t>(stop_event);
    return SG_OK;
}

extern "C" size_t sg_validate_workspace_bytes(void) { return 256; }

extern "C" int sg_validate_coo(const uint32_t* d_idx, const uint64_t* d_in_off, uint32_t n, uint64_t M,
                               uint64_t total, void* d_ws, size_t ws_bytes, void* stream)
{
    if (!d_in_off || !d_ws || n == 0 || (total > 0 && !d_idx)) return SG_EINVAL;
    if (ws_bytes < sg_validate_workspace_bytes()) return SG_ECAPACITY;
    hipStream_t st = as_stream(stream);
    uint32_t* flags = static_cast<uint32_t*>(d_ws);
    int rc = fill_u32(flags, 4, 0, st);
    if (rc) return rc;
    uint64_t blocks = ceil_div(total > n + 1 ? total : n + 1, 256);
    if (blocks > 2048) blocks = 2048;
    validate_kernel<<<(unsigned)blocks, 256, 0, st>>>(d_idx, d_in_off, n, M, total, flags);
    SG_TRY_LAUNCH();
    uint32_t h[4];
    SG_TRY(hipMemcpyAsync(h, flags, sizeof(h), hipMemcpyDeviceToHost, st));
    SG_TRY(hipStreamSynchronize(st));
    if (h[0] || h[1]) return SG_ERANGE;
    if (h[2]) return SG_EUNSORTED;
    return SG_OK;
}

// sg_host.h -- host-side helpers shared by the entry points of libsg:
// status codes, workspace carving, the modulo divider, launch checks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/sg.h"
#include "sg_device.h"

namespace sg {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
inline uint64_t align_up(uint64_t a, uint64_t b) { return ceil_div(a, b) * b; }

// Carves aligned sub-buffers out of one caller workspace.  Used twice per
// call: once with base == nullptr to size the workspace, once to place it.
struct Carver {
    char* base;
    uint64_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(uint64_t count)
    {
        off = align_up(off, 256);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
    uint64_t bytes() const { return align_up(off, 256) + 256; }
};

inline Divider make_divider(uint32_t P)
{
    Divider d;
    d.P = P;
    if ((P & (P - 1u)) == 0u) {
        d.mul = 0;
        d.shift = 0;
        d.pow2 = 1;
        return d;
    }
    uint32_t l = 0;
    while ((1ull << l) < P) ++l; // l = ceil(log2 P)
    uint64_t m = ((1ull << 32) * ((1ull << l) - P)) / P + 1ull;
    d.mul = (uint32_t)m;
    d.shift = l - 1;
    d.pow2 = 0;
    return d;
}

#define SG_TRY_LAUNCH()                                      \
    do {                                                     \
        if (hipGetLastError() != hipSuccess) return SG_EHIP; \
    } while (0)

#define SG_TRY(x)                                 \
    do {                                          \
        if ((x) != hipSuccess) return SG_EHIP;    \
    } while (0)

// Fill a device range with a 32-bit value from a kernel (graph-safe: no
// memset node is recorded when a caller captures the stream).
int fill_u32(uint32_t* d, uint64_t count, uint32_t v, hipStream_t st);
int fill_u64(uint64_t* d, uint64_t count, uint64_t v, hipStream_t st);

// Blocks of a persistent kernel resident on the current device at once
// (occupancy x compute units), at most cap; cached per device and kernel.
int resident_blocks(const void* kernel, int threads, int cap, int* out);

// Small results that an entry point returns on the host travel in one copy
// into a pinned staging buffer of the process (grown on demand).  The lock
// is held from the copy to the end of the unpacking.
struct HostStage {
    std::unique_lock<std::mutex> lock;
    void* ptr = nullptr;
};
int host_stage(size_t bytes, HostStage* out);


// measurement hook (see sg_probe_set in sg.h)
struct Probe {
    int id;
    hipEvent_t start, stop;
};
extern Probe g_probe;
inline void probe_begin(int id, hipStream_t st)
{
    if (g_probe.id == id && g_probe.start) (void)hipEventRecord(g_probe.start, st);
}
inline void probe_end(int id, hipStream_t st)
{
    if (g_probe.id == id && g_probe.stop) (void)hipEventRecord(g_probe.stop, st);
}

} // namespace sg

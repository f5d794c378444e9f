// Device memory of the allocation-free Muon step (muon_owner_step_noalloc):
// one file-scope array per device holding that step's work list and
// intermediates, and the kernel that uploads a work list through kernel
// arguments (no host staging buffer, nothing allocated).
//
// The array belongs to this file's code object, which the HIP runtime loads
// on a device the first time one of this file's symbols is used there; the
// regular entry points never touch it, so only callers of the allocation-free
// step hold its memory.  Each device holds its own copy at its own address,
// until the process ends.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "device_common.h"
#include "mo_kernels.h"

static __device__ __align__(256) uint8_t scratch[MO_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

// One piece of a work list, passed by value as a kernel argument.
constexpr int WL_CHUNK = 3584;
struct WlChunk {
    u32x4 q[WL_CHUNK / 16];
};

// Thread t copies bytes [16 t, 16 t + 16) of the chunk when they are < n.
__global__ __launch_bounds__(WL_CHUNK / 16) void wl_upload_kernel(uint8_t* dst, WlChunk c, uint32_t n) {
    const uint32_t t = threadIdx.x;
    if (16 * t < n) reinterpret_cast<u32x4*>(dst)[t] = c.q[t];
}

}  // namespace

// Device address of this device's `scratch` (the current device), taken once
// per device with hipGetSymbolAddress and kept; the array's name is only a
// host-side stand-in and is never passed to a kernel or a copy.
hipError_t mo_static_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// Copies `bytes` (a multiple of 16) of host memory to dst on s, WL_CHUNK bytes
// per launch, carried in the launch's arguments.
hipError_t mo_launch_wl_upload(uint8_t* dst, const uint8_t* src, size_t bytes, hipStream_t s) {
    if (bytes % 16) return hipErrorInvalidValue;
    for (size_t off = 0; off < bytes; off += WL_CHUNK) {
        const uint32_t n = uint32_t(bytes - off < size_t(WL_CHUNK) ? bytes - off : size_t(WL_CHUNK));
        WlChunk c;
        std::memset(&c, 0, sizeof(c));
        std::memcpy(&c, src + off, n);
        hipLaunchKernelGGL(wl_upload_kernel, dim3(1), dim3(WL_CHUNK / 16), 0, s, dst + off, c, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// verify_noalloc.hip -- fixed device scratch for the allocation-free verify GEMM
// entry point (vq_gemm_q4_0_noalloc).
//
// The walk form of the verify GEMM needs device memory beyond its inputs and
// outputs: one arrival counter per workgroup and wave, and the fp32 partial
// sums of tile groups cut between two workgroups' ranges.  vq_gemm_q4_0 takes
// that memory from the caller (a workspace); callers that cannot allocate
// (code under HIP graph capture, tight serving loops) get it from the array
// below instead: a file-scope device array of kNoallocScratchBytes, one copy
// per GPU the library runs on, held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever handed to a kernel.
#include <atomic>
#include <mutex>

#include "vq_device.h"
#include "vq_internal.h"

namespace vq {

namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_lock;

// Clears the arrival counters (a kernel, so that a caller capturing the
// stream records no memset node).
__global__ __launch_bounds__(256) void zero_counters_kernel(uint32_t *p, int n) {
    const int i = (int)(blockIdx.x * 256 + threadIdx.x);
    if (i < n)
        p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> guard(g_scratch_lock);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            // set-up, once per device, with that device current: the array's
            // address on this device, and the counters at zero (every call
            // leaves them at zero again)
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return e != hipSuccess ? e : hipErrorInvalidSymbol;
            constexpr int n = (int)(kWalkCounterBytes / 4);
            hipLaunchKernelGGL(zero_counters_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                               static_cast<uint32_t *>(p), n);
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace vq

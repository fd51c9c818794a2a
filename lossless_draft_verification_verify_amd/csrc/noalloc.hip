// Static device scratch for spec_verify_noalloc: the workspace of a verify
// call held in a file-scope device array, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops).
//
// The array lives in the library's code object, so each GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In host
// code the name `scratch` is only a host-side stand-in for that symbol: its
// device address comes from hipGetSymbolAddress, asked once per device with
// the device current, and only that address is ever passed to a kernel.
//
// Every call on one GPU shares the array: calls that overlap in time on one
// GPU (two streams, or two host threads) race.  Each call clears the part it
// uses with a fill kernel before its verify launches, so it does not depend on
// how an earlier call ended.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "sv_plan.h"

static __device__ __align__(256) unsigned char scratch[sv::kNoAllocScratchBytes];

namespace sv {
namespace {

constexpr int kMaxDevices = 128;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void k_zero16(uint4 *p, size_t n16) {
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += size_t(gridDim.x) * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

int noalloc_scratch(int dev, void **out) {
    *out = nullptr;
    if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return int(e);
        if (!ptr) return int(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return 0;
}

int launch_zero(void *p, size_t bytes, void *stream) {
    const size_t n16 = bytes / 16;           // callers pass a multiple of 256
    if (n16 == 0) return 0;
    const unsigned grid = unsigned(std::min<size_t>((n16 + 255) / 256, 1024));
    hipLaunchKernelGGL(k_zero16, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint4 *>(p), n16);
    return int(hipGetLastError());
}

}  // namespace sv

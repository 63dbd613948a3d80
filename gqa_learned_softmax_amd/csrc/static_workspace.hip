// The workspace of sinkattn_decode_static: a file-scope device array that the library owns, for
// callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation). Every GPU the library runs on holds one copy of it, from the time the code
// object is loaded until the process ends; every call on that GPU shares it.
#include <mutex>

#include "launch.h"

namespace sinkattn {
namespace {

__device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

// Zeroes n 32-bit words (a kernel rather than hipMemsetAsync, so that a first call made under
// graph capture records a kernel node, never a memset node).
__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_device_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_decode_workspace(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_device_ptr[dev] == nullptr) {
        // First use on this device (the current one): the array's device address. In host code
        // the name `scratch` is only a stand-in; the pointer below is what kernels are given.
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        // The arrival counters at its start must be zero before their first use; every call
        // that completes leaves them zero again. The whole array is cleared once, on the
        // caller's stream, ahead of the call's own kernels.
        clear_words<<<dim3(1024), dim3(256), 0, stream>>>(static_cast<uint32_t*>(ptr),
                                                        static_cast<int64_t>(kStaticWorkspaceBytes / 4));
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        g_device_ptr[dev] = ptr;
    }
    *out = g_device_ptr[dev];
    return hipSuccess;
}

}  // namespace sinkattn

// scratch.hip -- the device-resident scratch of skv_attn_splitkv_decode_noalloc.
//
// That entry point serves callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its
// partial states and arrival counters live in one file-scope device array that
// every GPU the library runs on holds until the process ends.  Host code never
// passes the array's name to a kernel (in host code that name is only a stand-in
// for the symbol): each device's address is looked up once with
// hipGetSymbolAddress and cached, and only that address reaches kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace skv {

// Arrival counters (kTicketBlockBytes, first) then the partial states, laid out
// exactly as the workspace of skv_attn_splitkv_decode.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];      // device address of `scratch`, per device
bool g_zeroed[kMaxDevices];    // counters cleared by an executed (not captured) fill

}  // namespace

hipError_t noalloc_scratch(void** ptr, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    if (!g_zeroed[dev]) {
        // The counters must start at zero (every decode call returns them to zero).
        // A fill kernel rather than hipMemsetAsync keeps this safe under graph
        // capture; a captured fill only counts once it has really run, so the flag
        // is set only outside capture.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, (uint32_t*)g_ptr[dev],
                           (int64_t)(kTicketBlockBytes / sizeof(uint32_t)));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (cs == hipStreamCaptureStatusNone) g_zeroed[dev] = true;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace skv

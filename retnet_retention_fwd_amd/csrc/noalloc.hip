// The chunkwise forward for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops and harnesses that forbid allocation): the same call as
// retention_chunkwise_fwd, with the segment-state scratch it needs taken from a
// fixed-size device array of the library instead of a caller workspace.
//
// The array is a file-scope __device__ variable: each device the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never uses the
// variable's name as a device pointer (in host code it is only a stand-in): the device
// address is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.  Nothing here allocates or frees memory.

#include "../../include/retention.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = RETN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of `scratch` on device `dev` (looked up once, with dev current).
void* scratch_on(int dev) {
    std::call_once(g_once[dev], [dev] {
        int prev = 0;
        hipError_t e = hipGetDevice(&prev);
        if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
        void* p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != dev) (void)hipSetDevice(prev);
        g_err[dev] = e;
        g_ptr[dev] = e == hipSuccess ? p : nullptr;
    });
    return g_ptr[dev];
}

}  // namespace

extern "C" retn_status retention_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v,
                                                       const float* gamma, void* o, const float* state_in,
                                                       float* state_out, int B, int H, int N, int dk, int dv,
                                                       int chunk, retn_dtype dtype, void* stream) {
    // the scratch this call needs (0 for invalid sizes, which the forward rejects)
    const size_t need = retention_workspace_bytes(B, H, N, dk, dv, chunk, dtype, 0);
    if (need > kScratchBytes) return RETN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        // the stream's device (the calling thread's current device for the null stream)
        int dev = -1;
        hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                         : hipGetDevice(&dev);
        if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return RETN_ERR_HIP;
        ws = scratch_on(dev);
        if (ws == nullptr) return RETN_ERR_HIP;
    }
    return retention_chunkwise_fwd(q, k, v, gamma, o, state_in, state_out, B, H, N, dk, dv, chunk, dtype, ws,
                                   ws != nullptr ? kScratchBytes : 0, stream);
}

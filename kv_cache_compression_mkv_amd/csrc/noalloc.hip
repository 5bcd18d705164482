// Scratch memory of the allocation-free decode entry point
// (mkv_decode_attn_noalloc): a file-scope device array that stands in for the
// caller's workspace, for callers that cannot allocate device memory.
//
// In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and cached, and only that address is handed to kernels.
// Each device holds its own copy of the array from the library's first use on
// it until the process ends. Every call on one device shares it, so calls
// that overlap on one device race; the decode writes every scratch byte it
// later reads within the same call, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mkv_internal.h"

static __device__ __align__(256) unsigned char scratch[MKV_SCRATCH_BYTES];

namespace mkv {

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_addr[MAX_DEVICES];  // device address of `scratch` per device, once known

}  // namespace

hipError_t scratch_address(hipStream_t stream, void **ptr) {
    *ptr = nullptr;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return e;
        dev = (int)sd;
    }
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_addr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace mkv

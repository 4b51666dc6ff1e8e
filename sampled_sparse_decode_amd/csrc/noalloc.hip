// Device scratch of santa_decode_attention_noalloc: a file-scope array in
// device memory, so callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc) still get a
// workspace. Every GPU the library runs on holds one copy of the array until
// the process ends; calls that overlap on one GPU share it and race.
//
// In host code the array's name is only a stand-in for the symbol, not a
// device address. Its address on each device is looked up once, with that
// device current, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "santa_internal.h"

namespace santa {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

santa_status noalloc_scratch(void *stream, void **ptr) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return SANTA_ERR_HIP;
    int dev = cur;
    if (st != nullptr) {
        hipDevice_t sd = 0;
        if (hipStreamGetDevice(st, &sd) != hipSuccess) return SANTA_ERR_HIP;
        dev = int(sd);
    }
    if (dev < 0 || dev >= kMaxDevices) return SANTA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return SANTA_ERR_HIP;
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return SANTA_ERR_HIP;
        if (err != hipSuccess || p == nullptr) return SANTA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SANTA_OK;
}

}  // namespace santa

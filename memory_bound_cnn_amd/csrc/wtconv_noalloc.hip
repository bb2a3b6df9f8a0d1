// wtconv_backward_noalloc: the fused backward pass with its scratch (the
// weight-gradient partial records that wtconv_backward keeps in the caller's
// workspace) in a fixed device array, so that the call allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wtc_internal.h"

namespace wtc {
namespace {

// One copy per GPU, held until the process ends.  In host code `scratch` names
// a host-side stand-in, never the device array: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[WTCONV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's array, looked up once per device
// with that device current.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WTC_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WTC_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return WTC_OK;
}

}  // namespace
}  // namespace wtc

extern "C" int wtconv_backward_noalloc(const wtc_desc* d, const void* x, const void* g, const float* w0,
                                       const float* s0, const float* wl, const float* sl, void* dx, float* dw0,
                                       float* ds0, float* db0, float* dwl, float* dsl, void* stream) {
    int st = wtc::backward_check(d, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl);
    if (st != WTC_OK) return st;
    const size_t need = wtconv_backward_workspace(d);
    if (need > WTCONV_NOALLOC_SCRATCH_BYTES) return WTC_ESCRATCH;
    void* ws = nullptr;
    if ((st = wtc::scratch_address(&ws)) != WTC_OK) return st;
    return wtconv_backward(d, x, g, w0, s0, wl, sl, dx, dw0, ds0, db0, dwl, dsl, ws, WTCONV_NOALLOC_SCRATCH_BYTES,
                           stream);
}

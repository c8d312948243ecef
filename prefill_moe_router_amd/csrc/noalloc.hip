// noalloc.hip -- moe_forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the workspace is a fixed-size array in the library's own device memory.
//
// The array `scratch` is a file-scope __device__ symbol.  Its name in host code is
// only a host-side stand-in: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is ever
// handed to kernels or copies.  Each device that runs the library holds its own
// copy until the process ends.  Every call on one device shares that device's
// array, so calls that overlap on one device (other streams, other threads) race.
#include <mutex>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct DeviceScratch {
    void *ptr = nullptr;     // device address of `scratch` on this device
    bool cleared = false;    // the clear of the first call has been enqueued
};

std::mutex g_mutex;
DeviceScratch g_dev[kMaxDevices];

__global__ __launch_bounds__(256) void clear_scratch_kernel(uint4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0, 0, 0, 0);
}

// the device error word (byte 0 of the workspace) moves to the caller's int and clears
__global__ void take_error_kernel(int32_t *ws_err, int32_t *out) {
    *out = *ws_err;
    *ws_err = 0;
}

// The current device's scratch address, looked up once per device (set-up: the first
// call on each device, with that device current).
hipError_t device_scratch(DeviceScratch **out) {
    int dev = 0;
    hipError_t r = hipGetDevice(&dev);
    if (r != hipSuccess) return r;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceScratch &d = g_dev[dev];
    if (!d.ptr) {
        void *p = nullptr;
        r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r != hipSuccess) return r;
        if (!p) return hipErrorInvalidSymbol;
        d.ptr = p;
    }
    *out = &d;
    return hipSuccess;
}

// The first call on a device enqueues a clear of the whole array on `st` before its
// launches (the workspace contract: zero before first use).  A graph that captures that
// call clears the array at every replay, which is equally correct.
hipError_t clear_once(DeviceScratch &d, hipStream_t st) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (d.cleared) return hipSuccess;
    hipLaunchKernelGGL(clear_scratch_kernel, dim3(1024), dim3(256), 0, st, static_cast<uint4 *>(d.ptr),
                       kScratchBytes / 16);
    const hipError_t r = hipGetLastError();
    if (r == hipSuccess) d.cleared = true;
    return r;
}

}  // namespace

}  // namespace moe

extern "C" moe_status moe_forward_noalloc(const moe_shape *shape, const void *x, const void *w_router,
                                          const float *bias, const moe_expert_weights *w, void *y,
                                          int32_t *topk_ids_out, float *topk_w_out, int32_t *device_err,
                                          void *stream) {
    using namespace moe;
    const size_t need = moe_workspace_size(shape);
    if (need == 0) return MOE_ERR_INVALID_ARG;
    if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
    if (device_err && (reinterpret_cast<uintptr_t>(device_err) & 15u)) return MOE_ERR_INVALID_ARG;
    DeviceScratch *d = nullptr;
    if (device_scratch(&d) != hipSuccess) return MOE_ERR_HIP;
    // every argument is checked before anything is enqueued
    const moe_status chk =
        forward_check(shape, x, w_router, bias, w, y, topk_ids_out, topk_w_out, d->ptr, kScratchBytes);
    if (chk != MOE_OK || shape->num_tokens == 0) return chk;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (clear_once(*d, st) != hipSuccess) return MOE_ERR_HIP;
    const moe_status s =
        forward_impl(shape, x, w_router, bias, w, y, topk_ids_out, topk_w_out, d->ptr, kScratchBytes, st, nullptr, 0);
    if (s != MOE_OK || !device_err) return s;
    hipLaunchKernelGGL(take_error_kernel, dim3(1), dim3(1), 0, st, static_cast<int32_t *>(d->ptr), device_err);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

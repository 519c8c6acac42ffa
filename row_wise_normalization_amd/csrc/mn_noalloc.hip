// mn_noalloc.hip -- the RMSNorm backward for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses
// that forbid hipMalloc): the same kernels as mn_rmsnorm_backward, with the
// per-workgroup dgamma partial rows (and the hand-off words of the one-launch
// backward of small problems) in a fixed device array of this library
// instead of a caller workspace.
//
// The array lives in each device's copy of the code object until the
// process ends. Host code never passes the array's own name to a kernel: in
// host code that name is only a stand-in for the symbol. Its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the kernels receive.
#include "mn_norm.h"

#include <mutex>

#include "mn_internal.hpp"

namespace mn {
mn_status record_device_error(hipError_t e);  // mn_api.cpp
}

namespace {

// Largest RMSNorm partial-row area: at most 512 rows of up to 3072 columns
// or 256 rows of up to 8192 columns, 8 MiB (checked against
// mn_norm_workspace_bytes for every shape by the host tests).
constexpr size_t kScratchBytes = (size_t)8 << 20;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

// Device address of `dev`'s copy of the scratch array, looked up on first
// use with `dev` current.
mn_status scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return MN_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return mn::record_device_error(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return mn::record_device_error(e);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = (cur != dev) ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return mn::record_device_error(e);
        if (back != hipSuccess) return mn::record_device_error(back);
        if (p == nullptr) return MN_ERR_DEVICE;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MN_OK;
}

}  // namespace

extern "C" {

size_t mn_noalloc_scratch_bytes(void) { return kScratchBytes; }

mn_status mn_rmsnorm_backward_noalloc(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                                      const mn_f16* dY, mn_f16* dX, float* dgamma, int64_t N,
                                      int64_t D, void* stream)
{
    // argument errors first, as the workspace entry point reports them, and
    // before anything touches a device
    if (!X || !gamma || !rstd || !dY || !dX || !dgamma) return MN_ERR_NULL;
    const size_t need = mn_norm_workspace_bytes(MN_RMSNORM, N, D);
    if (need == 0) return MN_ERR_SHAPE;
    if (need > kScratchBytes) return MN_ERR_WORKSPACE;
    // the device the work is enqueued on
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev)
                          : hipGetDevice(&dev);
    if (e != hipSuccess) return mn::record_device_error(e);
    void* ws = nullptr;
    const mn_status s = scratch_address(dev, &ws);
    if (s != MN_OK) return s;
    // every workgroup writes its whole partial row before stage 2 reads it,
    // so nothing in the array has to start at zero
    return mn_rmsnorm_backward(X, gamma, rstd, dY, dX, dgamma, N, D, ws, kScratchBytes, stream);
}

}  // extern "C"

// iabn_forward_train_noalloc: the training forward with its workspace in a
// static device array instead of a caller's buffer, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Declared in iabn.h.
//
// The array lives in this code object; every device the library runs on holds
// its own copy from module load until the process ends.  Host code never passes
// the array's name to a kernel or a copy (on the host it only stands for the
// symbol): the device address of the current device's copy is looked up once per
// device with hipGetSymbolAddress and cached, and that address is what the
// kernels get, as the workspace argument of iabn_forward_train.
#include <stdint.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "iabn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[IABN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of scratch on each device (null until looked up).
std::atomic<void*> g_scratch_addr[kMaxDevices];

// The current device's copy of scratch, looked up on its first use there.
iabn_status scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return IABN_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return IABN_ERR_UNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return IABN_ERR_HIP;
        }
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return IABN_OK;
}

}  // namespace

extern "C" iabn_status iabn_forward_train_noalloc(
    void* x_inout, int64_t N, int64_t C, int64_t H, int64_t W, iabn_layout layout,
    iabn_dtype dtype, const float* gamma, const float* beta, float* running_mean,
    float* running_var, float* save_mean, float* save_invstd, iabn_act act, float act_param,
    float eps, float momentum, hipStream_t stream)
{
    // the size check is host arithmetic only: a request beyond the array is
    // rejected before any HIP call
    const size_t need = iabn_workspace_size(N, C, H, W, layout, dtype);
    if (need > size_t(IABN_NOALLOC_SCRATCH_BYTES)) return IABN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        // every other argument checked first: with no workspace the call returns
        // IABN_ERR_WORKSPACE, launching nothing, exactly when the rest is valid
        const iabn_status v = iabn_forward_train(
            x_inout, N, C, H, W, layout, dtype, gamma, beta, running_mean, running_var,
            save_mean, save_invstd, act, act_param, eps, momentum, nullptr, 0, stream);
        if (v != IABN_ERR_WORKSPACE) return v;
        const iabn_status st = scratch_address(&ws);
        if (st != IABN_OK) return st;
    }
    return iabn_forward_train(x_inout, N, C, H, W, layout, dtype, gamma, beta, running_mean,
                              running_var, save_mean, save_invstd, act, act_param, eps, momentum,
                              ws, need > 0 ? size_t(IABN_NOALLOC_SCRATCH_BYTES) : 0, stream);
}

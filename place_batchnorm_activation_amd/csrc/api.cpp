// C ABI of the In-Place ABN library: argument validation (before any HIP call),
// plan selection, and launches on the caller's stream.  Declared in iabn.h.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include <hip/hip_runtime_api.h>

#include "fused.hpp"
#include "iabn.h"
#include "launch.hpp"
#include "plan.hpp"

using namespace iabn;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool finite_pos(float v) { return v > 0.f && isfinite(v); }

iabn_status check_shape(int64_t N, int64_t C, int64_t H, int64_t W, iabn_layout layout,
                        iabn_dtype dtype)
{
    if (layout != IABN_NCHW && layout != IABN_NHWC) return IABN_ERR_INVALID_ARG;
    if (dtype != IABN_F32 && dtype != IABN_BF16 && dtype != IABN_F16) return IABN_ERR_INVALID_ARG;
    if (N < 0 || C < 0 || H < 0 || W < 0) return IABN_ERR_INVALID_ARG;
    // keep every index product well inside int64 and every grid inside 2^31 workgroups
    const double numel = double(N) * double(C) * double(H) * double(W);
    if (numel > 9.0e15) return IABN_ERR_UNSUPPORTED;
    return IABN_OK;
}

iabn_status check_act(iabn_act act, float a)
{
    switch (act) {
    case IABN_ACT_IDENTITY: return IABN_OK;
    case IABN_ACT_LEAKY_RELU:
    case IABN_ACT_ELU: return finite_pos(a) ? IABN_OK : IABN_ERR_INVALID_ARG;
    default: return IABN_ERR_INVALID_ARG;
    }
}

iabn_status check_channel_vec(const float* p, bool required)
{
    if (!p) return required ? IABN_ERR_INVALID_ARG : IABN_OK;
    return aligned(p, 4) ? IABN_OK : IABN_ERR_MISALIGNED;
}

iabn_status check_tensor(const void* p, iabn_dtype dtype)
{
    if (!p) return IABN_ERR_INVALID_ARG;
    return aligned(p, dtype == IABN_F32 ? 4 : 2) ? IABN_OK : IABN_ERR_MISALIGNED;
}

// Workspace bytes of the split kernels, whichever of the vector and scalar plans
// a call takes.
size_t split_bytes(int64_t N, int64_t C, int64_t H, int64_t W, iabn_layout layout,
                   iabn_dtype dtype)
{
    const size_t a = make_plan(N, C, H, W, layout, dtype, false).bytes;
    if (!vec_shape_ok(C, H * W, layout, dtype)) return a;
    const size_t b = make_plan(N, C, H, W, layout, dtype, true).bytes;
    return a > b ? a : b;
}

// Workgroups the current device runs at once with one per CU: its CU count
// (cached per device).  Without a device (planning only) the MI355X's 256.
int64_t coresident_grid()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int cus = cache[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0) {
            (void)hipGetLastError();
            return 256;
        }
        cache[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// Whether plans may take the kernels whose workgroups wait on one another (the
// NCHW channel groups, the NHWC slice groups and the streamed slice kernels):
// iabn_set_grouped_kernels, initially on unless the environment variable
// IABN_GROUPED_KERNELS is "0".
std::atomic<int> g_grouped{-1};

bool grouped_allowed()
{
    int v = g_grouped.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = getenv("IABN_GROUPED_KERNELS");
        v = (e && e[0] == '0' && e[1] == '\0') ? 0 : 1;
        int expect = -1;
        g_grouped.compare_exchange_strong(expect, v, std::memory_order_relaxed);
        v = g_grouped.load(std::memory_order_relaxed);
    }
    return v != 0;
}

// act < 0: the stage entry points, which always run the split kernels.
// allow_groups: whether grouped kernels may be planned (by default the
// process-wide setting; the workspace size always plans them, so that one
// workspace serves either setting).
Plan plan_for(int64_t N, int64_t C, int64_t H, int64_t W, iabn_layout layout, iabn_dtype dtype,
              bool ptrs16, int act = -1, int allow_groups = -1)
{
    // the grid a grouped kernel may span: the device's CU count, or 0 (no groups)
    const bool groups = allow_groups < 0 ? grouped_allowed() : allow_groups != 0;
    auto group_grid = [&]() -> int64_t { return groups ? coresident_grid() : 0; };
    const bool vec = ptrs16 && vec_shape_ok(C, H * W, layout, dtype);
    Plan p = make_plan(N, C, H, W, layout, dtype, vec);
    if (act >= 0 && p.layout == kNCHW && p.vec && p.numel > 0) {
        const int64_t vc = p.m / p.V;
        const int f = fused_fwd_pick(vc);
        if (f >= 0 && fused_worthwhile(p, fused_fwd_threads(f))) p.fused_variant = f;
        const int b = fused_bwd_pick(vc);
        if (b >= 0 && fused_worthwhile(p, fused_bwd_threads(b))) p.fused_bwd_variant = b;
        if (p.fused_variant < 0 || p.fused_bwd_variant < 0) {
            // a channel larger than one workgroup holds, or too few channels to
            // fill the chip: a group of workgroups per channel
            const NchwGroupChoice g = fused_nchw_group_pick(p, group_grid());
            if (g.group > 1) {
                p.fused_variant = g.fwd;
                p.fused_bwd_variant = g.bwd;
                p.nchw_group = g.group;
                // the exchange goes past every split-kernel section, which other
                // calls on the same workspace may write: one epoch per channel
                // (padded to 32 words), four tagged words per member and channel
                p.off_xchg = (size_t)align_up((int64_t)split_bytes(N, C, H, W, layout, dtype), 256);
                p.bytes = p.off_xchg +
                          sizeof(uint64_t) * (size_t)nhwc_exchange_words(C, g.group, C);
            }
        }
    }
    if (act < 0 && p.layout == kNHWC && p.vec && p.numel > 0) {
        // the split kernels only; note whether the training forward would stream
        p.fwd_streamed = fused_nhwc_pick(p, group_grid()).variant < 0 &&
                         fused_stream_pick(p, group_grid()).variant >= 0;
    }
    if (act >= 0) {
        const bool nhwc_vec = p.layout == kNHWC && p.vec && p.numel > 0;
        const NhwcChoice nc = fused_nhwc_pick(p, nhwc_vec ? group_grid() : 0);
        p.nhwc_variant = nc.variant;
        p.nhwc_group = nc.group;
        p.scalar_variant = fused_scalar_pick(p);
        int64_t lpr = 1;
        if (nc.variant >= 0) {
            switch (nc.variant) {
#define IABN_ROW(ID, T, LPR, NR) case ID: lpr = LPR; break;
                IABN_FUSED_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
            default: break;
            }
        } else if (nhwc_vec) {
            const NhwcChoice sc = fused_stream_pick(p, group_grid());
            p.stream_variant = sc.variant;
            p.fwd_streamed = sc.variant >= 0;
            if (sc.variant >= 0) {
                p.nhwc_group = sc.group;
                if (stream_bwd_worthwhile(p, sc.variant, sc.group)) p.stream_bwd_variant = sc.variant;
                switch (sc.variant) {
#define IABN_ROW(ID, T, LPR, NRF, LF, UF, NRB, LB, UB) case ID: lpr = LPR; break;
                    IABN_STREAM_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
                default: break;
                }
            }
        }
        if ((nc.variant >= 0 || p.stream_variant >= 0) && p.nhwc_group > 1) {
            // the exchange goes past every split-kernel section, which other calls
            // on the same workspace may write
            p.off_xchg = (size_t)align_up((int64_t)split_bytes(N, C, H, W, layout, dtype), 256);
            p.bytes = p.off_xchg + sizeof(uint64_t) *
                      (size_t)nhwc_exchange_words(C / p.V / lpr, p.nhwc_group, C);
        }
    }
    return p;
}

size_t workspace_bytes_for(int64_t N, int64_t C, int64_t H, int64_t W, iabn_layout layout,
                           iabn_dtype dtype)
{
    const size_t a = split_bytes(N, C, H, W, layout, dtype);
    if (!vec_shape_ok(C, H * W, layout, dtype)) return a;
    // the group exchange (act plays no part in its choice), planned whatever the
    // process-wide setting of grouped kernels
    const size_t b = plan_for(N, C, H, W, layout, dtype, true, IABN_ACT_IDENTITY, 1).bytes;
    return a > b ? a : b;
}

iabn_status check_workspace(const void* ws, size_t bytes, const Plan& pl)
{
    if (pl.bytes == 0) return IABN_OK;
    if (!ws || bytes < pl.bytes) return IABN_ERR_WORKSPACE;
    return aligned(ws, 16) ? IABN_OK : IABN_ERR_MISALIGNED;
}

iabn_status launched()
{
    return hipGetLastError() == hipSuccess ? IABN_OK : IABN_ERR_HIP;
}

bool overlap(const void* a, const void* b, size_t bytes)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bytes && y < x + bytes;
}

#define IABN_TRY(expr)                          \
    do {                                        \
        const iabn_status st_ = (expr);         \
        if (st_ != IABN_OK) return st_;         \
    } while (0)

// Validation shared by iabn_forward_train and iabn_forward_stats.
iabn_status check_forward_train(const void* x, int64_t N, int64_t C, int64_t H, int64_t W,
                                iabn_layout layout, iabn_dtype dtype, const float* gamma,
                                const float* beta, float* rm, float* rv, float* save_mean,
                                float* save_invstd, float eps, float momentum)
{
    IABN_TRY(check_shape(N, C, H, W, layout, dtype));
    if (!(eps >= 0.f) || !isfinite(eps)) return IABN_ERR_INVALID_ARG;
    if (!(momentum >= 0.f && momentum <= 1.f)) return IABN_ERR_INVALID_ARG;
    if ((rm == nullptr) != (rv == nullptr)) return IABN_ERR_INVALID_ARG;
    if (C == 0) return IABN_OK;
    if (N * H * W < 2) return IABN_ERR_INVALID_ARG;
    IABN_TRY(check_tensor(x, dtype));
    IABN_TRY(check_channel_vec(gamma, true));
    IABN_TRY(check_channel_vec(beta, true));
    IABN_TRY(check_channel_vec(rm, false));
    IABN_TRY(check_channel_vec(rv, false));
    IABN_TRY(check_channel_vec(save_mean, true));
    IABN_TRY(check_channel_vec(save_invstd, true));
    return IABN_OK;
}

iabn_status check_backward(const void* y, const void* dy, const void* dx, int64_t N, int64_t C,
                           int64_t H, int64_t W, iabn_layout layout, iabn_dtype dtype,
                           iabn_act act, float a)
{
    IABN_TRY(check_shape(N, C, H, W, layout, dtype));
    IABN_TRY(check_act(act, a));
    if (C == 0) return IABN_OK;
    if (N * H * W < 2) return IABN_ERR_INVALID_ARG;
    IABN_TRY(check_tensor(y, dtype));
    IABN_TRY(check_tensor(dy, dtype));
    IABN_TRY(check_tensor(dx, dtype));
    const size_t bytes = size_t(N * C * H * W) * (dtype == IABN_F32 ? 4 : 2);
    if (overlap(dx, y, bytes)) return IABN_ERR_INVALID_ARG;
    if (dx != dy && overlap(dx, dy, bytes)) return IABN_ERR_INVALID_ARG;
    return IABN_OK;
}

}  // namespace

extern "C" {

const char* iabn_status_string(iabn_status status)
{
    switch (status) {
    case IABN_OK: return "ok";
    case IABN_ERR_INVALID_ARG: return "invalid argument";
    case IABN_ERR_UNSUPPORTED: return "unsupported";
    case IABN_ERR_WORKSPACE: return "workspace missing or too small";
    case IABN_ERR_MISALIGNED: return "misaligned pointer";
    case IABN_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int iabn_version(void) { return 200; }

int iabn_set_grouped_kernels(int enabled)
{
    const int prev = grouped_allowed() ? 1 : 0;
    if (enabled >= 0) g_grouped.store(enabled ? 1 : 0, std::memory_order_relaxed);
    return prev;
}

iabn_status iabn_workspace_status(void* workspace, size_t workspace_bytes, int clear,
                                  int* timed_out, hipStream_t stream)
{
    if (!timed_out) return IABN_ERR_INVALID_ARG;
    *timed_out = 0;
    if (!workspace || workspace_bytes < kWsHeaderBytes) return IABN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return IABN_ERR_MISALIGNED;
    uint64_t word = 0;
    if (hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return IABN_ERR_HIP;
    *timed_out = word == kExchangeTimeout ? 1 : 0;
    if (clear && *timed_out) {
        if (hipMemsetAsync(workspace, 0, sizeof word, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return IABN_ERR_HIP;
    }
    return IABN_OK;
}

size_t iabn_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, iabn_layout layout,
                           iabn_dtype dtype)
{
    if (check_shape(N, C, H, W, layout, dtype) != IABN_OK) return 0;
    if (N * C * H * W == 0) return 0;
    return workspace_bytes_for(N, C, H, W, layout, dtype);
}

iabn_status iabn_forward_stats(const void* x, int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype, const float* gamma,
                               const float* beta, float* running_mean, float* running_var,
                               float* save_mean, float* save_invstd, float eps, float momentum,
                               void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    IABN_TRY(check_forward_train(x, N, C, H, W, layout, dtype, gamma, beta, running_mean,
                                 running_var, save_mean, save_invstd, eps, momentum));
    if (C == 0) return IABN_OK;
    const Plan pl = plan_for(N, C, H, W, layout, dtype, aligned(x, 16));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pl));
    launch_forward_stats(pl, x, gamma, beta, running_mean, running_var, save_mean, save_invstd,
                         eps, momentum, workspace, stream);
    return launched();
}

iabn_status iabn_forward_apply(void* x_inout, int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype, iabn_act act,
                               float act_param, void* workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    IABN_TRY(check_shape(N, C, H, W, layout, dtype));
    IABN_TRY(check_act(act, act_param));
    if (C == 0) return IABN_OK;
    if (N * H * W < 2) return IABN_ERR_INVALID_ARG;
    IABN_TRY(check_tensor(x_inout, dtype));
    const Plan pl = plan_for(N, C, H, W, layout, dtype, aligned(x_inout, 16));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pl));
    launch_forward_apply(pl, x_inout, act, act_param, workspace, stream);
    return launched();
}

iabn_status iabn_forward_train(void* x_inout, int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype, const float* gamma,
                               const float* beta, float* running_mean, float* running_var,
                               float* save_mean, float* save_invstd, iabn_act act,
                               float act_param, float eps, float momentum, void* workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    IABN_TRY(check_act(act, act_param));
    IABN_TRY(check_forward_train(x_inout, N, C, H, W, layout, dtype, gamma, beta, running_mean,
                                 running_var, save_mean, save_invstd, eps, momentum));
    if (C == 0) return IABN_OK;
    const Plan pl = plan_for(N, C, H, W, layout, dtype, aligned(x_inout, 16), act);
    IABN_TRY(check_workspace(workspace, workspace_bytes, pl));
    if (pl.fused_variant >= 0) {
        launch_forward_fused_nchw(pl, x_inout, gamma, beta, running_mean, running_var, save_mean,
                                  save_invstd, eps, momentum, act, act_param, workspace, stream);
        return launched();
    }
    if (pl.scalar_variant >= 0) {
        launch_forward_fused_scalar(pl, x_inout, gamma, beta, running_mean, running_var,
                                    save_mean, save_invstd, eps, momentum, act, act_param,
                                    stream);
        return launched();
    }
    if (pl.nhwc_variant >= 0) {
        launch_forward_fused_nhwc(pl, x_inout, gamma, beta, running_mean, running_var, save_mean,
                                  save_invstd, eps, momentum, act, act_param, workspace, stream);
        return launched();
    }
    if (pl.stream_variant >= 0) {
        launch_forward_stream_nhwc(pl, x_inout, gamma, beta, running_mean, running_var, save_mean,
                                   save_invstd, eps, momentum, act, act_param, workspace, stream);
        return launched();
    }
    launch_forward_stats(pl, x_inout, gamma, beta, running_mean, running_var, save_mean,
                         save_invstd, eps, momentum, workspace, stream);
    launch_forward_apply(pl, x_inout, act, act_param, workspace, stream);
    return launched();
}

iabn_status iabn_forward_eval(void* x_inout, int64_t N, int64_t C, int64_t H, int64_t W,
                              iabn_layout layout, iabn_dtype dtype, const float* gamma,
                              const float* beta, const float* running_mean,
                              const float* running_var, iabn_act act, float act_param, float eps,
                              hipStream_t stream)
{
    IABN_TRY(check_shape(N, C, H, W, layout, dtype));
    IABN_TRY(check_act(act, act_param));
    if (!(eps >= 0.f) || !isfinite(eps)) return IABN_ERR_INVALID_ARG;
    if (N * C * H * W == 0) return IABN_OK;
    IABN_TRY(check_tensor(x_inout, dtype));
    IABN_TRY(check_channel_vec(gamma, true));
    IABN_TRY(check_channel_vec(beta, true));
    IABN_TRY(check_channel_vec(running_mean, true));
    IABN_TRY(check_channel_vec(running_var, true));
    const Plan pl = plan_for(N, C, H, W, layout, dtype, aligned(x_inout, 16));
    launch_forward_eval(pl, x_inout, gamma, beta, running_mean, running_var, eps, act, act_param,
                        stream);
    return launched();
}

iabn_status iabn_backward_reduce(const void* y, const void* dy, int64_t N, int64_t C, int64_t H,
                                 int64_t W, iabn_layout layout, iabn_dtype dtype,
                                 const float* gamma, const float* beta, const float* save_invstd,
                                 float* dgamma, float* dbeta, iabn_act act, float act_param,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    // dx plays no part in the reduction; dy stands in for it in the shared checks
    IABN_TRY(check_shape(N, C, H, W, layout, dtype));
    IABN_TRY(check_act(act, act_param));
    if (C == 0) return IABN_OK;
    if (N * H * W < 2) return IABN_ERR_INVALID_ARG;
    IABN_TRY(check_tensor(y, dtype));
    IABN_TRY(check_tensor(dy, dtype));
    IABN_TRY(check_channel_vec(gamma, true));
    IABN_TRY(check_channel_vec(beta, true));
    IABN_TRY(check_channel_vec(save_invstd, true));
    IABN_TRY(check_channel_vec(dgamma, true));
    IABN_TRY(check_channel_vec(dbeta, true));
    const Plan pl = plan_for(N, C, H, W, layout, dtype, aligned(y, 16) && aligned(dy, 16));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pl));
    launch_backward_reduce(pl, y, dy, gamma, beta, save_invstd, dgamma, dbeta, act, act_param,
                           workspace, stream);
    return launched();
}

iabn_status iabn_backward_apply(const void* y, const void* dy, void* dx, int64_t N, int64_t C,
                                int64_t H, int64_t W, iabn_layout layout, iabn_dtype dtype,
                                iabn_act act, float act_param, void* workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    IABN_TRY(check_backward(y, dy, dx, N, C, H, W, layout, dtype, act, act_param));
    if (C == 0) return IABN_OK;
    const Plan pl = plan_for(N, C, H, W, layout, dtype,
                             aligned(y, 16) && aligned(dy, 16) && aligned(dx, 16));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pl));
    launch_backward_apply(pl, y, dy, dx, act, act_param, workspace, stream);
    return launched();
}

iabn_status iabn_backward(const void* y, const void* dy, void* dx, int64_t N, int64_t C,
                          int64_t H, int64_t W, iabn_layout layout, iabn_dtype dtype,
                          const float* gamma, const float* beta, const float* save_invstd,
                          float* dgamma, float* dbeta, iabn_act act, float act_param,
                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    IABN_TRY(check_backward(y, dy, dx, N, C, H, W, layout, dtype, act, act_param));
    if (C == 0) return IABN_OK;
    IABN_TRY(check_channel_vec(gamma, true));
    IABN_TRY(check_channel_vec(beta, true));
    IABN_TRY(check_channel_vec(save_invstd, true));
    IABN_TRY(check_channel_vec(dgamma, true));
    IABN_TRY(check_channel_vec(dbeta, true));
    const Plan pr = plan_for(N, C, H, W, layout, dtype, aligned(y, 16) && aligned(dy, 16));
    const Plan pa = plan_for(N, C, H, W, layout, dtype,
                             aligned(y, 16) && aligned(dy, 16) && aligned(dx, 16), act);
    IABN_TRY(check_workspace(workspace, workspace_bytes, pr));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pa));
    if (pa.fused_bwd_variant >= 0) {
        launch_backward_fused_nchw(pa, y, dy, dx, gamma, beta, save_invstd, dgamma, dbeta, act,
                                   act_param, workspace, stream);
        return launched();
    }
    if (pa.scalar_variant >= 0) {
        launch_backward_fused_scalar(pa, y, dy, dx, gamma, beta, save_invstd, dgamma, dbeta, act,
                                     act_param, stream);
        return launched();
    }
    if (pa.nhwc_variant >= 0) {
        launch_backward_fused_nhwc(pa, y, dy, dx, gamma, beta, save_invstd, dgamma, dbeta, act,
                                   act_param, workspace, stream);
        return launched();
    }
    if (pa.stream_bwd_variant >= 0) {
        launch_backward_stream_nhwc(pa, y, dy, dx, gamma, beta, save_invstd, dgamma, dbeta, act,
                                    act_param, workspace, stream);
        return launched();
    }
    launch_backward_reduce(pr, y, dy, gamma, beta, save_invstd, dgamma, dbeta, act, act_param,
                           workspace, stream);
    launch_backward_apply(pa, y, dy, dx, act, act_param, workspace, stream);
    return launched();
}

iabn_status iabn_backward_eval(const void* y, const void* dy, void* dx, int64_t N, int64_t C,
                               int64_t H, int64_t W, iabn_layout layout, iabn_dtype dtype,
                               const float* gamma, const float* beta, const float* running_var,
                               float eps, float* dgamma, float* dbeta, iabn_act act,
                               float act_param, void* workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    IABN_TRY(check_shape(N, C, H, W, layout, dtype));
    IABN_TRY(check_act(act, act_param));
    if (!(eps >= 0.f) || !isfinite(eps)) return IABN_ERR_INVALID_ARG;
    if ((dgamma == nullptr) != (dbeta == nullptr)) return IABN_ERR_INVALID_ARG;
    if (C == 0) return IABN_OK;
    if (N * H * W < 1) return IABN_ERR_INVALID_ARG;
    IABN_TRY(check_tensor(y, dtype));
    IABN_TRY(check_tensor(dy, dtype));
    IABN_TRY(check_tensor(dx, dtype));
    const size_t bytes = size_t(N * C * H * W) * (dtype == IABN_F32 ? 4 : 2);
    if (overlap(dx, y, bytes)) return IABN_ERR_INVALID_ARG;
    if (dx != dy && overlap(dx, dy, bytes)) return IABN_ERR_INVALID_ARG;
    IABN_TRY(check_channel_vec(gamma, true));
    IABN_TRY(check_channel_vec(beta, true));
    IABN_TRY(check_channel_vec(running_var, true));
    IABN_TRY(check_channel_vec(dgamma, false));
    IABN_TRY(check_channel_vec(dbeta, false));
    const Plan pr = plan_for(N, C, H, W, layout, dtype, aligned(y, 16) && aligned(dy, 16));
    const Plan pa = plan_for(N, C, H, W, layout, dtype,
                             aligned(y, 16) && aligned(dy, 16) && aligned(dx, 16));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pr));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pa));
    if (dgamma) {
        launch_backward_eval_grads(pa, y, dy, dx, gamma, beta, running_var, eps, dgamma, dbeta,
                                   act, act_param, workspace, stream);
    } else {
        launch_eval_consts(pa, gamma, beta, running_var, eps, workspace, stream);
        launch_backward_apply(pa, y, dy, dx, act, act_param, workspace, stream);
    }
    return launched();
}

iabn_status iabn_forward_train_ckpt(void* x_inout, void* y, int64_t N, int64_t C, int64_t H,
                                    int64_t W, iabn_layout layout, iabn_dtype dtype,
                                    const float* gamma, const float* beta, float* running_mean,
                                    float* running_var, float* save_mean, float* save_invstd,
                                    iabn_act act, float act_param, float eps, float momentum,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    IABN_TRY(check_act(act, act_param));
    IABN_TRY(check_forward_train(x_inout, N, C, H, W, layout, dtype, gamma, beta, running_mean,
                                 running_var, save_mean, save_invstd, eps, momentum));
    if (C == 0) return IABN_OK;
    IABN_TRY(check_tensor(y, dtype));
    const size_t bytes = size_t(N * C * H * W) * (dtype == IABN_F32 ? 4 : 2);
    if (overlap(y, x_inout, bytes)) return IABN_ERR_INVALID_ARG;
    const Plan pl = plan_for(N, C, H, W, layout, dtype, aligned(x_inout, 16) && aligned(y, 16));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pl));
    launch_forward_stats(pl, x_inout, gamma, beta, running_mean, running_var, save_mean,
                         save_invstd, eps, momentum, workspace, stream);
    launch_ckpt_forward_apply(pl, x_inout, y, gamma, beta, save_invstd, act, act_param, workspace,
                              stream);
    return launched();
}

iabn_status iabn_recompute_from_xhat(const void* xhat, void* y, int64_t N, int64_t C, int64_t H,
                                     int64_t W, iabn_layout layout, iabn_dtype dtype,
                                     const float* gamma, const float* beta, iabn_act act,
                                     float act_param, hipStream_t stream)
{
    IABN_TRY(check_shape(N, C, H, W, layout, dtype));
    IABN_TRY(check_act(act, act_param));
    if (N * C * H * W == 0) return IABN_OK;
    IABN_TRY(check_tensor(xhat, dtype));
    IABN_TRY(check_tensor(y, dtype));
    IABN_TRY(check_channel_vec(gamma, true));
    IABN_TRY(check_channel_vec(beta, true));
    const size_t bytes = size_t(N * C * H * W) * (dtype == IABN_F32 ? 4 : 2);
    if (y != xhat && overlap(y, xhat, bytes)) return IABN_ERR_INVALID_ARG;
    const Plan pl = plan_for(N, C, H, W, layout, dtype, aligned(xhat, 16) && aligned(y, 16));
    launch_ckpt_recompute(pl, xhat, y, gamma, beta, act, act_param, stream);
    return launched();
}

iabn_status iabn_backward_ckpt(const void* xhat, const void* dy, void* dx, int64_t N, int64_t C,
                               int64_t H, int64_t W, iabn_layout layout, iabn_dtype dtype,
                               const float* gamma, const float* beta, const float* save_invstd,
                               float* dgamma, float* dbeta, iabn_act act, float act_param,
                               void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    IABN_TRY(check_backward(xhat, dy, dx, N, C, H, W, layout, dtype, act, act_param));
    if (C == 0) return IABN_OK;
    IABN_TRY(check_channel_vec(gamma, true));
    IABN_TRY(check_channel_vec(beta, true));
    IABN_TRY(check_channel_vec(save_invstd, true));
    IABN_TRY(check_channel_vec(dgamma, true));
    IABN_TRY(check_channel_vec(dbeta, true));
    const Plan pr = plan_for(N, C, H, W, layout, dtype, aligned(xhat, 16) && aligned(dy, 16));
    const Plan pa = plan_for(N, C, H, W, layout, dtype,
                             aligned(xhat, 16) && aligned(dy, 16) && aligned(dx, 16));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pr));
    IABN_TRY(check_workspace(workspace, workspace_bytes, pa));
    launch_backward_reduce_xhat(pr, xhat, dy, gamma, beta, save_invstd, dgamma, dbeta, act,
                                act_param, workspace, stream);
    launch_ckpt_dx(pa, xhat, dy, dx, gamma, beta, act, act_param, workspace, stream);
    return launched();
}

int iabn_describe_plan(int64_t N, int64_t C, int64_t H, int64_t W, iabn_layout layout,
                       iabn_dtype dtype, iabn_act act, int aligned16, char* buf, size_t len)
{
    if (check_shape(N, C, H, W, layout, dtype) != IABN_OK) return -1;
    if (act != IABN_ACT_IDENTITY && act != IABN_ACT_LEAKY_RELU && act != IABN_ACT_ELU) return -1;
    const Plan p = plan_for(N, C, H, W, layout, dtype, aligned16 != 0, act);
    char fwd[96], bwd[96], nd[48] = "", sd[48] = "";
    switch (p.nhwc_variant) {
#define IABN_ROW(ID, T, LPR, NR) case ID: snprintf(nd, sizeof nd, "%dx%dx%d", T, LPR, NR); break;
        IABN_FUSED_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: break;
    }
    if (p.nhwc_variant >= 0 && p.nhwc_group > 1) {
        const size_t n = strlen(nd);
        snprintf(nd + n, sizeof nd - n, ",group%d", p.nhwc_group);
    }
    char sd_f[48] = "", sd_b[48] = "";
    switch (p.stream_variant) {
#define IABN_ROW(ID, T, LPR, NRF, LF, UF, NRB, LB, UB)                                   \
    case ID:                                                                            \
        snprintf(sd_f, sizeof sd_f, "%dx%dx(%d+%d)+%d,group%d", T, LPR, NRF, LF, UF,       \
                 p.nhwc_group);                                                         \
        snprintf(sd_b, sizeof sd_b, "%dx%dx(%d+%d)+%d,group%d", T, LPR, NRB, LB, UB,       \
                 p.nhwc_group);                                                         \
        break;
        IABN_STREAM_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: break;
    }
    switch (p.scalar_variant) {
#define IABN_ROW(ID, T, NR) case ID: snprintf(sd, sizeof sd, "%dx%d", T, NR); break;
        IABN_FUSED_SCALAR_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: break;
    }
    if (p.fused_variant >= 0) {
        int T = 0, NR = 0;
        switch (p.fused_variant) {
#define IABN_ROW(ID, T_, NR_) case ID: T = T_; NR = NR_; break;
            IABN_FUSED_FWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
        default: break;
        }
        if (p.nchw_group > 1)
            snprintf(fwd, sizeof fwd, "channel_resident(%dx%d,group%d)", T, NR, p.nchw_group);
        else
            snprintf(fwd, sizeof fwd, "channel_resident(%dx%d)", T, NR);
    } else if (p.scalar_variant >= 0) {
        snprintf(fwd, sizeof fwd, "channel_resident_scalar(%s)", sd);
    } else if (p.nhwc_variant >= 0) {
        snprintf(fwd, sizeof fwd, "slice_resident(%s)", nd);
    } else if (p.stream_variant >= 0) {
        snprintf(fwd, sizeof fwd, "slice_streamed(%s)", sd_f);
    } else {
        snprintf(fwd, sizeof fwd, "split(stats:%lldx%d,apply:%lldx%d,%s)",
                 (long long)p.reduce_blocks, kThreads, (long long)apply_grid(p, act), kThreads,
                 p.vec ? "vec16" : "scalar");
    }
    if (p.fused_bwd_variant >= 0) {
        int T = 0, NR = 0;
        bool dyr = false;
        switch (p.fused_bwd_variant) {
#define IABN_ROW(ID, T_, NRV_, NRL_, G_, DYR_) case ID: T = T_; NR = NRV_ + NRL_; dyr = DYR_; break;
            IABN_FUSED_BWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
        default: break;
        }
        if (p.nchw_group > 1)
            snprintf(bwd, sizeof bwd, "channel_resident(%dx%d,%s,group%d)", T, NR,
                     dyr ? "dy_resident" : "dy_streamed", p.nchw_group);
        else
            snprintf(bwd, sizeof bwd, "channel_resident(%dx%d,%s)", T, NR,
                     dyr ? "dy_resident" : "dy_streamed");
    } else if (p.scalar_variant >= 0) {
        snprintf(bwd, sizeof bwd, "channel_resident_scalar(%s,dy_resident)", sd);
    } else if (p.nhwc_variant >= 0) {
        snprintf(bwd, sizeof bwd, "slice_resident(%s)", nd);
    } else if (p.stream_bwd_variant >= 0) {
        snprintf(bwd, sizeof bwd, "slice_streamed(%s)", sd_b);
    } else {
        snprintf(bwd, sizeof bwd, "split(reduce:%lldx%d,apply:%lldx%d,%s)",
                 (long long)p.reduce_blocks_bwd, kThreads, (long long)dx_grid(p, act), kThreads,
                 p.vec ? "vec16" : "scalar");
    }
    return snprintf(buf, len, "forward=%s backward=%s", fwd, bwd);
}

}  // extern "C"

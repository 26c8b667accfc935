// Channel-resident NCHW kernels: variant tables (shared by the host plan and the
// kernel instantiations) and launchers.
//
// A variant is (workgroup size T, vectors per thread NR held in VGPRs); it holds
// up to T*NR 16-byte vectors of one channel.  512-thread workgroups run two waves
// per SIMD, which leaves each thread up to 256 VGPRs.  The plan takes the
// smallest variant that holds the channel.
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.hpp"

// X(id, T, NR)
#define IABN_FUSED_FWD_VARIANTS(X) \
    X(0, 256, 1)                   \
    X(1, 256, 2)                   \
    X(2, 256, 4)                   \
    X(3, 256, 8)                   \
    X(4, 256, 13)                  \
    X(5, 512, 16)                  \
    X(6, 512, 32)                  \
    X(7, 512, 49)

// X(id, T, NR, DYR): DYR = dy resident too; otherwise dy is streamed twice
#define IABN_FUSED_BWD_VARIANTS(X) \
    X(0, 256, 1, true)             \
    X(1, 256, 2, true)             \
    X(2, 256, 4, true)             \
    X(3, 256, 8, true)             \
    X(4, 256, 13, true)            \
    X(5, 512, 16, false)           \
    X(6, 512, 32, false)           \
    X(7, 512, 49, false)

namespace iabn {

struct FusedVariant { int id, T, NR; bool dyr; };

inline int fused_fwd_pick(int64_t vc)
{
    static const FusedVariant tbl[] = {
#define IABN_ROW(ID, T, NR) {ID, T, NR, false},
        IABN_FUSED_FWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
    };
    for (const auto& v : tbl)
        if (int64_t(v.T) * v.NR >= vc) return v.id;
    return -1;
}

inline int fused_bwd_pick(int64_t vc)
{
    static const FusedVariant tbl[] = {
#define IABN_ROW(ID, T, NR, DYR) {ID, T, NR, DYR},
        IABN_FUSED_BWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
    };
    for (const auto& v : tbl)
        if (int64_t(v.T) * v.NR >= vc) return v.id;
    return -1;
}

inline int fused_fwd_threads(int id)
{
    switch (id) {
#define IABN_ROW(ID, T, NR) case ID: return T;
        IABN_FUSED_FWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: return 0;
    }
}

inline int fused_bwd_threads(int id)
{
    switch (id) {
#define IABN_ROW(ID, T, NR, DYR) case ID: return T;
        IABN_FUSED_BWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: return 0;
    }
}

// Whether the channel-resident kernels fill enough of the chip to beat the
// split path: they run one workgroup per channel.
// ELU's inverse and forward expand to long inline sequences; with the largest
// variants the fully unrolled loops exceed the unroller's limit and the resident
// array would fall back to scratch memory, so ELU stays on the smaller variants.
constexpr int kEluMaxFwdVariant = 6;
constexpr int kEluMaxBwdVariant = 4;

inline bool fused_worthwhile(const Plan& p, int threads)
{
    // 32-bit byte offsets address the tensor
    if (p.layout != kNCHW || !p.vec || p.numel * p.esize >= (int64_t(1) << 32)) return false;
    const int64_t bytes = p.numel * p.esize;
    return p.C * threads >= int64_t(256) * 256 || bytes <= (int64_t(4) << 20);
}

void launch_forward_fused_nchw(const Plan& pl, void* x, const float* gamma, const float* beta,
                               float* rm, float* rv, float* sm, float* si, float eps, float mom,
                               int act, float a, hipStream_t s);

void launch_backward_fused_nchw(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* invstd,
                                float* dgamma, float* dbeta, int act, float a, hipStream_t s);

}  // namespace iabn

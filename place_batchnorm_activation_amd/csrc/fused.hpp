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

// X(id, T, NRV, NRL, G, DYR).  DYR: y and dy both resident, NRV vectors each in
// VGPRs (3S of traffic).  Otherwise y is resident, NRV vectors per thread in VGPRs
// and NRL in LDS, and dy is streamed twice in groups of G (4S).
#define IABN_FUSED_BWD_VARIANTS(X)   \
    X(0, 256, 1, 0, 1, true)         \
    X(1, 256, 2, 0, 1, true)         \
    X(2, 256, 4, 0, 1, true)         \
    X(3, 256, 8, 0, 1, true)         \
    X(4, 256, 13, 0, 1, true)        \
    X(5, 512, 16, 0, 6, false)       \
    X(6, 512, 24, 8, 8, false)       \
    X(7, 512, 33, 16, 8, false)

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
#define IABN_ROW(ID, T, NRV, NRL, G, DYR) {ID, T, NRV + NRL, DYR},
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
#define IABN_ROW(ID, T, NRV, NRL, G, DYR) case ID: return T;
        IABN_FUSED_BWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: return 0;
    }
}

// Whether the channel-resident kernels fill enough of the chip to beat the
// split path: they run one workgroup per channel.
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

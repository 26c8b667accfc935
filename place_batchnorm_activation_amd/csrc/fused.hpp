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

// Slice-resident NHWC kernels.  X(id, T, LPR, NR): T threads; LPR 16-byte lanes
// of every row per workgroup (a slice of LPR*V channels); NR rows per thread, so
// one workgroup holds (T/LPR)*NR rows.  The backward keeps y and dy both resident
// (8*NR VGPRs of data), which bounds NR at 512 threads.  A -D definition of the
// macro replaces the table.
#ifndef IABN_FUSED_NHWC_VARIANTS
#define IABN_FUSED_NHWC_VARIANTS(X) \
    X(0, 256, 1, 2)                  \
    X(1, 256, 1, 4)                  \
    X(2, 256, 1, 8)                  \
    X(3, 256, 1, 13)                 \
    X(4, 512, 1, 13)                 \
    X(5, 512, 1, 18)                 \
    X(6, 512, 2, 4)                  \
    X(7, 512, 2, 8)                  \
    X(8, 512, 2, 13)                 \
    X(9, 512, 2, 18)
#endif

// Channel-resident NCHW kernels on single elements, for shapes the 16-byte
// vectors cannot take (H*W not a multiple of the vector width, e.g. 7x7 maps, or
// pointers not 16-byte aligned).  X(id, T, NR): NR elements per thread, y and dy
// both resident in the backward.
#define IABN_FUSED_SCALAR_VARIANTS(X) \
    X(0, 256, 2)                       \
    X(1, 256, 4)                       \
    X(2, 256, 8)                       \
    X(3, 256, 16)                      \
    X(4, 512, 16)                      \
    X(5, 512, 32)                      \
    X(6, 512, 48)

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

// Slice-resident NHWC variant for a problem, or -1.  Wider slices (LPR = 2: a
// wave reads 32 bytes of each of 32 rows instead of 16 bytes of 64) coalesce
// better, so they are preferred while they still give at least 128 workgroups;
// then the first variant (table order) whose workgroup holds all m rows.  The
// kernels are taken when the slices fill the chip, or when the tensor is small
// enough for launch latency to rule and each workgroup's rows are few (measured:
// 32 workgroups of 6272 rows lose to the split path, 64 of 1568 win).  32-bit
// vector indices address the tensor.
inline int fused_nhwc_pick(const Plan& p)
{
    if (p.layout != kNHWC || !p.vec || p.numel == 0) return -1;
    if (p.numel * p.esize >= (int64_t(1) << 32)) return -1;
    const int64_t cv = p.C / p.V;
    const int64_t bytes = p.numel * p.esize;
    struct Row { int id, T, LPR, NR; };
    static const Row tbl[] = {
#define IABN_ROW(ID, T, LPR, NR) {ID, T, LPR, NR},
        IABN_FUSED_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
    };
    const int want = (cv % 2 == 0 && cv / 2 >= 128) ? 2 : 1;
    for (int pass = 0; pass < 2; ++pass) {
        for (const auto& v : tbl) {
            if ((pass == 0) != (v.LPR == want)) continue;
            if (cv % v.LPR != 0 || int64_t(v.T / v.LPR) * v.NR < p.m) continue;
            const int64_t blocks = cv / v.LPR;
            if (blocks * v.T >= int64_t(256) * 256 || (bytes <= (int64_t(4) << 20) && p.m <= 4096))
                return v.id;
            return -1;
        }
    }
    return -1;
}

// Scalar channel-resident variant for an NCHW problem off the vector path, or -1:
// the smallest that holds the channel's m elements, taken on the same terms as
// the vector kernels (the chip filled, or a tensor under 4 MB).
inline int fused_scalar_pick(const Plan& p)
{
    if (p.layout != kNCHW || p.vec || p.numel == 0) return -1;
    if (p.numel * p.esize >= (int64_t(1) << 32)) return -1;
    struct Row { int id, T, NR; };
    static const Row tbl[] = {
#define IABN_ROW(ID, T, NR) {ID, T, NR},
        IABN_FUSED_SCALAR_VARIANTS(IABN_ROW)
#undef IABN_ROW
    };
    const int64_t bytes = p.numel * p.esize;
    for (const auto& v : tbl) {
        if (int64_t(v.T) * v.NR < p.m) continue;
        if (p.C * v.T >= int64_t(256) * 256 || bytes <= (int64_t(4) << 20)) return v.id;
        return -1;
    }
    return -1;
}

void launch_forward_fused_nchw(const Plan& pl, void* x, const float* gamma, const float* beta,
                               float* rm, float* rv, float* sm, float* si, float eps, float mom,
                               int act, float a, hipStream_t s);

void launch_backward_fused_nchw(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* invstd,
                                float* dgamma, float* dbeta, int act, float a, hipStream_t s);

void launch_forward_fused_scalar(const Plan& pl, void* x, const float* gamma, const float* beta,
                                 float* rm, float* rv, float* sm, float* si, float eps, float mom,
                                 int act, float a, hipStream_t s);

void launch_backward_fused_scalar(const Plan& pl, const void* y, const void* dy, void* dx,
                                  const float* gamma, const float* beta, const float* invstd,
                                  float* dgamma, float* dbeta, int act, float a, hipStream_t s);

void launch_forward_fused_nhwc(const Plan& pl, void* x, const float* gamma, const float* beta,
                               float* rm, float* rv, float* sm, float* si, float eps, float mom,
                               int act, float a, hipStream_t s);

void launch_backward_fused_nhwc(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* invstd,
                                float* dgamma, float* dbeta, int act, float a, hipStream_t s);

}  // namespace iabn

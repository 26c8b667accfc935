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
    X(9, 512, 2, 18)                 \
    X(10, 512, 4, 4)                 \
    X(11, 512, 4, 7)                 \
    X(12, 512, 4, 13)                \
    X(13, 512, 8, 7)                 \
    X(14, 512, 8, 13)
#endif

// Streamed slice kernels (NHWC maps too large to hold).  X(id, T, LPR, NRF, LF,
// UF, NRB, LB, UB): T threads, LPR lanes per row; the forward keeps NRF rows per
// thread in registers and the next LF in LDS, and streams the rest UF rows per
// thread at a time; the backward likewise with NRB, LB and UB (y and dy both).
// LF and LB are multiples of UF and UB; the LDS rows take 128 KB, beside up to
// 17 KB for the scatter and the two-level exchange.
#ifndef IABN_STREAM_NHWC_VARIANTS
#define IABN_STREAM_NHWC_VARIANTS(X)   \
    X(0, 512, 4, 28, 16, 4, 14, 8, 2)  \
    X(1, 512, 8, 28, 16, 4, 14, 8, 2)
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

// The largest group a forward variant may run in: variants holding more than 32
// vectors a thread compile only the one-level exchange (fused_nchw.hip,
// kFwdTwoLevel), so their groups stay under the two-level size of 16.
inline int fused_fwd_group_max(int id)
{
    switch (id) {
#define IABN_ROW(ID, T, NR) case ID: return NR > 32 ? 15 : 64;
        IABN_FUSED_FWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: return 0;
    }
}

inline bool fused_bwd_dy_resident(int id)
{
    switch (id) {
#define IABN_ROW(ID, T, NRV, NRL, G, DYR) case ID: return DYR;
        IABN_FUSED_BWD_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: return false;
    }
}

// Channels one workgroup cannot hold, or too few channels to fill the chip: G
// workgroups (members) share a channel, member j holding its vectors
// [j*ceil(vc/G), ...), and swap their fp64 sums through the workspace (the
// exchange of the NHWC groups, one channel a slice).  The largest power of two
// G (2 to 64) with C*G within max_grid (every member runs at once) whose share
// fits a forward and a y-resident, dy-streaming backward variant (and a group
// size the forward variant allows), if the grid then fills the chip (or the
// tensor is small).  Both passes use that G.
struct NchwGroupChoice {
    int fwd = -1, bwd = -1, group = 1;
};

inline NchwGroupChoice fused_nchw_group_pick(const Plan& p, int64_t max_grid)
{
    NchwGroupChoice none;
    if (p.layout != kNCHW || !p.vec || p.numel == 0) return none;
    const int64_t bytes = p.numel * p.esize;
    if (bytes >= (int64_t(1) << 32)) return none;
    const int64_t vc = p.m / p.V;
    for (int g = 64; g >= 2; g /= 2) {
        if (p.C * g > max_grid) continue;
        const int64_t share = ceil_div(vc, g);
        if ((g - 1) * share >= vc) continue;        // every member holds vectors
        const int f = fused_fwd_pick(share), b = fused_bwd_pick(share);
        if (f < 0 || b < 0 || fused_bwd_dy_resident(b) || g > fused_fwd_group_max(f)) continue;
        const int64_t threads = p.C * g * fused_fwd_threads(f);
        if (threads < int64_t(256) * 256 && bytes > (int64_t(4) << 20)) return none;
        NchwGroupChoice c;
        c.fwd = f;
        c.bwd = b;
        c.group = g;
        return c;
    }
    return none;
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

// Slice-resident NHWC plan: variant and group size (variant -1: not used).  A
// group of G > 1 workgroups shares one slice, each holding a contiguous block of
// ceil(m/G) rows; the members swap their partial sums through the workspace
// while all of them stay resident, so the grid must not exceed what the device
// runs at once (max_grid, one workgroup per CU; 0 forbids groups).
struct NhwcChoice {
    int variant = -1;
    int group = 1;
};

// Choice, from cold timings of every (variant, G) on ResNet-50 NHWC shapes:
//  0. A tensor under 4 MB: one lane per row and 256 threads, at most 2 (else 4)
//     rows per thread, the smallest group (up to 8) that holds the rows -- on so
//     little data the count of workgroups, each a CU's load pipeline, matters
//     most.
//  1. The widest LPR in the table (a wave reads LPR*16 contiguous bytes of each
//     row; one lane per row coalesces poorly): the smallest group (up to 32)
//     whose ceil(m/G) rows fit a variant of at most 4 rows per thread, else 8,
//     else 13 (more rows per thread lengthen each member's load -> reduce ->
//     store round trip more than extra members cost).  G = 1 here needs the chip
//     filled or a small tensor.
//  2. One workgroup per slice at any LPR, the chip filled (T*slices >= 256*256)
//     or a small tensor (under 4 MB with at most 4096 rows), where launch latency
//     rules.
// Groups need slices % 8 == 0 (a group's members on one XCD) and a grid within
// max_grid.  32-bit vector indices address the tensor.
inline NhwcChoice fused_nhwc_pick(const Plan& p, int64_t max_grid)
{
    NhwcChoice none;
    if (p.layout != kNHWC || !p.vec || p.numel == 0) return none;
    if (p.numel * p.esize >= (int64_t(1) << 32)) return none;
    const int64_t cv = p.C / p.V;
    const int64_t bytes = p.numel * p.esize;
    struct Row { int id, T, LPR, NR; };
    static const Row tbl[] = {
#define IABN_ROW(ID, T, LPR, NR) {ID, T, LPR, NR},
        IABN_FUSED_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
    };
    const bool small = bytes <= (int64_t(4) << 20) && p.m <= 4096;
    auto fills = [&](int64_t grid, int T) { return grid * T >= int64_t(256) * 256; };
    // the smallest variant of width lpr, at most nr_cap rows per thread, holding rows
    auto holding = [&](int lpr, int nr_cap, int64_t rows) -> const Row* {
        const Row* best = nullptr;
        for (const auto& v : tbl)
            if (v.LPR == lpr && v.NR <= nr_cap && int64_t(v.T / lpr) * v.NR >= rows &&
                (!best || int64_t(v.T) * v.NR < int64_t(best->T) * best->NR))
                best = &v;
        return best;
    };
    // a tensor under 4 MB: as many workgroups as possible, each thread holding at
    // most 2, else 4 rows (one lane per row, 256 threads), groups of at most 8
    if (bytes <= (int64_t(4) << 20)) {
        for (int nr_cap : {2, 4}) {
            for (int g = 1; g <= 8; g *= 2) {
                const int64_t grid = cv * g;
                const int64_t mg = ceil_div(p.m, g);
                if (g > 1 && (cv % 8 != 0 || grid > max_grid || (g - 1) * mg >= p.m)) break;
                const Row* v = holding(1, nr_cap, mg);
                if (v && v->T == 256) {
                    NhwcChoice c;
                    c.variant = v->id;
                    c.group = g;
                    return c;
                }
            }
        }
    }
    // Eight lanes per row (whole lines per workgroup) only with 7 or 13 rows a
    // thread and groups of at most 8: there the backward, whose four-lane stores
    // leave partial lines (1.38 S written), gains (64x2048x7x7 bf16: 14.3 against
    // 15.6 us; 128x2048x7x7: 21.8 against 27.5) and the forward holds even; with
    // 4 rows a thread or the two-level exchange of larger groups it lost (32x2048x7x7:
    // 10.9 against 10.3; 64x1024x7x7 in groups of 16: 13.6 against 10.8).
    // The smallest group of width lpr whose members hold their rows in variants of
    // at most nr_cap rows per thread (none: variant -1).
    auto grouped = [&](int lpr, int nr_cap) -> NhwcChoice {
        NhwcChoice c;
        if (cv % lpr != 0) return c;
        const int64_t slices = cv / lpr;
        const int gmax = lpr == 8 ? 8 : 32;
        for (int g = 1; g <= gmax; g *= 2) {
            const int64_t grid = slices * g;
            const int64_t mg = ceil_div(p.m, g);
            if (g > 1 && (slices % 8 != 0 || grid > max_grid || (g - 1) * mg >= p.m)) break;
            const Row* v = holding(lpr, nr_cap, mg);
            if (v && (g > 1 || fills(grid, v->T) || small)) {
                c.variant = v->id;
                c.group = g;
                return c;
            }
        }
        return c;
    };
    for (int nr_cap : {4, 8, 13}) {
        for (int lpr : {8, 4, 2}) {
            NhwcChoice c = grouped(lpr, nr_cap);
            if (c.variant < 0) continue;
            // At most 4 rows a thread, where four lanes need the two-level exchange
            // (groups of 16 or more members), two lanes in a smaller group are faster
            // (8x512x28x28 bf16: 19.6 against 22.5 us a step in groups of 8 against
            // 16; 64x256x14x14: 21.5 against 23.5 in 16 against 32).  With more rows
            // a thread the two-lane backward, whose stores leave quarter lines,
            // loses (32x512x28x28 at 13 rows: 48.7 against 42.8).
            if (lpr == 4 && nr_cap == 4 && c.group >= 16) {
                const NhwcChoice c2 = grouped(2, nr_cap);
                if (c2.variant >= 0 && c2.group < c.group) return c2;
            }
            return c;
        }
    }
    for (int lpr : {2, 1}) {
        if (cv % lpr != 0) continue;
        const Row* v = holding(lpr, 1 << 30, p.m);
        if (v && (fills(cv / lpr, v->T) || small)) {
            NhwcChoice c;
            c.variant = v->id;
            return c;
        }
    }
    return none;
}

// Streamed slice plan for an NHWC map (variant -1: not used): eight lanes per row
// (each workgroup writes whole 128-byte lines: the 2x256x512x512 forward went from
// 138 to 128 us), else four (two lost to the split path on 64-channel 112x112
// maps), whose slices, in groups of a power of two from 8 to 64, make a grid of
// exactly max_grid workgroups (every CU streams), every member getting rows.
// Taken where the resident kernels cannot hold the rows.
inline NhwcChoice fused_stream_pick(const Plan& p, int64_t max_grid)
{
    NhwcChoice none;
    if (p.layout != kNHWC || !p.vec || p.numel == 0) return none;
    if (p.numel * p.esize >= (int64_t(1) << 32)) return none;
    const int64_t cv = p.C / p.V;
    struct Row { int id, T, LPR; };
    static const Row tbl[] = {
#define IABN_ROW(ID, T, LPR, NRF, LF, UF, NRB, LB, UB) {ID, T, LPR},
        IABN_STREAM_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
    };
    for (int lpr : {8, 4}) {
        if (cv % lpr != 0) continue;
        const int64_t slices = cv / lpr;
        int g = 64;
        while (g >= 8 && slices * g > max_grid) g /= 2;
        if (g < 8 || slices * g != max_grid || (g - 1) * ceil_div(p.m, g) >= p.m) continue;
        for (const auto& v : tbl) {
            if (v.LPR != lpr) continue;
            NhwcChoice c;
            c.variant = v.id;
            c.group = g;
            return c;
        }
    }
    return none;
}

// Whether the streamed backward beats the split one: measured so where at least
// half of each thread's rows stay on chip (y and dy both held, in registers or
// LDS); with fewer, re-reading two streams at this kernel's occupancy loses to
// the split kernels (2x256x512x512 bf16, 17% of the rows held: 245.9 against
// 239.2 us for the backward, though it moves 4.66 S against 5 S).
inline bool stream_bwd_worthwhile(const Plan& p, int variant, int group)
{
    switch (variant) {
#define IABN_ROW(ID, T, LPR, NRF, LF, UF, NRB, LB, UB) \
    case ID: return ceil_div(ceil_div(p.m, group), T / LPR) <= 2 * (NRB + LB);
        IABN_STREAM_NHWC_VARIANTS(IABN_ROW)
#undef IABN_ROW
    default: return false;
    }
}

// Workspace words of the group exchange: one epoch per slice (padded to 32
// words), then per slice, member and channel four tagged words.
inline int64_t nhwc_exchange_words(int64_t slices, int64_t group, int64_t C)
{
    return group > 1 ? align_up(slices, 32) + 4 * group * C : 0;
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
                               int act, float a, void* ws, hipStream_t s);

void launch_backward_fused_nchw(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* invstd,
                                float* dgamma, float* dbeta, int act, float a, void* ws,
                                hipStream_t s);

void launch_forward_fused_scalar(const Plan& pl, void* x, const float* gamma, const float* beta,
                                 float* rm, float* rv, float* sm, float* si, float eps, float mom,
                                 int act, float a, hipStream_t s);

void launch_backward_fused_scalar(const Plan& pl, const void* y, const void* dy, void* dx,
                                  const float* gamma, const float* beta, const float* invstd,
                                  float* dgamma, float* dbeta, int act, float a, hipStream_t s);

void launch_forward_fused_nhwc(const Plan& pl, void* x, const float* gamma, const float* beta,
                               float* rm, float* rv, float* sm, float* si, float eps, float mom,
                               int act, float a, void* ws, hipStream_t s);

void launch_backward_fused_nhwc(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* invstd,
                                float* dgamma, float* dbeta, int act, float a, void* ws,
                                hipStream_t s);

void launch_forward_stream_nhwc(const Plan& pl, void* x, const float* gamma, const float* beta,
                                float* rm, float* rv, float* sm, float* si, float eps, float mom,
                                int act, float a, void* ws, hipStream_t s);

void launch_backward_stream_nhwc(const Plan& pl, const void* y, const void* dy, void* dx,
                                 const float* gamma, const float* beta, const float* invstd,
                                 float* dgamma, float* dbeta, int act, float a, void* ws,
                                 hipStream_t s);

}  // namespace iabn

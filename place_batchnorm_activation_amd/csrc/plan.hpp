// Tiling plan for the In-Place ABN kernels (host side).
//
// A plan depends only on the shape, layout, dtype, whether the 128-bit vector
// path applies and (the slice-resident NHWC groups) the device's CU count, so a
// given problem always reduces in the same order on a given device and the
// results are bitwise reproducible.
//
// Reduction tiling (forward statistics and backward sums).  Every channel's m
// elements are cut into P "partials":
//   NCHW: the channel-local index j = n*HW + hw is cut into runs of `unit`
//         elements (the last one ragged); one workgroup per (channel, partial):
//         grid = C * P.
//   NHWC: the C channels are cut into `slices` of `tpr` vectors (tpr threads per
//         row, rpi = 256/tpr rows per step), the m rows into row groups of rpi
//         rows; workgroup (slice, p) takes row groups p, p + P, p + 2P, ...:
//         grid = slices * P, slice index fastest.
// Each workgroup writes one partial per channel it covers, partial-major
// (index p*C + c), and its element count; a finishing kernel combines the P
// partials of a channel in a fixed order.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace iabn {

constexpr int kThreads = 256;          // workgroup size of every kernel
constexpr int kWave = 64;              // CDNA wavefront
// finishing kernels: 1024 threads = kFinChannels channels x kFinPhases phases
constexpr int kFinThreads = 1024;
constexpr int kFinChannels = 16;
constexpr int kFinPhases = kFinThreads / kFinChannels;

enum Layout { kNCHW = 0, kNHWC = 1 };
enum DType { kF32 = 0, kBF16 = 1, kF16 = 2 };
enum Act { kIdentity = 0, kLeaky = 1, kElu = 2 };

// Host-side dispatch onto compile-time storage dtype and activation: calls f with
// std::integral_constant<int, value>, so a launcher names its kernel template
// once for every combination.
template <class F>
inline void with_dtype(int dtype, F&& f)
{
    switch (dtype) {
    case kF32: f(std::integral_constant<int, kF32>{}); break;
    case kBF16: f(std::integral_constant<int, kBF16>{}); break;
    case kF16: f(std::integral_constant<int, kF16>{}); break;
    default: break;
    }
}

template <class F>
inline void with_act(int act, F&& f)
{
    switch (act) {
    case kLeaky: f(std::integral_constant<int, kLeaky>{}); break;
    case kElu: f(std::integral_constant<int, kElu>{}); break;
    default: f(std::integral_constant<int, kIdentity>{}); break;
    }
}

// Elements per 16-byte access.
constexpr int vec_width(int dtype) { return dtype == kF32 ? 4 : 8; }

// Every workspace starts with a header of this many bytes.  Its first 8 bytes
// are the exchange status word: a group member whose bounded wait for a partner
// runs out stores kExchangeTimeout there (group.hpp), and the word keeps it
// until the caller clears it (iabn_workspace_status).
constexpr size_t kWsHeaderBytes = 256;
constexpr uint64_t kExchangeTimeout = 0x69616E6254494D45ull;   // any other value: none

struct Plan {
    int64_t N = 0, C = 0, HW = 0, m = 0, numel = 0;
    int layout = 0, dtype = 0, esize = 4;
    bool vec = false;    // 128-bit accesses
    int V = 1;           // elements per access
    // reduction tiling
    int64_t P = 1;       // partials per channel
    int64_t unit = 1;    // NCHW: channel-local elements per partial; NHWC: row groups
    int tpr = 1;         // NHWC: threads per row
    int64_t slices = 1;  // NHWC: channel slices
    int64_t reduce_blocks = 0;
    // the backward's reduction (NHWC: its own, smaller grid; NCHW: P, reduce_blocks)
    int64_t P_bwd = 1;
    int64_t reduce_blocks_bwd = 0;
    // elementwise tiling
    int64_t apply_blocks = 0;
    int64_t apply_blocks_elu = 0;   // the same grid for ELU (more arithmetic to hide)
    bool fixed_col = false;  // NHWC: each thread keeps one channel group for the whole walk
    // channel-resident NCHW kernels (-1: not used for this problem)
    int fused_variant = -1;
    int fused_bwd_variant = -1;
    // workgroups per channel of those kernels (channels one workgroup cannot
    // hold); their exchange sits at off_xchg like the NHWC groups'
    int nchw_group = 1;
    // slice-resident NHWC kernels (-1: not used), workgroups per slice, and the
    // workspace section of their exchange (groups only)
    int nhwc_variant = -1;
    int nhwc_group = 1;
    size_t off_xchg = 0;
    // streamed slice kernels, forward and backward (-1: not used; the backward
    // then takes the split path); their group size is nhwc_group
    int stream_variant = -1;
    int stream_bwd_variant = -1;
    // whether the training forward of this shape takes the streamed slice kernel
    // (set also in plans made without an activation, which never take it: the
    // split backward's walk order follows it)
    bool fwd_streamed = false;
    // channel-resident NCHW kernels on single elements (-1: not used)
    int scalar_variant = -1;
    // workspace sections (bytes, 256-aligned)
    size_t off_part_a = 0, off_part_b = 0, off_const = kWsHeaderBytes, off_count = 0, bytes = 0;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The elementwise grid for an activation.
inline int64_t apply_grid(const Plan& p, int act)
{
    return act == kElu ? p.apply_blocks_elu : p.apply_blocks;
}
inline int64_t align_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
inline int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

inline int64_t gcd64(int64_t a, int64_t b)
{
    while (b) { const int64_t t = a % b; a = b; b = t; }
    return a;
}

// Walk order of the NHWC split backward, chosen by measuring the step (the
// forward, then the backward on the same tensor): where the forward of the same
// shape is the streamed slice kernel, the sums pass walks the tensor from the end
// down and the dx pass from the start up; otherwise the sums walk up and the dx
// pass down.  Either way the dx pass starts on the rows the sums read last (the
// likeliest still to sit in the Infinity Cache).  Measured, fwd + bwd, cold:
// 2x256x512x512 bf16 (streamed forward) 373.8 -> 385.9 Gelem/s with the sums
// walking down; 32x64x112x112 bf16 (split forward) 82.0 -> 79.0 us with them
// walking up.
inline bool bwd_sums_from_end(const Plan& p) { return p.layout == kNHWC && p.fwd_streamed; }

// The NHWC backward dx pass after a streamed forward (the order above): one
// workgroup per CU streamed faster than two on the maps that take it
// (2x256x512x512, fwd + bwd, cold: bf16 383.4 -> 387.5 Gelem/s, dx pass 137.3 ->
// 130.9 us; f16 380.6 -> 386.3; f32 156.6 -> 168.4), while the split path's other
// elementwise passes keep two per CU (with one, the ResNet-50 NCHW split steps
// were 1-10% slower).  ELU keeps its wider grid.
#ifndef IABN_DX_BLOCKS_STREAMED
#define IABN_DX_BLOCKS_STREAMED 256
#endif
constexpr int64_t kDxBlocksStreamed = IABN_DX_BLOCKS_STREAMED;
inline int64_t dx_grid(const Plan& p, int act)
{
    const int64_t g = apply_grid(p, act);
    if (act == kElu || !bwd_sums_from_end(p) || !p.fixed_col || kDxBlocksStreamed >= g) return g;
    const int64_t cv = p.C / p.V;
    const int64_t need = cv / gcd64(cv, kThreads);  // keeps each thread on one channel group
    return kDxBlocksStreamed % need == 0 ? kDxBlocksStreamed : g;
}

// Workgroups an elementwise kernel launches at most.  Two per CU for leaky ReLU
// and identity: like the reductions, the elementwise passes stream faster with a
// narrower window of addresses in flight (the split path's steps on ResNet-50
// shapes, summed: 1366 us at 512 workgroups, 1413 at 1024, 1452 at 2048).  ELU's
// transcendentals need more waves to hide them (bf16 NHWC dx pass on
// 2x256x512x512: 164 us at 2048 workgroups, 185 at 512), so it keeps 2048.
#ifndef IABN_APPLY_BLOCKS_MAX
#define IABN_APPLY_BLOCKS_MAX 512
#endif
#ifndef IABN_APPLY_BLOCKS_MAX_ELU
#define IABN_APPLY_BLOCKS_MAX_ELU 2048
#endif
constexpr int64_t kApplyBlocksMax = IABN_APPLY_BLOCKS_MAX;
constexpr int64_t kApplyBlocksMaxElu = IABN_APPLY_BLOCKS_MAX_ELU;
// Workgroups a reduction aims for.
#ifndef IABN_REDUCE_BLOCKS_TARGET
#define IABN_REDUCE_BLOCKS_TARGET 2048
#endif
constexpr int64_t kReduceBlocksTarget = IABN_REDUCE_BLOCKS_TARGET;
// NHWC reductions: long-lived workgroups walking row groups with a stride, one
// per CU, each with a few row groups in flight per pipeline stage.  A narrower
// window of addresses in flight streams faster than two workgroups per CU or
// deeper stages (2x256x512x512 bf16, cold: statistics 57 against 62 us at 512
// workgroups; backward sums 104.5 against 115 at 512 x 8 row groups).  The
// statistics (P) and the backward sums (P_bwd) have a grid each.
#ifndef IABN_NHWC_REDUCE_BLOCKS
#define IABN_NHWC_REDUCE_BLOCKS 256
#endif
constexpr int64_t kNhwcReduceBlocks = IABN_NHWC_REDUCE_BLOCKS;
#ifndef IABN_NHWC_BWD_REDUCE_BLOCKS
#define IABN_NHWC_BWD_REDUCE_BLOCKS 256
#endif
constexpr int64_t kNhwcBwdReduceBlocks = IABN_NHWC_BWD_REDUCE_BLOCKS;

inline Plan make_plan(int64_t N, int64_t C, int64_t H, int64_t W, int layout, int dtype, bool vec)
{
    Plan p;
    p.N = N; p.C = C; p.HW = H * W; p.m = N * p.HW; p.numel = p.m * C;
    p.layout = layout; p.dtype = dtype;
    p.esize = dtype == kF32 ? 4 : 2;
    p.vec = vec;
    p.V = vec ? 16 / p.esize : 1;
    if (p.numel == 0) return p;
    const int V = p.V;

    if (layout == kNCHW) {
        // vectors never straddle planes: HW % V == 0 on the vector path
        const int64_t vc = p.m / V;                          // vectors per channel
        const int64_t want = ceil_div(kReduceBlocksTarget, C);
        const int64_t cap = max64(1, ceil_div(vc, 2 * kThreads));  // >= ~2 vectors per thread
        int64_t P = max64(1, min64(want, cap));
        p.unit = ceil_div(vc, P) * V;
        p.P = ceil_div(p.m, p.unit);
        p.reduce_blocks = C * p.P;
        p.P_bwd = p.P;
        p.reduce_blocks_bwd = p.reduce_blocks;
    } else {
        const int64_t cv = C / V;                            // vectors per row
        // partial traffic (8 B per channel and partial) kept to ~2% of the data
        const int64_t p_budget = max64(1, (p.m * p.esize) / 400);
        int tpr = 1;
        while (tpr < cv && tpr < kThreads) tpr <<= 1;
        auto groups = [&](int t) { return ceil_div(p.m, int64_t(kThreads / t)); };
        auto choose_P = [&](int t) {
            const int64_t p_iter = max64(1, groups(t) / 4);  // >= ~4 row groups per workgroup
            return max64(1, min64(p_budget, p_iter));
        };
        int64_t slices = ceil_div(cv, tpr);
        int64_t P = choose_P(tpr);
        // narrower slices (down to 4 lanes, 64 bytes per row segment) while short of work
        while (slices * P < kNhwcReduceBlocks / 2 && tpr > 4) {
            tpr >>= 1;
            slices = ceil_div(cv, tpr);
            P = choose_P(tpr);
        }
        const int64_t P_bwd = min64(P, max64(1, ceil_div(kNhwcBwdReduceBlocks, slices)));
        P = min64(P, max64(1, ceil_div(kNhwcReduceBlocks, slices)));
        p.tpr = tpr;
        p.slices = slices;
        p.unit = groups(tpr);                               // row groups in all
        p.P = min64(P, p.unit);
        p.reduce_blocks = slices * p.P;
        p.P_bwd = min64(P_bwd, p.unit);
        p.reduce_blocks_bwd = slices * p.P_bwd;
    }

    const int64_t nvec = p.numel / V;
    p.apply_blocks = max64(1, min64(kApplyBlocksMax, ceil_div(nvec, kThreads)));
    p.apply_blocks_elu = max64(1, min64(kApplyBlocksMaxElu, ceil_div(nvec, kThreads)));
    if (layout == kNHWC) {
        // keep each thread on one channel group: stride (blocks*256) % (C/V) == 0
        const int64_t cv = C / V;
        const int64_t need = cv / gcd64(cv, kThreads);      // blocks must be a multiple of this
        if (need <= min64(kApplyBlocksMax, kApplyBlocksMaxElu)) {
            p.apply_blocks = max64(need, (p.apply_blocks / need) * need);
            p.apply_blocks_elu = max64(need, (p.apply_blocks_elu / need) * need);
            p.fixed_col = true;
        }
    }

    // The header comes first (the exchange status word), then the constants, at
    // offsets that do not depend on the plan, so that a stage planned for the
    // vector path and one planned for the scalar path (different pointer
    // alignment) agree on where they are.
    size_t off = kWsHeaderBytes;
    const size_t part_bytes = (size_t)(max64(p.P, p.P_bwd) * C) * sizeof(float);
    p.off_const = off;  off = (size_t)align_up((int64_t)(off + (size_t)C * 16), 256);
    p.off_part_a = off; off = (size_t)align_up((int64_t)(off + part_bytes), 256);
    p.off_part_b = off; off = (size_t)align_up((int64_t)(off + part_bytes), 256);
    p.off_count = off;  off = (size_t)align_up((int64_t)(off + (size_t)p.P * sizeof(float)), 256);
    p.bytes = off;
    return p;
}

// Whether the 128-bit path applies to this shape (pointer alignment is checked apart).
inline bool vec_shape_ok(int64_t C, int64_t HW, int layout, int dtype)
{
    const int V = 16 / (dtype == kF32 ? 4 : 2);
    return layout == kNCHW ? (HW % V == 0) : (C % V == 0);
}

}  // namespace iabn

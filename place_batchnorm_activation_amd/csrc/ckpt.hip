// Optimized checkpointing (section 3 of the paperlayer summary of "In-Place
// Activated BatchNorm for Memory-Optimized Training of DNNs", "Proposed
// Checkpointing"): the block keeps the normalised xhat instead of its input x.
// The layer output y is rebuilt as act(gamma*xhat + beta) when the following
// layer's backward needs it, and the BN backward reads xhat itself instead of
// recomputing it.  This is the method the pages compare InPlace-ABN II against.
//
// The statistics and the backward sums run the split path's kernels (fwd.hip;
// bwd.hip with its xhat decode).  The elementwise passes that differ are here:
//   kCkptFwd       xhat = ((x - K) - d)*invstd rounded to the storage dtype and
//                  written over x, and y = act(fmaf(gamma, xhat, beta)) from
//                  that rounded xhat into its own buffer, so that y has the bits
//                  the recompute gives later;
//   kCkptRecompute y = act(fmaf(gamma, xhat, beta));
//   kCkptDx        z = fmaf(gamma, xhat, beta), dz = act'(z)*dy,
//                  dx = A*dz + B*xhat + Cc, with A = gamma*invstd,
//                  B = -A*dgamma/m, Cc = -A*dbeta/m.
// z is one fused multiply-add of binary32 operands, so its sign, which picks the
// activation's branch, is that of the exact gamma*xhat + beta.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace iabn {

namespace {

enum CkptMode { kCkptFwd = 0, kCkptRecompute = 1, kCkptDx = 2 };

struct CkptArgs {
    const float4* consts;   // kCkptFwd: {K, d, s, beta}; kCkptDx: {A, B, Cc, beta}
    const float* gamma;
    const float* beta;
    const float* invstd;    // kCkptFwd only
};

// A channel's values: kCkptFwd {K, d, invstd}, kCkptDx {A, B, Cc}, and gamma, beta.
struct CkptChan {
    float k0, k1, k2, g, b;
};

template <int MODE>
__device__ __forceinline__ CkptChan ckpt_chan(const CkptArgs& ar, int64_t c)
{
    CkptChan k;
    k.g = ar.gamma[c];
    k.b = ar.beta[c];
    k.k0 = k.k1 = k.k2 = 0.f;
    if constexpr (MODE == kCkptFwd) {
        const float4 q = ar.consts[c];
        k.k0 = q.x;
        k.k1 = q.y;
        k.k2 = ar.invstd[c];
    } else if constexpr (MODE == kCkptDx) {
        const float4 q = ar.consts[c];
        k.k0 = q.x;
        k.k1 = q.y;
        k.k2 = q.z;
    }
    return k;
}

// A value as stored in dtype DT and read back.
template <int DT>
__device__ __forceinline__ float as_stored(float v)
{
    if constexpr (DT == kF32) return v;
    else return unpack1<DT>(pack1<DT>(v));
}

// One vector of V elements at element index i; v0 holds in0's values (and v1
// in1's for kCkptDx), loaded by the caller.
template <int DT, int V, int ACT, int MODE>
__device__ __forceinline__ void ckpt_vec(float (&v0)[V], const float (&v1)[V], void* out0,
                                         void* out1, int64_t i, const CkptChan (&k)[V], float a)
{
    if constexpr (MODE == kCkptFwd) {
        // xhat is rounded once, and those values are both stored (exactly: they
        // are representable) and used for y.  The fp32 product goes through an
        // empty asm first: without it the compiler rounded the product to fp16 in
        // one instruction (v_fma_mix, one rounding) for y but through fp32 (two
        // roundings) for the store, and the two could differ in the last bit.
        float y[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float p = ((v0[e] - k[e].k0) - k[e].k1) * k[e].k2;
            asm volatile("" : "+v"(p));
            v0[e] = as_stored<DT>(p);
            y[e] = act_forward<ACT, DT == kF32>(fmaf(k[e].g, v0[e], k[e].b), a);
        }
        store_out<DT, V>(out0, i, v0);
        store_out<DT, V>(out1, i, y);
    } else if constexpr (MODE == kCkptRecompute) {
#pragma unroll
        for (int e = 0; e < V; ++e) v0[e] = act_forward<ACT, DT == kF32>(fmaf(k[e].g, v0[e], k[e].b), a);
        store_out<DT, V>(out0, i, v0);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float dz = act_slope_at<ACT>(fmaf(k[e].g, v0[e], k[e].b), a) * v1[e];
            v0[e] = fmaf(k[e].k0, dz, fmaf(k[e].k1, v0[e], k[e].k2));
        }
        store_out<DT, V>(out0, i, v0);
    }
}

constexpr int kUnrollC = 4;

// NCHW: grid-stride over 16-byte vectors (or single elements), the channel of
// each tracked by a carry walk.  in1 is read only for kCkptDx.
template <int DT, int V, int ACT, int MODE>
__global__ __launch_bounds__(kThreads) void k_ckpt_nchw(
    const void* in0, const void* in1, void* out0, void* out1, int64_t nvec, int64_t C,
    int64_t HWv, CkptArgs ar, float a)
{
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    FlatNCHWWalk w;
    w.init(v < nvec ? v : 0, C, HWv, stride);
    for (; v + (kUnrollC - 1) * stride < nvec; v += kUnrollC * stride) {
        float x0[kUnrollC][V], x1[kUnrollC][V];
        CkptChan k[kUnrollC][V];
#pragma unroll
        for (int u = 0; u < kUnrollC; ++u) {
            load_elems<DT, V>(in0, (v + u * stride) * V, x0[u]);
            if constexpr (MODE == kCkptDx) load_elems<DT, V>(in1, (v + u * stride) * V, x1[u]);
            const CkptChan kc = ckpt_chan<MODE>(ar, w.c);
#pragma unroll
            for (int e = 0; e < V; ++e) k[u][e] = kc;
            w.step();
        }
#pragma unroll
        for (int u = 0; u < kUnrollC; ++u)
            ckpt_vec<DT, V, ACT, MODE>(x0[u], x1[u], out0, out1, (v + u * stride) * V, k[u], a);
    }
    for (; v < nvec; v += stride) {
        float x0[V], x1[V];
        CkptChan k[V];
        load_elems<DT, V>(in0, v * V, x0);
        if constexpr (MODE == kCkptDx) load_elems<DT, V>(in1, v * V, x1);
        const CkptChan kc = ckpt_chan<MODE>(ar, w.c);
#pragma unroll
        for (int e = 0; e < V; ++e) k[e] = kc;
        w.step();
        ckpt_vec<DT, V, ACT, MODE>(x0, x1, out0, out1, v * V, k, a);
    }
}

// NHWC: vector v covers channels (v % Cv)*V .. +V.  With FIXED the stride is a
// multiple of Cv and each thread loads its V channels' values once.
template <int DT, int V, int ACT, int MODE, bool FIXED>
__global__ __launch_bounds__(kThreads) void k_ckpt_nhwc(
    const void* in0, const void* in1, void* out0, void* out1, int64_t nvec, int64_t Cv,
    CkptArgs ar, float a)
{
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if constexpr (FIXED) {
        if (v >= nvec) return;
        const int64_t c0 = (v % Cv) * V;
        CkptChan k[V];
#pragma unroll
        for (int e = 0; e < V; ++e) k[e] = ckpt_chan<MODE>(ar, c0 + e);
        for (; v + (kUnrollC - 1) * stride < nvec; v += kUnrollC * stride) {
            float x0[kUnrollC][V], x1[kUnrollC][V];
#pragma unroll
            for (int u = 0; u < kUnrollC; ++u) {
                load_elems<DT, V>(in0, (v + u * stride) * V, x0[u]);
                if constexpr (MODE == kCkptDx) load_elems<DT, V>(in1, (v + u * stride) * V, x1[u]);
            }
#pragma unroll
            for (int u = 0; u < kUnrollC; ++u)
                ckpt_vec<DT, V, ACT, MODE>(x0[u], x1[u], out0, out1, (v + u * stride) * V, k, a);
        }
        for (; v < nvec; v += stride) {
            float x0[V], x1[V];
            load_elems<DT, V>(in0, v * V, x0);
            if constexpr (MODE == kCkptDx) load_elems<DT, V>(in1, v * V, x1);
            ckpt_vec<DT, V, ACT, MODE>(x0, x1, out0, out1, v * V, k, a);
        }
    } else {
        for (; v < nvec; v += stride) {
            const int64_t c0 = (v % Cv) * V;
            CkptChan k[V];
#pragma unroll
            for (int e = 0; e < V; ++e) k[e] = ckpt_chan<MODE>(ar, c0 + e);
            float x0[V], x1[V];
            load_elems<DT, V>(in0, v * V, x0);
            if constexpr (MODE == kCkptDx) load_elems<DT, V>(in1, v * V, x1);
            ckpt_vec<DT, V, ACT, MODE>(x0, x1, out0, out1, v * V, k, a);
        }
    }
}

template <int MODE>
void launch_ckpt(const Plan& pl, const void* in0, const void* in1, void* out0, void* out1,
                 const CkptArgs& ar, int act, float a, hipStream_t s)
{
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            constexpr int DT = decltype(d)::value, ACT = decltype(ac)::value;
            auto go = [&](auto vv) {
                constexpr int V = decltype(vv)::value;
                const int64_t nvec = pl.numel / V;
                const dim3 grid(unsigned(apply_grid(pl, ACT)));
                if (pl.layout == kNCHW)
                    hipLaunchKernelGGL((k_ckpt_nchw<DT, V, ACT, MODE>), grid, dim3(kThreads), 0, s,
                                       in0, in1, out0, out1, nvec, pl.C, pl.HW / V, ar, a);
                else if (pl.fixed_col)
                    hipLaunchKernelGGL((k_ckpt_nhwc<DT, V, ACT, MODE, true>), grid, dim3(kThreads),
                                       0, s, in0, in1, out0, out1, nvec, pl.C / V, ar, a);
                else
                    hipLaunchKernelGGL((k_ckpt_nhwc<DT, V, ACT, MODE, false>), grid,
                                       dim3(kThreads), 0, s, in0, in1, out0, out1, nvec, pl.C / V,
                                       ar, a);
            };
            if (pl.vec) go(std::integral_constant<int, vec_width(DT)>{});
            else go(std::integral_constant<int, 1>{});
        });
    });
}

}  // namespace

// ---------------------------------------------------------------------------
// host launchers

void launch_ckpt_forward_apply(const Plan& pl, void* x, void* y, const float* gamma,
                               const float* beta, const float* invstd, int act, float a, void* ws,
                               hipStream_t s)
{
    const CkptArgs ar{reinterpret_cast<const float4*>(static_cast<char*>(ws) + pl.off_const),
                      gamma, beta, invstd};
    launch_ckpt<kCkptFwd>(pl, x, nullptr, x, y, ar, act, a, s);
}

void launch_ckpt_recompute(const Plan& pl, const void* xhat, void* y, const float* gamma,
                           const float* beta, int act, float a, hipStream_t s)
{
    const CkptArgs ar{nullptr, gamma, beta, nullptr};
    launch_ckpt<kCkptRecompute>(pl, xhat, nullptr, y, nullptr, ar, act, a, s);
}

void launch_ckpt_dx(const Plan& pl, const void* xhat, const void* dy, void* dx,
                    const float* gamma, const float* beta, int act, float a, void* ws,
                    hipStream_t s)
{
    const CkptArgs ar{reinterpret_cast<const float4*>(static_cast<char*>(ws) + pl.off_const),
                      gamma, beta, nullptr};
    launch_ckpt<kCkptDx>(pl, xhat, dy, dx, nullptr, ar, act, a, s);
}

}  // namespace iabn

// Backward kernels of In-Place Activated BatchNorm: everything from the stored
// output y (section 3 of the paperlayer summary of "In-Place Activated BatchNorm
// for Memory-Optimized Training of DNNs", "INPLACE-ABN" I and II, and the
// Appendix on rebuilding the discarded buffers during the backward pass).
//
// Per element, in registers: z = act^-1(y), dz = act'(z)*dy (both read off y),
// and t = z - beta_c, so that xhat = t/gamma_c.
//
// Three launches:
//   bwd_reduce_*  one workgroup per (channel tile, partial): sums of dz and dz*t
//   bwd_finalize  16 channels x 64 phases per workgroup, fixed-order fp64 sums:
//                 dbeta = sum dz, dgamma = (sum dz*t)/gamma, and the constants
//                 {A = gamma*invstd, B = -A*dgamma/(m*gamma), Cc = -A*dbeta/m, beta}
//   bwd_apply     dx = A*dz + B*(z - beta) + Cc
//                    = gamma*invstd*(dz - dbeta/m - xhat*dgamma/m)
// The affine recovery is thus folded into O(1) per-channel constants (form II),
// while the reductions keep the centred t = z - beta of form I so that a large
// |beta/gamma| does not cancel.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace iabn {

#ifndef IABN_REDUCE_UNROLL
#define IABN_REDUCE_UNROLL 4
#endif
constexpr int kUnrollB = IABN_REDUCE_UNROLL;
// NHWC reduction: row groups of y and dy in flight per thread, per pipeline stage.
// Fewer distinct addresses in flight stream faster, down to two: with one
// workgroup per CU, 4 had run faster than 8; after the streamed forward whose
// rows are dealt interleaved, the 2x256x512x512 bf16 step (sums walking down)
// took 371.5, 397.9-398.4, 389.9 and 391.0 Gelem/s at 1, 2, 3 and 4 (the sums
// pass 123.5, 99.6, 103.7 and 104.3 us a call); the ResNet-50 NHWC split steps
// were unchanged or up to 3% faster at 2.
#ifndef IABN_NHWC_REDUCE_UNROLL
#define IABN_NHWC_REDUCE_UNROLL 2
#endif
constexpr int kUnrollN = IABN_NHWC_REDUCE_UNROLL;

// XH: the stored value is xhat (optimized checkpointing) instead of y.  Its
// decode gives the slope at z = fmaf(gamma, xhat, beta) and t = xhat, so the
// sums become dbeta = sum dz and dgamma = sum dz*t directly (k_bwd_finalize with
// xhat_sums).
template <int ACT, bool XH, bool P>
__device__ __forceinline__ void decode(float v, float g, float b, float a, float inv_a, float& t,
                                       float& slope)
{
    if constexpr (XH) {
        slope = act_slope_at<ACT>(fmaf(g, v, b), a);
        t = v;
    } else {
        float z;
        act_invert<ACT, P>(v, a, inv_a, z, slope);
        t = z - b;
    }
}

template <int ACT, int V, bool XH, bool P>
__device__ __forceinline__ void accumulate(const float (&y)[V], const float (&dy)[V],
                                           const float (&beta)[V], const float (&gam)[V], float a,
                                           float inv_a, float (&sdz)[V], float (&sdzt)[V])
{
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float t, slope;
        decode<ACT, XH, P>(y[e], gam[e], beta[e], a, inv_a, t, slope);
        const float dz = slope * dy[e];
        sdz[e] += dz;
        sdzt[e] = fmaf(dz, t, sdzt[e]);
    }
}

// The same sums, and dx = A*dz written over dy's values (the backward with frozen
// statistics, where dx needs no reduction: A = gamma/sqrt(running_var + eps)).
template <int ACT, int V, bool P>
__device__ __forceinline__ void accumulate_dx(const float (&y)[V], float (&dy)[V],
                                              const float (&beta)[V], const float (&A)[V],
                                              float a, float inv_a, float (&sdz)[V],
                                              float (&sdzt)[V])
{
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float z, slope;
        act_invert<ACT, P>(y[e], a, inv_a, z, slope);
        const float dz = slope * dy[e];
        sdz[e] += dz;
        sdzt[e] = fmaf(dz, z - beta[e], sdzt[e]);
        dy[e] = A[e] * dz;
    }
}

// A = gamma/sqrt(running_var + eps) in fp64, rounded once.
__device__ __forceinline__ float frozen_scale(const float* gamma, const float* var, float eps,
                                              int64_t c)
{
    return float(double(gamma[c]) / sqrt(double(var[c]) + double(eps)));
}

// ---------------------------------------------------------------------------
// NCHW: workgroup b covers channel c = b / P, partial p = b % P.
// DX: also writes dx for the backward with frozen statistics (each element of dy
// is read by the thread that then writes the same element of dx, so dx may be dy).
// XH: y holds xhat (optimized checkpointing; not with DX).
template <int DT, int V, int ACT, bool DX, bool XH = false>
__global__ __launch_bounds__(kThreads) void k_bwd_reduce_nchw(
    const void* __restrict__ y, const void* dy, int64_t C, int64_t HW, int64_t m,
    int64_t unit, int64_t P, const float* __restrict__ beta, float a, float inv_a,
    float* __restrict__ part_dz, float* __restrict__ part_dzt, void* dx,
    const float* __restrict__ gamma, const float* __restrict__ frozen_var, float eps)
{
    static_assert(!(DX && XH), "the frozen-statistics pass reads y");
    const int64_t b = blockIdx.x;
    const int64_t c = b / P;
    const int64_t p = b - c * P;
    const int64_t HWv = HW / V;
    const int64_t j1 = dmin(p * unit + unit, m) / V;
    int64_t j = p * unit / V + threadIdx.x;

    float bc[V], gc[V], sdz[V], sdzt[V], A[V];
    const float bb = beta[c];
    const float gg = XH ? gamma[c] : 0.f;
    const float Ac = DX ? frozen_scale(gamma, frozen_var, eps, c) : 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) {
        bc[e] = bb;
        gc[e] = gg;
        A[e] = Ac;
        sdz[e] = 0.f;
        sdzt[e] = 0.f;
    }

    ChannelWalk w;
    w.init(j < j1 ? j : 0, c, C, HWv, kThreads);
    for (; j + (kUnrollB - 1) * kThreads < j1; j += kUnrollB * kThreads) {
        float vy[kUnrollB][V], vd[kUnrollB][V];
        int64_t ad[kUnrollB];
#pragma unroll
        for (int u = 0; u < kUnrollB; ++u) {
            ad[u] = w.addr * V;
            load_elems<DT, V>(y, ad[u], vy[u]);
            load_elems<DT, V>(dy, ad[u], vd[u]);
            w.step();
        }
#pragma unroll
        for (int u = 0; u < kUnrollB; ++u) {
            if constexpr (DX) {
                accumulate_dx<ACT, V, DT == kF32>(vy[u], vd[u], bc, A, a, inv_a, sdz, sdzt);
                store_out<DT, V>(dx, ad[u], vd[u]);
            } else {
                accumulate<ACT, V, XH, DT == kF32>(vy[u], vd[u], bc, gc, a, inv_a, sdz, sdzt);
            }
        }
    }
    for (; j < j1; j += kThreads) {
        float vy[V], vd[V];
        const int64_t ad = w.addr * V;
        load_elems<DT, V>(y, ad, vy);
        load_elems<DT, V>(dy, ad, vd);
        w.step();
        if constexpr (DX) {
            accumulate_dx<ACT, V, DT == kF32>(vy, vd, bc, A, a, inv_a, sdz, sdzt);
            store_out<DT, V>(dx, ad, vd);
        } else {
            accumulate<ACT, V, XH, DT == kF32>(vy, vd, bc, gc, a, inv_a, sdz, sdzt);
        }
    }
    float S1 = 0.f, S2 = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) { S1 += sdz[e]; S2 += sdzt[e]; }
    S1 = wave_sum(S1);
    S2 = wave_sum(S2);
    __shared__ float sh[2][kThreads / kWave];
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) { sh[0][wave] = S1; sh[1][wave] = S2; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float t1 = sh[0][0], t2 = sh[1][0];
#pragma unroll
        for (int k = 1; k < kThreads / kWave; ++k) { t1 += sh[0][k]; t2 += sh[1][k]; }
        part_dz[p * C + c] = t1;
        part_dzt[p * C + c] = t2;
    }
}

// ---------------------------------------------------------------------------
// NHWC: workgroup b covers channel slice b % slices and partial b / slices, i.e.
// row groups p, p + P, ... of rpi = 256/tpr rows (as the statistics kernel).
template <int DT, int V, int ACT, bool DX, bool XH = false>
__global__ __launch_bounds__(kThreads) void k_bwd_reduce_nhwc(
    const void* __restrict__ y, const void* dy, int64_t m, int64_t Cv, int tpr,
    int64_t slices, int64_t groups, int64_t P, const float* __restrict__ beta, float a,
    float inv_a, float* __restrict__ part_dz, float* __restrict__ part_dzt, void* dx,
    const float* __restrict__ gamma, const float* __restrict__ frozen_var, float eps,
    bool from_end)
{
    static_assert(!(DX && XH), "the frozen-statistics pass reads y");
    const int64_t b = blockIdx.x;
    const int64_t p = b / slices;
    const int64_t sl = b - p * slices;
    const int t = threadIdx.x;
    const int rs = t / tpr;
    const int rpi = kThreads / tpr;
    const int64_t col = sl * tpr + (t - rs * tpr);
    const bool active = col < Cv;

    float bc[V], gc[V], sdz[V], sdzt[V], A[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        bc[e] = 0.f;
        gc[e] = 0.f;
        A[e] = 0.f;
        sdz[e] = 0.f;
        sdzt[e] = 0.f;
    }
    // one element of the reduction; with DX also dx at storage index i (elements)
    auto one = [&](float (&vy)[V], float (&vd)[V], int64_t i) {
        if constexpr (DX) {
            accumulate_dx<ACT, V, DT == kF32>(vy, vd, bc, A, a, inv_a, sdz, sdzt);
            store_out<DT, V>(dx, i, vd);
        } else {
            accumulate<ACT, V, XH, DT == kF32>(vy, vd, bc, gc, a, inv_a, sdz, sdzt);
        }
    };
    if (active) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            bc[e] = beta[col * V + e];
            if constexpr (XH) gc[e] = gamma[col * V + e];
            if constexpr (DX) A[e] = frozen_scale(gamma, frozen_var, eps, col * V + e);
        }
        if constexpr (V == Raw16<DT>::V) {
            // software pipeline over complete row groups (branch-free): the next
            // kUnrollN groups of y and dy load while the current ones are summed;
            // the rest, at most one ragged group per workgroup, runs checked
            const int64_t full = m / rpi;
            const uint4* yv = reinterpret_cast<const uint4*>(y);
            const uint4* dv = reinterpret_cast<const uint4*>(dy);
            // row group g's place in the walk: from the end of the tensor down if
            // from_end (the ragged last group, if any, keeps its place)
            auto rg = [&](int64_t g) { return from_end && g < full ? full - 1 - g : g; };
            auto load_set = [&](uint4 (&by)[kUnrollN], uint4 (&bd)[kUnrollN], int64_t g0) {
#pragma unroll
                for (int u = 0; u < kUnrollN; ++u) {
                    const int64_t i = (rg(g0 + u * P) * rpi + rs) * Cv + col;
                    by[u] = yv[i];
                    bd[u] = dv[i];
                }
            };
            auto add_set = [&](const uint4 (&by)[kUnrollN], const uint4 (&bd)[kUnrollN],
                               int64_t g0) {
#pragma unroll
                for (int u = 0; u < kUnrollN; ++u) {
                    float vy[V], vd[V];
                    unpack16<DT>(by[u], vy);
                    unpack16<DT>(bd[u], vd);
                    one(vy, vd, ((rg(g0 + u * P) * rpi + rs) * Cv + col) * V);
                }
            };
            // sets of kUnrollN complete groups, pipelined as in the statistics
            const int64_t span = int64_t(kUnrollN) * P;
            const int64_t first_bad = full - (kUnrollN - 1) * P;
            const int64_t ns = first_bad > p ? (first_bad - p + span - 1) / span : 0;
            int64_t g = p + ns * span;
            if (ns > 0) {
                uint4 Ay[kUnrollN], Ad[kUnrollN], By[kUnrollN], Bd[kUnrollN];
                load_set(Ay, Ad, p);
                int64_t j = 0;
                for (; j + 1 < ns; j += 2) {
                    load_set(By, Bd, p + (j + 1) * span);
                    __builtin_amdgcn_sched_barrier(0);
                    add_set(Ay, Ad, p + j * span);
                    load_set(Ay, Ad, p + (j + 2 < ns ? j + 2 : ns - 1) * span);
                    __builtin_amdgcn_sched_barrier(0);
                    add_set(By, Bd, p + (j + 1) * span);
                }
                if (j < ns) add_set(Ay, Ad, p + j * span);
            }
            for (; g < groups; g += P) {
                const int64_t r = rg(g) * rpi + rs;
                if (r < m) {
                    float vy[V], vd[V];
                    unpack16<DT>(yv[r * Cv + col], vy);
                    unpack16<DT>(dv[r * Cv + col], vd);
                    one(vy, vd, (r * Cv + col) * V);
                }
            }
        } else {
            for (int64_t g = p; g < groups; g += P) {
                const int64_t r = g * rpi + rs;
                if (r < m) {
                    float vy[V], vd[V];
                    load_elems<DT, V>(y, (r * Cv + col) * V, vy);
                    load_elems<DT, V>(dy, (r * Cv + col) * V, vd);
                    one(vy, vd, (r * Cv + col) * V);
                }
            }
        }
    }
    __shared__ float sh_a[V][kThreads];
    __shared__ float sh_b[V][kThreads];
#pragma unroll
    for (int e = 0; e < V; ++e) { sh_a[e][t] = sdz[e]; sh_b[e][t] = sdzt[e]; }
    for (int s = rpi / 2; s >= 1; s >>= 1) {
        __syncthreads();
        if (rs < s) {
            const int o = t + s * tpr;
#pragma unroll
            for (int e = 0; e < V; ++e) { sdz[e] += sh_a[e][o]; sdzt[e] += sh_b[e][o]; }
        }
        __syncthreads();
        if (rs < s) {
#pragma unroll
            for (int e = 0; e < V; ++e) { sh_a[e][t] = sdz[e]; sh_b[e][t] = sdzt[e]; }
        }
    }
    if (rs == 0 && active) {
        const int64_t base = p * Cv * V + col * V;
        store_floats<V>(part_dz + base, sdz);
        store_floats<V>(part_dzt + base, sdzt);
    }
}

// ---------------------------------------------------------------------------
// Finishing the sums: thread t of a 1024-thread workgroup takes channel
// t % kFinChannels and partials p = t / kFinChannels + k*kFinPhases, adds them in
// fp64, and the phases are added in a fixed order.
//
// frozen_var non-null: the statistics are the frozen running ones (the backward
// through the inference forward), so dx = gamma*dz/sqrt(frozen_var + eps): the
// constants become {A, 0, 0, beta}, and dgamma, dbeta are the same sums.
// xhat_sums: the second sums are of dz*xhat (optimized checkpointing), so dgamma
// is their total and dx = A*dz + B*xhat + Cc with B = -A*dgamma/m.
__global__ __launch_bounds__(kFinThreads) void k_bwd_finalize(
    int64_t C, int64_t m, int64_t P, const float* __restrict__ part_dz,
    const float* __restrict__ part_dzt, const float* __restrict__ gamma,
    const float* __restrict__ beta, const float* __restrict__ invstd,
    const float* __restrict__ frozen_var, float eps,
    float* __restrict__ dgamma, float* __restrict__ dbeta, float4* __restrict__ consts,
    bool xhat_sums = false)
{
    const int cl = threadIdx.x % kFinChannels;
    const int ph = threadIdx.x / kFinChannels;
    const int64_t c = int64_t(blockIdx.x) * kFinChannels + cl;
    // the finishing thread's per-channel inputs, fetched before the sums
    const bool fin = ph == 0 && c < C;
    float g_c = 1.f, b_c = 0.f, s_c = 0.f;
    if (fin) {
        g_c = gamma[c];
        b_c = beta[c];
        s_c = frozen_var ? frozen_var[c] : invstd[c];
    }
    double s1 = 0.0, s2 = 0.0;
    if (c < C) {
        // partials in order, four at a time with their loads issued together
        int64_t p = ph;
        for (; p + 3 * kFinPhases < P; p += 4 * kFinPhases) {
            float a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = part_dz[(p + u * kFinPhases) * C + c];
                b[u] = part_dzt[(p + u * kFinPhases) * C + c];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) { s1 += double(a[u]); s2 += double(b[u]); }
        }
        for (; p < P; p += kFinPhases) {
            s1 += double(part_dz[p * C + c]);
            s2 += double(part_dzt[p * C + c]);
        }
    }
    __shared__ double sh1[kFinPhases][kFinChannels];
    __shared__ double sh2[kFinPhases][kFinChannels];
    sh1[ph][cl] = s1;
    sh2[ph][cl] = s2;
    __syncthreads();
    if (!fin) return;
    for (int k = 1; k < kFinPhases; ++k) { s1 += sh1[k][cl]; s2 += sh2[k][cl]; }
    const double g = double(g_c);
    const double db = s1;
    const double dg = xhat_sums ? s2 : s2 / g;
    dbeta[c] = float(db);
    dgamma[c] = float(dg);
    if (frozen_var) {
        consts[c] = make_float4(float(g / sqrt(double(s_c) + double(eps))), 0.f, 0.f, b_c);
        return;
    }
    const double A = g * double(s_c);
    const double md = double(m);
    const double B = xhat_sums ? -A * dg / md : -A * dg / (md * g);
    consts[c] = make_float4(float(A), float(B), float(-A * db / md), b_c);
}

// The dx constants of the backward through the inference forward when dgamma and
// dbeta are not wanted: {gamma/sqrt(running_var + eps), 0, 0, beta} per channel.
__global__ __launch_bounds__(kThreads) void k_eval_consts(
    int64_t C, const float* __restrict__ gamma, const float* __restrict__ beta,
    const float* __restrict__ running_var, float eps, float4* __restrict__ consts)
{
    const int64_t c = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (c >= C) return;
    consts[c] = make_float4(float(double(gamma[c]) / sqrt(double(running_var[c]) + double(eps))),
                            0.f, 0.f, beta[c]);
}

// ---------------------------------------------------------------------------
// dx = A*dz + B*(z - beta) + Cc.  dx may be the same buffer as dy: each element
// of dy is read by the thread that then writes the same element of dx.
template <int ACT, int V, bool P>
__device__ __forceinline__ void dx_one(const float (&vy)[V], float (&vd)[V], const float4 (&k)[V],
                                       float a, float inv_a)
{
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float z, slope;
        act_invert<ACT, P>(vy[e], a, inv_a, z, slope);
        const float dz = slope * vd[e];
        vd[e] = fmaf(k[e].x, dz, fmaf(k[e].y, z - k[e].w, k[e].z));
    }
}

template <int DT, int V, int ACT>
__global__ __launch_bounds__(kThreads) void k_bwd_apply_nchw(
    const void* __restrict__ y, const void* dy, void* dx, int64_t nvec, int64_t C, int64_t HWv,
    const float4* __restrict__ consts, float a, float inv_a)
{
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    FlatNCHWWalk w;
    w.init(v < nvec ? v : 0, C, HWv, stride);
    for (; v + (kUnrollB - 1) * stride < nvec; v += kUnrollB * stride) {
        float vy[kUnrollB][V], vd[kUnrollB][V];
        float4 k[kUnrollB][V];
#pragma unroll
        for (int u = 0; u < kUnrollB; ++u) {
            load_elems<DT, V>(y, (v + u * stride) * V, vy[u]);
            load_elems<DT, V>(dy, (v + u * stride) * V, vd[u]);
            const float4 kc = consts[w.c];
#pragma unroll
            for (int e = 0; e < V; ++e) k[u][e] = kc;
            w.step();
        }
#pragma unroll
        for (int u = 0; u < kUnrollB; ++u) {
            dx_one<ACT, V, DT == kF32>(vy[u], vd[u], k[u], a, inv_a);
            store_out<DT, V>(dx, (v + u * stride) * V, vd[u]);
        }
    }
    for (; v < nvec; v += stride) {
        float vy[V], vd[V];
        float4 k[V];
        load_elems<DT, V>(y, v * V, vy);
        load_elems<DT, V>(dy, v * V, vd);
        const float4 kc = consts[w.c];
#pragma unroll
        for (int e = 0; e < V; ++e) k[e] = kc;
        w.step();
        dx_one<ACT, V, DT == kF32>(vy, vd, k, a, inv_a);
        store_out<DT, V>(dx, v * V, vd);
    }
}

template <int DT, int V, int ACT, bool FIXED>
__global__ __launch_bounds__(kThreads) void k_bwd_apply_nhwc(
    const void* __restrict__ y, const void* dy, void* dx, int64_t nvec, int64_t Cv,
    const float4* __restrict__ consts, float a, float inv_a, bool from_end)
{
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if constexpr (FIXED) {
        if (v >= nvec) return;
        const int64_t c0 = (v % Cv) * V;
        float4 k[V];
#pragma unroll
        for (int e = 0; e < V; ++e) k[e] = consts[c0 + e];
        if constexpr (V == Raw16<DT>::V && ACT != kElu) {
            // The thread's n vectors, from the end of the tensor down if from_end,
            // else up (starting where the sums pass ended: those rows are the
            // likeliest still to sit in the Infinity Cache), in sets of kUnrollB:
            // set j + 1 loads while set j is written.
            // The loop has no exit between its stages (the last load of an even
            // count is a spare reload), so the compiler keeps both sets in flight.
            // ELU keeps the plain loop below: its wider grid needs the registers
            // the second set would take (bf16: 159 against 193 us).
            const int64_t n = (nvec - 1 - v) / stride + 1;
            const int64_t top = v + (n - 1) * stride;
            const int64_t step = from_end ? -stride : stride;
            const int64_t first = from_end ? top : v;
            const int64_t ns = n / kUnrollB;
            const uint4* yv = reinterpret_cast<const uint4*>(y);
            const uint4* dv = reinterpret_cast<const uint4*>(dy);
            auto load_set = [&](uint4 (&qy)[kUnrollB], uint4 (&qd)[kUnrollB], int64_t js) {
#pragma unroll
                for (int u = 0; u < kUnrollB; ++u) {
                    const int64_t w = first + (js * kUnrollB + u) * step;
                    qy[u] = yv[w];
                    qd[u] = dv[w];
                }
            };
            auto put = [&](const uint4& qy, const uint4& qd, int64_t w) {
                float vy[V], vd[V];
                unpack16<DT>(qy, vy);
                unpack16<DT>(qd, vd);
                dx_one<ACT, V, DT == kF32>(vy, vd, k, a, inv_a);
                store_out<DT, V>(dx, w * V, vd);
            };
            auto put_set = [&](const uint4 (&qy)[kUnrollB], const uint4 (&qd)[kUnrollB], int64_t js) {
#pragma unroll
                for (int u = 0; u < kUnrollB; ++u) put(qy[u], qd[u], first + (js * kUnrollB + u) * step);
            };
            if (ns > 0) {
                uint4 ya[kUnrollB], da[kUnrollB], yb[kUnrollB], db[kUnrollB];
                load_set(ya, da, 0);
                int64_t js = 0;
                for (; js + 1 < ns; js += 2) {
                    load_set(yb, db, js + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    put_set(ya, da, js);
                    load_set(ya, da, js + 2 < ns ? js + 2 : ns - 1);
                    __builtin_amdgcn_sched_barrier(0);
                    put_set(yb, db, js + 1);
                }
                if (js < ns) put_set(ya, da, js);
            }
            for (int64_t i2 = ns * kUnrollB; i2 < n; ++i2) {
                const int64_t w = first + i2 * step;
                put(yv[w], dv[w], w);
            }
            return;
        }
        if (from_end) {
            // walk from the end down
            const int64_t v0 = v;
            v = v0 + ((nvec - 1 - v0) / stride) * stride;
            for (; v - (kUnrollB - 1) * stride >= v0; v -= kUnrollB * stride) {
                float vy[kUnrollB][V], vd[kUnrollB][V];
#pragma unroll
                for (int u = 0; u < kUnrollB; ++u) {
                    load_elems<DT, V>(y, (v - u * stride) * V, vy[u]);
                    load_elems<DT, V>(dy, (v - u * stride) * V, vd[u]);
                }
#pragma unroll
                for (int u = 0; u < kUnrollB; ++u) {
                    dx_one<ACT, V, DT == kF32>(vy[u], vd[u], k, a, inv_a);
                    store_out<DT, V>(dx, (v - u * stride) * V, vd[u]);
                }
            }
            for (; v >= v0; v -= stride) {
                float vy[V], vd[V];
                load_elems<DT, V>(y, v * V, vy);
                load_elems<DT, V>(dy, v * V, vd);
                dx_one<ACT, V, DT == kF32>(vy, vd, k, a, inv_a);
                store_out<DT, V>(dx, v * V, vd);
            }
            return;
        }
        for (; v + (kUnrollB - 1) * stride < nvec; v += kUnrollB * stride) {
            float vy[kUnrollB][V], vd[kUnrollB][V];
#pragma unroll
            for (int u = 0; u < kUnrollB; ++u) {
                load_elems<DT, V>(y, (v + u * stride) * V, vy[u]);
                load_elems<DT, V>(dy, (v + u * stride) * V, vd[u]);
            }
#pragma unroll
            for (int u = 0; u < kUnrollB; ++u) {
                dx_one<ACT, V, DT == kF32>(vy[u], vd[u], k, a, inv_a);
                store_out<DT, V>(dx, (v + u * stride) * V, vd[u]);
            }
        }
        for (; v < nvec; v += stride) {
            float vy[V], vd[V];
            load_elems<DT, V>(y, v * V, vy);
            load_elems<DT, V>(dy, v * V, vd);
            dx_one<ACT, V, DT == kF32>(vy, vd, k, a, inv_a);
            store_out<DT, V>(dx, v * V, vd);
        }
    } else {
        for (; v < nvec; v += stride) {
            const int64_t c0 = (v % Cv) * V;
            float vy[V], vd[V];
            float4 k[V];
#pragma unroll
            for (int e = 0; e < V; ++e) k[e] = consts[c0 + e];
            load_elems<DT, V>(y, v * V, vy);
            load_elems<DT, V>(dy, v * V, vd);
            dx_one<ACT, V, DT == kF32>(vy, vd, k, a, inv_a);
            store_elems<DT, V>(dx, v * V, vd);
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers

// The frozen-statistics arguments (dx, gamma, frozen_var, eps) are used only with DX.
struct FrozenDx {
    void* dx = nullptr;
    const float* gamma = nullptr;
    const float* var = nullptr;
    float eps = 0.f;
};

template <int DT, int V, int ACT, bool DX, bool XH>
static void launch_reduce_dva(const Plan& pl, const void* y, const void* dy, const float* beta,
                              float a, float ia, float* pa, float* pb, const FrozenDx& f,
                              hipStream_t s)
{
    if (pl.layout == kNCHW)
        hipLaunchKernelGGL((k_bwd_reduce_nchw<DT, V, ACT, DX, XH>), dim3(pl.reduce_blocks),
                           dim3(kThreads), 0, s, y, dy, pl.C, pl.HW, pl.m, pl.unit, pl.P, beta, a,
                           ia, pa, pb, f.dx, f.gamma, f.var, f.eps);
    else
        hipLaunchKernelGGL((k_bwd_reduce_nhwc<DT, V, ACT, DX, XH>), dim3(pl.reduce_blocks_bwd),
                           dim3(kThreads), 0, s, y, dy, pl.m, pl.C / V, pl.tpr, pl.slices, pl.unit,
                           pl.P_bwd, beta, a, ia, pa, pb, f.dx, f.gamma, f.var, f.eps,
                           bwd_sums_from_end(pl));
}

// XH: the reduction reads xhat instead of y (f.gamma carries gamma for it).
template <bool DX, bool XH = false>
static void launch_reduce(const Plan& pl, const void* y, const void* dy, const float* beta,
                          int act, float a, float ia, float* pa, float* pb, const FrozenDx& f,
                          hipStream_t s)
{
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            constexpr int DT = decltype(d)::value, ACT = decltype(ac)::value;
            if (pl.vec)
                launch_reduce_dva<DT, vec_width(DT), ACT, DX, XH>(pl, y, dy, beta, a, ia, pa, pb,
                                                                  f, s);
            else
                launch_reduce_dva<DT, 1, ACT, DX, XH>(pl, y, dy, beta, a, ia, pa, pb, f, s);
        });
    });
}

void launch_backward_reduce(const Plan& pl, const void* y, const void* dy, const float* gamma,
                            const float* beta, const float* invstd, float* dgamma, float* dbeta,
                            int act, float a, void* ws, hipStream_t s)
{
    char* wsb = static_cast<char*>(ws);
    float* pa = reinterpret_cast<float*>(wsb + pl.off_part_a);
    float* pb = reinterpret_cast<float*>(wsb + pl.off_part_b);
    float4* consts = reinterpret_cast<float4*>(wsb + pl.off_const);
    const float ia = act == kIdentity ? 1.f : 1.f / a;
    launch_reduce<false>(pl, y, dy, beta, act, a, ia, pa, pb, FrozenDx{}, s);
    hipLaunchKernelGGL(k_bwd_finalize, dim3(unsigned(ceil_div(pl.C, kFinChannels))),
                       dim3(kFinThreads), 0, s, pl.C, pl.m, pl.P_bwd, pa, pb, gamma, beta, invstd,
                       static_cast<const float*>(nullptr), 0.f, dgamma, dbeta, consts);
}

void launch_backward_reduce_xhat(const Plan& pl, const void* xhat, const void* dy,
                                 const float* gamma, const float* beta, const float* invstd,
                                 float* dgamma, float* dbeta, int act, float a, void* ws,
                                 hipStream_t s)
{
    char* wsb = static_cast<char*>(ws);
    float* pa = reinterpret_cast<float*>(wsb + pl.off_part_a);
    float* pb = reinterpret_cast<float*>(wsb + pl.off_part_b);
    float4* consts = reinterpret_cast<float4*>(wsb + pl.off_const);
    FrozenDx g;
    g.gamma = gamma;
    launch_reduce<false, true>(pl, xhat, dy, beta, act, a, 1.f, pa, pb, g, s);
    hipLaunchKernelGGL(k_bwd_finalize, dim3(unsigned(ceil_div(pl.C, kFinChannels))),
                       dim3(kFinThreads), 0, s, pl.C, pl.m, pl.P_bwd, pa, pb, gamma, beta, invstd,
                       static_cast<const float*>(nullptr), 0.f, dgamma, dbeta, consts, true);
}

void launch_backward_eval_grads(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* running_var,
                                float eps, float* dgamma, float* dbeta, int act, float a,
                                void* ws, hipStream_t s)
{
    char* wsb = static_cast<char*>(ws);
    float* pa = reinterpret_cast<float*>(wsb + pl.off_part_a);
    float* pb = reinterpret_cast<float*>(wsb + pl.off_part_b);
    float4* consts = reinterpret_cast<float4*>(wsb + pl.off_const);
    const float ia = act == kIdentity ? 1.f : 1.f / a;
    launch_reduce<true>(pl, y, dy, beta, act, a, ia, pa, pb, FrozenDx{dx, gamma, running_var, eps},
                        s);
    hipLaunchKernelGGL(k_bwd_finalize, dim3(unsigned(ceil_div(pl.C, kFinChannels))),
                       dim3(kFinThreads), 0, s, pl.C, pl.m, pl.P_bwd, pa, pb, gamma, beta,
                       static_cast<const float*>(nullptr), running_var, eps, dgamma, dbeta,
                       consts);
}

void launch_eval_consts(const Plan& pl, const float* gamma, const float* beta,
                        const float* running_var, float eps, void* ws, hipStream_t s)
{
    float4* consts = reinterpret_cast<float4*>(static_cast<char*>(ws) + pl.off_const);
    hipLaunchKernelGGL(k_eval_consts, dim3(unsigned(ceil_div(pl.C, kThreads))), dim3(kThreads), 0,
                       s, pl.C, gamma, beta, running_var, eps, consts);
}

template <int DT, int V, int ACT>
static void launch_bapply_dva(const Plan& pl, const void* y, const void* dy, void* dx,
                              const float4* k, float a, float ia, hipStream_t s)
{
    const int64_t nvec = pl.numel / V;
    const dim3 grid(unsigned(dx_grid(pl, ACT)));
    if (pl.layout == kNCHW)
        hipLaunchKernelGGL((k_bwd_apply_nchw<DT, V, ACT>), grid, dim3(kThreads), 0, s, y, dy, dx,
                           nvec, pl.C, pl.HW / V, k, a, ia);
    else if (pl.fixed_col)
        hipLaunchKernelGGL((k_bwd_apply_nhwc<DT, V, ACT, true>), grid, dim3(kThreads), 0, s, y, dy,
                           dx, nvec, pl.C / V, k, a, ia, !bwd_sums_from_end(pl));
    else
        hipLaunchKernelGGL((k_bwd_apply_nhwc<DT, V, ACT, false>), grid, dim3(kThreads), 0, s, y,
                           dy, dx, nvec, pl.C / V, k, a, ia, !bwd_sums_from_end(pl));
}

template <int DT, int V>
static void launch_bapply_dv(const Plan& pl, const void* y, const void* dy, void* dx,
                             const float4* k, int act, float a, float ia, hipStream_t s)
{
    switch (act) {
    case kLeaky: launch_bapply_dva<DT, V, kLeaky>(pl, y, dy, dx, k, a, ia, s); break;
    case kElu: launch_bapply_dva<DT, V, kElu>(pl, y, dy, dx, k, a, ia, s); break;
    default: launch_bapply_dva<DT, V, kIdentity>(pl, y, dy, dx, k, a, ia, s); break;
    }
}

void launch_backward_apply(const Plan& pl, const void* y, const void* dy, void* dx, int act,
                           float a, void* ws, hipStream_t s)
{
    const float4* k = reinterpret_cast<const float4*>(static_cast<char*>(ws) + pl.off_const);
    const float ia = act == kIdentity ? 1.f : 1.f / a;
    with_dtype(pl.dtype, [&](auto d) {
        constexpr int DT = decltype(d)::value;
        if (pl.vec) launch_bapply_dv<DT, vec_width(DT)>(pl, y, dy, dx, k, act, a, ia, s);
        else launch_bapply_dv<DT, 1>(pl, y, dy, dx, k, act, a, ia, s);
    });
}

}  // namespace iabn

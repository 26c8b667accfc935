// Forward kernels of In-Place Activated BatchNorm (training and inference).
//
// Training forward (section 3 of the paperlayer summary of "In-Place Activated
// BatchNorm for Memory-Optimized Training of DNNs", "Batch Normalization Review"
// and "INPLACE-ABN"): per-channel empirical mean and biased variance over the
// m = N*H*W elements, then y = act(gamma*xhat + beta) written over x, so that
// the layer keeps a single buffer.
//
// Three launches:
//   stats_*      one workgroup per (channel tile, partial); streams x once and
//                writes (mean, M2) of its elements, shifted by a pivot K_c
//   fwd_finalize the partials of a channel as fp64 shifted sums, added in a fixed
//                order; statistics, running statistics, and the constants
//                {K_c, d_c = mean_c - K_c, s_c = gamma_c*invstd_c, beta_c}
//   fwd_apply    elementwise y = act(((x - K_c) - d_c)*s_c + beta_c), in place
//
// The pivot K_c is the channel's first element (n = 0, h = 0, w = 0).  x - K_c
// is exact in fp32 whenever x is within a factor two of K_c, so the centred value
// keeps full precision even when |mean| >> std: the mean is only ever handled as
// the small offset d_c, never as an fp32 number of its own.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace iabn {

#ifndef IABN_REDUCE_UNROLL
#define IABN_REDUCE_UNROLL 4
#endif
constexpr int kUnroll = IABN_REDUCE_UNROLL;
// NHWC statistics: row groups in flight per thread and pipeline stage
#ifndef IABN_NHWC_STATS_UNROLL
#define IABN_NHWC_STATS_UNROLL 4
#endif
constexpr int kUnrollS = IABN_NHWC_STATS_UNROLL;

// ---------------------------------------------------------------------------
// NCHW statistics: workgroup b covers channel c = b / P, partial p = b % P, i.e.
// the channel-local elements [p*unit, min((p+1)*unit, m)).
template <int DT, int V>
__global__ __launch_bounds__(kThreads) void k_stats_nchw(
    const void* __restrict__ x, int64_t C, int64_t HW, int64_t m, int64_t unit, int64_t P,
    float* __restrict__ part_mean, float* __restrict__ part_m2, float* __restrict__ count)
{
    const int64_t b = blockIdx.x;
    const int64_t c = b / P;
    const int64_t p = b - c * P;
    const int64_t HWv = HW / V;
    const int64_t j1 = dmin(p * unit + unit, m) / V;
    int64_t j = p * unit / V + threadIdx.x;

    const float K = load_one<DT>(x, c * HW);
    float s1[V], s2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) { s1[e] = 0.f; s2[e] = 0.f; }
    int cnt = 0;

    ChannelWalk w;
    w.init(j < j1 ? j : 0, c, C, HWv, kThreads);
    // main loop: kUnroll vectors in flight per thread
    for (; j + (kUnroll - 1) * kThreads < j1; j += kUnroll * kThreads) {
        float v[kUnroll][V];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            load_elems<DT, V>(x, w.addr * V, v[u]);
            w.step();
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float d = v[u][e] - K;
                s1[e] += d;
                s2[e] = fmaf(d, d, s2[e]);
            }
        cnt += kUnroll;
    }
    for (; j < j1; j += kThreads) {
        float v[V];
        load_elems<DT, V>(x, w.addr * V, v);
        w.step();
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float d = v[e] - K;
            s1[e] += d;
            s2[e] = fmaf(d, d, s2[e]);
        }
        cnt += 1;
    }

    float S1 = 0.f, S2 = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) { S1 += s1[e]; S2 += s2[e]; }
    float n = float(cnt * V);
    float mean = cnt ? S1 / n : 0.f;
    float m2 = cnt ? fmaxf(S2 - S1 * mean, 0.f) : 0.f;
    wave_chan(n, mean, m2);

    __shared__ float sh[3][kThreads / kWave];
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        sh[0][wave] = n; sh[1][wave] = mean; sh[2][wave] = m2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float tn = sh[0][0], tm = sh[1][0], t2 = sh[2][0];
#pragma unroll
        for (int k = 1; k < kThreads / kWave; ++k) chan_merge(tn, tm, t2, sh[0][k], sh[1][k], sh[2][k]);
        part_mean[p * C + c] = tm;
        part_m2[p * C + c] = t2;
        if (c == 0) count[p] = tn;
    }
}

// ---------------------------------------------------------------------------
// NHWC statistics: workgroup b covers channel slice sl = b % slices (tpr vectors
// of V channels) and partial p = b / slices, i.e. row groups p, p + P, p + 2P, ...
// of rpi = 256/tpr rows.  Thread t owns channel vector col = sl*tpr + t % tpr
// and row slot t / tpr of every group; the row slots are then merged by an LDS
// tree.  On the 16-byte path the walk is software-pipelined: the next kUnroll
// row groups are loaded (as raw bits) while the current ones are summed.
template <int DT, int V>
__device__ __forceinline__ void stats_add(const float (&v)[V], const float (&K)[V], float (&s1)[V],
                                          float (&s2)[V])
{
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const float d = v[e] - K[e];
        s1[e] += d;
        s2[e] = fmaf(d, d, s2[e]);
    }
}

template <int DT, int V>
__global__ __launch_bounds__(kThreads) void k_stats_nhwc(
    const void* __restrict__ x, int64_t m, int64_t Cv, int tpr, int64_t slices, int64_t groups,
    int64_t P, float* __restrict__ part_mean, float* __restrict__ part_m2,
    float* __restrict__ count)
{
    const int64_t b = blockIdx.x;
    const int64_t p = b / slices;
    const int64_t sl = b - p * slices;
    const int t = threadIdx.x;
    const int rs = t / tpr;               // row slot
    const int rpi = kThreads / tpr;       // rows per group
    const int64_t col = sl * tpr + (t - rs * tpr);
    const bool active = col < Cv;

    float K[V];
    float s1[V], s2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) { K[e] = 0.f; s1[e] = 0.f; s2[e] = 0.f; }
    int cnt = 0;
    if (active) {
        load_elems<DT, V>(x, col * V, K);
        if constexpr (V == Raw16<DT>::V) {
            // complete row groups (every row present) run a branch-free pipeline;
            // the rest, at most one ragged group per workgroup, runs checked
            const int64_t full = m / rpi;
            const uint4* xv = reinterpret_cast<const uint4*>(x);
            auto load_set = [&](uint4 (&buf)[kUnrollS], int64_t g0) {
#pragma unroll
                for (int u = 0; u < kUnrollS; ++u) buf[u] = xv[((g0 + u * P) * rpi + rs) * Cv + col];
            };
            auto add_set = [&](const uint4 (&buf)[kUnrollS]) {
#pragma unroll
                for (int u = 0; u < kUnrollS; ++u) {
                    float v[V];
                    unpack16<DT>(buf[u], v);
                    stats_add<DT, V>(v, K, s1, s2);
                }
                cnt += kUnrollS;
            };
            // Sets of kUnrollS complete groups, g = p + j*kUnrollS*P for j < ns.  Set
            // j + 1 loads while set j is summed; the loop has no exit in between
            // (the last load of an even count is a spare reload of the final set),
            // so the compiler keeps the two sets in flight together.
            const int64_t span = int64_t(kUnrollS) * P;
            const int64_t first_bad = full - (kUnrollS - 1) * P;   // sets starting here are ragged
            const int64_t ns = first_bad > p ? (first_bad - p + span - 1) / span : 0;
            int64_t g = p + ns * span;
            if (ns > 0) {
                uint4 A[kUnrollS], B[kUnrollS];
                load_set(A, p);
                int64_t j = 0;
                for (; j + 1 < ns; j += 2) {
                    load_set(B, p + (j + 1) * span);
                    __builtin_amdgcn_sched_barrier(0);
                    add_set(A);
                    load_set(A, p + (j + 2 < ns ? j + 2 : ns - 1) * span);
                    __builtin_amdgcn_sched_barrier(0);
                    add_set(B);
                }
                if (j < ns) add_set(A);
            }
            for (; g < groups; g += P) {
                const int64_t r = g * rpi + rs;
                if (r < m) {
                    float v[V];
                    unpack16<DT>(xv[r * Cv + col], v);
                    stats_add<DT, V>(v, K, s1, s2);
                    ++cnt;
                }
            }
        } else {
            for (int64_t g = p; g < groups; g += P) {
                const int64_t r = g * rpi + rs;
                if (r < m) {
                    float v[V];
                    load_elems<DT, V>(x, (r * Cv + col) * V, v);
                    stats_add<DT, V>(v, K, s1, s2);
                    ++cnt;
                }
            }
        }
    }
    float n = float(cnt);
    float mean[V], m2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        mean[e] = cnt ? s1[e] / n : 0.f;
        m2[e] = cnt ? fmaxf(s2[e] - s1[e] * mean[e], 0.f) : 0.f;
    }

    __shared__ float sh_n[kThreads];
    __shared__ float sh_mean[V][kThreads];
    __shared__ float sh_m2[V][kThreads];
    sh_n[t] = n;
#pragma unroll
    for (int e = 0; e < V; ++e) { sh_mean[e][t] = mean[e]; sh_m2[e][t] = m2[e]; }
    for (int s = rpi / 2; s >= 1; s >>= 1) {
        __syncthreads();
        if (rs < s) {
            const int o = t + s * tpr;
            const float nb = sh_n[o];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float nn = n;
                chan_merge(nn, mean[e], m2[e], nb, sh_mean[e][o], sh_m2[e][o]);
            }
            if (nb > 0.f) n += nb;
        }
        __syncthreads();
        if (rs < s) {
            sh_n[t] = n;
#pragma unroll
            for (int e = 0; e < V; ++e) { sh_mean[e][t] = mean[e]; sh_m2[e][t] = m2[e]; }
        }
    }
    if (rs == 0 && active) {
        const int64_t base = p * Cv * V + col * V;
        store_floats<V>(part_mean + base, mean);
        store_floats<V>(part_m2 + base, m2);
    }
    if (t == 0 && sl == 0) count[p] = n;
}

// ---------------------------------------------------------------------------
// Finishing the statistics.  A 1024-thread workgroup covers kFinChannels
// channels; thread t takes channel t % kFinChannels and partials
// p = t / kFinChannels + k*kFinPhases.  Each partial (n_p, mean_p, M2_p) becomes
// the shifted sums n_p*mean_p and M2_p + n_p*mean_p^2, added in fp64 in a fixed
// order (phases in turn, then partials within a phase); then
//   mean = S1/m, M2 = S2 - S1*mean, var = M2/m  (all fp64),
// and the statistics, the running statistics and the apply constants.
template <int DT>
__global__ __launch_bounds__(kFinThreads) void k_fwd_finalize(
    const void* __restrict__ x, int layout, int64_t C, int64_t HW, int64_t m, int64_t P,
    const float* __restrict__ part_mean, const float* __restrict__ part_m2,
    const float* __restrict__ count, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* __restrict__ running_mean,
    float* __restrict__ running_var, float* __restrict__ save_mean,
    float* __restrict__ save_invstd, float eps, float momentum, float4* __restrict__ consts)
{
    const int cl = threadIdx.x % kFinChannels;
    const int ph = threadIdx.x / kFinChannels;
    const int64_t c = int64_t(blockIdx.x) * kFinChannels + cl;
    // the finishing thread's per-channel inputs, fetched before the sums
    const bool fin = ph == 0 && c < C;
    float K = 0.f, g_c = 0.f, b_c = 0.f, rm_c = 0.f, rv_c = 0.f;
    if (fin) {
        K = load_one<DT>(x, layout == kNCHW ? c * HW : c);
        g_c = gamma[c];
        b_c = beta[c];
        if (running_mean) { rm_c = running_mean[c]; rv_c = running_var[c]; }
    }
    double S1 = 0.0, S2 = 0.0;
    if (c < C) {
        // partials p = ph, ph + kFinPhases, ... in order; four at a time with their
        // loads issued together
        int64_t p = ph;
        for (; p + 3 * kFinPhases < P; p += 4 * kFinPhases) {
            float n[4], mu[4], m2[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t q = p + u * kFinPhases;
                n[u] = count[q];
                mu[u] = part_mean[q * C + c];
                m2[u] = part_m2[q * C + c];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const double nn = double(n[u]), mm = double(mu[u]);
                S1 = fma(nn, mm, S1);
                S2 += fma(nn * mm, mm, double(m2[u]));
            }
        }
        for (; p < P; p += kFinPhases) {
            const double n = double(count[p]);
            const double mu = double(part_mean[p * C + c]);
            S1 = fma(n, mu, S1);
            S2 += fma(n * mu, mu, double(part_m2[p * C + c]));
        }
    }
    __shared__ double sh1[kFinPhases][kFinChannels];
    __shared__ double sh2[kFinPhases][kFinChannels];
    sh1[ph][cl] = S1;
    sh2[ph][cl] = S2;
    __syncthreads();
    if (!fin) return;
    for (int k = 1; k < kFinPhases; ++k) { S1 += sh1[k][cl]; S2 += sh2[k][cl]; }
    const double mean = S1 / double(m);
    const double var = fmax(S2 - S1 * mean, 0.0) / double(m);
    const double invstd = 1.0 / sqrt(var + double(eps));
    const double mu = double(K) + mean;
    save_mean[c] = float(mu);
    save_invstd[c] = float(invstd);
    if (running_mean) {
        const double mom = double(momentum);
        running_mean[c] = float((1.0 - mom) * double(rm_c) + mom * mu);
        running_var[c] = float((1.0 - mom) * double(rv_c) + mom * var * double(m) / double(m - 1));
    }
    consts[c] = make_float4(K, float(mean), float(double(g_c) * invstd), b_c);
}

// ---------------------------------------------------------------------------
// Elementwise y = act(z), in place, z formed by the constants' own rule.
//
// Training reads (K, d, s, beta) from the workspace: z = ((x - K) - d)*s + beta,
// K a sample of the channel and d = mean - K, so every term stays on the scale
// of the channel's spread and z's error on that of the output.
//
// Inference forms z = (x - running_mean)*s + beta, s = gamma/sqrt(running_var +
// eps), from frozen statistics that need not lie near the data: the product and
// beta can cancel to outputs far smaller than either, where fp32 rounding of
// x - running_mean and of s would be seen.  So x - running_mean is kept exactly
// as a pair of floats (Knuth's two-sum), s as a pair (hi, lo) from an fp64
// reciprocal square root refined by one Newton step, the cancelling product and
// beta meet in one fused multiply-add, and the small terms come after it.
struct TrainConsts {
    const float4* consts;
    __device__ __forceinline__ float4 get(int64_t c) const { return consts[c]; }
    static __device__ __forceinline__ float z(float v, const float4& k)
    {
        return fmaf((v - k.x) - k.y, k.z, k.w);
    }
};
struct EvalConsts {
    const float* gamma;
    const float* beta;
    const float* rm;
    const float* rv;
    float eps;
    // (running_mean, s_lo, s_hi, beta)
    __device__ __forceinline__ float4 get(int64_t c) const
    {
        const double q = double(rv[c]) + double(eps);
        double r = __builtin_amdgcn_rsq(q);
        // the hardware estimate's relative error squared; 0 and inf stay as they
        // are (1/sqrt(0) = inf)
        if (q > 0.0 && q < __builtin_huge_val()) r *= fma(-0.5 * q * r, r, 1.5);
        const double sc = double(gamma[c]) * r;
        const float hi = float(sc);
        return make_float4(rm[c], float(sc - double(hi)), hi, beta[c]);
    }
    static __device__ __forceinline__ float z(float v, const float4& k)
    {
        const float dh = v - k.x;
        const float bb = dh - v;
        const float dl = (v - (dh - bb)) + (-k.x - bb);    // dh + dl == v - k.x
        const float z0 = fmaf(dh, k.z, k.w);
        // a non-finite difference leaves the terms' error undefined: z0 is the result
        return __builtin_isfinite(dh) ? z0 + fmaf(dh, k.y, dl * k.z) : z0;
    }
};

template <int ACT, int V, typename CS, bool P>
__device__ __forceinline__ void apply_one(float (&v)[V], const float4& k, float a)
{
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = act_forward<ACT, P>(CS::z(v[e], k), a);
}

template <int DT, int V, int ACT, typename CS>
__global__ __launch_bounds__(kThreads) void k_apply_nchw(
    void* x, int64_t nvec, int64_t C, int64_t HWv, CS cs, float a)
{
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    FlatNCHWWalk w;
    w.init(v < nvec ? v : 0, C, HWv, stride);
    for (; v + (kUnroll - 1) * stride < nvec; v += kUnroll * stride) {
        float val[kUnroll][V];
        float4 k[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            load_elems<DT, V>(x, (v + u * stride) * V, val[u]);
            k[u] = cs.get(w.c);
            w.step();
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            apply_one<ACT, V, CS, DT == kF32>(val[u], k[u], a);
            store_out<DT, V>(x, (v + u * stride) * V, val[u]);
        }
    }
    for (; v < nvec; v += stride) {
        float val[V];
        load_elems<DT, V>(x, v * V, val);
        const float4 k = cs.get(w.c);
        w.step();
        apply_one<ACT, V, CS, DT == kF32>(val, k, a);
        store_out<DT, V>(x, v * V, val);
    }
}

// NHWC: vector v covers channels (v % Cv)*V .. +V.  With FIXED the stride is a
// multiple of Cv and each thread loads its V channel constants once.
template <int DT, int V, int ACT, bool FIXED, typename CS>
__global__ __launch_bounds__(kThreads) void k_apply_nhwc(
    void* x, int64_t nvec, int64_t Cv, CS cs, float a)
{
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if constexpr (FIXED) {
        if (v >= nvec) return;
        const int64_t c0 = (v % Cv) * V;
        float4 k[V];
#pragma unroll
        for (int e = 0; e < V; ++e) k[e] = cs.get(c0 + e);
        if constexpr (IABN_APPLY_REVERSE) {
            // walk from the end of the tensor down: the rows the statistics pass read
            // last are the likeliest still to sit in the Infinity Cache.  (A software
            // pipeline, the next set's loads ahead of this set's stores as in the dx
            // pass, made this in-place pass slower: 99 against 87 us on a
            // 2x256x512x512 bf16 map.)
            const int64_t v0 = v;
            v = v0 + ((nvec - 1 - v0) / stride) * stride;
            for (; v - (kUnroll - 1) * stride >= v0; v -= kUnroll * stride) {
                float val[kUnroll][V];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) load_elems<DT, V>(x, (v - u * stride) * V, val[u]);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        val[u][e] = act_forward<ACT, DT == kF32>(CS::z(val[u][e], k[e]), a);
                    store_out<DT, V>(x, (v - u * stride) * V, val[u]);
                }
            }
            for (; v >= v0; v -= stride) {
                float val[V];
                load_elems<DT, V>(x, v * V, val);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    val[e] = act_forward<ACT, DT == kF32>(CS::z(val[e], k[e]), a);
                store_out<DT, V>(x, v * V, val);
            }
            return;
        }
        for (; v + (kUnroll - 1) * stride < nvec; v += kUnroll * stride) {
            float val[kUnroll][V];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) load_elems<DT, V>(x, (v + u * stride) * V, val[u]);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    val[u][e] = act_forward<ACT, DT == kF32>(CS::z(val[u][e], k[e]), a);
                store_out<DT, V>(x, (v + u * stride) * V, val[u]);
            }
        }
        for (; v < nvec; v += stride) {
            float val[V];
            load_elems<DT, V>(x, v * V, val);
#pragma unroll
            for (int e = 0; e < V; ++e)
                val[e] = act_forward<ACT, DT == kF32>(CS::z(val[e], k[e]), a);
            store_out<DT, V>(x, v * V, val);
        }
    } else {
        for (; v < nvec; v += stride) {
            const int64_t c0 = (v % Cv) * V;
            float val[V];
            load_elems<DT, V>(x, v * V, val);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float4 k = cs.get(c0 + e);
                val[e] = act_forward<ACT, DT == kF32>(CS::z(val[e], k), a);
            }
            store_elems<DT, V>(x, v * V, val);
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers

template <int DT, int V>
static void launch_stats_dv(const Plan& pl, const void* x, float* pa, float* pb, float* cnt,
                            hipStream_t s)
{
    if (pl.layout == kNCHW)
        hipLaunchKernelGGL((k_stats_nchw<DT, V>), dim3(pl.reduce_blocks), dim3(kThreads), 0, s,
                           x, pl.C, pl.HW, pl.m, pl.unit, pl.P, pa, pb, cnt);
    else
        hipLaunchKernelGGL((k_stats_nhwc<DT, V>), dim3(pl.reduce_blocks), dim3(kThreads), 0, s,
                           x, pl.m, pl.C / V, pl.tpr, pl.slices, pl.unit, pl.P, pa, pb, cnt);
}

void launch_forward_stats(const Plan& pl, const void* x, const float* gamma, const float* beta,
                          float* running_mean, float* running_var, float* save_mean,
                          float* save_invstd, float eps, float momentum, void* ws, hipStream_t s)
{
    char* wsb = static_cast<char*>(ws);
    float* pa = reinterpret_cast<float*>(wsb + pl.off_part_a);
    float* pb = reinterpret_cast<float*>(wsb + pl.off_part_b);
    float4* consts = reinterpret_cast<float4*>(wsb + pl.off_const);
    float* cnt = reinterpret_cast<float*>(wsb + pl.off_count);
    const dim3 grid(unsigned(ceil_div(pl.C, kFinChannels)));
    with_dtype(pl.dtype, [&](auto d) {
        constexpr int DT = decltype(d)::value;
        if (pl.vec) launch_stats_dv<DT, vec_width(DT)>(pl, x, pa, pb, cnt, s);
        else launch_stats_dv<DT, 1>(pl, x, pa, pb, cnt, s);
        hipLaunchKernelGGL((k_fwd_finalize<DT>), grid, dim3(kFinThreads), 0, s, x, pl.layout,
                           pl.C, pl.HW, pl.m, pl.P, pa, pb, cnt, gamma, beta, running_mean,
                           running_var, save_mean, save_invstd, eps, momentum, consts);
    });
}

template <int DT, int V, int ACT, typename CS>
static void launch_apply_dva(const Plan& pl, void* x, CS cs, float a, hipStream_t s)
{
    const int64_t nvec = pl.numel / V;
    const dim3 grid(unsigned(apply_grid(pl, ACT)));
    if (pl.layout == kNCHW)
        hipLaunchKernelGGL((k_apply_nchw<DT, V, ACT, CS>), grid, dim3(kThreads), 0, s, x, nvec,
                           pl.C, pl.HW / V, cs, a);
    else if (pl.fixed_col)
        hipLaunchKernelGGL((k_apply_nhwc<DT, V, ACT, true, CS>), grid, dim3(kThreads), 0, s, x,
                           nvec, pl.C / V, cs, a);
    else
        hipLaunchKernelGGL((k_apply_nhwc<DT, V, ACT, false, CS>), grid, dim3(kThreads), 0, s, x,
                           nvec, pl.C / V, cs, a);
}

template <int DT, int V, typename CS>
static void launch_apply_dv(const Plan& pl, void* x, CS cs, int act, float a, hipStream_t s)
{
    switch (act) {
    case kLeaky: launch_apply_dva<DT, V, kLeaky>(pl, x, cs, a, s); break;
    case kElu: launch_apply_dva<DT, V, kElu>(pl, x, cs, a, s); break;
    default: launch_apply_dva<DT, V, kIdentity>(pl, x, cs, a, s); break;
    }
}

template <typename CS>
static void launch_apply(const Plan& pl, void* x, CS cs, int act, float a, hipStream_t s)
{
    with_dtype(pl.dtype, [&](auto d) {
        constexpr int DT = decltype(d)::value;
        if (pl.vec) launch_apply_dv<DT, vec_width(DT)>(pl, x, cs, act, a, s);
        else launch_apply_dv<DT, 1>(pl, x, cs, act, a, s);
    });
}

void launch_forward_apply(const Plan& pl, void* x, int act, float a, void* ws, hipStream_t s)
{
    TrainConsts cs{reinterpret_cast<const float4*>(static_cast<char*>(ws) + pl.off_const)};
    launch_apply(pl, x, cs, act, a, s);
}

void launch_forward_eval(const Plan& pl, void* x, const float* gamma, const float* beta,
                         const float* rm, const float* rv, float eps, int act, float a,
                         hipStream_t s)
{
    EvalConsts cs{gamma, beta, rm, rv, eps};
    launch_apply(pl, x, cs, act, a, s);
}

}  // namespace iabn

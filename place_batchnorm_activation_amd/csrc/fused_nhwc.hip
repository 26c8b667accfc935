// Slice-resident NHWC kernels: one workgroup owns a slice of channels (LPR 16-byte
// lanes of every row, i.e. LPR*V channels) across all m rows and keeps it in VGPRs
// between the reduction and the elementwise pass -- the NHWC counterpart of the
// channel-resident NCHW kernels, for maps whose rows are short (small N*H*W) and
// whose channels are many.
//
// Forward (section 3 of the paperlayer summary of "In-Place Activated BatchNorm
// for Memory-Optimized Training of DNNs", "Batch Normalization Review" and
// "INPLACE-ABN"): sums of x - K and (x - K)^2 per channel, K the channel's first
// element (one pivot for the whole channel, so the sums simply add) -> fp64
// totals across the row slots -> statistics -> y from the registers, written
// over x (2S).
// Backward ("INPLACE-ABN" I/II, Appendix): y and dy resident; sums of dz and
// dz*(z - beta) -> per-channel constants -> dx (3S).
//
// Thread t owns lane t % LPR of the slice and rows t / LPR + k*RPS (RPS = T/LPR,
// k < NR).  Workgroups are mapped to slices XCD by XCD (nhwc_slice_of), so
// neighbouring slices -- which share cache lines when a slice is narrower than a
// line -- meet in one L2.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "fused.hpp"

namespace iabn {

namespace {

__device__ __forceinline__ uint32_t opaque_u(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ float opaque_f(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ uint4 opaque_q(uint4 q)
{
    asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
    return q;
}

__device__ __forceinline__ void st16_nt(void* base, uint32_t vec, const uint4& q)
{
    const u32x4_t v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(base) + vec);
}

// Workgroup totals over the row slots, stage one: threads t and t' hold the same
// channels when t % LPR == t' % LPR.  Inside the wave a reduce-scatter butterfly:
// at xor offset OFF (32, 16, ...) a lane keeps half of its NV values -- the upper
// half when lane & OFF -- and adds the partner's copy of that half, so it sends
// NV/2 + NV/4 + ... values rather than NV per level.  Once one value is left, the
// levels down to LPR are plain butterfly sums, in fp64.  Value q of lane position
// l then sits in lane (q << (6 - log2 NV)) | l of every wave; each lane leaves its
// value in sh[wave][lane] (the caller waits on the barrier).
template <int OFF, int LPR, int N>
struct ScatterLevels {
    static constexpr int kEnd = ScatterLevels<OFF / 2, LPR, N / 2>::kEnd;
    static __device__ __forceinline__ void run(float* a, uint32_t lane)
    {
        constexpr int H = N / 2;
        const bool up = (lane & OFF) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float send = up ? a[i] : a[i + H];
            const float keep = up ? a[i + H] : a[i];
            a[i] = keep + __shfl_xor(send, OFF, kWave);
        }
        ScatterLevels<OFF / 2, LPR, H>::run(a, lane);
    }
};

template <int OFF, int LPR>
struct ScatterLevels<OFF, LPR, 1> {
    static constexpr int kEnd = OFF;             // first plain level
    static __device__ __forceinline__ void run(float*, uint32_t) {}
};

template <int OFF, int LPR>
__device__ __forceinline__ double plain_levels(double a)
{
    if constexpr (OFF >= LPR && OFF >= 1) {
        a += __shfl_xor(a, OFF, kWave);
        return plain_levels<OFF / 2, LPR>(a);
    } else {
        return a;
    }
}

// Keeps values loaded at the top in registers up to this point, so the compiler
// cannot sink their loads into the code after the barrier (where each would cost a
// memory round trip on the critical path).
__device__ __forceinline__ void pin_loaded(float& a, float& b)
{
    asm volatile("" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ void pin_loaded(float& a, float& b, float& c)
{
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c));
}

// ok ? a : b on raw 16-byte vectors, as bit masks (a ?: on vectors tends to become
// a branch, and with it a wait for the load behind a).
__device__ __forceinline__ uint4 select16(bool ok, const uint4& a, const uint4& b)
{
    const uint32_t mk = 0u - uint32_t(ok);
    return make_uint4((a.x & mk) | (b.x & ~mk), (a.y & mk) | (b.y & ~mk),
                      (a.z & mk) | (b.z & ~mk), (a.w & mk) | (b.w & ~mk));
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

template <int LPR, int NV>
__device__ __forceinline__ void wave_scatter(float (&v)[NV], double (*sh)[kWave])
{
    static_assert((1 << ilog2(NV)) == NV && NV * LPR <= kWave, "values per lane position");
    const uint32_t lane = threadIdx.x & (kWave - 1);
    ScatterLevels<kWave / 2, LPR, NV>::run(v, lane);
    constexpr int kEnd = ScatterLevels<kWave / 2, LPR, NV>::kEnd;
    sh[threadIdx.x / kWave][lane] = plain_levels<kEnd, LPR>(double(v[0]));
}

// Stage two: the total of value q for lane position l, the waves summed in order.
template <int T, int NV>
__device__ __forceinline__ double lds_total(const double (*sh)[kWave], uint32_t q, uint32_t l)
{
    const uint32_t src = (q << (6 - ilog2(NV))) | l;
    double acc = sh[0][src];
#pragma unroll
    for (int w = 1; w < T / kWave; ++w) acc += sh[w][src];
    return acc;
}

}  // namespace

// ---------------------------------------------------------------------------
// One or two workgroups per CU at a time: the hint keeps the scheduler from
// trading loads in flight for an occupancy these kernels never reach.
#define IABN_SLICE_OCCUPANCY __attribute__((amdgpu_waves_per_eu(1, 2)))

template <int DT, int ACT, int T, int LPR, int NR>
__global__ __launch_bounds__(T) IABN_SLICE_OCCUPANCY void k_fwd_fused_nhwc(
    void* x, uint32_t m, uint32_t Cv, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* __restrict__ running_mean,
    float* __restrict__ running_var, float* __restrict__ save_mean,
    float* __restrict__ save_invstd, float eps, float momentum, float a)
{
    constexpr int V = Raw16<DT>::V;
    constexpr uint32_t RPS = T / LPR;
    const uint32_t slices = Cv / LPR;
    const uint32_t s = nhwc_slice_of(blockIdx.x, slices);
    const uint32_t t = threadIdx.x;
    const uint32_t lane = t % LPR, rs = t / LPR;
    const uint32_t col = s * LPR + lane;            // 16-byte vector column of the row
    const uint32_t c0 = col * V;                    // first channel of this thread
    const uint4* xv = reinterpret_cast<const uint4*>(x);

    // pivot K: row 0 of each channel, loaded first since every sum needs it.  Slots
    // past the last row load row m-1 (no branch); the sums below take K's bits for
    // them, which add exactly zero.
    const uint4 kraw = xv[col];
    __builtin_amdgcn_sched_barrier(0);
    uint4 r[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) r[k] = xv[min(rs + k * RPS, m - 1) * Cv + col];
    // Per-channel values for the finishing threads, loaded last (they are needed
    // last) but up front, so that no global load sits between the two barriers:
    // thread t < V*LPR finishes channel cf.  Unconditional loads (the other threads
    // read channel 0): a branch would wait for them on the spot.
    const bool fin = t < V * LPR;
    const uint32_t cf = fin ? (s * LPR + t % LPR) * V + t / LPR : 0;
    uint32_t k_bits = DT == kF32 ? static_cast<const uint32_t*>(x)[cf]
                                 : uint32_t(static_cast<const uint16_t*>(x)[cf]);
    float g_f = gamma[cf];
    const float* rm_src = running_mean ? running_mean : gamma;
    const float* rv_src = running_mean ? running_var : gamma;
    float rm_f = rm_src[cf], rv_f = rv_src[cf];
    float b_c[V];
#pragma unroll
    for (int e = 0; e < V; ++e) b_c[e] = beta[c0 + e];
    // every load above is issued before any of the arithmetic below (a select or a
    // conversion next to a load would make the compiler wait for it there)
    __builtin_amdgcn_sched_barrier(0);

    float K[V];
    unpack16<DT>(kraw, K);

    float sums[2 * V];
#pragma unroll
    for (int e = 0; e < 2 * V; ++e) sums[e] = 0.f;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        float v[V];
        unpack16<DT>(select16(rs + k * RPS < m, r[k], kraw), v);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float d = v[e] - K[e];
            sums[e] += d;
            sums[V + e] = fmaf(d, d, sums[V + e]);
        }
    }
    __shared__ double sh[T / kWave][kWave];
    __shared__ float coef[2][V][LPR];
    pin_loaded(g_f, rm_f, rv_f);
    asm volatile("" : "+v"(k_bits));
    wave_scatter<LPR, 2 * V>(sums, sh);
    __syncthreads();

    // statistics in fp64, one thread per channel: d = mean - K, M2 = S2 - S1*d
    if (fin) {
        const uint32_t e = t / LPR, l = t % LPR;
        const double S1 = lds_total<T, 2 * V>(sh, e, l);
        const double S2 = lds_total<T, 2 * V>(sh, V + e, l);
        const double md = double(m);
        const double dm = S1 / md;
        const double var = fmax(S2 - S1 * dm, 0.0) / md;
        const double invstd = 1.0 / sqrt(var + double(eps));
        const double mu = double(DT == kF32 ? __uint_as_float(k_bits) : unpack1<DT>(uint16_t(k_bits))) + dm;
        save_mean[cf] = float(mu);
        save_invstd[cf] = float(invstd);
        if (running_mean) {
            const double mom = double(momentum);
            running_mean[cf] = float((1.0 - mom) * double(rm_f) + mom * mu);
            running_var[cf] = float((1.0 - mom) * double(rv_f) + mom * var * md / (md - 1.0));
        }
        coef[0][e][l] = float(dm);
        coef[1][e][l] = float(double(g_f) * invstd);
    }
    __syncthreads();
    float d[V], sc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        d[e] = coef[0][e][lane];
        sc[e] = coef[1][e][lane];
    }

    const uint32_t rs2 = opaque_u(rs);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const uint32_t row = rs2 + k * RPS;
        float v[V];
        unpack16<DT>(opaque_q(r[k]), v);
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = act_forward<ACT>(fmaf((v[e] - K[e]) - d[e], sc[e], b_c[e]), a);
        if (row < m) st16_nt(x, row * Cv + col, pack16<DT>(v));
    }
}

// ---------------------------------------------------------------------------
template <int DT, int ACT, int T, int LPR, int NR>
__global__ __launch_bounds__(T) IABN_SLICE_OCCUPANCY void k_bwd_fused_nhwc(
    const void* __restrict__ y, const void* dy, void* dx, uint32_t m, uint32_t Cv,
    const float* __restrict__ gamma, const float* __restrict__ beta,
    const float* __restrict__ invstd, float* __restrict__ dgamma, float* __restrict__ dbeta,
    float a, float inv_a)
{
    constexpr int V = Raw16<DT>::V;
    constexpr uint32_t RPS = T / LPR;
    const uint32_t slices = Cv / LPR;
    const uint32_t s = nhwc_slice_of(blockIdx.x, slices);
    const uint32_t t = threadIdx.x;
    const uint32_t lane = t % LPR, rs = t / LPR;
    const uint32_t col = s * LPR + lane;
    const uint32_t c0 = col * V;
    const uint4* yv = reinterpret_cast<const uint4*>(y);
    const uint4* dv = reinterpret_cast<const uint4*>(dy);

    // per-channel values for the finishing threads, fetched up front
    const bool fin = t < V * LPR;
    const uint32_t cf = fin ? (s * LPR + t % LPR) * V + t / LPR : 0;
    float g_f = gamma[cf], i_f = invstd[cf];

    // slots past the last row load row m-1 (no branch); the sums below take
    // dy = 0 for them, so dz = 0 adds exactly zero
    uint4 ry[NR], rd[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const uint32_t i = min(rs + k * RPS, m - 1) * Cv + col;
        ry[k] = yv[i];
        rd[k] = dv[i];
    }
    // every load above is issued before any of the arithmetic below
    __builtin_amdgcn_sched_barrier(0);
    float b_c[V];
#pragma unroll
    for (int e = 0; e < V; ++e) b_c[e] = beta[c0 + e];

    float sums[2 * V];
#pragma unroll
    for (int e = 0; e < 2 * V; ++e) sums[e] = 0.f;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        float vy[V], vd[V];
        unpack16<DT>(ry[k], vy);
        unpack16<DT>(select16(rs + k * RPS < m, rd[k], make_uint4(0, 0, 0, 0)), vd);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float z, slope;
            act_invert<ACT>(vy[e], a, inv_a, z, slope);
            const float dz = slope * vd[e];
            sums[e] += dz;
            sums[V + e] = fmaf(dz, z - b_c[e], sums[V + e]);
        }
    }
    __shared__ double sh[T / kWave][kWave];
    __shared__ float coef[3][V][LPR];
    pin_loaded(g_f, i_f);
    wave_scatter<LPR, 2 * V>(sums, sh);
    __syncthreads();

    // per-channel constants in fp64, one thread per channel
    if (fin) {
        const uint32_t e = t / LPR, l = t % LPR;
        const double db = lds_total<T, 2 * V>(sh, e, l);
        const double g = double(g_f);
        const double dg = lds_total<T, 2 * V>(sh, V + e, l) / g;
        dbeta[cf] = float(db);
        dgamma[cf] = float(dg);
        const double A = g * double(i_f);
        const double md = double(m);
        coef[0][e][l] = float(A);
        coef[1][e][l] = float(-A * dg / (md * g));
        coef[2][e][l] = float(-A * db / md);
    }
    __syncthreads();
    float kA[V], kB[V], kC[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        kA[e] = coef[0][e][lane];
        kB[e] = coef[1][e][lane];
        kC[e] = coef[2][e][lane];
    }

    const uint32_t rs2 = opaque_u(rs);
    const float a2 = opaque_f(a), ia2 = opaque_f(inv_a);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const uint32_t row = rs2 + k * RPS;
        float vy[V], vd[V];
        unpack16<DT>(opaque_q(ry[k]), vy);
        unpack16<DT>(opaque_q(rd[k]), vd);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float z, slope;
            act_invert<ACT>(vy[e], a2, ia2, z, slope);
            const float dz = slope * vd[e];
            vd[e] = fmaf(kA[e], dz, fmaf(kB[e], z - b_c[e], kC[e]));
        }
        if (row < m) st16_nt(dx, row * Cv + col, pack16<DT>(vd));
    }
}

// ---------------------------------------------------------------------------
// host side

template <int DT, int ACT>
static void launch_nhwc_fwd_da(const Plan& pl, void* x, const float* gamma, const float* beta,
                               float* rm, float* rv, float* sm, float* si, float eps, float mom,
                               float a, hipStream_t s)
{
    const uint32_t m = uint32_t(pl.m), Cv = uint32_t(pl.C / pl.V);
    switch (pl.nhwc_variant) {
#define IABN_CASE(ID, T, LPR, NR)                                                                  \
    case ID:                                                                                       \
        hipLaunchKernelGGL((k_fwd_fused_nhwc<DT, ACT, T, LPR, NR>), dim3(Cv / LPR), dim3(T), 0, s, \
                           x, m, Cv, gamma, beta, rm, rv, sm, si, eps, mom, a);                    \
        break;
        IABN_FUSED_NHWC_VARIANTS(IABN_CASE)
#undef IABN_CASE
    default: break;
    }
}

void launch_forward_fused_nhwc(const Plan& pl, void* x, const float* gamma, const float* beta,
                               float* rm, float* rv, float* sm, float* si, float eps, float mom,
                               int act, float a, hipStream_t s)
{
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            launch_nhwc_fwd_da<decltype(d)::value, decltype(ac)::value>(
                pl, x, gamma, beta, rm, rv, sm, si, eps, mom, a, s);
        });
    });
}

template <int DT, int ACT>
static void launch_nhwc_bwd_da(const Plan& pl, const void* y, const void* dy, void* dx,
                               const float* gamma, const float* beta, const float* invstd,
                               float* dgamma, float* dbeta, float a, float ia, hipStream_t s)
{
    const uint32_t m = uint32_t(pl.m), Cv = uint32_t(pl.C / pl.V);
    switch (pl.nhwc_variant) {
#define IABN_CASE(ID, T, LPR, NR)                                                                  \
    case ID:                                                                                       \
        hipLaunchKernelGGL((k_bwd_fused_nhwc<DT, ACT, T, LPR, NR>), dim3(Cv / LPR), dim3(T), 0, s, \
                           y, dy, dx, m, Cv, gamma, beta, invstd, dgamma, dbeta, a, ia);           \
        break;
        IABN_FUSED_NHWC_VARIANTS(IABN_CASE)
#undef IABN_CASE
    default: break;
    }
}

void launch_backward_fused_nhwc(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* invstd,
                                float* dgamma, float* dbeta, int act, float a, hipStream_t s)
{
    const float ia = act == kIdentity ? 1.f : 1.f / a;
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            launch_nhwc_bwd_da<decltype(d)::value, decltype(ac)::value>(
                pl, y, dy, dx, gamma, beta, invstd, dgamma, dbeta, a, ia, s);
        });
    });
}

}  // namespace iabn

// Channel-resident NCHW kernels: one workgroup owns one channel and keeps its
// data in VGPRs between the reduction and the elementwise pass, so there are no
// partials, no finishing launch and no second read of the same bytes.
//
// Forward (section 3 of the paperlayer summary of "In-Place Activated BatchNorm
// for Memory-Optimized Training of DNNs", "Batch Normalization Review" and
// "INPLACE-ABN"): load the channel, pivot-shifted sums -> Chan merge across the
// workgroup -> statistics in fp64 -> y = act(((x - K) - d)*s + beta) from the
// registers, written over x.  HBM traffic: read S, write S.
//
// Backward ("INPLACE-ABN" I/II, Appendix): y (and dy when it fits) stay
// resident; sums of dz and dz*(z - beta) -> per-channel constants -> dx.  When
// dy does not fit it is streamed twice.  HBM traffic: 3S, or 4S with dy
// streamed.
//
// Thread t of the workgroup owns the channel's 16-byte vectors j = t + k*T,
// k < NR.  Addresses are 32-bit byte offsets from the uniform tensor base (the
// plan only picks these kernels for tensors under 4 GiB), one VGPR per vector.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "fused.hpp"
#include "group.hpp"

namespace iabn {

__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off)
{
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + (off << 4));
}

__device__ __forceinline__ void st16(void* base, uint32_t off, const uint4& q)
{
    if constexpr (IABN_FUSED_NT_STORE) {
        const u32x4_t v = {q.x, q.y, q.z, q.w};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(static_cast<char*>(base) + (off << 4)));
    } else {
        *reinterpret_cast<uint4*>(static_cast<char*>(base) + (off << 4)) = q;
    }
}

// A copy of v the compiler cannot see through: the second pass recomputes its
// addresses instead of keeping the first pass's offsets alive in VGPRs.
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ float opaquef(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Same for a resident vector: its unpacked / transformed values are recomputed in
// the second pass rather than kept from the first.
__device__ __forceinline__ uint4 opaque4(uint4 q)
{
    asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
    return q;
}

// Streamed loads are issued in groups of kStreamGroup; the compiler may not hoist
// loads across the group boundary, which bounds the VGPRs they occupy.
constexpr int kStreamGroup = 4;

__device__ __forceinline__ void group_fence() { asm volatile("" ::: "memory"); }

// Block-wide Chan merge; every thread returns the workgroup's (n, mean, M2).
template <int T>
__device__ __forceinline__ void block_chan(float& n, float& mean, float& m2)
{
    constexpr int NW = T / kWave;
    __shared__ float sh[3][NW];
    wave_chan(n, mean, m2);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) { sh[0][wave] = n; sh[1][wave] = mean; sh[2][wave] = m2; }
    __syncthreads();
    float tn = sh[0][0], tm = sh[1][0], t2 = sh[2][0];
#pragma unroll
    for (int k = 1; k < NW; ++k) chan_merge(tn, tm, t2, sh[0][k], sh[1][k], sh[2][k]);
    n = tn; mean = tm; m2 = t2;
}

// Block-wide sums in a fixed order; every thread returns the totals.
template <int T>
__device__ __forceinline__ void block_sum2(float& a, float& b)
{
    constexpr int NW = T / kWave;
    __shared__ float sh[2][NW];
    a = wave_sum(a);
    b = wave_sum(b);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) { sh[0][wave] = a; sh[1][wave] = b; }
    __syncthreads();
    float ta = sh[0][0], tb = sh[1][0];
#pragma unroll
    for (int k = 1; k < NW; ++k) { ta += sh[0][k]; tb += sh[1][k]; }
    a = ta; b = tb;
}

// A grouped forward whose share takes nearly all the registers (49 vectors a
// thread) compiles only the one-level exchange: with the two-level path in, it
// spilled about 24 VGPRs around the exchange.  The plan never gives it a group
// of kTwoLevelGroup members or more (fused_nchw_group_pick).
template <int NR>
constexpr bool kFwdTwoLevel = NR <= 32;

// ---------------------------------------------------------------------------
template <int DT, int ACT, int T, int NR, bool GRP>
__global__ __launch_bounds__(T) void k_fwd_fused_nchw(
    void* x, uint32_t C, uint32_t HW, uint32_t m, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* __restrict__ running_mean,
    float* __restrict__ running_var, float* __restrict__ save_mean,
    float* __restrict__ save_invstd, float eps, float momentum, float a, SliceGroup grp)
{
    constexpr int V = Raw16<DT>::V;
    // channel and member: with GRP a group of G workgroups shares a channel,
    // member j holding the channel's vectors [j*mg, min(Vc, (j+1)*mg)); without,
    // one workgroup holds it all (and the kernel carries no exchange code)
    const uint32_t c = GRP ? blockIdx.x / grp.G : blockIdx.x;
    const uint32_t member = GRP ? blockIdx.x - c * grp.G : 0u;
    const uint32_t t = threadIdx.x;
    const uint32_t HWv = HW / V;
    const uint32_t Vc = m / V;
    const uint32_t v0 = GRP ? member * grp.mg : 0u;
    const uint32_t v1 = GRP ? min(Vc, v0 + grp.mg) : Vc;
    const float K = load_one<DT>(x, int64_t(c) * HW);
    // per-channel parameters fetched up front, off the critical path
    const float g_c = gamma[c];
    const float b = beta[c];
    float rm_c = 0.f, rv_c = 0.f;
    if (t == 0 && running_mean) { rm_c = running_mean[c]; rv_c = running_var[c]; }

    uint64_t epoch = 0;
    if (GRP && t == 0) epoch = atomic_ld(grp.xchg + c);
    uint4 r[NR];
    ChannelWalk32 w;
    w.init(v0 + t, c, C, HWv, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        r[k] = (v0 + t + k * T < v1) ? ld16(x, w.off) : make_uint4(0, 0, 0, 0);
        w.step();
    }

    float s1[V], s2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) { s1[e] = 0.f; s2[e] = 0.f; }
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if (v0 + t + k * T < v1) {
            float v[V];
            unpack16<DT>(r[k], v);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float d = v[e] - K;
                s1[e] += d;
                s2[e] = fmaf(d, d, s2[e]);
            }
            ++cnt;
        }
    }
    float S1 = 0.f, S2 = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) { S1 += s1[e]; S2 += s2[e]; }
    float n = float(cnt * V);
    float mean = cnt ? S1 / n : 0.f;
    float m2 = cnt ? fmaxf(S2 - S1 * mean, 0.f) : 0.f;
    __shared__ uint64_t tok_sh;
    if (GRP && t == 0) tok_sh = group_token(grp, c, epoch);
    block_chan<T>(n, mean, m2);

    // statistics in fp64 (every thread computes the same values).  A group adds
    // its members' shifted sums, sum(x - K) = n*mean and sum((x - K)^2) = M2 +
    // n*mean^2, in fp64 and in a fixed order (group_sums).
    double dm = double(mean), var = double(m2) / double(m);
    if constexpr (GRP) {
        __shared__ double tot_sh[2];
        double s1 = double(n) * double(mean);
        double s2 = double(m2) + double(n) * double(mean) * double(mean);
        group_sums<1, T, (kFwdTwoLevel<NR> ? 4 : 1), kFwdTwoLevel<NR>>(grp, c, C, member, tok_sh,
                                                                  t == 0, s1, s2);
        if (t == 0) {
            tot_sh[0] = s1;
            tot_sh[1] = s2;
        }
        __syncthreads();
        const double md = double(m);
        dm = tot_sh[0] / md;
        var = fmax(tot_sh[1] - tot_sh[0] * dm, 0.0) / md;
        if (member == 0 && t == 0) atomic_st(grp.xchg + c, epoch + 1);
    }
    const double invstd = 1.0 / sqrt(var + double(eps));
    const float d = float(dm);
    const float s = float(double(g_c) * invstd);
    if (t == 0 && member == 0) {
        const double mu = double(K) + dm;
        save_mean[c] = float(mu);
        save_invstd[c] = float(invstd);
        if (running_mean) {
            const double mom = double(momentum);
            running_mean[c] = float((1.0 - mom) * double(rm_c) + mom * mu);
            running_var[c] = float((1.0 - mom) * double(rv_c) + mom * var * double(m) / double(m - 1));
        }
    }

    const uint32_t t2 = opaque(t);
    w.init(v0 + t2, c, C, HWv, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if (v0 + t2 + k * T < v1) {
            float v[V];
            unpack16<DT>(opaque4(r[k]), v);
#pragma unroll
            for (int e = 0; e < V; ++e) v[e] = act_forward<ACT, DT == kF32>(fmaf((v[e] - K) - d, s, b), a);
            st16(x, w.off, pack16<DT>(v));
        }
        w.step();
    }
}

// ---------------------------------------------------------------------------
// DYR: dy resident as well (3S); otherwise dy is streamed twice (4S).
template <int DT, int ACT, int T, int NR, bool DYR>
__global__ __launch_bounds__(T) void k_bwd_fused_nchw(
    const void* __restrict__ y, const void* dy, void* dx, uint32_t C, uint32_t HW, uint32_t m,
    const float* __restrict__ gamma, const float* __restrict__ beta,
    const float* __restrict__ invstd, float* __restrict__ dgamma, float* __restrict__ dbeta,
    float a, float inv_a)
{
    constexpr int V = Raw16<DT>::V;
    const uint32_t c = blockIdx.x;
    const uint32_t t = threadIdx.x;
    const uint32_t HWv = HW / V;
    const uint32_t Vc = m / V;
    const float bc = beta[c];
    const float g_c = gamma[c];
    const float is_c = invstd[c];

    constexpr bool kKeepZ = DYR && DT == kF32;
    uint4 ry[NR];
    uint4 rd[DYR ? NR : 1];
    ChannelWalk32 w;
    w.init(t, c, C, HWv, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const bool ok = t + k * T < Vc;
        ry[k] = ok ? ld16(y, w.off) : make_uint4(0, 0, 0, 0);
        if constexpr (DYR) rd[k] = ok ? ld16(dy, w.off) : make_uint4(0, 0, 0, 0);
        w.step();
    }
    float sdz = 0.f, sdzt = 0.f;
    const uint32_t t1 = opaque(t);
    if constexpr (!DYR) w.init(t1, c, C, HWv, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if constexpr (!DYR) if (k % kStreamGroup == 0) group_fence();
        if (t1 + k * T < Vc) {
            float vy[V], vd[V];
            unpack16<DT>(ry[k], vy);
            if constexpr (DYR) unpack16<DT>(rd[k], vd);
            else unpack16<DT>(ld16(dy, w.off), vd);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float z, slope;
                act_invert<ACT, DT == kF32>(vy[e], a, inv_a, z, slope);
                const float dz = slope * vd[e];
                sdz += dz;
                sdzt = fmaf(dz, z - bc, sdzt);
                vy[e] = z;
                vd[e] = dz;
            }
            // fp32 storage with dy resident: z and dz take the places of y and dy,
            // so the dx pass does not invert the activation again (ELU: a log1p
            // an element)
            if constexpr (kKeepZ) {
                ry[k] = pack16<DT>(vy);
                rd[k] = pack16<DT>(vd);
            }
        }
        if constexpr (!DYR) w.step();
    }
    block_sum2<T>(sdz, sdzt);

    const double g = double(g_c);
    const double db = double(sdz);
    const double dg = double(sdzt) / g;
    if (t == 0) {
        dbeta[c] = float(db);
        dgamma[c] = float(dg);
    }
    const double A = g * double(is_c);
    const double md = double(m);
    const float kA = float(A), kB = float(-A * dg / (md * g)), kC = float(-A * db / md);

    const uint32_t t2 = opaque(t);
    const float a2 = opaquef(a), ia2 = opaquef(inv_a), bc2 = opaquef(bc);
    w.init(t2, c, C, HWv, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if constexpr (!DYR) if (k % kStreamGroup == 0) group_fence();
        if (t2 + k * T < Vc) {
            float vy[V], vd[V];
            unpack16<DT>(opaque4(ry[k]), vy);
            if constexpr (DYR) unpack16<DT>(opaque4(rd[k]), vd);
            else unpack16<DT>(ld16(dy, w.off), vd);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float z, dz;
                if constexpr (kKeepZ) {
                    z = vy[e];
                    dz = vd[e];
                } else {
                    float slope;
                    act_invert<ACT, DT == kF32>(vy[e], a2, ia2, z, slope);
                    dz = slope * vd[e];
                }
                vd[e] = fmaf(kA, dz, fmaf(kB, z - bc2, kC));
            }
            st16(dx, w.off, pack16<DT>(vd));
        }
        w.step();
    }
}

// ---------------------------------------------------------------------------
// Backward for channels too large to keep y and dy both on chip: y stays
// resident (NRV vectors per thread in VGPRs, NRL in LDS) and dy is streamed
// twice, through a two-group software pipeline: the G loads of the next group
// are in flight while the current group is consumed.  HBM traffic 4S.
template <int DT, int ACT, int T, int NRV, int NRL, int G, bool GRP>
__global__ __launch_bounds__(T) void k_bwd_stream_nchw(
    const void* __restrict__ y, const void* dy, void* dx, uint32_t C, uint32_t HW, uint32_t m,
    const float* __restrict__ gamma, const float* __restrict__ beta,
    const float* __restrict__ invstd, float* __restrict__ dgamma, float* __restrict__ dbeta,
    float a, float inv_a, SliceGroup grp)
{
    constexpr int V = Raw16<DT>::V;
    constexpr int NR = NRV + NRL;
    constexpr int NG = (NR + G - 1) / G;
    __shared__ uint4 ly[NRL > 0 ? NRL * T : 1];
    // channel and member, as in the forward
    const uint32_t c = GRP ? blockIdx.x / grp.G : blockIdx.x;
    const uint32_t member = GRP ? blockIdx.x - c * grp.G : 0u;
    const uint32_t t = threadIdx.x;
    const uint32_t HWv = HW / V;
    const uint32_t Vc = m / V;
    const uint32_t v0 = GRP ? member * grp.mg : 0u;
    const uint32_t v1 = GRP ? min(Vc, v0 + grp.mg) : Vc;
    uint64_t epoch = 0;
    if (GRP && t == 0) epoch = atomic_ld(grp.xchg + c);
    const float bc = beta[c];
    const float g_c = gamma[c];
    const float is_c = invstd[c];

    // y: registers, then this thread's own LDS slots (read back only by this thread)
    uint4 ry[NRV];
    ChannelWalk32 w;
    w.init(v0 + t, c, C, HWv, T);
#pragma unroll
    for (int k = 0; k < NRV; ++k) {
        ry[k] = (v0 + t + k * T < v1) ? ld16(y, w.off) : make_uint4(0, 0, 0, 0);
        w.step();
    }
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
        if (v0 + t + (NRV + k) * T < v1) ly[k * T + t] = ld16(y, w.off);
        w.step();
    }

    // pass 1: sums over dy streamed in groups of G
    float sdz = 0.f, sdzt = 0.f;
    {
        const uint32_t t1 = opaque(t), u1 = v0 + t1;   // thread; its first channel vector
        ChannelWalk32 wd;
        wd.init(u1, c, C, HWv, T);
        uint4 buf[2][G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            buf[0][i] = (i < NR && u1 + i * T < v1) ? ld16(dy, wd.off) : make_uint4(0, 0, 0, 0);
            wd.step();
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            group_fence();
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int k = (gi + 1) * G + i;
                if (k < NR) {
                    buf[(gi + 1) & 1][i] = (u1 + k * T < v1) ? ld16(dy, wd.off) : make_uint4(0, 0, 0, 0);
                    wd.step();
                }
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int k = gi * G + i;
                if (k < NR && u1 + k * T < v1) {
                    float vy[V], vd[V];
                    unpack16<DT>(k < NRV ? ry[k < NRV ? k : 0] : ly[(k >= NRV ? k - NRV : 0) * T + t1], vy);
                    unpack16<DT>(buf[gi & 1][i], vd);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        float z, slope;
                        act_invert<ACT, DT == kF32>(vy[e], a, inv_a, z, slope);
                        const float dz = slope * vd[e];
                        sdz += dz;
                        sdzt = fmaf(dz, z - bc, sdzt);
                    }
                }
            }
        }
    }
    __shared__ uint64_t tok_sh;
    if (GRP && t == 0) tok_sh = group_token(grp, c, epoch);
    block_sum2<T>(sdz, sdzt);

    // a group adds its members' sums in fp64, in a fixed order (group_sums)
    double sum_dz = double(sdz), sum_dzt = double(sdzt);
    if constexpr (GRP) {
        __shared__ double tot_sh[2];
        group_sums<1, T, 2>(grp, c, C, member, tok_sh, t == 0, sum_dz, sum_dzt);
        if (t == 0) {
            tot_sh[0] = sum_dz;
            tot_sh[1] = sum_dzt;
        }
        __syncthreads();
        sum_dz = tot_sh[0];
        sum_dzt = tot_sh[1];
        if (member == 0 && t == 0) atomic_st(grp.xchg + c, epoch + 1);
    }
    const double g = double(g_c);
    const double db = sum_dz;
    const double dg = sum_dzt / g;
    if (t == 0 && member == 0) {
        dbeta[c] = float(db);
        dgamma[c] = float(dg);
    }
    const double A = g * double(is_c);
    const double md = double(m);
    const float kA = float(A), kB = float(-A * dg / (md * g)), kC = float(-A * db / md);

    // pass 2: dy streamed again, dx written
    {
        const uint32_t t2 = opaque(t), u2 = v0 + t2;
        const float a2 = opaquef(a), ia2 = opaquef(inv_a), bc2 = opaquef(bc);
        ChannelWalk32 wd, wx;
        wd.init(u2, c, C, HWv, T);
        wx.init(u2, c, C, HWv, T);
        uint4 buf[2][G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            buf[0][i] = (i < NR && u2 + i * T < v1) ? ld16(dy, wd.off) : make_uint4(0, 0, 0, 0);
            wd.step();
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            group_fence();
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int k = (gi + 1) * G + i;
                if (k < NR) {
                    buf[(gi + 1) & 1][i] = (u2 + k * T < v1) ? ld16(dy, wd.off) : make_uint4(0, 0, 0, 0);
                    wd.step();
                }
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int k = gi * G + i;
                if (k < NR) {
                    if (u2 + k * T < v1) {
                        float vy[V], vd[V];
                        unpack16<DT>(k < NRV ? opaque4(ry[k < NRV ? k : 0])
                                           : ly[(k >= NRV ? k - NRV : 0) * T + t2], vy);
                        unpack16<DT>(buf[gi & 1][i], vd);
#pragma unroll
                        for (int e = 0; e < V; ++e) {
                            float z, slope;
                            act_invert<ACT, DT == kF32>(vy[e], a2, ia2, z, slope);
                            const float dz = slope * vd[e];
                            vd[e] = fmaf(kA, dz, fmaf(kB, z - bc2, kC));
                        }
                        st16(dx, wx.off, pack16<DT>(vd));
                    }
                    wx.step();
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Channel-resident kernels on single elements (planes whose length is not a
// multiple of the vector width, or pointers off 16-byte alignment).  Thread t
// owns channel-local elements j = t + k*T, k < NR, walked with ChannelWalk32 in
// element units; each element's raw bits stay in one VGPR between the passes.

template <int DT>
__device__ __forceinline__ uint32_t ld_elem(const void* base, uint32_t off)
{
    if constexpr (DT == kF32) return static_cast<const uint32_t*>(base)[off];
    else return static_cast<const uint16_t*>(base)[off];
}

template <int DT>
__device__ __forceinline__ float elem_float(uint32_t bits)
{
    if constexpr (DT == kF32) return __uint_as_float(bits);
    else return unpack1<DT>(uint16_t(bits));
}

template <int DT>
__device__ __forceinline__ void st_elem(void* base, uint32_t off, float v)
{
    if constexpr (DT == kF32) {
        float* p = static_cast<float*>(base) + off;
        if constexpr (IABN_FUSED_NT_STORE) __builtin_nontemporal_store(v, p);
        else *p = v;
    } else {
        uint16_t* p = static_cast<uint16_t*>(base) + off;
        if constexpr (IABN_FUSED_NT_STORE) __builtin_nontemporal_store(pack1<DT>(v), p);
        else *p = pack1<DT>(v);
    }
}

template <int DT, int ACT, int T, int NR>
__global__ __launch_bounds__(T) void k_fwd_fused_nchw_s(
    void* x, uint32_t C, uint32_t HW, uint32_t m, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* __restrict__ running_mean,
    float* __restrict__ running_var, float* __restrict__ save_mean,
    float* __restrict__ save_invstd, float eps, float momentum, float a)
{
    const uint32_t c = blockIdx.x;
    const uint32_t t = threadIdx.x;
    const float K = load_one<DT>(x, int64_t(c) * HW);
    const float g_c = gamma[c];
    const float b = beta[c];
    float rm_c = 0.f, rv_c = 0.f;
    if (t == 0 && running_mean) { rm_c = running_mean[c]; rv_c = running_var[c]; }

    uint32_t r[NR];
    ChannelWalk32 w;
    w.init(t, c, C, HW, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        r[k] = (t + k * T < m) ? ld_elem<DT>(x, w.off) : 0u;
        w.step();
    }
    float s1 = 0.f, s2 = 0.f;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if (t + k * T < m) {
            const float d = elem_float<DT>(r[k]) - K;
            s1 += d;
            s2 = fmaf(d, d, s2);
            ++cnt;
        }
    }
    float n = float(cnt);
    float mean = cnt ? s1 / n : 0.f;
    float m2 = cnt ? fmaxf(s2 - s1 * mean, 0.f) : 0.f;
    block_chan<T>(n, mean, m2);

    const double var = double(m2) / double(m);
    const double invstd = 1.0 / sqrt(var + double(eps));
    const float d = float(mean);
    const float sc = float(double(g_c) * invstd);
    if (t == 0) {
        const double mu = double(K) + double(mean);
        save_mean[c] = float(mu);
        save_invstd[c] = float(invstd);
        if (running_mean) {
            const double mom = double(momentum);
            running_mean[c] = float((1.0 - mom) * double(rm_c) + mom * mu);
            running_var[c] = float((1.0 - mom) * double(rv_c) + mom * var * double(m) / double(m - 1));
        }
    }

    const uint32_t t2 = opaque(t);
    w.init(t2, c, C, HW, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if (t2 + k * T < m) {
            const float v = elem_float<DT>(opaque(r[k]));
            st_elem<DT>(x, w.off, act_forward<ACT, DT == kF32>(fmaf((v - K) - d, sc, b), a));
        }
        w.step();
    }
}

template <int DT, int ACT, int T, int NR>
__global__ __launch_bounds__(T) void k_bwd_fused_nchw_s(
    const void* __restrict__ y, const void* dy, void* dx, uint32_t C, uint32_t HW, uint32_t m,
    const float* __restrict__ gamma, const float* __restrict__ beta,
    const float* __restrict__ invstd, float* __restrict__ dgamma, float* __restrict__ dbeta,
    float a, float inv_a)
{
    const uint32_t c = blockIdx.x;
    const uint32_t t = threadIdx.x;
    const float bc = beta[c];
    const float g_c = gamma[c];
    const float is_c = invstd[c];

    uint32_t ry[NR], rd[NR];
    ChannelWalk32 w;
    w.init(t, c, C, HW, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const bool ok = t + k * T < m;
        ry[k] = ok ? ld_elem<DT>(y, w.off) : 0u;
        rd[k] = ok ? ld_elem<DT>(dy, w.off) : 0u;
        w.step();
    }
    // every element sits in a 32-bit register of its own: z and dz take the
    // places of y and dy, so the dx pass does not invert the activation again
    float sdz = 0.f, sdzt = 0.f;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if (t + k * T < m) {
            float z, slope;
            act_invert<ACT, DT == kF32>(elem_float<DT>(ry[k]), a, inv_a, z, slope);
            const float dz = slope * elem_float<DT>(rd[k]);
            sdz += dz;
            sdzt = fmaf(dz, z - bc, sdzt);
            ry[k] = __float_as_uint(z);
            rd[k] = __float_as_uint(dz);
        }
    }
    block_sum2<T>(sdz, sdzt);

    const double g = double(g_c);
    const double db = double(sdz);
    const double dg = double(sdzt) / g;
    if (t == 0) {
        dbeta[c] = float(db);
        dgamma[c] = float(dg);
    }
    const double A = g * double(is_c);
    const double md = double(m);
    const float kA = float(A), kB = float(-A * dg / (md * g)), kC = float(-A * db / md);

    const uint32_t t2 = opaque(t);
    const float bc2 = opaquef(bc);
    w.init(t2, c, C, HW, T);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        if (t2 + k * T < m) {
            const float z = __uint_as_float(opaque(ry[k]));
            const float dz = __uint_as_float(opaque(rd[k]));
            st_elem<DT>(dx, w.off, fmaf(kA, dz, fmaf(kB, z - bc2, kC)));
        }
        w.step();
    }
}

// ---------------------------------------------------------------------------
// host side

// The group of the channel-resident kernels: G workgroups per channel, mg
// vectors each (G = 1: the whole channel, no exchange words).
static SliceGroup channel_group(const Plan& pl, void* ws)
{
    SliceGroup g;
    const int64_t vc = pl.m / pl.V;
    g.G = uint32_t(pl.nchw_group);
    g.mg = uint32_t(pl.nchw_group > 1 ? ceil_div(vc, pl.nchw_group) : vc);
    g.xchg = pl.nchw_group > 1
                 ? reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + pl.off_xchg)
                 : nullptr;
    g.salt = process_salt();
    g.status = static_cast<uint64_t*>(ws);      // the workspace header's status word
    return g;
}

template <int DT, int ACT>
static void launch_fwd_da(const Plan& pl, void* x, const float* gamma, const float* beta,
                          float* rm, float* rv, float* sm, float* si, float eps, float mom,
                          float a, void* ws, hipStream_t s)
{
    const uint32_t C = uint32_t(pl.C), HW = uint32_t(pl.HW), m = uint32_t(pl.m);
    const SliceGroup grp = channel_group(pl, ws);
    switch (pl.fused_variant) {
#define IABN_FWD_CASE(ID, T, NR)                                                                  \
    case ID:                                                                                      \
        if (grp.G > 1)                                                                            \
            hipLaunchKernelGGL((k_fwd_fused_nchw<DT, ACT, T, NR, true>), dim3(C * grp.G), dim3(T), \
                               0, s, x, C, HW, m, gamma, beta, rm, rv, sm, si, eps, mom, a, grp); \
        else                                                                                      \
            hipLaunchKernelGGL((k_fwd_fused_nchw<DT, ACT, T, NR, false>), dim3(C), dim3(T), 0, s, \
                               x, C, HW, m, gamma, beta, rm, rv, sm, si, eps, mom, a, grp);       \
        break;
        IABN_FUSED_FWD_VARIANTS(IABN_FWD_CASE)
#undef IABN_FWD_CASE
    default: break;
    }
}

void launch_forward_fused_nchw(const Plan& pl, void* x, const float* gamma, const float* beta,
                               float* rm, float* rv, float* sm, float* si, float eps, float mom,
                               int act, float a, void* ws, hipStream_t s)
{
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            launch_fwd_da<decltype(d)::value, decltype(ac)::value>(
                pl, x, gamma, beta, rm, rv, sm, si, eps, mom, a, ws, s);
        });
    });
}

template <int DT, int ACT>
static void launch_bwd_da(const Plan& pl, const void* y, const void* dy, void* dx,
                          const float* gamma, const float* beta, const float* invstd,
                          float* dgamma, float* dbeta, float a, float ia, void* ws, hipStream_t s)
{
    const uint32_t C = uint32_t(pl.C), HW = uint32_t(pl.HW), m = uint32_t(pl.m);
    const SliceGroup grp = channel_group(pl, ws);
    const uint32_t grid = C * grp.G;     // (the table's G names its dy stream groups)
    const bool grouped = grp.G > 1;
    switch (pl.fused_bwd_variant) {
#define IABN_BWD_CASE(ID, T, NRV, NRL, G, DYR)                                                      \
    case ID:                                                                                       \
        if constexpr (DYR)                                                                         \
            hipLaunchKernelGGL((k_bwd_fused_nchw<DT, ACT, T, NRV, true>), dim3(C), dim3(T), 0, s, \
                               y, dy, dx, C, HW, m, gamma, beta, invstd, dgamma, dbeta, a, ia);    \
        else if (grouped)                                                                          \
            hipLaunchKernelGGL((k_bwd_stream_nchw<DT, ACT, T, NRV, NRL, G, true>), dim3(grid),     \
                               dim3(T), 0, s, y, dy, dx, C, HW, m, gamma, beta, invstd, dgamma,    \
                               dbeta, a, ia, grp);                                                 \
        else                                                                                       \
            hipLaunchKernelGGL((k_bwd_stream_nchw<DT, ACT, T, NRV, NRL, G, false>), dim3(C),       \
                               dim3(T), 0, s, y, dy, dx, C, HW, m, gamma, beta, invstd, dgamma,    \
                               dbeta, a, ia, grp);                                                 \
        break;
        IABN_FUSED_BWD_VARIANTS(IABN_BWD_CASE)
#undef IABN_BWD_CASE
    default: break;
    }
}

void launch_backward_fused_nchw(const Plan& pl, const void* y, const void* dy, void* dx,
                                const float* gamma, const float* beta, const float* invstd,
                                float* dgamma, float* dbeta, int act, float a, void* ws,
                                hipStream_t s)
{
    const float ia = act == kIdentity ? 1.f : 1.f / a;
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            launch_bwd_da<decltype(d)::value, decltype(ac)::value>(
                pl, y, dy, dx, gamma, beta, invstd, dgamma, dbeta, a, ia, ws, s);
        });
    });
}

template <int DT, int ACT>
static void launch_fwd_s_da(const Plan& pl, void* x, const float* gamma, const float* beta,
                            float* rm, float* rv, float* sm, float* si, float eps, float mom,
                            float a, hipStream_t s)
{
    const uint32_t C = uint32_t(pl.C), HW = uint32_t(pl.HW), m = uint32_t(pl.m);
    switch (pl.scalar_variant) {
#define IABN_CASE(ID, T, NR)                                                                      \
    case ID:                                                                                      \
        hipLaunchKernelGGL((k_fwd_fused_nchw_s<DT, ACT, T, NR>), dim3(C), dim3(T), 0, s, x, C, HW, \
                           m, gamma, beta, rm, rv, sm, si, eps, mom, a);                          \
        break;
        IABN_FUSED_SCALAR_VARIANTS(IABN_CASE)
#undef IABN_CASE
    default: break;
    }
}

void launch_forward_fused_scalar(const Plan& pl, void* x, const float* gamma, const float* beta,
                                 float* rm, float* rv, float* sm, float* si, float eps, float mom,
                                 int act, float a, hipStream_t s)
{
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            launch_fwd_s_da<decltype(d)::value, decltype(ac)::value>(
                pl, x, gamma, beta, rm, rv, sm, si, eps, mom, a, s);
        });
    });
}

template <int DT, int ACT>
static void launch_bwd_s_da(const Plan& pl, const void* y, const void* dy, void* dx,
                            const float* gamma, const float* beta, const float* invstd,
                            float* dgamma, float* dbeta, float a, float ia, hipStream_t s)
{
    const uint32_t C = uint32_t(pl.C), HW = uint32_t(pl.HW), m = uint32_t(pl.m);
    switch (pl.scalar_variant) {
#define IABN_CASE(ID, T, NR)                                                                      \
    case ID:                                                                                      \
        hipLaunchKernelGGL((k_bwd_fused_nchw_s<DT, ACT, T, NR>), dim3(C), dim3(T), 0, s, y, dy, dx, \
                           C, HW, m, gamma, beta, invstd, dgamma, dbeta, a, ia);                  \
        break;
        IABN_FUSED_SCALAR_VARIANTS(IABN_CASE)
#undef IABN_CASE
    default: break;
    }
}

void launch_backward_fused_scalar(const Plan& pl, const void* y, const void* dy, void* dx,
                                  const float* gamma, const float* beta, const float* invstd,
                                  float* dgamma, float* dbeta, int act, float a, hipStream_t s)
{
    const float ia = act == kIdentity ? 1.f : 1.f / a;
    with_dtype(pl.dtype, [&](auto d) {
        with_act(act, [&](auto ac) {
            launch_bwd_s_da<decltype(d)::value, decltype(ac)::value>(
                pl, y, dy, dx, gamma, beta, invstd, dgamma, dbeta, a, ia, s);
        });
    });
}

}  // namespace iabn

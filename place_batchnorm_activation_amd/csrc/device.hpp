// Device helpers for the In-Place ABN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace iabn {

__device__ __forceinline__ int64_t dmin(int64_t a, int64_t b) { return a < b ? a : b; }

// ---------------------------------------------------------------------------
// storage access: V consecutive elements <-> V floats.
// fp32: V = 4 (one 128-bit access) or 1.  bf16 and fp16: V = 8 (one 128-bit
// access) or 1.  Loads widen exactly; stores round to nearest even.

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two 16-bit elements of a 32-bit word (low half first) <-> two floats.
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi)
{
    if constexpr (DT == kBF16) {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xffff0000u);
    } else {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, w);
        lo = float(h.x);
        hi = float(h.y);
    }
}

// fp32 -> bf16 (v_cvt_pk_bf16_f32) or fp16 (v_cvt_f16_f32), nearest even; fp16
// overflows to infinity and keeps its subnormals.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (DT == kBF16) {
        const bf16x2_t t = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, t);
    } else {
        const f16x2_t t = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, t);
    }
}

template <int DT>
__device__ __forceinline__ float unpack1(uint16_t b)
{
    if constexpr (DT == kBF16) return __uint_as_float(uint32_t(b) << 16);
    else return float(__builtin_bit_cast(_Float16, b));
}

template <int DT>
__device__ __forceinline__ uint16_t pack1(float v)
{
    if constexpr (DT == kBF16) return __builtin_bit_cast(uint16_t, (__bf16)v);
    else return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Raw 16-byte vector <-> floats, for loops that keep loads in flight as raw bits.
template <int DT>
struct Raw16 { static constexpr int V = DT == kF32 ? 4 : 8; };

template <int DT>
__device__ __forceinline__ void unpack16(const uint4& q, float (&v)[Raw16<DT>::V])
{
    if constexpr (DT == kF32) {
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    } else {
        unpack2<DT>(q.x, v[0], v[1]);
        unpack2<DT>(q.y, v[2], v[3]);
        unpack2<DT>(q.z, v[4], v[5]);
        unpack2<DT>(q.w, v[6], v[7]);
    }
}

template <int DT>
__device__ __forceinline__ uint4 pack16(const float (&v)[Raw16<DT>::V])
{
    if constexpr (DT == kF32) {
        return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                          __float_as_uint(v[3]));
    } else {
        return make_uint4(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]), pack2<DT>(v[4], v[5]),
                          pack2<DT>(v[6], v[7]));
    }
}

template <int DT, int V>
__device__ __forceinline__ void load_elems(const void* base, int64_t i, float (&v)[V])
{
    if constexpr (DT == kF32) {
        const float* p = static_cast<const float*>(base) + i;
        if constexpr (V == 4) {
            const float4 q = *reinterpret_cast<const float4*>(p);
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else {
            static_assert(V == 1, "fp32 access width");
            v[0] = *p;
        }
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(base) + i;
        if constexpr (V == 8) {
            unpack16<DT>(*reinterpret_cast<const uint4*>(p), v);
        } else {
            static_assert(V == 1, "16-bit access width");
            v[0] = unpack1<DT>(*p);
        }
    }
}

template <int DT, int V>
__device__ __forceinline__ void store_elems(void* base, int64_t i, const float (&v)[V])
{
    if constexpr (DT == kF32) {
        float* p = static_cast<float*>(base) + i;
        if constexpr (V == 4) {
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            *p = v[0];
        }
    } else {
        uint16_t* p = static_cast<uint16_t*>(base) + i;
        if constexpr (V == 8) {
            *reinterpret_cast<uint4*>(p) = pack16<DT>(v);
        } else {
            *p = pack1<DT>(v[0]);
        }
    }
}

// V consecutive fp32 values (16-byte aligned when V is a multiple of 4).
template <int V>
__device__ __forceinline__ void store_floats(float* p, const float (&v)[V])
{
    if constexpr (V % 4 == 0) {
#pragma unroll
        for (int k = 0; k < V; k += 4)
            *reinterpret_cast<float4*>(p + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k) p[k] = v[k];
    }
}

// Store of V elements with the non-temporal hint (streaming data that is not read
// again soon); same values as store_elems.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int DT, int V>
__device__ __forceinline__ void store_elems_nt(void* base, int64_t i, const float (&v)[V])
{
    if constexpr (V * (DT == kF32 ? 4 : 2) == 16) {
        const uint4 q = pack16<DT>(v);
        const u32x4_t w = {q.x, q.y, q.z, q.w};
        char* p = static_cast<char*>(base) + i * (DT == kF32 ? 4 : 2);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    } else {
        store_elems<DT, V>(base, i, v);
    }
}

// Elementwise outputs (y, dx) are written with the non-temporal hint: they are
// not read again within the call, and keeping them out of the way leaves the
// Infinity Cache to the inputs being re-read and spares the next kernel the
// write-back of dirty lines (measured on the bf16 NHWC segmentation map: the
// following statistics pass went from 75 to 55 us).  The split forward's NHWC
// elementwise pass walks the tensor from the end down (the rows the statistics
// read last are the likeliest to be cached).
#ifndef IABN_APPLY_NT_STORE
#define IABN_APPLY_NT_STORE 1
#endif
#ifndef IABN_APPLY_REVERSE
#define IABN_APPLY_REVERSE 1
#endif
#ifndef IABN_FUSED_NT_STORE
#define IABN_FUSED_NT_STORE 1
#endif

template <int DT, int V>
__device__ __forceinline__ void store_out(void* base, int64_t i, const float (&v)[V])
{
    if constexpr (IABN_APPLY_NT_STORE) store_elems_nt<DT, V>(base, i, v);
    else store_elems<DT, V>(base, i, v);
}

template <int DT>
__device__ __forceinline__ float load_one(const void* base, int64_t i)
{
    float v[1];
    load_elems<DT, 1>(base, i, v);
    return v[0];
}

// ---------------------------------------------------------------------------
// invertible activations.  Forward branches on z > 0; the backward reads the
// branch off the stored y (y > 0), which agrees with z > 0 for every slope > 0.

// ELU's two transcendentals, with relative accuracy of a few ulps over the
// whole ELU branch, also where the result is tiny (a channel whose z all sit
// near 0, as running statistics in eval mode or a small gamma can make them;
// exp(z) - 1 and ln(1 + u) formed directly lose their digits there).  Each
// forms a series for arguments near 0 and the hardware's exp2 or log2 for the
// rest, and selects (no branch):
//   expm1(z), z <= 0: on [-0.35, 0] the Taylor series to z^7 (the first term
//     left out is below 2^-25 of the sum); below -0.35, exp2(z*log2(e)) - 1,
//     whose magnitude there exceeds 0.29, so the roundings of exp2 and of its
//     argument stay a few ulps of it;
//   log1p(u), -1 < u <= 0: above -0.29, ln(1 + u) = 2*atanh(s) with
//     s = u/(2 + u), |s| < 0.17, by the series 2s(1 + s^2/3 + s^4/5 + s^6/7 +
//     s^8/9) (first term left out below 2^-28 of the sum); at or below it,
//     log2(1 + u)*ln2, where |ln(1 + u)| >= 0.34 and 1 + u is rounded at most
//     by half an ulp of 2^-1.
// Emulated in fp32 (fused multiply-adds, correctly rounded exp2, log2 and
// reciprocal): at most 2.4 ulps (expm1) and 3.5 ulps (log1p) from the exact
// values; the hardware's exp2, log2 and reciprocal are within an ulp of those.
__device__ __forceinline__ float elu_expm1(float z)
{
    float p = 1.f / 5040.f;
    p = fmaf(p, z, 1.f / 720.f);
    p = fmaf(p, z, 1.f / 120.f);
    p = fmaf(p, z, 1.f / 24.f);
    p = fmaf(p, z, 1.f / 6.f);
    p = fmaf(p, z, 0.5f);
    p = fmaf(p, z, 1.f);
    const float near0 = p * z;
    const float far = __builtin_amdgcn_exp2f(z * 1.44269504088896341f) - 1.f;
    return z > -0.35f ? near0 : far;                   // NaN takes exp2's NaN
}

__device__ __forceinline__ float elu_log1p(float u)
{
    const float s = u * __builtin_amdgcn_rcpf(2.f + u);
    const float t = s * s;
    float q = 1.f / 9.f;
    q = fmaf(q, t, 1.f / 7.f);
    q = fmaf(q, t, 1.f / 5.f);
    q = fmaf(q, t, 1.f / 3.f);
    q = fmaf(q, t, 1.f);
    const float near0 = 2.f * s * q;
    const float far = __builtin_amdgcn_logf(1.f + u) * 0.693147180559945309f;
    return u > -0.29f ? near0 : far;
}

// The direct forms on the hardware units alone: exp2(z*log2(e)) - 1, and
// ln(w) - ((w - 1) - u)/w with w = 1 + u (the first-order correction for the
// rounding of w: Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991).  Their error is about an ulp of 1 in
// absolute terms, under the rounding of 16-bit storage for every value above
// the fp16 subnormal range, so every kernel on 16-bit storage uses them: there
// the forms above would cost registers and ALU time and gain nothing.
__device__ __forceinline__ float elu_expm1_direct(float z)
{
    return __builtin_amdgcn_exp2f(z * 1.44269504088896341f) - 1.f;
}

__device__ __forceinline__ float elu_log1p_direct(float u)
{
    const float w = 1.f + u;
    return __builtin_amdgcn_logf(w) * 0.693147180559945309f
           - ((w - 1.f) - u) * __builtin_amdgcn_rcpf(w);
}

// PRECISE: ELU through elu_expm1 / elu_log1p, else through the direct forms.
template <int ACT, bool PRECISE>
__device__ __forceinline__ float act_forward(float z, float a)
{
    if constexpr (ACT == kLeaky) return z > 0.f ? z : a * z;
    else if constexpr (ACT == kElu) {
        // both arms formed and one selected: as a branch around the series, each
        // element's chain would run alone, with no other element's to fill its
        // latencies.  A NaN z keeps its NaN (it is not clamped to 0).
        const float zn = z > 0.f ? 0.f : z;
        const float e = PRECISE ? elu_expm1(zn) : elu_expm1_direct(zn);
        return z > 0.f ? z : a * e;
    } else return z;
}

// From a stored y: the pre-activation z = act^-1(y) and the slope act'(z).
// ELU: act'(z) = alpha*exp(z) = y + alpha; the inverse clamps y/alpha at -1 + 2^-24.
template <int ACT, bool PRECISE>
__device__ __forceinline__ void act_invert(float y, float a, float inv_a, float& z, float& slope)
{
    if constexpr (ACT == kLeaky) {
        const bool pos = y > 0.f;
        z = pos ? y : y * inv_a;
        slope = pos ? 1.f : a;
    } else if constexpr (ACT == kElu) {
        const bool pos = y > 0.f;
        const float u = fmaxf(y * inv_a, -1.f + 0x1p-24f);
        // formed for every element and selected, as in act_forward
        const float lz = PRECISE ? elu_log1p(u) : elu_log1p_direct(u);
        z = pos ? y : lz;
        slope = pos ? 1.f : y + a;
    } else {
        z = y;
        slope = 1.f;
    }
}

// act'(z) from the pre-activation itself (optimized checkpointing rebuilds z =
// gamma*xhat + beta with one fused multiply-add, whose sign is exact):
// leaky ReLU a, ELU alpha*exp(z), on the non-positive side.
template <int ACT>
__device__ __forceinline__ float act_slope_at(float z, float a)
{
    if constexpr (ACT == kLeaky) return z > 0.f ? 1.f : a;
    else if constexpr (ACT == kElu)
        return z > 0.f ? 1.f : a * __builtin_amdgcn_exp2f(z * 1.44269504088896341f);
    else return 1.f;
}

// ---------------------------------------------------------------------------
// Chan et al. pairwise update of (count, mean, M2): merge b into a.  The weight
// nb/(n+nb) takes the hardware reciprocal in fp32 (1 ulp), an exact division in fp64.
__device__ __forceinline__ float merge_weight(float nb, float nn) { return nb * __builtin_amdgcn_rcpf(nn); }
__device__ __forceinline__ double merge_weight(double nb, double nn) { return nb / nn; }

template <typename F>
__device__ __forceinline__ void chan_merge(F& n, F& mean, F& m2, F nb, F mb, F m2b)
{
    if (nb > F(0)) {
        const F nn = n + nb;
        const F f = merge_weight(nb, nn);
        const F d = mb - mean;
        mean = mean + d * f;
        m2 = m2 + m2b + d * d * n * f;
        n = nn;
    }
}

// lane 0 of the wave ends with the Chan merge of all 64 lanes, in a fixed order
template <typename F>
__device__ __forceinline__ void wave_chan(F& n, F& mean, F& m2)
{
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
        const F nb = __shfl_xor(n, off, kWave);
        const F mb = __shfl_xor(mean, off, kWave);
        const F m2b = __shfl_xor(m2, off, kWave);
        chan_merge(n, mean, m2, nb, mb, m2b);
    }
}

template <typename F>
__device__ __forceinline__ F wave_sum(F v)
{
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// Walk of an NCHW channel: channel-local vector index j = n*HWv + o maps to the
// global vector address (n*C + c)*HWv + o.  Advancing j by a fixed stride needs
// no division: o += r, n += q with a carry.
struct ChannelWalk {
    int64_t addr;      // global vector address of the current position
    int64_t o;         // offset inside the plane (vectors)
    int64_t hwv;       // vectors per plane
    int64_t d_addr;    // address step without carry: q*C*HWv + r
    int64_t d_carry;   // extra step on carry: C*HWv - HWv
    int64_t r;

    __host__ __device__ __forceinline__ void init(int64_t j, int64_t c, int64_t C, int64_t HWv, int64_t stride)
    {
        const int64_t n = j / HWv;
        o = j - n * HWv;
        hwv = HWv;
        addr = (n * C + c) * HWv + o;
        const int64_t q = stride / HWv;
        r = stride - q * HWv;
        d_addr = q * C * HWv + r;
        d_carry = C * HWv - HWv;
    }
    __host__ __device__ __forceinline__ void step()
    {
        o += r;
        addr += d_addr;
        if (o >= hwv) { o -= hwv; addr += d_carry; }
    }
};

// ChannelWalk in 32-bit vector offsets (tensors under 2^28 vectors, 4 GiB).
struct ChannelWalk32 {
    uint32_t off, o, hwv, d_off, d_carry, r;
    __host__ __device__ __forceinline__ void init(uint32_t j, uint32_t c, uint32_t C, uint32_t HWv,
                                                  uint32_t stride)
    {
        const uint32_t n = j / HWv;
        o = j - n * HWv;
        hwv = HWv;
        off = (n * C + c) * HWv + o;
        const uint32_t q = stride / HWv;
        r = stride - q * HWv;
        d_off = q * C * HWv + r;
        d_carry = C * HWv - HWv;
    }
    __host__ __device__ __forceinline__ void step()
    {
        o += r;
        off += d_off;
        if (o >= hwv) { o -= hwv; off += d_carry; }
    }
};

// Slice taken by workgroup b of a slice-resident NHWC launch (one workgroup per
// slice).  Workgroups are dealt to the 8 XCDs round-robin (b runs on XCD b % 8), so
// when the slice count divides by 8 each XCD takes a contiguous run of slices:
// neighbouring slices share cache lines and then meet in one L2.  A permutation of
// [0, slices).
__host__ __device__ __forceinline__ uint32_t nhwc_slice_of(uint32_t b, uint32_t slices)
{
    return (slices % 8 == 0) ? (b % 8) * (slices / 8) + b / 8 : b;
}

// Slice and member of workgroup b when G workgroups share each slice (G == 1:
// nhwc_slice_of).  With slices % 8 == 0 the G members of a slice are workgroups
// b, b + 8, ..., so they run on one XCD (one L2), and XCD x takes slices
// x*(slices/8) onwards.  A bijection of [0, slices*G) onto (slice, member) pairs.
__host__ __device__ __forceinline__ void nhwc_slice_member(uint32_t b, uint32_t slices,
                                                           uint32_t G, uint32_t& s,
                                                           uint32_t& member)
{
    if (G == 1) {
        s = nhwc_slice_of(b, slices);
        member = 0;
    } else {
        const uint32_t j = b / 8;
        member = j % G;
        s = (b % 8) * (slices / 8) + j / G;
    }
}

// Slice and member of workgroup b of a streamed slice launch (G % 8 == 0):
// XCD x = b % 8 takes members x, x + 8, ... of every slice, so that all slices of
// one member's rows -- whole 128-byte lines -- meet in one L2.  A bijection of
// [0, slices*G) onto (slice, member) pairs.
__host__ __device__ __forceinline__ void nhwc_stream_member(uint32_t b, uint32_t slices,
                                                            uint32_t& s, uint32_t& member)
{
    const uint32_t q = b / 8;
    s = q % slices;
    member = b % 8 + 8 * (q / slices);
}

// Slice and member of workgroup b of a slice-resident launch: groups of 8 or more
// members are placed member-major (nhwc_stream_member), so that every line's
// writers -- the slices of one row range -- share an L2 however narrow the
// slices; smaller groups slice-major (nhwc_slice_member).
__host__ __device__ __forceinline__ void nhwc_group_member(uint32_t b, uint32_t slices,
                                                           uint32_t G, uint32_t& s,
                                                           uint32_t& member)
{
    if (G >= 8) nhwc_stream_member(b, slices, s, member);
    else nhwc_slice_member(b, slices, G, s, member);
}

// Walk of a flat NCHW tensor: vector v has channel ((v / HWv) % C).  Advancing v
// by a fixed stride updates the in-plane offset and the channel with carries.
struct FlatNCHWWalk {
    int64_t o, c, hwv, C, r, qc;
    __host__ __device__ __forceinline__ void init(int64_t v, int64_t C_, int64_t HWv, int64_t stride)
    {
        hwv = HWv; C = C_;
        const int64_t plane = v / HWv;
        o = v - plane * HWv;
        c = plane % C;
        const int64_t q = stride / HWv;
        r = stride - q * HWv;
        qc = q % C;
    }
    __host__ __device__ __forceinline__ void step()
    {
        o += r;
        c += qc;
        if (o >= hwv) { o -= hwv; c += 1; }
        if (c >= C) c -= C;
    }
};

}  // namespace iabn

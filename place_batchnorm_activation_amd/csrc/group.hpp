// Group exchange of fp64 partial sums between the workgroups (members) that
// share one slice of a tensor -- a slice of channels (NHWC) or one channel
// (NCHW) -- with no fence and no reset launch.
//
// Every word is a relaxed 64-bit atomic {32-bit tag, 32-bit half of an fp64
// value}; a partial is accepted when the tags of its words equal the halves of
// this call's 64-bit token.  The token mixes a per-process salt, the slice and a
// per-slice epoch that the kernels keep in the workspace: member 0 advances the
// epoch once every member's sums have arrived (each member read it before
// publishing), so the next call -- a graph replay too -- uses a fresh token and
// words left by earlier calls never match.  The members must run at once (the
// host keeps the grid within the CU count); each wait is bounded, and past it
// the sums become NaN instead of the device hanging, and the workspace's status
// word records the timeout for the host to query.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace iabn {

// The salt of every exchange token of this process (host).
uint64_t process_salt();

namespace {

// splitmix64's output mix (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014), a bijection of 64-bit words.
__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t atomic_ld(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_st(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t half)
{
    return (uint64_t(tag) << 32) | half;
}

// Bounded wait of the exchange, in polls (each a round trip to L2 and a sleep):
// well over a second.
constexpr uint32_t kMaxPolls = 1u << 21;

// A wait ran out: the workspace's status word (null: none to set) records it.
__device__ __forceinline__ void group_timed_out(uint64_t* status)
{
    if (status) atomic_st(status, kExchangeTimeout);
}

// Members per slice at most (the plans never form larger groups).
constexpr uint32_t kMaxGroup = 64;

// This member's two fp64 sums of channel ch, as four tagged words.  words: the
// slice's first word; nch: channels per slice.
__device__ __forceinline__ void group_publish(uint64_t* words, uint32_t member, uint32_t nch,
                                              uint32_t ch, uint64_t tok, double s1, double s2)
{
    const uint32_t tlo = uint32_t(tok), thi = uint32_t(tok >> 32);
    const uint64_t b1 = uint64_t(__double_as_longlong(s1)), b2 = uint64_t(__double_as_longlong(s2));
    uint64_t* w = words + (size_t(member) * nch + ch) * 4;
    atomic_st(w + 0, tagged(tlo, uint32_t(b1 >> 32)));
    atomic_st(w + 1, tagged(thi, uint32_t(b1)));
    atomic_st(w + 2, tagged(tlo, uint32_t(b2 >> 32)));
    atomic_st(w + 3, tagged(thi, uint32_t(b2)));
}

// Member j's sums of channel ch, once all four words carry this call's tags
// (bounded wait; NaN after it, and the timeout recorded in *status).
__device__ __forceinline__ void group_fetch(const uint64_t* words, uint32_t j, uint32_t nch,
                                            uint32_t ch, uint64_t tok, double& v1, double& v2,
                                            uint64_t* status)
{
    const uint32_t tlo = uint32_t(tok), thi = uint32_t(tok >> 32);
    const uint64_t* w = words + (size_t(j) * nch + ch) * 4;
    v1 = v2 = __longlong_as_double(0x7FF8000000000000ll);
    for (uint32_t poll = 0; poll <= kMaxPolls; ++poll) {
        const uint64_t w0 = atomic_ld(w + 0), w1 = atomic_ld(w + 1);
        const uint64_t w2 = atomic_ld(w + 2), w3 = atomic_ld(w + 3);
        if (uint32_t(w0 >> 32) == tlo && uint32_t(w1 >> 32) == thi &&
            uint32_t(w2 >> 32) == tlo && uint32_t(w3 >> 32) == thi) {
            v1 = __longlong_as_double(int64_t((w0 << 32) | uint32_t(w1)));
            v2 = __longlong_as_double(int64_t((w2 << 32) | uint32_t(w3)));
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    group_timed_out(status);
}

// Members FB at a time: the sums of channel ch of members j0 .. j0 + FB - 1
// (< G; this member's own taken from s1, s2), all their words loaded at once on
// every poll, so that partners that have all published cost one round trip.
// NaN for a member not received within the bounded wait (recorded in *status).
template <uint32_t FB>
__device__ __forceinline__ void group_fetch_batch(const uint64_t* words, uint32_t j0, uint32_t G,
                                                  uint32_t member, uint32_t nch, uint32_t ch,
                                                  uint64_t tok, double s1, double s2,
                                                  double (&v1)[FB], double (&v2)[FB],
                                                  uint64_t* status)
{
    const uint32_t tlo = uint32_t(tok), thi = uint32_t(tok >> 32);
    bool need[FB];
    uint32_t left = 0;
#pragma unroll
    for (uint32_t q = 0; q < FB; ++q) {
        const uint32_t j = j0 + q;
        v1[q] = j == member ? s1 : __longlong_as_double(0x7FF8000000000000ll);
        v2[q] = j == member ? s2 : __longlong_as_double(0x7FF8000000000000ll);
        need[q] = j < G && j != member;
        left += need[q] ? 1u : 0u;
    }
    for (uint32_t poll = 0; left != 0 && poll <= kMaxPolls; ++poll) {
        uint64_t w[FB][4];
#pragma unroll
        for (uint32_t q = 0; q < FB; ++q) {
            if (need[q]) {
                const uint64_t* src = words + (size_t(j0 + q) * nch + ch) * 4;
                w[q][0] = atomic_ld(src + 0);
                w[q][1] = atomic_ld(src + 1);
                w[q][2] = atomic_ld(src + 2);
                w[q][3] = atomic_ld(src + 3);
            }
        }
#pragma unroll
        for (uint32_t q = 0; q < FB; ++q) {
            if (need[q] && uint32_t(w[q][0] >> 32) == tlo && uint32_t(w[q][1] >> 32) == thi &&
                uint32_t(w[q][2] >> 32) == tlo && uint32_t(w[q][3] >> 32) == thi) {
                v1[q] = __longlong_as_double(int64_t((w[q][0] << 32) | uint32_t(w[q][1])));
                v2[q] = __longlong_as_double(int64_t((w[q][2] << 32) | uint32_t(w[q][3])));
                need[q] = false;
                --left;
            }
        }
        if (left != 0) __builtin_amdgcn_s_sleep(1);
    }
    if (left != 0) group_timed_out(status);
}

}  // namespace

// Group exchange arguments: the workspace words (epochs, then the tagged sums),
// the per-process salt, members per slice, rows per member, and the workspace's
// status word (where a wait that runs out is recorded; null: not recorded).
struct SliceGroup {
    uint64_t* xchg;
    uint64_t salt;
    uint32_t G;
    uint32_t mg;
    uint64_t* status = nullptr;
};

namespace {

__device__ __forceinline__ uint64_t group_token(const SliceGroup& grp, uint32_t s, uint64_t epoch)
{
    return mix64(grp.salt ^ mix64(epoch ^ (uint64_t(s) << 40)));
}

// First word of slice s's tagged sums (after the epochs, padded to 32 words).
__device__ __forceinline__ uint64_t* group_words(const SliceGroup& grp, uint32_t s,
                                                 uint32_t slices, uint32_t nch)
{
    return grp.xchg + ((slices + 31u) & ~31u) + size_t(s) * grp.G * nch * 4;
}

// Groups of at least this many members exchange in two levels, member 0's
// threads loading up to kPairBatch (member, channel) pairs at once.
constexpr uint32_t kTwoLevelGroup = 16;
constexpr uint32_t kPairBatch = 4;

// Sums over all members (G > 1), called by every thread of the workgroup: the
// finishing thread of channel t (t < NCH) passes its member's sums s1, s2 and
// gets back the sums over members 0..G-1, added in a fixed order (member order
// in one-level groups; in two-level ones the order given below), so that every
// member derives the same bits on every run.
//  - G < kTwoLevelGroup: each finishing thread publishes and then reads the other
//    members, FB at a time (measured: reading them with one thread per
//    (member, channel) loads the memory system with polls and is slower).
//  - Larger groups, in two levels: every member but 0 publishes; member 0 reads
//    them, each of its threads loading up to kPairBatch (member, channel) pairs at
//    once, adds, and publishes the totals in its own slot, which the others read.
//    Member 0 stages one partial sum per thread in LDS (16 bytes a thread), not
//    every member's partials, which leaves the streamed kernels LDS for rows.
// FB: members read per poll in one-level groups.  Eight (every partner of a group
// of 8 in one round trip) made the slice-resident NHWC kernels 5-7% faster on
// groups of 8; the other kernels keep four, which left them as fast and their
// register allocation unchanged.
// TWO: whether the two-level path is compiled in.  A kernel whose plan never
// gives it kTwoLevelGroup members or more leaves it out, which spares the
// registers its batched loads take (a kernel holding its data in nearly all of
// them spilled around it).
template <uint32_t NCH, int T, uint32_t FB = 4, bool TWO = true>
__device__ __forceinline__ void group_sums(const SliceGroup& grp, uint32_t s, uint32_t slices,
                                           uint32_t member, uint64_t tok, bool fin, double& s1,
                                           double& s2)
{
    uint64_t* words = group_words(grp, s, slices, NCH);
    const uint32_t t = threadIdx.x;
    if (!TWO || grp.G < kTwoLevelGroup) {
        if (fin) {
            group_publish(words, member, NCH, t, tok, s1, s2);
            double t1 = 0.0, t2 = 0.0;
            for (uint32_t j0 = 0; j0 < grp.G; j0 += FB) {
                double v1[FB], v2[FB];
                group_fetch_batch<FB>(words, j0, grp.G, member, NCH, t, tok, s1, s2, v1, v2,
                                       grp.status);
#pragma unroll
                for (uint32_t q = 0; q < FB; ++q) {
                    if (j0 + q < grp.G) {
                        t1 += v1[q];
                        t2 += v2[q];
                    }
                }
            }
            s1 = t1;
            s2 = t2;
        }
        return;
    }
    if constexpr (!TWO) return;
    if (member != 0) {
        if (fin) {
            group_publish(words, member, NCH, t, tok, s1, s2);
            group_fetch(words, 0, NCH, t, tok, s1, s2, grp.status);
        }
        return;
    }
    // Member 0: thread t takes the pairs t, t + T, t + 2T, ... of the (member,
    // channel) pairs of members 1..G-1 -- one channel, t % NCH, since NCH divides
    // T -- kPairBatch at a time, and adds each batch, in order, once all of it
    // has arrived; the finishing thread of a channel (t < NCH) starts from member
    // 0's own sums.  The channel's total is then the sums of threads t, t + NCH,
    // t + 2 NCH, ... added in that order: a fixed order, whatever the order of
    // arrival (with one thread, member order).
    static_assert(T % NCH == 0, "a thread's pairs share one channel");
    __shared__ double part[2][T];
    const uint32_t tlo = uint32_t(tok), thi = uint32_t(tok >> 32);
    const uint32_t npairs = (grp.G - 1) * NCH;
    double a1 = fin ? s1 : 0.0, a2 = fin ? s2 : 0.0;
    for (uint32_t p0 = 0; p0 < npairs; p0 += kPairBatch * T) {
        bool need[kPairBatch];
        double v1[kPairBatch], v2[kPairBatch];
        uint32_t left = 0;
#pragma unroll
        for (uint32_t q = 0; q < kPairBatch; ++q) {
            need[q] = p0 + q * T + t < npairs;
            left += need[q] ? 1u : 0u;
            v1[q] = v2[q] = __longlong_as_double(0x7FF8000000000000ll);   // NaN unless received
        }
        const bool any = left != 0;
        for (uint32_t poll = 0; left != 0 && poll <= kMaxPolls; ++poll) {
            uint64_t w[kPairBatch][4];
#pragma unroll
            for (uint32_t q = 0; q < kPairBatch; ++q) {
                if (need[q]) {
                    const uint32_t pair = p0 + q * T + t;
                    const uint64_t* src = words + (size_t(1 + pair / NCH) * NCH + pair % NCH) * 4;
                    w[q][0] = atomic_ld(src + 0);
                    w[q][1] = atomic_ld(src + 1);
                    w[q][2] = atomic_ld(src + 2);
                    w[q][3] = atomic_ld(src + 3);
                }
            }
#pragma unroll
            for (uint32_t q = 0; q < kPairBatch; ++q) {
                if (need[q] && uint32_t(w[q][0] >> 32) == tlo && uint32_t(w[q][1] >> 32) == thi &&
                    uint32_t(w[q][2] >> 32) == tlo && uint32_t(w[q][3] >> 32) == thi) {
                    v1[q] = __longlong_as_double(int64_t((w[q][0] << 32) | uint32_t(w[q][1])));
                    v2[q] = __longlong_as_double(int64_t((w[q][2] << 32) | uint32_t(w[q][3])));
                    need[q] = false;
                    --left;
                }
            }
            if (left != 0) __builtin_amdgcn_s_sleep(1);
        }
        if (left != 0) group_timed_out(grp.status);
        if (any) {
#pragma unroll
            for (uint32_t q = 0; q < kPairBatch; ++q) {
                if (p0 + q * T + t < npairs) {
                    a1 += v1[q];
                    a2 += v2[q];
                }
            }
        }
    }
    part[0][t] = a1;
    part[1][t] = a2;
    __syncthreads();
    if (fin) {
        // threads t + k NCH, k < G - 1, hold channel t's other members
        const uint32_t nthr = uint32_t(T / NCH) < grp.G - 1 ? uint32_t(T / NCH) : grp.G - 1;
        s1 = part[0][t];
        s2 = part[1][t];
        for (uint32_t k = 1; k < nthr; ++k) {
            s1 += part[0][k * NCH + t];
            s2 += part[1][k * NCH + t];
        }
        group_publish(words, 0, NCH, t, tok, s1, s2);
    }
}

}  // namespace

}  // namespace iabn

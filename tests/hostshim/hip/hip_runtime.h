// Host stand-ins for the few HIP names the group exchange header uses, so that
// tests/group_check.cpp can run the exchange with one host thread per workgroup
// (one thread per workgroup: threadIdx.x is 0, LDS is per thread, and a
// workgroup barrier has nothing to wait for).  Test infrastructure only.
#pragma once

#include <cstdint>
#include <cstring>
#include <thread>

#define __device__
#define __forceinline__ inline
#define __shared__ static thread_local
#define __HIP_MEMORY_SCOPE_AGENT 3

struct HostThreadIdx {
    unsigned x, y, z;
};
inline thread_local HostThreadIdx threadIdx{0, 0, 0};

inline void __syncthreads() {}

#define __builtin_amdgcn_s_sleep(n) std::this_thread::yield()

template <class T>
inline T __hip_atomic_load(const T* p, int order, int)
{
    return __atomic_load_n(p, order);
}

template <class T>
inline void __hip_atomic_store(T* p, T v, int order, int)
{
    __atomic_store_n(p, v, order);
}

inline long long __double_as_longlong(double d)
{
    long long v;
    std::memcpy(&v, &d, sizeof v);
    return v;
}

inline double __longlong_as_double(long long v)
{
    double d;
    std::memcpy(&d, &v, sizeof d);
    return d;
}

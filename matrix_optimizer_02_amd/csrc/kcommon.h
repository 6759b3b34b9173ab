// Device helpers shared by the HIP kernels of libdmuon_ns (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dmuon_internal.h"

namespace dmuon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern; the
// conversion down rounds to nearest even (gfx950 has a hardware instruction
// for it, which the compiler selects for __bf16 conversions).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static __forceinline__ float load(const float* p) { return *p; }
    __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
    __device__ static __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Streaming vector accesses for the bandwidth-bound passes, which touch every
// byte once: non-temporal loads and stores (measured on a 4 GiB copy: 6.07
// TB/s against 5.73 with ordinary accesses).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename V>
__device__ __forceinline__ V ld_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}
template <typename V>
__device__ __forceinline__ void st_stream(void* p, V v) {
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

// Four consecutive elements <-> float4 (aligned to 4 elements), streaming.
__device__ __forceinline__ float4 load4(const float* p) {
    const f32x4_t v = ld_stream<f32x4_t>(p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load4(const uint16_t* p) {
    const u32x2_t u = ld_stream<u32x2_t>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void store4(float* p, float4 v) { st_stream<f32x4_t>(p, f32x4_t{v.x, v.y, v.z, v.w}); }
__device__ __forceinline__ void store4(uint16_t* p, float4 v) {
    u32x2_t u;
    u.x = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    u.y = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
    st_stream<u32x2_t>(p, u);
}

// Largest i in [0, n) with key(i) <= x, for a non-decreasing key (key(0) <= x).
// (A one-round variant -- each lane comparing one key, the count of a ballot
// giving i -- measured no faster on the 28- and 67-record launches.)
template <typename F>
__device__ __forceinline__ int upper_index(int n, int64_t x, F key) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (key(mid) <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Deterministic block sum of one float per thread (fixed reduction tree).
template <int THREADS>
__device__ __forceinline__ float block_sum(float v, float* red) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float total = 0.f;
    #pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) total += red[w];
    __syncthreads();
    return total;
}

}  // namespace dmuon

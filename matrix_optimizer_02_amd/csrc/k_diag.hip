// Measurement kernels: the practical ceilings that the benchmark reports next
// to the published peaks, measured on the same device in the same run.
//   copy  -- a streaming copy (non-temporal 16-byte accesses, four per lane in
//            flight): the HBM read + write rate a bandwidth-bound pass can reach;
//   mix   -- the byte mix of one of the library's bandwidth-bound passes (the
//            same dtypes, streams and read/write ratio) on flat contiguous
//            arrays: what that pass's traffic can reach without its tiling;
//   mfma  -- back-to-back v_mfma_f32_32x32x16_bf16 on operands that change every
//            instruction (pseudo-random bf16 values, as the products of the
//            Newton-Schulz iteration see), no memory traffic: the matrix-core
//            rate the chip sustains within its power limit;
//   clock -- one wave that reads the shader-clock counter and the constant
//            100 MHz wall clock at fixed wall-clock intervals: run on a side
//            stream beside other work, it gives the shader clock of its XCD
//            while that work ran.
// Page basis: the project's benchmark section states the hardware, precision
// and method behind every figure (DMuon project documentation, "基准测试").
#include "kcommon.h"
#include "launch.h"

namespace dmuon {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyVec = 4;  // 16-byte groups per lane per round

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(f32x4_t* __restrict__ dst,
                                                            const f32x4_t* __restrict__ src, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kCopyThreads * kCopyVec;
    for (int64_t base = ((int64_t)blockIdx.x * kCopyThreads * kCopyVec) + threadIdx.x; base < n16; base += stride) {
        f32x4_t v[kCopyVec];
        #pragma unroll
        for (int u = 0; u < kCopyVec; ++u) {
            const int64_t i = base + (int64_t)u * kCopyThreads;
            if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
        }
        #pragma unroll
        for (int u = 0; u < kCopyVec; ++u) {
            const int64_t i = base + (int64_t)u * kCopyThreads;
            if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

// kind 0, prep: read a (bf16) and b (fp32), write b and c (bf16), 12 bytes an
// element; kind 1, apply: read a and b (bf16), write b, 6 bytes; kind 2,
// AdamW: read a and b (bf16) and c, c + n (fp32), write a, c and c + n, 22
// bytes.  Four elements a group, four groups per lane in flight, grid-stride.
template <int KIND>
__global__ __launch_bounds__(kCopyThreads) void mix_kernel(void* a, void* b, void* c, int64_t n4) {
    const int64_t n = 4 * n4;
    const int64_t stride = (int64_t)gridDim.x * kCopyThreads * kCopyVec;
    for (int64_t base = ((int64_t)blockIdx.x * kCopyThreads * kCopyVec) + threadIdx.x; base < n4; base += stride) {
        float4 x[kCopyVec], y[kCopyVec], z[kCopyVec], w[kCopyVec];
        #pragma unroll
        for (int u = 0; u < kCopyVec; ++u) {
            const int64_t e = 4 * (base + (int64_t)u * kCopyThreads);
            if (e >= n) continue;
            if (KIND == 0) {
                x[u] = load4(static_cast<const uint16_t*>(a) + e);
                y[u] = load4(static_cast<const float*>(b) + e);
            } else if (KIND == 1) {
                x[u] = load4(static_cast<const uint16_t*>(a) + e);
                y[u] = load4(static_cast<const uint16_t*>(b) + e);
            } else {
                x[u] = load4(static_cast<const uint16_t*>(a) + e);
                y[u] = load4(static_cast<const uint16_t*>(b) + e);
                z[u] = load4(static_cast<const float*>(c) + e);
                w[u] = load4(static_cast<const float*>(c) + n + e);
            }
        }
        #pragma unroll
        for (int u = 0; u < kCopyVec; ++u) {
            const int64_t e = 4 * (base + (int64_t)u * kCopyThreads);
            if (e >= n) continue;
            if (KIND == 0) {
                const float4 m = make_float4(fmaf(0.95f, y[u].x, x[u].x), fmaf(0.95f, y[u].y, x[u].y),
                                             fmaf(0.95f, y[u].z, x[u].z), fmaf(0.95f, y[u].w, x[u].w));
                store4(static_cast<float*>(b) + e, m);
                store4(static_cast<uint16_t*>(c) + e,
                       make_float4(fmaf(0.95f, m.x, x[u].x), fmaf(0.95f, m.y, x[u].y), fmaf(0.95f, m.z, x[u].z),
                                   fmaf(0.95f, m.w, x[u].w)));
            } else if (KIND == 1) {
                store4(static_cast<uint16_t*>(b) + e,
                       make_float4(fmaf(-1e-3f, x[u].x, y[u].x), fmaf(-1e-3f, x[u].y, y[u].y),
                                   fmaf(-1e-3f, x[u].z, y[u].z), fmaf(-1e-3f, x[u].w, y[u].w)));
            } else {
                float p[4] = {x[u].x, x[u].y, x[u].z, x[u].w}, g[4] = {y[u].x, y[u].y, y[u].z, y[u].w};
                float m[4] = {z[u].x, z[u].y, z[u].z, z[u].w}, v[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    m[q] = fmaf(0.9f, m[q], 0.1f * g[q]);
                    v[q] = fmaf(0.999f, v[q], 1e-3f * g[q] * g[q]);
                    p[q] = fmaf(-1e-4f, m[q] / (sqrtf(v[q]) + 1e-8f), p[q]);
                }
                store4(static_cast<uint16_t*>(a) + e, make_float4(p[0], p[1], p[2], p[3]));
                store4(static_cast<float*>(c) + e, make_float4(m[0], m[1], m[2], m[3]));
                store4(static_cast<float*>(c) + n + e, make_float4(v[0], v[1], v[2], v[3]));
            }
        }
    }
}

// splitmix64 of a counter: the operand bits of lane, pair and operand.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Eight bf16 values with random signs and mantissas and magnitudes in [0.5, 2).
__device__ __forceinline__ bf16x8 random_bf16x8(uint64_t key) {
    typedef short shortx8 __attribute__((ext_vector_type(8)));
    shortx8 v;
    #pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const uint64_t z = mix64(key * 8 + e);
        #pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t b = (uint32_t)(z >> (32 * h));
            v[e + h] = (short)(((b & 1u) << 15) | ((126u + ((b >> 1) & 1u)) << 7) | ((b >> 2) & 0x7fu));
        }
    }
    return __builtin_bit_cast(bf16x8, v);
}

constexpr int kMfmaThreads = 512;

__global__ __launch_bounds__(kMfmaThreads, 1) void mfma_kernel(float* out, int32_t iters) {
    const uint64_t lane_key = (uint64_t)blockIdx.x * kMfmaThreads + threadIdx.x;
    bf16x8 a[8], b[8];
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = random_bf16x8(lane_key * 16 + j);
        b[j] = random_bf16x8(lane_key * 16 + 8 + j);
    }
    floatx16 acc[8];
    #pragma unroll
    for (int j = 0; j < 8; ++j)
        #pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    // eight independent accumulators; each instruction takes another operand pair
    for (int i = 0; i < iters; i += 8) {
        #pragma unroll
        for (int ii = 0; ii < 8; ++ii)
            #pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + ii) & 7], b[(3 * j + ii) & 7], acc[j], 0, 0, 0);
    }
    float s = 0.f;
    #pragma unroll
    for (int j = 0; j < 8; ++j)
        #pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    out[lane_key] = s;  // keeps the products live
}

// One wave: lane 0 records `samples` (shader cycles, wall ticks) pairs, the
// k-th once the wall clock has advanced k * interval ticks from the first.
// The wall clock is monotonic, so every wait ends.
__global__ void clock_kernel(long long* out, int32_t samples, int32_t interval) {
    const long long w0 = wall_clock64();
    for (int i = 0; i < samples; ++i) {
        const long long due = w0 + (long long)i * interval;
        long long w = wall_clock64();
        while (w < due) {
            __builtin_amdgcn_s_sleep(8);
            w = wall_clock64();
        }
        const long long c = clock64();
        if (threadIdx.x == 0) {
            out[2 * i] = c;
            out[2 * i + 1] = w;
        }
    }
}

}  // namespace
}  // namespace dmuon

using namespace dmuon;

extern "C" dmuon_status dmuon_diag_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (dst == nullptr || src == nullptr || bytes == 0 || bytes % 16 != 0 ||
        (reinterpret_cast<uintptr_t>(dst) & 15u) != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
        return DMUON_ERR_INVALID_ARG;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), s0 = reinterpret_cast<uintptr_t>(src);
    if (d0 < s0 + bytes && s0 < d0 + bytes) return DMUON_ERR_INVALID_ARG;  // overlapping
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t blocks = (n16 + kCopyThreads * kCopyVec - 1) / (kCopyThreads * kCopyVec);
    if (blocks > 256 * 64) blocks = 256 * 64;  // a grid-stride loop covers the rest
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<f32x4_t*>(dst), static_cast<const f32x4_t*>(src), n16);
    return hipGetLastError() == hipSuccess ? DMUON_OK : DMUON_ERR_HIP;
}

extern "C" dmuon_status dmuon_diag_mix(int32_t kind, void* a, void* b, void* c, size_t n, void* stream) {
    if (kind < 0 || kind > 2 || n == 0 || n % 4 != 0 || n > ((size_t)1 << 40)) return DMUON_ERR_INVALID_ARG;
    const size_t a_bytes = 2 * n, b_bytes = kind == 0 ? 4 * n : 2 * n, c_bytes = kind == 0 ? 2 * n : 8 * n;
    void* ptrs[3] = {a, b, c};
    const size_t sizes[3] = {a_bytes, b_bytes, kind == 1 ? 0 : c_bytes};
    for (int i = 0; i < 3; ++i) {
        if (sizes[i] == 0) continue;
        if (ptrs[i] == nullptr || (reinterpret_cast<uintptr_t>(ptrs[i]) & 15u) != 0) return DMUON_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j) {
            if (sizes[j] == 0) continue;
            const uintptr_t x = reinterpret_cast<uintptr_t>(ptrs[i]), y = reinterpret_cast<uintptr_t>(ptrs[j]);
            if (x < y + sizes[j] && y < x + sizes[i]) return DMUON_ERR_INVALID_ARG;  // overlapping
        }
    }
    const int64_t n4 = (int64_t)(n / 4);
    int64_t blocks = (n4 + kCopyThreads * kCopyVec - 1) / (kCopyThreads * kCopyVec);
    if (blocks > 256 * 64) blocks = 256 * 64;  // a grid-stride loop covers the rest
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(kCopyThreads);
    if (kind == 0) hipLaunchKernelGGL(mix_kernel<0>, grid, block, 0, s, a, b, c, n4);
    else if (kind == 1) hipLaunchKernelGGL(mix_kernel<1>, grid, block, 0, s, a, b, c, n4);
    else hipLaunchKernelGGL(mix_kernel<2>, grid, block, 0, s, a, b, c, n4);
    return hipGetLastError() == hipSuccess ? DMUON_OK : DMUON_ERR_HIP;
}

extern "C" dmuon_status dmuon_diag_clock(long long* out, int32_t samples, int32_t interval, void* stream) {
    // at most about 100 s of sampling: samples x interval ticks of 10 ns
    if (out == nullptr || samples < 2 || interval < 1 || (long long)samples * interval > 10000000000LL)
        return DMUON_ERR_INVALID_ARG;
    hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out, samples, interval);
    return hipGetLastError() == hipSuccess ? DMUON_OK : DMUON_ERR_HIP;
}

extern "C" dmuon_status dmuon_diag_mfma(float* out, int32_t blocks, int32_t iters, void* stream) {
    if (out == nullptr || blocks < 1 || iters < 8 || iters % 8 != 0) return DMUON_ERR_INVALID_ARG;
    hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream),
                       out, iters);
    return hipGetLastError() == hipSuccess ? DMUON_OK : DMUON_ERR_HIP;
}

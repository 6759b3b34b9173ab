// AdamW step for the parameters that do not go through Muon (gfx950): one
// grouped, bandwidth-bound launch over a list of tensors of any sizes.
//   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
//   p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// fp32 arithmetic and fp32 moments; the parameter and the gradient are bf16
// or fp32, the parameter rounded once (to nearest even) when stored as bf16.
//
// Page basis: the optimizer takes a separate AdamW learning rate for the
// parameters that its predicate does not route to Muon (DMuon project
// documentation, quick-start snippet and the VLA/VLM paragraph).
//
// Each block covers kAdamBlock consecutive elements of one tensor, 8 per
// thread: two float4 of each moment, one 16-byte (bf16) or two float4 (fp32)
// groups of the parameter and the gradient.  A tensor whose length is not a
// multiple of 8 finishes with a per-element tail in its last block.
#include "kcommon.h"
#include "launch.h"

namespace dmuon {
namespace {

constexpr int kAdamThreads = 256;
constexpr int kPerThread = 8;

struct Vec8 {
    float x[8];
};

__device__ __forceinline__ Vec8 load8(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    return Vec8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
__device__ __forceinline__ Vec8 load8(const uint16_t* p) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    Vec8 r;
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.x[2 * i] = __uint_as_float(w[i] << 16);
        r.x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    return r;
}
__device__ __forceinline__ void store8(float* p, const Vec8& v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v.x[0], v.x[1], v.x[2], v.x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v.x[4], v.x[5], v.x[6], v.x[7]);
}
__device__ __forceinline__ void store8(uint16_t* p, const Vec8& v) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16(v.x[0]) | ((uint32_t)f32_to_bf16(v.x[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(v.x[2]) | ((uint32_t)f32_to_bf16(v.x[3]) << 16);
    u.z = (uint32_t)f32_to_bf16(v.x[4]) | ((uint32_t)f32_to_bf16(v.x[5]) << 16);
    u.w = (uint32_t)f32_to_bf16(v.x[6]) | ((uint32_t)f32_to_bf16(v.x[7]) << 16);
    *reinterpret_cast<uint4*>(p) = u;
}

// one element; decay, then both moments, then the bias-corrected step
__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v, const AdamArgs& a) {
    p *= a.decay;
    m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
    v = fmaf(a.beta2, v, a.one_minus_beta2 * g * g);
    const float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
    p = fmaf(-a.step_size, m / denom, p);
}

template <typename PT, typename GT>
__device__ __forceinline__ void adamw_block(const AdamArgs& a, const AdamRec& r, int64_t local) {
    PT* P = static_cast<PT*>(r.p);
    const GT* G = static_cast<const GT*>(r.g);
    const int64_t base = local * kAdamBlock;
    const int64_t e0 = base + (int64_t)threadIdx.x * kPerThread;
    const int64_t vec_end = r.n & ~(int64_t)(kPerThread - 1);  // whole 8-element groups
    if (e0 + kPerThread <= vec_end) {
        Vec8 p = load8(P + e0), m = load8(r.m + e0), v = load8(r.v + e0);
        const Vec8 g = load8(G + e0);
        #pragma unroll
        for (int i = 0; i < kPerThread; ++i) adamw_elem(p.x[i], g.x[i], m.x[i], v.x[i], a);
        store8(P + e0, p);
        store8(r.m + e0, m);
        store8(r.v + e0, v);
    } else if (e0 < r.n) {
        // the tensor's last partial group: element by element
        for (int64_t e = e0; e < r.n && e < e0 + kPerThread; ++e) {
            float p = Elem<PT>::load(P + e), m = r.m[e], v = r.v[e];
            adamw_elem(p, Elem<GT>::load(G + e), m, v, a);
            Elem<PT>::store(P + e, p);
            r.m[e] = m;
            r.v[e] = v;
        }
    }
}

__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(AdamArgs a) {
    const int64_t bid = blockIdx.x;
    const int i = upper_index(a.count, bid, [&](int k) { return a.rec[k].block_begin; });
    const AdamRec& r = a.rec[i];
    const int64_t local = bid - r.block_begin;
    if (r.p_dtype == DMUON_BF16) {
        if (r.g_dtype == DMUON_BF16) adamw_block<uint16_t, uint16_t>(a, r, local);
        else adamw_block<uint16_t, float>(a, r, local);
    } else {
        if (r.g_dtype == DMUON_BF16) adamw_block<float, uint16_t>(a, r, local);
        else adamw_block<float, float>(a, r, local);
    }
}

}  // namespace

hipError_t launch_adamw(const AdamArgs& a, hipStream_t stream) {
    if (a.total_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)a.total_blocks), dim3(kAdamThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dmuon

// The three Newton-Schulz products in fp32 (the path taken for fp32
// gradients), same grouped launches and epilogues as the bf16 MFMA kernels:
// Gram A = s X X^T and square B = b A + c A A^T on upper-triangle tiles with
// mirrored stores, and X' = s (a X + B X) into the other X copy (computed as
// X'^T tiles: rows of the long side, columns of the short side).  Products are
// computed with fp32 FMA on 64 x 64 tiles, 256 threads, 4 x 4 outputs per
// thread, K staged through two LDS stages 16 at a time.
//
// Page basis: as for the bf16 kernels -- X X^T on the full matrix, one
// triangle of the symmetric products (DMuon explainer on gist.science, second
// section 2.1 Efficiente Gram Newton-Schulz Iteratie).
#include "kcommon.h"
#include "launch.h"

namespace dmuon {
namespace {

constexpr int kT = 64;
constexpr int kBKf = 16;

__device__ __forceinline__ void tri_decode_f(int t, int tm, int& I, int& J) {
    int i = 0;
    while (t >= tm - i) {
        t -= tm - i;
        ++i;
    }
    I = i;
    J = i + t;
}

template <int PHASE>
__global__ __launch_bounds__(256) void ns_gemm_f32_kernel(GemmArgs args) {
    // two LDS stages: slab k + 1 is fetched into registers while slab k is
    // multiplied, then written to the other stage, so one barrier per slab
    // suffices and the global load latency overlaps the FMAs
    __shared__ float Ps[2][kBKf][kT + 4];
    __shared__ float Qs[2][kBKf][kT + 4];

    const int bid = blockIdx.x;
    int s = 0;
    for (int i = 1; i < args.nseg; ++i)
        if (bid >= args.seg[i].first_block) s = i;
    const GemmSeg& sg = args.seg[s];
    const int local = bid - sg.first_block;
    const int slot = local / sg.tiles_per_mat;
    const int t = local - slot * sg.tiles_per_mat;
    const int plan_idx = sg.plan_base + slot;

    int I, J;
    const float *P, *Q;
    int64_t ldk, K;
    if (PHASE == kBX) {
        I = t / sg.tm;  // long-side tile
        J = t - I * sg.tm;
        P = reinterpret_cast<const float*>(args.ws + sg.p_off + slot * sg.x_stride);  // X: m x n
        Q = reinterpret_cast<const float*>(args.ws + sg.q_off + slot * sg.a_stride);
        ldk = sg.m_pad;
        K = sg.m_pad;
    } else {
        tri_decode_f(t, sg.tm, I, J);
        P = Q = reinterpret_cast<const float*>(args.ws + sg.p_off + slot * (PHASE == kGram ? sg.x_stride : sg.a_stride));
        ldk = PHASE == kGram ? sg.n_pad : sg.m_pad;
        K = ldk;
    }
    const float* Qt = Q + (int64_t)J * kT * ldk;

    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int lrow = tid >> 2, lk = (tid & 3) * 4;
    const int kk = tid >> 4, jj = (tid & 15) * 4;  // B X: X row k0 + kk, long-side columns jj .. jj + 3
    auto fetch = [&](int64_t k0, float4& pv, float4& qv) {
        if (PHASE == kBX)
            pv = *reinterpret_cast<const float4*>(P + (k0 + kk) * sg.n_pad + (int64_t)I * kT + jj);
        else
            pv = *reinterpret_cast<const float4*>(P + ((int64_t)I * kT + lrow) * ldk + k0 + lk);
        qv = *reinterpret_cast<const float4*>(Qt + lrow * ldk + k0 + lk);
    };
    auto stage = [&](int b, const float4& pv, const float4& qv) {
        if (PHASE == kBX) {
            // P[j][k] = X[k][j]
            Ps[b][kk][jj + 0] = pv.x; Ps[b][kk][jj + 1] = pv.y; Ps[b][kk][jj + 2] = pv.z; Ps[b][kk][jj + 3] = pv.w;
        } else {
            Ps[b][lk + 0][lrow] = pv.x; Ps[b][lk + 1][lrow] = pv.y; Ps[b][lk + 2][lrow] = pv.z; Ps[b][lk + 3][lrow] = pv.w;
        }
        Qs[b][lk + 0][lrow] = qv.x; Qs[b][lk + 1][lrow] = qv.y; Qs[b][lk + 2][lrow] = qv.z; Qs[b][lk + 3][lrow] = qv.w;
    };
    float acc[4][4] = {};
    float4 pv, qv;
    fetch(0, pv, qv);
    stage(0, pv, qv);
    __syncthreads();
    int b = 0;
    for (int64_t k0 = 0; k0 < K; k0 += kBKf) {
        const bool more = k0 + kBKf < K;
        if (more) fetch(k0 + kBKf, pv, qv);
        #pragma unroll
        for (int k = 0; k < kBKf; ++k) {
            const float4 av = *reinterpret_cast<const float4*>(&Ps[b][k][ty * 4]);
            const float4 bv = *reinterpret_cast<const float4*>(&Qs[b][k][tx * 4]);
            const float ar[4] = {av.x, av.y, av.z, av.w};
            const float br[4] = {bv.x, bv.y, bv.z, bv.w};
            #pragma unroll
            for (int i = 0; i < 4; ++i)
                #pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
        }
        // stage b ^ 1 was last read in the previous slab, before the barrier
        // that ended it; every thread is done with stage b after this one
        if (more) stage(b ^ 1, pv, qv);
        __syncthreads();
        b ^= 1;
    }

    // thread owns rows ty*4 + i and columns tx*4 + j of the 64 x 64 tile
    const float first_scale = sg.first_iter ? args.scale[plan_idx] : 1.0f;
    const int64_t r0 = (int64_t)I * kT + ty * 4, c0 = (int64_t)J * kT + tx * 4;
    if (PHASE == kBX) {
        // rows r of the tile are long-side indices, columns c short-side ones:
        // X'[c][r] = s (a X[c][r] + acc[r][c])
        const int64_t ldn = sg.n_pad;
        const float* Xs = P;
        float* Xd = reinterpret_cast<float*>(args.ws + sg.o_off + slot * sg.x_stride);
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 xs = *reinterpret_cast<const float4*>(Xs + (c0 + j) * ldn + r0);
            const float4 o = make_float4(first_scale * fmaf(args.a, xs.x, acc[0][j]),
                                         first_scale * fmaf(args.a, xs.y, acc[1][j]),
                                         first_scale * fmaf(args.a, xs.z, acc[2][j]),
                                         first_scale * fmaf(args.a, xs.w, acc[3][j]));
            *reinterpret_cast<float4*>(Xd + (c0 + j) * ldn + r0) = o;
        }
    } else {
        const int64_t ld = sg.m_pad;
        float* Out = reinterpret_cast<float*>(args.ws + sg.o_off + slot * sg.a_stride);
        const float alpha = PHASE == kGram ? first_scale * first_scale : args.c;
        float o[4][4];
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 ain = make_float4(0.f, 0.f, 0.f, 0.f);
            if (PHASE == kSquare) ain = *reinterpret_cast<const float4*>(P + (r0 + i) * ld + c0);
            const float ar[4] = {ain.x, ain.y, ain.z, ain.w};
            #pragma unroll
            for (int j = 0; j < 4; ++j) {
                float val = alpha * acc[i][j];
                if (PHASE == kSquare) val = fmaf(args.b, ar[j], val);
                o[i][j] = val;
            }
            *reinterpret_cast<float4*>(Out + (r0 + i) * ld + c0) = make_float4(o[i][0], o[i][1], o[i][2], o[i][3]);
        }
        if (I != J) {
            #pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4*>(Out + (c0 + j) * ld + r0) = make_float4(o[0][j], o[1][j], o[2][j], o[3][j]);
        }
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t stream) {
    if (a.total_blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)a.total_blocks), block(256);
    switch (a.phase) {
        case kGram: hipLaunchKernelGGL(ns_gemm_f32_kernel<kGram>, grid, block, 0, stream, a); break;
        case kSquare: hipLaunchKernelGGL(ns_gemm_f32_kernel<kSquare>, grid, block, 0, stream, a); break;
        case kBX: hipLaunchKernelGGL(ns_gemm_f32_kernel<kBX>, grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;  // fp32 buckets run the short-side recurrence only
    }
    return hipGetLastError();
}

}  // namespace dmuon

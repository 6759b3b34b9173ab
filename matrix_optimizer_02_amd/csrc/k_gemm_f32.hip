// The three Newton-Schulz products in fp32 (the path taken for fp32
// gradients), same grouped launches as the bf16 kernels: Gram A = s X X^T and
// square B = b A + c A A^T on upper-triangle tiles with mirrored stores, and
// X' = s (a X + B X) into the other X copy (computed as X'^T tiles: rows of
// the long side, columns of the short side).
//
// Matrix cores in fp32: v_mfma_f32_32x32x2_f32, one 32 x 32 output tile per
// workgroup of four waves.  Each wave sums a quarter of K into its own 32 x 32
// accumulator; the quarters are added in a fixed order (wave 0 + 1 + 2 + 3)
// through LDS, so results do not depend on timing.  The fp32 workloads are
// small (a single 256 x 512 matrix is the headline one): their launches are
// latency-bound, so the tile is small and K is split four ways to put more
// CUs on each product, and operands go from global memory straight into
// registers, a block of four 16-deep groups ahead of the one being multiplied.
//
// Operand layout per MFMA: lane l supplies row l % 32 of each operand at one
// k; the instruction sums two k, lanes 0-31 giving the first and 32-63 the
// second.  A lane's 8 MFMAs of a 16-deep group take k = 0..7 (lanes 0-31)
// and 8..15 (lanes 32-63) of the group, so each lane reads 8 consecutive k of
// its row (two 16-byte loads for K-contiguous rows).
//
// Page basis: as for the bf16 kernels -- X X^T on the full matrix, one
// triangle of the symmetric products (DMuon explainer on gist.science, second
// section 2.1 Efficiente Gram Newton-Schulz Iteratie).
#include "kcommon.h"
#include "launch.h"

namespace dmuon {
namespace {

constexpr int kT = 32;      // output tile edge
constexpr int kGroup = 16;  // k per group (8 MFMAs)
constexpr int kBlock = 4;   // groups per prefetch block

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
    __shared__ float red[3][16][64];     // partial tiles of waves 1..3, [wave - 1][register][lane]
    __shared__ float tile[kT][kT + 1];   // the summed tile, rows i, columns j

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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, half = lane >> 5;
    // this wave's quarter of K (K is a multiple of 64, so each quarter of 16)
    const int64_t kq = K / 4, kbeg = (int64_t)wave * kq;
    const int G = (int)(kq / kGroup);
    // the lane's rows: P row I T + r (B X: column I T + r of X, read k-major), Q row J T + r
    const float* prow = PHASE == kBX ? P + (int64_t)I * kT + r : P + ((int64_t)I * kT + r) * ldk;
    const float* qrow = Q + ((int64_t)J * kT + r) * ldk;

    auto load_group = [&](int g, float (&a)[8], float (&b)[8]) {
        const int64_t k = kbeg + (int64_t)g * kGroup + 8 * half;
        if (PHASE == kBX) {
            const int64_t ldn = sg.n_pad;
            #pragma unroll
            for (int u = 0; u < 8; ++u) a[u] = prow[(k + u) * ldn];
        } else {
            const float4 lo = *reinterpret_cast<const float4*>(prow + k);
            const float4 hi = *reinterpret_cast<const float4*>(prow + k + 4);
            a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
            a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
        }
        const float4 lo = *reinterpret_cast<const float4*>(qrow + k);
        const float4 hi = *reinterpret_cast<const float4*>(qrow + k + 4);
        b[0] = lo.x; b[1] = lo.y; b[2] = lo.z; b[3] = lo.w;
        b[4] = hi.x; b[5] = hi.y; b[6] = hi.z; b[7] = hi.w;
    };
    floatx16 acc;
    #pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    float a0[kBlock][8], b0[kBlock][8], a1[kBlock][8], b1[kBlock][8];
    auto load_block = [&](int blk, float (&a)[kBlock][8], float (&b)[kBlock][8]) {
        #pragma unroll
        for (int g = 0; g < kBlock; ++g)
            if (blk * kBlock + g < G) load_group(blk * kBlock + g, a[g], b[g]);
    };
    auto mul_block = [&](int blk, float (&a)[kBlock][8], float (&b)[kBlock][8]) {
        #pragma unroll
        for (int g = 0; g < kBlock; ++g) {
            if (blk * kBlock + g < G) {
                #pragma unroll
                for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[g][u], b[g][u], acc, 0, 0, 0);
            }
        }
    };
    // blocks alternate between two register sets: block b + 1 loads while block b multiplies
    load_block(0, a0, b0);
    for (int blk = 0; blk * kBlock < G; blk += 2) {
        if ((blk + 1) * kBlock < G) load_block(blk + 1, a1, b1);
        mul_block(blk, a0, b0);
        if ((blk + 1) * kBlock < G) {
            if ((blk + 2) * kBlock < G) load_block(blk + 2, a0, b0);
            mul_block(blk + 1, a1, b1);
        }
    }

    // the quarters, added in a fixed order; acc[v] is row 8 (v / 4) + 4 half + v % 4, column r
    if (wave > 0) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) red[wave - 1][v][lane] = acc[v];
    }
    __syncthreads();
    if (wave == 0) {
        #pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float sum = ((acc[v] + red[0][v][lane]) + red[1][v][lane]) + red[2][v][lane];
            tile[8 * (v / 4) + 4 * half + (v % 4)][r] = sum;
        }
    }
    __syncthreads();

    // epilogue: thread t takes row i = t / 8 and columns 4 (t % 8) .. + 3 of the tile
    const float first_scale = sg.first_iter ? args.scale[plan_idx] : 1.0f;
    const int ei = tid >> 3, ej = (tid & 7) * 4;
    if (PHASE == kBX) {
        // tile rows are long-side indices, columns short-side ones: X'[c][r] = s (a X[c][r] + C[r][c]);
        // thread t writes X' row c = J T + t / 8, columns r = I T + 4 (t % 8) .. + 3
        const int64_t ldn = sg.n_pad;
        const int64_t c = (int64_t)J * kT + ei, r0 = (int64_t)I * kT + ej;
        const float4 xs = *reinterpret_cast<const float4*>(P + c * ldn + r0);
        float* Xd = reinterpret_cast<float*>(args.ws + sg.o_off + slot * sg.x_stride);
        const float4 o = make_float4(first_scale * fmaf(args.a, xs.x, tile[ej + 0][ei]),
                                     first_scale * fmaf(args.a, xs.y, tile[ej + 1][ei]),
                                     first_scale * fmaf(args.a, xs.z, tile[ej + 2][ei]),
                                     first_scale * fmaf(args.a, xs.w, tile[ej + 3][ei]));
        *reinterpret_cast<float4*>(Xd + c * ldn + r0) = o;
    } else {
        const int64_t ld = sg.m_pad;
        float* Out = reinterpret_cast<float*>(args.ws + sg.o_off + slot * sg.a_stride);
        const float alpha = PHASE == kGram ? first_scale * first_scale : args.c;
        const int64_t gi = (int64_t)I * kT + ei, gj = (int64_t)J * kT + ej;
        float4 ain = make_float4(0.f, 0.f, 0.f, 0.f);
        if (PHASE == kSquare) ain = *reinterpret_cast<const float4*>(P + gi * ld + gj);
        const float ar[4] = {ain.x, ain.y, ain.z, ain.w};
        float o[4];
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            float val = alpha * tile[ei][ej + j];
            if (PHASE == kSquare) val = fmaf(args.b, ar[j], val);
            o[j] = val;
        }
        *reinterpret_cast<float4*>(Out + gi * ld + gj) = make_float4(o[0], o[1], o[2], o[3]);
        if (I != J) {
            // the mirror block: the final values, transposed through the tile
            __syncthreads();
            #pragma unroll
            for (int j = 0; j < 4; ++j) tile[ei][ej + j] = o[j];
            __syncthreads();
            // thread t writes mirror row J T + t / 8, columns I T + 4 (t % 8) .. + 3
            const float4 m = make_float4(tile[ej + 0][ei], tile[ej + 1][ei], tile[ej + 2][ei], tile[ej + 3][ei]);
            *reinterpret_cast<float4*>(Out + ((int64_t)J * kT + ei) * ld + (int64_t)I * kT + ej) = m;
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

int f32_kernel_tile() { return kT; }

}  // namespace dmuon

// The three Newton-Schulz products on bf16 MFMA (gfx950), one grouped launch
// per phase over every bucket of the batch:
//   Gram    A  = s X X^T           upper-triangle tiles only, mirrored store
//   square  B  = b A + c A A^T     (A A = A A^T: A is symmetric) upper tiles only
//   BX      X' = s (a X + B X)     computed as X'^T = s (a X^T + X^T B^T), B = B^T,
//                                  stored both as X'^T and (transposed) as X'
// s is 1 / (||U||_F + eps) in the first iteration (s^2 for the Gram) and 1
// afterwards.  Every product is an "NT" product C[i][j] = sum_k P[i][k] Q[j][k]
// whose operands are K-contiguous rows, which is why X is kept in both
// orientations.
//
// Page basis: X X^T is the dominant product and, being symmetric, is computed
// as one triangle only, halving its arithmetic (DMuon explainer on
// gist.science, second section 2.1 Efficiente Gram Newton-Schulz Iteratie,
// "Benutting van Symmetrie"); matrices of similar shapes run jointly to keep
// the GPU occupied and amortise dispatch (same section, "Batching").
//
// Tile: T x T outputs per 256-thread workgroup (T = 256 or 128), 4 waves in a
// 2 x 2 grid, each wave (T/2) x (T/2) outputs as (T/64)^2 blocks of
// v_mfma_f32_32x32x16_bf16; K staged through LDS in 64-wide slabs, two
// stages, 16-byte chunks XOR-swizzled by row so that the fragment reads of
// eight consecutive rows hit eight distinct bank groups.
#include "kcommon.h"
#include "launch.h"

namespace dmuon {
namespace {

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kBK = 64;          // K slab
constexpr int kRowBytes = kBK * 2;  // one LDS row of a slab: 128 bytes, 8 chunks of 16 bytes

template <int T>
struct TileCfg {
    static constexpr int WT = T / 2;           // wave tile
    static constexpr int F = WT / 32;          // MFMA blocks per wave per dim
    static constexpr int kDmaPerOp = T / 32;   // 1 KB direct loads per wave per operand per slab
    static constexpr int kOperandBytes = T * kRowBytes;
    static constexpr int kStageBytes = 2 * kOperandBytes;
};

__device__ __forceinline__ void tri_decode(int t, int tm, int& I, int& J) {
    int i = 0;
    while (t >= tm - i) {
        t -= tm - i;
        ++i;
    }
    I = i;
    J = i + t;
}

template <int T, int PHASE>
__global__ __launch_bounds__(256, 1) void ns_gemm_bf16_kernel(GemmArgs args) {
    using C = TileCfg<T>;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::kStageBytes];

    // ---- which tile of which matrix --------------------------------------------
    const int bid = blockIdx.x;
    int s = 0;
    for (int i = 1; i < args.nseg; ++i)
        if (bid >= args.seg[i].first_block) s = i;
    const GemmSeg& sg = args.seg[s];
    const int local = bid - sg.first_block;
    const int slot = local / sg.tiles_per_mat;
    const int t = local - slot * sg.tiles_per_mat;
    const int plan_idx = sg.plan_base + slot;

    int I, J;  // tile coordinates in the output (row tile, column tile)
    const uint16_t *P, *Q;
    int64_t ldk;  // leading dimension (= K extent) of P and Q
    int64_t K;
    if (PHASE == kBX) {
        I = t / sg.tm;  // long-side tile (rows of X^T)
        J = t - I * sg.tm;
        P = reinterpret_cast<const uint16_t*>(args.ws + sg.xt_src_off + slot * sg.x_stride);
        Q = reinterpret_cast<const uint16_t*>(args.ws + sg.b_off + slot * sg.a_stride);
        ldk = sg.m_pad;
        K = sg.m_pad;
    } else {
        tri_decode(t, sg.tm, I, J);
        const int64_t off = PHASE == kGram ? sg.x_off + slot * sg.x_stride : sg.a_off + slot * sg.a_stride;
        P = Q = reinterpret_cast<const uint16_t*>(args.ws + off);
        ldk = PHASE == kGram ? sg.n_pad : sg.m_pad;
        K = ldk;
    }
    const uint16_t* Pt = P + (int64_t)I * T * ldk;  // first row of this tile's P panel
    const uint16_t* Qt = Q + (int64_t)J * T * ldk;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    // ---- global -> LDS (direct), two stages ------------------------------------------
    // A slab is 64 K-values of T rows per operand: 128-byte LDS rows, 8 chunks of
    // 16 bytes.  One global_load_lds_dwordx4 of a wave fills 1 KB = 8 rows: lane l
    // writes physical chunk l % 8 of row 8 q + l / 8.  Logical chunk ch of row r is
    // stored at physical chunk ch ^ (r % 8) ^ ((r / 8) % 2), so the fragment reads
    // of 8 (or 16) consecutive rows at one logical chunk hit distinct banks.
    auto dma = [&](int64_t k0, int stage) {
        char* sbase = smem + stage * C::kStageBytes;
        #pragma unroll
        for (int i = 0; i < C::kDmaPerOp; ++i) {
            const int q = wave * C::kDmaPerOp + i;  // 1 KB block (8 rows) of the operand tile
            const int row = 8 * q + (lane >> 3);
            const int lc = (lane & 7) ^ (lane >> 3) ^ (q & 1);
            const int64_t go = (int64_t)row * ldk + k0 + lc * 8;
            __builtin_amdgcn_global_load_lds((gptr_t)(Pt + go), (lptr_t)(sbase + q * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gptr_t)(Qt + go),
                                             (lptr_t)(sbase + C::kOperandBytes + q * 1024), 16, 0, 0);
        }
    };

    floatx16 acc[C::F][C::F];
    #pragma unroll
    for (int i = 0; i < C::F; ++i)
        #pragma unroll
        for (int j = 0; j < C::F; ++j)
            #pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int lrow = lane & 31, khalf = lane >> 5;
    const int swz = (lane & 7) ^ ((lane >> 3) & 1);
    const int a_row0 = (wr * C::WT + lrow) * kRowBytes;
    const int b_row0 = (wc * C::WT + lrow) * kRowBytes;
    bf16x8 fa0[C::F], fb0[C::F], fa1[C::F], fb1[C::F];

#define DMUON_READ(FA, FB, BASE, KS)                                                              \
    do {                                                                                          \
        const int pc_ = ((((KS) * 2 + khalf) ^ swz) << 4);                                        \
        _Pragma("unroll") for (int i_ = 0; i_ < C::F; ++i_)                                       \
            FA[i_] = *reinterpret_cast<const bf16x8*>((BASE) + a_row0 + i_ * 32 * kRowBytes + pc_); \
        _Pragma("unroll") for (int j_ = 0; j_ < C::F; ++j_)                                       \
            FB[j_] = *reinterpret_cast<const bf16x8*>((BASE) + C::kOperandBytes + b_row0 +          \
                                                      j_ * 32 * kRowBytes + pc_);                 \
    } while (0)
#define DMUON_MFMA(FA, FB)                                                                        \
    do {                                                                                          \
        _Pragma("unroll") for (int i_ = 0; i_ < C::F; ++i_)                                       \
            _Pragma("unroll") for (int j_ = 0; j_ < C::F; ++j_)                                   \
                acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i_], FB[j_], acc[i_][j_], 0, 0, 0); \
    } while (0)

    const int KT = (int)(K / kBK);
    dma(0, 0);
    if (KT > 1) dma(kBK, 1);
    // The compiler does not count direct-to-LDS loads in its barrier waits:
    // every wait for them below is explicit.  Slab 0 has landed once only
    // slab 1's loads (issued after it) may still be outstanding.
    static_assert(2 * C::kDmaPerOp == 16 || 2 * C::kDmaPerOp == 8, "vmcnt below");
    if (KT == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (2 * C::kDmaPerOp == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();
    DMUON_READ(fa0, fb0, smem, 0);
    for (int kt = 0; kt < KT; ++kt) {
        const char* cur = smem + (kt & 1) * C::kStageBytes;
        DMUON_READ(fa1, fb1, cur, 1);
        DMUON_MFMA(fa0, fb0);
        DMUON_READ(fa0, fb0, cur, 2);
        DMUON_MFMA(fa1, fb1);
        DMUON_READ(fa1, fb1, cur, 3);
        DMUON_MFMA(fa0, fb0);
        if (kt + 1 < KT) {
            // this wave's loads of slab kt + 1 (the only ones outstanding) have
            // landed; the barrier then publishes every wave's share and makes
            // sure every wave is done reading slab kt before it is overwritten
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (kt + 2 < KT) dma((int64_t)(kt + 2) * kBK, kt & 1);
            DMUON_READ(fa0, fb0, smem + ((kt + 1) & 1) * C::kStageBytes, 0);
        }
        DMUON_MFMA(fa1, fb1);
    }
#undef DMUON_READ
#undef DMUON_MFMA

    // ---- epilogue -----------------------------------------------------------------
    // acc[i][j][v] holds output row  wr*WT + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4
    //                  and column  wc*WT + 32 j + lane % 32   of the T x T tile.
    const float first_scale = args.first_iter ? args.scale[plan_idx] : 1.0f;
    if (PHASE == kBX) {
        const int64_t ldm = sg.m_pad, ldn = sg.n_pad;
        const uint16_t* XTs = P;
        uint16_t* XTd = reinterpret_cast<uint16_t*>(args.ws + sg.xt_dst_off + slot * sg.x_stride);
        uint16_t* X = reinterpret_cast<uint16_t*>(args.ws + sg.x_off + slot * sg.x_stride);
        const float a = args.a;
        #pragma unroll
        for (int i = 0; i < C::F; ++i)
            #pragma unroll
            for (int j = 0; j < C::F; ++j)
                #pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int64_t r0 = (int64_t)I * T + wr * C::WT + i * 32 + 8 * v4 + 4 * khalf;  // long-side index
                    const int64_t c = (int64_t)J * T + wc * C::WT + j * 32 + lrow;              // short-side index
                    uint16_t o[4];
                    #pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int64_t e = (r0 + v) * ldm + c;
                        const float val = first_scale * fmaf(a, bf16_to_f32(XTs[e]), acc[i][j][4 * v4 + v]);
                        o[v] = f32_to_bf16(val);
                        XTd[e] = o[v];
                    }
                    uint2 pk;
                    pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                    pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                    *reinterpret_cast<uint2*>(X + c * ldn + r0) = pk;
                }
    } else {
        const int64_t ld = sg.m_pad;
        const int64_t out_off = PHASE == kGram ? sg.a_off + slot * sg.a_stride : sg.b_off + slot * sg.a_stride;
        uint16_t* Out = reinterpret_cast<uint16_t*>(args.ws + out_off);
        const uint16_t* Ain = P;  // A, for the square phase's b A term
        const float alpha = PHASE == kGram ? first_scale * first_scale : args.c;
        const float beta = args.b;
        const bool mirror = I != J;
        #pragma unroll
        for (int i = 0; i < C::F; ++i)
            #pragma unroll
            for (int j = 0; j < C::F; ++j)
                #pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int64_t r0 = (int64_t)I * T + wr * C::WT + i * 32 + 8 * v4 + 4 * khalf;
                    const int64_t c = (int64_t)J * T + wc * C::WT + j * 32 + lrow;
                    uint16_t o[4];
                    #pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int64_t e = (r0 + v) * ld + c;
                        float val = alpha * acc[i][j][4 * v4 + v];
                        if (PHASE == kSquare) val = fmaf(beta, bf16_to_f32(Ain[e]), val);
                        o[v] = f32_to_bf16(val);
                        Out[e] = o[v];
                    }
                    if (mirror) {
                        uint2 pk;
                        pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                        pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                        *reinterpret_cast<uint2*>(Out + c * ld + r0) = pk;
                    }
                }
    }
}

template <int T>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.total_blocks), block(256);
    switch (a.phase) {
        case kGram: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kGram>), grid, block, 0, stream, a); break;
        case kSquare: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kSquare>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kBX>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(int tile, const GemmArgs& a, hipStream_t stream) {
    if (a.total_blocks <= 0) return hipSuccess;
    if (tile == 256) return launch_tile<256>(a, stream);
    if (tile == 128) return launch_tile<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace dmuon

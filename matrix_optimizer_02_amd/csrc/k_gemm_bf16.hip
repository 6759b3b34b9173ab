// The three Newton-Schulz products on bf16 MFMA (gfx950), one grouped launch
// per phase over every bucket of the batch:
//   Gram    A  = s X X^T           upper-triangle tiles only, mirrored store
//   square  B  = b A + c A A^T     (A A = A A^T: A is symmetric) upper tiles only
//   BX      X' = s (a X + B X)     into the other X copy
// s is 1 / (||U||_F + eps) in the first iteration (s^2 for the Gram) and 1
// afterwards.  Each product is computed as C[i][j] = sum_k P[i][k] Q[j][k]:
// for the Gram and square P = Q = X or A, whose rows are K-contiguous; for B X
// the output tile is X'^T (rows along the long side n, columns along the short
// side m), P[j][k] = X[k][j] is fetched from the K-major X slab with the gfx950
// transposing LDS read, and Q = B.
//
// Page basis: X X^T is the dominant product and, being symmetric, is computed
// as one triangle only, halving its arithmetic (DMuon explainer on
// gist.science, second section 2.1 Efficiente Gram Newton-Schulz Iteratie,
// "Benutting van Symmetrie"); matrices of similar shapes run jointly to keep
// the GPU occupied and amortise dispatch (same section, "Batching").
//
// Tile: T x T outputs per 256-thread workgroup (T = 256 or 128), 4 waves in a
// 2 x 2 grid, each wave (T/2) x (T/2) outputs as (T/64)^2 blocks of
// v_mfma_f32_32x32x16_bf16.  K is staged through LDS in slabs by direct
// global->LDS loads, S stages deep; 16-byte chunks are XOR-swizzled by row so
// that the fragment reads hit distinct banks.  Each MFMA k-step is its own
// scheduling region: its MFMAs interleaved with the next k-step's fragment
// reads.  The B X epilogue stages the output tile through LDS so that both the
// a X read and the X' write are coalesced 16-byte accesses.
#include "kcommon.h"
#include "launch.h"
#include "tile_map.h"

#ifndef DMUON_BK
#define DMUON_BK 64
#endif
#ifndef DMUON_STAGES_256
#define DMUON_STAGES_256 2
#endif
#ifndef DMUON_XCD_REMAP
#define DMUON_XCD_REMAP 0
#endif
#ifndef DMUON_BANDED
#define DMUON_BANDED 1
#endif
#ifndef DMUON_L2_PREFETCH
#define DMUON_L2_PREFETCH 0
#endif

namespace dmuon {
namespace {

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kBK = DMUON_BK;            // K slab: 32 or 64
constexpr int kRowBytes = kBK * 2;       // one LDS row of a K-contiguous slab
constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per such row
constexpr int kDmaRows = 1024 / kRowBytes;  // rows one 1 KB wave load fills
static_assert(kBK == 32 || kBK == 64, "slab width");

template <int T, int S>
struct TileCfg {
    static constexpr int WT = T / 2;               // wave tile
    static constexpr int F = WT / 32;              // MFMA blocks per wave per dim
    static constexpr int kDmaPerOp = T * kRowBytes / 1024 / 4;  // 1 KB loads per wave per operand per slab
    static constexpr int kDmaPerSlab = 2 * kDmaPerOp;
    static constexpr int kOperandBytes = T * kRowBytes;
    static constexpr int kStageBytes = 2 * kOperandBytes;
    // B X: the P slab is kBK rows (k) of T long-side values
    static constexpr int kPRowBytes = 2 * T;
    static constexpr int kPChunks = kPRowBytes / 16;
    static constexpr int kPDmaRows = 1024 / kPRowBytes;
};

// K-contiguous slab rows: logical chunk ch of row r sits at ch ^ swizzle(r), so
// the fragment reads of 8 (or 16) consecutive rows at one logical chunk hit
// distinct bank groups whether the LDS serves 128 or 256 bytes a clock.
__device__ __forceinline__ int swizzle(int r) {
    if (kBK == 32) return ((r >> 1) ^ (r >> 3)) & 3;
    return (r & 7) ^ ((r >> 3) & 1);
}

// B X P slab (rows k, long-side columns): a transposing read takes 4 rows of
// one 16-lane group; rows r..r+3 get chunk offsets 0, 4, 10, 14 so that the
// 8 chunks of a group (and the 16 of two groups) fall in distinct bank groups.
__device__ __forceinline__ int swizzle_p(int r) { return (0xEA40 >> ((r & 3) * 4)) & 15; }

// B X epilogue tile (rows short side, long-side columns): one chunk swizzle
// per row, over the row's T / 8 chunks.
template <int T>
__device__ __forceinline__ int swizzle_e(int r) { return r & (T / 8 - 1); }

template <int T, int PHASE, int S>
__global__ __launch_bounds__(256, 1) void ns_gemm_bf16_kernel(GemmArgs args) {
    using C = TileCfg<T, S>;
    // S stages, then 1 KB that L2 prefetches land in (never read)
    __shared__ __attribute__((aligned(1024))) char smem[S * C::kStageBytes + 1024];
    constexpr bool kPrefetch = DMUON_L2_PREFETCH && S == 2 && kBK == 64;
    static_assert(PHASE != kBX || S * C::kStageBytes >= 2 * T * T, "B X epilogue tile fits the stages");

    // ---- which tile of which matrix --------------------------------------------
    int s, local;
    if (DMUON_XCD_REMAP) {
        xcd_map((int)blockIdx.x, args.nseg,
                [&](int i) { return args.seg[i].count * args.seg[i].tiles_per_mat; },
                [&](int i) { return args.seg[i].first_block; }, s, local);
    } else {
        s = 0;
        for (int i = 1; i < args.nseg; ++i)
            if ((int)blockIdx.x >= args.seg[i].first_block) s = i;
        local = (int)blockIdx.x - args.seg[s].first_block;
    }
    const GemmSeg& sg = args.seg[s];
    const int slot = local / sg.tiles_per_mat;
    const int t = local - slot * sg.tiles_per_mat;
    const int plan_idx = sg.plan_base + slot;

    int I, J;  // tile coordinates in the output (row tile, column tile)
    const uint16_t *P, *Q;
    int64_t ldq;  // leading dimension of Q's rows (= K extent)
    if (PHASE == kBX) {
        if (DMUON_BANDED) {
            bx_decode_banded(t, sg.tn, sg.tm, I, J);  // I: long-side tile, J: short-side tile
        } else {
            I = t / sg.tm;
            J = t - I * sg.tm;
        }
        P = reinterpret_cast<const uint16_t*>(args.ws + sg.x_src_off + slot * sg.x_stride);  // X: m x n
        Q = reinterpret_cast<const uint16_t*>(args.ws + sg.b_off + slot * sg.a_stride);
        ldq = sg.m_pad;
    } else {
        if (DMUON_BANDED) {
            tri_decode_banded(t, sg.tm, I, J);
        } else {
            int tt = t, i = 0;
            while (tt >= sg.tm - i) {
                tt -= sg.tm - i;
                ++i;
            }
            I = i;
            J = i + tt;
        }
        const int64_t off = PHASE == kGram ? sg.x_src_off + slot * sg.x_stride : sg.a_off + slot * sg.a_stride;
        P = Q = reinterpret_cast<const uint16_t*>(args.ws + off);
        ldq = PHASE == kGram ? sg.n_pad : sg.m_pad;
    }
    const int64_t K = ldq;
    const uint16_t* Qt = Q + (int64_t)J * T * ldq;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    // ---- global -> LDS (direct), S stages ---------------------------------------------
    // One global_load_lds_dwordx4 of a wave fills 1 KB of LDS: lane l writes
    // bytes 16 l .. 16 l + 15 of it, so it fetches the global chunk that the
    // swizzle places there.
    auto dma = [&](int64_t k0, int stage) {
        char* sbase = smem + stage * C::kStageBytes;
        #pragma unroll
        for (int i = 0; i < C::kDmaPerOp; ++i) {
            const int q = wave * C::kDmaPerOp + i;  // 1 KB block of the operand slab
            const uint16_t* gp;
            if (PHASE == kBX) {
                // P slab: X rows k0 .. k0 + kBK - 1, long-side columns I T .. I T + T - 1
                const int row = C::kPDmaRows * q + lane / C::kPChunks;
                const int lc = (lane % C::kPChunks) ^ swizzle_p(row);
                gp = P + (k0 + row) * sg.n_pad + (int64_t)I * T + lc * 8;
            } else {
                const int row = kDmaRows * q + lane / kChunks;
                const int lc = (lane % kChunks) ^ swizzle(row);
                gp = P + ((int64_t)I * T + row) * ldq + k0 + lc * 8;
            }
            __builtin_amdgcn_global_load_lds((gptr_t)gp, (lptr_t)(sbase + q * 1024), 16, 0, 0);
            const int qrow = kDmaRows * q + lane / kChunks;
            const int qlc = (lane % kChunks) ^ swizzle(qrow);
            __builtin_amdgcn_global_load_lds((gptr_t)(Qt + (int64_t)qrow * ldq + k0 + qlc * 8),
                                             (lptr_t)(sbase + C::kOperandBytes + q * 1024), 16, 0, 0);
        }
    };

    // L2 prefetch of a slab: every 128-byte line of both operand slabs is
    // touched by one lane (4 bytes, landing in the scratch KB), so the slab's
    // direct loads issued one slab later hit L2.  Every wave issues the same
    // number of them (one per operand; T = 128 touches some lines twice), which
    // keeps the load counts the waits rely on uniform.
    constexpr int kLinesPerOp = T * kRowBytes / 128;  // = kBK * 2 T / 128 for the B X P slab
    constexpr int kPfPerOp = kLinesPerOp / 256 > 0 ? kLinesPerOp / 256 : 1;
    auto prefetch = [&](int64_t k0) {
        char* scratch = smem + S * C::kStageBytes;
        #pragma unroll
        for (int i = 0; i < kPfPerOp; ++i) {
            const int id = ((wave * kPfPerOp + i) * 64 + lane) % kLinesPerOp;  // line of the slab
            const uint16_t* gp;
            if (PHASE == kBX) {
                constexpr int kLinesPerRow = 2 * T / 128;
                gp = P + (k0 + id / kLinesPerRow) * sg.n_pad + (int64_t)I * T + (id % kLinesPerRow) * 64;
            } else {
                gp = P + ((int64_t)I * T + id) * ldq + k0;
            }
            __builtin_amdgcn_global_load_lds((gptr_t)gp, (lptr_t)scratch, 4, 0, 0);
            __builtin_amdgcn_global_load_lds((gptr_t)(Qt + (int64_t)id * ldq + k0), (lptr_t)scratch, 4, 0, 0);
        }
    };
    constexpr int kPfPerSlab = kPrefetch ? 2 * kPfPerOp : 0;  // prefetch loads per wave per slab

    floatx16 acc[C::F][C::F];
    #pragma unroll
    for (int i = 0; i < C::F; ++i)
        #pragma unroll
        for (int j = 0; j < C::F; ++j)
            #pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int lrow = lane & 31, khalf = lane >> 5;
    const int swz = swizzle(lrow);  // fragment rows start at multiples of 32
    const int a_row0 = (wr * C::WT + lrow) * kRowBytes;
    const int b_row0 = (wc * C::WT + lrow) * kRowBytes;
    // B X transposing read: lane 16 g + s of a 16-lane group g addresses row
    // (s / 4) and columns 4 (s % 4) .. + 3 of a 4 x 16 block; it receives that
    // block's column s, i.e. 4 consecutive k of output row jbase + s.
    const int tr_g = lane >> 4, tr_s = lane & 15;
    const int tr_row = 8 * (tr_g >> 1) + (tr_s >> 2);                 // + 16 ks + 4 half
    const int tr_col = wr * C::WT + 16 * (tr_g & 1) + 4 * (tr_s & 3);  // + 32 fi
    const int tr_sw = swizzle_p(tr_s >> 2);                           // rows are 4-aligned
    bf16x8 fa[2][C::F], fb[2][C::F];

#define DMUON_READ_A(BUF, BASE, KS)                                                               \
    do {                                                                                          \
        if (PHASE == kBX) {                                                                       \
            _Pragma("unroll") for (int i_ = 0; i_ < C::F; ++i_) {                                 \
                shortx4 h_[2];                                                                    \
                _Pragma("unroll") for (int t_ = 0; t_ < 2; ++t_) {                                \
                    const int r_ = 16 * (KS) + 4 * t_ + tr_row;                                   \
                    const int c_ = tr_col + 32 * i_;                                              \
                    const int o_ = r_ * C::kPRowBytes + (((c_ >> 3) ^ tr_sw) << 4) + (c_ & 7) * 2; \
                    h_[t_] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                             \
                        (lds_shortx4*)((__attribute__((address_space(3))) char*)(BASE) + o_));    \
                }                                                                                 \
                const shortx8 w_ = __builtin_shufflevector(h_[0], h_[1], 0, 1, 2, 3, 4, 5, 6, 7); \
                fa[BUF][i_] = __builtin_bit_cast(bf16x8, w_);                                     \
            }                                                                                     \
        } else {                                                                                  \
            const int pc_ = ((((KS) * 2 + khalf) ^ swz) << 4);                                    \
            _Pragma("unroll") for (int i_ = 0; i_ < C::F; ++i_)                                   \
                fa[BUF][i_] = *reinterpret_cast<const bf16x8*>((BASE) + a_row0 + i_ * 32 * kRowBytes + pc_); \
        }                                                                                         \
    } while (0)
#define DMUON_READ(BUF, BASE, KS)                                                                 \
    do {                                                                                          \
        DMUON_READ_A(BUF, BASE, KS);                                                              \
        const int pc_ = ((((KS) * 2 + khalf) ^ swz) << 4);                                        \
        _Pragma("unroll") for (int j_ = 0; j_ < C::F; ++j_)                                       \
            fb[BUF][j_] = *reinterpret_cast<const bf16x8*>((BASE) + C::kOperandBytes + b_row0 +     \
                                                           j_ * 32 * kRowBytes + pc_);            \
    } while (0)
#define DMUON_MFMA(BUF)                                                                           \
    do {                                                                                          \
        _Pragma("unroll") for (int i_ = 0; i_ < C::F; ++i_)                                       \
            _Pragma("unroll") for (int j_ = 0; j_ < C::F; ++j_)                                   \
                acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[BUF][i_], fb[BUF][j_],   \
                                                                      acc[i_][j_], 0, 0, 0);      \
    } while (0)

    // Wait until at most n of this wave's loads are in flight (loads complete in
    // issue order).  The compiler does not count direct-to-LDS loads in its own
    // waits, so every wait for them is explicit.
    static_assert(S >= 2 && S <= 5, "waits cover up to 4 slabs in flight");
    static_assert(C::kDmaPerSlab == 16 || C::kDmaPerSlab == 8 || C::kDmaPerSlab == 4, "vmcnt encodings");
    auto wait_vm = [&](int n) {
        switch (n) {
            case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
            case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
            case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
            case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
            case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
            case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
            case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
            case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
            case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
            case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;  // 0, or drain
        }
    };
    auto wait_slabs = [&](int slabs) { wait_vm(slabs <= 0 ? 0 : slabs * C::kDmaPerSlab); };

    const int KT = (int)(K / kBK);
    // prologue: slabs 0 .. S-1 into stages 0 .. S-1 (and the L2 prefetch of
    // slab S); wait for slab 0
    #pragma unroll
    for (int st = 0; st < S; ++st)
        if (st < KT) dma((int64_t)st * kBK, st);
    if (kPrefetch) {
        const bool pf = S < KT;
        if (pf) prefetch((int64_t)S * kBK);
        wait_vm(KT > 1 ? C::kDmaPerSlab + (pf ? kPfPerSlab : 0) : 0);
    } else {
        wait_slabs(min(S, KT) - 1);
    }
    __syncthreads();
    DMUON_READ(0, smem, 0);
    constexpr int KS = kBK / 16;  // MFMA k-steps per slab (even)
    constexpr int NREAD = (PHASE == kBX ? 3 : 2) * C::F;  // fragment reads per k-step
    constexpr int NMFMA = C::F * C::F;                    // MFMAs per k-step
    // One k-step as its own scheduling region: each of the first MFMAs is
    // followed by one fragment read for the next k-step, so the reads are in
    // flight while the matrix pipe is busy and have landed before they are used
    // (the MFMA leading the region only waits on reads issued a region earlier).
#define DMUON_INTERLEAVE()                                                                        \
    do {                                                                                          \
        _Pragma("unroll") for (int g_ = 0; g_ < (NREAD < NMFMA ? NREAD : NMFMA); ++g_) {          \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */                         \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* DS read */                      \
        }                                                                                         \
        if (NMFMA > NREAD) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NREAD, 0);         \
        if (NREAD > NMFMA) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NMFMA, 0);         \
        __builtin_amdgcn_sched_barrier(0);                                                        \
    } while (0)
    // all slabs but the last: the last k-step also waits for the next slab,
    // refills the freed stage and reads the next slab's first fragments
    for (int kt = 0; kt + 1 < KT; ++kt) {
        const int stage = kt % S;
        const char* cur = smem + stage * C::kStageBytes;
        #pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            DMUON_READ((ks + 1) & 1, cur, ks + 1);
            DMUON_MFMA(ks & 1);
            DMUON_INTERLEAVE();
        }
        // Issued so far: slabs 0 .. min(kt + S - 1, KT - 1).  Slab kt + 1 has
        // landed once only the ones after it are in flight; the barrier then
        // publishes every wave's share and makes sure every wave is done
        // reading slab kt, whose stage is refilled with slab kt + S.
        if (kPrefetch) {
            // S = 2: issued after slab kt + 1's loads is only the prefetch of slab kt + 2
            wait_vm(kt + 2 < KT ? kPfPerSlab : 0);
        } else {
            wait_slabs(min(kt + S - 1, KT - 1) - (kt + 1));
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if (kt + S < KT) dma((int64_t)(kt + S) * kBK, stage);
        if (kPrefetch && kt + S + 1 < KT) prefetch((int64_t)(kt + S + 1) * kBK);
        __builtin_amdgcn_sched_barrier(0);
        DMUON_READ(0, smem + ((kt + 1) % S) * C::kStageBytes, 0);
        DMUON_MFMA((KS - 1) & 1);
        DMUON_INTERLEAVE();
    }
    {   // the last slab
        const char* cur = smem + ((KT - 1) % S) * C::kStageBytes;
        #pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            DMUON_READ((ks + 1) & 1, cur, ks + 1);
            DMUON_MFMA(ks & 1);
            DMUON_INTERLEAVE();
        }
        DMUON_MFMA((KS - 1) & 1);
    }
#undef DMUON_INTERLEAVE
#undef DMUON_READ
#undef DMUON_READ_A
#undef DMUON_MFMA

    // ---- epilogue -----------------------------------------------------------------
    // acc[i][j][v] holds output row  wr*WT + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4
    //                  and column  wc*WT + 32 j + lane % 32   of the T x T tile.
    const float first_scale = args.first_iter ? args.scale[plan_idx] : 1.0f;
    if (PHASE == kBX) {
        // Tile rows are long-side indices r, columns short-side indices c:
        // X'[c][r] = s (a X[c][r] + acc[r][c]).  The X tile (T rows c, T
        // columns r) goes through LDS: loaded whole, updated in place by each
        // lane's own elements, stored whole.
        constexpr int kERowBytes = 2 * T, kEChunks = T / 8;
        const int64_t ldn = sg.n_pad;
        const uint16_t* Xs = P + (int64_t)J * T * ldn + (int64_t)I * T;
        uint16_t* Xd = reinterpret_cast<uint16_t*>(args.ws + sg.x_dst_off + slot * sg.x_stride) +
                       (int64_t)J * T * ldn + (int64_t)I * T;
        __syncthreads();  // every wave is done with the last slab
        constexpr int kLoads = T * kERowBytes / 1024 / 4;  // 1 KB loads per wave
        #pragma unroll 8
        for (int i = 0; i < kLoads; ++i) {
            const int q = wave * kLoads + i;
            const int row = (1024 / kERowBytes) * q + lane / kEChunks;
            const int lc = (lane % kEChunks) ^ swizzle_e<T>(row);
            __builtin_amdgcn_global_load_lds((gptr_t)(Xs + row * ldn + lc * 8), (lptr_t)(smem + q * 1024),
                                             16, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const float a = args.a;
        #pragma unroll
        for (int i = 0; i < C::F; ++i)
            #pragma unroll
            for (int j = 0; j < C::F; ++j)
                #pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int r0 = wr * C::WT + i * 32 + 8 * v4 + 4 * khalf;  // long-side (column of X)
                    const int c = wc * C::WT + j * 32 + lrow;                 // short-side (row of X)
                    char* p = smem + c * kERowBytes + (((r0 >> 3) ^ swizzle_e<T>(c)) << 4) + (r0 & 7) * 2;
                    const uint2 x = *reinterpret_cast<const uint2*>(p);
                    const float x0 = __uint_as_float(x.x << 16), x1 = __uint_as_float(x.x & 0xffff0000u);
                    const float x2 = __uint_as_float(x.y << 16), x3 = __uint_as_float(x.y & 0xffff0000u);
                    uint2 o;
                    o.x = (uint32_t)f32_to_bf16(first_scale * fmaf(a, x0, acc[i][j][4 * v4 + 0])) |
                          ((uint32_t)f32_to_bf16(first_scale * fmaf(a, x1, acc[i][j][4 * v4 + 1])) << 16);
                    o.y = (uint32_t)f32_to_bf16(first_scale * fmaf(a, x2, acc[i][j][4 * v4 + 2])) |
                          ((uint32_t)f32_to_bf16(first_scale * fmaf(a, x3, acc[i][j][4 * v4 + 3])) << 16);
                    *reinterpret_cast<uint2*>(p) = o;
                }
        __syncthreads();
        constexpr int kStores = T * kEChunks / 256;
        #pragma unroll 8
        for (int i = 0; i < kStores; ++i) {
            const int q = tid + 256 * i;
            const int row = q / kEChunks, lc = q % kEChunks;
            const uint4 v = *reinterpret_cast<const uint4*>(smem + row * kERowBytes +
                                                            ((lc ^ swizzle_e<T>(row)) << 4));
            *reinterpret_cast<uint4*>(Xd + row * ldn + lc * 8) = v;
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

// Pipeline depth per tile size.  A T = 256 stage is 64 KB with 64-wide slabs
// (32 KB with 32-wide), a T = 128 stage a quarter of that.
template <int T> struct Depth;
template <> struct Depth<256> { static constexpr int S = DMUON_STAGES_256; };
template <> struct Depth<128> { static constexpr int S = kBK == 32 ? 4 : 2; };

template <int T>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream) {
    constexpr int S = Depth<T>::S;
    const dim3 grid((unsigned)a.total_blocks), block(256);
    switch (a.phase) {
        case kGram: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kGram, S>), grid, block, 0, stream, a); break;
        case kSquare: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kSquare, S>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kBX, S>), grid, block, 0, stream, a); break;
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

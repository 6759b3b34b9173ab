// The Newton-Schulz products on bf16 MFMA (gfx950), one grouped launch per
// phase over every bucket of the batch:
//   Gram    A  = s X X^T           upper-triangle tiles only, mirrored store
//   square  B' = a I + b A + c A A^T   (A A = A A^T: A is symmetric) upper tiles only
//   BX      X' = s B' X            into the other X copy; in the last
//                                  iteration (FUSED instance) the epilogue
//                                  writes the parameter update W' instead
//   prod    C  = P Q               P, Q symmetric and commuting (the Gram-space
//                                  recurrence's products), upper tiles only
// X' = a X + B X is computed as (a I + B) X: the a X term rides on B's
// diagonal, so the B X epilogue never reads X back.
// s is 1 / (||U||_F + eps) in the first iteration (s^2 for the Gram) and 1
// afterwards.  Each product is computed as C[i][j] = sum_k P[i][k] Q[j][k]:
// for the Gram and square P = Q = X or A, whose rows are K-contiguous (for the
// prod two distinct symmetric m x m matrices, rows again K-contiguous); for B X
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
// Each launch is persistent: one workgroup per CU (two for T = 128) takes
// tiles from its XCD's queue until none is left, and the next tile's first
// slab loads while the current tile's output is written (see the kernel).
//
// Tile: T x T outputs per workgroup (T = 256 or 128).  T = 256: 8 waves in a
// 2 x 4 grid, two per SIMD, each 128 x 64 outputs as 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 (128 accumulator registers, so two waves fit a
// SIMD and one wave's fragment reads and loads overlap the other's MFMAs).
// T = 128: 4 waves in a 2 x 2 grid, each 64 x 64.  Every output element is
// accumulated by one wave in the same k order either way.  K is staged
// through LDS in 64-deep slabs by direct global->LDS loads, the P operand in
// two buffers and the Q operand in three: while slab s is multiplied, P of
// slab s + 1 and Q of slab s + 2 load (the five buffers take the CU's whole
// 160 KB for T = 256).  16-byte chunks are XOR-swizzled by row so that the
// fragment reads hit distinct banks.  Each MFMA k-step is its own scheduling
// region: its MFMAs interleaved with the next k-step's fragment reads and
// with half of one operand's later slab.  Every epilogue stages the output
// tile through LDS, so that global reads and writes are whole 16-byte chunks
// of rows.
#include "kcommon.h"
#include "launch.h"
#include "tile_map.h"

#include <cmath>


namespace dmuon {
namespace {

typedef __attribute__((address_space(3))) void* lptr_t;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kBK = 64;                     // K slab
constexpr int kRowBytes = kBK * 2;          // one LDS row of a K-contiguous slab
constexpr int kChunks = kRowBytes / 16;     // 16-byte chunks per such row
constexpr int kDmaRows = 1024 / kRowBytes;  // rows one 1 KB wave load fills
constexpr int KS = kBK / 16;                // MFMA k-steps per slab

// T = 256: 8 waves in a 2 x 4 grid, each 128 x 64 outputs, two waves per
// SIMD; T = 128: 4 waves in a 2 x 2 grid, each 64 x 64.
template <int T>
struct TileCfg {
    static constexpr int NW = T == 256 ? 8 : 4;    // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int WC = NW / 2;              // waves across the tile's columns (2 down its rows)
    static constexpr int RW = T / 2, CW = T / WC;  // rows, columns of one wave's sub-tile
    static constexpr int FI = RW / 32, FJ = CW / 32;  // MFMA blocks per wave per dim
    static constexpr int kOperandBytes = T * kRowBytes;
    static constexpr int kStageBytes = 2 * kOperandBytes;
    // B X: the P slab is kBK rows (k) of T long-side values
    static constexpr int kPRowBytes = 2 * T;
    static constexpr int kPChunks = kPRowBytes / 16;
    static constexpr int kPDmaRows = 1024 / kPRowBytes;
    // epilogue tile: T rows of T bf16, staged through two operand buffers in kEHalves pieces
    static constexpr int kERowBytes = 2 * T;
    static constexpr int kEChunks = T / 8;
    static constexpr int kEHalves = T * kERowBytes / kStageBytes;
};

// Wait until at most N of the wave's vector-memory loads are in flight (loads
// complete in issue order).  The compiler does not count direct-to-LDS loads
// in the waits it places before barriers, so every such wait is explicit.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One wave-wide direct load: 64 lanes x 16 bytes from global memory into the
// 1 KB of LDS at byte offset lds (wave-uniform), lane l's bytes landing at
// lds + 16 l.  Written as inline assembly so that the compiler, which cannot
// tell the slab buffers apart, does not make every later LDS read wait for
// it: the kernel orders these loads itself, with explicit waits and barriers.
// Every direct load of the kernel goes through here, so the compiler never
// holds a value of its own in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "m0", "memory");
}
// The same with a wave-uniform base address and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
                 : "m0", "memory");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(lptr_t)p;
}

// K-contiguous slab rows: logical chunk ch of row r sits at ch ^ swizzle(r), so
// the fragment reads of 8 (or 16) consecutive rows at one logical chunk hit
// distinct bank groups whether the LDS serves 128 or 256 bytes a clock.
__device__ __forceinline__ int swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// B X P slab (rows k, long-side columns): a transposing read takes 4 rows of
// one 16-lane group; rows r..r+3 get chunk offsets 0, 4, 10, 14 so that the
// 8 chunks of a group (and the 16 of two groups) fall in distinct bank groups.
__device__ __forceinline__ int swizzle_p(int r) { return (0xEA40 >> ((r & 3) * 4)) & 15; }

// Epilogue tile: one chunk swizzle per row, over the row's T / 8 chunks.
template <int T>
__device__ __forceinline__ int swizzle_e(int r) { return r & (T / 8 - 1); }

// A tile of a launch: segment, matrix slot and output tile (I, J).
struct TileInfo {
    int s, slot, I, J;
};

// Where a tile's slabs come from: wave-uniform bases and strides (every side
// is below 2^27 elements, so strides and K fit 32 bits), and each lane's
// 32-bit offsets (two, by load parity).
struct LoadPlan {
    const char* p_base;
    const char* q_base;
    int32_t p_k, p_q, q_q, k_rot, K;
    uint32_t voff_p[2], voff_q[2];
};

// Persistent: each workgroup computes tiles until its XCD's queue is empty.
// The launch's tiles are dealt to the XCDs exactly as a grid of one
// workgroup per tile would deal them (xcd_map of block ids x, x + 8, x + 16,
// ... to XCD x; the hardware places block b on XCD b % 8).  The k-th
// workgroup of XCD x starts with that XCD's k-th tile and then takes the next
// untaken one, counted by the XCD's counter (so tiles of one XCD run in
// their dealt order, longest segments first).  Consecutive tiles of a
// workgroup overlap: the last two slabs of a tile load the next tile's first
// P slab and first two Q slabs, and the epilogue stages the output through
// the buffers of the tile's last slab, so the next tile's loads are in flight
// while the output is written.  Every output element is still accumulated by
// one wave in one k order, so results do not depend on which workgroup takes
// which tile.  FUSED selects the square's variant with b A folded into its
// accumulators, and B X's variant whose epilogue can write parameter updates
// (the last iteration's launch); the other phases ignore it.
template <int T, int PHASE, bool FUSED>
__global__ __launch_bounds__(TileCfg<T>::NT, 1) void ns_gemm_bf16_kernel(GemmArgs args) {
    using C = TileCfg<T>;
    // P buffers 0, 1, then Q buffers 0, 1, 2, kOperandBytes each
    __shared__ __attribute__((aligned(1024))) char smem[5 * C::kOperandBytes];
    static_assert(C::kEHalves * C::kStageBytes == T * C::kERowBytes, "epilogue pieces fill two buffers each");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    // wave w runs on SIMD w % 4; with wr = w % 2, wc = w / 2 the waves holding
    // one half of the tile's columns (the epilogue's pieces) sit on all four
    const int wr = wave % 2, wc = wave / 2;

    // ---- this workgroup's queue ------------------------------------------------------
    const int x = (int)(blockIdx.x % kXcds);
    const int wgs_x = ((int)gridDim.x - x + kXcds - 1) / kXcds;  // workgroups on XCD x
    const int total = args.total_blocks;
    const int count_x = total > x ? (total - x + kXcds - 1) / kXcds : 0;  // tiles dealt to XCD x

    auto decode = [&](int kq, TileInfo& ti) {
        int local;
        xcd_map(x + kXcds * kq, args.nseg, [&](int i) { return args.seg[i].count * args.seg[i].tiles_per_mat; },
                [&](int i) { return args.seg[i].first_block; }, [&](int i) { return args.seg[i].xcd_remap != 0; },
                ti.s, local);
        const GemmSeg& sg = args.seg[ti.s];
        ti.slot = local / sg.tiles_per_mat;
        const int t = local - ti.slot * sg.tiles_per_mat;
        if (PHASE == kBX)
            bx_decode_banded(t, sg.tn, sg.tm, ti.I, ti.J);  // I: long-side tile, J: short-side tile
        else
            tri_decode_banded(t, sg.tm, ti.I, ti.J);
    };
    // The P operand (B X: X, read k-major) of a tile's matrix, and the leading
    // dimension of the K-contiguous rows (Q's, and P's outside B X): the K extent.
    auto operand_p = [&](const TileInfo& ti) -> const uint16_t* {
        const GemmSeg& sg = args.seg[ti.s];
        return reinterpret_cast<const uint16_t*>(
            args.ws + sg.p_off + ti.slot * (PHASE == kBX || PHASE == kGram ? sg.x_stride : sg.a_stride));
    };
    auto k_extent = [&](const TileInfo& ti) -> int32_t {
        const GemmSeg& sg = args.seg[ti.s];
        return (int32_t)(PHASE == kGram ? sg.n_pad : sg.m_pad);
    };

    // ---- global -> LDS (direct) ------------------------------------------------------
    // One global_load_lds_dwordx4 of a wave fills 1 KB of LDS: lane l writes
    // bytes 16 l .. 16 l + 15 of it, so it fetches the global chunk that the
    // swizzle places there.  Load q (= wave kDmaPerOp + i) of an operand slab
    // covers rows R q .. R q + R - 1 of it (R = 1 KB / row bytes), lane l row
    // R q + l / (chunks per row); the address splits into a wave-uniform part
    // (slab, q) and a per-lane part that depends on q only through the
    // swizzle, i.e. through q's parity (kDmaPerOp is even).
    //   K-contiguous rows (Gram, square P; every Q): R = 8, chunk swizzle
    //   (l / 8) ^ (q & 1).
    //   B X P slab (rows k of X): R = 2 (T = 256) or 4, chunk swizzle
    //   swizzle_p of the row, whose two low bits hold 2 (q & 1) + l / 32 or l / 16.
    // Waves that issue the slab loads.  In B X, waves 0 .. 3 (one of each pair
    // sharing a SIMD) issue all of them, so the MFMAs of waves 4 .. 7 never
    // wait behind loads of their own (B X 1% faster, same box; the other
    // phases measured 0.6-5.5% slower that way); elsewhere every wave loads.
    constexpr int kLoaders = PHASE == kBX && C::NW == 8 ? 4 : C::NW;
    constexpr int kDmaPerOp = T * kRowBytes / 1024 / kLoaders;  // 1 KB loads per loader wave per operand per slab
    static_assert(kDmaPerOp % 2 == 0, "load parity");
    auto plan_loads = [&](const TileInfo& ti, LoadPlan& lp) {
        const GemmSeg& sg = args.seg[ti.s];
        const int32_t ldq = k_extent(ti);
        const int32_t p_row_ld = PHASE == kBX ? (int32_t)sg.n_pad : ldq;  // P slab row stride (elements)
        const uint16_t* P = operand_p(ti);
        const uint16_t* Q = PHASE == kBX || PHASE == kProd
                                ? reinterpret_cast<const uint16_t*>(args.ws + sg.q_off + ti.slot * sg.a_stride)
                                : P;
        #pragma unroll
        for (int par = 0; par < 2; ++par) {
            if (PHASE == kBX) {
                const int row = C::kPDmaRows * par + lane / C::kPChunks;
                const int lc = (lane % C::kPChunks) ^ swizzle_p(row);
                lp.voff_p[par] = (uint32_t)(2 * ((lane / C::kPChunks) * p_row_ld + lc * 8));
            } else {
                const int lc = (lane % kChunks) ^ swizzle(kDmaRows * par + lane / kChunks);
                lp.voff_p[par] = (uint32_t)(2 * ((lane / kChunks) * p_row_ld + lc * 8));
            }
            const int lc = (lane % kChunks) ^ swizzle(kDmaRows * par + lane / kChunks);
            lp.voff_q[par] = (uint32_t)(2 * ((lane / kChunks) * ldq + lc * 8));
        }
        // wave-uniform byte addresses: P slab at k0 = p_base + k0 p_k + q p_q
        lp.p_base = reinterpret_cast<const char*>(P) +
                    (PHASE == kBX ? 2 * (int64_t)ti.I * T : 2 * (int64_t)ti.I * T * ldq);
        lp.q_base = reinterpret_cast<const char*>(Q + (int64_t)ti.J * T * ldq);
        lp.p_k = PHASE == kBX ? 2 * (int32_t)sg.n_pad : 2;
        lp.p_q = PHASE == kBX ? 2 * C::kPDmaRows * (int32_t)sg.n_pad : 16 * ldq;
        lp.q_q = 16 * ldq;
        lp.K = ldq;
        // The square's K loop starts right after block I of k (A columns I T ..),
        // so that the tile's last T / kBK slabs are that block: the folded b A
        // term reads it there (and the read-back path finds it in L2).  K is a
        // multiple of T.
        lp.k_rot = 0;
        if (PHASE == kSquare) {
            lp.k_rot = (ti.I + 1) * T;
            if (lp.k_rot >= lp.K) lp.k_rot -= lp.K;
        }
    };
    // Loads i0 .. i1-1 (of kDmaPerOp) of the P or Q slab at loop position k0
    // of the tile lp describes into the buffer at dst.
    auto rot = [&](const LoadPlan& lp, int32_t k0) {
        k0 += lp.k_rot;
        return k0 >= lp.K ? k0 - lp.K : k0;
    };
    auto dma_p = [&](const LoadPlan& lp, int32_t k0, char* dst, int i0, int i1) {
        if (kLoaders < C::NW && wave >= kLoaders) return;
        const char* base = lp.p_base + (int64_t)rot(lp, k0) * lp.p_k;
        #pragma unroll
        for (int i = i0; i < i1; ++i) {
            const int q = wave * kDmaPerOp + i;  // 1 KB block of the operand slab
            dma16(base + (int64_t)q * lp.p_q, lp.voff_p[i & 1], lds_offset(dst + q * 1024));
        }
    };
    auto dma_q = [&](const LoadPlan& lp, int32_t k0, char* dst, int i0, int i1) {
        if (kLoaders < C::NW && wave >= kLoaders) return;
        const char* base = lp.q_base + 2 * (int64_t)rot(lp, k0);
        #pragma unroll
        for (int i = i0; i < i1; ++i) {
            const int q = wave * kDmaPerOp + i;
            dma16(base + (int64_t)q * lp.q_q, lp.voff_q[i & 1], lds_offset(dst + q * 1024));
        }
    };
    // A slab's loads go out in halves, one per scheduling region (P's in the
    // region after the barrier and in k-step 0, Q's in k-steps 1 and 2), so the
    // address unit never takes a whole slab's loads at once while the matrix
    // pipe waits behind them.
    constexpr int kHalf = kDmaPerOp / 2;

    floatx16 acc[C::FI][C::FJ];
    const int lrow = lane & 31, khalf = lane >> 5;
    // The square's b A term, folded into the accumulators: B' = c (A A^T +
    // (b / c) A) + a I.  K is rotated so that the tile's last T / kBK slabs are
    // block I of k, where Q's fragments are A[J T + c][I T + k'] = A[I T + k'][J T + c]
    // (A is symmetric); one more MFMA per fragment against (b / c) times the
    // identity (rows k' of the tile) adds (b / c) A[I T + r][J T + c] to
    // acc[r][c].  b / c goes in as two bf16 parts, so it keeps about 16 bits.
    // FUSED (the launch takes it when c != 0 and |b / c| <= 64; the quintic's
    // b / c is -2.35): for other coefficients the epilogue reads A's block back
    // instead, in a kernel of its own.
    constexpr bool sq_fold = PHASE == kSquare && FUSED;
    const float sq_bc = sq_fold ? args.b / args.c : 0.f;
    const __bf16 sq_hi = (__bf16)sq_bc;
    const __bf16 sq_lo = (__bf16)(sq_bc - (float)sq_hi);
    const int swz = swizzle(lrow);  // fragment rows start at multiples of 32
    const int a_row0 = (wr * C::RW + lrow) * kRowBytes;
    const int b_row0 = (wc * C::CW + lrow) * kRowBytes;
    // B X transposing read: lane 16 g + s of a 16-lane group g addresses row
    // (s / 4) and columns 4 (s % 4) .. + 3 of a 4 x 16 block; it receives that
    // block's column s, i.e. 4 consecutive k of output row jbase + s.
    const int tr_g = lane >> 4, tr_s = lane & 15;
    const int tr_row = 8 * (tr_g >> 1) + (tr_s >> 2);                 // + 16 ks + 4 half
    const int tr_col = wr * C::RW + 16 * (tr_g & 1) + 4 * (tr_s & 3);  // + 32 fi
    const int tr_sw = swizzle_p(tr_s >> 2);                           // rows are 4-aligned
    bf16x8 fa[2][C::FI], fb[2][C::FJ];

#define DMUON_READ_A(BUF, BASE, KS_)                                                              \
    do {                                                                                          \
        if (PHASE == kBX) {                                                                       \
            _Pragma("unroll") for (int i_ = 0; i_ < C::FI; ++i_) {                                \
                shortx4 h_[2];                                                                    \
                _Pragma("unroll") for (int t_ = 0; t_ < 2; ++t_) {                                \
                    const int r_ = 16 * (KS_) + 4 * t_ + tr_row;                                  \
                    const int c_ = tr_col + 32 * i_;                                              \
                    const int o_ = r_ * C::kPRowBytes + (((c_ >> 3) ^ tr_sw) << 4) + (c_ & 7) * 2; \
                    h_[t_] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                             \
                        (lds_shortx4*)((__attribute__((address_space(3))) char*)(BASE) + o_));    \
                }                                                                                 \
                const shortx8 w_ = __builtin_shufflevector(h_[0], h_[1], 0, 1, 2, 3, 4, 5, 6, 7); \
                fa[BUF][i_] = __builtin_bit_cast(bf16x8, w_);                                     \
            }                                                                                     \
        } else {                                                                                  \
            const int pc_ = ((((KS_) * 2 + khalf) ^ swz) << 4);                                   \
            _Pragma("unroll") for (int i_ = 0; i_ < C::FI; ++i_)                                  \
                fa[BUF][i_] = *reinterpret_cast<const bf16x8*>((BASE) + a_row0 + i_ * 32 * kRowBytes + pc_); \
        }                                                                                         \
    } while (0)
#define DMUON_READ(BUF, PB, QB, KS_)                                                              \
    do {                                                                                          \
        DMUON_READ_A(BUF, PB, KS_);                                                               \
        const int pc_ = ((((KS_) * 2 + khalf) ^ swz) << 4);                                       \
        _Pragma("unroll") for (int j_ = 0; j_ < C::FJ; ++j_)                                      \
            fb[BUF][j_] = *reinterpret_cast<const bf16x8*>((QB) + b_row0 + j_ * 32 * kRowBytes + pc_); \
    } while (0)
#define DMUON_MFMA(BUF)                                                                           \
    do {                                                                                          \
        _Pragma("unroll") for (int i_ = 0; i_ < C::FI; ++i_)                                      \
            _Pragma("unroll") for (int j_ = 0; j_ < C::FJ; ++j_)                                  \
                acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[BUF][i_], fb[BUF][j_],   \
                                                                      acc[i_][j_], 0, 0, 0);      \
    } while (0)

    constexpr int NREAD = (PHASE == kBX ? 2 : 1) * C::FI + C::FJ;  // fragment reads per k-step
    constexpr int NMFMA = C::FI * C::FJ;                          // MFMAs per k-step
    // loads per region in the MFMAs' scheduling groups (none where they sit
    // behind the loader waves' branch)
    constexpr int NV = kLoaders == C::NW ? kHalf : 0;
    // One k-step as its own scheduling region: each of the first MFMAs is
    // followed by one fragment read for the next k-step (and, where the region
    // carries a piece of a slab's loads, by one of those), so the reads are in
    // flight while the matrix pipe is busy and have landed before they are used
    // (the MFMA leading the region only waits on reads issued a region earlier).
#define DMUON_INTERLEAVE(NV)                                                                      \
    do {                                                                                          \
        _Pragma("unroll") for (int g_ = 0; g_ < NMFMA; ++g_) {                                    \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */                         \
            if (g_ < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* DS read */      \
            if (g_ < (NV)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  /* VMEM */         \
        }                                                                                         \
        if (NREAD > NMFMA) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NMFMA, 0);         \
        if ((NV) > NMFMA) __builtin_amdgcn_sched_group_barrier(0x010, (NV) - NMFMA, 0);           \
        __builtin_amdgcn_sched_barrier(0);                                                        \
    } while (0)
    // The folded b A term for k-step KS_ of slab KT_ (Q's fragments in fb[BUF_]):
    // k' = 16 KS_ + (position of the slab in block I) kBK + the lane's 8 k;
    // rows r of the tile with r = k' get (b / c) on the diagonal of the
    // identity fragment, in the 32-row fragment i that holds them.
#define DMUON_SQ_FOLD(KT_, KS_, BUF_)                                                             \
    do {                                                                                          \
        if (sq_fold) {                                                                            \
            const int sp_ = (KT_) - (KT - T / kBK);                                               \
            const int g_ = sp_ * kBK + 16 * (KS_) - wr * C::RW;  /* rows of this k-step, wave-relative */ \
            if (sp_ >= 0 && g_ >= 0 && g_ < C::RW) {                                              \
                const int i0_ = g_ >> 5;                                                          \
                const int d_ = lrow + 32 * i0_ - g_ - 8 * khalf;                                  \
                bf16x8 hi_, lo_;                                                                  \
                _Pragma("unroll") for (int e_ = 0; e_ < 8; ++e_) {                                \
                    hi_[e_] = d_ == e_ ? sq_hi : (__bf16)0.f;                                     \
                    lo_[e_] = d_ == e_ ? sq_lo : (__bf16)0.f;                                     \
                }                                                                                 \
                _Pragma("unroll") for (int i_ = 0; i_ < C::FI; ++i_) {                            \
                    if (i_ == i0_) {                                                              \
                        _Pragma("unroll") for (int j_ = 0; j_ < C::FJ; ++j_) {                    \
                            acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi_, fb[BUF_][j_], acc[i_][j_], 0, 0, 0); \
                            acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo_, fb[BUF_][j_], acc[i_][j_], 0, 0, 0); \
                        }                                                                         \
                    }                                                                             \
                }                                                                                 \
            }                                                                                     \
        }                                                                                         \
    } while (0)
    // k-step KS_ (0 .. KS - 2) of the slab in buffers PB_, QB_: the MFMAs of
    // k-step KS_, the fragment reads of k-step KS_ + 1 and the loads LD_.
#define DMUON_KSTEP(KS_, PB_, QB_, LD_)                                                           \
    do {                                                                                          \
        LD_;                                                                                      \
        DMUON_READ(((KS_) + 1) & 1, PB_, QB_, (KS_) + 1);                                         \
        DMUON_MFMA((KS_) & 1);                                                                    \
        DMUON_INTERLEAVE(NV);                                                                     \
    } while (0)

    // ---- epilogue ---------------------------------------------------------------------
    // acc[i][j][v] holds output row  wr*RW + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4
    //                  and column  wc*CW + 32 j + lane % 32   of the T x T tile,
    // i.e. four consecutive rows r0 .. r0 + 3 of one column c per (i, j, v / 4).
    // The tile goes through LDS transposed, as E[c][r] = C[r][c]: each lane's
    // four values are one 8-byte piece of a row of E.  E is staged through the
    // last slab's two buffers in kEHalves pieces of kERows rows (columns c)
    // each, the waves holding a piece's columns writing it.
    constexpr int kERows = T / C::kEHalves;
    const int my_piece = (wc * C::CW) / kERows;
    // E lives in two buffers of kOperandBytes (the P and Q buffers of the
    // tile's last slab): rows 0 .. kERegRows - 1 in the first, the rest in the
    // second.
    constexpr int kERegRows = C::kOperandBytes / C::kERowBytes;
    static_assert(2 * kERegRows == kERows, "a piece of E fills the two buffers");
    struct EBuf {
        char* a;
        char* b;
    };
    auto erow = [&](const EBuf& E, int c) -> char* {
        return (c < kERegRows ? E.a : E.b) + (c & (kERegRows - 1)) * C::kERowBytes;
    };
    // kERows rows of 2 T bytes from global (row stride ld elements) into E, whole.
    auto load_piece = [&](int eln, const EBuf& ebuf, const uint16_t* src, int64_t ld) {
        constexpr int kLoads = kERows * C::kERowBytes / 1024 / C::NW;  // 1 KB loads per wave
        #pragma unroll 8
        for (int i = 0; i < kLoads; ++i) {
            const int q = wave * kLoads + i;
            const int row = (1024 / C::kERowBytes) * q + eln / C::kEChunks;
            const int lc = (eln % C::kEChunks) ^ swizzle_e<T>(row);
            // the 1 KB block q holds whole E rows, all in one of E's two buffers
            dma16(src + row * ld + lc * 8, lds_offset(erow(ebuf, (1024 / C::kERowBytes) * q)));
        }
        wait_vm<0>();
        __syncthreads();
    };
    // E row c, columns r .. r + 3 (r a multiple of 4)
    auto e_ptr = [&](const EBuf& ebuf, int c, int r) -> char* {
        return erow(ebuf, c) + (((r >> 3) ^ swizzle_e<T>(c)) << 4) + (r & 7) * 2;
    };
    // E rows to global rows (row stride ld elements), whole 16-byte chunks.
    auto store_rows = [&](int etid, const EBuf& ebuf, uint16_t* dst, int64_t ld) {
        constexpr int kStores = kERows * C::kEChunks / C::NT;
        #pragma unroll 8
        for (int i = 0; i < kStores; ++i) {
            const int q = etid + C::NT * i;
            const int row = q / C::kEChunks, lc = q % C::kEChunks;
            const uint4 v = *reinterpret_cast<const uint4*>(erow(ebuf, row) + ((lc ^ swizzle_e<T>(row)) << 4));
            *reinterpret_cast<uint4*>(dst + row * ld + lc * 8) = v;
        }
    };
    // E columns to global rows: global row r gets E[c .. c + 7][r].  A
    // transposing read of a 16-lane group takes rows c0 .. c0 + 3 of E at
    // columns r0 .. r0 + 15 (source lane 4 k + q addresses row c0 + k, columns
    // r0 + 4 q .. + 3) and hands lane i the four values E[c0 .. c0 + 3][r0 + i];
    // two such reads give a lane 8 consecutive c of one r.  A wave covers 16
    // rows r and 32 columns c per store, the 4 groups taking 8 columns each.
    auto store_cols = [&](int eln, const EBuf& ebuf, uint16_t* dst, int64_t ld) {
        const int g = eln >> 4, i16 = eln & 15, k = i16 >> 2, q = i16 & 3;
        constexpr int kRowBlocks = T / 16, kColBlocks = kERows / 32;
        #pragma unroll 4
        for (int it = 0; it < kRowBlocks * kColBlocks / C::NW; ++it) {
            const int w = C::NW * it + wave;
            const int r0 = (w % kRowBlocks) * 16, cb = (w / kRowBlocks) * 32 + 8 * g;
            shortx4 h[2];
            #pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_shortx4*)((__attribute__((address_space(3))) char*)e_ptr(ebuf, cb + 4 * hh + k, r0 + 4 * q)));
            const shortx8 v = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
            *reinterpret_cast<shortx8*>(dst + (int64_t)(r0 + i16) * ld + cb) = v;
        }
    };
    // The parameter update written by the last B X launch (FUSED), for a bf16
    // parameter: per element W' = keep W + coef O (or, for the output of an
    // orthogonalisation, W' = O), O being the bf16 value X' would get and
    // keep, coef the apply pass's own factors, so the result is the apply
    // pass's bit for bit.  Waves 0 .. 3 (kUpdWaves) do the update: they hold
    // the accumulators of piece 0 of E, and load parameter chunks into
    // registers only once those are staged, so the accumulators of piece 1
    // (waves 4 .. 7) and the parameter chunks are never live together.
    //   piece 0: waves 0 .. 3 stage it; barrier; they load W's chunks of piece
    //            0, update and store them, then load those of piece 1
    //   piece 1: barrier (E free); waves 4 .. 7 stage it; barrier; waves 0 .. 3
    //            update and store it
    // (T = 128: one piece, all four waves.)  Each worker lane takes kUpd
    // 16-byte chunks (8 bf16) of a piece: along parameter rows for a wide or
    // square matrix (W[c][r]: E's rows, as store_rows), along E's columns for a
    // tall one (W[r][c]: through the transposing read, as store_cols).
    constexpr int kUpdWaves = 4;
    static_assert(C::kEHalves == 1 ? C::NW == kUpdWaves : (C::kEHalves == 2 && C::NW == 2 * kUpdWaves),
                  "the update waves hold piece 0");
    constexpr int kUpd = kERows * C::kEChunks / (64 * kUpdWaves);
    static_assert((T / 16) * (kERows / 32) / kUpdWaves == kUpd, "both layouts take kUpd chunks a lane");
    auto update_epilogue = [&](const TileInfo& ti, const EBuf& ebuf, const auto* rec, auto&& stage, int etid) {
        const int64_t rows = rec->rows, cols = rec->cols;
        const bool tall = rec->transposed != 0;
        uint16_t* const W = static_cast<uint16_t*>(rec->dst);  // bf16 (fused records only)
        const float coef = -args.lr * rec->upd_scale;
        const float keep = 1.0f - args.lr * args.wd;
        const int ut = etid & (64 * kUpdWaves - 1);  // lane among the update waves
        const int g = (ut & 63) >> 4, i16 = ut & 15, k4 = i16 >> 2, q4 = i16 & 3, uw = ut >> 6;
        constexpr int kRowBlocks = T / 16;
        // chunk u of piece h: the parameter row and column it covers (cols a
        // multiple of 8: a chunk is inside the matrix or wholly outside),
        // and where its O values sit in E
        auto chunk = [&](int h, int u, int64_t& prow, int64_t& pcol, int& erow_, int& ecol) {
            const int c0 = ti.J * T + h * kERows, r0 = ti.I * T;
            if (!tall) {  // W[c][r]: E row = c, chunk along r
                const int qq = ut + 64 * kUpdWaves * u;
                erow_ = qq / C::kEChunks;
                ecol = 8 * (qq % C::kEChunks);
                prow = c0 + erow_;
                pcol = r0 + ecol;
            } else {  // W[r][c]: 8 consecutive c of one r
                const int wv = kUpdWaves * u + uw;
                const int rr = (wv % kRowBlocks) * 16, cb = (wv / kRowBlocks) * 32 + 8 * g;
                erow_ = cb;
                ecol = rr;
                prow = r0 + rr + i16;
                pcol = c0 + cb;
            }
        };
        auto inside = [&](int64_t prow, int64_t pcol) { return prow < rows && pcol < cols; };
        // The W loads are unconditional (a chunk outside the matrix reads the
        // first one and is never stored) and each w[u] is marked used on every
        // path where the update consumes it: a load left pending on some path
        // of the tile loop made the compiler wait for all memory traffic
        // before every later load into the same registers, so the 16 loads of
        // a piece went out one round trip at a time.
        u32x4_t w[kUpd];
        auto load_w = [&](int h) {
            if (!args.update) return;
            #pragma unroll
            for (int u = 0; u < kUpd; ++u) {
                int64_t prow, pcol;
                int er, ec;
                chunk(h, u, prow, pcol, er, ec);
                w[u] = ld_stream<u32x4_t>(W + (inside(prow, pcol) ? prow * cols + pcol : 0));
            }
        };
        auto update = [&](int h) {
            #pragma unroll
            for (int u = 0; u < kUpd; ++u) {
                int64_t prow, pcol;
                int er, ec;
                chunk(h, u, prow, pcol, er, ec);
                if (args.update) asm volatile("" : "+v"(w[u]));
                u32x4_t o;
                if (!tall) {
                    o = *reinterpret_cast<const u32x4_t*>(erow(ebuf, er) + (((ec >> 3) ^ swizzle_e<T>(er)) << 4));
                } else {
                    // every lane takes part in the transposing reads: the empty
                    // asm keeps them out of the branch below
                    shortx4 hv[2];
                    #pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_shortx4*)((__attribute__((address_space(3))) char*)e_ptr(ebuf, er + 4 * hh + k4, ec + 4 * q4)));
                    o = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
                    asm volatile("" : "+v"(o));
                }
                if (inside(prow, pcol)) {
                    if (args.update) {
                        #pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t ov = o[e], wv = w[u][e];
                            const float lo = fmaf(coef, __uint_as_float(ov << 16), keep * __uint_as_float(wv << 16));
                            const float hi = fmaf(coef, __uint_as_float(ov & 0xffff0000u),
                                                  keep * __uint_as_float(wv & 0xffff0000u));
                            o[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                        }
                    }
                    st_stream<u32x4_t>(W + prow * cols + pcol, o);
                }
            }
        };
        if constexpr (C::kEHalves == 1) {
            stage(0);
            __syncthreads();
            load_w(0);
            update(0);
        } else {
            if (my_piece == 0) stage(0);
            __syncthreads();
            if (wave < kUpdWaves) {
                load_w(0);
                update(0);
                load_w(1);
            }
            __syncthreads();  // E is free again
            if (my_piece == 1) stage(1);
            __syncthreads();
            if (wave < kUpdWaves) update(1);
        }
    };
    auto epilogue = [&](const TileInfo& ti, const EBuf& ebuf) {
        // Lane indices passed through an empty asm statement: the epilogue's
        // per-lane addresses are then computed here, once per tile, rather
        // than hoisted out of the tile loop into registers the main loop needs.
        int etid = tid;
        asm volatile("" : "+v"(etid));
        const int eln = etid & 63, elrow = eln & 31, ekhalf = eln >> 5;
        // likewise the segment's fields: loaded here, not kept through the main loop
        int es = ti.s;
        asm volatile("" : "+s"(es));
        const GemmSeg& sg = args.seg[es];
        const int plan_idx = sg.plan_base + ti.slot;
        // a scalar load: a vector load here would make the compiler wait for
        // every load in flight, the next tile's slab included
        typedef const __attribute__((address_space(4))) float cfloat_t;
        const float first_scale = sg.first_iter ? *(cfloat_t*)(uintptr_t)(args.scale + plan_idx) : 1.0f;
        if (PHASE == kBX) {
            // Tile rows are long-side indices r, columns short-side indices c:
            // X'[c][r] = s acc[r][c]; E is the X' tile (T rows c, T columns r).
            const int64_t ldn = sg.n_pad;
            uint16_t* Xd = reinterpret_cast<uint16_t*>(args.ws + sg.o_off + ti.slot * sg.x_stride) +
                           (int64_t)ti.J * T * ldn + (int64_t)ti.I * T;
            bool fused = false;
            if constexpr (FUSED) {
                // the last segment's closing product of a matrix whose record
                // says fused: the epilogue writes its update instead of X'
                typedef const __attribute__((address_space(4))) DevMatRec crec_t;
                const crec_t* rec = reinterpret_cast<const crec_t*>(reinterpret_cast<uintptr_t>(args.recs + plan_idx));
                fused = sg.fuse != 0 && rec->fused != 0;
                // piece h of E from the accumulators of the waves holding its columns
                auto stage = [&](int h) {
                    #pragma unroll
                    for (int i = 0; i < C::FI; ++i)
                        #pragma unroll
                        for (int j = 0; j < C::FJ; ++j)
                            #pragma unroll
                            for (int v4 = 0; v4 < 4; ++v4) {
                                const int r0 = wr * C::RW + i * 32 + 8 * v4 + 4 * ekhalf;
                                const int c = wc * C::CW + j * 32 + elrow - h * kERows;
                                uint2 o;
                                o.x = (uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 0]) |
                                      ((uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 1]) << 16);
                                o.y = (uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 2]) |
                                      ((uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 3]) << 16);
                                *reinterpret_cast<uint2*>(e_ptr(ebuf, c, r0)) = o;
                            }
                };
                if (fused) update_epilogue(ti, ebuf, rec, stage, etid);
            }
            if (!fused) {
                // (the same staging as the fused path's, written out: the
                // lambda here changes this kernel's register allocation)
                #pragma unroll
                for (int h = 0; h < C::kEHalves; ++h) {
                    if (my_piece == h) {
                        #pragma unroll
                        for (int i = 0; i < C::FI; ++i)
                            #pragma unroll
                            for (int j = 0; j < C::FJ; ++j)
                                #pragma unroll
                                for (int v4 = 0; v4 < 4; ++v4) {
                                    const int r0 = wr * C::RW + i * 32 + 8 * v4 + 4 * ekhalf;
                                    const int c = wc * C::CW + j * 32 + elrow - h * kERows;
                                    uint2 o;
                                    o.x = (uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 0]) |
                                          ((uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 1]) << 16);
                                    o.y = (uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 2]) |
                                          ((uint32_t)f32_to_bf16(first_scale * acc[i][j][4 * v4 + 3]) << 16);
                                    *reinterpret_cast<uint2*>(e_ptr(ebuf, c, r0)) = o;
                                }
                    }
                    __syncthreads();
                    store_rows(etid, ebuf, Xd + (int64_t)h * kERows * ldn, ldn);
                    if (h + 1 < C::kEHalves) __syncthreads();  // before the next piece overwrites E
                }
            }
        } else {
            // Out[I T + r][J T + c] = C[r][c] = E[c][r] and, off the diagonal, the
            // mirror Out[J T + c][I T + r] = E[c][r].  E's rows are rows of block
            // (J, I); on the diagonal that block is the tile itself (symmetric).
            // The square's b A term reads A's block (J, I) = block (I, J)^T into E
            // first (A is symmetric and stored whole).
            const int64_t ld = sg.m_pad;
            uint16_t* Out = reinterpret_cast<uint16_t*>(args.ws + sg.o_off + ti.slot * sg.a_stride);
            const float alpha = PHASE == kGram ? first_scale * first_scale : PHASE == kSquare ? args.c : 1.0f;
            const float beta = args.b;
            #pragma unroll
            for (int h = 0; h < C::kEHalves; ++h) {
                if (PHASE == kSquare && !sq_fold)
                    load_piece(eln, ebuf,
                               reinterpret_cast<const uint16_t*>(args.ws + sg.p_off + ti.slot * sg.a_stride) +
                                   ((int64_t)ti.J * T + h * kERows) * ld + (int64_t)ti.I * T,
                               ld);
                if (my_piece == h) {
                    #pragma unroll
                    for (int i = 0; i < C::FI; ++i)
                        #pragma unroll
                        for (int j = 0; j < C::FJ; ++j)
                            #pragma unroll
                            for (int v4 = 0; v4 < 4; ++v4) {
                                const int r0 = wr * C::RW + i * 32 + 8 * v4 + 4 * ekhalf;
                                const int cg = wc * C::CW + j * 32 + elrow;  // column in the tile
                                char* p = e_ptr(ebuf, cg - h * kERows, r0);
                                float v[4];
                                #pragma unroll
                                for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][4 * v4 + e];
                                if (PHASE == kSquare) {
                                    if (!sq_fold) {
                                        const uint2 xa = *reinterpret_cast<const uint2*>(p);
                                        v[0] = fmaf(beta, __uint_as_float(xa.x << 16), v[0]);
                                        v[1] = fmaf(beta, __uint_as_float(xa.x & 0xffff0000u), v[1]);
                                        v[2] = fmaf(beta, __uint_as_float(xa.y << 16), v[2]);
                                        v[3] = fmaf(beta, __uint_as_float(xa.y & 0xffff0000u), v[3]);
                                    }
                                    if (ti.I == ti.J) {  // the a I term on the diagonal
                                        #pragma unroll
                                        for (int e = 0; e < 4; ++e)
                                            if (r0 + e == cg) v[e] += args.a;
                                    }
                                }
                                uint2 o;
                                o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                                o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                                *reinterpret_cast<uint2*>(p) = o;
                            }
                }
                __syncthreads();
                store_rows(etid, ebuf, Out + ((int64_t)ti.J * T + h * kERows) * ld + (int64_t)ti.I * T, ld);
                if (ti.I != ti.J)
                    store_cols(eln, ebuf, Out + (int64_t)ti.I * T * ld + (int64_t)ti.J * T + h * kERows, ld);
                if (h + 1 < C::kEHalves) __syncthreads();  // before the next piece overwrites E
            }
        }
    };

    // ---- the tiles of this workgroup ------------------------------------------------------
    // Slab g of the workgroup (counted across its tiles) has its P operand in
    // P buffer g % 2 and its Q operand in Q buffer g % 3.  While slab s of a
    // tile is multiplied, its P of slab s + 1 and its Q of slab s + 2 load,
    // into the buffers slabs s - 1 and s - 1 have left: P's halves in the
    // region after the barrier and in k-step 0, Q's in k-steps 1 and 2.  The
    // end of slab s waits for slab s + 1 (P issued in this slab, Q in the one
    // before): loads complete in issue order, so waiting until at most the
    // kDmaPerOp Q loads of slab s + 2 are in flight lands it (stores in between
    // only make such a wait longer), and the barrier after it lands it for the
    // waves that issue no loads.  Past the tile's end these loads are the
    // next tile's: Q of its slab 0 in slab KT - 2, P of slab 0 and Q of slab 1
    // in slab KT - 1.  The next tile is read from the queue at the end of slab
    // KT - 3 (at the tile's start when it has two slabs), through the Q buffer
    // that slab has left and its next tile's Q loads will fill, and its loads
    // are planned in slab KT - 2, after this tile's last P loads.
    auto pbuf = [&](int b) { return smem + b * C::kOperandBytes; };
    auto qbuf = [&](int b) { return smem + (2 + b) * C::kOperandBytes; };
    auto next3 = [](int b) { return b == 2 ? 0 : b + 1; };
    int kq = (int)(blockIdx.x / kXcds);  // this workgroup's first tile of its XCD's queue
    if (kq < count_x) {
        TileInfo cur;
        decode(kq, cur);
        LoadPlan L;
        plan_loads(cur, L);
        int gp = 0, gq = 0;  // the current slab's P and Q buffers
        // prologue: P and Q of slab 0, Q of slab 1; wait for slab 0
        dma_p(L, 0, pbuf(0), 0, kDmaPerOp);
        dma_q(L, 0, qbuf(0), 0, kDmaPerOp);
        dma_q(L, kBK, qbuf(1), 0, kDmaPerOp);
        wait_vm<kDmaPerOp>();
        __syncthreads();
        for (;;) {
            // the queue position of the tile after this one; its value is used
            // only in slab KT - 2 (the compiler waits for it there)
            uint32_t taken = 0;
            if (tid == 0) {
                // the index through a vector register: otherwise the compiler
                // turns the one-lane atomic into a wave-wide one whose result it
                // needs (and waits for, with every load in flight) right away.
                // The pointer itself keeps its global address space: a flat
                // atomic would also hold up every LDS wait until it returns.
                int qx = x;
                asm volatile("" : "+v"(qx));
                taken = atomicAdd(args.queue + qx, 1u);
            }
            #pragma unroll
            for (int i = 0; i < C::FI; ++i)
                #pragma unroll
                for (int j = 0; j < C::FJ; ++j)
                    #pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
            const int KT = (int)(L.K / kBK);  // >= 2: K is a multiple of the tile
            bool has_next = false;
            TileInfo nxt = cur;
            // The next tile, from the queue: every wave passes the atomic's
            // result through the empty asm (so that the compiler's wait for it
            // sits here on every path), thread 0 posts it in the free Q buffer
            // mail, and the buffer takes no loads before every wave has read it.
            auto next_tile = [&](char* mail) {
                asm volatile("" : "+v"(taken));
                if (tid == 0) *reinterpret_cast<int*>(mail) = wgs_x + (int)taken;
                __syncthreads();
                const int kn = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(mail));
                __syncthreads();
                has_next = kn < count_x;
                if (has_next) decode(kn, nxt);
            };
            if (KT == 2) next_tile(qbuf(next3(next3(gq))));
            // region after the barrier of slab 0: half of P of slab 1 (this tile's:
            // K covers at least two slabs), k-step 0 fragments
            __builtin_amdgcn_sched_barrier(0);
            dma_p(L, kBK, pbuf(gp ^ 1), 0, kHalf);
            DMUON_READ(0, pbuf(gp), qbuf(gq), 0);
            DMUON_INTERLEAVE(NV);
            for (int kt = 0;; ++kt) {
                char* const pb = pbuf(gp);
                char* const qb = qbuf(gq);
                // P of slab kt + 1 (the next tile's slab 0 at the tile's last slab)
                const int32_t kp = kt + 1 < KT ? (kt + 1) * kBK : 0;
                DMUON_KSTEP(0, pb, qb, dma_p(L, kp, pbuf(gp ^ 1), kHalf, kDmaPerOp));
                DMUON_SQ_FOLD(kt, 0, 0);
                if (kt + 2 == KT) plan_loads(nxt, L);  // this tile's loads are all issued
                // Q of slab kt + 2 (past the end: the next tile's slab 0 or 1)
                const int32_t kqo = (kt + 2 < KT ? kt + 2 : kt + 2 - KT) * kBK;
                char* const qd = qbuf(next3(next3(gq)));
                DMUON_KSTEP(1, pb, qb, dma_q(L, kqo, qd, 0, kHalf));
                DMUON_SQ_FOLD(kt, 1, 1);
                DMUON_KSTEP(2, pb, qb, dma_q(L, kqo, qd, kHalf, kDmaPerOp));
                DMUON_SQ_FOLD(kt, 2, 0);
                if (kt + 1 == KT) break;
                wait_vm<kDmaPerOp>();  // slab kt + 1 (Q of slab kt + 2 may be in flight)
                __syncthreads();
                if (kt + 3 == KT) next_tile(qb);  // slab kt's Q buffer takes the next tile's slab 0
                gp ^= 1;
                gq = next3(gq);
                // the region after the barrier: half of P of slab kt + 2 (the next
                // tile's slab 0 when kt + 2 is this tile's end), slab kt + 1's k-step
                // 0 fragments, slab kt's k-step 3 MFMAs
                const int32_t kp2 = kt + 2 < KT ? (kt + 2) * kBK : 0;
                __builtin_amdgcn_sched_barrier(0);
                dma_p(L, kp2, pbuf(gp ^ 1), 0, kHalf);
                DMUON_READ(0, pbuf(gp), qbuf(gq), 0);
                DMUON_MFMA((KS - 1) & 1);
                DMUON_INTERLEAVE(NV);
                DMUON_SQ_FOLD(kt, KS - 1, (KS - 1) & 1);
            }
            DMUON_MFMA((KS - 1) & 1);  // the last slab's k-step 3
            DMUON_SQ_FOLD(KT - 1, KS - 1, (KS - 1) & 1);
            __syncthreads();           // every wave is done with the last slab's buffers
            epilogue(cur, EBuf{pbuf(gp), qbuf(gq)});
            // The queue ticket stays live through the epilogue.  Otherwise the
            // compiler reuses its register there and, counting none of the direct
            // loads, first waits for every load in flight (the next tile's first
            // slabs included); its wait for the ticket falls here instead, where
            // the tile-start wait below waits as long.
            asm volatile("" ::"v"(taken));
            if (!has_next) break;
            // The next tile: P of its slab 0 and Q of its slabs 0 and 1 were issued
            // in this tile's last two slabs, the epilogue's stores after them.
            // Slab 0 is waited for and published; vector memory operations
            // complete in issue order, stores included, so this also waits for
            // all but the last kDmaPerOp stores (leaving more of them in flight
            // measured no faster).
            __syncthreads();
            wait_vm<kDmaPerOp>();
            __syncthreads();
            gp ^= 1;
            gq = next3(gq);
            cur = nxt;
        }
    }
#undef DMUON_KSTEP
#undef DMUON_SQ_FOLD
#undef DMUON_INTERLEAVE
#undef DMUON_READ
#undef DMUON_READ_A
#undef DMUON_MFMA
    // no load into LDS may outlive the workgroup; then the last workgroup of
    // the launch empties the queues for the next launch
    wait_vm<0>();
    if (tid == 0) {
        __threadfence();
        const uint32_t done = atomicAdd(args.queue + kXcds, 1u);
        if (done == gridDim.x - 1) {
            for (int i = 0; i <= kXcds; ++i) args.queue[i] = 0u;
        }
    }
}

// Workgroups per XCD of a persistent launch: one per CU for 256-tiles (their
// five 32 KB operand buffers fill a CU's LDS), two per CU for 128-tiles; never more than
// the XCD has tiles.
template <int T>
int persistent_grid(int tiles) {
    constexpr int kCusPerXcd = 32, kPerCu = T == 256 ? 1 : 2;
    const int per_xcd = (tiles + kXcds - 1) / kXcds;
    return kXcds * (per_xcd < kCusPerXcd * kPerCu ? per_xcd : kCusPerXcd * kPerCu);
}

template <int T>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)persistent_grid<T>(a.total_blocks)), block(TileCfg<T>::NT);
    // the square folds its b A term into the accumulators when b / c is moderate
    const bool fold = a.c != 0.f && std::fabs(a.b / a.c) <= 64.f;
    // B X writes parameter updates from its epilogue when a segment asks for it
    bool fuse = false;
    for (int i = 0; i < a.nseg; ++i) fuse = fuse || a.seg[i].fuse != 0;
    switch (a.phase) {
        case kGram: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kGram, true>), grid, block, 0, stream, a); break;
        case kSquare:
            if (fold) hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kSquare, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kSquare, false>), grid, block, 0, stream, a);
            break;
        case kBX:
            if (fuse) hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kBX, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kBX, false>), grid, block, 0, stream, a);
            break;
        case kProd: hipLaunchKernelGGL((ns_gemm_bf16_kernel<T, kProd, true>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
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

// Internal types shared by the planner (host C++) and the HIP launchers.
// Nothing here is part of the C ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/dmuon_ns.h"

namespace dmuon {

constexpr int kPathF32 = DMUON_F32;
constexpr int kPathBF16 = DMUON_BF16;

// Elementwise kernels work on 64 x 64 tiles of the padded stored-orientation
// matrix; every tile granularity is a multiple of 64.  A prep or apply block
// takes kTilesPerBlock neighbouring tiles along the stored row (the last block
// of a row fewer when the row has an odd number of tiles): twice the bytes in
// flight per block, measured 3-4% faster than one tile on the 8B-model shapes.
constexpr int kPrepTile = 64;
constexpr int kTilesPerBlock = 2;
// Blocks of a prep pass over an r_pad x c_pad grid and of an apply pass over
// a rows x cols matrix.
inline int64_t prep_blocks_of(int64_t r_pad, int64_t c_pad) {
    return (r_pad / kPrepTile) * ((c_pad / kPrepTile + kTilesPerBlock - 1) / kTilesPerBlock);
}
inline int64_t apply_blocks_of(int64_t rows, int64_t cols) {
    const int64_t tc = (cols + kPrepTile - 1) / kPrepTile;
    return ((rows + kPrepTile - 1) / kPrepTile) * ((tc + kTilesPerBlock - 1) / kTilesPerBlock);
}
constexpr std::size_t kAlign = 256;
// Gram-space iterations between restarts unless the plan options say
// otherwise: 2 on buckets of padded short side up to 1024, 3 above.  Measured
// against the fp64 oracle on Gaussian inputs (5 iterations, relative O error):
// restarting every 3 iterations costs the small buckets accuracy (256 x 1536:
// 1.4e-2 against 9.1e-3 every 2; 1024 x 4096: 1.4e-2 against 8.9e-3), while
// the large ones do better every 3 (4096 x 14336: 8.6e-3 against 1.1e-2).
constexpr int32_t kDefaultGramRestartSmall = 2;
constexpr int32_t kDefaultGramRestartLarge = 3;
constexpr int64_t kGramRestartSmallMaxM = 1024;
inline int32_t default_gram_restart(int64_t m_pad) {
    return m_pad <= kGramRestartSmallMaxM ? kDefaultGramRestartSmall : kDefaultGramRestartLarge;
}
// The automatic rule's accuracy guard for the Gram-space form.  In bf16 the
// Gram space resolves small singular values worse than the short side, and
// it saves the least work where it loses the most accuracy: near-square
// matrices (at n = 1.5 m it executes 11-14% fewer flops for about 1.5 times
// the short side's error) and small short sides (whose products are latency-
// rather than flop-bound).  Measured against the fp64 oracle on Gaussian
// inputs, every bucket of padded short side >= 1024 whose members have
// n >= 3 m stays within 1.2e-2 relative error; the default therefore takes
// the Gram space only there.
constexpr int64_t kGramMinPaddedM = 1024;
constexpr int64_t kGramMinAspect = 3;
inline bool gram_auto_shape(int path, int64_t m_pad, int64_t n_pad) {
    return path == kPathBF16 && n_pad > m_pad && m_pad >= kGramMinPaddedM;
}
inline bool gram_auto_member(int64_t m, int64_t n) { return n >= kGramMinAspect * m; }
// Phases whose launch deals each XCD a contiguous run of a bucket's tiles by
// default: the B X product (bit 2), whose X panels are then reused in that
// XCD's L2.
constexpr uint32_t kDefaultXcdMask = 1u << 2;
constexpr uint32_t kAllPhasesMask = 0xFu;
// Buckets small enough to run every iteration in one workgroup with X in LDS
// (k_resident.hip): bf16 path, padded short side 128, padded long side at
// most 512, short-side iterations.
constexpr int64_t kResidentM = 128;
constexpr int64_t kResidentMaxN = 512;
inline bool resident_shape(int path, int64_t m_pad, int64_t n_pad) {
    return path == kPathBF16 && m_pad == kResidentM && n_pad >= kResidentM && n_pad <= kResidentMaxN;
}
// Longest side a bf16-gradient matrix may have: the bf16 kernels address up
// to 8 rows of a slab with one 32-bit byte offset per lane.
constexpr int64_t kMaxBf16Side = int64_t(1) << 27;

inline std::size_t align_up(std::size_t x, std::size_t a = kAlign) { return (x + a - 1) / a * a; }

// The persistent bf16 product launches take tiles from one queue per XCD: a
// counter per XCD and a count of finished workgroups (the last one resets all
// of them for the next launch), in the workspace.
constexpr int kQueueWords = 16;

struct MatPlan {
    int64_t rows, cols;
    int32_t grad_dtype, param_dtype;
    int64_t m, n;          // short, long side
    int32_t transposed;    // rows > cols
    int32_t bucket, slot;  // bucket in execution order, slot inside it
    int32_t plan_index;    // position in bucket-major execution order
    int64_t m_pad, n_pad;
    int64_t cost;          // 4 m^2 n + 2 m^3 of the real shape
    int64_t r_pad, c_pad;  // padded dims in the stored orientation
    int64_t prep_tiles;    // 64x64 tiles of the padded stored-orientation grid
    int64_t partial_off;   // first norm partial of this matrix
};

struct BucketPlan {
    int32_t path;          // kPathF32 | kPathBF16
    int32_t algo;          // DMUON_ALGO_SHORT_SIDE | DMUON_ALGO_GRAM_SPACE
    int32_t seg_len;       // iterations per segment: 1 (short side) or the Gram-space restart interval
    uint32_t xcd_mask;     // bf16: phases (bit per Phase) whose launch deals each XCD a contiguous tile run
    double cost_ms;        // measured per-matrix cost from a tuned entry, 0 if none
    int32_t apply_pass;    // 1: the update is written by the elementwise pass, never by B X
    int32_t tile;          // tile granularity g
    int64_t m_pad, n_pad;
    std::vector<int32_t> members;  // input indices, slot order
    int32_t plan_base;     // plan index of slot 0
    int64_t exec_cost;     // count * (4 m_pad^2 n_pad + 2 m_pad^3)
    int32_t esize;         // bytes per element of X / A / B
    // byte offsets of the bucket's arrays in the workspace; slot s of array Y
    // starts at off_Y + s * (its per-matrix size).  X (m_pad x n_pad) is kept in
    // two copies that the iterations ping-pong between.  Gram-space buckets
    // hold three more m_pad x m_pad arrays (off_g[0..2]); together with A and
    // B they carry the recurrence's A_k, Q_k, P_k, P_{k+1} and the product
    // A_k Q_k, whose roles rotate over the iterations.
    std::size_t off_x0, off_x1, off_a, off_b;
    std::size_t off_g[3];
};

}  // namespace dmuon

struct dmuon_plan {
    std::vector<dmuon::MatPlan> mats;        // input order
    std::vector<dmuon::BucketPlan> buckets;  // execution order
    std::vector<int32_t> order;              // plan index -> input index
    int64_t total_prep_tiles = 0;
    // off_queue: the grouped launches' tile-queue counters (dmuon::kQueueWords
    // uint32), zeroed at the start of every call
    std::size_t off_records = 0, off_scale = 0, off_partials = 0, off_queue = 0;
    std::size_t workspace_bytes = 0;
};

namespace dmuon {

// Per-matrix record kept in the workspace (device side), written at the start
// of every call.  Indexed by plan index.
struct DevMatRec {
    const void* src;       // gradient (step) or input (orthogonalisation)
    float* mom;            // momentum, nullptr for orthogonalisation
    void* dst;             // parameter (step) or output (orthogonalisation)
    int64_t x_off0;        // byte offset of this matrix's X copy 0 in the workspace
    int64_t x_off1;        // ... of X copy 1
    int64_t partial_off;   // first norm partial
    int64_t prep_begin;    // first prep block of this matrix (prefix sum)
    int64_t apply_begin;   // first apply block of this matrix (prefix sum)
    int32_t rows, cols;
    int32_t r_pad, c_pad;  // padded stored-orientation dims
    int32_t transposed;
    int32_t src_dtype, dst_dtype, path;
    float upd_scale;       // sqrt(max(1, rows / cols))
    int32_t final_copy;    // X copy (0 | 1) that holds the orthogonalised matrix
    int32_t fused;         // 1: the kernel ending the iteration (the last B X launch's
                           // epilogue, or the resident kernel) writes dst (update or
                           // output); X is not written back and the apply pass skips it
};

// Whether a step with `steps` iterations writes matrix mp's update from the
// kernel that finishes its iterations (else the apply pass writes it), in a
// bucket that keeps the default route: the resident kernel writes any
// parameter of its buckets; the last B X launch writes a bf16 parameter with
// cols a multiple of 8 (16-byte chunks of whole rows) of a bf16 bucket of
// tiled launches.
inline bool update_fused(const BucketPlan& bp, const MatPlan& mp, int32_t steps) {
    if (steps <= 0 || bp.apply_pass != 0) return false;
    const bool resident = bp.algo == DMUON_ALGO_SHORT_SIDE && resident_shape(bp.path, bp.m_pad, bp.n_pad);
    if (resident) return true;
    return bp.path == kPathBF16 && mp.param_dtype == DMUON_BF16 && mp.cols % 8 == 0;
}

// Apply kernel: each block covers kApplyElems elements of the real matrix.
constexpr int kApplyThreads = 256;
constexpr int kApplyElems = kApplyThreads * 8;

}  // namespace dmuon

// Host-side launchers of the HIP kernels (internal to libdmuon_ns).
#pragma once

#include <hip/hip_runtime.h>

#include <vector>

#include "dmuon_internal.h"

namespace dmuon {

// ---- elementwise passes (k_elementwise.hip) ----------------------------------

constexpr int kRecChunk = 24;  // records carried by one table-writing launch

struct RecChunk {
    DevMatRec* table;
    uint32_t* queue;  // the tile-queue counters, zeroed by the launch carrying record 0
    int32_t first;
    int32_t n;
    DevMatRec rec[kRecChunk];
};

hipError_t launch_write_records(const RecChunk& chunk, hipStream_t stream);

struct PrepArgs {
    const DevMatRec* recs;
    int32_t count;
    char* ws;
    float* partials;
    float beta;
    int32_t nesterov;
    int32_t has_momentum;  // 0: orthogonalisation (U = input)
    int64_t total_blocks;
};
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);

hipError_t launch_finalize_norms(const DevMatRec* recs, int32_t count, const float* partials,
                                 float* scale, float eps, hipStream_t stream);

struct ApplyArgs {
    const DevMatRec* recs;
    int32_t count;
    const char* ws;
    const float* scale;
    int32_t use_scale;     // ns_steps == 0: multiply by 1 / (||U|| + eps)
    int32_t update;        // 1: W' = W (1 - lr wd) - lr s O ; 0: dst = O
    float lr;
    float weight_decay;
    int64_t total_blocks;
};
hipError_t launch_apply(const ApplyArgs& a, hipStream_t stream);

// ---- Newton-Schulz products (k_gemm_bf16.hip, k_gemm_f32.hip) ---------------

// Products of one grouped launch, C[i][j] = sum_k P[i][k] Q[j][k]:
//   kGram    P = Q = X (m_pad x n_pad)       O = s^2 C          triangle, mirrored
//   kSquare  P = Q = A                       O = a I + b A + c C  triangle, mirrored
//   kBX      P = X^T (read from X), Q = B'   O = s C^T  (m_pad x n_pad)
//   kProd    P, Q two symmetric m x m        O = C              triangle, mirrored
// kProd serves the Gram-space recurrence, whose operands all commute, so the
// product of two of them is symmetric.
enum Phase : int32_t { kGram = 0, kSquare = 1, kBX = 2, kProd = 3 };
constexpr int kMaxSeg = 24;

// One bucket's share of a grouped launch.  Operand and output arrays are given
// as bucket base byte offsets in the workspace; slot s adds s times the
// per-slot size: x_stride for m_pad x n_pad arrays (the Gram's P and Q, the
// B X product's P and O), a_stride for m_pad x m_pad ones.
struct GemmSeg {
    int32_t first_block;    // first block id of this segment in the launch
    int32_t tiles_per_mat;  // output tiles per matrix
    int32_t tm;             // tiles along the short side (m_pad / tile)
    int32_t tn;             // tiles along the long side (n_pad / tile)
    int32_t count;          // matrices in the bucket
    int32_t plan_base;      // plan index of slot 0
    int32_t first_iter;     // apply the normalisation scale s (Gram s^2, B X s)
    int32_t xcd_remap;      // bf16: each XCD takes a contiguous run of this segment's tiles
    int32_t fuse;           // B X closing the last segment: for matrices whose record says
                            // fused, the epilogue writes dst (update or output) instead of X'
    int64_t m_pad, n_pad;
    int64_t p_off, q_off, o_off;  // operand P, operand Q (kProd, kBX), output
    int64_t x_stride, a_stride;   // per-slot bytes
};

struct GemmArgs {
    char* ws;
    uint32_t* queue;     // bf16: kQueueWords counters, zero at launch (kXcds tile counters, then the
                         // count of finished workgroups); the launch's last workgroup zeroes them again
    const float* scale;  // per plan index: 1 / (||U|| + eps)
    const DevMatRec* recs;  // per plan index (read by B X segments with fuse set)
    float lr, wd;           // the update W' = W (1 - lr wd) - lr s O of such segments ...
    int32_t update;         // ... when 1; 0: dst = O
    float a, b, c;
    int32_t phase;
    int32_t nseg;
    int32_t total_blocks;
    GemmSeg seg[kMaxSeg];
};

hipError_t launch_gemm_bf16(int tile, const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t stream);
// Output tile edge of the fp32 kernels (their buckets are padded to 64, a multiple of it).
int f32_kernel_tile();

// ---- AdamW for the non-Muon parameters (k_adamw.hip) ------------------------

constexpr int kAdamBlock = 2048;  // elements per block
constexpr int kAdamChunk = 64;    // tensors carried by one launch (kernel-argument table)

struct AdamRec {
    void* p;              // parameter (bf16 | fp32), updated in place
    const void* g;        // gradient (bf16 | fp32)
    float* m;             // first moment
    float* v;             // second moment
    int64_t n;            // elements (>= 1)
    int64_t block_begin;  // first block of this tensor in the launch
    int32_t p_dtype, g_dtype;
};

struct AdamArgs {
    float decay;           // 1 - lr wd
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float step_size;       // lr / (1 - beta1^t)
    float inv_sqrt_bc2;    // 1 / sqrt(1 - beta2^t)
    float eps;
    int32_t count;
    int64_t total_blocks;
    AdamRec rec[kAdamChunk];
};

hipError_t launch_adamw(const AdamArgs& a, hipStream_t stream);

// ---- small matrices resident in LDS (k_resident.hip) ---------------------------

struct ResidentBucket {
    int32_t plan_base;  // first plan index of the bucket's matrices
    int32_t count;
    int64_t n_pad;
};

// All ns_steps (> 0) iterations of the given buckets' matrices: X from each
// record's copy 0, the normalisation from the record's norm partials (summed
// as finalize_norms sums them), and the result into the parameter (update, or
// output: W' as the apply pass computes it) for a fused record, else into the
// X copy final_copy.
struct ResidentStep {
    const float* partials;
    float eps, a, b, c;
    int32_t steps;
    int32_t update;  // 1: W' = W (1 - lr wd) - lr s O ; 0: dst = O
    float lr, wd;
};
hipError_t launch_resident(const DevMatRec* recs, char* ws, const ResidentStep& st,
                           const std::vector<ResidentBucket>& buckets, hipStream_t stream);

}  // namespace dmuon

// Bandwidth-bound passes of the owner-side Muon step (gfx950):
//   prep   -- momentum accumulation, the Nesterov look-ahead U, U cast to the
//             NS operand dtype and written as X (m x n, short side first:
//             transposed for tall matrices, zero padded), and per-tile partial
//             sums of U^2;
//   norms  -- per matrix, the fixed-order sum of those partials:
//             scale = 1 / (||U||_F + eps);
//   apply  -- the parameter update W' = W (1 - lr wd) - lr s O, or the output
//             O, read from the final X back in the stored orientation
//             (transposed through LDS for tall matrices).
// The normalisation itself is folded into the first Newton-Schulz
// iteration's epilogues (A0 = scale^2 U U^T, X1 = scale (a U + B0 U)), so U
// is read from HBM once.
//
// Page basis: NS acts on the momentum-aggregated gradient (DMuon explainer on
// gist.science, "Technische Samenvatting" section 1); the owner holds the
// optimizer state and applies the update to the full matrix (section 2.1
// Owner-Centric Executiestrategie; DMuon abstract).
#include "kcommon.h"
#include "launch.h"

namespace dmuon {
namespace {

constexpr int kThreads = 256;

__global__ void write_records_kernel(RecChunk c) {
    const int i = threadIdx.x;
    if (i < c.n) c.table[c.first + i] = c.rec[i];
    if (c.first == 0 && i < kQueueWords) c.queue[i] = 0u;  // the call's tile queues start empty
}

// Sum of squares of four values, in one fixed order of explicit operations.
__device__ __forceinline__ float sumsq4(float4 v) {
    float s = v.x * v.x;
    s = fmaf(v.y, v.y, s);
    s = fmaf(v.z, v.z, s);
    return fmaf(v.w, v.w, s);
}

// ---- prep ---------------------------------------------------------------------
// One block per 64 x 64 tile of the padded stored-orientation matrix.  Thread
// t covers columns 4 (t % 16) .. +3 of rows t / 16 + 16 p, p = 0..3.  X is
// m_pad x n_pad: for a wide or square matrix it is U itself, for a tall one
// U^T, written from the LDS copy of the tile so both sides stay coalesced.
// The norm partials are taken in X's orientation -- each thread sums the
// squares of the float4 groups it writes to X, and the partial of X tile
// (i, j) sits at index i * (X tiles per row) + j -- so a tall matrix and its
// transpose get bitwise the same norm.
template <typename T, bool VEC>
__device__ __forceinline__ void prep_tile(const PrepArgs& a, const DevMatRec& r, int64_t local,
                                          float (*tile)[kPrepTile + 1], float* red) {
    const int64_t tiles_c = r.c_pad / kPrepTile;
    const int64_t rho0 = (local / tiles_c) * kPrepTile;
    const int64_t kap0 = (local % tiles_c) * kPrepTile;
    const int t = threadIdx.x, cg = t & 15, rr = t >> 4;
    const T* G = static_cast<const T*>(r.src);
    float* M = r.mom;
    T* X = reinterpret_cast<T*>(a.ws + r.x_off0);
    const float beta = a.beta;
    float ss = 0.f;
    // every row's loads first, so that all of them are in flight at once (the
    // stores below could alias them as far as the compiler knows)
    float4 gv[4], mv[4];
    if (VEC) {
        #pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t rho = rho0 + rr + 16 * p, kap = kap0 + 4 * cg;
            if (rho < r.rows && kap < r.cols) {
                gv[p] = load4(G + rho * r.cols + kap);
                if (a.has_momentum) mv[p] = load4(M + rho * r.cols + kap);
            }
        }
    }
    #pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = rr + 16 * p;
        const int64_t rho = rho0 + row;
        const int64_t kap = kap0 + 4 * cg;
        float u[4] = {0.f, 0.f, 0.f, 0.f};
        if (rho < r.rows) {
            const int64_t e = rho * r.cols + kap;
            if (VEC) {
                if (kap < r.cols) {
                    const float4 g = gv[p];
                    float4 uu = g;
                    if (a.has_momentum) {
                        const float4 m = mv[p];
                        float4 mn;
                        mn.x = fmaf(beta, m.x, g.x);
                        mn.y = fmaf(beta, m.y, g.y);
                        mn.z = fmaf(beta, m.z, g.z);
                        mn.w = fmaf(beta, m.w, g.w);
                        store4(M + e, mn);
                        if (a.nesterov) {
                            uu.x = fmaf(beta, mn.x, g.x);
                            uu.y = fmaf(beta, mn.y, g.y);
                            uu.z = fmaf(beta, mn.z, g.z);
                            uu.w = fmaf(beta, mn.w, g.w);
                        } else {
                            uu = mn;
                        }
                    }
                    u[0] = uu.x; u[1] = uu.y; u[2] = uu.z; u[3] = uu.w;
                }
            } else {
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (kap + q < r.cols) {
                        const float g = Elem<T>::load(G + e + q);
                        float uq = g;
                        if (a.has_momentum) {
                            const float mn = fmaf(beta, M[e + q], g);
                            M[e + q] = mn;
                            uq = a.nesterov ? fmaf(beta, mn, g) : mn;
                        }
                        u[q] = uq;
                    }
                }
            }
        }
        if (!r.transposed) {
            const float4 v = make_float4(u[0], u[1], u[2], u[3]);
            ss += sumsq4(v);
            store4(X + rho * r.c_pad + kap, v);
        } else {
            #pragma unroll
            for (int q = 0; q < 4; ++q) tile[row][4 * cg + q] = u[q];
        }
    }
    if (r.transposed) {
        __syncthreads();
        #pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row_e = rr + 16 * p;  // column offset in the stored orientation
            const float4 v = make_float4(tile[4 * cg + 0][row_e], tile[4 * cg + 1][row_e],
                                         tile[4 * cg + 2][row_e], tile[4 * cg + 3][row_e]);
            ss += sumsq4(v);
            store4(X + (kap0 + row_e) * r.r_pad + rho0 + 4 * cg, v);
        }
    }
    const float total = block_sum<kThreads>(ss, red);
    // X tile index: stored tile (rt, ct) is X tile (ct, rt) for a tall matrix
    const int64_t xi = r.transposed ? (local % tiles_c) * (r.r_pad / kPrepTile) + local / tiles_c : local;
    if (t == 0) a.partials[r.partial_off + xi] = total;
}

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
    __shared__ float tile[kPrepTile][kPrepTile + 1];
    __shared__ float red[kThreads / 64];
    const int64_t bid = blockIdx.x;
    const int i = upper_index(a.count, bid, [&](int k) { return a.recs[k].prep_begin; });
    const DevMatRec r = a.recs[i];
    const int64_t local = bid - r.prep_begin;
    const bool vec = (r.cols & 3) == 0;
    if (r.path == kPathBF16) {
        if (vec) prep_tile<uint16_t, true>(a, r, local, tile, red);
        else prep_tile<uint16_t, false>(a, r, local, tile, red);
    } else {
        if (vec) prep_tile<float, true>(a, r, local, tile, red);
        else prep_tile<float, false>(a, r, local, tile, red);
    }
}

// ---- norms ----------------------------------------------------------------------
// One block per matrix; every thread sums a fixed stride of the partials, then
// a fixed reduction tree: the result does not depend on scheduling.
__global__ __launch_bounds__(kThreads) void finalize_norms_kernel(const DevMatRec* recs, const float* partials,
                                                                   float* scale, float eps) {
    __shared__ float red[kThreads / 64];
    const DevMatRec r = recs[blockIdx.x];
    const int64_t n = (r.r_pad / kPrepTile) * (r.c_pad / kPrepTile);
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += kThreads) s += partials[r.partial_off + i];
    const float total = block_sum<kThreads>(s, red);
    if (threadIdx.x == 0) scale[blockIdx.x] = 1.0f / (sqrtf(total) + eps);
}

// ---- apply ----------------------------------------------------------------------
// One block per 64 x 64 tile of the real (unpadded) matrix, stored orientation.
// O is the final X (m_pad x n_pad) for a wide or square matrix and its
// transpose for a tall one; the transposed tile goes through LDS.
template <typename FT, typename DT, bool VEC>
__device__ __forceinline__ void apply_tile(const ApplyArgs& a, const DevMatRec& r, int plan_idx,
                                           int64_t local, float (*tile)[kPrepTile + 1]) {
    const int64_t tiles_c = (r.cols + kPrepTile - 1) / kPrepTile;
    const int64_t rho0 = (local / tiles_c) * kPrepTile;
    const int64_t kap0 = (local % tiles_c) * kPrepTile;
    const int t = threadIdx.x, cg = t & 15, rr = t >> 4;
    const FT* F = reinterpret_cast<const FT*>(a.ws + (r.final_copy ? r.x_off1 : r.x_off0));
    DT* W = static_cast<DT*>(r.dst);
    const float sigma = a.use_scale ? a.scale[plan_idx] : 1.0f;
    const float coef = -a.lr * r.upd_scale * sigma;
    const float keep = 1.0f - a.lr * a.weight_decay;
    if (r.transposed) {
        // X rows kap0 .. kap0 + 63, columns rho0 .. rho0 + 63 (inside the padding)
        #pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = rr + 16 * p;
            const float4 v = load4(F + (kap0 + row) * r.r_pad + rho0 + 4 * cg);
            tile[4 * cg + 0][row] = v.x;
            tile[4 * cg + 1][row] = v.y;
            tile[4 * cg + 2][row] = v.z;
            tile[4 * cg + 3][row] = v.w;
        }
        __syncthreads();
    }
    #pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = rr + 16 * p;
        const int64_t rho = rho0 + row;
        const int64_t kap = kap0 + 4 * cg;
        if (rho >= r.rows) continue;
        const int64_t e = rho * r.cols + kap;
        float o[4];
        if (r.transposed) {
            #pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = tile[row][4 * cg + q];
        } else {
            const float4 v = load4(F + rho * r.c_pad + kap);
            o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
        }
        if (VEC) {
            if (kap >= r.cols) continue;
            float4 w;
            if (a.update) {
                w = load4(W + e);
                w.x = fmaf(coef, o[0], keep * w.x);
                w.y = fmaf(coef, o[1], keep * w.y);
                w.z = fmaf(coef, o[2], keep * w.z);
                w.w = fmaf(coef, o[3], keep * w.w);
            } else {
                w = make_float4(sigma * o[0], sigma * o[1], sigma * o[2], sigma * o[3]);
            }
            store4(W + e, w);
        } else {
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (kap + q >= r.cols) break;
                float w;
                if (a.update) w = fmaf(coef, o[q], keep * Elem<DT>::load(W + e + q));
                else w = sigma * o[q];
                Elem<DT>::store(W + e + q, w);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void apply_kernel(ApplyArgs a) {
    __shared__ float tile[kPrepTile][kPrepTile + 1];
    const int64_t bid = blockIdx.x;
    const int i = upper_index(a.count, bid, [&](int k) { return a.recs[k].apply_begin; });
    const DevMatRec r = a.recs[i];
    const int64_t local = bid - r.apply_begin;
    const bool vec = (r.cols & 3) == 0;
    const bool fb = r.path == kPathBF16, db = r.dst_dtype == DMUON_BF16;
#define DMUON_APPLY(FT, DT)                                  \
    do {                                                     \
        if (vec) apply_tile<FT, DT, true>(a, r, i, local, tile);   \
        else apply_tile<FT, DT, false>(a, r, i, local, tile);      \
    } while (0)
    if (fb && db) DMUON_APPLY(uint16_t, uint16_t);
    else if (fb) DMUON_APPLY(uint16_t, float);
    else if (db) DMUON_APPLY(float, uint16_t);
    else DMUON_APPLY(float, float);
#undef DMUON_APPLY
}

}  // namespace

hipError_t launch_write_records(const RecChunk& chunk, hipStream_t stream) {
    hipLaunchKernelGGL(write_records_kernel, dim3(1), dim3(64), 0, stream, chunk);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream) {
    if (a.total_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)a.total_blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_finalize_norms(const DevMatRec* recs, int32_t count, const float* partials,
                                 float* scale, float eps, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(finalize_norms_kernel, dim3(count), dim3(kThreads), 0, stream, recs,
                       partials, scale, eps);
    return hipGetLastError();
}

hipError_t launch_apply(const ApplyArgs& a, hipStream_t stream) {
    if (a.total_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(apply_kernel, dim3((unsigned)a.total_blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dmuon

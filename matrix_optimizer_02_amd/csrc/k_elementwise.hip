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
// One block per kTilesPerBlock neighbouring 64 x 64 tiles along a row of the
// padded stored-orientation matrix; every load of the block is issued before
// the first tile is worked on.  In each tile thread t covers columns
// 4 (t % 16) .. +3 of rows t / 16 + 16 p, p = 0..3.  X is m_pad x n_pad: for
// a wide or square matrix it is U itself, for a tall one U^T, written from
// the LDS copy of the tile so both sides stay coalesced.  The norm partials
// are taken in X's orientation -- thread t sums the squares of the float4
// groups it writes to X, rows t / 16 + 16 p and columns 4 (t % 16) .. +3 of
// the X tile, in that order, the waves' sums are added in wave order, and the
// partial of X tile (i, j) sits at index i * (X tiles per row) + j -- so a
// tall matrix and its transpose get bitwise the same norm.
template <typename T, bool VEC>
__device__ __forceinline__ void prep_block(const PrepArgs& a, const DevMatRec& r, int64_t local,
                                           float (*tile)[kPrepTile + 1], float (*red)[kThreads / 64]) {
    constexpr int TC = kTilesPerBlock;
    const int64_t tiles_c = r.c_pad / kPrepTile;
    const int64_t bpr = (tiles_c + TC - 1) / TC;
    const int64_t rt = local / bpr, ct0 = (local % bpr) * TC;
    const int nt = (int)(tiles_c - ct0 < TC ? tiles_c - ct0 : TC);  // tiles in this block
    const int64_t rho0 = rt * kPrepTile;
    const int t = threadIdx.x, cg = t & 15, rr = t >> 4;
    const T* G = static_cast<const T*>(r.src);
    float* M = r.mom;
    T* X = reinterpret_cast<T*>(a.ws + r.x_off0);
    const float beta = a.beta;
    // every tile's loads first, so that all of them are in flight at once (the
    // stores below could alias them as far as the compiler knows)
    float4 gv[TC][4], mv[TC][4];
    if (VEC) {
        #pragma unroll
        for (int c = 0; c < TC; ++c) {
            if (c >= nt) break;
            #pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int64_t rho = rho0 + rr + 16 * p, kap = (ct0 + c) * kPrepTile + 4 * cg;
                if (rho < r.rows && kap < r.cols) {
                    gv[c][p] = load4(G + rho * r.cols + kap);
                    if (a.has_momentum) mv[c][p] = load4(M + rho * r.cols + kap);
                }
            }
        }
    }
    float ss[TC];
    #pragma unroll
    for (int c = 0; c < TC; ++c) {
        ss[c] = 0.f;
        if (c >= nt) break;
        const int64_t kap0 = (ct0 + c) * kPrepTile;
        const int64_t kap = kap0 + 4 * cg;
        if (r.transposed && c > 0) __syncthreads();  // the previous tile's LDS reads are done
        #pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = rr + 16 * p;
            const int64_t rho = rho0 + row;
            float u[4] = {0.f, 0.f, 0.f, 0.f};
            if (rho < r.rows) {
                const int64_t e = rho * r.cols + kap;
                if (VEC) {
                    if (kap < r.cols) {
                        const float4 g = gv[c][p];
                        float4 uu = g;
                        if (a.has_momentum) {
                            const float4 m = mv[c][p];
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
                ss[c] += sumsq4(v);
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
                ss[c] += sumsq4(v);
                store4(X + (kap0 + row_e) * r.r_pad + rho0 + 4 * cg, v);
            }
        }
    }
    // one partial per tile: the wave sums (fixed shuffle tree), then the waves in order
    const int lane = t & 63, wave = t >> 6;
    #pragma unroll
    for (int c = 0; c < TC; ++c) {
        float v = ss[c];
        #pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[c][wave] = v;
    }
    __syncthreads();
    if (t < nt) {
        float total = red[t][0];
        #pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) total += red[t][w];
        // X tile index: stored tile (rt, ct) is X tile (ct, rt) for a tall matrix
        const int64_t ct = ct0 + t;
        const int64_t xi = r.transposed ? ct * (r.r_pad / kPrepTile) + rt : rt * tiles_c + ct;
        a.partials[r.partial_off + xi] = total;
    }
}

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
    __shared__ float tile[kPrepTile][kPrepTile + 1];
    __shared__ float red[kTilesPerBlock][kThreads / 64];
    const int64_t bid = blockIdx.x;
    const int i = upper_index(a.count, bid, [&](int k) { return a.recs[k].prep_begin; });
    const DevMatRec r = a.recs[i];
    const int64_t local = bid - r.prep_begin;
    const bool vec = (r.cols & 3) == 0;
    if (r.path == kPathBF16) {
        if (vec) prep_block<uint16_t, true>(a, r, local, tile, red);
        else prep_block<uint16_t, false>(a, r, local, tile, red);
    } else {
        if (vec) prep_block<float, true>(a, r, local, tile, red);
        else prep_block<float, false>(a, r, local, tile, red);
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
// One block per kTilesPerBlock neighbouring 64 x 64 tiles along a row of the
// real (unpadded) matrix, stored orientation; thread t covers columns
// 4 (t % 16) .. +3 of rows t / 16 + 16 p of each tile.  O is the final X
// (m_pad x n_pad) for a wide or square matrix and its transpose for a tall
// one; the transposed tile goes through LDS.  The block's O loads are issued
// before the first tile is worked on; each parameter row is loaded where it is
// updated (loading the parameter rows up front as well measured 30% slower on
// the 8B-model shapes).
template <typename FT, typename DT, bool VEC>
__device__ __forceinline__ void apply_block(const ApplyArgs& a, const DevMatRec& r, int plan_idx,
                                            int64_t local, float (*tile)[kPrepTile + 1]) {
    constexpr int TC = kTilesPerBlock;
    const int64_t tiles_c = (r.cols + kPrepTile - 1) / kPrepTile;
    const int64_t bpr = (tiles_c + TC - 1) / TC;
    const int64_t ct0 = (local % bpr) * TC;
    const int nt = (int)(tiles_c - ct0 < TC ? tiles_c - ct0 : TC);
    const int64_t rho0 = (local / bpr) * kPrepTile;
    const int t = threadIdx.x, cg = t & 15, rr = t >> 4;
    const FT* F = reinterpret_cast<const FT*>(a.ws + (r.final_copy ? r.x_off1 : r.x_off0));
    DT* W = static_cast<DT*>(r.dst);
    const float sigma = a.use_scale ? a.scale[plan_idx] : 1.0f;
    const float coef = -a.lr * r.upd_scale * sigma;
    const float keep = 1.0f - a.lr * a.weight_decay;
    float4 fv[TC][4];
    #pragma unroll
    for (int c = 0; c < TC; ++c) {
        if (c >= nt) break;
        const int64_t kap0 = (ct0 + c) * kPrepTile;
        #pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = rr + 16 * p;
            const int64_t rho = rho0 + row, kap = kap0 + 4 * cg;
            if (r.transposed) {
                // X rows kap0 .. kap0 + 63, columns rho0 .. rho0 + 63 (inside the padding)
                fv[c][p] = load4(F + (kap0 + row) * r.r_pad + rho0 + 4 * cg);
            } else if (rho < r.rows) {
                fv[c][p] = load4(F + rho * r.c_pad + kap);
            }
        }
    }
    #pragma unroll
    for (int c = 0; c < TC; ++c) {
        if (c >= nt) break;
        const int64_t kap = (ct0 + c) * kPrepTile + 4 * cg;
        if (r.transposed) {
            if (c > 0) __syncthreads();  // the previous tile's LDS reads are done
            #pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int row = rr + 16 * p;
                tile[4 * cg + 0][row] = fv[c][p].x;
                tile[4 * cg + 1][row] = fv[c][p].y;
                tile[4 * cg + 2][row] = fv[c][p].z;
                tile[4 * cg + 3][row] = fv[c][p].w;
            }
            __syncthreads();
        }
        #pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = rr + 16 * p;
            const int64_t rho = rho0 + row;
            if (rho >= r.rows) continue;
            const int64_t e = rho * r.cols + kap;
            float o[4];
            if (r.transposed) {
                #pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = tile[row][4 * cg + q];
            } else {
                o[0] = fv[c][p].x; o[1] = fv[c][p].y; o[2] = fv[c][p].z; o[3] = fv[c][p].w;
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
        if (vec) apply_block<FT, DT, true>(a, r, i, local, tile);   \
        else apply_block<FT, DT, false>(a, r, i, local, tile);      \
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

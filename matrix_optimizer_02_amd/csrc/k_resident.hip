// Newton-Schulz for small bf16 matrices (padded short side 128, padded long
// side at most 512), one workgroup per matrix for all iterations: X (128 x
// n_pad bf16, up to 128 KB) and the 128 x 128 A / B' array (32 KB) stay in
// LDS, so an iteration costs three barriers instead of three grouped launches.
// Launches of such single-tile products are latency-bound (a few microseconds
// each, whatever their size), which is what this kernel removes.  It also
// takes over the per-matrix launches around the iteration: it sums the
// matrix's norm partials itself and, on the default route, writes the
// parameter update (or the output) from the final X in LDS, so neither the
// finalize nor the apply pass runs for its matrices.
//
// The arithmetic is the tiled kernels' short-side iteration, with the same
// operand and output roundings: per iteration, with s = 1 / (||U||_F + eps) in
// the first and 1 afterwards,
//   A  = s^2 X X^T                     (bf16)
//   B' = a I + b A + c A A             (bf16; A A = A A^T, A is symmetric)
//   X' = s B' X                        (bf16, in place: column strip by strip)
// All 16 32 x 32 blocks of A and of A A are computed (the triangle saving is
// not worth a second pass at this size).  Page basis: matrices of similar
// small shapes are batched so that they keep the GPU busy and amortise
// dispatch (DMuon explainer on gist.science, second section 2.1, "Batching").
//
// LDS rows (X: 2 n_pad bytes, A: 256 bytes, both multiples of 256) hold
// 16-byte chunks XOR-swizzled by row within aligned groups of 16 chunks:
//   f(r) = 2 (r mod 4) + (r / 4 mod 2) + 8 (r / 8 mod 2)
// so the fragment reads of 16 consecutive rows at one logical chunk, and the
// transposing reads of 4 consecutive rows at two adjacent chunks, fall in
// distinct bank groups.
#include "kcommon.h"
#include "launch.h"


namespace dmuon {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kM = (int)kResidentM;         // padded short side
constexpr int kMaxN = (int)kResidentMaxN;   // largest padded long side
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kARowBytes = 2 * kM;          // 256
constexpr int kXBytes = kM * kMaxN * 2;     // 128 KB
constexpr int kABytes = kM * kARowBytes;    // 32 KB

__device__ __forceinline__ int rswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

// Byte offset of element (r, c) (c a multiple of 4 for 8-byte accesses, of 8
// for 16-byte ones) in an LDS array with rows of row_bytes.
__device__ __forceinline__ int loff(int r, int c, int row_bytes) {
    return r * row_bytes + ((((c >> 3) ^ rswz(r))) << 4) + (c & 7) * 2;
}

__device__ __forceinline__ bf16x8 ld8(const char* base, int off) {
    return *reinterpret_cast<const bf16x8*>(base + off);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// C = P P^T over K (= 128 rows of P, K-contiguous, in LDS with rows of
// row_bytes): wave w computes blocks (w / 2, 2 (w % 2) + j), j = 0, 1;
// acc[j][v] is row 32 (w / 2) + 8 (v / 4) + 4 (lane / 32) + v % 4, column
// 32 (2 (w % 2) + j) + lane % 32.
__device__ __forceinline__ void sym_product(const char* P, int row_bytes, int K, int wave, int lane,
                                            floatx16 (&acc)[2]) {
    const int lrow = lane & 31, khalf = lane >> 5;
    const int ra = 32 * (wave >> 1) + lrow;
    const int rb0 = 64 * (wave & 1) + lrow;
    #pragma unroll
    for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    // the next k-step's fragments are read before this one's MFMAs
    bf16x8 fa = ld8(P, loff(ra, 8 * khalf, row_bytes));
    bf16x8 fb0 = ld8(P, loff(rb0, 8 * khalf, row_bytes));
    bf16x8 fb1 = ld8(P, loff(rb0 + 32, 8 * khalf, row_bytes));
    #pragma unroll 1
    for (int k = 16; k < K; k += 16) {
        const int c = k + 8 * khalf;
        const bf16x8 na = ld8(P, loff(ra, c, row_bytes));
        const bf16x8 nb0 = ld8(P, loff(rb0, c, row_bytes));
        const bf16x8 nb1 = ld8(P, loff(rb0 + 32, c, row_bytes));
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb0, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb1, acc[1], 0, 0, 0);
        fa = na;
        fb0 = nb0;
        fb1 = nb1;
    }
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb1, acc[1], 0, 0, 0);
}

struct ResidentSeg {
    int32_t plan_base, count, n_pad, first_block;
};

struct ResidentArgs {
    const DevMatRec* recs;
    char* ws;
    const float* partials;
    float eps, a, b, c;
    int32_t steps;
    int32_t update;
    float lr, wd;
    int32_t nseg;
    ResidentSeg seg[kMaxSeg];
};

// Per thread, kB 16-byte chunks of X are moved at a time, their global loads
// all issued before the first is used.  The chunk count (16 n_pad) is a
// multiple of kThreads but not always of kB kThreads: an index past the end
// is taken modulo the count, which repeats a chunk of the same batch
// (straight-line code, no branch between the loads).
constexpr int kB = 8;
__device__ __forceinline__ int wrap(int q, int total) { return q < total ? q : q - total; }

// The parameter (or output) of a fused record, from the final X in LDS: O is X
// for a wide matrix and X^T for a tall one; W' = keep W + coef O element by
// element with coef = -lr sqrt(max(1, rows / cols)) and keep = 1 - lr wd,
// rounded once to the parameter's type (the apply pass's arithmetic), or
// O itself without the update.  A chunk is 8 consecutive elements of a
// parameter row; a tall matrix's chunks are columns of X, read with the
// transposing LDS read by groups of 16 lanes (16 parameter rows, one 8-column
// block).  VEC (cols a multiple of 8): 16- or 32-byte accesses per chunk;
// otherwise element by element.  Chunks outside the matrix (padding, or a
// repeated index) load from element 0 and store nothing.
template <typename DT, bool TALL, bool VEC>
__device__ __forceinline__ void write_param(const char* X, int xrow, int n, const DevMatRec& rec,
                                            const ResidentArgs& args, int tid) {
    constexpr bool kBF = sizeof(DT) == 2;
    const int rows = rec.rows, cols = rec.cols;  // rows cols <= kM kMaxN: int offsets
    DT* const W = static_cast<DT*>(rec.dst);
    const bool update = args.update != 0;
    const float coef = -args.lr * rec.upd_scale;
    const float keep = 1.0f - args.lr * args.wd;
    const int total = kM * n / 8;
    const int t16 = tid & 15;
    for (int q0 = 0; q0 < total; q0 += kB * kThreads) {
        u32x4_t o[kB];
        int off[kB], pcol[kB];
        bool ok[kB];
        u32x4_t wb[kB];       // VEC, bf16
        f32x4_t wf[kB][2];    // VEC, fp32
        float ws[kB][8];      // element by element
        #pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int qr = q0 + u * kThreads + tid;
            const int q = wrap(qr, total);
            int prow;
            if (!TALL) {
                prow = q / (n / 8);
                pcol[u] = 8 * (q % (n / 8));
                o[u] = *reinterpret_cast<const u32x4_t*>(X + loff(prow, pcol[u], xrow));
            } else {
                // group q / 16: parameter rows 16 (gq / 16) + t16, columns 8 (gq % 16) ..
                const int gq = q >> 4;
                const int k0 = 8 * (gq & 15), r0 = 16 * (gq >> 4);
                prow = r0 + t16;
                pcol[u] = k0;
                shortx4 hv[2];
                #pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_shortx4*)((__attribute__((address_space(3))) char*)X +
                                       loff(k0 + 4 * hh + (t16 >> 2), r0 + 4 * (t16 & 3), xrow)));
                o[u] = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
                // every lane takes part in the transposing reads: keep them
                // out of the branches below
                asm volatile("" : "+v"(o[u]));
            }
            ok[u] = qr < total && prow < rows && pcol[u] < cols;
            off[u] = ok[u] ? prow * cols + pcol[u] : 0;
        }
        if (update) {
            #pragma unroll
            for (int u = 0; u < kB; ++u) {
                if (VEC) {
                    if constexpr (kBF) {
                        wb[u] = ld_stream<u32x4_t>(W + off[u]);
                    } else {
                        wf[u][0] = ld_stream<f32x4_t>(W + off[u]);
                        wf[u][1] = ld_stream<f32x4_t>(W + off[u] + 4);
                    }
                } else {
                    #pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ws[u][e] = Elem<DT>::load(W + (ok[u] && pcol[u] + e < cols ? off[u] + e : 0));
                }
            }
        }
        #pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (!ok[u]) continue;
            float v[8];
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = __uint_as_float(o[u][e] << 16);
                v[2 * e + 1] = __uint_as_float(o[u][e] & 0xffff0000u);
            }
            if (update) {
                float w[8];
                #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (!VEC) w[e] = ws[u][e];
                    else if constexpr (kBF)
                        w[e] = (e & 1) ? __uint_as_float(wb[u][e / 2] & 0xffff0000u) : __uint_as_float(wb[u][e / 2] << 16);
                    else w[e] = wf[u][e / 4][e % 4];
                }
                #pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = fmaf(coef, v[e], keep * w[e]);
            }
            DT* const dst = W + off[u];
            if (VEC) {
                if constexpr (kBF) {
                    u32x4_t s;
                    #pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[e] = (uint32_t)f32_to_bf16(v[2 * e]) | ((uint32_t)f32_to_bf16(v[2 * e + 1]) << 16);
                    st_stream<u32x4_t>(dst, s);
                } else {
                    st_stream<f32x4_t>(dst, f32x4_t{v[0], v[1], v[2], v[3]});
                    st_stream<f32x4_t>(dst + 4, f32x4_t{v[4], v[5], v[6], v[7]});
                }
            } else {
                #pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (pcol[u] + e < cols) Elem<DT>::store(dst + e, v[e]);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads, 1) void ns_resident_kernel(ResidentArgs args) {
    __shared__ __attribute__((aligned(1024))) char smem[kXBytes + kABytes];
    char* const X = smem;
    char* const Ar = smem + kXBytes;

    int s = 0;
    while (s + 1 < args.nseg && (int)blockIdx.x >= args.seg[s + 1].first_block) ++s;
    const ResidentSeg& sg = args.seg[s];
    const int pi = sg.plan_base + ((int)blockIdx.x - sg.first_block);
    const DevMatRec& rec = args.recs[pi];
    const int n = sg.n_pad;
    const int xrow = 2 * n;  // X row bytes
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 31, khalf = lane >> 5;

    // s = 1 / (||U||_F + eps) from the record's norm partials, summed as
    // finalize_norms sums them (there: thread t adds partials t, t + 256, ..,
    // the waves reduce by butterfly and thread 0 adds the wave sums in order;
    // with at most 64 partials only wave 0's sum is nonzero, so every lane of
    // each wave here forms the same value bit for bit)
    static_assert((kM / kPrepTile) * (kMaxN / kPrepTile) <= 64, "one partial a lane");
    const int np = (rec.r_pad / kPrepTile) * (rec.c_pad / kPrepTile);
    float nsum = 0.f;
    if (lane < np) nsum += args.partials[rec.partial_off + lane];
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) nsum += __shfl_xor(nsum, off, 64);
    const float s0 = 1.0f / (sqrtf(nsum) + args.eps);

    // X (the prepared U, copy 0) into LDS, kB loads in flight per thread (a
    // repeated chunk is stored twice, with the same bytes)
    const uint4* xg = reinterpret_cast<const uint4*>(args.ws + rec.x_off0);
    const int chunks = kM * n / 8;
    for (int q0 = 0; q0 < chunks; q0 += kB * kThreads) {
        uint4 xv[kB];
        #pragma unroll
        for (int u = 0; u < kB; ++u) xv[u] = xg[wrap(q0 + u * kThreads + tid, chunks)];
        #pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int q = wrap(q0 + u * kThreads + tid, chunks);
            *reinterpret_cast<uint4*>(X + loff(q / (n / 8), 8 * (q % (n / 8)), xrow)) = xv[u];
        }
    }

    const float a = args.a, b = args.b, c = args.c;
    for (int it = 0; it < args.steps; ++it) {
        const float sc = it == 0 ? s0 : 1.0f;
        __syncthreads();  // X' complete; every wave done with B'

        // ---- A = s^2 X X^T, stored transposed (A is symmetric) -------------------
        floatx16 acc[2];
        sym_product(X, xrow, n, wave, lane, acc);
        const float s2 = sc * sc;
        #pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 64 * (wave & 1) + 32 * j + lrow;
            #pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int r0 = 32 * (wave >> 1) + 8 * v4 + 4 * khalf;
                uint2 o;
                o.x = pack2(s2 * acc[j][4 * v4 + 0], s2 * acc[j][4 * v4 + 1]);
                o.y = pack2(s2 * acc[j][4 * v4 + 2], s2 * acc[j][4 * v4 + 3]);
                *reinterpret_cast<uint2*>(Ar + loff(col, r0, kARowBytes)) = o;
            }
        }
        __syncthreads();

        // ---- B' = a I + b A + c A A ------------------------------------------------
        sym_product(Ar, kARowBytes, kM, wave, lane, acc);
        uint2 av[2][4];  // A at this lane's outputs, read as A[col][r0 .. r0 + 3]
        #pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 64 * (wave & 1) + 32 * j + lrow;
            #pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int r0 = 32 * (wave >> 1) + 8 * v4 + 4 * khalf;
                av[j][v4] = *reinterpret_cast<const uint2*>(Ar + loff(col, r0, kARowBytes));
            }
        }
        __syncthreads();  // every wave done reading A
        #pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 64 * (wave & 1) + 32 * j + lrow;
            #pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int r0 = 32 * (wave >> 1) + 8 * v4 + 4 * khalf;
                float v[4];
                v[0] = fmaf(b, bf_lo(av[j][v4].x), c * acc[j][4 * v4 + 0]);
                v[1] = fmaf(b, bf_hi(av[j][v4].x), c * acc[j][4 * v4 + 1]);
                v[2] = fmaf(b, bf_lo(av[j][v4].y), c * acc[j][4 * v4 + 2]);
                v[3] = fmaf(b, bf_hi(av[j][v4].y), c * acc[j][4 * v4 + 3]);
                #pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (r0 + e == col) v[e] += a;
                uint2 o;
                o.x = pack2(v[0], v[1]);
                o.y = pack2(v[2], v[3]);
                *reinterpret_cast<uint2*>(Ar + loff(col, r0, kARowBytes)) = o;
            }
        }
        __syncthreads();

        // ---- X' = s B' X, one 32-column strip of X at a time per wave ---------------
        // Output block rows are X columns r (long side), columns are X rows i:
        // acc[ib][v] is X'[32 ib + lane % 32][r0 + 8 (v / 4) + 4 (lane / 32) + v % 4].
        // The X operand is read with the transposing LDS read: lane 16 g + t of
        // group g addresses X row k0 + t / 4, columns 4 (t % 4) .. + 3 of the
        // group's 16 columns and receives 4 consecutive k of column t.
        const int tr_g = lane >> 4, tr_t = lane & 15;
        for (int strip = wave; strip < n / 32; strip += kWaves) {
            const int rb = 32 * strip;
            floatx16 bx[4];
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib)
                #pragma unroll
                for (int v = 0; v < 16; ++v) bx[ib][v] = 0.f;
            // fragments of k-step k: X (transposing reads) and the four B' rows
            auto frag = [&](int k, bf16x8& fa, bf16x8 (&fb)[4]) {
                shortx4 h[2];
                #pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int row = k + 8 * (tr_g >> 1) + 4 * t + (tr_t >> 2);
                    const int col = rb + 16 * (tr_g & 1) + 4 * (tr_t & 3);
                    h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_shortx4*)((__attribute__((address_space(3))) char*)X + loff(row, col, xrow)));
                }
                fa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) fb[ib] = ld8(Ar, loff(32 * ib + lrow, k + 8 * khalf, kARowBytes));
            };
            bf16x8 fa, fb[4];
            frag(0, fa, fb);
            #pragma unroll
            for (int k = 16; k <= kM; k += 16) {
                bf16x8 na, nb[4];
                if (k < kM) frag(k, na, nb);
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) bx[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb[ib], bx[ib], 0, 0, 0);
                if (k < kM) {
                    fa = na;
                    #pragma unroll
                    for (int ib = 0; ib < 4; ++ib) fb[ib] = nb[ib];
                }
            }
            // this wave alone reads and writes columns rb .. rb + 31 of X
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const int i = 32 * ib + lrow;
                #pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int r0 = rb + 8 * v4 + 4 * khalf;
                    uint2 o;
                    o.x = pack2(sc * bx[ib][4 * v4 + 0], sc * bx[ib][4 * v4 + 1]);
                    o.y = pack2(sc * bx[ib][4 * v4 + 2], sc * bx[ib][4 * v4 + 3]);
                    *reinterpret_cast<uint2*>(X + loff(i, r0, xrow)) = o;
                }
            }
        }
    }
    __syncthreads();

    if (rec.fused) {
        const bool tall = rec.transposed != 0, vec = (rec.cols & 7) == 0;
#define DMUON_WRITE(DT)                                                          \
        do {                                                                     \
            if (tall) {                                                          \
                if (vec) write_param<DT, true, true>(X, xrow, n, rec, args, tid);   \
                else write_param<DT, true, false>(X, xrow, n, rec, args, tid);      \
            } else {                                                             \
                if (vec) write_param<DT, false, true>(X, xrow, n, rec, args, tid);  \
                else write_param<DT, false, false>(X, xrow, n, rec, args, tid);     \
            }                                                                    \
        } while (0)
        if (rec.dst_dtype == DMUON_BF16) DMUON_WRITE(uint16_t);
        else DMUON_WRITE(float);
#undef DMUON_WRITE
        return;
    }
    // else the result into the X copy that the apply pass reads
    uint4* xo = reinterpret_cast<uint4*>(args.ws + (rec.final_copy ? rec.x_off1 : rec.x_off0));
    for (int q = tid; q < chunks; q += kThreads) {
        const int r = q / (n / 8), c8 = 8 * (q % (n / 8));
        xo[q] = *reinterpret_cast<const uint4*>(X + loff(r, c8, xrow));
    }
}

}  // namespace

hipError_t launch_resident(const DevMatRec* recs, char* ws, const ResidentStep& st,
                           const std::vector<ResidentBucket>& buckets, hipStream_t stream) {
    ResidentArgs ra{};
    ra.recs = recs;
    ra.ws = ws;
    ra.partials = st.partials;
    ra.eps = st.eps;
    ra.a = st.a;
    ra.b = st.b;
    ra.c = st.c;
    ra.steps = st.steps;
    ra.update = st.update;
    ra.lr = st.lr;
    ra.wd = st.wd;
    auto flush = [&]() -> hipError_t {
        if (ra.nseg == 0) return hipSuccess;
        const int total = ra.seg[ra.nseg - 1].first_block + ra.seg[ra.nseg - 1].count;
        hipLaunchKernelGGL(ns_resident_kernel, dim3(total), dim3(kThreads), 0, stream, ra);
        ra.nseg = 0;
        return hipGetLastError();
    };
    int32_t blocks = 0;
    for (const ResidentBucket& rb : buckets) {
        if (rb.n_pad < kM || rb.n_pad > kMaxN || rb.n_pad % 128 != 0 || rb.count <= 0) return hipErrorInvalidValue;
        if (ra.nseg == kMaxSeg || (int64_t)blocks + rb.count > (int64_t)INT32_MAX) {
            hipError_t e = flush();
            if (e != hipSuccess) return e;
            blocks = 0;
        }
        ResidentSeg& sg = ra.seg[ra.nseg++];
        sg.plan_base = rb.plan_base;
        sg.count = rb.count;
        sg.n_pad = (int32_t)rb.n_pad;
        sg.first_block = blocks;
        blocks += rb.count;
    }
    return flush();
}

}  // namespace dmuon

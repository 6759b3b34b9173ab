// C-ABI entry points of libdmuon_ns that enqueue device work: argument checks,
// the per-call matrix table, and the launch sequence of one step
//   records -> prep (momentum, U, X, norm partials) -> norms
//   -> ns_steps x (Gram, square, prod, BX), each phase a grouped launch per
//      tile class (prod: two, for the Gram-space buckets); the last BX writes
//      the update (or output) of the bf16 matrices it can from its epilogue
//   -> apply (update or output) of the others.
// No device memory is allocated and nothing is synchronised: everything is
// enqueued on the caller's stream.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "dmuon_internal.h"
#include "launch.h"

using namespace dmuon;

namespace {

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A caller buffer's byte range and whether the call writes it.
struct Span {
    uintptr_t lo, hi;
    bool written;
};

// True when no two of the spans overlap where one of them is written.  Read-
// only spans may overlap each other (the same gradient passed twice is
// harmless).  Sorted by start, a span overlaps an earlier one exactly when it
// starts below that one's end, so one sweep suffices.
bool disjoint_where_written(std::vector<Span>& v) {
    std::sort(v.begin(), v.end(), [](const Span& x, const Span& y) { return x.lo < y.lo; });
    uintptr_t end_any = 0, end_written = 0;
    for (const Span& sp : v) {
        if (sp.lo < end_written || (sp.written && sp.lo < end_any)) return false;
        end_any = std::max(end_any, sp.hi);
        if (sp.written) end_written = std::max(end_written, sp.hi);
    }
    return true;
}

size_t dtype_bytes(int32_t dt) { return dt == DMUON_BF16 ? 2 : 4; }

// The matrices' byte ranges for an overlap check: read-only sources, fp32
// momenta (when given) and destinations, and the workspace the plan uses.
bool args_disjoint(const dmuon_plan* plan, const void* const* src, float* const* mom, const void* const* dst,
                   const void* workspace) {
    std::vector<Span> v;
    v.reserve(3 * plan->mats.size() + 1);
    for (size_t i = 0; i < plan->mats.size(); ++i) {
        const MatPlan& mp = plan->mats[i];
        const uintptr_t e = (uintptr_t)(mp.rows * mp.cols);
        auto add = [&](const void* p, size_t esz, bool w) {
            v.push_back({reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + e * esz, w});
        };
        add(src[i], dtype_bytes(mp.grad_dtype), false);
        if (mom) add(mom[i], 4, true);
        add(dst[i], dtype_bytes(mp.param_dtype), true);
    }
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace);
    v.push_back({w0, w0 + plan->workspace_bytes, true});
    return disjoint_where_written(v);
}

struct StepParams {
    const void* const* src;
    float* const* mom;     // nullptr: orthogonalisation
    void* const* dst;
    int update;
    float lr, beta, wd, eps, a, b, c;
    int ns_steps, nesterov;
};

// Checks shared by the step and orthogonalisation entry points (mom ==
// nullptr: orthogonalisation).  Every pointer non-null and 16-byte aligned,
// the workspace large enough and 256-byte aligned, and no written buffer
// (momentum, destination, workspace) overlapping any other buffer of the call.
dmuon_status check_call(const dmuon_plan* plan, const void* const* src, float* const* mom, bool need_mom,
                        const void* const* dst, void* workspace, size_t workspace_bytes) {
    if (plan == nullptr) return DMUON_ERR_INVALID_ARG;
    const size_t count = plan->mats.size();
    if (count == 0) return DMUON_OK;
    if (src == nullptr || dst == nullptr || (need_mom && mom == nullptr)) return DMUON_ERR_INVALID_ARG;
    for (size_t i = 0; i < count; ++i) {
        if (!aligned16(src[i]) || !aligned16(dst[i]) || (need_mom && !aligned16(mom[i])))
            return DMUON_ERR_INVALID_ARG;
    }
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0 ||
        workspace_bytes < plan->workspace_bytes)
        return DMUON_ERR_WORKSPACE;
    try {
        if (!args_disjoint(plan, src, need_mom ? mom : nullptr, dst, workspace)) return DMUON_ERR_INVALID_ARG;
    } catch (...) {
        return DMUON_ERR_ALLOC;
    }
    return DMUON_OK;
}

struct TileClass {
    int path;
    int tile;
};
constexpr TileClass kClasses[] = {{kPathBF16, 256}, {kPathBF16, 128}, {kPathF32, 64}};

// One bucket's product in a grouped launch: operand and output arrays as
// bucket base byte offsets in the workspace.
struct SegSpec {
    const BucketPlan* bp;
    int64_t p_off, q_off, o_off;
    int32_t first_iter;
    int32_t fuse = 0;  // B X closing the last segment (the epilogue writes the fused matrices' dst)
};

// One grouped launch per tile class over the given products of one phase.
hipError_t launch_segs(char* ws, uint32_t* queue, const float* scale, const DevMatRec* recs,
                       const StepParams& sp, int phase, const std::vector<SegSpec>& segs, hipStream_t stream) {
    for (const TileClass& tc : kClasses) {
        GemmArgs ga{};
        ga.ws = ws;
        ga.queue = queue;
        ga.scale = scale;
        ga.a = sp.a;
        ga.b = sp.b;
        ga.c = sp.c;
        ga.recs = recs;
        ga.lr = sp.lr;
        ga.wd = sp.wd;
        ga.update = sp.update;
        ga.phase = phase;
        auto flush = [&]() -> hipError_t {
            if (ga.nseg == 0) return hipSuccess;
            hipError_t e = tc.path == kPathBF16 ? launch_gemm_bf16(tc.tile, ga, stream)
                                                : launch_gemm_f32(ga, stream);
            ga.nseg = 0;
            ga.total_blocks = 0;
            return e;
        };
        for (const SegSpec& ss : segs) {
            const BucketPlan& bp = *ss.bp;
            if (bp.path != tc.path || bp.tile != tc.tile) continue;
            // the kernel's output tile: the bucket's on the bf16 path, the fp32 kernels' own on fp32
            const int64_t ktile = bp.path == kPathF32 ? f32_kernel_tile() : bp.tile;
            const int64_t tm = bp.m_pad / ktile, tn = bp.n_pad / ktile;
            const int64_t blocks = (int64_t)bp.members.size() * (phase == kBX ? tm * tn : tm * (tm + 1) / 2);
            if (ga.nseg == kMaxSeg || (int64_t)ga.total_blocks + blocks > (int64_t)INT32_MAX) {
                hipError_t e = flush();
                if (e != hipSuccess) return e;
            }
            GemmSeg& s = ga.seg[ga.nseg++];
            s.tm = (int32_t)tm;
            s.tn = (int32_t)tn;
            s.tiles_per_mat = phase == kBX ? s.tm * s.tn : s.tm * (s.tm + 1) / 2;
            s.count = (int32_t)bp.members.size();
            s.plan_base = bp.plan_base;
            s.first_iter = ss.first_iter;
            s.xcd_remap = (int32_t)((bp.xcd_mask >> phase) & 1u);
            s.fuse = phase == kBX && bp.path == kPathBF16 ? ss.fuse : 0;
            s.first_block = ga.total_blocks;
            s.m_pad = bp.m_pad;
            s.n_pad = bp.n_pad;
            s.p_off = ss.p_off;
            s.q_off = ss.q_off;
            s.o_off = ss.o_off;
            s.x_stride = bp.m_pad * bp.n_pad * bp.esize;
            s.a_stride = bp.m_pad * bp.m_pad * bp.esize;
            ga.total_blocks += s.count * s.tiles_per_mat;
        }
        hipError_t e = flush();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// A bucket's m x m arrays (bucket base offsets) in their current roles: A_j,
// Q_j, P_j, the next P and the product T = A_j Q_j.  Short-side buckets only
// ever use the first two (A and B); Gram-space buckets rotate the five.
struct Roles {
    int64_t a, q, p, p2, t;
};

// Iterations per segment that this call runs a bucket with.  Along directions
// that X_0 barely spans, P grows like a^j within a segment; beyond 2^64 the
// call runs the bucket on the short side instead.
int32_t seg_len_for(const BucketPlan& bp, const StepParams& sp) {
    if (bp.seg_len <= 1) return 1;
    const double growth = (double)bp.seg_len * std::log2(std::max(1.0, (double)std::fabs(sp.a)));
    return growth <= 64.0 ? bp.seg_len : 1;
}

dmuon_status run_impl(const dmuon_plan* p, const StepParams& sp, void* workspace, hipStream_t stream,
                      void* const* events);

// The enqueue sequence behind every step entry point.  run_impl makes every
// host allocation of the call before its first enqueue, so a failed one
// (the only exceptions it can raise) comes back as ALLOC with nothing
// enqueued, and no exception crosses the ABI.
dmuon_status run(const dmuon_plan* p, const StepParams& sp, void* workspace, hipStream_t stream,
                 void* const* events = nullptr) {
    try {
        return run_impl(p, sp, workspace, stream, events);
    } catch (...) {
        return DMUON_ERR_ALLOC;
    }
}

// events == nullptr: plain run.  Otherwise events[0] is recorded before the
// first launch and events[1 + k] after phase k, phases being: prep (records,
// momentum/cast, norms), then per iteration Gram, square, prod, BX (each
// possibly empty), then apply.
dmuon_status run_impl(const dmuon_plan* p, const StepParams& sp, void* workspace, hipStream_t stream,
                      void* const* events) {
    const int32_t count = (int32_t)p->mats.size();
    if (count == 0) return DMUON_OK;
    int ev = 0;
    auto mark = [&]() -> bool {
        if (events == nullptr) return true;
        return hipEventRecord(static_cast<hipEvent_t>(events[ev++]), stream) == hipSuccess;
    };
    char* ws = static_cast<char*>(workspace);
    DevMatRec* table = reinterpret_cast<DevMatRec*>(ws + p->off_records);
    float* scale = reinterpret_cast<float*>(ws + p->off_scale);
    float* partials = reinterpret_cast<float*>(ws + p->off_partials);
    uint32_t* queue = reinterpret_cast<uint32_t*>(ws + p->off_queue);
    const int steps = sp.ns_steps;
    const size_t nb = p->buckets.size();
    std::vector<int32_t> seg(nb);
    for (size_t b = 0; b < nb; ++b) seg[b] = seg_len_for(p->buckets[b], sp);
    // small short-side buckets whose iterations run in one launch, in LDS
    std::vector<char> resident(nb, 0);
    std::vector<ResidentBucket> resident_list;
    for (size_t b = 0; b < nb; ++b) {
        const BucketPlan& bp = p->buckets[b];
        if (steps > 0 && bp.algo == DMUON_ALGO_SHORT_SIDE && resident_shape(bp.path, bp.m_pad, bp.n_pad)) {
            resident[b] = 1;
            resident_list.push_back({bp.plan_base, (int32_t)bp.members.size(), bp.n_pad});
        }
    }

    // Every host container of the call, sized now: nothing below allocates
    // once the first launch is enqueued.
    std::vector<Roles> roles(nb);
    std::vector<int32_t> xcur(nb, 0);  // X copy holding the current iterate
    std::vector<int32_t> j(nb), lc(nb);
    std::vector<SegSpec> segs;
    segs.reserve(2 * nb);  // a phase takes at most two products per bucket

    if (!mark()) return DMUON_ERR_HIP;
    // per-matrix records, plan order, written into the workspace by small launches
    RecChunk chunk{};
    chunk.table = table;
    chunk.queue = queue;
    int64_t prep_blocks = 0, apply_blocks = 0;
    for (int32_t pi = 0; pi < count; ++pi) {
        const int32_t in = p->order[pi];
        const MatPlan& mp = p->mats[in];
        const BucketPlan& bp = p->buckets[mp.bucket];
        const int64_t xsz = bp.m_pad * bp.n_pad * bp.esize;
        DevMatRec r{};
        r.src = sp.src[in];
        r.mom = sp.mom ? sp.mom[in] : nullptr;
        r.dst = sp.dst[in];
        r.x_off0 = (int64_t)bp.off_x0 + mp.slot * xsz;
        r.x_off1 = (int64_t)bp.off_x1 + mp.slot * xsz;
        r.partial_off = mp.partial_off;
        r.prep_begin = prep_blocks;
        prep_blocks += prep_blocks_of(mp.r_pad, mp.c_pad);
        // the last B X launch writes this update, or the apply pass does
        r.fused = update_fused(bp, mp, steps);
        r.apply_begin = apply_blocks;
        if (!r.fused) apply_blocks += apply_blocks_of(mp.rows, mp.cols);
        r.rows = (int32_t)mp.rows;
        r.cols = (int32_t)mp.cols;
        r.r_pad = (int32_t)mp.r_pad;
        r.c_pad = (int32_t)mp.c_pad;
        r.transposed = mp.transposed;
        r.src_dtype = mp.grad_dtype;
        r.dst_dtype = mp.param_dtype;
        r.path = bp.path;
        r.upd_scale = (float)std::sqrt(std::max(1.0, (double)mp.rows / (double)mp.cols));
        // every segment's closing product moves X into the other copy
        const int32_t L = seg[mp.bucket];
        r.final_copy = ((steps + L - 1) / L) % 2;
        chunk.rec[chunk.n++] = r;
        if (chunk.n == kRecChunk || pi == count - 1) {
            if (launch_write_records(chunk, stream) != hipSuccess) return DMUON_ERR_HIP;
            chunk.first += chunk.n;
            chunk.n = 0;
        }
    }

    PrepArgs pa{};
    pa.recs = table;
    pa.count = count;
    pa.ws = ws;
    pa.partials = partials;
    pa.beta = sp.beta;
    pa.nesterov = sp.nesterov ? 1 : 0;
    pa.has_momentum = sp.mom ? 1 : 0;
    pa.total_blocks = prep_blocks;
    if (launch_prep(pa, stream) != hipSuccess) return DMUON_ERR_HIP;
    // the resident kernel sums its matrices' partials itself; the others read
    // the scale array
    bool need_scale = false;
    for (size_t b = 0; b < nb; ++b) need_scale = need_scale || !resident[b];
    if (need_scale && launch_finalize_norms(table, count, partials, scale, sp.eps, stream) != hipSuccess)
        return DMUON_ERR_HIP;
    if (!mark()) return DMUON_ERR_HIP;
    // the resident buckets' whole iteration (timed with iteration 0's Gram phase)
    if (!resident_list.empty()) {
        ResidentStep rs{partials, sp.eps, sp.a, sp.b, sp.c, steps, sp.update, sp.lr, sp.wd};
        if (launch_resident(table, ws, rs, resident_list, stream) != hipSuccess) return DMUON_ERR_HIP;
    }

    // The iterations as segments of seg[b] iterations per bucket (1: the
    // short side).  Iteration k is position j = k mod L of its segment, whose
    // length Lc is L, or less for the last one.  A segment takes
    //   j = 0:      A = s^2 X X^T from the current X copy (s: first segment only)
    //   every j:    Q_j = a I + b A + c A A
    //   j >= 1:     P_{j+1} = Q_j P_j            (P_1 = Q_0)
    //   j < Lc - 1: T = A Q_j, then A = Q_j T
    //   j = Lc - 1: X' = s P_Lc X into the other X copy
    // so a segment of one iteration is exactly the short-side iteration.
    for (size_t b = 0; b < nb; ++b) {
        const BucketPlan& bp = p->buckets[b];
        roles[b] = Roles{(int64_t)bp.off_a, (int64_t)bp.off_b, (int64_t)bp.off_g[0], (int64_t)bp.off_g[1],
                         (int64_t)bp.off_g[2]};
    }
    auto xoff = [&](size_t b, int copy) {
        return (int64_t)(copy == 0 ? p->buckets[b].off_x0 : p->buckets[b].off_x1);
    };
    auto phase_done = [&](int phase) -> bool {
        const bool ok = launch_segs(ws, queue, scale, table, sp, phase, segs, stream) == hipSuccess;
        segs.clear();
        return ok;
    };
    for (int it = 0; it < steps; ++it) {
        for (size_t b = 0; b < nb; ++b) {
            j[b] = it % seg[b];
            lc[b] = std::min(seg[b], steps - (it - j[b]));
        }
        for (size_t b = 0; b < nb; ++b)
            if (!resident[b] && j[b] == 0)
                segs.push_back({&p->buckets[b], xoff(b, xcur[b]), 0, roles[b].a, it == 0 ? 1 : 0});
        if (!phase_done(kGram) || !mark()) return DMUON_ERR_HIP;

        for (size_t b = 0; b < nb; ++b)
            if (!resident[b]) segs.push_back({&p->buckets[b], roles[b].a, 0, roles[b].q, 0});
        if (!phase_done(kSquare) || !mark()) return DMUON_ERR_HIP;

        for (size_t b = 0; b < nb; ++b) {
            const Roles& r = roles[b];
            if (resident[b]) continue;
            if (j[b] >= 1) segs.push_back({&p->buckets[b], r.q, r.p, r.p2, 0});
            if (j[b] < lc[b] - 1) segs.push_back({&p->buckets[b], r.a, r.q, r.t, 0});
        }
        if (!phase_done(kProd)) return DMUON_ERR_HIP;
        for (size_t b = 0; b < nb; ++b)
            if (!resident[b] && j[b] < lc[b] - 1)
                segs.push_back({&p->buckets[b], roles[b].q, roles[b].t, roles[b].a, 0});
        if (!phase_done(kProd) || !mark()) return DMUON_ERR_HIP;

        for (size_t b = 0; b < nb; ++b) {
            if (resident[b] || j[b] != lc[b] - 1) continue;
            const int64_t pfin = j[b] == 0 ? roles[b].q : roles[b].p2;  // P_Lc
            segs.push_back({&p->buckets[b], xoff(b, xcur[b]), pfin, xoff(b, 1 - xcur[b]), it == j[b] ? 1 : 0,
                            it == steps - 1 ? 1 : 0});
        }
        if (!phase_done(kBX) || !mark()) return DMUON_ERR_HIP;

        for (size_t b = 0; b < nb; ++b) {
            Roles& r = roles[b];
            if (j[b] == lc[b] - 1) {
                xcur[b] = 1 - xcur[b];  // segment closed; its arrays are free again
            } else if (j[b] == 0) {
                std::swap(r.p, r.q);  // P_1 = Q_0; the next Q goes where P's array was
            } else {
                std::swap(r.p, r.p2);
            }
        }
    }

    ApplyArgs aa{};
    aa.recs = table;
    aa.count = count;
    aa.ws = ws;
    aa.scale = scale;
    aa.use_scale = steps == 0 ? 1 : 0;
    aa.update = sp.update;
    aa.lr = sp.lr;
    aa.weight_decay = sp.wd;
    aa.total_blocks = apply_blocks;
    if (launch_apply(aa, stream) != hipSuccess) return DMUON_ERR_HIP;
    if (!mark()) return DMUON_ERR_HIP;
    return DMUON_OK;
}

}  // namespace

extern "C" dmuon_status muon_step_batched(const dmuon_plan* plan, const void* const* grads,
                                          float* const* momenta, void* const* params,
                                          const dmuon_hparams* hp, void* workspace,
                                          size_t workspace_bytes, void* stream) {
    if (plan == nullptr || hp == nullptr || hp->ns_steps < 0) return DMUON_ERR_INVALID_ARG;
    dmuon_status st = check_call(plan, grads, momenta, true, params, workspace, workspace_bytes);
    if (st != DMUON_OK || plan->mats.empty()) return st;
    StepParams sp{grads, momenta, params, 1, hp->lr, hp->beta, hp->weight_decay, hp->eps,
                  hp->a, hp->b, hp->c, hp->ns_steps, hp->nesterov};
    return run(plan, sp, workspace, static_cast<hipStream_t>(stream));
}

extern "C" dmuon_status ns_orthogonalize_batched(const dmuon_plan* plan, const void* const* inputs,
                                                 void* const* outputs, int32_t ns_steps, float a,
                                                 float b, float c, float eps, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
    if (plan == nullptr || ns_steps < 0) return DMUON_ERR_INVALID_ARG;
    dmuon_status st = check_call(plan, inputs, nullptr, false, outputs, workspace, workspace_bytes);
    if (st != DMUON_OK || plan->mats.empty()) return st;
    StepParams sp{inputs, nullptr, outputs, 0, 0.f, 0.f, 0.f, eps, a, b, c, ns_steps, 0};
    return run(plan, sp, workspace, static_cast<hipStream_t>(stream));
}

extern "C" int32_t muon_step_event_count(int32_t ns_steps) {
    return ns_steps < 0 || ns_steps > (INT32_MAX - 3) / 4 ? -1 : 3 + 4 * ns_steps;
}

extern "C" dmuon_status muon_step_batched_profiled(const dmuon_plan* plan, const void* const* grads,
                                                   float* const* momenta, void* const* params,
                                                   const dmuon_hparams* hp, void* workspace,
                                                   size_t workspace_bytes, void* stream,
                                                   void* const* events, int32_t num_events) {
    if (plan == nullptr || hp == nullptr || hp->ns_steps < 0 || events == nullptr ||
        muon_step_event_count(hp->ns_steps) < 0 || num_events < muon_step_event_count(hp->ns_steps))
        return DMUON_ERR_INVALID_ARG;
    for (int32_t i = 0; i < num_events; ++i)
        if (events[i] == nullptr) return DMUON_ERR_INVALID_ARG;
    dmuon_status st = check_call(plan, grads, momenta, true, params, workspace, workspace_bytes);
    if (st != DMUON_OK || plan->mats.empty()) return st;
    StepParams sp{grads, momenta, params, 1, hp->lr, hp->beta, hp->weight_decay, hp->eps,
                  hp->a, hp->b, hp->c, hp->ns_steps, hp->nesterov};
    return run(plan, sp, workspace, static_cast<hipStream_t>(stream), events);
}

extern "C" dmuon_status dmuon_events_create(int32_t n, void** events) {
    if (n < 0 || (n > 0 && events == nullptr)) return DMUON_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) {
            for (int32_t j = 0; j < i; ++j) (void)hipEventDestroy(static_cast<hipEvent_t>(events[j]));
            return DMUON_ERR_HIP;
        }
        events[i] = e;
    }
    return DMUON_OK;
}

extern "C" dmuon_status dmuon_events_elapsed_ms(void* start, void* stop, float* ms) {
    if (start == nullptr || stop == nullptr || ms == nullptr) return DMUON_ERR_INVALID_ARG;
    if (hipEventSynchronize(static_cast<hipEvent_t>(stop)) != hipSuccess) return DMUON_ERR_HIP;
    if (hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) != hipSuccess)
        return DMUON_ERR_HIP;
    return DMUON_OK;
}

extern "C" dmuon_status dmuon_events_destroy(int32_t n, void** events) {
    if (n < 0 || (n > 0 && events == nullptr)) return DMUON_ERR_INVALID_ARG;
    dmuon_status st = DMUON_OK;
    for (int32_t i = 0; i < n; ++i)
        if (events[i] != nullptr && hipEventDestroy(static_cast<hipEvent_t>(events[i])) != hipSuccess)
            st = DMUON_ERR_HIP;
    return st;
}

extern "C" dmuon_status adamw_step_batched(int32_t count, const int64_t* numels, const int32_t* param_dtypes,
                                           const int32_t* grad_dtypes, void* const* params,
                                           const void* const* grads, float* const* exp_avgs,
                                           float* const* exp_avg_sqs, const dmuon_adamw_hparams* hp,
                                           void* stream) {
    if (count < 0 || hp == nullptr) return DMUON_ERR_INVALID_ARG;
    if (hp->step < 1 || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) ||
        !(hp->eps > 0.0) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
        return DMUON_ERR_INVALID_ARG;
    if (count == 0) return DMUON_OK;
    if (numels == nullptr || param_dtypes == nullptr || grad_dtypes == nullptr || params == nullptr ||
        grads == nullptr || exp_avgs == nullptr || exp_avg_sqs == nullptr)
        return DMUON_ERR_INVALID_ARG;
    for (int32_t i = 0; i < count; ++i) {
        if (numels[i] < 0) return DMUON_ERR_INVALID_ARG;
        const int32_t pd = param_dtypes[i], gd = grad_dtypes[i];
        if ((pd != DMUON_F32 && pd != DMUON_BF16) || (gd != DMUON_F32 && gd != DMUON_BF16))
            return DMUON_ERR_INVALID_ARG;
        if (numels[i] == 0) continue;
        if (!aligned16(params[i]) || !aligned16(grads[i]) || !aligned16(exp_avgs[i]) || !aligned16(exp_avg_sqs[i]))
            return DMUON_ERR_INVALID_ARG;
    }
    // no written buffer (parameter, moments) may overlap another buffer of the call
    try {
        std::vector<Span> v;
        v.reserve(4 * (size_t)count);
        for (int32_t i = 0; i < count; ++i) {
            if (numels[i] == 0) continue;
            const uintptr_t n = (uintptr_t)numels[i];
            auto add = [&](const void* q, size_t esz, bool w) {
                v.push_back({reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + n * esz, w});
            };
            add(params[i], dtype_bytes(param_dtypes[i]), true);
            add(grads[i], dtype_bytes(grad_dtypes[i]), false);
            add(exp_avgs[i], 4, true);
            add(exp_avg_sqs[i], 4, true);
        }
        if (!disjoint_where_written(v)) return DMUON_ERR_INVALID_ARG;
    } catch (...) {
        return DMUON_ERR_ALLOC;
    }
    // every launch's block count fits the grid, checked before the first one
    // is enqueued (the launches below group the tensors the same way)
    {
        int32_t i = 0;
        while (i < count) {
            int32_t n = 0;
            int64_t blocks = 0;
            for (; i < count && n < kAdamChunk; ++i) {
                if (numels[i] == 0) continue;
                ++n;
                blocks += (numels[i] + kAdamBlock - 1) / kAdamBlock;
            }
            if (blocks > (int64_t)0x7fffffff) return DMUON_ERR_UNSUPPORTED;
        }
    }
    // bias corrections in double on the host, handed to the kernel in fp32
    const double t = (double)hp->step;
    const double bc1 = 1.0 - std::pow(hp->beta1, t), bc2 = 1.0 - std::pow(hp->beta2, t);
    AdamArgs a{};
    a.decay = (float)(1.0 - hp->lr * hp->weight_decay);
    a.beta1 = (float)hp->beta1;
    a.one_minus_beta1 = (float)(1.0 - hp->beta1);
    a.beta2 = (float)hp->beta2;
    a.one_minus_beta2 = (float)(1.0 - hp->beta2);
    a.step_size = (float)(hp->lr / bc1);
    a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    a.eps = (float)hp->eps;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t i = 0;
    while (i < count) {
        a.count = 0;
        a.total_blocks = 0;
        for (; i < count && a.count < kAdamChunk; ++i) {
            if (numels[i] == 0) continue;
            AdamRec& r = a.rec[a.count++];
            r.p = params[i];
            r.g = grads[i];
            r.m = exp_avgs[i];
            r.v = exp_avg_sqs[i];
            r.n = numels[i];
            r.block_begin = a.total_blocks;
            r.p_dtype = param_dtypes[i];
            r.g_dtype = grad_dtypes[i];
            a.total_blocks += (numels[i] + kAdamBlock - 1) / kAdamBlock;
        }
        if (launch_adamw(a, s) != hipSuccess) return DMUON_ERR_HIP;
    }
    return DMUON_OK;
}

// ---- the step without any allocation ---------------------------------------------
// For callers that cannot allocate device memory: the workspace is this
// file-scope device array, one copy per GPU, held from the library's load on
// that GPU until the process ends.  Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the symbol); it uses the
// device address hipGetSymbolAddress gives for the current GPU, looked up once
// per GPU on the entry point's first call there.  Every call on a GPU shares
// that GPU's array: calls on one GPU that overlap in time race on it.  No part
// of it needs to start at zero (every kernel writes what it later reads).
static __device__ __align__(256) char scratch[DMUON_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // per device, null until looked up

dmuon_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DMUON_ERR_HIP;
    if (dev >= kMaxScratchDevices) return DMUON_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return DMUON_ERR_HIP;
        if ((reinterpret_cast<uintptr_t>(ptr) & (kAlign - 1)) != 0) return DMUON_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DMUON_OK;
}

}  // namespace

extern "C" dmuon_status muon_step_batched_noalloc(const dmuon_plan* plan, const void* const* grads,
                                                  float* const* momenta, void* const* params,
                                                  const dmuon_hparams* hp, void* stream) {
    if (plan == nullptr || hp == nullptr || hp->ns_steps < 0) return DMUON_ERR_INVALID_ARG;
    if (plan->mats.empty()) return DMUON_OK;
    if (plan->workspace_bytes > (size_t)DMUON_NOALLOC_SCRATCH_BYTES) return DMUON_ERR_WORKSPACE;
    void* ws = nullptr;
    try {
        const dmuon_status st = scratch_of_current_device(&ws);
        if (st != DMUON_OK) return st;
    } catch (...) {  // the lock
        return DMUON_ERR_HIP;
    }
    dmuon_status st = check_call(plan, grads, momenta, true, params, ws, DMUON_NOALLOC_SCRATCH_BYTES);
    if (st != DMUON_OK) return st;
    StepParams sp{grads, momenta, params, 1, hp->lr, hp->beta, hp->weight_decay, hp->eps,
                  hp->a, hp->b, hp->c, hp->ns_steps, hp->nesterov};
    return run(plan, sp, ws, static_cast<hipStream_t>(stream));
}

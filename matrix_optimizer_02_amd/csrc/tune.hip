// Per-shape autotuning: time candidate configurations of every bucket on the
// device and keep the fastest as a tuning entry (dmuon_tune_entry), which
// muon_plan_ex then applies.
//
// Page basis: the execution stack autotunes kernel configurations for each
// matrix shape and caches the result, and balances work by per-shape costs
// measured at start-up (DMuon explainer on gist.science, sections 2.3 and
// 2.4; section 4 credits autotuning and batching with 16% of the speed-up).
// Here the candidates are what this library can vary per bucket: the output
// tile, the XCD order of the tile launches and the form of the recurrence.
//
// Host code only: each trial is an ordinary ns_orthogonalize_batched call on a
// plan holding one bucket (or, for the final check of the forms, the whole
// batch), timed with HIP events on the caller's stream.
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "dmuon_internal.h"

using namespace dmuon;

namespace {

struct Candidate {
    int32_t tile, algo;
    uint32_t xcd;
};

dmuon_plan_opts base_opts(const dmuon_plan_opts* opts) {
    dmuon_plan_opts o{};
    if (opts) o = *opts;
    o.tuned = nullptr;
    o.tuned_count = 0;
    return o;
}

// Candidates for bucket bp of a plan built with options o.
std::vector<Candidate> candidates(const BucketPlan& bp, const dmuon_plan_opts& o) {
    std::vector<Candidate> out;
    if (bp.path != kPathBF16) {
        out.push_back({bp.tile, DMUON_ALGO_SHORT_SIDE, kDefaultXcdMask});
        return out;
    }
    // a resident bucket has nothing to vary: one workgroup per matrix, in LDS
    if (bp.algo == DMUON_ALGO_SHORT_SIDE && resident_shape(bp.path, bp.m_pad, bp.n_pad)) {
        out.push_back({bp.tile, DMUON_ALGO_SHORT_SIDE, kDefaultXcdMask});
        return out;
    }
    std::vector<int32_t> tiles;
    if (bp.m_pad % 256 == 0 && bp.n_pad % 256 == 0) tiles.push_back(256);
    tiles.push_back(128);
    // the planner's own choice bounds the forms: a forced form stays, and the
    // automatic rule's accuracy guard decides whether the Gram space is tried
    std::vector<int32_t> algos;
    if (o.algo == DMUON_ALGO_GRAM_SPACE) {
        algos.push_back(DMUON_ALGO_GRAM_SPACE);
    } else {
        algos.push_back(DMUON_ALGO_SHORT_SIDE);
        if (bp.algo == DMUON_ALGO_GRAM_SPACE) algos.push_back(DMUON_ALGO_GRAM_SPACE);
    }
    for (int32_t t : tiles)
        for (int32_t a : algos)
            for (uint32_t x : {0u, kDefaultXcdMask, kAllPhasesMask}) out.push_back({t, a, x});
    return out;
}

dmuon_tune_entry entry_for(const BucketPlan& bp, const Candidate& c) {
    dmuon_tune_entry e{};
    e.path = bp.path;
    e.tile = c.tile;
    e.padded_m = bp.m_pad;
    e.padded_n = bp.n_pad;
    e.algo = c.algo;
    e.gram_restart = 0;
    e.xcd_remap = c.xcd;
    return e;
}

struct PlanHolder {
    dmuon_plan* p = nullptr;
    ~PlanHolder() { muon_plan_destroy(p); }
};

struct EventPair {
    hipEvent_t e[2] = {nullptr, nullptr};
    ~EventPair() {
        for (hipEvent_t x : e)
            if (x) (void)hipEventDestroy(x);
    }
};

// The arguments every timed trial shares.
struct Trial {
    int32_t ns_steps;
    float a, b, c;
    int32_t reps;
    void* workspace;
    size_t workspace_bytes;
    hipStream_t stream;
    EventPair* ev;
};

// Milliseconds per ns_orthogonalize_batched call of the plan built from descs
// with options o and the given entries: one untimed call, then t.reps timed.
dmuon_status time_plan(const Trial& t, const dmuon_matrix_desc* descs, int32_t count, const void* const* inputs,
                       void* const* outputs, const dmuon_plan_opts& o, const dmuon_tune_entry* entries,
                       int32_t n_entries, double* ms_per_call) {
    dmuon_plan_opts oc = o;
    oc.tuned = entries;
    oc.tuned_count = n_entries;
    PlanHolder plan;
    dmuon_status st = muon_plan_ex(descs, count, &oc, &plan.p);
    if (st != DMUON_OK) return st;
    const float eps = 1e-7f;
    auto call = [&]() {
        return ns_orthogonalize_batched(plan.p, inputs, outputs, t.ns_steps, t.a, t.b, t.c, eps, t.workspace,
                                        t.workspace_bytes, t.stream);
    };
    if ((st = call()) != DMUON_OK) return st;  // warm-up
    if (hipEventRecord(t.ev->e[0], t.stream) != hipSuccess) return DMUON_ERR_HIP;
    for (int32_t r = 0; r < t.reps; ++r)
        if ((st = call()) != DMUON_OK) return st;
    float ms = 0.f;
    if (hipEventRecord(t.ev->e[1], t.stream) != hipSuccess || hipEventSynchronize(t.ev->e[1]) != hipSuccess ||
        hipEventElapsedTime(&ms, t.ev->e[0], t.ev->e[1]) != hipSuccess)
        return DMUON_ERR_HIP;
    *ms_per_call = (double)ms / t.reps;
    return DMUON_OK;
}

}  // namespace

extern "C" dmuon_status muon_autotune_workspace_bytes(const dmuon_matrix_desc* descs, int32_t count,
                                                      const dmuon_plan_opts* opts, size_t* bytes) {
    if (bytes == nullptr) return DMUON_ERR_INVALID_ARG;
    const dmuon_plan_opts o = base_opts(opts);
    PlanHolder base;
    dmuon_status st = muon_plan_ex(descs, count, &o, &base.p);
    if (st != DMUON_OK) return st;
    size_t need = base.p->workspace_bytes;
    try {
        // per bucket, the candidate with the largest workspace: a whole-batch
        // plan of those bounds every combination (a bucket's padded dims are
        // fixed, so its share of the workspace depends on its form alone)
        std::vector<dmuon_tune_entry> largest;
        for (const BucketPlan& bp : base.p->buckets) {
            std::vector<dmuon_matrix_desc> sub;
            for (int32_t i : bp.members) sub.push_back(descs[i]);
            size_t largest_bytes = 0;
            dmuon_tune_entry largest_entry{};
            for (const Candidate& c : candidates(bp, o)) {
                const dmuon_tune_entry e = entry_for(bp, c);
                dmuon_plan_opts oc = o;
                oc.tuned = &e;
                oc.tuned_count = 1;
                PlanHolder trial;
                st = muon_plan_ex(sub.data(), (int32_t)sub.size(), &oc, &trial.p);
                if (st != DMUON_OK) return st;
                need = std::max(need, trial.p->workspace_bytes);
                if (trial.p->workspace_bytes >= largest_bytes) {
                    largest_bytes = trial.p->workspace_bytes;
                    largest_entry = e;
                }
            }
            largest.push_back(largest_entry);
        }
        if (!largest.empty()) {
            dmuon_plan_opts oc = o;
            oc.tuned = largest.data();
            oc.tuned_count = (int32_t)largest.size();
            PlanHolder whole;
            st = muon_plan_ex(descs, count, &oc, &whole.p);
            if (st != DMUON_OK) return st;
            need = std::max(need, whole.p->workspace_bytes);
        }
    } catch (const std::bad_alloc&) {
        return DMUON_ERR_ALLOC;
    }
    *bytes = need;
    return DMUON_OK;
}

extern "C" dmuon_status muon_autotune(const dmuon_matrix_desc* descs, int32_t count, const dmuon_plan_opts* opts,
                                      const void* const* inputs, void* const* outputs, int32_t ns_steps, float a,
                                      float b, float c, int32_t reps, void* workspace, size_t workspace_bytes,
                                      void* stream, dmuon_tune_entry* out, int32_t out_capacity,
                                      int32_t* out_count) {
    if (out_count == nullptr || reps < 1 || ns_steps < 0 || (count > 0 && (inputs == nullptr || outputs == nullptr)))
        return DMUON_ERR_INVALID_ARG;
    *out_count = 0;
    const dmuon_plan_opts o = base_opts(opts);
    PlanHolder base;
    dmuon_status st = muon_plan_ex(descs, count, &o, &base.p);
    if (st != DMUON_OK) return st;
    const int32_t nb = (int32_t)base.p->buckets.size();
    if (nb > 0 && (out == nullptr || out_capacity < nb)) return DMUON_ERR_INVALID_ARG;
    size_t need = 0;
    st = muon_autotune_workspace_bytes(descs, count, opts, &need);
    if (st != DMUON_OK) return st;
    if (nb > 0 && (workspace == nullptr || workspace_bytes < need)) return DMUON_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    EventPair ev;
    if (nb > 0 && (hipEventCreate(&ev.e[0]) != hipSuccess || hipEventCreate(&ev.e[1]) != hipSuccess))
        return DMUON_ERR_HIP;
    const Trial t{ns_steps, a, b, c, reps, workspace, workspace_bytes, s, &ev};
    try {
        std::vector<dmuon_tune_entry> best_short(nb);
        std::vector<char> has_short(nb, 0);
        for (int32_t bi = 0; bi < nb; ++bi) {
            const BucketPlan& bp = base.p->buckets[bi];
            std::vector<dmuon_matrix_desc> sub;
            std::vector<const void*> in;
            std::vector<void*> outp;
            for (int32_t i : bp.members) {
                sub.push_back(descs[i]);
                in.push_back(inputs[i]);
                outp.push_back(outputs[i]);
            }
            const double per_matrix = 1.0 / (double)bp.members.size();
            double best_ms = -1.0, short_ms = -1.0;
            dmuon_tune_entry best{};
            for (const Candidate& cand : candidates(bp, o)) {
                dmuon_tune_entry e = entry_for(bp, cand);
                double ms = 0.0;
                st = time_plan(t, sub.data(), (int32_t)sub.size(), in.data(), outp.data(), o, &e, 1, &ms);
                if (st != DMUON_OK) return st;
                e.cost_ms_per_matrix = ms * per_matrix;
                if (best_ms < 0.0 || ms < best_ms) {
                    best_ms = ms;
                    best = e;
                }
                if (cand.algo == DMUON_ALGO_SHORT_SIDE && (short_ms < 0.0 || ms < short_ms)) {
                    short_ms = ms;
                    best_short[bi] = e;
                    has_short[bi] = 1;
                }
            }
            out[bi] = best;
        }
        // The Gram-space buckets of a batch add product launches that the other
        // buckets do not have; with small matrices their latency can outweigh
        // what the Gram space saves, which no bucket timed alone shows.  So the
        // whole batch is timed with the chosen entries and with every
        // Gram-space entry replaced by its bucket's fastest short-side one, and
        // the faster set is kept.
        std::vector<dmuon_tune_entry> alt(out, out + nb);
        bool differs = false;
        for (int32_t bi = 0; bi < nb; ++bi)
            if (out[bi].algo == DMUON_ALGO_GRAM_SPACE && has_short[bi]) {
                alt[bi] = best_short[bi];
                differs = true;
            }
        if (differs) {
            double chosen_ms = 0.0, alt_ms = 0.0;
            if ((st = time_plan(t, descs, count, inputs, outputs, o, out, nb, &chosen_ms)) != DMUON_OK ||
                (st = time_plan(t, descs, count, inputs, outputs, o, alt.data(), nb, &alt_ms)) != DMUON_OK)
                return st;
            if (alt_ms < chosen_ms) std::copy(alt.begin(), alt.end(), out);
        }
    } catch (const std::bad_alloc&) {
        return DMUON_ERR_ALLOC;
    }
    *out_count = nb;
    return DMUON_OK;
}

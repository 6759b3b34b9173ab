// Batch planner: buckets matrices of similar shape, pads them to the tile
// granularity, orders the work by computational cost and lays out the
// workspace.  Host-only C++, no device work.
//
// Page basis: matrices with similar shapes are batched and their
// Newton-Schulz recurrence runs jointly, amortising kernel dispatch over many
// small matrices (DMuon explainer on gist.science, second section 2.1,
// "Batching"; section 4 credits autotuning and batching with 16% of the
// speed-up); work is balanced by computational cost (DMuon abstract).  The
// cost of one iteration on an m x n matrix (m <= n) is taken as
// 4 m^2 n + 2 m^3: the products X X^T, A A and B X.
//
// Each bf16 bucket of padded short side >= 1024 whose matrices all have a long
// side of at least three times the short one runs, by default, the Gram-space
// form of the recurrence (DMuon explainer on gist.science, second section 2.1
// Efficiente Gram Newton-Schulz Iteratie): most of its products are m x m;
// with the default restart every 3 iterations, 5 iterations cost
// 6 m^2 n + 14 m^3 instead of 15 m^2 n + 5 m^3 (9 m^2 n + 11 m^3 on buckets of
// padded short side 1024, which restart every 2 iterations).
// The bucket ordering keeps the cost above.
#include <algorithm>
#include <climits>
#include <map>
#include <new>
#include <tuple>

#include "dmuon_internal.h"

using namespace dmuon;

namespace {

int64_t ceil_to(int64_t x, int64_t g) { return (x + g - 1) / g * g; }

int64_t dense_cost(int64_t m, int64_t n) { return 4 * m * m * n + 2 * m * m * m; }

int32_t tile_granularity(int32_t path, int64_t m) {
    if (path == kPathF32) return 64;
    return m <= 128 ? 128 : 256;
}

bool valid_dtype(int32_t d) { return d == DMUON_F32 || d == DMUON_BF16; }

struct InvalidEntry {};  // a tuned entry that applies to a bucket but cannot run it
struct TooLarge {};      // a bucket whose launch would exceed 32-bit block ids

}  // namespace

extern "C" dmuon_status muon_plan_ex(const dmuon_matrix_desc* descs, int32_t count, const dmuon_plan_opts* opts,
                                     dmuon_plan** out) {
    if (out == nullptr || count < 0 || (count > 0 && descs == nullptr)) return DMUON_ERR_INVALID_ARG;
    *out = nullptr;
    const int32_t algo_opt = opts ? opts->algo : DMUON_ALGO_AUTO;
    if (algo_opt != DMUON_ALGO_AUTO && algo_opt != DMUON_ALGO_SHORT_SIDE && algo_opt != DMUON_ALGO_GRAM_SPACE)
        return DMUON_ERR_INVALID_ARG;
    if (opts && opts->gram_restart < 0) return DMUON_ERR_INVALID_ARG;
    // 0: each bucket's default interval (default_gram_restart of its padded short side)
    const int32_t restart_opt = opts ? opts->gram_restart : 0;
    const int32_t ntuned = opts ? opts->tuned_count : 0;
    if (ntuned < 0 || (ntuned > 0 && opts->tuned == nullptr)) return DMUON_ERR_INVALID_ARG;
    for (int32_t i = 0; i < count; ++i) {
        const dmuon_matrix_desc& d = descs[i];
        if (d.rows < 1 || d.cols < 1 || !valid_dtype(d.grad_dtype) || !valid_dtype(d.param_dtype))
            return DMUON_ERR_INVALID_ARG;
        if (d.rows >= (int64_t(1) << 30) || d.cols >= (int64_t(1) << 30)) return DMUON_ERR_UNSUPPORTED;
        // the bf16 kernels address a row stride with 32-bit lane offsets
        if (d.grad_dtype == DMUON_BF16 && std::max(d.rows, d.cols) > kMaxBf16Side) return DMUON_ERR_UNSUPPORTED;
    }
    dmuon_plan* p = new (std::nothrow) dmuon_plan();
    if (p == nullptr) return DMUON_ERR_ALLOC;
    try {
        p->mats.resize(count);
        // bucket key -> bucket under construction (first-appearance index kept)
        std::map<std::tuple<int32_t, int64_t, int64_t>, int32_t> key_to_tmp;
        std::vector<BucketPlan> tmp;
        for (int32_t i = 0; i < count; ++i) {
            const dmuon_matrix_desc& d = descs[i];
            MatPlan& mp = p->mats[i];
            mp.rows = d.rows;
            mp.cols = d.cols;
            mp.grad_dtype = d.grad_dtype;
            mp.param_dtype = d.param_dtype;
            mp.m = std::min(d.rows, d.cols);
            mp.n = std::max(d.rows, d.cols);
            mp.transposed = d.rows > d.cols ? 1 : 0;
            mp.cost = dense_cost(mp.m, mp.n);
            const int32_t path = d.grad_dtype;  // the gradient dtype selects the path
            const int32_t g = tile_granularity(path, mp.m);
            mp.m_pad = ceil_to(mp.m, g);
            mp.n_pad = ceil_to(mp.n, g);
            mp.r_pad = mp.transposed ? mp.n_pad : mp.m_pad;
            mp.c_pad = mp.transposed ? mp.m_pad : mp.n_pad;
            mp.prep_tiles = (mp.r_pad / kPrepTile) * (mp.c_pad / kPrepTile);
            auto key = std::make_tuple(path, mp.m_pad, mp.n_pad);
            auto it = key_to_tmp.find(key);
            int32_t b;
            if (it == key_to_tmp.end()) {
                b = (int32_t)tmp.size();
                key_to_tmp.emplace(key, b);
                BucketPlan bp{};
                bp.path = path;
                bp.tile = g;
                bp.m_pad = mp.m_pad;
                bp.n_pad = mp.n_pad;
                bp.esize = path == kPathBF16 ? 2 : 4;
                tmp.push_back(bp);
            } else {
                b = it->second;
            }
            tmp[b].members.push_back(i);
        }
        // Recurrence form.  The Gram space does less work once the padded long
        // side exceeds the padded short one.  By default it is kept to buckets
        // of padded short side >= 1024 whose every member has n >= 3 m (the
        // accuracy guard of gram_auto_shape / gram_auto_member): a near-square
        // matrix has small singular values, which the Gram space resolves
        // worse, and there it saves little; a small short side's products are
        // latency-bound, so the flops it saves buy little time.  fp32 buckets
        // keep the short side.
        auto auto_gram = [&](const BucketPlan& bp) {
            bool ok = gram_auto_shape(bp.path, bp.m_pad, bp.n_pad);
            for (int32_t i : bp.members) ok = ok && gram_auto_member(p->mats[i].m, p->mats[i].n);
            return ok;
        };
        for (auto& bp : tmp) {
            const int32_t restart = restart_opt > 0 ? restart_opt : default_gram_restart(bp.m_pad);
            bool gram = bp.path == kPathBF16 && algo_opt != DMUON_ALGO_SHORT_SIDE;
            if (gram && algo_opt == DMUON_ALGO_AUTO) gram = auto_gram(bp);
            bp.algo = gram ? DMUON_ALGO_GRAM_SPACE : DMUON_ALGO_SHORT_SIDE;
            bp.seg_len = gram ? restart : 1;
            bp.xcd_mask = kDefaultXcdMask;
            bp.cost_ms = 0.0;
            bp.apply_pass = 0;
            // a tuned entry for this shape overrides the defaults above
            const dmuon_tune_entry* e = nullptr;
            for (int32_t t = 0; t < ntuned && e == nullptr; ++t) {
                const dmuon_tune_entry& c = opts->tuned[t];
                if (c.path == bp.path && c.padded_m == bp.m_pad && c.padded_n == bp.n_pad) e = &c;
            }
            if (e == nullptr) continue;
            const bool tile_ok = e->tile == 0 ||
                                 (bp.path == kPathBF16 ? (e->tile == 128 || e->tile == 256) : e->tile == 64);
            if (!tile_ok || (e->tile != 0 && (bp.m_pad % e->tile != 0 || bp.n_pad % e->tile != 0)) ||
                (e->algo != DMUON_ALGO_AUTO && e->algo != DMUON_ALGO_SHORT_SIDE && e->algo != DMUON_ALGO_GRAM_SPACE) ||
                (e->algo == DMUON_ALGO_GRAM_SPACE && bp.path != kPathBF16) || e->gram_restart < 0 ||
                (e->xcd_remap != DMUON_XCD_REMAP_DEFAULT && (e->xcd_remap & ~kAllPhasesMask) != 0) ||
                (e->apply_pass != 0 && e->apply_pass != 1) || !(e->cost_ms_per_matrix >= 0.0))
                throw InvalidEntry();
            if (e->tile != 0) bp.tile = e->tile;
            // Entries are keyed by padded dims, so one measured on some shapes
            // may meet a bucket whose real members fail the automatic rule's
            // accuracy guard (2047 x 3000 pads like 2000 x 3000): under the
            // automatic option such a bucket keeps the short side.
            const bool entry_gram_refused =
                e->algo == DMUON_ALGO_GRAM_SPACE && algo_opt == DMUON_ALGO_AUTO && !auto_gram(bp);
            if (e->algo != DMUON_ALGO_AUTO && !entry_gram_refused) {
                bp.algo = e->algo;
                bp.seg_len = e->algo == DMUON_ALGO_GRAM_SPACE ? restart : 1;
            }
            if (bp.algo == DMUON_ALGO_GRAM_SPACE && e->gram_restart > 0) bp.seg_len = e->gram_restart;
            if (e->xcd_remap != DMUON_XCD_REMAP_DEFAULT) bp.xcd_mask = e->xcd_remap;
            bp.cost_ms = e->cost_ms_per_matrix;
            bp.apply_pass = e->apply_pass;
        }
        // a bucket's launch must stay within 32-bit block ids (B X has the
        // most tiles per matrix)
        for (const auto& bp : tmp) {
            const int64_t tiles = (bp.m_pad / bp.tile) * (bp.n_pad / bp.tile);
            if ((int64_t)bp.members.size() * tiles > (int64_t)INT32_MAX) throw TooLarge();
        }
        // order buckets by executed cost, descending -- measured, when every
        // bucket has a measured cost, else dense; stable sort keeps first
        // appearance on ties
        bool measured = !tmp.empty();
        for (auto& bp : tmp) {
            bp.exec_cost = (int64_t)bp.members.size() * dense_cost(bp.m_pad, bp.n_pad);
            measured = measured && bp.cost_ms > 0.0;
        }
        std::vector<int32_t> idx(tmp.size());
        for (size_t i = 0; i < idx.size(); ++i) idx[i] = (int32_t)i;
        std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
            if (measured)
                return (double)tmp[x].members.size() * tmp[x].cost_ms > (double)tmp[y].members.size() * tmp[y].cost_ms;
            return tmp[x].exec_cost > tmp[y].exec_cost;
        });
        p->buckets.reserve(tmp.size());
        for (int32_t b : idx) p->buckets.push_back(std::move(tmp[b]));

        // plan order, slots, norm partial offsets
        p->order.reserve(count);
        int64_t partials = 0;
        for (int32_t b = 0; b < (int32_t)p->buckets.size(); ++b) {
            BucketPlan& bp = p->buckets[b];
            bp.plan_base = (int32_t)p->order.size();
            for (int32_t s = 0; s < (int32_t)bp.members.size(); ++s) {
                MatPlan& mp = p->mats[bp.members[s]];
                mp.bucket = b;
                mp.slot = s;
                mp.plan_index = (int32_t)p->order.size();
                p->order.push_back(bp.members[s]);
            }
        }
        for (int32_t pi = 0; pi < count; ++pi) {
            MatPlan& mp = p->mats[p->order[pi]];
            mp.partial_off = partials;
            partials += mp.prep_tiles;
        }
        p->total_prep_tiles = partials;

        // workspace layout
        std::size_t off = 0;
        p->off_records = off;
        off = align_up(off + sizeof(DevMatRec) * (std::size_t)count);
        p->off_scale = off;
        off = align_up(off + sizeof(float) * (std::size_t)count);
        p->off_partials = off;
        off = align_up(off + sizeof(float) * (std::size_t)partials);
        p->off_queue = off;
        off = align_up(off + sizeof(uint32_t) * (std::size_t)kQueueWords);
        for (BucketPlan& bp : p->buckets) {
            const std::size_t cnt = bp.members.size();
            const std::size_t xsz = (std::size_t)bp.m_pad * bp.n_pad * bp.esize;
            const std::size_t asz = (std::size_t)bp.m_pad * bp.m_pad * bp.esize;
            bp.off_x0 = off;  off = align_up(off + cnt * xsz);
            bp.off_x1 = off;  off = align_up(off + cnt * xsz);
            bp.off_a = off;   off = align_up(off + cnt * asz);
            bp.off_b = off;   off = align_up(off + cnt * asz);
            for (int g = 0; g < 3; ++g) {
                bp.off_g[g] = off;
                if (bp.algo == DMUON_ALGO_GRAM_SPACE) off = align_up(off + cnt * asz);
            }
        }
        p->workspace_bytes = count == 0 ? 0 : off;
    } catch (const std::bad_alloc&) {
        delete p;
        return DMUON_ERR_ALLOC;
    } catch (const InvalidEntry&) {
        delete p;
        return DMUON_ERR_INVALID_ARG;
    } catch (const TooLarge&) {
        delete p;
        return DMUON_ERR_UNSUPPORTED;
    }
    *out = p;
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan(const dmuon_matrix_desc* descs, int32_t count, dmuon_plan** out) {
    return muon_plan_ex(descs, count, nullptr, out);
}

extern "C" dmuon_status muon_plan_workspace_bytes(const dmuon_plan* plan, size_t* bytes) {
    if (plan == nullptr || bytes == nullptr) return DMUON_ERR_INVALID_ARG;
    *bytes = plan->workspace_bytes;
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan_info(const dmuon_plan* plan, int32_t* count, int32_t* num_buckets) {
    if (plan == nullptr) return DMUON_ERR_INVALID_ARG;
    if (count) *count = (int32_t)plan->mats.size();
    if (num_buckets) *num_buckets = (int32_t)plan->buckets.size();
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan_query(const dmuon_plan* plan, int32_t idx, int32_t* bucket,
                                        int32_t* slot, int32_t* transposed, int64_t* padded_m,
                                        int64_t* padded_n, int64_t* ns_cost) {
    if (plan == nullptr || idx < 0 || idx >= (int32_t)plan->mats.size()) return DMUON_ERR_INVALID_ARG;
    const MatPlan& mp = plan->mats[idx];
    if (bucket) *bucket = mp.bucket;
    if (slot) *slot = mp.slot;
    if (transposed) *transposed = mp.transposed;
    if (padded_m) *padded_m = mp.m_pad;
    if (padded_n) *padded_n = mp.n_pad;
    if (ns_cost) *ns_cost = mp.cost;
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan_bucket(const dmuon_plan* plan, int32_t bucket, int32_t* path,
                                         int64_t* padded_m, int64_t* padded_n, int32_t* count,
                                         int32_t* tile) {
    if (plan == nullptr || bucket < 0 || bucket >= (int32_t)plan->buckets.size())
        return DMUON_ERR_INVALID_ARG;
    const BucketPlan& bp = plan->buckets[bucket];
    if (path) *path = bp.path;
    if (padded_m) *padded_m = bp.m_pad;
    if (padded_n) *padded_n = bp.n_pad;
    if (count) *count = (int32_t)bp.members.size();
    if (tile) *tile = bp.tile;
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan_bucket_algo(const dmuon_plan* plan, int32_t bucket, int32_t* algo,
                                             int32_t* gram_restart) {
    if (plan == nullptr || bucket < 0 || bucket >= (int32_t)plan->buckets.size()) return DMUON_ERR_INVALID_ARG;
    if (algo) *algo = plan->buckets[bucket].algo;
    if (gram_restart) *gram_restart = plan->buckets[bucket].seg_len;
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan_bucket_resident(const dmuon_plan* plan, int32_t bucket, int32_t* resident) {
    if (plan == nullptr || resident == nullptr || bucket < 0 || bucket >= (int32_t)plan->buckets.size())
        return DMUON_ERR_INVALID_ARG;
    const BucketPlan& bp = plan->buckets[bucket];
    *resident = bp.algo == DMUON_ALGO_SHORT_SIDE && resident_shape(bp.path, bp.m_pad, bp.n_pad) ? 1 : 0;
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan_update_fused(const dmuon_plan* plan, int32_t idx, int32_t ns_steps,
                                              int32_t* fused) {
    if (plan == nullptr || fused == nullptr || idx < 0 || idx >= (int32_t)plan->mats.size() || ns_steps < 0)
        return DMUON_ERR_INVALID_ARG;
    const MatPlan& mp = plan->mats[idx];
    *fused = update_fused(plan->buckets[mp.bucket], mp, ns_steps) ? 1 : 0;
    return DMUON_OK;
}

extern "C" dmuon_status muon_plan_bucket_config(const dmuon_plan* plan, int32_t bucket, dmuon_tune_entry* out) {
    if (plan == nullptr || out == nullptr || bucket < 0 || bucket >= (int32_t)plan->buckets.size())
        return DMUON_ERR_INVALID_ARG;
    const BucketPlan& bp = plan->buckets[bucket];
    dmuon_tune_entry e{};
    e.path = bp.path;
    e.tile = bp.tile;
    e.padded_m = bp.m_pad;
    e.padded_n = bp.n_pad;
    e.algo = bp.algo;
    e.gram_restart = bp.seg_len;
    e.xcd_remap = bp.xcd_mask;
    e.apply_pass = bp.apply_pass;
    e.cost_ms_per_matrix = bp.cost_ms;
    *out = e;
    return DMUON_OK;
}

extern "C" void muon_plan_destroy(dmuon_plan* plan) { delete plan; }

extern "C" const char* dmuon_status_string(dmuon_status status) {
    switch (status) {
        case DMUON_OK: return "ok";
        case DMUON_ERR_INVALID_ARG: return "invalid argument";
        case DMUON_ERR_UNSUPPORTED: return "unsupported";
        case DMUON_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case DMUON_ERR_HIP: return "HIP runtime error";
        case DMUON_ERR_ALLOC: return "host allocation failed";
    }
    return "unknown status";
}

extern "C" const char* dmuon_version(void) { return "0.1.0"; }

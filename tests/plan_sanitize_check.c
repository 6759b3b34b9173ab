/* Plain C99 driver of the planning half of the C ABI, built with the host
 * sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) together with the
 * planner source.  It builds plans for many pseudo-random matrix sets, with
 * every option and with tuned entries (valid and invalid), reads every
 * per-matrix and per-bucket entry back, checks the plan's invariants and
 * releases it.  Any out-of-bounds access, leak, overflow or misaligned access
 * in the planner ends the run with a sanitizer report. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "dmuon_ns.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64 */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

static int fail(const char* what, int a) {
    printf("FAIL %s %d\n", what, a);
    return 1;
}

static int check_plan(const dmuon_plan* plan, const dmuon_matrix_desc* descs, int32_t count) {
    int32_t n = -1, nb = -1;
    size_t ws = 0;
    if (muon_plan_info(plan, &n, &nb) != DMUON_OK || n != count) return fail("info", count);
    if (muon_plan_workspace_bytes(plan, &ws) != DMUON_OK || (count > 0 && ws == 0)) return fail("workspace", count);
    int32_t* seen = (int32_t*)calloc((size_t)(nb > 0 ? nb : 1), sizeof(int32_t));
    if (seen == NULL) return fail("calloc", 0);
    for (int32_t i = 0; i < count; ++i) {
        int32_t b = -1, slot = -1, tr = -1, path = -1, cnt = 0, tile = 0;
        int64_t pm = 0, pn = 0, cost = 0, bm = 0, bn = 0;
        if (muon_plan_query(plan, i, &b, &slot, &tr, &pm, &pn, &cost) != DMUON_OK) return fail("query", i);
        const int64_t m = descs[i].rows < descs[i].cols ? descs[i].rows : descs[i].cols;
        const int64_t nn = descs[i].rows < descs[i].cols ? descs[i].cols : descs[i].rows;
        if (b < 0 || b >= nb || tr != (descs[i].rows > descs[i].cols)) return fail("bucket/transpose", i);
        if (pm < m || pn < nn || cost != 4 * m * m * nn + 2 * m * m * m) return fail("pad/cost", i);
        if (muon_plan_bucket(plan, b, &path, &bm, &bn, &cnt, &tile) != DMUON_OK) return fail("bucket", i);
        if (bm != pm || bn != pn || path != descs[i].grad_dtype || slot < 0 || slot >= cnt) return fail("slot", i);
        if (tile <= 0 || pm % tile != 0 || pn % tile != 0) return fail("tile", i);
        seen[b] += 1;
    }
    for (int32_t b = 0; b < nb; ++b) {
        int32_t cnt = 0, algo = 0, restart = 0, res = -1;
        dmuon_tune_entry e;
        if (muon_plan_bucket(plan, b, NULL, NULL, NULL, &cnt, NULL) != DMUON_OK || cnt != seen[b])
            return fail("bucket count", b);
        if (muon_plan_bucket_algo(plan, b, &algo, &restart) != DMUON_OK || restart < 1) return fail("algo", b);
        if (muon_plan_bucket_resident(plan, b, &res) != DMUON_OK || (res != 0 && res != 1)) return fail("res", b);
        if (muon_plan_bucket_config(plan, b, &e) != DMUON_OK || e.algo != algo) return fail("config", b);
    }
    free(seen);
    return 0;
}

int main(void) {
    enum { kSets = 400, kMaxCount = 24 };
    dmuon_matrix_desc descs[kMaxCount];
    dmuon_tune_entry tuned[8];
    for (int set = 0; set < kSets; ++set) {
        const int32_t count = (int32_t)pick(0, kMaxCount);
        for (int32_t i = 0; i < count; ++i) {
            const int big = pick(0, 9) == 0;
            descs[i].rows = pick(1, big ? 9000 : 700);
            descs[i].cols = pick(1, big ? 9000 : 700);
            descs[i].grad_dtype = (int32_t)pick(0, 1);
            descs[i].param_dtype = (int32_t)pick(0, 1);
        }
        /* tuned entries keyed on shapes of this set, some of them invalid */
        const int32_t ntuned = count > 0 ? (int32_t)pick(0, 8) : 0;
        for (int32_t t = 0; t < ntuned; ++t) {
            const dmuon_matrix_desc* d = &descs[pick(0, count - 1)];
            const int64_t m = d->rows < d->cols ? d->rows : d->cols, n = d->rows < d->cols ? d->cols : d->rows;
            const int64_t g = d->grad_dtype == DMUON_F32 ? 64 : (m <= 128 ? 128 : 256);
            tuned[t].path = d->grad_dtype;
            tuned[t].tile = (int32_t)(pick(0, 3) == 0 ? 0 : (d->grad_dtype == DMUON_F32 ? 64 : (pick(0, 1) ? 128 : 256)));
            tuned[t].padded_m = (m + g - 1) / g * g;
            tuned[t].padded_n = (n + g - 1) / g * g;
            tuned[t].algo = (int32_t)pick(0, 3); /* 3 is invalid */
            tuned[t].gram_restart = (int32_t)pick(-1, 4);
            tuned[t].xcd_remap = pick(0, 5) == 0 ? DMUON_XCD_REMAP_DEFAULT : (uint32_t)pick(0, 31);
            tuned[t].apply_pass = (int32_t)pick(0, 20) == 0 ? 2 : (int32_t)pick(0, 1); /* 2 is invalid */
            tuned[t].cost_ms_per_matrix = (double)pick(0, 100) / 10.0;
        }
        dmuon_plan_opts opts;
        opts.algo = (int32_t)pick(0, 2);
        opts.gram_restart = (int32_t)pick(0, 5);
        opts.tuned = ntuned > 0 ? tuned : NULL;
        opts.tuned_count = ntuned;
        dmuon_plan* plan = NULL;
        const dmuon_status st = muon_plan_ex(descs, count, pick(0, 4) == 0 ? NULL : &opts, &plan);
        if (st == DMUON_OK) {
            if (plan == NULL) return fail("null plan", set);
            if (check_plan(plan, descs, count) != 0) return fail("plan", set);
            muon_plan_destroy(plan);
        } else if (st != DMUON_ERR_INVALID_ARG || plan != NULL) {
            return fail("status", set);
        }
    }
    /* argument errors */
    dmuon_plan* plan = NULL;
    if (muon_plan(NULL, 3, &plan) != DMUON_ERR_INVALID_ARG) return fail("null descs", 0);
    if (muon_plan(descs, -1, &plan) != DMUON_ERR_INVALID_ARG) return fail("negative count", 0);
    descs[0].rows = (int64_t)1 << 30;
    descs[0].cols = 4;
    descs[0].grad_dtype = DMUON_F32;
    if (muon_plan(descs, 1, &plan) != DMUON_ERR_UNSUPPORTED) return fail("huge dim", 0);
    if (muon_plan_query(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL) != DMUON_ERR_INVALID_ARG) return fail("query", 0);
    muon_plan_destroy(NULL);
    printf("OK\n");
    return 0;
}

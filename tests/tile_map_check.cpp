// Host check of the grouped-launch tile maps (tile_map.h): every block of a
// launch maps to exactly one (segment, matrix, tile) and every tile is covered,
// each tile coordinate lies inside its grid, and each XCD's share of a segment
// is one contiguous run whose size differs from the other XCDs' by at most 1.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <tuple>
#include <vector>

#include "tile_map.h"

using namespace dmuon;

static int fail(const char* what, int a, int b) {
    std::printf("FAIL %s %d %d\n", what, a, b);
    return 1;
}

int check_tri(int tm) {
    std::set<std::pair<int, int>> seen;
    const int n = tm * (tm + 1) / 2;
    for (int t = 0; t < n; ++t) {
        int I, J;
        tri_decode_banded(t, tm, I, J);
        if (!(0 <= I && I <= J && J < tm)) return fail("tri range", tm, t);
        if (!seen.insert({I, J}).second) return fail("tri duplicate", tm, t);
    }
    return (int)seen.size() == n ? 0 : fail("tri coverage", tm, (int)seen.size());
}

int check_bx(int tn, int tm) {
    std::set<std::pair<int, int>> seen;
    for (int t = 0; t < tn * tm; ++t) {
        int I, J;
        bx_decode_banded(t, tn, tm, I, J);
        if (!(0 <= I && I < tn && 0 <= J && J < tm)) return fail("bx range", tn * 1000 + tm, t);
        if (!seen.insert({I, J}).second) return fail("bx duplicate", tn * 1000 + tm, t);
    }
    return (int)seen.size() == tn * tm ? 0 : fail("bx coverage", tn, tm);
}

int check_launch(const std::vector<int>& totals, const std::vector<int>& remap) {
    std::vector<int> first(totals.size());
    int sum = 0;
    for (size_t s = 0; s < totals.size(); ++s) {
        first[s] = sum;
        sum += totals[s];
    }
    std::set<std::pair<int, int>> seen;
    // per (segment, xcd): the locals it received, in block order
    std::vector<std::vector<std::vector<int>>> runs(totals.size(), std::vector<std::vector<int>>(kXcds));
    for (int b = 0; b < sum; ++b) {
        int s, local;
        xcd_map(b, (int)totals.size(), [&](int i) { return totals[i]; }, [&](int i) { return first[i]; },
                [&](int i) { return remap[i] != 0; }, s, local);
        // a segment left in the hardware's order maps block b to tile b - first(s)
        if (s >= 0 && s < (int)totals.size() && !remap[s] && local != b - first[s]) return fail("plain order", b, s);
        if (s < 0 || s >= (int)totals.size() || local < 0 || local >= totals[s]) return fail("map range", b, s);
        if (!seen.insert({s, local}).second) return fail("map duplicate", b, s);
        runs[s][b % kXcds].push_back(local);
    }
    if ((int)seen.size() != sum) return fail("map coverage", sum, (int)seen.size());
    for (size_t s = 0; s < totals.size(); ++s) {
        int lo = 1 << 30, hi = 0;
        for (int x = 0; x < kXcds; ++x) {
            const auto& r = runs[s][x];
            const int step = remap[s] ? 1 : kXcds;  // contiguous run, or every 8th tile
            for (size_t i = 1; i < r.size(); ++i)
                if (r[i] != r[i - 1] + step) return fail("run not contiguous", (int)s, x);
            lo = std::min(lo, (int)r.size());
            hi = std::max(hi, (int)r.size());
        }
        if (hi - lo > 1) return fail("unbalanced shares", (int)s, hi - lo);
    }
    return 0;
}

int main() {
    int bad = 0;
    for (int tm = 1; tm <= 80; ++tm) bad |= check_tri(tm);
    for (int tn = 1; tn <= 80; tn += 3)
        for (int tm = 1; tm <= 40; ++tm) bad |= check_bx(tn, tm);
    const std::vector<std::vector<int>> launches = {
        {1}, {7}, {8}, {9}, {136 * 12, 136 * 8, 10 * 8}, {896 * 12, 256 * 8, 64 * 8},
        {3, 5, 7, 11, 13}, {1, 1, 1, 1, 1, 1, 1, 1, 1}, {21 * 56, 1 * 56, 6 * 84}, {105 * 28, 74 * 14 * 84}};
    for (const auto& l : launches) {
        bad |= check_launch(l, std::vector<int>(l.size(), 1));
        bad |= check_launch(l, std::vector<int>(l.size(), 0));
    }
    std::srand(7);
    for (int trial = 0; trial < 400; ++trial) {
        std::vector<int> l(1 + std::rand() % 6), r(l.size());
        for (auto& v : l) v = 1 + std::rand() % 700;
        for (auto& v : r) v = std::rand() % 2;  // mixed orders in one launch
        bad |= check_launch(l, r);
    }
    std::printf(bad ? "FAILED\n" : "OK\n");
    return bad;
}

// Block -> tile maps of the grouped Newton-Schulz launches.  Plain integer
// code, usable from device code and from host-side checks.
#pragma once

#if defined(__HIPCC__)
#define DMUON_HD __host__ __device__ __forceinline__
#else
#define DMUON_HD inline
#endif

namespace dmuon {

constexpr int kXcds = 8;     // XCDs of an MI355X; the hardware deals blocks round-robin
constexpr int kTriBand = 4;  // rows per band of a triangle schedule
constexpr int kBxBand = 8;   // short-side columns per band of the B X schedule

DMUON_HD int imin(int a, int b) { return a < b ? a : b; }

// Triangle tile t (band order) -> (I, J), I <= J, of a tm x tm tile grid.
// Bands of kTriBand rows; inside a band, column by column, rows inner, so a
// run of 32 consecutive tiles spans 4 row panels and ~8 column panels.
DMUON_HD void tri_decode_banded(int t, int tm, int& I, int& J) {
    for (int b0 = 0; b0 < tm; b0 += kTriBand) {
        const int h = imin(kTriBand, tm - b0);
        const int tri = h * (h + 1) / 2;  // columns b0 .. b0+h-1 hold 1 .. h tiles
        const int band_total = tri + (tm - b0 - h) * h;
        if (t >= band_total) {
            t -= band_total;
            continue;
        }
        if (t < tri) {
            int j = 0;
            while (t >= j + 1) {
                t -= j + 1;
                ++j;
            }
            J = b0 + j;
            I = b0 + t;
        } else {
            t -= tri;
            J = b0 + h + t / h;
            I = b0 + t % h;
        }
        return;
    }
    I = J = 0;  // not reached for t in range
}

// B X tile t (band order) -> (I: long-side tile in [0, tn), J: short-side
// tile in [0, tm)).  Bands of kBxBand short-side columns; inside a band, row
// by row, columns inner.
DMUON_HD void bx_decode_banded(int t, int tn, int tm, int& I, int& J) {
    const int band_tiles = kBxBand * tn;
    const int band = t / band_tiles;
    const int r = t - band * band_tiles;
    const int w = imin(kBxBand, tm - band * kBxBand);
    I = r / w;
    J = band * kBxBand + r % w;
}

// Block id -> (segment s, tile index within the segment).  Segment s holds
// total(s) tiles and starts at block first(s) (the running sum).  The
// hardware deals blocks to XCDs round-robin (XCD = id % 8), and segment s's
// tiles are dealt the same way, continuing where segment s - 1 stopped: XCD x
// takes the tiles whose offset rho = (x - first(s)) mod 8 matches, k-th slot
// after k.  With remap(s) each XCD takes its share of the segment as one
// contiguous run of tiles (neighbouring tiles share operand panels in that
// XCD's L2); without it, tile rho + 8 k, which is the plain order
// local = block - first(s).
template <typename Total, typename First, typename Remap>
DMUON_HD void xcd_map(int bid, int nseg, Total total, First first, Remap remap, int& s, int& local) {
    const int x = bid % kXcds;
    int k = bid / kXcds;
    for (s = 0; s < nseg; ++s) {
        const int tot = total(s);
        const int q = tot / kXcds, rem = tot % kXcds;
        const int rho = (x - first(s) % kXcds + kXcds) % kXcds;
        const int share = q + (rho < rem ? 1 : 0);
        if (k < share) {
            local = remap(s) ? rho * q + imin(rho, rem) + k : rho + kXcds * k;
            return;
        }
        k -= share;
    }
    s = nseg - 1;  // not reached for bid < the launch's block count
    local = 0;
}

}  // namespace dmuon

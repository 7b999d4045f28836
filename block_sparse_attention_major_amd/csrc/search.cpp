// Offline dual-window search on the host (Compact Attention page, Fig. 3
// caption: windows shrunk step by step under a recall constraint tau and a
// cost constraint lambda; Fig. 4 caption: from full coverage in every
// temporal-distance group; Fig. 1 caption part (3): two windows per group).
//
// The pages give no formula; the reading implemented here (the header at
// sparse_attn_search_windows states it in full):
//  - tile pair (i, j) weighs w = round(A[i][j] c_i 2^24) (integers, so every
//    sum is exact and independent of order) and costs c_i c_j;
//  - a group's kept offsets (dy, dx) are the union of two origin-anchored
//    rectangles, wide (y, X) and tall (Y, x), -1 <= y <= Y, -1 <= x <= X;
//  - from full coverage, each step applies the admissible single-strip
//    shrink with the least weight lost per cost saved.
// Everything reduces to per-group tables of weight and cost by offset, so a
// step costs O(groups * ny * nx) whatever the number of tiles.
#include "sparse_attn.h"

#include <cmath>
#include <cstdint>
#include <vector>

#include "common.h"

namespace {

struct Region {
    int y, X, Y, x;  // wide window (ry y, rx X), tall window (ry Y, rx x)
    bool covers(int dy, int dx) const { return (dy <= y && dx <= X) || (dy <= Y && dx <= x); }
};

// The five shrink moves of a region; false when the move does not apply.
bool apply_move(const Region &r, int move, Region &out)
{
    out = r;
    switch (move) {
    case 0:  // notch the corner of a rectangle
        if (!(r.y == r.Y && r.x == r.X && r.Y >= 0 && r.X >= 0))
            return false;
        out.y = r.y - 1;
        out.x = r.x - 1;
        return true;
    case 1:
        if (r.y < 0)
            return false;
        out.y = r.y - 1;
        return true;
    case 2:
        if (r.x < 0)
            return false;
        out.x = r.x - 1;
        return true;
    case 3:
        if (r.Y < 0)
            return false;
        out.Y = r.Y - 1;
        out.y = r.y < out.Y ? r.y : out.Y;
        return true;
    case 4:
        if (r.X < 0)
            return false;
        out.X = r.X - 1;
        out.x = r.x < out.X ? r.x : out.X;
        return true;
    }
    return false;
}

struct Candidate {
    int64_t dw, dc;
    int group, move;
};

// Ranking of candidates: least weight lost per cost saved (a move that saves
// no cost loses no weight and comes first), then the larger saved cost, then
// the lower group and move number.
bool ranks_before(const Candidate &a, const Candidate &b)
{
    if (a.dc == 0 || b.dc == 0) {
        if ((a.dc == 0) != (b.dc == 0))
            return a.dc == 0;
    } else {
        const __int128 lhs = (__int128)a.dw * b.dc, rhs = (__int128)b.dw * a.dc;
        if (lhs != rhs)
            return lhs < rhs;
    }
    if (a.dc != b.dc)
        return a.dc > b.dc;
    if (a.group != b.group)
        return a.group < b.group;
    return a.move < b.move;
}

}  // namespace

namespace sa {

// Search of one head.  tiles: coordinates and real counts; A: [nT][nT].
int search_head(const Layout &L, const float *A, const sparse_attn_window_group *gin, int G, double tau,
                double lambda, sparse_attn_window_group *gout, double *recall, double *cost)
{
    const int nT = L.nT, ny = L.ny, nx = L.nx;
    std::vector<int> ta(nT), tb(nT), te(nT);
    std::vector<int64_t> tc(nT);
    for (int t = 0; t < nT; ++t) {
        const TileBox bx = tile_box(L, t);
        ta[t] = bx.a;
        tb[t] = bx.b;
        te[t] = bx.e;
        tc[t] = (int64_t)bx.et * bx.ey * bx.ex;
    }
    // Per group, weight and cost by offset.
    const size_t cells = (size_t)ny * nx;
    std::vector<int64_t> gw((size_t)G * cells, 0), gc((size_t)G * cells, 0);
    int64_t w_total = 0, c_total = 0;
    for (int i = 0; i < nT; ++i) {
        for (int j = 0; j < nT; ++j) {
            const int64_t w =
                (int64_t)std::nearbyint((double)A[(size_t)i * nT + j] * (double)tc[i] * 16777216.0);
            const int64_t c = tc[i] * tc[j];
            w_total += w;
            c_total += c;
            const int da = std::abs(ta[i] - ta[j]);
            const int dy = std::abs(tb[i] - tb[j]), dx = std::abs(te[i] - te[j]);
            for (int g = 0; g < G; ++g) {
                if (da >= gin[g].dt_lo && (gin[g].dt_hi < 0 || da <= gin[g].dt_hi)) {
                    gw[(size_t)g * cells + (size_t)dy * nx + dx] += w;
                    gc[(size_t)g * cells + (size_t)dy * nx + dx] += c;
                    break;  // groups are disjoint
                }
            }
        }
    }
    std::vector<Region> reg(G, Region{ny - 1, nx - 1, ny - 1, nx - 1});
    int64_t kept_w = 0, kept_c = 0;
    for (size_t u = 0; u < gw.size(); ++u) {
        kept_w += gw[u];
        kept_c += gc[u];
    }
    const int64_t need = (int64_t)std::ceil(tau * (double)w_total);
    for (;;) {
        bool found = false;
        Candidate best{};
        Region best_region{};
        for (int g = 0; g < G; ++g) {
            for (int mv = 0; mv < 5; ++mv) {
                Region nr;
                if (!apply_move(reg[g], mv, nr))
                    continue;
                int64_t dw = 0, dc = 0;
                bool any = false;
                for (int dy = 0; dy < ny; ++dy)
                    for (int dx = 0; dx < nx; ++dx)
                        if (reg[g].covers(dy, dx) && !nr.covers(dy, dx)) {
                            any = true;
                            dw += gw[(size_t)g * cells + (size_t)dy * nx + dx];
                            dc += gc[(size_t)g * cells + (size_t)dy * nx + dx];
                        }
                if (!any || kept_w - dw < need)
                    continue;
                if (!std::isinf(lambda) &&
                    !((double)dw * (double)c_total <= lambda * (double)dc * (double)w_total))
                    continue;
                const Candidate cand{dw, dc, g, mv};
                if (!found || ranks_before(cand, best)) {
                    found = true;
                    best = cand;
                    best_region = nr;
                }
            }
        }
        if (!found)
            break;
        reg[best.group] = best_region;
        kept_w -= best.dw;
        kept_c -= best.dc;
    }
    for (int g = 0; g < G; ++g) {
        gout[g] = gin[g];
        gout[g].ry[0] = reg[g].y;
        gout[g].rx[0] = reg[g].X;
        gout[g].ry[1] = reg[g].Y;
        gout[g].rx[1] = reg[g].x;
    }
    *recall = w_total > 0 ? (double)kept_w / (double)w_total : 0.0;
    *cost = c_total > 0 ? (double)kept_c / (double)c_total : 0.0;
    return SPARSE_ATTN_OK;
}

}  // namespace sa

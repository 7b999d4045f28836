// Host-side checks of the library under AddressSanitizer and
// UndefinedBehaviorSanitizer (built and run by tests/test_sanitizers.py on
// the CPU): layout planning, argument validation, the Hilbert sequence, the
// host window search and the status strings, with the kernel launchers
// replaced by stubs that fail (no path exercised here reaches them).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "sparse_attn.h"
#include "common.h"
#include "mix_probe.h"

namespace sa {
hipError_t launch_permute_rows(const Layout &, int, const void *, void *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_permute_tile_columns(const Layout &, const void *, void *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_unpermute_rows(const Layout &, int, const void *, void *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_compile_mask(const Layout &, int, const uint8_t *, const MaskBuffers &, const MaskBuffers &,
                               hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention_mfma(const Layout &, const AttnParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention_rows(const Layout &, const AttnParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention_f32(const Layout &, const AttnParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_select_topk(const Layout &, int, const void *, const void *, const int *, float, float *, float *,
                              uint8_t *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_select_scope(const Layout &, int, const void *, const void *, float, float, int, float *, float *,
                               int *, int *, uint8_t *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_tile_mass(const Layout &, const void *, const void *, float, float *, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_attention_generic(const Layout &, int, const AttnParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mix_probe(int, int, int, int, long long *, float *, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sa

static int g_fail = 0;
#define EXPECT(cond)                                                                   \
    do {                                                                               \
        if (!(cond)) {                                                                 \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
            ++g_fail;                                                                  \
        }                                                                              \
    } while (0)

static sparse_attn_config cfg(int heads, int d, int T, int H, int W, int tt, int th, int tw, int dtype, int order = 0)
{
    sparse_attn_config c{};
    c.heads = heads;
    c.head_dim = d;
    c.grid[0] = T; c.grid[1] = H; c.grid[2] = W;
    c.tile[0] = tt; c.tile[1] = th; c.tile[2] = tw;
    c.dtype = dtype;
    c.softmax_scale = 0.f;
    c.order = order;
    return c;
}

int main()
{
    // Status strings, including unknown codes.
    for (int s = -2; s < 10; ++s)
        EXPECT(sparse_attn_status_string(s) != nullptr);

    // Invalid configurations fail before planning.
    sparse_attn_handle *h = nullptr;
    EXPECT(sparse_attn_create(nullptr, &h) == SPARSE_ATTN_INVALID_ARG);
    const sparse_attn_config bad[] = {
        cfg(0, 128, 4, 8, 8, 1, 4, 4, 1), cfg(1, 96, 4, 8, 8, 1, 4, 4, 1), cfg(1, 128, 4, 8, 8, 2, 8, 16, 1),
        cfg(1, 128, 0, 8, 8, 1, 4, 4, 1), cfg(1, 128, 4, 8, 8, 1, 4, 4, 7), cfg(1, 128, 4, 8, 8, 1, 4, 4, 1, 5),
        cfg(40, 128, 2000, 800, 800, 1, 8, 16, 1)};
    for (const auto &c : bad) {
        h = nullptr;
        EXPECT(sparse_attn_create(&c, &h) != SPARSE_ATTN_OK && h == nullptr);
        EXPECT(std::strlen(sparse_attn_last_error(nullptr)) > 0);
    }
    sparse_attn_destroy(nullptr);

    // Valid configurations: layout, sizes, search and validation paths.
    const sparse_attn_config good[] = {
        cfg(2, 64, 4, 8, 8, 1, 4, 4, 0),          cfg(3, 128, 8, 30, 40, 1, 8, 16, 1),
        cfg(2, 128, 3, 20, 36, 1, 8, 16, 1),      cfg(2, 64, 5, 3, 3, 2, 3, 3, 0),
        cfg(2, 128, 3, 17, 33, 1, 8, 16, 1, 1),   cfg(1, 128, 1, 1, 1, 1, 1, 1, 1),
        cfg(40, 128, 21, 45, 80, 1, 8, 16, 1)};
    std::mt19937 rng(7);
    for (const auto &c : good) {
        h = nullptr;
        EXPECT(sparse_attn_create(&c, &h) == SPARSE_ATTN_OK && h != nullptr);
        if (!h)
            continue;
        sparse_attn_layout_info L{};
        EXPECT(sparse_attn_layout(h, &L) == SPARSE_ATTN_OK);
        EXPECT(sparse_attn_layout(h, nullptr) == SPARSE_ATTN_INVALID_ARG);
        size_t b = 0;
        EXPECT(sparse_attn_mask_bytes(h, 0, &b) == SPARSE_ATTN_OK && b > 0);
        EXPECT(sparse_attn_mask_bytes(h, 17, &b) == SPARSE_ATTN_OK);
        EXPECT(sparse_attn_workspace_bytes(h, &b) == SPARSE_ATTN_OK && b == L.ws_bytes);
        EXPECT(sparse_attn_order_bytes(h, &b) == SPARSE_ATTN_OK);

        // Forward-path validation before any device work.
        alignas(16) static char fake[64];
        void *p = fake;
        EXPECT(sparse_attn_forward(h, nullptr, p, p, p, p, 1 << 20, nullptr) == SPARSE_ATTN_INVALID_ARG);
        EXPECT(sparse_attn_forward(h, fake + 1, p, p, p, p, 1 << 20, nullptr) != SPARSE_ATTN_OK);
        int st = sparse_attn_forward(h, p, p, p, p, p, 0, nullptr);
        EXPECT(st != SPARSE_ATTN_OK);
        EXPECT(sparse_attn_attend(h, p, L.ws_bytes, nullptr) != SPARSE_ATTN_OK);  // no mask yet
        if (2 * L.ws_offset_k > SPARSE_ATTN_NOALLOC_SCRATCH_BYTES && c.order == 0)
            EXPECT(sparse_attn_forward_noalloc(h, p, p, p, p, nullptr) == SPARSE_ATTN_UNSUPPORTED);

        // Malformed masks fail with BAD_MASK before any upload.
        std::vector<sparse_attn_window_group> groups(c.heads * 2);
        std::vector<int32_t> gph(c.heads, 2);
        for (int hh = 0; hh < c.heads; ++hh) {
            groups[2 * hh] = {0, 1, {1, 0}, {0, 1}};
            groups[2 * hh + 1] = {1, -1, {0, -1}, {2, -1}};  // overlaps the first group: invalid
        }
        sparse_attn_mask m{};
        m.kind = SPARSE_ATTN_MASK_DUAL_WINDOW;
        m.groups = groups.data();
        m.groups_per_head = gph.data();
        EXPECT(sparse_attn_set_mask(h, &m, p, size_t(1) << 40, nullptr) == SPARSE_ATTN_BAD_MASK);
        m.kind = 9;
        EXPECT(sparse_attn_set_mask(h, &m, p, size_t(1) << 40, nullptr) != SPARSE_ATTN_OK);

        // The host window search on random masses (rows normalised), for
        // several tau and lambda, with valid and invalid arguments.
        if (L.tiles <= 700) {
            const int64_t nT = L.tiles;
            std::vector<float> mass(size_t(c.heads) * nT * nT);
            std::uniform_real_distribution<float> u(0.f, 1.f);
            for (int64_t r = 0; r < c.heads * nT; ++r) {
                double s = 0;
                for (int64_t j = 0; j < nT; ++j)
                    s += (mass[r * nT + j] = u(rng));
                for (int64_t j = 0; j < nT; ++j)
                    mass[r * nT + j] = float(mass[r * nT + j] / s);
            }
            std::vector<sparse_attn_window_group> gin(c.heads * 3), gout(c.heads * 3);
            std::vector<int32_t> g3(c.heads, 3);
            for (int hh = 0; hh < c.heads; ++hh) {
                gin[3 * hh] = {0, 0, {0, 0}, {0, 0}};
                gin[3 * hh + 1] = {1, 2, {0, 0}, {0, 0}};
                gin[3 * hh + 2] = {3, -1, {0, 0}, {0, 0}};
            }
            std::vector<double> rec(c.heads), cost(c.heads);
            for (double tau : {0.0, 0.5, 0.9, 1.0})
                for (double lam : {double(INFINITY), 2.0, 0.5}) {
                    EXPECT(sparse_attn_search_windows(h, mass.data(), gin.data(), g3.data(), tau, lam, gout.data(),
                                                      rec.data(), cost.data()) == SPARSE_ATTN_OK);
                    for (int hh = 0; hh < c.heads; ++hh)
                        EXPECT(rec[hh] >= tau - 1e-12 && rec[hh] <= 1.0 + 1e-12 && cost[hh] >= 0 && cost[hh] <= 1);
                }
            EXPECT(sparse_attn_search_windows(h, mass.data(), gin.data(), g3.data(), 1.5, INFINITY, gout.data(),
                                              rec.data(), cost.data()) == SPARSE_ATTN_INVALID_ARG);
            EXPECT(sparse_attn_search_windows(h, nullptr, gin.data(), g3.data(), 0.5, INFINITY, gout.data(),
                                              rec.data(), cost.data()) == SPARSE_ATTN_INVALID_ARG);
            EXPECT(sparse_attn_search_windows(h, mass.data(), groups.data(), gph.data(), 0.5, INFINITY, gout.data(),
                                              rec.data(), cost.data()) == SPARSE_ATTN_BAD_MASK);
        }
        EXPECT(sparse_attn_last_error(h) != nullptr);
        sparse_attn_destroy(h);
    }
    std::printf("host checks done, %d failure(s)\n", g_fail);
    return g_fail ? 1 : 0;
}

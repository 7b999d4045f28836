// Host side of the C-ABI: argument checks, layout planning, buffer carving
// and kernel orchestration.  No device memory is allocated here: every device
// buffer is the caller's.  Every check runs before the first enqueue.
#include "sparse_attn.h"

#include <cmath>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <string>
#include <vector>

#include "common.h"
#include "mix_probe.h"

struct sparse_attn_handle {
    sparse_attn_config cfg;
    sa::Layout L;
    int elem_bytes;
    int kernel;
    float scale;
    // compiled mask
    bool has_mask = false;
    sa::MaskBuffers mb{};  // row lists
    sa::MaskBuffers pb{};  // pair lists (matrix-core kernel only; R = 0 otherwise)
    // host copy of the last dual-window spec (source of the upload)
    std::vector<int32_t> spec;
    // Hilbert order: raster token of each sequence position (host copy, the
    // source of sparse_attn_set_order's upload)
    std::vector<int32_t> seq;
    bool has_order = false;
    // host copy of the last per-head k of the tile selection (upload source)
    std::vector<int32_t> kh;
    std::string err;
};

namespace {

thread_local std::string g_create_err;

int fail(sparse_attn_handle *h, int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (h)
        h->err = buf;
    else
        g_create_err = buf;
    return code;
}

int hip_fail(sparse_attn_handle *h, hipError_t e, const char *what)
{
    return fail(h, SPARSE_ATTN_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Mask-buffer carving: row-list arrays, then (matrix-core kernel) pair-list
// arrays, then the row index list [cap] and (matrix-core kernel) the pair
// index list [cap].  A pair list is never longer than the two row lists it
// merges, so cap entries hold it whenever they hold the rows.
struct MaskLayout {
    size_t row_ptr, len, order, chunk, bucket, status, groups, group_off;
    size_t p_row_ptr, p_len, p_order, p_chunk, p_bucket, p_flag;
    size_t cols;  // start of the index lists
    int R, nchunks, P, pnchunks;
};

MaskLayout mask_layout(const sa::Layout &L, bool pairs)
{
    MaskLayout m{};
    m.R = L.heads * L.nT;
    m.nchunks = (m.R + sa::kMaskChunk - 1) / sa::kMaskChunk;
    m.P = pairs ? L.heads * L.nP : 0;
    m.pnchunks = (m.P + sa::kMaskChunk - 1) / sa::kMaskChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = sa::align256(off + bytes);
        return at;
    };
    m.row_ptr = take(4 * size_t(m.R + 1));
    m.len = take(4 * size_t(m.R));
    m.order = take(4 * size_t(m.R));
    m.chunk = take(4 * size_t(m.nchunks) * size_t(L.nT + 1));
    m.bucket = take(4 * size_t(L.nT + 1));
    m.status = take(64);
    m.groups = take(4 * 6 * size_t(L.heads) * SPARSE_ATTN_MAX_GROUPS);
    m.group_off = take(4 * size_t(L.heads + 1));
    if (pairs) {
        m.p_row_ptr = take(4 * size_t(m.P + 1));
        m.p_len = take(4 * size_t(m.P));
        m.p_order = take(4 * size_t(m.P));
        m.p_chunk = take(4 * size_t(m.pnchunks) * size_t(L.nT + 1));
        m.p_bucket = take(4 * size_t(L.nT + 1));
        m.p_flag = take(4 * size_t(m.P));
    }
    m.cols = off;
    return m;
}

// Bytes of a mask buffer whose index lists hold cap entries.
size_t mask_buffer_bytes(const MaskLayout &m, long long cap)
{
    const size_t rows_end = m.cols + 4 * size_t(cap);
    return m.P > 0 ? sa::align256(rows_end) + 4 * size_t(cap) : rows_end;
}

long long max_pairs(const sa::Layout &L) { return (long long)L.heads * L.nT * L.nT; }

struct WsLayout {
    size_t q, k, v, o, total;
};

WsLayout ws_layout(const sparse_attn_handle *h)
{
    const size_t t = sa::align256(size_t(h->L.heads) * h->L.Npad * h->L.D * h->elem_bytes);
    return WsLayout{0, t, 2 * t, 3 * t, 4 * t};
}

size_t io_bytes(const sparse_attn_handle *h)
{
    return size_t(h->L.heads) * h->L.N * h->L.D * h->elem_bytes;
}

int check_handle(const sparse_attn_handle *h) { return h ? SPARSE_ATTN_OK : SPARSE_ATTN_INVALID_ARG; }

int check_ws(sparse_attn_handle *h, const void *ws, size_t ws_bytes)
{
    if (!ws)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "workspace pointer is null");
    if (!aligned16(ws))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "workspace is not 16-byte aligned");
    const size_t need = ws_layout(h).total;
    if (ws_bytes < need)
        return fail(h, SPARSE_ATTN_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %zu needed",
                    ws_bytes, need);
    return SPARSE_ATTN_OK;
}

// Checks a caller tensor in raster token order (every call that takes one
// moves tokens between the raster and the tiles, which in the Hilbert order
// needs the uploaded sequence map).
int check_io(sparse_attn_handle *h, const void *p, const char *name)
{
    if (!p)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "%s is null", name);
    if (!aligned16(p))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "%s is not 16-byte aligned", name);
    if (h->cfg.order == SPARSE_ATTN_ORDER_HILBERT && !h->has_order)
        return fail(h, SPARSE_ATTN_NO_ORDER, "the Hilbert order needs sparse_attn_set_order first");
    return SPARSE_ATTN_OK;
}

// Validates the temporal-distance groups of a dual-window spec (and, with
// windows, their half-extents); off gets the per-head group offsets.
int check_groups(sparse_attn_handle *h, const sparse_attn_window_group *groups, const int32_t *gph,
                 bool windows, std::vector<int32_t> &off)
{
    const int heads = h->L.heads;
    off.assign(heads + 1, 0);
    for (int hh = 0; hh < heads; ++hh) {
        const int ng = gph[hh];
        if (ng < 1 || ng > SPARSE_ATTN_MAX_GROUPS)
            return fail(h, SPARSE_ATTN_BAD_MASK, "head %d has %d groups (1..%d allowed)", hh, ng,
                        SPARSE_ATTN_MAX_GROUPS);
        off[hh + 1] = off[hh] + ng;
    }
    for (int hh = 0; hh < heads; ++hh) {
        long long prev_hi = -1;
        for (int g = off[hh]; g < off[hh + 1]; ++g) {
            const sparse_attn_window_group &G = groups[g];
            const bool last = g + 1 == off[hh + 1];
            if (G.dt_lo < 0 || (G.dt_hi < 0 && G.dt_hi != -1) || (G.dt_hi >= 0 && G.dt_hi < G.dt_lo))
                return fail(h, SPARSE_ATTN_BAD_MASK, "head %d group %d: bad distance range [%d, %d]", hh,
                            g - off[hh], G.dt_lo, G.dt_hi);
            if (G.dt_hi == -1 && !last)
                return fail(h, SPARSE_ATTN_BAD_MASK,
                            "head %d group %d: an unbounded group must be the last", hh, g - off[hh]);
            if (G.dt_lo <= prev_hi)
                return fail(h, SPARSE_ATTN_BAD_MASK,
                            "head %d group %d: groups must be sorted and disjoint", hh, g - off[hh]);
            for (int w = 0; windows && w < 2; ++w) {
                if (G.ry[w] < -1 || G.rx[w] < -1)
                    return fail(h, SPARSE_ATTN_BAD_MASK,
                                "head %d group %d window %d: half-extents must be >= -1", hh, g - off[hh], w);
            }
            prev_hi = G.dt_hi;
        }
    }
    return SPARSE_ATTN_OK;
}

// Index of cell (t, y, x) on the 3D Hilbert curve over a 2^k cube, after
// J. Skilling, "Programming the Hilbert curve", AIP Conf. Proc. 707 (2004):
// the axes (t, y, x) are turned into the transposed Hilbert index (undo the
// reflections and exchanges level by level from the top, Gray-encode across
// the axes, correct the lower bits), whose bits are read level by level
// from the top, t's first.
uint64_t hilbert_key(int k, uint32_t t, uint32_t y, uint32_t x)
{
    uint32_t c[3] = {t, y, x};
    for (int lvl = k - 1; lvl >= 1; --lvl) {
        const uint32_t bit = 1u << lvl, below = bit - 1;
        for (int a = 0; a < 3; ++a) {
            if (c[a] & bit) {
                c[0] ^= below;
            } else {
                const uint32_t swap = (c[0] ^ c[a]) & below;
                c[0] ^= swap;
                c[a] ^= swap;
            }
        }
    }
    for (int a = 1; a < 3; ++a)
        c[a] ^= c[a - 1];
    uint32_t fix = 0;
    for (int lvl = k - 1; lvl >= 1; --lvl)
        if (c[2] & (1u << lvl))
            fix ^= (1u << lvl) - 1;
    uint64_t key = 0;
    for (int lvl = k - 1; lvl >= 0; --lvl)
        for (int a = 0; a < 3; ++a)
            key = (key << 1) | (((c[a] ^ fix) >> lvl) & 1u);
    return key;
}

// Raster tokens of a T x H x W grid in Hilbert rank order: cells ranked by
// their index on the curve over the smallest enclosing 2^k cube.
std::vector<int32_t> hilbert_sequence(int T, int H, int W, int k)
{
    const long long N = (long long)T * H * W;
    std::vector<std::pair<uint64_t, int32_t>> keyed(N);
    for (long long n = 0; n < N; ++n) {
        const uint32_t t = uint32_t(n / ((long long)H * W)), y = uint32_t((n / W) % H),
                       x = uint32_t(n % W);
        keyed[n] = {hilbert_key(k, t, y, x), int32_t(n)};
    }
    std::sort(keyed.begin(), keyed.end());
    std::vector<int32_t> seq(N);
    for (long long r = 0; r < N; ++r)
        seq[r] = keyed[r].second;
    return seq;
}

// Attention parameters over permuted K and V at kbuf and vbuf; q and o are
// left for the caller to set.
sa::AttnParams attn_params_kv(const sparse_attn_handle *h, const void *kbuf, const void *vbuf)
{
    sa::AttnParams p;
    p.q = nullptr;
    p.k = kbuf;
    p.v = vbuf;
    p.o = nullptr;
    p.raster = 0;
    p.lse = nullptr;
    p.rows = sa::ListSet{h->mb.row_ptr, h->mb.cols, h->mb.order, h->mb.cap};
    p.pairs = sa::ListSet{h->pb.row_ptr, h->pb.cols, h->pb.order, h->pb.cap};
    p.pair_flag = h->pb.flag;
    p.scale_log2 = h->scale * 1.4426950408889634f;
    // Consecutive work items of one XCD take 32 consecutive (longest-first)
    // rows, so query tiles that share key tiles share that XCD's L2.
    p.xcd_chunk = 32;
    p.div_plane = sa::make_fastdiv(uint32_t(h->L.ny) * uint32_t(h->L.nx));
    p.div_row = sa::make_fastdiv(uint32_t(h->L.nx));
    return p;
}

// Attention parameters over the four regions of a forward workspace.
sa::AttnParams attn_params(const sparse_attn_handle *h, void *ws)
{
    const WsLayout w = ws_layout(h);
    char *b = static_cast<char *>(ws);
    sa::AttnParams p = attn_params_kv(h, b + w.k, b + w.v);
    p.q = b + w.q;
    p.o = b + w.o;
    return p;
}

hipError_t launch_attention(const sparse_attn_handle *h, const sa::AttnParams &p, hipStream_t s)
{
    if (h->kernel == SPARSE_ATTN_KERNEL_MFMA_F32)
        return sa::launch_attention_f32(h->L, p, s);
    if (h->kernel != SPARSE_ATTN_KERNEL_MFMA_BF16)
        return sa::launch_attention_generic(h->L, h->elem_bytes, p, s);
    // The pair kernel skips pairs it does not serve and the row kernel
    // tiles the pair kernel serves; a pairing that gives one kernel nothing
    // leaves its launch out.
    const int pairing = h->pb.pairing;
    hipError_t e = hipSuccess;
    if (pairing != SPARSE_ATTN_PAIRING_NONE)
        e = sa::launch_attention_mfma(h->L, p, s);
    if (e == hipSuccess && pairing != SPARSE_ATTN_PAIRING_ALL)
        e = sa::launch_attention_rows(h->L, p, s);
    return e;
}

size_t lse_bytes(const sparse_attn_handle *h) { return size_t(h->L.heads) * h->L.N * sizeof(float); }

// The pairing in effect on the bf16 matrix-core path (AUTO resolved); -1 for
// the fp32 matrix-core and vector-ALU kernels.
int pairing_of(const sparse_attn_handle *h)
{
    if (h->kernel != SPARSE_ATTN_KERNEL_MFMA_BF16)
        return -1;
    if (h->cfg.pairing != SPARSE_ATTN_PAIRING_AUTO)
        return h->cfg.pairing;
    return (long long)h->L.heads * h->L.nP <= sa::kSmallLayoutPairs ? SPARSE_ATTN_PAIRING_NONE
                                                                   : SPARSE_ATTN_PAIRING_OVERLAP;
}

// Scratch of sparse_attn_forward_noalloc: the permuted K and V live in this
// file-scope device array instead of a caller workspace.  Each device that
// runs the library holds its own copy until the process ends.  In host code
// `scratch` only names the symbol; its device address (per device) comes from
// hipGetSymbolAddress and is the only thing passed to kernels.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices] = {};

// Bytes of scratch the no-allocation forward needs: K then V, each region
// 256-byte aligned, as in the workspace.
size_t scratch_need(const sparse_attn_handle *h) { return 2 * ws_layout(h).k; }

// The current device's scratch address, looked up once per device.
int scratch_address(sparse_attn_handle *h, char **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(h, e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(h, SPARSE_ATTN_UNSUPPORTED, "device %d is beyond the %d the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(h, e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = static_cast<char *>(p);
    }
    *out = g_scratch_ptr[dev];
    return SPARSE_ATTN_OK;
}

}  // namespace

extern "C" {

const char *sparse_attn_status_string(int status)
{
    switch (status) {
    case SPARSE_ATTN_OK: return "ok";
    case SPARSE_ATTN_INVALID_ARG: return "invalid argument";
    case SPARSE_ATTN_UNSUPPORTED: return "unsupported configuration";
    case SPARSE_ATTN_BAD_MASK: return "malformed mask";
    case SPARSE_ATTN_WORKSPACE_TOO_SMALL: return "buffer too small";
    case SPARSE_ATTN_NO_MASK: return "no mask set";
    case SPARSE_ATTN_NO_ORDER: return "no Hilbert sequence set";
    case SPARSE_ATTN_HIP_ERROR: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *sparse_attn_last_error(const sparse_attn_handle *h)
{
    return h ? h->err.c_str() : g_create_err.c_str();
}

int sparse_attn_create(const sparse_attn_config *cfg, sparse_attn_handle **out)
{
    if (!cfg || !out)
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "cfg and out must be non-null");
    *out = nullptr;
    const sparse_attn_config &c = *cfg;
    if (c.heads < 1)
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "heads must be >= 1");
    for (int a = 0; a < 3; ++a) {
        if (c.grid[a] < 1 || c.tile[a] < 1)
            return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "grid and tile sizes must be >= 1");
    }
    if (c.dtype != SPARSE_ATTN_F32 && c.dtype != SPARSE_ATTN_BF16)
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "dtype must be F32 or BF16");
    if (!(c.softmax_scale >= 0.f) || std::isinf(c.softmax_scale))
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "softmax_scale must be finite and >= 0");
    if (c.head_dim != 64 && c.head_dim != 128)
        return fail(nullptr, SPARSE_ATTN_UNSUPPORTED, "head_dim must be 64 or 128");
    const long long B = (long long)c.tile[0] * c.tile[1] * c.tile[2];
    if (B > 128)
        return fail(nullptr, SPARSE_ATTN_UNSUPPORTED, "tile volume %lld exceeds 128", B);
    if (c.order != SPARSE_ATTN_ORDER_TILES && c.order != SPARSE_ATTN_ORDER_HILBERT)
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "order must be TILES or HILBERT");
    if (c.pairing < SPARSE_ATTN_PAIRING_AUTO || c.pairing > SPARSE_ATTN_PAIRING_NONE)
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "pairing must be AUTO, OVERLAP, ALL or NONE");
    const long long N0 = (long long)c.grid[0] * c.grid[1] * c.grid[2];
    if (N0 >= (1ll << 31))
        return fail(nullptr, SPARSE_ATTN_UNSUPPORTED, "%lld tokens do not fit 32-bit token ids", N0);
    int cube_k = 0;
    while ((1ll << cube_k) < std::max({c.grid[0], c.grid[1], c.grid[2]}))
        ++cube_k;
    if (c.order == SPARSE_ATTN_ORDER_HILBERT && cube_k > 21)
        return fail(nullptr, SPARSE_ATTN_UNSUPPORTED, "the Hilbert order takes grid sides up to 2^21");

    sa::Layout L{};
    if (c.order == SPARSE_ATTN_ORDER_TILES) {
        L.T = c.grid[0];
        L.H = c.grid[1];
        L.W = c.grid[2];
        // A tile larger than the grid is allowed: it is clipped like any
        // edge tile (its slots per tile are set with the kernel below).
        L.tt = c.tile[0];
        L.th = c.tile[1];
        L.tw = c.tile[2];
    } else {
        // Hilbert order: the tokens in rank order form a 1 x 1 x N grid cut
        // into tiles of 1 x 1 x B (the last one clipped).
        L.T = 1;
        L.H = 1;
        L.W = (int)N0;
        L.tt = 1;
        L.th = 1;
        L.tw = (int)B;
    }
    L.seq_tok = nullptr;
    L.nt = (L.T + L.tt - 1) / L.tt;
    L.ny = (L.H + L.th - 1) / L.th;
    L.nx = (L.W + L.tw - 1) / L.tw;
    const long long nT = (long long)L.nt * L.ny * L.nx;
    const long long N = (long long)L.T * L.H * L.W;
    // This bound also keeps tile ids below 2^16, the width pair-list entries
    // give them.
    if (nT * nT * c.heads >= (1ll << 31))
        return fail(nullptr, SPARSE_ATTN_UNSUPPORTED,
                    "heads * tiles^2 = %lld does not fit 32-bit index lists", nT * nT * c.heads);
    // bf16 runs on the bf16 matrix-core kernels, whose blocks are 128 slots
    // for any tile volume (a smaller tile leaves slots empty); fp32 on the
    // fp32 matrix-core kernel, B slots per tile, while a head's rows fit its
    // 32-bit buffer offsets; the vector-ALU kernel (B slots per tile) takes
    // the rest and every layout on request.
    int kernel = SPARSE_ATTN_KERNEL_GENERIC;
    if (!c.vector_alu && c.dtype == SPARSE_ATTN_BF16)
        kernel = SPARSE_ATTN_KERNEL_MFMA_BF16;
    else if (!c.vector_alu && nT * B * c.head_dim * 4 < (1ll << 31))
        kernel = SPARSE_ATTN_KERNEL_MFMA_F32;
    L.nT = (int)nT;
    L.S = kernel == SPARSE_ATTN_KERNEL_MFMA_BF16 ? 128 : (int)B;
    L.heads = c.heads;
    L.D = c.head_dim;
    L.N = N;
    L.Npad = nT * L.S;
    // Pair query tiles along y, t or x: an axis of even extent first (no
    // tile left alone), preferring y, then t, then x.
    {
        const int n[3] = {L.nt, L.ny, L.nx};
        const int pref[3] = {1, 0, 2};
        L.pax = -1;
        for (int a : pref)
            if (L.pax < 0 && n[a] >= 2 && n[a] % 2 == 0)
                L.pax = a;
        for (int a : pref)
            if (L.pax < 0 && n[a] >= 2)
                L.pax = a;
        for (int a = 0; a < 3; ++a)
            L.pn[a] = a == L.pax ? (n[a] + 1) / 2 : n[a];
        L.nP = L.pn[0] * L.pn[1] * L.pn[2];
    }

    auto *h = new sparse_attn_handle();
    h->cfg = c;
    h->L = L;
    if (c.order == SPARSE_ATTN_ORDER_HILBERT)
        h->seq = hilbert_sequence(c.grid[0], c.grid[1], c.grid[2], cube_k);
    h->elem_bytes = c.dtype == SPARSE_ATTN_F32 ? 4 : 2;
    h->kernel = kernel;
    h->scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.0f / std::sqrt((float)c.head_dim);
    *out = h;
    return SPARSE_ATTN_OK;
}

void sparse_attn_destroy(sparse_attn_handle *h) { delete h; }

int sparse_attn_layout(const sparse_attn_handle *h, sparse_attn_layout_info *info)
{
    if (!h || !info)
        return SPARSE_ATTN_INVALID_ARG;
    const WsLayout w = ws_layout(h);
    info->tokens = h->L.N;
    info->tiles = h->L.nT;
    info->tile_grid[0] = h->L.nt;
    info->tile_grid[1] = h->L.ny;
    info->tile_grid[2] = h->L.nx;
    info->tile_volume = h->L.tt * h->L.th * h->L.tw;
    info->slot_stride = h->L.S;
    info->slots = h->L.Npad;
    info->kernel = h->kernel;
    info->v_layout = h->kernel == SPARSE_ATTN_KERNEL_MFMA_BF16 ? SPARSE_ATTN_LAYOUT_TILE_COLUMNS
                                                               : SPARSE_ATTN_LAYOUT_ROWS;
    info->ws_offset_q = w.q;
    info->ws_offset_k = w.k;
    info->ws_offset_v = w.v;
    info->ws_offset_o = w.o;
    info->ws_bytes = w.total;
    info->pair_axis = h->L.pax;
    for (int a = 0; a < 3; ++a)
        info->pair_grid[a] = h->L.pn[a];
    info->pairs = h->L.nP;
    info->order = h->cfg.order;
    info->pairing = pairing_of(h);
    return SPARSE_ATTN_OK;
}

int sparse_attn_order_bytes(const sparse_attn_handle *h, size_t *bytes)
{
    if (!h || !bytes)
        return SPARSE_ATTN_INVALID_ARG;
    *bytes = 4 * h->seq.size();
    return SPARSE_ATTN_OK;
}

int sparse_attn_set_order(sparse_attn_handle *h, void *order_buf, size_t bytes, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    if (h->cfg.order != SPARSE_ATTN_ORDER_HILBERT)
        return SPARSE_ATTN_OK;
    if (!order_buf || !aligned16(order_buf))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "order_buf must be non-null and 16-byte aligned");
    const size_t need = 4 * h->seq.size();
    if (bytes < need)
        return fail(h, SPARSE_ATTN_WORKSPACE_TOO_SMALL, "order buffer holds %zu bytes, %zu needed", bytes,
                    need);
    const hipError_t e = hipMemcpyAsync(order_buf, h->seq.data(), need, hipMemcpyHostToDevice,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(h, e, "uploading the Hilbert sequence");
    h->L.seq_tok = static_cast<const int *>(order_buf);
    h->has_order = true;
    return SPARSE_ATTN_OK;
}

int sparse_attn_mask_bytes(const sparse_attn_handle *h, int64_t max_nnz, size_t *bytes)
{
    if (!h || !bytes)
        return SPARSE_ATTN_INVALID_ARG;
    const long long cap = (max_nnz <= 0 || max_nnz > max_pairs(h->L)) ? max_pairs(h->L) : max_nnz;
    *bytes = mask_buffer_bytes(mask_layout(h->L, h->kernel == SPARSE_ATTN_KERNEL_MFMA_BF16), cap);
    return SPARSE_ATTN_OK;
}

int sparse_attn_workspace_bytes(const sparse_attn_handle *h, size_t *bytes)
{
    if (!h || !bytes)
        return SPARSE_ATTN_INVALID_ARG;
    *bytes = ws_layout(h).total;
    return SPARSE_ATTN_OK;
}

int sparse_attn_set_mask(sparse_attn_handle *h, const sparse_attn_mask *m, void *mask_buf,
                         size_t bytes, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    if (!m || !mask_buf)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "mask and mask_buf must be non-null");
    if (!aligned16(mask_buf))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "mask_buf is not 16-byte aligned");
    const sa::Layout &L = h->L;
    const bool pairs = h->kernel == SPARSE_ATTN_KERNEL_MFMA_BF16;
    const MaskLayout ml = mask_layout(L, pairs);
    const long long want = (m->max_nnz <= 0 || m->max_nnz > max_pairs(L)) ? max_pairs(L) : m->max_nnz;
    const size_t need = mask_buffer_bytes(ml, want);
    if (bytes < need)
        return fail(h, SPARSE_ATTN_WORKSPACE_TOO_SMALL, "mask_buf holds %zu bytes, %zu needed", bytes,
                    need);

    std::vector<int32_t> spec;  // groups (6 ints each), then offsets (heads + 1)
    if (m->kind == SPARSE_ATTN_MASK_BITMAP) {
        if (!m->bitmap)
            return fail(h, SPARSE_ATTN_INVALID_ARG, "bitmap mask without a bitmap pointer");
    } else if (m->kind == SPARSE_ATTN_MASK_DUAL_WINDOW) {
        if (!m->groups || !m->groups_per_head)
            return fail(h, SPARSE_ATTN_INVALID_ARG, "dual-window mask without groups");
        std::vector<int32_t> off;
        int st;
        if ((st = check_groups(h, m->groups, m->groups_per_head, true, off)))
            return st;
        for (int g = 0; g < off[L.heads]; ++g) {
            const sparse_attn_window_group &G = m->groups[g];
            spec.insert(spec.end(), {G.dt_lo, G.dt_hi, G.ry[0], G.ry[1], G.rx[0], G.rx[1]});
        }
        spec.insert(spec.end(), off.begin(), off.end());
    } else {
        return fail(h, SPARSE_ATTN_BAD_MASK, "unknown mask kind %d", m->kind);
    }

    char *base = static_cast<char *>(mask_buf);
    sa::MaskBuffers mb{};
    mb.row_ptr = reinterpret_cast<int *>(base + ml.row_ptr);
    mb.len = reinterpret_cast<int *>(base + ml.len);
    mb.order = reinterpret_cast<int *>(base + ml.order);
    mb.chunk = reinterpret_cast<int *>(base + ml.chunk);
    mb.bucket = reinterpret_cast<int *>(base + ml.bucket);
    mb.status = reinterpret_cast<int *>(base + ml.status);
    mb.groups = reinterpret_cast<int *>(base + ml.groups);
    mb.group_off = reinterpret_cast<int *>(base + ml.group_off);
    mb.cols = reinterpret_cast<int *>(base + ml.cols);
    mb.cap = want;
    mb.R = ml.R;
    mb.nchunks = ml.nchunks;
    mb.pair = 0;
    mb.flag = nullptr;
    mb.dplane = sa::make_fastdiv(uint32_t(L.ny) * uint32_t(L.nx));
    mb.drow = sa::make_fastdiv(uint32_t(L.nx));
    sa::MaskBuffers pb{};
    if (pairs) {
        pb = mb;
        pb.row_ptr = reinterpret_cast<int *>(base + ml.p_row_ptr);
        pb.len = reinterpret_cast<int *>(base + ml.p_len);
        pb.order = reinterpret_cast<int *>(base + ml.p_order);
        pb.chunk = reinterpret_cast<int *>(base + ml.p_chunk);
        pb.bucket = reinterpret_cast<int *>(base + ml.p_bucket);
        pb.status = mb.status + 4;
        pb.cols = reinterpret_cast<int *>(base + sa::align256(ml.cols + 4 * size_t(want)));
        pb.R = ml.P;
        pb.nchunks = ml.pnchunks;
        pb.pair = 1;
        pb.flag = reinterpret_cast<int *>(base + ml.p_flag);
        pb.pairing = pairing_of(h);
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    h->has_mask = false;
    if (m->kind == SPARSE_ATTN_MASK_DUAL_WINDOW) {
        h->spec = std::move(spec);
        const size_t ngroups = (h->spec.size() - (L.heads + 1)) / 6;
        hipError_t e = hipMemcpyAsync(mb.groups, h->spec.data(), ngroups * 6 * 4,
                                      hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(mb.group_off, h->spec.data() + ngroups * 6, (L.heads + 1) * 4,
                               hipMemcpyHostToDevice, s);
        if (e != hipSuccess)
            return hip_fail(h, e, "uploading the window spec");
    }
    const hipError_t e = sa::launch_compile_mask(
        L, m->kind == SPARSE_ATTN_MASK_BITMAP ? 0 : 1, m->bitmap, mb, pb, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "mask compile launch");
    h->mb = mb;
    h->pb = pb;
    h->has_mask = true;
    return SPARSE_ATTN_OK;
}

int sparse_attn_permute_inputs(sparse_attn_handle *h, const void *q, const void *k, const void *v,
                               void *ws, size_t ws_bytes, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, q, "q")) || (st = check_io(h, k, "k")) || (st = check_io(h, v, "v")) ||
        (st = check_ws(h, ws, ws_bytes)))
        return st;
    const size_t n = io_bytes(h);
    const WsLayout w = ws_layout(h);
    for (const void *p : {q, k, v})
        if (overlaps(p, n, ws, w.total))
            return fail(h, SPARSE_ATTN_INVALID_ARG, "inputs must not overlap the workspace");
    char *b = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_permute_rows(h->L, h->elem_bytes, q, b + w.q, s);
    if (e == hipSuccess)
        e = sa::launch_permute_rows(h->L, h->elem_bytes, k, b + w.k, s);
    if (e == hipSuccess)
        e = h->kernel == SPARSE_ATTN_KERNEL_MFMA_BF16
                ? sa::launch_permute_tile_columns(h->L, v, b + w.v, s)
                : sa::launch_permute_rows(h->L, h->elem_bytes, v, b + w.v, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "permute launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_attend(sparse_attn_handle *h, void *ws, size_t ws_bytes, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_ws(h, ws, ws_bytes)))
        return st;
    if (!h->has_mask)
        return fail(h, SPARSE_ATTN_NO_MASK, "set_mask must be called before attention");
    const hipError_t e = launch_attention(h, attn_params(h, ws), static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(h, e, "attention launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_unpermute_output(sparse_attn_handle *h, void *ws, size_t ws_bytes, void *o,
                                 void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, o, "o")) || (st = check_ws(h, ws, ws_bytes)))
        return st;
    const WsLayout w = ws_layout(h);
    if (overlaps(o, io_bytes(h), ws, w.total))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "o must not overlap the workspace");
    const hipError_t e = sa::launch_unpermute_rows(h->L, h->elem_bytes, static_cast<char *>(ws) + w.o,
                                                   o, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(h, e, "unpermute launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_permute_kv(sparse_attn_handle *h, const void *k, const void *v, void *ws,
                           size_t ws_bytes, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, k, "k")) || (st = check_io(h, v, "v")) || (st = check_ws(h, ws, ws_bytes)))
        return st;
    const size_t n = io_bytes(h);
    const WsLayout w = ws_layout(h);
    for (const void *p : {k, v})
        if (overlaps(p, n, ws, w.total))
            return fail(h, SPARSE_ATTN_INVALID_ARG, "inputs must not overlap the workspace");
    char *b = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_permute_rows(h->L, h->elem_bytes, k, b + w.k, s);
    if (e == hipSuccess)
        e = h->kernel == SPARSE_ATTN_KERNEL_MFMA_BF16
                ? sa::launch_permute_tile_columns(h->L, v, b + w.v, s)
                : sa::launch_permute_rows(h->L, h->elem_bytes, v, b + w.v, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "permute launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_attend_raster(sparse_attn_handle *h, const void *q, void *o, float *lse, void *ws,
                              size_t ws_bytes, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, q, "q")) || (st = check_io(h, o, "o")) || (st = check_ws(h, ws, ws_bytes)))
        return st;
    if (lse && !aligned16(lse))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "lse is not 16-byte aligned");
    if (!h->has_mask)
        return fail(h, SPARSE_ATTN_NO_MASK, "set_mask must be called before attention");
    const size_t n = io_bytes(h);
    const WsLayout w = ws_layout(h);
    if (overlaps(o, n, q, n) || overlaps(o, n, ws, w.total) || overlaps(q, n, ws, w.total))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "q, o and the workspace must not overlap");
    if (lse && (overlaps(lse, lse_bytes(h), q, n) || overlaps(lse, lse_bytes(h), o, n) ||
                overlaps(lse, lse_bytes(h), ws, w.total)))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "lse must not overlap q, o or the workspace");
    sa::AttnParams p = attn_params(h, ws);
    p.q = q;
    p.o = o;
    p.raster = 1;
    p.lse = lse;
    const hipError_t e = launch_attention(h, p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(h, e, "attention launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_forward_lse(sparse_attn_handle *h, const void *q, const void *k, const void *v,
                            void *o, float *lse, void *ws, size_t ws_bytes, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, q, "q")) || (st = check_io(h, k, "k")) || (st = check_io(h, v, "v")) ||
        (st = check_io(h, o, "o")) || (st = check_ws(h, ws, ws_bytes)))
        return st;
    if (lse && !aligned16(lse))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "lse is not 16-byte aligned");
    if (!h->has_mask)
        return fail(h, SPARSE_ATTN_NO_MASK, "set_mask must be called before forward");
    const size_t n = io_bytes(h);
    for (const void *p : {q, k, v})
        if (overlaps(o, n, p, n) || (lse && overlaps(lse, lse_bytes(h), p, n)))
            return fail(h, SPARSE_ATTN_INVALID_ARG, "o and lse must not overlap q, k or v");
    if (lse && overlaps(lse, lse_bytes(h), o, n))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "lse must not overlap o");
    const size_t wt = ws_layout(h).total;
    for (const void *p : {q, k, v, static_cast<const void *>(o)})
        if (overlaps(p, n, ws, wt))
            return fail(h, SPARSE_ATTN_INVALID_ARG, "q, k, v and o must not overlap the workspace");
    if (lse && overlaps(lse, lse_bytes(h), ws, wt))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "lse must not overlap the workspace");
    // Every check of the two stages has passed here, so nothing is enqueued
    // unless both launch.
    if ((st = sparse_attn_permute_kv(h, k, v, ws, ws_bytes, stream)))
        return st;
    return sparse_attn_attend_raster(h, q, o, lse, ws, ws_bytes, stream);
}

int sparse_attn_forward(sparse_attn_handle *h, const void *q, const void *k, const void *v, void *o,
                        void *ws, size_t ws_bytes, void *stream)
{
    return sparse_attn_forward_lse(h, q, k, v, o, nullptr, ws, ws_bytes, stream);
}

int sparse_attn_forward_noalloc(sparse_attn_handle *h, const void *q, const void *k, const void *v, void *o,
                                void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, q, "q")) || (st = check_io(h, k, "k")) || (st = check_io(h, v, "v")) ||
        (st = check_io(h, o, "o")))
        return st;
    const size_t need = scratch_need(h);
    if (need > kScratchBytes)
        return fail(h, SPARSE_ATTN_UNSUPPORTED,
                    "the permuted K and V need %zu bytes; the no-allocation forward holds at most %zu "
                    "(use sparse_attn_forward with a workspace)",
                    need, kScratchBytes);
    if (!h->has_mask)
        return fail(h, SPARSE_ATTN_NO_MASK, "set_mask must be called before forward");
    const size_t n = io_bytes(h);
    for (const void *p : {q, k, v})
        if (overlaps(o, n, p, n))
            return fail(h, SPARSE_ATTN_INVALID_ARG, "o must not overlap q, k or v");
    char *kbuf = nullptr;
    if ((st = scratch_address(h, &kbuf)))
        return st;
    // The workspace's K and V regions, carved from the scratch array.
    const WsLayout w = ws_layout(h);
    char *vbuf = kbuf + (w.v - w.k);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_permute_rows(h->L, h->elem_bytes, k, kbuf, s);
    if (e == hipSuccess)
        e = h->kernel == SPARSE_ATTN_KERNEL_MFMA_BF16 ? sa::launch_permute_tile_columns(h->L, v, vbuf, s)
                                                      : sa::launch_permute_rows(h->L, h->elem_bytes, v, vbuf, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "permute launch");
    sa::AttnParams p = attn_params_kv(h, kbuf, vbuf);
    p.q = q;
    p.o = o;
    p.raster = 1;
    p.lse = nullptr;
    e = launch_attention(h, p, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "attention launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_tile_mass(sparse_attn_handle *h, const void *q, const void *k, void *ws,
                          size_t ws_bytes, float *mass, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, q, "q")) || (st = check_io(h, k, "k")) || (st = check_ws(h, ws, ws_bytes)))
        return st;
    if (!mass || !aligned16(mass))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "mass must be non-null and 16-byte aligned");
    if (h->kernel != SPARSE_ATTN_KERNEL_MFMA_BF16)
        return fail(h, SPARSE_ATTN_UNSUPPORTED, "the tile mass runs on the matrix-core path (bf16)");
    const sa::Layout &L = h->L;
    const size_t n = io_bytes(h), mb = size_t(L.heads) * L.nT * L.nT * sizeof(float);
    const WsLayout w = ws_layout(h);
    for (const void *p : {q, k})
        if (overlaps(p, n, ws, w.total) || overlaps(mass, mb, p, n))
            return fail(h, SPARSE_ATTN_INVALID_ARG, "q, k, mass and the workspace must not overlap");
    if (overlaps(mass, mb, ws, w.total))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "mass must not overlap the workspace");
    char *b = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_permute_rows(L, h->elem_bytes, q, b + w.q, s);
    if (e == hipSuccess)
        e = sa::launch_permute_rows(L, h->elem_bytes, k, b + w.k, s);
    if (e == hipSuccess)
        e = sa::launch_tile_mass(L, b + w.q, b + w.k, h->scale * 1.4426950408889634f, mass, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "tile mass");
    return SPARSE_ATTN_OK;
}

int sparse_attn_search_windows(sparse_attn_handle *h, const float *mass,
                               const sparse_attn_window_group *groups_in, const int32_t *groups_per_head,
                               double tau, double lambda, sparse_attn_window_group *groups_out,
                               double *recall, double *cost)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    if (!mass || !groups_in || !groups_per_head || !groups_out || !recall || !cost)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "null argument");
    if (!(tau >= 0.0 && tau <= 1.0))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "tau must lie in [0, 1]");
    if (!(lambda > 0.0))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "lambda must be > 0 (infinity disables it)");
    std::vector<int32_t> off;
    int st;
    if ((st = check_groups(h, groups_in, groups_per_head, false, off)))
        return st;
    const sa::Layout &L = h->L;
    for (int hh = 0; hh < L.heads; ++hh)
        sa::search_head(L, mass + (size_t)hh * L.nT * L.nT, groups_in + off[hh], off[hh + 1] - off[hh], tau,
                        lambda, groups_out + off[hh], recall + hh, cost + hh);
    return SPARSE_ATTN_OK;
}

int sparse_attn_select_topk(sparse_attn_handle *h, const int32_t *k_per_head, void *ws,
                            size_t ws_bytes, uint8_t *bitmap, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_ws(h, ws, ws_bytes)))
        return st;
    if (!k_per_head || !bitmap)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "k_per_head and bitmap must be non-null");
    const sa::Layout &L = h->L;
    for (int hh = 0; hh < L.heads; ++hh)
        if (k_per_head[hh] < 0 || k_per_head[hh] > L.nT)
            return fail(h, SPARSE_ATTN_INVALID_ARG, "k_per_head[%d] = %d is outside 0..%d", hh,
                        k_per_head[hh], L.nT);
    if (L.nT > sa::kSelectMaxTiles)
        return fail(h, SPARSE_ATTN_UNSUPPORTED, "tile selection takes at most %d tiles (%d)",
                    sa::kSelectMaxTiles, L.nT);
    // Scratch in the output region: tile means of Q and K (fp32), then k.
    const WsLayout w = ws_layout(h);
    const size_t means = sa::align256(size_t(L.heads) * L.nT * L.D * 4);
    if (2 * means + 4 * size_t(L.heads) > w.total - w.o)
        return fail(h, SPARSE_ATTN_UNSUPPORTED, "tiles of %d slots are too small for the selection scratch",
                    L.S);
    char *b = static_cast<char *>(ws);
    float *qbar = reinterpret_cast<float *>(b + w.o);
    float *kbar = reinterpret_cast<float *>(b + w.o + means);
    int *kh = reinterpret_cast<int *>(b + w.o + 2 * means);
    hipStream_t s = static_cast<hipStream_t>(stream);
    h->kh.assign(k_per_head, k_per_head + L.heads);
    hipError_t e = hipMemcpyAsync(kh, h->kh.data(), 4 * size_t(L.heads), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = sa::launch_select_topk(L, h->elem_bytes, b + w.q, b + w.k, kh, h->scale, qbar, kbar, bitmap,
                                   s);
    if (e != hipSuccess)
        return hip_fail(h, e, "tile selection");
    return SPARSE_ATTN_OK;
}

int sparse_attn_select_scope(sparse_attn_handle *h, float rho, int32_t k_fixed, void *ws, size_t ws_bytes,
                             uint8_t *bitmap, int32_t *base, int32_t *keep, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_ws(h, ws, ws_bytes)))
        return st;
    const sa::Layout &L = h->L;
    if (!bitmap)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "bitmap must be non-null");
    if (!std::isfinite(rho))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "rho must be finite");
    if (k_fixed < 0 || k_fixed > L.nT)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "k_fixed = %d is outside 0..%d", k_fixed, L.nT);
    if (L.nT > sa::kSelectMaxTiles)
        return fail(h, SPARSE_ATTN_UNSUPPORTED, "tile selection takes at most %d tiles (%d)",
                    sa::kSelectMaxTiles, L.nT);
    // Scratch in the output region: tile means of Q and K (fp32), then the
    // base and final counts (when the caller passes no arrays for them).
    const WsLayout w = ws_layout(h);
    const size_t means = sa::align256(size_t(L.heads) * L.nT * L.D * 4);
    const size_t counts = sa::align256(size_t(L.heads) * L.nT * 4);
    if (2 * means + 2 * counts > w.total - w.o)
        return fail(h, SPARSE_ATTN_UNSUPPORTED, "tiles of %d slots are too small for the selection scratch",
                    L.S);
    const size_t bm = size_t(L.heads) * L.nT * L.nT, nc = size_t(L.heads) * L.nT * 4;
    if (overlaps(bitmap, bm, ws, w.total) || (base && overlaps(base, nc, ws, w.total)) ||
        (keep && overlaps(keep, nc, ws, w.total)) || (base && overlaps(base, nc, bitmap, bm)) ||
        (keep && overlaps(keep, nc, bitmap, bm)) || (base && keep && overlaps(base, nc, keep, nc)))
        return fail(h, SPARSE_ATTN_INVALID_ARG, "bitmap, base, keep and the workspace must not overlap");
    char *b = static_cast<char *>(ws);
    float *qbar = reinterpret_cast<float *>(b + w.o);
    float *kbar = reinterpret_cast<float *>(b + w.o + means);
    int *bs = base ? base : reinterpret_cast<int *>(b + w.o + 2 * means);
    int *kp = keep ? keep : reinterpret_cast<int *>(b + w.o + 2 * means + counts);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_select_scope(L, h->elem_bytes, b + w.q, b + w.k, h->scale, rho, k_fixed, qbar,
                                           kbar, bs, kp, bitmap, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "tile selection");
    return SPARSE_ATTN_OK;
}

int sparse_attn_permute(sparse_attn_handle *h, const void *src, void *dst, int32_t layout,
                        void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, src, "src")) || (st = check_io(h, dst, "dst")))
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (layout == SPARSE_ATTN_LAYOUT_ROWS) {
        e = sa::launch_permute_rows(h->L, h->elem_bytes, src, dst, s);
    } else if (layout == SPARSE_ATTN_LAYOUT_TILE_COLUMNS) {
        if (h->elem_bytes != 2 || h->L.S % 8 != 0)
            return fail(h, SPARSE_ATTN_UNSUPPORTED,
                        "tile-column layout needs bf16 and a tile volume divisible by 8");
        e = sa::launch_permute_tile_columns(h->L, src, dst, s);
    } else {
        return fail(h, SPARSE_ATTN_INVALID_ARG, "unknown layout %d", layout);
    }
    if (e != hipSuccess)
        return hip_fail(h, e, "permute launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_unpermute(sparse_attn_handle *h, const void *src, void *dst, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    int st;
    if ((st = check_io(h, src, "src")) || (st = check_io(h, dst, "dst")))
        return st;
    const hipError_t e =
        sa::launch_unpermute_rows(h->L, h->elem_bytes, src, dst, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(h, e, "unpermute launch");
    return SPARSE_ATTN_OK;
}

int sparse_attn_read_index_lists(sparse_attn_handle *h, int32_t *row_ptr, int32_t *cols,
                                 int64_t cols_capacity, int32_t *order, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    if (!row_ptr || !order || (!cols && cols_capacity > 0) || cols_capacity < 0)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "null destination");
    if (!h->has_mask)
        return fail(h, SPARSE_ATTN_NO_MASK, "no mask set");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int R = h->mb.R;
    hipError_t e = hipMemcpyAsync(row_ptr, h->mb.row_ptr, 4 * size_t(R + 1), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(order, h->mb.order, 4 * size_t(R), hipMemcpyDeviceToDevice, s);
    const long long n = std::min<long long>(cols_capacity, h->mb.cap);
    if (e == hipSuccess && n > 0)
        e = hipMemcpyAsync(cols, h->mb.cols, 4 * size_t(n), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "copying index lists");
    return SPARSE_ATTN_OK;
}

int sparse_attn_read_pair_lists(sparse_attn_handle *h, int32_t *row_ptr, int32_t *cols,
                                int64_t cols_capacity, int32_t *order, int32_t *flag, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    if (!row_ptr || !order || !flag || (!cols && cols_capacity > 0) || cols_capacity < 0)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "null destination");
    if (h->kernel != SPARSE_ATTN_KERNEL_MFMA_BF16)
        return fail(h, SPARSE_ATTN_UNSUPPORTED, "pair lists exist for the bf16 matrix-core kernels only");
    if (!h->has_mask)
        return fail(h, SPARSE_ATTN_NO_MASK, "no mask set");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int P = h->pb.R;
    hipError_t e = hipMemcpyAsync(row_ptr, h->pb.row_ptr, 4 * size_t(P + 1), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(order, h->pb.order, 4 * size_t(P), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(flag, h->pb.flag, 4 * size_t(P), hipMemcpyDeviceToDevice, s);
    const long long n = std::min<long long>(cols_capacity, h->pb.cap);
    if (e == hipSuccess && n > 0)
        e = hipMemcpyAsync(cols, h->pb.cols, 4 * size_t(n), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess)
        return hip_fail(h, e, "copying pair lists");
    return SPARSE_ATTN_OK;
}

int sparse_attn_mask_info(sparse_attn_handle *h, int64_t *nnz, int32_t *overflow, void *stream)
{
    if (check_handle(h))
        return SPARSE_ATTN_INVALID_ARG;
    if (!nnz || !overflow)
        return fail(h, SPARSE_ATTN_INVALID_ARG, "null output");
    if (!h->has_mask)
        return fail(h, SPARSE_ATTN_NO_MASK, "no mask set");
    int32_t st[2];
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(st, h->mb.status, sizeof st, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return hip_fail(h, e, "reading mask status");
    *nnz = st[0];
    *overflow = st[1];
    return SPARSE_ATTN_OK;
}

}  // extern "C"

int sparse_attn_mix_probe(int32_t waves_per_simd, int32_t pingpong, int32_t cus, int32_t iters, int64_t *cycles,
                          float *sink, void *stream)
{
    if (waves_per_simd < 1 || waves_per_simd > 3)
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "waves_per_simd must be 1, 2 or 3");
    if (pingpong != 0 && (pingpong != 1 || waves_per_simd != 2))
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "pingpong must be 0, or 1 with waves_per_simd 2");
    if (cus < 1 || cus > 65536 || iters < 1 || iters > (1 << 20))
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "cus must be in 1..65536 and iters in 1..2^20");
    if (!cycles || !sink || reinterpret_cast<uintptr_t>(cycles) % 8 || reinterpret_cast<uintptr_t>(sink) % 4)
        return fail(nullptr, SPARSE_ATTN_INVALID_ARG, "cycles and sink must be non-null and aligned");
    const hipError_t e = sa::launch_mix_probe(waves_per_simd, pingpong, cus, iters,
                                              reinterpret_cast<long long *>(cycles), sink,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SPARSE_ATTN_OK : hip_fail(nullptr, e, "mix probe launch");
}

"""Python binding of libsparse_attn (block-sparse video attention forward for
MI355X / gfx950).

A thin ctypes layer with the same names as the C-ABI in
include/sparse_attn.h: it marshals torch tensors (device memory) and streams
into pointers and raises SparseAttnError on a non-zero status.  Every step of
the computation runs in the HIP library; there is no fallback path.  The
library must have been built (block_sparse_attention_major_amd/build.py);
importing this module fails loudly if it is missing.

``SparseAttention`` is a small convenience wrapper that allocates the mask
buffer and workspace with torch and calls the same entry points.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python block_sparse_attention_major_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

SPARSE_ATTN_OK = 0
SPARSE_ATTN_INVALID_ARG = 1
SPARSE_ATTN_UNSUPPORTED = 2
SPARSE_ATTN_BAD_MASK = 3
SPARSE_ATTN_WORKSPACE_TOO_SMALL = 4
SPARSE_ATTN_NO_MASK = 5
SPARSE_ATTN_HIP_ERROR = 6
SPARSE_ATTN_NO_ORDER = 7
SPARSE_ATTN_ORDER_TILES = 0
SPARSE_ATTN_ORDER_HILBERT = 1
SPARSE_ATTN_PAIRING_AUTO = 0
SPARSE_ATTN_PAIRING_OVERLAP = 1
SPARSE_ATTN_PAIRING_ALL = 2
SPARSE_ATTN_PAIRING_NONE = 3
_PAIRINGS = {"auto": SPARSE_ATTN_PAIRING_AUTO, "overlap": SPARSE_ATTN_PAIRING_OVERLAP,
             "all": SPARSE_ATTN_PAIRING_ALL, "none": SPARSE_ATTN_PAIRING_NONE}

SPARSE_ATTN_F32 = 0
SPARSE_ATTN_BF16 = 1
SPARSE_ATTN_MASK_BITMAP = 0
SPARSE_ATTN_MASK_DUAL_WINDOW = 1
SPARSE_ATTN_LAYOUT_ROWS = 0
SPARSE_ATTN_LAYOUT_TILE_COLUMNS = 1
SPARSE_ATTN_KERNEL_MFMA_BF16 = 0
SPARSE_ATTN_KERNEL_GENERIC = 1
SPARSE_ATTN_KERNEL_MFMA_F32 = 2
SPARSE_ATTN_MAX_GROUPS = 8

EXPORTED = [
    "sparse_attn_create", "sparse_attn_destroy", "sparse_attn_layout", "sparse_attn_mask_bytes",
    "sparse_attn_workspace_bytes", "sparse_attn_order_bytes", "sparse_attn_set_order",
    "sparse_attn_set_mask", "sparse_attn_forward", "sparse_attn_forward_noalloc",
    "sparse_attn_forward_lse", "sparse_attn_permute_kv", "sparse_attn_attend_raster",
    "sparse_attn_permute_inputs", "sparse_attn_attend", "sparse_attn_unpermute_output",
    "sparse_attn_permute", "sparse_attn_unpermute", "sparse_attn_read_index_lists",
    "sparse_attn_read_pair_lists", "sparse_attn_select_topk", "sparse_attn_select_scope",
    "sparse_attn_tile_mass",
    "sparse_attn_search_windows", "sparse_attn_mix_probe",
    "sparse_attn_mask_info", "sparse_attn_status_string", "sparse_attn_last_error",
]


class sparse_attn_config(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("grid", ctypes.c_int32 * 3), ("tile", ctypes.c_int32 * 3),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("order", ctypes.c_int32), ("pairing", ctypes.c_int32),
                ("vector_alu", ctypes.c_int32)]


class sparse_attn_window_group(ctypes.Structure):
    _fields_ = [("dt_lo", ctypes.c_int32), ("dt_hi", ctypes.c_int32),
                ("ry", ctypes.c_int32 * 2), ("rx", ctypes.c_int32 * 2)]


class sparse_attn_mask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("bitmap", ctypes.c_void_p),
                ("groups", ctypes.c_void_p), ("groups_per_head", ctypes.c_void_p),
                ("max_nnz", ctypes.c_int64)]


class sparse_attn_layout_info(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("tile_grid", ctypes.c_int32 * 3), ("tile_volume", ctypes.c_int32),
                ("slots", ctypes.c_int64), ("kernel", ctypes.c_int32), ("v_layout", ctypes.c_int32),
                ("ws_offset_q", ctypes.c_size_t), ("ws_offset_k", ctypes.c_size_t),
                ("ws_offset_v", ctypes.c_size_t), ("ws_offset_o", ctypes.c_size_t),
                ("ws_bytes", ctypes.c_size_t), ("pair_axis", ctypes.c_int32),
                ("pair_grid", ctypes.c_int32 * 3), ("pairs", ctypes.c_int64),
                ("order", ctypes.c_int32), ("pairing", ctypes.c_int32),
                ("slot_stride", ctypes.c_int32)]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_P = ctypes.POINTER
_sigs = {
    "sparse_attn_create": ([_P(sparse_attn_config), _P(_vp)], ctypes.c_int),
    "sparse_attn_destroy": ([_vp], None),
    "sparse_attn_layout": ([_vp, _P(sparse_attn_layout_info)], ctypes.c_int),
    "sparse_attn_mask_bytes": ([_vp, _i64, _P(_sz)], ctypes.c_int),
    "sparse_attn_workspace_bytes": ([_vp, _P(_sz)], ctypes.c_int),
    "sparse_attn_order_bytes": ([_vp, _P(_sz)], ctypes.c_int),
    "sparse_attn_set_order": ([_vp, _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_set_mask": ([_vp, _P(sparse_attn_mask), _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_forward": ([_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_forward_noalloc": ([_vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "sparse_attn_forward_lse": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_permute_kv": ([_vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_attend_raster": ([_vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_permute_inputs": ([_vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_attend": ([_vp, _vp, _sz, _vp], ctypes.c_int),
    "sparse_attn_unpermute_output": ([_vp, _vp, _sz, _vp, _vp], ctypes.c_int),
    "sparse_attn_permute": ([_vp, _vp, _vp, _i32, _vp], ctypes.c_int),
    "sparse_attn_unpermute": ([_vp, _vp, _vp, _vp], ctypes.c_int),
    "sparse_attn_read_index_lists": ([_vp, _vp, _vp, _i64, _vp, _vp], ctypes.c_int),
    "sparse_attn_read_pair_lists": ([_vp, _vp, _vp, _i64, _vp, _vp, _vp], ctypes.c_int),
    "sparse_attn_select_topk": ([_vp, _vp, _vp, _sz, _vp, _vp], ctypes.c_int),
    "sparse_attn_select_scope": ([_vp, ctypes.c_float, _i32, _vp, _sz, _vp, _vp, _vp, _vp], ctypes.c_int),
    "sparse_attn_tile_mass": ([_vp, _vp, _vp, _vp, _sz, _vp, _vp], ctypes.c_int),
    "sparse_attn_search_windows": ([_vp, _vp, _vp, _vp, ctypes.c_double, ctypes.c_double, _vp, _vp,
                                    _vp], ctypes.c_int),
    "sparse_attn_mix_probe": ([_i32, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "sparse_attn_mask_info": ([_vp, _P(_i64), _P(_i32), _vp], ctypes.c_int),
    "sparse_attn_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sparse_attn_last_error": ([_vp], ctypes.c_char_p),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class SparseAttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{sparse_attn_status_string(status)} ({status}): {message}")
        self.status = status
        self.message = message


def sparse_attn_status_string(status):
    return _lib.sparse_attn_status_string(int(status)).decode()


def sparse_attn_last_error(h=None):
    return _lib.sparse_attn_last_error(h.ptr if h is not None else None).decode()


class Handle:
    """Owns a sparse_attn_handle*; destroyed with sparse_attn_destroy."""

    def __init__(self, ptr, cfg):
        self.ptr = ptr
        self.cfg = cfg
        self._sizes = None

    @property
    def sizes(self):
        """Byte sizes of the caller buffers, from the planned layout."""
        if self._sizes is None:
            L = sparse_attn_layout(self)
            heads, d = self.cfg.heads, self.cfg.head_dim
            elem = 4 if self.cfg.dtype == SPARSE_ATTN_F32 else 2
            N, nT, slots = L["tokens"], L["tiles"], L["slots"]
            self._sizes = {
                "elem": elem, "heads": heads, "tiles": nT, "pairs": L["pairs"],
                "io": heads * N * d * elem,          # q, k, v, o in raster order
                "slots": heads * slots * d * elem,   # a tile-major tensor
                "lse": heads * N * 4,
                "bitmap": heads * nT * nT,
                "mass": heads * nT * nT * 4,
            }
        return self._sizes

    def __del__(self):
        # At interpreter exit the module's globals may already be gone.
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.sparse_attn_destroy(self.ptr)
            self.ptr = None


def _check(status, h=None):
    if status != SPARSE_ATTN_OK:
        raise SparseAttnError(status, sparse_attn_last_error(h))


def _dptr(t, name):
    """Device pointer of a torch tensor (or None / raw int)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _sized(t, name, nbytes, elem=None, at_least=False):
    """Device pointer of t after checking that it holds exactly (or, with
    at_least, at least) nbytes bytes of elements of size elem: the C ABI
    takes no sizes for these buffers, so a mis-sized tensor is refused here,
    before anything is enqueued."""
    if t is None or isinstance(t, int):
        return _dptr(t, name)
    if elem is not None and t.element_size() != elem:
        raise ValueError(f"{name}: elements of {t.element_size()} bytes, expected {elem}")
    got = t.numel() * t.element_size()
    if (got < nbytes) if at_least else (got != nbytes):
        raise ValueError(f"{name}: {got} bytes, expected {'at least ' if at_least else ''}{nbytes}")
    return _dptr(t, name)


def _host_heads(a, name, heads):
    """A host int32 array with one entry per head."""
    a = np.ascontiguousarray(a, dtype=np.int32).reshape(-1)
    if a.shape[0] != heads:
        raise ValueError(f"{name}: {a.shape[0]} entries, expected one per head ({heads})")
    return a


def _host_groups(groups, gph, heads):
    """Window groups [G, 6] and groups per head, checked against each other
    and the head count."""
    g = np.ascontiguousarray(groups, dtype=np.int32).reshape(-1, 6)
    gph = _host_heads(gph, "groups_per_head", heads)
    if g.shape[0] != int(gph.astype(np.int64).sum()):
        raise ValueError(f"groups: {g.shape[0]} rows, expected sum(groups_per_head) = {int(gph.sum())}")
    return g, gph


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    return t.numel() * t.element_size()


def sparse_attn_create(heads, head_dim, grid, tile, dtype, softmax_scale=0.0,
                       order=SPARSE_ATTN_ORDER_TILES, pairing=SPARSE_ATTN_PAIRING_AUTO,
                       vector_alu=False):
    """dtype: "bf16"/"f32" or SPARSE_ATTN_BF16/SPARSE_ATTN_F32; order:
    "tiles"/"hilbert" or SPARSE_ATTN_ORDER_*; pairing: "auto"/"overlap"/
    "all"/"none" or SPARSE_ATTN_PAIRING_*; vector_alu: run on the vector-ALU
    kernel instead of the matrix-core kernels."""
    if isinstance(dtype, str):
        dtype = {"bf16": SPARSE_ATTN_BF16, "f32": SPARSE_ATTN_F32}[dtype]
    if isinstance(order, str):
        order = {"tiles": SPARSE_ATTN_ORDER_TILES, "hilbert": SPARSE_ATTN_ORDER_HILBERT}[order]
    if isinstance(pairing, str):
        pairing = _PAIRINGS[pairing]
    cfg = sparse_attn_config(int(heads), int(head_dim), (ctypes.c_int32 * 3)(*grid),
                             (ctypes.c_int32 * 3)(*tile), int(dtype), float(softmax_scale),
                             int(order), int(pairing), int(bool(vector_alu)))
    out = _vp()
    st = _lib.sparse_attn_create(ctypes.byref(cfg), ctypes.byref(out))
    if st != SPARSE_ATTN_OK:
        raise SparseAttnError(st, sparse_attn_last_error(None))
    return Handle(out.value, cfg)


def sparse_attn_destroy(h):
    if h.ptr:
        _lib.sparse_attn_destroy(h.ptr)
        h.ptr = None


def sparse_attn_layout(h):
    info = sparse_attn_layout_info()
    _check(_lib.sparse_attn_layout(h.ptr, ctypes.byref(info)), h)
    return {f: (list(getattr(info, f)) if f in ("tile_grid", "pair_grid") else getattr(info, f))
            for f, _ in sparse_attn_layout_info._fields_}


def sparse_attn_mask_bytes(h, max_nnz=0):
    n = _sz()
    _check(_lib.sparse_attn_mask_bytes(h.ptr, int(max_nnz), ctypes.byref(n)), h)
    return n.value


def sparse_attn_workspace_bytes(h):
    n = _sz()
    _check(_lib.sparse_attn_workspace_bytes(h.ptr, ctypes.byref(n)), h)
    return n.value


def sparse_attn_order_bytes(h):
    n = _sz()
    _check(_lib.sparse_attn_order_bytes(h.ptr, ctypes.byref(n)), h)
    return n.value


def sparse_attn_set_order(h, order_buf, stream=None):
    """Upload the Hilbert rank -> token map into order_buf (device tensor of
    at least sparse_attn_order_bytes bytes; kept alive by the caller)."""
    _check(_lib.sparse_attn_set_order(h.ptr, _dptr(order_buf, "order_buf"),
                                      _nbytes(order_buf) if order_buf is not None else 0,
                                      _stream(stream)), h)


def sparse_attn_set_mask(h, mask_buf, bitmap=None, groups=None, groups_per_head=None, max_nnz=0,
                         stream=None):
    """Bitmap mask: `bitmap` is a device uint8 tensor [heads, nT, nT].
    Dual-window mask: `groups` int32 [G, 6] rows (dt_lo, dt_hi, ry0, ry1, rx0,
    rx1) and `groups_per_head` int32 [heads], host arrays."""
    m = sparse_attn_mask()
    keep = []
    if bitmap is not None:
        m.kind = SPARSE_ATTN_MASK_BITMAP
        m.bitmap = _sized(bitmap, "bitmap", h.sizes["bitmap"], elem=1)
    else:
        g, gph = _host_groups(groups, groups_per_head, h.cfg.heads)
        keep += [g, gph]
        m.kind = SPARSE_ATTN_MASK_DUAL_WINDOW
        m.groups = g.ctypes.data
        m.groups_per_head = gph.ctypes.data
    m.max_nnz = int(max_nnz)
    _check(_lib.sparse_attn_set_mask(h.ptr, ctypes.byref(m), _dptr(mask_buf, "mask_buf"),
                                     _nbytes(mask_buf), _stream(stream)), h)
    del keep


def _io(h, t, name):
    return _sized(t, name, h.sizes["io"], elem=h.sizes["elem"])


def _lse(h, t):
    return _sized(t, "lse", h.sizes["lse"], elem=4)


def sparse_attn_forward(h, q, k, v, o, ws, stream=None):
    _check(_lib.sparse_attn_forward(h.ptr, _io(h, q, "q"), _io(h, k, "k"), _io(h, v, "v"), _io(h, o, "o"),
                                    _dptr(ws, "ws"), _nbytes(ws), _stream(stream)), h)


SPARSE_ATTN_NOALLOC_SCRATCH_BYTES = 128 << 20


def sparse_attn_forward_noalloc(h, q, k, v, o, stream=None):
    """Forward without a workspace: the permuted K and V use the library's
    fixed per-device scratch array (at most SPARSE_ATTN_NOALLOC_SCRATCH_BYTES;
    larger layouts fail with UNSUPPORTED).  Calls overlapping in time on one
    device race on that array."""
    _check(_lib.sparse_attn_forward_noalloc(h.ptr, _io(h, q, "q"), _io(h, k, "k"), _io(h, v, "v"),
                                            _io(h, o, "o"), _stream(stream)), h)


def sparse_attn_forward_lse(h, q, k, v, o, lse, ws, stream=None):
    """Forward that also writes lse (device fp32 [heads, N], or None)."""
    _check(_lib.sparse_attn_forward_lse(h.ptr, _io(h, q, "q"), _io(h, k, "k"), _io(h, v, "v"),
                                        _io(h, o, "o"), _lse(h, lse), _dptr(ws, "ws"),
                                        _nbytes(ws), _stream(stream)), h)


def sparse_attn_permute_kv(h, k, v, ws, stream=None):
    _check(_lib.sparse_attn_permute_kv(h.ptr, _io(h, k, "k"), _io(h, v, "v"), _dptr(ws, "ws"),
                                       _nbytes(ws), _stream(stream)), h)


def sparse_attn_attend_raster(h, q, o, ws, lse=None, stream=None):
    _check(_lib.sparse_attn_attend_raster(h.ptr, _io(h, q, "q"), _io(h, o, "o"), _lse(h, lse),
                                          _dptr(ws, "ws"), _nbytes(ws), _stream(stream)), h)


def sparse_attn_permute_inputs(h, q, k, v, ws, stream=None):
    _check(_lib.sparse_attn_permute_inputs(h.ptr, _io(h, q, "q"), _io(h, k, "k"), _io(h, v, "v"),
                                           _dptr(ws, "ws"), _nbytes(ws), _stream(stream)), h)


def sparse_attn_attend(h, ws, stream=None):
    _check(_lib.sparse_attn_attend(h.ptr, _dptr(ws, "ws"), _nbytes(ws), _stream(stream)), h)


def sparse_attn_unpermute_output(h, ws, o, stream=None):
    _check(_lib.sparse_attn_unpermute_output(h.ptr, _dptr(ws, "ws"), _nbytes(ws), _io(h, o, "o"),
                                             _stream(stream)), h)


def sparse_attn_permute(h, src, dst, layout=SPARSE_ATTN_LAYOUT_ROWS, stream=None):
    _check(_lib.sparse_attn_permute(h.ptr, _io(h, src, "src"),
                                    _sized(dst, "dst", h.sizes["slots"], elem=h.sizes["elem"]), int(layout),
                                    _stream(stream)), h)


def sparse_attn_unpermute(h, src, dst, stream=None):
    _check(_lib.sparse_attn_unpermute(h.ptr, _sized(src, "src", h.sizes["slots"], elem=h.sizes["elem"]),
                                      _io(h, dst, "dst"), _stream(stream)), h)


def sparse_attn_read_index_lists(h, row_ptr, cols, order, stream=None):
    R = h.sizes["heads"] * h.sizes["tiles"]
    _check(_lib.sparse_attn_read_index_lists(h.ptr, _sized(row_ptr, "row_ptr", 4 * (R + 1), elem=4, at_least=True),
                                             _sized(cols, "cols", 0, elem=4, at_least=True),
                                             cols.numel() if cols is not None else 0,
                                             _sized(order, "order", 4 * R, elem=4, at_least=True),
                                             _stream(stream)), h)


def sparse_attn_select_topk(h, k_per_head, ws, bitmap, stream=None):
    """Top-k tile bitmap from the permuted Q and K in ws (run
    sparse_attn_permute_inputs on ws first); bitmap: device uint8
    [heads, nT, nT]."""
    kh = _host_heads([int(x) for x in k_per_head], "k_per_head", h.cfg.heads)
    _check(_lib.sparse_attn_select_topk(h.ptr, kh.ctypes.data, _dptr(ws, "ws"), _nbytes(ws),
                                        _sized(bitmap, "bitmap", h.sizes["bitmap"], elem=1),
                                        _stream(stream)), h)


def sparse_attn_select_scope(h, rho, k_fixed, ws, bitmap, base=None, keep=None, stream=None):
    """Tile bitmap with the per-head Top-k estimate from the permuted Q and K
    in ws: per query tile the hybrid Top-p (rho) / fixed Top-k (k_fixed key
    tiles) base count, the head's weighted estimate, then each row's
    max(base, k_head) best key tiles.  base, keep: optional device int32
    [heads, nT] that receive the counts."""
    n = h.sizes["heads"] * h.sizes["tiles"] * 4
    _check(_lib.sparse_attn_select_scope(h.ptr, float(rho), int(k_fixed), _dptr(ws, "ws"), _nbytes(ws),
                                         _sized(bitmap, "bitmap", h.sizes["bitmap"], elem=1),
                                         _sized(base, "base", n, elem=4), _sized(keep, "keep", n, elem=4),
                                         _stream(stream)), h)


def sparse_attn_read_pair_lists(h, row_ptr, cols, order, flag, stream=None):
    mfma = sparse_attn_layout(h)["kernel"] == SPARSE_ATTN_KERNEL_MFMA_BF16
    R = h.sizes["heads"] * h.sizes["pairs"] if mfma else 0  # (UNSUPPORTED otherwise)
    _check(_lib.sparse_attn_read_pair_lists(h.ptr, _sized(row_ptr, "row_ptr", 4 * (R + 1), elem=4, at_least=True),
                                            _sized(cols, "cols", 0, elem=4, at_least=True),
                                            cols.numel() if cols is not None else 0,
                                            _sized(order, "order", 4 * R, elem=4, at_least=True),
                                            _sized(flag, "flag", 4 * R, elem=4, at_least=True),
                                            _stream(stream)), h)


def sparse_attn_mask_info(h, stream=None):
    nnz, ovf = _i64(), _i32()
    _check(_lib.sparse_attn_mask_info(h.ptr, ctypes.byref(nnz), ctypes.byref(ovf), _stream(stream)), h)
    return nnz.value, bool(ovf.value)


def sparse_attn_mix_probe(waves_per_simd, cus, iters, cycles, sink, pingpong=False, stream=None):
    """Diagnostic: the attention stage's instruction mix with nothing else
    in the way, in the row kernel's schedule (waves_per_simd unsynchronised
    waves per SIMD) or, with pingpong (waves_per_simd 2), the pair kernel's.
    cycles: device int64 tensor of cus * waves_per_simd * 4 elements (each
    wave's loop cycles, out); sink: device fp32 tensor of
    cus * waves_per_simd * 256 elements.  Asynchronous on `stream`."""
    n = int(cus) * int(waves_per_simd)
    cp = _sized(cycles, "cycles", n * 4 * 8, elem=8)
    sp = _sized(sink, "sink", n * 256 * 4, elem=4)
    _check(_lib.sparse_attn_mix_probe(int(waves_per_simd), int(bool(pingpong)), int(cus), int(iters), cp, sp,
                                      _stream(stream)))


class SparseAttention:
    """Convenience wrapper: one handle plus torch-allocated mask buffer and
    workspace on `device`."""

    def __init__(self, heads, head_dim, grid, tile, dtype="bf16", softmax_scale=0.0, device="cuda"):
        import torch
        self.torch = torch
        self.h = sparse_attn_create(heads, head_dim, grid, tile, dtype, softmax_scale)
        self.layout = sparse_attn_layout(self.h)
        self.device = device
        self.heads, self.head_dim = heads, head_dim
        self.ws = torch.empty(sparse_attn_workspace_bytes(self.h), dtype=torch.uint8, device=device)
        self.mask_buf = None

    def _mask_buf(self, max_nnz):
        need = sparse_attn_mask_bytes(self.h, max_nnz)
        if self.mask_buf is None or self.mask_buf.numel() < need:
            self.mask_buf = self.torch.empty(need, dtype=self.torch.uint8, device=self.device)
        return self.mask_buf

    def set_mask_bitmap(self, bitmap, max_nnz=0, stream=None):
        sparse_attn_set_mask(self.h, self._mask_buf(max_nnz), bitmap=bitmap, max_nnz=max_nnz,
                             stream=stream)

    def set_mask_windows(self, groups, groups_per_head, max_nnz=0, stream=None):
        sparse_attn_set_mask(self.h, self._mask_buf(max_nnz), groups=groups,
                             groups_per_head=groups_per_head, max_nnz=max_nnz, stream=stream)

    def forward(self, q, k, v, o=None, stream=None):
        if o is None:
            o = self.torch.empty_like(q)
        sparse_attn_forward(self.h, q, k, v, o, self.ws, stream)
        return o

    def close(self):
        """Destroys the handle (host state); the torch buffers go with the object."""
        if self.h is not None:
            sparse_attn_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def sparse_attn_tile_mass(h, q, k, ws, mass, stream=None):
    """Full-attention mass per tile pair into mass (device fp32 [heads, nT, nT])."""
    _check(_lib.sparse_attn_tile_mass(h.ptr, _io(h, q, "q"), _io(h, k, "k"), _dptr(ws, "ws"), _nbytes(ws),
                                      _sized(mass, "mass", h.sizes["mass"], elem=4), _stream(stream)), h)


def sparse_attn_search_windows(h, mass, groups, groups_per_head, tau, lam=float("inf")):
    """Host search.  mass: host float32 [heads, nT, nT]; groups: int32 [G, 6]
    rows (dt_lo, dt_hi, ...) (windows ignored); returns (groups [G, 6] with
    the searched windows, recall [heads], cost [heads])."""
    heads = h.cfg.heads
    nT = h.sizes["tiles"]
    m = np.ascontiguousarray(mass, dtype=np.float32)
    if m.size != heads * nT * nT:
        raise ValueError(f"mass: {m.size} values, expected heads * nT * nT = {heads * nT * nT}")
    g, gph = _host_groups(groups, groups_per_head, heads)
    out = np.zeros_like(g)
    rec = np.zeros(heads)
    cst = np.zeros(heads)
    _check(_lib.sparse_attn_search_windows(h.ptr, m.ctypes.data, g.ctypes.data, gph.ctypes.data,
                                           float(tau), float(lam), out.ctypes.data, rec.ctypes.data,
                                           cst.ctypes.data), h)
    return out, rec, cst

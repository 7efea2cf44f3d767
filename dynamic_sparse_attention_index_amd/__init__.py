"""Python binding of the vertical-slash sparse attention library (libvsattn.so).

Argument marshalling only: every step of the path runs in the gfx950 HIP
kernels behind the C ABI declared in include/vs_attn.h. PyTorch provides device
memory and streams. If the library has not been built, calling any entry point
raises; there is no fallback implementation.

Entry points (same names and meaning as the C ABI):
    vs_index_build, vs_block_mask, vs_attn_fwd, vs_merge_lse,
    vs_attn_bwd_prep, vs_attn_bwd, vs_convert_f16
plus helpers to size workspaces and hold a mask buffer (``Mask``).
"""
import contextlib
import ctypes
import os

import torch

from . import _build

# VS_ATTN_LIB names another build of the same library (the host-sanitizer
# build of the ABI checks); by default the in-tree libvsattn.so is loaded.
LIB_PATH = os.environ.get("VS_ATTN_LIB", _build.LIB)
# The same library with bounds checks on every mask value the attention
# kernels turn into an address (built beside it; see vs_debug_bounds_count).
DEBUG_LIB_PATH = _build.DEBUG_LIB

VS_OK, VS_ERR_ARG, VS_ERR_UNSUPPORTED, VS_ERR_WORKSPACE, VS_ERR_CAPACITY, VS_ERR_HIP = 0, -1, -2, -3, -4, -5
VS_ERR_RANGE = -6
VS_F32, VS_BF16, VS_F16 = 0, 1, 2
LAYOUTS = {"contig": 0, "striped": 1, "zigzag": 2, "striped1": 3}
TILE_DIAG = 0x40000000
TILE_MASK = 0x3FFFFFFF

EXPORTED = [
    "vs_status_string", "vs_index_workspace_size", "vs_index_build", "vs_index_rank_stats", "vs_index_rank_mass",
    "vs_index_select_workspace_size", "vs_index_select", "vs_index_select_budget", "vs_mask_bytes", "vs_mask_init",
    "vs_block_mask", "vs_attn_fwd", "vs_merge_lse", "vs_attn_bwd_prep", "vs_attn_bwd", "vs_attn_bwd_parts",
    "vs_convert_f16", "vs_index_select_group_workspace_size", "vs_index_select_group", "vs_attn_fwd_packed",
    "vs_attn_bwd_prep_f16", "vs_index_build_noalloc", "vs_attn_fwd_ring", "vs_attn_bwd_ring",
    "vs_block_mask_ring", "vs_debug_bounds_enabled", "vs_debug_bounds_count",
]
VS_BWD_DQ, VS_BWD_DKDV, VS_BWD_DKDV_VERT, VS_BWD_ALL, VS_BWD_OVERWRITE = 1, 2, 4, 7, 8


class VsTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int64), ("D", ctypes.c_int32), ("stride_h", ctypes.c_int64),
                ("stride_n", ctypes.c_int64)]


class VsLayout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("P", ctypes.c_int32), ("n_global", ctypes.c_int64)]


_P32 = ctypes.POINTER(ctypes.c_int32)


class VsMask(ctypes.Structure):
    _fields_ = [("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("QB", ctypes.c_int32), ("KB", ctypes.c_int32),
                ("T", ctypes.c_int32), ("W", ctypes.c_int32), ("lay", VsLayout), ("tile_cap", ctypes.c_int64),
                ("rank", ctypes.c_int32), ("src", ctypes.c_int32),
                ("tile_ptr", ctypes.c_void_p), ("tile_col", ctypes.c_void_p), ("csc_ptr", ctypes.c_void_p),
                ("csc_row", ctypes.c_void_p), ("vloc", ctypes.c_void_p), ("vloc_cnt", ctypes.c_void_p),
                ("vcum", ctypes.c_void_p), ("vert_end", ctypes.c_void_p), ("slash_bits", ctypes.c_void_p),
                ("n_active", ctypes.c_void_p), ("status", ctypes.c_void_p)]


class VsError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


_lib = None
_loaded = {}


def lib():
    """Load libvsattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Route every entry point through another build of the library at `path`
    (the bounds-checked debug build, DEBUG_LIB_PATH) inside the block."""
    global _lib
    prev = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def _load(path):
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    if True:
        L = ctypes.CDLL(path)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.vs_status_string.restype = ctypes.c_char_p
        L.vs_status_string.argtypes = [i32]
        L.vs_index_workspace_size.restype = sz
        L.vs_index_workspace_size.argtypes = [i32, i32, i64, i32, i32]
        L.vs_index_build.restype = i32
        L.vs_index_build.argtypes = [VsTensor, VsTensor, VsLayout, f32, f32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.vs_index_build_noalloc.restype = i32
        L.vs_index_build_noalloc.argtypes = [VsTensor, VsTensor, VsLayout, f32, f32, vp, vp, vp, vp, vp, vp, vp]
        L.vs_index_rank_stats.restype = i32
        L.vs_index_rank_stats.argtypes = [VsTensor, VsTensor, VsLayout, i32, f32, vp, vp, sz, vp]
        L.vs_index_rank_mass.restype = i32
        L.vs_index_rank_mass.argtypes = [VsTensor, VsTensor, VsLayout, i32, f32, vp, vp, vp, vp, sz, vp]
        L.vs_index_select.restype = i32
        L.vs_index_select.argtypes = [vp, vp, i32, i64, f32, vp, vp, vp, vp, vp, sz, vp]
        L.vs_index_select_budget.restype = i32
        L.vs_index_select_budget.argtypes = [vp, vp, i32, i64, i32, f32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.vs_index_select_workspace_size.restype = sz
        L.vs_index_select_workspace_size.argtypes = [i32, i64]
        L.vs_mask_bytes.restype = sz
        L.vs_mask_bytes.argtypes = [i32, i32, VsLayout, i64]
        L.vs_mask_init.restype = i32
        L.vs_mask_init.argtypes = [ctypes.POINTER(VsMask), vp, sz, i32, i32, VsLayout, i64]
        L.vs_block_mask.restype = i32
        L.vs_block_mask.argtypes = [vp, vp, i64, vp, vp, i64, i32, i32, ctypes.POINTER(VsMask), vp]
        L.vs_attn_fwd.restype = i32
        L.vs_attn_fwd.argtypes = [VsTensor, VsTensor, VsTensor, ctypes.POINTER(VsMask), f32, vp, vp, i32, vp]
        L.vs_merge_lse.restype = i32
        L.vs_merge_lse.argtypes = [vp, vp, vp, vp, i32, i64, i32, vp]
        L.vs_index_select_group_workspace_size.restype = sz
        L.vs_index_select_group_workspace_size.argtypes = [i32, i32, i64]
        L.vs_index_select_group.restype = i32
        L.vs_index_select_group.argtypes = [vp, vp, i32, i32, i64, f32, vp, vp, vp, vp, vp, sz, vp]
        L.vs_attn_fwd_packed.restype = i32
        L.vs_attn_fwd_packed.argtypes = [VsTensor, VsTensor, VsTensor, ctypes.POINTER(VsMask), f32, vp, vp, i32, vp,
                                         vp]
        L.vs_attn_bwd_prep_f16.restype = i32
        L.vs_attn_bwd_prep_f16.argtypes = [vp, vp, vp, i32, i64, i32, vp, vp, vp]
        L.vs_convert_f16.restype = i32
        L.vs_convert_f16.argtypes = [vp, vp, i64, vp, vp]
        L.vs_attn_bwd_prep.restype = i32
        L.vs_attn_bwd_prep.argtypes = [vp, VsTensor, vp, vp]
        L.vs_attn_bwd.restype = i32
        L.vs_attn_bwd.argtypes = [VsTensor, VsTensor, VsTensor, VsTensor, vp, vp, ctypes.POINTER(VsMask), f32,
                                  vp, vp, vp, vp]
        L.vs_block_mask_ring.restype = i32
        L.vs_block_mask_ring.argtypes = [vp, vp, i64, vp, vp, i64, i32, ctypes.POINTER(VsMask), i32, vp]
        L.vs_attn_fwd_ring.restype = i32
        L.vs_attn_fwd_ring.argtypes = [VsTensor, VsTensor, VsTensor, ctypes.POINTER(VsMask), i32, f32, vp, vp, i32,
                                       vp]
        L.vs_attn_bwd_ring.restype = i32
        L.vs_attn_bwd_ring.argtypes = [VsTensor, VsTensor, VsTensor, VsTensor, vp, vp, ctypes.POINTER(VsMask), i32,
                                       f32, vp, vp, vp, i32, vp]
        L.vs_attn_bwd_parts.restype = i32
        L.vs_attn_bwd_parts.argtypes = [VsTensor, VsTensor, VsTensor, VsTensor, vp, vp, ctypes.POINTER(VsMask),
                                        f32, vp, vp, vp, i32, vp]
        L.vs_debug_bounds_enabled.restype = i32
        L.vs_debug_bounds_enabled.argtypes = []
        L.vs_debug_bounds_count.restype = i32
        L.vs_debug_bounds_count.argtypes = [vp, i32, vp]
    _loaded[path] = L
    return L


def status_string(code):
    try:
        return lib().vs_status_string(code).decode()
    except RuntimeError:
        return str(code)


def _check(code, what):
    if code != VS_OK:
        raise VsError(code, what)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _cptr(t):
    """Pointer of a dense buffer argument (the ABI's plain float* arrays are
    contiguous [H, N(, D)]); a strided view would be read or written wrongly."""
    if not t.is_contiguous():
        raise VsError(VS_ERR_ARG, "non-contiguous buffer passed where the ABI takes a dense array")
    return ctypes.c_void_p(t.data_ptr())


def as_vs_tensor(t: torch.Tensor) -> VsTensor:
    """[H, N, D] torch view -> vs_tensor (no copy)."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a [H, N, D] tensor with contiguous D")
    if t.dtype == torch.bfloat16:
        dt = VS_BF16
    elif t.dtype == torch.float16:
        dt = VS_F16
    elif t.dtype == torch.float32:
        dt = VS_F32
    else:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return VsTensor(t.data_ptr(), dt, t.shape[0], t.shape[1], t.shape[2], t.stride(0), t.stride(1))


def layout(kind: str = "contig", P: int = 1, n_global: int = 0) -> VsLayout:
    return VsLayout(LAYOUTS[kind], P, n_global)


def index_workspace_size(Hq, Hkv, n_global, D, last_q=64) -> int:
    return int(lib().vs_index_workspace_size(Hq, Hkv, n_global, D, last_q))


def vs_index_build(q_last, k, lay: VsLayout, scale, top_p, vert_score, slash_score, vert_idx, vert_cnt,
                   slash_idx, slash_cnt, ws, stream=None):
    _check(lib().vs_index_build(as_vs_tensor(q_last), as_vs_tensor(k), lay, scale, top_p, _ptr(vert_score),
                                _ptr(slash_score), _ptr(vert_idx), _ptr(vert_cnt), _ptr(slash_idx),
                                _ptr(slash_cnt), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "vs_index_build")


def vs_index_build_noalloc(q_last, k, lay: VsLayout, scale, top_p, vert_score, slash_score, vert_idx, vert_cnt,
                           slash_idx, slash_cnt, stream=None):
    """vs_index_build with the library's own per-GPU scratch instead of a
    caller workspace (no allocation in the call)."""
    _check(lib().vs_index_build_noalloc(as_vs_tensor(q_last), as_vs_tensor(k), lay, scale, top_p, _ptr(vert_score),
                                        _ptr(slash_score), _ptr(vert_idx), _ptr(vert_cnt), _ptr(slash_idx),
                                        _ptr(slash_cnt), _stream(stream)),
           "vs_index_build_noalloc")


def vs_index_rank_stats(q_last, k_local, lay: VsLayout, rank, scale, stats, ws, stream=None):
    _check(lib().vs_index_rank_stats(as_vs_tensor(q_last), as_vs_tensor(k_local), lay, rank, scale, _cptr(stats),
                                     _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "vs_index_rank_stats")


def vs_index_rank_mass(q_last, k_local, lay: VsLayout, rank, scale, all_stats, vert_score, slash_score, ws,
                       stream=None):
    _check(lib().vs_index_rank_mass(as_vs_tensor(q_last), as_vs_tensor(k_local), lay, rank, scale,
                                    _cptr(all_stats), _cptr(vert_score), _cptr(slash_score), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "vs_index_rank_mass")


def index_select_workspace_size(Hq, n_global) -> int:
    return int(lib().vs_index_select_workspace_size(Hq, n_global))


def vs_index_select(vert_score, slash_score, Hq, n_global, top_p, vert_idx, vert_cnt, slash_idx, slash_cnt, ws,
                    stream=None):
    _check(lib().vs_index_select(_cptr(vert_score), _cptr(slash_score), Hq, n_global, top_p, _ptr(vert_idx),
                                 _ptr(vert_cnt), _ptr(slash_idx), _ptr(slash_cnt), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "vs_index_select")


VS_BUDGET_TOP_P = 0
VS_BUDGET_TOP_K = 1
VS_BUDGET_JOINT_TOP_P = 2


def vs_index_select_budget(vert_score, slash_score, Hq, n_global, budget, top_p, k_vert, k_slash, vert_idx, vert_cnt,
                           slash_idx, slash_cnt, ws, stream=None):
    _check(lib().vs_index_select_budget(_cptr(vert_score), _cptr(slash_score), Hq, n_global, int(budget), top_p,
                                        int(k_vert), int(k_slash), _ptr(vert_idx), _ptr(vert_cnt), _ptr(slash_idx),
                                        _ptr(slash_cnt), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "vs_index_select_budget")


class Mask:
    """A caller-owned device buffer carved into a vs_mask descriptor."""

    def __init__(self, Hq, Hkv, lay: VsLayout, tile_cap, device="cuda"):
        nbytes = int(lib().vs_mask_bytes(Hq, Hkv, lay, tile_cap))
        if nbytes == 0:
            raise VsError(VS_ERR_ARG, "vs_mask_bytes")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.desc = VsMask()
        _check(lib().vs_mask_init(ctypes.byref(self.desc), _ptr(self.buf), nbytes, Hq, Hkv, lay, tile_cap),
               "vs_mask_init")

    def _view(self, name, n, dtype):
        off = getattr(self.desc, name) - self.buf.data_ptr()
        esz = torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + n * esz].view(dtype)

    def arrays(self):
        d = self.desc
        n_csr, n_col = d.Hq * d.QB, d.tile_cap
        return {
            "tile_ptr": self._view("tile_ptr", n_csr + 1, torch.int32),
            "tile_col": self._view("tile_col", n_col, torch.int32),
            "csc_ptr": self._view("csc_ptr", d.Hq * d.KB + 1, torch.int32),
            "csc_row": self._view("csc_row", n_col, torch.int32),
            "vloc": self._view("vloc", d.Hq * d.KB * 64, torch.int32),
            "vloc_cnt": self._view("vloc_cnt", d.Hq, torch.int32),
            "vcum": self._view("vcum", d.Hq * (d.KB + 1), torch.int32),
            "vert_end": self._view("vert_end", d.Hq * d.QB, torch.int32),
            "slash_bits": self._view("slash_bits", d.Hq * d.W, torch.int32),
            "n_active": self._view("n_active", d.Hq * d.QB, torch.int64),
            "status": self._view("status", 1, torch.int32),
        }


def vs_block_mask(vert_idx, vert_cnt, slash_idx, slash_cnt, rank, step, mask: Mask, stream=None):
    _check(lib().vs_block_mask(_ptr(vert_idx), _ptr(vert_cnt), vert_idx.stride(0), _ptr(slash_idx),
                               _ptr(slash_cnt), slash_idx.stride(0), rank, step, ctypes.byref(mask.desc),
                               _stream(stream)), "vs_block_mask")


def vs_attn_fwd(q, k, v, mask: Mask, scale, o, lse, accumulate=0, stream=None):
    _check(lib().vs_attn_fwd(as_vs_tensor(q), as_vs_tensor(k), as_vs_tensor(v), ctypes.byref(mask.desc), scale,
                             _cptr(o), _cptr(lse), int(accumulate), _stream(stream)), "vs_attn_fwd")


def vs_attn_fwd_packed(q, k, v, mask: Mask, scale, o, lse, status, accumulate=0, stream=None):
    _check(lib().vs_attn_fwd_packed(as_vs_tensor(q), as_vs_tensor(k), as_vs_tensor(v), ctypes.byref(mask.desc),
                                    scale, _cptr(o), _cptr(lse), int(accumulate), _cptr(status), _stream(stream)),
           "vs_attn_fwd_packed")


def index_select_group_workspace_size(Hq, Hkv, n_global):
    return lib().vs_index_select_group_workspace_size(Hq, Hkv, n_global)


def vs_index_select_group(vert_score, slash_score, Hq, Hkv, n_global, top_p, vert_idx, vert_cnt, slash_idx,
                          slash_cnt, ws, stream=None):
    _check(lib().vs_index_select_group(_cptr(vert_score), _cptr(slash_score), Hq, Hkv, n_global, top_p,
                                       _cptr(vert_idx), _cptr(vert_cnt), _cptr(slash_idx), _cptr(slash_cnt),
                                       _cptr(ws), ws.numel(), _stream(stream)), "vs_index_select_group")


def vs_merge_lse(o_acc, lse_acc, o_step, lse_step, stream=None):
    Hq, Nq, D = o_acc.shape
    _check(lib().vs_merge_lse(_cptr(o_acc), _cptr(lse_acc), _cptr(o_step), _cptr(lse_step), Hq, Nq, D,
                              _stream(stream)), "vs_merge_lse")


def vs_convert_f16(src, dst, status, stream=None):
    """dst (float16) = exact fp16 copy of src (bfloat16), both dense with the
    same number of elements; status: one int32 device word the caller set to
    VS_OK, which receives VS_ERR_RANGE if a value is outside fp16's range."""
    if src.dtype != torch.bfloat16 or dst.dtype != torch.float16 or status.dtype != torch.int32:
        raise ValueError("vs_convert_f16 takes bfloat16 src, float16 dst and an int32 status word")
    if src.numel() != dst.numel():
        raise ValueError("src and dst differ in size")
    _check(lib().vs_convert_f16(_cptr(src), _cptr(dst), src.numel(), _cptr(status), _stream(stream)),
           "vs_convert_f16")


def vs_attn_bwd_prep_f16(o, dout, dout_f16, delta, status, stream=None):
    """delta from bf16 dout [Hq, Nq, D] (dense), writing its fp16 copy dout_f16."""
    if dout.dtype != torch.bfloat16 or dout_f16.dtype != torch.float16 or dout.shape != dout_f16.shape:
        raise ValueError("vs_attn_bwd_prep_f16 takes bfloat16 dout and a float16 dout_f16 of the same shape")
    Hq, Nq, D = dout.shape
    _check(lib().vs_attn_bwd_prep_f16(_cptr(o), _cptr(dout), _cptr(dout_f16), Hq, Nq, D, _cptr(delta),
                                      _cptr(status), _stream(stream)), "vs_attn_bwd_prep_f16")


def vs_attn_bwd_prep(o, dout, delta, stream=None):
    _check(lib().vs_attn_bwd_prep(_cptr(o), as_vs_tensor(dout), _cptr(delta), _stream(stream)), "vs_attn_bwd_prep")


def vs_attn_bwd(q, k, v, dout, lse, delta, mask: Mask, scale, dq, dk, dv, stream=None):
    _check(lib().vs_attn_bwd(as_vs_tensor(q), as_vs_tensor(k), as_vs_tensor(v), as_vs_tensor(dout), _cptr(lse),
                             _cptr(delta), ctypes.byref(mask.desc), scale, _cptr(dq), _cptr(dk), _cptr(dv),
                             _stream(stream)), "vs_attn_bwd")


def vs_attn_bwd_parts(q, k, v, dout, lse, delta, mask: Mask, scale, dq, dk, dv, parts, stream=None):
    _check(lib().vs_attn_bwd_parts(as_vs_tensor(q), as_vs_tensor(k), as_vs_tensor(v), as_vs_tensor(dout),
                                   _cptr(lse), _cptr(delta), ctypes.byref(mask.desc), scale, _cptr(dq), _cptr(dk),
                                   _cptr(dv), int(parts), _stream(stream)), "vs_attn_bwd_parts")


def _mask_array(masks):
    arr = (VsMask * len(masks))()
    for i, m in enumerate(masks):
        arr[i] = m.desc
    return arr


def vs_attn_fwd_ring(q, k_all, v_all, masks, scale, o, lse, accumulate=0, stream=None):
    """One rank's ring steps (`masks`: one Mask per step, filled by
    vs_block_mask) in one launch; k_all/v_all hold every shard in storage order."""
    arr = _mask_array(masks)
    _check(lib().vs_attn_fwd_ring(as_vs_tensor(q), as_vs_tensor(k_all), as_vs_tensor(v_all), arr, len(masks), scale,
                                  _cptr(o), _cptr(lse), int(accumulate), _stream(stream)), "vs_attn_fwd_ring")


def vs_attn_bwd_ring(q, k_all, v_all, dout, lse, delta, masks, scale, dq, dk_all, dv_all, parts=VS_BWD_ALL,
                     stream=None):
    arr = _mask_array(masks)
    _check(lib().vs_attn_bwd_ring(as_vs_tensor(q), as_vs_tensor(k_all), as_vs_tensor(v_all), as_vs_tensor(dout),
                                  _cptr(lse), _cptr(delta), arr, len(masks), scale, _cptr(dq), _cptr(dk_all),
                                  _cptr(dv_all), int(parts), _stream(stream)), "vs_attn_bwd_ring")


def vs_block_mask_ring(vert_idx, vert_cnt, slash_idx, slash_cnt, rank, masks, stream=None):
    """Steps 0 .. len(masks)-1 of `rank` into `masks` (Mask objects of one shape)."""
    arr = _mask_array(masks)
    _check(lib().vs_block_mask_ring(_ptr(vert_idx), _ptr(vert_cnt), vert_idx.stride(0), _ptr(slash_idx),
                                    _ptr(slash_cnt), slash_idx.stride(0), rank, arr, len(masks), _stream(stream)),
           "vs_block_mask_ring")
    for m, d in zip(masks, arr):     # the library set each descriptor's rank and visible shard
        m.desc = d


def debug_bounds_enabled() -> bool:
    return bool(lib().vs_debug_bounds_enabled())


def debug_bounds_count(reset: bool = True, stream=None) -> int:
    """Out-of-range mask values the attention kernels met since the last reset
    (always 0 for the release build, which has no checks)."""
    n = ctypes.c_int32(0)
    _check(lib().vs_debug_bounds_count(ctypes.byref(n), 1 if reset else 0, _stream(stream)), "vs_debug_bounds_count")
    return int(n.value)

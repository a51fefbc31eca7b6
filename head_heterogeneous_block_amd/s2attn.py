"""Python binding of libs2attn (include/s2attn.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the method: it checks device / dtype / dimensions, passes
``data_ptr()``, strides and torch's current HIP stream, and raises S2Error on
a non-zero status.  The library must be built (``__graft_entry__.build()``);
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # imported first: the library then binds torch's HIP runtime

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libs2attn.so")

S2_OK, S2_EINVAL, S2_EUNSUPPORTED, S2_ECAPACITY, S2_EHIP = range(5)
S2_F32, S2_BF16 = 0, 1
S2_BLOCK = 64
_STATUS_NAMES = {0: "S2_OK", 1: "S2_EINVAL", 2: "S2_EUNSUPPORTED", 3: "S2_ECAPACITY", 4: "S2_EHIP"}
_DTYPES = {torch.float32: S2_F32, torch.bfloat16: S2_BF16}

EXPORTED = ["s2_abi_version", "s2_last_error", "s2_layout_nnz", "s2_build_layout", "s2_attn_fwd_workspace",
            "s2_attn_fwd",
            "s2_attn_decode_workspace", "s2_attn_decode", "s2_build_layout_t", "s2_attn_bwd_workspace",
            "s2_attn_bwd", "s2_attn_decode_paged_workspace", "s2_attn_decode_paged", "s2_validate_layout",
            "s2_transpose_layout_workspace", "s2_transpose_layout", "s2_attn_fwd_varlen", "s2_block_minmax",
            "s2_select_blocks", "s2_attn_decode_rows_workspace", "s2_attn_decode_rows", "s2_block_minmax_paged",
            "s2_attn_decode_paged_rows_workspace", "s2_attn_decode_paged_rows", "s2_attn_decode_noalloc"]


class S2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _Pattern(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("local_blocks", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("dense", ctypes.POINTER(ctypes.c_uint8))]


class _Layout(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("num_q_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libs2attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.s2_abi_version.restype = i32
    lib.s2_last_error.restype = ctypes.c_char_p
    lib.s2_layout_nnz.argtypes = [ctypes.POINTER(_Pattern), i32, p64]
    lib.s2_build_layout.argtypes = [ctypes.POINTER(_Pattern), i32, vp, vp, i64, vp]
    lib.s2_attn_fwd_workspace.argtypes = [ctypes.POINTER(sz)]
    lib.s2_attn_fwd.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32, i32,
                                vp, p64, vp, p64, vp, p64, vp, p64, vp, vp, sz, f32, vp]
    lib.s2_attn_decode_workspace.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32,
                                             ctypes.POINTER(sz)]
    lib.s2_attn_decode_noalloc.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32, vp, p64, vp, p64, vp, p64,
                                           vp, i32, vp, p64, vp, i32, f32, vp]
    lib.s2_attn_decode.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32, vp, p64, vp, p64, vp, p64,
                                   vp, i32, vp, p64, vp, i32, vp, sz, f32, vp]
    lib.s2_build_layout_t.argtypes = [ctypes.POINTER(_Pattern), i32, vp, vp, i64, vp]
    lib.s2_attn_bwd_workspace.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    lib.s2_attn_bwd.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(_Layout), i32, i32, i32, i32,
                                vp, p64, vp, p64, vp, p64, vp, p64, vp, p64, vp,
                                vp, p64, vp, p64, vp, p64, vp, sz, f32, vp]
    lib.s2_attn_decode_paged_workspace.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32, i32,
                                                   ctypes.POINTER(sz)]
    lib.s2_attn_decode_paged.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32, i32, vp, p64, vp, p64,
                                         vp, p64, i32, i32, vp, i64, i32, vp, vp, p64, vp, i32, vp, sz,
                                         f32, vp]
    lib.s2_attn_fwd_varlen.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32, i32, vp, vp, p64, vp, p64,
                                       vp, p64, vp, p64, vp, vp, sz, f32, vp]
    lib.s2_validate_layout.argtypes = [ctypes.POINTER(_Layout), vp, vp]
    lib.s2_transpose_layout_workspace.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(sz)]
    lib.s2_transpose_layout.argtypes = [ctypes.POINTER(_Layout), vp, vp, i64, vp, sz, vp]
    lib.s2_block_minmax.argtypes = [i32, i32, i32, i32, vp, p64, vp, i32, vp, vp, i32, vp]
    lib.s2_select_blocks.argtypes = [i32, i32, i32, i32, i32, vp, p64, vp, vp, i32, vp, i32, i32, vp, vp, i64, vp]
    lib.s2_block_minmax_paged.argtypes = [i32, i32, i32, i32, vp, p64, i32, i32, vp, i64, i32, vp, vp, vp, i32, vp]
    lib.s2_attn_decode_paged_rows_workspace.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.s2_attn_decode_paged_rows.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, vp, p64, vp, p64, vp, p64,
                                              i32, i32, vp, i64, i32, vp, vp, p64, vp, i32, vp, sz, f32, vp]
    lib.s2_attn_decode_rows_workspace.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.s2_attn_decode_rows.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp, p64, vp, p64, vp, p64, vp, i32,
                                        vp, p64, vp, i32, vp, sz, f32, vp]
    for name in EXPORTED[2:]:
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != S2_OK:
        raise S2Error(status, library().s2_last_error().decode())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _strides(t: torch.Tensor):
    return (ctypes.c_int64 * t.dim())(*t.stride())


@dataclass
class Pattern:
    """HHST pattern: window of `local_blocks` key blocks ending at the diagonal,
    head-offset strided blocks (j + h) % stride == 0, optional dense heads."""
    num_heads: int
    local_blocks: int
    stride: int
    dense_heads: tuple = ()
    block_size: int = S2_BLOCK

    def _c(self):
        flags = (ctypes.c_uint8 * max(1, self.num_heads))()
        for h in self.dense_heads:
            if 0 <= h < self.num_heads:
                flags[h] = 1
        pt = _Pattern(self.num_heads, self.block_size, self.local_blocks, self.stride,
                      ctypes.cast(flags, ctypes.POINTER(ctypes.c_uint8)))
        return pt, flags


@dataclass
class Layout:
    """CSR layout on the device (row_ptr int32 [H*nqb+1], col_idx int32 [nnz])."""
    num_heads: int
    num_q_blocks: int
    nnz: int
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    block_size: int = S2_BLOCK

    def _c(self):
        return _Layout(self.num_heads, self.num_q_blocks, self.block_size, self.nnz,
                       self.row_ptr.data_ptr(), self.col_idx.data_ptr())


def s2_abi_version() -> int:
    return int(library().s2_abi_version())


def s2_last_error() -> str:
    return library().s2_last_error().decode()


def s2_layout_nnz(pattern: Pattern, num_q_blocks: int) -> int:
    pt, _keep = pattern._c()
    n = ctypes.c_int64(0)
    _check(library().s2_layout_nnz(ctypes.byref(pt), num_q_blocks, ctypes.byref(n)))
    return int(n.value)


def s2_build_layout(pattern: Pattern, num_q_blocks: int, device="cuda", row_ptr=None,
                    col_idx=None) -> Layout:
    device = torch.device(device)
    nnz = s2_layout_nnz(pattern, num_q_blocks)
    rows = pattern.num_heads * num_q_blocks
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=device)
    if col_idx is None:
        col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr / col_idx must be int32")
    if row_ptr.numel() < rows + 1:
        raise ValueError("row_ptr too small")
    pt, _keep = pattern._c()
    _check(library().s2_build_layout(ctypes.byref(pt), num_q_blocks, row_ptr.data_ptr(),
                                     col_idx.data_ptr(), col_idx.numel(), _stream(device)))
    return Layout(pattern.num_heads, num_q_blocks, nnz, row_ptr, col_idx, pattern.block_size)


def s2_build_layout_t(pattern: Pattern, num_q_blocks: int, device="cuda", col_ptr=None,
                      row_idx=None) -> Layout:
    """Column view of the pattern's layout (query blocks per key block), as a Layout
    whose row_ptr / col_idx are the column pointers / query-block indices."""
    device = torch.device(device)
    nnz = s2_layout_nnz(pattern, num_q_blocks)
    cols = pattern.num_heads * num_q_blocks
    if col_ptr is None:
        col_ptr = torch.empty(cols + 1, dtype=torch.int32, device=device)
    if row_idx is None:
        row_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)
    if col_ptr.dtype != torch.int32 or row_idx.dtype != torch.int32:
        raise ValueError("col_ptr / row_idx must be int32")
    if col_ptr.numel() < cols + 1:
        raise ValueError("col_ptr too small")
    pt, _keep = pattern._c()
    _check(library().s2_build_layout_t(ctypes.byref(pt), num_q_blocks, col_ptr.data_ptr(),
                                       row_idx.data_ptr(), row_idx.numel(), _stream(device)))
    return Layout(pattern.num_heads, num_q_blocks, nnz, col_ptr, row_idx, pattern.block_size)


def s2_validate_layout(layout: Layout) -> None:
    """Check a layout on the device (synchronous); raises S2Error naming the first bad row."""
    dev = layout.row_ptr.device
    scratch = torch.empty(1, dtype=torch.int64, device=dev)
    ly = layout._c()
    _check(library().s2_validate_layout(ctypes.byref(ly), scratch.data_ptr(), _stream(dev)))


def layout_from_csr(row_ptr: torch.Tensor, col_idx: torch.Tensor, num_heads: int, num_q_blocks: int,
                    validate: bool = True) -> Layout:
    """A caller-built layout: device int32 row_ptr [H * nqb + 1] (head-major rows) and
    col_idx [nnz], strictly ascending key blocks j <= i in each row."""
    _dev_tensor("row_ptr", row_ptr, 1, torch.int32)
    _dev_tensor("col_idx", col_idx, 1, torch.int32)
    if row_ptr.numel() != num_heads * num_q_blocks + 1 or not row_ptr.is_contiguous() \
            or not col_idx.is_contiguous():
        raise ValueError("row_ptr must be contiguous [num_heads * num_q_blocks + 1], col_idx contiguous")
    ly = Layout(num_heads, num_q_blocks, int(col_idx.numel()), row_ptr, col_idx)
    if validate:
        s2_validate_layout(ly)
    return ly


def s2_transpose_layout_workspace(layout: Layout) -> int:
    n = ctypes.c_size_t(0)
    ly = layout._c()
    _check(library().s2_transpose_layout_workspace(ctypes.byref(ly), ctypes.byref(n)))
    return int(n.value)


def s2_transpose_layout(layout: Layout, col_ptr=None, row_idx=None, workspace=None) -> Layout:
    """Column view of any valid layout (query blocks per key block), as a Layout."""
    dev = layout.row_ptr.device
    cols = layout.num_heads * layout.num_q_blocks
    if col_ptr is None:
        col_ptr = torch.empty(cols + 1, dtype=torch.int32, device=dev)
    if row_idx is None:
        row_idx = torch.empty(max(layout.nnz, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(s2_transpose_layout_workspace(layout), dtype=torch.uint8, device=dev)
    ly = layout._c()
    _check(library().s2_transpose_layout(ctypes.byref(ly), col_ptr.data_ptr(), row_idx.data_ptr(), row_idx.numel(),
                                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                         _stream(dev)))
    return Layout(layout.num_heads, layout.num_q_blocks, layout.nnz, col_ptr, row_idx, layout.block_size)


def _dev_tensor(name, t, ndim, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def s2_attn_fwd_workspace() -> int:
    n = ctypes.c_size_t(0)
    _check(library().s2_attn_fwd_workspace(ctypes.byref(n)))
    return int(n.value)


def _fwd_workspace(workspace, device):
    """The caller's forward workspace, or a new one (any content is valid)."""
    need = s2_attn_fwd_workspace()
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _dev_tensor("workspace", workspace, 1)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    return workspace


def s2_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: Layout,
                sm_scale: float = 0.0, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                want_lse: bool = True, workspace: torch.Tensor | None = None):
    """q, k, v: [B, H, N, D] (fp32 or bf16, any strides with D contiguous).

    Returns (o, lse); o has q's dtype and shape, lse is fp32 [B, H, N] (or None).
    workspace: s2_attn_fwd_workspace() bytes of device memory, any content (a new
    one is made if None); launches in flight together need separate workspaces."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(name, t, 4, q.dtype)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, N, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _dev_tensor("out", out, 4, q.dtype)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H, N)):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    ws = _fwd_workspace(workspace, q.device)
    ly = layout._c()
    _check(library().s2_attn_fwd(
        ctypes.byref(ly), _DTYPES[q.dtype], B, N, D,
        q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
        out.data_ptr(), _strides(out), lse.data_ptr() if lse is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), float(sm_scale), _stream(q.device)))
    return out, lse


def _varlen_args(q, k, v, cu_seqlens, out, lse, workspace, sm_scale):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dev_tensor(name, t, 3, torch.bfloat16)
    _dev_tensor("cu_seqlens", cu_seqlens, 1, torch.int32)
    T, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, k, v and out must all be [T_total, H, D]")
    if not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous int32 [B + 1] tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (H, T)):
        raise ValueError("lse must be a contiguous fp32 [H, T_total] tensor")
    return (S2_BF16, cu_seqlens.numel() - 1, T, D, cu_seqlens.data_ptr(), q.data_ptr(), _strides(q),
            k.data_ptr(), _strides(k), v.data_ptr(), _strides(v), out.data_ptr(), _strides(out),
            lse.data_ptr() if lse is not None else None,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), float(sm_scale))


def s2_attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                       layout: Layout, sm_scale: float = 0.0, out: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, want_lse: bool = True,
                       workspace: torch.Tensor | None = None):
    """Packed variable-length forward.  q, k, v: bf16 [T_total, H, D] (D contiguous);
    cu_seqlens: device int32 [B + 1].  Returns (o [T_total, H, D], lse fp32 [H, T_total] or None)."""
    _dev_tensor("q", q, 3, torch.bfloat16)
    T, H, D = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if want_lse and lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    ws = _fwd_workspace(workspace, q.device)
    ly = layout._c()
    _check(library().s2_attn_fwd_varlen(ctypes.byref(ly),
                                        *_varlen_args(q, k, v, cu_seqlens, out, lse, ws, sm_scale),
                                        _stream(q.device)))
    return out, lse


def s2_attn_decode_workspace(layout: Layout, B: int, D: int, splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    ly = layout._c()
    _check(library().s2_attn_decode_workspace(ctypes.byref(ly), B, D, splits, ctypes.byref(n)))
    return int(n.value)


def s2_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seq_lens: torch.Tensor, layout: Layout, splits: int = 0, sm_scale: float = 0.0,
                   workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, want_lse: bool = True):
    """q: [B, H, D]; k_cache, v_cache: [B, H, cache_len, D]; seq_lens: int32 [B] on the device.

    Returns (o [B, H, D] in q's dtype, lse fp32 [B, H] or None)."""
    _dev_tensor("q", q, 3)
    _dev_tensor("k_cache", k_cache, 4, q.dtype)
    _dev_tensor("v_cache", v_cache, 4, q.dtype)
    _dev_tensor("seq_lens", seq_lens, 1, torch.int32)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[:2] != (B, H) or k_cache.shape[3] != D:
        raise ValueError("cache shapes must be [B, H, cache_len, D] matching q")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    cache_len = k_cache.shape[2]
    if out is None:
        out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = s2_attn_decode_workspace(layout, B, D, splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ly = layout._c()
    _check(library().s2_attn_decode(
        ctypes.byref(ly), _DTYPES[q.dtype], B, D, q.data_ptr(), _strides(q),
        k_cache.data_ptr(), _strides(k_cache), v_cache.data_ptr(), _strides(v_cache),
        seq_lens.data_ptr(), cache_len, out.data_ptr(), _strides(out),
        lse.data_ptr() if lse is not None else None, splits, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), float(sm_scale), _stream(q.device)))
    return out, lse


S2_NOALLOC_SCRATCH_BYTES = 16 << 20


def s2_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           seq_lens: torch.Tensor, layout: Layout, out: torch.Tensor,
                           lse: torch.Tensor | None = None, splits: int = 0, sm_scale: float = 0.0):
    """s2_attn_decode without a workspace: the library's static per-GPU scratch holds the
    split partials, and nothing is allocated (the caller passes out and lse).  Calls
    that overlap in time on one GPU race; calls in stream order are safe."""
    _dev_tensor("q", q, 3)
    _dev_tensor("k_cache", k_cache, 4, q.dtype)
    _dev_tensor("v_cache", v_cache, 4, q.dtype)
    _dev_tensor("seq_lens", seq_lens, 1, torch.int32)
    _dev_tensor("out", out, 3, q.dtype)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[:2] != (B, H) or k_cache.shape[3] != D:
        raise ValueError("cache shapes must be [B, H, cache_len, D] matching q")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B, H, D]")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H)):
        raise ValueError("lse must be a contiguous fp32 [B, H] tensor")
    ly = layout._c()
    _check(library().s2_attn_decode_noalloc(
        ctypes.byref(ly), _DTYPES[q.dtype], B, D, q.data_ptr(), _strides(q),
        k_cache.data_ptr(), _strides(k_cache), v_cache.data_ptr(), _strides(v_cache),
        seq_lens.data_ptr(), k_cache.shape[2], out.data_ptr(), _strides(out),
        lse.data_ptr() if lse is not None else None, splits, float(sm_scale), _stream(q.device)))
    return out, lse


def s2_attn_decode_paged_workspace(layout: Layout, B: int, num_kv_heads: int, D: int,
                                   splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    ly = layout._c()
    _check(library().s2_attn_decode_paged_workspace(ctypes.byref(ly), B, num_kv_heads, D, splits,
                                                    ctypes.byref(n)))
    return int(n.value)


def _paged_args(q, k_pages, v_pages, block_table, seq_lens, layout: Layout, out, lse, workspace,
                splits: int, sm_scale: float):
    _dev_tensor("q", q, 3)
    _dev_tensor("k_pages", k_pages, 4, q.dtype)
    _dev_tensor("v_pages", v_pages, 4, q.dtype)
    _dev_tensor("block_table", block_table, 2, torch.int32)
    _dev_tensor("seq_lens", seq_lens, 1, torch.int32)
    _dev_tensor("out", out, 3, q.dtype)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, D = q.shape
    num_pages, Hkv, P, Dk = k_pages.shape
    if v_pages.shape != k_pages.shape or Dk != D:
        raise ValueError("k_pages and v_pages must be [num_pages, num_kv_heads, page_size, D]")
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B, H, D]")
    if block_table.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [B, max_pages] with unit inner stride")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H)):
        raise ValueError("lse must be a contiguous fp32 [B, H] tensor")
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if workspace is not None \
        else (None, 0)
    return (_DTYPES[q.dtype], B, Hkv, D, q.data_ptr(), _strides(q), k_pages.data_ptr(), _strides(k_pages),
            v_pages.data_ptr(), _strides(v_pages), num_pages, P, block_table.data_ptr(),
            block_table.stride(0), block_table.shape[1], seq_lens.data_ptr(), out.data_ptr(),
            _strides(out), lse.data_ptr() if lse is not None else None, splits, ws[0], ws[1],
            float(sm_scale))


def s2_attn_decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, layout: Layout,
                         splits: int = 0, sm_scale: float = 0.0, workspace: torch.Tensor | None = None,
                         out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                         want_lse: bool = True):
    """Serving decode over a paged cache.  q: [B, H, D]; k_pages, v_pages:
    [num_pages, H_kv, page_size, D] (H_kv divides H); block_table: int32 [B, max_pages];
    seq_lens: int32 [B].  Returns (o [B, H, D] in q's dtype, lse fp32 [B, H] or None)."""
    _dev_tensor("q", q, 3)
    B, H, D = q.shape
    if out is None:
        out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = s2_attn_decode_paged_workspace(layout, B, k_pages.shape[1], D, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ly = layout._c()
    _check(library().s2_attn_decode_paged(
        ctypes.byref(ly), *_paged_args(q, k_pages, v_pages, block_table, seq_lens, layout, out, lse,
                                       workspace, splits, sm_scale), _stream(q.device)))
    return out, lse


def s2_attn_bwd_workspace(B: int, H: int, N: int) -> int:
    n = ctypes.c_size_t(0)
    _check(library().s2_attn_bwd_workspace(B, H, N, ctypes.byref(n)))
    return int(n.value)


def s2_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                dout: torch.Tensor, lse: torch.Tensor, layout: Layout, layout_t: Layout,
                sm_scale: float = 0.0, dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """q, k, v, o, dout: bf16 [B, H, N, D] (D contiguous); lse: fp32 [B, H, N] from the
    forward; layout_t: s2_build_layout_t of the same pattern.  Returns (dq, dk, dv)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev_tensor(name, t, 4, torch.bfloat16)
    B, H, N, D = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have q's shape")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q, memory_format=torch.contiguous_format)
        _dev_tensor(name, t, 4, torch.bfloat16)
        outs.append(t)
    dq, dk, dv = outs
    need = s2_attn_bwd_workspace(B, H, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ly, lt = layout._c(), layout_t._c()
    _check(library().s2_attn_bwd(
        ctypes.byref(ly), ctypes.byref(lt), _DTYPES[q.dtype], B, N, D,
        q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
        o.data_ptr(), _strides(o), dout.data_ptr(), _strides(dout), lse.data_ptr(),
        dq.data_ptr(), _strides(dq), dk.data_ptr(), _strides(dk), dv.data_ptr(), _strides(dv),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), float(sm_scale),
        _stream(q.device)))
    return dq, dk, dv


class PreparedFwd:
    """s2_attn_fwd with its arguments marshalled once (for tight loops and benches).

    Calling it enqueues the same launch on torch's current stream; the tensors
    passed at construction must stay alive and unchanged in shape/strides."""

    def __init__(self, q, k, v, layout: Layout, out, lse=None, sm_scale: float = 0.0, workspace=None):
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            _dev_tensor(name, t, 4, q.dtype)
        self._lib = library()
        self._ly = layout._c()
        ws = _fwd_workspace(workspace, q.device)
        self._keep = (q, k, v, out, lse, layout, ws)
        self._strides = [_strides(t) for t in (q, k, v, out)]
        B, _, N, D = q.shape
        self._args = (ctypes.byref(self._ly), _DTYPES[q.dtype], B, N, D,
                      q.data_ptr(), self._strides[0], k.data_ptr(), self._strides[1],
                      v.data_ptr(), self._strides[2], out.data_ptr(), self._strides[3],
                      lse.data_ptr() if lse is not None else None,
                      ws.data_ptr(), ws.numel() * ws.element_size(), float(sm_scale))
        self._device = q.device

    def __call__(self):
        _check(self._lib.s2_attn_fwd(*self._args, _stream(self._device)))


class PreparedBwd:
    """s2_attn_bwd with its arguments marshalled once; the tensors passed at
    construction must stay alive and unchanged in shape/strides."""

    def __init__(self, q, k, v, o, dout, lse, layout: Layout, layout_t: Layout, dq, dk, dv,
                 workspace, sm_scale: float = 0.0):
        for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                        ("dk", dk), ("dv", dv)):
            _dev_tensor(name, t, 4, torch.bfloat16)
        self._lib = library()
        self._ly, self._lt = layout._c(), layout_t._c()
        self._keep = (q, k, v, o, dout, lse, dq, dk, dv, workspace, layout, layout_t)
        st = [_strides(t) for t in (q, k, v, o, dout, dq, dk, dv)]
        self._strides = st
        B, _, N, D = q.shape
        self._args = (ctypes.byref(self._ly), ctypes.byref(self._lt), _DTYPES[q.dtype], B, N, D,
                      q.data_ptr(), st[0], k.data_ptr(), st[1], v.data_ptr(), st[2],
                      o.data_ptr(), st[3], dout.data_ptr(), st[4], lse.data_ptr(),
                      dq.data_ptr(), st[5], dk.data_ptr(), st[6], dv.data_ptr(), st[7],
                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                      float(sm_scale))
        self._device = q.device

    def __call__(self):
        _check(self._lib.s2_attn_bwd(*self._args, _stream(self._device)))


class PreparedLayout:
    """s2_build_layout into fixed row_ptr / col_idx buffers, arguments marshalled once."""

    def __init__(self, pattern: Pattern, num_q_blocks: int, layout: Layout):
        self._lib = library()
        self._pt, self._flags = pattern._c()
        self._args = (ctypes.byref(self._pt), num_q_blocks, layout.row_ptr.data_ptr(),
                      layout.col_idx.data_ptr(), layout.col_idx.numel())
        self._keep = layout
        self._device = layout.row_ptr.device

    def __call__(self):
        _check(self._lib.s2_build_layout(*self._args, _stream(self._device)))


class PreparedDecode:
    """s2_attn_decode with its arguments marshalled once."""

    def __init__(self, q, k_cache, v_cache, seq_lens, layout: Layout, out, lse, workspace,
                 splits: int = 0, sm_scale: float = 0.0):
        _dev_tensor("q", q, 3)
        self._lib = library()
        self._ly = layout._c()
        self._keep = (q, k_cache, v_cache, seq_lens, out, lse, workspace, layout)
        st = [_strides(t) for t in (q, k_cache, v_cache, out)]
        self._st = st
        B, _, D = q.shape
        self._args = (ctypes.byref(self._ly), _DTYPES[q.dtype], B, D, q.data_ptr(), st[0],
                      k_cache.data_ptr(), st[1], v_cache.data_ptr(), st[2], seq_lens.data_ptr(),
                      k_cache.shape[2], out.data_ptr(), st[3],
                      lse.data_ptr() if lse is not None else None, splits, workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), float(sm_scale))
        self._device = q.device

    def __call__(self):
        _check(self._lib.s2_attn_decode(*self._args, _stream(self._device)))


class PreparedDecodePaged:
    """s2_attn_decode_paged with its arguments marshalled once."""

    def __init__(self, q, k_pages, v_pages, block_table, seq_lens, layout: Layout, out, lse=None,
                 workspace=None, splits: int = 0, sm_scale: float = 0.0):
        self._lib = library()
        self._ly = layout._c()
        self._keep = (q, k_pages, v_pages, block_table, seq_lens, out, lse, workspace, layout)
        self._args = _paged_args(q, k_pages, v_pages, block_table, seq_lens, layout, out, lse,
                                 workspace, splits, sm_scale)
        self._device = q.device

    def __call__(self):
        _check(self._lib.s2_attn_decode_paged(ctypes.byref(self._ly), *self._args,
                                              _stream(self._device)))


class PreparedFwdVarlen:
    """s2_attn_fwd_varlen with its arguments marshalled once."""

    def __init__(self, q, k, v, cu_seqlens, layout: Layout, out, lse=None, sm_scale: float = 0.0,
                 workspace=None):
        self._lib = library()
        self._ly = layout._c()
        ws = _fwd_workspace(workspace, q.device)
        self._keep = (q, k, v, cu_seqlens, out, lse, layout, ws)
        self._args = _varlen_args(q, k, v, cu_seqlens, out, lse, ws, sm_scale)
        self._device = q.device

    def __call__(self):
        _check(self._lib.s2_attn_fwd_varlen(ctypes.byref(self._ly), *self._args, _stream(self._device)))


# ---- query-aware block lists (per-block key bounds, top-budget rows, decode over them) ----

def s2_block_minmax(k_cache: torch.Tensor, seq_lens: torch.Tensor, num_blocks: int | None = None,
                    kmin: torch.Tensor | None = None, kmax: torch.Tensor | None = None):
    """Channel-wise key minima and maxima per 64-token block.

    k_cache: [B, H, cache_len, D]; seq_lens: int32 [B] on the device.  Returns
    (kmin, kmax), [B, H, num_blocks, D] contiguous in the keys' dtype; blocks at
    or past a sequence's length keep whatever the buffers held."""
    _dev_tensor("k_cache", k_cache, 4)
    _dev_tensor("seq_lens", seq_lens, 1, torch.int32)
    if k_cache.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k_cache.dtype}")
    B, H, L, D = k_cache.shape
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    nb = -(-L // S2_BLOCK) if num_blocks is None else num_blocks
    shape = (B, H, nb, D)
    if kmin is None:
        kmin = torch.empty(shape, dtype=k_cache.dtype, device=k_cache.device)
    if kmax is None:
        kmax = torch.empty(shape, dtype=k_cache.dtype, device=k_cache.device)
    for name, t in (("kmin", kmin), ("kmax", kmax)):
        _dev_tensor(name, t, 4, k_cache.dtype)
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {list(shape)} tensor")
    _check(library().s2_block_minmax(_DTYPES[k_cache.dtype], B, H, D, k_cache.data_ptr(), _strides(k_cache),
                                      seq_lens.data_ptr(), L, kmin.data_ptr(), kmax.data_ptr(), nb,
                                      _stream(k_cache.device)))
    return kmin, kmax


def _select_args(q, kmin, kmax, seq_lens, budget: int, cache_len: int, row_ptr, col_idx):
    _dev_tensor("q", q, 3)
    _dev_tensor("kmin", kmin, 4, q.dtype)
    _dev_tensor("kmax", kmax, 4, q.dtype)
    _dev_tensor("seq_lens", seq_lens, 1, torch.int32)
    _dev_tensor("row_ptr", row_ptr, 1, torch.int32)
    _dev_tensor("col_idx", col_idx, 1, torch.int32)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, D = q.shape
    Hkv = kmin.shape[1]
    if kmin.shape != kmax.shape or kmin.shape[0] != B or kmin.shape[3] != D or H % Hkv != 0:
        raise ValueError("kmin and kmax must be [B, H_kv, num_blocks, D] matching q, H_kv dividing H")
    if not (kmin.is_contiguous() and kmax.is_contiguous()):
        raise ValueError("kmin and kmax must be contiguous")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    if row_ptr.numel() != B * H + 1 or not row_ptr.is_contiguous() or not col_idx.is_contiguous():
        raise ValueError("row_ptr must be a contiguous int32 [B * H + 1] tensor and col_idx contiguous")
    return (_DTYPES[q.dtype], B, H, Hkv, D, q.data_ptr(), _strides(q), kmin.data_ptr(), kmax.data_ptr(),
            kmin.shape[2], seq_lens.data_ptr(), cache_len, budget, row_ptr.data_ptr(), col_idx.data_ptr(),
            col_idx.numel())


def s2_select_blocks(q: torch.Tensor, kmin: torch.Tensor, kmax: torch.Tensor, seq_lens: torch.Tensor,
                     budget: int, cache_len: int, row_ptr: torch.Tensor | None = None,
                     col_idx: torch.Tensor | None = None):
    """Per-(sequence, head) lists of the query's block and the budget - 1 earlier
    blocks with the largest key-bound scores.  kmin, kmax: [B, H_kv, num_blocks, D]
    (query head h ranks K/V head h // (H / H_kv)).  cache_len: the longest
    sequence the bounds can cover (for a paged cache, max_pages * page_size).
    Returns (row_ptr [B*H+1], col_idx), int32 on the device; row b * H + h belongs
    to sequence b, head h."""
    B, H, _ = q.shape
    if row_ptr is None:
        row_ptr = torch.empty(B * H + 1, dtype=torch.int32, device=q.device)
    if col_idx is None:
        col_idx = torch.empty(B * H * min(budget, -(-cache_len // S2_BLOCK)), dtype=torch.int32,
                              device=q.device)
    _check(library().s2_select_blocks(*_select_args(q, kmin, kmax, seq_lens, budget, cache_len, row_ptr,
                                                    col_idx), _stream(q.device)))
    return row_ptr, col_idx


def s2_attn_decode_rows_workspace(B: int, H: int, D: int, max_row_blocks: int, splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(library().s2_attn_decode_rows_workspace(B, H, D, max_row_blocks, splits, ctypes.byref(n)))
    return int(n.value)


def _rows_args(q, k_cache, v_cache, seq_lens, row_ptr, col_idx, max_row_blocks: int, out, lse, workspace,
               splits: int, sm_scale: float):
    _dev_tensor("q", q, 3)
    _dev_tensor("k_cache", k_cache, 4, q.dtype)
    _dev_tensor("v_cache", v_cache, 4, q.dtype)
    _dev_tensor("seq_lens", seq_lens, 1, torch.int32)
    _dev_tensor("row_ptr", row_ptr, 1, torch.int32)
    _dev_tensor("col_idx", col_idx, 1, torch.int32)
    _dev_tensor("out", out, 3, q.dtype)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[:2] != (B, H) or k_cache.shape[3] != D:
        raise ValueError("cache shapes must be [B, H, cache_len, D] matching q")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    if row_ptr.numel() != B * H + 1:
        raise ValueError("row_ptr must hold B * H + 1 entries")
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B, H, D]")
    return (_DTYPES[q.dtype], B, H, D, row_ptr.data_ptr(), col_idx.data_ptr(), max_row_blocks,
            q.data_ptr(), _strides(q), k_cache.data_ptr(), _strides(k_cache), v_cache.data_ptr(),
            _strides(v_cache), seq_lens.data_ptr(), k_cache.shape[2], out.data_ptr(), _strides(out),
            lse.data_ptr() if lse is not None else None, splits, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), float(sm_scale))


def s2_attn_decode_rows(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        seq_lens: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                        max_row_blocks: int, splits: int = 0, sm_scale: float = 0.0,
                        workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None, want_lse: bool = True):
    """Decode over per-(sequence, head) block lists (row b * H + h of the CSR).
    Returns (o [B, H, D] in q's dtype, lse fp32 [B, H] or None)."""
    B, H, D = q.shape
    if out is None:
        out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(s2_attn_decode_rows_workspace(B, H, D, max_row_blocks, splits),
                                dtype=torch.uint8, device=q.device)
    _check(library().s2_attn_decode_rows(*_rows_args(q, k_cache, v_cache, seq_lens, row_ptr, col_idx,
                                                     max_row_blocks, out, lse, workspace, splits, sm_scale),
                                         _stream(q.device)))
    return out, lse


class PreparedSelectDecode:
    """One query-aware decode step with its arguments marshalled once:
    s2_select_blocks (the query's block and the budget - 1 best earlier blocks
    per (sequence, head), from the block bounds) then s2_attn_decode_rows."""

    def __init__(self, q, k_cache, v_cache, seq_lens, kmin, kmax, budget: int, out, lse=None,
                 splits: int = 0, sm_scale: float = 0.0):
        B, H, D = q.shape
        L = k_cache.shape[2]
        longest = min(budget, -(-L // S2_BLOCK))
        self.row_ptr = torch.empty(B * H + 1, dtype=torch.int32, device=q.device)
        self.col_idx = torch.empty(B * H * longest, dtype=torch.int32, device=q.device)
        self.workspace = torch.empty(s2_attn_decode_rows_workspace(B, H, D, longest, splits),
                                     dtype=torch.uint8, device=q.device)
        self._lib = library()
        self._keep = (q, k_cache, v_cache, seq_lens, kmin, kmax, out, lse)
        self._sel = _select_args(q, kmin, kmax, seq_lens, budget, L, self.row_ptr, self.col_idx)
        self._dec = _rows_args(q, k_cache, v_cache, seq_lens, self.row_ptr, self.col_idx, longest, out, lse,
                               self.workspace, splits, sm_scale)
        self._device = q.device

    def __call__(self):
        st = _stream(self._device)
        _check(self._lib.s2_select_blocks(*self._sel, st))
        _check(self._lib.s2_attn_decode_rows(*self._dec, st))


def s2_block_minmax_paged(k_pages: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                          num_blocks: int | None = None, kmin: torch.Tensor | None = None,
                          kmax: torch.Tensor | None = None):
    """Per-block key bounds over a paged cache.  k_pages: [num_pages, H_kv, page_size, D];
    block_table: int32 [B, max_pages]; seq_lens: int32 [B].  Returns (kmin, kmax),
    [B, H_kv, num_blocks, D] contiguous in the keys' dtype."""
    _dev_tensor("k_pages", k_pages, 4)
    _dev_tensor("block_table", block_table, 2, torch.int32)
    _dev_tensor("seq_lens", seq_lens, 1, torch.int32)
    if k_pages.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k_pages.dtype}")
    num_pages, Hkv, P, D = k_pages.shape
    B, width = block_table.shape
    if block_table.stride(1) != 1 or seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("block_table must be int32 [B, max_pages] with unit inner stride, seq_lens int32 [B]")
    nb = -(-(width * P) // S2_BLOCK) if num_blocks is None else num_blocks
    shape = (B, Hkv, nb, D)
    if kmin is None:
        kmin = torch.empty(shape, dtype=k_pages.dtype, device=k_pages.device)
    if kmax is None:
        kmax = torch.empty(shape, dtype=k_pages.dtype, device=k_pages.device)
    for name, t in (("kmin", kmin), ("kmax", kmax)):
        _dev_tensor(name, t, 4, k_pages.dtype)
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {list(shape)} tensor")
    _check(library().s2_block_minmax_paged(_DTYPES[k_pages.dtype], B, Hkv, D, k_pages.data_ptr(),
                                           _strides(k_pages), num_pages, P, block_table.data_ptr(),
                                           block_table.stride(0), width, seq_lens.data_ptr(), kmin.data_ptr(),
                                           kmax.data_ptr(), nb, _stream(k_pages.device)))
    return kmin, kmax


def s2_attn_decode_paged_rows_workspace(B: int, H: int, num_kv_heads: int, D: int, max_row_blocks: int,
                                        splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(library().s2_attn_decode_paged_rows_workspace(B, H, num_kv_heads, D, max_row_blocks, splits,
                                                         ctypes.byref(n)))
    return int(n.value)


def _paged_rows_args(q, k_pages, v_pages, block_table, seq_lens, row_ptr, col_idx, max_row_blocks: int, out,
                     lse, workspace, splits: int, sm_scale: float):
    _dev_tensor("row_ptr", row_ptr, 1, torch.int32)
    _dev_tensor("col_idx", col_idx, 1, torch.int32)
    B, H, _ = q.shape
    if row_ptr.numel() != B * H + 1:
        raise ValueError("row_ptr must hold B * H + 1 entries")
    a = _paged_args(q, k_pages, v_pages, block_table, seq_lens, None, out, lse, workspace, splits, sm_scale)
    # (dtype, B, H_kv, D, ...) -> (dtype, B, H, H_kv, D, row_ptr, col_idx, max_row_blocks, ...)
    return (a[0], a[1], H, a[2], a[3], row_ptr.data_ptr(), col_idx.data_ptr(), max_row_blocks) + a[4:]


def s2_attn_decode_paged_rows(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor, row_ptr: torch.Tensor,
                              col_idx: torch.Tensor, max_row_blocks: int, splits: int = 0, sm_scale: float = 0.0,
                              workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                              lse: torch.Tensor | None = None, want_lse: bool = True):
    """Serving decode over per-(sequence, head) block lists (row b * H + h)."""
    B, H, D = q.shape
    if out is None:
        out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = s2_attn_decode_paged_rows_workspace(B, H, k_pages.shape[1], D, max_row_blocks, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(library().s2_attn_decode_paged_rows(
        *_paged_rows_args(q, k_pages, v_pages, block_table, seq_lens, row_ptr, col_idx, max_row_blocks, out, lse,
                          workspace, splits, sm_scale), _stream(q.device)))
    return out, lse


class PreparedSelectDecodePaged:
    """One query-aware serving-decode step with its arguments marshalled once:
    s2_select_blocks over the paged cache's block bounds, then s2_attn_decode_paged_rows."""

    def __init__(self, q, k_pages, v_pages, block_table, seq_lens, kmin, kmax, budget: int, out, lse=None,
                 splits: int = 0, sm_scale: float = 0.0):
        B, H, D = q.shape
        L = block_table.shape[1] * k_pages.shape[2]  # the longest sequence the tables reach
        longest = min(budget, -(-L // S2_BLOCK))
        self.row_ptr = torch.empty(B * H + 1, dtype=torch.int32, device=q.device)
        self.col_idx = torch.empty(B * H * longest, dtype=torch.int32, device=q.device)
        need = s2_attn_decode_paged_rows_workspace(B, H, k_pages.shape[1], D, longest, splits)
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        self._lib = library()
        self._keep = (q, k_pages, v_pages, block_table, seq_lens, kmin, kmax, out, lse)
        self._sel = _select_args(q, kmin, kmax, seq_lens, budget, L, self.row_ptr, self.col_idx)
        self._dec = _paged_rows_args(q, k_pages, v_pages, block_table, seq_lens, self.row_ptr, self.col_idx, longest,
                                     out, lse, self.workspace if need > 0 else None, splits, sm_scale)
        self._device = q.device

    def __call__(self):
        st = _stream(self._device)
        _check(self._lib.s2_select_blocks(*self._sel, st))
        _check(self._lib.s2_attn_decode_paged_rows(*self._dec, st))

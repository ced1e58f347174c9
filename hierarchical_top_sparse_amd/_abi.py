"""ctypes binding of libllsa.so: one Python function per C entry point, same names.

Argument marshalling only: tensors become device pointers, lists of tensors become pointer
arrays, the stream defaults to torch's current stream.  Every step of the computation runs in
the HIP library; there is no fallback.  Each call verifies that the tensors it hands over have
the sizes the C ABI assumes (the C side cannot see buffer sizes), then raises LlsaError on
any non-zero status.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllsa.so")
_lib = None

LLSA_F32, LLSA_BF16 = 0, 1
LLSA_LAYOUT_MORTON, LLSA_LAYOUT_RASTER = 0, 1
LLSA_MAX_LEVELS = 6
LLSA_ABI_VERSION = 5   # the llsa_problem layout and entry points this binding marshals


class LlsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(what)
        self.status = status


class LlsaProblemC(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("batch", "heads", "height", "width", "head_dim", "block", "levels", "topk",
                 "enrich")] + [("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                               ("layout", ctypes.c_int32), ("enrich_levels", ctypes.c_int32),
                               ("coarse_unit_weight", ctypes.c_int32),
                               ("coarse_exclude_overlap", ctypes.c_int32)]


@dataclass(frozen=True)
class Problem:
    batch: int
    heads: int
    height: int
    width: int
    levels: int
    topk: int = 8
    enrich: int = 1
    head_dim: int = 64
    block: int = 16
    scale: float = 0.0
    dtype: int = LLSA_BF16
    layout: int = LLSA_LAYOUT_RASTER
    enrich_levels: int = 0        # with enrich: only coarse levels 2..1+m (0 = all)
    coarse_unit_weight: int = 0   # 1: coarse keys weighted 1 instead of B^l
    coarse_exclude_overlap: int = 0   # 1: drop coarse keys over a finer selected key

    @property
    def fine_k(self) -> int:
        """Picks per 16-token query block as the attention reads them: topk * block / 16."""
        return self.topk * self.block // 16

    def csc_dims(self, l: int):
        """(rows = cols, k) of the level-l selection the backward transposes: level 1 in
        16-token blocks, levels >= 2 as selected."""
        return (self.n // 16, self.fine_k) if l == 1 else (self.n_level(l), self.topk)

    @property
    def coarse_levels(self) -> int:
        """Coarse levels whose keys enrich the attention."""
        if not self.enrich or self.levels < 2:
            return 0
        return self.levels - 1 if not self.enrich_levels else min(self.enrich_levels,
                                                                   self.levels - 1)

    @property
    def n(self) -> int:
        return self.height * self.width

    def n_level(self, l: int) -> int:
        return self.n // self.block ** l

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == LLSA_BF16 else torch.float32

    def c(self) -> LlsaProblemC:
        return LlsaProblemC(self.batch, self.heads, self.height, self.width, self.head_dim,
                            self.block, self.levels, self.topk, int(self.enrich),
                            float(self.scale), self.dtype, self.layout, self.enrich_levels,
                            self.coarse_unit_weight, self.coarse_exclude_overlap)


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m hierarchical_top_sparse_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.llsa_abi_version.restype = ctypes.c_int32
        if L.llsa_abi_version() != LLSA_ABI_VERSION:
            raise RuntimeError(f"{_LIB_PATH} has ABI version {L.llsa_abi_version()}, the binding "
                               f"expects {LLSA_ABI_VERSION}: rebuild it")
        P = ctypes.POINTER(LlsaProblemC)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pp = ctypes.POINTER(ctypes.c_void_p)
        sigs = {
            "llsa_abi_version": ([], i32),
            "llsa_status_str": ([i32], ctypes.c_char_p),
            "llsa_last_error": ([], ctypes.c_char_p),
            "llsa_check": ([P], i32),
            "llsa_workspace_bytes": ([P, ctypes.POINTER(sz), ctypes.POINTER(sz)], i32),
            "llsa_reorder": ([P, vp, vp, i32, vp], i32),
            "llsa_pool": ([P, vp, vp, vp, pp, pp, pp, vp], i32),
            "llsa_select": ([P, pp, pp, pp, i32, i32, vp], i32),
            "llsa_pool_select": ([P, vp, vp, vp, pp, pp, pp, pp, vp], i32),
            "llsa_attn_fwd": ([P, vp, vp, vp, pp, pp, pp, vp, vp, vp], i32),
            "llsa_index_transpose_workspace": ([i32, i32, i32, i32, ctypes.POINTER(sz)], i32),
            "llsa_index_transpose": ([i32, i32, i32, i32, vp, vp, vp, vp, sz, vp], i32),
            "llsa_index_transpose_levels_workspace": ([P, ctypes.POINTER(sz)], i32),
            "llsa_index_transpose_levels": ([P, pp, pp, pp, vp, sz, vp], i32),
            "llsa_attn_bwd": ([P, vp, vp, vp, vp, vp, pp, pp, pp, pp, pp, vp, vp, vp, vp, sz,
                               vp], i32),
            "llsa_dense_attn_fwd": ([i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp],
                                    i32),
            "llsa_dense_attn_bwd": ([i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp], i32),
            "llsa_block_mask": ([P, vp, vp, vp], i32),
            "llsa_calib_copy": ([vp, vp, sz, vp], i32),
            "llsa_calib_mfma": ([vp, i32, i32, vp], i32),
            "llsa_expand_blocks": ([P, vp, vp, vp], i32),
            "llsa_attn_bwd_masked": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
                                     i32),
            "llsa_profile_enable": ([i32], i32),
            "llsa_attn_bwd_noalloc": ([P, vp, vp, vp, vp, vp, pp, pp, pp, pp, pp, vp, vp, vp, vp],
                                      i32),
            "llsa_profile_read": ([ctypes.c_char_p, sz], i32),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def exported_symbols() -> list:
    return ["llsa_abi_version", "llsa_status_str", "llsa_last_error", "llsa_check",
            "llsa_workspace_bytes", "llsa_reorder", "llsa_pool", "llsa_select",
            "llsa_pool_select", "llsa_attn_fwd",
            "llsa_index_transpose_workspace", "llsa_index_transpose", "llsa_attn_bwd",
            "llsa_dense_attn_fwd", "llsa_dense_attn_bwd", "llsa_block_mask", "llsa_expand_blocks",
            "llsa_attn_bwd_masked", "llsa_calib_copy", "llsa_calib_mfma", "llsa_profile_enable",
            "llsa_profile_read", "llsa_attn_bwd_noalloc", "llsa_index_transpose_levels",
            "llsa_index_transpose_levels_workspace"]


def _raise(status: int, name: str):
    if status != 0:
        L = lib()
        msg = L.llsa_last_error().decode()
        raise LlsaError(status, f"{name}: {L.llsa_status_str(status).decode()}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ptrs(ts, count=LLSA_MAX_LEVELS):
    arr = (ctypes.c_void_p * count)()
    for i, t in enumerate(ts or []):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, shape, dtype, name):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} "
                         f"{t.dtype}")


def _tok_shape(p: Problem):
    return (p.batch, p.heads, p.n, p.head_dim)


def _lv_shape(p: Problem, l: int):
    return (p.batch, p.heads, p.n_level(l), p.head_dim)


def _fine_sel_shape(p: Problem):
    return (p.batch, p.heads, p.n // 16, p.fine_k)


def _sel_shape(p: Problem, l: int):
    return (p.batch, p.heads, p.n_level(l), p.topk)


# ------------------------------------------------------------------------------ entry points


def llsa_abi_version() -> int:
    return lib().llsa_abi_version()


def llsa_status_str(status: int) -> str:
    return lib().llsa_status_str(status).decode()


def llsa_last_error() -> str:
    return lib().llsa_last_error().decode()


def llsa_check(p: Problem) -> int:
    """Host-only validation; returns the status code (does not raise)."""
    return lib().llsa_check(ctypes.byref(p.c()))


def llsa_workspace_bytes(p: Problem):
    f, b = ctypes.c_size_t(), ctypes.c_size_t()
    _raise(lib().llsa_workspace_bytes(ctypes.byref(p.c()), ctypes.byref(f), ctypes.byref(b)),
           "llsa_workspace_bytes")
    return f.value, b.value


def llsa_reorder(p: Problem, x, y, inverse: bool, stream=None):
    _expect(x, _tok_shape(p), p.torch_dtype, "x")
    _expect(y, _tok_shape(p), p.torch_dtype, "y")
    _raise(lib().llsa_reorder(ctypes.byref(p.c()), _ptr(x), _ptr(y), int(inverse),
                              _stream(stream)), "llsa_reorder")


def llsa_pool(p: Problem, q, k, v, q_lv, k_lv, v_lv, stream=None):
    for name, x, lv in (("q", q, q_lv), ("k", k, k_lv), ("v", v, v_lv)):
        _expect(x, _tok_shape(p), p.torch_dtype, name)
        if x is not None:
            if len(lv) != p.levels:
                raise ValueError(f"{name}_lv needs {p.levels} entries")
            for l, t in enumerate(lv, start=1):
                _expect(t, _lv_shape(p, l), torch.float32, f"{name}_lv[{l - 1}]")
    _raise(lib().llsa_pool(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v),
                           _ptrs(q_lv if q is not None else None),
                           _ptrs(k_lv if k is not None else None),
                           _ptrs(v_lv if v is not None else None), _stream(stream)),
           "llsa_pool")


def llsa_select(p: Problem, q_lv, k_lv, sel, level_hi=None, level_lo=1, stream=None):
    level_hi = p.levels if level_hi is None else level_hi
    for l in range(level_lo, level_hi + 1):
        _expect(q_lv[l - 1], _lv_shape(p, l), torch.float32, f"q_lv[{l - 1}]")
        _expect(k_lv[l - 1], _lv_shape(p, l), torch.float32, f"k_lv[{l - 1}]")
        _expect(sel[l - 1], _sel_shape(p, l), torch.int32, f"sel[{l - 1}]")
    if level_hi < p.levels:
        _expect(sel[level_hi], _sel_shape(p, level_hi + 1), torch.int32, "parent sel")
    _raise(lib().llsa_select(ctypes.byref(p.c()), _ptrs(q_lv), _ptrs(k_lv), _ptrs(sel),
                             level_hi, level_lo, _stream(stream)), "llsa_select")


def llsa_pool_select(p: Problem, q, k, v, q_lv, k_lv, v_lv, sel, stream=None):
    """llsa_pool(q, k, v) then llsa_select of levels L..1, as one call (V's pooling rides in
    the selection launches where the library can)."""
    _expect(q, _tok_shape(p), p.torch_dtype, "q")
    _expect(k, _tok_shape(p), p.torch_dtype, "k")
    _expect(v, _tok_shape(p), p.torch_dtype, "v")
    for name, x, lv in (("q", q, q_lv), ("k", k, k_lv), ("v", v, v_lv)):
        if x is None:
            continue
        if len(lv) != p.levels:
            raise ValueError(f"{name}_lv needs {p.levels} entries")
        for l, t in enumerate(lv, start=1):
            _expect(t, _lv_shape(p, l), torch.float32, f"{name}_lv[{l - 1}]")
    for l in range(1, p.levels + 1):
        _expect(sel[l - 1], _sel_shape(p, l), torch.int32, f"sel[{l - 1}]")
    _raise(lib().llsa_pool_select(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptrs(q_lv),
                                  _ptrs(k_lv), _ptrs(v_lv if v is not None else None),
                                  _ptrs(sel), _stream(stream)), "llsa_pool_select")


def llsa_attn_fwd(p: Problem, q, k, v, k_lv, v_lv, sel, o, lse, stream=None):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _expect(t, _tok_shape(p), p.torch_dtype, name)
    _expect(lse, (p.batch, p.heads, p.n), torch.float32, "lse")
    _expect(sel[0], _fine_sel_shape(p), torch.int32, "sel[0]")
    if p.coarse_levels:
        for l in range(2, 2 + p.coarse_levels):
            _expect(k_lv[l - 1], _lv_shape(p, l), torch.float32, f"k_lv[{l - 1}]")
            _expect(v_lv[l - 1], _lv_shape(p, l), torch.float32, f"v_lv[{l - 1}]")
            _expect(sel[l - 1], _sel_shape(p, l), torch.int32, f"sel[{l - 1}]")
    _raise(lib().llsa_attn_fwd(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptrs(k_lv),
                               _ptrs(v_lv), _ptrs(sel), _ptr(o), _ptr(lse), _stream(stream)),
           "llsa_attn_fwd")


def llsa_expand_blocks(p: Problem, sel1, fine, stream=None):
    """Level-1 picks of B-token blocks as the 16-token blocks they cover (a copy for B = 16)."""
    _expect(sel1, _sel_shape(p, 1), torch.int32, "sel1")
    _expect(fine, _fine_sel_shape(p), torch.int32, "fine")
    _raise(lib().llsa_expand_blocks(ctypes.byref(p.c()), _ptr(sel1), _ptr(fine), _stream(stream)),
           "llsa_expand_blocks")


def llsa_index_transpose_workspace(nmat: int, rows: int, cols: int, k: int) -> int:
    b = ctypes.c_size_t()
    _raise(lib().llsa_index_transpose_workspace(nmat, rows, cols, k, ctypes.byref(b)),
           "llsa_index_transpose_workspace")
    return b.value


def llsa_index_transpose(nmat, rows, cols, k, csr, csc_off, csc_rows, ws, stream=None):
    if csr.numel() != nmat * rows * k or csr.dtype != torch.int32 or not csr.is_contiguous():
        raise ValueError("csr must hold nmat*rows*k contiguous int32")
    if csc_off.numel() != nmat * (cols + 1) or csc_off.dtype != torch.int32:
        raise ValueError("csc_off must hold nmat*(cols+1) int32")
    if csc_rows.numel() != nmat * rows * k or csc_rows.dtype != torch.int32:
        raise ValueError("csc_rows must hold nmat*rows*k int32")
    _raise(lib().llsa_index_transpose(nmat, rows, cols, k, _ptr(csr), _ptr(csc_off),
                                      _ptr(csc_rows), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "llsa_index_transpose")


def llsa_index_transpose_levels_workspace(p: Problem) -> int:
    b = ctypes.c_size_t()
    _raise(lib().llsa_index_transpose_levels_workspace(ctypes.byref(p.c()), ctypes.byref(b)),
           "llsa_index_transpose_levels_workspace")
    return b.value


def llsa_index_transpose_levels(p: Problem, sel, csc_off, csc_rows, ws, stream=None):
    """CSR -> CSC of every level the backward reads (sel[0]: level 1 as 16-token blocks)."""
    for l in range(1, 2 + p.coarse_levels):
        rows, kk = p.csc_dims(l)
        _expect(sel[l - 1], _fine_sel_shape(p) if l == 1 else _sel_shape(p, l), torch.int32,
                f"sel[{l - 1}]")
        _expect(csc_off[l - 1], (p.batch, p.heads, rows + 1), torch.int32, f"csc_off[{l - 1}]")
        _expect(csc_rows[l - 1], (p.batch, p.heads, rows * kk), torch.int32,
                f"csc_rows[{l - 1}]")
    _raise(lib().llsa_index_transpose_levels(ctypes.byref(p.c()), _ptrs(sel), _ptrs(csc_off),
                                             _ptrs(csc_rows), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)),
           "llsa_index_transpose_levels")


def _check_bwd_args(p: Problem, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off, csc_rows, dq, dk,
                    dv):
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _expect(t, _tok_shape(p), p.torch_dtype, name)
    _expect(lse, (p.batch, p.heads, p.n), torch.float32, "lse")
    levels = 1 + p.coarse_levels
    for l in range(1, levels + 1):
        rows, kk = p.csc_dims(l)
        _expect(sel[l - 1], _fine_sel_shape(p) if l == 1 else _sel_shape(p, l), torch.int32,
                f"sel[{l - 1}]")
        _expect(csc_off[l - 1], (p.batch, p.heads, rows + 1), torch.int32, f"csc_off[{l - 1}]")
        _expect(csc_rows[l - 1], (p.batch, p.heads, rows * kk), torch.int32,
                f"csc_rows[{l - 1}]")
        if l >= 2:
            _expect(k_lv[l - 1], _lv_shape(p, l), torch.float32, f"k_lv[{l - 1}]")
            _expect(v_lv[l - 1], _lv_shape(p, l), torch.float32, f"v_lv[{l - 1}]")


def llsa_attn_bwd(p: Problem, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off, csc_rows, dq, dk,
                  dv, ws, stream=None):
    _check_bwd_args(p, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off, csc_rows, dq, dk, dv)
    _raise(lib().llsa_attn_bwd(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                               _ptr(lse), _ptrs(k_lv), _ptrs(v_lv), _ptrs(sel),
                               _ptrs(csc_off), _ptrs(csc_rows), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "llsa_attn_bwd")


LLSA_NOALLOC_SCRATCH_BYTES = 96 << 20   # the allocation-free backward's workspace limit


def llsa_attn_bwd_noalloc(p: Problem, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off, csc_rows,
                          dq, dk, dv, stream=None):
    _check_bwd_args(p, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off, csc_rows, dq, dk, dv)
    _raise(lib().llsa_attn_bwd_noalloc(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(dout), _ptr(lse), _ptrs(k_lv), _ptrs(v_lv),
                                       _ptrs(sel), _ptrs(csc_off), _ptrs(csc_rows), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _stream(stream)),
           "llsa_attn_bwd_noalloc")


def _mask_shape(p: Problem):
    return (p.batch, p.heads, p.n_level(1), p.n_level(1))


def llsa_block_mask(p: Problem, sel1, mask, stream=None):
    """Dense level-1 block mask (uint8 [b, H, n_1, n_1]) of Sel_1: the mask-based comparator."""
    _expect(sel1, _sel_shape(p, 1), torch.int32, "sel1")
    _expect(mask, _mask_shape(p), torch.uint8, "mask")
    _raise(lib().llsa_block_mask(ctypes.byref(p.c()), _ptr(sel1), _ptr(mask), _stream(stream)),
           "llsa_block_mask")


def llsa_attn_bwd_masked(p: Problem, q, k, v, dout, lse, sel1, mask, dq, dk, dv, ws,
                         stream=None):
    """llsa_attn_bwd without coarse keys, its key-major pass scanning the block mask."""
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _expect(t, _tok_shape(p), p.torch_dtype, name)
    _expect(lse, (p.batch, p.heads, p.n), torch.float32, "lse")
    _expect(sel1, _sel_shape(p, 1), torch.int32, "sel1")
    _expect(mask, _mask_shape(p), torch.uint8, "mask")
    _raise(lib().llsa_attn_bwd_masked(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(dout), _ptr(lse), _ptr(sel1), _ptr(mask), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "llsa_attn_bwd_masked")


def _dense_shapes(q):
    if q.dim() < 2:
        raise ValueError("dense attention tensors are [..., n, head_dim]")
    n, d = q.shape[-2], q.shape[-1]
    return q.numel() // (n * d), n, d


def llsa_dense_attn_fwd(q, k, v, o, lse, scale=0.0, stream=None):
    """Dense softmax attention over [..., n, 64] bf16 (the full-attention baseline)."""
    bh, n, d = _dense_shapes(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _expect(t, tuple(q.shape), torch.bfloat16, name)
    _expect(lse, tuple(q.shape[:-1]), torch.float32, "lse")
    _raise(lib().llsa_dense_attn_fwd(bh, n, d, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(lse), _stream(stream)), "llsa_dense_attn_fwd")


def llsa_dense_attn_bwd(q, k, v, dout, lse, dq, dk, dv, d_rows, scale=0.0, stream=None):
    bh, n, d = _dense_shapes(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _expect(t, tuple(q.shape), torch.bfloat16, name)
    _expect(lse, tuple(q.shape[:-1]), torch.float32, "lse")
    _expect(d_rows, tuple(q.shape[:-1]), torch.float32, "d_rows")
    _raise(lib().llsa_dense_attn_bwd(bh, n, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                     _ptr(d_rows), _stream(stream)), "llsa_dense_attn_bwd")


def llsa_calib_copy(src, dst, stream=None):
    """Plain streaming copy of a contiguous tensor into another of the same size."""
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("src and dst must have the same size in bytes")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    _raise(lib().llsa_calib_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                                 _stream(stream)), "llsa_calib_copy")


def llsa_calib_mfma(out, blocks: int, iters: int, stream=None):
    """MFMA-only loop; out: fp32 [blocks * 256]."""
    _expect(out, (blocks * 256,), torch.float32, "out")
    _raise(lib().llsa_calib_mfma(_ptr(out), int(blocks), int(iters), _stream(stream)),
           "llsa_calib_mfma")


def llsa_profile_enable(on: bool):
    _raise(lib().llsa_profile_enable(int(on)), "llsa_profile_enable")


def llsa_profile_read() -> dict:
    """{kernel name: (launches, total_ms)} since the last read (waits for the events)."""
    buf = ctypes.create_string_buffer(1 << 16)
    _raise(lib().llsa_profile_read(buf, len(buf)), "llsa_profile_read")
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out

"""Python binding of libasa.so: content-aware block-sparse attention on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the library's HIP
kernels; torch supplies device memory and the current stream.  There is no CPU
fallback: importing this package fails if the built library is missing.

Entry points (same names as the C ABI in include/asa.h):
    asa_build_mask(q, k, blk, mode, ...)   -> (row_ptr, col_idx)
    asa_build_mask_noalloc(q, k, blk, mode, out=(row_ptr, col_idx), ...) -> same, no allocation
    asa_static_mask(B, H, N, blk, patterns, device) -> (row_ptr, col_idx)
    asa_attention_fwd(q, k, v, row_ptr, col_idx, blk, ...) -> O
    asa_attention_fwd_split(q, k, v, row_ptr, col_idx, blk, split_blocks=...) -> O
    asa_attention_bwd(q, k, v, o, dout, lse, row_ptr, col_idx, blk, ...) -> (dQ, dK, dV)
    asa_pattern_search(q, k, v, blk, candidates, ...) -> (choice, loss, mse)
"""
import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libasa.so")

ASA_F32, ASA_BF16 = 0, 1
ADAPTIVE, FULL, SKIP, DIAG, MULTIDIAG, VSTRIPE, FRAME_TILE = 0, 1, 2, 3, 4, 5, 6
TOPK, TAU = 0, 1


class asa_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("blk", ctypes.c_int32), ("in_dtype", ctypes.c_int32)]


class asa_adaptive(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("k", ctypes.c_int32), ("tau", ctypes.c_double),
                ("k_cap", ctypes.c_int32), ("n_text", ctypes.c_int32), ("keep_diag", ctypes.c_int32)]


class asa_head_pattern(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("param", ctypes.c_int32)]


class asa_csr(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("order", ctypes.c_void_p)]


EXPORTS = {
    "asa_version": (ctypes.c_int32, []),
    "asa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "asa_last_error": (ctypes.c_char_p, []),
    "asa_csr_capacity": (ctypes.c_int64, [ctypes.POINTER(asa_shape)]),
    "asa_build_mask_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(asa_shape)]),
    "asa_static_mask_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(asa_shape)]),
    "asa_build_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(asa_shape),
                                      ctypes.POINTER(asa_adaptive), ctypes.POINTER(asa_head_pattern),
                                      ctypes.POINTER(asa_csr), ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]),
    "asa_build_mask_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(asa_shape),
                                              ctypes.POINTER(asa_adaptive), ctypes.POINTER(asa_head_pattern),
                                              ctypes.POINTER(asa_csr), ctypes.c_void_p]),
    "asa_static_mask": (ctypes.c_int, [ctypes.POINTER(asa_shape), ctypes.POINTER(asa_head_pattern),
                                       ctypes.POINTER(asa_csr), ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]),
    "asa_attention_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.POINTER(asa_shape), ctypes.POINTER(asa_csr),
                                         ctypes.POINTER(asa_head_pattern), ctypes.c_float, ctypes.c_void_p]),
    "asa_attention_fwd_lse": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.POINTER(asa_shape), ctypes.POINTER(asa_csr),
                                             ctypes.POINTER(asa_head_pattern), ctypes.c_float, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "asa_attention_fwd_split_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(asa_shape), ctypes.c_int32]),
    "asa_attention_fwd_split": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.POINTER(asa_shape), ctypes.POINTER(asa_csr),
                                               ctypes.POINTER(asa_head_pattern), ctypes.c_float, ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "asa_attention_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(asa_shape)]),
    "asa_attention_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(asa_shape),
                                         ctypes.POINTER(asa_csr), ctypes.POINTER(asa_head_pattern),
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "asa_pattern_search_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(asa_shape), ctypes.c_int32]),
    "asa_pattern_search": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.POINTER(asa_shape), ctypes.POINTER(asa_head_pattern),
                                          ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_float,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python block_sparse_attention_asa_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        try:
            fn = getattr(lib, name)
        except AttributeError:
            raise ImportError(f"{LIB_PATH} does not export {name} (built from older sources); "
                              f"run `python block_sparse_attention_asa_amd/build.py`") from None
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class AsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.asa_last_error().decode(errors="replace")
        name = lib.asa_status_string(status).decode()
        super().__init__(f"{where}: {name} ({status}): {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise AsaError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ASA_BF16
    if t.dtype == torch.float32:
        return ASA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _shape_of(q: torch.Tensor, blk: int) -> asa_shape:
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    B, H, N, d = q.shape
    return asa_shape(B, H, N, d, blk, _dtype_code(q))


def _patterns(patterns: Optional[Sequence[Tuple[int, int]]], H: int):
    if patterns is None:
        return None
    if len(patterns) != H:
        raise ValueError(f"need {H} head patterns, got {len(patterns)}")
    arr = (asa_head_pattern * H)()
    for h, (pid, prm) in enumerate(patterns):
        arr[h].id, arr[h].param = int(pid), int(prm)
    return arr


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _require_device(*ts: torch.Tensor):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def num_blocks(N: int, blk: int) -> int:
    return (N + blk - 1) // blk


def asa_csr_capacity(B: int, H: int, N: int, blk: int) -> int:
    shp = asa_shape(B, H, N, 64, blk, ASA_BF16)
    return int(lib.asa_csr_capacity(ctypes.byref(shp)))


def _alloc_csr(B, H, N, blk, device):
    shp = asa_shape(B, H, N, 64, blk, ASA_BF16)
    cap = int(lib.asa_csr_capacity(ctypes.byref(shp)))
    if cap < 0:
        # a shape the builders reject: the builder call itself validates the shape first
        # and raises AsaError with its status and message; these buffers are never touched
        return (torch.zeros(1, dtype=torch.int32, device=device),
                torch.zeros(1, dtype=torch.int32, device=device))
    rows = B * H * num_blocks(N, blk)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=device)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
    return row_ptr, col_idx


def _csr_buffers(out, with_order, B, H, N, blk, device):
    """(row_ptr, col_idx, order or None): the caller's buffers or fresh ones."""
    if out is not None:
        if len(out) not in (2, 3):
            raise ValueError("out must be (row_ptr, col_idx) or (row_ptr, col_idx, order)")
        row_ptr, col_idx = out[0], out[1]
        order = out[2] if len(out) == 3 else None
        _require_device(row_ptr, col_idx)
        if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
            raise TypeError("row_ptr and col_idx must be int32")
        if row_ptr.numel() != B * H * num_blocks(N, blk) + 1:
            raise ValueError("row_ptr length does not match [B, H, Nb] rows")
    else:
        row_ptr, col_idx = _alloc_csr(B, H, N, blk, device)
        order = None
    if order is None and with_order:
        order = torch.empty(row_ptr.numel() - 1, dtype=torch.int32, device=row_ptr.device)
    if order is not None:
        _require_device(order)
        if order.dtype != torch.int32 or order.numel() != row_ptr.numel() - 1:
            raise ValueError("order must be int32 with one entry per CSR row")
    return row_ptr, col_idx, order


def _csr_struct(row_ptr, col_idx, order):
    return asa_csr(row_ptr.data_ptr(), col_idx.data_ptr(), col_idx.numel(),
                   order.data_ptr() if order is not None else None)


def asa_build_mask(q: torch.Tensor, k: torch.Tensor, blk: int, mode: int, *, k_top: int = 0,
                   tau: float = 0.0, k_cap: int = 0, n_text: int = 0, keep_diag: int = 1,
                   patterns: Optional[Sequence[Tuple[int, int]]] = None,
                   out: Optional[Tuple[torch.Tensor, ...]] = None, with_order: bool = False,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Adaptive block mask (plus forced / static blocks) as CSR (row_ptr, col_idx).

    col_idx is sized for the worst case; its first row_ptr[-1] entries are valid.  With
    with_order (or a 3-tuple `out`), also returns the attention schedule `order` (rows
    longest first inside each XCD range; see asa.h).
    """
    _require_device(q, k)
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must have the same shape and dtype")
    shp = _shape_of(q, blk)
    B, H, N, _ = q.shape
    row_ptr, col_idx, order = _csr_buffers(out, with_order, B, H, N, blk, q.device)
    csr = _csr_struct(row_ptr, col_idx, order)
    ad = asa_adaptive(mode, k_top, tau, k_cap, n_text, keep_diag)
    need = int(lib.asa_build_mask_workspace_size(ctypes.byref(shp)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    pats = _patterns(patterns, H)
    _check(lib.asa_build_mask(q.data_ptr(), k.data_ptr(), ctypes.byref(shp), ctypes.byref(ad),
                              pats, ctypes.byref(csr), workspace.data_ptr(), workspace.numel(),
                              _stream(q.device, stream)), "asa_build_mask")
    return (row_ptr, col_idx) if order is None else (row_ptr, col_idx, order)


NOALLOC_SCRATCH_BYTES = 32 << 20


def asa_build_mask_noalloc(q: torch.Tensor, k: torch.Tensor, blk: int, mode: int, *,
                           out: Tuple[torch.Tensor, ...], k_top: int = 0, tau: float = 0.0,
                           k_cap: int = 0, n_text: int = 0, keep_diag: int = 1,
                           patterns: Optional[Sequence[Tuple[int, int]]] = None, stream=None):
    """asa_build_mask into caller-supplied CSR buffers `out` = (row_ptr, col_idx[, order]),
    with the library's static device scratch as workspace: the call allocates nothing.
    Shapes whose workspace exceeds NOALLOC_SCRATCH_BYTES raise AsaError."""
    _require_device(q, k)
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must have the same shape and dtype")
    if out is None:
        raise ValueError("out = (row_ptr, col_idx[, order]) is required: this call allocates nothing")
    shp = _shape_of(q, blk)
    B, H, N, _ = q.shape
    row_ptr, col_idx, order = _csr_buffers(out, False, B, H, N, blk, q.device)
    csr = _csr_struct(row_ptr, col_idx, order)
    ad = asa_adaptive(mode, k_top, tau, k_cap, n_text, keep_diag)
    _check(lib.asa_build_mask_noalloc(q.data_ptr(), k.data_ptr(), ctypes.byref(shp), ctypes.byref(ad),
                                      _patterns(patterns, H), ctypes.byref(csr), _stream(q.device, stream)),
           "asa_build_mask_noalloc")
    return (row_ptr, col_idx) if order is None else (row_ptr, col_idx, order)


def asa_static_mask(B: int, H: int, N: int, blk: int, patterns: Sequence[Tuple[int, int]],
                    device, *, out=None, with_order: bool = False,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """Static-pattern block mask as CSR (row_ptr, col_idx[, order])."""
    device = torch.device(device)
    shp = asa_shape(B, H, N, 64, blk, ASA_BF16)
    row_ptr, col_idx, order = _csr_buffers(out, with_order, B, H, N, blk, device)
    csr = _csr_struct(row_ptr, col_idx, order)
    need = int(lib.asa_static_mask_workspace_size(ctypes.byref(shp)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    pats = _patterns(patterns, H)
    if pats is None:
        raise ValueError("patterns are required")
    _check(lib.asa_static_mask(ctypes.byref(shp), pats, ctypes.byref(csr), workspace.data_ptr(),
                               workspace.numel(), _stream(device, stream)), "asa_static_mask")
    return (row_ptr, col_idx) if order is None else (row_ptr, col_idx, order)


def asa_attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                      col_idx: torch.Tensor, blk: int, *,
                      patterns: Optional[Sequence[Tuple[int, int]]] = None,
                      out_dtype: torch.dtype = torch.float32, scale: float = 0.0,
                      order: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block-sparse attention over the kept tiles of the CSR mask; returns O [B,H,N,d].

    `order`, from a mask builder's with_order, sets the processing order of the rows; the
    result does not depend on it.  `lse` (float32 [B,H,N]), if given, receives the log of
    each query's softmax normaliser (what asa_attention_bwd needs).
    """
    _require_device(q, k, v, row_ptr, col_idx)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    shp = _shape_of(q, blk)
    B, H, N, d = q.shape
    if row_ptr.numel() != B * H * num_blocks(N, blk) + 1:
        raise ValueError("row_ptr length does not match [B, H, Nb] rows")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    _require_device(out)
    if tuple(out.shape) != (B, H, N, d):
        raise ValueError(f"out must have shape {(B, H, N, d)}, got {tuple(out.shape)}")
    o_code = _dtype_code(out)
    if order is not None:
        _require_device(order)
        if order.dtype != torch.int32 or order.numel() != row_ptr.numel() - 1:
            raise ValueError("order must be int32 with one entry per CSR row")
    csr = _csr_struct(row_ptr, col_idx, order)
    pats = _patterns(patterns, H)
    if lse is None:
        _check(lib.asa_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), o_code,
                                     ctypes.byref(shp), ctypes.byref(csr), pats, float(scale),
                                     _stream(q.device, stream)), "asa_attention_fwd")
    else:
        _require_device(lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be float32 [B, H, N]")
        _check(lib.asa_attention_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), o_code,
                                         ctypes.byref(shp), ctypes.byref(csr), pats, float(scale),
                                         lse.data_ptr(), _stream(q.device, stream)), "asa_attention_fwd_lse")
    return out


def asa_attention_fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                            col_idx: torch.Tensor, blk: int, *, split_blocks: int = 0,
                            patterns: Optional[Sequence[Tuple[int, int]]] = None,
                            out_dtype: torch.dtype = torch.float32, scale: float = 0.0,
                            order: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """asa_attention_fwd with rows of more than `split_blocks` kept blocks split over several
    workgroups and merged afterwards (0 = choose from the shape).  Returns O [B,H,N,d]."""
    _require_device(q, k, v, row_ptr, col_idx)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    shp = _shape_of(q, blk)
    B, H, N, d = q.shape
    if row_ptr.numel() != B * H * num_blocks(N, blk) + 1:
        raise ValueError("row_ptr length does not match [B, H, Nb] rows")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    _require_device(out)
    if tuple(out.shape) != (B, H, N, d):
        raise ValueError(f"out must have shape {(B, H, N, d)}, got {tuple(out.shape)}")
    if order is not None:
        _require_device(order)
        if order.dtype != torch.int32 or order.numel() != row_ptr.numel() - 1:
            raise ValueError("order must be int32 with one entry per CSR row")
    if lse is not None:
        _require_device(lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be float32 [B, H, N]")
    need = int(lib.asa_attention_fwd_split_workspace_size(ctypes.byref(shp), int(split_blocks)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    csr = _csr_struct(row_ptr, col_idx, order)
    _check(lib.asa_attention_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dtype_code(out),
                                       ctypes.byref(shp), ctypes.byref(csr), _patterns(patterns, H), float(scale),
                                       lse.data_ptr() if lse is not None else None, int(split_blocks),
                                       workspace.data_ptr() if workspace is not None else None,
                                       workspace.numel() if workspace is not None else 0,
                                       _stream(q.device, stream)), "asa_attention_fwd_split")
    return out


def asa_attention_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                      dout: torch.Tensor, lse: torch.Tensor, row_ptr: torch.Tensor,
                      col_idx: torch.Tensor, blk: int, *,
                      patterns: Optional[Sequence[Tuple[int, int]]] = None, scale: float = 0.0,
                      order: Optional[torch.Tensor] = None,
                      grads: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients (dQ, dK, dV), float32 [B,H,N,d], of sum(dout * O) for the block-sparse
    attention O = asa_attention_fwd(q, k, v, row_ptr, col_idx, blk) with its `lse`.
    `order` (a mask builder's schedule) sets the dQ pass's row order, as for the forward."""
    _require_device(q, k, v, o, dout, lse, row_ptr, col_idx)
    if not (q.shape == k.shape == v.shape == o.shape == dout.shape):
        raise ValueError("q, k, v, o and dout must share one shape")
    if not (q.dtype == k.dtype == v.dtype == dout.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("the backward takes q, k, v and dout of one dtype, bfloat16 or float32")
    shp = _shape_of(q, blk)
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 [B, H, N]")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != B * H * num_blocks(N, blk) + 1:
        raise ValueError("row_ptr length does not match [B, H, Nb] rows")
    if order is not None:
        _require_device(order)
        if order.dtype != torch.int32 or order.numel() != row_ptr.numel() - 1:
            raise ValueError("order must be int32 with one entry per CSR row")
    if grads is None:
        grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=q.device) for _ in range(3))
    dq, dk, dv = grads
    _require_device(dq, dk, dv)
    for g in grads:
        if g.dtype != torch.float32 or g.shape != q.shape:
            raise ValueError("gradients are float32 with the shape of q")
    need = int(lib.asa_attention_bwd_workspace_size(ctypes.byref(shp)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    csr = _csr_struct(row_ptr, col_idx, order)
    pats = _patterns(patterns, H)
    _check(lib.asa_attention_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _dtype_code(o),
                                 dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                 ctypes.byref(shp), ctypes.byref(csr), pats, float(scale),
                                 workspace.data_ptr(), workspace.numel(), _stream(q.device, stream)),
           "asa_attention_bwd")
    return dq, dk, dv


def asa_pattern_search(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, blk: int,
                       candidates: Sequence[Tuple[int, int]], *, lam: float = 0.01, eps: float = 0.1,
                       scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                       out: Optional[Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]] = None,
                       stream=None):
    """Per-head pattern choice of one layer: returns (choice int32 [H], loss float64 [H, n],
    mse float64 [H, n]) on the device.  choice 0 = full attention, i = candidates[i - 1]."""
    _require_device(q, k, v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must share one shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    shp = _shape_of(q, blk)
    B, H, N, d = q.shape
    n = len(candidates)
    arr = (asa_head_pattern * max(n, 1))()
    for i, (pid, prm) in enumerate(candidates):
        arr[i].id, arr[i].param = int(pid), int(prm)
    if out is None:
        out = (torch.empty(H, dtype=torch.int32, device=q.device),
               torch.empty((H, n), dtype=torch.float64, device=q.device),
               torch.empty((H, n), dtype=torch.float64, device=q.device))
    choice, loss, mse = out
    _require_device(choice, loss, *( [mse] if mse is not None else []))
    if choice.dtype != torch.int32 or choice.numel() != H:
        raise ValueError("choice must be int32 [H]")
    if loss.dtype != torch.float64 or loss.numel() != H * n:
        raise ValueError("loss must be float64 [H, n]")
    if mse is not None and (mse.dtype != torch.float64 or mse.numel() != H * n):
        raise ValueError("mse must be float64 [H, n]")
    need = int(lib.asa_pattern_search_workspace_size(ctypes.byref(shp), n))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.asa_pattern_search(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(shp), arr, n,
                                  float(lam), float(eps), float(scale),
                                  loss.data_ptr(), mse.data_ptr() if mse is not None else None,
                                  choice.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                  _stream(q.device, stream)),
           "asa_pattern_search")
    return choice, loss, mse


__all__ = ["asa_build_mask", "asa_build_mask_noalloc", "NOALLOC_SCRATCH_BYTES", "asa_static_mask", "asa_attention_fwd", "asa_attention_fwd_split",
           "asa_attention_bwd", "asa_pattern_search",
           "asa_csr_capacity",
           "AsaError", "lib", "LIB_PATH", "EXPORTS", "num_blocks",
           "ADAPTIVE", "FULL", "SKIP", "DIAG", "MULTIDIAG", "VSTRIPE", "FRAME_TILE", "TOPK", "TAU"]

"""Python binding of the fused linear cross-entropy engine for MI355X.

Two layers, both argument marshalling only -- every step of the computation runs
in the HIP kernels of ``libflce.so``:

* ``flce_workspace_size``, ``flce_forward``, ``flce_backward``,
  ``flce_chunked_workspace_size``, ``flce_chunked``, ``flce_scale_grads`` and
  ``flce_status_string`` mirror the C ABI of ``include/flce.h`` one to one and
  take raw device addresses (Python ints) and sizes;
* ``linear_cross_entropy(hidden, weight, labels, ignore_index=-100,
  shift=False, reduction="mean", mode="recompute")`` is the tensor-level call
  with autograd, the argument set of the ``linear_cross_entropy`` call in the
  LoRA-SFT blog post's CCE patch; ``mode="chunked"`` computes the gradients
  during the forward with the row-chunk schedule.  PyTorch only provides device
  memory and the current stream.

Importing the package loads ``libflce.so`` and fails loudly if it is missing;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "FLCE_OK", "FLCE_DTYPE_F32", "FLCE_DTYPE_BF16", "FLCE_REDUCTION_MEAN",
    "FLCE_REDUCTION_SUM", "FLCE_REDUCTION_NONE", "FlceError", "flce_workspace_size", "flce_forward",
    "flce_forward_noalloc", "FLCE_NOALLOC_SCRATCH_BYTES",
    "flce_backward", "flce_chunked_workspace_size", "flce_chunked", "flce_scale_grads",
    "flce_convert_grads",
    "flce_shard_forward", "flce_shard_merge_workspace_size", "flce_shard_merge",
    "flce_shard_backward",
    "flce_status_string", "linear_cross_entropy", "library_path",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce.so")

# mirrors include/flce.h
FLCE_OK = 0
FLCE_ERR_NULL = 1
FLCE_ERR_SHAPE = 2
FLCE_ERR_ALIGN = 3
FLCE_ERR_DTYPE = 4
FLCE_ERR_REDUCTION = 5
FLCE_ERR_WORKSPACE = 6
FLCE_ERR_HIP = 7
FLCE_ERR_LABEL_RANGE = 8
FLCE_ERR_ALIAS = 9
FLCE_ERR_TOO_LARGE = 10
FLCE_NOALLOC_SCRATCH_BYTES = 160 << 20
FLCE_DTYPE_F32 = 0
FLCE_DTYPE_BF16 = 1
FLCE_REDUCTION_MEAN = 0
FLCE_REDUCTION_SUM = 1
FLCE_REDUCTION_NONE = 2

EXPORTS = ("flce_workspace_size", "flce_forward", "flce_forward_noalloc", "flce_backward",
           "flce_shard_forward", "flce_shard_merge_workspace_size", "flce_shard_merge",
           "flce_shard_backward", "flce_chunked_workspace_size", "flce_chunked",
           "flce_scale_grads", "flce_convert_grads", "flce_status_string")


class FlceError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {flce_status_string(code)} (status {code})")


def _load() -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime under the same soname; load it first so
    # that this library binds to that one runtime and shares its streams.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python lm_head_linear_flce_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.flce_workspace_size.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(sz)]
    lib.flce_workspace_size.restype = i32
    lib.flce_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i64, i32, i32,
                                 vp, vp, vp, vp, vp, sz, vp]
    lib.flce_forward.restype = i32
    lib.flce_forward_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i64, i32, i32,
                                         vp, vp, vp, vp, vp]
    lib.flce_forward_noalloc.restype = i32
    lib.flce_backward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i64, i32, i32,
                                  vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.flce_backward.restype = i32
    lib.flce_shard_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i64,
                                       i32, vp, vp, vp, vp, sz, vp]
    lib.flce_shard_forward.restype = i32
    lib.flce_shard_merge_workspace_size.argtypes = [i64, i64, ctypes.POINTER(sz)]
    lib.flce_shard_merge_workspace_size.restype = i32
    lib.flce_shard_merge.argtypes = [vp, vp, i32, vp, i64, i64, i64, i64, i32, i32, vp, vp,
                                     vp, vp, vp, sz, vp]
    lib.flce_shard_merge.restype = i32
    lib.flce_shard_backward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i64,
                                        i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.flce_shard_backward.restype = i32
    lib.flce_chunked_workspace_size.argtypes = [i64, i64, i64, i64, i32, i64,
                                                ctypes.POINTER(sz)]
    lib.flce_chunked_workspace_size.restype = i32
    lib.flce_chunked.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i64, i32, i32, i64,
                                 vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.flce_chunked.restype = i32
    lib.flce_scale_grads.argtypes = [vp, vp, i64, vp, vp, i64, i32, vp, vp]
    lib.flce_scale_grads.restype = i32
    lib.flce_convert_grads.argtypes = [vp, vp, i64, i32, vp, i32, vp]
    lib.flce_convert_grads.restype = i32
    lib.flce_status_string.argtypes = [i32]
    lib.flce_status_string.restype = ctypes.c_char_p
    return lib


_LIB = _load()


def library_path() -> str:
    return LIB_PATH


# ---------------------------------------------------------------------------
# C ABI, one to one (device addresses as Python ints, 0 = NULL)
# ---------------------------------------------------------------------------

def flce_status_string(code: int) -> str:
    return _LIB.flce_status_string(int(code)).decode()


def flce_workspace_size(B: int, T: int, H: int, V: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    rc = _LIB.flce_workspace_size(B, T, H, V, dtype, ctypes.byref(out))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_workspace_size")
    return int(out.value)


def flce_forward(X, W, labels, B, T, H, V, dtype, ignore_index, reduction, shift,
                 loss, lse, n_valid, status, workspace, workspace_bytes, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_forward(X or None, W or None, labels or None, B, T, H, V, dtype,
                             ignore_index, reduction, int(bool(shift)), loss or None,
                             lse or None, n_valid or None, status or None,
                             workspace or None, workspace_bytes, stream or None)


def flce_forward_noalloc(X, W, labels, B, T, H, V, dtype, ignore_index, reduction, shift,
                         loss, lse, n_valid, status, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_forward_noalloc(X or None, W or None, labels or None, B, T, H, V, dtype,
                                     ignore_index, reduction, int(bool(shift)), loss or None,
                                     lse or None, n_valid or None, status or None,
                                     stream or None)


def flce_backward(X, W, labels, B, T, H, V, dtype, ignore_index, reduction, shift,
                  lse, grad_scale, dX, dW, grad_dtype, dW_accumulate, status, workspace,
                  workspace_bytes, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_backward(X or None, W or None, labels or None, B, T, H, V, dtype,
                              ignore_index, reduction, int(bool(shift)), lse or None,
                              grad_scale or None, dX or None, dW or None, grad_dtype,
                              int(bool(dW_accumulate)), status or None, workspace or None,
                              workspace_bytes, stream or None)


def flce_shard_forward(X, W, labels, B, T, H, V, v_begin, V_total, dtype, ignore_index,
                       shift, lse, zt, status, workspace, workspace_bytes, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_shard_forward(X or None, W or None, labels or None, B, T, H, V, v_begin,
                                   V_total, dtype, ignore_index, int(bool(shift)), lse or None,
                                   zt or None, status or None, workspace or None,
                                   workspace_bytes, stream or None)


def flce_shard_merge_workspace_size(B: int, T: int) -> int:
    out = ctypes.c_size_t(0)
    rc = _LIB.flce_shard_merge_workspace_size(B, T, ctypes.byref(out))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_shard_merge_workspace_size")
    return int(out.value)


def flce_shard_merge(lse_shards, zt_shards, shards, labels, B, T, V_total, ignore_index,
                     shift, reduction, loss, lse, n_valid, status, workspace,
                     workspace_bytes, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_shard_merge(lse_shards or None, zt_shards or None, shards,
                                 labels or None, B, T, V_total, ignore_index,
                                 int(bool(shift)), reduction, loss or None, lse or None,
                                 n_valid or None, status or None, workspace or None,
                                 workspace_bytes, stream or None)


def flce_shard_backward(X, W, labels, B, T, H, V, v_begin, V_total, dtype, ignore_index,
                        reduction, shift, lse, grad_scale, dX_partial, dW, grad_dtype,
                        dW_accumulate, status, workspace, workspace_bytes, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_shard_backward(X or None, W or None, labels or None, B, T, H, V, v_begin,
                                    V_total, dtype, ignore_index, reduction, int(bool(shift)),
                                    lse or None, grad_scale or None, dX_partial or None,
                                    dW or None, grad_dtype, int(bool(dW_accumulate)),
                                    status or None, workspace or None, workspace_bytes,
                                    stream or None)


def flce_chunked_workspace_size(B: int, T: int, H: int, V: int, dtype: int,
                                chunk_rows: int = 0) -> int:
    out = ctypes.c_size_t(0)
    rc = _LIB.flce_chunked_workspace_size(B, T, H, V, dtype, chunk_rows, ctypes.byref(out))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_chunked_workspace_size")
    return int(out.value)


def flce_chunked(X, W, labels, B, T, H, V, dtype, ignore_index, reduction, shift,
                 chunk_rows, grad_scale, loss, lse, n_valid, dX, dW, grad_dtype,
                 dW_accumulate, status, workspace, workspace_bytes, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_chunked(X or None, W or None, labels or None, B, T, H, V, dtype,
                             ignore_index, reduction, int(bool(shift)), chunk_rows,
                             grad_scale or None, loss or None, lse or None, n_valid or None,
                             dX or None, dW or None, grad_dtype, int(bool(dW_accumulate)),
                             status or None, workspace or None, workspace_bytes,
                             stream or None)


def flce_scale_grads(dX_in, dX, nx, dW_in, dW, nw, grad_dtype, scale, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_scale_grads(dX_in or None, dX or None, nx, dW_in or None, dW or None, nw,
                                 grad_dtype, scale or None, stream or None)


def flce_convert_grads(src, dst, n, dst_dtype, scale, accumulate, stream) -> int:
    """Returns the status code (0 on success); raises nothing."""
    return _LIB.flce_convert_grads(src or None, dst or None, n, dst_dtype, scale or None,
                                   int(bool(accumulate)), stream or None)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FLCE_DTYPE_BF16
    if t.dtype == torch.float32:
        return FLCE_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _reduction_code(reduction: str) -> int:
    if reduction == "mean":
        return FLCE_REDUCTION_MEAN
    if reduction == "sum":
        return FLCE_REDUCTION_SUM
    if reduction == "none":
        return FLCE_REDUCTION_NONE
    raise ValueError(f"unsupported reduction {reduction!r} (mean, sum or none)")


def _shape(hidden, weight, labels):
    if labels.dim() == 2:
        B, T = labels.shape
    elif labels.dim() == 1:
        B, T = 1, labels.shape[0]
    else:
        raise ValueError("labels must be [B, T] or [N]")
    H = hidden.shape[-1]
    if hidden.numel() != B * T * H:
        raise ValueError(f"hidden {tuple(hidden.shape)} does not match labels "
                         f"{tuple(labels.shape)}")
    if weight.dim() != 2 or weight.shape[1] != H:
        raise ValueError(f"weight must be [V, {H}], got {tuple(weight.shape)}")
    return int(B), int(T), int(H), int(weight.shape[0])


def _check_tensors(hidden, weight, labels):
    torch = _torch()
    for name, t in (("hidden", hidden), ("weight", weight), ("labels", labels)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if hidden.dtype != weight.dtype:
        raise TypeError("hidden and weight must have the same dtype")
    if labels.dtype != torch.int64:
        raise TypeError("labels must be int64")
    if hidden.device != weight.device or hidden.device != labels.device:
        raise ValueError("all tensors must be on one device")


def _stream_handle(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def workspace(B, T, H, V, dtype_code, device):
    torch = _torch()
    nbytes = flce_workspace_size(B, T, H, V, dtype_code)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device), nbytes


def forward(hidden, weight, labels, ignore_index=-100, shift=False, reduction="mean",
            ws=None):
    """(loss, lse, n_valid, status) as device tensors, no host synchronisation;
    loss is a scalar, or [B*T] per-row losses for reduction="none"."""
    torch = _torch()
    _check_tensors(hidden, weight, labels)
    B, T, H, V = _shape(hidden, weight, labels)
    dt = _dtype_code(hidden)
    dev = hidden.device
    if ws is None:
        ws, nbytes = workspace(B, T, H, V, dt, dev)
    else:
        nbytes = ws.numel()
    loss = torch.empty((B * T,) if reduction == "none" else (), dtype=torch.float32,
                       device=dev)
    lse = torch.empty(B * T, dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int64, device=dev)
    status = torch.empty((), dtype=torch.int32, device=dev)
    rc = flce_forward(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), B, T, H, V,
                      dt, int(ignore_index), _reduction_code(reduction), shift,
                      loss.data_ptr(), lse.data_ptr(), n_valid.data_ptr(),
                      status.data_ptr(), ws.data_ptr(), nbytes, _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward")
    return loss, lse, n_valid, status


def _dw_out(dW, weight, out_dtype, accumulate):
    torch = _torch()
    if dW is None:
        if accumulate:
            raise ValueError("accumulate=True needs the dW tensor to add to")
        return torch.empty(weight.shape, dtype=out_dtype, device=weight.device)
    if (dW.shape != weight.shape or dW.dtype != out_dtype or dW.device != weight.device
            or not dW.is_contiguous()):
        raise ValueError("dW must be a contiguous tensor shaped like weight, in the "
                         "gradient dtype, on the same device")
    return dW


def backward(hidden, weight, labels, lse, grad_scale=None, ignore_index=-100,
             shift=False, reduction="mean", grad_dtype=None, ws=None, dW=None,
             accumulate=False):
    """(dX, dW, status); grad_scale is a device float32 scalar, or [B*T] per-row
    values for reduction="none", or None (= 1).  dW: optional output tensor;
    accumulate=True adds the gradient to it."""
    torch = _torch()
    _check_tensors(hidden, weight, labels)
    B, T, H, V = _shape(hidden, weight, labels)
    dt = _dtype_code(hidden)
    gd = dt if grad_dtype is None else _dtype_code(torch.empty(0, dtype=grad_dtype))
    out_dtype = torch.float32 if gd == FLCE_DTYPE_F32 else hidden.dtype
    dev = hidden.device
    if ws is None:
        ws, nbytes = workspace(B, T, H, V, dt, dev)
    else:
        nbytes = ws.numel()
    dX = torch.empty(hidden.shape, dtype=out_dtype, device=dev)
    dW = _dw_out(dW, weight, out_dtype, accumulate)
    status = torch.empty((), dtype=torch.int32, device=dev)
    gs = 0
    if grad_scale is not None:
        grad_scale = grad_scale.to(device=dev, dtype=torch.float32).contiguous()
        gs = grad_scale.data_ptr()
    lse = lse.to(device=dev, dtype=torch.float32).contiguous()
    rc = flce_backward(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), B, T, H,
                       V, dt, int(ignore_index), _reduction_code(reduction), shift,
                       lse.data_ptr(), gs, dX.data_ptr(), dW.data_ptr(), gd, accumulate,
                       status.data_ptr(), ws.data_ptr(), nbytes, _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_backward")
    return dX, dW, status


def shard_forward(hidden, weight_shard, labels, v_begin, V_total, ignore_index=-100,
                  shift=False, ws=None):
    """(lse_shard, zt_shard, status) of one vocabulary shard."""
    torch = _torch()
    _check_tensors(hidden, weight_shard, labels)
    B, T, H, V = _shape(hidden, weight_shard, labels)
    dt = _dtype_code(hidden)
    dev = hidden.device
    if ws is None:
        ws, nbytes = workspace(B, T, H, V, dt, dev)
    else:
        nbytes = ws.numel()
    lse = torch.empty(B * T, dtype=torch.float32, device=dev)
    zt = torch.empty(B * T, dtype=torch.float32, device=dev)
    status = torch.empty((), dtype=torch.int32, device=dev)
    rc = flce_shard_forward(hidden.data_ptr(), weight_shard.data_ptr(), labels.data_ptr(), B,
                            T, H, V, int(v_begin), int(V_total), dt, int(ignore_index), shift,
                            lse.data_ptr(), zt.data_ptr(), status.data_ptr(), ws.data_ptr(),
                            nbytes, _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_shard_forward")
    return lse, zt, status


def shard_merge(lse_shards, zt_shards, labels, V_total, ignore_index=-100, shift=False,
                reduction="mean"):
    """(loss, lse, n_valid, status) from the stacked shard outputs [shards, B*T]."""
    torch = _torch()
    lse_shards = lse_shards.to(torch.float32).contiguous()
    zt_shards = zt_shards.to(torch.float32).contiguous()
    if labels.dim() == 2:
        B, T = labels.shape
    else:
        B, T = 1, labels.shape[0]
    dev = labels.device
    nbytes = flce_shard_merge_workspace_size(B, T)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    loss = torch.empty((B * T,) if reduction == "none" else (), dtype=torch.float32,
                       device=dev)
    lse = torch.empty(B * T, dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int64, device=dev)
    status = torch.empty((), dtype=torch.int32, device=dev)
    rc = flce_shard_merge(lse_shards.data_ptr(), zt_shards.data_ptr(), lse_shards.shape[0],
                          labels.contiguous().data_ptr(), int(B), int(T), int(V_total),
                          int(ignore_index), shift, _reduction_code(reduction),
                          loss.data_ptr(), lse.data_ptr(), n_valid.data_ptr(),
                          status.data_ptr(), ws.data_ptr(), nbytes, _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_shard_merge")
    return loss, lse, n_valid, status


def shard_backward(hidden, weight_shard, labels, lse, v_begin, V_total, grad_scale=None,
                   ignore_index=-100, shift=False, reduction="mean", grad_dtype=None,
                   ws=None, dW=None, accumulate=False):
    """(dX_partial fp32, dW_shard, status) of one vocabulary shard."""
    torch = _torch()
    _check_tensors(hidden, weight_shard, labels)
    B, T, H, V = _shape(hidden, weight_shard, labels)
    dt = _dtype_code(hidden)
    gd = dt if grad_dtype is None else _dtype_code(torch.empty(0, dtype=grad_dtype))
    out_dtype = torch.float32 if gd == FLCE_DTYPE_F32 else hidden.dtype
    dev = hidden.device
    if ws is None:
        ws, nbytes = workspace(B, T, H, V, dt, dev)
    else:
        nbytes = ws.numel()
    dXp = torch.empty(hidden.shape, dtype=torch.float32, device=dev)
    dW = _dw_out(dW, weight_shard, out_dtype, accumulate)
    status = torch.empty((), dtype=torch.int32, device=dev)
    gs = 0
    if grad_scale is not None:
        grad_scale = grad_scale.to(device=dev, dtype=torch.float32).contiguous()
        gs = grad_scale.data_ptr()
    lse = lse.to(device=dev, dtype=torch.float32).contiguous()
    rc = flce_shard_backward(hidden.data_ptr(), weight_shard.data_ptr(), labels.data_ptr(), B,
                             T, H, V, int(v_begin), int(V_total), dt, int(ignore_index),
                             _reduction_code(reduction), shift, lse.data_ptr(), gs,
                             dXp.data_ptr(), dW.data_ptr(), gd, accumulate,
                             status.data_ptr(), ws.data_ptr(), nbytes, _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_shard_backward")
    return dXp, dW, status


def chunked_workspace(B, T, H, V, dtype_code, device, chunk_rows=0):
    torch = _torch()
    nbytes = flce_chunked_workspace_size(B, T, H, V, dtype_code, chunk_rows)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device), nbytes


def _convert(src, dst, accumulate=False, scale=None):
    """dst = round(scale * src (+ dst)) through flce_convert_grads."""
    rc = flce_convert_grads(src.data_ptr(), dst.data_ptr(), src.numel(), _dtype_code(dst),
                            0 if scale is None else scale.data_ptr(), accumulate,
                            _stream_handle(src.device))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_convert_grads")


def chunked(hidden, weight, labels, grad_scale=None, ignore_index=-100, shift=False,
            reduction="mean", grad_dtype=None, ws=None, chunk_rows=0, dW=None,
            accumulate=False, round_once=False):
    """(loss, lse, n_valid, dX, dW, status) from one flce_chunked call; a
    caller-provided ws must come from chunked_workspace with the same
    chunk_rows.  round_once=True with bf16 gradients keeps dX and dW in FP32
    over all row chunks (flce_chunked with FP32 outputs) and rounds them once
    (flce_convert_grads), at the price of FP32 temporaries; otherwise a bf16
    dW is rounded once per row chunk."""
    torch = _torch()
    _check_tensors(hidden, weight, labels)
    B, T, H, V = _shape(hidden, weight, labels)
    dt = _dtype_code(hidden)
    gd = dt if grad_dtype is None else _dtype_code(torch.empty(0, dtype=grad_dtype))
    if round_once and gd == FLCE_DTYPE_BF16:
        loss, lse, n_valid, dX32, dW32, status = chunked(
            hidden, weight, labels, grad_scale, ignore_index, shift, reduction,
            torch.float32, ws, chunk_rows)
        dX = torch.empty(hidden.shape, dtype=hidden.dtype, device=hidden.device)
        _convert(dX32, dX)
        dW = _dw_out(dW, weight, hidden.dtype, accumulate)
        _convert(dW32, dW, accumulate=accumulate)
        return loss, lse, n_valid, dX, dW, status
    out_dtype = torch.float32 if gd == FLCE_DTYPE_F32 else hidden.dtype
    dev = hidden.device
    if ws is None:
        ws, nbytes = chunked_workspace(B, T, H, V, dt, dev, chunk_rows)
    else:
        nbytes = ws.numel()
    loss = torch.empty((B * T,) if reduction == "none" else (), dtype=torch.float32,
                       device=dev)
    lse = torch.empty(B * T, dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int64, device=dev)
    status = torch.empty((), dtype=torch.int32, device=dev)
    dX = torch.empty(hidden.shape, dtype=out_dtype, device=dev)
    dW = _dw_out(dW, weight, out_dtype, accumulate)
    gs = 0
    if grad_scale is not None:
        grad_scale = grad_scale.to(device=dev, dtype=torch.float32).contiguous()
        gs = grad_scale.data_ptr()
    rc = flce_chunked(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), B, T, H, V,
                      dt, int(ignore_index), _reduction_code(reduction), shift,
                      int(chunk_rows), gs,
                      loss.data_ptr(), lse.data_ptr(), n_valid.data_ptr(), dX.data_ptr(),
                      dW.data_ptr(), gd, accumulate, status.data_ptr(), ws.data_ptr(), nbytes,
                      _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_chunked")
    return loss, lse, n_valid, dX, dW, status


def _autograd_function():
    torch = _torch()

    class LinearCrossEntropy(torch.autograd.Function):
        @staticmethod
        def forward(ctx, hidden, weight, labels, ignore_index, shift, reduction):
            loss, lse, _, _ = forward(hidden, weight, labels, ignore_index, shift,
                                      reduction)
            ctx.save_for_backward(hidden, weight, labels, lse)
            ctx.args = (ignore_index, shift, reduction)
            return loss.reshape(labels.shape) if reduction == "none" else loss

        @staticmethod
        def backward(ctx, grad_out):
            hidden, weight, labels, lse = ctx.saved_tensors
            ignore_index, shift, reduction = ctx.args
            g = grad_out.reshape(-1) if reduction == "none" else grad_out.reshape(())
            dX, dW, _ = backward(hidden, weight, labels, lse, grad_scale=g,
                                 ignore_index=ignore_index, shift=shift,
                                 reduction=reduction)
            return dX, dW, None, None, None, None

    class LinearCrossEntropyChunked(torch.autograd.Function):
        """Gradients formed in the forward (flce_chunked, grad_scale 1, FP32
        sums over all row chunks), scaled by the upstream gradient and
        rounded once to the input dtype in the backward (flce_convert_grads,
        out of place: a second backward through a retained graph scales the
        saved sums afresh)."""

        @staticmethod
        def forward(ctx, hidden, weight, labels, ignore_index, shift, reduction):
            loss, _, _, dX, dW, _ = chunked(hidden, weight, labels,
                                            ignore_index=ignore_index, shift=shift,
                                            reduction=reduction, grad_dtype=torch.float32)
            ctx.save_for_backward(dX, dW)
            ctx.out_dtype = hidden.dtype
            return loss

        @staticmethod
        def backward(ctx, grad_out):
            dX, dW = ctx.saved_tensors
            g = grad_out.reshape(()).to(dtype=torch.float32).contiguous()
            gX = torch.empty(dX.shape, dtype=ctx.out_dtype, device=dX.device)
            gW = torch.empty(dW.shape, dtype=ctx.out_dtype, device=dW.device)
            _convert(dX, gX, scale=g)
            _convert(dW, gW, scale=g)
            return gX, gW, None, None, None, None

    return LinearCrossEntropy, LinearCrossEntropyChunked


_FN = None


def linear_cross_entropy(hidden, weight, labels, ignore_index=-100, shift=False,
                         reduction="mean", mode="recompute"):
    """Fused ``cross_entropy(hidden @ weight.T, targets)`` without the logits.

    hidden [B, T, H] or [N, H]; weight [V, H]; labels [B, T] (or [N], one
    sequence); bfloat16 or float32 on the GPU.  Returns a float32 scalar loss
    (reduction "mean" or "sum") or per-token losses shaped like labels
    ("none"; 0 on ignored tokens, their negatives are the target log-probs),
    which backpropagate into hidden and weight.  mode="recompute"
    (forward, then a backward that recomputes the logits; extra memory linear
    in N) or "chunked" (gradients formed during the forward over row chunks;
    one logits pass, extra memory proportional to a chunk of rows times V)."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    if reduction not in ("mean", "sum", "none"):
        raise ValueError(f"unsupported reduction {reduction!r} (mean, sum or none)")
    if mode not in ("recompute", "chunked"):
        raise ValueError(f"unsupported mode {mode!r} (recompute or chunked)")
    if mode == "chunked" and reduction == "none":
        # the chunked mode forms the gradients before the upstream gradient
        # exists; a per-token one cannot be applied afterwards
        raise ValueError('mode="chunked" needs a scalar loss (mean or sum)')
    fn = _FN[0] if mode == "recompute" else _FN[1]
    return fn.apply(hidden.contiguous(), weight.contiguous(), labels.contiguous(),
                    int(ignore_index), bool(shift), reduction)

"""ctypes binding of liblce03.so (include/flce.h), same function names.

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity, turned into raw pointers and handed to the C ABI together with the
current HIP stream. Every computation happens in the library's HIP kernels.
PyTorch is used to allocate device memory (outputs and workspace, when the
caller does not pass them) and to name the stream. A non-OK status raises
FlceError. The library is loaded on first use; if it has not been built the
import fails loudly (there is no fallback).
"""

import ctypes
import os
import re

import torch  # loads the HIP runtime that the library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblce03.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "flce.h")

F32, BF16, F16 = 0, 1, 2
REDUCTIONS = {"none": 0, "sum": 1, "mean": 2}
OK, E_INVALID_ARG, E_WORKSPACE, E_UNSUPPORTED, E_TARGET, E_HIP = range(6)
TIMING_KINDS = {"logits_gemm": 0, "row_ce": 1, "grad_x_gemm": 2, "grad_w_gemm": 3, "other": 4}

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_int = ctypes.c_int

_SIGNATURES = {
    "flce_status_string": (ctypes.c_char_p, [_int]),
    "flce_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _i64]),
    "flce_plan": (_int, [_i64, _i64, _i64, _int, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i32)]),
    "flce_forward_backward": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _i32, _int,
                                     _vp, _vp, _vp, _vp, _vp, _sz, _i64, _vp]),
    "flce_forward_backward_ex": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _i32, _int,
                                        _int, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _vp]),
    "ce_workspace_bytes": (_sz, [_i64, _i64]),
    "ce_forward_backward": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _i32, _int, _vp, _vp, _sz, _vp]),
    "ce_forward_backward_noalloc": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _i32, _int, _vp, _vp]),
    "ce_shard_stats": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _int, _i32, _vp, _vp, _vp, _vp,
                              _sz, _vp]),
    "flce_shard_stats": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _i32,
                                _vp, _vp, _vp, _vp, _sz, _i64, _vp]),
    "ce_combine_shard_stats": (_int, [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i32, _int, _vp, _vp,
                                      _vp, _sz, _vp]),
    "flce_shard_backward": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _i32,
                                   _int, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _vp]),
    "flce_shard_backward_ex": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int,
                                      _i32, _int, _vp, _int, _vp, _vp, _vp, _vp, _sz, _i64, _vp]),
    "flce_shift_labels": (_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "flce_dpo_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _int, _i64]),
    "flce_dpo_forward_backward": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _i32, _vp,
                                         ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _vp]),
    "flce_dpo_forward_backward_ex": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _i32,
                                            _vp, ctypes.c_float, _int, _vp, _vp, _vp, _vp, _vp,
                                            _sz, _i64, _vp]),
    "flce_jsd_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _i64]),
    "flce_jsd_forward_backward_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                            _int, _i32, _int, ctypes.c_float, _int, _vp, _vp,
                                            _vp, _vp, _sz, _i64, _vp]),
    "flce_jsd_forward_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                                         _i32, _int, ctypes.c_float, _vp, _vp, _vp, _vp, _sz,
                                         _i64, _vp]),
    "flce_multihead_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _int, _i64]),
    "flce_multihead_forward_backward": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                                               _i32, _int, _vp, _vp, _vp, _vp, _vp, _sz, _i64,
                                               _vp]),
    "flce_multihead_forward_backward_ex": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                  _int, _i32, _int, _int, _vp, _vp, _vp, _vp, _vp,
                                                  _sz, _i64, _vp]),
    "flce_check_device_error": (_int, [_vp, _vp]),
    "flce_set_row_packing": (_int, [_int]),
    "flce_workspace_parts": (_int, [_i64, _i64, _i64, _int, _i64, ctypes.POINTER(_sz)]),
    "flce_timing_enable": (_int, [_int]),
    "flce_timing_read": (_int, [_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "flce_timing_reset": (_int, []),
}

_lib = None


class FlceError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_text(status)})")


def header_functions():
    """Names of the functions include/flce.h declares."""
    with open(HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)


def lib():
    """The loaded library (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m linear_cross_entropy_03_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_text(status):
    return lib().flce_status_string(int(status)).decode()


flce_status_string = status_text


def _check(status, where):
    if status != OK:
        raise FlceError(status, where)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32, bfloat16 or float16")


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _red(reduction):
    try:
        return REDUCTIONS[reduction]
    except KeyError:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}") from None


def flce_workspace_bytes(N, H, V, dtype=BF16, chunk_rows=0):
    return int(lib().flce_workspace_bytes(N, H, V, dtype, chunk_rows))


def ce_workspace_bytes(N, V):
    return int(lib().ce_workspace_bytes(N, V))


def flce_plan(N, H, V, dtype=BF16, chunk_rows=0):
    """(rows per chunk, grad_X K-splits) the planner picks."""
    c = _i64()
    s = _i32()
    _check(lib().flce_plan(N, H, V, dtype, chunk_rows, ctypes.byref(c), ctypes.byref(s)), "flce_plan")
    return int(c.value), int(s.value)


WORKSPACE_PARTS = ("rows", "chunk_logits", "split_partials", "pack_lists")


def flce_workspace_parts(N, H, V, dtype=BF16, chunk_rows=0):
    """The planner's workspace regions in bytes, by name (they sum to
    flce_workspace_bytes)."""
    arr = (_sz * len(WORKSPACE_PARTS))()
    _check(lib().flce_workspace_parts(N, H, V, dtype, chunk_rows, arr), "flce_workspace_parts")
    return dict(zip(WORKSPACE_PARTS, (int(v) for v in arr)))


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _grad_arg(want, shape, device, dtype=None):
    """A gradient output: the given tensor, a new one (True; float32 unless
    dtype is given), or None."""
    if isinstance(want, torch.Tensor):
        return want
    return _empty(shape, dtype or torch.float32, device) if want else None


def flce_forward_backward(X, W, targets, bias=None, ignore_index=-100, reduction="mean",
                          grad_X=True, grad_W=True, grad_bias=None, loss=None, workspace=None,
                          chunk_rows=0, stream=None, grad_dtype="f32"):
    """Fused linear cross-entropy forward + backward.

    X [N, H] and W [V, H] (and bias [V]) share one dtype (float32, bfloat16 or
    float16); targets is int32 [N]. grad_X / grad_W / grad_bias: a
    preallocated tensor, True (allocate), or False/None (skip; grad_bias
    defaults to bias is not None). grad_dtype "f32" gives float32 gradients;
    "input" gives them in X's 16-bit dtype (flce_forward_backward_ex).
    Returns (loss, grad_X, grad_W, grad_bias).
    """
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    dt = _dtype_code(X)
    if grad_dtype not in ("f32", "input"):
        raise ValueError("grad_dtype must be 'f32' or 'input'")
    g16 = grad_dtype == "input"
    gtorch = X.dtype if g16 else torch.float32
    if grad_bias is None:
        grad_bias = bias is not None
    gX = _grad_arg(grad_X, (N, H), dev, gtorch)
    gW = _grad_arg(grad_W, (V, H), dev, gtorch)
    gb = _grad_arg(grad_bias, (V,), dev, gtorch)
    if loss is None:
        loss = _empty((N,) if reduction == "none" else (1,), torch.float32, dev)
    if workspace is None:
        workspace = _empty((max(1, flce_workspace_bytes(N, H, V, dt, chunk_rows)),), torch.uint8, dev)
    args = [_ptr(X, "X"), _ptr(W, "W", X.dtype), _ptr(bias, "bias", X.dtype),
            _ptr(targets, "targets", torch.int32), N, H, V, dt, ignore_index, _red(reduction)]
    rest = [_ptr(loss, "loss", torch.float32), _ptr(gX, "grad_X", gtorch),
            _ptr(gW, "grad_W", gtorch), _ptr(gb, "grad_bias", gtorch),
            _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), chunk_rows,
            _stream(stream)]
    if g16:
        st = lib().flce_forward_backward_ex(*args, dt, *rest)
        _check(st, "flce_forward_backward_ex")
    else:
        st = lib().flce_forward_backward(*args, *rest)
        _check(st, "flce_forward_backward")
    return loss, gX, gW, gb


def flce_multihead_workspace_bytes(N, H, V, K, dtype=BF16, chunk_rows=0):
    return int(lib().flce_multihead_workspace_bytes(N, H, V, K, dtype, chunk_rows))


def flce_multihead_forward_backward(X, W, targets, bias=None, ignore_index=-100, reduction="mean",
                                    grad_X=True, grad_W=True, grad_bias=None, loss=None,
                                    workspace=None, chunk_rows=0, stream=None, grad_dtype="f32"):
    """K heads over shared X [N, H]: W [K, V, H], targets [K, N] (int32),
    bias [K, V] or None. Returns (loss [K] or [K, N], grad_X (sum over heads),
    grad_W [K, V, H], grad_bias [K, V]); grad_dtype as in flce_forward_backward."""
    N, H = X.shape
    K, V, _ = W.shape
    dev = X.device
    dt = _dtype_code(X)
    if grad_dtype not in ("f32", "input"):
        raise ValueError("grad_dtype must be 'f32' or 'input'")
    g16 = grad_dtype == "input"
    gtorch = X.dtype if g16 else torch.float32
    if grad_bias is None:
        grad_bias = bias is not None
    gX = _grad_arg(grad_X, (N, H), dev, gtorch)
    gW = _grad_arg(grad_W, (K, V, H), dev, gtorch)
    gb = _grad_arg(grad_bias, (K, V), dev, gtorch)
    if loss is None:
        loss = _empty((K, N) if reduction == "none" else (K,), torch.float32, dev)
    if workspace is None:
        workspace = _empty((max(1, flce_multihead_workspace_bytes(N, H, V, K, dt, chunk_rows)),),
                           torch.uint8, dev)
    args = [_ptr(X, "X"), _ptr(W, "W", X.dtype), _ptr(bias, "bias", X.dtype),
            _ptr(targets, "targets", torch.int32), N, H, V, K, dt, ignore_index, _red(reduction)]
    rest = [_ptr(loss, "loss", torch.float32), _ptr(gX, "grad_X", gtorch),
            _ptr(gW, "grad_W", gtorch), _ptr(gb, "grad_bias", gtorch),
            _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), chunk_rows,
            _stream(stream)]
    if g16:
        st = lib().flce_multihead_forward_backward_ex(*args, dt, *rest)
        _check(st, "flce_multihead_forward_backward_ex")
    else:
        st = lib().flce_multihead_forward_backward(*args, *rest)
        _check(st, "flce_multihead_forward_backward")
    return loss, gX, gW, gb


def ce_forward_backward(logits, targets, ignore_index=-100, reduction="mean", grad_logits=True,
                        loss=None, workspace=None, stream=None):
    """Cross-entropy over given logits [N, V] with its gradient.

    grad_logits: a tensor (may be `logits` itself for in-place), True
    (allocate), or False/None (loss only). Returns (loss, grad_logits).
    """
    N, V = logits.shape
    dev = logits.device
    dt = _dtype_code(logits)
    if isinstance(grad_logits, torch.Tensor):
        g = grad_logits
    elif grad_logits:
        g = torch.empty_like(logits)
    else:
        g = None
    if loss is None:
        loss = _empty((N,) if reduction == "none" else (1,), torch.float32, dev)
    if workspace is None:
        workspace = _empty((max(1, ce_workspace_bytes(N, V)),), torch.uint8, dev)
    st = lib().ce_forward_backward(
        _ptr(logits, "logits"), _ptr(g, "grad_logits", logits.dtype),
        _ptr(targets, "targets", torch.int32), N, V, dt, ignore_index, _red(reduction),
        _ptr(loss, "loss", torch.float32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "ce_forward_backward")
    return loss, g


def ce_forward_backward_noalloc(logits, targets, ignore_index=-100, reduction="mean",
                                grad_logits=True, loss=None, stream=None):
    """ce_forward_backward through the entry point that takes no workspace
    (its scratch is the library's per-device static array; N <= 4194304).
    Outputs are the caller's (allocated here with torch when not given)."""
    N, V = logits.shape
    dt = _dtype_code(logits)
    if isinstance(grad_logits, torch.Tensor):
        g = grad_logits
    elif grad_logits:
        g = torch.empty_like(logits)
    else:
        g = None
    if loss is None:
        loss = _empty((N,) if reduction == "none" else (1,), torch.float32, logits.device)
    st = lib().ce_forward_backward_noalloc(
        _ptr(logits, "logits"), _ptr(g, "grad_logits", logits.dtype),
        _ptr(targets, "targets", torch.int32), N, V, dt, ignore_index, _red(reduction),
        _ptr(loss, "loss", torch.float32), _stream(stream))
    _check(st, "ce_forward_backward_noalloc")
    return loss, g


def ce_shard_stats(logits_shard, targets, vocab_start, V_global, ignore_index=-100,
                   out=None, workspace=None, stream=None):
    """Per-row (max, sumexp, target logit) of one vocabulary shard."""
    N, Vl = logits_shard.shape
    dev = logits_shard.device
    m, s, t = out if out is not None else tuple(_empty((N,), torch.float32, dev) for _ in range(3))
    if workspace is None:
        workspace = _empty((max(1, ce_workspace_bytes(N, V_global)),), torch.uint8, dev)
    st = lib().ce_shard_stats(
        _ptr(logits_shard, "logits_shard"), _ptr(targets, "targets", torch.int32), N, Vl,
        vocab_start, V_global, _dtype_code(logits_shard), ignore_index,
        _ptr(m, "row_max", torch.float32), _ptr(s, "row_sumexp", torch.float32),
        _ptr(t, "row_target_logit", torch.float32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "ce_shard_stats")
    return m, s, t


def flce_shard_stats(X, W_shard, targets, vocab_start, V_global, bias_shard=None,
                     ignore_index=-100, out=None, workspace=None, chunk_rows=0, stream=None):
    """Shard statistics of X W_shard^T (+ bias_shard) without holding the logits."""
    N, H = X.shape
    Vl = W_shard.shape[0]
    dev = X.device
    dt = _dtype_code(X)
    m, s, t = out if out is not None else tuple(_empty((N,), torch.float32, dev) for _ in range(3))
    if workspace is None:
        workspace = _empty((max(1, flce_workspace_bytes(N, H, Vl, dt, chunk_rows)),), torch.uint8, dev)
    st = lib().flce_shard_stats(
        _ptr(X, "X"), _ptr(W_shard, "W_shard", X.dtype), _ptr(bias_shard, "bias_shard", X.dtype),
        _ptr(targets, "targets", torch.int32), N, H, Vl, vocab_start, V_global, dt, ignore_index,
        _ptr(m, "row_max", torch.float32), _ptr(s, "row_sumexp", torch.float32),
        _ptr(t, "row_target_logit", torch.float32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), chunk_rows, _stream(stream))
    _check(st, "flce_shard_stats")
    return m, s, t


def ce_combine_shard_stats(shard_max, shard_sumexp, shard_target_logit, targets, V_global,
                           ignore_index=-100, reduction="mean", row_lse=None, loss=None,
                           workspace=None, stream=None):
    """Global per-row lse and the loss from P shards' statistics ([P, N] each).
    Returns (loss, row_lse)."""
    P, N = shard_max.shape
    dev = shard_max.device
    red = _red(reduction)
    if row_lse is None:
        row_lse = _empty((N,), torch.float32, dev)
    if loss is None:
        loss = _empty((N,) if reduction == "none" else (1,), torch.float32, dev)
    if workspace is None:
        workspace = _empty((max(1, ce_workspace_bytes(N, V_global)),), torch.uint8, dev)
    st = lib().ce_combine_shard_stats(
        _ptr(shard_max, "shard_max", torch.float32), _ptr(shard_sumexp, "shard_sumexp", torch.float32),
        _ptr(shard_target_logit, "shard_target_logit", torch.float32), P, N,
        _ptr(targets, "targets", torch.int32), V_global, ignore_index, red,
        _ptr(row_lse, "row_lse", torch.float32), _ptr(loss, "loss", torch.float32),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "ce_combine_shard_stats")
    return loss, row_lse


def _grad_type(X, grad_dtype):
    """(16-bit?, torch dtype) of the gradient outputs for grad_dtype "f32" or "input"."""
    if grad_dtype not in ("f32", "input"):
        raise ValueError("grad_dtype must be 'f32' or 'input'")
    g16 = grad_dtype == "input"
    return g16, (X.dtype if g16 else torch.float32)


def flce_shard_backward(X, W_shard, targets, row_lse, vocab_start, V_global, bias_shard=None,
                        ignore_index=-100, reduction="mean", grad_X=True, grad_W=True,
                        grad_bias=None, workspace=None, chunk_rows=0, stream=None,
                        grad_dtype="f32"):
    """One vocabulary shard's part of the FLCE gradients, given the global
    row lse. Gradient arguments: True = allocate, False/None = skip, or a
    tensor to write into; grad_dtype "input" writes them in X's 16-bit dtype
    (flce_shard_backward_ex). Returns (grad_X partial, grad_W_shard, grad_bias_shard)."""
    N, H = X.shape
    Vl = W_shard.shape[0]
    dev = X.device
    dt = _dtype_code(X)
    red = _red(reduction)
    g16, gtorch = _grad_type(X, grad_dtype)
    if grad_bias is None:
        grad_bias = bias_shard is not None
    gX = _grad_arg(grad_X, (N, H), dev, gtorch)
    gW = _grad_arg(grad_W, (Vl, H), dev, gtorch)
    gb = _grad_arg(grad_bias, (Vl,), dev, gtorch)
    if workspace is None:
        workspace = _empty((max(1, flce_workspace_bytes(N, H, Vl, dt, chunk_rows)),), torch.uint8, dev)
    head = [_ptr(X, "X"), _ptr(W_shard, "W_shard", X.dtype), _ptr(bias_shard, "bias_shard", X.dtype),
            _ptr(targets, "targets", torch.int32), N, H, Vl, vocab_start, V_global, dt, ignore_index,
            red, _ptr(row_lse, "row_lse", torch.float32)]
    tail = [_ptr(gX, "grad_X", gtorch), _ptr(gW, "grad_W_shard", gtorch),
            _ptr(gb, "grad_bias_shard", gtorch), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), chunk_rows, _stream(stream)]
    if g16:
        _check(lib().flce_shard_backward_ex(*head, dt, *tail), "flce_shard_backward_ex")
    else:
        _check(lib().flce_shard_backward(*head, *tail), "flce_shard_backward")
    return gX, gW, gb


def flce_jsd_workspace_bytes(N, H_s, V, dtype=BF16, chunk_rows=0):
    return int(lib().flce_jsd_workspace_bytes(N, H_s, V, dtype, chunk_rows))


def flce_jsd_forward_backward(X_s, W_s, X_t, W_t, targets, temperature=1.0, ignore_index=-100,
                              reduction="mean", grad_X=True, grad_W=True, loss=None,
                              workspace=None, chunk_rows=0, stream=None, grad_dtype="f32"):
    """Jensen-Shannon distillation of a student head (X_s, W_s) towards a
    frozen teacher head (X_t, W_t); grad_dtype "input" writes the gradients in
    X_s's 16-bit dtype (flce_jsd_forward_backward_ex). Returns (loss, grad_X_s, grad_W_s)."""
    N, Hs = X_s.shape
    V = W_s.shape[0]
    Ht = X_t.shape[1]
    dev = X_s.device
    dt = _dtype_code(X_s)
    g16, gtorch = _grad_type(X_s, grad_dtype)
    gX = _grad_arg(grad_X, (N, Hs), dev, gtorch)
    gW = _grad_arg(grad_W, (V, Hs), dev, gtorch)
    if loss is None:
        loss = _empty((N,) if reduction == "none" else (1,), torch.float32, dev)
    if workspace is None:
        workspace = _empty((max(1, flce_jsd_workspace_bytes(N, Hs, V, dt, chunk_rows)),),
                           torch.uint8, dev)
    head = [_ptr(X_s, "X_s"), _ptr(W_s, "W_s", X_s.dtype), _ptr(X_t, "X_t", X_s.dtype),
            _ptr(W_t, "W_t", X_s.dtype), _ptr(targets, "targets", torch.int32), N, Hs, Ht, V, dt,
            ignore_index, _red(reduction), float(temperature)]
    tail = [_ptr(loss, "loss", torch.float32), _ptr(gX, "grad_X_s", gtorch),
            _ptr(gW, "grad_W_s", gtorch), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), chunk_rows, _stream(stream)]
    if g16:
        _check(lib().flce_jsd_forward_backward_ex(*head, dt, *tail), "flce_jsd_forward_backward_ex")
    else:
        _check(lib().flce_jsd_forward_backward(*head, *tail), "flce_jsd_forward_backward")
    return loss, gX, gW


def flce_dpo_workspace_bytes(n_pairs, seq_len, H, V, dtype=BF16, chunk_rows=0):
    return int(lib().flce_dpo_workspace_bytes(n_pairs, seq_len, H, V, dtype, chunk_rows))


def flce_dpo_forward_backward(X, W, targets, n_pairs, seq_len, ref_logps, beta=0.1,
                              ignore_index=-100, grad_X=True, grad_W=True, pair_loss=True,
                              loss=None, workspace=None, chunk_rows=0, stream=None,
                              grad_dtype="f32"):
    """DPO over 2 * n_pairs sequences of seq_len rows (chosen first);
    grad_dtype "input" writes the gradients in X's 16-bit dtype
    (flce_dpo_forward_backward_ex). Returns (loss [1], pair_loss [n_pairs] or
    None, grad_X, grad_W)."""
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    dt = _dtype_code(X)
    g16, gtorch = _grad_type(X, grad_dtype)
    gX = _grad_arg(grad_X, (N, H), dev, gtorch)
    gW = _grad_arg(grad_W, (V, H), dev, gtorch)
    pl = pair_loss if isinstance(pair_loss, torch.Tensor) else (
        _empty((max(1, n_pairs),), torch.float32, dev) if pair_loss else None)
    if loss is None:
        loss = _empty((1,), torch.float32, dev)
    if workspace is None:
        workspace = _empty((max(1, flce_dpo_workspace_bytes(n_pairs, seq_len, H, V, dt, chunk_rows)),),
                           torch.uint8, dev)
    head = [_ptr(X, "X"), _ptr(W, "W", X.dtype), _ptr(targets, "targets", torch.int32), n_pairs,
            seq_len, H, V, dt, ignore_index, _ptr(ref_logps, "ref_logps", torch.float32), float(beta)]
    tail = [_ptr(loss, "loss", torch.float32), _ptr(pl, "pair_loss", torch.float32),
            _ptr(gX, "grad_X", gtorch), _ptr(gW, "grad_W", gtorch), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), chunk_rows, _stream(stream)]
    if g16:
        _check(lib().flce_dpo_forward_backward_ex(*head, dt, *tail), "flce_dpo_forward_backward_ex")
    else:
        _check(lib().flce_dpo_forward_backward(*head, *tail), "flce_dpo_forward_backward")
    return loss, pl, gX, gW


def flce_shift_labels(labels, ignore_index=-100, out=None, stream=None):
    """Causal-LM targets [B*S] from labels [B, S] (int32)."""
    Bn, S = labels.shape
    if out is None:
        out = _empty((Bn * S,), torch.int32, labels.device)
    _check(lib().flce_shift_labels(_ptr(labels, "labels", torch.int32), Bn, S, ignore_index,
                                   _ptr(out, "targets", torch.int32), _stream(stream)),
           "flce_shift_labels")
    return out


def flce_check_device_error(workspace, stream=None):
    """Status of the last call that used `workspace` (waits for the stream)."""
    return int(lib().flce_check_device_error(_ptr(workspace, "workspace"), _stream(stream)))


def flce_set_row_packing(enable=True):
    """Turn row packing of ignored rows on or off; returns the previous setting."""
    return bool(lib().flce_set_row_packing(1 if enable else 0))


def flce_timing_enable(enable=True):
    _check(lib().flce_timing_enable(1 if enable else 0), "flce_timing_enable")


def flce_timing_read(kind):
    ms = ctypes.c_double()
    n = _i64()
    _check(lib().flce_timing_read(TIMING_KINDS.get(kind, kind), ctypes.byref(ms), ctypes.byref(n)),
           "flce_timing_read")
    return float(ms.value), int(n.value)


def flce_timing_reset():
    _check(lib().flce_timing_reset(), "flce_timing_reset")

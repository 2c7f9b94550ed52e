"""Python binding of the dense-layer training path for MI355X (gfx950).

A thin ctypes layer over libdense_layers_amd.so: it checks tensor devices,
dtypes and contiguity, allocates outputs and workspaces with PyTorch (device
memory and streams are the only things PyTorch provides here), and passes raw
pointers plus the current HIP stream to the C ABI.  Every step of the
computation runs in the library's HIP kernels; there is no CPU fallback and
importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libdense_layers_amd.so")

DL_F32, DL_BF16, DL_F16 = 0, 1, 2
ACT_IDENTITY, ACT_RELU, ACT_GELU_TANH = 0, 1, 2
OPT_SGD, OPT_ADAMW, OPT_ADAM = 0, 1, 2
LR_CONSTANT, LR_STEP, LR_WARMUP_COSINE, LR_WARMUP_LINEAR = 0, 1, 2, 3
STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "ALIASING",
          4: "WORKSPACE_TOO_SMALL", 5: "HIP_ERROR", 6: "LABEL_OUT_OF_RANGE"}

_ACTS = {"identity": ACT_IDENTITY, "relu": ACT_RELU, "gelu_tanh": ACT_GELU_TANH,
         None: ACT_IDENTITY}


class DenseError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                              ctypes.c_double, ctypes.c_size_t)


class DLLayer(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_int64), ("out", ctypes.c_int64),
                ("act", ctypes.c_int32),
                ("W", _vp), ("b", _vp), ("dW", _vp), ("db", _vp),
                ("mW", _vp), ("vW", _vp), ("mb", _vp), ("vb", _vp),
                ("eW", _vp), ("eb", _vp)]


class DLLrSchedule(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("warmup", ctypes.c_int64),
                ("total", ctypes.c_int64), ("step_size", ctypes.c_int64),
                ("min_lr", ctypes.c_double), ("gamma", ctypes.c_double)]


class DLLossScaler(ctypes.Structure):
    _fields_ = [("scale", _vp), ("growth_tracker", _vp), ("found_inf", _vp),
                ("growth_factor", ctypes.c_double), ("backoff_factor", ctypes.c_double),
                ("growth_interval", ctypes.c_int32)]


class DLOpt(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("lr", ctypes.c_double),
                ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64), ("step_dev", ctypes.c_void_p),
                ("max_grad_norm", ctypes.c_double), ("ema_decay", ctypes.c_double),
                ("schedule", ctypes.POINTER(DLLrSchedule)),
                ("scaler", ctypes.POINTER(DLLossScaler)),
                ("grad_norm", _vp)]


class DLParam(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("w", _vp), ("g", _vp), ("m", _vp), ("v", _vp),
                ("ema", _vp), ("w_bf16", _vp)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_c = {
    "dl_last_error": _sig("dl_last_error", ctypes.c_char_p, []),
    "dense_last_error": _sig("dense_last_error", ctypes.c_char_p, []),
    "dl_set_validate": _sig("dl_set_validate", _i32, [_i32]),
    "dl_empty_launches": _sig("dl_empty_launches", _i32, [_vp, _i32]),
    "dl_build_target": _sig("dl_build_target", ctypes.c_char_p, []),
    "dense_act_fwd": _sig("dense_act_fwd", _i32,
                          [_vp, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "dense_act_vjp": _sig("dense_act_vjp", _i32,
                          [_vp, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, _vp, _i32, _vp, _vp, _sz]),
    "dense_act_vjp_scaled": _sig("dense_act_vjp_scaled", _i32,
                                 [_vp, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "dense_cast_f16_scaled": _sig("dense_cast_f16_scaled", _i32,
                                  [_vp, _i64, _vp, _vp, _vp, _vp, _sz]),
    "dense_cast_f16_scaled_workspace_size": _sig("dense_cast_f16_scaled_workspace_size", _sz,
                                                 [_i64]),
    "dense_act_vjp_workspace_size": _sig("dense_act_vjp_workspace_size", _sz,
                                         [_i32, _i32, _i64, _i64, _i64]),
    "softmax_xent_fwd_bwd": _sig("softmax_xent_fwd_bwd", _i32,
                                 [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "softmax_xent_workspace_size": _sig("softmax_xent_workspace_size", _sz, [_i64, _i64]),
    "dense_xent_fwd": _sig("dense_xent_fwd", _i32,
                           [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _vp, _sz]),
    "dense_xent_fwd_workspace_size": _sig("dense_xent_fwd_workspace_size", _sz,
                                          [_i64, _i64, _i64]),
    "dense_xent_vjp": _sig("dense_xent_vjp", _i32,
                           [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _vp, _sz]),
    "dense_xent_vjp_workspace_size": _sig("dense_xent_vjp_workspace_size", _sz,
                                          [_i64, _i64, _i64]),
    "softmax_xent_fwd_bwd_noalloc": _sig("softmax_xent_fwd_bwd_noalloc", _i32,
                                         [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "sgd_step": _sig("sgd_step", _i32, [_vp, _i64, _vp, _vp, _f64]),
    "adamw_step": _sig("adamw_step", _i32,
                       [_vp, _i64, _vp, _vp, _vp, _vp, _f64, _f64, _f64, _f64, _f64, _i64]),
    "dense_cast_bf16": _sig("dense_cast_bf16", _i32, [_vp, _i64, _vp, _vp]),
    "dense_cast_bf16_t": _sig("dense_cast_bf16_t", _i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "dense_cast_f16": _sig("dense_cast_f16", _i32, [_vp, _i64, _vp, _vp]),
    "dense_cast_f16_t": _sig("dense_cast_f16_t", _i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "mlp_train_step": _sig("mlp_train_step", _i32,
                           [_vp, _i64, _i32, ctypes.POINTER(DLLayer), _vp, _vp,
                            ctypes.POINTER(DLOpt), _vp, _vp, _sz]),
    "mlp_train_step_mse": _sig("mlp_train_step_mse", _i32,
                               [_vp, _i64, _i32, ctypes.POINTER(DLLayer), _vp, _vp,
                                ctypes.POINTER(DLOpt), _vp, _vp, _sz]),
    "mlp_train_step_workspace_size": _sig("mlp_train_step_workspace_size", _sz,
                                          [_i64, _i32, ctypes.POINTER(DLLayer)]),
    "adam_step": _sig("adam_step", _i32,
                      [_vp, _i64, _vp, _vp, _vp, _vp, _f64, _f64, _f64, _f64, _f64, _i64]),
    "ema_update": _sig("ema_update", _i32, [_vp, _i64, _vp, _vp, _f64]),
    "clip_grad_norm": _sig("clip_grad_norm", _i32,
                           [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_i64), _f64, _vp,
                            _vp, _sz]),
    "clip_grad_norm_workspace_size": _sig("clip_grad_norm_workspace_size", _sz,
                                          [_i32, ctypes.POINTER(_i64)]),
    "optimizer_step": _sig("optimizer_step", _i32,
                           [_vp, ctypes.POINTER(DLOpt), _i32, ctypes.POINTER(DLParam), _vp, _sz]),
    "optimizer_step_workspace_size": _sig("optimizer_step_workspace_size", _sz,
                                          [_i32, ctypes.POINTER(DLParam)]),
    "mse_loss_fwd_bwd": _sig("mse_loss_fwd_bwd", _i32,
                             [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz]),
    "mse_loss_workspace_size": _sig("mse_loss_workspace_size", _sz, [_i64, _i64]),
    "dl_lr_at": _sig("dl_lr_at", _f64, [ctypes.POINTER(DLLrSchedule), _f64, _i64]),
    "dl_profile_begin": _sig("dl_profile_begin", _i32, [_i32]),
    "dl_profile_end": _sig("dl_profile_end", _i32, [_i32, _vp, _vp]),
    "dl_set_mlp_fusion": _sig("dl_set_mlp_fusion", _i32, [_i32]),
}

EXPORTS = ["dl_last_error", "dense_last_error", "dl_set_validate", "dl_empty_launches",
           "dl_build_target", "dense_act_fwd", "dense_act_vjp",
           "dense_act_vjp_scaled", "dense_cast_f16_scaled", "dense_cast_f16_scaled_workspace_size",
           "dense_act_vjp_workspace_size", "softmax_xent_fwd_bwd",
           "softmax_xent_workspace_size", "softmax_xent_fwd_bwd_noalloc", "dense_xent_fwd",
           "dense_xent_fwd_workspace_size", "dense_xent_vjp", "dense_xent_vjp_workspace_size",
           "sgd_step",
           "adamw_step",
           "dense_cast_bf16", "dense_cast_bf16_t", "dense_cast_f16", "dense_cast_f16_t",
           "mlp_train_step", "mlp_train_step_mse",
           "mlp_train_step_workspace_size", "adam_step", "ema_update", "clip_grad_norm",
           "clip_grad_norm_workspace_size", "optimizer_step", "optimizer_step_workspace_size",
           "mse_loss_fwd_bwd", "mse_loss_workspace_size", "dl_lr_at",
           "dl_profile_begin", "dl_profile_end", "dl_set_mlp_fusion"]


def build_target() -> str:
    return _c["dl_build_target"]().decode()


def profile_begin(capacity: int = 4096):
    """Start timing every launch this library makes from this thread."""
    _check(_c["dl_profile_begin"](capacity))


def profile_end(max_records: int = 4096):
    """Stop timing; returns [(launch name, milliseconds)] in launch order."""
    ms = (ctypes.c_float * max_records)()
    names = ctypes.create_string_buffer(48 * max_records)
    n = _c["dl_profile_end"](max_records, ms, names)
    if n < 0:
        raise DenseError(-n, _c["dl_last_error"]().decode())
    k = min(n, max_records)
    raw = names.raw
    return [(raw[i * 48:(i + 1) * 48].split(b"\0", 1)[0].decode(), float(ms[i])) for i in range(k)]


def set_mlp_fusion(level: int) -> int:
    """Fusion level of mlp_train_step on this thread (2: tail kernel, 1: head
    kernel only); returns the previous level."""
    prev = _c["dl_set_mlp_fusion"](level)
    if prev < 0:
        raise DenseError(-prev, _c["dl_last_error"]().decode())
    return prev


def set_validate(on: bool) -> bool:
    """Validate mode on this thread: cross-entropy calls check their labels
    on the device first (one stream synchronisation) and raise
    LABEL_OUT_OF_RANGE instead of producing NaN rows.  Returns the previous
    setting."""
    return bool(_c["dl_set_validate"](1 if on else 0))


def empty_launches(n: int, device=None):
    """n empty-kernel launches on the current stream (the launch floor)."""
    dev = torch.device("cuda") if device is None else device
    _check(_c["dl_empty_launches"](torch.cuda.current_stream(dev).cuda_stream, n))


def _check(status: int):
    if status != 0:
        raise DenseError(status, _c["dense_last_error"]().decode())


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DL_F32
    if t.dtype == torch.bfloat16:
        return DL_BF16
    if t.dtype == torch.float16:
        return DL_F16
    raise ValueError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")


def _act(act) -> int:
    return _ACTS[act] if not isinstance(act, int) else act


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- dense layer

def dense_act_fwd(X: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor] = None,
                  act=ACT_IDENTITY, Y: Optional[torch.Tensor] = None,
                  Z: Optional[torch.Tensor] = None, save_z: bool = False):
    """Y = act(X W^T + b); returns (Y, Z or None)."""
    _dev(X, "X")
    dt = X.dtype
    B, n_in = X.shape
    n_out = W.shape[0]
    _dev(W, "W", dt, (n_out, n_in))
    if b is not None:
        _dev(b, "b", torch.float32, (n_out,))
    if Y is None:
        Y = torch.empty((B, n_out), dtype=dt, device=X.device)
    _dev(Y, "Y", dt, (B, n_out))
    if Z is None and save_z:
        Z = torch.empty((B, n_out), dtype=dt, device=X.device)
    if Z is not None:
        _dev(Z, "Z", dt, (B, n_out))
    _check(_c["dense_act_fwd"](_stream(X), _dtype_code(X), _act(act), B, n_in, n_out,
                               _ptr(X), _ptr(W), _ptr(b), _ptr(Y), _ptr(Z)))
    return Y, Z


def dense_act_vjp_workspace_size(dtype: int, act, B: int, n_in: int, n_out: int) -> int:
    return int(_c["dense_act_vjp_workspace_size"](dtype, _act(act), B, n_in, n_out))


def dense_act_vjp(dY: torch.Tensor, saved: Optional[torch.Tensor], X: Optional[torch.Tensor],
                  W: torch.Tensor, act=ACT_IDENTITY, need_dx: bool = True,
                  need_dw: bool = True, dX: Optional[torch.Tensor] = None,
                  dW: Optional[torch.Tensor] = None, db: Optional[torch.Tensor] = None,
                  dx_act=ACT_IDENTITY, dx_saved: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, Wt: Optional[torch.Tensor] = None,
                  dy_scale: Optional[torch.Tensor] = None):
    """G = dY * act'(saved); returns (dX or None, dW or None, db or None).

    With dx_act != identity the returned dX is dX * dx_act'(dx_saved).  Wt,
    when given, is W transposed ([in, out]); dX then reads it instead of W.
    dy_scale (device float32 [1]): dY holds the cotangent times that scale
    (see dense_cast_f16_scaled); dW and db are divided by it, dX keeps it."""
    _dev(dY, "dY")
    dt = dY.dtype
    B, n_out = dY.shape
    n_in = W.shape[1]
    _dev(W, "W", dt, (n_out, n_in))
    if X is not None:
        _dev(X, "X", dt, (B, n_in))
    if saved is not None:
        _dev(saved, "saved", dt, (B, n_out))
    if need_dx and dX is None:
        dX = torch.empty((B, n_in), dtype=dt, device=dY.device)
    if dX is not None:
        _dev(dX, "dX", dt, (B, n_in))
    if need_dw:
        if dW is None:
            dW = torch.empty((n_out, n_in), dtype=torch.float32, device=dY.device)
        if db is None:
            db = torch.empty((n_out,), dtype=torch.float32, device=dY.device)
    if dW is not None:
        _dev(dW, "dW", torch.float32, (n_out, n_in))
    if db is not None:
        _dev(db, "db", torch.float32, (n_out,))
    if dx_saved is not None:
        _dev(dx_saved, "dx_saved", dt, (B, n_in))
    if Wt is not None:
        _dev(Wt, "Wt", dt, (n_in, n_out))
    code = _dtype_code(dY)
    need = dense_act_vjp_workspace_size(code, act, B, n_in, n_out)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dY.device)
    args = (_stream(dY), code, _act(act), B, n_in, n_out, _ptr(dY), _ptr(saved), _ptr(X), _ptr(W),
            _ptr(Wt), _ptr(dX), _ptr(dW), _ptr(db), _act(dx_act), _ptr(dx_saved), _ptr(ws),
            0 if ws is None else ws.numel())
    if dy_scale is not None:
        _dev(dy_scale, "dy_scale", torch.float32, (1,))
        _check(_c["dense_act_vjp_scaled"](*args, _ptr(dy_scale)))
    else:
        _check(_c["dense_act_vjp"](*args))
    return dX, dW, db


# ---------------------------------------------------------------- loss

def softmax_xent_workspace_size(B: int, C: int) -> int:
    return int(_c["softmax_xent_workspace_size"](B, C))


def softmax_xent_fwd_bwd(logits: torch.Tensor, labels: torch.Tensor,
                         dlogits: Optional[torch.Tensor] = None, inplace: bool = False,
                         row_loss: Optional[torch.Tensor] = None,
                         loss: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None):
    """Mean softmax cross-entropy and its gradient; returns (loss[1], dlogits)."""
    _dev(logits, "logits", torch.float32)
    B, C = logits.shape
    _dev(labels, "labels", torch.int32, (B,))
    if inplace:
        dlogits = logits
    elif dlogits is None:
        dlogits = torch.empty_like(logits)
    _dev(dlogits, "dlogits", torch.float32, (B, C))
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=logits.device)
    if row_loss is not None:
        _dev(row_loss, "row_loss", torch.float32, (B,))
    need = softmax_xent_workspace_size(B, C)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, logits.device)
    _check(_c["softmax_xent_fwd_bwd"](_stream(logits), B, C, _ptr(logits), _ptr(labels),
                                      _ptr(loss), _ptr(row_loss), _ptr(dlogits), _ptr(ws),
                                      ws.numel()))
    return loss, dlogits


def dense_xent_fwd(X: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor],
                   labels: torch.Tensor, logits: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, loss: Optional[torch.Tensor] = None,
                   row_loss: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Fused classifier head, forward: logits = X W^T + b, lse per row, mean
    softmax cross-entropy.  Returns (loss[1], logits, lse)."""
    _dev(X, "X", torch.float32)
    B, n_in = X.shape
    _dev(W, "W", torch.float32)
    C = W.shape[0]
    _dev(W, "W", torch.float32, (C, n_in))
    if b is not None:
        _dev(b, "b", torch.float32, (C,))
    _dev(labels, "labels", torch.int32, (B,))
    if logits is None:
        logits = torch.empty(B, C, dtype=torch.float32, device=X.device)
    if lse is None:
        lse = torch.empty(B, dtype=torch.float32, device=X.device)
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=X.device)
    _dev(logits, "logits", torch.float32, (B, C))
    _dev(lse, "lse", torch.float32, (B,))
    if row_loss is not None:
        _dev(row_loss, "row_loss", torch.float32, (B,))
    need = _c["dense_xent_fwd_workspace_size"](B, n_in, C)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, X.device)
    _check(_c["dense_xent_fwd"](_stream(X), B, n_in, C, _ptr(X), _ptr(W), _ptr(b), _ptr(labels),
                                _ptr(logits), _ptr(lse), _ptr(loss), _ptr(row_loss), _ptr(ws),
                                0 if ws is None else ws.numel()))
    return loss, logits, lse


def dense_xent_vjp(logits: torch.Tensor, lse: torch.Tensor, labels: torch.Tensor,
                   X: Optional[torch.Tensor], W: Optional[torch.Tensor],
                   dX: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None,
                   db: Optional[torch.Tensor] = None, need_dx: bool = True,
                   need_dw: bool = True, ws: Optional[torch.Tensor] = None):
    """Fused classifier head, backward from the forward's logits and lse:
    returns (dX, dW, db) (None where not requested)."""
    _dev(logits, "logits", torch.float32)
    B, C = logits.shape
    _dev(lse, "lse", torch.float32, (B,))
    _dev(labels, "labels", torch.int32, (B,))
    n_in = (X if X is not None else W).shape[1]
    if need_dx:
        _dev(W, "W", torch.float32, (C, n_in))
        if dX is None:
            dX = torch.empty(B, n_in, dtype=torch.float32, device=logits.device)
        _dev(dX, "dX", torch.float32, (B, n_in))
    if need_dw:
        _dev(X, "X", torch.float32, (B, n_in))
        if dW is None:
            dW = torch.empty(C, n_in, dtype=torch.float32, device=logits.device)
        if db is None:
            db = torch.empty(C, dtype=torch.float32, device=logits.device)
        _dev(dW, "dW", torch.float32, (C, n_in))
        _dev(db, "db", torch.float32, (C,))
    need = _c["dense_xent_vjp_workspace_size"](B, n_in, C)
    if need > 0 and (ws is None or ws.numel() < need):
        ws = _workspace(need, logits.device)
    _check(_c["dense_xent_vjp"](_stream(logits), B, n_in, C, _ptr(logits), _ptr(lse),
                                _ptr(labels), _ptr(X), _ptr(W),
                                _ptr(dX) if need_dx else None, _ptr(dW) if need_dw else None,
                                _ptr(db) if need_dw else None, _ptr(ws),
                                0 if ws is None else ws.numel()))
    return (dX if need_dx else None), (dW if need_dw else None), (db if need_dw else None)


XENT_NOALLOC_MAX_ROWS = 1 << 20


def softmax_xent_fwd_bwd_noalloc(logits: torch.Tensor, labels: torch.Tensor,
                                 dlogits: torch.Tensor, loss: torch.Tensor,
                                 row_loss: Optional[torch.Tensor] = None):
    """softmax_xent_fwd_bwd into caller-provided outputs, with no workspace:
    the library's own per-device scratch holds the per-row losses (at most
    XENT_NOALLOC_MAX_ROWS rows unless row_loss is given).  Allocates
    nothing; calls overlapping in time on one GPU race on the scratch."""
    _dev(logits, "logits", torch.float32)
    B, C = logits.shape
    _dev(labels, "labels", torch.int32, (B,))
    _dev(dlogits, "dlogits", torch.float32, (B, C))
    _dev(loss, "loss", torch.float32, (1,))
    if row_loss is not None:
        _dev(row_loss, "row_loss", torch.float32, (B,))
    _check(_c["softmax_xent_fwd_bwd_noalloc"](_stream(logits), B, C, _ptr(logits),
                                              _ptr(labels), _ptr(loss), _ptr(row_loss),
                                              _ptr(dlogits)))
    return loss, dlogits


# ---------------------------------------------------------------- optimizers

def sgd_step(w: torch.Tensor, g: torch.Tensor, lr: float):
    _dev(w, "w", torch.float32)
    _dev(g, "g", torch.float32, tuple(w.shape))
    _check(_c["sgd_step"](_stream(w), w.numel(), _ptr(w), _ptr(g), lr))
    return w


def adamw_step(w, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, step: int):
    for t, n in ((w, "w"), (g, "g"), (m, "m"), (v, "v")):
        _dev(t, n, torch.float32, tuple(w.shape))
    _check(_c["adamw_step"](_stream(w), w.numel(), _ptr(w), _ptr(g), _ptr(m), _ptr(v), lr,
                            beta1, beta2, eps, weight_decay, step))
    return w


def adam_step(w, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
              weight_decay: float, step: int):
    """Adam with coupled (L2) weight decay, in place on w, m, v."""
    for t, n in ((w, "w"), (g, "g"), (m, "m"), (v, "v")):
        _dev(t, n, torch.float32, tuple(w.shape))
    _check(_c["adam_step"](_stream(w), w.numel(), _ptr(w), _ptr(g), _ptr(m), _ptr(v), lr,
                           beta1, beta2, eps, weight_decay, step))
    return w


def ema_update(ema: torch.Tensor, w: torch.Tensor, decay: float):
    """ema <- decay ema + (1 - decay) w, in place."""
    _dev(ema, "ema", torch.float32)
    _dev(w, "w", torch.float32, tuple(ema.shape))
    _check(_c["ema_update"](_stream(w), w.numel(), _ptr(ema), _ptr(w), decay))
    return ema


def clip_grad_norm(grads: Sequence[torch.Tensor], max_norm: float,
                   total_norm: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Scale the gradients in place so their global 2-norm is at most max_norm;
    returns the device norm (before clipping)."""
    grads = list(grads)
    for k, g in enumerate(grads):
        _dev(g, f"grads[{k}]", torch.float32)
    dev = grads[0].device
    if total_norm is None:
        total_norm = torch.empty(1, dtype=torch.float32, device=dev)
    ptrs = (_vp * len(grads))(*[_ptr(g) for g in grads])
    ns = (_i64 * len(grads))(*[g.numel() for g in grads])
    need = int(_c["clip_grad_norm_workspace_size"](len(grads), ns))
    ws = _workspace(need, dev)
    _check(_c["clip_grad_norm"](_stream(grads[0]), len(grads), ptrs, ns, max_norm,
                                _ptr(total_norm), _ptr(ws), 0 if ws is None else ws.numel()))
    return total_norm


class Schedule:
    """Learning-rate schedule over optimizer steps t >= 1 (see dl_lr_schedule_t)."""

    def __init__(self, kind: int = LR_CONSTANT, warmup: int = 0, total: int = 1,
                 min_lr: float = 0.0, step_size: int = 1, gamma: float = 1.0):
        self.c = DLLrSchedule(kind, warmup, total, step_size, min_lr, gamma)

    def lr_at(self, lr: float, step: int) -> float:
        return float(_c["dl_lr_at"](ctypes.byref(self.c), lr, step))


class LossScaler:
    """Dynamic loss scale held in device memory (scale, growth tracker and the
    last step's found_inf flag), updated by the optimizer on the device."""

    def __init__(self, device, init_scale: float = 65536.0, growth_factor: float = 2.0,
                 backoff_factor: float = 0.5, growth_interval: int = 2000):
        self.scale = torch.full((1,), init_scale, dtype=torch.float32, device=device)
        self.growth_tracker = torch.zeros(1, dtype=torch.int32, device=device)
        self.found_inf = torch.zeros(1, dtype=torch.int32, device=device)
        self.c = DLLossScaler(_ptr(self.scale), _ptr(self.growth_tracker), _ptr(self.found_inf),
                              growth_factor, backoff_factor, growth_interval)


def _opt_struct(kind, lr, beta1, beta2, eps, weight_decay, step, step_dev, max_grad_norm,
                ema_decay, schedule, scaler, grad_norm) -> DLOpt:
    o = DLOpt(kind, lr, beta1, beta2, eps, weight_decay, step, _ptr(step_dev), max_grad_norm,
              ema_decay)
    if schedule is not None:
        o.schedule = ctypes.pointer(schedule.c)
    if scaler is not None:
        o.scaler = ctypes.pointer(scaler.c)
    o.grad_norm = _ptr(grad_norm)
    return o


class Param:
    """One array for optimizer_step: value w, gradient g, Adam moments m and v,
    and optionally its average and a bf16 copy of the updated value."""

    def __init__(self, w, g, m=None, v=None, ema=None, w_bf16=None):
        _dev(w, "w", torch.float32)
        for t, n in ((g, "g"), (m, "m"), (v, "v"), (ema, "ema")):
            if t is not None:
                _dev(t, n, torch.float32, tuple(w.shape))
        if w_bf16 is not None:
            _dev(w_bf16, "w_bf16", torch.bfloat16, tuple(w.shape))
        self.w, self.g, self.m, self.v, self.ema, self.w_bf16 = w, g, m, v, ema, w_bf16

    def struct(self) -> DLParam:
        return DLParam(self.w.numel(), _ptr(self.w), _ptr(self.g), _ptr(self.m), _ptr(self.v),
                       _ptr(self.ema), _ptr(self.w_bf16))


def optimizer_step(params: Sequence[Param], kind: int = OPT_ADAMW, lr: float = 1e-3,
                   beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                   weight_decay: float = 0.0, step: int = 1, step_dev=None,
                   max_grad_norm: float = 0.0, ema_decay: float = 0.0, schedule=None,
                   scaler=None, grad_norm=None, ws=None):
    """One fused multi-array update (see optimizer_step in the C header)."""
    params = list(params)
    table = (DLParam * len(params))(*[p.struct() for p in params])
    opt = _opt_struct(kind, lr, beta1, beta2, eps, weight_decay, step, step_dev, max_grad_norm,
                      ema_decay, schedule, scaler, grad_norm)
    dev = params[0].w.device
    if ws is None:
        need = int(_c["optimizer_step_workspace_size"](len(params), table))
        ws = _workspace(need, dev)
    _check(_c["optimizer_step"](_stream(params[0].w), ctypes.byref(opt), len(params), table,
                                _ptr(ws), 0 if ws is None else ws.numel()))


def optimizer_step_workspace_size(params: Sequence[Param]) -> int:
    params = list(params)
    table = (DLParam * len(params))(*[p.struct() for p in params])
    return int(_c["optimizer_step_workspace_size"](len(params), table))


def mse_loss_workspace_size(B: int, C: int) -> int:
    return int(_c["mse_loss_workspace_size"](B, C))


def mse_loss_fwd_bwd(pred: torch.Tensor, target: torch.Tensor,
                     dpred: Optional[torch.Tensor] = None, loss: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, in_place: bool = False):
    """Mean squared error over all elements and its gradient; returns (loss, dpred)."""
    _dev(pred, "pred", torch.float32)
    if pred.dim() != 2:
        raise ValueError("pred must be [B, C]")
    B, C = pred.shape
    _dev(target, "target", torch.float32, (B, C))
    if in_place:
        dpred = pred
    elif dpred is None:
        dpred = torch.empty_like(pred)
    _dev(dpred, "dpred", torch.float32, (B, C))
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=pred.device)
    if ws is None:
        ws = _workspace(mse_loss_workspace_size(B, C), pred.device)
    _check(_c["mse_loss_fwd_bwd"](_stream(pred), B, C, _ptr(pred), _ptr(target), _ptr(loss),
                                  _ptr(dpred), _ptr(ws), 0 if ws is None else ws.numel()))
    return loss, dpred


def _cast_t(name, tdt, src, dst, dst_t, copy, transposed):
    _dev(src, "src", torch.float32)
    rows, cols = src.shape
    if copy and dst is None:
        dst = torch.empty((rows, cols), dtype=tdt, device=src.device)
    if transposed and dst_t is None:
        dst_t = torch.empty((cols, rows), dtype=tdt, device=src.device)
    if dst is not None:
        _dev(dst, "dst", tdt, (rows, cols))
    if dst_t is not None:
        _dev(dst_t, "dst_t", tdt, (cols, rows))
    _check(_c[name](_stream(src), rows, cols, _ptr(src), _ptr(dst), _ptr(dst_t)))
    return dst, dst_t


def _cast(name, tdt, src, dst):
    _dev(src, "src", torch.float32)
    if dst is None:
        dst = torch.empty(src.shape, dtype=tdt, device=src.device)
    _dev(dst, "dst", tdt, tuple(src.shape))
    _check(_c[name](_stream(src), src.numel(), _ptr(src), _ptr(dst)))
    return dst


def dense_cast_bf16_t(src: torch.Tensor, dst: Optional[torch.Tensor] = None,
                      dst_t: Optional[torch.Tensor] = None, copy: bool = True,
                      transposed: bool = True):
    """bf16 copy of a [rows, cols] matrix and/or its transpose; returns (dst, dst_t)."""
    return _cast_t("dense_cast_bf16_t", torch.bfloat16, src, dst, dst_t, copy, transposed)


def dense_cast_bf16(src: torch.Tensor, dst: Optional[torch.Tensor] = None):
    return _cast("dense_cast_bf16", torch.bfloat16, src, dst)


def dense_cast_f16_t(src: torch.Tensor, dst: Optional[torch.Tensor] = None,
                     dst_t: Optional[torch.Tensor] = None, copy: bool = True,
                     transposed: bool = True):
    """Half copy (clamped to +-65504) of a [rows, cols] matrix and/or its
    transpose; returns (dst, dst_t)."""
    return _cast_t("dense_cast_f16_t", torch.float16, src, dst, dst_t, copy, transposed)


def dense_cast_f16(src: torch.Tensor, dst: Optional[torch.Tensor] = None):
    return _cast("dense_cast_f16", torch.float16, src, dst)


def dense_cast_f16_scaled(src: torch.Tensor, dst: Optional[torch.Tensor] = None,
                          scale: Optional[torch.Tensor] = None):
    """Half copy of a gradient operand times a power-of-two scale chosen from
    its largest finite magnitude; returns (dst, scale) with scale a device
    float32 [1] (pass it as dense_act_vjp's dy_scale)."""
    _dev(src, "src", torch.float32)
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.float16, device=src.device)
    _dev(dst, "dst", torch.float16, tuple(src.shape))
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=src.device)
    n = src.numel()
    ws = _workspace(int(_c["dense_cast_f16_scaled_workspace_size"](n)), src.device)
    _check(_c["dense_cast_f16_scaled"](_stream(src), n, _ptr(src), _ptr(dst), _ptr(scale),
                                       _ptr(ws), 0 if ws is None else ws.numel()))
    return dst, scale


# ---------------------------------------------------------------- MLP step

class MLP:
    """Parameters, gradients and optimizer moments of an MLP on one device,
    plus the ctypes layer table and workspace that mlp_train_step needs.
    The tensors are ordinary torch tensors the caller may read or replace
    in place; the table holds their pointers."""

    def __init__(self, Ws: Sequence[torch.Tensor], bs: Sequence[torch.Tensor],
                 acts: Sequence[int], batch: int, adamw: bool, ema: bool = False):
        self.L = len(Ws)
        dev = Ws[0].device
        self.W = [_dev(w, f"W{l}", torch.float32).contiguous() for l, w in enumerate(Ws)]
        self.b = [_dev(x, f"b{l}", torch.float32).contiguous() for l, x in enumerate(bs)]
        self.dW = [torch.zeros_like(w) for w in self.W]
        self.db = [torch.zeros_like(x) for x in self.b]
        if adamw:
            self.mW = [torch.zeros_like(w) for w in self.W]
            self.vW = [torch.zeros_like(w) for w in self.W]
            self.mb = [torch.zeros_like(x) for x in self.b]
            self.vb = [torch.zeros_like(x) for x in self.b]
        else:
            self.mW = self.vW = self.mb = self.vb = [None] * self.L
        # parameter averages, starting from the initial parameters
        if ema:
            self.eW = [w.clone() for w in self.W]
            self.eb = [x.clone() for x in self.b]
        else:
            self.eW = self.eb = [None] * self.L
        self.acts = [_act(a) for a in acts]
        self.batch = batch
        self.table = (DLLayer * self.L)()
        for l in range(self.L):
            out, n_in = self.W[l].shape
            self.table[l] = DLLayer(n_in, out, self.acts[l], _ptr(self.W[l]), _ptr(self.b[l]),
                                    _ptr(self.dW[l]), _ptr(self.db[l]), _ptr(self.mW[l]),
                                    _ptr(self.vW[l]), _ptr(self.mb[l]), _ptr(self.vb[l]),
                                    _ptr(self.eW[l]), _ptr(self.eb[l]))
        need = mlp_train_step_workspace_size(batch, self.table)
        self.ws = _workspace(need, dev)
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.step_count = 0
        # steps taken, on the device (AdamW with device_step=True)
        self.step_dev = torch.zeros(1, dtype=torch.int64, device=dev)


def mlp_train_step_workspace_size(B: int, table) -> int:
    return int(_c["mlp_train_step_workspace_size"](B, len(table), table))


def mlp_train_step(mlp: MLP, X: torch.Tensor, labels: torch.Tensor, kind: int = OPT_SGD,
                   lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
                   eps: float = 1e-8, weight_decay: float = 0.0,
                   step: Optional[int] = None, device_step: bool = False,
                   max_grad_norm: float = 0.0, ema_decay: float = 0.0, schedule=None,
                   scaler=None, grad_norm: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One forward / softmax-xent / backward / optimizer step; returns the
    device loss tensor (computed before the update).  With device_step the
    step count lives in mlp.step_dev and advances on the device (the form a
    captured graph can replay, and the one a loss scaler needs, since a
    skipped step does not count)."""
    _dev(X, "X", torch.float32, (mlp.batch, mlp.W[0].shape[1]))
    _dev(labels, "labels", torch.int32, (mlp.batch,))
    if step is None:
        step = mlp.step_count + 1
    mlp.step_count = step
    opt = _opt_struct(kind, lr, beta1, beta2, eps, weight_decay, step,
                      mlp.step_dev if device_step else None, max_grad_norm, ema_decay, schedule,
                      scaler, grad_norm)
    _check(_c["mlp_train_step"](_stream(X), mlp.batch, mlp.L, mlp.table, _ptr(X),
                                _ptr(labels), ctypes.byref(opt), _ptr(mlp.loss), _ptr(mlp.ws),
                                0 if mlp.ws is None else mlp.ws.numel()))
    return mlp.loss


def mlp_train_step_mse(mlp: MLP, X: torch.Tensor, targets: torch.Tensor, kind: int = OPT_SGD,
                       lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
                       eps: float = 1e-8, weight_decay: float = 0.0,
                       step: Optional[int] = None, device_step: bool = False,
                       max_grad_norm: float = 0.0, ema_decay: float = 0.0, schedule=None,
                       scaler=None, grad_norm: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mlp_train_step with the mean squared error against float32 targets
    [B, C] as the loss."""
    _dev(X, "X", torch.float32, (mlp.batch, mlp.W[0].shape[1]))
    _dev(targets, "targets", torch.float32, (mlp.batch, mlp.W[-1].shape[0]))
    if step is None:
        step = mlp.step_count + 1
    mlp.step_count = step
    opt = _opt_struct(kind, lr, beta1, beta2, eps, weight_decay, step,
                      mlp.step_dev if device_step else None, max_grad_norm, ema_decay, schedule,
                      scaler, grad_norm)
    _check(_c["mlp_train_step_mse"](_stream(X), mlp.batch, mlp.L, mlp.table, _ptr(X),
                                    _ptr(targets), ctypes.byref(opt), _ptr(mlp.loss),
                                    _ptr(mlp.ws), 0 if mlp.ws is None else mlp.ws.numel()))
    return mlp.loss


class StepGraph:
    """One whole training step captured as a stream graph and replayed: the
    launches of mlp_train_step are recorded once (on a side stream, as torch
    requires) and replay() issues them again with one call.  X and labels are
    the tensors the graph reads, so new data goes in by copying into them.
    Adam, AdamW, schedules and loss scaling run with the device step count,
    so every replay is the next step.
    The library allocates nothing and records no memory fills, so the graph
    holds only its kernels."""

    def __init__(self, mlp: MLP, X: torch.Tensor, labels: torch.Tensor, kind: int = OPT_SGD,
                 **opt):
        self.mlp, self.X, self.labels = mlp, X, labels
        self.kind, self.opt = kind, opt
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=X.device)
        side.wait_stream(torch.cuda.current_stream(X.device))
        with torch.cuda.stream(side):
            with torch.cuda.graph(self.graph, stream=side):
                dev = kind != OPT_SGD or opt.get("schedule") is not None or \
                    opt.get("scaler") is not None
                mlp_train_step(mlp, X, labels, kind, device_step=dev, **opt)
        torch.cuda.current_stream(X.device).wait_stream(side)

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        return self.mlp.loss

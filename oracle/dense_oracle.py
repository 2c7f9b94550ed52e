"""Float64 CPU oracle for the fused dense layer training path.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the bench's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

Every function computes in float64 with plain NumPy.  ``np.matmul`` is the
one library primitive used (as the matrix product of a definition); there is
no blocking, fusion or reordering beyond what each definition states.  Values
that cross a call boundary are rounded to their contract dtype by the caller
(``round_f32`` / ``round_bf16``); inside a call everything stays float64.

Notation follows the pages: X is [B, in] (rows are samples), W is [out, in]
(the PyTorch-style ``Linear(in, out)`` layout of the MuNet page, "Python
training", and the Orthon page, "Quick start"), b is [out], Z = X W^T + b is
the pre-activation, Y = act(Z), G = dY * act'(Z).

Readings of passages the pages leave open (each listed in the design notes):
* ReLU'(0) = 0, so the mask is Z > 0 strictly.
* GELU is the tanh form with constants sqrt(2/pi) and 0.044715.
* The cross-entropy loss is the mean over the batch, labels are int32 indices.
* AdamW is decoupled decay applied before the moment update, bias-corrected,
  eps = 1e-8, one parameter group (biases decayed too), t counts from 1.
* SGD is plain: no momentum, no decay.
* Adam takes coupled (L2) decay: g + wd w enters both moments.
* Gradient clipping scales every gradient of the step by
  min(1, max_norm / (||g||_2 + 1e-6)), the norm taken over all arrays at once
  (of the unscaled gradients when a loss scale is in use).
* EMA: e <- d e + (1 - d) w after each applied update.
* LR schedules count scheduler steps k = t - 1 from 0 (see ``lr_at``).
* MSE is the mean over all B*C elements of (p - t)^2.
* Dynamic loss scaling: the loss (hence every gradient) is multiplied by S; a
  step whose scaled gradients hold a NaN or Inf is skipped and S is
  multiplied by the backoff factor; after `interval` applied steps in a row S
  is multiplied by the growth factor.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

ACT_IDENTITY = 0
ACT_RELU = 1
ACT_GELU_TANH = 2

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
_GELU_CUBIC = 0.044715


# ---------------------------------------------------------------------------
# Rounding to the contract dtypes
# ---------------------------------------------------------------------------

def round_f32(a) -> np.ndarray:
    """Round to float32 (IEEE round-to-nearest-even), returned as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round to bfloat16, nearest value with ties to even, NaN kept.

    The low-precision convention of the MuNet page ("Configuration", the
    precision setting).  bf16 is the top 16
    bits of an IEEE float32; the value is first rounded to float32, then the
    low half is rounded away with ties going to the even upper half.
    Returned as float64 holding bf16-representable values.
    """
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lower = u & 0xFFFF
    upper = u >> 16
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    upper = upper + round_up.astype(np.uint64)
    out = (upper << 16).astype(np.uint32).view(np.float32)
    out = np.where(nan, f, out)
    return out.astype(np.float64)


F16_MAX = 65504.0


def round_f16_sat(a) -> np.ndarray:
    """Round to IEEE half precision, nearest value with ties to even,
    clamped to +-65504, NaN kept.

    The half input convention of the MuNet page ("Configuration", the mixed
    precision setting).  The value is first rounded to float32 (as the float32
    accumulator holds it), then to half by NumPy's round-half-to-even cast;
    a result that overflowed to +-inf (a finite value at or past the
    rounding threshold, or an infinite input) becomes +-65504.  Returned as
    float64 holding half-representable values.
    """
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    with np.errstate(over="ignore"):
        h = f.astype(np.float16).astype(np.float64)
    return np.where(np.isinf(h), np.copysign(F16_MAX, h), h)


def f16_safe_scale(a) -> float:
    """Power-of-two scale of a gradient operand before half conversion (the
    MuNet page, "Configuration", precision mixed_safe: each half gradient
    operand is scaled by a power of two, which is exact, so that very small
    cotangents survive the conversion with their relative accuracy).  With m the largest finite |a|: s = 2^(14 - floor(log2 m)),
    which puts m * s in [2^14, 2^15) (one binade below the half maximum);
    s = 1 when m is 0 or there is no finite value."""
    a = np.asarray(a, dtype=np.float64)
    fin = np.abs(a[np.isfinite(a)])
    m = float(fin.max()) if fin.size else 0.0
    if m == 0.0:
        return 1.0
    e = math.floor(math.log2(m))
    # log2 of a value just below a power of two can round up to it
    if 2.0 ** e > m:
        e -= 1
    elif 2.0 ** (e + 1) <= m:
        e += 1
    return 2.0 ** (14 - e)


# ---------------------------------------------------------------------------
# Activations (noeira.nn docs, "The design in one page": LinearAct fuses
# MatMul + Bias + Activation; the derivative is the act' of the vjp)
# ---------------------------------------------------------------------------

def _gelu_tanh_inner(z: np.ndarray) -> np.ndarray:
    return np.tanh(_SQRT_2_OVER_PI * (z + _GELU_CUBIC * z * z * z))


def act_fwd(z: np.ndarray, act: int) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    if act == ACT_IDENTITY:
        return z.copy()
    if act == ACT_RELU:
        return np.where(z > 0.0, z, 0.0)
    if act == ACT_GELU_TANH:
        return 0.5 * z * (1.0 + _gelu_tanh_inner(z))
    raise ValueError(f"unknown activation {act}")


def act_grad(z: np.ndarray, act: int) -> np.ndarray:
    """d act / d z evaluated at the pre-activation z."""
    z = np.asarray(z, dtype=np.float64)
    if act == ACT_IDENTITY:
        return np.ones_like(z)
    if act == ACT_RELU:
        return np.where(z > 0.0, 1.0, 0.0)
    if act == ACT_GELU_TANH:
        t = _gelu_tanh_inner(z)
        du = _SQRT_2_OVER_PI * (1.0 + 3.0 * _GELU_CUBIC * z * z)
        return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * du
    raise ValueError(f"unknown activation {act}")


# ---------------------------------------------------------------------------
# Dense layer forward and vector-Jacobian product
# ---------------------------------------------------------------------------

def dense_act_fwd(X, W, b, act: int) -> Tuple[np.ndarray, np.ndarray]:
    """Forward of LinearAct: Z = X W^T + b, Y = act(Z).

    noeira.nn docs, "The design in one page" (each module implements forward;
    LinearAct is MatMul+Bias+Activation in one kernel).  Returns (Y, Z) in
    float64.  ``b`` may be None (no bias).
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    Z = X @ W.T
    if b is not None:
        Z = Z + np.asarray(b, dtype=np.float64)[None, :]
    return act_fwd(Z, act), Z


def dense_act_vjp(dY, Zsaved, X, W, act: int, need_dx: bool = True,
                  mask: Optional[np.ndarray] = None):
    """Vector-Jacobian product of LinearAct.

    noeira.nn docs, "The design in one page" (each module implements vjp; the
    backward pass is the composition of the modules' vjps).  With
    G = dY * act'(Z):  dX = G W,  dW = G^T X,  db = sum over rows of G.

    ``mask`` (optional) replaces act'(Z) entirely; it is how a caller adopts
    the other side's ReLU decision for pre-activations within rounding of 0
    (see ``rounding_bands.relu_kink_band``).  Returns (dX or None, dW, db) in float64.
    """
    dY = np.asarray(dY, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    d = act_grad(Zsaved, act) if mask is None else np.asarray(mask, np.float64)
    G = dY * d
    dX = G @ W if need_dx else None
    dW = G.T @ X
    db = G.sum(axis=0)
    return dX, dW, db


# ---------------------------------------------------------------------------
# Softmax cross-entropy, forward and backward
# ---------------------------------------------------------------------------

def softmax_xent_fwd_bwd(logits, labels, batch_total: Optional[int] = None
                         ) -> Tuple[float, np.ndarray, np.ndarray]:
    """Mean softmax cross-entropy over the batch and its gradient.

    Orthon page, "Selected Orthon vs. PyTorch results" (one fused kernel reads
    the logits once for the forward and backward of cross entropy); netcl page,
    "The Training Step Lifecycle" (cross_entropy(logits, y) closes the step).
    Per row i with label y_i:  m = max_j z_ij,  s = sum_j exp(z_ij - m),
    lse = m + ln s,  l_i = lse - z_{i,y_i},  p_ij = exp(z_ij - m)/s,
    dz_ij = (p_ij - [j == y_i]) / B,  loss = (1/B) sum_i l_i.
    B is the number of rows, or ``batch_total`` when these rows are a block
    of a larger batch (rows are independent, so a batch may be taken in
    blocks of rows with the divisor of the whole batch).
    Returns (loss, dlogits, per-row loss) in float64.
    """
    z = np.asarray(logits, dtype=np.float64)
    y = np.asarray(labels)
    B, C = z.shape
    if y.shape != (B,):
        raise ValueError("labels must be [B]")
    if np.any(y < 0) or np.any(y >= C):
        raise ValueError("label out of range")
    n = B if batch_total is None else int(batch_total)
    if n < B:
        raise ValueError("batch_total is smaller than the block")
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    rows = np.arange(B)
    row_loss = lse - z[rows, y]
    p = e / s
    onehot = np.zeros_like(p)
    onehot[rows, y] = 1.0
    dz = (p - onehot) / n
    return float(row_loss.sum() / n), dz, row_loss


def softmax_lse(logits) -> np.ndarray:
    """Per-row log-sum-exp, lse_i = m_i + ln sum_j exp(z_ij - m_i) with
    m_i = max_j z_ij (the same row statistics as softmax_xent_fwd_bwd; a
    fused head keeps lse so that its backward can form softmax(z) =
    exp(z - lse) from the logits again)."""
    z = np.asarray(logits, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]


# ---------------------------------------------------------------------------
# Optimizers (MuNet page, "What runs today": SGD and AdamW; noeira.nn docs,
# "The design in one page": a Param owns val, grd and Adam's m and v, the
# moments starting at zero on the first stateful step)
# ---------------------------------------------------------------------------

def sgd_step(w, g, lr: float) -> np.ndarray:
    """w <- w - lr * g (plain SGD, no momentum or decay)."""
    return np.asarray(w, np.float64) - lr * np.asarray(g, np.float64)


def adamw_step(w, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, t: int):
    """One decoupled-weight-decay Adam step (t >= 1).

    w <- w (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
    m_hat = m / (1 - b1^t);  v_hat = v / (1 - b2^t);
    w <- w - lr m_hat / (sqrt(v_hat) + eps).
    Returns (w, m, v) in float64.
    """
    if t < 1:
        raise ValueError("AdamW step counts from 1")
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    w = w * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    w = w - lr * m_hat / (np.sqrt(v_hat) + eps)
    return w, m, v


def adam_step(w, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
              weight_decay: float, t: int):
    """One Adam step with coupled (L2) weight decay (t >= 1).

    noeira.nn docs, "Optimizers & losses" and the Orthon page, "Core
    capabilities" (Adam next to SGD and AdamW).  The decay is added to the
    gradient, so it passes through both moments:
    g' = g + wd w;  m <- b1 m + (1 - b1) g';  v <- b2 v + (1 - b2) g'^2;
    w <- w - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
    Returns (w, m, v) in float64.
    """
    if t < 1:
        raise ValueError("Adam step counts from 1")
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64) + weight_decay * w
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    return w - lr * m_hat / (np.sqrt(v_hat) + eps), m, v


CLIP_EPS = 1e-6


def global_grad_norm(grads) -> float:
    """The 2-norm of all gradient arrays taken together (MuNet page, "What
    runs today": gradient clipping; noeira.nn docs, "Optimizers & losses")."""
    total = 0.0
    for g in grads:
        g = np.asarray(g, np.float64)
        total += float(np.sum(g * g))
    return math.sqrt(total)


def clip_coef(norm: float, max_norm: float) -> float:
    """Factor applied to every gradient: min(1, max_norm / (norm + 1e-6))."""
    return min(1.0, max_norm / (norm + CLIP_EPS))


def ema_update(e, w, decay: float) -> np.ndarray:
    """Exponential moving average of the parameters (MuNet page, "What runs
    today": EMA in the compiled step): e <- decay e + (1 - decay) w."""
    return decay * np.asarray(e, np.float64) + (1.0 - decay) * np.asarray(w, np.float64)


LR_CONSTANT = 0
LR_STEP = 1
LR_WARMUP_COSINE = 2
LR_WARMUP_LINEAR = 3


def lr_at(kind: int, base_lr: float, t: int, warmup: int = 0, total: int = 1,
          min_lr: float = 0.0, step_size: int = 1, gamma: float = 1.0) -> float:
    """Learning rate of optimizer step t >= 1 (noeira.nn docs, "Optimizers &
    losses": LR schedules).  With k = t - 1 scheduler steps taken:
    constant: base;  step: base gamma^floor(k / step_size);
    warmup-cosine: base (k + 1) / warmup for k < warmup, then
      min + (base - min) (1 + cos(pi min(k - warmup, T) / T)) / 2,
      T = total - warmup;
    warmup-linear: the same warmup, then min + (base - min) (T - min(k - warmup, T)) / T.
    """
    if t < 1:
        raise ValueError("steps count from 1")
    k = t - 1
    if kind == LR_CONSTANT:
        return base_lr
    if kind == LR_STEP:
        return base_lr * gamma ** (k // step_size)
    if kind in (LR_WARMUP_COSINE, LR_WARMUP_LINEAR):
        if k < warmup:
            return base_lr * (k + 1) / warmup
        T = total - warmup
        if T <= 0:
            return min_lr
        j = min(k - warmup, T)
        if kind == LR_WARMUP_COSINE:
            return min_lr + (base_lr - min_lr) * (1.0 + math.cos(math.pi * j / T)) / 2.0
        return min_lr + (base_lr - min_lr) * (T - j) / T
    raise ValueError(f"unknown schedule {kind}")


def mse_loss_fwd_bwd(pred, target) -> Tuple[float, np.ndarray]:
    """Mean squared error and its gradient (MuNet page, "Python training":
    the step's mse_loss; noeira.nn docs, package layout: MSE among the
    losses).  loss = (1/(B C)) sum (p - t)^2,  dpred = 2 (p - t) / (B C)."""
    p = np.asarray(pred, np.float64)
    t = np.asarray(target, np.float64)
    if p.shape != t.shape:
        raise ValueError("pred and target shapes differ")
    n = p.size
    d = p - t
    return float(np.sum(d * d) / n), 2.0 * d / n


class LossScaler:
    """Dynamic loss scale (Orthon page, "Core capabilities": the scaler drops
    a step whose gradients hold Inf / NaN and lowers the scale, and raises it
    after a run of good steps).  ``update`` takes
    whether this step's scaled gradients held a NaN or Inf."""

    def __init__(self, scale: float = 65536.0, growth_factor: float = 2.0,
                 backoff_factor: float = 0.5, growth_interval: int = 2000):
        self.scale = float(scale)
        self.growth_factor = float(growth_factor)
        self.backoff_factor = float(backoff_factor)
        self.growth_interval = int(growth_interval)
        self.tracker = 0

    def update(self, found_inf: bool) -> None:
        if found_inf:
            self.scale = float(np.float32(self.scale * self.backoff_factor))
            self.tracker = 0
            return
        self.tracker += 1
        if self.tracker == self.growth_interval:
            self.scale = float(np.float32(self.scale * self.growth_factor))
            self.tracker = 0


def grad_control(scaled_grads, max_norm: float = 0.0, scale: float = 1.0):
    """What the optimizer applies to gradients handed over multiplied by the
    loss scale: (found_inf, norm of the unscaled gradients, multiplier).
    found_inf: a NaN or Inf among the scaled (stored) gradients.  The
    multiplier is coef / scale, coef = clip_coef(norm, max_norm) when
    max_norm > 0, else 1."""
    found = any(not np.all(np.isfinite(np.asarray(g, np.float64))) for g in scaled_grads)
    norm = global_grad_norm([np.asarray(g, np.float64) / scale for g in scaled_grads])
    coef = clip_coef(norm, max_norm) if max_norm > 0 else 1.0
    return found, norm, coef / scale


def optimizer_update(kind: str, w, g, m, v, opt, t: int, lr: float):
    """One element-wise update of an array by kind ("sgd", "adam", "adamw")
    with learning rate lr; returns (w, m, v) in float64 (m, v None for SGD)."""
    if kind == "sgd":
        return sgd_step(w, g, lr), None, None
    args = (lr, opt.beta1, opt.beta2, opt.eps, opt.weight_decay, t)
    if kind == "adamw":
        return adamw_step(w, g, m, v, *args)
    if kind == "adam":
        return adam_step(w, g, m, v, *args)
    raise ValueError(f"unknown optimizer {kind}")


def opt_lr(opt, t: int) -> float:
    """The optimizer's learning rate at step t: its schedule if it has one."""
    sched = getattr(opt, "schedule", None)
    if sched is None:
        return opt.lr
    return lr_at(sched.kind, opt.lr, t, sched.warmup, sched.total, sched.min_lr,
                 sched.step_size, sched.gamma)


# ---------------------------------------------------------------------------
# One MLP training step
# ---------------------------------------------------------------------------

class MLPState:
    """Parameters and optimizer state, stored in float32 between steps.
    ``eW`` / ``eb`` hold the parameters' moving averages once ``enable_ema``
    has set them to copies of the parameters."""

    def __init__(self, W: Sequence[np.ndarray], b: Sequence[np.ndarray]):
        self.W = [round_f32(w) for w in W]
        self.b = [round_f32(x) for x in b]
        self.mW = [np.zeros_like(w) for w in self.W]
        self.vW = [np.zeros_like(w) for w in self.W]
        self.mb = [np.zeros_like(x) for x in self.b]
        self.vb = [np.zeros_like(x) for x in self.b]
        self.eW = None
        self.eb = None
        self.t = 0

    def enable_ema(self) -> None:
        self.eW = [w.copy() for w in self.W]
        self.eb = [x.copy() for x in self.b]


def mlp_train_step(state: MLPState, X, labels, acts: Sequence[int], opt,
                   relu_masks: Optional[List[Optional[np.ndarray]]] = None,
                   scaler: Optional[LossScaler] = None, targets=None):
    """Forward, loss, backward and optimizer update of an MLP.

    MuNet page, "Python training" (the compiled step: zero grads, loss,
    backward, optimizer step, the loss returned as computed before the update)
    and noeira.nn docs, "A complete example" (the LinearReLU, LinearReLU,
    Linear network trained with a per-batch optimizer step).  The backward
    pass composes the layers' vjps from the last layer to the first; the first
    layer's dX is not needed.

    The loss is softmax cross-entropy against ``labels``, or, when
    ``targets`` is given (labels None), the mean squared error against them.

    ``opt`` has ``kind`` ("sgd", "adam", "adamw"), ``lr``, ``beta1``,
    ``beta2``, ``eps``, ``weight_decay`` and optionally ``max_grad_norm``
    (> 0: clip the global gradient norm), ``ema_decay`` (moving averages in
    ``state.eW`` / ``state.eb``) and ``schedule`` (see ``opt_lr``).  With a
    ``scaler`` the gradients are formed for the loss times its scale, a step
    with non-finite scaled gradients is skipped (no parameter, moment,
    average or step-count change) and the scale is updated.
    ``relu_masks[l]``, when given, replaces layer l's ReLU mask (used only to
    adopt the other side's decision inside the rounding band).  Updates
    ``state`` in place (rounded to float32) and returns a dict with the loss
    (pre-update, unscaled), the float64 gradients (times the loss scale, as
    the backward forms them), whether the step was skipped, the norm and
    multiplier applied, each layer's masked upstream gradient G (unscaled),
    its input h and pre-activation Z.
    """
    L = len(state.W)
    h = [np.asarray(X, dtype=np.float64)]
    Zs = []
    for l in range(L):
        Y, Z = dense_act_fwd(h[-1], state.W[l], state.b[l], acts[l])
        Zs.append(Z)
        h.append(Y)
    if targets is None:
        loss, dz, row_loss = softmax_xent_fwd_bwd(h[-1], labels)
    else:
        loss, dz = mse_loss_fwd_bwd(h[-1], targets)
        row_loss = None
    grads_W: List[np.ndarray] = [None] * L
    grads_b: List[np.ndarray] = [None] * L
    Gs: List[np.ndarray] = [None] * L
    dY = dz
    for l in reversed(range(L)):
        mask = None if relu_masks is None else relu_masks[l]
        dX, dW, db = dense_act_vjp(dY, Zs[l], h[l], state.W[l], acts[l],
                                   need_dx=(l > 0), mask=mask)
        grads_W[l], grads_b[l] = dW, db
        Gs[l] = dY * (act_grad(Zs[l], acts[l]) if mask is None else mask)
        dY = dX
    # gradient control: the backward ran on the scaled loss, so the stored
    # gradients are S g; the finite check looks at them in float32
    S = scaler.scale if scaler is not None else 1.0
    scaled = [round_f32(S * g) for g in grads_W + grads_b]
    max_norm = getattr(opt, "max_grad_norm", 0.0) or 0.0
    found, norm, mul = grad_control(scaled, max_norm, S) if (scaler or max_norm > 0) \
        else (False, None, 1.0)
    coef = mul * S
    result = {"loss": loss, "row_loss": row_loss,
              "dW": [S * g for g in grads_W], "db": [S * g for g in grads_b],
              "skipped": found, "norm": norm, "coef": coef,
              "G": Gs, "Z": Zs, "h": h, "dlogits": dz}
    if scaler is not None:
        scaler.update(found)
    if found:
        return result
    state.t += 1
    lr = opt_lr(opt, state.t)
    decay = getattr(opt, "ema_decay", None)
    for l in range(L):
        for name, mname, vname, ename, g in (("W", "mW", "vW", "eW", grads_W[l]),
                                            ("b", "mb", "vb", "eb", grads_b[l])):
            arrs = getattr(state, name)
            ms, vs = getattr(state, mname), getattr(state, vname)
            w, m, v = optimizer_update(opt.kind, arrs[l], coef * g, ms[l], vs[l],
                                       opt, state.t, lr)
            arrs[l] = round_f32(w)
            if m is not None:
                ms[l], vs[l] = round_f32(m), round_f32(v)
            if decay is not None:
                es = getattr(state, ename)
                es[l] = round_f32(ema_update(es[l], arrs[l], decay))
    return result

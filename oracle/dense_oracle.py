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
    """Round to bfloat16 with round-to-nearest-even, NaN preserved.

    The low-precision convention of the MuNet page ("Configuration", the
    precision setting: round to nearest, NaN preserved).  bf16 is the top 16
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
    (see ``relu_kink_band``).  Returns (dX or None, dW, db) in float64.
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


def relu_kink_band(X, W, b) -> np.ndarray:
    """Per-element rounding bound of the float32 pre-activation.

    tau_ij = gamma_K * (sum_k |x_ik w_jk| + |b_j|), gamma_K = K u/(1 - K u),
    u = 2^-24: the standard bound on a K-term float32 dot product.  Where
    |z_ij| <= tau_ij, both sides of the ReLU kink are correct results.
    """
    X = np.abs(np.asarray(X, dtype=np.float64))
    W = np.abs(np.asarray(W, dtype=np.float64))
    K = X.shape[1] + 1
    u = 2.0 ** -24
    gamma = K * u / (1.0 - K * u)
    s = X @ W.T
    if b is not None:
        s = s + np.abs(np.asarray(b, dtype=np.float64))[None, :]
    return gamma * s


# ---------------------------------------------------------------------------
# Softmax cross-entropy, forward and backward
# ---------------------------------------------------------------------------

def softmax_xent_fwd_bwd(logits, labels) -> Tuple[float, np.ndarray, np.ndarray]:
    """Mean softmax cross-entropy over the batch and its gradient.

    Orthon page, "Selected Orthon vs. PyTorch results" (one fused kernel reads
    the logits once for the forward and backward of cross entropy); netcl page,
    "The Training Step Lifecycle" (cross_entropy(logits, y) closes the step).
    Per row i with label y_i:  m = max_j z_ij,  s = sum_j exp(z_ij - m),
    lse = m + ln s,  l_i = lse - z_{i,y_i},  p_ij = exp(z_ij - m)/s,
    dz_ij = (p_ij - [j == y_i]) / B,  loss = (1/B) sum_i l_i.
    Returns (loss, dlogits, per-row loss) in float64.
    """
    z = np.asarray(logits, dtype=np.float64)
    y = np.asarray(labels)
    B, C = z.shape
    if y.shape != (B,):
        raise ValueError("labels must be [B]")
    if np.any(y < 0) or np.any(y >= C):
        raise ValueError("label out of range")
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    rows = np.arange(B)
    row_loss = lse - z[rows, y]
    p = e / s
    onehot = np.zeros_like(p)
    onehot[rows, y] = 1.0
    dz = (p - onehot) / B
    return float(row_loss.sum() / B), dz, row_loss


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


# ---------------------------------------------------------------------------
# One MLP training step
# ---------------------------------------------------------------------------

class MLPState:
    """Parameters and optimizer state, stored in float32 between steps."""

    def __init__(self, W: Sequence[np.ndarray], b: Sequence[np.ndarray]):
        self.W = [round_f32(w) for w in W]
        self.b = [round_f32(x) for x in b]
        self.mW = [np.zeros_like(w) for w in self.W]
        self.vW = [np.zeros_like(w) for w in self.W]
        self.mb = [np.zeros_like(x) for x in self.b]
        self.vb = [np.zeros_like(x) for x in self.b]
        self.t = 0


def mlp_train_step(state: MLPState, X, labels, acts: Sequence[int], opt,
                   relu_masks: Optional[List[Optional[np.ndarray]]] = None):
    """Forward, softmax-xent, backward and optimizer update of an MLP.

    MuNet page, "Python training" (the compiled step: zero grads, loss,
    backward, optimizer step, the loss returned as computed before the update)
    and noeira.nn docs, "A complete example" (the LinearReLU, LinearReLU,
    Linear network trained with a per-batch optimizer step).  The backward
    pass composes the layers' vjps from the last layer to the first; the first
    layer's dX is not needed.

    ``opt`` has ``kind`` ("sgd"/"adamw"), ``lr``, ``beta1``, ``beta2``,
    ``eps``, ``weight_decay``.  ``relu_masks[l]``, when given, replaces layer
    l's ReLU mask (used only to adopt the other side's decision inside the
    rounding band).  Updates ``state`` in place (rounded to float32) and
    returns a dict with the loss (pre-update), the float64 gradients, each
    layer's masked upstream gradient G, its input h and pre-activation Z.
    """
    L = len(state.W)
    h = [np.asarray(X, dtype=np.float64)]
    Zs = []
    for l in range(L):
        Y, Z = dense_act_fwd(h[-1], state.W[l], state.b[l], acts[l])
        Zs.append(Z)
        h.append(Y)
    loss, dz, row_loss = softmax_xent_fwd_bwd(h[-1], labels)
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
    state.t += 1
    for l in range(L):
        if opt.kind == "sgd":
            state.W[l] = round_f32(sgd_step(state.W[l], grads_W[l], opt.lr))
            state.b[l] = round_f32(sgd_step(state.b[l], grads_b[l], opt.lr))
        elif opt.kind == "adamw":
            args = (opt.lr, opt.beta1, opt.beta2, opt.eps, opt.weight_decay,
                    state.t)
            w, m, v = adamw_step(state.W[l], grads_W[l], state.mW[l],
                                 state.vW[l], *args)
            state.W[l], state.mW[l], state.vW[l] = (round_f32(w), round_f32(m),
                                                    round_f32(v))
            w, m, v = adamw_step(state.b[l], grads_b[l], state.mb[l],
                                 state.vb[l], *args)
            state.b[l], state.mb[l], state.vb[l] = (round_f32(w), round_f32(m),
                                                    round_f32(v))
        else:
            raise ValueError(f"unknown optimizer {opt.kind}")
    return {"loss": loss, "row_loss": row_loss, "dW": grads_W, "db": grads_b,
            "G": Gs, "Z": Zs, "h": h, "dlogits": dz}

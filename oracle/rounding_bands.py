"""Float32 rounding bounds: where several results are correct.

TEST INFRASTRUCTURE, part of the oracle package.  Only the tests, the package
smoke check and the bench's CPU-baseline leg may import it; the HIP library
never does, and nothing here is shared with it.

A float32 evaluation of a sum of n terms, in any order and any tree shape,
lies within gamma_n * (sum of the terms' magnitudes) of the exact sum, with
gamma_n = n u / (1 - n u) and u = 2^-24 (the standard bound for summation and
inner products: N. J. Higham, "Accuracy and Stability of Numerical
Algorithms", 2nd ed., section 3.1; a rounded product is one more rounding of
its term, so n counts products, and a bias adds one term).  Where a decision
depends on a value inside such a bound -- the ReLU mask z > 0 at a
pre-activation within rounding of zero, the AdamW update near eps -- an
implementation in float32 may land on either side and still be correct.

The functions below give those bounds elementwise, in float64, including how
a deviation of an operand (the other side's float32 copy of an earlier
layer's output or gradient) carries into the next result.  The parity tests
widen a comparison only inside them.  None of this changes what the oracle
computes; it only says how far a correct float32 result may lie from it.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

U32 = 2.0 ** -24  # unit roundoff of float32 (round to nearest)

ACT_IDENTITY = 0
ACT_RELU = 1


def gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u) for float32, n >= 0 terms."""
    if n < 0 or n * U32 >= 1.0:
        raise ValueError(f"gamma_n undefined for n = {n}")
    return n * U32 / (1.0 - n * U32)


def dot_band(X, W, b=None, dX=None) -> np.ndarray:
    """Bound on |z' - z| for z = X W^T + b.

    z is exact (float64 stands in for exact here); z' is any float32
    evaluation, in any order, of X' W^T + b where the operand X' the other
    side holds satisfies |X' - X| <= dX elementwise (dX None: X' = X).
    Each z_ij is a sum of K products and the bias, n = K + 1 terms, so
      tau_ij = gamma_{K+1} (sum_k (|x_ik| + dx_ik) |w_jk| + |b_j|)
               + sum_k dx_ik |w_jk|
    (the first part: rounding of the sum of the perturbed terms; the second:
    the exact effect of the perturbation).  W and b are the same float32
    values on both sides.
    """
    aX = np.abs(np.asarray(X, dtype=np.float64))
    aW = np.abs(np.asarray(W, dtype=np.float64))
    K = aX.shape[1]
    if dX is not None:
        aX = aX + np.asarray(dX, dtype=np.float64)
    s = aX @ aW.T
    if b is not None:
        s = s + np.abs(np.asarray(b, dtype=np.float64))[None, :]
    tau = gamma(K + 1) * s
    if dX is not None:
        tau = tau + np.asarray(dX, dtype=np.float64) @ aW.T
    return tau


def relu_kink_band(X, W, b, dX=None) -> np.ndarray:
    """The ReLU decision band: where |z| <= dot_band(X, W, b, dX), the float32
    pre-activation may have either sign, and both masks are correct."""
    return dot_band(X, W, b, dX)


def act_out_dev(z, tau, act: int) -> np.ndarray:
    """Bound on |y' - y| for y = act(z), where y' is the float32 rounding of
    act(z') and |z' - z| <= tau.  Identity and ReLU move no value by more
    than its argument moves (1-Lipschitz), and the float32 rounding of the
    result adds at most u |y'| <= u (|z| + tau):  tau + u (|z| + tau)."""
    if act not in (ACT_IDENTITY, ACT_RELU):
        raise ValueError("act_out_dev covers identity and ReLU")
    z = np.abs(np.asarray(z, dtype=np.float64))
    tau = np.asarray(tau, dtype=np.float64)
    return tau + U32 * (z + tau)


def xent_grad_band(z, tau, batch_total: int, scale: float = 1.0, labels=None,
                   form: str = "softmax") -> np.ndarray:
    """Bound on |g' - g| for the softmax cross-entropy gradient
    g = scale (softmax(z) - onehot) / batch_total per row, when g' is formed
    in float32 from logits z' with |z' - z| <= tau (elementwise).

    form "softmax" (one pass over a row held whole): the row max m'
    (exact), the exponentials e'_j = exp(z'_j - m') with the argument
    rounded twice (the difference, then its scaling to base 2: relative
    error 2u|z_j - m| in the result) and the exponential itself within 4u,
    their float32 sum s' in any order (gamma_C), p'_j = e'_j / s' (one
    rounding).
    form "lse" (a row split into column tiles, as a GEMM epilogue sees it):
    per tile t its max m_t and s_t = sum exp(z - m_t), then
    s' = sum_t s_t exp(m_t - m) (each term two exponentials and a product:
    relative error (2|z_j - m| + 9) u), lse' = m + log s' (log within 2u of
    its result, the sum rounded once), and p'_j / B formed again from the
    logits as one base-2 exponential 2^(z log2 e - (lse log2 e + log2 B))
    (the exponent offset and the exponent each rounded, the exponential
    within 4u: relative error 2u (|z_j - lse| + |lse| + ln B) + 4u).
    Either way g' is then p' minus the one-hot times 1/batch_total, itself
    rounded and times the loss scale (four roundings: gamma_4).

    With delta_j = tau_j + max_k tau_k (the shift of z_j - m, since the max
    moves by at most max_k tau_k) and rho_j the rounding just listed:
      eps_j = exp(delta_j) (1 + rho_j) - 1     (|e'_j / e_j - 1|)
      eps_s = (sum_j e_j eps_j + gamma_C sum_j e_j (1 + eps_j)) / s
    "softmax":
      dp_j = p_j ((1 + eps_j)(1 + u) / (1 - eps_s) - 1),
      and since the p'_j of a row add up to 1 within gamma_{C+2}, a
      probability moves by no more than the others in all:
      dp_j <= sum_{k != j} dp_k + gamma_{C+2} (tighter for a dominant class).
    "lse":
      Lambda = max_k tau_k - log(1 - eps_s) + 2u |log s| + u |lse|,
      dp_j = p_j (exp(tau_j + Lambda) (1 + 2u (|z_j - lse| + |lse| + ln B)
                  + 4u) - 1).
    Then |g'_j - g_j| <= (scale / B) (dp_j + gamma_4 (|p_j - onehot_j| + dp_j)).
    Without ``labels`` the bound takes |p_j - onehot_j| <= 1.  Both
    probabilities lie in [0, 1], so dp_j never exceeds 1 (plus rounding);
    a row whose logit deviation leaves the sum unbounded (eps_s >= 1) gets
    that cap for every class.
    """
    if form not in ("softmax", "lse"):
        raise ValueError(f"unknown form {form}")
    z = np.asarray(z, dtype=np.float64)
    tau = np.asarray(tau, dtype=np.float64)
    B, C = z.shape
    # A deviation beyond the exponential's range makes eps (and the sum's
    # bound) inf or, where a tiny probability meets it, NaN: such rows are
    # caught by `lost` below, so the floating-point flags are not errors.
    with np.errstate(over="ignore", invalid="ignore"):
        return _xent_grad_band(z, tau, B, C, batch_total, labels, scale, form)


def _xent_grad_band(z, tau, B, C, batch_total, labels, scale, form):
    m = z.max(axis=1, keepdims=True)
    d = z - m                                   # <= 0
    e = np.exp(d)
    s = e.sum(axis=1, keepdims=True)
    tmax = tau.max(axis=1, keepdims=True)
    # eps = exp(tau + max tau) (1 + rho) - 1, rho = (c0 - 2 d) u, built in place
    eps = tau + tmax
    np.exp(eps, out=eps)
    d *= -2.0 * U32
    d += 1.0 + (4.0 if form == "softmax" else 9.0) * U32
    eps *= d
    eps -= 1.0
    del d
    es = (e * eps).sum(axis=1, keepdims=True)
    eps_s = (es + gamma(C) * (s + es)) / s
    # rows whose logits may move so far that the sum is not bounded away
    # from zero: only |p' - p| <= 1 (+ rounding) is left there
    lost = ~(eps_s < 1.0)                       # NaN included
    eps_s = np.where(lost, 0.0, eps_s)
    p = e
    p /= s                                      # e is not needed past here
    if form == "softmax":
        dp = eps
        dp += 1.0
        dp *= (1.0 + U32) / (1.0 - eps_s)
        dp -= 1.0
        dp *= p                                 # p ((1 + eps)(1 + u) / (1 - eps_s) - 1)
        others = dp.sum(axis=1, keepdims=True) - dp
        others += gamma(C + 2)
        np.minimum(dp, others, out=dp)
        del others
    else:
        del eps
        logs = np.log(s)
        lse = m + logs
        lam = tmax - np.log1p(-eps_s) + 2.0 * U32 * np.abs(logs) + U32 * np.abs(lse)
        dp = z - lse
        np.abs(dp, out=dp)
        dp += np.abs(lse) + np.log(batch_total)
        dp *= 2.0 * U32
        dp += 1.0 + 4.0 * U32                   # 1 + 2u (|z - lse| + |lse| + ln B) + 4u
        dp *= np.exp(tau + lam)
        dp -= 1.0
        dp *= p
    cap = 1.0 + 4.0 * U32  # two probabilities in [0, 1], each rounded
    np.minimum(dp, cap, out=dp)
    dp[lost[:, 0]] = cap
    if labels is None:
        dist = np.ones_like(p)
    else:
        dist = p
        rows = np.arange(B)
        dist[rows, np.asarray(labels)] = 1.0 - dist[rows, np.asarray(labels)]
    dist += dp
    dist *= gamma(4)
    dist += dp
    dist *= abs(scale) / batch_total
    return dist


def sum_band(G, h, dG=None, dh=None, n: Optional[int] = None) -> np.ndarray:
    """Bound on |s' - s| for s = G^T h (a sum over the rows, as in
    dW = G^T X; db is the case h = ones), s' any float32 evaluation of
    G'^T h' with |G' - G| <= dG and |h' - h| <= dh elementwise:
      gamma_n (|G| + dG)^T (|h| + dh) + dG^T (|h| + dh) + |G|^T dh,
    n the number of terms of each sum: the rows of G, or ``n`` when G and h
    are one block of rows of a longer sum (the bound is then a sum over
    blocks of these terms, all taken with the whole sum's gamma_n).
    """
    aG = np.abs(np.asarray(G, dtype=np.float64))
    ah = np.abs(np.asarray(h, dtype=np.float64))
    gn = gamma(aG.shape[0] if n is None else int(n))
    if dG is None and dh is None:
        return gn * (aG.T @ ah)
    dG = np.zeros_like(aG) if dG is None else np.asarray(dG, dtype=np.float64)
    dh = np.zeros_like(ah) if dh is None else np.asarray(dh, dtype=np.float64)
    hp = ah + dh
    return (gn * aG + (1.0 + gn) * dG).T @ hp + aG.T @ dh


def mlp_forward_bands(X, Ws: Sequence[np.ndarray], bs: Sequence[np.ndarray],
                      acts: Sequence[int], masks: Optional[Sequence] = None):
    """Forward bands of an MLP chain evaluated in float32 from the same input
    X and parameters: for each layer, the band tau_l of its pre-activation
    (dot_band with the deviation of its input, which is the previous layer's
    act_out_dev) and the deviation bound dh_l of its input.  ``masks[l]``
    (optional) is the ReLU mask the comparison adopted for layer l; the
    layer outputs follow it exactly as the oracle's re-evaluation does.
    Returns (taus, dhs, hs, zs) lists in float64: hs[l] is layer l's input,
    zs[l] its pre-activation (the oracle's values)."""
    h = np.asarray(X, dtype=np.float64)
    dh = None
    taus: List[np.ndarray] = []
    dhs: List[Optional[np.ndarray]] = []
    hs: List[np.ndarray] = []
    zs: List[np.ndarray] = []
    for l in range(len(Ws)):
        W = np.asarray(Ws[l], dtype=np.float64)
        b = None if bs[l] is None else np.asarray(bs[l], dtype=np.float64)
        z = h @ W.T
        if b is not None:
            z = z + b[None, :]
        tau = dot_band(h, W, b, dh)
        taus.append(tau)
        dhs.append(dh)
        hs.append(h)
        zs.append(z)
        if acts[l] == ACT_RELU:
            mk = (z > 0.0) if masks is None or masks[l] is None else np.asarray(masks[l]) > 0
            y = np.where(mk, z, 0.0)
        elif acts[l] == ACT_IDENTITY:
            y = z
        else:
            raise ValueError("mlp_forward_bands covers identity and ReLU layers")
        dh = act_out_dev(z, tau, acts[l])
        h = y
    return taus, dhs, hs, zs


def dx_band(G, W, dG, mask=None) -> np.ndarray:
    """Bound on the deviation of a layer's input gradient dX = (G W) * mask
    (mask: the adopted 0/1 ReLU mask of the layer below, or None) when G W is
    evaluated in float32 from G' with |G' - G| <= dG: a dot_band over the K =
    out terms of each sum, then the mask (the same on both sides)."""
    aW = np.abs(np.asarray(W, dtype=np.float64))
    aG = np.abs(np.asarray(G, dtype=np.float64))
    K = aG.shape[1]
    dG = np.asarray(dG, dtype=np.float64)
    band = gamma(K) * ((aG + dG) @ aW) + dG @ aW
    if mask is not None:
        band = band * np.asarray(mask, dtype=np.float64)
    return band

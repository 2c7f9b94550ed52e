"""Pins of the float32 rounding bounds the parity tests use to decide where
several results are correct (oracle/rounding_bands.py).

Each bound is pinned from both sides, by float32 arithmetic evaluated here
and not by its own formula:
* below: no float32 evaluation order (random permutations, left to right,
  pairwise) of the perturbed operands escapes the bound;
* above: a family of inputs whose left-to-right float32 sum loses almost
  the whole bound (x = [1, u, u, ...]: every + u is a tie that rounds back
  to 1) shows the bound is within a small factor of the worst case, so a
  bound several times too wide fails.
"""
import numpy as np
import pytest

import oracle as O

U = 2.0 ** -24


def _f32_dot_orders(x, w, b, rng, n_orders=4):
    """Float32 evaluations of b + sum_k x_k w_k in several orders: left to
    right, right to left, random permutations, and pairwise."""
    x = np.asarray(x, np.float32)
    w = np.asarray(w, np.float32)
    prods = (x * w).astype(np.float32)
    outs = []
    orders = [np.arange(len(x)), np.arange(len(x))[::-1]]
    orders += [rng.permutation(len(x)) for _ in range(n_orders)]
    for idx in orders:
        acc = np.float32(b)
        for k in idx:
            acc = np.float32(acc + prods[k])
        outs.append(float(acc))
    terms = [np.float32(b)] + list(prods)
    while len(terms) > 1:  # pairwise tree
        nxt = [np.float32(terms[i] + terms[i + 1]) for i in range(0, len(terms) - 1, 2)]
        if len(terms) % 2:
            nxt.append(terms[-1])
        terms = nxt
    outs.append(float(terms[0]))
    return outs


def test_gamma_values():
    assert O.gamma(0) == 0.0
    assert O.gamma(1) == U / (1 - U)
    # n u / (1 - n u) at n = 2^10: 2^-14 / (1 - 2^-14)
    assert O.gamma(1024) == 2.0 ** -14 / (1 - 2.0 ** -14)
    with pytest.raises(ValueError):
        O.gamma(2 ** 24)


def test_dot_band_holds_for_every_float32_order():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((6, 300)).astype(np.float32)
    W = rng.standard_normal((5, 300)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    tau = O.relu_kink_band(X, W, b)
    exact = X.astype(np.float64) @ W.astype(np.float64).T + b
    for i in range(6):
        for j in range(5):
            for v in _f32_dot_orders(X[i], W[j], b[j], rng):
                assert abs(v - exact[i, j]) <= tau[i, j]


def test_dot_band_near_attained_by_ties():
    """x = [1, u, ..., u] (K terms), w = 1, b = 0: left to right, each + u is
    a tie that rounds to even (back to 1), losing (K - 1) u in all.  The
    bound must hold there and be less than 1.5 times that loss."""
    for K in (8, 16, 64):
        x = np.full(K, U, np.float32)
        x[0] = 1.0
        w = np.ones(K, np.float32)
        acc = np.float32(0.0)
        for k in range(K):
            acc = np.float32(acc + x[k] * w[k])
        exact = 1.0 + (K - 1) * U
        lost = exact - float(acc)
        assert lost == (K - 1) * U
        tau = float(O.relu_kink_band(x[None, :], w[None, :], np.zeros(1))[0, 0])
        assert lost <= tau < 1.5 * lost, (K, lost, tau)


def test_dot_band_covers_perturbed_operand():
    """An operand X' within dX of X: every float32 evaluation of X' W^T + b
    stays inside dot_band(X, W, b, dX) around the exact X W^T + b, including
    the worst case, where every deviation pushes the same way (W > 0, X' =
    X + dX)."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((4, 120))
    W = np.abs(rng.standard_normal((3, 120))).astype(np.float32)
    b = rng.standard_normal(3).astype(np.float32)
    dX = np.abs(rng.standard_normal((4, 120))) * 1e-3
    tau = O.dot_band(X, W, b, dX)
    exact = X @ W.astype(np.float64).T + b
    signs = [np.ones_like(X), -np.ones_like(X)] + [rng.choice([-1.0, 1.0], size=X.shape)
                                                   for _ in range(2)]
    for sg in signs:
        Xp = (X + dX * sg).astype(np.float32)
        for i in range(4):
            for j in range(3):
                for v in _f32_dot_orders(Xp[i], W[j], b[j], rng, 2):
                    assert abs(v - exact[i, j]) <= tau[i, j]


def test_dot_band_perturbation_term_is_tight():
    """x = [1, 1], w = [1, 1], x' = x + d (exact in float32): z' - z = 2d
    exactly; the bound holds and is within 1.01 of it (the rounding part is
    a few u on top of d = 2^-10)."""
    d = 2.0 ** -10
    x = np.ones((1, 2))
    w = np.ones((1, 2), np.float32)
    tau = float(O.dot_band(x, w, None, np.full((1, 2), d))[0, 0])
    zp = np.float32(np.float32(1 + d) + np.float32(1 + d))
    dev = float(zp) - 2.0
    assert dev == 2 * d
    assert dev <= tau < 1.01 * dev


def test_act_out_dev():
    z = np.array([-1.0, 0.0, 3.0])
    tau = np.array([1e-6, 1e-6, 1e-6])
    dev = O.act_out_dev(z, tau, O.ACT_RELU)
    # ReLU of z' with |z' - z| <= tau, then float32 rounding, stays within dev
    for zp in (z - tau, z + tau):
        yp = np.maximum(zp, 0.0).astype(np.float32).astype(np.float64)
        assert np.all(np.abs(yp - np.maximum(z, 0.0)) <= dev)
    with pytest.raises(ValueError):
        O.act_out_dev(z, tau, O.ACT_GELU_TANH)


def _f32_softmax_grad(zp, y, B, rng):
    """Float32 softmax-xent gradient of one row, summation in random order."""
    zp = np.asarray(zp, np.float32)
    m = np.float32(zp.max())
    e = np.exp((zp - m).astype(np.float32)).astype(np.float32)
    s = np.float32(0.0)
    for k in rng.permutation(len(e)):
        s = np.float32(s + e[k])
    p = (e / s).astype(np.float32)
    oh = np.zeros_like(p)
    oh[y] = 1.0
    return ((p - oh).astype(np.float32) * np.float32(1.0 / B)).astype(np.float64)


def test_xent_grad_band_holds():
    rng = np.random.default_rng(21)
    B, C = 8, 50
    z = rng.standard_normal((B, C)) * 3.0
    y = rng.integers(0, C, B)
    tau = np.abs(rng.standard_normal((B, C))) * 1e-4
    band = O.xent_grad_band(z, tau, B)
    band_y = O.xent_grad_band(z, tau, B, labels=y)
    assert np.all(band_y <= band)
    band = band_y
    _, g, _ = O.softmax_xent_fwd_bwd(z, y)
    for trial in range(4):
        zp = z + tau * rng.choice([-1.0, 1.0], size=z.shape)
        for i in range(B):
            gp = _f32_softmax_grad(zp[i], y[i], B, rng)
            assert np.all(np.abs(gp - g[i]) <= band[i])


def test_xent_grad_band_is_tight_for_a_dominant_class():
    """One dominant logit raised by tau and the rest lowered by tau moves
    its probability by about p (1 - p) 2 tau; the bound stays within 4x."""
    t = 1e-3
    z = np.array([[4.0, 0.0, 0.0, 0.0, 0.0]])
    tau = np.full_like(z, t)
    band = O.xent_grad_band(z, tau, 1, labels=np.array([1]))
    zp = z + np.array([[t, -t, -t, -t, -t]])
    e = np.exp(zp - zp.max())
    p1 = e / e.sum()
    e0 = np.exp(z - z.max())
    p0 = e0 / e0.sum()
    dev = abs(p1[0, 0] - p0[0, 0])
    assert dev <= band[0, 0] < 4.0 * dev


def test_sum_band_holds_and_is_near_attained():
    rng = np.random.default_rng(31)
    n = 200
    G = rng.standard_normal((n, 3))
    h = rng.standard_normal((n, 2))
    dG = np.abs(rng.standard_normal((n, 3))) * 1e-6
    dh = np.abs(rng.standard_normal((n, 2))) * 1e-6
    band = O.sum_band(G, h, dG, dh)
    exact = G.T @ h
    for trial in range(3):
        Gp = (G + dG * rng.choice([-1.0, 1.0], size=G.shape)).astype(np.float32)
        hp = (h + dh * rng.choice([-1.0, 1.0], size=h.shape)).astype(np.float32)
        for a in range(3):
            for c in range(2):
                for v in _f32_dot_orders(Gp[:, a], hp[:, c], 0.0, rng, 2):
                    assert abs(v - exact[a, c]) <= band[a, c]
    # the tie family: n rows, G = [1, u, ..., u], h = 1
    for n in (16, 128):
        g = np.full((n, 1), U)
        g[0] = 1.0
        acc = np.float32(0.0)
        for k in range(n):
            acc = np.float32(acc + np.float32(g[k, 0]))
        lost = 1.0 + (n - 1) * U - float(acc)
        b = float(O.sum_band(g, np.ones((n, 1)))[0, 0])
        assert lost <= b < 1.5 * lost


def test_mlp_forward_bands_cover_a_float32_chain():
    """A tiny ReLU MLP evaluated in float32 (float32 matmul, then ReLU):
    every layer's pre-activation stays inside its propagated band, and the
    band of layer 2 on is wider than the local rounding bound alone."""
    rng = np.random.default_rng(41)
    X = rng.standard_normal((64, 40)).astype(np.float32)
    Ws = [rng.standard_normal((30, 40)).astype(np.float32) * 0.3,
          rng.standard_normal((20, 30)).astype(np.float32) * 0.3,
          rng.standard_normal((5, 20)).astype(np.float32) * 0.3]
    bs = [rng.standard_normal(n).astype(np.float32) * 0.1 for n in (30, 20, 5)]
    acts = [O.ACT_RELU, O.ACT_RELU, O.ACT_IDENTITY]
    taus, dhs, hs, zs = O.mlp_forward_bands(X, Ws, bs, acts)
    h32 = X
    for l in range(3):
        z32 = (h32 @ Ws[l].T + bs[l]).astype(np.float32)
        dev = np.abs(z32.astype(np.float64) - zs[l])
        assert np.all(dev <= taus[l]), l
        if l > 0:
            local = O.dot_band(hs[l], Ws[l], bs[l])
            assert np.all(taus[l] > local)
        h32 = np.maximum(z32, 0.0) if acts[l] == O.ACT_RELU else z32


def test_dx_band_covers_float32_products():
    rng = np.random.default_rng(51)
    G = rng.standard_normal((16, 12))
    W = rng.standard_normal((12, 9)).astype(np.float32)
    dG = np.abs(rng.standard_normal(G.shape)) * 1e-6
    mask = (rng.standard_normal((16, 9)) > 0).astype(np.float64)
    band = O.dx_band(G, W, dG, mask)
    exact = (G @ W.astype(np.float64)) * mask
    for trial in range(3):
        Gp = (G + dG * rng.choice([-1.0, 1.0], size=G.shape)).astype(np.float32)
        for i in range(16):
            for k in range(9):
                for v in _f32_dot_orders(Gp[i], W[:, k], 0.0, rng, 2):
                    assert abs(v * mask[i, k] - exact[i, k]) <= band[i, k]


def test_sum_band_by_blocks_equals_whole():
    rng = np.random.default_rng(61)
    G = rng.standard_normal((300, 4))
    h = rng.standard_normal((300, 3))
    dG = np.abs(rng.standard_normal(G.shape)) * 1e-7
    whole = O.sum_band(G, h, dG)
    blocks = sum(O.sum_band(G[i:i + 100], h[i:i + 100], dG[i:i + 100], n=300)
                 for i in range(0, 300, 100))
    assert np.allclose(blocks, whole, rtol=1e-12, atol=0)


def test_xent_grad_band_saturates_for_huge_logit_deviation():
    """A logit deviation that leaves the softmax unconstrained bounds each
    probability's move by 1 (plus rounding), never more, never an error."""
    z = np.array([[0.0, 1.0, 2.0]])
    band = O.xent_grad_band(z, np.full_like(z, 5.0), 4, labels=np.array([1]))
    assert np.all(band <= (1.0 + 4 * U) * (1 + O.gamma(4)) / 4 * 1.0001 + O.gamma(4) / 4)
    assert np.all(band >= 1.0 / 4)


def test_xent_grad_band_caps_rows_whose_bound_overflows():
    """A deviation past the exponential's range, on a row where another
    class's exponential underflows (0 times inf in the sum's bound), still
    bounds every probability's move by the cap, with no NaN; rows with a
    small deviation keep their finite, smaller band."""
    z = np.array([[0.0, -800.0, 1.0], [0.0, 1.0, 2.0]])
    tau = np.array([[400.0, 400.0, 400.0], [1e-6, 1e-6, 1e-6]])
    band = O.xent_grad_band(z, tau, 4, labels=np.array([1, 0]))
    cap = (1.0 + 4 * U) * (1 + O.gamma(4)) / 4 * 1.0001 + O.gamma(4) / 4
    assert np.all(np.isfinite(band))
    assert np.all(band[0] >= 1.0 / 4) and np.all(band[0] <= cap)
    assert np.all(band[1] < 1e-5)


def _f32_lse_grad(zp, y, B, tile, rng):
    """Float32 softmax-xent gradient of one row formed as the fused head does:
    per column tile its max and sum of exp, the tiles combined in order,
    lse = m + log s, then exp(z - lse) / B from the logits as one base-2
    exponential, minus 1 / B at the label."""
    zp = np.asarray(zp, np.float32)
    C = len(zp)
    parts = []
    for t0 in range(0, C, tile):
        zt = zp[t0:t0 + tile]
        mt = np.float32(zt.max())
        st = np.float32(0.0)
        for k in rng.permutation(len(zt)):
            st = np.float32(st + np.exp(np.float32(zt[k] - mt)))
        parts.append((mt, st))
    m = np.float32(max(mt for mt, _ in parts))
    s = np.float32(0.0)
    for mt, st in parts:
        s = np.float32(s + np.float32(st * np.exp(np.float32(mt - m))))
    lse = np.float32(m + np.log(s))
    l2e = np.float32(1.4426950408889634)
    c = np.float32(lse * l2e + np.float32(np.log2(B)))
    g = np.exp2((zp * l2e - c).astype(np.float32)).astype(np.float32)  # exp(z - lse) / B
    g[y] = np.float32(g[y] - np.float32(1.0 / B))
    return g.astype(np.float64)


def test_xent_grad_band_lse_form_holds():
    rng = np.random.default_rng(23)
    B, C = 6, 300
    z = rng.standard_normal((B, C)) * 3.0
    y = rng.integers(0, C, B)
    tau = np.abs(rng.standard_normal((B, C))) * 1e-4
    band = O.xent_grad_band(z, tau, B, labels=y, form="lse")
    _, g, _ = O.softmax_xent_fwd_bwd(z, y)
    for trial in range(3):
        zp = z + tau * rng.choice([-1.0, 1.0], size=z.shape)
        for i in range(B):
            for tile in (32, 128):
                gp = _f32_lse_grad(zp[i], y[i], B, tile, rng)
                assert np.all(np.abs(gp - g[i]) <= band[i])


def test_xent_grad_band_lse_form_is_tight():
    """Lower every logit but the largest by tau and raise that one: a minor
    class's probability moves by about p (1 + p_max) tau... within 3x of the
    bound."""
    t = 1e-3
    z = np.array([[4.0, 0.0, 0.0, 0.0, 0.0]])
    tau = np.full_like(z, t)
    band = O.xent_grad_band(z, tau, 1, labels=np.array([0]), form="lse")
    zp = z + np.array([[t, -t, -t, -t, -t]])
    e = np.exp(zp - zp.max())
    p1 = e / e.sum()
    e0 = np.exp(z - z.max())
    p0 = e0 / e0.sum()
    dev = abs(p1[0, 1] - p0[0, 1])
    assert dev <= band[0, 1] < 3.0 * dev

"""Pins of the float64 oracle to things other than itself.

Each check ties an oracle function to a closed form, an invariant, a finite
difference, a brute-force loop on a tiny input, or an independent library
routine (SciPy, or PyTorch's CPU float64 ops, which share no code with the
oracle).  None of them retypes the oracle's own formula.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

ACTS = [O.ACT_IDENTITY, O.ACT_RELU, O.ACT_GELU_TANH]


def rel_norm(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(a - ref)) / (denom if denom > 0 else 1.0))


# ---------------------------------------------------------------- rounding

def test_round_bf16_hand_values():
    one = 1.0
    assert O.round_bf16(one) == 1.0
    # halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0
    # halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): goes up
    assert O.round_bf16(1.0 + 2.0 ** -7 + 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above halfway rounds up
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert O.round_bf16(-3.0) == -3.0
    assert np.isnan(O.round_bf16(np.nan))
    assert O.round_bf16(np.inf) == np.inf


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x32), ref)


def test_round_f16_sat_hand_values():
    e = 2.0 ** -24  # smallest half subnormal
    cases = [(1.0, 1.0), (65504.0, 65504.0), (65519.0, 65504.0), (65520.0, 65504.0),
             (1e9, 65504.0), (-1e9, -65504.0), (np.inf, 65504.0), (-np.inf, -65504.0),
             (e, e), (0.5 * e, 0.0), (1.5 * e, 2 * e), (2.5 * e, 2 * e),
             (1.0 + 2.0 ** -11, 1.0), (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),
             (-2.0 ** -14, -2.0 ** -14), (0.1, 0.0999755859375)]
    got = O.round_f16_sat(np.array([c[0] for c in cases]))
    for (x, want), g in zip(cases, got):
        assert g == want, (x, g, want)
    assert np.isnan(O.round_f16_sat(np.array([np.nan]))[0])


def test_round_f16_sat_matches_torch_cast_in_range():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 11, 20000))).astype(np.float32)
    x = x[np.abs(x) < 65504.0]
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(O.round_f16_sat(x), ref)


def test_f16_safe_scale_hand_values():
    assert O.f16_safe_scale(np.array([1.0, -0.5])) == 2.0 ** 14
    assert O.f16_safe_scale(np.array([3.0])) == 2.0 ** 13
    assert O.f16_safe_scale(np.array([-2.0 ** 15])) == 0.5
    assert O.f16_safe_scale(np.array([1e-7, np.nan, np.inf])) == 2.0 ** 38
    assert O.f16_safe_scale(np.zeros(5)) == 1.0
    assert O.f16_safe_scale(np.array([np.nan])) == 1.0
    # just below a power of two stays in the lower binade
    x = np.nextafter(1.0, 0.0)
    assert O.f16_safe_scale(np.array([x])) == 2.0 ** 15


def test_f16_safe_scale_places_max_in_top_binade_and_keeps_relative_accuracy():
    rng = np.random.default_rng(7)
    for mag in (1e-9, 1e-7, 3e-5, 1.0, 700.0):
        a = (rng.standard_normal(4000) * mag).astype(np.float32).astype(np.float64)
        s = O.f16_safe_scale(a)
        assert math.log2(s) == int(math.log2(s))  # a power of two
        m = np.max(np.abs(a)) * s
        assert 2.0 ** 14 <= m < 2.0 ** 15
        back = O.round_f16_sat(a * s) / s
        big = np.abs(a) > np.max(np.abs(a)) * 2.0 ** -10  # inside the half normal range after scaling
        assert np.max(np.abs(back - a)[big] / np.abs(a)[big]) <= 2.0 ** -11
    # without the scale, cotangents of 1e-7 lose their relative accuracy
    a = rng.standard_normal(4000) * 1e-7
    plain = O.round_f16_sat(a)
    assert np.median(np.abs(plain - a) / np.abs(a)) > 0.05


def test_round_f32_hand_values():
    """Round-to-nearest-even into float32, from hand-derived values."""
    u = 2.0 ** -24
    cases = [
        (1.0 + u, 1.0),                       # tie between 1 and 1 + 2u: even is 1
        (1.0 + 3 * u, 1.0 + 4 * u),           # tie between 1 + 2u and 1 + 4u: even is 1 + 4u
        (1.0 + u * 1.0000001, 1.0 + 2 * u),   # just past the tie rounds up
        (1.0 + 2 * u, 1.0 + 2 * u),           # representable: unchanged
        (0.1, 13421773 * 2.0 ** -27),         # 0x3DCCCCCD
        (-7.0, -7.0),
        (2.0 ** -149, 2.0 ** -149),           # smallest subnormal
        (2.0 ** -150, 0.0),                   # tie with 0: even is 0
        (3 * 2.0 ** -150, 2.0 ** -148),       # tie between 1 and 2 subnormal units: 2
        (2.0 ** 128 * (1 - 2.0 ** -25), float("inf")),  # rounds past the largest float
        (2.0 ** 128 * (1 - 2.0 ** -24), 2.0 ** 128 * (1 - 2.0 ** -24)),  # largest float
    ]
    for x, want in cases:
        with np.errstate(over="ignore"):
            got = O.round_f32(np.array([x]))[0]
        assert got == want, (x, got, want)
    assert np.isnan(O.round_f32(np.array([np.nan]))[0])


# ---------------------------------------------------------------- activations

def test_relu_regions():
    z = np.linspace(-5, 5, 1001)
    y = O.act_fwd(z, O.ACT_RELU)
    assert np.array_equal(y[z > 0], z[z > 0])
    assert np.all(y[z <= 0] == 0.0)
    d = O.act_grad(z, O.ACT_RELU)
    assert np.all(d[z > 0] == 1.0) and np.all(d[z <= 0] == 0.0)
    # ReLU'(0) = 0 (mask is Z > 0 strictly)
    assert O.act_grad(np.array([0.0]), O.ACT_RELU)[0] == 0.0


def test_identity():
    z = np.linspace(-3, 3, 7)
    assert np.array_equal(O.act_fwd(z, O.ACT_IDENTITY), z)
    assert np.all(O.act_grad(z, O.ACT_IDENTITY) == 1.0)


def test_gelu_closed_forms():
    z = np.linspace(-8, 8, 4001)
    g = O.act_fwd(z, O.ACT_GELU_TANH)
    d = O.act_grad(z, O.ACT_GELU_TANH)
    assert O.act_fwd(np.array([0.0]), O.ACT_GELU_TANH)[0] == 0.0
    assert O.act_grad(np.array([0.0]), O.ACT_GELU_TANH)[0] == 0.5
    # gelu(z) - gelu(-z) = z  (x Phi(x) with an odd-symmetric Phi - 1/2)
    assert np.max(np.abs(g - O.act_fwd(-z, O.ACT_GELU_TANH) - z)) < 1e-12
    # gelu'(z) + gelu'(-z) = 1
    assert np.max(np.abs(d + O.act_grad(-z, O.ACT_GELU_TANH) - 1.0)) < 1e-12
    big = np.array([30.0, 50.0])
    assert np.allclose(O.act_fwd(big, O.ACT_GELU_TANH), big, rtol=0, atol=1e-12)
    assert np.allclose(O.act_grad(big, O.ACT_GELU_TANH), 1.0, atol=1e-12)
    assert np.allclose(O.act_fwd(-big, O.ACT_GELU_TANH), 0.0, atol=1e-12)


def test_gelu_matches_torch_tanh_gelu():
    z = np.linspace(-10, 10, 20001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh")
    assert np.max(np.abs(O.act_fwd(z, O.ACT_GELU_TANH) - ref.numpy())) < 1e-14
    # and it stays within 1e-3 of the exact (erf) GELU it approximates
    exact = 0.5 * z * (1.0 + scipy.special.erf(z / math.sqrt(2.0)))
    assert np.max(np.abs(O.act_fwd(z, O.ACT_GELU_TANH) - exact)) < 1e-3


def test_gelu_grad_matches_torch_autograd():
    z = torch.linspace(-6, 6, 1201, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(z, approximate="tanh").sum().backward()
    ref = z.grad.numpy()
    assert np.max(np.abs(O.act_grad(z.detach().numpy(), O.ACT_GELU_TANH) - ref)) < 1e-13


@pytest.mark.parametrize("act", ACTS)
def test_act_grad_central_difference(act):
    z = np.linspace(-4, 4, 801)
    z = z[np.abs(z) > 1e-3]  # away from the ReLU kink
    h = 1e-5
    fd = (O.act_fwd(z + h, act) - O.act_fwd(z - h, act)) / (2 * h)
    assert np.max(np.abs(fd - O.act_grad(z, act))) < 1e-8


# ---------------------------------------------------------------- dense fwd

def _brute_fwd(X, W, b, act):
    B, K = X.shape
    N = W.shape[0]
    Z = np.zeros((B, N))
    for i in range(B):
        for j in range(N):
            s = 0.0 if b is None else float(b[j])
            for k in range(K):
                s += float(X[i, k]) * float(W[j, k])
            Z[i, j] = s
    return Z


def _tiny_layer(seed, B, n_in, n_out, away_from_kink=True):
    rng = np.random.default_rng(seed)
    for _ in range(1000):
        X = rng.standard_normal((B, n_in))
        W = rng.standard_normal((n_out, n_in))
        b = rng.standard_normal(n_out)
        Z = X @ W.T + b
        if not away_from_kink or np.min(np.abs(Z)) > 1e-2:
            return X, W, b
    raise RuntimeError("could not draw a kink-free layer")


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 4), (6, 2, 5), (4, 6, 3)])
def test_dense_fwd_brute_force(act, shape):
    X, W, b = _tiny_layer(11, *shape, away_from_kink=False)
    Y, Z = O.dense_act_fwd(X, W, b, act)
    Zb = _brute_fwd(X, W, b, act)
    assert np.max(np.abs(Z - Zb)) < 1e-12
    # act applied elementwise, checked against a library routine
    tz = torch.from_numpy(Zb)
    ref = {O.ACT_IDENTITY: tz, O.ACT_RELU: torch.relu(tz),
           O.ACT_GELU_TANH: torch.nn.functional.gelu(tz, approximate="tanh")}[act]
    assert np.max(np.abs(Y - ref.numpy())) < 1e-12


def test_dense_fwd_no_bias_matches_library_matmul():
    X, W, b = _tiny_layer(3, 50, 70, 30, away_from_kink=False)
    Y, Z = O.dense_act_fwd(X, W, None, O.ACT_IDENTITY)
    ref = torch.nn.functional.linear(torch.from_numpy(X), torch.from_numpy(W))
    assert rel_norm(Z, ref.numpy()) < 1e-13


# ---------------------------------------------------------------- vjp

@pytest.mark.parametrize("act", ACTS)
def test_vjp_central_difference(act):
    """L = sum(R * act(X W^T + b)); dL/dX, dL/dW, dL/db by central FD."""
    B, n_in, n_out = 3, 5, 4
    X, W, b = _tiny_layer(5, B, n_in, n_out)
    R = np.random.default_rng(6).standard_normal((B, n_out))

    def loss(X_, W_, b_):
        return float(np.sum(R * O.dense_act_fwd(X_, W_, b_, act)[0]))

    _, Z = O.dense_act_fwd(X, W, b, act)
    dX, dW, db = O.dense_act_vjp(R, Z, X, W, act)

    def fd(arr, which):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            h = 1e-6 * max(1.0, abs(arr[idx]))
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = [X, W, b]
            args_m = [X, W, b]
            args_p[which], args_m[which] = p, m
            out[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        return out

    assert rel_norm(dX, fd(X, 0)) < 1e-5
    assert rel_norm(dW, fd(W, 1)) < 1e-5
    assert rel_norm(db, fd(b, 2)) < 1e-5


@pytest.mark.parametrize("act", ACTS)
def test_vjp_db_is_column_sum_of_masked_grad(act):
    X, W, b = _tiny_layer(8, 7, 6, 5, away_from_kink=False)
    dY = np.random.default_rng(9).standard_normal((7, 5))
    _, Z = O.dense_act_fwd(X, W, b, act)
    _, dW, db = O.dense_act_vjp(dY, Z, X, W, act)
    # masked upstream gradient built with a library activation derivative
    tz = torch.from_numpy(Z).requires_grad_(True)
    f = {O.ACT_IDENTITY: lambda t: t, O.ACT_RELU: torch.relu,
         O.ACT_GELU_TANH: lambda t: torch.nn.functional.gelu(t, approximate="tanh")}[act]
    f(tz).backward(torch.from_numpy(dY))
    G = tz.grad.numpy()
    for j in range(5):
        assert abs(db[j] - sum(G[i, j] for i in range(7))) < 1e-12
    # dW as a sum of outer products, in loops
    dWb = np.zeros_like(dW)
    for i in range(7):
        for j in range(5):
            for k in range(6):
                dWb[j, k] += G[i, j] * X[i, k]
    assert np.max(np.abs(dW - dWb)) < 1e-12


def test_vjp_need_dx_false():
    X, W, b = _tiny_layer(1, 3, 4, 2)
    _, Z = O.dense_act_fwd(X, W, b, O.ACT_RELU)
    dX, dW, db = O.dense_act_vjp(np.ones((3, 2)), Z, X, W, O.ACT_RELU,
                                 need_dx=False)
    assert dX is None and dW.shape == (2, 4) and db.shape == (2,)


# ---------------------------------------------------------------- xent

def test_xent_by_row_blocks_with_batch_total():
    """Rows are independent: the batch taken in blocks of rows, each with
    the whole batch as the divisor, gives the same dlogits and row losses,
    and the block losses add up to the batch loss."""
    rng = np.random.default_rng(71)
    z = rng.standard_normal((12, 9)) * 2.0
    y = rng.integers(0, 9, 12).astype(np.int32)
    loss, dz, row = O.softmax_xent_fwd_bwd(z, y)
    parts = [O.softmax_xent_fwd_bwd(z[i:i + 4], y[i:i + 4], batch_total=12) for i in (0, 4, 8)]
    assert abs(sum(p[0] for p in parts) - loss) < 1e-14
    assert np.allclose(np.concatenate([p[1] for p in parts]), dz, rtol=1e-14, atol=1e-17)
    assert np.array_equal(np.concatenate([p[2] for p in parts]), row)
    with pytest.raises(ValueError):
        O.softmax_xent_fwd_bwd(z, y, batch_total=11)


def test_softmax_lse_matches_scipy_and_row_loss():
    from scipy.special import logsumexp
    rng = np.random.default_rng(72)
    z = rng.standard_normal((7, 40)) * 5.0 + 100.0
    y = rng.integers(0, 40, 7).astype(np.int32)
    lse = O.softmax_lse(z)
    assert np.allclose(lse, logsumexp(z, axis=1), rtol=1e-15, atol=1e-12)
    _, _, row = O.softmax_xent_fwd_bwd(z, y)
    assert np.allclose(row, lse - z[np.arange(7), y], rtol=1e-13, atol=1e-12)


def _xent_case(seed, B, C, scale=3.0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, C)) * scale
    y = rng.integers(0, C, size=B).astype(np.int32)
    return z, y


def test_xent_matches_library_routines():
    z, y = _xent_case(0, 37, 13)
    loss, dz, row = O.softmax_xent_fwd_bwd(z, y)
    p = scipy.special.softmax(z, axis=1)
    onehot = np.eye(13)[y]
    assert rel_norm(dz, (p - onehot) / 37) < 1e-14
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z),
                                            torch.from_numpy(y).long())
    assert abs(loss - ref.item()) < 1e-14
    lse = scipy.special.logsumexp(z, axis=1)
    assert np.max(np.abs(row - (lse - z[np.arange(37), y]))) < 1e-13


def test_xent_invariants():
    z, y = _xent_case(1, 29, 40)
    B = 29
    loss, dz, row = O.softmax_xent_fwd_bwd(z, y)
    onehot = np.eye(40)[y]
    p = dz * B + onehot
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12   # softmax rows sum to 1
    assert np.all(p > 0)
    assert np.max(np.abs(dz.sum(axis=1))) < 1e-15        # dz rows sum to 0
    assert loss >= 0 and np.all(row >= 0)
    # shift invariance of each row
    shift = np.random.default_rng(2).standard_normal((B, 1)) * 50
    loss2, dz2, _ = O.softmax_xent_fwd_bwd(z + shift, y)
    assert abs(loss2 - loss) < 1e-12 and np.max(np.abs(dz2 - dz)) < 1e-15


@pytest.mark.parametrize("C", [1, 2, 10, 1000])
def test_xent_zero_logits(C):
    B = 5
    y = np.arange(B, dtype=np.int32) % C
    loss, dz, _ = O.softmax_xent_fwd_bwd(np.zeros((B, C)), y)
    assert abs(loss - math.log(C)) < 1e-15
    ref = (np.full((B, C), 1.0 / C) - np.eye(C)[y]) / B
    assert np.max(np.abs(dz - ref)) < 1e-17


def test_xent_central_difference():
    z, y = _xent_case(3, 4, 7)
    _, dz, _ = O.softmax_xent_fwd_bwd(z, y)
    fd = np.zeros_like(z)
    for idx in np.ndindex(z.shape):
        h = 1e-6
        p, m = z.copy(), z.copy()
        p[idx] += h
        m[idx] -= h
        fd[idx] = (O.softmax_xent_fwd_bwd(p, y)[0]
                   - O.softmax_xent_fwd_bwd(m, y)[0]) / (2 * h)
    assert rel_norm(dz, fd) < 1e-7


def test_xent_rejects_bad_labels():
    with pytest.raises(ValueError):
        O.softmax_xent_fwd_bwd(np.zeros((2, 3)), np.array([0, 3], np.int32))
    with pytest.raises(ValueError):
        O.softmax_xent_fwd_bwd(np.zeros((2, 3)), np.array([-1, 0], np.int32))


# ---------------------------------------------------------------- optimizers

def test_sgd_one_step():
    rng = np.random.default_rng(0)
    w, g = rng.standard_normal(100), rng.standard_normal(100)
    out = O.sgd_step(w, g, 1e-3)
    for i in range(100):
        assert out[i] == w[i] - 1e-3 * g[i]
    # torch's plain SGD
    tw = torch.from_numpy(w.copy()).requires_grad_(True)
    opt = torch.optim.SGD([tw], lr=1e-3)
    tw.grad = torch.from_numpy(g)
    opt.step()
    assert np.max(np.abs(tw.detach().numpy() - out)) < 1e-15


def test_adamw_step1_closed_form():
    rng = np.random.default_rng(1)
    w, g = rng.standard_normal(64), rng.standard_normal(64)
    g[:4] = 0.0
    lr, wd, eps = 1e-3, 0.01, 1e-8
    w1, m1, v1 = O.adamw_step(w, g, np.zeros(64), np.zeros(64), lr, 0.9, 0.999,
                              eps, wd, 1)
    # at t = 1: m_hat = g, v_hat = g^2
    ref = w * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.max(np.abs(w1 - ref)) < 1e-15
    # g = 0 gives pure decay
    assert np.array_equal(w1[:4], w[:4] * (1 - lr * wd))
    assert np.max(np.abs(m1 - 0.1 * g)) < 1e-16
    assert np.max(np.abs(v1 - 0.001 * g * g)) < 1e-16


def test_adamw_step2_hand_form():
    g1, g2, w0 = 0.3, -0.7, 1.25
    lr, b1, b2, eps, wd = 1e-2, 0.9, 0.999, 1e-8, 0.1
    w, m, v = O.adamw_step(np.array([w0]), np.array([g1]), np.zeros(1),
                           np.zeros(1), lr, b1, b2, eps, wd, 1)
    w, m, v = O.adamw_step(w, np.array([g2]), m, v, lr, b1, b2, eps, wd, 2)
    m2 = (1 - b1) * (b1 * g1 + g2)
    v2 = (1 - b2) * (b2 * g1 * g1 + g2 * g2)
    w1 = w0 * (1 - lr * wd) - lr * g1 / (abs(g1) + eps)
    w2 = w1 * (1 - lr * wd) - lr * (m2 / (1 - b1 ** 2)) / (
        math.sqrt(v2 / (1 - b2 ** 2)) + eps)
    assert abs(w[0] - w2) < 1e-15 and abs(m[0] - m2) < 1e-17
    assert abs(v[0] - v2) < 1e-18


def test_adamw_matches_torch_adamw_many_steps():
    rng = np.random.default_rng(2)
    w0 = rng.standard_normal(500)
    grads = [rng.standard_normal(500) for _ in range(30)]
    tw = torch.from_numpy(w0.copy()).requires_grad_(True)
    opt = torch.optim.AdamW([tw], lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                            weight_decay=0.01)
    w, m, v = w0.copy(), np.zeros(500), np.zeros(500)
    for t, g in enumerate(grads, start=1):
        tw.grad = torch.from_numpy(g.copy())
        opt.step()
        w, m, v = O.adamw_step(w, g, m, v, 1e-3, 0.9, 0.999, 1e-8, 0.01, t)
    assert rel_norm(w, tw.detach().numpy()) < 1e-13
    st = opt.state[tw]
    assert rel_norm(m, st["exp_avg"].numpy()) < 1e-13
    assert rel_norm(v, st["exp_avg_sq"].numpy()) < 1e-13


def test_adamw_rejects_step0():
    with pytest.raises(ValueError):
        O.adamw_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1),
                     1e-3, 0.9, 0.999, 1e-8, 0.0, 0)


# ---------------------------------------------------------------- MLP step

class _Opt:
    def __init__(self, kind, lr=1e-3, wd=0.0):
        self.kind, self.lr, self.beta1, self.beta2 = kind, lr, 0.9, 0.999
        self.eps, self.weight_decay = 1e-8, wd


def _tiny_mlp(seed, dims, B):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((B, dims[0])).astype(np.float32)
    y = rng.integers(0, dims[-1], size=B).astype(np.int32)
    W = [(rng.standard_normal((dims[l + 1], dims[l])) * 0.8).astype(np.float32)
         for l in range(len(dims) - 1)]
    b = [(rng.standard_normal(dims[l + 1]) * 0.3).astype(np.float32)
         for l in range(len(dims) - 1)]
    return X, y, W, b


def test_mlp_step_gradients_central_difference():
    dims, B = [5, 4, 3, 3], 4
    acts = [O.ACT_RELU, O.ACT_RELU, O.ACT_IDENTITY]
    X, y, W, b = _tiny_mlp(7, dims, B)
    st = O.MLPState(W, b)
    out = O.mlp_train_step(st, X, y, acts, _Opt("sgd", lr=0.0))
    for Z in out["Z"][:-1]:
        assert np.min(np.abs(Z)) > 1e-4  # FD stays on one side of each kink

    def loss_of(Ws, bs):
        h = np.asarray(X, np.float64)
        for l in range(3):
            h = O.dense_act_fwd(h, Ws[l], bs[l], acts[l])[0]
        return O.softmax_xent_fwd_bwd(h, y)[0]

    Ws = [w.astype(np.float64) for w in W]
    bs = [x.astype(np.float64) for x in b]
    for l in range(3):
        for arr, grad in ((Ws[l], out["dW"][l]), (bs[l], out["db"][l])):
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                h = 1e-6
                arr[idx] += h
                lp = loss_of(Ws, bs)
                arr[idx] -= 2 * h
                lm = loss_of(Ws, bs)
                arr[idx] += h
                fd[idx] = (lp - lm) / (2 * h)
            assert rel_norm(grad, fd) < 1e-5


@pytest.mark.parametrize("kind", ["sgd", "adamw"])
def test_mlp_trajectory_matches_torch_float64(kind):
    """Five steps of the oracle against PyTorch modules/optimizers in float64
    (fresh float32 rounding of the state each step on the oracle side)."""
    dims, B = [6, 5, 4, 3], 8
    acts = [O.ACT_RELU, O.ACT_RELU, O.ACT_IDENTITY]
    X, y, W, b = _tiny_mlp(3, dims, B)
    opt = _Opt(kind, lr=1e-2, wd=0.01 if kind == "adamw" else 0.0)
    st = O.MLPState(W, b)
    layers = [torch.nn.Linear(dims[l], dims[l + 1]).double() for l in range(3)]
    with torch.no_grad():
        for l in range(3):
            layers[l].weight.copy_(torch.from_numpy(W[l].astype(np.float64)))
            layers[l].bias.copy_(torch.from_numpy(b[l].astype(np.float64)))
    model = torch.nn.Sequential(layers[0], torch.nn.ReLU(), layers[1],
                                torch.nn.ReLU(), layers[2])
    if kind == "sgd":
        topt = torch.optim.SGD(model.parameters(), lr=opt.lr)
    else:
        topt = torch.optim.AdamW(model.parameters(), lr=opt.lr,
                                 betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    tx = torch.from_numpy(X.astype(np.float64))
    ty = torch.from_numpy(y).long()
    for _ in range(5):
        topt.zero_grad()
        tl = torch.nn.functional.cross_entropy(model(tx), ty)
        tl.backward()
        grads = [(layers[l].weight.grad.numpy().copy(),
                  layers[l].bias.grad.numpy().copy()) for l in range(3)]
        topt.step()
        out = O.mlp_train_step(st, X, y, acts, opt)
        assert abs(out["loss"] - tl.item()) < 1e-6 * abs(tl.item())
        for l in range(3):
            assert rel_norm(out["dW"][l], grads[l][0]) < 1e-5
            assert rel_norm(out["db"][l], grads[l][1]) < 1e-5
    for l in range(3):
        assert rel_norm(st.W[l], layers[l].weight.detach().numpy()) < 1e-5
        assert rel_norm(st.b[l], layers[l].bias.detach().numpy()) < 1e-5


def test_mlp_loss_is_pre_update():
    dims, B = [4, 3, 2], 6
    X, y, W, b = _tiny_mlp(9, dims, B)
    acts = [O.ACT_RELU, O.ACT_IDENTITY]
    st = O.MLPState(W, b)
    h = O.dense_act_fwd(X, st.W[0], st.b[0], acts[0])[0]
    h = O.dense_act_fwd(h, st.W[1], st.b[1], acts[1])[0]
    before = O.softmax_xent_fwd_bwd(h, y)[0]
    out = O.mlp_train_step(st, X, y, acts, _Opt("sgd", lr=0.5))
    assert out["loss"] == before

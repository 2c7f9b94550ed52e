"""Pins of the oracle's optimizer, loss and gradient-control variants: closed
forms, hand-computed trajectories, invariants, and the special cases that
reduce to PyTorch's own CPU routines (torch.optim.Adam, clip_grad_norm_,
mse_loss, the lr_scheduler classes, the GradScaler update), all float64."""
import math

import numpy as np
import pytest
import torch

import oracle as O

from tests.test_oracle_pins import rel_norm, _tiny_mlp


# ---------------------------------------------------------------- Adam (coupled)

def test_adam_step1_closed_form():
    rng = np.random.default_rng(11)
    w, g = rng.standard_normal(64), rng.standard_normal(64)
    lr, wd, eps = 1e-3, 0.05, 1e-8
    w1, m1, v1 = O.adam_step(w, g, np.zeros(64), np.zeros(64), lr, 0.9, 0.999, eps, wd, 1)
    gp = g + wd * w  # the decay enters the gradient
    assert np.max(np.abs(w1 - (w - lr * gp / (np.abs(gp) + eps)))) < 1e-15
    assert np.max(np.abs(m1 - 0.1 * gp)) < 1e-16
    assert np.max(np.abs(v1 - 0.001 * gp * gp)) < 1e-16


def test_adam_constant_gradient_closed_form():
    """With wd = 0 and a constant gradient, m_hat = g and v_hat = g^2 at every
    step, so each step moves lr g / (|g| + eps)."""
    g, w = np.array([0.25, -2.0, 1e-3]), np.array([1.0, 0.5, -0.75])
    m, v = np.zeros(3), np.zeros(3)
    lr, eps = 1e-2, 1e-8
    for t in range(1, 8):
        w, m, v = O.adam_step(w, g, m, v, lr, 0.9, 0.999, eps, 0.0, t)
    ref = np.array([1.0, 0.5, -0.75]) - 7 * lr * g / (np.abs(g) + eps)
    assert np.max(np.abs(w - ref)) < 1e-14


def test_adam_matches_torch_adam_many_steps():
    rng = np.random.default_rng(12)
    w0 = rng.standard_normal(400)
    tw = torch.from_numpy(w0.copy()).requires_grad_(True)
    opt = torch.optim.Adam([tw], lr=2e-3, betas=(0.8, 0.99), eps=1e-8, weight_decay=0.03)
    w, m, v = w0.copy(), np.zeros(400), np.zeros(400)
    for t in range(1, 31):
        g = rng.standard_normal(400)
        tw.grad = torch.from_numpy(g.copy())
        opt.step()
        w, m, v = O.adam_step(w, g, m, v, 2e-3, 0.8, 0.99, 1e-8, 0.03, t)
    assert rel_norm(w, tw.detach().numpy()) < 1e-13
    st = opt.state[tw]
    assert rel_norm(m, st["exp_avg"].numpy()) < 1e-13
    assert rel_norm(v, st["exp_avg_sq"].numpy()) < 1e-13


def test_adam_and_adamw_agree_without_decay_and_differ_with_it():
    rng = np.random.default_rng(13)
    w, g = rng.standard_normal(32), rng.standard_normal(32)
    z = np.zeros(32)
    a = O.adam_step(w, g, z, z, 1e-2, 0.9, 0.999, 1e-8, 0.0, 1)[0]
    b = O.adamw_step(w, g, z, z, 1e-2, 0.9, 0.999, 1e-8, 0.0, 1)[0]
    assert np.array_equal(a, b)
    a = O.adam_step(w, g, z, z, 1e-2, 0.9, 0.999, 1e-8, 0.1, 1)[0]
    b = O.adamw_step(w, g, z, z, 1e-2, 0.9, 0.999, 1e-8, 0.1, 1)[0]
    assert np.max(np.abs(a - b)) > 1e-6


# ---------------------------------------------------------------- clipping

def test_global_norm_and_clip_coef_hand_values():
    grads = [np.array([3.0]), np.array([[0.0, 4.0]])]
    assert O.global_grad_norm(grads) == 5.0
    assert O.clip_coef(5.0, 1.0) == 1.0 / (5.0 + 1e-6)
    assert O.clip_coef(5.0, 10.0) == 1.0
    assert O.global_grad_norm([np.zeros(7)]) == 0.0


def test_clip_matches_torch_clip_grad_norm():
    rng = np.random.default_rng(14)
    arrays = [rng.standard_normal(s) for s in ((7, 5), (5,), (3, 7), (3,))]
    for max_norm in (0.5, 3.0, 100.0):
        ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in arrays]
        for t, a in zip(ts, arrays):
            t.grad = torch.from_numpy(a.copy())
        total = torch.nn.utils.clip_grad_norm_(ts, max_norm)
        norm = O.global_grad_norm(arrays)
        assert abs(norm - total.item()) < 1e-13 * norm
        c = O.clip_coef(norm, max_norm)
        for t, a in zip(ts, arrays):
            assert np.max(np.abs(t.grad.numpy() - c * a)) < 1e-15


def test_grad_control_finite_check_and_multiplier():
    g = [np.array([6.0, 8.0]), np.array([0.0])]
    found, norm, mul = O.grad_control(g, max_norm=1.0, scale=2.0)
    assert not found and norm == 5.0  # norm of the unscaled gradients
    assert mul == (1.0 / (5.0 + 1e-6)) / 2.0
    found, _, mul = O.grad_control(g, max_norm=0.0, scale=4.0)
    assert not found and mul == 0.25
    for bad in (np.nan, np.inf, -np.inf):
        assert O.grad_control([np.array([1.0, bad])], 0.0, 1.0)[0]


# ---------------------------------------------------------------- EMA

def test_ema_constant_parameter_closed_form():
    w, e0, d = np.array([2.0, -1.0, 0.5]), np.array([0.0, 3.0, 0.5]), 0.9
    e = e0.copy()
    for _ in range(10):
        e = O.ema_update(e, w, d)
    assert np.max(np.abs(e - (w + d ** 10 * (e0 - w)))) < 1e-15


def test_ema_matches_torch_ema_avg_fn():
    rng = np.random.default_rng(15)
    fn = torch.optim.swa_utils.get_ema_avg_fn(0.99)
    e = rng.standard_normal(50)
    te = torch.from_numpy(e.copy())
    for n in range(5):
        w = rng.standard_normal(50)
        te = fn(te, torch.from_numpy(w), torch.tensor(n))
        e = O.ema_update(e, w, 0.99)
    assert np.max(np.abs(e - te.numpy())) < 1e-15


# ---------------------------------------------------------------- LR schedules

def test_lr_schedule_hand_values():
    base, mn = 1.0, 0.1
    assert O.lr_at(O.LR_CONSTANT, 0.3, 17) == 0.3
    assert [O.lr_at(O.LR_STEP, base, t, step_size=3, gamma=0.5) for t in range(1, 8)] == \
        [1.0, 1.0, 1.0, 0.5, 0.5, 0.5, 0.25]
    cos = lambda t: O.lr_at(O.LR_WARMUP_COSINE, base, t, warmup=4, total=14, min_lr=mn)
    assert [cos(t) for t in (1, 2, 4)] == [0.25, 0.5, 1.0]
    assert cos(5) == 1.0  # k = warmup: the cosine's start
    assert abs(cos(10) - (base + mn) / 2) < 1e-15  # k - warmup = T / 2
    assert cos(15) == mn and cos(100) == mn
    lin = lambda t: O.lr_at(O.LR_WARMUP_LINEAR, base, t, warmup=2, total=6, min_lr=mn)
    assert [lin(t) for t in (1, 2, 3)] == [0.5, 1.0, 1.0]
    assert abs(lin(5) - 0.55) < 1e-15 and lin(7) == mn and lin(50) == mn
    with pytest.raises(ValueError):
        O.lr_at(O.LR_CONSTANT, 1.0, 0)


def _torch_lrs(make, steps, base):
    p = torch.nn.Parameter(torch.zeros(1, dtype=torch.float64))
    opt = torch.optim.SGD([p], lr=base)
    sch = make(opt)
    out = []
    for _ in range(steps):
        out.append(opt.param_groups[0]["lr"])
        opt.step()
        sch.step()
    return out


def test_lr_schedules_match_torch_schedulers():
    L = torch.optim.lr_scheduler
    base, mn, W, T = 0.5, 0.02, 5, 40
    ref = _torch_lrs(lambda o: L.StepLR(o, step_size=7, gamma=0.3), 30, base)
    got = [O.lr_at(O.LR_STEP, base, t, step_size=7, gamma=0.3) for t in range(1, 31)]
    assert np.max(np.abs(np.array(got) - ref)) < 1e-15
    ref = _torch_lrs(lambda o: L.SequentialLR(o, [
        L.LinearLR(o, start_factor=1.0 / W, end_factor=1.0, total_iters=W - 1),
        L.CosineAnnealingLR(o, T_max=T - W, eta_min=mn)], milestones=[W]), T, base)
    got = [O.lr_at(O.LR_WARMUP_COSINE, base, t, warmup=W, total=T, min_lr=mn)
           for t in range(1, T + 1)]
    assert np.max(np.abs(np.array(got) - ref)) < 1e-12


# ---------------------------------------------------------------- MSE

def test_mse_constant_offset_closed_form():
    rng = np.random.default_rng(16)
    t = rng.standard_normal((5, 3))
    loss, d = O.mse_loss_fwd_bwd(t + 0.5, t)
    assert abs(loss - 0.25) < 1e-15
    assert np.max(np.abs(d - 2 * 0.5 / 15)) < 1e-16


def test_mse_matches_torch_and_central_difference():
    rng = np.random.default_rng(17)
    p, t = rng.standard_normal((6, 4)), rng.standard_normal((6, 4))
    loss, d = O.mse_loss_fwd_bwd(p, t)
    tp = torch.from_numpy(p.copy()).requires_grad_(True)
    tl = torch.nn.functional.mse_loss(tp, torch.from_numpy(t))
    tl.backward()
    assert abs(loss - tl.item()) < 1e-15
    assert np.max(np.abs(d - tp.grad.numpy())) < 1e-16
    h = 1e-6
    for idx in [(0, 0), (3, 2), (5, 3)]:
        q = p.copy()
        q[idx] += h
        lp = O.mse_loss_fwd_bwd(q, t)[0]
        q[idx] -= 2 * h
        lm = O.mse_loss_fwd_bwd(q, t)[0]
        assert abs((lp - lm) / (2 * h) - d[idx]) < 1e-8


# ---------------------------------------------------------------- loss scaler

def test_loss_scaler_hand_trajectory():
    s = O.LossScaler(scale=8.0, growth_factor=2.0, backoff_factor=0.5, growth_interval=2)
    seen = []
    for found in (False, False, True, False, False, False):
        s.update(found)
        seen.append((s.scale, s.tracker))
    assert seen == [(8.0, 1), (16.0, 0), (8.0, 0), (8.0, 1), (16.0, 0), (16.0, 1)]


def test_loss_scaler_matches_torch_update_scale():
    rng = np.random.default_rng(18)
    s = O.LossScaler(scale=1024.0, growth_factor=2.0, backoff_factor=0.25, growth_interval=3)
    ts = torch.tensor([1024.0])
    tg = torch.tensor([0], dtype=torch.int32)
    for found in rng.random(60) < 0.2:
        s.update(bool(found))
        torch._amp_update_scale_(ts, tg, torch.tensor([1.0 if found else 0.0]), 2.0, 0.25, 3)
        assert s.scale == ts.item() and s.tracker == tg.item()


# ---------------------------------------------------------------- MLP step variants

class _Opt:
    def __init__(self, kind, lr=1e-2, wd=0.0, max_grad_norm=0.0, ema_decay=None,
                 schedule=None):
        self.kind, self.lr, self.beta1, self.beta2 = kind, lr, 0.9, 0.999
        self.eps, self.weight_decay = 1e-8, wd
        self.max_grad_norm, self.ema_decay, self.schedule = max_grad_norm, ema_decay, schedule


class _Sched:
    def __init__(self, kind, warmup=0, total=1, min_lr=0.0, step_size=1, gamma=1.0):
        self.kind, self.warmup, self.total, self.min_lr = kind, warmup, total, min_lr
        self.step_size, self.gamma = step_size, gamma


def _torch_mlp(dims, W, b):
    layers = [torch.nn.Linear(dims[l], dims[l + 1]).double() for l in range(len(dims) - 1)]
    with torch.no_grad():
        for l, ly in enumerate(layers):
            ly.weight.copy_(torch.from_numpy(W[l].astype(np.float64)))
            ly.bias.copy_(torch.from_numpy(b[l].astype(np.float64)))
    mods = []
    for l, ly in enumerate(layers):
        mods.append(ly)
        if l + 1 < len(layers):
            mods.append(torch.nn.ReLU())
    return layers, torch.nn.Sequential(*mods)


@pytest.mark.parametrize("case", ["adam", "clip", "ema", "schedule", "mse"])
def test_mlp_step_variants_match_torch_float64(case):
    dims, B = [6, 5, 4, 3], 8
    acts = [O.ACT_RELU, O.ACT_RELU, O.ACT_IDENTITY]
    X, y, W, b = _tiny_mlp(21, dims, B)
    kind = "adam" if case == "adam" else "adamw"
    sched = _Sched(O.LR_WARMUP_COSINE, warmup=2, total=6, min_lr=1e-3) if case == "schedule" else None
    opt = _Opt(kind, lr=2e-2, wd=0.02, max_grad_norm=0.3 if case == "clip" else 0.0,
               ema_decay=0.8 if case == "ema" else None, schedule=sched)
    targets = None
    if case == "mse":
        targets = np.random.default_rng(5).standard_normal((B, dims[-1])).astype(np.float32)
    st = O.MLPState(W, b)
    if case == "ema":
        st.enable_ema()
    layers, model = _torch_mlp(dims, W, b)
    params = list(model.parameters())
    if kind == "adam":
        topt = torch.optim.Adam(params, lr=opt.lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.02)
    else:
        topt = torch.optim.AdamW(params, lr=opt.lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.02)
    if sched is not None:
        Ls = torch.optim.lr_scheduler
        tsched = Ls.SequentialLR(topt, [
            Ls.LinearLR(topt, start_factor=0.5, end_factor=1.0, total_iters=1),
            Ls.CosineAnnealingLR(topt, T_max=4, eta_min=1e-3)], milestones=[2])
    ema = [p.detach().clone() for p in params]
    tx = torch.from_numpy(X.astype(np.float64))
    clipped = 0
    for _ in range(6):
        topt.zero_grad()
        out_t = model(tx)
        if case == "mse":
            tl = torch.nn.functional.mse_loss(out_t, torch.from_numpy(targets.astype(np.float64)))
        else:
            tl = torch.nn.functional.cross_entropy(out_t, torch.from_numpy(y).long())
        tl.backward()
        if case == "clip":
            n = torch.nn.utils.clip_grad_norm_(params, 0.3)
            clipped += int(n.item() > 0.3)
        topt.step()
        if sched is not None:
            tsched.step()
        with torch.no_grad():
            for e, p in zip(ema, params):
                e.mul_(0.8).add_(0.2 * p)
        out = O.mlp_train_step(st, X, None if case == "mse" else y, acts, opt, targets=targets)
        assert abs(out["loss"] - tl.item()) < 1e-6 * abs(tl.item())
        assert not out["skipped"]
    if case == "clip":
        assert clipped >= 3  # the clip was active on most steps
    for l in range(3):
        assert rel_norm(st.W[l], layers[l].weight.detach().numpy()) < 1e-5
        assert rel_norm(st.b[l], layers[l].bias.detach().numpy()) < 1e-5
        if case == "ema":
            assert rel_norm(st.eW[l], ema[2 * l].numpy()) < 1e-5
            assert rel_norm(st.eb[l], ema[2 * l + 1].numpy()) < 1e-5


def test_mlp_clip_bounds_the_sgd_update():
    """With SGD and an active clip the whole update has norm lr * max_norm."""
    dims, B = [5, 4, 3], 6
    acts = [O.ACT_RELU, O.ACT_IDENTITY]
    X, y, W, b = _tiny_mlp(22, dims, B)
    st = O.MLPState(W, b)
    before = [a.copy() for a in st.W + st.b]
    out = O.mlp_train_step(st, X, y, acts, _Opt("sgd", lr=0.1, max_grad_norm=1e-3))
    assert out["norm"] > 1e-3
    step = math.sqrt(sum(np.sum((a - c) ** 2) for a, c in zip(st.W + st.b, before)))
    assert abs(step - 0.1 * 1e-3) < 1e-3 * 0.1 * 1e-3


def test_mlp_scaler_skips_non_finite_step_and_backs_off():
    dims, B = [5, 4, 3], 6
    acts = [O.ACT_RELU, O.ACT_IDENTITY]
    X, y, W, b = _tiny_mlp(23, dims, B)
    st = O.MLPState(W, b)
    sc = O.LossScaler(scale=2.0 ** 10, growth_interval=2)
    bad = X.copy()
    bad[2, 1] = np.nan
    before = [a.copy() for a in st.W + st.b]
    out = O.mlp_train_step(st, bad, y, acts, _Opt("adamw"), scaler=sc)
    assert out["skipped"] and st.t == 0 and sc.scale == 2.0 ** 9
    assert all(np.array_equal(a, c) for a, c in zip(st.W + st.b, before))
    ref = O.MLPState(W, b)
    for k in range(2):  # two applied steps: the second one doubles the scale
        out = O.mlp_train_step(st, X, y, acts, _Opt("adamw"), scaler=sc)
        O.mlp_train_step(ref, X, y, acts, _Opt("adamw"))
        assert not out["skipped"]
    assert sc.scale == 2.0 ** 10 and st.t == 2
    # a power-of-two loss scale changes nothing else
    assert all(np.array_equal(a, c) for a, c in zip(st.W + st.b, ref.W + ref.b))


def test_mlp_resume_from_saved_state_is_exact():
    dims, B = [6, 5, 3], 7
    acts = [O.ACT_RELU, O.ACT_IDENTITY]
    X, y, W, b = _tiny_mlp(24, dims, B)
    opt = _Opt("adamw", wd=0.01, ema_decay=0.9)
    straight = O.MLPState(W, b)
    straight.enable_ema()
    for _ in range(4):
        O.mlp_train_step(straight, X, y, acts, opt)
    first = O.MLPState(W, b)
    first.enable_ema()
    for _ in range(2):
        O.mlp_train_step(first, X, y, acts, opt)
    # what a checkpoint holds: parameters, moments, averages and the step count
    resumed = O.MLPState([w.astype(np.float32) for w in first.W],
                         [x.astype(np.float32) for x in first.b])
    for name in ("mW", "vW", "mb", "vb", "eW", "eb"):
        setattr(resumed, name, [a.copy() for a in getattr(first, name)])
    resumed.t = first.t
    for _ in range(2):
        O.mlp_train_step(resumed, X, y, acts, opt)
    for name in ("W", "b", "mW", "vW", "mb", "vb", "eW", "eb"):
        for a, c in zip(getattr(resumed, name), getattr(straight, name)):
            assert np.array_equal(a, c)

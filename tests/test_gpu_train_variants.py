"""Parity of the optimizer, loss-scaling, clipping, EMA, schedule and MSE
paths with the float64 oracle, through the C ABI.

Same bar as the other parity tests: float32 results within a normwise
relative error of 1e-4 (1e-6 for the element-wise updates), the loss within
1e-5 relative, integer and bit-level results exactly.  Where a result is
exact by construction (a power-of-two loss scale, a skipped step, a resumed
run, a replayed graph) the GPU is compared with itself bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as si
from tests.gpu_util import F32_TOL, LOSS_TOL, assert_close, device, misaligned, to_dev, to_np
from tests.test_gpu_parity import (_adopted_masks, _assert_close_band, _copy_state,
                                   _gpu_relu_masks, _grad_bands, _load_state)

pytestmark = pytest.mark.gpu

UPD_TOL = 1e-6  # element-wise float32 updates against the float64 oracle


@pytest.fixture(scope="module")
def dl():
    device()
    import dense_layers_amd
    return dense_layers_amd


class _Opt:
    """Optimizer settings in the form both sides read."""

    def __init__(self, kind, lr=1e-2, wd=0.0, max_grad_norm=0.0, ema_decay=None, schedule=None):
        self.kind, self.lr, self.beta1, self.beta2 = kind, lr, 0.9, 0.999
        self.eps, self.weight_decay = 1e-8, wd
        self.max_grad_norm, self.ema_decay, self.schedule = max_grad_norm, ema_decay, schedule


class _Sched:
    def __init__(self, kind, warmup=0, total=1, min_lr=0.0, step_size=1, gamma=1.0):
        self.kind, self.warmup, self.total, self.min_lr = kind, warmup, total, min_lr
        self.step_size, self.gamma = step_size, gamma


def _kind(dl, name):
    return {"sgd": dl.OPT_SGD, "adamw": dl.OPT_ADAMW, "adam": dl.OPT_ADAM}[name]


def _dl_sched(dl, s):
    if s is None:
        return None
    return dl.Schedule(s.kind, warmup=s.warmup, total=s.total, min_lr=s.min_lr,
                       step_size=s.step_size, gamma=s.gamma)


# ------------------------------------------------------------------ element-wise steps

SIZES = [1, 3, 4096, 16389, (1 << 20) + 3]


@pytest.mark.parametrize("n", SIZES)
def test_adam_ten_steps(dl, n):
    w = si.random_matrix(300, (n,))
    wd, md, vd = to_dev(w), torch.zeros(n, device=device()), torch.zeros(n, device=device())
    wr, mr, vr = O.round_f32(w), np.zeros(n), np.zeros(n)
    for t in range(1, 11):
        g = si.random_matrix(310 + t, (n,), scale=0.1)
        dl.adam_step(wd, to_dev(g), md, vd, 1e-3, 0.9, 0.999, 1e-8, 0.05, t)
        wr, mr, vr = [O.round_f32(a) for a in
                      O.adam_step(wr, g, mr, vr, 1e-3, 0.9, 0.999, 1e-8, 0.05, t)]
    assert_close(to_np(wd), wr, UPD_TOL, "w")
    assert_close(to_np(md), mr, 1e-5, "m")
    assert_close(to_np(vd), vr, 1e-5, "v")


@pytest.mark.parametrize("n", [1, 4097, (1 << 18) + 1])
def test_ema_update(dl, n):
    e = si.random_matrix(320, (n,))
    ed = to_dev(e)
    for k in range(3):
        w = si.random_matrix(321 + k, (n,))
        dl.ema_update(ed, to_dev(w), 0.95)
        e = O.round_f32(O.ema_update(e, w, 0.95))
    assert_close(to_np(ed), e, UPD_TOL, "ema")


def _grad_set(seed, sizes, scale=1.0):
    return [si.random_matrix(seed + k, (n,), scale=scale) for k, n in enumerate(sizes)]


CLIP_SIZES = [[5], [3, 4100, 1], [(1 << 20) + 7, 999], [17 + 31 * k for k in range(40)]]


@pytest.mark.parametrize("sizes", CLIP_SIZES, ids=["one", "ragged", "large", "40_arrays"])
@pytest.mark.parametrize("max_norm", [0.5, 1e6])
def test_clip_grad_norm(dl, sizes, max_norm):
    gs = _grad_set(330, sizes)
    gd = [to_dev(g) for g in gs]
    before = [g.clone() for g in gd]
    norm = dl.clip_grad_norm(gd, max_norm)
    ref_norm = O.global_grad_norm(gs)
    assert abs(norm.item() - ref_norm) <= 1e-6 * ref_norm
    c = O.clip_coef(ref_norm, max_norm)
    if c == 1.0:
        for a, b in zip(gd, before):
            assert torch.equal(a, b)  # no clipping leaves every bit as it was
    for a, g in zip(gd, gs):
        assert_close(to_np(a), c * g, UPD_TOL, "clipped")


def test_clip_grad_norm_misaligned(dl):
    gs = _grad_set(340, [1001, 2050])
    gd = [misaligned(to_dev(g)) for g in gs]
    dl.clip_grad_norm(gd, 0.25)
    c = O.clip_coef(O.global_grad_norm(gs), 0.25)
    for a, g in zip(gd, gs):
        assert_close(to_np(a), c * g, UPD_TOL, "clipped")


# ------------------------------------------------------------------ fused multi-array step

def _params(dl, seed, sizes, adam, ema, bf16, misalign=False):
    host, devp = [], []
    for k, n in enumerate(sizes):
        w = si.random_matrix(seed + 3 * k, (n,))
        e = si.random_matrix(seed + 3 * k + 1, (n,)) if ema else None
        host.append({"w": O.round_f32(w), "m": np.zeros(n), "v": np.zeros(n),
                     "e": None if e is None else O.round_f32(e)})
        t = (lambda a: misaligned(to_dev(a))) if misalign else to_dev
        p = dl.Param(t(w), torch.zeros(n, device=device()),
                     torch.zeros(n, device=device()) if adam else None,
                     torch.zeros(n, device=device()) if adam else None,
                     t(e) if ema else None,
                     torch.empty(n, dtype=torch.bfloat16, device=device()) if bf16 else None)
        devp.append(p)
    return host, devp


def _oracle_multi_step(host, grads, opt, t, scale=1.0):
    """The oracle's fused step over arrays given gradients times `scale`;
    returns whether it was skipped."""
    scaled = [O.round_f32(scale * g) for g in grads]
    found, _, mul = O.grad_control(scaled, opt.max_grad_norm or 0.0, scale)
    if found:
        return True
    lr = O.opt_lr(opt, t)
    for h, g in zip(host, scaled):
        w, m, v = O.optimizer_update(opt.kind, h["w"], mul * g, h["m"], h["v"], opt, t, lr)
        h["w"] = O.round_f32(w)
        if m is not None:
            h["m"], h["v"] = O.round_f32(m), O.round_f32(v)
        if h["e"] is not None:
            h["e"] = O.round_f32(O.ema_update(h["e"], h["w"], opt.ema_decay))
    return False


MULTI_CASES = {
    "sgd_clip": dict(kind="sgd", clip=0.3),
    "adamw_ema_bf16": dict(kind="adamw", ema=0.9, bf16=True),
    "adam_clip_ema": dict(kind="adam", clip=2.0, ema=0.5),
    "adamw_schedule_host": dict(kind="adamw", sched=_Sched(O.LR_WARMUP_COSINE, 2, 6, 1e-4)),
    "sgd_step_schedule_device": dict(kind="sgd", sched=_Sched(O.LR_STEP, step_size=2, gamma=0.5),
                                     dev=True),
    "adamw_all_device": dict(kind="adamw", clip=1.0, ema=0.8, bf16=True, dev=True,
                             sched=_Sched(O.LR_WARMUP_LINEAR, 1, 5, 1e-3)),
}


@pytest.mark.parametrize("case", sorted(MULTI_CASES))
@pytest.mark.parametrize("sizes", [[1, 4096, 5001], [64 + 13 * k for k in range(37)]],
                         ids=["ragged", "37_arrays"])
def test_optimizer_step_matches_oracle(dl, case, sizes):
    c = MULTI_CASES[case]
    adam = c["kind"] != "sgd"
    opt = _Opt(c["kind"], lr=1e-2, wd=0.01, max_grad_norm=c.get("clip", 0.0),
               ema_decay=c.get("ema"), schedule=c.get("sched"))
    host, devp = _params(dl, 400, sizes, adam, "ema" in c, c.get("bf16", False))
    step_dev = torch.zeros(1, dtype=torch.int64, device=device()) if c.get("dev") else None
    norm = torch.zeros(1, device=device())
    for t in range(1, 5):
        grads = _grad_set(500 + 50 * t, sizes, scale=0.3)
        for p, g in zip(devp, grads):
            p.g.copy_(torch.from_numpy(g.astype(np.float32)))
        dl.optimizer_step(devp, _kind(dl, c["kind"]), lr=opt.lr, weight_decay=opt.weight_decay,
                          step=t, step_dev=step_dev, max_grad_norm=opt.max_grad_norm,
                          ema_decay=opt.ema_decay or 0.0, schedule=_dl_sched(dl, opt.schedule),
                          grad_norm=norm)
        assert not _oracle_multi_step(host, grads, opt, t)
        if opt.max_grad_norm > 0:
            ref = O.global_grad_norm(grads)
            assert abs(norm.item() - ref) <= 1e-6 * ref
    if step_dev is not None:
        assert step_dev.item() == 4
    for p, h in zip(devp, host):
        assert_close(to_np(p.w), h["w"], UPD_TOL if not adam else 1e-5, "w")
        if adam:
            assert_close(to_np(p.m), h["m"], 1e-5, "m")
            assert_close(to_np(p.v), h["v"], 1e-5, "v")
        if p.ema is not None:
            assert_close(to_np(p.ema), h["e"], 1e-5, "ema")
        if p.w_bf16 is not None:
            # the copy is the RNE rounding of the updated value, bit for bit
            assert torch.equal(p.w_bf16, p.w.to(torch.bfloat16))
            assert_close(to_np(p.w_bf16), h["w"], 1e-2, "w_bf16")


def test_optimizer_step_misaligned_arrays(dl):
    sizes = [1001, 4099]
    opt = _Opt("adamw", lr=1e-2, wd=0.01, ema_decay=0.9)
    host, devp = _params(dl, 600, sizes, True, True, False, misalign=True)
    grads = _grad_set(610, sizes)
    for p, g in zip(devp, grads):
        p.g.copy_(torch.from_numpy(g.astype(np.float32)))
    dl.optimizer_step(devp, dl.OPT_ADAMW, lr=1e-2, weight_decay=0.01, step=1, ema_decay=0.9)
    _oracle_multi_step(host, grads, opt, 1)
    for p, h in zip(devp, host):
        assert_close(to_np(p.w), h["w"], 1e-5, "w")
        assert_close(to_np(p.ema), h["e"], 1e-5, "ema")


def test_optimizer_step_loss_scaler(dl):
    """Gradients handed over times S: a finite step is the unscaled step, a
    step with a NaN or Inf is skipped and backs the scale off, and the scale
    grows after `interval` applied steps."""
    sizes = [300, 5000]
    opt = _Opt("adamw", lr=1e-2, wd=0.01)
    host, devp = _params(dl, 700, sizes, True, False, False)
    sc = dl.LossScaler(device(), init_scale=1024.0, growth_interval=2)
    osc = O.LossScaler(scale=1024.0, growth_interval=2)
    step_dev = torch.zeros(1, dtype=torch.int64, device=device())
    t = 0
    for k, poison in enumerate([False, True, False, False, True, False]):
        grads = _grad_set(710 + 10 * k, sizes, scale=0.2)
        S = osc.scale
        scaled = [S * g for g in grads]
        if poison:
            scaled[1][17] = np.inf if k == 1 else np.nan
        for p, g in zip(devp, scaled):
            p.g.copy_(torch.from_numpy(g.astype(np.float32)))
        before = [p.w.clone() for p in devp]
        dl.optimizer_step(devp, dl.OPT_ADAMW, lr=1e-2, weight_decay=0.01, step_dev=step_dev,
                          scaler=sc)
        skipped = _oracle_multi_step(host, [g / S for g in scaled], opt, t + 1, scale=S) \
            if not poison else True
        osc.update(poison)
        assert skipped == poison
        if not poison:
            t += 1
        assert sc.found_inf.item() == int(poison)
        assert sc.scale.item() == osc.scale and sc.growth_tracker.item() == osc.tracker
        assert step_dev.item() == t
        if poison:
            for a, b in zip(devp, before):
                assert torch.equal(a.w, b)
    for p, h in zip(devp, host):
        assert_close(to_np(p.w), h["w"], 1e-5, "w")
        assert_close(to_np(p.m), h["m"], 1e-5, "m")


# ------------------------------------------------------------------ MSE

MSE_SHAPES = [(1, 1), (7, 3), (64, 10), (1000, 1000), (4096, 4097), (16384, 1024)]


@pytest.mark.parametrize("shape", MSE_SHAPES)
def test_mse_loss(dl, shape):
    p = si.random_matrix(800, shape)
    t = si.random_matrix(801, shape)
    loss, dp = dl.mse_loss_fwd_bwd(to_dev(p), to_dev(t))
    rl, rd = O.mse_loss_fwd_bwd(p, t)
    assert abs(loss.item() - rl) <= LOSS_TOL * rl
    assert_close(to_np(dp), rd, UPD_TOL, "dpred")


def test_mse_loss_in_place_misaligned_and_loss_only(dl):
    p = si.random_matrix(810, (333, 77))
    t = si.random_matrix(811, (333, 77))
    rl, rd = O.mse_loss_fwd_bwd(p, t)
    pd = misaligned(to_dev(p))
    loss, dp = dl.mse_loss_fwd_bwd(pd, misaligned(to_dev(t)), in_place=True)
    assert dp.data_ptr() == pd.data_ptr()
    assert abs(loss.item() - rl) <= LOSS_TOL * rl
    assert_close(to_np(dp), rd, UPD_TOL, "dpred in place")
    ws = torch.empty(dl.mse_loss_workspace_size(333, 77), dtype=torch.uint8, device=device())
    loss2 = torch.empty(1, device=device())
    p2, t2 = to_dev(p), to_dev(t)  # held until the call has run
    st = dl._c["mse_loss_fwd_bwd"](dl._stream(p2), 333, 77, dl._ptr(p2), dl._ptr(t2),
                                   dl._ptr(loss2), None, dl._ptr(ws), ws.numel())
    assert st == 0 and abs(loss2.item() - rl) <= LOSS_TOL * rl


def test_mse_loss_bit_reproducible(dl):
    p, t = to_dev(si.random_matrix(820, (4096, 4097))), to_dev(si.random_matrix(821, (4096, 4097)))
    a = dl.mse_loss_fwd_bwd(p, t)
    b = dl.mse_loss_fwd_bwd(p, t)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------ MLP step variants

VARIANT_WORKLOADS = {
    "fused_head": si.Workload("var_fused", 31, 96, [50, 40, 10], [O.ACT_RELU, O.ACT_IDENTITY],
                              "kaiming", "uniform001", "f32", si.SGD),
    "xent_17": si.Workload("var_xent", 32, 120, [60, 40, 17], [O.ACT_RELU, O.ACT_IDENTITY],
                           "kaiming", "uniform001", "f32", si.SGD),
    "split_k": si.Workload("var_split", 33, 2048, [784, 256, 10], [O.ACT_RELU, O.ACT_IDENTITY],
                           "kaiming", "uniform001", "f32", si.SGD),
    # the tail's narrow-batch form, finishing the split-K forward of layer 1
    "narrow_tail": si.Workload("var_narrow", 34, 64, [784, 256, 128, 10],
                               [O.ACT_RELU, O.ACT_RELU, O.ACT_IDENTITY], "kaiming", "uniform001",
                               "f32", si.SGD),
}


def _mlp(dl, inp, w, adam, ema):
    return dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                  adamw=adam, ema=ema)


def _gpu_variant_step(dl, mlp, Xd, yd, opt, t, device_step, scaler=None, grad_norm=None):
    return dl.mlp_train_step(mlp, Xd, yd, _kind(dl, opt.kind), lr=opt.lr,
                             weight_decay=opt.weight_decay, step=t, device_step=device_step,
                             max_grad_norm=opt.max_grad_norm, ema_decay=opt.ema_decay or 0.0,
                             schedule=_dl_sched(dl, opt.schedule), scaler=scaler,
                             grad_norm=grad_norm)


VARIANTS = {
    "sgd_clip": dict(opt=_Opt("sgd", lr=0.05, max_grad_norm=0.2)),
    "sgd_ema": dict(opt=_Opt("sgd", lr=0.05, ema_decay=0.7)),
    "sgd_cosine_device": dict(opt=_Opt("sgd", lr=0.1,
                                       schedule=_Sched(O.LR_WARMUP_COSINE, 1, 3, 0.01)), dev=True),
    "sgd_step_host": dict(opt=_Opt("sgd", lr=0.1, schedule=_Sched(O.LR_STEP, step_size=1,
                                                                  gamma=0.5))),
    "sgd_scaled_clip": dict(opt=_Opt("sgd", lr=0.05, max_grad_norm=0.3), scale=2.0 ** 12,
                            dev=True),
}


@pytest.mark.parametrize("work", sorted(VARIANT_WORKLOADS))
@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_mlp_step_variant_matches_oracle(dl, work, variant):
    """Three steps; before each, the GPU takes the oracle's state and both
    run one step, compared element by element."""
    v = VARIANTS[variant]
    w = VARIANT_WORKLOADS[work]
    opt = v["opt"]
    inp = si.generate(w)
    ema = opt.ema_decay is not None
    mlp = _mlp(dl, inp, w, False, ema)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    st = O.MLPState(inp.W, inp.b)
    if ema:
        st.enable_ema()
    norm = torch.zeros(1, device=device())
    for t in range(1, 4):
        _load_state(mlp, st)
        if ema:
            for l in range(mlp.L):
                mlp.eW[l].copy_(torch.from_numpy(st.eW[l].astype(np.float32)))
                mlp.eb[l].copy_(torch.from_numpy(st.eb[l].astype(np.float32)))
        mlp.step_dev.fill_(t - 1)
        scaler = osc = None
        if "scale" in v:
            scaler = dl.LossScaler(device(), init_scale=v["scale"], growth_interval=1000)
            osc = O.LossScaler(scale=v["scale"], growth_interval=1000)
        masks, _ = _adopted_masks(_gpu_relu_masks(dl, inp.X, st.W, st.b, w.acts), st, inp.X,
                                  w.acts)
        ref = O.mlp_train_step(st, inp.X, inp.labels, w.acts, opt, relu_masks=masks,
                               scaler=osc)
        loss = float(_gpu_variant_step(dl, mlp, Xd, yd, opt, t, v.get("dev", False), scaler,
                                       norm).item())
        assert abs(loss - ref["loss"]) <= LOSS_TOL * abs(ref["loss"])
        assert not ref["skipped"]
        if opt.max_grad_norm > 0 or scaler is not None:
            assert abs(norm.item() - ref["norm"]) <= 1e-5 * ref["norm"]
        for l in range(mlp.L):
            assert_close(to_np(mlp.dW[l]), ref["dW"][l], F32_TOL, f"step {t} dW{l}")
            assert_close(to_np(mlp.db[l]), ref["db"][l], F32_TOL, f"step {t} db{l}")
            assert_close(to_np(mlp.W[l]), st.W[l], F32_TOL, f"step {t} W{l}")
            assert_close(to_np(mlp.b[l]), st.b[l], F32_TOL, f"step {t} b{l}")
            if ema:
                assert_close(to_np(mlp.eW[l]), st.eW[l], F32_TOL, f"step {t} eW{l}")
                assert_close(to_np(mlp.eb[l]), st.eb[l], F32_TOL, f"step {t} eb{l}")
        if v.get("dev"):
            assert mlp.step_dev.item() == t


def _adam_spread(w0, g, dg, m0, v0, o, t):
    args = (o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, t)
    c = O.adam_step(w0, g, m0, v0, *args)
    p = O.adam_step(w0, g + dg, m0, v0, *args)
    m = O.adam_step(w0, g - dg, m0, v0, *args)
    return [np.maximum(np.abs(pi - ci), np.abs(mi - ci)) for ci, pi, mi in zip(c, p, m)]


@pytest.mark.parametrize("work", ["fused_head", "split_k"])
def test_mlp_step_adam_matches_oracle(dl, work):
    w = VARIANT_WORKLOADS[work]
    opt = _Opt("adam", lr=1e-3, wd=0.01)
    inp = si.generate(w)
    mlp = _mlp(dl, inp, w, True, False)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    st = O.MLPState(inp.W, inp.b)
    for t in range(1, 4):
        _load_state(mlp, st)
        masks, _ = _adopted_masks(_gpu_relu_masks(dl, inp.X, st.W, st.b, w.acts), st, inp.X,
                                  w.acts)
        before = _copy_state(st)
        ref = O.mlp_train_step(st, inp.X, inp.labels, w.acts, opt, relu_masks=masks)
        loss = float(_gpu_variant_step(dl, mlp, Xd, yd, opt, t, False).item())
        assert abs(loss - ref["loss"]) <= LOSS_TOL * abs(ref["loss"])
        bands_w, bands_b = _grad_bands(ref, before, inp.X, w.acts, masks, labels=inp.labels)
        for l in range(mlp.L):
            dgW, dgb = bands_w[l], bands_b[l]
            for got, want, w0, g, dg, m0, v0 in (
                    (mlp.W[l], st.W[l], before.W[l], ref["dW"][l], dgW, before.mW[l],
                     before.vW[l]),
                    (mlp.b[l], st.b[l], before.b[l], ref["db"][l], dgb, before.mb[l],
                     before.vb[l])):
                bw, _, _ = _adam_spread(w0, g, dg, m0, v0, opt, t)
                _assert_close_band(to_np(got), want, bw, F32_TOL, f"step {t} layer {l}")


@pytest.mark.parametrize("work", sorted(VARIANT_WORKLOADS))
def test_mlp_power_of_two_loss_scale_is_exact(dl, work):
    """With S = 2^k every scaled gradient is exactly S times the one formed
    with S = 1, so the update is bit-identical, and dW holds exactly S times
    the S = 1 dW."""
    w = VARIANT_WORKLOADS[work]
    inp = si.generate(w)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    a = _mlp(dl, inp, w, True, True)
    b = _mlp(dl, inp, w, True, True)
    one = dl.LossScaler(device(), init_scale=1.0, growth_interval=1000)
    sc = dl.LossScaler(device(), init_scale=2.0 ** 14, growth_interval=1000)
    for t in range(1, 4):
        dl.mlp_train_step(a, Xd, yd, dl.OPT_ADAMW, lr=1e-3, weight_decay=0.01, device_step=True,
                          ema_decay=0.9, scaler=one)
        dl.mlp_train_step(b, Xd, yd, dl.OPT_ADAMW, lr=1e-3, weight_decay=0.01, device_step=True,
                          ema_decay=0.9, scaler=sc)
        assert torch.equal(a.loss, b.loss)
    for l in range(a.L):
        assert torch.equal(b.dW[l], a.dW[l] * 2.0 ** 14)
        for x, y in ((a.W, b.W), (a.b, b.b), (a.mW, b.mW), (a.vW, b.vW), (a.eW, b.eW)):
            assert torch.equal(x[l], y[l])
    assert sc.found_inf.item() == 0 and b.step_dev.item() == 3


@pytest.mark.parametrize("work", sorted(VARIANT_WORKLOADS))
def test_mlp_non_finite_step_is_skipped(dl, work):
    w = VARIANT_WORKLOADS[work]
    inp = si.generate(w)
    X = inp.X.copy()
    X[3, 5] = np.nan
    Xd, Xbad, yd = to_dev(inp.X), to_dev(X), to_dev(inp.labels)
    mlp = _mlp(dl, inp, w, True, True)
    sc = dl.LossScaler(device(), init_scale=256.0, growth_interval=2)
    dl.mlp_train_step(mlp, Xd, yd, dl.OPT_ADAMW, lr=1e-3, device_step=True, ema_decay=0.9,
                      scaler=sc, max_grad_norm=1.0)
    state = [t.clone() for t in mlp.W + mlp.b + mlp.mW + mlp.vW + mlp.eW + mlp.eb]
    # the NaN input reaches the first layer's dW (ReLU maps a NaN
    # pre-activation to 0 on both sides, so the loss itself may stay finite)
    dl.mlp_train_step(mlp, Xbad, yd, dl.OPT_ADAMW, lr=1e-3, device_step=True, ema_decay=0.9,
                      scaler=sc, max_grad_norm=1.0)
    assert torch.isnan(mlp.dW[0]).any()
    assert sc.found_inf.item() == 1 and sc.scale.item() == 128.0 and sc.growth_tracker.item() == 0
    assert mlp.step_dev.item() == 1
    for a, b in zip(state, mlp.W + mlp.b + mlp.mW + mlp.vW + mlp.eW + mlp.eb):
        assert torch.equal(a, b)
    for _ in range(2):
        dl.mlp_train_step(mlp, Xd, yd, dl.OPT_ADAMW, lr=1e-3, device_step=True, ema_decay=0.9,
                          scaler=sc, max_grad_norm=1.0)
    assert sc.found_inf.item() == 0 and sc.scale.item() == 256.0 and mlp.step_dev.item() == 3


def test_mlp_resume_from_saved_state_is_exact(dl):
    """Four steps straight against two steps, a copy of everything a
    checkpoint holds into fresh buffers, and two more steps: bit-identical."""
    w = VARIANT_WORKLOADS["split_k"]
    inp = si.generate(w)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    kw = dict(lr=1e-3, weight_decay=0.01, device_step=True, ema_decay=0.9, max_grad_norm=1.0,
              schedule=dl.Schedule(dl.LR_WARMUP_COSINE, warmup=1, total=10, min_lr=1e-4))
    straight = _mlp(dl, inp, w, True, True)
    for _ in range(4):
        dl.mlp_train_step(straight, Xd, yd, dl.OPT_ADAMW, **kw)
    first = _mlp(dl, inp, w, True, True)
    for _ in range(2):
        dl.mlp_train_step(first, Xd, yd, dl.OPT_ADAMW, **kw)
    saved = {k: [t.cpu().clone() for t in getattr(first, k)]
             for k in ("W", "b", "mW", "vW", "mb", "vb", "eW", "eb")}
    saved_step = first.step_dev.cpu().clone()
    del first
    resumed = dl.MLP([t.to(device()) for t in saved["W"]], [t.to(device()) for t in saved["b"]],
                     w.acts, w.batch, adamw=True, ema=True)
    for k in ("mW", "vW", "mb", "vb", "eW", "eb"):
        for dst, src in zip(getattr(resumed, k), saved[k]):
            dst.copy_(src)
    resumed.step_dev.copy_(saved_step)
    for _ in range(2):
        dl.mlp_train_step(resumed, Xd, yd, dl.OPT_ADAMW, **kw)
    for k in ("W", "b", "mW", "vW", "mb", "vb", "eW", "eb"):
        for a, b in zip(getattr(resumed, k), getattr(straight, k)):
            assert torch.equal(a, b), k
    assert torch.equal(resumed.loss, straight.loss)


def test_graph_replay_with_clip_scaler_ema_schedule(dl):
    """The step with every option captured once and replayed: each replay
    equals the eager step from the same state, bit for bit."""
    w = VARIANT_WORKLOADS["split_k"]
    inp = si.generate(w)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    kw = dict(lr=1e-3, weight_decay=0.01, ema_decay=0.9, max_grad_norm=0.5,
              schedule=dl.Schedule(dl.LR_WARMUP_LINEAR, warmup=2, total=8, min_lr=1e-5))
    eager = _mlp(dl, inp, w, True, True)
    sc_e = dl.LossScaler(device(), init_scale=1024.0, growth_interval=2)
    graphed = _mlp(dl, inp, w, True, True)
    sc_g = dl.LossScaler(device(), init_scale=1024.0, growth_interval=2)
    dl.mlp_train_step(eager, Xd, yd, dl.OPT_ADAMW, device_step=True, scaler=sc_e, **kw)
    dl.mlp_train_step(graphed, Xd, yd, dl.OPT_ADAMW, device_step=True, scaler=sc_g, **kw)
    g = dl.StepGraph(graphed, Xd, yd, dl.OPT_ADAMW, scaler=sc_g, **kw)
    for _ in range(3):
        g.replay()
        dl.mlp_train_step(eager, Xd, yd, dl.OPT_ADAMW, device_step=True, scaler=sc_e, **kw)
        torch.cuda.synchronize()
        for k in ("W", "b", "mW", "vW", "eW"):
            for a, b in zip(getattr(graphed, k), getattr(eager, k)):
                assert torch.equal(a, b), k
        assert torch.equal(sc_g.scale, sc_e.scale)
        assert graphed.step_dev.item() == eager.step_dev.item()


# ------------------------------------------------------------------ MLP step with MSE

from tests.test_gpu_parity import _adamw_spread  # noqa: E402

MSE_VARIANTS = {
    "sgd": dict(opt=_Opt("sgd", lr=0.05)),
    "sgd_clip_ema_scaled": dict(opt=_Opt("sgd", lr=0.05, max_grad_norm=0.1, ema_decay=0.6),
                                scale=2.0 ** 8, dev=True),
    "adamw": dict(opt=_Opt("adamw", lr=1e-3, wd=0.01)),
}


@pytest.mark.parametrize("work", sorted(VARIANT_WORKLOADS))
@pytest.mark.parametrize("variant", sorted(MSE_VARIANTS))
def test_mlp_step_mse_matches_oracle(dl, work, variant):
    v = MSE_VARIANTS[variant]
    w = VARIANT_WORKLOADS[work]
    opt = v["opt"]
    inp = si.generate(w)
    T = si.random_matrix(990, (w.batch, w.dims[-1]))
    adam = opt.kind != "sgd"
    ema = opt.ema_decay is not None
    mlp = _mlp(dl, inp, w, adam, ema)
    Xd, Td = to_dev(inp.X), to_dev(T)
    st = O.MLPState(inp.W, inp.b)
    if ema:
        st.enable_ema()
    for t in range(1, 4):
        _load_state(mlp, st)
        if ema:
            for l in range(mlp.L):
                mlp.eW[l].copy_(torch.from_numpy(st.eW[l].astype(np.float32)))
                mlp.eb[l].copy_(torch.from_numpy(st.eb[l].astype(np.float32)))
        mlp.step_dev.fill_(t - 1)
        scaler = osc = None
        if "scale" in v:
            scaler = dl.LossScaler(device(), init_scale=v["scale"], growth_interval=1000)
            osc = O.LossScaler(scale=v["scale"], growth_interval=1000)
        masks, _ = _adopted_masks(_gpu_relu_masks(dl, inp.X, st.W, st.b, w.acts), st, inp.X,
                                  w.acts)
        before = _copy_state(st)
        ref = O.mlp_train_step(st, inp.X, None, w.acts, opt, relu_masks=masks, scaler=osc,
                               targets=T)
        loss = float(dl.mlp_train_step_mse(
            mlp, Xd, Td, _kind(dl, opt.kind), lr=opt.lr, weight_decay=opt.weight_decay, step=t,
            device_step=v.get("dev", False), max_grad_norm=opt.max_grad_norm,
            ema_decay=opt.ema_decay or 0.0, scaler=scaler).item())
        assert abs(loss - ref["loss"]) <= LOSS_TOL * abs(ref["loss"])
        for l in range(mlp.L):
            assert_close(to_np(mlp.dW[l]), ref["dW"][l], F32_TOL, f"step {t} dW{l}")
            assert_close(to_np(mlp.db[l]), ref["db"][l], F32_TOL, f"step {t} db{l}")
            if adam:
                dgW = _grad_bands(ref, before, inp.X, w.acts, masks, loss="mse")[0][l]
                bw, _, _ = _adamw_spread(before.W[l], ref["dW"][l], dgW, before.mW[l],
                                         before.vW[l], opt, t)
                _assert_close_band(to_np(mlp.W[l]), st.W[l], bw, F32_TOL, f"step {t} W{l}")
            else:
                assert_close(to_np(mlp.W[l]), st.W[l], F32_TOL, f"step {t} W{l}")
                assert_close(to_np(mlp.b[l]), st.b[l], F32_TOL, f"step {t} b{l}")
            if ema:
                assert_close(to_np(mlp.eW[l]), st.eW[l], F32_TOL, f"step {t} eW{l}")

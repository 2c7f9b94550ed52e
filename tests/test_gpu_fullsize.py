"""Parity at the full workload sizes, with the same entry points, shapes and
therefore the same launch plans as bench.py.

* wide MLP (1024-4096-4096-4096-1000, batch 16384, SGD): one whole training
  step against the full float64 oracle step.
* transformer MLP (1024 -> 4096 GELU -> 1024, 32768 tokens, bf16): the
  forward and both vjps against the full float64 oracle.
* transformer MLP with the oracle chain rounded to bf16 wherever a tensor
  crosses a call boundary (H, Z, Y, the masked gradient dZ1, dX), as the
  bf16 contract of these calls says.
* classifier head (65536 x 768 -> 32000, AdamW at t = 1): 8.4 GB of
  logits, more bytes than a 32-bit offset reaches.  The float64 oracle runs
  the whole batch in blocks of rows (rows are independent; every block is
  scaled by the whole batch): the loss, every row loss, dX, dW and db, and
  the AdamW state after the step are compared in full, the logits and
  dlogits on 4096 seeded rows.
"""
import os
import threading
import time

import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as si
from tests.gpu_util import BF16_TOL, F32_TOL, LOSS_TOL, assert_close, device, to_dev, to_np
from tests.test_gpu_parity import (_adamw_spread, _adopted_masks, _assert_close_band,
                                   _gpu_relu_masks)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dl():
    device()
    import dense_layers_amd
    return dense_layers_amd


def test_mlp_wide_full_batch_sgd_step(dl):
    w = si.WORKLOADS["mlp_wide"]
    inp = si.generate(w)
    mlp = dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                 adamw=False)
    st = O.MLPState(inp.W, inp.b)
    gm = _gpu_relu_masks(dl, inp.X, st.W, st.b, w.acts)
    masks, adopted = _adopted_masks(gm, st, inp.X, w.acts)
    print(f"adopted ReLU decisions within the rounding band: {adopted}")
    W0 = [np.array(a, dtype=np.float64) for a in inp.W]
    b0 = [np.array(a, dtype=np.float64) for a in inp.b]
    loss = float(dl.mlp_train_step(mlp, to_dev(inp.X), to_dev(inp.labels), dl.OPT_SGD,
                                   lr=w.optim.lr, step=1).item())
    ref = O.mlp_train_step(st, inp.X, inp.labels, w.acts, w.optim, relu_masks=masks)
    assert abs(loss - ref["loss"]) <= LOSS_TOL * abs(ref["loss"]), (loss, ref["loss"])
    for l in range(mlp.L):
        assert_close(to_np(mlp.dW[l]), ref["dW"][l], F32_TOL, f"dW{l}")
        assert_close(to_np(mlp.db[l]), ref["db"][l], F32_TOL, f"db{l}")
        assert_close(to_np(mlp.W[l]), st.W[l], F32_TOL, f"W{l}")
        assert_close(to_np(mlp.b[l]), st.b[l], F32_TOL, f"b{l}")
        # the update itself, which a normwise check of W hides under W:
        # both sides round W - lr dW to float32 once (at most one ulp apart)
        # on top of lr times the gradient's own difference
        for name, got, want, p0, g in (("W", mlp.W[l], st.W[l], W0[l], ref["dW"][l]),
                                       ("b", mlp.b[l], st.b[l], b0[l], ref["db"][l])):
            d_gpu = to_np(got).astype(np.float64) - p0
            d_ref = np.asarray(want, dtype=np.float64) - p0
            tol = w.optim.lr * F32_TOL * np.abs(g).max() + 2.0 ** -23 * np.abs(p0).max()
            err = np.abs(d_gpu - d_ref).max()
            print(f"{name}{l} update: max |ref| {np.abs(d_ref).max():.3e}, error {err:.3e}, "
                  f"bound {tol:.3e}")
            assert err <= tol, (name, l, err, tol)


def test_tmlp_bf16_full_tokens(dl):
    w = si.WORKLOADS["tmlp_bf16"]
    inp = si.generate(w)
    bf = torch.bfloat16
    X = to_dev(inp.X, bf)
    dY = to_dev(inp.dY, bf)
    Wm = [to_dev(a) for a in inp.W]
    b = [to_dev(a) for a in inp.b]
    Wb, Wbt = zip(*[dl.dense_cast_bf16_t(a) for a in Wm])
    H, Z = dl.dense_act_fwd(X, Wb[0], b[0], dl.ACT_GELU_TANH, save_z=True)
    Y, _ = dl.dense_act_fwd(H, Wb[1], b[1], dl.ACT_IDENTITY)
    Y_np, H_np = to_np(Y), to_np(H)
    # vjp of layer 2 folds gelu'(Z1) into its dX (in place over Z1)
    dZ, dW2, db2 = dl.dense_act_vjp(dY, None, H, Wb[1], dl.ACT_IDENTITY, dX=Z,
                                    dx_act=dl.ACT_GELU_TANH, dx_saved=Z, Wt=Wbt[1])
    dX, dW1, db1 = dl.dense_act_vjp(dZ, None, X, Wb[0], dl.ACT_IDENTITY, Wt=Wbt[0])
    torch.cuda.synchronize()

    # the oracle chain, each boundary tensor rounded to bf16 (X, dY and the
    # W copies are bf16 already; H, Z and Y leave the forwards in bf16; the
    # second vjp writes dZ1 = (dY W2) * gelu'(Z1) in bf16 with Z1 read from
    # its bf16 copy; dX leaves in bf16)
    r = O.round_bf16
    W1, W2 = r(inp.W[0]), r(inp.W[1])
    _, Z1 = O.dense_act_fwd(inp.X, W1, inp.b[0], O.ACT_GELU_TANH)
    rZ = r(Z1)
    rH = r(O.act_fwd(Z1, O.ACT_GELU_TANH))
    rY = r(O.dense_act_fwd(rH, W2, inp.b[1], O.ACT_IDENTITY)[0])
    assert_close(H_np, rH, BF16_TOL, "H")
    assert_close(Y_np, rY, BF16_TOL, "Y")
    rdH, rdW2, rdb2 = O.dense_act_vjp(inp.dY, None, rH, W2, O.ACT_IDENTITY)
    rdZ = r(rdH * O.act_grad(rZ, O.ACT_GELU_TANH))
    rdX, rdW1, rdb1 = O.dense_act_vjp(rdZ, None, inp.X, W1, O.ACT_IDENTITY)
    assert_close(to_np(dW2), rdW2, BF16_TOL, "dW2")
    assert_close(to_np(db2), rdb2, BF16_TOL, "db2")
    assert_close(to_np(dZ), rdZ, BF16_TOL, "dZ1")
    assert_close(to_np(dW1), rdW1, BF16_TOL, "dW1")
    assert_close(to_np(db1), rdb1, BF16_TOL, "db1")
    assert_close(to_np(dX), r(rdX), BF16_TOL, "dX")


# ------------------------------------------------------------ classifier head

HEAD_SAMPLE_ROWS = 4096


def _head_sample(B):
    rng = np.random.default_rng(5)
    s = np.sort(rng.choice(B, HEAD_SAMPLE_ROWS - 2, replace=False))
    return np.unique(np.concatenate([s, [0, B - 1]]))


HEAD_BLOCK = 512


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def head_ref():
    """One classifier-head step of the float64 oracle at full size: forward,
    softmax-xent and vjp over blocks of rows (each with the whole batch as
    the divisor), then AdamW at t = 1 on W and b.  Also the float32 rounding
    band of dW and db (sums over all 65536 rows), for the update's
    comparison near zero gradients.  Rows are independent, so the blocks are
    shared among threads (thread t takes blocks t, t + T, ...; BLAS on one
    thread each) and the per-thread sums are added in thread order."""
    from threadpoolctl import threadpool_limits
    w = si.WORKLOADS["head_xent"]
    inp = si.generate(w)
    B, d, C = w.batch, w.dims[0], w.dims[1]
    W, b, y = inp.W[0].astype(np.float64), inp.b[0].astype(np.float64), inp.labels
    X = inp.X
    sample = _head_sample(B)
    ref = {"row": np.empty(B), "lse": np.empty(B), "dX": np.empty((B, d)),
           "z_s": np.empty((len(sample), C)), "dz_s": np.empty((len(sample), C))}
    nt = _threads()
    blocks = list(range(0, B, HEAD_BLOCK))
    acc = [None] * nt
    t0 = time.time()

    def work(t):
        dW, db = np.zeros((C, d)), np.zeros(C)
        bw, bb = np.zeros((C, d)), np.zeros(C)
        bwl, bbl = np.zeros((C, d)), np.zeros(C)
        for r0 in blocks[t::nt]:
            r1 = min(B, r0 + HEAD_BLOCK)
            Xc = X[r0:r1].astype(np.float64)
            _, Z = O.dense_act_fwd(Xc, W, b, O.ACT_IDENTITY)
            _, dz, rl = O.softmax_xent_fwd_bwd(Z, y[r0:r1], batch_total=B)
            ref["row"][r0:r1] = rl
            ref["lse"][r0:r1] = O.softmax_lse(Z)
            tau = O.dot_band(Xc, W, b)
            dG = O.xent_grad_band(Z, tau, B, labels=y[r0:r1])
            dGl = O.xent_grad_band(Z, tau, B, labels=y[r0:r1], form="lse")
            del tau
            dXc, dWc, dbc = O.dense_act_vjp(dz, None, Xc, W, O.ACT_IDENTITY)
            ref["dX"][r0:r1] = dXc
            dW += dWc
            db += dbc
            h1 = np.hstack([Xc, np.ones((r1 - r0, 1))])
            band = O.sum_band(dz, h1, dG, n=B)
            bw += band[:, :d]
            bb += band[:, d]
            band = O.sum_band(dz, h1, dGl, n=B)
            bwl += band[:, :d]
            bbl += band[:, d]
            ins = (sample >= r0) & (sample < r1)
            ref["z_s"][ins] = Z[sample[ins] - r0]
            ref["dz_s"][ins] = dz[sample[ins] - r0]
        acc[t] = (dW, db, bw, bb, bwl, bbl)

    with threadpool_limits(limits=1):
        threads = [threading.Thread(target=work, args=(t,)) for t in range(nt)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
    assert all(a is not None for a in acc), "an oracle thread failed"
    for key, i in (("dW", 0), ("db", 1), ("bw", 2), ("bb", 3), ("bw_lse", 4), ("bb_lse", 5)):
        total = acc[0][i].copy()
        for t in range(1, nt):
            total += acc[t][i]
        ref[key] = total
    print(f"oracle of the full head step on {nt} threads: {time.time() - t0:.1f} s", flush=True)
    ref["loss"] = float(ref["row"].sum() / B)
    o = w.optim
    args = (o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, 1)
    for name, p0, g in (("W", W, ref["dW"]), ("b", b, ref["db"])):
        z0 = np.zeros_like(g)
        w1, m1, v1 = O.adamw_step(p0, g, z0, z0, *args)
        ref[name + "1"], ref["m" + name], ref["v" + name] = (O.round_f32(w1), O.round_f32(m1),
                                                            O.round_f32(v1))
    ref["inp"], ref["w"], ref["sample"] = inp, w, sample
    return ref


def _gpu_head_step(dl, ref):
    """The classifier-head step exactly as bench.py runs it (same entry
    points, shapes and launch plans), with the sampled logits and dlogits
    rows gathered on the side.  Returns float64 host arrays."""
    inp, w, sample = ref["inp"], ref["w"], ref["sample"]
    o = w.optim
    B, d, C = w.batch, w.dims[0], w.dims[1]
    X, y = to_dev(inp.X), to_dev(inp.labels)
    W, b = to_dev(inp.W[0]), to_dev(inp.b[0])
    srows = torch.from_numpy(sample).to(device())
    logits, _ = dl.dense_act_fwd(X, W, b, dl.ACT_IDENTITY)
    z_s = logits[srows].cpu()
    row = torch.empty(B, device=device())
    loss, dz = dl.softmax_xent_fwd_bwd(logits, y, inplace=True, row_loss=row)
    dz_s = dz[srows].cpu()
    dX, dW, db = dl.dense_act_vjp(dz, None, X, W, dl.ACT_IDENTITY)
    del logits, dz
    mW, vW = torch.zeros_like(W), torch.zeros_like(W)
    mb, vb = torch.zeros_like(b), torch.zeros_like(b)
    dl.adamw_step(W, dW, mW, vW, o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, 1)
    dl.adamw_step(b, db, mb, vb, o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, 1)
    torch.cuda.synchronize()
    out = {"loss": float(loss.item()), "row": to_np(row), "dX": to_np(dX), "dW": to_np(dW),
           "db": to_np(db), "W1": to_np(W), "mW": to_np(mW), "vW": to_np(vW), "b1": to_np(b),
           "mb": to_np(mb), "vb": to_np(vb), "z_s": z_s.double().numpy(),
           "dz_s": dz_s.double().numpy()}
    return out


def _check_head(got, ref, what, band_keys=("bw", "bb")):
    inp, w = ref["inp"], ref["w"]
    o = w.optim
    assert abs(got["loss"] - ref["loss"]) <= LOSS_TOL * abs(ref["loss"]), \
        (what, got["loss"], ref["loss"])
    assert_close(got["row"], ref["row"], F32_TOL, f"{what}: row losses")
    if "z_s" in got:
        assert_close(got["z_s"], ref["z_s"], F32_TOL, f"{what}: sampled logits rows")
    if "dz_s" in got:
        assert_close(got["dz_s"], ref["dz_s"], F32_TOL, f"{what}: sampled dlogits rows")
    if "lse" in got:
        assert_close(got["lse"], ref["lse"], F32_TOL, f"{what}: lse")
    assert_close(got["dX"], ref["dX"], F32_TOL, f"{what}: dX")
    assert_close(got["dW"], ref["dW"], F32_TOL, f"{what}: dW")
    assert_close(got["db"], ref["db"], F32_TOL, f"{what}: db")
    for name, p0, g, band in (("W", inp.W[0], ref["dW"], ref[band_keys[0]]),
                              ("b", inp.b[0], ref["db"], ref[band_keys[1]])):
        z0 = np.zeros_like(g)
        bw, bm, bv = _adamw_spread(p0.astype(np.float64), g, band, z0, z0, o, 1)
        n = _assert_close_band(got[name + "1"], ref[name + "1"], bw, F32_TOL,
                               f"{what}: {name} after AdamW")
        _assert_close_band(got["m" + name], ref["m" + name], bm, F32_TOL, f"{what}: m{name}")
        _assert_close_band(got["v" + name], ref["v" + name], bv, F32_TOL, f"{what}: v{name}")
        print(f"{what}: {name} updates inside the band of an ill-conditioned gradient: "
              f"{n} of {g.size}")


@pytest.mark.timeout(1200)
def test_head_xent_full_size_composed(dl, head_ref):
    assert head_ref["w"].batch * head_ref["w"].dims[1] * 4 > 2 ** 32
    _check_head(_gpu_head_step(dl, head_ref), head_ref, "composed head")


def _gpu_head_step_fused(dl, ref):
    """The classifier-head step through the fused head (dense_xent_fwd /
    dense_xent_vjp), as bench.py runs it by default."""
    inp, w, sample = ref["inp"], ref["w"], ref["sample"]
    o = w.optim
    B = w.batch
    X, y = to_dev(inp.X), to_dev(inp.labels)
    W, b = to_dev(inp.W[0]), to_dev(inp.b[0])
    srows = torch.from_numpy(sample).to(device())
    row = torch.empty(B, device=device())
    loss, logits, lse = dl.dense_xent_fwd(X, W, b, y, row_loss=row)
    z_s = logits[srows].cpu()
    dX, dW, db = dl.dense_xent_vjp(logits, lse, y, X, W)
    del logits
    mW, vW = torch.zeros_like(W), torch.zeros_like(W)
    mb, vb = torch.zeros_like(b), torch.zeros_like(b)
    dl.adamw_step(W, dW, mW, vW, o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, 1)
    dl.adamw_step(b, db, mb, vb, o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, 1)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "row": to_np(row), "lse": to_np(lse), "dX": to_np(dX),
            "dW": to_np(dW), "db": to_np(db), "W1": to_np(W), "mW": to_np(mW), "vW": to_np(vW),
            "b1": to_np(b), "mb": to_np(mb), "vb": to_np(vb), "z_s": z_s.double().numpy()}


@pytest.mark.timeout(1200)
def test_head_xent_full_size_fused(dl, head_ref):
    _check_head(_gpu_head_step_fused(dl, head_ref), head_ref, "fused head", ("bw_lse", "bb_lse"))

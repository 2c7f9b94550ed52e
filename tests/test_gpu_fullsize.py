"""Parity at the full workload sizes, with the same entry points, shapes and
therefore the same launch plans as bench.py.

* wide MLP (1024-4096-4096-4096-1000, batch 16384, SGD): one whole training
  step against the full float64 oracle step.
* transformer MLP (1024 -> 4096 GELU -> 1024, 32768 tokens, bf16): the
  forward and both vjps against the full float64 oracle.
* classifier head (65536 x 768 -> 32000): 8.4 GB of logits, more bytes than
  a 32-bit offset reaches.  The oracle checks sampled rows one by one
  (row losses, dlogits rows, dX rows); dW and db are checked through
  properties that hold at any size, evaluated in float64 from the GPU's own
  dlogits: dW v = dlogits^T (X v) for random v, and db = column sums of
  dlogits.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as si
from tests.gpu_util import BF16_TOL, F32_TOL, LOSS_TOL, assert_close, device, to_dev, to_np
from tests.test_gpu_parity import _adopted_masks, _gpu_relu_masks

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
    loss = float(dl.mlp_train_step(mlp, to_dev(inp.X), to_dev(inp.labels), dl.OPT_SGD,
                                   lr=w.optim.lr, step=1).item())
    ref = O.mlp_train_step(st, inp.X, inp.labels, w.acts, w.optim, relu_masks=masks)
    assert abs(loss - ref["loss"]) <= LOSS_TOL * abs(ref["loss"]), (loss, ref["loss"])
    for l in range(mlp.L):
        assert_close(to_np(mlp.dW[l]), ref["dW"][l], F32_TOL, f"dW{l}")
        assert_close(to_np(mlp.db[l]), ref["db"][l], F32_TOL, f"db{l}")
        assert_close(to_np(mlp.W[l]), st.W[l], F32_TOL, f"W{l}")
        assert_close(to_np(mlp.b[l]), st.b[l], F32_TOL, f"b{l}")


def test_tmlp_bf16_full_tokens(dl):
    w = si.WORKLOADS["tmlp_bf16"]
    inp = si.generate(w)
    bf = torch.bfloat16
    T, d, f = w.batch, w.dims[0], w.dims[1]
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

    W1, W2 = O.round_bf16(inp.W[0]), O.round_bf16(inp.W[1])
    rH, rZ = O.dense_act_fwd(inp.X, W1, inp.b[0], O.ACT_GELU_TANH)
    rY, _ = O.dense_act_fwd(rH, W2, inp.b[1], O.ACT_IDENTITY)
    assert_close(H_np, rH, BF16_TOL, "H")
    assert_close(Y_np, rY, BF16_TOL, "Y")
    rdH, rdW2, rdb2 = O.dense_act_vjp(inp.dY, None, rH, W2, O.ACT_IDENTITY)
    rdX, rdW1, rdb1 = O.dense_act_vjp(rdH, rZ, inp.X, W1, O.ACT_GELU_TANH)
    assert_close(to_np(dW2), rdW2, BF16_TOL, "dW2")
    assert_close(to_np(db2), rdb2, BF16_TOL, "db2")
    assert_close(to_np(dZ), rdH * O.act_grad(rZ, O.ACT_GELU_TANH), BF16_TOL, "dZ1")
    assert_close(to_np(dW1), rdW1, BF16_TOL, "dW1")
    assert_close(to_np(db1), rdb1, BF16_TOL, "db1")
    assert_close(to_np(dX), rdX, BF16_TOL, "dX")


def test_head_xent_full_rows(dl):
    w = si.WORKLOADS["head_xent"]
    inp = si.generate(w)
    B, d, C = w.batch, w.dims[0], w.dims[1]
    assert B * C * 4 > 2 ** 32
    X, y = to_dev(inp.X), to_dev(inp.labels)
    W, b = to_dev(inp.W[0]), to_dev(inp.b[0])
    logits, _ = dl.dense_act_fwd(X, W, b, dl.ACT_IDENTITY)
    row = torch.empty(B, device=device())
    loss, dz = dl.softmax_xent_fwd_bwd(logits, y, inplace=True, row_loss=row)
    dX, dW, db = dl.dense_act_vjp(dz, None, X, W, dl.ACT_IDENTITY)
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, B, 250), [0, B - 1]]))
    zr, _ = O.dense_act_fwd(inp.X[rows], inp.W[0], inp.b[0], O.ACT_IDENTITY)
    _, _, rrow = O.softmax_xent_fwd_bwd(zr, inp.labels[rows])
    p = np.exp(zr - zr.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    rdz = (p - np.eye(C)[inp.labels[rows]]) / B
    rows_t = torch.from_numpy(rows).to(device())
    assert_close(to_np(row[rows_t]), rrow, F32_TOL, "sampled row losses")
    assert_close(to_np(dz[rows_t]), rdz, F32_TOL, "sampled dlogits rows")
    assert_close(to_np(dX[rows_t]), rdz @ inp.W[0].astype(np.float64), F32_TOL, "sampled dX rows")
    # the mean is the fixed-order mean of the per-row losses
    mean = float(row.double().mean().item())
    assert abs(float(loss.item()) - mean) <= 1e-6 * abs(mean)
    # dW and db against the GPU's own dlogits, in float64 on the device
    v = torch.randn(d, dtype=torch.float64, device=device(), generator=torch.Generator(
        device=device()).manual_seed(7))
    xv = X.double() @ v
    lhs = dW.double() @ v
    rhs = torch.zeros(C, dtype=torch.float64, device=device())
    colsum = torch.zeros(C, dtype=torch.float64, device=device())
    for s in range(0, B, 4096):
        blk = dz[s:s + 4096].double()
        rhs += blk.t() @ xv[s:s + 4096]
        colsum += blk.sum(dim=0)
    assert_close(lhs.cpu().numpy(), rhs.cpu().numpy(), F32_TOL, "dW v")
    assert_close(to_np(db), colsum.cpu().numpy(), F32_TOL, "db")

"""The MLP step's tail kernel (the last hidden layer's forward, the narrow
head's forward + softmax-xent + vjp, and the hidden layer's dX in one pass
over the rows) against the composition it replaces.

The 32-row form runs every product in the same order as level 1, so every
output of a training step (loss, dW, db, W, b, Adam moments, parameter
averages, the loss scale) must be bit-identical at level 2 (tail) and level 1
(head kernel alone, the hidden layer as GEMMs), over shapes with ragged row
tiles, partial 32-column blocks, a hidden layer right after the input (no
dX), a deeper network, one class, and the loss-scale / clipping / EMA options.

A small batch through a 256-wide hidden input with 128 or 256 outputs takes
the narrow form instead (16-row tiles on the 16x16x4 MFMA, which also
finishes a split-K forward of the layer before it): its sums run in another
order, so those shapes are checked against the float64 oracle, as are the
fused step's odd shapes.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as si
from tests.gpu_util import device, to_dev
from tests.test_gpu_parity import _check_one_step

pytestmark = pytest.mark.gpu

R, I = O.ACT_RELU, O.ACT_IDENTITY

# (dims, batch, activations)
SHAPES = {
    "c1_64": ([784, 256, 128, 10], 64, [R, R, I]),
    "c2_8192": ([784, 256, 128, 10], 8192, [R, R, I]),
    "ragged_1000": ([784, 256, 128, 10], 1000, [R, R, I]),
    "narrow_77": ([40, 24, 16, 5], 77, [R, R, I]),
    "partial_blocks_300": ([64, 72, 96, 16], 300, [R, R, I]),
    "identity_hidden_45": ([48, 40, 56, 7], 45, [R, I, I]),
    "two_layers_129": ([256, 40, 3], 129, [R, I]),
    "four_layers_50": ([33, 48, 200, 120, 7], 50, [R, R, R, I]),
    "one_class_40": ([16, 16, 8, 1], 40, [R, R, I]),
    "many_tiles_9000": ([96, 64, 32, 4], 9000, [R, R, I]),
    # fully unrolled kernel forms: 256-wide hidden input, 256 or 128 outputs
    "unrolled_256_256_100": ([64, 256, 256, 10], 100, [R, R, I]),
    "unrolled_no_dx_70": ([256, 128, 10], 70, [R, I]),
    "unrolled_8200": ([784, 256, 128, 10], 8200, [R, R, I]),
    "unrolled_256_256_8300": ([64, 256, 256, 10], 8300, [R, R, I]),
    # narrow form; the first two also fold the split-K forward of layer 1
    "fold_13": ([784, 256, 128, 10], 13, [R, R, I]),
    "fold_100": ([600, 256, 128, 10], 100, [R, R, I]),
    # narrow form at the class-count edges: one class, and 16 over a 256-wide layer
    "narrow_one_class_50": ([64, 256, 128, 1], 50, [R, R, I]),
    "narrow_16_classes_33": ([64, 256, 256, 16], 33, [R, I, I]),
}


def _narrow(name):
    """Whether the step takes the tail's narrow-batch form for this shape."""
    dims, B, _ = SHAPES[name]
    L = len(dims) - 1
    return L >= 2 and dims[L - 2] == 256 and dims[L - 1] in (128, 256) and dims[L] <= 16 \
        and B <= 8192


BIT_SHAPES = sorted(n for n in SHAPES if not _narrow(n))
NARROW_SHAPES = sorted(n for n in SHAPES if _narrow(n))


@pytest.fixture(scope="module")
def dl():
    device()
    import dense_layers_amd
    return dense_layers_amd


def _workload(name, optim):
    dims, B, acts = SHAPES[name]
    return si.Workload(f"tail_{name}", 11, B, dims, acts, "kaiming", "uniform001", "f32", optim)


def _mlp(dl, inp, w, adamw, ema):
    return dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                  adamw=adamw, ema=ema)


OPTS = {
    "sgd": dict(kind="sgd"),
    "adamw": dict(kind="adamw"),
    "adamw_clip_scaler_ema": dict(kind="adamw", clip=0.5, ema=0.9, scaler=True),
}


def _step(dl, mlp, Xd, yd, c, t, scaler):
    kind = dl.OPT_ADAMW if c["kind"] == "adamw" else dl.OPT_SGD
    return dl.mlp_train_step(mlp, Xd, yd, kind, lr=1e-2, weight_decay=0.01, step=t,
                             device_step=scaler is not None, max_grad_norm=c.get("clip", 0.0),
                             ema_decay=c.get("ema", 0.0), scaler=scaler)


def _tensors(mlp, loss, scaler):
    out = [loss]
    for l in range(mlp.L):
        out += [mlp.W[l], mlp.b[l], mlp.dW[l], mlp.db[l]]
        for t in (mlp.mW[l], mlp.vW[l], mlp.mb[l], mlp.vb[l], mlp.eW[l], mlp.eb[l]):
            if t is not None:
                out.append(t)
    if scaler is not None:
        out += [scaler.scale]
    return [t.clone() for t in out]


def test_shape_split():
    assert NARROW_SHAPES == ["c1_64", "c2_8192", "fold_100", "fold_13", "narrow_16_classes_33",
                             "narrow_one_class_50", "ragged_1000", "unrolled_256_256_100",
                             "unrolled_no_dx_70"]


@pytest.mark.parametrize("opt", sorted(OPTS))
@pytest.mark.parametrize("shape", BIT_SHAPES)
def test_tail_bit_identical_to_head_only(dl, shape, opt):
    c = OPTS[opt]
    w = _workload(shape, si.SGD)
    inp = si.generate(w)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    runs = []
    for level in (1, 2):
        prev = dl.set_mlp_fusion(level)
        try:
            mlp = _mlp(dl, inp, w, c["kind"] == "adamw", "ema" in c)
            scaler = (dl.LossScaler(device(), init_scale=2.0 ** 10, growth_interval=2)
                      if c.get("scaler") else None)
            per_step = []
            for t in (1, 2, 3):
                loss = _step(dl, mlp, Xd, yd, c, t, scaler)
                per_step.append(_tensors(mlp, loss, scaler))
            torch.cuda.synchronize()
        finally:
            dl.set_mlp_fusion(prev)
        runs.append(per_step)
    for t, (a, b) in enumerate(zip(*runs), start=1):
        for i, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), f"step {t}, tensor {i}: fused tail differs from head-only"
    assert np.isfinite(float(runs[1][-1][0].item()))


@pytest.mark.parametrize("shape", ["narrow_77", "partial_blocks_300", "two_layers_129",
                                   "four_layers_50", "one_class_40", "identity_hidden_45"]
                         + NARROW_SHAPES)
@pytest.mark.parametrize("optim", ["sgd", "adamw"])
def test_tail_step_matches_oracle(dl, shape, optim):
    o = si.SGD if optim == "sgd" else si.ADAMW
    w = _workload(shape, o)
    inp = si.generate(w)
    mlp = _mlp(dl, inp, w, optim == "adamw", False)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    st = O.MLPState(inp.W, inp.b)
    for t in (1, 2):
        _check_one_step(dl, w, inp, mlp, Xd, yd, st)
        O.mlp_train_step(st, inp.X, inp.labels, w.acts, w.optim)


def test_fusion_level_is_per_thread_setting(dl):
    prev = dl.set_mlp_fusion(1)
    assert dl.set_mlp_fusion(prev) == 1

"""A whole training step captured as a stream graph and replayed
(StepGraph): every replay must leave the parameters, moments and loss
bit-identical to the same step run eagerly, with unrelated eager work and
synchronizations between the replays; and AdamW with the device step count
must match AdamW with the host step count."""
import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as si
from tests.gpu_util import F32_TOL, assert_close, device, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dl():
    device()
    import dense_layers_amd
    return dense_layers_amd


def _mlp(dl, w, inp):
    return dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                  adamw=(w.optim.kind == "adamw"))


def _state(mlp):
    ts = mlp.W + mlp.b + mlp.dW + mlp.db + [mlp.loss]
    if mlp.mW[0] is not None:
        ts += mlp.mW + mlp.vW + mlp.mb + mlp.vb
    return [t.clone() for t in ts]


def _opt(w):
    o = w.optim
    if o.kind == "adamw":
        return dict(lr=o.lr, beta1=o.beta1, beta2=o.beta2, eps=o.eps,
                    weight_decay=o.weight_decay)
    return dict(lr=o.lr)


@pytest.mark.parametrize("name,batch", [("mlp_small", 64), ("mlp_adamw", 512),
                                        ("mlp_wide", 128)])
def test_graph_replays_match_eager_steps(dl, name, batch):
    w = si.WORKLOADS[name].scaled(batch)
    inp = si.generate(w)
    kind = dl.OPT_ADAMW if w.optim.kind == "adamw" else dl.OPT_SGD
    dev_step = kind == dl.OPT_ADAMW
    eager, graphed = _mlp(dl, w, inp), _mlp(dl, w, inp)
    Xe, ye = to_dev(inp.X), to_dev(inp.labels)
    Xg, yg = to_dev(inp.X), to_dev(inp.labels)
    # one eager step on each first (the graph is captured from a warm library)
    dl.mlp_train_step(eager, Xe, ye, kind, device_step=dev_step, **_opt(w))
    dl.mlp_train_step(graphed, Xg, yg, kind, device_step=dev_step, **_opt(w))
    g = dl.StepGraph(graphed, Xg, yg, kind, **_opt(w))
    other = torch.randn(256, 256, device=device())
    for t in range(2, 7):
        g.replay()
        torch.cuda.synchronize()
        dl.mlp_train_step(eager, Xe, ye, kind, device_step=dev_step, **_opt(w))
        other = torch.tanh(other @ other.t().contiguous() * 1e-3)  # unrelated eager work
        torch.cuda.synchronize()
        for a, b in zip(_state(eager), _state(graphed)):
            assert torch.equal(a, b), f"replay {t} differs from the eager step"
    if dev_step:
        assert int(graphed.step_dev.item()) == 6 and int(eager.step_dev.item()) == 6


def test_adamw_device_step_matches_host_step(dl):
    w = si.WORKLOADS["mlp_adamw"].scaled(256)
    inp = si.generate(w)
    a, b = _mlp(dl, w, inp), _mlp(dl, w, inp)
    X, y = to_dev(inp.X), to_dev(inp.labels)
    for t in range(1, 5):
        dl.mlp_train_step(a, X, y, dl.OPT_ADAMW, step=t, **_opt(w))
        dl.mlp_train_step(b, X, y, dl.OPT_ADAMW, device_step=True, **_opt(w))
    torch.cuda.synchronize()
    for l in range(a.L):
        assert_close(to_np(b.W[l]), to_np(a.W[l]).astype(np.float64), F32_TOL, f"W{l}")
        assert_close(to_np(b.mW[l]), to_np(a.mW[l]).astype(np.float64), F32_TOL, f"mW{l}")
        assert_close(to_np(b.vW[l]), to_np(a.vW[l]).astype(np.float64), F32_TOL, f"vW{l}")

"""Host-side checks of the optimizer, loss-scaling and MSE entry points that
need no GPU: the learning-rate schedule (a host function, compared with the
oracle), workspace queries, and argument checks that reject a call before
anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle as O


@pytest.fixture(scope="module")
def dl():
    import dense_layers_amd
    return dense_layers_amd


FAKE = 0x100000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kind,kw", [
    (0, {}),
    (1, dict(step_size=7, gamma=0.3)),
    (2, dict(warmup=5, total=40, min_lr=0.02)),
    (2, dict(warmup=0, total=25, min_lr=0.0)),
    (3, dict(warmup=3, total=17, min_lr=1e-4)),
    (3, dict(warmup=4, total=4, min_lr=0.1)),  # no decay phase: min_lr after warmup
])
def test_host_schedule_matches_oracle(dl, kind, kw):
    s = dl.Schedule(kind, **kw)
    for t in range(1, 60):
        got = s.lr_at(0.5, t)
        ref = O.lr_at(kind, 0.5, t, **kw)
        assert abs(got - ref) <= 1e-15 * abs(ref), (t, got, ref)


def test_host_schedule_rejects(dl):
    assert np.isnan(dl.Schedule(1, step_size=0).lr_at(0.1, 3))
    assert np.isnan(dl.Schedule(9).lr_at(0.1, 3))
    assert np.isnan(dl.Schedule(0).lr_at(0.1, 0))
    assert dl._c["dl_lr_at"](None, 0.25, 7) == 0.25


def test_train_workspace_queries(dl):
    c = dl._c
    ns = (ctypes.c_int64 * 2)(10, 5000)
    n = c["clip_grad_norm_workspace_size"](2, ns)
    assert n > 0 and n % 256 == 0
    assert c["clip_grad_norm_workspace_size"](0, ns) == 0
    ns[0] = 0
    assert c["clip_grad_norm_workspace_size"](2, ns) == 0
    assert dl.mse_loss_workspace_size(64, 10) == 256
    assert dl.mse_loss_workspace_size(0, 10) == 0
    # the MLP step reserves the gradient-control partials
    table = (dl.DLLayer * 1)()
    table[0] = dl.DLLayer(784, 10, 0)
    assert dl.mlp_train_step_workspace_size(64, table) > 64 * 10 * 4


def _param(dl, base, n, adam=True):
    step = n * 4 + 256
    return dl.DLParam(n, base, base + step, base + 2 * step if adam else None,
                      base + 3 * step if adam else None)


def test_optimizer_step_rejects_bad_arguments(dl):
    c = dl._c
    table = (dl.DLParam * 2)(_param(dl, FAKE, 100), _param(dl, FAKE + (1 << 20), 50))
    opt = dl.DLOpt(1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    # missing moments for an Adam kind
    bad = (dl.DLParam * 1)(_param(dl, FAKE, 100, adam=False))
    assert c["optimizer_step"](None, ctypes.byref(opt), 1, bad, None, 0) == 1
    # two params share memory
    both = (dl.DLParam * 2)(_param(dl, FAKE, 100), _param(dl, FAKE + 200, 50))
    assert c["optimizer_step"](None, ctypes.byref(opt), 2, both, None, 0) == 3
    # clipping needs the workspace
    opt.max_grad_norm = 1.0
    assert c["optimizer_step"](None, ctypes.byref(opt), 2, table, None, 0) == 4
    opt.max_grad_norm = 0.0
    # a loss scaler with Adam needs a device step count
    sc = dl.DLLossScaler(FAKE + (1 << 24), FAKE + (1 << 24) + 256, FAKE + (1 << 24) + 512,
                         2.0, 0.5, 100)
    opt.scaler = ctypes.pointer(sc)
    assert c["optimizer_step"](None, ctypes.byref(opt), 2, table, FAKE + (1 << 25), 1 << 20) == 1
    assert "device step count" in c["dl_last_error"]().decode()
    opt.scaler = None
    # bad schedule, bad kind, step 0
    sch = dl.DLLrSchedule(1, 0, 0, 0, 0.0, 0.5)
    opt.schedule = ctypes.pointer(sch)
    assert c["optimizer_step"](None, ctypes.byref(opt), 2, table, None, 0) == 1
    opt.schedule = None
    opt.kind = 7
    assert c["optimizer_step"](None, ctypes.byref(opt), 2, table, None, 0) == 1
    opt.kind, opt.step = 2, 0
    assert c["optimizer_step"](None, ctypes.byref(opt), 2, table, None, 0) == 1
    # EMA decay out of range where an average is present
    opt.step = 1
    opt.ema_decay = 1.5
    table[0].ema = FAKE + (1 << 22)
    assert c["optimizer_step"](None, ctypes.byref(opt), 2, table, None, 0) == 1


def test_other_train_entry_points_reject(dl):
    c = dl._c
    assert c["adam_step"](None, 16, FAKE, FAKE + 64, FAKE + 128, FAKE + 192, 1e-3, 0.9, 0.999,
                          1e-8, 0.0, 0) == 1
    assert c["adam_step"](None, 16, FAKE, FAKE + 64, FAKE + 64, FAKE + 192, 1e-3, 0.9, 0.999,
                          1e-8, 0.0, 1) == 3
    assert c["ema_update"](None, 16, FAKE, FAKE + 32, 0.9) == 3
    assert c["ema_update"](None, 16, FAKE, FAKE + 64, -0.1) == 1
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE + 100)
    ns = (ctypes.c_int64 * 2)(100, 100)
    assert c["clip_grad_norm"](None, 2, ptrs, ns, 1.0, None, FAKE + (1 << 20), 1 << 16) == 3
    ptrs[1] = FAKE + 4096
    assert c["clip_grad_norm"](None, 2, ptrs, ns, 0.0, None, FAKE + (1 << 20), 1 << 16) == 1
    assert c["clip_grad_norm"](None, 2, ptrs, ns, 1.0, None, None, 0) == 4
    # MSE: empty, workspace too small, dpred partly over pred
    assert c["mse_loss_fwd_bwd"](None, 0, 4, FAKE, FAKE + 4096, FAKE + 8192, None, None, 0) == 1
    assert c["mse_loss_fwd_bwd"](None, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, None, None, 0) == 4
    assert c["mse_loss_fwd_bwd"](None, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, FAKE + 4,
                                 FAKE + 16384, 256) == 3


def test_mlp_step_rejects_partial_averages(dl):
    c = dl._c
    table = (dl.DLLayer * 2)()
    table[0] = dl.DLLayer(8, 4, 1, FAKE, FAKE + 256, FAKE + 512, FAKE + 768)
    table[1] = dl.DLLayer(4, 3, 0, FAKE + 1024, FAKE + 1280, FAKE + 1536, FAKE + 1792)
    table[0].eW, table[0].eb = FAKE + 4096, FAKE + 8192
    opt = dl.DLOpt(0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    opt.ema_decay = 0.9
    assert c["mlp_train_step"](None, 2, 2, table, FAKE, FAKE, ctypes.byref(opt), FAKE, FAKE,
                               1 << 20) == 1
    assert "all layers or none" in c["dl_last_error"]().decode()

"""Parity of the half-precision ("mixed") operand path with the float64
oracle, through the C ABI: forward and vjp on both 16-bit GEMM kernels and
every tile they choose, saturation at +-65504 instead of overflow, NaN kept,
and the half working copies bit for bit.  Inputs are drawn half-exact, so the
only roundings are those of the path itself (results within 5e-3 normwise,
about ten half ulps: a result passes at most two half roundings)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as si
from tests.gpu_util import F16_TOL, assert_close, device, to_dev, to_np

pytestmark = pytest.mark.gpu

H = torch.float16
ACTS = [O.ACT_IDENTITY, O.ACT_RELU, O.ACT_GELU_TANH]


@pytest.fixture(scope="module")
def dl():
    device()
    import dense_layers_amd
    return dense_layers_amd


def _m(seed, shape, scale=1.0):
    return si.random_matrix(seed, shape, scale=scale, f16_exact=True)


# (B, in, out): general kernel (K not a multiple of 64), the 128x128 tile, the
# 256x256 tile, ragged edges
SHAPES = [(1, 8, 8), (77, 130, 90), (300, 1024, 512), (1024, 1024, 4096), (513, 4096, 1024),
          (1000, 200, 1000)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("act", ACTS)
def test_dense_fwd_f16(dl, shape, act):
    B, n_in, n_out = shape
    X = _m(900, (B, n_in))
    Wm = si.random_matrix(901, (n_out, n_in), scale=0.02)
    b = si.random_matrix(902, (n_out,), scale=0.01)
    Wh = dl.dense_cast_f16(to_dev(Wm))
    Y, Z = dl.dense_act_fwd(to_dev(X, H), Wh, to_dev(b), act, save_z=True)
    assert Y.dtype == H and Z.dtype == H
    refY, refZ = O.dense_act_fwd(X, O.round_f16_sat(Wm), b, act)
    assert_close(to_np(Z), refZ, F16_TOL, "Z")
    assert_close(to_np(Y), refY, F16_TOL, "Y")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
def test_dense_vjp_f16(dl, shape, act):
    B, n_in, n_out = shape
    X, W = _m(910, (B, n_in)), _m(911, (n_out, n_in), 0.02)
    Z, dY = _m(912, (B, n_out)), _m(913, (B, n_out))
    dX, dW, db = dl.dense_act_vjp(to_dev(dY, H), to_dev(Z, H), to_dev(X, H), to_dev(W, H), act)
    rdX, rdW, rdb = O.dense_act_vjp(dY, Z, X, W, act)
    assert dX.dtype == H and dW.dtype == torch.float32
    assert_close(to_np(dX), rdX, F16_TOL, "dX")
    assert_close(to_np(dW), rdW, F16_TOL, "dW")
    assert_close(to_np(db), rdb, F16_TOL, "db")


@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
@pytest.mark.parametrize("B", [8200, 4104])
def test_f16_large_and_persistent_tiles_fwd(dl, act, B):
    """4104 rows: the 256x256 tile, one workgroup per tile; 8200 rows with
    8200 outputs: the persistent form.  Ragged in M and N."""
    n_in, n_out = 192, 8200 if B == 8200 else 4120
    X, W = _m(920, (B, n_in)), _m(921, (n_out, n_in), 0.05)
    b = si.random_matrix(922, (n_out,), scale=0.01)
    Y, Z = dl.dense_act_fwd(to_dev(X, H), to_dev(W, H), to_dev(b), act, save_z=True)
    refY, refZ = O.dense_act_fwd(X, W, b, act)
    assert_close(to_np(Z), refZ, F16_TOL, "Z")
    assert_close(to_np(Y), refY, F16_TOL, "Y")


@pytest.mark.parametrize("use_wt", [False, True])
def test_f16_large_tile_dx_with_prev_gelu(dl, use_wt):
    B, n_in, n_out = 4104, 4120, 192
    W = _m(930, (n_out, n_in), 0.05)
    Z, dY, Hs = _m(931, (B, n_out)), _m(932, (B, n_out)), _m(933, (B, n_in))
    Wd = to_dev(W, H)
    Wt = Wd.t().contiguous() if use_wt else None
    dX, _, _ = dl.dense_act_vjp(to_dev(dY, H), to_dev(Z, H), None, Wd, O.ACT_GELU_TANH,
                                need_dw=False, Wt=Wt, dx_act=O.ACT_GELU_TANH,
                                dx_saved=to_dev(Hs, H))
    rdX = O.dense_act_vjp(dY, Z, np.zeros((B, n_in)), W, O.ACT_GELU_TANH)[0]
    rdX = rdX * O.act_grad(Hs, O.ACT_GELU_TANH)
    assert_close(to_np(dX), rdX, F16_TOL, "dX")


@pytest.mark.parametrize("shape", [(2048, 1032, 2000), (1024, 1000, 200)])
def test_f16_weight_gradient_tiles(dl, shape):
    """Half weight gradients of two sizes (the register-staged 128x128 tile,
    split along the batch), ragged in both output dimensions."""
    B, n_in, n_out = shape
    X, dY = _m(940, (B, n_in)), _m(941, (B, n_out))
    W = _m(942, (n_out, n_in), 0.05)
    _, dW, db = dl.dense_act_vjp(to_dev(dY, H), None, to_dev(X, H), to_dev(W, H),
                                 O.ACT_IDENTITY, need_dx=False)
    _, rdW, rdb = O.dense_act_vjp(dY, None, X, W, O.ACT_IDENTITY, need_dx=False)
    assert_close(to_np(dW), rdW, F16_TOL, "dW")
    assert_close(to_np(db), rdb, F16_TOL, "db")


@pytest.mark.parametrize("n_in", [64, 60])  # the direct-to-LDS kernel, the general one
@pytest.mark.parametrize("act", ACTS)
def test_f16_outputs_saturate_and_keep_nan(dl, n_in, act):
    """Pre-activations far past the half range come out as +-65504 (never
    inf) in Y and Z, exactly as the oracle's saturating rounding gives; a NaN
    input row stays NaN."""
    B, n_out = 64, 96
    rng = np.random.default_rng(950)
    X = np.where(rng.random((B, n_in)) < 0.5, 256.0, -256.0).astype(np.float32)
    W = np.where(rng.random((n_out, n_in)) < 0.5, 256.0, 1.0).astype(np.float32)
    X[5, 3] = np.nan
    Y, Z = dl.dense_act_fwd(to_dev(X, H), to_dev(W, H), None, act, save_z=True)
    refY, refZ = O.dense_act_fwd(X, W, None, act)
    gy, gz = Y.float().cpu().numpy(), Z.float().cpu().numpy()
    ry, rz = O.round_f16_sat(refY), O.round_f16_sat(refZ)
    assert np.isnan(gz[5]).all() and np.isnan(rz[5]).all()
    keep = np.ones(B, bool)
    keep[5] = False
    assert not np.isinf(gy).any() and not np.isinf(gz).any()
    sat = np.abs(rz[keep]) == 65504.0
    assert sat.mean() > 0.5  # most outputs overflow the half range
    assert np.array_equal(gz[keep][sat], rz[keep][sat])
    sat_y = np.abs(ry[keep]) == 65504.0
    assert np.array_equal(gy[keep][sat_y], ry[keep][sat_y])


CAST_SHAPES = [(1, 1), (63, 130), (1024, 4096), (100, 68), (4, 8)]


@pytest.mark.parametrize("shape", CAST_SHAPES)
def test_cast_f16_bit_exact(dl, shape):
    W = si.random_matrix(960, shape, scale=30000.0)
    flat = W.reshape(-1)
    flat[:: 7] *= 10.0  # some values past the half range
    flat[1:: 97] = np.inf
    flat[2:: 101] = -np.inf
    flat[3:: 89] = np.nan
    ref = O.round_f16_sat(W).astype(np.float16).view(np.uint16)
    d, dt = dl.dense_cast_f16_t(to_dev(W))
    d1 = dl.dense_cast_f16(to_dev(W.reshape(-1)))
    got = d.view(torch.int16).cpu().numpy().view(np.uint16)
    got_t = dt.view(torch.int16).cpu().numpy().view(np.uint16)
    got1 = d1.view(torch.int16).cpu().numpy().view(np.uint16)
    nan = np.isnan(W)
    for g, r, m in ((got, ref, nan), (got_t, ref.T, nan.T), (got1, ref.reshape(-1), nan.reshape(-1))):
        assert np.array_equal(g[~m], r[~m])
        assert np.isnan(g[m].view(np.float16)).all()


# ------------------------------------------------------------------ mixed_safe

@pytest.mark.parametrize("mag", [1e-9, 1e-7, 3e-5, 1.0, 700.0])
def test_cast_f16_scaled_bit_exact(dl, mag):
    a = si.random_matrix(970, (257, 129), scale=mag)
    a.reshape(-1)[5] = np.nan
    a.reshape(-1)[9] = np.inf
    h, sc = dl.dense_cast_f16_scaled(to_dev(a))
    s = O.f16_safe_scale(a)
    assert sc.item() == s
    ref = O.round_f16_sat(a * s).astype(np.float16).view(np.uint16)
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    nan = np.isnan(a)
    assert np.array_equal(got[~nan], ref[~nan]) and np.isnan(got[nan].view(np.float16)).all()


VJP_SCALED_SHAPES = [(77, 130, 90), (1024, 1024, 512), (1024, 1000, 200), (4104, 256, 4120)]


@pytest.mark.parametrize("shape", VJP_SCALED_SHAPES)
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
def test_vjp_scaled_keeps_tiny_cotangents(dl, shape, act):
    """Cotangents of 1e-7 (below the half normal range): through the scaled
    half copy every product keeps half accuracy against the exact vjp; the
    plain half copy loses it."""
    B, n_in, n_out = shape
    X, W, Z = _m(980, (B, n_in)), _m(981, (n_out, n_in), 0.05), _m(982, (B, n_out))
    dY = si.random_matrix(983, (B, n_out), scale=1e-7)
    Xd, Wd, Zd = to_dev(X, H), to_dev(W, H), to_dev(Z, H)
    dYh, sc = dl.dense_cast_f16_scaled(to_dev(dY))
    dX, dW, db = dl.dense_act_vjp(dYh, Zd, Xd, Wd, act, dy_scale=sc)
    exact = O.dense_act_vjp(dY, Z, X, W, act)
    s = O.f16_safe_scale(dY)
    assert sc.item() == s
    # dX keeps the scale (the next gradient operand); dW, db come out unscaled
    assert_close(to_np(dX) / s, exact[0], F16_TOL, "dX / s")
    assert_close(to_np(dW), exact[1], F16_TOL, "dW")
    assert_close(to_np(db), exact[2], F16_TOL, "db")
    # the oracle of the scaled operand itself, to the same bar
    rdX, rdW, rdb = O.dense_act_vjp(O.round_f16_sat(dY * s) / s, Z, X, W, act)
    assert_close(to_np(dW), rdW, F16_TOL, "dW (scaled operand)")
    plain = dl.dense_cast_f16(to_dev(dY))
    pX, _, _ = dl.dense_act_vjp(plain, Zd, Xd, Wd, act)
    from tests.gpu_util import normwise
    assert normwise(to_np(pX), exact[0]) > 0.05


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_vjp_power_of_two_scale_is_exact(dl, dtype):
    """dY times 2^12 with dy_scale = 2^12: dW and db bit for bit the unscaled
    ones, dX bit for bit 2^12 times the unscaled dX (where that is a normal
    number of the dtype), in every dtype (float32
    accumulation, the division before the float32 store, a power of two).
    Half takes the identity activation and a dY with no half subnormal: a
    masked gradient or a cotangent in half's subnormal range unscaled but not
    scaled is where the scaled form is the more accurate one."""
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": H}[dtype]
    act = O.ACT_IDENTITY if dtype == "f16" else O.ACT_GELU_TANH
    for B, n_in, n_out in ((1024, 1000, 200), (1024, 1024, 512)):
        X, W, Z = _m(990, (B, n_in)), _m(991, (n_out, n_in), 0.05), _m(992, (B, n_out))
        dY = _m(993, (B, n_out), 0.01)
        if dtype == "f16":  # every dY a normal half in both runs
            dY = np.where(np.abs(dY) < 2.0 ** -14, np.copysign(2.0 ** -14, dY), dY).astype(np.float32)
        Xd, Wd, Zd = to_dev(X, tdt), to_dev(W, tdt), to_dev(Z, tdt)
        a = dl.dense_act_vjp(to_dev(dY, tdt), Zd, Xd, Wd, act)
        sc = torch.full((1,), 4096.0, device=device())
        b = dl.dense_act_vjp(to_dev(dY * 4096.0, tdt), Zd, Xd, Wd, act, dy_scale=sc)
        # (where the unscaled half dX is subnormal, or rounded up from there
        # to the smallest normal, the scaled one is the more precise;
        # elsewhere the two agree bit for bit)
        normal = a[0].float().abs() > 2.0 ** -14
        assert torch.equal(b[0][normal], (a[0] * 4096.0)[normal])
        assert normal.float().mean() > 0.95
        assert torch.equal(b[1], a[1]) and torch.equal(b[2], a[2])

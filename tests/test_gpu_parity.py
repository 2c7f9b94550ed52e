"""Parity of the HIP path with the float64 oracle, through the C ABI.

Every case draws seeded inputs once, runs the GPU kernels and the oracle on
the same values, and compares element by element: float32 results within a
normwise relative error of 1e-4, the loss within 1e-5 relative, bf16-operand
results within 2e-2, integer and bit-level results exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as si
from tests.gpu_util import (BF16_TOL, F32_TOL, LOSS_TOL, assert_close, device, misaligned, normwise,
                            to_dev, to_np)

pytestmark = pytest.mark.gpu

ACTS = [O.ACT_IDENTITY, O.ACT_RELU, O.ACT_GELU_TANH]


@pytest.fixture(scope="module")
def dl():
    device()
    import dense_layers_amd
    return dense_layers_amd


def _layer(seed, B, n_in, n_out, bias=True):
    X = si.random_matrix(seed, (B, n_in))
    W = si.random_matrix(seed + 1, (n_out, n_in), scale=1.0 / math.sqrt(n_in))
    b = si.random_matrix(seed + 2, (n_out,), scale=0.1) if bias else None
    return X, W, b


# ------------------------------------------------------------------ forward

# (the last two: 576 tiles of 128 x 256, ragged in K and N, so the forward
# runs on the 8-wave tile; with N = 2101 its rows take the bounds-checked
# stores)
FWD_SHAPES = [(1, 1, 1), (7, 10, 33), (129, 127, 65), (64, 784, 256), (300, 1000, 129),
              (513, 256, 1000), (256, 1024, 4096), (8192, 128, 10), (33, 4100, 70),
              (8200, 300, 250), (8192, 100, 2100), (8192, 100, 2101)]


@pytest.mark.parametrize("shape", FWD_SHAPES)
@pytest.mark.parametrize("act", ACTS)
def test_dense_fwd_f32(dl, shape, act):
    B, n_in, n_out = shape
    X, W, b = _layer(10, B, n_in, n_out, bias=(B % 2 == 1))
    Y, Z = dl.dense_act_fwd(to_dev(X), to_dev(W), None if b is None else to_dev(b), act,
                            save_z=True)
    refY, refZ = O.dense_act_fwd(X, W, b, act)
    assert_close(to_np(Z), refZ, F32_TOL, "Z")
    assert_close(to_np(Y), refY, F32_TOL, "Y")


def test_dense_fwd_f32_misaligned_operands(dl):
    B, n_in, n_out = 97, 64, 80
    X, W, b = _layer(11, B, n_in, n_out)
    Xd, Wd = misaligned(to_dev(X)), misaligned(to_dev(W))
    Y, _ = dl.dense_act_fwd(Xd, Wd, to_dev(b), O.ACT_RELU)
    assert_close(to_np(Y), O.dense_act_fwd(X, W, b, O.ACT_RELU)[0], F32_TOL, "Y")


def test_dense_fwd_is_bit_reproducible(dl):
    X, W, b = _layer(12, 1000, 512, 300)
    a = dl.dense_act_fwd(to_dev(X), to_dev(W), to_dev(b), O.ACT_GELU_TANH)[0]
    c = dl.dense_act_fwd(to_dev(X), to_dev(W), to_dev(b), O.ACT_GELU_TANH)[0]
    assert torch.equal(a, c)


def test_dense_fwd_on_side_stream(dl):
    X, W, b = _layer(13, 300, 200, 100)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Xd, Wd, bd = to_dev(X), to_dev(W), to_dev(b)
        Y, _ = dl.dense_act_fwd(Xd, Wd, bd, O.ACT_RELU)
    s.synchronize()
    assert_close(to_np(Y), O.dense_act_fwd(X, W, b, O.ACT_RELU)[0], F32_TOL, "Y")


# ------------------------------------------------------------------ vjp

# (the last two: a dX of 576 tiles of 128 x 256, ragged in K and N, on the
# 8-wave tile; with in = 2101 its weight operand takes the bounds-checked
# loads)
VJP_SHAPES = [(1, 1, 1), (7, 10, 33), (129, 127, 65), (64, 784, 256), (8192, 784, 256),
              (8192, 128, 10), (1000, 300, 513), (4096, 1024, 1000), (700, 1000, 300),
              (2000, 1000, 1000), (8200, 250, 300), (8192, 2100, 100), (8192, 2101, 100)]


@pytest.mark.parametrize("shape", VJP_SHAPES)
@pytest.mark.parametrize("act", ACTS)
def test_dense_vjp_f32(dl, shape, act):
    B, n_in, n_out = shape
    X, W, b = _layer(20, B, n_in, n_out)
    Z = O.round_f32(O.dense_act_fwd(X, W, b, O.ACT_IDENTITY)[1]).astype(np.float32)
    dY = si.random_matrix(23, (B, n_out), scale=1e-2)
    dX, dW, db = dl.dense_act_vjp(to_dev(dY), to_dev(Z), to_dev(X), to_dev(W), act)
    rdX, rdW, rdb = O.dense_act_vjp(dY, Z, X, W, act)
    assert_close(to_np(dX), rdX, F32_TOL, "dX")
    assert_close(to_np(dW), rdW, F32_TOL, "dW")
    assert_close(to_np(db), rdb, F32_TOL, "db")


@pytest.mark.parametrize("shape", [(777, 300, 129), (8192, 2100, 100)])
@pytest.mark.parametrize("dx_act", [O.ACT_RELU, O.ACT_GELU_TANH])
def test_dense_vjp_folds_previous_activation(dl, dx_act, shape):
    """dX epilogue multiplies by the previous layer's act'(saved), in place
    (also on the 8-wave 128 x 256 tile)."""
    B, n_in, n_out = shape
    X, W, b = _layer(30, B, n_in, n_out)
    Zprev = si.random_matrix(31, (B, n_in))
    dY = si.random_matrix(32, (B, n_out))
    Zp = to_dev(Zprev)
    dX, dW, db = dl.dense_act_vjp(to_dev(dY), None, to_dev(X), to_dev(W), O.ACT_IDENTITY,
                                  dX=Zp, dx_act=dx_act, dx_saved=Zp)
    rdX, rdW, rdb = O.dense_act_vjp(dY, None, X, W, O.ACT_IDENTITY)
    assert dX.data_ptr() == Zp.data_ptr()
    assert_close(to_np(dX), rdX * O.act_grad(Zprev, dx_act), F32_TOL, "folded dX")
    assert_close(to_np(dW), rdW, F32_TOL, "dW")
    assert_close(to_np(db), rdb, F32_TOL, "db")


def test_dense_vjp_skips_outputs(dl):
    B, n_in, n_out = 100, 50, 40
    X, W, b = _layer(40, B, n_in, n_out)
    dY = si.random_matrix(41, (B, n_out))
    dX, dW, db = dl.dense_act_vjp(to_dev(dY), None, to_dev(X), to_dev(W), O.ACT_IDENTITY,
                                  need_dx=False)
    assert dX is None
    rdX, rdW, rdb = O.dense_act_vjp(dY, None, X, W, O.ACT_IDENTITY)
    assert_close(to_np(dW), rdW, F32_TOL, "dW")
    dX, dW, db = dl.dense_act_vjp(to_dev(dY), None, None, to_dev(W), O.ACT_IDENTITY,
                                  need_dw=False)
    assert dW is None and db is None
    assert_close(to_np(dX), rdX, F32_TOL, "dX")


def test_dense_vjp_is_bit_reproducible(dl):
    B, n_in, n_out = 8192, 784, 256   # split-K path
    X, W, b = _layer(50, B, n_in, n_out)
    dY = si.random_matrix(51, (B, n_out))
    args = (to_dev(dY), None, to_dev(X), to_dev(W), O.ACT_IDENTITY)
    r1 = dl.dense_act_vjp(*args)
    r2 = dl.dense_act_vjp(*args)
    for a, c in zip(r1, r2):
        assert torch.equal(a, c)


# ------------------------------------------------------------------ bf16

BF16_SHAPES = [(1, 8, 8), (77, 130, 90), (300, 1024, 512), (1024, 1024, 4096), (513, 4096, 1024),
               (300, 1000, 1000), (1000, 200, 1000)]


@pytest.mark.parametrize("shape", BF16_SHAPES)
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
def test_dense_fwd_bf16(dl, shape, act):
    B, n_in, n_out = shape
    X = si.random_matrix(60, (B, n_in), bf16_exact=True)
    Wm = si.random_matrix(61, (n_out, n_in), scale=0.02)
    b = si.random_matrix(62, (n_out,), scale=0.01)
    Wb = dl.dense_cast_bf16(to_dev(Wm))
    Y, Z = dl.dense_act_fwd(to_dev(X, torch.bfloat16), Wb, to_dev(b), act, save_z=True)
    Wr = O.round_bf16(Wm)
    refY, refZ = O.dense_act_fwd(X, Wr, b, act)
    assert_close(to_np(Z), refZ, BF16_TOL, "Z")
    assert_close(to_np(Y), refY, BF16_TOL, "Y")


@pytest.mark.parametrize("shape", BF16_SHAPES)
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
def test_dense_vjp_bf16(dl, shape, act):
    B, n_in, n_out = shape
    X = si.random_matrix(70, (B, n_in), bf16_exact=True)
    W = si.random_matrix(71, (n_out, n_in), scale=0.02, bf16_exact=True)
    Z = si.random_matrix(72, (B, n_out), bf16_exact=True)
    dY = si.random_matrix(73, (B, n_out), bf16_exact=True)
    bf = torch.bfloat16
    dX, dW, db = dl.dense_act_vjp(to_dev(dY, bf), to_dev(Z, bf), to_dev(X, bf), to_dev(W, bf),
                                  act)
    rdX, rdW, rdb = O.dense_act_vjp(dY, Z, X, W, act)
    assert dX.dtype == bf and dW.dtype == torch.float32
    assert_close(to_np(dX), rdX, BF16_TOL, "dX")
    assert_close(to_np(dW), rdW, BF16_TOL, "dW")
    assert_close(to_np(db), rdb, BF16_TOL, "db")


# Shapes that reach the direct-to-LDS bf16 kernel's 256x256 tile (at least
# 256 such tiles, K a multiple of 64) with ragged M and N, and its 128x128
# tile on a ragged, split-K weight gradient.
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
def test_bf16_large_tile_fwd_ragged(dl, act):
    B, n_in, n_out = 4104, 192, 4120
    X = si.random_matrix(230, (B, n_in), bf16_exact=True)
    W = si.random_matrix(231, (n_out, n_in), scale=0.05, bf16_exact=True)
    b = si.random_matrix(232, (n_out,), scale=0.01)
    bf = torch.bfloat16
    Y, Z = dl.dense_act_fwd(to_dev(X, bf), to_dev(W, bf), to_dev(b), act, save_z=True)
    refY, refZ = O.dense_act_fwd(X, W, b, act)
    assert_close(to_np(Z), refZ, BF16_TOL, "Z")
    assert_close(to_np(Y), refY, BF16_TOL, "Y")


@pytest.mark.parametrize("use_wt", [False, True])
def test_bf16_large_tile_dx_ragged(dl, use_wt):
    B, n_in, n_out = 4104, 4120, 192
    X = si.random_matrix(240, (B, n_in), bf16_exact=True)
    W = si.random_matrix(241, (n_out, n_in), scale=0.05, bf16_exact=True)
    Z = si.random_matrix(242, (B, n_out), bf16_exact=True)
    dY = si.random_matrix(243, (B, n_out), bf16_exact=True)
    bf = torch.bfloat16
    Wd = to_dev(W, bf)
    Wt = Wd.t().contiguous() if use_wt else None
    dX, _, _ = dl.dense_act_vjp(to_dev(dY, bf), to_dev(Z, bf), None, Wd, O.ACT_GELU_TANH,
                                need_dw=False, Wt=Wt)
    rdX, _, _ = O.dense_act_vjp(dY, Z, X, W, O.ACT_GELU_TANH, need_dx=True)
    assert_close(to_np(dX), rdX, BF16_TOL, "dX")


# At least four 256x256 tiles per CU: the tile runs persistent (each
# workgroup walks several tiles with one pipeline), ragged in M and N.
# 8200 x 8200: 1089 tiles (items taken in plain order); 8192 x 8200: 1056
# tiles (items taken in the XCD-grouped band order).
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
@pytest.mark.parametrize("B", [8200, 8192])
def test_bf16_persistent_fwd_ragged(dl, act, B):
    n_in, n_out = 64, 8200
    X = si.random_matrix(260, (B, n_in), bf16_exact=True)
    W = si.random_matrix(261, (n_out, n_in), scale=0.1, bf16_exact=True)
    b = si.random_matrix(262, (n_out,), scale=0.01)
    bf = torch.bfloat16
    save_z = act != O.ACT_IDENTITY
    Y, Z = dl.dense_act_fwd(to_dev(X, bf), to_dev(W, bf), to_dev(b), act, save_z=save_z)
    refY, refZ = O.dense_act_fwd(X, W, b, act)
    if save_z:
        assert_close(to_np(Z), refZ, BF16_TOL, "Z")
    assert_close(to_np(Y), refY, BF16_TOL, "Y")


def test_bf16_persistent_dx_ragged(dl):
    B, n_in, n_out = 8200, 8200, 64
    X = si.random_matrix(270, (B, n_in), bf16_exact=True)
    W = si.random_matrix(271, (n_out, n_in), scale=0.1, bf16_exact=True)
    Z = si.random_matrix(272, (B, n_out), bf16_exact=True)
    dY = si.random_matrix(273, (B, n_out), bf16_exact=True)
    H = si.random_matrix(274, (B, n_in), bf16_exact=True)
    bf = torch.bfloat16
    # dX of this layer with the previous layer's GELU derivative folded in
    dX, _, _ = dl.dense_act_vjp(to_dev(dY, bf), to_dev(Z, bf), None, to_dev(W, bf),
                                O.ACT_GELU_TANH, need_dw=False, dx_act=O.ACT_GELU_TANH,
                                dx_saved=to_dev(H, bf))
    rdX, _, _ = O.dense_act_vjp(dY, Z, X, W, O.ACT_GELU_TANH, need_dx=True)
    rdX = rdX * O.act_grad(H, O.ACT_GELU_TANH)
    assert_close(to_np(dX), rdX, BF16_TOL, "dX")


# Output rows whose length is not a multiple of 4: no row allows 16-byte
# access, so every wave of the direct-load epilogue takes its per-element
# path for the stores, the bias and the saved activations.  4104 x 4106:
# 289 tiles of 256 x 256 (one workgroup each); 8200 x 8202: 1089 tiles
# (persistent).
@pytest.mark.parametrize("B, n_out", [(4104, 4106), (8200, 8202)])
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_GELU_TANH])
def test_bf16_fwd_unaligned_rows(dl, act, B, n_out):
    n_in = 64
    X = si.random_matrix(280, (B, n_in), bf16_exact=True)
    W = si.random_matrix(281, (n_out, n_in), scale=0.1, bf16_exact=True)
    b = si.random_matrix(282, (n_out,), scale=0.01)
    bf = torch.bfloat16
    save_z = act != O.ACT_IDENTITY
    Y, Z = dl.dense_act_fwd(to_dev(X, bf), to_dev(W, bf), to_dev(b), act, save_z=save_z)
    refY, refZ = O.dense_act_fwd(X, W, b, act)
    if save_z:
        assert_close(to_np(Z), refZ, BF16_TOL, "Z")
    assert_close(to_np(Y), refY, BF16_TOL, "Y")


@pytest.mark.parametrize("B, n_in", [(4104, 4106), (8200, 8202)])
def test_bf16_dx_unaligned_rows(dl, B, n_in):
    n_out = 64
    X = si.random_matrix(290, (B, n_in), bf16_exact=True)
    W = si.random_matrix(291, (n_out, n_in), scale=0.1, bf16_exact=True)
    Z = si.random_matrix(292, (B, n_out), bf16_exact=True)
    dY = si.random_matrix(293, (B, n_out), bf16_exact=True)
    H = si.random_matrix(294, (B, n_in), bf16_exact=True)
    bf = torch.bfloat16
    Wd = to_dev(W, bf)
    # the transposed copy keeps the direct-load kernel (an M/N-major W would
    # need n_in % 8 == 0); the previous layer's GELU derivative folded in
    dX, _, _ = dl.dense_act_vjp(to_dev(dY, bf), to_dev(Z, bf), None, Wd, O.ACT_GELU_TANH,
                                need_dw=False, dx_act=O.ACT_GELU_TANH, dx_saved=to_dev(H, bf),
                                Wt=Wd.t().contiguous())
    rdX, _, _ = O.dense_act_vjp(dY, Z, X, W, O.ACT_GELU_TANH, need_dx=True)
    rdX = rdX * O.act_grad(H, O.ACT_GELU_TANH)
    assert_close(to_np(dX), rdX, BF16_TOL, "dX")


def test_bf16_dw_wide_tile_ragged(dl):
    """A large weight gradient (register-staged 128x128 tiles, split along
    the batch), ragged in both output dimensions."""
    B, n_in, n_out = 2048, 1032, 2000
    X = si.random_matrix(280, (B, n_in), bf16_exact=True)
    W = si.random_matrix(281, (n_out, n_in), scale=0.05, bf16_exact=True)
    dY = si.random_matrix(282, (B, n_out), bf16_exact=True)
    bf = torch.bfloat16
    _, dW, db = dl.dense_act_vjp(to_dev(dY, bf), None, to_dev(X, bf), to_dev(W, bf),
                                 O.ACT_IDENTITY, need_dx=False)
    _, rdW, rdb = O.dense_act_vjp(dY, None, X, W, O.ACT_IDENTITY, need_dx=False)
    assert_close(to_np(dW), rdW, BF16_TOL, "dW")
    assert_close(to_np(db), rdb, BF16_TOL, "db")


def test_bf16_dw_split_ragged(dl):
    B, n_in, n_out = 1024, 1000, 200
    X = si.random_matrix(250, (B, n_in), bf16_exact=True)
    W = si.random_matrix(251, (n_out, n_in), scale=0.05, bf16_exact=True)
    dY = si.random_matrix(252, (B, n_out), bf16_exact=True)
    bf = torch.bfloat16
    dX, dW, db = dl.dense_act_vjp(to_dev(dY, bf), None, to_dev(X, bf), to_dev(W, bf),
                                  O.ACT_IDENTITY)
    rdX, rdW, rdb = O.dense_act_vjp(dY, None, X, W, O.ACT_IDENTITY)
    assert_close(to_np(dW), rdW, BF16_TOL, "dW")
    assert_close(to_np(db), rdb, BF16_TOL, "db")
    assert_close(to_np(dX), rdX, BF16_TOL, "dX")


def test_bf16_fp32_consistency(dl):
    """With bf16-exact operands the fp32 path must meet 1e-4 on the same
    oracle, so the bf16 tolerance hides only output rounding."""
    B, n_in, n_out = 300, 1024, 512
    X = si.random_matrix(80, (B, n_in), bf16_exact=True)
    W = si.random_matrix(81, (n_out, n_in), scale=0.02, bf16_exact=True)
    b = si.random_matrix(82, (n_out,), scale=0.01)
    Y32, _ = dl.dense_act_fwd(to_dev(X), to_dev(W), to_dev(b), O.ACT_GELU_TANH)
    Y16, _ = dl.dense_act_fwd(to_dev(X, torch.bfloat16), to_dev(W, torch.bfloat16), to_dev(b),
                              O.ACT_GELU_TANH)
    ref = O.dense_act_fwd(X, W, b, O.ACT_GELU_TANH)[0]
    assert_close(to_np(Y32), ref, F32_TOL, "fp32 path")
    assert_close(to_np(Y16), O.round_bf16(ref), 1e-2, "bf16 path vs rounded oracle")


def test_cast_bf16_bit_exact(dl):
    rng = np.random.default_rng(90)
    x = (rng.standard_normal(100003) * np.exp(rng.uniform(-30, 30, 100003))).astype(np.float32)
    specials = np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, np.inf, -np.inf, 65504.0,
                         3.4e38, 1e-40], dtype=np.float32)
    x[: specials.size] = specials
    got = dl.dense_cast_bf16(to_dev(x)).view(torch.int16).cpu().numpy().view(np.uint16)
    ref = O.round_bf16(x).astype(np.float32).view(np.uint32) >> 16
    assert np.array_equal(got, ref.astype(np.uint16))
    nan = dl.dense_cast_bf16(to_dev(np.array([np.nan], np.float32)))
    assert torch.isnan(nan.float()).all()


# ------------------------------------------------------------------ softmax xent

XENT_SHAPES = [(1, 1), (5, 10), (64, 10), (8192, 10), (100, 33), (77, 256), (64, 257),
               (130, 1000), (3, 2047), (17, 2049), (8, 4096), (4, 32000), (2, 32001),
               (3, 40000), (300, 31),
               # a whole-workgroup row whose last waves hold no class at all
               (9, 2052)]


@pytest.mark.parametrize("shape", XENT_SHAPES)
def test_softmax_xent(dl, shape):
    B, C = shape
    z = si.random_matrix(100 + C, (B, C), scale=3.0)
    y = si.random_labels(101, B, C)
    row = torch.empty(B, dtype=torch.float32, device=device())
    loss, dz = dl.softmax_xent_fwd_bwd(to_dev(z), to_dev(y), row_loss=row)
    rloss, rdz, rrow = O.softmax_xent_fwd_bwd(z, y)
    assert abs(float(loss.item()) - rloss) <= LOSS_TOL * abs(rloss)
    assert_close(to_np(dz), rdz, F32_TOL, "dlogits")
    assert_close(to_np(row), rrow, F32_TOL, "row loss")


def test_softmax_xent_in_place(dl):
    B, C = 513, 1000
    z = si.random_matrix(110, (B, C), scale=5.0)
    y = si.random_labels(111, B, C)
    zd = to_dev(z)
    loss, dz = dl.softmax_xent_fwd_bwd(zd, to_dev(y), inplace=True)
    assert dz.data_ptr() == zd.data_ptr()
    rloss, rdz, _ = O.softmax_xent_fwd_bwd(z, y)
    assert abs(float(loss.item()) - rloss) <= LOSS_TOL * abs(rloss)
    assert_close(to_np(dz), rdz, F32_TOL, "dlogits")


def test_softmax_xent_labels_read_back_exactly(dl):
    y = si.random_labels(112, 4096, 32000)
    yd = to_dev(y)
    z = to_dev(np.zeros((4096, 32000), np.float32))
    loss, dz = dl.softmax_xent_fwd_bwd(z, yd)
    assert np.array_equal(yd.cpu().numpy(), y)
    assert abs(float(loss.item()) - math.log(32000)) < 1e-5 * math.log(32000)


def test_softmax_xent_bad_label_gives_nan_not_fault(dl):
    z = si.random_matrix(120, (4, 10))
    y = np.array([0, 10, 3, -1], dtype=np.int32)
    row = torch.empty(4, dtype=torch.float32, device=device())
    loss, dz = dl.softmax_xent_fwd_bwd(to_dev(z), to_dev(y), row_loss=row)
    r = row.cpu().numpy()
    assert math.isnan(float(loss.item()))
    assert np.isnan(r[1]) and np.isnan(r[3]) and np.isfinite(r[0]) and np.isfinite(r[2])


def test_validate_mode_rejects_bad_labels_before_any_output(dl):
    """Validate mode: a label outside [0, C) is LABEL_OUT_OF_RANGE, and the
    outputs keep what they held; good labels give the same bits as without
    validation."""
    B, C = 300, 40
    z = to_dev(si.random_matrix(121, (B, C)))
    y = si.random_labels(122, B, C)
    prev = dl.set_validate(True)
    try:
        for bad in (C, -1, 2 ** 31 - 1):
            yb = y.copy()
            yb[B // 2] = bad
            dz = torch.full((B, C), 7.0, device=device())
            loss = torch.full((1,), 7.0, device=device())
            with pytest.raises(dl.DenseError) as ei:
                dl.softmax_xent_fwd_bwd(z, to_dev(yb), dlogits=dz, loss=loss)
            assert ei.value.status == 6
            assert bool(torch.all(dz == 7.0)) and float(loss.item()) == 7.0
        l1, d1 = dl.softmax_xent_fwd_bwd(z, to_dev(y))
    finally:
        dl.set_validate(prev)
    l0, d0 = dl.softmax_xent_fwd_bwd(z, to_dev(y))
    assert torch.equal(d0, d1) and torch.equal(l0, l1)


def test_validate_mode_in_the_mlp_step(dl):
    w = si.WORKLOADS["mlp_small"]
    inp = si.generate(w)
    mlp = dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                 adamw=False)
    W0 = [t.clone() for t in mlp.W]
    yb = inp.labels.copy()
    yb[3] = 10
    prev = dl.set_validate(True)
    try:
        with pytest.raises(dl.DenseError) as ei:
            dl.mlp_train_step(mlp, to_dev(inp.X), to_dev(yb), dl.OPT_SGD, lr=w.optim.lr)
        assert ei.value.status == 6
        assert all(torch.equal(a, b) for a, b in zip(W0, mlp.W))
        loss = dl.mlp_train_step(mlp, to_dev(inp.X), to_dev(inp.labels), dl.OPT_SGD,
                                 lr=w.optim.lr)
    finally:
        dl.set_validate(prev)
    st = O.MLPState(inp.W, inp.b)
    ref = O.mlp_train_step(st, inp.X, inp.labels, w.acts, w.optim)
    assert abs(float(loss.item()) - ref["loss"]) <= LOSS_TOL * abs(ref["loss"])


# ------------------------------------------------ fused classifier head
#
# dense_xent_fwd / dense_xent_vjp: the forward GEMM leaves logits and
# per-tile row statistics, a row pass forms lse and the losses, and the dX /
# dW GEMMs form the loss gradient from the logits as they stage them.
# (B, in, C): several tiles with ragged tails; a class count and an input
# width that are not multiples of 4 (bounds-checked loads everywhere); the
# 32000-class head on 1000 rows; a batch whose weight gradient is split
# along K; the degenerate single-class and single-row heads; and a dX (576
# tiles) and a weight gradient (585 tiles, ragged in classes and batch) with
# more tiles than the chip holds at once, which walk tile rows per XCD; and
# a dX on 516 ragged 128 x 256 tiles of 8 waves, also walking tile rows.
XENT_HEAD_SHAPES = [(300, 96, 1000), (257, 64, 2049), (1000, 768, 32000), (64, 33, 130),
                    (8192, 96, 1000), (5, 16, 3), (1, 8, 1), (77, 40, 1),
                    (8192, 1152, 1000), (520, 1152, 8200), (16461, 1000, 300)]


@pytest.mark.parametrize("shape", XENT_HEAD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dense_xent_head_matches_oracle(dl, shape):
    B, n_in, C = shape
    seed = 700 + B % 97 + C % 89
    X = si.random_matrix(seed, (B, n_in))
    W = si.random_matrix(seed + 1, (C, n_in), scale=0.3 / math.sqrt(n_in))
    b = si.random_matrix(seed + 2, (C,), scale=0.1)
    y = si.random_labels(seed + 3, B, C)
    Xd, Wd, bd, yd = to_dev(X), to_dev(W), to_dev(b), to_dev(y)
    row = torch.empty(B, device=device())
    loss, logits, lse = dl.dense_xent_fwd(Xd, Wd, bd, yd, row_loss=row)
    dX, dW, db = dl.dense_xent_vjp(logits, lse, yd, Xd, Wd)
    torch.cuda.synchronize()
    _, Z = O.dense_act_fwd(X, W, b, O.ACT_IDENTITY)
    rloss, rdz, rrow = O.softmax_xent_fwd_bwd(Z, y)
    rdX, rdW, rdb = O.dense_act_vjp(rdz, None, X, W, O.ACT_IDENTITY)
    assert abs(float(loss.item()) - rloss) <= LOSS_TOL * max(abs(rloss), 1e-30) + 1e-7, \
        (float(loss.item()), rloss)
    assert_close(to_np(logits), Z, F32_TOL, "logits")
    assert_close(to_np(lse), O.softmax_lse(Z), F32_TOL, "lse")
    assert_close(to_np(row), rrow, F32_TOL, "row losses")
    assert_close(to_np(dX), rdX, F32_TOL, "dX")
    assert_close(to_np(dW), rdW, F32_TOL, "dW")
    assert_close(to_np(db), rdb, F32_TOL, "db")


def test_dense_xent_head_is_bit_reproducible_and_options(dl):
    """Two runs give the same bits; dX alone, dW/db alone and no bias match
    the full call; the workspace queries answer."""
    B, n_in, C = 513, 128, 5000
    X = to_dev(si.random_matrix(760, (B, n_in)))
    W = to_dev(si.random_matrix(761, (C, n_in), scale=0.05))
    y = to_dev(si.random_labels(762, B, C))
    l1, z1, s1 = dl.dense_xent_fwd(X, W, None, y)
    l2, z2, s2 = dl.dense_xent_fwd(X, W, None, y)
    assert torch.equal(l1, l2) and torch.equal(z1, z2) and torch.equal(s1, s2)
    a = dl.dense_xent_vjp(z1, s1, y, X, W)
    bx = dl.dense_xent_vjp(z1, s1, y, None, W, need_dw=False)
    bw = dl.dense_xent_vjp(z1, s1, y, X, None, need_dx=False)
    assert torch.equal(a[0], bx[0]) and bx[1] is None
    assert torch.equal(a[1], bw[1]) and torch.equal(a[2], bw[2]) and bw[0] is None
    c = dl._c
    assert c["dense_xent_fwd_workspace_size"](B, n_in, C) >= B * 8 * ((C + 127) // 128)
    assert c["dense_xent_vjp_workspace_size"](65536, 768, 32000) == 65536 * 8 + 256


def test_dense_xent_head_validate_mode(dl):
    B, n_in, C = 40, 16, 50
    X = to_dev(si.random_matrix(770, (B, n_in)))
    W = to_dev(si.random_matrix(771, (C, n_in), scale=0.2))
    y = si.random_labels(772, B, C)
    y[7] = C
    logits = torch.full((B, C), 5.0, device=device())
    prev = dl.set_validate(True)
    try:
        with pytest.raises(dl.DenseError) as ei:
            dl.dense_xent_fwd(X, W, None, to_dev(y), logits=logits)
        assert ei.value.status == 6
        assert bool(torch.all(logits == 5.0))
    finally:
        dl.set_validate(prev)


# ------------------------------------------------------------------ optimizers

OPT_SIZES = [1, 3, 4096, 16389, (1 << 20) + 3]


@pytest.mark.parametrize("n", OPT_SIZES)
def test_sgd(dl, n):
    w = si.random_matrix(130, (n,))
    g = si.random_matrix(131, (n,))
    wd = to_dev(w)
    dl.sgd_step(wd, to_dev(g), 1e-3)
    got = to_np(wd)
    # the kernel's arithmetic is float32, so its step is lr rounded to float32:
    # with that step the update is correct to one float32 ulp
    ref32 = O.round_f32(O.sgd_step(w, g, float(np.float32(1e-3))))
    ulp = np.spacing(np.abs(ref32).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref32) <= ulp)
    assert_close(got, O.sgd_step(w, g, 1e-3), 1e-6, "w")


@pytest.mark.parametrize("n", OPT_SIZES)
def test_adamw_ten_steps(dl, n):
    w = si.random_matrix(140, (n,))
    wd, md, vd = to_dev(w), torch.zeros(n, device=device()), torch.zeros(n, device=device())
    wr, mr, vr = O.round_f32(w), np.zeros(n), np.zeros(n)
    for t in range(1, 11):
        g = si.random_matrix(150 + t, (n,), scale=0.1)
        dl.adamw_step(wd, to_dev(g), md, vd, 1e-3, 0.9, 0.999, 1e-8, 0.01, t)
        wr, mr, vr = [O.round_f32(a) for a in
                      O.adamw_step(wr, g, mr, vr, 1e-3, 0.9, 0.999, 1e-8, 0.01, t)]
    assert_close(to_np(wd), wr, 1e-6, "w")
    assert_close(to_np(md), mr, 1e-5, "m")
    assert_close(to_np(vd), vr, 1e-5, "v")


def test_adamw_zero_gradient_is_pure_decay(dl):
    w = si.random_matrix(160, (1000,))
    wd = to_dev(w)
    z = torch.zeros(1000, device=device())
    dl.adamw_step(wd, z.clone(), z.clone(), z.clone(), 1e-2, 0.9, 0.999, 1e-8, 0.1, 1)
    assert_close(to_np(wd), O.round_f32(w * (1 - 1e-3)), 1e-7, "decay")


# ------------------------------------------------------------------ MLP step
#
# A step is compared on identical inputs: the GPU buffers are loaded with the
# oracle's own state (W, b, m, v) before the step, the oracle never reads a
# GPU value, and the two results of that one step are compared.  Two places
# admit several correct results, and there the comparison widens only by
# what float32 rounding allows:
#   * a ReLU pre-activation within its float32 rounding band of zero may be
#     decided either way; the oracle is re-evaluated with the GPU's decision
#     there (any disagreement outside the band fails);
#   * the AdamW update lr * m_hat / (sqrt(v_hat) + eps) is ill-conditioned for
#     gradients near eps; each element may deviate by the spread of the
#     oracle's own update when its gradient moves within the float32 rounding
#     bound of the weight-gradient sum.


def _gpu_relu_masks(dl, X, Ws, bs, acts):
    """GPU forward, layer by layer (the same kernels and launch plan as the
    fused step), returning each layer's ReLU decision Y > 0."""
    h = to_dev(X)
    masks = []
    for l in range(len(Ws)):
        h, _ = dl.dense_act_fwd(h, to_dev(np.asarray(Ws[l], np.float32)),
                                to_dev(np.asarray(bs[l], np.float32)), acts[l])
        masks.append((h > 0).cpu().numpy() if acts[l] == O.ACT_RELU else None)
    return masks


def _adopted_masks(gpu_masks, state, X, acts):
    """Oracle masks, replaced by the GPU's decision only where the oracle's
    pre-activation lies within its float32 rounding band of zero: the band
    of the layer's own sum plus what the deviation of the layer's float32
    input (the earlier layers' bands, carried forward) can move it by.
    Returns (masks, adopted count); fails on a disagreement outside it."""
    taus, _, _, zs = O.mlp_forward_bands(X, state.W, state.b, acts)
    out, adopted, total = [], 0, 0
    for l in range(len(state.W)):
        if acts[l] == O.ACT_RELU:
            Z = zs[l]
            own = Z > 0
            near = np.abs(Z) <= taus[l]
            diff = own != gpu_masks[l]
            assert not np.any(diff & ~near), f"layer {l}: ReLU decision differs outside the band"
            adopted += int(np.sum(diff & near))
            total += Z.size
            out.append(np.where(near, gpu_masks[l], own).astype(np.float64))
        else:
            out.append(None)
    # The band is the worst case (every rounding error aligned, carried
    # through the layers): far wider than the float32 results actually
    # stray.  What keeps the comparison sharp is that the two sides decide
    # differently only a scattering of times (49 of 2e8 pre-activations in
    # the wide MLP's step), so more than 1e-5 of them (plus 16) fails.
    assert adopted <= 1e-5 * total + 16, f"{adopted} ReLU decisions differ of {total}"
    return out, adopted


def _grad_bands(ref, before, X, acts, masks, loss="xent", scale=1.0, labels=None):
    """Float32 rounding bands of every weight and bias gradient of one MLP
    step, from the oracle's step result `ref` and the state `before` it:
    the loss gradient's band from the logits' forward band, then each
    layer's dW = G^T h and db = sum G bands from the deviations of its G
    (carried down through the dX products) and of its input h (carried up
    through the forward).  Lists (dW bands, db bands), times the loss
    scale like the gradients themselves."""
    L = len(before.W)
    taus, dhs, hs, zs = O.mlp_forward_bands(X, before.W, before.b, acts)
    B = hs[0].shape[0]
    if loss == "xent":
        dG = O.xent_grad_band(zs[-1], taus[-1], B, labels=labels)
    else:  # mean squared error: 2 (p - t) / (B C), four roundings
        n = zs[-1].size
        dG = (2.0 / n) * (taus[-1] + O.gamma(4) * (np.abs(ref["G"][-1]) * n / 2.0 + taus[-1]))
    bw, bb = [None] * L, [None] * L
    for l in reversed(range(L)):
        G = ref["G"][l]
        bw[l] = scale * O.sum_band(G, hs[l], dG, dhs[l])
        bb[l] = scale * O.sum_band(G, np.ones((B, 1)), dG, None)[:, 0]
        if l > 0:
            mk = masks[l - 1] if masks is not None and masks[l - 1] is not None else \
                O.act_grad(zs[l - 1], acts[l - 1])
            dG = O.dx_band(G, before.W[l], dG, mk)
    return bw, bb


def _adamw_spread(w0, g, dg, m0, v0, o, t):
    """Largest change of the oracle's AdamW result (w, m, v) when g moves by
    +-dg."""
    args = (o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, t)
    c = O.adamw_step(w0, g, m0, v0, *args)
    p = O.adamw_step(w0, g + dg, m0, v0, *args)
    m = O.adamw_step(w0, g - dg, m0, v0, *args)
    return [np.maximum(np.abs(pi - ci), np.abs(mi - ci)) for ci, pi, mi in zip(c, p, m)]


def _assert_close_band(got, ref, band, tol, what):
    """got within tol (normwise) of ref once each element may also move by
    its band.  The band admits elements whose update is ill-conditioned in
    the gradient: a gradient so close to zero that the float32 sum may turn
    the update's sign, or within a few tens of eps, where
    m_hat / (sqrt(v_hat) + eps) still moves with its gradient's last digits.
    Those are counted, and more than 1e-3 of the elements (plus 8) fails: in
    the workloads here that share stays near or below 2.5e-4 (the classifier
    head's biases, whose gradients are (sum of ~2 softmax masses - count) / B
    and cancel to within 30 eps for about one class in a hundred), so a
    kernel that goes wrong on more than a scattering of elements fails."""
    scale = np.max(np.abs(ref))
    dev = np.abs(got - ref)
    excess = dev - band
    err = float(np.max(excess) / scale) if scale > 0 else float(np.max(excess))
    assert err < tol, f"{what}: error beyond the rounding band {err:.3e} >= {tol:.1e}"
    admitted = int(np.sum(dev >= tol * scale)) if scale > 0 else 0
    assert admitted <= 1e-3 * dev.size + 8, f"{what}: band admits {admitted} of {dev.size}"
    return admitted


def _load_state(mlp, st):
    for l in range(mlp.L):
        mlp.W[l].copy_(torch.from_numpy(st.W[l].astype(np.float32)))
        mlp.b[l].copy_(torch.from_numpy(st.b[l].astype(np.float32)))
        if mlp.mW[l] is not None:
            mlp.mW[l].copy_(torch.from_numpy(st.mW[l].astype(np.float32)))
            mlp.vW[l].copy_(torch.from_numpy(st.vW[l].astype(np.float32)))
            mlp.mb[l].copy_(torch.from_numpy(st.mb[l].astype(np.float32)))
            mlp.vb[l].copy_(torch.from_numpy(st.vb[l].astype(np.float32)))


def _copy_state(st):
    c = O.MLPState(st.W, st.b)
    c.mW = [a.copy() for a in st.mW]
    c.vW = [a.copy() for a in st.vW]
    c.mb = [a.copy() for a in st.mb]
    c.vb = [a.copy() for a in st.vb]
    c.t = st.t
    return c


def _opt_kind(dl, w):
    return dl.OPT_ADAMW if w.optim.kind == "adamw" else dl.OPT_SGD


def _gpu_step(dl, mlp, w, Xd, yd, t):
    o = w.optim
    return dl.mlp_train_step(mlp, Xd, yd, _opt_kind(dl, w), lr=o.lr, beta1=o.beta1,
                             beta2=o.beta2, eps=o.eps, weight_decay=o.weight_decay, step=t)


def _check_one_step(dl, w, inp, mlp, Xd, yd, st):
    """Load the oracle state `st` (before step st.t + 1) into the GPU, run one
    step on both sides and compare everything the step produces."""
    t = st.t + 1
    _load_state(mlp, st)
    gm = _gpu_relu_masks(dl, inp.X, st.W, st.b, w.acts)
    masks, adopted = _adopted_masks(gm, st, inp.X, w.acts)
    before = _copy_state(st)
    ref_st = _copy_state(st)
    ref = O.mlp_train_step(ref_st, inp.X, inp.labels, w.acts, w.optim, relu_masks=masks)
    loss = float(_gpu_step(dl, mlp, w, Xd, yd, t).item())
    assert abs(loss - ref["loss"]) <= LOSS_TOL * abs(ref["loss"]), (t, loss, ref["loss"])
    o = w.optim
    bands_w, bands_b = _grad_bands(ref, before, inp.X, w.acts, masks, labels=inp.labels)
    for l in range(mlp.L):
        dgW, dgb = bands_w[l], bands_b[l]
        assert_close(to_np(mlp.dW[l]), ref["dW"][l], F32_TOL, f"step {t} dW{l}")
        assert_close(to_np(mlp.db[l]), ref["db"][l], F32_TOL, f"step {t} db{l}")
        pairs = [("W", mlp.W[l], ref_st.W[l], before.W[l], ref["dW"][l], dgW, before.mW[l],
                  before.vW[l], mlp.mW[l], mlp.vW[l], ref_st.mW[l], ref_st.vW[l]),
                 ("b", mlp.b[l], ref_st.b[l], before.b[l], ref["db"][l], dgb, before.mb[l],
                  before.vb[l], mlp.mb[l], mlp.vb[l], ref_st.mb[l], ref_st.vb[l])]
        for name, got, want, w0, g, dg, m0, v0, gm_, gv_, wm_, wv_ in pairs:
            if o.kind == "adamw":
                bw, bm, bv = _adamw_spread(w0, g, dg, m0, v0, o, t)
                _assert_close_band(to_np(got), want, bw, F32_TOL, f"step {t} {name}{l}")
                _assert_close_band(to_np(gm_), wm_, bm, F32_TOL, f"step {t} m{name}{l}")
                _assert_close_band(to_np(gv_), wv_, bv, F32_TOL, f"step {t} v{name}{l}")
            else:
                assert_close(to_np(got), want, F32_TOL, f"step {t} {name}{l}")
                _assert_sgd_update(to_np(got), want, w0, g, o.lr, f"step {t} {name}{l}")
    return ref["loss"], adopted


def _assert_sgd_update(got, want, p0, g, lr, what):
    """The SGD update p - p0 on its own, which a normwise check of p hides
    under p itself: both sides round p0 - lr g to float32 once (at most one
    ulp of p apart), on top of lr times the gradient's own normwise
    difference (F32_TOL, checked before)."""
    p0 = np.asarray(p0, dtype=np.float64)
    d_gpu = np.asarray(got, dtype=np.float64) - p0
    d_ref = np.asarray(want, dtype=np.float64) - p0
    scale = max(np.abs(p0).max(), np.abs(np.asarray(want, dtype=np.float64)).max())
    tol = lr * F32_TOL * np.abs(g).max() + 2.0 ** -23 * scale
    err = np.abs(d_gpu - d_ref).max()
    assert err <= tol, (what, err, tol, np.abs(d_ref).max())


def _trajectory(dl, w, steps, check_steps, batch=None):
    """Run the oracle free for `steps` steps; before each step in
    `check_steps` compare one GPU step started from the oracle's state."""
    if batch is not None:
        w = w.scaled(batch)
    inp = si.generate(w)
    mlp = dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                 adamw=(w.optim.kind == "adamw"))
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    st = O.MLPState(inp.W, inp.b)
    for t in range(1, steps + 1):
        if t in check_steps:
            _check_one_step(dl, w, inp, mlp, Xd, yd, st)
        if t < steps:
            O.mlp_train_step(st, inp.X, inp.labels, w.acts, w.optim)


def test_mlp_small_one_sgd_step(dl):
    _trajectory(dl, si.WORKLOADS["mlp_small"], 1, {1})


def test_mlp_small_ragged_batch(dl):
    _trajectory(dl, si.WORKLOADS["mlp_small"], 3, {1, 3}, batch=37)


def test_mlp_adamw_full_batch_steps(dl):
    """Full state (loss, dW, db, W, b, m, v) at steps 1, 2, 10 and 100 of the
    8192-sample AdamW run, each GPU step started from the oracle's state."""
    _trajectory(dl, si.WORKLOADS["mlp_adamw"], 100, {1, 2, 10, 100})


def test_mlp_adamw_all_100_losses(dl):
    """Every one of the 100 steps of the 8192-sample AdamW run: the GPU loss,
    computed from the oracle's state at that step, against the oracle's loss;
    and the trajectory the GPU follows on its own, reported beside it."""
    w = si.WORKLOADS["mlp_adamw"]
    inp = si.generate(w)
    mlp = dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                 adamw=True)
    free = dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                  adamw=True)
    Xd, yd = to_dev(inp.X), to_dev(inp.labels)
    st = O.MLPState(inp.W, inp.b)
    rel, free_loss, ref_loss = [], [], []
    for t in range(1, 101):
        _load_state(mlp, st)
        got = float(_gpu_step(dl, mlp, w, Xd, yd, t).item())
        free_loss.append(float(_gpu_step(dl, free, w, Xd, yd, t).item()))
        ref = O.mlp_train_step(st, inp.X, inp.labels, w.acts, w.optim)["loss"]
        ref_loss.append(ref)
        rel.append(abs(got - ref) / abs(ref))
    free_rel = max(abs(a - b) / b for a, b in zip(free_loss, ref_loss))
    print(f"max rel loss error {max(rel):.2e}; free-running GPU vs oracle: {free_rel:.2e}")
    assert max(rel) < LOSS_TOL, (int(np.argmax(rel)), max(rel))
    assert ref_loss[-1] < ref_loss[0] and free_loss[-1] < free_loss[0]
    # The GPU's own 100-step trajectory against the oracle's.  Two float32
    # trajectories part once an AdamW update near a zero gradient goes the
    # other way (an element then moves 2 lr away and its later gradients
    # differ), and the parting grows from step to step, so no rounding bound
    # covers it: this is an envelope that a broken update or gradient would
    # leave at once (their errors are of the order of the loss and of lr
    # per element per step), not a parity check.  Measured on MI355X: loss
    # 1.1e-3 relative at the worst step; W1 (784 inputs, the most elements
    # with near-zero gradients) 7.3e-2 normwise, the other arrays 4e-3 to
    # 3.6e-2.  A missing or sign-reversed update would put elements up to
    # 2 lr t = 0.2 apart, of the order of the arrays' largest elements, so
    # the envelope is the loss within 1e-2 and each array within 0.25.
    errs = {}
    for l in range(free.L):
        for name, got, want in (("W", free.W[l], st.W[l]), ("b", free.b[l], st.b[l])):
            errs[f"{name}{l}"] = normwise(to_np(got), want)
    print("free-running state after 100 steps, normwise: " +
          ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert free_rel < 1e-2, free_rel
    assert max(errs.values()) < 0.25, errs


def test_mlp_wide_reduced_batch(dl):
    _trajectory(dl, si.WORKLOADS["mlp_wide"], 1, {1}, batch=256)


def test_head_xent_reduced_batch(dl):
    _trajectory(dl, si.WORKLOADS["head_xent"], 2, {1, 2}, batch=256)


# The narrow-head path of the step (last Linear + softmax-xent + its vjp in
# one kernel, for <= 16 classes and <= 256 inputs) at its corners, and the
# unfused path just past them.
_HEADS = {
    "single_layer": si.Workload("head_single", 21, 100, [64, 10], [O.ACT_IDENTITY], "kaiming",
                                "uniform001", "f32", si.ADAMW),
    "max_head_ragged": si.Workload("head_max", 22, 77, [96, 256, 16], [O.ACT_RELU, O.ACT_IDENTITY],
                                   "kaiming", "uniform001", "f32", si.SGD),
    "one_slice": si.Workload("head_small_batch", 23, 20, [50, 30, 7], [O.ACT_RELU, O.ACT_IDENTITY],
                             "kaiming", "uniform001", "f32", si.ADAMW),
    "many_tiles": si.Workload("head_tiles", 24, 5000, [40, 64, 12], [O.ACT_RELU, O.ACT_IDENTITY],
                              "kaiming", "uniform001", "f32", si.ADAMW),
    "identity_hidden": si.Workload("head_linear", 25, 200, [30, 20, 5],
                                   [O.ACT_IDENTITY, O.ACT_IDENTITY], "kaiming", "uniform001", "f32",
                                   si.SGD),
    "unfused_17_classes": si.Workload("head_17", 26, 300, [60, 40, 17],
                                      [O.ACT_RELU, O.ACT_IDENTITY], "kaiming", "uniform001", "f32",
                                      si.SGD),
}


@pytest.mark.parametrize("case", sorted(_HEADS))
def test_mlp_step_head_shapes(dl, case):
    _trajectory(dl, _HEADS[case], 2, {1, 2})


def test_mlp_step_bit_reproducible(dl):
    w = si.WORKLOADS["mlp_adamw"]
    inp = si.generate(w)
    outs = []
    for _ in range(2):
        mlp = dl.MLP([to_dev(a) for a in inp.W], [to_dev(a) for a in inp.b], w.acts, w.batch,
                     adamw=True)
        for t in range(1, 4):
            dl.mlp_train_step(mlp, to_dev(inp.X), to_dev(inp.labels), dl.OPT_ADAMW,
                              weight_decay=0.01, step=t)
        outs.append([a.clone() for a in mlp.W + mlp.b + mlp.mW + mlp.vW])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_profile_hook_times_each_launch(dl):
    X, W, b = _layer(200, 512, 256, 128)
    Xd, Wd, bd = to_dev(X), to_dev(W), to_dev(b)
    dl.profile_begin(16)
    dl.dense_act_fwd(Xd, Wd, bd, O.ACT_RELU)
    dY = to_dev(si.random_matrix(201, (512, 128)))
    dl.dense_act_vjp(dY, None, Xd, Wd, O.ACT_IDENTITY)
    recs = dl.profile_end(16)
    names = [n for n, _ in recs]
    assert names[0] == "fwd_gemm" and "dw_gemm" in names and names[-1] == "dx_gemm"
    assert all(ms > 0 for _, ms in recs)
    # outside a profiling window nothing is recorded
    dl.dense_act_fwd(Xd, Wd, bd, O.ACT_RELU)
    dl.profile_begin(0)
    assert dl.profile_end(0) == []


@pytest.mark.parametrize("shape", [(1, 1), (63, 130), (1024, 4096), (4096, 1000), (100, 68), (4, 8)])
def test_cast_bf16_transposed_bit_exact(dl, shape):
    W = si.random_matrix(210, shape, scale=0.02)
    d, dt = dl.dense_cast_bf16_t(to_dev(W))
    ref = (O.round_bf16(W).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = d.view(torch.int16).cpu().numpy().view(np.uint16)
    got_t = dt.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref) and np.array_equal(got_t, ref.T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(300, 1000, 1000), (513, 1024, 4096), (77, 130, 90)])
def test_dense_vjp_with_transposed_weight(dl, dtype, shape):
    """dX through the transposed weight (read along the contraction index)
    equals dX through W, and both match the oracle."""
    B, n_in, n_out = shape
    bf = dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32
    X = si.random_matrix(220, (B, n_in), bf16_exact=bf)
    W = si.random_matrix(221, (n_out, n_in), scale=0.02, bf16_exact=bf)
    dY = si.random_matrix(222, (B, n_out), bf16_exact=bf)
    Wd = to_dev(W, tdt)
    Wt = Wd.t().contiguous()
    dX, dW, db = dl.dense_act_vjp(to_dev(dY, tdt), None, to_dev(X, tdt), Wd, O.ACT_IDENTITY,
                                  Wt=Wt)
    dX2, _, _ = dl.dense_act_vjp(to_dev(dY, tdt), None, None, Wd, O.ACT_IDENTITY, need_dw=False)
    rdX, rdW, rdb = O.dense_act_vjp(dY, None, X, W, O.ACT_IDENTITY)
    tol = BF16_TOL if bf else F32_TOL
    assert_close(to_np(dX), rdX, tol, "dX via Wt")
    assert_close(to_np(dX2), rdX, tol, "dX via W")
    assert_close(to_np(dW), rdW, tol, "dW")

"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the header declares, reports its target, answers workspace
queries, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dense_layers_amd.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def dl():
    import dense_layers_amd
    return dense_layers_amd


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["dense_act_fwd", "dense_act_vjp", "softmax_xent_fwd_bwd", "sgd_step",
              "adamw_step", "mlp_train_step", "dense_cast_bf16", "dl_last_error",
              "dense_last_error", "dl_set_validate"]:
        assert n in names


def test_last_error_names_and_validate_switch(dl):
    c = dl._c
    # a rejected call (no GPU work: the size check comes first)
    assert c["sgd_step"](None, 0, None, None, 1e-3) == 1
    assert c["dense_last_error"]() == c["dl_last_error"]() and b"sgd_step" in c["dense_last_error"]()
    assert dl.set_validate(True) is False
    assert dl.set_validate(False) is True
    assert dl.STATUS[6] == "LABEL_OUT_OF_RANGE"


def test_library_exports_every_declared_symbol(dl):
    lib = ctypes.CDLL(dl.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), n
    assert sorted(_declared_functions()) == sorted(dl.EXPORTS)


def test_build_target(dl):
    assert dl.build_target() == "gfx950"


def test_workspace_queries(dl):
    # identity activation, no split-K needed: nothing
    assert dl.dense_act_vjp_workspace_size(dl.DL_F32, dl.ACT_IDENTITY, 16384, 4096, 4096) == 0
    # GELU needs the masked gradient (bf16, 256-byte aligned)
    n = dl.dense_act_vjp_workspace_size(dl.DL_BF16, dl.ACT_GELU_TANH, 32768, 1024, 4096)
    assert n >= 32768 * 4096 * 2 and n % 256 == 0
    # long-K weight gradient of a narrow layer gets split-K partials
    assert dl.dense_act_vjp_workspace_size(dl.DL_F32, dl.ACT_IDENTITY, 8192, 784, 256) > 0
    assert dl.softmax_xent_workspace_size(65536, 32000) == 65536 * 4
    assert dl.dense_act_vjp_workspace_size(dl.DL_F32, 7, 1, 1, 1) == 0
    assert dl.softmax_xent_workspace_size(0, 10) == 0


def test_mlp_workspace_query(dl):
    dims = [784, 256, 128, 10]
    table = (dl.DLLayer * 3)()
    for l in range(3):
        table[l] = dl.DLLayer(dims[l], dims[l + 1], 1 if l < 2 else 0)
    n = dl.mlp_train_step_workspace_size(8192, table)
    assert n >= 8192 * (256 + 128 + 10) * 4 + 8192 * 4
    assert n % 256 == 0


def _raw(dl):
    return ctypes.CDLL(dl.LIB_PATH)


def test_rejects_bad_arguments_without_launching(dl):
    c = dl._c
    fake = 0x100000  # never dereferenced: every call below fails validation first
    # bad dtype
    assert c["dense_act_fwd"](None, 9, 0, 4, 4, 4, fake, fake, None, fake + 4096, None) == 1
    # bad activation
    assert c["dense_act_fwd"](None, 0, 9, 4, 4, 4, fake, fake, None, fake + 4096, None) == 1
    # zero size
    assert c["dense_act_fwd"](None, 0, 0, 0, 4, 4, fake, fake, None, fake + 4096, None) == 1
    # missing X
    assert c["dense_act_fwd"](None, 0, 0, 4, 4, 4, None, fake, None, fake + 4096, None) == 1
    assert "X, W and Y" in c["dl_last_error"]().decode()
    # Y overlapping X
    assert c["dense_act_fwd"](None, 0, 0, 4, 4, 4, fake, fake + 8192, None, fake + 16, None) == 3
    # vjp: GELU without the saved pre-activation
    assert c["dense_act_vjp"](None, 0, 2, 4, 4, 4, fake, None, fake, fake, None, None, None, None,
                              0, None, None, 0) == 1
    # vjp: db without dW
    assert c["dense_act_vjp"](None, 0, 0, 4, 4, 4, fake, None, fake, fake, None, None, None,
                              fake + 8192, 0, None, None, 0) == 2
    # vjp: workspace too small (split-K partials needed)
    assert c["dense_act_vjp"](None, 0, 0, 8192, 784, 256, fake, None, fake + (1 << 30),
                              fake + (1 << 31), None, None, fake + (1 << 32), None, 0, None,
                              None, 0) == 4
    # xent: missing labels, workspace too small, partial overlap of dlogits
    assert c["softmax_xent_fwd_bwd"](None, 4, 10, fake, None, fake, None, fake, fake, 1024) == 1
    assert c["softmax_xent_fwd_bwd"](None, 4, 10, fake, fake + 4096, fake + 8192, None,
                                     fake + 16384, fake + 32768, 0) == 4
    assert c["softmax_xent_fwd_bwd"](None, 4, 10, fake, fake + 4096, fake + 8192, None,
                                     fake + 4, fake + 32768, 256) == 3
    # optimizers
    assert c["sgd_step"](None, 0, fake, fake + 64, 0.1) == 1
    assert c["sgd_step"](None, 16, fake, fake + 4, 0.1) == 3
    assert c["adamw_step"](None, 16, fake, fake + 64, fake + 128, fake + 192, 1e-3, 0.9, 0.999,
                           1e-8, 0.0, 0) == 1
    assert c["adamw_step"](None, 16, fake, fake + 64, fake + 64, fake + 192, 1e-3, 0.9, 0.999,
                           1e-8, 0.0, 1) == 3
    assert c["adamw_step"](None, 16, fake, fake + 64, fake + 128, fake + 192, 1e-3, 1.5, 0.999,
                           1e-8, 0.0, 1) == 1
    assert c["dense_cast_bf16"](None, 16, fake, fake + 8) == 3
    assert c["dense_cast_bf16_t"](None, 4, 4, fake, None, None) == 1
    assert c["dense_cast_bf16_t"](None, 4, 4, fake, fake + 32, None) == 3


def test_mlp_step_rejects_bad_layers(dl):
    c = dl._c
    fake = 0x100000
    table = (dl.DLLayer * 2)()
    table[0] = dl.DLLayer(8, 4, 1, fake, fake + 256, fake + 512, fake + 768)
    table[1] = dl.DLLayer(5, 3, 0, fake + 1024, fake + 1280, fake + 1536, fake + 1792)
    opt = dl.DLOpt(0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    # layer 1's in (5) != layer 0's out (4)
    assert c["mlp_train_step"](None, 2, 2, table, fake, fake, ctypes.byref(opt), fake, fake,
                               1 << 20) == 1
    table[1] = dl.DLLayer(4, 3, 1, fake + 1024, fake + 1280, fake + 1536, fake + 1792)
    # ReLU on the last layer is not supported (the loss pass overwrites its output)
    assert c["mlp_train_step"](None, 2, 2, table, fake, fake, ctypes.byref(opt), fake, fake,
                               1 << 20) == 2
    table[1] = dl.DLLayer(4, 3, 0, fake + 1024, fake + 1280, fake + 1536, fake + 1792)
    # AdamW without moments
    opt = dl.DLOpt(1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    assert c["mlp_train_step"](None, 2, 2, table, fake, fake, ctypes.byref(opt), fake, fake,
                               1 << 20) == 1
    # bad optimizer kind
    opt = dl.DLOpt(5, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    assert c["mlp_train_step"](None, 2, 2, table, fake, fake, ctypes.byref(opt), fake, fake,
                               1 << 20) == 1


def test_mlp_fusion_level_setting(dl):
    prev = dl.set_mlp_fusion(1)
    assert prev == 2  # default: the tail kernel where it fits
    assert dl.set_mlp_fusion(2) == 1
    for bad in (0, 3, -1):
        with pytest.raises(dl.DenseError):
            dl.set_mlp_fusion(bad)
    assert dl.set_mlp_fusion(2) == 2  # unchanged by the rejected levels


def test_xent_noalloc_rejects_before_any_device_work(dl):
    """The no-allocation cross-entropy checks sizes, pointers, aliasing and
    its scratch limit on the host first (fake pointers are never touched)."""
    c = dl._c["softmax_xent_fwd_bwd_noalloc"]
    fake = 1 << 40
    big = dl.XENT_NOALLOC_MAX_ROWS + 1
    assert c(None, big, 10, fake, fake + (1 << 30), fake + (2 << 30), None, fake + (3 << 30)) == 4
    assert b"scratch" in dl._c["dense_last_error"]()
    assert c(None, 0, 10, fake, fake, fake, None, fake) == 1
    assert c(None, 4, 10, fake, None, fake, None, fake) == 1
    assert c(None, 4, 10, fake, fake, fake, None, fake) == 3

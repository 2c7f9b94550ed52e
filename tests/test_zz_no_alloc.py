"""The cross-entropy entry point that allocates nothing
(softmax_xent_fwd_bwd_noalloc), called through the C ABI, against the
workspace entry point (softmax_xent_fwd_bwd) on the same inputs: the same
kernels run, so every output must match bit for bit.  Two calls in a row on
one device share the library's scratch; the second, smaller one must not
see anything of the first."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.gpu_util import device, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dl():
    device()
    import dense_layers_amd
    return dense_layers_amd


def _noalloc(dl, logits, labels, dlogits, loss, row_loss=None):
    B, C = logits.shape
    stream = torch.cuda.current_stream(logits.device).cuda_stream
    ptr = (lambda t: None if t is None else t.data_ptr())
    return dl._c["softmax_xent_fwd_bwd_noalloc"](stream, B, C, ptr(logits), ptr(labels),
                                                 ptr(loss), ptr(row_loss), ptr(dlogits))


def _case(seed, B, C):
    z = to_dev(si.random_matrix(seed, (B, C), scale=3.0))
    y = to_dev(si.random_labels(seed + 1, B, C))
    return z, y


# first call, then a smaller one on the same device
PAIRS = [((4096, 1000), (1000, 1000)), ((600, 32000), (257, 32000)), ((2000, 10), (37, 10)),
         ((3000, 2052), (5, 2052))]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}x{p[0][1]}->{p[1][0]}")
def test_noalloc_matches_workspace_entry_on_two_calls(dl, pair):
    for k, (B, C) in enumerate(pair):
        z, y = _case(900 + 10 * k + C % 7, B, C)
        ref_loss, ref_dz = dl.softmax_xent_fwd_bwd(z, y)
        ref_row = torch.empty(B, device=device())
        dl.softmax_xent_fwd_bwd(z, y, row_loss=ref_row)
        dz = torch.full((B, C), float("nan"), device=device())
        loss = torch.full((1,), float("nan"), device=device())
        assert _noalloc(dl, z, y, dz, loss) == 0, dl._c["dense_last_error"]()
        torch.cuda.synchronize()
        assert torch.equal(loss, ref_loss), (B, C, float(loss.item()), float(ref_loss.item()))
        assert torch.equal(dz, ref_dz), (B, C)
        row = torch.full((B,), float("nan"), device=device())
        dz2 = torch.empty_like(dz)
        assert _noalloc(dl, z, y, dz2, loss, row) == 0
        torch.cuda.synchronize()
        assert torch.equal(row, ref_row) and torch.equal(dz2, ref_dz)


def test_noalloc_in_place(dl):
    z, y = _case(950, 513, 4000)
    ref_loss, ref_dz = dl.softmax_xent_fwd_bwd(z, y)
    loss = torch.empty(1, device=device())
    assert _noalloc(dl, z, y, z, loss) == 0
    torch.cuda.synchronize()
    assert torch.equal(z, ref_dz) and torch.equal(loss, ref_loss)


def test_noalloc_rejects_rows_past_its_scratch(dl):
    """More rows than the scratch holds: a clear error and nothing launched
    (the check comes before any device work), unless row_loss is given."""
    B = dl.XENT_NOALLOC_MAX_ROWS + 1
    fake = 1 << 40  # never dereferenced: the size check fails first
    stream = torch.cuda.current_stream(device()).cuda_stream
    st = dl._c["softmax_xent_fwd_bwd_noalloc"](stream, B, 10, fake, fake + (1 << 30),
                                               fake + (2 << 30), None, fake + (3 << 30))
    assert st == 4
    assert b"scratch" in dl._c["dense_last_error"]()
    assert dl._c["softmax_xent_fwd_bwd_noalloc"](stream, 0, 10, fake, fake, fake, None, fake) == 1


def test_noalloc_largest_scratch_batch(dl):
    """The largest batch the scratch holds, with a narrow class count."""
    B, C = dl.XENT_NOALLOC_MAX_ROWS, 10
    z, y = _case(960, B, C)
    ref_loss, ref_dz = dl.softmax_xent_fwd_bwd(z, y)
    dz, loss = torch.empty_like(z), torch.empty(1, device=device())
    assert _noalloc(dl, z, y, dz, loss) == 0
    torch.cuda.synchronize()
    assert torch.equal(loss, ref_loss) and torch.equal(dz, ref_dz)
    assert np.isfinite(float(loss.item()))

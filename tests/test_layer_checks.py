"""Argument checks of the layer classes, on the CPU: every malformed tensor is
rejected with ValueError before any library call is made (the binding's launch
functions are replaced by ones that fail the test if reached)."""

import pytest
import torch

from orthogonal_reparameterized_cnp_amd import binding as B
from orthogonal_reparameterized_cnp_amd import layer as L


@pytest.fixture
def no_launch(monkeypatch):
    def boom(*a, **k):
        raise AssertionError("a library call was made before the arguments were checked")

    for name in ("poetx_linear_fwd", "poetx_linear_bwd", "poetx_linear_bwd_dx", "poetx_spo_fwd", "poetx_spo_bwd"):
        monkeypatch.setattr(B, name, boom)


def _layer(mode="xfast"):
    return L.PoetxLinear(96, 80, 32, "bf16", "bf16", device="cpu", mode=mode)


def _fake_forward(lay, T):
    """State a forward of T tokens would leave (no kernel runs on the CPU)."""
    lay.H_save = torch.empty(B.poetx_saved_bytes(lay.desc, T), dtype=torch.uint8)
    lay.T = T


@pytest.mark.parametrize(
    "X, msg",
    [
        (torch.zeros(8, 95, dtype=torch.bfloat16), "shape"),
        (torch.zeros(8, 96, dtype=torch.float32), "dtype"),
        (torch.zeros(96, 8, dtype=torch.bfloat16).t(), "contiguous"),
        (torch.zeros(8, 96, dtype=torch.bfloat16), "GPU"),
        (torch.zeros(8, 2, 96, dtype=torch.bfloat16), "2-D"),
    ],
)
def test_forward_rejects(no_launch, X, msg):
    with pytest.raises(ValueError, match=msg):
        _layer().forward(X)


def test_forward_rejects_bad_output(no_launch):
    with pytest.raises(ValueError, match="Y has shape"):
        _layer().forward(torch.zeros(8, 96, dtype=torch.bfloat16), Y=torch.zeros(8, 79, dtype=torch.bfloat16))


def test_backward_needs_forward_of_same_tokens(no_launch):
    lay = _layer()
    X, dZ = torch.zeros(8, 96, dtype=torch.bfloat16), torch.zeros(8, 80, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="saved state"):
        lay.backward(X, dZ)
    _fake_forward(lay, 16)
    with pytest.raises(ValueError, match="forward of 16"):
        lay.backward(X, dZ)


@pytest.mark.parametrize(
    "kw, msg",
    [
        (dict(dZ=torch.zeros(8, 81, dtype=torch.bfloat16)), "dZ has shape"),
        (dict(dZ=torch.zeros(7, 80, dtype=torch.bfloat16)), "dZ has shape"),
        (dict(dZ=torch.zeros(8, 80, dtype=torch.float32)), "dZ has dtype"),
        (dict(dX=torch.zeros(8, 95, dtype=torch.bfloat16)), "dX has shape"),
        (dict(dq_R=torch.zeros(2, 496)), "dq_R has shape"),
        (dict(dq_P=torch.zeros(3, 496, dtype=torch.float64)), "dq_P has"),
        (dict(), "GPU"),
    ],
)
def test_backward_rejects(no_launch, kw, msg):
    lay = _layer()
    _fake_forward(lay, 8)
    args = dict(dZ=torch.zeros(8, 80, dtype=torch.bfloat16))
    args.update(kw)
    dZ = args.pop("dZ")
    with pytest.raises(ValueError, match=msg):
        lay.backward(torch.zeros(8, 96, dtype=torch.bfloat16), dZ, **args)


def test_xout_backward_checks_y(no_launch):
    lay = _layer("xout")
    _fake_forward(lay, 8)
    X, dZ = torch.zeros(8, 96, dtype=torch.bfloat16), torch.zeros(8, 80, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="pass Y"):
        lay.backward(X, dZ)
    with pytest.raises(ValueError, match="Y has shape"):
        lay.backward(X, dZ, Y=torch.zeros(4, 80, dtype=torch.bfloat16))


def test_group_backward_checks(no_launch):
    lay = _layer()
    g = L.PoetxGroup.__new__(L.PoetxGroup)  # the checks run before the group's own buffers are used
    g.layers, g.device = [lay], lay.device
    _fake_forward(lay, 8)
    with pytest.raises(ValueError, match="dZ has shape"):
        g.backward_dx(0, torch.zeros(8, 96, dtype=torch.bfloat16), torch.zeros(8, 96, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="forward of 8"):
        g.backward_dx(0, torch.zeros(9, 96, dtype=torch.bfloat16), torch.zeros(9, 80, dtype=torch.bfloat16))


def test_spo_factor_checks(no_launch):
    f = L.PoetxSpoFactor(64, 16, "block", "bf16", device="cpu")
    with pytest.raises(ValueError, match="X has shape"):
        f.forward(torch.zeros(4, 63, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        f.forward(torch.zeros(4, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="forward of None"):
        f.backward(torch.zeros(4, 64, dtype=torch.bfloat16))
    f.T = 4
    with pytest.raises(ValueError, match="dY has dtype"):
        f.backward(torch.zeros(4, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="dq has shape"):
        f.backward(torch.zeros(4, 64, dtype=torch.bfloat16), dq=torch.zeros(3, 120))

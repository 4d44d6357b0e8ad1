"""Group calls (poetx_linear_fwd_group, poetx_linear_bwd_dx_group): the forwards and the backwards to dX
of several linears with their block products in shared launches, and their W~ contractions that are
too small to fill the GPU alone (fewer than 256 tiles of 256 x 256) in one launch per K where together
they do.  Every output must be bit-identical to the linear's own calls (the same kernels take the same
operands in the same order).

The cases reach: one contraction alone next to two grouped ones, forward and backward (q, k, v shapes:
8192 tokens, widths 2048 / 1024 / 1024 under 1024 inputs; the backward groups k and v and leaves q, of
another K, alone), one input shared by every linear of a call, int8 weights (widened codes, column
scales in the grouped launch, once next to a bf16 linear without scales), a group of contractions too
small to launch together, streamed sides with a partial last block and a ragged K (1300 = 5 x 256 + 20,
contracted over its zero padding to 1344), sides too short to stream (ragged T, partial blocks), the
Xmem and Xout backwards, and fp32 layers (one call per linear)."""

import pytest
import torch

from orthogonal_reparameterized_cnp_amd.layer import PoetxGroup
from tests.poetx_cases import dev, make_layer
from workloads.gen import custom_linear_inputs

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

# act, mode, b, [(m, n, w)], T, one shared input
CASES = [
    ("bf16", "xfast", 512, [(1024, 2048, "bf16"), (1024, 1024, "bf16"), (1024, 1024, "bf16")], 8192, True),
    ("bf16", "xfast", 512, [(1024, 1024, "i8"), (1024, 1024, "i8")], 8192, True),
    ("bf16", "xfast", 512, [(1024, 1024, "i8"), (1024, 1024, "bf16")], 8192, False),
    ("bf16", "xfast", 512, [(4096, 1024, "bf16"), (1024, 4096, "bf16")], 2048, False),
    ("bf16", "xfast", 256, [(1300, 600, "bf16"), (1300, 1100, "bf16")], 2048, True),
    ("bf16", "xmem", 256, [(600, 520, "bf16"), (256, 300, "bf16")], 300, False),
    ("bf16", "xout", 512, [(1024, 1536, "bf16"), (600, 520, "bf16")], 256, False),
    ("f32", "xfast", 32, [(96, 50, "f32"), (33, 64, "f32")], 70, False),
]


@pytest.mark.parametrize("act,mode,b,shapes,T,shared", CASES)
def test_group_calls_bit_identical(act, mode, b, shapes, T, shared):
    print(f"group calls act={act} mode={mode} b={b} shapes={shapes} T={T} shared={shared}", flush=True)
    inps = [custom_linear_inputs(m, n, b, T, act, w, 0.05, seed=13 * m + n + i) for i, (m, n, w) in enumerate(shapes)]
    single, grouped = [make_layer(inp, mode) for inp in inps], [make_layer(inp, mode) for inp in inps]
    ga, gb = PoetxGroup(single, batch_grads=True), PoetxGroup(grouped, batch_grads=True)
    ga.build()
    gb.build()
    X0 = dev(inps[0].X, act)
    Xs = [X0 if shared else dev(inp.X, act) for inp in inps]
    dZs = [dev(inp.dZ, act) for inp in inps]
    idx = list(range(len(inps)))
    Ya = [lay.forward(X) for lay, X in zip(single, Xs)]
    Yb = gb.forward(idx, Xs)
    out_y = mode == "xout"
    dXa = [ga.backward_dx(i, X, dZ, Y=Y if out_y else None) for i, X, dZ, Y in zip(idx, Xs, dZs, Ya)]
    dXb = gb.backward_dx_many(idx, dZs, Ys=Yb if out_y else None)
    dqa, dqb = ga.backward_q(), gb.backward_q()
    torch.cuda.synchronize()
    for i in idx:
        assert torch.equal(Ya[i], Yb[i]), f"linear {i}: Y differs from its own forward"
        assert torch.equal(dXa[i], dXb[i]), f"linear {i}: dX differs from its own backward"
        for k, side in enumerate("RP"):
            assert torch.equal(dqa[i][k], dqb[i][k]), f"linear {i}: dq_{side} differs"


def test_group_call_arguments():
    inps = [custom_linear_inputs(m, n, 64, 64, "bf16", "bf16", 0.05, seed=m) for m, n in [(128, 64), (64, 128)]]
    group = PoetxGroup([make_layer(inp) for inp in inps], batch_grads=True)
    X0, X1 = dev(inps[0].X, "bf16"), dev(inps[1].X, "bf16")
    with pytest.raises(ValueError):
        group.forward([0, 0], [X0, X0])  # the same linear twice
    with pytest.raises(ValueError):
        group.forward([0, 1], [X0])  # one input short
    with pytest.raises(ValueError):
        group.forward([0, 1], [X0, X1[:32]])  # different T
    with pytest.raises(ValueError):
        group.forward([0, 1], [X1, X0])  # inputs of the wrong width
    Y0, Y1 = group.forward([0, 1], [X0, X1])
    dZ0, dZ1 = dev(inps[0].dZ, "bf16"), dev(inps[1].dZ, "bf16")
    with pytest.raises(ValueError):
        group.backward_dx_many([0, 1], [dZ0[:32], dZ1[:32]])  # T differs from the forwards'
    dX0, dX1 = group.backward_dx_many([0, 1], [dZ0, dZ1])
    group.backward_q()
    torch.cuda.synchronize()
    assert dX0.shape == (64, 128) and dX1.shape == (64, 64)


@pytest.mark.parametrize(
    "act,b,shapes,T",
    [("bf16", 512, [(1024, 2048), (1024, 1024), (1024, 1024)], 1024), ("bf16", 256, [(600, 520), (600, 300)], 300),
     ("f32", 32, [(96, 50), (96, 64)], 70)],
)
def test_group_shared_dx_is_the_sum(act, b, shapes, T):
    """Linears that read one input and pass one dX tensor receive the sum of their input gradients: within
    the rounding of the separate bf16 results (each off by at most half a unit of its own value, the sum
    rounded once), and within 1e-6 in fp32; the block gradients, and so dq, do not change."""
    print(f"group shared dX act={act} b={b} shapes={shapes} T={T}", flush=True)
    inps = [custom_linear_inputs(m, n, b, T, act, act, 0.05, seed=29 * m + n + i) for i, (m, n) in enumerate(shapes)]
    single, grouped = [make_layer(inp) for inp in inps], [make_layer(inp) for inp in inps]
    ga, gb = PoetxGroup(single, batch_grads=True), PoetxGroup(grouped, batch_grads=True)
    ga.build()
    gb.build()
    X = dev(inps[0].X, act)
    dZs = [dev(inp.dZ, act) for inp in inps]
    idx = list(range(len(inps)))
    for lay in single:
        lay.forward(X)
    gb.forward(idx, [X] * len(idx))
    dXa = [ga.backward_dx(i, X, dZ) for i, dZ in zip(idx, dZs)]
    D = torch.empty_like(dXa[0])
    out = gb.backward_dx_many(idx, dZs, dXs=[D] * len(idx))
    assert all(o is D for o in out)
    dqa, dqb = ga.backward_q(), gb.backward_q()
    torch.cuda.synchronize()
    parts = torch.stack([x.double() for x in dXa])
    want, got = parts.sum(0), D.double()
    if act == "bf16":
        bound = 2.0 ** -8 * (parts.abs().sum(0) + got.abs()) + 1e-30
    else:
        bound = 1e-6 * (parts.abs().sum(0) + got.abs()) + 1e-30
    worst = ((got - want).abs() / bound).max().item()
    print(f"  summed dX: worst error / bound {worst:.3f}", flush=True)
    assert worst <= 1.0
    for i in idx:
        for k in range(2):
            assert torch.equal(dqa[i][k], dqb[i][k])

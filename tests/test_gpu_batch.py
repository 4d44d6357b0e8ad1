"""Batched CNP entry points (poetx_cnp_build_batch, poetx_linear_bwd_dx +
poetx_cnp_backward_batch, and its form poetx_cnp_backward_batch_reuse that
reads the build's dense Q and S, which the group uses after its build):
bit-identical to the per-side / per-linear calls, and the batched backward
checked against the fp64 oracle.

Sides of different lengths (partial last blocks, r = 2 .. b) share each batch,
so the block-to-side lookup of the kernels is exercised at its boundaries.
The batched block gradients (poetx_linear_bwd_dx_sides + poetx_block_grads_batch)
split the token range for the whole batch, so their dq is compared with the
per-linear calls to fp32 rounding and with the oracle."""

import numpy as np
import pytest
import torch

from orthogonal_reparameterized_cnp_amd import binding as B
from orthogonal_reparameterized_cnp_amd.layer import PoetxGroup
from tests.poetx_cases import assert_close, assert_dead_slots_zero, dev, host, make_layer, run_oracle
from workloads.gen import custom_linear_inputs

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


@pytest.mark.parametrize(
    "act,b,dims",
    [("bf16", 64, [256, 96, 300, 64, 130]), ("f32", 32, [96, 50, 33]), ("bf16", 512, [4096, 1024, 600, 14336])],
)
def test_cnp_build_batch_bit_identical(act, b, dims):
    print(f"cnp_build_batch act={act} b={b} dims={dims}", flush=True)
    adt = B.DTYPES[act]
    w = "f32" if act == "f32" else "bf16"
    u8 = dict(dtype=torch.uint8, device="cuda")
    qs, single, batch = [], [], []
    for i, d in enumerate(dims):
        inp = custom_linear_inputs(d, 1, b, 1, act, w, 0.05, seed=100 + i)
        q = dev(inp.q_R, "f32")
        qs.append(q)
        ws = torch.empty(B.poetx_workspace_size(B.desc(d, 1, b, act, w), 0, B.POETX_OP_CNP), **u8)
        g = torch.full((B.poetx_g_bytes(d, b, adt),), 7, **u8)
        B.poetx_cnp_build(q, d, b, adt, g, ws, ws.numel())
        single.append(g)
        batch.append(torch.full_like(g, 9))
    ws = torch.empty(B.poetx_cnp_batch_workspace_size(dims, b, adt), **u8)
    B.poetx_cnp_build_batch(qs, dims, b, adt, batch, ws, ws.numel())
    torch.cuda.synchronize()
    for d, g1, g2 in zip(dims, single, batch):
        assert torch.equal(g1, g2), f"side d={d}: batched G differs from the single build"


CASES = [
    ("bf16", 64, [(256, 96), (130, 200), (64, 64)], 300, True),
    ("f32", 32, [(96, 50), (33, 64)], 70, True),
    ("bf16", 512, [(1024, 1536), (600, 520)], 256, True),
    ("bf16", 512, [(4096, 1024), (4096, 4096), (14336, 4096)], 1024, False),
    # token-split block gradients: ragged T (one split), T = 6 * 64 (six splits of one K tile),
    # 11 and 5 K tiles over 6 and 3 splits (uneven), partial blocks
    ("bf16", 256, [(600, 520), (256, 300)], 300, True),
    ("bf16", 256, [(700, 256)], 384, True),
    ("bf16", 256, [(700, 256)], 704, True),
    ("bf16", 512, [(1024, 512)], 320, True),
]


@pytest.mark.parametrize("act,b,shapes,T,oracle", CASES)
def test_group_backward(act, b, shapes, T, oracle):
    _group_case(act, b, shapes, T, oracle, "xfast")


@pytest.mark.parametrize("act,b,shapes,T", [("bf16", 512, [(1024, 1536), (600, 520)], 256),
                                             ("bf16", 256, [(700, 256)], 384)])
def test_group_backward_xmem(act, b, shapes, T):
    """Grouped Xmem linears (H recomputed in backward_dx) against per-linear Xfast calls: bit-identical."""
    _group_case(act, b, shapes, T, False, "xmem")


@pytest.mark.parametrize("act,b,shapes,T", [("bf16", 512, [(1024, 1536), (600, 520)], 256)])
def test_group_backward_xout(act, b, shapes, T):
    """Grouped Xout linears (H taken back from Y in backward_dx) against per-linear Xout calls:
    bit-identical."""
    _group_case(act, b, shapes, T, False, "xout")


def _group_case(act, b, shapes, T, oracle, mode):
    print(f"group backward act={act} b={b} shapes={shapes} T={T} mode={mode}", flush=True)
    inps = [custom_linear_inputs(m, n, b, T, act, act, 0.05, seed=11 * m + n) for m, n in shapes]
    # per-side builds; Xmem against Xfast (bit-identical), Xout against Xout (its dq_P differs)
    single = [make_layer(inp, "xout" if mode == "xout" else "xfast") for inp in inps]
    grouped = [make_layer(inp, mode) for inp in inps]
    group = PoetxGroup(grouped)
    group.build()  # rebuild every side's G in one batch
    torch.cuda.synchronize()
    for a, g in zip(single, grouped):
        assert torch.equal(a.g_R, g.g_R) and torch.equal(a.g_P, g.g_P)
    outs = []
    for i, (inp, a, g) in enumerate(zip(inps, single, grouped)):
        X, dZ = dev(inp.X, inp.act), dev(inp.dZ, inp.act)
        Ya = a.forward(X)
        Yg = g.forward(X)
        out_y = mode == "xout"
        dX_a, dqR_a, dqP_a = a.backward(X, dZ, Y=Ya if out_y else None)
        dX_g = group.backward_dx(i, X, dZ, Y=Yg if out_y else None)
        outs.append((dX_a, dqR_a, dqP_a, dX_g))
    dqs = group.backward_q()
    torch.cuda.synchronize()
    for (dX_a, dqR_a, dqP_a, dX_g), (dqR_g, dqP_g) in zip(outs, dqs):
        assert torch.equal(dX_a, dX_g)
        assert torch.equal(dqR_a, dqR_g)
        assert torch.equal(dqP_a, dqP_g)
    if oracle:
        for inp, (_, _, _, dX_g), (dqR_g, dqP_g) in zip(inps, outs, dqs):
            ref = run_oracle(inp)
            assert_close("dX", host(dX_g, act), ref["dX"], act)
            assert_close("dq_R", host(dqR_g, "f32"), ref["dq_R"], act)
            assert_close("dq_P", host(dqP_g, "f32"), ref["dq_P"], act)


def test_backward_reads_saved_input_not_x():
    """The backward takes the gathered input from the forward's saved state: passing no X (or a
    different X) gives bit-identical results."""
    print("backward without X", flush=True)
    inp = custom_linear_inputs(520, 300, 256, 200, "bf16", "bf16", 0.05, seed=21)
    lay = make_layer(inp)
    X, dZ = dev(inp.X, "bf16"), dev(inp.dZ, "bf16")
    lay.forward(X)
    ref = [t.clone() for t in lay.backward(X, dZ)]
    T = X.shape[0]
    dX = torch.empty_like(ref[0])
    dq_R, dq_P = torch.empty_like(ref[1]), torch.empty_like(ref[2])
    B.poetx_linear_bwd(lay.desc, T, None, dZ, lay.perm_R, lay.perm_P, lay.Wt, lay.g_R, lay.g_P, lay.q_R, lay.q_P,
                       lay.H_save, dX, dq_R, dq_P, lay.ws, lay.ws.numel())
    torch.cuda.synchronize()
    assert torch.equal(dX, ref[0]) and torch.equal(dq_R, ref[1]) and torch.equal(dq_P, ref[2])


BATCH_GRAD_CASES = [
    # full blocks over several linears (one shared token split), ragged T, partial blocks, fp32
    ("bf16", 512, [(4096, 1024), (4096, 4096), (14336, 4096)], 1024, False),
    ("bf16", 512, [(1024, 1536), (600, 520)], 256, True),
    ("bf16", 256, [(600, 520), (256, 300)], 300, True),
    ("bf16", 256, [(700, 256)], 704, True),
    ("f32", 32, [(96, 50), (33, 64)], 70, True),
]


@pytest.mark.parametrize("act,b,shapes,T,oracle", BATCH_GRAD_CASES)
def test_group_batch_grads(act, b, shapes, T, oracle):
    """Block gradients of every side in shared launches (poetx_block_grads_batch): dX bit-identical to the
    per-linear calls, dq close to theirs, and within the usual bounds of the oracle.  The two differ only
    in the fp32 order of the token-split sums of U; in bf16 the chain rule reads U rounded to bf16, where
    such a difference can move an element by one unit (2^-8 relative), hence the bf16 bound."""
    print(f"group batch_grads act={act} b={b} shapes={shapes} T={T}", flush=True)
    inps = [custom_linear_inputs(m, n, b, T, act, act, 0.05, seed=7 * m + n) for m, n in shapes]
    single = [make_layer(inp) for inp in inps]
    grouped = [make_layer(inp) for inp in inps]
    group = PoetxGroup(grouped, batch_grads=True)
    group.build()
    outs = []
    for i, (inp, a, g) in enumerate(zip(inps, single, grouped)):
        X, dZ = dev(inp.X, inp.act), dev(inp.dZ, inp.act)
        a.forward(X)
        g.forward(X)
        dX_a, dqR_a, dqP_a = a.backward(X, dZ)
        dX_g = group.backward_dx(i, X, dZ)
        outs.append((dX_a, dqR_a, dqP_a, dX_g))
    dqs = group.backward_q()
    torch.cuda.synchronize()
    for (dX_a, dqR_a, dqP_a, dX_g), (dqR_g, dqP_g) in zip(outs, dqs):
        assert torch.equal(dX_a, dX_g)
        for name, x, y in (("dq_R", dqR_g, dqR_a), ("dq_P", dqP_g, dqP_a)):
            x, y = x.double().cpu(), y.double().cpu()
            rel = ((x - y).norm() / max(y.norm().item(), 1e-30)).item()
            print(f"  {name}: relative difference to the per-linear call {rel:.2e}", flush=True)
            assert rel <= (2e-3 if act == "bf16" else 1e-5), f"{name}: {rel:.2e}"
    for inp, (dqR_g, dqP_g) in zip(inps, dqs):
        assert_dead_slots_zero("dq_R", dqR_g, inp.m, inp.b)
        assert_dead_slots_zero("dq_P", dqP_g, inp.n, inp.b)
    if oracle:
        for inp, (_, _, _, dX_g), (dqR_g, dqP_g) in zip(inps, outs, dqs):
            ref = run_oracle(inp)
            assert_close("dX", host(dX_g, act), ref["dX"], act)
            assert_close("dq_R", host(dqR_g, "f32"), ref["dq_R"], act)
            assert_close("dq_P", host(dqP_g, "f32"), ref["dq_P"], act)


def test_group_batch_grads_needs_every_linear():
    inps = [custom_linear_inputs(m, n, 64, 64, "bf16", "bf16", 0.05, seed=m) for m, n in [(128, 64), (64, 128)]]
    group = PoetxGroup([make_layer(inp) for inp in inps], batch_grads=True)
    X, dZ = dev(inps[0].X, "bf16"), dev(inps[0].dZ, "bf16")
    group.layers[0].forward(X)
    group.backward_dx(0, X, dZ)
    with pytest.raises(ValueError):
        group.backward_q()


def test_group_chain_rule_with_and_without_the_group_build():
    """backward_q reads the dense Q and S of the group build that came before it, once; without a group
    build (the G built per linear) it forms them itself.  Both give the per-linear dq bit for bit."""
    shapes, b, T = [(600, 520), (256, 300)], 256, 300
    inps = [custom_linear_inputs(m, n, b, T, "bf16", "bf16", 0.05, seed=5 * m + n) for m, n in shapes]
    single = [make_layer(inp) for inp in inps]
    grouped = [make_layer(inp) for inp in inps]  # each built per linear
    group = PoetxGroup(grouped)
    refs = []
    for inp, a in zip(inps, single):
        X, dZ = dev(inp.X, "bf16"), dev(inp.dZ, "bf16")
        a.forward(X)
        refs.append(a.backward(X, dZ)[1:])

    def step():
        for i, (inp, g) in enumerate(zip(inps, grouped)):
            X, dZ = dev(inp.X, "bf16"), dev(inp.dZ, "bf16")
            g.forward(X)
            group.backward_dx(i, X, dZ)
        return group.backward_q()

    for use_group_build in (False, True, False):
        if use_group_build:
            group.build()
        assert group.built == use_group_build
        dqs = step()
        torch.cuda.synchronize()
        assert not group.built  # a group build serves one backward_q
        for (dqR, dqP), (rR, rP) in zip(dqs, refs):
            assert torch.equal(dqR, rR) and torch.equal(dqP, rP), f"group build {use_group_build}"

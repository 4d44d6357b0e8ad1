"""The layer's CNP build, forward and backward captured into one HIP graph
(torch.cuda.CUDAGraph on the library's stream) and replayed: every replay,
with eager work and synchronisations between them, must reproduce the eager
results bit for bit.  The calls allocate nothing and record no memsets, so
the captured launches are the eager ones."""

from __future__ import annotations

import pytest
import torch

from orthogonal_reparameterized_cnp_amd.layer import PoetxGroup
from tests.poetx_cases import dev, make_layer
from workloads.gen import custom_linear_inputs

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


@pytest.mark.parametrize(
    "m,n,b,T,act,w,mode",
    [
        (320, 200, 64, 96, "bf16", "bf16", "xfast"),   # register loops, partial blocks
        (1024, 1536, 512, 512, "bf16", "bf16", "xfast"),  # direct-to-LDS contractions, streamed block products
        (1024, 1536, 512, 512, "bf16", "bf16", "xout"),
        (512, 384, 128, 256, "bf16", "i8", "xmem"),
        (96, 64, 32, 40, "f32", "f32", "xfast"),
    ],
)
def test_layer_step_replays_in_a_graph(m, n, b, T, act, w, mode):
    print(f"graph {m}x{n} b={b} T={T} {act}/{w} {mode}", flush=True)
    inp = custom_linear_inputs(m, n, b, T, act, w, 0.02, seed=51)
    lay = make_layer(inp, mode)
    X, dZ = dev(inp.X, act), dev(inp.dZ, act)
    Y = torch.empty(T, n, dtype=X.dtype, device="cuda")
    dX = torch.empty(T, m, dtype=X.dtype, device="cuda")
    dq_R, dq_P = torch.empty_like(lay.q_R), torch.empty_like(lay.q_P)
    outs = (Y, dX, dq_R, dq_P)

    def step():
        lay.build()
        lay.forward(X, Y)
        lay.backward(X, dZ, dX, dq_R, dq_P, Y=Y if mode == "xout" else None)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for k in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("Y", "dX", "dq_R", "dq_P"), outs, ref):
            assert torch.equal(got.view(torch.uint8) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.uint8) if want.dtype == torch.bfloat16 else want), \
                f"replay {k}: {name} differs from the eager result"


@pytest.mark.parametrize("batch_grads", [False, True])
def test_group_step_replays_in_a_graph(batch_grads):
    """Several linears with the batched CNP calls (the benchmark's step shape, small), with the block
    gradients per linear or in one batch after the backwards (the eager step before the capture sizes
    the batch's workspace, so the capture allocates nothing)."""
    shapes = [(256, 256), (256, 128), (512, 256)]
    b, T, act = 128, 128, "bf16"
    lays, Xs, dZs = [], [], []
    for i, (m, n) in enumerate(shapes):
        inp = custom_linear_inputs(m, n, b, T, act, "bf16", 0.02, seed=60 + i)
        lays.append(make_layer(inp))
        Xs.append(dev(inp.X, act))
        dZs.append(dev(inp.dZ, act))
    group = PoetxGroup(lays, batch_grads=batch_grads)
    Ys = [torch.empty(T, l.n, dtype=torch.bfloat16, device="cuda") for l in lays]
    dXs = [torch.empty(T, l.m, dtype=torch.bfloat16, device="cuda") for l in lays]
    dqs = [(torch.empty_like(l.q_R), torch.empty_like(l.q_P)) for l in lays]

    def step():
        group.build()
        for l, X, Y in zip(lays, Xs, Ys):
            l.forward(X, Y)
        for i in reversed(range(len(lays))):
            group.backward_dx(i, Xs[i], dZs[i], dXs[i])
        group.backward_q(dqs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    flat = Ys + dXs + [x for p in dqs for x in p]
    ref = [t.clone() for t in flat]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for k in range(3):
        for t in flat:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(flat, ref):
            assert torch.equal(got.view(torch.uint8) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.uint8) if want.dtype == torch.bfloat16 else want), f"replay {k}"


def test_chain_step_replays_in_a_graph():
    """Two factors per side (a fully stochastic and a block-stochastic outer
    factor around the linear): the SPO calls capture like the layer calls."""
    from orthogonal_reparameterized_cnp_amd.layer import PoetxChain, PoetxSpoFactor
    from workloads.gen import spo_inputs

    m, n, b, T, act = 320, 200, 64, 96, "bf16"
    inp = custom_linear_inputs(m, n, b, T, act, "bf16", 0.02, seed=71)
    lin = make_layer(inp)
    facs = []
    for d, kind, seed in ((m, "full", 72), (n, "block", 73)):
        si = spo_inputs(d, b, kind, T, act, 0.02, seed=seed)
        f = PoetxSpoFactor(d, b, kind, act)
        f.load(dev(si.idx, "i32"), dev(si.q, "f32"))
        facs.append(f)
    chain = PoetxChain(lin, [facs[0]], [facs[1]])
    X, dZ = dev(inp.X, act), dev(inp.dZ, act)
    res = {}

    def step():
        chain.build()
        res["Y"] = chain.forward(X)
        res["dX"], res["dq_oR"], res["dq_lin"], res["dq_oP"] = chain.backward(dZ)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (res["Y"], res["dX"], res["dq_oR"][0], *res["dq_lin"], res["dq_oP"][0])]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    outs = (res["Y"], res["dX"], res["dq_oR"][0], *res["dq_lin"], res["dq_oP"][0])
    for k in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got.view(torch.uint8) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.uint8) if want.dtype == torch.bfloat16 else want), f"replay {k}"

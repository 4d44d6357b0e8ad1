"""Parity with the fp64 oracle at the workloads' full sizes, in the launch
configurations the benchmark times (256 x 256 direct-to-LDS contractions,
row-streamed block products at b = 256 and 512, one-row gathers), plus the
paths that only full sizes reach: a ragged 5461-wide edge with K = 5461 on the
256 x 256 register loop, the b = 512 paths on an exact identity, and the merge
of a Llama-13B int8 layer.

The oracle recomputes what it can afford at these sizes: sampled token rows of
Y and dX (each row depends on that row of the input only) and sampled blocks of
dq_R, dq_P, each a sum over all tokens (including a partial last block)."""

import numpy as np
import pytest
import torch

import oracle as O
from tests.poetx_cases import (assert_close, assert_dead_slots_zero, compare_layer, dev, host, make_layer, run_gpu,
                               run_oracle)
from workloads import WORKLOADS, make_linear_inputs
from workloads.gen import custom_linear_inputs

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

FULL = [(wl, lin) for wl in ("llama8b", "llama13b_int8", "llama1p3b") for lin in range(7)]


@pytest.mark.parametrize("wl,lin", FULL, ids=[f"{w}-{l}" for w, l in FULL])
def test_full_size_sampled(wl, lin):
    W_ = WORKLOADS[wl]
    print(f"full size {wl} linear {lin} ({W_.linears[lin].m}x{W_.linears[lin].n}, T={W_.T})", flush=True)
    inp = make_linear_inputs(W_, lin)
    out = run_gpu(inp)
    kind = inp.act
    rng = np.random.default_rng(100 + lin)
    rows = np.sort(rng.choice(inp.T, 32, replace=False))
    X = O.to_f64(inp.X[rows], kind)
    dZ = O.to_f64(inp.dZ[rows], kind)
    W = O.to_f64(inp.W0, inp.w, inp.w_scale)
    q_R, q_P = inp.q_R.astype(np.float64), inp.q_P.astype(np.float64)
    G_R, G_P = O.side_G(q_R, inp.m, inp.b), O.side_G(q_P, inp.n, inp.b)
    f = O.forward(X, W, inp.perm_R, inp.perm_P, G_R, G_P)
    assert_close("Y rows", host(out["Y"], kind)[rows], f.Y, kind)
    g = O.backward(X, dZ, W, inp.perm_R, inp.perm_P, q_R, q_P, inp.b)
    assert_close("dX rows", host(out["dX"], kind)[rows], g.dX, kind)
    del f, g
    nbR, nbP = inp.q_R.shape[0], inp.q_P.shape[0]
    bR, bP = sorted({0, nbR - 1}), sorted({nbP // 2, nbP - 1})
    ref = O.block_grads(O.to_f64(inp.X, kind), O.to_f64(inp.dZ, kind), W, inp.perm_R, inp.perm_P, q_R, q_P, inp.b,
                        bR, bP)
    dqR, dqP = host(out["dq_R"], "f32"), host(out["dq_P"], "f32")
    for k in bR:
        assert_close(f"dq_R[{k}]", dqR[k], ref[("R", k)], kind)
    for k in bP:
        assert_close(f"dq_P[{k}]", dqP[k], ref[("P", k)], kind)
    assert_dead_slots_zero("dq_R", out["dq_R"], inp.m, inp.b)
    assert_dead_slots_zero("dq_P", out["dq_P"], inp.n, inp.b)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def test_identity_bit_exact_b512():
    """W0 = I and q = 0 at 4096 x 4096, b = 512, 1024 tokens: the streamed block products,
    the 256 x 256 direct-to-LDS contractions and the one-row gathers and scatters must
    reproduce Y = X and dX = dZ bit for bit (every product multiplies by 1 or 0)."""
    m, T = 4096, 1024
    print(f"identity m=n={m} b=512 T={T}", flush=True)
    inp = custom_linear_inputs(m, m, 512, T, "bf16", "bf16", 0.0, seed=41)
    inp.W0 = np.zeros((m, m), dtype=np.uint16)
    inp.W0[np.arange(m), np.arange(m)] = 0x3F80
    inp.q_R[:] = 0
    inp.q_P[:] = 0
    out = run_gpu(inp)
    np.testing.assert_array_equal(_bits(out["Y"]), _bits(dev(inp.X, "bf16")))
    np.testing.assert_array_equal(_bits(out["dX"]), _bits(dev(inp.dZ, "bf16")))


def test_ragged_wide_register_loop():
    """A forward contraction with 16 x 17 = 272 output tiles of 256 x 256 (enough to take the
    256-wide tile), a ragged last tile column (n = 4100) and K = 1300, not a multiple of 64:
    every tile runs the 256 x 256 register loop with its bounds checks."""
    print("ragged 1300x4100 b=256 T=4096", flush=True)
    inp = custom_linear_inputs(1300, 4100, 256, 4096, "bf16", "bf16", 0.01, seed=17)
    compare_layer(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("lin", [0, 4, 6])
def test_merge_full_size_int8(lin):
    """poetx_merge_reinit of a Llama-13B int8 linear at its full shape against the oracle's
    merge (R W P with the CNP blocks, new permutations), and the int8 requantisation of the
    same fp32 values, bit for bit."""
    wl = WORKLOADS["llama13b_int8"]
    inp = make_linear_inputs(wl, lin, T=1, with_dz=False)
    m, n, b = inp.m, inp.n, inp.b
    print(f"merge llama13b_int8 linear {lin} ({m}x{n})", flush=True)
    lay = make_layer(inp)
    seed_R, seed_P = 7000 + lin, 8000 + lin
    lay.merge_reinit(seed_R, seed_P)
    torch.cuda.synchronize()
    newR, newP = O.perm_from_seed(seed_R, m), O.perm_from_seed(seed_P, n)
    np.testing.assert_array_equal(lay.perm_R.cpu().numpy(), newR)
    np.testing.assert_array_equal(lay.perm_P.cpu().numpy(), newP)
    assert not lay.q_R.any() and not lay.q_P.any()
    Wq = lay.merged_f32().cpu().numpy()[:, :n]
    G_R = O.side_G(inp.q_R.astype(np.float64), m, b)
    G_P = O.side_G(inp.q_P.astype(np.float64), n, b)
    Wt_old = O.premerge(O.to_f64(inp.W0, "i8", inp.w_scale), inp.perm_R, inp.perm_P)
    ref = O.merge_reinit(Wt_old, inp.perm_R, inp.perm_P, G_R, G_P, seed_R, seed_P)
    del Wt_old
    # the products run in fp32, but the blocks enter as the layer's bf16 G - I, so the bound is bf16's
    assert_close("merged W", Wq.astype(np.float64), ref.Wt_new, "bf16")
    code, scale = O.quantize_int8_f32(Wq)
    np.testing.assert_array_equal(lay.weight_values()[:, :n].cpu().numpy(), code)
    np.testing.assert_array_equal(lay.weight_scales()[:n].cpu().numpy(), scale)


@pytest.mark.parametrize("wl", ["llama8b", "llama1p3b"])
def test_layer_batched_grads_full_size(wl):
    """The decoder layer as the benchmark runs it: the block gradients of all 14 sides in shared launches
    (one token split for the whole batch) after the seven backwards.  dX is bit-identical to the
    per-linear calls and dq matches theirs to the bf16 rounding of U (the per-linear results are
    checked against the oracle above); one dq block per side of the widest linear is also checked
    against the oracle directly."""
    from orthogonal_reparameterized_cnp_amd.layer import PoetxGroup

    W_ = WORKLOADS[wl]
    print(f"batched block gradients {wl}, T={W_.T}", flush=True)
    inps = [make_linear_inputs(W_, i) for i in range(len(W_.linears))]
    lays = [make_layer(inp) for inp in inps]
    group = PoetxGroup(lays, batch_grads=True)
    group.build()
    Xs = [dev(inp.X, inp.act) for inp in inps]
    dZs = [dev(inp.dZ, inp.act) for inp in inps]
    for lay, X in zip(lays, Xs):
        lay.forward(X)
    dXs = [None] * len(lays)
    for i in reversed(range(len(lays))):
        dXs[i] = group.backward_dx(i, Xs[i], dZs[i])
    dqs = group.backward_q()
    torch.cuda.synchronize()
    for i, (inp, lay) in enumerate(zip(inps, lays)):
        dX_a, dqR_a, dqP_a = lay.backward(Xs[i], dZs[i])
        assert torch.equal(dX_a, dXs[i]), f"linear {i}: dX differs from the per-linear call"
        for name, x, y in (("dq_R", dqs[i][0], dqR_a), ("dq_P", dqs[i][1], dqP_a)):
            x, y = x.double().cpu(), y.double().cpu()
            rel = ((x - y).norm() / max(y.norm().item(), 1e-30)).item()
            print(f"  linear {i} {name}: relative difference to the per-linear call {rel:.2e}", flush=True)
            assert rel <= 2e-3, f"linear {i} {name}: {rel:.2e}"
        assert_dead_slots_zero("dq_R", dqs[i][0], inp.m, inp.b)
        assert_dead_slots_zero("dq_P", dqs[i][1], inp.n, inp.b)
    # the oracle on the widest linear (gate): the last block of each side
    gi = max(range(len(inps)), key=lambda i: inps[i].m * inps[i].n)
    inp = inps[gi]
    W = O.to_f64(inp.W0, inp.w, inp.w_scale)
    q_R, q_P = inp.q_R.astype(np.float64), inp.q_P.astype(np.float64)
    bR, bP = [inp.q_R.shape[0] - 1], [inp.q_P.shape[0] - 1]
    ref = O.block_grads(O.to_f64(inp.X, inp.act), O.to_f64(inp.dZ, inp.act), W, inp.perm_R, inp.perm_P, q_R, q_P,
                        inp.b, bR, bP)
    assert_close(f"dq_R[{bR[0]}]", host(dqs[gi][0], "f32")[bR[0]], ref[("R", bR[0])], inp.act)
    assert_close(f"dq_P[{bP[0]}]", host(dqs[gi][1], "f32")[bP[0]], ref[("P", bP[0])], inp.act)

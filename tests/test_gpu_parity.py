"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the same
seeded inputs.  Needs an MI355X; every test is marked `gpu`."""

import numpy as np
import pytest
import torch

import oracle as O
from orthogonal_reparameterized_cnp_amd.layer import lead
from tests.poetx_cases import TOL, assert_close, compare_layer, dev, host, make_layer, run_gpu, run_oracle
from workloads import WORKLOADS, make_linear_inputs
from workloads.gen import custom_linear_inputs

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.numpy()


# ----------------------------------------------------------------------------
# CNP block builder
# ----------------------------------------------------------------------------
@pytest.mark.parametrize(
    "d,b,act,std",
    [(256, 32, "f32", 0.02), (200, 64, "f32", 0.05), (200, 64, "bf16", 0.05), (1376, 256, "bf16", 0.01),
     (1024, 512, "bf16", 0.005), (5461, 256, "bf16", 0.01)],
)
def test_cnp_build(d, b, act, std):
    inp = custom_linear_inputs(d, d, b, 1, act, "f32" if act == "f32" else "bf16", std, seed=d + b)
    lay = make_layer(inp)
    torch.cuda.synchronize()
    g = lay.g_slices("R")
    delta, delta_t = host(g[0], act), host(g[1], act)
    for k, (s, r) in enumerate(O.side_blocks(d, b)):
        Q = O.unpack_skew(inp.q_R[k].astype(np.float64), r, b)
        ref = O.cnp(Q) - np.eye(r)
        assert_close(f"Delta[{k}]", delta[k, :r, :r], ref, act)
        assert np.array_equal(delta_t[k], delta[k].T), "slice 1 must be the exact transpose of slice 0"
        assert not delta[k, r:, :].any() and not delta[k, :, r:].any(), "entries outside the live block must be 0"


# ----------------------------------------------------------------------------
# pre-merge: pure data movement, bit-exact
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("w,act", [("f32", "f32"), ("bf16", "bf16"), ("i8", "bf16")])
def test_premerge_bit_exact(w, act):
    inp = custom_linear_inputs(300, 131, 64, 1, act, w, 0.01, seed=7)
    lay = make_layer(inp)
    torch.cuda.synchronize()
    got = _bits(lay.weight_values())[:, : inp.n]
    want = np.ascontiguousarray(O.premerge(inp.W0, inp.perm_R, inp.perm_P))
    if w == "bf16":
        want = want.view(np.int16)
    np.testing.assert_array_equal(got, want)
    if w == "bf16":
        # the transposed copy the forward reads: exact transpose, zero past column m
        wt = _bits(lay.weight_t())
        np.testing.assert_array_equal(wt[:, : inp.m], want.T)
        assert not wt[:, inp.m :].any()
    if w == "i8":
        np.testing.assert_array_equal(_bits(lay.weight_scales())[: inp.n], inp.w_scale[inp.perm_P])


# ----------------------------------------------------------------------------
# exactness: W0 = I and q = 0 make every product multiply by 1 and add exact zeros
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("act,b", [("f32", 64), ("bf16", 64), ("bf16", 48)])
def test_identity_weight_bit_exact(act, b):
    m = 192
    inp = custom_linear_inputs(m, m, b, 70, act, act, 0.0, seed=3)
    eye = np.eye(m, dtype=np.float32)
    inp.W0 = eye if act == "f32" else (eye.view(np.uint32) >> 16).astype(np.uint16)
    inp.q_R[:] = 0
    inp.q_P[:] = 0
    out = run_gpu(inp)
    np.testing.assert_array_equal(_bits(out["Y"]), _bits(dev(inp.X, act)))
    np.testing.assert_array_equal(_bits(out["dX"]), _bits(dev(inp.dZ, act)))


# ----------------------------------------------------------------------------
# whole layer at the workloads' shapes
# ----------------------------------------------------------------------------
def test_layer_linear256_fp32():
    inp = make_linear_inputs(WORKLOADS["linear256_fp32"], 0)
    compare_layer(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("lin", range(7))
def test_layer_llama60m(lin):
    inp = make_linear_inputs(WORKLOADS["llama60m"], lin)
    compare_layer(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("lin", [0, 4, 6])
def test_layer_llama1p3b_odd_width(lin):
    inp = make_linear_inputs(WORKLOADS["llama1p3b"], lin, T=512)
    compare_layer(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize(
    "m,n,b,T,act",
    [(200, 131, 64, 77, "bf16"), (200, 131, 64, 77, "f32"), (96, 300, 32, 1, "bf16"), (130, 130, 128, 300, "bf16"),
     (64, 64, 64, 513, "bf16"), (33, 17, 8, 5, "f32"), (520, 1030, 256, 260, "bf16"),
     # block sizes that are not a multiple of 8: every b x b row pitch is odd, so the 16-byte epilogue
     # stores fall back to element stores (and a partial last block of 1 column on the P side)
     (111, 75, 37, 50, "bf16"), (45, 79, 13, 9, "f32"),
     # row-streamed block products (enough row tiles): ragged T and a partial last block of b = 256 / 512
     (2048, 1300, 256, 1000, "bf16"), (1536, 2600, 512, 700, "bf16")],
)
def test_layer_ragged(m, n, b, T, act):
    inp = custom_linear_inputs(m, n, b, T, act, act, 0.05, seed=m * 7 + n)
    compare_layer(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("m,n,T", [(1024, 1536, 256), (600, 520, 100), (2048, 2560, 600)])
def test_layer_int8(m, n, T):
    inp = custom_linear_inputs(m, n, 512 if m >= 1024 else 128, T, "bf16", "i8", 0.005, seed=m + n)
    compare_layer(inp, run_gpu(inp), run_oracle(inp))


# ----------------------------------------------------------------------------
# Xmem (H recomputed in the backward): bit-identical to Xfast
# ----------------------------------------------------------------------------
@pytest.mark.parametrize(
    "m,n,b,T,act,w",
    [(520, 1030, 256, 260, "bf16", "bf16"), (600, 520, 128, 100, "bf16", "i8"), (200, 131, 64, 77, "f32", "f32"),
     (1024, 1536, 512, 512, "bf16", "bf16")],
)
def test_xmem_matches_xfast(m, n, b, T, act, w):
    inp = custom_linear_inputs(m, n, b, T, act, w, 0.02, seed=m + n + T)
    fast = run_gpu(inp, mode="xfast")
    mem = run_gpu(inp, mode="xmem")
    for k in ("Y", "dX", "dq_R", "dq_P"):
        assert torch.equal(_bits_t(fast[k]), _bits_t(mem[k])), f"{k} differs between xfast and xmem"
    # the xmem saved state is the gathered input alone: X[:, perm_R], bit for bit
    lay = mem["layer"]
    Xt = lay.H_save.view(_dt(act))[: T * lead(m)].view(T, lead(m))[:, :m]
    want = dev(inp.X, act)[:, torch.from_numpy(inp.perm_R.astype(np.int64)).cuda()]
    assert torch.equal(_bits_t(Xt), _bits_t(want))


def _dt(act):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[act]


def _bits_t(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# ----------------------------------------------------------------------------
# Xout (H taken back from the output, the checkpoint b = G_P z) against the
# oracle's h_output backward; dX and dq_R bit-identical to Xfast
# ----------------------------------------------------------------------------
@pytest.mark.parametrize(
    "m,n,b,T,act,w",
    [(520, 1030, 256, 260, "bf16", "bf16"), (2048, 2560, 512, 600, "bf16", "i8"), (200, 131, 64, 77, "f32", "f32"),
     (1024, 1536, 512, 512, "bf16", "bf16")],
)
def test_xout_matches_oracle(m, n, b, T, act, w):
    print(f"xout m={m} n={n} b={b} T={T} act={act} w={w}", flush=True)
    inp = custom_linear_inputs(m, n, b, T, act, w, 0.02, seed=m + 3 * n + T)
    out = run_gpu(inp, mode="xout")
    ref = run_oracle(inp, h_output=True)
    kind = inp.act
    assert_close("Y", host(out["Y"], kind), ref["Y"], kind)
    assert_close("dX", host(out["dX"], kind), ref["dX"], kind)
    assert_close("dq_R", host(out["dq_R"], "f32"), ref["dq_R"], kind)
    assert_close("dq_P", host(out["dq_P"], "f32"), ref["dq_P"], kind)
    fast = run_gpu(inp, mode="xfast")
    for k in ("Y", "dX", "dq_R"):
        assert torch.equal(out[k], fast[k]), k


def test_empty_batch():
    inp = custom_linear_inputs(128, 96, 32, 1, "bf16", "bf16", 0.01, seed=5)
    lay = make_layer(inp)
    X = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    Y = lay.forward(X)
    dX, dq_R, dq_P = lay.backward(X, torch.empty(0, 96, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert Y.shape == (0, 96)
    assert not dq_R.any() and not dq_P.any()


def test_backward_is_deterministic():
    inp = make_linear_inputs(WORKLOADS["llama60m"], 4)
    lay = make_layer(inp)
    X, dZ = dev(inp.X, "bf16"), dev(inp.dZ, "bf16")
    lay.forward(X)
    a = [t.clone() for t in lay.backward(X, dZ)]
    b = [t.clone() for t in lay.backward(X, dZ)]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        np.testing.assert_array_equal(_bits(x), _bits(y))


# ----------------------------------------------------------------------------
# merge-then-reinitialise
# ----------------------------------------------------------------------------
@pytest.mark.parametrize(
    "m,n,b,act,w,std",
    [(256, 256, 32, "f32", "f32", 0.02), (300, 131, 64, "bf16", "bf16", 0.02), (1024, 1536, 512, "bf16", "i8", 0.005),
     (520, 200, 128, "bf16", "i8", 0.01)],
)
def test_merge_reinit(m, n, b, act, w, std):
    inp = custom_linear_inputs(m, n, b, 64, act, w, std, seed=m + 3 * n)
    lay = make_layer(inp)
    X = dev(inp.X, act)
    Y0 = host(lay.forward(X), act)
    seed_R, seed_P = 1000 + m, 2000 + n
    lay.merge_reinit(seed_R, seed_P)
    torch.cuda.synchronize()
    newR, newP = O.perm_from_seed(seed_R, m), O.perm_from_seed(seed_P, n)
    np.testing.assert_array_equal(lay.perm_R.cpu().numpy(), newR)
    np.testing.assert_array_equal(lay.perm_P.cpu().numpy(), newP)
    assert not lay.q_R.any() and not lay.q_P.any()
    # fp32 merged weight before rounding, new pre-merged order
    Wq = lay.merged_f32().cpu().numpy()[:, :n]
    G_R = O.side_G(inp.q_R.astype(np.float64), m, b)
    G_P = O.side_G(inp.q_P.astype(np.float64), n, b)
    Wt_old = O.premerge(O.to_f64(inp.W0, w, inp.w_scale), inp.perm_R, inp.perm_P)
    ref = O.merge_reinit(Wt_old, inp.perm_R, inp.perm_P, G_R, G_P, seed_R, seed_P)
    assert_close("merged W", Wq.astype(np.float64), ref.Wt_new, act)
    # rounding / requantisation decided in fp32 on the same values
    vals = _bits(lay.weight_values())[:, :n]
    if w == "f32":
        np.testing.assert_array_equal(vals, Wq)
    elif w == "bf16":
        np.testing.assert_array_equal(vals.view(np.uint16), O.round_bf16(Wq.astype(np.float64)))
        np.testing.assert_array_equal(_bits(lay.weight_t())[:, :m], vals.T)
    else:
        code, scale = O.quantize_int8_f32(Wq)
        np.testing.assert_array_equal(vals, code)
        np.testing.assert_array_equal(_bits(lay.weight_scales())[:n], scale)
    # the layer function is unchanged by the merge (factors restart at the identity)
    lay.build()
    Y1 = host(lay.forward(X), act)
    lim = {"f32": 1e-5, "bf16": 1e-2}[act] if w != "i8" else 2e-2
    ma = np.linalg.norm(Y1 - Y0) / np.linalg.norm(Y0)
    print(f"  fwd after/before merge: rel fro {ma:.3e}")
    assert ma <= lim

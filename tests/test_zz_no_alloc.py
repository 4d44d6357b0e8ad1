"""poetx_cnp_build_noalloc (workspace in the library's fixed device array)
against poetx_cnp_build (caller workspace), through the C ABI: bit-identical G
buffers on consecutive calls, the second on a smaller side, so the second call
runs on scratch the first one left dirty."""

import numpy as np
import pytest
import torch

from orthogonal_reparameterized_cnp_amd import binding as B

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

ADT = {"f32": B.POETX_F32, "bf16": B.POETX_BF16}


def _q(d, b, std, seed):
    nb = -(-d // b)
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.standard_normal((nb, b * (b - 1) // 2)) * std).astype(np.float32)).cuda()


def _build_with_workspace(q, d, b, adt):
    g = torch.empty(B.poetx_g_bytes(d, b, adt), dtype=torch.uint8, device="cuda")
    need = B.poetx_workspace_size(B.desc(d, 1, b, "f32" if adt == B.POETX_F32 else "bf16",
                                         "f32" if adt == B.POETX_F32 else "bf16"), 0, B.POETX_OP_CNP)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    B.poetx_cnp_build(q, d, b, adt, g, ws, ws.numel())
    return g


@pytest.mark.parametrize(
    "cases",
    [
        # the largest side of the Llama-8B layer (28 blocks of 512), then a smaller ragged one
        [(14336, 512, "bf16", 0.005), (1376, 256, "bf16", 0.01)],
        # fp32 blocks, then a smaller side with a partial block
        [(512, 128, "f32", 0.02), (200, 64, "f32", 0.05)],
    ],
)
def test_noalloc_matches_cnp_build(cases):
    for i, (d, b, act, std) in enumerate(cases):
        print(f"noalloc call {i}: d={d} b={b} {act}", flush=True)
        adt = ADT[act]
        q = _q(d, b, std, seed=d + b)
        ref = _build_with_workspace(q, d, b, adt)
        g = torch.full_like(ref, 0xA5)  # every byte of G must be written
        B.poetx_cnp_build_noalloc(q, d, b, adt, g)
        torch.cuda.synchronize()
        assert torch.equal(g, ref), f"call {i}: G differs from poetx_cnp_build"


def test_noalloc_rejects_oversized_side():
    # 48 blocks of 512 in bf16 need 72 MiB of workspace, more than the fixed array's 60 MiB
    d, b = 48 * 512, 512
    q = torch.zeros(48, b * (b - 1) // 2, dtype=torch.float32, device="cuda")
    g = torch.zeros(B.poetx_g_bytes(d, b, B.POETX_BF16), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.PoetxError) as e:
        B.poetx_cnp_build_noalloc(q, d, b, B.POETX_BF16, g)
    assert e.value.status == B.POETX_E_WORKSPACE
    torch.cuda.synchronize()
    assert not g.any(), "nothing may be written on an error"

"""The five synthetic workloads, named by what they are.

Shapes follow Llama decoder layers; each linear is W0 in R^{m x n} with
m = input features and n = output features, so the layer maps a [T, m] token
matrix to [T, n].  b is the block size of the block-stochastic factors, T the
number of tokens (batch x sequence, flattened).
"""

from dataclasses import dataclass, field
from typing import List, Tuple


@dataclass(frozen=True)
class LinearShape:
    name: str
    m: int  # input features (rows of W0)
    n: int  # output features (columns of W0)


@dataclass(frozen=True)
class Workload:
    key: str
    wid: int  # numeric id used in the seed sequence
    linears: Tuple[LinearShape, ...]
    b: int
    T: int
    act: str  # dtype of X, dZ, Y, dX: "f32" or "bf16"
    w: str  # storage dtype of W0: "f32", "bf16" or "i8"
    q_std: float
    merge_every: int = 0  # merge-then-reinit period (0: not part of the workload)
    description: str = ""
    meta: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def input_groups(self) -> Tuple[Tuple[int, ...], ...]:
        """The linears in layer order, grouped by the input they read: q, k and v share the attention
        input and gate and up the MLP input; every other linear reads its own."""
        shared = ({"q", "k", "v"}, {"gate", "up"})
        groups, i = [], 0
        while i < len(self.linears):
            g = [i]
            for s in shared:
                if self.linears[i].name in s:
                    while i + len(g) < len(self.linears) and self.linears[i + len(g)].name in s:
                        g.append(i + len(g))
            groups.append(tuple(g))
            i += len(g)
        return tuple(groups)

    @property
    def flop_per_token_gemm(self) -> float:
        # fwd H = A W + bwd dA = dH W^T: 2 contractions of 2*m*n each
        return float(sum(4 * L.m * L.n for L in self.linears))


def _llama(key, wid, hidden, kv, inter, b, T, w, q_std, merge_every=0, desc=""):
    lin = (
        LinearShape("q", hidden, hidden),
        LinearShape("k", hidden, kv),
        LinearShape("v", hidden, kv),
        LinearShape("o", hidden, hidden),
        LinearShape("gate", hidden, inter),
        LinearShape("up", hidden, inter),
        LinearShape("down", inter, hidden),
    )
    return Workload(key, wid, lin, b, T, "bf16", w, q_std, merge_every, desc)


WORKLOADS = {
    w.key: w
    for w in (
        Workload(
            "linear256_fp32",
            1,
            (LinearShape("lin", 256, 256),),
            b=32,
            T=64,
            act="f32",
            w="f32",
            q_std=0.02,
            description="one 256x256 linear, b=32 (8 blocks per side), 64 tokens, all fp32",
        ),
        _llama("llama60m", 2, 512, 512, 1376, 256, 2048, "bf16", 0.01,
               desc="Llama-60M decoder layer, b=256 (last block 96), 2048 tokens, bf16"),
        _llama("llama1p3b", 3, 2048, 2048, 5461, 256, 16384, "bf16", 0.01,
               desc="Llama-1.3B decoder layer, b=256 (last block 85), 16384 tokens, bf16"),
        _llama("llama8b", 4, 4096, 1024, 14336, 512, 8192, "bf16", 0.005,
               desc="Llama-8B decoder layer, b=512, 8192 tokens, bf16"),
        _llama("llama13b_int8", 5, 5120, 5120, 13824, 512, 8192, "i8", 0.005, merge_every=200,
               desc="Llama-13B decoder layer, b=512, 8192 tokens, int8 W0 + fp32 column scale"),
    )
}


def get_workload(key: str) -> Workload:
    if key not in WORKLOADS:
        raise KeyError(f"unknown workload {key!r}; known: {sorted(WORKLOADS)}")
    return WORKLOADS[key]


def all_linears(w: Workload) -> List[LinearShape]:
    return list(w.linears)

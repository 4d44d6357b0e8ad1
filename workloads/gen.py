"""Seeded generators for one POET-X linear's inputs.

Every tensor is drawn from numpy's PCG64 seeded by SeedSequence([workload id,
linear index, tensor id, ...]) with tensor ids 0 = W0, 1 = q_R, 2 = q_P, 3 = X,
4 = dZ, 5 = perm_R, 6 = perm_P (and 7 = dq, 8, 9 = optimiser moments).  Matrices are drawn in fixed chunks of 512 rows,
chunk c from SeedSequence([..., c]), so the values do not depend on how many
threads fill them.  Values are drawn in float64 and rounded once to the storage
type; bf16 tensors are returned as uint16 bit patterns so both consumers see
identical bits.

W0 follows the normalized-Gaussian initialisation of the POET notes
("Reparameterized LLM Training via Orthogonal Equivalence Transformation",
section 4, initialisation schemes): N(0, 1) entries with every output column
(every neuron) scaled to unit L2 norm.  For int8 storage the codes are a
clipped, rounded Gaussian and the per-column fp32 scale is chosen so that each
dequantised column has unit norm; this is an input recipe, not the layer's
requantisation rule.

Packed skew parameters q are N(0, std^2) for every packed slot, including the
slots of a partial last block that the layer must ignore: they are left
non-zero on purpose so that both implementations are checked to ignore them.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

from .configs import Workload

TENSOR_W0, TENSOR_QR, TENSOR_QP, TENSOR_X, TENSOR_DZ, TENSOR_PR, TENSOR_PP, TENSOR_DQ, TENSOR_M1, TENSOR_M2 = range(10)


def packed_len(b: int) -> int:
    """Number of stored values per b x b block (strict upper triangle)."""
    return b * (b - 1) // 2


CHUNK_ROWS = 512


def _rng(wid: int, lin: int, tensor: int, extra: int = 0) -> np.random.Generator:
    words = [wid, lin, tensor] + ([extra] if extra else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(words)))


def _chunked_normal(words, shape, finish: Callable[[np.ndarray], np.ndarray], out_dtype) -> np.ndarray:
    """N(0, 1) matrix drawn in 512-row chunks (chunk c seeded by words + [c]) in
    parallel threads; `finish` maps each float64 chunk to its stored form."""
    rows, cols = shape
    out = np.empty(shape, dtype=out_dtype)
    starts = list(range(0, rows, CHUNK_ROWS))

    def fill(c):
        r0 = starts[c]
        r1 = min(rows, r0 + CHUNK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words) + [c])))
        out[r0:r1] = finish(g.standard_normal((r1 - r0, cols)))

    if len(starts) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); uint16 bits.
    Exact for every finite input: the largest finite pattern plus the rounding
    bias stays below 2^32, so 32-bit arithmetic does not wrap."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(dtype)


@dataclass
class LinearInputs:
    m: int
    n: int
    b: int
    T: int
    act: str  # "f32" | "bf16"
    w: str  # "f32" | "bf16" | "i8"
    W0: np.ndarray  # [m, n]: float32, uint16 (bf16 bits) or int8 codes
    w_scale: Optional[np.ndarray]  # [n] float32 when w == "i8"
    q_R: np.ndarray  # [ceil(m/b), b(b-1)/2] float32
    q_P: np.ndarray  # [ceil(n/b), b(b-1)/2] float32
    perm_R: np.ndarray  # [m] int32
    perm_P: np.ndarray  # [n] int32
    X: np.ndarray  # [T, m] float32 or uint16
    dZ: Optional[np.ndarray]  # [T, n] float32 or uint16


def normalized_gaussian(words, m: int, n: int, dtype: str) -> np.ndarray:
    g = _chunked_normal(words, (m, n), lambda c: c, np.float64)
    g /= np.linalg.norm(g, axis=0, keepdims=True)
    return _store(g, dtype)


def int8_gaussian(words, m: int, n: int):
    codes = _chunked_normal(words, (m, n), lambda c: np.clip(np.rint(c * (127.0 / 4.0)), -127, 127), np.int8)
    norms = np.sqrt(np.einsum("ij,ij->j", codes, codes, dtype=np.float64))
    norms[norms == 0] = 1.0
    return codes, (1.0 / norms).astype(np.float32)


def _act_matrix(words, T: int, d: int, dtype: str) -> np.ndarray:
    return _chunked_normal(words, (T, d), lambda c: _store(c, dtype), np.float32 if dtype == "f32" else np.uint16)


def make_linear_inputs(
    wl: Workload,
    lin: int,
    T: Optional[int] = None,
    with_dz: bool = True,
    q_scale: float = 1.0,
) -> LinearInputs:
    """Inputs of linear `lin` of workload `wl`.  `T` overrides the token count
    (parity tests use fewer tokens than the timed workload); `q_scale`
    multiplies the q standard deviation (0 gives q = 0)."""
    L = wl.linears[lin]
    m, n, b = L.m, L.n, wl.b
    T = wl.T if T is None else T
    wid = wl.wid
    if wl.w == "i8":
        W0, w_scale = int8_gaussian([wid, lin, TENSOR_W0], m, n)
    else:
        W0, w_scale = normalized_gaussian([wid, lin, TENSOR_W0], m, n, wl.w), None
    nbR, nbP = -(-m // b), -(-n // b)
    std = wl.q_std * q_scale
    q_R = (_rng(wid, lin, TENSOR_QR).standard_normal((nbR, packed_len(b))) * std).astype(np.float32)
    q_P = (_rng(wid, lin, TENSOR_QP).standard_normal((nbP, packed_len(b))) * std).astype(np.float32)
    perm_R = _rng(wid, lin, TENSOR_PR).permutation(m).astype(np.int32)
    perm_P = _rng(wid, lin, TENSOR_PP).permutation(n).astype(np.int32)
    X = _act_matrix([wid, lin, TENSOR_X, T], T, m, wl.act)
    dZ = _act_matrix([wid, lin, TENSOR_DZ, T], T, n, wl.act) if with_dz else None
    return LinearInputs(m, n, b, T, wl.act, wl.w, W0, w_scale, q_R, q_P, perm_R, perm_P, X, dZ)


def custom_linear_inputs(
    m: int, n: int, b: int, T: int, act: str, w: str, q_std: float, seed: int
) -> LinearInputs:
    """Same recipe at an arbitrary shape (edge-case tests: ragged blocks, tiny sizes)."""
    from .configs import LinearShape

    wl = Workload("custom", 1000 + seed, (LinearShape("x", m, n),), b, T, act, w, q_std)
    return make_linear_inputs(wl, 0)


def optimizer_inputs(lens, seed: int, q_std: float = 0.01, g_std: float = 4.0):
    """Packed parameters, gradients and two moment arrays for sides of lens[i]
    slots (float32): q ~ N(0, q_std^2), dq ~ N(0, g_std^2), first moment
    ~ N(0, (g_std/3)^2), second moment g_std^2 (N(0, 1)^2 + 1/4), kept away
    from zero like a running mean of squares.  Returns [(q, dq, m1, m2)]."""
    out = []
    for i, L in enumerate(lens):
        wid = 3000 + seed
        q = (_rng(wid, i, TENSOR_QR).standard_normal(L) * q_std).astype(np.float32)
        dq = (_rng(wid, i, TENSOR_DQ).standard_normal(L) * g_std).astype(np.float32)
        m1 = (_rng(wid, i, TENSOR_M1).standard_normal(L) * (g_std / 3.0)).astype(np.float32)
        m2 = ((_rng(wid, i, TENSOR_M2).standard_normal(L) ** 2 + 0.25) * g_std**2).astype(np.float32)
        out.append((q, dq, m1, m2))
    return out


def loop_batches(m: int, n: int, T: int, act: str, steps: int, seed: int):
    """(X, dZ) storage arrays for `steps` training steps of one linear."""
    wid = 4000 + seed
    return [
        (_act_matrix([wid, s, TENSOR_X, T], T, m, act), _act_matrix([wid, s, TENSOR_DZ, T], T, n, act))
        for s in range(steps)
    ]


@dataclass
class SpoInputs:
    d: int
    b: int
    kind: str  # "block" | "full"
    T: int
    act: str
    idx: np.ndarray  # [d] permutation (block) or [b] distinct columns (full), int32
    q: np.ndarray  # [nb, b(b-1)/2] float32, nb = ceil(d/b) (block) or 1 (full)
    X: np.ndarray  # [T, d]
    dY: np.ndarray  # [T, d]


def spo_inputs(d: int, b: int, kind: str, T: int, act: str, q_std: float, seed: int) -> SpoInputs:
    """Inputs of one SPO factor: a numpy-drawn permutation or ordered b-subset
    of the d columns, N(0, q_std^2) packed parameters (dead slots included),
    N(0, 1) X and dY."""
    wid = 5000 + seed
    perm = _rng(wid, 0, TENSOR_PR).permutation(d).astype(np.int32)
    idx = perm if kind == "block" else perm[:b].copy()
    nb = -(-d // b) if kind == "block" else 1
    q = (_rng(wid, 0, TENSOR_QR).standard_normal((nb, packed_len(b))) * q_std).astype(np.float32)
    X = _act_matrix([wid, 0, TENSOR_X, T], T, d, act)
    dY = _act_matrix([wid, 0, TENSOR_DZ, T], T, d, act)
    return SpoInputs(d, b, kind, T, act, idx, q, X, dY)

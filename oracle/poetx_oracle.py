"""fp64 CPU oracle of the POET-X linear layer (plain definitions, numpy).

TEST INFRASTRUCTURE.  Only tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the HIP library and
never calls it.

Sources (web pages about POET-X and its parent method POET):
  [ZC]  "在单张 H100 上预训练 13B 模型：POET-X 如何把正交变换的内存开销砍到 1/3"
        (zhichai.net blog on POET-X); sections 第一斧 .. 第五斧.
  [WS]  "[Project POET-X] Scaling Orthogonal Equivalence: Training 13B LLMs with
        LoRA-level Memory Efficiency" (wispaper.ai blog); numbered methodology
        sections and "Quantized Training (POET-XQ)".
  [PN]  "Reparameterized LLM Training via Orthogonal Equivalence Transformation"
        (NeurIPS 2025 paper notes on POET); 方法详解: 整体框架, 关键设计 1-4,
        训练策略.
  [GS]  "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
        Transformation" (gist.science summary); Resumo técnico, 2. Metodologia.

Conventions (where the pages leave the step open, the plainest reading):
  * W0 is m x n (m inputs, n outputs); tokens are rows, so the layer
    y = (R W0 P)^T x of [PN] 整体框架 reads Y = X R W0 P for X in R^{T x m}.
  * A permutation is an index array pi with Psi[i, pi[i]] = 1, so
    X Psi^T = X[:, pi] and (Z Psi)[:, pi[i]] = Z[:, i].
  * One block-stochastic factor per side ([PN] 关键设计 1, c = 1) in the
    layer calls: R = Psi_R^T Diag(G_R^0 .. G_R^{nb-1}) Psi_R, nb = ceil(m / b).
    A partial last block of r < b rows is its own r x r CNP block.  Products
    of c factors, block-stochastic or fully stochastic (I + D(S)(G - I)D(S)^T
    for an ordered b-subset S, D(S)[S[j], j] = 1), are spo_* and chain_*.
  * Each block G is the Cayley-Neumann form with k = 3 ([PN] 关键设计 2, [ZC]
    第四斧 item 2): G = I + 2(Q + Q^2 + Q^3) + Q^4 of a skew-symmetric Q.
  * Q is stored as its strict upper triangle in row-major order with the full
    block stride b ([ZC] 第四斧 item 1): slot p(i, j) = i*b - i(i+1)/2 + (j-i-1)
    holds Q[i, j] (i < j), and Q[j, i] = -Q[i, j].  Slots with j >= r in a
    partial block are ignored and receive a zero gradient.
  * Gradients are the exact gradients of this forward (intermediate H kept),
    projected onto the packed parameters: dq[p(i,j)] = dQ[i,j] - dQ[j,i].
  * The checkpoint of [ZC] 第五斧 (b = G_P z: the pre-P activation taken back
    from the output instead of stored) is the opt-in h_from_output below.  In
    row form it reads H' = Y[:, pi_P] Diag(G_P)^T.  It inverts the P side only
    for orthogonal blocks; for CNP blocks H' = H Diag((I - Q^4)^2).
  * The optimiser that moves the packed q is not named by the pages, which
    only say that it keeps state for the packed half ([ZC] 第四斧 item 1): it
    is read as Adam with decoupled weight decay (adam_step).  The training
    loop (train_steps) restarts q and the moments at every merge.
"""

from __future__ import annotations

import copy
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

MASK64 = (1 << 64) - 1

# ----------------------------------------------------------------------------
# dtype decoding (the oracle's own widening of the stored bit patterns)
# ----------------------------------------------------------------------------


def to_f64(a: np.ndarray, dtype: str, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Storage -> float64.  bf16 arrives as uint16 bit patterns; int8 codes are
    multiplied by their per-column scale (dequantisation, [WS] POET-XQ)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    if dtype == "i8":
        out = np.asarray(a, dtype=np.int8).astype(np.float64)
        if scale is not None:
            out = out * np.asarray(scale, dtype=np.float32).astype(np.float64)[None, :]
        return out
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# packed skew-symmetric storage ([ZC] 第四斧 item 1; [WS] CNP "Half-Storage")
# ----------------------------------------------------------------------------


def packed_len(b: int) -> int:
    return b * (b - 1) // 2


def packed_index(i: int, j: int, b: int) -> int:
    """Slot of Q[i, j], i < j, in the row-major strict upper triangle of a b x b block."""
    assert 0 <= i < j < b
    return i * b - i * (i + 1) // 2 + (j - i - 1)


def _triu(b: int):
    # numpy enumerates the strict upper triangle row by row: the same order as packed_index
    return np.triu_indices(b, 1)


def unpack_skew(qk: np.ndarray, r: int, b: int) -> np.ndarray:
    """r x r skew-symmetric Q of one block from its packed slots (block stride b)."""
    qk = np.asarray(qk, dtype=np.float64)
    assert qk.shape == (packed_len(b),)
    iu, ju = _triu(b)
    live = ju < r
    Q = np.zeros((r, r))
    Q[iu[live], ju[live]] = qk[live]
    Q[ju[live], iu[live]] = -qk[live]
    return Q


def pack_skew_grad(dQ: np.ndarray, b: int) -> np.ndarray:
    """Gradient w.r.t. the packed slots: dq = dQ[i,j] - dQ[j,i]; dead slots 0."""
    r = dQ.shape[0]
    iu, ju = _triu(b)
    live = ju < r
    out = np.zeros(packed_len(b))
    out[live] = dQ[iu[live], ju[live]] - dQ[ju[live], iu[live]]
    return out


# ----------------------------------------------------------------------------
# Cayley-Neumann parameterisation ([PN] 关键设计 2; [ZC] 第四斧 item 2)
# ----------------------------------------------------------------------------


def cnp(Q: np.ndarray) -> np.ndarray:
    """G = I + 2(Q + Q^2 + Q^3) + Q^4: the k = 3 Neumann truncation of the Cayley
    transform, multiplied out."""
    I = np.eye(Q.shape[0])
    Q2 = Q @ Q
    Q3 = Q2 @ Q
    Q4 = Q3 @ Q
    return I + 2.0 * (Q + Q2 + Q3) + Q4


def cnp_neumann(Q: np.ndarray, k: int) -> np.ndarray:
    """(I + Q)(I + Q + ... + Q^k): the truncated Cayley form of [PN] 关键设计 2."""
    I = np.eye(Q.shape[0])
    S = I.copy()
    P = I.copy()
    for _ in range(k):
        P = P @ Q
        S = S + P
    return (I + Q) @ S


def cayley(Q: np.ndarray) -> np.ndarray:
    """Exact Cayley transform (I + Q)(I - Q)^{-1} ([PN] 关键设计 2)."""
    I = np.eye(Q.shape[0])
    return (I + Q) @ np.linalg.solve(I - Q, I)


def cnp_adjoint(Q: np.ndarray, U: np.ndarray) -> np.ndarray:
    """Gradient of <U, cnp(Q)> w.r.t. an unconstrained Q, using Q^T = -Q.

    Each term A E B of the differential of G contributes A^T U B^T:
    dQ = 2U - 2(QU + UQ) + 2(Q^2 U + Q U Q + U Q^2)
         - (Q^3 U + Q^2 U Q + Q U Q^2 + U Q^3)."""
    Q2 = Q @ Q
    Q3 = Q2 @ Q
    return (
        2.0 * U
        - 2.0 * (Q @ U + U @ Q)
        + 2.0 * (Q2 @ U + Q @ U @ Q + U @ Q2)
        - (Q3 @ U + Q2 @ U @ Q + Q @ U @ Q2 + U @ Q3)
    )


# ----------------------------------------------------------------------------
# block-stochastic factors ([PN] 关键设计 1, block stochastic SPO with c = 1)
# ----------------------------------------------------------------------------


def side_blocks(d: int, b: int):
    """(start, size) of the ceil(d/b) diagonal blocks of one side."""
    return [(s, min(b, d - s)) for s in range(0, d, b)]


def side_Q(q: np.ndarray, d: int, b: int) -> List[np.ndarray]:
    return [unpack_skew(q[k], r, b) for k, (_, r) in enumerate(side_blocks(d, b))]


def side_G(q: np.ndarray, d: int, b: int, exact: bool = False) -> List[np.ndarray]:
    f = cayley if exact else cnp
    return [f(Q) for Q in side_Q(q, d, b)]


def perm_matrix(perm: np.ndarray) -> np.ndarray:
    """Psi with Psi[i, perm[i]] = 1."""
    d = len(perm)
    Psi = np.zeros((d, d))
    Psi[np.arange(d), perm] = 1.0
    return Psi


def block_diag(blocks: Sequence[np.ndarray]) -> np.ndarray:
    d = sum(B.shape[0] for B in blocks)
    D = np.zeros((d, d))
    s = 0
    for B in blocks:
        r = B.shape[0]
        D[s : s + r, s : s + r] = B
        s += r
    return D


def dense_factor(perm: np.ndarray, blocks: Sequence[np.ndarray]) -> np.ndarray:
    """R = Psi^T Diag(G^0 ..) Psi as a dense matrix (tiny sizes only)."""
    Psi = perm_matrix(perm)
    return Psi.T @ block_diag(blocks) @ Psi


def apply_blocks(Z: np.ndarray, blocks: Sequence[np.ndarray], transpose: bool = False) -> np.ndarray:
    """Row form of the block-diagonal product Z Diag(G) (or Z Diag(G)^T), one
    block of columns at a time ([ZC] 第三斧: the blocks as a batch)."""
    out = np.empty_like(Z)
    s = 0
    for G in blocks:
        r = G.shape[0]
        out[:, s : s + r] = Z[:, s : s + r] @ (G.T if transpose else G)
        s += r
    return out


# ----------------------------------------------------------------------------
# permutation merge ([ZC] 第二斧; [GS] 2. Metodologia, 4 -> 2 permutations)
# ----------------------------------------------------------------------------


def premerge(W: np.ndarray, perm_R: np.ndarray, perm_P: np.ndarray) -> np.ndarray:
    """W~ = Psi_R W Psi_P^T = W[perm_R, :][:, perm_P]."""
    return W[perm_R][:, perm_P]


# ----------------------------------------------------------------------------
# forward / backward ([ZC] 第一斧 input-centric order; [WS] section 1)
# ----------------------------------------------------------------------------


@dataclass
class Fwd:
    Y: np.ndarray
    H: np.ndarray
    A: np.ndarray
    Xt: np.ndarray
    Wt: np.ndarray


def forward(X, W, perm_R, perm_P, G_R, G_P) -> Fwd:
    """Input-centric forward with fp64 W (dequantised if stored int8):
    Xt = X[:, pi_R]; A = Xt Diag(G_R); H = A W~; Zt = H Diag(G_P); Y[:, pi_P] = Zt."""
    Xt = X[:, perm_R]
    A = apply_blocks(Xt, G_R)
    Wt = premerge(W, perm_R, perm_P)
    H = A @ Wt
    Zt = apply_blocks(H, G_P)
    Y = np.empty_like(Zt)
    Y[:, perm_P] = Zt
    return Fwd(Y, H, A, Xt, Wt)


def forward_weight_centric(X, W, R, P) -> np.ndarray:
    """Original (weight-centric) order: build R W P, then apply it ([ZC] 第一斧)."""
    return X @ (R @ W @ P)


@dataclass
class Bwd:
    dX: np.ndarray
    dG_R: List[np.ndarray]
    dG_P: List[np.ndarray]
    dq_R: np.ndarray
    dq_P: np.ndarray


def h_from_output(Y, perm_P, G_P) -> np.ndarray:
    """[ZC] 第五斧: b = G_P z, the pre-P activation recovered from the layer output
    (z = G_P^T b in column form).  Row form: H' = Y[:, pi_P] Diag(G_P)^T."""
    return apply_blocks(Y[:, perm_P], G_P, transpose=True)


def backward(X, dZ, W, perm_R, perm_P, q_R, q_P, b, h_output: bool = False) -> Bwd:
    """Exact gradients of forward() w.r.t. X and the packed q of both sides.
    h_output: dG_P uses H' = h_from_output(Y, ..) in place of the forward's H
    (the checkpoint variant; dX and dq_R do not involve H)."""
    m, n = W.shape
    Q_R, Q_P = side_Q(q_R, m, b), side_Q(q_P, n, b)
    G_R, G_P = [cnp(Q) for Q in Q_R], [cnp(Q) for Q in Q_P]
    f = forward(X, W, perm_R, perm_P, G_R, G_P)
    dZt = dZ[:, perm_P]
    H = h_from_output(f.Y, perm_P, G_P) if h_output else f.H
    dG_P = [H[:, s : s + r].T @ dZt[:, s : s + r] for s, r in side_blocks(n, b)]
    dH = apply_blocks(dZt, G_P, transpose=True)
    dA = dH @ f.Wt.T
    dG_R = [f.Xt[:, s : s + r].T @ dA[:, s : s + r] for s, r in side_blocks(m, b)]
    dXt = apply_blocks(dA, G_R, transpose=True)
    dX = np.empty_like(dXt)
    dX[:, perm_R] = dXt
    dq_R = np.stack([pack_skew_grad(cnp_adjoint(Q, U), b) for Q, U in zip(Q_R, dG_R)])
    dq_P = np.stack([pack_skew_grad(cnp_adjoint(Q, U), b) for Q, U in zip(Q_P, dG_P)])
    return Bwd(dX, dG_R, dG_P, dq_R, dq_P)


def cnp_grad_packed(q: np.ndarray, dG: Sequence[np.ndarray], d: int, b: int) -> np.ndarray:
    """Packed dq of one side from the block gradients dG (CNP chain rule + skew projection)."""
    return np.stack([pack_skew_grad(cnp_adjoint(Q, U), b) for Q, U in zip(side_Q(q, d, b), dG)])


# ----------------------------------------------------------------------------
# permutation generator: SplitMix64 (Steele, Lea, Flood 2014) + Durstenfeld shuffle
# ----------------------------------------------------------------------------


def splitmix64_stream(seed: int):
    """Successive SplitMix64 outputs for a 64-bit seed: the state advances by the
    golden-ratio increment and each state is put through the two xor-shift-multiply
    rounds of the published finaliser."""
    state = seed & MASK64
    while True:
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        yield z ^ (z >> 31)


def perm_from_seed(seed: int, d: int) -> np.ndarray:
    """Durstenfeld's Fisher-Yates shuffle of the identity: for i = d-1 .. 1 draw
    j = floor(u * (i + 1) / 2^64) from the next 64-bit output u and swap p[i], p[j]."""
    p = list(range(d))
    g = splitmix64_stream(seed)
    for i in range(d - 1, 0, -1):
        j = (next(g) * (i + 1)) >> 64
        p[i], p[j] = p[j], p[i]
    return np.asarray(p, dtype=np.int32)


# ----------------------------------------------------------------------------
# 8-bit weights (POET-XQ, [WS] "Quantized Training"; [GS] 2. Metodologia)
# ----------------------------------------------------------------------------


def quantize_int8_f32(W: np.ndarray):
    """Symmetric per-output-column absmax quantisation, every decision in fp32:
    scale_j = fp32(max_i |W_ij|) / 127 (an all-zero column gets scale 1),
    code = clamp(round_half_even(W / scale_j), -127, 127)."""
    W = np.asarray(W, dtype=np.float32)
    amax = np.max(np.abs(W), axis=0)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    code = np.rint(W / scale[None, :])
    return np.clip(code, -127, 127).astype(np.int8), scale


def round_bf16(a64: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 (each step round to nearest even); uint16 bits."""
    u = np.ascontiguousarray(a64.astype(np.float32)).view(np.uint32).astype(np.uint64)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# merge-then-reinitialise ([PN] 关键设计 3 and 训练策略)
# ----------------------------------------------------------------------------


@dataclass
class Merge:
    W_new: np.ndarray  # merged weight R W P in the natural layout (fp64)
    Wt_new: np.ndarray  # re-permuted for the new permutations (fp64)
    perm_R: np.ndarray
    perm_P: np.ndarray


def merge_reinit(Wt, perm_R, perm_P, G_R, G_P, seed_R, seed_P) -> Merge:
    """Fold the current factors into the weight and draw new permutations.

    Wt is the pre-merged weight of the current permutations (fp64).  The merged
    weight is W' = R W P = Psi_R^T (Diag(G_R) W~ Diag(G_P)) Psi_P; after the merge
    the factors restart at the identity (q = 0) with permutations drawn from the
    seeds, so the new pre-merged weight is W'[pi_R'][:, pi_P']."""
    m, n = Wt.shape
    M = apply_blocks(apply_blocks(Wt.T, G_R, transpose=True).T, G_P)  # Diag(G_R) W~ Diag(G_P)
    W_new = np.empty_like(M)
    W_new[np.ix_(perm_R, perm_P)] = M
    pR, pP = perm_from_seed(seed_R, m), perm_from_seed(seed_P, n)
    return Merge(W_new, premerge(W_new, pR, pP), pR, pP)


# ----------------------------------------------------------------------------
# sampled outputs at full size
# ----------------------------------------------------------------------------


def block_grads(X, dZ, W, perm_R, perm_P, q_R, q_P, b, blocks_R, blocks_P):
    """Packed dq of selected blocks only, with the sums over all tokens.

    Same definitions as backward(): dG_P^k = H_k^T dZt_k needs only the block's
    columns of H = A W~, and dG_R^k = Xt_k^T dA_k only the block's columns of
    dA = dH W~^T, so the cost is a few block-wide products instead of the whole
    layer.  Returns {("R"|"P", k): dq_k}."""
    m, n = W.shape
    Q_R, Q_P = side_Q(q_R, m, b), side_Q(q_P, n, b)
    G_R, G_P = [cnp(Q) for Q in Q_R], [cnp(Q) for Q in Q_P]
    Wt = premerge(W, perm_R, perm_P)
    Xt = X[:, perm_R]
    dZt = dZ[:, perm_P]
    out = {}
    sbP = side_blocks(n, b)
    if blocks_P:
        A = apply_blocks(Xt, G_R)
        for k in blocks_P:
            s, r = sbP[k]
            Hk = A @ Wt[:, s : s + r]
            out[("P", k)] = pack_skew_grad(cnp_adjoint(Q_P[k], Hk.T @ dZt[:, s : s + r]), b)
    if blocks_R:
        dH = apply_blocks(dZt, G_P, transpose=True)
        sbR = side_blocks(m, b)
        for k in blocks_R:
            s, r = sbR[k]
            dAk = dH @ Wt[s : s + r, :].T
            out[("R", k)] = pack_skew_grad(cnp_adjoint(Q_R[k], Xt[:, s : s + r].T @ dAk), b)
    return out


# ----------------------------------------------------------------------------
# optimiser step on the packed parameters and the training cadence
# ([ZC] 第四斧 item 1: the optimiser keeps state only for the packed half;
#  [PN] 训练策略 and 关键设计 3: an inner loop on the small orthogonal
#  parameters, merged into the weight every T_m steps and then restarted)
# ----------------------------------------------------------------------------


@dataclass
class AdamHP:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


def adam_step(q, g, m1, m2, t: int, hp: AdamHP):
    """One Adam step (Kingma & Ba 2015: exponential moving averages of the
    gradient and of its square, each divided by its bias correction 1 - beta^t)
    with decoupled weight decay (Loshchilov & Hutter 2019: the decay term is
    added to the normalised step, not to the gradient).  fp64; t is the 1-based
    number of steps since the moments were zero.  Returns new (q, m1, m2)."""
    q, g, m1, m2 = (np.asarray(a, dtype=np.float64) for a in (q, g, m1, m2))
    m1 = hp.beta1 * m1 + (1.0 - hp.beta1) * g
    m2 = hp.beta2 * m2 + (1.0 - hp.beta2) * g * g
    m_hat = m1 / (1.0 - hp.beta1**t)
    v_hat = m2 / (1.0 - hp.beta2**t)
    q = q - hp.lr * (m_hat / (np.sqrt(v_hat) + hp.eps) + hp.weight_decay * q)
    return q, m1, m2


def store_weight_values(W64: np.ndarray, w: str) -> np.ndarray:
    """Values of a weight after it is stored in dtype w: fp32 and bf16 round to
    nearest even, int8 is requantised per column (quantize_int8_f32) and read
    back as code x scale.  "f64" keeps the values unrounded."""
    if w == "f64":
        return np.array(W64, dtype=np.float64)
    if w == "f32":
        return W64.astype(np.float32).astype(np.float64)
    if w == "bf16":
        return to_f64(round_bf16(W64), "bf16")
    if w == "i8":
        code, scale = quantize_int8_f32(W64)
        return to_f64(code, "i8", scale)
    raise ValueError(w)


@dataclass
class TrainState:
    Wt: np.ndarray  # pre-merged weight values W0[pi_R][:, pi_P] (fp64 of the stored dtype)
    perm_R: np.ndarray
    perm_P: np.ndarray
    q_R: np.ndarray
    q_P: np.ndarray
    m1_R: np.ndarray
    m2_R: np.ndarray
    m1_P: np.ndarray
    m2_P: np.ndarray
    t: int  # steps since the moments were last zero


def natural_weight(Wt: np.ndarray, perm_R: np.ndarray, perm_P: np.ndarray) -> np.ndarray:
    """W0 from its pre-merged form: W0[pi_R[i], pi_P[j]] = W~[i, j]."""
    W = np.empty_like(Wt)
    W[np.ix_(perm_R, perm_P)] = Wt
    return W


def train_steps(state: TrainState, b: int, w: str, batches, hp: AdamHP, merge_every: int, merge_seeds,
                first_step: int = 1) -> TrainState:
    """The inner loop of [PN] 训练策略 on one linear, one step per (X, dZ) batch.

    Step s (counted from first_step): build G from q, take the exact gradient
    dq of both sides (backward()), and move q by one adam_step with the count
    of steps since the last restart.  When merge_every > 0 and s is a multiple
    of it, merge the factors built from the updated q into the weight
    (merge_reinit with merge_seeds(s) -> (seed_R, seed_P)), store the new
    pre-merged weight in dtype w, and restart: q = 0, both moments 0, count 0.
    The moments are cleared because the new permutations give every packed
    slot a different pair of coordinates (the pages do not say; plainest
    reading)."""
    st = copy.deepcopy(state)
    m, n = st.Wt.shape
    for s, (X, dZ) in enumerate(batches, start=first_step):
        W = natural_weight(st.Wt, st.perm_R, st.perm_P)
        g = backward(X, dZ, W, st.perm_R, st.perm_P, st.q_R, st.q_P, b)
        st.t += 1
        st.q_R, st.m1_R, st.m2_R = adam_step(st.q_R, g.dq_R, st.m1_R, st.m2_R, st.t, hp)
        st.q_P, st.m1_P, st.m2_P = adam_step(st.q_P, g.dq_P, st.m1_P, st.m2_P, st.t, hp)
        if merge_every > 0 and s % merge_every == 0:
            seed_R, seed_P = merge_seeds(s)
            mg = merge_reinit(st.Wt, st.perm_R, st.perm_P, side_G(st.q_R, m, b), side_G(st.q_P, n, b),
                              seed_R, seed_P)
            st.Wt = store_weight_values(mg.Wt_new, w)
            st.perm_R, st.perm_P = mg.perm_R, mg.perm_P
            for k in ("q_R", "q_P", "m1_R", "m2_R", "m1_P", "m2_P"):
                setattr(st, k, np.zeros_like(getattr(st, k)))
            st.t = 0
    return st


# ----------------------------------------------------------------------------
# more than one SPO factor per side, and the fully stochastic factor
# ([PN] 关键设计 1: R is a product of c primitives, each block-stochastic
#  Psi^T Diag(G^1 .. G^nb) Psi or fully stochastic I + D(S)(G - I)D(S)^T)
# ----------------------------------------------------------------------------


@dataclass
class SpoFactor:
    kind: str  # "block": idx is a permutation of all d columns; "full": idx is an ordered b-subset
    idx: np.ndarray
    q: np.ndarray  # packed parameters [nb, b(b-1)/2]; nb = 1 for "full"
    d: int
    b: int

    def blocks(self) -> List[np.ndarray]:
        return side_G(self.q, self.d if self.kind == "block" else self.b, self.b)


def selection_matrix(S: np.ndarray, d: int) -> np.ndarray:
    """D(S) in R^{d x b}: column j is the unit vector e_{S[j]}."""
    D = np.zeros((d, len(S)))
    D[np.asarray(S), np.arange(len(S))] = 1.0
    return D


def spo_dense(f: SpoFactor) -> np.ndarray:
    """The factor as an explicit d x d matrix (tiny sizes)."""
    if f.kind == "block":
        return dense_factor(f.idx, f.blocks())
    D = selection_matrix(f.idx, f.d)
    return np.eye(f.d) + D @ (f.blocks()[0] - np.eye(f.b)) @ D.T


def spo_forward(X: np.ndarray, f: SpoFactor):
    """Row form Y = X F of one factor; also returns the gathered input it keeps.
    block: Xt = X[:, pi], Y[:, pi] = Xt Diag(G).  full: Xt = X[:, S], Y = X with
    Y[:, S] = Xt G (the other columns pass through)."""
    Xt = X[:, f.idx]
    if f.kind == "block":
        Y = np.empty_like(X)
        Y[:, f.idx] = apply_blocks(Xt, f.blocks())
    else:
        Y = np.array(X, dtype=np.float64)
        Y[:, f.idx] = Xt @ f.blocks()[0]
    return Y, Xt


def spo_backward(Xt: np.ndarray, dY: np.ndarray, f: SpoFactor):
    """Exact gradients of spo_forward: dX = dY F^T and the packed dq of the
    factor's blocks (dG_k = Xt_k^T dY[:, idx]_k, then the CNP chain rule)."""
    dA = dY[:, f.idx]
    G = f.blocks()
    if f.kind == "block":
        dG = [Xt[:, s : s + r].T @ dA[:, s : s + r] for s, r in side_blocks(f.d, f.b)]
        dX = np.empty_like(dY)
        dX[:, f.idx] = apply_blocks(dA, G, transpose=True)
        return dX, cnp_grad_packed(f.q, dG, f.d, f.b)
    dX = np.array(dY, dtype=np.float64)
    dX[:, f.idx] = dA @ G[0].T
    return dX, cnp_grad_packed(f.q, [Xt.T @ dA], f.b, f.b)


def chain_forward(X, W, R: Sequence[SpoFactor], P: Sequence[SpoFactor]) -> np.ndarray:
    """Y = X R_1 .. R_c W0 P_1 .. P_c, one factor at a time in row form."""
    Y = X
    for f in R:
        Y = spo_forward(Y, f)[0]
    Y = Y @ W
    for f in P:
        Y = spo_forward(Y, f)[0]
    return Y


def chain_backward(X, dZ, W, R: Sequence[SpoFactor], P: Sequence[SpoFactor]):
    """Exact dX and the packed dq of every factor (lists in the order of R and P)."""
    ins_R, Y = [], X
    for f in R:
        Y, Xt = spo_forward(Y, f)
        ins_R.append(Xt)
    Y = Y @ W
    ins_P = []
    for f in P:
        Y, Xt = spo_forward(Y, f)
        ins_P.append(Xt)
    g, dq_P = dZ, [None] * len(P)
    for k in reversed(range(len(P))):
        g, dq_P[k] = spo_backward(ins_P[k], g, P[k])
    g = g @ W.T
    dq_R = [None] * len(R)
    for k in reversed(range(len(R))):
        g, dq_R[k] = spo_backward(ins_R[k], g, R[k])
    return g, dq_R, dq_P


def chain_merge(W, R: Sequence[SpoFactor], P: Sequence[SpoFactor]) -> np.ndarray:
    """Merge every factor of a chain into the weight ([PN] 关键设计 3 for R and P
    built as products of c primitives, 关键设计 1): W' = R_1 .. R_c W P_1 .. P_c
    with the factors as explicit matrices (tiny sizes), so that chain_forward
    with W' and no factors equals chain_forward with W and the factors."""
    Wn = np.asarray(W, dtype=np.float64)
    for f in reversed(list(R)):
        Wn = spo_dense(f) @ Wn
    for f in P:
        Wn = Wn @ spo_dense(f)
    return Wn


def spo_block_grads(X: np.ndarray, dY: np.ndarray, f: SpoFactor, blocks: Sequence[int]):
    """Packed dq of selected blocks of one factor, with the sums over all rows:
    dG_k = X[:, cols_k]^T dY[:, cols_k] for the block's columns cols_k of idx,
    then the CNP chain rule (the same definitions as spo_backward, restricted
    to the blocks asked for).  Returns {k: dq_k}."""
    de = f.d if f.kind == "block" else f.b
    sb = side_blocks(de, f.b)
    Q = side_Q(f.q, de, f.b)
    out = {}
    for k in blocks:
        s, r = sb[k]
        cols = np.asarray(f.idx[s : s + r])
        out[k] = pack_skew_grad(cnp_adjoint(Q[k], X[:, cols].T @ dY[:, cols]), f.b)
    return out

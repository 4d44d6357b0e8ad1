"""Pins of the oracle's SPO factors beyond the layer's one-per-side form:
fully stochastic factors I + D(S)(G - I)D(S)^T and chains of c factors per
side, each against something other than the oracle's row-form code: explicit
dense matrices built from D(S) and Psi, the special case where a fully
stochastic factor covers every coordinate (a one-block block-stochastic
factor), the adjoint identity, central finite differences, and the c = 1
chain against the layer's own (already pinned) forward and backward."""

import numpy as np
import pytest

import oracle as O


def _factor(rng, kind, d, b, std=0.1):
    if kind == "block":
        idx = rng.permutation(d).astype(np.int32)
        nb = -(-d // b)
    else:
        idx = rng.permutation(d)[:b].astype(np.int32)
        nb = 1
    return O.SpoFactor(kind, idx, rng.standard_normal((nb, O.packed_len(b))) * std, d, b)


CASES = [("block", 11, 4), ("block", 8, 8), ("full", 11, 4), ("full", 9, 9), ("full", 7, 2)]


@pytest.mark.parametrize("kind,d,b", CASES)
def test_spo_forward_matches_dense(kind, d, b):
    rng = np.random.default_rng(1)
    f = _factor(rng, kind, d, b)
    X = rng.standard_normal((5, d))
    Y, Xt = O.spo_forward(X, f)
    np.testing.assert_allclose(Y, X @ O.spo_dense(f), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(Xt, X[:, f.idx])


def test_selection_matrix_explicit():
    D = O.selection_matrix(np.array([3, 0]), 4)
    np.testing.assert_array_equal(D, [[0, 1], [0, 0], [0, 0], [1, 0]])


def test_full_factor_covering_everything_is_one_block():
    """S = pi (all d coordinates, b = d): D(S) = Psi^T, so the fully stochastic
    factor equals the block-stochastic one with a single d x d block."""
    rng = np.random.default_rng(2)
    d = 9
    full = _factor(rng, "full", d, d)
    block = O.SpoFactor("block", full.idx, full.q, d, d)
    np.testing.assert_allclose(O.spo_dense(full), O.spo_dense(block), rtol=0, atol=1e-14)


def test_full_factor_leaves_other_columns():
    rng = np.random.default_rng(3)
    f = _factor(rng, "full", 12, 5)
    X = rng.standard_normal((4, 12))
    Y, _ = O.spo_forward(X, f)
    rest = np.setdiff1d(np.arange(12), f.idx)
    np.testing.assert_array_equal(Y[:, rest], X[:, rest])
    # and the factor is orthogonal up to the CNP defect (I - Q^4)^2
    F = O.spo_dense(f)
    Q = O.side_Q(f.q, f.b, f.b)[0]
    Dm = O.selection_matrix(f.idx, 12)
    defect = np.linalg.matrix_power(np.eye(5) - np.linalg.matrix_power(Q, 4), 2)
    np.testing.assert_allclose(F @ F.T, np.eye(12) + Dm @ (defect - np.eye(5)) @ Dm.T, atol=1e-13)


@pytest.mark.parametrize("kind,d,b", CASES)
def test_spo_backward_adjoint_and_fd(kind, d, b):
    rng = np.random.default_rng(4)
    f = _factor(rng, kind, d, b, std=0.2)
    X = rng.standard_normal((6, d))
    dY = rng.standard_normal((6, d))
    _, Xt = O.spo_forward(X, f)
    dX, dq = O.spo_backward(Xt, dY, f)
    np.testing.assert_allclose(dX, dY @ O.spo_dense(f).T, rtol=0, atol=1e-12)
    h = 1e-6
    fd = np.zeros_like(f.q)
    for k in range(f.q.shape[0]):
        for p in range(f.q.shape[1]):
            qp, qm = f.q.copy(), f.q.copy()
            qp[k, p] += h
            qm[k, p] -= h
            Lp = np.sum(dY * O.spo_forward(X, O.SpoFactor(kind, f.idx, qp, d, b))[0])
            Lm = np.sum(dY * O.spo_forward(X, O.SpoFactor(kind, f.idx, qm, d, b))[0])
            fd[k, p] = (Lp - Lm) / (2 * h)
    np.testing.assert_allclose(dq, fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()))


def _chain(rng, m, n, kinds_R, kinds_P, b):
    R = [_factor(rng, k, m, b) for k in kinds_R]
    P = [_factor(rng, k, n, b) for k in kinds_P]
    W = rng.standard_normal((m, n))
    return R, P, W


def test_chain_matches_dense_product():
    rng = np.random.default_rng(5)
    m, n, b = 10, 7, 3
    R, P, W = _chain(rng, m, n, ["full", "block", "block"], ["block", "full"], b)
    X = rng.standard_normal((4, m))
    dense = X
    for f in R:
        dense = dense @ O.spo_dense(f)
    dense = dense @ W
    for f in P:
        dense = dense @ O.spo_dense(f)
    np.testing.assert_allclose(O.chain_forward(X, W, R, P), dense, rtol=0, atol=1e-12)


def test_chain_backward_fd():
    rng = np.random.default_rng(6)
    m, n, b = 8, 6, 3
    R, P, W = _chain(rng, m, n, ["block", "full"], ["full", "block"], b)
    X = rng.standard_normal((5, m))
    dZ = rng.standard_normal((5, n))
    dX, dq_R, dq_P = O.chain_backward(X, dZ, W, R, P)
    # dX: the adjoint of the dense chain
    M = np.eye(m)
    for f in R:
        M = M @ O.spo_dense(f)
    M = M @ W
    for f in P:
        M = M @ O.spo_dense(f)
    np.testing.assert_allclose(dX, dZ @ M.T, rtol=0, atol=1e-12)
    h = 1e-6
    for side, facs, dqs in (("R", R, dq_R), ("P", P, dq_P)):
        for i, f in enumerate(facs):
            for p in (0, 1, f.q.shape[1] - 1):
                vals = []
                for sgn in (1, -1):
                    q2 = f.q.copy()
                    q2[0, p] += sgn * h
                    g = O.SpoFactor(f.kind, f.idx, q2, f.d, f.b)
                    R2 = [g if (side == "R" and j == i) else x for j, x in enumerate(R)]
                    P2 = [g if (side == "P" and j == i) else x for j, x in enumerate(P)]
                    vals.append(np.sum(dZ * O.chain_forward(X, W, R2, P2)))
                assert abs(dqs[i][0, p] - (vals[0] - vals[1]) / (2 * h)) <= 1e-6 * max(1, abs(dqs[i][0, p]))


def test_chain_of_one_block_factor_per_side_is_the_layer():
    """c = 1 block-stochastic chains reproduce forward() and backward() of the layer."""
    rng = np.random.default_rng(7)
    m, n, b, T = 11, 9, 4, 5
    W = rng.standard_normal((m, n))
    pR, pP = rng.permutation(m).astype(np.int32), rng.permutation(n).astype(np.int32)
    qR = rng.standard_normal((-(-m // b), O.packed_len(b))) * 0.1
    qP = rng.standard_normal((-(-n // b), O.packed_len(b))) * 0.1
    X, dZ = rng.standard_normal((T, m)), rng.standard_normal((T, n))
    R = [O.SpoFactor("block", pR, qR, m, b)]
    P = [O.SpoFactor("block", pP, qP, n, b)]
    f = O.forward(X, W, pR, pP, O.side_G(qR, m, b), O.side_G(qP, n, b))
    np.testing.assert_allclose(O.chain_forward(X, W, R, P), f.Y, rtol=0, atol=1e-12)
    g = O.backward(X, dZ, W, pR, pP, qR, qP, b)
    dX, dq_R, dq_P = O.chain_backward(X, dZ, W, R, P)
    np.testing.assert_allclose(dX, g.dX, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq_R[0], g.dq_R, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq_P[0], g.dq_P, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind,d,b", [("block", 11, 4), ("full", 9, 4)])
def test_spo_block_grads_is_backward_restricted(kind, d, b):
    rng = np.random.default_rng(8)
    f = _factor(rng, kind, d, b, std=0.2)
    X, dY = rng.standard_normal((7, d)), rng.standard_normal((7, d))
    _, dq = O.spo_backward(O.spo_forward(X, f)[1], dY, f)
    sel = O.spo_block_grads(X, dY, f, range(dq.shape[0]))
    for k, v in sel.items():
        np.testing.assert_allclose(v, dq[k], rtol=0, atol=1e-12)


def test_chain_merge_preserves_the_function():
    """Merging every factor into the weight leaves the chain's function unchanged: the row-form
    chain with the factors equals the plain product with the merged weight and no factors."""
    rng = np.random.default_rng(8)
    m, n, b = 10, 7, 3
    R, P, W = _chain(rng, m, n, ["full", "block", "block"], ["block", "full"], b)
    X = rng.standard_normal((6, m))
    Wm = O.chain_merge(W, R, P)
    np.testing.assert_allclose(O.chain_forward(X, Wm, [], []), O.chain_forward(X, W, R, P), rtol=0, atol=1e-12)
    # the merged weight is not the original one (the factors were not the identity)
    assert np.abs(Wm - W).max() > 1e-3


def test_chain_merge_of_one_factor_per_side_is_the_layer_merge():
    """c = 1: the dense merge equals merge_reinit's merged weight (blockwise products on the
    pre-merged weight, scattered back to the natural order)."""
    rng = np.random.default_rng(9)
    m, n, b = 11, 9, 4
    W = rng.standard_normal((m, n))
    pR, pP = rng.permutation(m).astype(np.int32), rng.permutation(n).astype(np.int32)
    qR = rng.standard_normal((-(-m // b), O.packed_len(b))) * 0.1
    qP = rng.standard_normal((-(-n // b), O.packed_len(b))) * 0.1
    R = [O.SpoFactor("block", pR, qR, m, b)]
    P = [O.SpoFactor("block", pP, qP, n, b)]
    ref = O.merge_reinit(O.premerge(W, pR, pP), pR, pP, O.side_G(qR, m, b), O.side_G(qP, n, b), 1, 2)
    np.testing.assert_allclose(O.chain_merge(W, R, P), ref.W_new, rtol=0, atol=1e-12)

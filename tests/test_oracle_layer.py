"""Pins of the oracle's layer: forward, backward, permutation merge, merge-then-
reinitialise, 8-bit requantisation and the permutation generator, each against
something other than the oracle's own formula (dense brute force from explicit
permutation and block-diagonal matrices, closed forms, finite differences,
invariants, published known answers)."""

from pathlib import Path

import numpy as np
import pytest

import oracle as O

GOLD = Path(__file__).parent / "golden"


def _skew_q(rng, nb, b, std):
    return rng.standard_normal((nb, O.packed_len(b))) * std


def _problem(m, n, b, T, std, seed):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((m, n))
    W /= np.linalg.norm(W, axis=0, keepdims=True)
    q_R = _skew_q(rng, -(-m // b), b, std)
    q_P = _skew_q(rng, -(-n // b), b, std)
    return dict(
        X=rng.standard_normal((T, m)),
        dZ=rng.standard_normal((T, n)),
        W=W,
        q_R=q_R,
        q_P=q_P,
        perm_R=rng.permutation(m).astype(np.int32),
        perm_P=rng.permutation(n).astype(np.int32),
        b=b,
    )


SHAPES = [(8, 8, 4, 5), (13, 10, 4, 7), (12, 7, 5, 3), (9, 16, 16, 4), (6, 6, 1 + 5, 2)]


def _dense(p, exact=False):
    m, n = p["W"].shape
    GR = O.side_G(p["q_R"], m, p["b"], exact)
    GP = O.side_G(p["q_P"], n, p["b"], exact)
    return O.dense_factor(p["perm_R"], GR), O.dense_factor(p["perm_P"], GP), GR, GP


def test_side_blocks_partial():
    assert O.side_blocks(1376, 256) == [(0, 256), (256, 256), (512, 256), (768, 256), (1024, 256), (1280, 96)]
    assert O.side_blocks(5461, 256)[-1] == (5376, 85)
    assert len(O.side_blocks(14336, 512)) == 28


def test_perm_matrix_convention():
    # X Psi^T gathers columns, Z Psi scatters them
    perm = np.array([2, 0, 3, 1])
    Psi = O.perm_matrix(perm)
    X = np.arange(8.0).reshape(2, 4)
    np.testing.assert_array_equal(X @ Psi.T, X[:, perm])
    Z = X @ Psi
    np.testing.assert_array_equal(Z[:, perm], X)


@pytest.mark.parametrize("shape", SHAPES)
def test_input_centric_equals_weight_centric(shape):
    m, n, b, T = shape
    p = _problem(m, n, b, T, 0.2, sum(shape))
    R, P, GR, GP = _dense(p)
    y_wc = O.forward_weight_centric(p["X"], p["W"], R, P)
    y_ic = O.forward(p["X"], p["W"], p["perm_R"], p["perm_P"], GR, GP).Y
    np.testing.assert_allclose(y_ic, y_wc, atol=1e-13)
    # the four-permutation form equals the two-permutation form with W pre-merged
    PsiR, PsiP = O.perm_matrix(p["perm_R"]), O.perm_matrix(p["perm_P"])
    np.testing.assert_array_equal(PsiR @ p["W"] @ PsiP.T, O.premerge(p["W"], p["perm_R"], p["perm_P"]))


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_zero_q_gives_plain_linear(shape):
    m, n, b, T = shape
    p = _problem(m, n, b, T, 0.0, 1)
    R, P, GR, GP = _dense(p)
    np.testing.assert_array_equal(R, np.eye(m))
    f = O.forward(p["X"], p["W"], p["perm_R"], p["perm_P"], GR, GP)
    np.testing.assert_allclose(f.Y, p["X"] @ p["W"], atol=1e-14)
    g = O.backward(p["X"], p["dZ"], p["W"], p["perm_R"], p["perm_P"], p["q_R"], p["q_P"], b)
    np.testing.assert_allclose(g.dX, p["dZ"] @ p["W"].T, atol=1e-14)


def test_identity_weight_roundtrip_exact():
    # W = I, q = 0: Y = X and dX = dZ exactly in any summation order
    m = 24
    p = _problem(m, m, 8, 5, 0.0, 2)
    W = np.eye(m)
    GR, GP = O.side_G(p["q_R"], m, 8), O.side_G(p["q_P"], m, 8)
    f = O.forward(p["X"], W, p["perm_R"], p["perm_P"], GR, GP)
    np.testing.assert_array_equal(f.Y, p["X"])
    g = O.backward(p["X"], p["dZ"], W, p["perm_R"], p["perm_P"], p["q_R"], p["q_P"], 8)
    np.testing.assert_array_equal(g.dX, p["dZ"])


@pytest.mark.parametrize("shape", [(12, 10, 4, 3), (16, 16, 8, 3)])
def test_spectrum_preserved_with_exact_cayley(shape):
    m, n, b, T = shape
    p = _problem(m, n, b, T, 0.3, 5)
    R, P, _, _ = _dense(p, exact=True)
    s0 = np.linalg.svd(p["W"], compute_uv=False)
    s1 = np.linalg.svd(R @ p["W"] @ P, compute_uv=False)
    np.testing.assert_allclose(s1, s0, atol=1e-13)


def test_cnp_spectrum_bound():
    # with the truncated form the singular values shrink by at most (1 - mu_R^4)(1 - mu_P^4)
    p = _problem(16, 12, 4, 3, 0.3, 9)
    R, P, GR, GP = _dense(p)
    muR = max(np.max(np.abs(np.linalg.eigvals(O.unpack_skew(q, 4, 4)))) for q in p["q_R"])
    muP = max(np.max(np.abs(np.linalg.eigvals(O.unpack_skew(q, 4, 4)))) for q in p["q_P"])
    s0 = np.linalg.svd(p["W"], compute_uv=False)
    s1 = np.linalg.svd(R @ p["W"] @ P, compute_uv=False)
    assert np.all(s1 <= s0 * (1 + 1e-12))
    assert np.all(s1 >= s0 * (1 - muR**4) * (1 - muP**4) * (1 - 1e-12))
    assert np.max(np.abs(s1 - s0)) > 1e-6  # the truncation is visible


@pytest.mark.parametrize("shape", [(9, 7, 4, 3), (8, 12, 5, 2)])
def test_backward_finite_differences(shape):
    m, n, b, T = shape
    p = _problem(m, n, b, T, 0.2, 11)
    g = O.backward(p["X"], p["dZ"], p["W"], p["perm_R"], p["perm_P"], p["q_R"], p["q_P"], b)

    def loss(qR, qP, X):
        R = O.dense_factor(p["perm_R"], O.side_G(qR, m, b))
        P = O.dense_factor(p["perm_P"], O.side_G(qP, n, b))
        return np.sum(p["dZ"] * O.forward_weight_centric(X, p["W"], R, P))

    h = 1e-6
    for name, q, dq in (("R", p["q_R"], g.dq_R), ("P", p["q_P"], g.dq_P)):
        for k in range(q.shape[0]):
            for s in range(q.shape[1]):
                e = np.zeros_like(q)
                e[k, s] = h
                if name == "R":
                    fd = (loss(q + e, p["q_P"], p["X"]) - loss(q - e, p["q_P"], p["X"])) / (2 * h)
                else:
                    fd = (loss(p["q_R"], q + e, p["X"]) - loss(p["q_R"], q - e, p["X"])) / (2 * h)
                assert abs(fd - dq[k, s]) < 1e-7 * (1 + abs(fd)), (name, k, s, fd, dq[k, s])
    # Y is linear in X: <dX, V> = <dZ, Y(V)> for any V
    V = np.random.default_rng(0).standard_normal(p["X"].shape)
    assert np.isclose(np.sum(g.dX * V), loss(p["q_R"], p["q_P"], V), rtol=1e-12)


def test_merge_then_reinit_preserves_function():
    m, n, b, T = 13, 11, 4, 6
    p = _problem(m, n, b, T, 0.2, 21)
    GR, GP = O.side_G(p["q_R"], m, b), O.side_G(p["q_P"], n, b)
    f = O.forward(p["X"], p["W"], p["perm_R"], p["perm_P"], GR, GP)
    mg = O.merge_reinit(f.Wt, p["perm_R"], p["perm_P"], GR, GP, 123, 456)
    R, P = O.dense_factor(p["perm_R"], GR), O.dense_factor(p["perm_P"], GP)
    np.testing.assert_allclose(mg.W_new, R @ p["W"] @ P, atol=1e-14)
    np.testing.assert_array_equal(mg.perm_R, O.perm_from_seed(123, m))
    # after the merge the factors are the identity (q = 0) with the new permutations
    Z = np.zeros_like(p["q_R"]), np.zeros_like(p["q_P"])
    GR0, GP0 = O.side_G(Z[0], m, b), O.side_G(Z[1], n, b)
    f2 = O.forward(p["X"], mg.W_new, mg.perm_R, mg.perm_P, GR0, GP0)
    np.testing.assert_allclose(f2.Y, f.Y, atol=1e-13)
    np.testing.assert_array_equal(f2.Wt, mg.Wt_new)


def test_merge_with_zero_q_is_repermutation_only():
    m, n, b = 10, 9, 4
    p = _problem(m, n, b, 2, 0.0, 3)
    Wt = O.premerge(p["W"], p["perm_R"], p["perm_P"])
    GR, GP = O.side_G(p["q_R"], m, b), O.side_G(p["q_P"], n, b)
    mg = O.merge_reinit(Wt, p["perm_R"], p["perm_P"], GR, GP, 5, 6)
    np.testing.assert_array_equal(mg.W_new, p["W"])
    np.testing.assert_array_equal(mg.Wt_new, p["W"][mg.perm_R][:, mg.perm_P])


def test_splitmix64_known_answers():
    for line in (GOLD / "splitmix64_known_answers.txt").read_text().splitlines():
        if line.startswith("#") or not line.strip():
            continue
        seed, outs = line.split("|")
        g = O.splitmix64_stream(int(seed))
        assert [next(g) for _ in range(3)] == [int(x) for x in outs.split()]


def test_perm_from_seed_is_uniform_bijection():
    for d in (1, 2, 7, 1376):
        for s in range(3):
            p = O.perm_from_seed(s * 977 + d, d)
            assert sorted(p.tolist()) == list(range(d))
    # d = 2: j = floor(2u / 2^64) is 0 (swap) iff the first output is below 2^63
    for s in range(20):
        u = next(O.splitmix64_stream(s))
        assert O.perm_from_seed(s, 2).tolist() == ([1, 0] if u < 1 << 63 else [0, 1])
    # d = 3: all 6 orders, frequencies within 5 sigma of 1/6
    counts = {}
    N = 6000
    for s in range(N):
        k = tuple(O.perm_from_seed(s, 3).tolist())
        counts[k] = counts.get(k, 0) + 1
    assert len(counts) == 6
    sd = np.sqrt(N * (1 / 6) * (5 / 6))
    assert all(abs(c - N / 6) < 5 * sd for c in counts.values())


def test_quantize_int8_decisions():
    W = np.array(
        [[0.5, 0.0, -1.0], [-1.27, 0.0, 0.25], [0.005, 0.0, 0.5 * 1.0 / 127]], dtype=np.float32
    )
    code, scale = O.quantize_int8_f32(W)
    assert scale.dtype == np.float32 and code.dtype == np.int8
    assert scale[1] == 1.0 and np.all(code[:, 1] == 0)  # all-zero column
    assert scale[0] == np.float32(1.27) / np.float32(127)
    assert code[1, 0] == -127 and code[0, 2] == -127
    # the column max maps to +-127 and ties round to even
    assert code[2, 2] == 0  # 0.5 * step rounds to even (0)
    # dequantised error is at most half a step
    deq = code.astype(np.float64) * scale.astype(np.float64)[None, :]
    assert np.all(np.abs(deq - W) <= 0.5 * scale[None, :] * (1 + 1e-6))


def test_block_grads_match_full_backward():
    m, n, b, T = 13, 10, 4, 6
    p = _problem(m, n, b, T, 0.2, 31)
    g = O.backward(p["X"], p["dZ"], p["W"], p["perm_R"], p["perm_P"], p["q_R"], p["q_P"], b)
    sel = O.block_grads(p["X"], p["dZ"], p["W"], p["perm_R"], p["perm_P"], p["q_R"], p["q_P"], b, [0, 3], [2])
    np.testing.assert_allclose(sel[("R", 0)], g.dq_R[0], atol=1e-14)
    np.testing.assert_allclose(sel[("R", 3)], g.dq_R[3], atol=1e-14)
    np.testing.assert_allclose(sel[("P", 2)], g.dq_P[2], atol=1e-14)


# ----------------------------------------------------------------------------
# the checkpoint of [ZC] 第五斧: H taken back from the output
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("shape", SHAPES)
def test_h_from_output_closed_form(shape):
    """H' = Y[:, pi_P] Diag(G_P)^T equals H Diag((I - Q^4)^2) for CNP blocks: the
    Neumann truncation is the Cayley transform times (I - Q^4), so G G^T = (I - Q^4)^2.
    The right side is built from Q alone, without G, the output or the permutation."""
    m, n, b, T = shape
    p = _problem(m, n, b, T, 0.3, seed=m * 100 + n)
    G_R, G_P = O.side_G(p["q_R"], m, b), O.side_G(p["q_P"], n, b)
    f = O.forward(p["X"], p["W"], p["perm_R"], p["perm_P"], G_R, G_P)
    Hp = O.h_from_output(f.Y, p["perm_P"], G_P)
    corr = []
    for Q in O.side_Q(p["q_P"], n, b):
        E = np.eye(Q.shape[0]) - np.linalg.matrix_power(Q, 4)
        corr.append(E @ E)
    expect = f.H @ O.block_diag(corr)
    assert np.abs(Hp - expect).max() <= 1e-12 * np.abs(expect).max()
    # and it is not H itself (the q above is large enough to see the difference)
    assert np.abs(Hp - f.H).max() > 1e-6 * np.abs(f.H).max()


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_h_from_output_exact_for_orthogonal_blocks(shape):
    m, n, b, T = shape
    p = _problem(m, n, b, T, 0.3, seed=m + 7 * n)
    G_R, G_P = O.side_G(p["q_R"], m, b, exact=True), O.side_G(p["q_P"], n, b, exact=True)
    f = O.forward(p["X"], p["W"], p["perm_R"], p["perm_P"], G_R, G_P)
    Hp = O.h_from_output(f.Y, p["perm_P"], G_P)
    assert np.abs(Hp - f.H).max() <= 1e-12 * np.abs(f.H).max()


def test_h_output_backward_touches_only_dq_p():
    """dX and dq_R do not involve H; with q_P = 0 (G_P = I) H' = H and dq_P agrees too."""
    m, n, b, T = 12, 10, 4, 6
    p = _problem(m, n, b, T, 0.3, seed=5)
    args = (p["X"], p["dZ"], p["W"], p["perm_R"], p["perm_P"], p["q_R"], p["q_P"], b)
    g0, g1 = O.backward(*args), O.backward(*args, h_output=True)
    np.testing.assert_array_equal(g0.dX, g1.dX)
    np.testing.assert_array_equal(g0.dq_R, g1.dq_R)
    assert np.abs(g0.dq_P - g1.dq_P).max() > 0
    zero = (p["X"], p["dZ"], p["W"], p["perm_R"], p["perm_P"], p["q_R"], np.zeros_like(p["q_P"]), b)
    h0, h1 = O.backward(*zero), O.backward(*zero, h_output=True)
    assert np.abs(h0.dq_P - h1.dq_P).max() <= 1e-12 * np.abs(h0.dq_P).max()

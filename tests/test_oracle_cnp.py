"""Pins of the oracle's packing and Cayley-Neumann block against facts that do
not come from the oracle itself: exact closed forms, the factored form the pages
print, algebraic identities of the Cayley transform, and brute force."""

from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

import oracle as O

GOLD = Path(__file__).parent / "golden"


def _frac_list(s):
    return [float(Fraction(x)) for x in s.split()]


def _closed_form_cases():
    cases = []
    for line in (GOLD / "cnp_closed_forms.txt").read_text().splitlines():
        if not line.startswith("case"):
            continue
        name, q, G, C = [p.strip() for p in line.split("|")]
        q = _frac_list(q[2:])
        G = np.array(_frac_list(G[2:]))
        C = np.array(_frac_list(C[2:]))
        r = int(round(np.sqrt(len(G))))
        cases.append((name, r, q, G.reshape(r, r), C.reshape(r, r)))
    return cases


def _rand_skew(rng, r, std):
    A = rng.standard_normal((r, r)) * std
    return np.triu(A, 1) - np.triu(A, 1).T


def test_packed_index_order_b4():
    # row-major strict upper triangle of a 4 x 4 block
    want = {(0, 1): 0, (0, 2): 1, (0, 3): 2, (1, 2): 3, (1, 3): 4, (2, 3): 5}
    for (i, j), p in want.items():
        assert O.packed_index(i, j, 4) == p
    assert O.packed_len(4) == 6 and O.packed_len(512) == 130816


@pytest.mark.parametrize("b", [2, 3, 7, 32])
def test_unpack_matches_slot_formula(b):
    rng = np.random.default_rng(b)
    q = rng.standard_normal(O.packed_len(b))
    for r in sorted({b, max(1, b - 1), 1}):
        Q = O.unpack_skew(q, r, b)
        assert Q.shape == (r, r)
        for i in range(r):
            assert Q[i, i] == 0
            for j in range(i + 1, r):
                p = O.packed_index(i, j, b)
                assert Q[i, j] == q[p] and Q[j, i] == -q[p]


@pytest.mark.parametrize("b,r", [(5, 5), (5, 3), (6, 1)])
def test_pack_is_adjoint_of_unpack(b, r):
    # <U, unpack(q)> = <pack_grad(U), q> for every dense U: the packed gradient is
    # exactly the chain rule through Q_ij = q, Q_ji = -q; dead slots get 0
    rng = np.random.default_rng(3)
    q = rng.standard_normal(O.packed_len(b))
    U = rng.standard_normal((r, r))
    g = O.pack_skew_grad(U, b)
    assert np.isclose(np.sum(U * O.unpack_skew(q, r, b)), g @ q, rtol=1e-13)
    iu, ju = np.triu_indices(b, 1)
    assert np.all(g[ju >= r] == 0)


@pytest.mark.parametrize("case", _closed_form_cases(), ids=lambda c: c[0])
def test_cnp_closed_forms(case):
    name, r, q, G, C = case
    Q = O.unpack_skew(np.array(q), r, r)
    np.testing.assert_allclose(O.cnp(Q), G, rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.cayley(Q), C, rtol=0, atol=1e-15)


def test_partial_block_ignores_dead_slots():
    # a 3 x 3 block stored with stride b = 4: slots with j = 3 are dead
    case = [c for c in _closed_form_cases() if c[0] == "case 3x3"][0]
    _, _, (a, b_, c), G, _ = case
    q = np.array([a, b_, 99.0, c, -77.0, 55.0])  # dead slots hold garbage
    np.testing.assert_allclose(O.cnp(O.unpack_skew(q, 3, 4)), G, atol=1e-15)


@pytest.mark.parametrize("r,std", [(8, 0.1), (32, 0.02), (96, 0.01)])
def test_cnp_equals_factored_form(r, std):
    # the expanded form equals the truncated Cayley product (I+Q)(I+Q+Q^2+Q^3)
    Q = _rand_skew(np.random.default_rng(r), r, std)
    np.testing.assert_allclose(O.cnp(Q), O.cnp_neumann(Q, 3), atol=1e-14)
    # and k = 0 gives I + Q (the divergent case of the ablation), k -> inf the exact transform
    np.testing.assert_allclose(O.cnp_neumann(Q, 0), np.eye(r) + Q, atol=0)
    np.testing.assert_allclose(O.cnp_neumann(Q, 60), O.cayley(Q), atol=1e-13)


@pytest.mark.parametrize("r,std", [(16, 0.05), (64, 0.02)])
def test_cnp_cayley_identities(r, std):
    Q = _rand_skew(np.random.default_rng(100 + r), r, std)
    I = np.eye(r)
    G, C = O.cnp(Q), O.cayley(Q)
    Q4 = np.linalg.matrix_power(Q, 4)
    # Cayley of a skew matrix is orthogonal
    np.testing.assert_allclose(C.T @ C, I, atol=1e-13)
    # truncation error of the Neumann series: G = C (I - Q^4)
    np.testing.assert_allclose(G, C @ (I - Q4), atol=1e-14)
    # hence G^T G = (I - Q^4)^2 and sigma(G) = 1 - mu^4, mu = |eig(Q)|
    np.testing.assert_allclose(G.T @ G, (I - Q4) @ (I - Q4), atol=1e-14)
    mu = np.abs(np.linalg.eigvals(Q))
    np.testing.assert_allclose(np.sort(np.linalg.svd(G, compute_uv=False)), np.sort(1 - mu**4), atol=1e-13)
    # symmetric part I + 2Q^2 + Q^4, skew part 2(Q + Q^3)
    Q2 = Q @ Q
    np.testing.assert_allclose((G + G.T) / 2, I + 2 * Q2 + Q2 @ Q2, atol=1e-14)
    np.testing.assert_allclose((G - G.T) / 2, 2 * (Q + Q2 @ Q), atol=1e-14)


def test_cnp_zero_is_identity():
    for r in (1, 2, 17):
        np.testing.assert_array_equal(O.cnp(np.zeros((r, r))), np.eye(r))


@pytest.mark.parametrize("r", [4, 9])
def test_cnp_adjoint_finite_differences(r):
    # the 10-term adjoint agrees with central differences of <U, cnp(Q)> along
    # skew directions, and with the packed projection slot by slot
    rng = np.random.default_rng(7 + r)
    b = r + 2  # partial block in a wider stride
    q = rng.standard_normal(O.packed_len(b)) * 0.1
    U = rng.standard_normal((r, r))
    Q = O.unpack_skew(q, r, b)
    g = O.pack_skew_grad(O.cnp_adjoint(Q, U), b)
    h = 1e-6
    for p in range(O.packed_len(b)):
        e = np.zeros_like(q)
        e[p] = h
        fd = (np.sum(U * O.cnp(O.unpack_skew(q + e, r, b))) - np.sum(U * O.cnp(O.unpack_skew(q - e, r, b)))) / (2 * h)
        assert abs(fd - g[p]) < 1e-8 * (1 + abs(fd)), (p, fd, g[p])

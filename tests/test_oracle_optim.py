"""Pins of the oracle's optimiser step on packed q and of its training loop
(inner steps, merge, restart), each against something other than the oracle's
own formula: torch's AdamW (an independent implementation of the published
update), closed forms of Adam under constant gradients and under decay alone,
and invariants of the loop (the layer function survives a merge; the first
step after a restart has the first-step form)."""

import numpy as np
import pytest
import torch

import oracle as O


def _torch_adamw(q0, grads, hp):
    p = torch.nn.Parameter(torch.tensor(q0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay, foreach=False)
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    s = opt.state[p]
    return p.detach().numpy(), s["exp_avg"].numpy(), s["exp_avg_sq"].numpy()


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("betas", [(0.9, 0.999), (0.5, 0.9)])
def test_adam_matches_torch_adamw(wd, betas):
    rng = np.random.default_rng(5)
    hp = O.AdamHP(lr=0.01, beta1=betas[0], beta2=betas[1], eps=1e-6, weight_decay=wd)
    q0 = rng.standard_normal(300) * 0.02
    # gradients of mixed scale, including exact zeros
    grads = [rng.standard_normal(300) * np.exp(rng.uniform(-6, 3, 300)) * (rng.random(300) > 0.1) for _ in range(7)]
    q, m1, m2 = q0, np.zeros(300), np.zeros(300)
    for t, g in enumerate(grads, start=1):
        q, m1, m2 = O.adam_step(q, g, m1, m2, t, hp)
    rq, rm1, rm2 = _torch_adamw(q0, grads, hp)
    # torch forms the first moment by lerp, so rounding differs where the sum cancels
    for a, r in ((q, rq), (m1, rm1), (m2, rm2)):
        np.testing.assert_allclose(a, r, rtol=1e-12, atol=1e-14 * np.abs(r).max())


def test_adam_constant_gradient_closed_form():
    """With the same gradient every step the bias-corrected moments are exactly
    g and g^2, so each step moves q by lr g / (|g| + eps)."""
    hp = O.AdamHP(lr=0.003, beta1=0.9, beta2=0.99, eps=1e-3)
    g = np.array([2.0, -0.5, 1e-3, -7.0, 0.0])
    q0 = np.array([0.1, -0.2, 0.0, 0.3, 0.4])
    q, m1, m2 = q0, np.zeros(5), np.zeros(5)
    for t in range(1, 11):
        q, m1, m2 = O.adam_step(q, g, m1, m2, t, hp)
        np.testing.assert_allclose(q, q0 - t * hp.lr * g / (np.abs(g) + hp.eps), rtol=1e-12, atol=1e-15)


def test_adam_decay_only():
    """Zero gradient and zero moments: decoupled decay alone, q_t = q_0 (1 - lr wd)^t."""
    hp = O.AdamHP(lr=0.05, weight_decay=0.3)
    q0 = np.array([1.0, -2.0, 0.5])
    q, m1, m2 = q0, np.zeros(3), np.zeros(3)
    for t in range(1, 6):
        q, m1, m2 = O.adam_step(q, np.zeros(3), m1, m2, t, hp)
        np.testing.assert_allclose(q, q0 * (1 - hp.lr * hp.weight_decay) ** t, rtol=1e-14)
    assert not m1.any() and not m2.any()


# ---------------------------------------------------------------- the loop --


def _state(m, n, b, seed, q_std=0.0):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((m, n))
    W /= np.linalg.norm(W, axis=0, keepdims=True)
    pR, pP = rng.permutation(m).astype(np.int32), rng.permutation(n).astype(np.int32)
    z = lambda d: np.zeros((-(-d // b), O.packed_len(b)))
    q_R = rng.standard_normal(z(m).shape) * q_std
    q_P = rng.standard_normal(z(n).shape) * q_std
    return W, O.TrainState(O.premerge(W, pR, pP), pR, pP, q_R, q_P, z(m), z(m), z(n), z(n), 0)


def _batches(m, n, T, steps, seed):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal((T, m)), rng.standard_normal((T, n))) for _ in range(steps)]


def _seeds(s):
    return 1000 + s, 2000 + s


def _fn(st, X, b):
    """The layer function of a training state, evaluated on X."""
    m, n = st.Wt.shape
    W = O.natural_weight(st.Wt, st.perm_R, st.perm_P)
    return O.forward(X, W, st.perm_R, st.perm_P, O.side_G(st.q_R, m, b), O.side_G(st.q_P, n, b)).Y


def test_loop_zero_lr_only_repermutes():
    """lr = 0 and q = 0: the factors stay the identity, so each merge only
    re-permutes the weight: W~ = W0[pi_R'][:, pi_P'] for the last seeds, exactly."""
    m, n, b = 10, 7, 4
    W, st = _state(m, n, b, 1)
    out = O.train_steps(st, b, "f64", _batches(m, n, 3, 4, 2), O.AdamHP(lr=0.0), 2, _seeds)
    pR, pP = O.perm_from_seed(1004, m), O.perm_from_seed(2004, n)
    assert np.array_equal(out.perm_R, pR) and np.array_equal(out.perm_P, pP)
    assert np.array_equal(out.Wt, W[pR][:, pP])
    assert not out.q_R.any() and not out.q_P.any() and out.t == 0


@pytest.mark.parametrize("shape", [(10, 7, 4), (12, 12, 6)])
def test_loop_merge_preserves_function(shape):
    """A merge changes how the layer is stored, not what it computes: after the
    same steps, the run that merged at the last step (q = 0, new permutations)
    and the run that did not give the same output on a probe input."""
    m, n, b = shape
    W, st = _state(m, n, b, 3, q_std=0.05)
    batches = _batches(m, n, 4, 3, 4)
    hp = O.AdamHP(lr=0.02, eps=1e-3, weight_decay=0.01)
    merged = O.train_steps(st, b, "f64", batches, hp, 3, _seeds)
    plain = O.train_steps(st, b, "f64", batches, hp, 0, _seeds)
    assert merged.t == 0 and plain.t == 3 and not merged.q_R.any()
    assert not np.array_equal(merged.perm_R, st.perm_R)
    X = np.random.default_rng(9).standard_normal((5, m))
    ref = _fn(plain, X, b)
    np.testing.assert_allclose(_fn(merged, X, b), ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # and the steps did move the function away from the start
    assert np.abs(_fn(st, X, b) - ref).max() > 1e-3


def test_loop_first_step_after_restart():
    """One step after a merge the moments started from zero: m2 = (1 - b2) / (1 - b1)^2 m1^2
    in every slot, and q = -lr g / (|g| + eps) with g = m1 / (1 - b1)."""
    m, n, b = 9, 8, 4
    _, st = _state(m, n, b, 5, q_std=0.03)
    hp = O.AdamHP(lr=0.01, beta1=0.8, beta2=0.95, eps=1e-4)
    out = O.train_steps(st, b, "f64", _batches(m, n, 4, 3, 6), hp, 2, _seeds)
    assert out.t == 1
    for q, m1, m2 in ((out.q_R, out.m1_R, out.m2_R), (out.q_P, out.m1_P, out.m2_P)):
        g = m1 / (1 - hp.beta1)
        np.testing.assert_allclose(m2, (1 - hp.beta2) * g * g, rtol=1e-12, atol=0)
        np.testing.assert_allclose(q, -hp.lr * g / (np.abs(g) + hp.eps), rtol=1e-12, atol=1e-18)
        assert np.abs(g).max() > 0


def test_store_weight_values():
    W = np.array([[1.0 + 2**-30, -3.0], [0.5, 2.0]])
    assert O.store_weight_values(W, "f32")[0, 0] == 1.0
    assert O.store_weight_values(W, "bf16")[1, 1] == 2.0
    v = O.store_weight_values(W, "i8")
    np.testing.assert_allclose(v, W, rtol=0, atol=3.0 / 254 + 1e-12)
    assert np.array_equal(O.store_weight_values(W, "f64"), W)

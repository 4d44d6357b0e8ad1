"""The seeded input generator: determinism, shapes, dtypes, and the oracle's
decoding of the stored bit patterns."""

import numpy as np

import oracle as O
from workloads import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_linear_inputs


def test_workload_shapes():
    w = WORKLOADS["llama8b"]
    assert [(L.m, L.n) for L in w.linears] == [
        (4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096), (4096, 14336), (4096, 14336), (14336, 4096)
    ]
    assert w.b == 512 and w.T == 8192
    assert WORKLOADS["llama1p3b"].linears[4].n == 5461
    assert WORKLOADS["llama13b_int8"].w == "i8"


def test_bf16_rounding_known_values():
    x = np.array([1.0, -2.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-9, 3.0e38], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0);
    # 1 + 3*2^-9 is 3/4 of a step above 1 and rounds up to 1 + 2^-7
    assert bits.tolist() == [0x3F80, 0xC000, 0x3F80, 0x3F81, 0x7F62]
    np.testing.assert_array_equal(bf16_bits_to_f32(bits)[:2], [1.0, -2.0])
    np.testing.assert_array_equal(O.to_f64(bits, "bf16")[:4], [1.0, -2.0, 1.0, 1.0 + 2.0**-7])


def test_linear_inputs_deterministic_and_typed():
    w = WORKLOADS["llama60m"]
    a = make_linear_inputs(w, 6, T=16)
    b = make_linear_inputs(w, 6, T=16)
    assert (a.m, a.n) == (1376, 512)
    for f in ("W0", "q_R", "q_P", "perm_R", "perm_P", "X", "dZ"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.X.dtype == np.uint16 and a.X.shape == (16, 1376)
    assert a.q_R.shape == (6, 256 * 255 // 2) and a.q_R.dtype == np.float32
    assert sorted(a.perm_R.tolist()) == list(range(1376))
    W = O.to_f64(a.W0, "bf16")
    np.testing.assert_allclose(np.linalg.norm(W, axis=0), 1.0, atol=1e-2)
    # dead slots of the partial block are left non-zero on purpose
    iu, ju = np.triu_indices(256, 1)
    assert np.count_nonzero(a.q_R[-1][ju >= 96]) > 0


def test_int8_inputs():
    w = WORKLOADS["llama13b_int8"]
    a = make_linear_inputs(w, 1, T=4)
    assert a.W0.dtype == np.int8 and a.w_scale.shape == (5120,)
    assert np.abs(a.W0.astype(int)).max() <= 127
    W = O.to_f64(a.W0, "i8", a.w_scale)
    np.testing.assert_allclose(np.linalg.norm(W, axis=0), 1.0, rtol=1e-6)

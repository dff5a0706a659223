"""Pins for the oracle's predictor (scores = sigmoid(U relu(V x))).

Source: "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm",
section "The Prediction Problem" (the SparsityPredictor module: bias-free down and up
projections, ReLU between, sigmoid out).
"""
import math

import numpy as np
import pytest

from oracle import oracle as orc


def _np_scores(x, V, U):
    a = np.maximum(V @ x, 0.0)
    z = U @ a
    return a, z, 1.0 / (1.0 + np.exp(-z))


def _bf16(a32):
    """Round float32 values to bfloat16 bit patterns by truncating an already-representable value."""
    return (a32.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dt", [orc.F32, orc.F16, orc.BF16])
def test_predict_matches_numpy_float64(dt):
    rng = np.random.default_rng(7 + dt)
    d, r, f = 96, 24, 200
    x = rng.standard_normal(d)
    V = rng.standard_normal((r, d)) / math.sqrt(d)
    U = rng.standard_normal((f, r)) / math.sqrt(r)
    if dt == orc.F32:
        xs, Vs, Us = (a.astype(np.float32) for a in (x, V, U))
        xw, Vw, Uw = (a.astype(np.float64) for a in (xs, Vs, Us))
    elif dt == orc.F16:
        xs, Vs, Us = (a.astype(np.float16) for a in (x, V, U))
        xw, Vw, Uw = (a.astype(np.float64) for a in (xs, Vs, Us))
    else:
        xs, Vs, Us = (_bf16(a) for a in (x, V, U))
        xw, Vw, Uw = (_bf16_f64(a) for a in (xs, Vs, Us))
    a, z, s = orc.predict(xs, Vs, Us, dt)
    ra, rz, rs = _np_scores(xw, Vw, Uw)
    assert np.allclose(a, ra, rtol=1e-12, atol=1e-12)
    assert np.allclose(z, rz, rtol=1e-12, atol=1e-12)
    # each score is the double sigmoid rounded once to binary32
    assert np.array_equal(s, rs.astype(np.float32))


def test_doubled_factors_reduce_to_the_linear_map():
    """relu(t) - relu(-t) = t, so down = [V; -V], up = [U, -U] gives z = U V x exactly.

    Small integers keep every product and sum exact in double, so the comparison is ==."""
    rng = np.random.default_rng(3)
    d, r, f = 40, 12, 64
    x = rng.integers(-4, 5, d).astype(np.float32)
    V = rng.integers(-3, 4, (r, d)).astype(np.float32)
    U = rng.integers(-3, 4, (f, r)).astype(np.float32)
    V2 = np.concatenate([V, -V], axis=0)
    U2 = np.concatenate([U, -U], axis=1)
    _, z, _ = orc.predict(x, V2, U2, orc.F32)
    exact = [sum(int(U[j, i]) * sum(int(V[i, c]) * int(x[c]) for c in range(d)) for i in range(r))
             for j in range(f)]
    assert np.array_equal(z, np.array(exact, dtype=np.float64))


def test_worked_toy_example():
    """Hand-worked: x = (1, 2), V = [[2, 1]] gives V x = 4 and a = 4; U = (1, 0, -1)^T gives
    z = (4, 0, -4) and s = (1/(1+e^-4), 1/2, 1/(1+e^4)) rounded to binary32."""
    x = np.array([1, 2], np.float32)
    V = np.array([[2, 1]], np.float32)
    U = np.array([[1], [0], [-1]], np.float32)
    a, z, s = orc.predict(x, V, U, orc.F32)
    assert a.tolist() == [4.0]
    assert z.tolist() == [4.0, 0.0, -4.0]
    want = np.array([1 / (1 + math.exp(-4)), 0.5, 1 / (1 + math.exp(4))], np.float32)
    assert np.array_equal(s, want)
    # a negative hidden pre-activation is cut by the ReLU: V x = -1 -> a = 0 -> all scores 1/2
    a, z, s = orc.predict(x, np.array([[1, -1]], np.float32), U, orc.F32)
    assert a.tolist() == [0.0] and z.tolist() == [0.0, 0.0, 0.0] and s.tolist() == [0.5] * 3


def test_predict_rejects_bad_shapes():
    with pytest.raises(ValueError):
        orc.lib()  # ensure loaded
        rc = orc.lib().orc_predict(None, 0, None, 0, None, 0, 0, None, None, None)
        orc._check(rc, "orc_predict")

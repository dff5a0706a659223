"""Pins for the oracle's sparse and dense FFN.

Sources: "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm" --
"The Prediction Problem" (gather the active gate rows and matching down weights),
"The SiLU/GELU Challenge: TurboSparse" (ReLU-fied gated form down(relu(gate x) * up x)),
"Kernel-Level Implementation" (per-neuron dot product then max(acc, 0));
"Activation sparsity" -- "Implementation sketch" (the output over a partition of the active set
is the sum of the parts).
"""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as orc


def _layer(rng, d, f, dt, act=orc.RELU, bias=-0.3):
    x = rng.standard_normal(d)
    W1 = rng.standard_normal((f, d)) / math.sqrt(d)
    Wup = rng.standard_normal((f, d)) / math.sqrt(d) if act == orc.REGLU else None
    W2T = rng.standard_normal((f, d)) / math.sqrt(f)
    b1 = np.full(f, bias, np.float32)
    cast = {orc.F32: np.float32, orc.F16: np.float16}[dt]
    x, W1, W2T = x.astype(cast), W1.astype(cast), W2T.astype(cast)
    Wup = None if Wup is None else Wup.astype(cast)
    return x, W1, b1, Wup, W2T


def _np_masked(x, W1, b1, Wup, W2T, mask, act):
    x64, W164, W2T64 = x.astype(np.float64), W1.astype(np.float64), W2T.astype(np.float64)
    p = W164 @ x64 + b1.astype(np.float64)
    h = np.maximum(p, 0.0)
    if act == orc.REGLU:
        h = h * (Wup.astype(np.float64) @ x64)
    return W2T64.T @ (mask * h)


@pytest.mark.parametrize("dt", [orc.F32, orc.F16])
@pytest.mark.parametrize("act", [orc.RELU, orc.REGLU])
def test_sparse_matches_numpy_masked_dense(dt, act):
    rng = np.random.default_rng(11)
    d, f = 64, 300
    x, W1, b1, Wup, W2T = _layer(rng, d, f, dt, act)
    idx = np.sort(rng.choice(f, 45, replace=False)).astype(np.int32)
    mask = np.zeros(f)
    mask[idx] = 1.0
    h, y = orc.sparse_ffn(x, W1, b1, Wup, W2T, idx, act, dt)
    ref = _np_masked(x, W1, b1, Wup, W2T, mask, act)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert h.shape == (45,)


def test_brute_force_every_subset_small_f():
    rng = np.random.default_rng(2)
    d, f = 16, 8
    x, W1, b1, _, W2T = _layer(rng, d, f, orc.F32)
    for k in range(f + 1):
        for A in itertools.combinations(range(f), k):
            mask = np.zeros(f)
            mask[list(A)] = 1.0
            _, y = orc.sparse_ffn(x, W1, b1, None, W2T, np.array(A, np.int32), orc.RELU, orc.F32)
            ref = _np_masked(x, W1, b1, None, W2T, mask, orc.RELU)
            assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("act", [orc.RELU, orc.REGLU])
def test_all_neurons_equals_dense_bitwise(act):
    rng = np.random.default_rng(4)
    d, f = 48, 120
    x, W1, b1, Wup, W2T = _layer(rng, d, f, orc.F16, act)
    _, y_sparse = orc.sparse_ffn(x, W1, b1, Wup, W2T, np.arange(f, dtype=np.int32), act, orc.F16)
    _, y_dense = orc.dense_ffn(x, W1, b1, Wup, W2T, act, orc.F16)
    assert np.array_equal(y_sparse, y_dense)


def test_relu_true_set_equals_dense_bitwise():
    """Neurons outside the true set contribute exact zeros, so skipping them changes nothing."""
    rng = np.random.default_rng(9)
    d, f = 64, 400
    x, W1, b1, _, W2T = _layer(rng, d, f, orc.F32, bias=-0.5)
    T = orc.true_set(x, W1, b1, orc.F32)
    assert 0 < len(T) < f
    _, y_sparse = orc.sparse_ffn(x, W1, b1, None, W2T, T, orc.RELU, orc.F32)
    _, y_dense = orc.dense_ffn(x, W1, b1, None, W2T, orc.RELU, orc.F32)
    assert np.array_equal(y_sparse, y_dense)
    # dropping one true neuron does change the output (the test has teeth)
    _, y_drop = orc.sparse_ffn(x, W1, b1, None, W2T, T[1:], orc.RELU, orc.F32)
    assert not np.array_equal(y_drop, y_dense)


def test_additivity_over_a_partition():
    rng = np.random.default_rng(12)
    d, f = 32, 200
    x, W1, b1, Wup, W2T = _layer(rng, d, f, orc.F32, orc.REGLU)
    active = np.sort(rng.choice(f, 90, replace=False))
    hot = rng.random(f) < 0.3
    A = np.array([j for j in active if hot[j]], np.int32)
    B = np.array([j for j in active if not hot[j]], np.int32)
    _, y = orc.sparse_ffn(x, W1, b1, Wup, W2T, active.astype(np.int32), orc.REGLU, orc.F32)
    _, ya = orc.sparse_ffn(x, W1, b1, Wup, W2T, A, orc.REGLU, orc.F32)
    _, yb = orc.sparse_ffn(x, W1, b1, Wup, W2T, B, orc.REGLU, orc.F32)
    assert np.allclose(y, ya + yb, rtol=1e-12, atol=1e-13)


def test_neuron_permutation_invariance():
    rng = np.random.default_rng(13)
    d, f = 40, 150
    x, W1, b1, _, W2T = _layer(rng, d, f, orc.F32)
    b1 = rng.standard_normal(f).astype(np.float32) * 0.2
    idx = np.sort(rng.choice(f, 60, replace=False)).astype(np.int32)
    perm = rng.permutation(f)                 # new neuron n holds old neuron perm[n]
    inv = np.argsort(perm)
    idx2 = np.sort(inv[idx]).astype(np.int32)
    _, y = orc.sparse_ffn(x, W1, b1, None, W2T, idx, orc.RELU, orc.F32)
    _, y2 = orc.sparse_ffn(x, W1[perm].copy(), b1[perm].copy(), None, W2T[perm].copy(), idx2,
                           orc.RELU, orc.F32)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("act", [orc.RELU, orc.REGLU])
def test_integer_inputs_exact_against_python_integers(act):
    rng = np.random.default_rng(21)
    d, f = 24, 50
    x = rng.integers(-3, 4, d)
    W1 = rng.integers(-2, 3, (f, d))
    Wup = rng.integers(-2, 3, (f, d))
    W2T = rng.integers(-2, 3, (f, d))
    b1 = rng.integers(-2, 3, f)
    idx = np.sort(rng.choice(f, 20, replace=False)).astype(np.int32)
    h, y = orc.sparse_ffn(x.astype(np.float16), W1.astype(np.float16), b1.astype(np.float32),
                          Wup.astype(np.float16) if act == orc.REGLU else None,
                          W2T.astype(np.float16), idx, act, orc.F16)
    want = [0] * d
    for j in idx:
        p = sum(int(W1[j, c]) * int(x[c]) for c in range(d)) + int(b1[j])
        g = max(p, 0)
        if act == orc.REGLU:
            g *= sum(int(Wup[j, c]) * int(x[c]) for c in range(d))
        for c in range(d):
            want[c] += g * int(W2T[j, c])
    assert y.tolist() == [float(v) for v in want]


def test_reglu_with_unit_up_rows_is_relu_on_the_gate():
    rng = np.random.default_rng(22)
    d, f = 32, 64
    x, W1, b1, _, W2T = _layer(rng, d, f, orc.F32)
    x[0] = 1.0
    Wup = np.zeros((f, d), np.float32)
    Wup[:, 0] = 1.0                               # up_j . x = x_0 = 1
    idx = np.arange(0, f, 3, dtype=np.int32)
    _, y_gated = orc.sparse_ffn(x, W1, b1, Wup, W2T, idx, orc.REGLU, orc.F32)
    _, y_relu = orc.sparse_ffn(x, W1, b1, None, W2T, idx, orc.RELU, orc.F32)
    assert np.array_equal(y_gated, y_relu)


def test_no_bias_is_zero_bias_and_bad_index_is_rejected():
    rng = np.random.default_rng(23)
    x, W1, _, _, W2T = _layer(rng, 16, 20, orc.F32)
    idx = np.array([1, 5, 19], np.int32)
    _, y0 = orc.sparse_ffn(x, W1, None, None, W2T, idx, orc.RELU, orc.F32)
    _, yz = orc.sparse_ffn(x, W1, np.zeros(20, np.float32), None, W2T, idx, orc.RELU, orc.F32)
    assert np.array_equal(y0, yz)
    with pytest.raises(ValueError):
        orc.sparse_ffn(x, W1, None, None, W2T, np.array([20], np.int32), orc.RELU, orc.F32)
    _, y_empty = orc.sparse_ffn(x, W1, None, None, W2T, np.zeros(0, np.int32), orc.RELU, orc.F32)
    assert not y_empty.any()

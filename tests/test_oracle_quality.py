"""Pins for the oracle's recall/precision, batched (union) and stacked forms.

Sources: "Contextual Sparsity and Activation Predictors" -- "Precision, recall, and which error
hurts" (false positives cost bandwidth, false negatives drop output), "When it breaks" (a batch
reads the union of its tokens' sets; look-ahead is weakest early), "The predictor and its
budget" (x_{l+1} = x_l + f_l(x_l); predict layer l+1 from layer l's input).
"""
import math

import numpy as np
import pytest

from oracle import oracle as orc


def _doubled_predictor_layer(rng, d=10, r=4, f=60, bias=-2.5):
    """W1 = U V exactly (small integers) and a predictor with down = [V; -V], up = [U, -U], so the
    predictor's logit is exactly W1 x: its scores order neurons by their pre-activation."""
    V = rng.integers(-2, 3, (r, d)).astype(np.float32)
    U = rng.integers(-2, 3, (f, r)).astype(np.float32)
    x = rng.integers(-1, 2, d).astype(np.float32)
    W1 = (U.astype(np.int64) @ V.astype(np.int64)).astype(np.float32)
    b1 = np.full(f, bias, np.float32)
    return x, V, U, W1, b1, np.concatenate([V, -V], 0), np.concatenate([U, -U], 1)


@pytest.mark.parametrize("seed", range(5))
def test_recall_closed_form_for_an_exact_predictor(seed):
    rng = np.random.default_rng(seed)
    x, V, U, W1, b1, Vd, Ud = _doubled_predictor_layer(rng)
    _, z, s = orc.predict(x, Vd, Ud, orc.F32)
    T = orc.true_set(x, W1, b1, orc.F32)
    assert np.array_equal(z[T] + b1[T], (W1 @ x + b1)[T])
    # no member of the true set shares a score with a non-member (saturation ties at 1.0 can only
    # occur inside the true set, where they do not change recall or precision)
    outside = np.setdiff1d(np.arange(len(s)), T)
    assert s[T].min() > s[outside].max()
    f = W1.shape[0]
    nT = len(T)
    assert 0 < nT < f
    for k in range(0, f + 1, 3):
        A = orc.select_topk(s, k)
        rec, prec = orc.recall_precision(A, T)
        if k >= nT:
            assert rec == 1.0 and prec == pytest.approx(nT / k if k else 1.0)
        else:
            assert rec == pytest.approx(k / nT) and prec == 1.0


def test_recall_precision_empty_conventions():
    assert orc.recall_precision([], []) == (1.0, 1.0)
    assert orc.recall_precision([1, 2], []) == (1.0, 0.0)
    assert orc.recall_precision([], [3]) == (0.0, 1.0)


def _ffn(rng, d=24, f=90, act=orc.RELU):
    W1 = (rng.standard_normal((f, d)) / math.sqrt(d)).astype(np.float32)
    Wup = (rng.standard_normal((f, d)) / math.sqrt(d)).astype(np.float32) if act == orc.REGLU else None
    W2T = (rng.standard_normal((f, d)) / math.sqrt(f)).astype(np.float32)
    b1 = np.full(f, -0.2, np.float32)
    return W1, b1, Wup, W2T


@pytest.mark.parametrize("act", [orc.RELU, orc.REGLU])
def test_batched_invariants(act):
    rng = np.random.default_rng(31)
    W1, b1, Wup, W2T = _ffn(rng, act=act)
    f, d = W1.shape
    B = 5
    X = rng.standard_normal((B, d)).astype(np.float32)
    sets = [np.sort(rng.choice(f, rng.integers(0, 30), replace=False)).astype(np.int32) for _ in range(B)]
    # per-token: the same as running each token alone
    Y = orc.batched_ffn(X, sets, W1, b1, Wup, W2T, act, orc.F32)
    for t in range(B):
        assert np.array_equal(Y[t], orc.sparse_ffn(X[t], W1, b1, Wup, W2T, sets[t], act, orc.F32)[1])
    # batch of one: union and per-token agree
    Y1 = orc.batched_ffn(X[:1], sets[:1], W1, b1, Wup, W2T, act, orc.F32, union=True)
    assert np.array_equal(Y1[0], Y[0])
    # union of everything is the dense layer for every token
    full = [np.arange(f, dtype=np.int32)] + sets[1:]
    Yu = orc.batched_ffn(X, full, W1, b1, Wup, W2T, act, orc.F32, union=True)
    for t in range(B):
        assert np.array_equal(Yu[t], orc.dense_ffn(X[t], W1, b1, Wup, W2T, act, orc.F32)[1])
    # the union is the set union, and its bitmap is the OR of the tokens' bitmaps
    u = orc.union_of(sets, f)
    assert u.tolist() == sorted(set().union(*[set(s.tolist()) for s in sets]))
    ors = np.zeros((f + 31) // 32, np.uint32)
    for s in sets:
        ors |= orc.to_bitmap(s, f)
    assert np.array_equal(ors, orc.to_bitmap(u, f))


def test_bitmap_layout():
    bm = orc.to_bitmap(np.array([0, 31, 32, 70], np.int32), 71)
    assert bm.tolist() == [0x80000001, 0x00000001, 0x00000040]


def test_rms_normalize_matches_numpy():
    rng = np.random.default_rng(40)
    x = (rng.standard_normal(257) * 3.0).astype(np.float32)
    ref = x.astype(np.float64) / np.sqrt(np.mean(x.astype(np.float64) ** 2) + 1e-6)
    assert np.array_equal(orc.rms_normalize(x, orc.F32), ref.astype(np.float32))
    assert np.array_equal(orc.rms_normalize(x, orc.F16).view(np.uint16),
                          ref.astype(np.float16).view(np.uint16))
    got_bf = orc.rms_normalize(x, orc.BF16).astype(np.uint32)
    back = (got_bf << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(back - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)


def _stack_layers(rng, L, d, f, r, zero_out=False):
    layers = []
    for _ in range(L):
        V = (rng.standard_normal((r, d)) / math.sqrt(d)).astype(np.float16)
        U = (rng.standard_normal((f, r)) / math.sqrt(r)).astype(np.float16)
        W1 = (rng.standard_normal((f, d)) / math.sqrt(d)).astype(np.float16)
        W2T = (rng.standard_normal((f, d)) / math.sqrt(f)).astype(np.float16)
        if zero_out:
            W2T[:] = 0
        layers.append(dict(V=V, U=U, W1=W1, b1=np.full(f, -0.3, np.float32), Wup=None, W2T=W2T,
                           act=orc.RELU))
    return layers


def test_stack_single_layer_is_one_residual_block():
    rng = np.random.default_rng(41)
    d, f, r = 32, 96, 8
    layers = _stack_layers(rng, 1, d, f, r)
    x0 = rng.standard_normal(d).astype(np.float32)
    xL, sets, xhats = orc.stack_forward(x0, layers, orc.F16, k=20)
    L = layers[0]
    xh = orc.rms_normalize(x0, orc.F16)
    idx = orc.select_topk(orc.predict(xh, L["V"], L["U"], orc.F16)[2], 20)
    y = orc.sparse_ffn(xh, L["W1"], L["b1"], None, L["W2T"], idx, orc.RELU, orc.F16)[1]
    assert np.array_equal(sets[0], idx)
    assert np.array_equal(xL, (x0.astype(np.float64) + y).astype(np.float32))


def test_lookahead_equals_sync_when_the_stream_does_not_move():
    """With a zero down projection every block adds nothing, so layer l-1's input is exactly layer
    l's input and predicting one layer ahead must give the synchronous sets."""
    rng = np.random.default_rng(42)
    d, f, r = 32, 80, 8
    layers = _stack_layers(rng, 4, d, f, r, zero_out=True)
    x0 = rng.standard_normal(d).astype(np.float32)
    xs, sets_sync, _ = orc.stack_forward(x0, layers, orc.F16, k=16)
    xl, sets_la, _ = orc.stack_forward(x0, layers, orc.F16, k=16, lookahead=True)
    assert np.array_equal(xs, x0) and np.array_equal(xl, x0)
    # layer l in look-ahead mode uses layer l's predictor on layer l-1's input, which equals
    # layer l's own input here
    for a, b in zip(sets_sync, sets_la):
        assert np.array_equal(a, b)


def test_lookahead_uses_the_previous_layers_input():
    rng = np.random.default_rng(43)
    d, f, r = 32, 80, 8
    layers = _stack_layers(rng, 3, d, f, r)
    x0 = rng.standard_normal(d).astype(np.float32)
    _, sets, xhats = orc.stack_forward(x0, layers, orc.F16, k=16, lookahead=True)
    for l in (1, 2):
        s = orc.predict(xhats[l - 1], layers[l]["V"], layers[l]["U"], orc.F16)[2]
        assert np.array_equal(sets[l], orc.select_topk(s, 16))
    s0 = orc.predict(xhats[0], layers[0]["V"], layers[0]["U"], orc.F16)[2]
    assert np.array_equal(sets[0], orc.select_topk(s0, 16))

"""The oracle's multi-threaded loops change no bit of any result.

The oracle shares whole rows (predictor hidden units and scores, FFN activations) and whole column
blocks of the FFN output among OpenMP threads; each output element stays one double-precision sum
in ascending index order formed by one thread.  So predict, sparse_ffn and dense_ffn must return
bitwise-identical arrays for every thread count, including counts that do not divide the work
evenly and shapes with ragged column blocks.
"""
import numpy as np
import pytest

from oracle import oracle as orc


@pytest.fixture(autouse=True)
def _restore_threads():
    yield
    orc.set_threads(1)


def _layer(rng, d, f, r, dt):
    def st(shape, scale):
        v = rng.standard_normal(shape) * scale
        return v.astype(np.float32) if dt == orc.F32 else orc.round_to_storage(v, dt).reshape(shape)
    return dict(x=st((d,), 1.0), V=st((r, d), d ** -0.5), U=st((f, r), r ** -0.5),
                W1=st((f, d), d ** -0.5), Wup=st((f, d), d ** -0.5), W2T=st((f, d), f ** -0.5),
                b1=(rng.standard_normal(f) * 0.3).astype(np.float32))


@pytest.mark.parametrize("dt", [orc.F32, orc.F16, orc.BF16])
@pytest.mark.parametrize("act", [orc.RELU, orc.REGLU, orc.SILU])
def test_thread_count_changes_no_bit(dt, act):
    rng = np.random.default_rng(100 + 10 * dt + act)
    d, f, r = 700, 611, 40                        # 700 columns: blocks of 256, 256, 188
    L = _layer(rng, d, f, r, dt)
    Wup = L["Wup"] if act == orc.REGLU else None
    idx = np.sort(rng.permutation(f)[:203]).astype(np.int32)
    results = []
    for n in (1, 2, 3, 8):
        orc.set_threads(n)
        assert orc.get_threads() == n
        a, z, s = orc.predict(L["x"], L["V"], L["U"], dt)
        hs, ys = orc.sparse_ffn(L["x"], L["W1"], L["b1"], Wup, L["W2T"], idx, act, dt)
        hd, yd = orc.dense_ffn(L["x"], L["W1"], L["b1"], Wup, L["W2T"], act, dt)
        results.append((a, z, s, hs, ys, hd, yd))
    for other in results[1:]:
        for want, got in zip(results[0], other):
            assert want.dtype == got.dtype and np.array_equal(want, got)


def test_bad_thread_count_and_bad_index():
    with pytest.raises(ValueError):
        orc.set_threads(0)
    orc.set_threads(4)
    rng = np.random.default_rng(5)
    L = _layer(rng, 64, 50, 8, orc.F32)
    with pytest.raises(ValueError):
        orc.sparse_ffn(L["x"], L["W1"], L["b1"], None, L["W2T"], np.array([3, 50], np.int32),
                       orc.RELU, orc.F32)

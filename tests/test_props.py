"""Property tests over random shapes, ties, k and tau.

CPU part (the oracle against invariants the pages and the arithmetic fix, at shapes the fixed
pins do not reach: odd d and f, any k, random tie patterns, random tau):
  * top-k ("Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm", "The
    Prediction Problem") equals a stable descending sort cut at k (lower index first on ties),
    and the top-k sets are nested in k;
  * threshold ("Activation sparsity", "Implementation sketch") is {j : s_j >= tau} and shrinks as
    tau grows;
  * the sparse FFN over every neuron is the dense FFN; over a partition of a set it is the sum of
    the parts; for ReLU over the true positive set it is the dense output;
  * predictor scores lie in [0, 1] and follow a permutation of U's rows;
  * the union of a batch's sets is their set union ("Contextual Sparsity and Activation
    Predictors", "When it breaks") and the bitmap holds exactly the set.
GPU part (marked gpu): the HIP path through the C ABI against the oracle on random shapes with
ragged tails, random tie patterns and random k / tau; selection bit-exact, FFN outputs within
the normwise bars.  Examples are derandomized, so every run tries the same cases.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import contextual_sparsity_ffn_amd as csf
from csf_testutil import announce, assert_ffn_close, to_orc
from oracle import oracle as orc

CPU_SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                        suppress_health_check=[HealthCheck.too_slow])
GPU_SETTINGS = settings(max_examples=20, deadline=None, derandomize=True,
                        suppress_health_check=[HealthCheck.too_slow])

DTYPES = [(orc.F32, np.float32), (orc.F16, np.float16), (orc.BF16, None)]


def _scores(rng, f, levels):
    """f scores in [0, 1] on `levels` distinct values (few levels: heavy ties)."""
    return (np.floor(rng.random(f) * levels) / max(levels, 1)).astype(np.float32)


def _storage(rng, shape, dt, scale=1.0):
    v = rng.standard_normal(shape) * scale
    if dt == orc.F32:
        return v.astype(np.float32)
    return orc.round_to_storage(v, dt).reshape(shape)


# ---- selection ----------------------------------------------------------------------------------
@CPU_SETTINGS
@given(f=st.integers(0, 3000), levels=st.integers(1, 60), seed=st.integers(0, 2 ** 31 - 1),
       kfrac=st.floats(0.0, 1.0), k2frac=st.floats(0.0, 1.0))
def test_prop_topk_is_a_stable_sort_cut_and_nested(f, levels, seed, kfrac, k2frac):
    rng = np.random.default_rng(seed)
    s = _scores(rng, f, levels)
    k = int(round(kfrac * f))
    k2 = int(round(k2frac * f))
    A = orc.select_topk(s, k)
    assert A.tolist() == sorted(np.argsort(-s, kind="stable")[:k].tolist())
    A2 = orc.select_topk(s, k2)
    small, big = (A, A2) if k <= k2 else (A2, A)
    assert set(small.tolist()) <= set(big.tolist())


@CPU_SETTINGS
@given(f=st.integers(0, 3000), levels=st.integers(1, 60), seed=st.integers(0, 2 ** 31 - 1),
       pick=st.integers(0, 10 ** 6), t2=st.floats(0.0, 1.0, width=32))
def test_prop_threshold_is_the_superlevel_set_and_monotone(f, levels, seed, pick, t2):
    rng = np.random.default_rng(seed)
    s = _scores(rng, f, levels)
    tau = s[pick % f] if f else np.float32(0.5)         # a tau equal to a score: the >= edge
    A = orc.select_threshold(s, tau)
    assert A.tolist() == np.nonzero(s >= np.float32(tau))[0].tolist()
    B = orc.select_threshold(s, t2)
    lo, hi = (A, B) if float(tau) >= t2 else (B, A)
    assert set(lo.tolist()) <= set(hi.tolist())


# ---- FFN ------------------------------------------------------------------------------------------
@CPU_SETTINGS
@given(d=st.integers(1, 67), f=st.integers(1, 97), act=st.sampled_from([orc.RELU, orc.REGLU,
                                                                       orc.SILU, orc.SWIGLU]),
       dti=st.integers(0, 2), seed=st.integers(0, 2 ** 31 - 1), frac=st.floats(0.0, 1.0))
def test_prop_ffn_odd_shapes(d, f, act, dti, seed, frac):
    dt = DTYPES[dti][0]
    rng = np.random.default_rng(seed)
    x = _storage(rng, (d,), dt)
    W1 = _storage(rng, (f, d), dt, 1 / np.sqrt(d))
    W2T = _storage(rng, (f, d), dt, 1 / np.sqrt(f))
    Wup = _storage(rng, (f, d), dt, 1 / np.sqrt(d)) if act in (orc.REGLU, orc.SWIGLU) else None
    b1 = (rng.standard_normal(f) * 0.3).astype(np.float32)
    every = np.arange(f, dtype=np.int32)
    hd, yd = orc.dense_ffn(x, W1, b1, Wup, W2T, act, dt)
    hs, ys = orc.sparse_ffn(x, W1, b1, Wup, W2T, every, act, dt)
    assert np.array_equal(yd, ys) and np.array_equal(hd, hs)     # k = f is the dense layer
    # additivity over a random partition of a random set
    S = np.sort(rng.permutation(f)[: int(round(frac * f))]).astype(np.int32)
    mask = rng.random(S.shape[0]) < 0.5
    _, y = orc.sparse_ffn(x, W1, b1, Wup, W2T, S, act, dt)
    _, ya = orc.sparse_ffn(x, W1, b1, Wup, W2T, S[mask], act, dt)
    _, yb = orc.sparse_ffn(x, W1, b1, Wup, W2T, S[~mask], act, dt)
    scale = np.abs(ya).sum() + np.abs(yb).sum() + 1e-300
    assert np.abs(y - (ya + yb)).max() <= 1e-12 * scale
    if act == orc.RELU:
        T = orc.true_set(x, W1, b1, dt)
        _, yt = orc.sparse_ffn(x, W1, b1, None, W2T, T, act, dt)
        assert np.array_equal(yt, yd)                          # zeros add nothing


@CPU_SETTINGS
@given(d=st.integers(1, 67), r=st.integers(1, 33), f=st.integers(1, 97), dti=st.integers(0, 2),
       seed=st.integers(0, 2 ** 31 - 1))
def test_prop_predictor_range_and_row_permutation(d, r, f, dti, seed):
    dt = DTYPES[dti][0]
    rng = np.random.default_rng(seed)
    x = _storage(rng, (d,), dt)
    V = _storage(rng, (r, d), dt, 1 / np.sqrt(d))
    U = _storage(rng, (f, r), dt, 1 / np.sqrt(r))
    a, z, s = orc.predict(x, V, U, dt)
    assert (a >= 0).all() and (s >= 0).all() and (s <= 1).all()
    perm = rng.permutation(f)
    _, z2, s2 = orc.predict(x, V, np.ascontiguousarray(U[perm]), dt)
    assert np.array_equal(s2, s[perm]) and np.array_equal(z2, z[perm])


@CPU_SETTINGS
@given(f=st.integers(1, 300), B=st.integers(1, 8), seed=st.integers(0, 2 ** 31 - 1))
def test_prop_union_and_bitmap(f, B, seed):
    rng = np.random.default_rng(seed)
    sets = [np.sort(rng.permutation(f)[: rng.integers(0, f + 1)]).astype(np.int32)
            for _ in range(B)]
    U = orc.union_of(sets, f)
    ref = np.unique(np.concatenate(sets)) if sets else np.zeros(0)
    assert U.tolist() == ref.tolist()
    for s in sets:
        bm = orc.to_bitmap(s, f)
        assert sum(bin(int(w)).count("1") for w in bm) == len(s)
        got = [j for j in range(f) if (int(bm[j // 32]) >> (j % 32)) & 1]
        assert got == s.tolist()


# ---- GPU: the HIP path against the oracle on random shapes -------------------------------------
DEV = torch.device("cuda:0")
TORCH_DT = {orc.F32: torch.float32, orc.F16: torch.float16, orc.BF16: torch.bfloat16}


def _weights(g, shape, dtype, scale):
    return (torch.randn(shape, generator=g) * scale).to(dtype)


@pytest.mark.gpu
@GPU_SETTINGS
@given(f=st.integers(1, 60000), B=st.integers(1, 3), levels=st.integers(1, 5000),
       seed=st.integers(0, 2 ** 31 - 1), kfrac=st.floats(0.0, 1.0), tau=st.floats(0.0, 1.0))
def test_gpu_prop_selection_matches_the_oracle(f, B, levels, seed, kfrac, tau):
    announce(f"prop selection f={f} B={B} levels={levels} seed={seed}")
    rng = np.random.default_rng(seed)
    S = np.stack([_scores(rng, f, levels) for _ in range(B)])
    k = int(round(kfrac * f))
    Sd = torch.from_numpy(S).to(DEV)
    idx = csf.select_topk(Sd, k)
    tidx, tcount = csf.select_threshold(Sd, tau)
    torch.cuda.synchronize()
    for t in range(B):
        assert idx[t, :k].cpu().numpy().tolist() == orc.select_topk(S[t], k).tolist(), t
        n = int(tcount[t].item())
        assert tidx[t, :n].cpu().numpy().tolist() == orc.select_threshold(S[t], tau).tolist(), t


@pytest.mark.gpu
@GPU_SETTINGS
@given(d8=st.integers(1, 160), f=st.integers(1, 5000), act=st.sampled_from([csf.RELU, csf.REGLU,
                                                                            csf.SILU, csf.SWIGLU]),
       dti=st.integers(0, 2), seed=st.integers(0, 2 ** 31 - 1), frac=st.floats(0.0, 1.0),
       B=st.integers(1, 3))
def test_gpu_prop_sparse_ffn_matches_the_oracle(d8, f, act, dti, seed, frac, B):
    dt = DTYPES[dti][0]
    d = 8 * d8                                           # whole 16-byte rows for every type
    tdt = TORCH_DT[dt]
    announce(f"prop sparse_ffn d={d} f={f} act={act} dt={dt} B={B} seed={seed}")
    g = torch.Generator().manual_seed(seed)
    W1 = _weights(g, (f, d), tdt, d ** -0.5)
    Wup = _weights(g, (f, d), tdt, d ** -0.5) if act in (csf.REGLU, csf.SWIGLU) else None
    W2T = _weights(g, (f, d), tdt, f ** -0.5)
    b1 = torch.randn(f, generator=g) * 0.3
    X = _weights(g, (B, d), tdt, 1.0)
    m = int(round(frac * f))
    lists = [torch.sort(torch.randperm(f, generator=g)[:m]).values.to(torch.int32)
             for _ in range(B)]
    I = torch.stack(lists) if m else torch.zeros(B, 1, dtype=torch.int32)
    dv = lambda t: None if t is None else t.to(DEV)
    Y = csf.sparse_ffn(dv(X), dv(W1), dv(b1), dv(Wup), dv(W2T), dv(I), act=act,
                       max_count=m)
    torch.cuda.synchronize()
    for t in range(B):
        _, ref = orc.sparse_ffn(to_orc(X[t]), to_orc(W1), to_orc(b1),
                                None if Wup is None else to_orc(Wup), to_orc(W2T),
                                lists[t].numpy(), act, dt)
        if m == 0:
            assert not Y[t].any()
        else:
            assert_ffn_close(Y[t], ref, tdt, f"prop d={d} f={f} token {t}")


@pytest.mark.gpu
@GPU_SETTINGS
@given(d8=st.integers(1, 96), r8=st.integers(1, 24), f=st.integers(2, 6000),
       act=st.sampled_from([csf.RELU, csf.REGLU]), dti=st.integers(0, 2),
       seed=st.integers(0, 2 ** 31 - 1), kfrac=st.floats(0.0, 1.0), tau=st.floats(0.3, 0.7),
       use_k=st.booleans())
def test_gpu_prop_layer_matches_the_oracle(d8, r8, f, act, dti, seed, kfrac, tau, use_k):
    dt = DTYPES[dti][0]
    d, r = 8 * d8, 8 * r8
    tdt = TORCH_DT[dt]
    k = int(round(kfrac * f)) if use_k else None
    announce(f"prop layer d={d} r={r} f={f} act={act} dt={dt} k={k} tau={tau} seed={seed}")
    g = torch.Generator().manual_seed(seed)
    V = _weights(g, (r, d), tdt, d ** -0.5)
    U = _weights(g, (f, r), tdt, r ** -0.5)
    W1 = _weights(g, (f, d), tdt, d ** -0.5)
    Wup = _weights(g, (f, d), tdt, d ** -0.5) if act == csf.REGLU else None
    W2T = _weights(g, (f, d), tdt, f ** -0.5)
    b1 = torch.randn(f, generator=g) * 0.3
    x = _weights(g, (d,), tdt, 1.0)
    dv = lambda t: None if t is None else t.to(DEV)
    scores = torch.empty(f, dtype=torch.float32, device=DEV)
    idx = torch.empty(f, dtype=torch.int32, device=DEV)
    count = torch.empty(1, dtype=torch.int32, device=DEV)
    y = csf.sparse_ffn_layer(dv(x), dv(V), dv(U), dv(W1), dv(b1), dv(Wup), dv(W2T), k=k,
                             tau=None if use_k else tau, act=act, scores=scores, idx=idx,
                             count=count)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    _, _, s_ref = orc.predict(to_orc(x), to_orc(V), to_orc(U), dt)
    assert np.abs(s.astype(np.float64) - s_ref).max() <= 1e-5
    n = int(count.item())
    ix = idx[:n].cpu().numpy()
    want = orc.select_topk(s, k) if use_k else orc.select_threshold(s, tau)
    assert ix.tolist() == want.tolist()                   # bit-exact on the GPU's own scores
    _, ref = orc.sparse_ffn(to_orc(x), to_orc(W1), to_orc(b1),
                            None if Wup is None else to_orc(Wup), to_orc(W2T), ix, act, dt)
    if n == 0:
        assert not y.any()
    else:
        assert_ffn_close(y, ref, tdt, f"prop layer d={d} f={f}")

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bars: predictor scores within 1e-5 absolute; selection bit-exact when the oracle is fed the same
scores; FFN outputs within the normwise bars of csf_testutil (1e-5 float32, 2e-2 16-bit, plus the
tighter 1e-4 accumulation bound); integer-valued inputs bit-exact.
"""
import dataclasses

import numpy as np
import pytest
import torch

import contextual_sparsity_ffn_amd as csf
from contextual_sparsity_ffn_amd import workloads as wl
from csf_testutil import (ORC_DT, announce, assert_ffn_close, layer_to_orc, to_orc)
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _dev(t):
    return t.to(DEV)


def _layer(cfg):
    return wl.make_layer(cfg, device="cpu")


def _to_dev_layer(L):
    return wl.Layer(L.cfg, _dev(L.V), _dev(L.U), _dev(L.W1), _dev(L.b1),
                    None if L.Wup is None else _dev(L.Wup), _dev(L.W2T))


# shapes that span several workgroup tiles and end in ragged tails
PRED_CASES = [
    ("c0", wl.TINY_F32, 3),
    ("f16-ragged", wl.OPT175B.scaled(2600, 3001, 136), 2),
    ("bf16", wl.LLAMA_REGLU.scaled(4096, 1433, 256), 2),
    ("f16-r1024", wl.OPT175B.scaled(1024, 2050, 1024), 1),
    # one token: the persistent up projection (2048 workgroups over the row groups) with fewer
    # rows than one group, and with more groups than workgroups and a ragged last group
    ("f16-B1-tiny-f", wl.OPT175B.scaled(512, 7, 64), 1),
    ("f16-B1-many-groups-ragged", wl.OPT175B.scaled(512, 40001, 64), 1),
    ("f32-B1-many-groups-ragged", wl.TINY_F32.scaled(256, 33333, 64), 1),
    # batches of 4 or more 16-bit tokens with d, r multiples of 128 take the matrix-core predictor
    ("f16-B8-mfma", wl.OPT30B.scaled(1024, 2333, 128), 8),
    ("bf16-B20-mfma", wl.LLAMA_REGLU.scaled(512, 1433, 256), 20),
    ("f16-B37-mfma", wl.OPT175B.scaled(1024, 1000, 256), 37),
    ("f16-B5-r1024-mfma", wl.OPT175B.scaled(2048, 3001, 1024), 5),
    # r = 512: four K steps per wave, the most the register-resident up projection holds
    ("f16-B12-r512-mfma", wl.OPT30B.scaled(1024, 3001, 512), 12),
    ("bf16-B32-r512-mfma", wl.LLAMA_REGLU.scaled(512, 2049, 512), 32),
    ("f16-B6-ragged-valu", wl.OPT175B.scaled(2600, 3001, 136), 6),
]


@pytest.mark.parametrize("name,cfg,B", PRED_CASES, ids=[c[0] for c in PRED_CASES])
def test_predict_scores(name, cfg, B):
    announce(f"predict {name}")
    L = _layer(cfg)
    X = wl.make_tokens(cfg, B)
    s = csf.predict_active(_dev(X), _dev(L.V), _dev(L.U))
    torch.cuda.synchronize()
    o = layer_to_orc(L)
    for t in range(B):
        _, _, s_ref = orc.predict(to_orc(X[t]), o["V"], o["U"], o["dt"])
        diff = np.abs(s[t].cpu().numpy().astype(np.float64) - s_ref.astype(np.float64)).max()
        assert diff <= 1e-5, (name, t, diff)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_predict_large_hidden_keeps_its_range(dtype):
    """The batched matrix-core predictor multiplies relu(V x) with U as 16-bit terms; binary16
    holds magnitudes up to 65504, so a token whose hidden values reach 2^15 is split after a
    power-of-two scale.  Half the tokens get x scaled by 2^6 and V by 2^8 (largest hidden value
    well past 65504, checked on the oracle), with U scaled by 2^-14 so that their scores stay
    away from 0 and 1; exact powers of two, so the oracle sees the same stored values."""
    announce(f"predict large hidden {dtype}")
    cfg = wl.OPT30B.scaled(1024, 2333, 128)
    cfg = dataclasses.replace(cfg, dtype=dtype)
    L = _layer(cfg)
    B = 8
    X = wl.make_tokens(cfg, B).float()
    X[: B // 2] *= 2.0 ** 6
    X = X.to(dtype)
    V = (L.V.float() * 2.0 ** 8).to(dtype)
    U = (L.U.float() * 2.0 ** -14).to(dtype)
    s = csf.predict_active(_dev(X), _dev(V), _dev(U))
    torch.cuda.synchronize()
    assert torch.isfinite(s).all()
    dt = ORC_DT[dtype]
    mid = 0
    for t in range(B):
        a, _, s_ref = orc.predict(to_orc(X[t]), to_orc(V), to_orc(U), dt)
        if t < B // 2:
            assert a.max() > 65504, "the scaled tokens must need the wide range"
        mid += int(((s_ref > 0.05) & (s_ref < 0.95)).sum())
        diff = np.abs(s[t].cpu().numpy().astype(np.float64) - s_ref.astype(np.float64)).max()
        assert diff <= 1e-5, (t, diff)
    assert mid > B * cfg.f // 10, "scores must not all saturate"


def _score_patterns(f, g):
    u = torch.rand(f, generator=g)
    q = torch.round(torch.rand(f, generator=g) * 16) / 16            # heavy ties
    eq = torch.full((f,), 0.5)
    z = torch.where(torch.rand(f, generator=g) < 0.5, torch.tensor(-0.0), torch.tensor(0.0))
    sat = torch.where(torch.rand(f, generator=g) < 0.3, torch.tensor(1.0), torch.rand(f, generator=g))
    sig = torch.sigmoid(torch.randn(f, generator=g) * 2.45)
    # descending ramp: the k largest are the first k indices, so whole slices of a many-workgroup
    # selection lie above the boundary bucket (more members than any per-slice prefix holds)
    ramp = torch.linspace(1.0, 0.0, f)
    # a band narrower than one bucket (1/2048): more candidates than the direct ranking takes.
    # Distinct values, and the same band on a grid of 2^-22 (duplicates, but no one value
    # holding the k-th place alone), go through the radix passes; the tie patterns above take
    # the shortcut (the bucket's largest value fills the k-th place).
    band = 0.5 + torch.rand(f, generator=g) * 4e-4
    grid = torch.round(band * 2.0 ** 22) / 2.0 ** 22
    return {"uniform": u, "ties": q, "all-equal": eq, "signed-zero": z, "saturated": sat,
            "sigmoid": sig, "ramp": ramp, "band": band, "band-grid": grid}


SELECT_F = [1, 7, 1000, 1024, 1025, 3001, 30001, 49152, 65536]


@pytest.mark.parametrize("f", SELECT_F)
def test_select_topk_bit_exact(f):
    g = torch.Generator().manual_seed(f)
    pats = _score_patterns(f, g)
    for pname, s in pats.items():
        for k in sorted({0, 1, max(f // 20, 1), f // 2, max(f - 1, 0), f}):
            if k > f:
                continue
            announce(f"select_topk f={f} k={k} pattern={pname}")
            S = torch.stack([s, s.flip(0)]).float().contiguous()
            words = (f + 31) // 32
            bm = torch.empty(2, words, dtype=torch.int32, device=DEV)
            cnt = torch.empty(2, dtype=torch.int32, device=DEV)
            idx = csf.select_topk(_dev(S), k, count=cnt, bitmap=bm)
            torch.cuda.synchronize()
            for t in range(2):
                ref = orc.select_topk(S[t].numpy(), k)
                got = idx[t].cpu().numpy()
                assert np.array_equal(got, ref), (f, k, pname, t)
                assert cnt[t].item() == k
                want_bm = orc.to_bitmap(ref, f).view(np.int32)
                assert np.array_equal(bm[t].cpu().numpy(), want_bm), (f, k, pname, t)


@pytest.mark.parametrize("f", SELECT_F)
def test_select_threshold_bit_exact(f):
    g = torch.Generator().manual_seed(1000 + f)
    pats = _score_patterns(f, g)
    for pname, s in pats.items():
        for tau in (0.0, 0.25, 0.5, 0.9375, 1.0, 2.0):
            announce(f"select_threshold f={f} tau={tau} pattern={pname}")
            S = torch.stack([s, s.flip(0)]).float().contiguous()
            words = (f + 31) // 32
            bm = torch.empty(2, words, dtype=torch.int32, device=DEV)
            idx, cnt = csf.select_threshold(_dev(S), tau, bitmap=bm)
            torch.cuda.synchronize()
            for t in range(2):
                ref = orc.select_threshold(S[t].numpy(), tau)
                n = cnt[t].item()
                assert n == len(ref), (f, tau, pname, t)
                assert np.array_equal(idx[t, :n].cpu().numpy(), ref)
                assert np.array_equal(bm[t].cpu().numpy(), orc.to_bitmap(ref, f).view(np.int32))


def _topk_nan_last(s, k):
    """Top-k with the library's documented order for non-finite scores: a NaN ranks below every
    number (-inf included); otherwise score descending, -0.0 equal to +0.0, lower index first."""
    v = s.astype(np.float64)
    order = sorted(range(len(v)), key=lambda j: (1, 0.0, j) if np.isnan(v[j]) else (0, -v[j] + 0.0, j))
    return np.sort(np.array(order[:k], dtype=np.int64))


@pytest.mark.parametrize("f", [3001, 49152])
def test_select_topk_with_nan_scores(f):
    """NaN scores (e.g. from non-finite inputs) never leave the list short or stale: both the
    one-workgroup and the many-workgroup selections return exactly k neurons, NaN ranked last."""
    g = torch.Generator().manual_seed(77 + f)
    base = torch.rand(f, generator=g)
    few = base.clone()
    few[torch.rand(f, generator=g) < 0.1] = float("nan")
    most = torch.full((f,), float("nan"))
    keep = torch.randperm(f, generator=g)[: f // 50]
    most[keep] = base[keep]
    most[keep[:3]] = float("-inf")
    for pname, sc in (("some-nan", few), ("mostly-nan", most)):
        for k in (1, f // 20, f // 10, f // 2):
            announce(f"select_topk NaN f={f} k={k} pattern={pname}")
            S = torch.stack([sc, sc.flip(0)]).float().contiguous()
            cnt = torch.empty(2, dtype=torch.int32, device=DEV)
            idx = csf.select_topk(_dev(S), k, count=cnt)
            torch.cuda.synchronize()
            for t in range(2):
                ref = _topk_nan_last(S[t].numpy(), k)
                assert cnt[t].item() == k
                assert np.array_equal(idx[t].cpu().numpy(), ref), (f, k, pname, t)
            idx2, cnt2 = csf.select_threshold(_dev(S), 0.5)
            torch.cuda.synchronize()
            for t in range(2):
                v = S[t].numpy()
                ref = np.nonzero(v >= 0.5)[0]           # NaN compares false: never selected
                n = cnt2[t].item()
                assert n == len(ref) and np.array_equal(idx2[t, :n].cpu().numpy(), ref)


FFN_CASES = [
    ("c0-f32", wl.TINY_F32, 102),
    ("f16-ragged", wl.OPT175B.scaled(2600, 3001, 136), 150),
    ("f16-reglu", wl.dataclasses.replace(wl.LLAMA_REGLU.scaled(2600, 3001, 136), dtype=torch.float16), 301),
    ("bf16-reglu", wl.LLAMA_REGLU.scaled(4096, 1433, 256), 400),
    ("f16-wide", wl.OPT175B.scaled(12288, 700, 64), 333),
]


@pytest.mark.parametrize("name,cfg,count", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_sparse_ffn(name, cfg, count):
    announce(f"sparse_ffn {name}")
    L = _layer(cfg)
    Ld = _to_dev_layer(L)
    B = 3
    X = wl.make_tokens(cfg, B)
    g = torch.Generator().manual_seed(count)
    idx = torch.stack([torch.sort(torch.randperm(cfg.f, generator=g)[:count]).values
                       for _ in range(B)]).int()
    h = torch.empty(B, count, dtype=torch.float32, device=DEV)
    y = csf.sparse_ffn(_dev(X), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, _dev(idx), act=cfg.act, h=h)
    torch.cuda.synchronize()
    o = layer_to_orc(L)
    for t in range(B):
        h_ref, y_ref = orc.sparse_ffn(to_orc(X[t]), o["W1"], o["b1"], o["Wup"], o["W2T"],
                                      idx[t].numpy(), o["act"], o["dt"])
        assert_ffn_close(y[t], y_ref, cfg.dtype, f"{name} token {t}")
        hs = np.abs(h_ref).max()
        assert np.abs(h[t].cpu().double().numpy() - h_ref).max() <= 1e-4 * max(hs, 1e-30)
    # each token alone gives the same bits as the batch
    for t in range(B):
        y1 = csf.sparse_ffn(_dev(X[t]), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, _dev(idx[t]), act=cfg.act)
        assert torch.equal(y1, y[t])
    # a second run gives the same bits
    y2 = csf.sparse_ffn(_dev(X), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, _dev(idx), act=cfg.act)
    assert torch.equal(y2, y)


@pytest.mark.parametrize("act", [csf.RELU, csf.REGLU])
def test_sparse_ffn_integer_inputs_bit_exact(act):
    announce(f"sparse_ffn integer act={act}")
    g = torch.Generator().manual_seed(77)
    d, f, count, B = 2048 + 64, 1500, 200, 2
    x = torch.randint(-3, 4, (B, d), generator=g).half()
    W1 = torch.randint(-2, 3, (f, d), generator=g).half()
    Wup = torch.randint(-2, 3, (f, d), generator=g).half() if act == csf.REGLU else None
    W2T = torch.randint(-2, 3, (f, d), generator=g).half()
    b1 = torch.randint(-3, 4, (f,), generator=g).float()
    idx = torch.stack([torch.sort(torch.randperm(f, generator=g)[:count]).values for _ in range(B)]).int()
    y = csf.sparse_ffn(_dev(x), _dev(W1), _dev(b1), None if Wup is None else _dev(Wup), _dev(W2T),
                       _dev(idx), act=act)
    torch.cuda.synchronize()
    for t in range(B):
        _, y_ref = orc.sparse_ffn(to_orc(x[t]), to_orc(W1), to_orc(b1),
                                  None if Wup is None else to_orc(Wup), to_orc(W2T),
                                  idx[t].numpy(), act, orc.F16)
        # every partial sum is an integer below 2^24, so float32 accumulation is exact
        assert np.abs(y_ref).max() < 2 ** 24
        assert np.array_equal(y[t].cpu().double().numpy(), y_ref)


def test_sparse_ffn_device_counts_empty_and_bad_index():
    announce("sparse_ffn device counts / empty / bad index")
    cfg = wl.OPT175B.scaled(1024, 900, 64)
    L = _to_dev_layer(_layer(cfg))
    B, stride = 3, 64
    X = _dev(wl.make_tokens(cfg, B))
    g = torch.Generator().manual_seed(5)
    idx = torch.stack([torch.sort(torch.randperm(cfg.f, generator=g)[:stride]).values for _ in range(B)]).int()
    counts = torch.tensor([0, 17, 64], dtype=torch.int32)
    y = csf.sparse_ffn(X, L.W1, L.b1, None, L.W2T, _dev(idx), count=_dev(counts))
    torch.cuda.synchronize()
    assert not y[0].any()                                  # empty active set -> y = 0
    y17 = csf.sparse_ffn(X[1], L.W1, L.b1, None, L.W2T, _dev(idx[1, :17].contiguous()))
    y64 = csf.sparse_ffn(X[2], L.W1, L.b1, None, L.W2T, _dev(idx[2]))
    torch.cuda.synchronize()
    o = layer_to_orc(L)
    _, r17 = orc.sparse_ffn(to_orc(X[1]), o["W1"], o["b1"], None, o["W2T"], idx[1, :17].numpy(),
                            orc.RELU, orc.F16)
    assert_ffn_close(y[1], r17, cfg.dtype, "count 17")
    assert_ffn_close(y17, r17, cfg.dtype, "list of 17")
    assert torch.equal(y[2], y64)
    # an index outside [0, f) contributes nothing
    bad = idx[2].clone()
    bad[10] = cfg.f + 5
    bad[20] = -1
    yb = csf.sparse_ffn(X[2], L.W1, L.b1, None, L.W2T, _dev(bad))
    keep = np.delete(idx[2].numpy(), [10, 20])
    _, rb = orc.sparse_ffn(to_orc(X[2]), o["W1"], o["b1"], None, o["W2T"], keep, orc.RELU, orc.F16)
    torch.cuda.synchronize()
    assert_ffn_close(yb, rb, cfg.dtype, "bad index skipped")


DENSE_CASES = [
    ("c0-f32", wl.TINY_F32),
    ("f16-ragged", wl.OPT175B.scaled(2600, 3001, 136)),
    ("bf16-reglu", wl.LLAMA_REGLU.scaled(4096, 1433, 256)),
]


@pytest.mark.parametrize("name,cfg", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_ffn_and_full_list(name, cfg):
    announce(f"dense_ffn {name}")
    L = _layer(cfg)
    Ld = _to_dev_layer(L)
    X = wl.make_tokens(cfg, 2)
    y = csf.dense_ffn(_dev(X), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, act=cfg.act)
    full = torch.arange(cfg.f, dtype=torch.int32, device=DEV).repeat(2, 1).contiguous()
    ys = csf.sparse_ffn(_dev(X), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, full, act=cfg.act)
    torch.cuda.synchronize()
    assert torch.equal(y, ys)                              # the full list is the dense layer
    o = layer_to_orc(L)
    for t in range(2):
        _, y_ref = orc.dense_ffn(to_orc(X[t]), o["W1"], o["b1"], o["Wup"], o["W2T"], o["act"], o["dt"])
        assert_ffn_close(y[t], y_ref, cfg.dtype, f"dense {name} token {t}")


def test_relu_true_set_matches_dense():
    """For ReLU, the sparse step over the true active set gives the dense output (up to order)."""
    announce("true set vs dense")
    cfg = wl.OPT175B.scaled(2048, 4000, 128)
    L = _layer(cfg)
    Ld = _to_dev_layer(L)
    x = wl.make_tokens(cfg, 1)[0]
    o = layer_to_orc(L)
    T = orc.true_set(to_orc(x), o["W1"], o["b1"], o["dt"])
    y_sparse = csf.sparse_ffn(_dev(x), Ld.W1, Ld.b1, None, Ld.W2T, _dev(torch.from_numpy(T)))
    y_dense = csf.dense_ffn(_dev(x), Ld.W1, Ld.b1, None, Ld.W2T)
    torch.cuda.synchronize()
    _, y_ref = orc.dense_ffn(to_orc(x), o["W1"], o["b1"], None, o["W2T"], orc.RELU, o["dt"])
    assert_ffn_close(y_sparse, y_ref, cfg.dtype, "true set")
    assert_ffn_close(y_dense, y_ref, cfg.dtype, "dense")


LAYER_CASES = [
    ("c0", wl.TINY_F32, 6),
    ("f16-ragged-topk", wl.OPT175B.scaled(2600, 3001, 136), 3),
    ("bf16-reglu-threshold", wl.LLAMA_REGLU.scaled(4096, 1433, 256), 3),
    # threshold over 40001 scores (about 20000 entries)
    ("bf16-reglu-threshold-many", wl.LLAMA_REGLU.scaled(512, 40001, 64), 2),
    # up to 1024 neurons: scores and selection in one kernel
    ("bf16-reglu-small-threshold", wl.LLAMA_REGLU.scaled(1024, 700, 128), 3),
    ("f16-small-topk-ragged", wl.OPT175B.scaled(1000, 997, 72), 3),
]


def _check_layer_token(L, o, x, k, tau, what):
    f = L.cfg.f
    scores = torch.empty(f, dtype=torch.float32, device=DEV)
    idx = torch.empty(f, dtype=torch.int32, device=DEV)
    count = torch.empty(1, dtype=torch.int32, device=DEV)
    y = csf.sparse_ffn_layer(_dev(x), L.V, L.U, L.W1, L.b1, L.Wup, L.W2T, k=k, tau=tau,
                             act=L.cfg.act, scores=scores, idx=idx, count=count)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()
    _, _, s_ref = orc.predict(to_orc(x), o["V"], o["U"], o["dt"])
    assert np.abs(s_gpu.astype(np.float64) - s_ref).max() <= 1e-5, what
    n = count.item()
    ix = idx[:n].cpu().numpy()
    # selection is bit-exact when the oracle is fed the GPU's scores
    ref_sel = orc.select_topk(s_gpu, k) if k is not None else orc.select_threshold(s_gpu, tau)
    assert np.array_equal(ix, ref_sel), what
    # against the oracle's own scores, every disagreement sits within 1e-5 of the boundary
    own = orc.select_topk(s_ref, k) if k is not None else orc.select_threshold(s_ref, tau)
    theta = np.sort(s_ref)[::-1][k - 1] if (k is not None and k > 0) else tau
    for j in np.setxor1d(own, ix):
        assert abs(float(s_ref[j]) - float(theta)) < 1e-5, (what, j)
    _, y_ref = orc.sparse_ffn(to_orc(x), o["W1"], o["b1"], o["Wup"], o["W2T"], ix, o["act"], o["dt"])
    assert_ffn_close(y, y_ref, L.cfg.dtype, what)
    return ix


@pytest.mark.parametrize("name,cfg,ntok", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_end_to_end(name, cfg, ntok):
    L = _layer(cfg)
    Ld = _to_dev_layer(L)
    o = layer_to_orc(L)
    X = wl.make_tokens(cfg, ntok)
    for t in range(ntok):
        announce(f"layer {name} token {t}")
        _check_layer_token(Ld, o, X[t], cfg.k, cfg.tau if cfg.k is None else None, f"{name}/{t}")


@pytest.mark.parametrize("f", [1024, 3000])
def test_layer_selection_ties_go_to_the_lower_index(f):
    """Predictor up rows in identical pairs give identical scores: the selection (inside the
    predictor kernel for f <= 1024, the selection kernel above) must break the ties at the
    boundary by the lower neuron index, as the oracle does."""
    announce(f"layer ties f={f}")
    cfg = wl.TINY_F32.scaled(256, f, 64, k=f // 10 + 1)
    L = _layer(cfg)
    U = L.U.clone()
    U[1::2] = U[0::2][: U[1::2].shape[0]]
    L = wl.Layer(cfg, L.V, U, L.W1, L.b1, L.Wup, L.W2T)
    Ld = _to_dev_layer(L)
    o = layer_to_orc(L)
    X = wl.make_tokens(cfg, 3)
    for t in range(3):
        ix = _check_layer_token(Ld, o, X[t], cfg.k, None, f"ties f={f} token {t}")
        assert len(ix) == cfg.k


def test_layer_full_size_opt175b_shape():
    """The headline workload at full size (d=12288, f=49152, r=1024, f16, k=2458), one token,
    in the same launch configuration the benchmark times."""
    announce("layer full size c1")
    cfg = wl.OPT175B
    Ld = wl.make_layer(cfg, device=DEV)
    x = wl.make_tokens(cfg, 1, device=DEV)[0]
    o = layer_to_orc(Ld)
    ix = _check_layer_token(Ld, o, x, cfg.k, None, "c1 full")
    assert len(ix) == cfg.k


def test_layer_empty_selection_writes_zero():
    """k = 0, and a threshold above every score: the layer writes y = 0 (an empty list must not
    leave y as it was)."""
    cfg = wl.OPT175B.scaled(2048, 3001, 128)
    Ld = _to_dev_layer(_layer(cfg))
    x = _dev(wl.make_tokens(cfg, 1)[0])
    for k, tau in ((0, None), (None, 1.5)):
        announce(f"layer empty selection k={k} tau={tau}")
        y = torch.full((cfg.d,), 7.0, dtype=torch.float32, device=DEV)
        count = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=k, tau=tau,
                             act=cfg.act, y=y, count=count)
        torch.cuda.synchronize()
        assert int(count.item()) == 0 and not y.any(), (k, tau)


def test_layer_full_size_llama_reglu_threshold():
    """The LLaMA-class ReGLU layer at full size (d 4096, f 14336, r 256, bfloat16) in threshold
    mode (score >= 0.5), two tokens, in the launch configuration the benchmark uses; its
    one-kernel FFN equals the three-kernel form bit for bit."""
    cfg = wl.LLAMA_REGLU
    Ld = wl.make_layer(cfg, device=DEV)
    X = wl.make_tokens(cfg, 2, device=DEV)
    o = layer_to_orc(Ld)
    for t in range(2):
        announce(f"layer full size c2 token {t}")
        ix = _check_layer_token(Ld, o, X[t], None, cfg.tau, f"c2 full token {t}")
        assert 0 < len(ix) < cfg.f
        _fused_vs_separate(Ld, X[t], None, cfg.tau, cfg.act, f"c2 full one-kernel {t}")


FUSED_CASES = [
    ("c0", wl.TINY_F32, 3),
    ("f16-ragged-topk", wl.OPT175B.scaled(2600, 3001, 136), 3),
    ("bf16-reglu-threshold", wl.LLAMA_REGLU.scaled(4096, 1433, 256), 3),
    ("f32-many-slices", wl.TINY_F32.scaled(8192, 5000, 64, k=1200), 2),
]


def _fused_vs_separate(Ld, x, k, tau, act, what):
    """The layer's gathered FFN runs as one kernel that hands h and the partial rows from one
    workgroup to another inside the launch; y must equal, bit for bit, the three-kernel
    csf_sparse_ffn over the same list (same sums in the same order)."""
    f = Ld.cfg.f
    idx = torch.empty(f, dtype=torch.int32, device=DEV)
    count = torch.empty(1, dtype=torch.int32, device=DEV)
    y = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=k, tau=tau, act=act,
                             idx=idx, count=count)
    # the same list length bound (k, or f for a threshold with the count on the device), so the
    # same split of the down projection into chunks
    mc = k if k is not None else f
    lst = idx[:mc].reshape(1, mc)
    ys = csf.sparse_ffn(x.reshape(1, -1), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, lst, act=act,
                        count=None if k is not None else count, max_count=mc)
    torch.cuda.synchronize()
    assert int(count.item()) > 0, what
    assert torch.equal(y, ys.reshape(-1)), what


@pytest.mark.parametrize("name,cfg,ntok", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_layer_one_kernel_ffn_is_bit_identical(name, cfg, ntok):
    Ld = _to_dev_layer(_layer(cfg))
    X = wl.make_tokens(cfg, ntok)
    for t in range(ntok):
        announce(f"one-kernel FFN {name} token {t}")
        _fused_vs_separate(Ld, _dev(X[t]), cfg.k, cfg.tau if cfg.k is None else None, cfg.act,
                           f"{name}/{t}")


@pytest.mark.parametrize("act", [csf.REGLU, csf.SILU, csf.SWIGLU], ids=["reglu", "silu", "swiglu"])
def test_layer_one_kernel_ffn_nan_payload_is_not_the_sentinel(act):
    """A float32 token holding the NaN whose bits are all ones (the one-kernel FFN's mark for an
    unwritten h) carries it into h in the gated and SiLU forms (0 * NaN and NaN arithmetic keep
    the payload).  The up role stores such an h as the default NaN, so every column of y is NaN,
    as in the three-kernel form, instead of a wait running out and h being read as zero."""
    cfg = wl.TINY_F32
    Ld = _to_dev_layer(_layer(cfg))
    gated = act in (csf.REGLU, csf.SWIGLU)
    g = torch.Generator().manual_seed(77)
    Wup = _dev((torch.randn(cfg.f, cfg.d, generator=g) * 0.05).contiguous()) if gated else None
    x = _dev(wl.make_tokens(cfg, 1)[0]).clone()
    x.view(torch.int32)[3] = -1
    announce(f"one-kernel FFN NaN payload act={act}")
    y = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Wup, Ld.W2T, k=cfg.k, act=act)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()


def test_layer_one_kernel_ffn_full_size_repeated():
    """The headline shape, many calls back to back (the counters are cleared by each call's
    first kernel): every y bit-identical to the three-kernel form."""
    cfg = wl.OPT175B
    Ld = wl.make_layer(cfg, device=DEV)
    X = wl.make_tokens(cfg, 4, device=DEV)
    for rep in range(3):
        for t in range(4):
            announce(f"one-kernel FFN c1 rep {rep} token {t}")
            _fused_vs_separate(Ld, X[t], cfg.k, None, cfg.act, f"c1 {rep}/{t}")


# ---- post-gate zero-skip: rows with h = 0 are not read; y is the same up to summation order --------
ZS_CASES = [
    ("relu-f16", wl.OPT175B.scaled(2048, 3001, 128)),
    ("reglu-bf16-threshold", wl.LLAMA_REGLU.scaled(1024, 2500, 128)),
]


@pytest.mark.parametrize("name,cfg", ZS_CASES, ids=[c[0] for c in ZS_CASES])
def test_zero_skip_layer_and_ffn(name, cfg):
    announce(f"zero-skip {name}")
    L = _layer(cfg)
    Ld = _to_dev_layer(L)
    o = layer_to_orc(L)
    X = wl.make_tokens(cfg, 3)
    try:
        for t in range(3):
            x = _dev(X[t])
            k = cfg.k
            idx = torch.empty(k if k is not None else cfg.f, dtype=torch.int32, device=DEV)
            cnt = torch.empty(1, dtype=torch.int32, device=DEV)
            csf.set_ffn_flags(0)
            y0 = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=k, tau=cfg.tau,
                                      act=cfg.act, idx=idx, count=cnt)
            csf.set_ffn_flags(csf.FFN_SKIP_ZERO_H)
            y1 = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=k, tau=cfg.tau,
                                      act=cfg.act)
            y1b = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=k, tau=cfg.tau,
                                       act=cfg.act)
            torch.cuda.synchronize()
            n = int(cnt.item())
            sel = idx[:n].cpu().numpy()
            h_ref, y_ref = orc.sparse_ffn(to_orc(X[t]), o["W1"], o["b1"], o["Wup"], o["W2T"], sel,
                                          o["act"], o["dt"])
            assert (h_ref == 0).sum() > n // 4              # the skip has work to do
            assert_ffn_close(y0, y_ref, cfg.dtype, f"{name} plain token {t}")
            assert_ffn_close(y1, y_ref, cfg.dtype, f"{name} zero-skip token {t}")
            assert torch.equal(y1, y1b)                     # deterministic
        # the dense layer with the skip is the dense layer
        hd = torch.empty(1, cfg.f, dtype=torch.float32, device=DEV)
        yd = csf.dense_ffn(_dev(X[0]), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, act=cfg.act, h=hd)
        torch.cuda.synchronize()
        _, yd_ref = orc.dense_ffn(to_orc(X[0]), o["W1"], o["b1"], o["Wup"], o["W2T"], o["act"], o["dt"])
        assert_ffn_close(yd, yd_ref, cfg.dtype, f"{name} dense zero-skip")
    finally:
        csf.set_ffn_flags(0)


@pytest.mark.parametrize("act", [csf.RELU, csf.REGLU])
def test_zero_skip_integer_inputs_bit_exact(act):
    """Dropping exact zeros keeps integer arithmetic exact: bit-equal to the oracle."""
    announce(f"zero-skip integer act={act}")
    g = torch.Generator().manual_seed(123 + act)
    d, f, count, B = 1024, 1300, 400, 2
    x = torch.randint(-3, 4, (B, d), generator=g).half()
    W1 = torch.randint(-2, 3, (f, d), generator=g).half()
    Wup = torch.randint(-2, 3, (f, d), generator=g).half() if act == csf.REGLU else None
    W2T = torch.randint(-2, 3, (f, d), generator=g).half()
    b1 = torch.randint(-3, 4, (f,), generator=g).float()
    idx = torch.stack([torch.sort(torch.randperm(f, generator=g)[:count]).values for _ in range(B)]).int()
    try:
        csf.set_ffn_flags(csf.FFN_SKIP_ZERO_H)
        y = csf.sparse_ffn(_dev(x), _dev(W1), _dev(b1), None if Wup is None else _dev(Wup),
                           _dev(W2T), _dev(idx), act=act)
        torch.cuda.synchronize()
    finally:
        csf.set_ffn_flags(0)
    for t in range(B):
        h_ref, y_ref = orc.sparse_ffn(to_orc(x[t]), to_orc(W1), to_orc(b1),
                                      None if Wup is None else to_orc(Wup), to_orc(W2T),
                                      idx[t].numpy(), act, orc.F16)
        assert (h_ref == 0).sum() > count // 4
        assert np.array_equal(y[t].cpu().double().numpy(), y_ref)

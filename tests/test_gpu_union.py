"""GPU parity of the batched union FFN (csf_sparse_ffn_batched_union) against the oracle.

The oracle's batched form: token t over its own set (per-token semantics) or over the union of the
batch's sets (union semantics), each a plain double-precision sparse FFN.  Both kernel families
(vector-ALU gather, matrix-core MFMA) are compared at the FFN bars of csf_testutil; integer-valued
inputs must match bit for bit on both.  The sets come from each token's bitmap, so every case also
checks the union size the library reports.
"""
import dataclasses

import numpy as np
import pytest
import torch

import contextual_sparsity_ffn_amd as csf
from contextual_sparsity_ffn_amd import workloads as wl
from csf_testutil import announce, assert_ffn_close, layer_to_orc, to_orc
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _dev_layer(L):
    d = lambda t: None if t is None else t.to(DEV)
    return wl.Layer(L.cfg, d(L.V), d(L.U), d(L.W1), d(L.b1), d(L.Wup), d(L.W2T))


def _bitmaps(sets, f):
    words = np.stack([orc.to_bitmap(s, f) for s in sets])
    return torch.from_numpy(words.view(np.int32)).to(DEV)


def _random_sets(f, B, count, seed, shared=0.5):
    """B ascending sets of `count` neurons: a `shared` fraction drawn from one common pool, so the
    sets overlap the way clustered tokens do; the rest drawn per token."""
    g = torch.Generator().manual_seed(seed)
    pool = torch.randperm(f, generator=g)[: 2 * count]
    sets = []
    for _ in range(B):
        n_sh = int(count * shared)
        a = pool[torch.randperm(pool.numel(), generator=g)[:n_sh]]
        rest = torch.randperm(f, generator=g)
        rest = rest[~torch.isin(rest, a)][: count - n_sh]
        sets.append(np.sort(torch.cat([a, rest]).numpy()).astype(np.int32))
    return sets


def _run(Ld, X, bm, semantics, path, uc=None):
    Y, taken = csf.sparse_ffn_batched_union(X, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, bm, act=Ld.cfg.act,
                                            semantics=semantics, path=path, union_count=uc)
    torch.cuda.synchronize()
    return Y, taken


def _check(L, X, sets, Y, semantics, what):
    o = layer_to_orc(L)
    Yref = orc.batched_ffn(to_orc(X), sets, o["W1"], o["b1"], o["Wup"], o["W2T"], o["act"],
                           o["dt"], union=semantics == csf.SEM_UNION)
    for t in range(X.shape[0]):
        assert_ffn_close(Y[t], Yref[t], L.cfg.dtype, f"{what} token {t}")


# (name, config, B, active fraction): shapes span several tiles, f ends in a ragged word
CASES = [
    ("f16-B1", wl.OPT30B.scaled(512, 1000, 64), 1, 0.2),
    ("f16-B2", wl.OPT30B.scaled(512, 1000, 64), 2, 0.2),
    ("f16-B5", wl.OPT30B.scaled(512, 1000, 64), 5, 0.2),
    ("f16-B16", wl.OPT30B.scaled(768, 2333, 64), 16, 0.2),
    ("f16-B17", wl.OPT30B.scaled(768, 2333, 64), 17, 0.1),
    ("f16-B32", wl.OPT30B.scaled(1024, 1601, 64), 32, 0.2),
    ("bf16-reglu-B3", wl.LLAMA_REGLU.scaled(512, 1433, 64), 3, 0.3),
    ("bf16-reglu-B20", wl.LLAMA_REGLU.scaled(512, 1433, 64), 20, 0.3),
    ("bf16-swiglu-B2", wl.LLAMA_SWIGLU.scaled(512, 1433, 64), 2, 0.5),
    ("bf16-swiglu-B3", wl.LLAMA_SWIGLU.scaled(512, 1433, 64), 3, 0.5),
    ("bf16-swiglu-B20", wl.LLAMA_SWIGLU.scaled(512, 1433, 64), 20, 0.5),
    ("f16-silu-B8", dataclasses.replace(wl.OPT30B.scaled(512, 1000, 64), act=csf.SILU), 8, 0.3),
]
PATHS = [("gather", csf.PATH_GATHER), ("mfma", csf.PATH_MFMA)]


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
@pytest.mark.parametrize("name,cfg,B,frac", CASES, ids=[c[0] for c in CASES])
def test_batched_union_per_token(name, cfg, B, frac, pname, path):
    announce(f"batched union {name} {pname}")
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    X = wl.make_clustered_tokens(cfg, B)
    sets = _random_sets(cfg.f, B, max(1, int(cfg.f * frac)), seed=B * 1000 + cfg.d)
    uc = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    Y, taken = _run(Ld, X.to(DEV), _bitmaps(sets, cfg.f), csf.SEM_PER_TOKEN, path, uc)
    assert taken == path
    assert int(uc.item()) == len(orc.union_of(sets, cfg.f))
    _check(L, X, sets, Y, csf.SEM_PER_TOKEN, f"{name}/{pname}")
    # the same call again gives the same bits
    Y2, _ = _run(Ld, X.to(DEV), _bitmaps(sets, cfg.f), csf.SEM_PER_TOKEN, path)
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_batched_union_semantics_union(pname, path):
    announce(f"batched union semantics=union {pname}")
    cfg = wl.OPT30B.scaled(512, 1200, 64)
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    B = 6
    X = wl.make_clustered_tokens(cfg, B)
    sets = _random_sets(cfg.f, B, 150, seed=11)
    Y, _ = _run(Ld, X.to(DEV), _bitmaps(sets, cfg.f), csf.SEM_UNION, path)
    _check(L, X, sets, Y, csf.SEM_UNION, f"union/{pname}")
    # every neuron in every set: the union is the dense layer
    full = [np.arange(cfg.f, dtype=np.int32)] * B
    Yd, _ = _run(Ld, X.to(DEV), _bitmaps(full, cfg.f), csf.SEM_UNION, path)
    o = layer_to_orc(L)
    for t in range(B):
        ref = orc.dense_ffn(to_orc(X[t]), o["W1"], o["b1"], None, o["W2T"], o["act"], o["dt"])[1]
        assert_ffn_close(Yd[t], ref, cfg.dtype, f"dense/{pname} token {t}")


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
@pytest.mark.parametrize("act", [csf.RELU, csf.REGLU])
def test_batched_union_integer_inputs_bit_exact(act, pname, path):
    """Small integers: every h is an integer below 2^16, so hi + lo holds it exactly (hi rounds to
    a multiple of the binary16 spacing, the integer remainder lo is exact), every product is exact
    and every partial sum stays below 2^24: both kernel families must reproduce the oracle bit for
    bit."""
    announce(f"batched union integer act={act} {pname}")
    g = torch.Generator().manual_seed(91 + act)
    d, f, B = 768, 1111, 19
    x = torch.randint(-1, 2, (B, d), generator=g).half()
    W1 = torch.randint(-1, 2, (f, d), generator=g).half()
    Wup = torch.randint(-1, 2, (f, d), generator=g).half() if act == csf.REGLU else None
    W2T = torch.randint(-2, 3, (f, d), generator=g).half()
    b1 = torch.randint(-3, 4, (f,), generator=g).float()
    sets = _random_sets(f, B, 300, seed=3)
    cfg = dataclasses.replace(wl.OPT30B.scaled(d, f, 64), act=act)
    Ld = wl.Layer(cfg, None, None, W1.to(DEV), b1.to(DEV), None if Wup is None else Wup.to(DEV),
                  W2T.to(DEV))
    Y, _ = _run(Ld, x.to(DEV), _bitmaps(sets, f), csf.SEM_PER_TOKEN, path)
    Yref = orc.batched_ffn(to_orc(x), sets, to_orc(W1), to_orc(b1),
                           None if Wup is None else to_orc(Wup), to_orc(W2T), act, orc.F16)
    h_max = 0.0
    for t in range(B):
        h, _ = orc.sparse_ffn(to_orc(x[t]), to_orc(W1), to_orc(b1),
                              None if Wup is None else to_orc(Wup), to_orc(W2T), sets[t], act,
                              orc.F16)
        h_max = max(h_max, float(np.abs(h).max()))
    assert h_max < 65504 and np.abs(Yref).max() < 2 ** 24
    assert np.array_equal(Y.cpu().double().numpy(), Yref)


def test_batched_union_float32_and_auto_path():
    announce("batched union float32 / auto path")
    cfg = wl.TINY_F32                                    # d = 256, f = 1024, float32
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    B = 7
    X = wl.make_clustered_tokens(cfg, B)
    sets = _random_sets(cfg.f, B, cfg.k, seed=4)
    Y, taken = _run(Ld, X.to(DEV), _bitmaps(sets, cfg.f), csf.SEM_PER_TOKEN, csf.PATH_AUTO)
    assert taken == csf.PATH_GATHER                        # matrix cores take 16-bit types only
    _check(L, X, sets, Y, csf.SEM_PER_TOKEN, "f32")
    with pytest.raises(csf.CsfError):
        _run(Ld, X.to(DEV), _bitmaps(sets, cfg.f), csf.SEM_PER_TOKEN, csf.PATH_MFMA)
    # 16-bit: one token gathers, a batch of 8 takes the matrix cores
    c16 = wl.OPT30B.scaled(512, 1000, 64)
    L16 = _dev_layer(wl.make_layer(c16))
    X16 = wl.make_tokens(c16, 8).to(DEV)
    s16 = _random_sets(c16.f, 8, 100, seed=5)
    _, t1 = _run(L16, X16[:1].contiguous(), _bitmaps(s16[:1], c16.f), csf.SEM_PER_TOKEN, csf.PATH_AUTO)
    _, t8 = _run(L16, X16, _bitmaps(s16, c16.f), csf.SEM_PER_TOKEN, csf.PATH_AUTO)
    assert (t1, t8) == (csf.PATH_GATHER, csf.PATH_MFMA)


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_batched_union_empty_and_one_token_sets(pname, path):
    announce(f"batched union empty sets {pname}")
    cfg = wl.OPT30B.scaled(512, 999, 64)
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    B = 4
    X = wl.make_tokens(cfg, B)
    empty = [np.zeros(0, np.int32)] * B
    uc = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    Y, _ = _run(Ld, X.to(DEV), _bitmaps(empty, cfg.f), csf.SEM_PER_TOKEN, path, uc)
    assert int(uc.item()) == 0 and not Y.any()
    # only token 2 has neurons (including the last one, f - 1); the others must stay exactly 0
    sets = [np.zeros(0, np.int32), np.zeros(0, np.int32),
            np.array([0, 5, 31, 32, 500, cfg.f - 1], np.int32), np.zeros(0, np.int32)]
    Y, _ = _run(Ld, X.to(DEV), _bitmaps(sets, cfg.f), csf.SEM_PER_TOKEN, path, uc)
    assert int(uc.item()) == 6
    assert not Y[0].any() and not Y[1].any() and not Y[3].any()
    _check(L, X, sets, Y, csf.SEM_PER_TOKEN, f"one-token/{pname}")


@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_batched_union_matches_single_token_path(pname, path):
    """Per-token semantics: each token's row equals the single-token sparse FFN of its own list
    (to float32 rounding; the two sum in different orders)."""
    announce(f"batched union vs single-token {pname}")
    cfg = wl.OPT30B.scaled(1024, 3000, 64)
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    B = 9
    X = wl.make_clustered_tokens(cfg, B).to(DEV)
    sets = _random_sets(cfg.f, B, 600, seed=8)
    Y, _ = _run(Ld, X, _bitmaps(sets, cfg.f), csf.SEM_PER_TOKEN, path)
    for t in range(B):
        y1 = csf.sparse_ffn(X[t], Ld.W1, Ld.b1, None, Ld.W2T, torch.from_numpy(sets[t]).to(DEV))
        torch.cuda.synchronize()
        err = float((Y[t] - y1).abs().max() / y1.abs().max())
        assert err <= 1e-5, (t, err)


@pytest.mark.parametrize("B,path", [(4, csf.PATH_GATHER), (2, csf.PATH_MFMA), (8, csf.PATH_MFMA),
                                   (32, csf.PATH_MFMA)],
                         ids=["B4-gather", "B2-mfma", "B8-mfma", "B32-mfma"])
def test_batched_union_full_size_opt30b_shape(B, path):
    """The OPT-30B FFN shape (d 7168, f 28672, top-k 5734 per token) with sets chosen by the
    library's own predictor and top-k on clustered tokens, as the benchmark runs it."""
    announce(f"batched union full size B={B}")
    cfg = wl.OPT30B
    Ld = wl.make_layer(cfg, device=DEV)
    X = wl.make_clustered_tokens(cfg, B, device=DEV)
    scores = csf.predict_active(X, Ld.V, Ld.U)
    words = (cfg.f + 31) // 32
    bm = torch.zeros(B, words, dtype=torch.int32, device=DEV)
    idx = csf.select_topk(scores, cfg.k, bitmap=bm)
    uc = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y, taken = _run(Ld, X, bm, csf.SEM_PER_TOKEN, path, uc)
    assert taken == path
    sets = [idx[t].cpu().numpy() for t in range(B)]
    assert int(uc.item()) == len(orc.union_of(sets, cfg.f))
    o = dict(W1=to_orc(Ld.W1), b1=to_orc(Ld.b1), W2T=to_orc(Ld.W2T))
    for t in (0, B // 2, B - 1):                          # three tokens through the oracle
        _, ref = orc.sparse_ffn(to_orc(X[t]), o["W1"], o["b1"], None, o["W2T"], sets[t],
                                orc.RELU, orc.F16)
        assert_ffn_close(Y[t], ref, cfg.dtype, f"full B={B} token {t}")


@pytest.mark.parametrize("name,cfg,B", [
    ("f16-topk-B6", wl.OPT30B.scaled(768, 2333, 64), 6),
    ("bf16-reglu-threshold-B5", wl.LLAMA_REGLU.scaled(512, 1433, 64), 5),
    ("f16-topk-wide-B3", wl.OPT30B.scaled(256, 24576, 64), 3),   # many-workgroup top-k
    # a batch of one: the gather path runs the single-token layer (with the bitmap written)
    ("f16-topk-wide-B1", wl.OPT30B.scaled(256, 24576, 64), 1),
    ("bf16-reglu-threshold-B1", wl.LLAMA_REGLU.scaled(512, 1433, 64), 1),
    ("f16-topk-small-B1", wl.OPT30B.scaled(256, 1000, 64), 1),
], ids=["f16-topk-B6", "bf16-reglu-threshold-B5", "f16-topk-wide-B3", "f16-topk-wide-B1",
        "bf16-reglu-threshold-B1", "f16-topk-small-B1"])
def test_batched_layer_end_to_end(name, cfg, B):
    """Predict + select + union FFN in one call: the selected sets (bitmaps) equal the oracle's
    selection from the library's own scores, and Y matches the oracle over those sets."""
    announce(f"batched layer {name}")
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    X = wl.make_clustered_tokens(cfg, B)
    words = (cfg.f + 31) // 32
    bm = torch.zeros(B, words, dtype=torch.int32, device=DEV)
    for path in (csf.PATH_GATHER, csf.PATH_MFMA):
        uc = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        Y, taken = csf.sparse_ffn_batched_layer(X.to(DEV), Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T,
                                                k=cfg.k, tau=cfg.tau, act=cfg.act, path=path,
                                                bitmaps=bm, union_count=uc)
        scores = csf.predict_active(X.to(DEV), Ld.V, Ld.U)
        torch.cuda.synchronize()
        assert taken == path
        sets = []
        for t in range(B):
            s = scores[t].cpu().numpy()
            sel = orc.select_topk(s, cfg.k) if cfg.k is not None else orc.select_threshold(s, cfg.tau)
            assert np.array_equal(bm[t].cpu().numpy().view(np.uint32), orc.to_bitmap(sel, cfg.f))
            sets.append(sel)
        assert int(uc.item()) == len(orc.union_of(sets, cfg.f))
        _check(L, X, sets, Y, csf.SEM_PER_TOKEN, f"{name} path {path}")


@pytest.mark.parametrize("B", [2, 5, 32])
@pytest.mark.parametrize("pname,path", PATHS, ids=[p[0] for p in PATHS])
def test_batched_layer_equals_the_composed_calls(B, pname, path):
    """The batched layer in one enqueue against predict, select and the batched union FFN called
    one after another: the same bits, the same bitmaps and the same union size, for top-k, a
    threshold and an empty selection."""
    cfg = wl.OPT30B.scaled(1024, 3001, 128)
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    X = wl.make_clustered_tokens(cfg, B).to(DEV)
    words = (cfg.f + 31) // 32
    for k, tau in ((cfg.k, None), (None, 0.5), (0, None)):
        announce(f"batched layer vs composed B={B} {pname} k={k} tau={tau}")
        bm = torch.zeros(B, words, dtype=torch.int32, device=DEV)
        uc = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        Y, _ = csf.sparse_ffn_batched_layer(X, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=k,
                                            tau=tau, act=cfg.act, path=path, bitmaps=bm,
                                            union_count=uc)
        s = csf.predict_active(X, Ld.V, Ld.U)
        bm2 = torch.zeros(B, words, dtype=torch.int32, device=DEV)
        if k is not None:
            csf.select_topk(s, k, bitmap=bm2)
        else:
            csf.select_threshold(s, tau, bitmap=bm2)
        uc2 = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        Y2, _ = _run(Ld, X, bm2, csf.SEM_PER_TOKEN, path, uc2)
        torch.cuda.synchronize()
        assert torch.equal(bm, bm2)
        assert int(uc.item()) == int(uc2.item())
        assert torch.equal(Y, Y2)
        if k == 0:
            assert int(uc.item()) == 0 and not Y.any()


@pytest.mark.parametrize("name,cfg", [
    ("f16-topk-wide", wl.OPT30B.scaled(256, 24576, 64)),
    ("bf16-reglu-threshold", wl.LLAMA_REGLU.scaled(512, 1433, 64)),
], ids=["f16-topk-wide", "bf16-reglu-threshold"])
def test_batched_layer_batch_of_one_is_the_single_token_layer(name, cfg):
    """B = 1 on the gather path: the same bits as csf_sparse_ffn_layer for that token, the union
    size is the token's count, and the bitmap is its list."""
    announce(f"batched layer B=1 vs single-token layer {name}")
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    X = wl.make_tokens(cfg, 2)
    for t in range(2):
        x = X[t:t + 1].to(DEV).contiguous()
        words = (cfg.f + 31) // 32
        bm = torch.zeros(1, words, dtype=torch.int32, device=DEV)
        uc = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        Y, taken = csf.sparse_ffn_batched_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T,
                                                k=cfg.k, tau=cfg.tau, act=cfg.act,
                                                path=csf.PATH_AUTO, bitmaps=bm, union_count=uc)
        cnt = torch.empty(1, dtype=torch.int32, device=DEV)
        idx = torch.empty(cfg.k if cfg.k is not None else cfg.f, dtype=torch.int32, device=DEV)
        y1 = csf.sparse_ffn_layer(x[0], Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=cfg.k,
                                  tau=cfg.tau, act=cfg.act, idx=idx, count=cnt)
        torch.cuda.synchronize()
        assert taken == csf.PATH_GATHER
        assert torch.equal(Y[0], y1), (name, t)
        n = int(cnt.item())
        assert int(uc.item()) == n
        sel = idx[:n].cpu().numpy()
        assert np.array_equal(bm[0].cpu().numpy().view(np.uint32), orc.to_bitmap(sel, cfg.f))


@pytest.mark.parametrize("act", [csf.RELU, csf.SILU])
def test_batched_union_large_h_keeps_its_range(act):
    """binary16 holds magnitudes up to 65504, so the matrix-core path's 16-bit hi/lo split of h
    must not see h itself once a token's |h| reaches 2^15: that token's h is split after a
    power-of-two scale, and its outputs are scaled back.  W1 and b1 are scaled by 2^10 (every
    |h| in the thousands) and two tokens' inputs by a further 2^5, which takes their largest |h|
    past 2^16 (checked on the oracle's h); the others stay under 2^15.  Every output must be
    finite and meet the usual bars."""
    announce(f"batched union large h act={act}")
    cfg = dataclasses.replace(wl.OPT30B.scaled(512, 1000, 64), act=act)
    L0 = wl.make_layer(cfg)
    L = wl.Layer(cfg, L0.V, L0.U, (L0.W1.float() * 2.0 ** 10).to(cfg.dtype), L0.b1 * 2.0 ** 10,
                 L0.Wup, L0.W2T)
    Ld = _dev_layer(L)
    B = 6
    X = wl.make_clustered_tokens(cfg, B)
    sets = _random_sets(cfg.f, B, 300, seed=77)
    o = layer_to_orc(L)

    def h_max(x, t):
        h, _ = orc.sparse_ffn(to_orc(x), o["W1"], o["b1"], o["Wup"], o["W2T"], sets[t],
                              o["act"], o["dt"])
        return float(np.abs(h).max())

    for t in (1, 4):
        X[t] = (X[t].float() * 2.0 ** 5).to(cfg.dtype)
        assert h_max(X[t], t) >= 2.0 ** 16, "the scaled token must need the wide range"
    for t in (0, 2, 3, 5):
        assert h_max(X[t], t) < 2.0 ** 15
    Y, taken = _run(Ld, X.to(DEV), _bitmaps(sets, cfg.f), csf.SEM_PER_TOKEN, csf.PATH_MFMA)
    assert taken == csf.PATH_MFMA
    assert torch.isfinite(Y).all()
    _check(L, X, sets, Y, csf.SEM_PER_TOKEN, f"large-h act={act}")
    # the unscaled tokens' rows do not depend on the scaled ones: the same bits without them
    keep = [0, 2, 3, 5]
    Y2, _ = _run(Ld, X[keep].to(DEV), _bitmaps([sets[t] for t in keep], cfg.f),
                 csf.SEM_PER_TOKEN, csf.PATH_MFMA)
    err = float((Y[keep] - Y2).abs().max() / Y2.abs().max())
    assert err <= 1e-5, err

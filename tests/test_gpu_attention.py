"""GPU parity of attention-head sparsity (csf_sparse_attention_decode / _layer) against the oracle.

Bar: y and o within a normwise relative error of 1e-4 for every storage type.  Both sides read
the same weight and cache bytes; the difference is float32 against double arithmetic in the
projections and the logits.  Softmax turns a relative error e of the logits a into an absolute
error |a| e of the exponents, i.e. a relative error |a| e of the attention weights: with
|a| up to ~60 here (the sink logits) and e ~ 1e-6 (float32 dot products of a few thousand terms),
that is ~6e-5, so the FFN's 1e-5 float32 bar does not carry over and 1e-4 is the derived bound.
The appended cache entries are float32 results rounded once to the storage type on the GPU and
double results rounded once in the oracle: within one unit in the last place, plus the float32
accumulation error where the dot product cancels to a small value.  Every other cache element and
every length must be unchanged bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import contextual_sparsity_ffn_amd as csf
from contextual_sparsity_ffn_amd import workloads as wl
from csf_testutil import ORC_DT, announce, to_orc
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = 1e-4


def _dev(L):
    d = lambda t: None if t is None else t.to(DEV)
    return wl.AttnLayer(L.cfg, d(L.Vp), d(L.Up), d(L.Wq), d(L.Wk), d(L.Wv), d(L.WoT), d(L.bq),
                        d(L.Kc).clone(), d(L.Vc).clone(), d(L.lens).clone())


def _orc_state(L):
    return dict(x=None, Wq=to_orc(L.Wq), Wk=to_orc(L.Wk), Wv=to_orc(L.Wv), WoT=to_orc(L.WoT),
                bq=L.bq.cpu().numpy(), Kc=to_orc(L.Kc).copy(), Vc=to_orc(L.Vc).copy(),
                lens=L.lens.cpu().numpy().astype(np.int32).copy(), dt=ORC_DT[L.cfg.dtype])


def _err(g, ref):
    g = g.detach().double().cpu().numpy().reshape(ref.shape)
    s = np.abs(ref).max()
    return float(np.abs(g - ref).max() / s) if s > 0 else float(np.abs(g).max())


def _check_caches(Ld, o, before_K, before_V, dtype, what):
    """GPU caches against the oracle's: appended entries within one unit in the last place."""
    for name, gpu, ref, before in (("K", Ld.Kc, o["Kc"], before_K), ("V", Ld.Vc, o["Vc"], before_V)):
        g = to_orc(gpu)
        changed = np.any(ref != before, axis=-1) | np.any(g != before, axis=-1)
        same = ~changed
        assert np.array_equal(g[same], ref[same]), f"{what}: {name} cache changed outside the new rows"
        wide = lambda a: (a.astype(np.float64) if dtype != torch.bfloat16
                          else (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        gv, rv = wide(g[changed]), wide(ref[changed])
        # one unit in the last place of the storage type, plus the float32 accumulation error of
        # a d-term dot product (which dominates where the sum cancels to a small value)
        ulp = {torch.float32: 2.0 ** -23, torch.float16: 2.0 ** -10, torch.bfloat16: 2.0 ** -7}[dtype]
        scale = np.maximum(np.abs(rv).max(axis=-1, keepdims=True), 1.0)
        assert np.all(np.abs(gv - rv) <= ulp * np.abs(rv) + 2e-5 * scale), \
            f"{what}: {name} cache entries beyond one ulp"
    assert np.array_equal(Ld.lens.cpu().numpy(), o["lens"]), f"{what}: lengths"


CASES = [
    ("f32-tiny", wl.ATTN_TINY_F32, [0, 2, 5], [64, 3, 0, 71, 10, 64, 1, 2], False),
    ("f16-ragged", wl.ATTN_OPT175B.scaled(1000, 12, 64, 64, 300, extra=20),
     [0, 3, 4, 7, 11], [300, 0, 5, 318, 131, 128, 300, 2, 257, 1, 64, 129], False),
    ("f16-ragged-kvall", wl.ATTN_OPT175B.scaled(1000, 12, 64, 64, 300, extra=20),
     [1, 3, 10], [300, 0, 5, 318, 131, 128, 300, 2, 257, 1, 64, 129], True),
    ("bf16-dh128", dataclasses.replace(wl.ATTN_OPT175B.scaled(512, 6, 128, 64, 129, extra=8),
                                       dtype=torch.bfloat16), [0, 1, 2, 3, 4, 5],
     [129, 130, 0, 1, 127, 128], False),
    ("f32-dh64", dataclasses.replace(wl.ATTN_TINY_F32.scaled(512, 5, 64, 32, 200, extra=4),
                                     dtype=torch.float32), [4, 1],
     [200, 100, 0, 50, 202], False),
]


@pytest.mark.parametrize("name,cfg,heads,lens,kv_all", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(name, cfg, heads, lens, kv_all):
    announce(f"attention decode {name}")
    L = wl.make_attention_layer(cfg)
    L.lens = torch.tensor(lens, dtype=torch.int32)
    Ld = _dev(L)
    o = _orc_state(L)
    K0, V0 = o["Kc"].copy(), o["Vc"].copy()
    X = wl.make_attn_tokens(cfg, 2)
    for t in range(2):
        x = X[t]
        hl = torch.tensor(heads, dtype=torch.int32, device=DEV)
        og = torch.empty(len(heads), cfg.dh, dtype=torch.float32, device=DEV)
        y = csf.sparse_attention_decode(x.to(DEV), Ld.Wq, Ld.Wk, Ld.Wv, Ld.bq, None, None, Ld.WoT,
                                        Ld.Kc, Ld.Vc, Ld.lens, heads=hl, kv_all=kv_all, o=og)
        torch.cuda.synchronize()
        o_ref, y_ref = orc.attention_decode(to_orc(x), o["Wq"], o["Wk"], o["Wv"], o["bq"], None,
                                            None, o["WoT"], o["Kc"], o["Vc"], o["lens"],
                                            np.array(heads, np.int32), o["dt"], kv_all)
        assert _err(y, y_ref) <= TOL, (name, t, _err(y, y_ref))
        assert _err(og, o_ref) <= TOL, (name, t, _err(og, o_ref))
        _check_caches(Ld, o, K0, V0, cfg.dtype, f"{name} token {t}")
        K0, V0 = to_orc(Ld.Kc), to_orc(Ld.Vc)
        # keep the two sides on identical caches for the next token
        o["Kc"], o["Vc"] = K0.copy(), V0.copy()


def test_dense_step_and_determinism():
    cfg = wl.ATTN_OPT175B.scaled(1024, 8, 128, 64, 260, extra=4)
    announce("attention dense")
    L = wl.make_attention_layer(cfg)
    x = wl.make_attn_tokens(cfg, 1)[0]
    ys = []
    for rep in range(2):
        Ld = _dev(L)
        ys.append(csf.sparse_attention_decode(x.to(DEV), Ld.Wq, Ld.Wk, Ld.Wv, Ld.bq, None, None,
                                              Ld.WoT, Ld.Kc, Ld.Vc, Ld.lens))
        # the dense step is the list of every head
        Ld2 = _dev(L)
        ya = csf.sparse_attention_decode(x.to(DEV), Ld2.Wq, Ld2.Wk, Ld2.Wv, Ld2.bq, None, None,
                                         Ld2.WoT, Ld2.Kc, Ld2.Vc, Ld2.lens,
                                         heads=torch.arange(cfg.H, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(ya, ys[-1])
    assert torch.equal(ys[0], ys[1])
    o = _orc_state(L)
    _, y_ref = orc.attention_decode(to_orc(x), o["Wq"], o["Wk"], o["Wv"], o["bq"], None, None,
                                    o["WoT"], o["Kc"], o["Vc"], o["lens"],
                                    np.arange(cfg.H, dtype=np.int32), o["dt"])
    assert _err(ys[0], y_ref) <= TOL


def test_empty_list_bad_entries_and_full_cache():
    cfg = wl.ATTN_OPT175B.scaled(512, 6, 64, 32, 40, extra=2)
    announce("attention edge cases")
    L = wl.make_attention_layer(cfg)
    L.lens = torch.tensor([40, 42, 41, 0, 40, 40], dtype=torch.int32)    # head 1's cache is full
    x = wl.make_attn_tokens(cfg, 1)[0]
    # count = 0: nothing computed, nothing stored
    Ld = _dev(L)
    hl = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = csf.sparse_attention_decode(x.to(DEV), Ld.Wq, Ld.Wk, Ld.Wv, Ld.bq, None, None, Ld.WoT,
                                    Ld.Kc, Ld.Vc, Ld.lens, heads=hl, count=zero)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0
    assert torch.equal(Ld.Kc.cpu(), L.Kc) and torch.equal(Ld.lens.cpu(), L.lens)
    # entries outside [0, H) and a head whose cache is full are skipped
    Ld = _dev(L)
    hl = torch.tensor([-1, 1, 2, 3, 6, 5], dtype=torch.int32, device=DEV)
    og = torch.empty(6, cfg.dh, dtype=torch.float32, device=DEV)
    y = csf.sparse_attention_decode(x.to(DEV), Ld.Wq, Ld.Wk, Ld.Wv, Ld.bq, None, None, Ld.WoT,
                                    Ld.Kc, Ld.Vc, Ld.lens, heads=hl, o=og)
    torch.cuda.synchronize()
    o = _orc_state(L)
    o_ref, y_ref = orc.attention_decode(to_orc(x), o["Wq"], o["Wk"], o["Wv"], o["bq"], None, None,
                                        o["WoT"], o["Kc"], o["Vc"], o["lens"],
                                        np.array([2, 3, 5], np.int32), o["dt"])
    assert _err(y, y_ref) <= TOL
    ogc = og.cpu().numpy()
    assert np.all(ogc[[0, 1, 4]] == 0.0)
    assert _err(og[[2, 3, 5]], o_ref) <= TOL
    assert Ld.lens.cpu().tolist() == [40, 42, 42, 1, 40, 41]


LAYER_CASES = [
    ("f16-topk", wl.ATTN_OPT175B.scaled(1024, 16, 64, 64, 300, extra=4), None),
    ("f32-threshold", wl.ATTN_TINY_F32, 0.5),
]


@pytest.mark.parametrize("name,cfg,tau", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_end_to_end(name, cfg, tau):
    L = wl.make_attention_layer(cfg)
    Ld = _dev(L)
    o = _orc_state(L)
    X = wl.make_attn_tokens(cfg, 3)
    k = None if tau is not None else cfg.k
    for t in range(3):
        announce(f"attention layer {name} token {t}")
        scores = torch.empty(cfg.H, dtype=torch.float32, device=DEV)
        heads = torch.empty(cfg.H, dtype=torch.int32, device=DEV)
        count = torch.empty(1, dtype=torch.int32, device=DEV)
        y = csf.sparse_attention_layer(X[t].to(DEV), Ld.Vp, Ld.Up, Ld.Wq, Ld.Wk, Ld.Wv, Ld.bq,
                                       None, None, Ld.WoT, Ld.Kc, Ld.Vc, Ld.lens, k=k, tau=tau,
                                       scores=scores, heads=heads, count=count)
        torch.cuda.synchronize()
        s_gpu = scores.cpu().numpy()
        _, _, s_ref = orc.predict(to_orc(X[t]), to_orc(L.Vp), to_orc(L.Up), o["dt"])
        assert np.abs(s_gpu.astype(np.float64) - s_ref).max() <= 1e-5
        n = int(count.item())
        sel = heads[:n].cpu().numpy()
        ref_sel = orc.select_topk(s_gpu, k) if k is not None else orc.select_threshold(s_gpu, tau)
        assert np.array_equal(sel, ref_sel)
        _, y_ref = orc.attention_decode(to_orc(X[t]), o["Wq"], o["Wk"], o["Wv"], o["bq"], None,
                                        None, o["WoT"], o["Kc"], o["Vc"], o["lens"], sel, o["dt"])
        assert _err(y, y_ref) <= TOL, (name, t)
        assert np.array_equal(Ld.lens.cpu().numpy(), o["lens"])


def test_layer_full_size_opt175b_attention():
    """The OPT-175B attention shape (d 12288, 96 heads of 128, 2048 cached tokens, f16, top-19
    heads), one token, in the launch configuration the benchmark times."""
    announce("attention layer full size")
    cfg = wl.ATTN_OPT175B
    Ld = wl.make_attention_layer(cfg, device=DEV)
    o = _orc_state(Ld)
    x = wl.make_attn_tokens(cfg, 1, device=DEV)[0]
    scores = torch.empty(cfg.H, dtype=torch.float32, device=DEV)
    heads = torch.empty(cfg.k, dtype=torch.int32, device=DEV)
    count = torch.empty(1, dtype=torch.int32, device=DEV)
    y = csf.sparse_attention_layer(x, Ld.Vp, Ld.Up, Ld.Wq, Ld.Wk, Ld.Wv, Ld.bq, None, None, Ld.WoT,
                                   Ld.Kc, Ld.Vc, Ld.lens, k=cfg.k, scores=scores, heads=heads,
                                   count=count)
    torch.cuda.synchronize()
    sel = heads.cpu().numpy()
    assert np.array_equal(sel, orc.select_topk(scores.cpu().numpy(), cfg.k))
    _, y_ref = orc.attention_decode(to_orc(x), o["Wq"], o["Wk"], o["Wv"], o["bq"], None, None,
                                    o["WoT"], o["Kc"], o["Vc"], o["lens"], sel, o["dt"])
    assert _err(y, y_ref) <= TOL
    assert np.array_equal(Ld.lens.cpu().numpy(), o["lens"])

"""GPU parity of the hot-block layer (csf_sparse_ffn_layer_hot) and the static-locality helpers.

A power-law layer is profiled with the library's dense kernel, reordered hot first, and run with
its hot block always active and the predictor over the cold rows only.  Bars: the profiled firing
counts agree with the oracle's pre-activation signs (a count may differ only where a
pre-activation is within float32 rounding of 0); cold scores within 1e-5; the list bit-exact
against the oracle's composition fed the library's cold scores; y at the FFN bars; a hot block
of 0 is the plain layer, bit for bit.
"""
import numpy as np
import pytest
import torch

import contextual_sparsity_ffn_amd as csf
from contextual_sparsity_ffn_amd import locality, workloads as wl
from csf_testutil import announce, assert_ffn_close, to_orc
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _prepared(cfg, n_profile=96):
    L = wl.make_powerlaw_layer(cfg, device=DEV)
    P = wl.make_profile_tokens(cfg, n_profile, device=DEV)
    freq = locality.firing_frequency(L, P)
    order = locality.hot_first_order(freq)
    return L, P, freq, order, locality.reorder(L, order)


def test_firing_frequency_matches_oracle_signs():
    announce("locality firing frequency")
    cfg = wl.OPT30B.scaled(512, 1200, 64)
    L, P, freq, order, _ = _prepared(cfg, n_profile=48)
    torch.cuda.synchronize()
    o = dict(W1=to_orc(L.W1), b1=to_orc(L.b1), dt=orc.F16)
    counts = np.zeros(cfg.f)
    near = np.zeros(cfg.f, dtype=bool)
    for t in range(P.shape[0]):
        p = orc.preact(to_orc(P[t]), o["W1"], o["b1"], o["dt"])
        counts += p > 0
        near |= np.abs(p) < 1e-4 * np.abs(p).max()
    got = freq.cpu().double().numpy() * P.shape[0]
    diff = np.abs(got - counts)
    assert np.all(diff[~near] < 0.5) and np.all(diff <= P.shape[0])
    # the order is most frequent first, ties by index
    f_sorted = freq[order].cpu().numpy()
    assert np.all(np.diff(f_sorted) <= 0)


# f = 24576 leaves more than 20000 cold scores: the selection runs over many workgroups
@pytest.mark.parametrize("mode,f", [("topk", 3000), ("threshold", 3000), ("topk", 24576)])
def test_hot_layer_parity(mode, f):
    announce(f"locality hot layer {mode} f={f}")
    cfg = wl.OPT30B.scaled(1024, f, 128)
    L, P, freq, order, H = _prepared(cfg)
    hot = locality.hot_count(freq, 0.5, cap=cfg.k // 2)
    assert 0 < hot < cfg.f
    U_cold = H.U[hot:].contiguous()
    k_cold = cfg.k - hot if mode == "topk" else None
    tau = None if mode == "topk" else 0.5
    X = wl.make_tokens(cfg, 3)
    o = dict(V=to_orc(H.V), W1=to_orc(H.W1), b1=to_orc(H.b1), W2T=to_orc(H.W2T), dt=orc.F16)
    u_cold = to_orc(U_cold)
    for t in range(3):
        x = X[t].to(DEV)
        sc = torch.empty(cfg.f - hot, dtype=torch.float32, device=DEV)
        idx = torch.empty(cfg.f, dtype=torch.int32, device=DEV)
        cnt = torch.empty(1, dtype=torch.int32, device=DEV)
        y = csf.sparse_ffn_layer_hot(x, H.V, U_cold, H.W1, H.b1, None, H.W2T, hot, k=k_cold, tau=tau,
                                     scores=sc, idx=idx, count=cnt)
        torch.cuda.synchronize()
        n = int(cnt.item())
        gi = idx[:n].cpu().numpy()
        _, s_ref = orc.hot_layer_set(to_orc(X[t]), o["V"], u_cold, hot, o["dt"], k=k_cold, tau=tau)
        s_gpu = sc.cpu().numpy()
        assert np.abs(s_gpu.astype(np.float64) - s_ref).max() <= 1e-5
        cold = orc.select_topk(s_gpu, k_cold) if k_cold is not None else orc.select_threshold(s_gpu, tau)
        assert np.array_equal(gi, np.concatenate([np.arange(hot), cold + hot]).astype(np.int32))
        _, y_ref = orc.sparse_ffn(to_orc(X[t]), o["W1"], o["b1"], None, o["W2T"], gi, orc.RELU, orc.F16)
        assert_ffn_close(y, y_ref, cfg.dtype, f"hot layer {mode} token {t}")


@pytest.mark.parametrize("f", [2000, 24576])
def test_hot_block_of_zero_is_the_plain_layer(f):
    announce(f"locality hot = 0, f={f}")
    cfg = wl.OPT30B.scaled(1024, f, 128)
    L = wl.make_powerlaw_layer(cfg, device=DEV)
    x = wl.make_tokens(cfg, 1, device=DEV)[0]
    y0 = csf.sparse_ffn_layer(x, L.V, L.U, L.W1, L.b1, None, L.W2T, k=cfg.k)
    y1 = csf.sparse_ffn_layer_hot(x, L.V, L.U, L.W1, L.b1, None, L.W2T, 0, k=cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_reordered_layer_computes_the_same_function():
    announce("locality reorder")
    cfg = wl.OPT30B.scaled(768, 1500, 64)
    L, P, freq, order, H = _prepared(cfg, n_profile=32)
    X = wl.make_tokens(cfg, 2, device=DEV)
    y = csf.dense_ffn(X, L.W1, L.b1, None, L.W2T)
    yh = csf.dense_ffn(X, H.W1, H.b1, None, H.W2T)
    torch.cuda.synchronize()
    err = float((y - yh).abs().max() / y.abs().max())
    assert err < 1e-5, err

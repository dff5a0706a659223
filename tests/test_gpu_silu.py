"""GPU parity of the SiLU forms (SiLU, SwiGLU) and of the post-gate functional skip.

The kernels' SiLU is p / (1 + expf(-p)) in float32, the oracle's is the double-precision formula;
over a given active list both compute the same sum, so the FFN bars of csf_testutil apply
unchanged.  With the post-gate skip and a threshold tau > 0, a listed neuron is dropped when
|silu(p)| <= tau, a decision the kernel takes in float32 on its own p: for neurons whose
double-precision |silu(p)| lies within 1e-4 of tau either decision is correct, so the test reads
the kernel's decision for those (h = 0 or not) and checks every other one against the oracle.
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
AMBIGUOUS = 1e-4


def _dev_layer(L):
    d = lambda t: None if t is None else t.to(DEV)
    return wl.Layer(L.cfg, d(L.V), d(L.U), d(L.W1), d(L.b1), d(L.Wup), d(L.W2T))


def _silu_cfg(cfg, act=csf.SILU):
    return dataclasses.replace(cfg, act=act, wup_std=0.0 if act == csf.SILU else cfg.wup_std)


FFN_CASES = [
    ("silu-f32", _silu_cfg(wl.TINY_F32), 300),
    ("silu-f16-ragged", _silu_cfg(wl.OPT175B.scaled(2600, 3001, 136)), 777),
    ("swiglu-bf16", wl.LLAMA_SWIGLU.scaled(4096, 1433, 256), 700),
    ("swiglu-f16", dataclasses.replace(wl.LLAMA_SWIGLU.scaled(2600, 3001, 136), dtype=torch.float16),
     1501),
]


@pytest.mark.parametrize("name,cfg,count", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_sparse_and_dense_ffn_silu(name, cfg, count):
    announce(f"silu sparse_ffn {name}")
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    o = layer_to_orc(L)
    B = 3
    X = wl.make_tokens(cfg, B)
    g = torch.Generator().manual_seed(count)
    idx = torch.stack([torch.sort(torch.randperm(cfg.f, generator=g)[:count]).values
                       for _ in range(B)]).int()
    h = torch.empty(B, count, dtype=torch.float32, device=DEV)
    y = csf.sparse_ffn(X.to(DEV), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, idx.to(DEV), act=cfg.act, h=h)
    hd = torch.empty(B, cfg.f, dtype=torch.float32, device=DEV)
    yd = csf.dense_ffn(X.to(DEV), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, act=cfg.act, h=hd)
    torch.cuda.synchronize()
    for t in range(B):
        h_ref, y_ref = orc.sparse_ffn(to_orc(X[t]), o["W1"], o["b1"], o["Wup"], o["W2T"],
                                      idx[t].numpy(), o["act"], o["dt"])
        assert_ffn_close(y[t], y_ref, cfg.dtype, f"{name} sparse token {t}")
        assert np.abs(h[t].cpu().double().numpy() - h_ref).max() <= 1e-4 * np.abs(h_ref).max()
        assert np.count_nonzero(h_ref) == count            # SiLU has no exact zeros here
        hd_ref, yd_ref = orc.dense_ffn(to_orc(X[t]), o["W1"], o["b1"], o["Wup"], o["W2T"],
                                       o["act"], o["dt"])
        assert_ffn_close(yd[t], yd_ref, cfg.dtype, f"{name} dense token {t}")
        assert np.abs(hd[t].cpu().double().numpy() - hd_ref).max() <= 1e-4 * np.abs(hd_ref).max()
    y2 = csf.sparse_ffn(X.to(DEV), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, idx.to(DEV), act=cfg.act)
    assert torch.equal(y2, y)


LAYER_CASES = [
    ("swiglu-bf16-topk", wl.LLAMA_SWIGLU.scaled(4096, 1433, 256), None),
    ("silu-f16-threshold", _silu_cfg(wl.OPT175B.scaled(2048, 3001, 128)), 0.5),
]


@pytest.mark.parametrize("name,cfg,tau", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_end_to_end_silu(name, cfg, tau):
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    o = layer_to_orc(L)
    X = wl.make_tokens(cfg, 3)
    k = None if tau is not None else cfg.k
    for t in range(3):
        announce(f"silu layer {name} token {t}")
        f = cfg.f
        scores = torch.empty(f, dtype=torch.float32, device=DEV)
        idx = torch.empty(f, dtype=torch.int32, device=DEV)
        count = torch.empty(1, dtype=torch.int32, device=DEV)
        y = csf.sparse_ffn_layer(X[t].to(DEV), Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=k,
                                 tau=tau, act=cfg.act, scores=scores, idx=idx, count=count)
        torch.cuda.synchronize()
        s_gpu = scores.cpu().numpy()
        n = int(count.item())
        ix = idx[:n].cpu().numpy()
        ref_sel = orc.select_topk(s_gpu, k) if k is not None else orc.select_threshold(s_gpu, tau)
        assert np.array_equal(ix, ref_sel)
        _, y_ref = orc.sparse_ffn(to_orc(X[t]), o["W1"], o["b1"], o["Wup"], o["W2T"], ix,
                                  o["act"], o["dt"])
        assert_ffn_close(y, y_ref, cfg.dtype, f"{name} token {t}")


def test_layer_full_size_llama_swiglu():
    """The SwiGLU LLaMA-class layer at full size (d=4096, f=14336, r=256, bf16, k=7168)."""
    announce("silu layer full size swiglu")
    cfg = wl.LLAMA_SWIGLU
    Ld = wl.make_layer(cfg, device=DEV)
    o = layer_to_orc(Ld)
    x = wl.make_tokens(cfg, 1, device=DEV)[0]
    idx = torch.empty(cfg.k, dtype=torch.int32, device=DEV)
    count = torch.empty(1, dtype=torch.int32, device=DEV)
    scores = torch.empty(cfg.f, dtype=torch.float32, device=DEV)
    y = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=cfg.k, act=cfg.act,
                             scores=scores, idx=idx, count=count)
    torch.cuda.synchronize()
    assert int(count.item()) == cfg.k
    ix = idx.cpu().numpy()
    assert np.array_equal(ix, orc.select_topk(scores.cpu().numpy(), cfg.k))
    _, y_ref = orc.sparse_ffn(to_orc(x), o["W1"], o["b1"], o["Wup"], o["W2T"], ix, o["act"],
                              o["dt"])
    assert_ffn_close(y, y_ref, cfg.dtype, "swiglu full")


def _resolved_functional(x, o, listed, h_gpu, tau):
    """The listed neurons the oracle keeps (|silu(p)| > tau), with the kernel's decision taken for
    the ones within AMBIGUOUS of the threshold."""
    p = orc.preact(x, o["W1"], o["b1"], o["dt"])
    keep = []
    n_amb = 0
    for n, j in enumerate(listed):
        a = abs(orc.silu(p[j]))
        if abs(a - tau) <= AMBIGUOUS:
            n_amb += 1
            if h_gpu[n] != 0.0:
                keep.append(j)
        elif a > tau:
            keep.append(j)
    return np.array(keep, dtype=np.int32), n_amb


SKIP_CASES = [
    ("swiglu-bf16", wl.LLAMA_SWIGLU.scaled(2048, 2500, 128)),
    ("silu-f16", _silu_cfg(wl.LLAMA_SWIGLU.scaled(1024, 3001, 64), csf.SILU)),
]


@pytest.mark.parametrize("name,cfg", SKIP_CASES, ids=[c[0] for c in SKIP_CASES])
def test_functional_skip_layer_and_dense(name, cfg):
    """Post-gate skip with gate_tau = 0.1: the layer computes the predicted set cut to the
    neurons with |silu(p)| > 0.1 ([DV] "The Empirical Foundation"), the dense FFN the functional
    set itself."""
    cfg = dataclasses.replace(cfg, dtype=torch.float16) if cfg.act == csf.SILU else cfg
    announce(f"functional skip {name}")
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    o = layer_to_orc(L)
    X = wl.make_tokens(cfg, 3)
    tau = 0.1
    try:
        for t in range(3):
            x = X[t].to(DEV)
            idx = torch.empty(cfg.k, dtype=torch.int32, device=DEV)
            cnt = torch.empty(1, dtype=torch.int32, device=DEV)
            csf.set_ffn_flags(csf.FFN_SKIP_ZERO_H)
            csf.set_ffn_gate_threshold(tau)
            y = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=cfg.k,
                                     act=cfg.act, idx=idx, count=cnt)
            y_b = csf.sparse_ffn_layer(x, Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=cfg.k,
                                       act=cfg.act)
            # the FFN alone over the same list, with the per-entry h the kernel produced
            h = torch.empty(1, cfg.k, dtype=torch.float32, device=DEV)
            y_f = csf.sparse_ffn(x.unsqueeze(0), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T,
                                 idx.unsqueeze(0), act=cfg.act, h=h)
            hd = torch.empty(1, cfg.f, dtype=torch.float32, device=DEV)
            yd = csf.dense_ffn(x.unsqueeze(0), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, act=cfg.act, h=hd)
            torch.cuda.synchronize()
            listed = idx.cpu().numpy()
            xo = to_orc(X[t])
            keep, n_amb = _resolved_functional(xo, o, listed, h[0].cpu().numpy(), tau)
            assert 0 < len(keep) < len(listed)
            assert n_amb <= len(listed) // 100
            h_ref, y_ref = orc.sparse_ffn(xo, o["W1"], o["b1"], o["Wup"], o["W2T"], keep,
                                          o["act"], o["dt"])
            assert_ffn_close(y, y_ref, cfg.dtype, f"{name} layer token {t}")
            assert_ffn_close(y_f[0], y_ref, cfg.dtype, f"{name} ffn token {t}")
            assert torch.equal(y, y_b)
            # h of a kept entry is the plain activation, a dropped entry's is exactly 0
            hk = h[0].cpu().double().numpy()
            pos = np.searchsorted(listed, keep)
            assert np.abs(hk[pos] - h_ref).max() <= 1e-4 * np.abs(h_ref).max()
            assert np.count_nonzero(hk) == len(keep)
            # dense: the functional set itself
            keep_d, _ = _resolved_functional(xo, o, np.arange(cfg.f), hd[0].cpu().numpy(), tau)
            _, yd_ref = orc.sparse_ffn(xo, o["W1"], o["b1"], o["Wup"], o["W2T"], keep_d,
                                       o["act"], o["dt"])
            assert_ffn_close(yd[0], yd_ref, cfg.dtype, f"{name} dense token {t}")
        # tau = 0 with a SiLU gate drops nothing: the plain result, bit for bit
        csf.set_ffn_gate_threshold(0.0)
        y0 = csf.sparse_ffn_layer(X[0].to(DEV), Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, k=cfg.k,
                                  act=cfg.act)
        csf.set_ffn_flags(0)
        y0_plain = csf.sparse_ffn_layer(X[0].to(DEV), Ld.V, Ld.U, Ld.W1, Ld.b1, Ld.Wup, Ld.W2T,
                                        k=cfg.k, act=cfg.act)
        torch.cuda.synchronize()
        assert torch.equal(y0, y0_plain)
    finally:
        csf.set_ffn_flags(0)
        csf.set_ffn_gate_threshold(0.0)


def test_relu_gate_threshold_drops_small_activations():
    """The threshold applies to the ReLU forms as well: ReGLU with gate_tau > 0 keeps the neurons
    whose relu(gate) exceeds it."""
    cfg = wl.LLAMA_REGLU.scaled(1024, 2500, 128)
    announce("relu gate threshold")
    L = wl.make_layer(cfg)
    Ld = _dev_layer(L)
    o = layer_to_orc(L)
    X = wl.make_tokens(cfg, 2)
    p_scale = None
    try:
        for t in range(2):
            xo = to_orc(X[t])
            p = orc.preact(xo, o["W1"], o["b1"], o["dt"])
            if p_scale is None:
                p_scale = float(np.median(p[p > 0]))
            tau = p_scale
            csf.set_ffn_flags(csf.FFN_SKIP_ZERO_H)
            csf.set_ffn_gate_threshold(tau)
            hd = torch.empty(1, cfg.f, dtype=torch.float32, device=DEV)
            yd = csf.dense_ffn(X[t:t + 1].to(DEV), Ld.W1, Ld.b1, Ld.Wup, Ld.W2T, act=cfg.act, h=hd)
            torch.cuda.synchronize()
            hg = hd[0].cpu().numpy()
            keep = [j for j in range(cfg.f) if p[j] > tau + AMBIGUOUS * max(1.0, tau)
                    or (abs(p[j] - tau) <= AMBIGUOUS * max(1.0, tau) and hg[j] != 0.0)]
            keep = np.array(keep, dtype=np.int32)
            assert 0 < len(keep) < np.count_nonzero(p > 0)
            _, y_ref = orc.sparse_ffn(xo, o["W1"], o["b1"], o["Wup"], o["W2T"], keep, o["act"],
                                      o["dt"])
            assert_ffn_close(yd[0], y_ref, cfg.dtype, f"reglu gate threshold token {t}")
    finally:
        csf.set_ffn_flags(0)
        csf.set_ffn_gate_threshold(0.0)

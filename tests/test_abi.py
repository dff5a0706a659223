"""CPU-side checks of the C ABI: the library loads, exports every declared symbol, and rejects bad
arguments on the host with the documented status before anything is enqueued.

No call here passes validation, so no kernel is launched and no GPU is needed: the handle is
checked after every other argument, so argument errors are reported with a NULL handle, and a call
whose arguments are all valid stops at the NULL handle.  Device pointers are stand-in addresses
that the host code never dereferences.
"""
import ctypes
import json
import os
import re

import pytest

import contextual_sparsity_ffn_amd as csf
from contextual_sparsity_ffn_amd import _lib, workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.lib
OK, INVALID, UNSUPPORTED, MISALIGNED, WS_SMALL, HIP = range(6)
P = ctypes.c_void_p(0x7F0000001000)        # aligned stand-in device address (never dereferenced)
Q = ctypes.c_void_p(0x7F0000002008)        # 8-byte aligned only
NULL = None


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "csf.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(csf_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_version_and_status_strings():
    assert L.csf_abi_version() == 2
    assert L.csf_status_string(0) == b"CSF_OK"
    assert L.csf_status_string(4) == b"CSF_ERR_WORKSPACE_TOO_SMALL"
    assert L.csf_status_string(99) == b"CSF_ERR_UNKNOWN"


def test_handle_lifecycle_on_the_host():
    h = ctypes.c_void_p()
    assert L.csf_create(None, 0) == INVALID
    assert L.csf_destroy(None) == OK                       # NULL is accepted
    assert L.csf_get_device_info(None, None, None) == INVALID
    assert L.csf_set_ffn_flags(None, 0) == INVALID
    assert L.csf_set_ffn_gate_threshold(None, ctypes.c_float(0.0)) == INVALID
    assert L.csf_set_trace_events(None, None, 0) == INVALID
    rc = L.csf_create(ctypes.byref(h), -1)
    assert rc in (INVALID, HIP) and not h.value            # a bad index (or no runtime): no handle
    rc = L.csf_create(ctypes.byref(h), 0)
    assert rc in (OK, HIP)                                 # HIP: no device in this container
    if rc == OK:
        assert h.value
        assert L.csf_destroy(h) == OK


def test_valid_arguments_stop_at_a_missing_handle():
    assert L.csf_select_topk(NULL, P, 1, 100, 5, P, NULL, NULL, NULL, 0, NULL) == INVALID
    assert b"handle" in L.csf_last_error()
    assert L.csf_sparse_ffn(NULL, P, 1, 64, 100, csf.RELU, csf.F16, P, NULL, NULL, P, P, 10, NULL,
                            10, NULL, P, P, 1 << 24, NULL) == INVALID
    assert b"handle" in L.csf_last_error()


def test_workspace_sizes():
    assert csf.workspace_size(_lib.OP_SELECT_TOPK, 1, 12288, 49152) == 0
    assert csf.workspace_size(_lib.OP_PREDICT, 1, 12288, 49152, 1024, 0, csf.F16) >= 1024 * 4
    ffn = csf.workspace_size(_lib.OP_SPARSE_FFN, 1, 12288, 49152, 0, 2458, csf.F16)
    assert ffn >= (2458 + 12288) * 4
    layer = csf.workspace_size(_lib.OP_LAYER, 1, 12288, 49152, 1024, 2458, csf.F16)
    assert layer >= ffn + 49152 * 8
    assert csf.workspace_size(_lib.OP_SPARSE_FFN, 1, 0, 10) == 0      # invalid sizes -> 0
    assert csf.workspace_size(99, 1, 8, 8) == 0


def predict(x=P, B=1, d=64, V=P, r=16, U=P, f=100, dt=csf.F16, s=P, ws=P, wsb=1 << 20):
    return L.csf_predict_active(NULL, x, B, d, V, r, U, f, dt, s, ws, wsb, NULL)


def test_predict_validation():
    assert predict(d=60) == UNSUPPORTED                    # row not a multiple of 16 bytes
    assert predict(d=0) == INVALID
    assert predict(r=12) == UNSUPPORTED
    assert predict(r=8192) == UNSUPPORTED                  # beyond the kernel limit
    assert predict(f=0) == INVALID
    assert predict(dt=7) == INVALID
    assert predict(V=NULL) == INVALID
    assert predict(U=Q) == MISALIGNED
    assert predict(wsb=16) == WS_SMALL
    assert predict(ws=NULL) == INVALID
    assert predict(B=-1) == INVALID
    assert predict(B=0, x=NULL, s=NULL) == OK              # nothing to do, nothing enqueued
    assert predict(d=60) == UNSUPPORTED
    assert b"multiple of 16 bytes" in L.csf_last_error()


def test_select_validation():
    assert L.csf_select_topk(NULL, P, 1, 100, 101, P, NULL, NULL, NULL, 0, NULL) == INVALID
    assert L.csf_select_topk(NULL, P, 1, 100, -1, P, NULL, NULL, NULL, 0, NULL) == INVALID
    assert L.csf_select_topk(NULL, P, 1, 70000, 5, P, NULL, NULL, NULL, 0, NULL) == UNSUPPORTED
    assert L.csf_select_topk(NULL, P, 1, 100, 5, NULL, NULL, NULL, NULL, 0, NULL) == INVALID
    assert L.csf_select_topk(NULL, P, 1, 100, 5, P, Q, NULL, NULL, 0, NULL) == MISALIGNED
    assert L.csf_select_threshold(NULL, P, 1, 100, ctypes.c_float(float("nan")), P, P, NULL, NULL, 0,
                                  NULL) == INVALID
    assert L.csf_select_threshold(NULL, P, 1, 100, ctypes.c_float(0.5), P, NULL, NULL, NULL, 0,
                                  NULL) == INVALID                       # count is required
    assert L.csf_select_topk(NULL, NULL, 0, 100, 5, NULL, NULL, NULL, NULL, 0, NULL) == OK


def sparse(x=P, B=1, d=64, f=100, act=csf.RELU, dt=csf.F16, W1=P, b1=NULL, Wup=NULL, W2T=P,
           idx=P, stride=10, count=NULL, maxc=10, h=NULL, y=P, ws=P, wsb=1 << 24):
    return L.csf_sparse_ffn(NULL, x, B, d, f, act, dt, W1, b1, Wup, W2T, idx, stride, count, maxc,
                            h, y, ws, wsb, NULL)


def test_sparse_ffn_validation():
    assert sparse(maxc=11) == INVALID                      # max_count > idx_stride
    assert sparse(maxc=-1) == INVALID
    assert sparse(act=4) == INVALID
    assert sparse(act=-1) == INVALID
    assert sparse(act=csf.REGLU) == INVALID                # gated form needs Wup
    assert sparse(act=csf.SWIGLU) == INVALID               # gated form needs Wup
    assert sparse(Wup=P) == INVALID                        # ... and ReLU must not get one
    assert sparse(act=csf.SILU, Wup=P) == INVALID          # ... nor SiLU
    assert sparse(W2T=NULL) == INVALID
    assert sparse(b1=Q) == MISALIGNED
    assert sparse(d=12) == UNSUPPORTED
    assert sparse(d=64, dt=csf.F32, wsb=8) == WS_SMALL
    assert sparse(idx=NULL) == INVALID
    assert sparse(maxc=70000, stride=70000) == UNSUPPORTED   # longer than a list the kernels take
    assert L.csf_dense_ffn(NULL, P, 1, 64, 70000, csf.RELU, csf.F16, P, NULL, NULL, P, NULL, P, P,
                           1 << 30, NULL) == UNSUPPORTED


def test_layer_validation():
    def layer(k=5, tau=0.5, r=16, **kw):
        a = dict(x=P, d=64, f=100, act=csf.RELU, dt=csf.F16, V=P, U=P, W1=P, b1=NULL, Wup=NULL,
                 W2T=P, y=P, ws=P, wsb=1 << 24)
        a.update(kw)
        return L.csf_sparse_ffn_layer(NULL, a["x"], a["d"], a["f"], r, a["act"], a["dt"], a["V"], a["U"],
                                      a["W1"], a["b1"], a["Wup"], a["W2T"], k, ctypes.c_float(tau),
                                      a["y"], NULL, NULL, NULL, a["ws"], a["wsb"], NULL)
    assert layer(k=-2) == INVALID
    assert layer(k=101) == INVALID
    assert layer(k=-1, tau=float("nan")) == INVALID
    assert layer(r=10) == UNSUPPORTED
    assert layer(V=NULL) == INVALID
    assert layer(wsb=100) == WS_SMALL


def test_fault_injection_hook(monkeypatch):
    """CSF_FAULT_INJECT makes the named entry points fail with CSF_ERR_HIP once their arguments
    pass the host checks, before the handle check and before any launch; the binding turns the
    status into a CsfError that carries it."""
    monkeypatch.setenv("CSF_FAULT_INJECT", "csf_sparse_ffn")
    assert sparse() == HIP
    assert b"CSF_FAULT_INJECT" in L.csf_last_error() and b"nothing enqueued" in L.csf_last_error()
    assert sparse(maxc=11) == INVALID                      # argument checks still come first
    assert L.csf_select_topk(NULL, P, 1, 100, 5, P, NULL, NULL, NULL, 0, NULL) == INVALID
    assert b"handle" in L.csf_last_error()                 # an entry point not named: no hook
    monkeypatch.setenv("CSF_FAULT_INJECT", "csf_predict_active,csf_select_topk")
    assert predict() == HIP
    assert L.csf_select_topk(NULL, P, 1, 100, 5, P, NULL, NULL, NULL, 0, NULL) == HIP
    assert sparse() == INVALID
    assert predict(B=0, x=NULL, s=NULL) == OK              # nothing to dispatch: no failure
    monkeypatch.setenv("CSF_FAULT_INJECT", "csf_sparse_ffn_layer_")   # names match whole
    assert L.csf_sparse_ffn_layer(NULL, P, 64, 100, 16, csf.RELU, csf.F16, P, P, P, NULL, NULL, P,
                                  5, ctypes.c_float(0.5), P, NULL, NULL, NULL, P, 1 << 24,
                                  NULL) == INVALID
    monkeypatch.setenv("CSF_FAULT_INJECT", "all")
    assert L.csf_sparse_ffn_layer(NULL, P, 64, 100, 16, csf.RELU, csf.F16, P, P, P, NULL, NULL, P,
                                  5, ctypes.c_float(0.5), P, NULL, NULL, NULL, P, 1 << 24,
                                  NULL) == HIP
    with pytest.raises(csf.CsfError) as err:
        _lib._check(sparse())
    assert err.value.status == HIP and "CSF_FAULT_INJECT" in str(err.value)
    monkeypatch.setenv("CSF_FAULT_INJECT", "")
    assert sparse() == INVALID
    monkeypatch.delenv("CSF_FAULT_INJECT")
    assert sparse() == INVALID


def test_batched_union_validation():
    taken = ctypes.c_int(-1)

    def bu(X=P, B=4, d=256, f=100, act=csf.RELU, dt=csf.F16, W1=P, b1=NULL, Wup=NULL, W2T=P,
           bm=P, sem=0, path=0, Y=P, uc=NULL, ws=P, wsb=1 << 26):
        return L.csf_sparse_ffn_batched_union(NULL, X, B, d, f, act, dt, W1, b1, Wup, W2T, bm, sem, path,
                                              Y, uc, ctypes.byref(taken), ws, wsb, NULL)
    assert bu(B=33) == UNSUPPORTED                         # more tokens than one call takes
    assert bu(B=-1) == INVALID
    assert bu(f=70000) == UNSUPPORTED
    assert bu(sem=2) == INVALID
    assert bu(path=3) == INVALID
    assert bu(bm=NULL) == INVALID
    assert bu(bm=Q) == MISALIGNED
    assert bu(Y=NULL) == INVALID
    assert bu(uc=Q) == MISALIGNED
    assert bu(dt=csf.F32, path=2) == UNSUPPORTED           # matrix cores: 16-bit types only
    assert bu(d=264, path=2) == UNSUPPORTED                # ... and d % 256 == 0
    assert b"d % 256" in L.csf_last_error()
    assert bu(act=csf.REGLU) == INVALID
    assert bu(wsb=1024) == WS_SMALL
    # B = 0 enqueues nothing and reports the path the sizes would take
    assert bu(B=0, X=NULL, bm=NULL, Y=NULL, dt=csf.F32) == OK and taken.value == 1
    assert bu(B=0, X=NULL, bm=NULL, Y=NULL, path=2) == OK and taken.value == 2
    need = csf.workspace_size(_lib.OP_BATCHED_UNION, 32, 7168, 28672, 0, 0, csf.F16)
    # union list + h (float32, or hi/lo halves) + partial rows
    assert need >= 28672 * 4 + 32 * 28672 * 4 + 32 * 7168 * 4


def test_batched_layer_validation():
    taken = ctypes.c_int(-1)

    def bl(k=5, tau=0.5, r=16, B=4, V=P, bm=NULL, path=0, wsb=1 << 26):
        return L.csf_sparse_ffn_batched_layer(NULL, P, B, 256, 100, r, csf.RELU, csf.F16, V, P, P, NULL,
                                              NULL, P, k, ctypes.c_float(tau), 0, path, P, bm,
                                              NULL, ctypes.byref(taken), P, wsb, NULL)
    assert bl(k=-2) == INVALID
    assert bl(k=101) == INVALID
    assert bl(k=-1, tau=float("nan")) == INVALID
    assert bl(r=10) == UNSUPPORTED
    assert bl(V=NULL) == INVALID
    assert bl(bm=Q) == MISALIGNED
    assert bl(B=40) == UNSUPPORTED
    assert bl(wsb=64) == WS_SMALL
    assert bl(B=0) == OK
    lay = csf.workspace_size(_lib.OP_BATCHED_LAYER, 8, 7168, 28672, 512, 5734, csf.F16)
    assert lay > csf.workspace_size(_lib.OP_BATCHED_UNION, 8, 7168, 28672, 0, 0, csf.F16) + 8 * 28672 * 4


def test_stack_validation():
    lw = (_lib.LayerWeights * 2)(_lib.LayerWeights(P.value, P.value, P.value, None, P.value, None),
                                 _lib.LayerWeights(P.value, P.value, P.value, None, P.value, None))
    S1, S2 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)   # stand-in stream handles

    def st(layers=lw, L=2, k=5, tau=0.5, mode=0, norm=1, eps=1e-6, x=P, B=1, side=NULL, wsb=1 << 26,
           r=16, stream=NULL):
        return L_.csf_stack_forward(NULL, layers, L, 256, 100, r, csf.RELU, csf.F16, x, B, mode, k,
                                    ctypes.c_float(tau), norm, ctypes.c_float(eps), NULL, NULL,
                                    NULL, NULL, P, wsb, stream, side)
    L_ = L
    assert st(L=-1) == INVALID
    assert st(layers=None) == INVALID
    assert st(mode=2) == INVALID
    assert st(norm=2) == INVALID
    assert st(eps=-1.0) == INVALID
    assert st(mode=1) == INVALID                            # look-ahead without a side stream
    assert st(mode=1, side=S1, stream=S1) == INVALID        # ... or with the main stream as side
    assert st(k=101) == INVALID
    assert st(k=-1, tau=float("nan")) == INVALID
    assert st(r=10) == UNSUPPORTED
    assert st(x=Q) == MISALIGNED
    assert st(wsb=64) == WS_SMALL
    bad = (_lib.LayerWeights * 2)(lw[0], _lib.LayerWeights(P.value, None, P.value, None, P.value,
                                                           None))
    assert st(layers=bad) == INVALID
    assert b"layer 1" in L.csf_last_error()
    assert st(L=0) == OK and st(B=0) == OK                  # nothing to do
    need = csf.workspace_size(_lib.OP_STACK, 1, 7168, 28672, 512, 5734, csf.F16)
    assert need >= 2 * 7168 * 2 + 2 * 28672 * 4 + 2 * 5734 * 4


def test_ffn_options_need_a_live_handle():
    """The gathered FFN's options are state of a handle, not of the calling thread: without a
    handle they are rejected (the values themselves are checked in the GPU handle tests)."""
    assert L.csf_set_ffn_flags(NULL, csf.FFN_SKIP_ZERO_H) == INVALID
    assert L.csf_set_ffn_gate_threshold(NULL, ctypes.c_float(0.1)) == INVALID
    assert b"handle" in L.csf_last_error()


def test_k_from_ratio_matches_the_printed_figures():
    figs = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))
    for case in figs["k_from_ratio"]:
        assert csf.k_from_ratio(case["f"], case["ratio"]) == case["k"]
    # the workload sizes: 10% of 1024, 5% of 49152, 20% of 28672
    assert csf.k_from_ratio(1024, 0.10) == wl.TINY_F32.k == 102
    assert csf.k_from_ratio(49152, 0.05) == wl.OPT175B.k == 2458
    assert csf.k_from_ratio(28672, 0.20) == wl.OPT30B.k == 5734


def test_budget_figure_arithmetic():
    """An 11 GB FFN stack at 90% predicted sparsity leaves about 10 GB for the predictor."""
    b = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))["predictor_budget"]
    assert abs(b["dense_bytes_GB"] * b["predicted_sparsity"] - b["headroom_GB_approx"]) < 0.15
    # the headline workload's predictor is far inside that budget: (V + U) < s * dense bytes
    cfg = wl.OPT175B
    pred = 2 * (cfg.r * cfg.d + cfg.f * cfg.r)
    assert pred < 0.95 * wl.dense_bytes(cfg)


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(64, dtype=torch.float16)
    with pytest.raises(ValueError):
        csf.predict_active(x, torch.zeros(16, 64, dtype=torch.float16),
                           torch.zeros(100, 16, dtype=torch.float16))


def attn(x=P, d=256, H=8, dh=32, dt=csf.F16, Wq=P, Wk=P, Wv=P, bq=NULL, bk=NULL, bv=NULL, WoT=P,
         Kc=P, Vc=P, Tmax=64, lens=P, heads=P, count=NULL, maxh=4, kv_all=0, o=NULL, y=P, ws=P,
         wsb=1 << 26):
    return L.csf_sparse_attention_decode(NULL, x, d, H, dh, dt, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, Tmax,
                                         lens, heads, count, maxh, kv_all, o, y, ws, wsb, NULL)


def test_attention_validation():
    assert attn(dh=12) == UNSUPPORTED                     # 24-byte cached rows
    assert attn(dh=96) == UNSUPPORTED                     # 192 bytes: not a power of two
    assert attn(dh=512) == UNSUPPORTED                    # 1 KiB rows
    assert attn(dt=csf.F32, dh=4) == UNSUPPORTED          # 16-byte rows
    assert attn(H=0) == INVALID
    assert attn(Tmax=0) == INVALID
    assert attn(kv_all=2) == INVALID
    assert attn(Kc=NULL) == INVALID
    assert attn(lens=NULL) == INVALID
    assert attn(y=NULL) == INVALID
    assert attn(bq=Q) == MISALIGNED
    assert attn(maxh=9) == INVALID                        # more entries than heads
    assert attn(heads=NULL) == INVALID                    # the dense step needs max_heads == H
    assert attn(heads=NULL, maxh=8, count=P) == INVALID
    assert attn(H=1024, dh=128) == UNSUPPORTED            # H * dh beyond the row-list limit
    assert attn(d=12) == UNSUPPORTED
    assert attn(wsb=8) == WS_SMALL
    assert L.csf_sparse_attention_layer(NULL, P, 256, 8, 32, 64, csf.F16, P, P, P, P, P, NULL, NULL, NULL,
                                        P, P, P, 64, P, 9, 0.0, 0, NULL, NULL, NULL, NULL, P, P,
                                        1 << 26, NULL) == INVALID        # k > H
    assert L.csf_sparse_attention_layer(NULL, P, 256, 8, 32, 64, csf.F16, P, P, P, P, P, NULL, NULL, NULL,
                                        P, P, P, 64, P, -1, float("nan"), 0, NULL, NULL, NULL,
                                        NULL, P, P, 1 << 26, NULL) == INVALID   # NaN threshold
    assert L.csf_sparse_attention_layer(NULL, P, 256, 8, 32, 64, csf.F16, NULL, P, P, P, P, NULL, NULL,
                                        NULL, P, P, P, 64, P, 2, 0.0, 0, NULL, NULL, NULL, NULL, P,
                                        P, 1 << 26, NULL) == INVALID     # no predictor
    size = csf.attention_workspace_size
    assert size(_lib.OP_ATTN_DECODE, 12288, 96, 128, 0, 2112, 19, csf.F16) > 19 * 128 * 4 * 3
    assert size(_lib.OP_ATTN_LAYER, 12288, 96, 128, 256, 2112, 19, csf.F16) > \
        size(_lib.OP_ATTN_DECODE, 12288, 96, 128, 0, 2112, 19, csf.F16)
    assert size(_lib.OP_ATTN_DECODE, 12288, 96, 128, 0, 2112, 97, csf.F16) == 0
    assert size(_lib.OP_ATTN_LAYER, 12288, 96, 128, 0, 2112, 19, csf.F16) == 0
    assert size(_lib.OP_SPARSE_FFN, 12288, 96, 128, 0, 2112, 19, csf.F16) == 0

"""GPU checks of the library handle (csf_create / csf_destroy): it reports its device's facts, its
options belong to it alone, and a destroyed or foreign handle is refused before anything runs."""
import ctypes

import pytest
import torch

import contextual_sparsity_ffn_amd as csf
from contextual_sparsity_ffn_amd import _lib, workloads as wl
from csf_testutil import announce

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_handle_reports_the_device_compute_units():
    announce("handle device facts")
    ctx = csf.Context(0)
    try:
        assert ctx.compute_units == torch.cuda.get_device_properties(0).multi_processor_count
        dev, cus = ctypes.c_int(-1), ctypes.c_int(-1)
        assert _lib.lib.csf_get_device_info(ctx.handle, ctypes.byref(dev), ctypes.byref(cus)) == 0
        assert dev.value == 0 and cus.value == ctx.compute_units
    finally:
        ctx.close()


def test_bad_device_index_is_refused():
    h = ctypes.c_void_p()
    n = torch.cuda.device_count()
    assert _lib.lib.csf_create(ctypes.byref(h), n) == 1 and not h.value
    assert _lib.lib.csf_create(ctypes.byref(h), -1) == 1 and not h.value


def test_ffn_options_belong_to_their_handle():
    """The post-gate skip set on one handle changes that handle's calls only."""
    announce("per-handle FFN options")
    cfg = wl.OPT175B.scaled(2048, 3001, 128)
    L = wl.make_layer(cfg, device=DEV)
    x = wl.make_tokens(cfg, 1, device=DEV)[0]
    idx = torch.sort(torch.randperm(cfg.f, device=DEV)[:600]).values.int().reshape(1, -1)
    a, b = csf.Context(0), csf.Context(0)
    try:
        a.set_ffn_flags(csf.FFN_SKIP_ZERO_H)
        y_plain = csf.sparse_ffn(x, L.W1, L.b1, None, L.W2T, idx, ctx=b)
        y_skip = csf.sparse_ffn(x, L.W1, L.b1, None, L.W2T, idx, ctx=a)
        y_plain2 = csf.sparse_ffn(x, L.W1, L.b1, None, L.W2T, idx, ctx=b)
        torch.cuda.synchronize()
        assert torch.equal(y_plain, y_plain2)          # b never saw a's option
        # the skip drops zero terms: the same sum up to float32 order, not necessarily the bits
        assert (y_skip - y_plain).abs().max().item() <= 1e-4 * y_plain.abs().max().item()
        b.set_ffn_gate_threshold(0.0)
        with pytest.raises(csf.CsfError):
            a.set_ffn_gate_threshold(-1.0)             # validated: negative threshold
        with pytest.raises(csf.CsfError):
            a.set_ffn_flags(7)                          # unknown flag bits
    finally:
        a.close()
        b.close()


def test_destroyed_handle_is_refused():
    """A handle is looked up among the live ones: after csf_destroy it is refused (and a second
    destroy is an error), before anything is enqueued."""
    announce("destroyed handle")
    ctx = csf.Context(0)
    h = ctypes.c_void_p(ctx.handle.value)
    ctx.close()
    cfg = wl.TINY_F32
    s = torch.rand(1, cfg.f, device=DEV)
    idx = torch.full((1, cfg.k), -7, dtype=torch.int32, device=DEV)
    for handle in (h, None):
        rc = _lib.lib.csf_select_topk(handle, ctypes.c_void_p(s.data_ptr()), 1, cfg.f, cfg.k,
                                      ctypes.c_void_p(idx.data_ptr()), None, None, None, 0, None)
        assert rc == 1 and b"handle" in _lib.lib.csf_last_error()
    torch.cuda.synchronize()
    assert (idx == -7).all()                           # nothing ran
    assert _lib.lib.csf_destroy(h) == 1


def test_injected_failure_reaches_the_caller_and_launches_nothing(monkeypatch):
    """With CSF_FAULT_INJECT naming an entry point, the binding's call raises CsfError with
    CSF_ERR_HIP and the outputs keep their old contents (nothing ran); other entry points and,
    once the variable is cleared, the same one work as before."""
    announce("fault injection through the binding")
    cfg = wl.OPT175B.scaled(1024, 2000, 64)
    L = wl.make_layer(cfg, device=DEV)
    x = wl.make_tokens(cfg, 1, device=DEV)[0]
    idx = torch.arange(0, cfg.f, 7, dtype=torch.int32, device=DEV)
    y = torch.full((cfg.d,), 1234.5, dtype=torch.float32, device=DEV)
    monkeypatch.setenv("CSF_FAULT_INJECT", "csf_sparse_ffn")
    with pytest.raises(csf.CsfError) as err:
        csf.sparse_ffn(x, L.W1, L.b1, None, L.W2T, idx, y=y)
    torch.cuda.synchronize()
    assert err.value.status == 5 and "CSF_FAULT_INJECT" in str(err.value)
    assert bool((y == 1234.5).all())
    s = csf.predict_active(x.reshape(1, -1), L.V, L.U)       # not named: runs
    torch.cuda.synchronize()
    assert bool(torch.isfinite(s).all())
    monkeypatch.delenv("CSF_FAULT_INJECT")
    y2 = csf.sparse_ffn(x, L.W1, L.b1, None, L.W2T, idx, y=y)
    torch.cuda.synchronize()
    assert y2.data_ptr() == y.data_ptr() and not bool((y == 1234.5).any())

"""The no-allocation layer entry point (csf_sparse_ffn_layer_noalloc) against the workspace one
(csf_sparse_ffn_layer), through the C ABI: the same kernels on the library's static scratch, so
scores, lists and y are bit-identical.  Two calls in a row on the same scratch, the second with a
smaller layer; then a threshold layer; then a layer too large for the scratch, refused."""
import ctypes

import pytest
import torch

from contextual_sparsity_ffn_amd import _lib, workloads as wl
from csf_testutil import announce

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
L = _lib.lib
vp = ctypes.c_void_p


def _p(t):
    return None if t is None else vp(t.data_ptr())


def _run_both(h, Ld, x, k, tau):
    cfg = Ld.cfg
    d, f, r = cfg.d, cfg.f, cfg.r
    code = _lib.dtype_code(cfg.dtype)
    kk = -1 if k is None else k
    mc = f if kk < 0 else kk
    stream = vp(torch.cuda.current_stream(DEV).cuda_stream)
    outs = []
    for noalloc in (False, True):
        y = torch.full((d,), float("nan"), dtype=torch.float32, device=DEV)
        sc = torch.full((f,), -1.0, dtype=torch.float32, device=DEV)
        ix = torch.full((max(mc, 1),), -1, dtype=torch.int32, device=DEV)
        cn = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        common = (_p(x), d, f, r, cfg.act, code, _p(Ld.V), _p(Ld.U), _p(Ld.W1), _p(Ld.b1),
                  _p(Ld.Wup), _p(Ld.W2T), kk, ctypes.c_float(tau or 0.0), _p(y), _p(sc), _p(ix),
                  _p(cn))
        if noalloc:
            rc = L.csf_sparse_ffn_layer_noalloc(h, *common, stream)
        else:
            wsb = L.csf_workspace_size(h, _lib.OP_LAYER, 1, d, f, r, mc, code)
            ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
            rc = L.csf_sparse_ffn_layer(h, *common, _p(ws), wsb, stream)
        assert rc == 0, L.csf_last_error()
        torch.cuda.synchronize()
        outs.append((y, sc, ix, cn))
    (y0, s0, i0, c0), (y1, s1, i1, c1) = outs
    assert torch.equal(s0, s1)
    assert torch.equal(c0, c1)
    n = int(c0.item())
    assert n == (k if k is not None else n) and n > 0
    assert torch.equal(i0[:n], i1[:n])
    assert torch.equal(y0, y1)
    assert torch.isfinite(y1).all()


def test_noalloc_layer_matches_the_workspace_layer():
    h = vp()
    assert L.csf_create(ctypes.byref(h), 0) == 0
    try:
        # the headline shape first, then a smaller layer on the same scratch
        for cfg, ntok in ((wl.OPT175B, 2), (wl.OPT175B.scaled(2048, 3001, 128), 2)):
            Ld = wl.make_layer(cfg, device=DEV)
            X = wl.make_tokens(cfg, ntok, device=DEV)
            for t in range(ntok):
                announce(f"no-alloc layer d={cfg.d} f={cfg.f} token {t}")
                _run_both(h, Ld, X[t], cfg.k, None)
        # a threshold (gated, bfloat16) layer: the count comes from the device
        cfg = wl.LLAMA_REGLU.scaled(4096, 1433, 256)
        Ld = wl.make_layer(cfg, device=DEV)
        X = wl.make_tokens(cfg, 2, device=DEV)
        for t in range(2):
            announce(f"no-alloc threshold layer token {t}")
            _run_both(h, Ld, X[t], None, cfg.tau)
    finally:
        assert L.csf_destroy(h) == 0


def test_noalloc_refuses_a_layer_beyond_the_scratch():
    """d 32768, f 65536, r 4096 in threshold mode needs about 9.8 MiB of workspace: refused before
    anything is enqueued (the output keeps its contents)."""
    announce("no-alloc size limit")
    h = vp()
    assert L.csf_create(ctypes.byref(h), 0) == 0
    try:
        d, f, r = 32768, 65536, 4096
        assert L.csf_workspace_size(h, _lib.OP_LAYER, 1, d, f, r, f, _lib.F16) > 8 << 20
        x = torch.zeros(d, dtype=torch.float16, device=DEV)
        w = torch.zeros(16, dtype=torch.float16, device=DEV)     # never read: refused first
        y = torch.full((d,), 7.0, dtype=torch.float32, device=DEV)
        rc = L.csf_sparse_ffn_layer_noalloc(h, _p(x), d, f, r, _lib.RELU, _lib.F16, _p(w), _p(w),
                                            _p(w), None, None, _p(w), -1, ctypes.c_float(0.5),
                                            _p(y), None, None, None, None)
        assert rc == 2                                             # CSF_ERR_UNSUPPORTED
        assert b"static scratch" in L.csf_last_error()
        torch.cuda.synchronize()
        assert (y == 7.0).all()
    finally:
        assert L.csf_destroy(h) == 0

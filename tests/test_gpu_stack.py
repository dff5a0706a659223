"""GPU parity of the residual stack (csf_stack_forward), synchronous and look-ahead.

Teacher-forced against the oracle at every layer (a legitimate difference at a selection boundary
must not cascade into later layers): from the logged stream x_l, normalised input xhat_l and
active list A_l of the library's own run, each layer is checked on its own --
  * xhat_l is the rounding of x_l / sqrt(mean(x_l^2) + eps) (a one-unit difference only where the
    exact value sits at a rounding midpoint, within float32 rounding of the scale);
  * A_l is the oracle's selection from predictor_l(xhat_l) (synchronous) or predictor_l(xhat_{l-1})
    (look-ahead, l >= 1), up to neurons whose oracle score is within 1e-5 of the cut;
  * x_{l+1} - x_l matches the oracle's sparse FFN of xhat_l over A_l at the FFN bars.
A second check replays the look-ahead run with the library's single-layer entry points on one
stream and must reproduce it bit for bit: the side stream saw the right inputs, with no race.
"""
import numpy as np
import pytest
import torch

import contextual_sparsity_ffn_amd as csf
from contextual_sparsity_ffn_amd import workloads as wl
from csf_testutil import ORC_DT, announce, assert_ffn_close, layer_to_orc, to_orc
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
EPS = 1e-6


def _layers(cfg, L, device=DEV):
    return [wl.make_layer(cfg, device=device, layer=l) for l in range(L)]


def _run(layers, X, cfg, lookahead, norm=True):
    B, d = X.shape
    nl = len(layers)
    stride = cfg.k if cfg.k is not None else cfg.f
    x = X.float().to(DEV).contiguous()
    x_log = torch.empty(nl, B, d, dtype=torch.float32, device=DEV)
    xhat_log = torch.empty(nl, B, d, dtype=cfg.dtype, device=DEV)
    idx_log = torch.full((nl, B, stride), -1, dtype=torch.int32, device=DEV)
    count_log = torch.full((nl, B), -1, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream(device=DEV)
    csf.stack_forward(x, layers, k=cfg.k, tau=cfg.tau, act=cfg.act, lookahead=lookahead,
                      norm=norm, eps=EPS, x_log=x_log, xhat_log=xhat_log, idx_log=idx_log,
                      count_log=count_log, side_stream=side)
    torch.cuda.synchronize()
    return x, x_log, xhat_log, idx_log, count_log


def _check_xhat(x, xhat_gpu, dt, norm):
    """xhat_gpu is the storage rounding of x * scale, up to exact midpoint cases."""
    ref = orc.rms_normalize(x, ORC_DT[dt], EPS) if norm else orc.round_to_storage(x, ORC_DT[dt])
    g = orc.widen(to_orc(xhat_gpu), ORC_DT[dt])
    o = orc.widen(ref, ORC_DT[dt])
    bad = np.nonzero(g != o)[0]
    if bad.size:
        xd = x.astype(np.float64)
        scale = 1.0 / np.sqrt(np.mean(xd * xd) + EPS) if norm else 1.0
        v = xd[bad] * scale
        mid = 0.5 * (g[bad] + o[bad])
        # only a value within float32 rounding of a midpoint may round either way
        assert np.all(np.abs(v - mid) <= 4e-7 * np.abs(v) + 1e-30), (bad[:8], v[:8], g[bad][:8])
        assert bad.size <= max(2, x.size // 1000)


def _check_sets(gpu_idx, s_ref, k, tau):
    gpu = set(gpu_idx.tolist())
    if k is not None:
        ref = orc.select_topk(s_ref, k)
        theta = np.sort(s_ref.astype(np.float64))[::-1][k - 1] if k > 0 else np.inf
        assert len(gpu) == k
    else:
        ref = orc.select_threshold(s_ref, tau)
        theta = tau
    for j in gpu.symmetric_difference(set(ref.tolist())):
        assert abs(float(s_ref[j]) - theta) < 1e-5, (j, s_ref[j], theta)


def _teacher_forced(layers, cfg, X, lookahead, norm=True, check_layers=None):
    xL, x_log, xhat_log, idx_log, count_log = _run(layers, X, cfg, lookahead, norm)
    nl, B = x_log.shape[0], x_log.shape[1]
    for l in (range(nl) if check_layers is None else check_layers):
        o = layer_to_orc(wl.Layer(cfg, layers[l].V.cpu(), layers[l].U.cpu(), layers[l].W1.cpu(),
                                  layers[l].b1.cpu(), None if layers[l].Wup is None else layers[l].Wup.cpu(),
                                  layers[l].W2T.cpu()))
        x_next = (x_log[l + 1] if l + 1 < nl else xL).cpu().double().numpy()
        for t in range(B):
            x_l = x_log[l, t].cpu().numpy()
            _check_xhat(x_l, xhat_log[l, t], cfg.dtype, norm)
            src = xhat_log[l - 1, t] if (lookahead and l > 0) else xhat_log[l, t]
            _, _, s_ref = orc.predict(to_orc(src), o["V"], o["U"], o["dt"])
            cnt = int(count_log[l, t].item())
            gi = idx_log[l, t, :cnt].cpu().numpy()
            assert np.all(np.diff(gi) > 0)                       # ascending
            _check_sets(gi, s_ref, cfg.k, cfg.tau)
            _, y_ref = orc.sparse_ffn(to_orc(xhat_log[l, t]), o["W1"], o["b1"], o["Wup"], o["W2T"],
                                      gi, o["act"], o["dt"])
            y_gpu = torch.from_numpy(x_next[t] - x_l.astype(np.float64))
            assert_ffn_close(y_gpu, y_ref, cfg.dtype, f"layer {l} token {t}")
    return xL, x_log, xhat_log, idx_log, count_log


# B = 1 takes the one-kernel FFN (its hand-over state prepared by each block's normalisation
# kernel); B = 2 the three-kernel form
@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("lookahead", [False, True], ids=["sync", "lookahead"])
def test_stack_teacher_forced_topk(lookahead, B):
    announce(f"stack top-k lookahead={lookahead} B={B}")
    cfg = wl.OPT30B_STACK48.scaled(512, 2048, 64)
    layers = _layers(cfg, 4)
    X = wl.make_tokens(cfg, B)
    _teacher_forced(layers, cfg, X, lookahead)


@pytest.mark.parametrize("B", [1, 2])
def test_stack_teacher_forced_threshold_reglu_literal(B):
    announce(f"stack threshold reglu literal B={B}")
    cfg = wl.LLAMA_REGLU.scaled(512, 1433, 64)
    layers = _layers(cfg, 3)
    X = wl.make_tokens(cfg, B)
    _teacher_forced(layers, cfg, X, lookahead=True, norm=False)


def _replay(layers, cfg, X, x_log, xhat_log, idx_log, count_log, xL, lookahead):
    """Single-layer entry points on one stream, fed the logged inputs: must give the same bits."""
    nl = len(layers)
    for l in range(nl):
        src = xhat_log[l - 1] if (lookahead and l > 0) else xhat_log[l]
        s = csf.predict_active(src, layers[l].V, layers[l].U)
        if cfg.k is not None:
            idx = csf.select_topk(s, cfg.k)
            assert torch.equal(idx, idx_log[l]), f"layer {l}: selection differs"
            y = csf.sparse_ffn(xhat_log[l], layers[l].W1, layers[l].b1, layers[l].Wup,
                               layers[l].W2T, idx, act=cfg.act)
        else:
            idx, cnt = csf.select_threshold(s, cfg.tau)
            assert torch.equal(cnt, count_log[l])
            for t in range(idx.shape[0]):
                c = int(cnt[t])
                assert torch.equal(idx[t, :c], idx_log[l, t, :c])
            y = csf.sparse_ffn(xhat_log[l], layers[l].W1, layers[l].b1, layers[l].Wup,
                               layers[l].W2T, idx, act=cfg.act, count=cnt)
        nxt = x_log[l + 1] if l + 1 < nl else xL
        assert torch.equal(x_log[l] + y, nxt), f"layer {l}: residual stream differs"
    torch.cuda.synchronize()


@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("lookahead", [False, True], ids=["sync", "lookahead"])
def test_stack_replays_bit_exact_from_single_layer_calls(lookahead, B):
    announce(f"stack replay lookahead={lookahead} B={B}")
    cfg = wl.OPT30B_STACK48.scaled(1024, 3000, 128)
    layers = _layers(cfg, 6)
    X = wl.make_tokens(cfg, B)
    xL, x_log, xhat_log, idx_log, count_log = _run(layers, X, cfg, lookahead)
    _replay(layers, cfg, X, x_log, xhat_log, idx_log, count_log, xL, lookahead)
    # the same run again gives the same bits
    xL2, *_ = _run(layers, X, cfg, lookahead)
    assert torch.equal(xL, xL2)


def test_stack_single_layer_and_modes_agree_at_layer_zero():
    """L = 1: look-ahead has nothing to look ahead to, so both modes equal one block."""
    announce("stack L=1")
    cfg = wl.OPT30B_STACK48.scaled(512, 1024, 64)
    layers = _layers(cfg, 1)
    X = wl.make_tokens(cfg, 2)
    a = _run(layers, X, cfg, lookahead=False)[0]
    b = _run(layers, X, cfg, lookahead=True)[0]
    assert torch.equal(a, b)


def test_stack_full_size_opt30b_shape_lookahead():
    """Three blocks of the OPT-30B FFN shape (d 7168, f 28672, r 512, top-k 5734), batch 1,
    look-ahead: bitwise replay of all three, oracle check of the last one."""
    announce("stack full size")
    cfg = wl.OPT30B_STACK48
    layers = _layers(cfg, 3)
    X = wl.make_tokens(cfg, 1, device=DEV)
    xL, x_log, xhat_log, idx_log, count_log = _run(layers, X, cfg, lookahead=True)
    _replay(layers, cfg, X, x_log, xhat_log, idx_log, count_log, xL, lookahead=True)
    l = 2
    o = dict(W1=to_orc(layers[l].W1), b1=to_orc(layers[l].b1), W2T=to_orc(layers[l].W2T))
    _check_xhat(x_log[l, 0].cpu().numpy(), xhat_log[l, 0], cfg.dtype, True)
    _, y_ref = orc.sparse_ffn(to_orc(xhat_log[l, 0]), o["W1"], o["b1"], None, o["W2T"],
                              idx_log[l, 0].cpu().numpy(), orc.RELU, orc.F16)
    y_gpu = torch.from_numpy(xL[0].cpu().double().numpy() - x_log[l, 0].cpu().double().numpy())
    assert_ffn_close(y_gpu, y_ref, cfg.dtype, "full-size layer 2")


@pytest.mark.parametrize("lookahead", [False, True], ids=["sync", "lookahead"])
def test_stack_full_size_graph_replay_matches_eager(lookahead):
    """The captured-graph form at the OPT-30B FFN shape (d 7168, f 28672, r 512, top-k 5734),
    three blocks, batch 1 -- the launch configuration the benchmark times -- gives the eager bits
    on every replay."""
    announce(f"stack full size graph lookahead={lookahead}")
    cfg = wl.OPT30B_STACK48
    layers = _layers(cfg, 3)
    X = wl.make_tokens(cfg, 2).float().to(DEV)
    side = torch.cuda.Stream(device=DEV)
    ws = torch.empty(csf.workspace_size(8, 1, cfg.d, cfg.f, cfg.r, cfg.k, csf.F16), dtype=torch.uint8,
                     device=DEV)
    ref = []
    for t in range(2):
        x = X[t:t + 1].clone()
        csf.stack_forward(x, layers, k=cfg.k, lookahead=lookahead, side_stream=side, ws=ws)
        torch.cuda.synchronize()
        ref.append(x)
    assert not torch.equal(ref[0], ref[1])
    xg = torch.empty(1, cfg.d, dtype=torch.float32, device=DEV)
    for rep in range(3):
        for t in range(2):
            xg.copy_(X[t:t + 1])
            csf.stack_forward(xg, layers, k=cfg.k, lookahead=lookahead, side_stream=side, ws=ws,
                              graph=True)
            torch.cuda.synchronize()
            assert torch.equal(xg, ref[t]), (rep, t)


@pytest.mark.parametrize("lookahead", [False, True], ids=["sync", "lookahead"])
def test_stack_graph_replay_matches_eager(lookahead):
    """The captured-graph form gives the eager bits on every replay, with eager work (another
    stack call on other buffers) between the replays, and recaptures when an argument changes."""
    announce(f"stack graph lookahead={lookahead}")
    cfg = wl.OPT30B_STACK48.scaled(1024, 2048, 128)
    layers = _layers(cfg, 5)
    X = wl.make_tokens(cfg, 4).float().to(DEV)
    side = torch.cuda.Stream(device=DEV)
    ws = torch.empty(csf.workspace_size(8, 1, cfg.d, cfg.f, cfg.r, cfg.k, csf.F16), dtype=torch.uint8,
                     device=DEV)
    ws2 = torch.empty_like(ws)

    def eager(x0, w):
        x = x0.clone()
        csf.stack_forward(x, layers, k=cfg.k, lookahead=lookahead, side_stream=side, ws=w)
        torch.cuda.synchronize()
        return x

    ref = [eager(X[t:t + 1], ws) for t in range(4)]
    xg = torch.empty(1, cfg.d, dtype=torch.float32, device=DEV)
    for rep in range(3):
        for t in range(4):
            xg.copy_(X[t:t + 1])
            csf.stack_forward(xg, layers, k=cfg.k, lookahead=lookahead, side_stream=side, ws=ws,
                              graph=True)
            torch.cuda.synchronize()
            assert torch.equal(xg, ref[t]), (rep, t)
            other = eager(X[(t + 1) % 4:(t + 1) % 4 + 1], ws2)       # eager work in between
            assert torch.equal(other, ref[(t + 1) % 4])
    # a different output buffer is a different graph
    xh = torch.empty_like(xg)
    xh.copy_(X[2:3])
    csf.stack_forward(xh, layers, k=cfg.k, lookahead=lookahead, side_stream=side, ws=ws, graph=True)
    torch.cuda.synchronize()
    assert torch.equal(xh, ref[2])


def test_stack_layers_packed_once_give_the_same_bits():
    """StackLayers checks and packs the blocks once; stack_forward over it gives the bits of the
    list form, and refuses blocks checked for another activation or made for another d."""
    announce("stack StackLayers")
    cfg = wl.OPT30B_STACK48.scaled(1024, 2048, 128)
    layers = _layers(cfg, 4)
    X = wl.make_tokens(cfg, 1).float().to(DEV)
    side = torch.cuda.Stream(device=DEV)
    blocks = csf.StackLayers(layers)
    assert len(blocks) == 4
    for lookahead in (False, True):
        a = X.clone()
        b = X.clone()
        csf.stack_forward(a, layers, k=cfg.k, lookahead=lookahead, side_stream=side)
        csf.stack_forward(b, blocks, k=cfg.k, lookahead=lookahead, side_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(a, b), lookahead
    with pytest.raises(ValueError):
        csf.stack_forward(X.clone(), blocks, k=cfg.k, act=csf.SILU)
    with pytest.raises(ValueError):
        csf.stack_forward(torch.zeros(1, 512, dtype=torch.float32, device=DEV), blocks, k=cfg.k)

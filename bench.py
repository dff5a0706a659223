#!/usr/bin/env python3
"""Benchmark of the contextual-sparsity FFN step on one MI355X.

Workload: the OPT-175B FFN shape at batch 1 (d = 12288, f = 49152, predictor rank 1024, float16
weights with float32 accumulation, top-k = 2458 = 5% of f).  One step is one call of
csf_sparse_ffn_layer for one token: predictor, top-k selection and the gathered FFN.  Steps
rotate over several independently seeded layer instances (so the touched set is not served
from the 256 MB last-level cache) and over seeded tokens.

Printed: one JSON line.  `value` is the achieved bandwidth in GB/s on the bytes one step must
touch (V + U + the active rows of W1 and W2T + x), the metric's bandwidth form; the same line
gives microseconds per layer, the per-kernel times, the roofline of the dominant kernel, the
speed-up over the library's dense FFN, predictor recall/precision against the true active set,
and the CPU oracle's rate on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--no-cpu]
"""
import argparse
import ctypes
import functools
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-FFN µs/layer + HBM GB/s on touched bytes, batch 1, OPT-175B shape @5%"
PEAK_HBM_GBS = 8000.0
FFN_SEPARATE = ["gather_up", "gather_down", "reduce_partials"]


def layer_kernels(f, k, skip=False):
    """Kernels of csf_sparse_ffn_layer for one token: top-k over 20000 or more scores runs as
    two kernels (histogram, then classify, rank and emit), a smaller one as one, and up to 1024
    scores are selected inside the predictor's up-projection kernel.  The gathered FFN is one
    kernel (up rows, down rows and the reduction handed over inside it), or three with the
    post-gate skip."""
    ffn = FFN_SEPARATE if skip else ["ffn_fused"]
    if k is not None and k > 0 and f >= 20000:
        return ["pred_down", "pred_up", "select_hist", "select_finish"] + ffn
    if f <= 1024:     # scores and selection in one kernel
        return ["pred_down", "pred_up_select"] + ffn
    return ["pred_down", "pred_up", "select_topk" if k is not None else "select_threshold"] + ffn


KERNELS = layer_kernels(49152, 2458)


def _entry(name):
    """A C entry point with the default handle of the current device bound as its first
    argument (every step of the path runs in the library; this only marshals)."""
    from contextual_sparsity_ffn_amd import _lib
    return functools.partial(getattr(_lib.lib, name), _lib.context().handle)


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer instances rotated")
    ap.add_argument("--tokens", type=int, default=256)
    ap.add_argument("--trace-steps", type=int, default=400)
    ap.add_argument("--quality-tokens", type=int, default=32)
    ap.add_argument("--dense-steps", type=int, default=64)
    ap.add_argument("--cpu-tokens", type=int, default=12,
                    help="tokens of the single-thread oracle leg")
    ap.add_argument("--cpu-tokens-mt", type=int, default=64,
                    help="tokens of the multi-thread oracle leg")
    ap.add_argument("--no-hash", action="store_true",
                    help="skip the SHA-256 of the headline workload's tensors")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the HBM bandwidth probe (context for the metric)")
    ap.add_argument("--batched-steps", type=int, default=256,
                    help="steps per (batch size, path) of the OPT-30B-shape batched leg (0: skip)")
    ap.add_argument("--batched-layers", type=int, default=4)
    ap.add_argument("--batched-sizes", default="1,4,8,16,32",
                    help="comma-separated batch sizes of the batched leg")
    ap.add_argument("--zero-skip-steps", type=int, default=500,
                    help="steps of the post-gate zero-skip legs (0: skip them)")
    ap.add_argument("--silu-steps", type=int, default=300,
                    help="timed steps per variant of the SwiGLU functional-sparsity leg (0 = skip)")
    ap.add_argument("--attn-steps", type=int, default=200,
                    help="timed steps per variant of the attention-head sparsity leg (0 = skip)")
    ap.add_argument("--locality-steps", type=int, default=400,
                    help="steps of the hot-block (static locality) leg (0: skip it)")
    ap.add_argument("--stack-tokens", type=int, default=128,
                    help="tokens timed through the 48-layer OPT-30B-shape stack (0: skip)")
    ap.add_argument("--stack-layers", type=int, default=48)
    ap.add_argument("--stack-quality-tokens", type=int, default=32)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (to scale HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU path only: the library has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib, workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = wl.OPT175B
    d, f, r, k = cfg.d, cfg.f, cfg.r, cfg.k
    code = _lib.dtype_code(cfg.dtype)
    log(f"building {args.layers} layer instances of d={d} f={f} r={r} ({cfg.dtype})")
    layers = [wl.make_layer(cfg, device=dev, layer=l) for l in range(args.layers)]
    X = wl.make_tokens(cfg, args.tokens, device=dev)
    torch.cuda.synchronize()

    ws_bytes = csf.workspace_size(_lib.OP_LAYER, 1, d, f, r, k, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty(d, dtype=torch.float32, device=dev)
    scores = torch.empty(f, dtype=torch.float32, device=dev)
    idx = torch.empty(k, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    vp = ctypes.c_void_p

    def call_args(l, t, y_out=y, scores_out=None, idx_out=None):
        L = layers[l]
        return (vp(X[t].data_ptr()), d, f, r, cfg.act, code, vp(L.V.data_ptr()),
                vp(L.U.data_ptr()), vp(L.W1.data_ptr()), vp(L.b1.data_ptr()), None,
                vp(L.W2T.data_ptr()), k, ctypes.c_float(0.0), vp(y_out.data_ptr()),
                None if scores_out is None else vp(scores_out.data_ptr()),
                None if idx_out is None else vp(idx_out.data_ptr()), None,
                vp(ws.data_ptr()), ws_bytes, vp(stream.cuda_stream))

    plan = [call_args(s % args.layers, (s * 7) % args.tokens) for s in range(args.layers * args.tokens)]
    fn = _entry("csf_sparse_ffn_layer")

    def run(n, offset=0):
        for s in range(n):
            rc = fn(*plan[(offset + s) % len(plan)])
            if rc:
                raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())

    log(f"warmup {args.warmup} steps")
    run(args.warmup)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    run(args.steps, offset=args.warmup)
    e1.record(stream)
    enqueue = time.perf_counter() - wall0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    us_layer = ms_per_step * 1e3
    touched = wl.touched_bytes(cfg, k)
    value = touched / (ms_per_step * 1e-3) / 1e9
    log(f"{us_layer:.2f} us/layer, {value:.1f} GB/s on touched bytes (wall {wall:.3f}s, "
        f"host enqueue {enqueue / args.steps * 1e6:.1f} us/step)")

    # ---- per-step distribution: each of 256 steps bracketed by its own events ---------------
    nd = min(256, len(plan))
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nd)]
    for s_i in range(nd):
        sev[s_i][0].record(stream)
        rc = fn(*plan[(args.warmup + args.steps + s_i) % len(plan)])
        if rc:
            raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
        sev[s_i][1].record(stream)
    torch.cuda.synchronize()
    st_us = sorted(a.elapsed_time(b) * 1e3 for a, b in sev)
    step_dist = {"steps": nd, "p10_us": round(st_us[nd // 10], 3), "median_us": round(st_us[nd // 2], 3),
                 "p90_us": round(st_us[(9 * nd) // 10], 3)}

    # ---- per-kernel times from the library's trace hook (a separate pass) -------------------
    log(f"timing each kernel over {args.trace_steps} steps")
    nev = 2 * len(KERNELS)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.trace_steps)]
    for row in evs:                      # torch creates the HIP event on first record
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for s in range(args.trace_steps):
        csf.set_trace_events(evs[s])
        rc = fn(*plan[(args.warmup + args.steps + s) % len(plan)])
        if rc:
            raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
    csf.set_trace_events([])
    torch.cuda.synchronize()
    per_kernel = {}
    for i, name in enumerate(KERNELS):
        # the runtime records these at the kernel's own start and end
        ts = sorted(evs[s][2 * i].elapsed_time(evs[s][2 * i + 1]) * 1e3 for s in range(args.trace_steps))
        per_kernel[name] = {"avg_us": sum(ts) / len(ts), "p50_us": ts[len(ts) // 2]}
    es = 2  # float16
    kernel_bytes = {
        "pred_down": r * d * es + d * es + r * 4,
        "pred_up": f * r * es + r * 4 + f * 4,
        "select_hist": f * 4,
        "select_finish": f * 4 + k * 4,
        "ffn_fused": 2 * k * d * es + d * es + k * 4 + d * 4,
    }
    dom = max(KERNELS, key=lambda n: per_kernel[n]["avg_us"])
    dom_gbs = kernel_bytes[dom] / (per_kernel[dom]["avg_us"] * 1e-6) / 1e9
    # measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated), valid only
    # while the kernel sources are the ones the counters were taken from
    from contextual_sparsity_ffn_amd import profiling
    counters = profiling.load_counters(os.path.join(ROOT, "profiles", "layer_opt175b_hbm_counters.json"))
    traffic = None
    if counters and dom in counters["kernels"]:
        kc = counters["kernels"][dom]
        traffic = int(round(kc["fetch_bytes"] + kc["write_bytes"]))
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": kernel_bytes[dom],
                "avg_launch_us": round(per_kernel[dom]["avg_us"], 3)}
    for n in KERNELS:
        b = kernel_bytes[n]
        per_kernel[n]["GBps"] = round(b / (per_kernel[n]["avg_us"] * 1e-6) / 1e9, 1) if b else None
        per_kernel[n]["avg_us"] = round(per_kernel[n]["avg_us"], 3)
        per_kernel[n]["p50_us"] = round(per_kernel[n]["p50_us"], 3)

    # ---- dense FFN over the same layers ----------------------------------------------------
    log(f"dense FFN {args.dense_steps} steps")
    dws_bytes = csf.workspace_size(_lib.OP_DENSE_FFN, 1, d, f, 0, f, code)
    dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)
    hd = torch.empty(f, dtype=torch.float32, device=dev)
    dfn = _entry("csf_dense_ffn")

    def dense_call(l, t, h_out=None):
        L = layers[l]
        return dfn(vp(X[t].data_ptr()), 1, d, f, cfg.act, code, vp(L.W1.data_ptr()),
                   vp(L.b1.data_ptr()), None, vp(L.W2T.data_ptr()),
                   None if h_out is None else vp(h_out.data_ptr()), vp(y.data_ptr()),
                   vp(dws.data_ptr()), dws_bytes, vp(stream.cuda_stream))

    dense_us = None
    if args.dense_steps > 0:
        for s in range(4):
            dense_call(s % args.layers, s)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(args.dense_steps):
            dense_call(s % args.layers, s % args.tokens)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_us = e0.elapsed_time(e1) * 1e3 / args.dense_steps

    # ---- predictor quality: recall / precision against the true active set -------------------
    log(f"quality on {args.quality_tokens} tokens")
    rec, prec_list, tfrac = [], [], []
    for t in range(args.quality_tokens):
        l = t % args.layers
        rc = fn(*call_args(l, t, scores_out=scores, idx_out=idx))
        if rc:
            raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
        dense_call(l, t, h_out=hd)
        torch.cuda.synchronize()
        true = torch.nonzero(hd != 0).flatten()
        pred = idx.long()
        hit = torch.isin(pred, true).sum().item()
        nt = true.numel()
        rec.append(hit / nt if nt else 1.0)
        prec_list.append(hit / k if k else 1.0)
        tfrac.append(nt / f)

    prec = sum(prec_list) / len(prec_list) if prec_list else None

    # ---- optional plain copy for counter calibration -----------------------------------------
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ---- provenance: seeds and digests of the headline workload's tensors ---------------------
    seeds = {"rule": "seed(config, role, layer) = 1000000 config + 1000 role + layer; each tensor "
                     "drawn from its own torch.Generator on the GPU, float32, rounded once",
             "headline": {"config": cfg.index,
                          "roles": {"U": wl.ROLE_U, "V": wl.ROLE_V, "W1_noise": wl.ROLE_W1_NOISE,
                                    "W2T": wl.ROLE_W2T, "tokens": wl.ROLE_TOKENS,
                                    "bias_calibration": wl.ROLE_CALIB},
                          "layers": list(range(args.layers))},
             "other_legs": {name: c.index for name, c in (
                 ("zero_skip_gated", wl.LLAMA_REGLU), ("silu_functional", wl.LLAMA_SWIGLU),
                 ("batched_union", wl.OPT30B), ("static_locality", wl.OPT30B),
                 ("attention_heads", wl.ATTN_OPT175B), ("stack", wl.OPT30B_STACK48))}}
    digests = None
    if not args.no_hash:
        log("SHA-256 of the headline tensors")
        named = [("X", X)]
        for l, L in enumerate(layers):
            named += [(f"layer{l}.{n}", t) for n, t in (("V", L.V), ("U", L.U), ("W1", L.W1),
                                                        ("b1", L.b1), ("W2T", L.W2T))]
        digests = tensor_sha256(named)

    # ---- post-gate zero-skip on the same plan (an option, not the metric) ---------------------
    zero_skip = None
    if args.zero_skip_steps > 0:
        zero_skip = {"opt175b_layer": zero_skip_same_plan(args, fn, plan, stream, us_layer, prec,
                                                          cfg, k)}
        zero_skip["llama_reglu_layer"] = zero_skip_gated_leg(args, dev)

    silu = None
    if args.silu_steps > 0:
        silu = silu_functional_leg(args, dev)

    attn = None
    if args.attn_steps > 0:
        attn = attention_leg(args, dev)

    # ---- batched union leg (OPT-30B shape) --------------------------------------------------
    batched = None
    locality_res = None
    layer0 = layers[0]          # kept for the CPU baseline
    if args.batched_steps > 0 or args.locality_steps > 0:
        del layers
        torch.cuda.empty_cache()
    if args.locality_steps > 0:
        locality_res = static_locality_leg(args, dev)
    if args.batched_steps > 0:
        torch.cuda.empty_cache()
        batched = batched_union_leg(args, dev)

    stack = None
    if args.stack_tokens > 0:
        torch.cuda.empty_cache()
        stack = stack_leg(args, dev)

    probe = None if args.no_probe else bandwidth_probe(dev)

    # ---- CPU oracle baseline (rank 0, bounded sample) ----------------------------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, layer0, X, args.cpu_tokens, args.cpu_tokens_mt, touched)


    dense_b = wl.dense_bytes(cfg)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "OPT-175B-shape sparse FFN layer, batch 1: predict + top-k + gathered FFN",
                   "d": d, "f": f, "r": r, "k": k, "batch": 1, "act": "relu",
                   "weights": "float16, float32 accumulation", "layers_rotated": args.layers,
                   "tokens": args.tokens, "parallelism": "single GPU"},
        "us_per_layer": round(us_layer, 3),
        "us_per_step_distribution": step_dist,
        "bandwidth_probe": probe,
        "frac_of_dense_stream": round(value / (dense_b / (dense_us * 1e-6) / 1e9), 4) if dense_us else None,
        "host_enqueue_us_per_step": round(enqueue / args.steps * 1e6, 2),
        "tokens_per_s_per_layer": round(1e6 / us_layer, 1),
        "touched_bytes": touched,
        "frac_of_peak_hbm": round(value / PEAK_HBM_GBS, 4),
        "roofline": roofline,
        "kernels": per_kernel,
        "dense_us_per_layer": round(dense_us, 3) if dense_us else None,
        "dense_GBps": round(dense_b / (dense_us * 1e-6) / 1e9, 1) if dense_us else None,
        "speedup_vs_dense": round(dense_us / us_layer, 3) if dense_us else None,
        "speedup_bound_bytes": round(dense_b / touched, 3),
        "speedup_bound_active_frac": round(f / k, 3),
        "recall": round(sum(rec) / len(rec), 4) if rec else None,
        "precision": round(prec, 4) if prec is not None else None,
        "true_frac": round(sum(tfrac) / len(tfrac), 4) if tfrac else None,
        "pred_frac": round(k / f, 4),
        "cpu_baseline": cpu,
        "seeds": seeds,
        "tensor_sha256": digests,
        "zero_skip": zero_skip,
        "silu_functional": silu,
        "attention_heads": attn,
        "static_locality": locality_res,
        "batched_union": batched,
        "stack": stack,
    }
    print(json.dumps(out), flush=True)


PEAK_MFMA_F16_TFLOPS = 2500.0
UNION_KERNELS = ["union_list", "union_up", "union_down", "reduce_partials"]


def predictor_kernels(B, dtype_code, d, r):
    """Kernels the library's predictor launches for B tokens: the matrix-core form for batches of
    4 or more 16-bit tokens with d and r multiples of 128, else the vector-ALU pair."""
    if B >= 4 and dtype_code != 0 and d % 128 == 0 and r % 128 == 0:
        return ["pred_down", "pred_hidden", "pred_up"]
    return ["pred_down", "pred_up"]


def zero_skip_same_plan(args, fn, plan, stream, us_plain, prec, cfg, k):
    """The headline step with CSF_FFN_SKIP_ZERO_H: rows whose h is 0 (the predictor's false
    positives) skip their down row.  Bytes actually needed: V + U + k W1 rows + (precision k) W2T
    rows + x."""
    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib

    n = args.zero_skip_steps
    csf.set_ffn_flags(csf.FFN_SKIP_ZERO_H)
    try:
        for s in range(20):
            fn(*plan[s % len(plan)])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(n):
            rc = fn(*plan[(7 + s) % len(plan)])
            if rc:
                raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
        e1.record(stream)
        torch.cuda.synchronize()
    finally:
        csf.set_ffn_flags(0)
    us = e0.elapsed_time(e1) * 1e3 / n
    es = 2
    live = prec * k if prec is not None else None
    need = None
    if live is not None:
        need = (cfg.r * cfg.d + cfg.f * cfg.r + k * cfg.d + cfg.d) * es + live * cfg.d * es
    log(f"zero-skip OPT-175B layer: {us:.2f} us (plain {us_plain:.2f} us)")
    return {"us_per_layer": round(us, 3), "plain_us_per_layer": round(us_plain, 3),
            "speedup": round(us_plain / us, 4),
            "down_rows_read_per_token": round(live, 1) if live is not None else None,
            "bytes_needed": int(need) if need else None,
            "GBps_on_bytes_needed": round(need / (us * 1e-6) / 1e9, 1) if need else None}


def zero_skip_gated_leg(args, dev):
    """LLaMA-class gated layer (d 4096, f 14336, r 256, bfloat16, ReGLU, sigmoid >= 0.5): the
    recall-first predictor marks about half the neurons, a tenth fire.  Plain vs zero-skip (gate
    rows always; up and down rows only for positive gates)."""
    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib, workloads as wl

    cfg = wl.LLAMA_REGLU
    d, f, r = cfg.d, cfg.f, cfg.r
    code = _lib.dtype_code(cfg.dtype)
    nl = 8
    layers = [wl.make_layer(cfg, device=dev, layer=l) for l in range(nl)]
    X = wl.make_tokens(cfg, 64, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws_b = csf.workspace_size(_lib.OP_LAYER, 1, d, f, r, f, code)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    y = torch.empty(d, dtype=torch.float32, device=dev)
    idx = torch.empty(f, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    hd = torch.empty(f, dtype=torch.float32, device=dev)
    vp = ctypes.c_void_p
    fn = _entry("csf_sparse_ffn_layer")

    def call(l, t, idx_out=None, cnt_out=None):
        L = layers[l]
        return fn(vp(X[t].data_ptr()), d, f, r, cfg.act, code, vp(L.V.data_ptr()), vp(L.U.data_ptr()),
                  vp(L.W1.data_ptr()), vp(L.b1.data_ptr()), vp(L.Wup.data_ptr()), vp(L.W2T.data_ptr()),
                  -1, ctypes.c_float(cfg.tau), vp(y.data_ptr()), None,
                  None if idx_out is None else vp(idx_out.data_ptr()),
                  None if cnt_out is None else vp(cnt_out.data_ptr()), vp(ws.data_ptr()), ws_b,
                  vp(stream.cuda_stream))

    # predicted and live (positive-gate) counts over a sample of (layer, token) pairs; the true
    # set of a token is its positive-gate neurons (ReGLU h != 0 iff gate > 0 and up != 0), read
    # from the library's dense FFN; the scores give the sets of the other thresholds
    taus = (0.3, 0.4, 0.5, 0.6, 0.7, 0.8, 0.9)
    counts, lives, trues = [], [], []
    sweep = {tau: [0, 0, 0] for tau in taus}          # predicted, hits, true (summed)
    nq = 32
    for s in range(nq):
        l, t = s % nl, (5 * s) % 64
        call(l, t, idx, cnt)
        L = layers[l]
        csf.dense_ffn(X[t], L.W1, L.b1, L.Wup, L.W2T, act=cfg.act, h=hd)
        sc = csf.predict_active(X[t].reshape(1, -1), L.V, L.U)[0]
        torch.cuda.synchronize()
        n = int(cnt.item())
        true = hd != 0
        counts.append(n)
        lives.append(int(true[idx[:n].long()].sum()))
        trues.append(int(true.sum()))
        for tau in taus:
            sel = sc >= tau
            sweep[tau][0] += int(sel.sum())
            sweep[tau][1] += int((sel & true).sum())
            sweep[tau][2] += int(true.sum())
    count, live = sum(counts) / len(counts), sum(lives) / len(lives)
    ntrue = sum(trues) / len(trues)
    res = {"workload": "LLaMA-class gated layer, batch 1: d 4096, f 14336, r 256, bfloat16, ReGLU, "
                       "threshold sigmoid >= 0.5", "layers_rotated": nl,
           "predicted_mean": round(count, 1), "live_mean": round(live, 1),
           "quality": {"samples": nq, "recall": round(sum(lives) / max(sum(trues), 1), 4),
                       "precision": round(sum(lives) / max(sum(counts), 1), 4),
                       "true_frac": round(ntrue / f, 4), "pred_frac": round(count / f, 4),
                       "true_set": "neurons with a positive gate (h != 0) on the token's input"}}
    es = 2
    plain_bytes = (r * d + f * r + d) * es + count * 3 * d * es
    skip_bytes = (r * d + f * r + d) * es + count * d * es + live * 2 * d * es
    for mode, flags in (("plain", 0), ("zero_skip", csf.FFN_SKIP_ZERO_H)):
        csf.set_ffn_flags(flags)
        try:
            for s in range(20):
                call(s % nl, s % 64)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for s in range(args.zero_skip_steps):
                call(s % nl, (s * 7) % 64)
            e1.record(stream)
            torch.cuda.synchronize()
        finally:
            csf.set_ffn_flags(0)
        us = e0.elapsed_time(e1) * 1e3 / args.zero_skip_steps
        b = plain_bytes if mode == "plain" else skip_bytes
        res[mode] = {"us_per_layer": round(us, 3), "bytes_needed": int(b),
                     "GBps_on_bytes_needed": round(b / (us * 1e-6) / 1e9, 1)}
    res["speedup"] = round(res["plain"]["us_per_layer"] / res["zero_skip"]["us_per_layer"], 4)
    log(f"zero-skip gated layer: plain {res['plain']['us_per_layer']} us, skip "
        f"{res['zero_skip']['us_per_layer']} us (predicted {count:.0f}, live {live:.0f})")

    # threshold sweep on the predictor's own score scale: set size, recall, precision and the
    # plain layer's time at each tau (0.5 is the configured one)
    rows = []
    steps = max(50, args.zero_skip_steps // 4)
    for tau in taus:
        def call_tau(l, t):
            L = layers[l]
            return fn(vp(X[t].data_ptr()), d, f, r, cfg.act, code, vp(L.V.data_ptr()),
                      vp(L.U.data_ptr()), vp(L.W1.data_ptr()), vp(L.b1.data_ptr()),
                      vp(L.Wup.data_ptr()), vp(L.W2T.data_ptr()), -1, ctypes.c_float(tau),
                      vp(y.data_ptr()), None, None, None, vp(ws.data_ptr()), ws_b,
                      vp(stream.cuda_stream))
        for s in range(10):
            call_tau(s % nl, s % 64)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            call_tau(s % nl, (s * 7) % 64)
        e1.record(stream)
        torch.cuda.synchronize()
        npred, hits, ntr = sweep[tau]
        rows.append({"tau": tau, "pred_frac": round(npred / (nq * f), 4),
                     "recall": round(hits / max(ntr, 1), 4),
                     "precision": round(hits / max(npred, 1), 4),
                     "us_per_layer": round(e0.elapsed_time(e1) * 1e3 / steps, 3)})
    res["tau_sweep"] = {"samples": nq, "rows": rows,
                        "note": "sigmoid score >= tau over the same (layer, token) pairs as "
                                "quality; the layer timed without zero-skip"}
    log("tau sweep: " + ", ".join(f"{w['tau']}: frac {w['pred_frac']} rec {w['recall']} "
                                  f"prec {w['precision']} {w['us_per_layer']} us" for w in rows))
    del layers
    torch.cuda.empty_cache()
    return res


def silu_functional_leg(args, dev):
    """LLaMA-class SwiGLU layer (d 4096, f 14336, r 256, bfloat16, no bias, gate spread set for
    ~50% functional activity).  SiLU has no exact zeros, so every sparse variant approximates the
    dense layer; each is reported with its time and its relative L2 error against the library's
    dense SwiGLU FFN:
      topk_K        predictor top-K (the plain method) at K = 25%, 50%, 75% of f;
      topk_K+skip   the same list cut inside the FFN to |silu(gate)| > 0.1 (post-gate skip);
      functional    the dense FFN cut to |silu(gate)| > 0.1 (the functional set itself, no
                    predictor: the error floor of the 0.1 threshold);
      best_K        the K neurons of largest |h| (known only after the dense layer: the error
                    floor of any K-set).
    Recall and precision of the predicted set are against the functional set."""
    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib, workloads as wl

    cfg = wl.LLAMA_SWIGLU
    d, f, r = cfg.d, cfg.f, cfg.r
    code = _lib.dtype_code(cfg.dtype)
    gate_tau = 0.1
    nl, ntok, nq = 8, 64, 16
    layers = [wl.make_layer(cfg, device=dev, layer=l) for l in range(nl)]
    X = wl.make_tokens(cfg, ntok, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws_b = csf.workspace_size(_lib.OP_LAYER, 1, d, f, r, f, code)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    y = torch.empty(d, dtype=torch.float32, device=dev)
    vp = ctypes.c_void_p
    fn = _entry("csf_sparse_ffn_layer")
    ks = [f // 4, cfg.k, 3 * f // 4]

    def call(l, t, k, y_out=y, idx_out=None):
        L = layers[l]
        return fn(vp(X[t].data_ptr()), d, f, r, cfg.act, code, vp(L.V.data_ptr()),
                  vp(L.U.data_ptr()), vp(L.W1.data_ptr()), None, vp(L.Wup.data_ptr()),
                  vp(L.W2T.data_ptr()), k, ctypes.c_float(0.0), vp(y_out.data_ptr()), None,
                  None if idx_out is None else vp(idx_out.data_ptr()), None, vp(ws.data_ptr()),
                  ws_b, vp(stream.cuda_stream))

    def set_skip(on):
        csf.set_ffn_flags(csf.FFN_SKIP_ZERO_H if on else 0)
        csf.set_ffn_gate_threshold(gate_tau if on else 0.0)

    def timed(fn_step):
        for s in range(16):
            fn_step(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.silu_steps):
            fn_step(s)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.silu_steps

    # ---- quality over nq (layer, token) pairs -------------------------------------------------
    def rel(a, b):
        return float((a - b).norm() / b.norm())

    q = {f"topk_{k}": [] for k in ks}
    q.update({f"topk_{k}+skip": [] for k in ks})
    q.update({"functional": []})
    q.update({f"best_{k}": [] for k in ks})
    rec, prec, ffrac, live = [], [], [], {k: [] for k in ks}
    idx = torch.empty(f, dtype=torch.int32, device=dev)
    ys = torch.empty(d, dtype=torch.float32, device=dev)
    hd = torch.empty(1, f, dtype=torch.float32, device=dev)
    hg = torch.empty(1, f, dtype=torch.float32, device=dev)
    hk = torch.empty(1, f, dtype=torch.float32, device=dev)
    try:
        for s in range(nq):
            l, t = s % nl, (s * 5) % ntok
            L = layers[l]
            xt = X[t:t + 1]
            set_skip(False)
            yd = csf.dense_ffn(xt, L.W1, None, L.Wup, L.W2T, act=cfg.act, h=hd)[0].clone()
            # the gate activation silu(W1 x) alone: the ungated SiLU form over the same W1
            csf.dense_ffn(xt, L.W1, None, None, L.W2T, act=csf.SILU, h=hg)
            fset = torch.nonzero(hg[0].abs() > gate_tau).flatten()
            ffrac.append(fset.numel() / f)
            set_skip(True)
            yf = csf.dense_ffn(xt, L.W1, None, L.Wup, L.W2T, act=cfg.act)[0]
            q["functional"].append(rel(yf, yd))
            for k in ks:
                set_skip(False)
                rc = call(l, t, k, ys, idx)
                if rc:
                    raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
                torch.cuda.synchronize()
                q[f"topk_{k}"].append(rel(ys, yd))
                pred = idx[:k].long()
                if k == cfg.k:
                    hit = int(torch.isin(pred, fset).sum())
                    rec.append(hit / max(fset.numel(), 1))
                    prec.append(hit / k)
                set_skip(True)
                csf.sparse_ffn(xt, L.W1, None, L.Wup, L.W2T, idx[:k].unsqueeze(0), act=cfg.act,
                               h=hk[:, :k])
                rc = call(l, t, k, ys)
                if rc:
                    raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
                torch.cuda.synchronize()
                q[f"topk_{k}+skip"].append(rel(ys, yd))
                live[k].append(int((hk[0, :k] != 0).sum()))
                set_skip(False)
                best = torch.sort(torch.topk(hd[0].abs(), k).indices).values.int()
                yb = csf.sparse_ffn(xt, L.W1, None, L.Wup, L.W2T, best.unsqueeze(0), act=cfg.act)[0]
                torch.cuda.synchronize()
                q[f"best_{k}"].append(rel(yb, yd))
    finally:
        set_skip(False)

    mean = lambda v: sum(v) / len(v)
    es = 2
    pred_b = (r * d + f * r + d) * es
    res = {"workload": "LLaMA-class SwiGLU layer, batch 1: d 4096, f 14336, r 256, bfloat16, no "
                       "bias, std(W1 x) 0.3", "gate_tau": gate_tau, "layers_rotated": nl,
           "quality_pairs": nq, "functional_frac": round(mean(ffrac), 4),
           "recall_vs_functional": round(mean(rec), 4), "precision_vs_functional": round(mean(prec), 4),
           "rel_l2_err": {n: round(mean(v), 4) for n, v in q.items()}}

    # ---- timing ---------------------------------------------------------------------------------
    L0 = layers[0]
    dws_b = csf.workspace_size(_lib.OP_DENSE_FFN, 1, d, f, 0, f, code)
    dws = torch.empty(dws_b, dtype=torch.uint8, device=dev)
    dfn = _entry("csf_dense_ffn")

    def dense_step(s):
        L = layers[s % nl]
        rc = dfn(vp(X[(s * 7) % ntok].data_ptr()), 1, d, f, cfg.act, code, vp(L.W1.data_ptr()),
                 None, vp(L.Wup.data_ptr()), vp(L.W2T.data_ptr()), None, vp(y.data_ptr()),
                 vp(dws.data_ptr()), dws_b, vp(stream.cuda_stream))
        if rc:
            raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())

    us_dense = timed(dense_step)
    timing = {"dense": {"us_per_layer": round(us_dense, 3), "bytes": 3 * f * d * es}}
    try:
        for k in ks:
            for skip in (False, True):
                set_skip(skip)
                us = timed(lambda s: call(s % nl, (s * 7) % ntok, k))
                nb = pred_b + (k * d * es + mean(live[k]) * 2 * d * es if skip else k * 3 * d * es)
                timing[f"topk_{k}" + ("+skip" if skip else "")] = {
                    "us_per_layer": round(us, 3), "bytes_needed": int(nb),
                    "GBps_on_bytes_needed": round(nb / (us * 1e-6) / 1e9, 1),
                    "speedup_vs_dense": round(us_dense / us, 3)}
    finally:
        set_skip(False)
    # per-kernel times of the 50% layer, plain and with the skip (library trace hook)
    kern = {}
    try:
        for skip in (False, True):
            set_skip(skip)
            n = 50
            names = layer_kernels(f, cfg.k, skip)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(names))]
                   for _ in range(n)]
            for row in evs:
                for e in row:
                    e.record(stream)
            torch.cuda.synchronize()
            for s in range(n):
                csf.set_trace_events(evs[s])
                call(s % nl, (s * 7) % ntok, cfg.k)
            csf.set_trace_events([])
            torch.cuda.synchronize()
            kern["skip" if skip else "plain"] = {
                name: round(sum(evs[s][2 * i].elapsed_time(evs[s][2 * i + 1]) for s in range(n))
                            * 1e3 / n, 3) for i, name in enumerate(names)}
    finally:
        csf.set_trace_events([])
        set_skip(False)
    res["live_after_skip_mean"] = {str(k): round(mean(live[k]), 1) for k in ks}
    res["timing"] = timing
    res[f"kernels_avg_us_topk_{cfg.k}"] = kern
    log(f"SwiGLU functional: dense {us_dense:.1f} us; top-{cfg.k} "
        f"{timing[f'topk_{cfg.k}']['us_per_layer']} us err {res['rel_l2_err'][f'topk_{cfg.k}']}; "
        f"+skip {timing[f'topk_{cfg.k}+skip']['us_per_layer']} us err "
        f"{res['rel_l2_err'][f'topk_{cfg.k}+skip']}; functional-set err {res['rel_l2_err']['functional']}")
    del layers, L0
    torch.cuda.empty_cache()
    return res


ATTN_KERNELS = ["pred_down", "pred_up_select", "head_proj", "head_attn", "head_combine",
                "gather_down", "reduce_partials"]


def attention_leg(args, dev):
    """OPT-175B attention shape (d 12288, 96 heads of 128, 2048 cached tokens, f16): the head
    predictor + top-19 heads + the decode step over them, against the dense decode step (every
    head).  Each step appends the token's k, v to the computed heads' caches; the lengths are reset
    to the context before each timed variant.  Quality over 16 (layer, token) pairs: a head is
    active when its dense output has |o_h| > 0.1 (the silent heads sit at ~1e-3)."""
    import dataclasses
    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib, workloads as wl

    cfg = dataclasses.replace(wl.ATTN_OPT175B, extra=256)
    d, H, dh, r, k, T = cfg.d, cfg.H, cfg.dh, cfg.r, cfg.k, cfg.context
    code = _lib.dtype_code(cfg.dtype)
    nl, ntok = 4, 64
    steps = min(args.attn_steps, nl * (cfg.extra - 16))
    layers = [wl.make_attention_layer(cfg, device=dev, layer=l) for l in range(nl)]
    X = wl.make_attn_tokens(cfg, ntok, device=dev)
    lens0 = layers[0].lens.clone()
    stream = torch.cuda.current_stream(dev)
    vp = ctypes.c_void_p
    ws_b = csf.attention_workspace_size(_lib.OP_ATTN_LAYER, d, H, dh, r, cfg.Tmax, H, code)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    y = torch.empty(d, dtype=torch.float32, device=dev)
    heads = torch.empty(H, dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    lfn, dfn = _entry("csf_sparse_attention_layer"), _entry("csf_sparse_attention_decode")

    def reset():
        for L in layers:
            L.lens.copy_(lens0)

    def sparse_step(s, y_out=y, heads_out=None, count_out=None):
        L = layers[s % nl]
        rc = lfn(vp(X[(s * 7) % ntok].data_ptr()), d, H, dh, r, code, vp(L.Vp.data_ptr()),
                 vp(L.Up.data_ptr()), vp(L.Wq.data_ptr()), vp(L.Wk.data_ptr()), vp(L.Wv.data_ptr()),
                 vp(L.bq.data_ptr()), None, None, vp(L.WoT.data_ptr()), vp(L.Kc.data_ptr()),
                 vp(L.Vc.data_ptr()), cfg.Tmax, vp(L.lens.data_ptr()), k, ctypes.c_float(0.0), 0,
                 None, None if heads_out is None else vp(heads_out.data_ptr()),
                 None if count_out is None else vp(count_out.data_ptr()), None,
                 vp(y_out.data_ptr()), vp(ws.data_ptr()), ws_b, vp(stream.cuda_stream))
        if rc:
            raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())

    def dense_step(s, y_out=y, o_out=None):
        L = layers[s % nl]
        rc = dfn(vp(X[(s * 7) % ntok].data_ptr()), d, H, dh, code, vp(L.Wq.data_ptr()),
                 vp(L.Wk.data_ptr()), vp(L.Wv.data_ptr()), vp(L.bq.data_ptr()), None, None,
                 vp(L.WoT.data_ptr()), vp(L.Kc.data_ptr()), vp(L.Vc.data_ptr()), cfg.Tmax,
                 vp(L.lens.data_ptr()), None, None, H, 0,
                 None if o_out is None else vp(o_out.data_ptr()), vp(y_out.data_ptr()),
                 vp(ws.data_ptr()), ws_b, vp(stream.cuda_stream))
        if rc:
            raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())

    def timed(step):
        reset()
        for s in range(8):
            step(s)
        reset()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            step(s)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    us_sparse = timed(sparse_step)
    us_dense = timed(dense_step)

    # per-kernel times of the sparse layer (its seven kernels)
    reset()
    n = 40
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(16)] for _ in range(n)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for s in range(n):
        csf.set_trace_events(evs[s])
        sparse_step(s)
    csf.set_trace_events([])
    torch.cuda.synchronize()
    kern = {name: round(sum(evs[s][2 * i].elapsed_time(evs[s][2 * i + 1]) for s in range(n))
                        * 1e3 / n, 3) for i, name in enumerate(ATTN_KERNELS)}

    # quality: predicted heads against the heads the dense step finds active
    reset()
    o = torch.empty(H, dh, dtype=torch.float32, device=dev)
    yd = torch.empty(d, dtype=torch.float32, device=dev)
    ys = torch.empty(d, dtype=torch.float32, device=dev)
    yb = torch.empty(d, dtype=torch.float32, device=dev)
    rec, prec, act, err, err_best, err_act = [], [], [], [], [], []
    for q in range(16):
        L = layers[q % nl]
        xq = X[(q * 7) % ntok]
        reset()
        dense_step(q, y_out=yd, o_out=o)
        reset()
        sparse_step(q, y_out=ys, heads_out=heads, count_out=count)
        torch.cuda.synchronize()
        norms = o.norm(dim=1)
        active = torch.nonzero(norms > 0.1).flatten()
        pred = heads[:k].long()
        hit = int(torch.isin(pred, active).sum())
        rec.append(hit / max(active.numel(), 1))
        prec.append(hit / k)
        act.append(active.numel() / H)
        err.append(float((ys - yd).norm() / yd.norm()))
        for sel, acc in ((torch.sort(torch.topk(norms, k).indices).values, err_best),
                         (active, err_act)):
            reset()
            csf.sparse_attention_decode(xq, L.Wq, L.Wk, L.Wv, L.bq, None, None, L.WoT, L.Kc, L.Vc,
                                        L.lens, heads=sel.int().contiguous(), y=yb)
            torch.cuda.synchronize()
            acc.append(float((yb - yd).norm() / yd.norm()))
    reset()
    mean = lambda v: sum(v) / len(v)
    touched = wl.attn_touched_bytes(cfg, k, T)
    es = 2
    dense_b = 4 * H * dh * d * es + 2 * H * (T + 1) * dh * es + d * es
    res = {"workload": "OPT-175B attention decode step, batch 1: d 12288, 96 heads x 128, 2048 "
                       "cached tokens, float16, predictor rank 256, top-19 heads",
           "layers_rotated": nl, "steps": steps, "k_heads": k,
           "us_per_step": round(us_sparse, 3), "touched_bytes": touched,
           "GBps_on_touched": round(touched / (us_sparse * 1e-6) / 1e9, 1),
           "dense_us_per_step": round(us_dense, 3), "dense_bytes": dense_b,
           "dense_GBps": round(dense_b / (us_dense * 1e-6) / 1e9, 1),
           "speedup_vs_dense": round(us_dense / us_sparse, 3),
           "speedup_bound_bytes": round(dense_b / touched, 3),
           "active_frac": round(mean(act), 4), "recall_vs_active": round(mean(rec), 4),
           "precision_vs_active": round(mean(prec), 4),
           "rel_l2_err": {"predicted_top19": round(mean(err), 4),
                          "best_19_by_norm": round(mean(err_best), 4),
                          "active_set": round(mean(err_act), 4)},
           "kernels_avg_us": kern}
    log(f"attention heads: sparse {us_sparse:.1f} us, dense {us_dense:.1f} us, "
        f"recall {res['recall_vs_active']}, err {res['rel_l2_err']['predicted_top19']}")
    del layers
    torch.cuda.empty_cache()
    return res


def static_locality_leg(args, dev):
    """OPT-30B FFN shape with power-law firing (a few neurons fire for almost every token; the
    bias-free predictor cannot see it): the plain layer (top-k 5734 over all neurons) against the
    hot-first layer (profiled on 256 separately seeded tokens, reordered, neurons firing for at
    least half of them always computed, the rest of the same 5734 budget chosen by the predictor
    over the cold rows).  Time, recall of the true active set and predictor bytes for each."""
    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib, locality, workloads as wl

    cfg = wl.OPT30B
    d, f, r, k = cfg.d, cfg.f, cfg.r, cfg.k
    nl = 4
    log(f"static-locality leg: {nl} power-law layers of d={d} f={f}")
    plain, prepared = [], []
    for l in range(nl):
        L = wl.make_powerlaw_layer(cfg, device=dev, layer=l)
        freq = locality.firing_frequency(L, wl.make_profile_tokens(cfg, 256, device=dev))
        H = locality.reorder(L, locality.hot_first_order(freq))
        hot = locality.hot_count(freq, 0.5, cap=k // 2)
        plain.append(L)
        prepared.append((H, hot, H.U[hot:].contiguous()))
    X = wl.make_tokens(cfg, 64, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = _lib.dtype_code(cfg.dtype)
    ws_b = csf.workspace_size(_lib.OP_LAYER, 1, d, f, r, k, code)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    y = torch.empty(d, dtype=torch.float32, device=dev)
    idx = torch.empty(f, dtype=torch.int32, device=dev)
    H_all = torch.empty(1, f, dtype=torch.float32, device=dev)
    vp = ctypes.c_void_p
    fplain, fhot = _entry("csf_sparse_ffn_layer"), _entry("csf_sparse_ffn_layer_hot")

    def call_plain(l, t, idx_out=None):
        L = plain[l]
        return fplain(vp(X[t].data_ptr()), d, f, r, cfg.act, code, vp(L.V.data_ptr()),
                      vp(L.U.data_ptr()), vp(L.W1.data_ptr()), vp(L.b1.data_ptr()), None,
                      vp(L.W2T.data_ptr()), k, ctypes.c_float(0.0), vp(y.data_ptr()), None,
                      None if idx_out is None else vp(idx_out.data_ptr()), None, vp(ws.data_ptr()),
                      ws_b, vp(stream.cuda_stream))

    def call_hot(l, t, idx_out=None):
        H, hot, Uc = prepared[l]
        return fhot(vp(X[t].data_ptr()), d, f, r, cfg.act, code, vp(H.V.data_ptr()),
                    vp(Uc.data_ptr()), vp(H.W1.data_ptr()), vp(H.b1.data_ptr()), None,
                    vp(H.W2T.data_ptr()), hot, k - hot, ctypes.c_float(0.0), vp(y.data_ptr()), None,
                    None if idx_out is None else vp(idx_out.data_ptr()), None, vp(ws.data_ptr()),
                    ws_b, vp(stream.cuda_stream))

    hots = [p[1] for p in prepared]
    res = {"workload": "OPT-30B-shape layer with power-law firing (alpha 2, mean 0.2), batch 1, "
                       "active budget 5734", "layers_rotated": nl, "hot_per_layer": hots}
    for name, call, layers_of in (("plain", call_plain, lambda l: plain[l]),
                                  ("hot_block", call_hot, lambda l: prepared[l][0])):
        rec = []
        for t in range(16):
            l = t % nl
            rc = call(l, t, idx)
            if rc:
                raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
            Lq = layers_of(l)
            csf.dense_ffn(X[t:t + 1], Lq.W1, Lq.b1, None, Lq.W2T, h=H_all)
            torch.cuda.synchronize()
            true = H_all[0] > 0
            nt = int(true.sum())
            rec.append(int(true[idx[:k].long()].sum()) / nt if nt else 1.0)
        for s in range(20):
            call(s % nl, s % 64)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.locality_steps):
            call(s % nl, (s * 7) % 64)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.locality_steps
        hot_mean = sum(hots) / len(hots) if name == "hot_block" else 0
        pred_bytes = 2 * (r * d + (f - hot_mean) * r)
        res[name] = {"us_per_layer": round(us, 3), "recall": round(sum(rec) / len(rec), 4),
                     "predictor_bytes": int(pred_bytes)}
        log(f"  {name}: {us:.2f} us, recall {sum(rec) / len(rec):.3f}")
    del plain, prepared
    torch.cuda.empty_cache()
    return res


def batched_union_leg(args, dev):
    """OPT-30B FFN shape (d 7168, f 28672, r 512, top-k 5734 = 20%), clustered tokens (8 centroids
    + N(0, 0.3)), batches of B in {1, 4, 8, 16, 32}: one step is csf_sparse_ffn_batched_layer
    (predict, top-k with bitmaps, union FFN, per-token semantics) on both kernel families, plus
    the batched dense layer (every neuron, matrix-core path) at the same B."""
    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib, workloads as wl

    cfg = wl.OPT30B
    d, f, r, k = cfg.d, cfg.f, cfg.r, cfg.k
    code = _lib.dtype_code(cfg.dtype)
    nl = args.batched_layers
    log(f"batched leg: {nl} layer instances of d={d} f={f} r={r}")
    layers = [wl.make_layer(cfg, device=dev, layer=l) for l in range(nl)]
    ntok = 256
    X = wl.make_clustered_tokens(cfg, ntok, device=dev)
    stream = torch.cuda.current_stream(dev)
    vp = ctypes.c_void_p
    fn = _entry("csf_sparse_ffn_batched_layer")
    ufn = _entry("csf_sparse_ffn_batched_union")
    words = (f + 31) // 32
    full_bm = torch.full((32, words), -1, dtype=torch.int32, device=dev)
    full_bm[:, -1] = (1 << (f % 32)) - 1 if f % 32 else -1
    pred_bytes = 2 * (r * d + f * r)
    out = []
    for B in [int(b) for b in args.batched_sizes.split(",") if b]:
        Y = torch.empty(B, d, dtype=torch.float32, device=dev)
        uc = torch.zeros(1, dtype=torch.int32, device=dev)
        ws_b = csf.workspace_size(_lib.OP_BATCHED_LAYER, B, d, f, r, k, code)
        ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
        taken = ctypes.c_int(0)
        nb = ntok // B

        def args_for(s, path, ucount=None):
            L = layers[s % nl]
            Xb = X[(s % nb) * B:(s % nb) * B + B]
            return (vp(Xb.data_ptr()), B, d, f, r, cfg.act, code, vp(L.V.data_ptr()),
                    vp(L.U.data_ptr()), vp(L.W1.data_ptr()), vp(L.b1.data_ptr()), None,
                    vp(L.W2T.data_ptr()), k, ctypes.c_float(0.0), 0, path, vp(Y.data_ptr()), None,
                    None if ucount is None else vp(ucount.data_ptr()), ctypes.byref(taken),
                    vp(ws.data_ptr()), ws_b, vp(stream.cuda_stream))

        # union sizes of every (layer, batch) pair the timed loop visits
        usum = 0
        npairs = min(args.batched_steps, nl * nb)
        for s in range(npairs):
            fn(*args_for(s, _lib.PATH_GATHER, uc))
            usum += int(uc.item())
        u_mean = usum / npairs
        step_bytes = pred_bytes + u_mean * 2 * d * 2 + B * d * 2
        flops = 4.0 * B * u_mean * d
        row = {"B": B, "union_mean": round(u_mean, 1), "union_frac": round(u_mean / f, 4),
               "bytes_per_step": int(step_bytes)}
        for pname, path in (("gather", _lib.PATH_GATHER), ("mfma", _lib.PATH_MFMA)):
            plan = [args_for(s, path) for s in range(max(nl * nb, 1))]
            for s in range(16):
                rc = fn(*plan[s % len(plan)])
                if rc:
                    raise csf.CsfError(rc, _lib.lib.csf_last_error().decode())
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for s in range(args.batched_steps):
                fn(*plan[s % len(plan)])
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.batched_steps
            # per-kernel times (runtime-recorded start/end events)
            if B == 1 and path == _lib.PATH_GATHER:
                names = layer_kernels(f, k)      # a batch of one runs the single-token layer
            else:
                names = predictor_kernels(B, code, d, r) + ["select_topk"] + UNION_KERNELS
            nev = 2 * len(names)
            nt = min(64, args.batched_steps)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(nt)]
            for rowe in evs:
                for e in rowe:
                    e.record(stream)
            torch.cuda.synchronize()
            for s in range(nt):
                csf.set_trace_events(evs[s])
                fn(*plan[s % len(plan)])
            csf.set_trace_events([])
            torch.cuda.synchronize()
            kern = {n: round(sum(evs[s][2 * i].elapsed_time(evs[s][2 * i + 1]) for s in range(nt))
                             * 1e3 / nt, 2) for i, n in enumerate(names)}
            row[pname] = {"us_per_batch": round(us, 2), "tokens_per_s": round(B / us * 1e6, 1),
                          "GBps_touched": round(step_bytes / (us * 1e-6) / 1e9, 1),
                          "mfma_util": round(flops / (us * 1e-6) / (PEAK_MFMA_F16_TFLOPS * 1e12), 5),
                          "kernels_us": kern}
        # batched dense: every neuron for every token (union semantics, all-ones bitmaps)
        dws_b = csf.workspace_size(_lib.OP_BATCHED_UNION, B, d, f, 0, 0, code)
        dws = torch.empty(dws_b, dtype=torch.uint8, device=dev)
        dplan = [(vp(X[(s % nb) * B:(s % nb) * B + B].data_ptr()), B, d, f, cfg.act, code,
                  vp(layers[s % nl].W1.data_ptr()), vp(layers[s % nl].b1.data_ptr()), None,
                  vp(layers[s % nl].W2T.data_ptr()), vp(full_bm.data_ptr()), 1, _lib.PATH_MFMA,
                  vp(Y.data_ptr()), None, ctypes.byref(taken), vp(dws.data_ptr()), dws_b,
                  vp(stream.cuda_stream)) for s in range(nl)]
        for s in range(4):
            ufn(*dplan[s % nl])
        torch.cuda.synchronize()
        nd = max(8, args.batched_steps // 8)
        e0.record(stream)
        for s in range(nd):
            ufn(*dplan[s % nl])
        e1.record(stream)
        torch.cuda.synchronize()
        dus = e0.elapsed_time(e1) * 1e3 / nd
        row["dense_mfma_us"] = round(dus, 2)
        row["dense_GBps"] = round(2 * f * d * 2 / (dus * 1e-6) / 1e9, 1)
        best = min(row["gather"]["us_per_batch"], row["mfma"]["us_per_batch"])
        row["speedup_vs_dense"] = round(dus / best, 3)
        log(f"B={B}: union {u_mean:.0f} ({u_mean / f:.2f}), gather {row['gather']['us_per_batch']} us, "
            f"mfma {row['mfma']['us_per_batch']} us, dense {row['dense_mfma_us']} us")
        out.append(row)
        del ws, dws
    return {"workload": "OPT-30B-shape sparse FFN layer, clustered tokens, per-token semantics: "
                        "predict + top-k + union FFN",
            "d": d, "f": f, "r": r, "k": k, "layers_rotated": nl, "steps": args.batched_steps,
            "rows": out}


def stack_leg(args, dev):
    """48 residual blocks of the OPT-30B FFN shape (d 7168, f 28672, r 512, top-k 5734; about
    41 GB of weights), batch 1: tokens per second through the whole stack, synchronous vs
    look-ahead prediction, and each layer's recall of the true active set (the ReLU neurons that
    fire on that layer's actual normalised input)."""
    import torch
    import contextual_sparsity_ffn_amd as csf
    from contextual_sparsity_ffn_amd import _lib, workloads as wl

    cfg = wl.OPT30B_STACK48
    d, f, r, k = cfg.d, cfg.f, cfg.r, cfg.k
    nl = args.stack_layers
    log(f"stack leg: {nl} layers of d={d} f={f} r={r}")
    t0 = time.perf_counter()
    layers = [wl.make_layer(cfg, device=dev, layer=l) for l in range(nl)]
    torch.cuda.synchronize()
    log(f"  weights drawn in {time.perf_counter() - t0:.1f} s")
    ntok = max(args.stack_tokens, args.stack_quality_tokens) + 2
    X = wl.make_tokens(cfg, ntok, device=dev).float()
    side = torch.cuda.Stream(device=dev)
    stream = torch.cuda.current_stream(dev)
    code = _lib.dtype_code(cfg.dtype)
    ws = torch.empty(csf.workspace_size(_lib.OP_STACK, 1, d, f, r, k, code), dtype=torch.uint8,
                     device=dev)
    x = torch.empty(1, d, dtype=torch.float32, device=dev)
    blocks = csf.StackLayers(layers)          # checked and packed once, outside the timed calls
    res = {"workload": "48-layer OPT-30B-shape residual stack (pre-RMSNorm blocks), batch 1",
           "layers": nl, "d": d, "f": f, "r": r, "k": k,
           "bytes_per_token": nl * wl.touched_bytes(cfg, k)}
    for mode, ahead, graph in (("sync", False, False), ("lookahead", True, False),
                               ("sync_graph", False, True), ("lookahead_graph", True, True)):
        for t in range(2):
            x.copy_(X[t:t + 1])
            csf.stack_forward(x, blocks, k=k, lookahead=ahead, side_stream=side, ws=ws, graph=graph)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        host = 0.0
        e0.record(stream)
        for t in range(args.stack_tokens):
            x.copy_(X[2 + t:3 + t])
            h0 = time.perf_counter()
            csf.stack_forward(x, blocks, k=k, lookahead=ahead, side_stream=side, ws=ws, graph=graph)
            host += time.perf_counter() - h0
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.stack_tokens
        res[mode] = {"ms_per_token": round(ms, 4), "tokens_per_s": round(1e3 / ms, 2),
                     "GBps_touched": round(res["bytes_per_token"] / (ms * 1e-3) / 1e9, 1),
                     "us_per_layer": round(ms * 1e3 / nl, 2),
                     "host_enqueue_ms_per_token": round(host * 1e3 / args.stack_tokens, 3)}
        log(f"  {mode}: {ms:.3f} ms/token ({1e3 / ms:.1f} tok/s), host {host * 1e3 / args.stack_tokens:.3f} ms")
        # recall of each layer's set against the true set at that layer's actual input
        nq = args.stack_quality_tokens if not graph else 0
        if nq > 0:
            xhat_log = torch.empty(nl, 1, d, dtype=cfg.dtype, device=dev)
            idx_log = torch.empty(nl, 1, k, dtype=torch.int32, device=dev)
            H = torch.empty(1, f, dtype=torch.float32, device=dev)
            rec = torch.zeros(nl, dtype=torch.float64)
            for t in range(nq):
                x.copy_(X[t:t + 1])
                csf.stack_forward(x, blocks, k=k, lookahead=ahead, side_stream=side, ws=ws,
                                  xhat_log=xhat_log, idx_log=idx_log)
                for l in range(nl):
                    L = layers[l]
                    csf.dense_ffn(xhat_log[l], L.W1, L.b1, None, L.W2T, h=H)
                    true = H[0] > 0
                    nt = int(true.sum())
                    hit = int(true[idx_log[l, 0].long()].sum())
                    rec[l] += hit / nt if nt else 1.0
            rec /= nq
            res[mode]["recall_per_layer"] = [round(float(v), 4) for v in rec]
            res[mode]["recall_mean"] = round(float(rec.mean()), 4)
    # the recurrence as written (no normalisation): the stream's growth and the first layer
    # whose input no longer fits the 16-bit storage type
    x_log = torch.empty(nl, 1, d, dtype=torch.float32, device=dev)
    xhat_log = torch.empty(nl, 1, d, dtype=cfg.dtype, device=dev)
    lit = {}
    for norm in (True, False):
        x.copy_(X[0:1])
        csf.stack_forward(x, blocks, k=k, norm=norm, ws=ws, x_log=x_log, xhat_log=xhat_log)
        torch.cuda.synchronize()
        rms = x_log[:, 0].double().pow(2).mean(dim=1).sqrt()
        bad = [l for l in range(nl) if not bool(torch.isfinite(xhat_log[l, 0]).all())]
        lit["normalised" if norm else "literal"] = {
            "rms_per_layer": [float(f"{v:.4g}") for v in rms.tolist()],
            "first_layer_input_overflowing_f16": bad[0] if bad else None,
            "final_finite": bool(torch.isfinite(x).all())}
    lit["note"] = ("one token through the stack: x_{l+1} = x_l + FFN_l(xhat_l), xhat_l = "
                   "dtype(x_l / rms(x_l)) (normalised, the default) or dtype(x_l) (literal); "
                   "rms of x_l per layer, and the first layer whose rounded input holds inf")
    res["literal_recurrence"] = lit
    log(f"  literal recurrence: first f16 overflow at layer "
        f"{lit['literal']['first_layer_input_overflowing_f16']}")
    del layers, blocks
    torch.cuda.empty_cache()
    res["lookahead_speedup"] = round(res["sync"]["ms_per_token"] / res["lookahead"]["ms_per_token"], 4)
    res["lookahead_graph_speedup"] = round(res["sync_graph"]["ms_per_token"] /
                                           res["lookahead_graph"]["ms_per_token"], 4)
    res["dense_bound_tokens_per_s"] = round(8e12 / (nl * wl.dense_bytes(cfg)), 1)
    res["sparse_bound_tokens_per_s"] = round(8e12 / res["bytes_per_token"], 1)
    return res


def cpu_threads():
    """Host threads for the N-core oracle leg: the cores this process may run on, at most 16 (the
    host share that goes with one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(cfg, L, X, ntok, ntok_mt, touched):
    """The oracle as it stands (predict + top-k + sparse FFN per token, then the dense FFN) on the
    host: one thread on `ntok` tokens, then all of the host share's cores (OpenMP over rows and
    column blocks, the same sums in the same order) on `ntok_mt` tokens."""
    import numpy as np
    from oracle import oracle as orc

    def host(t):
        return t.detach().cpu().numpy()

    V, U, W1, W2T, b1 = host(L.V), host(L.U), host(L.W1), host(L.W2T), host(L.b1)
    n_mt = cpu_threads()
    xs = [host(X[t]) for t in range(max(ntok, ntok_mt))]
    orc.lib()
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    dense_b = (2 * cfg.f * cfg.d) * 2 + cfg.d * 2

    def sparse_leg(threads, n):
        orc.set_threads(threads)
        t0 = time.perf_counter()
        for x in xs[:n]:
            _, _, s = orc.predict(x, V, U, orc.F16)
            sel = orc.select_topk(s, cfg.k)
            orc.sparse_ffn(x, W1, b1, None, W2T, sel, orc.RELU, orc.F16)
        return time.perf_counter() - t0

    def dense_leg(threads, n):
        orc.set_threads(threads)
        t0 = time.perf_counter()
        for x in xs[:n]:
            orc.dense_ffn(x, W1, b1, None, W2T, orc.RELU, orc.F16)
        return time.perf_counter() - t0

    try:
        log(f"CPU oracle baseline: {ntok} tokens on 1 thread, {ntok_mt} on {n_mt} threads")
        t1 = sparse_leg(1, ntok)
        tn = sparse_leg(n_mt, ntok_mt)
        log("CPU oracle dense FFN: 1 token on 1 thread, 2 on all threads")
        td1 = dense_leg(1, 1)
        tdn = dense_leg(n_mt, 2)
    finally:
        orc.set_threads(1)

    def leg(dt, n, threads, nbytes):
        return {"value": round(nbytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
                "us_per_layer": round(dt / n * 1e6, 1), "tokens": n, "seconds": round(dt, 2)}

    single = leg(t1, ntok, 1, touched)
    multi = leg(tn, ntok_mt, n_mt, touched)
    return {"value": multi["value"], "unit": "GB/s", "cores": n_mt, "kind": "oracle",
            "us_per_layer": multi["us_per_layer"],
            "sample": f"{ntok_mt} tokens of one layer of the same shape (predict + top-k + sparse "
                      f"FFN) through the C oracle with double accumulation on {n_mt} OpenMP "
                      f"threads (whole rows and column blocks per thread, each sum in ascending "
                      f"order: bitwise the single-thread result), {tn:.1f} s",
            "single_thread": dict(single, sample=f"{ntok} tokens, one thread, {t1:.1f} s"),
            "dense": {"single_thread": leg(td1, 1, 1, dense_b), "multi_thread": leg(tdn, 2, n_mt, dense_b),
                      "sample": "the oracle's dense FFN (every neuron) on the first tokens"},
            "multi_thread_speedup": round(t1 / ntok / (tn / ntok_mt), 2),
            "host_cores_available": len(os.sched_getaffinity(0)), "host_cpu": model}


def tensor_sha256(named):
    """SHA-256 of each tensor's bytes (as stored: row-major, storage type), read back in chunks."""
    import hashlib
    import torch
    out = {}
    for name, t in named:
        h = hashlib.sha256()
        flat = t.detach().contiguous().reshape(-1).view(torch.uint8)
        step = 1 << 28
        for i in range(0, flat.numel(), step):
            h.update(flat[i:i + step].cpu().numpy().tobytes())
        out[name] = h.hexdigest()
    return out


def bandwidth_probe(dev):
    """HBM bandwidth of a plain 1 GiB device copy with PyTorch's own kernel (best of 5), for
    context.  The library's dense FFN, a pure streaming read of W1 and W2T (1.2 GB), is the
    read-side reference (dense_GBps)."""
    import torch
    n = 1 << 30
    a = torch.ones(n // 2, dtype=torch.float16, device=dev)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    t_copy = best(lambda: b.copy_(a))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": round(2 * n / t_copy / 1e9, 1), "bytes_copied": n,
            "how": "torch copy_ of 1 GiB (read + write counted)"}


if __name__ == "__main__":
    main()

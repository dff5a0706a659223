"""CPU oracle for the contextual-sparsity FFN step -- Python side.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path never imports it.

The arithmetic lives in ``csf_oracle.c`` (plain C loops, double-precision accumulation,
ascending index order).  This module loads it with ctypes, converts numpy arrays to the raw
storage the C code reads, and composes the C primitives into the per-token, batched and
stacked forms.  Composition is kept to plain Python loops so that each step can be read
against the pages:

  [DV] "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm"
  [CP] "Contextual Sparsity and Activation Predictors"
  [AS] "Activation sparsity" (wiki page), section "Implementation sketch"

Storage types: ``F32`` is float32, ``F16`` is float16, ``BF16`` is bfloat16 passed as its raw
``uint16`` bit pattern (numpy has no bfloat16 type).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, F16, BF16 = 0, 1, 2
RELU, REGLU, SILU, SWIGLU = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csf_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_NP_STORAGE = {F32: np.float32, F16: np.float16, BF16: np.uint16}


def build(force: bool = False) -> str:
    """Compile csf_oracle.c with gcc (no fast-math, so IEEE semantics hold)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-fopenmp", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        vp, i32, dbl, flt = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = dbl
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = dbl
        L.orc_f64_to_f16.argtypes = [dbl]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_f64_to_bf16.argtypes = [dbl]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_silu.argtypes = [dbl]
        L.orc_silu.restype = dbl
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = i32
        L.orc_get_threads.argtypes = []
        L.orc_get_threads.restype = i32
        L.orc_predict.argtypes = [vp, i32, vp, i32, vp, i32, i32, vp, vp, vp]
        L.orc_select_topk.argtypes = [vp, i32, i32, vp]
        L.orc_select_threshold.argtypes = [vp, i32, flt, vp]
        L.orc_sparse_ffn.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp]
        L.orc_dense_ffn.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.orc_preact.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.orc_rms_normalize.argtypes = [vp, i32, dbl, i32, vp]
        L.orc_attention_decode.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                           vp, i32, vp, vp, i32, i32, vp, vp]
        for name in ("orc_predict", "orc_select_topk", "orc_select_threshold", "orc_sparse_ffn",
                     "orc_dense_ffn", "orc_preact", "orc_rms_normalize", "orc_attention_decode"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads for the oracle's loops over independent outputs (1: serial).  Each output element
    is one sum in ascending index order whatever n is, so results do not depend on n."""
    if lib().orc_set_threads(int(n)) != 0:
        raise ValueError(f"thread count must be >= 1, got {n}")


def get_threads() -> int:
    return lib().orc_get_threads()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(a: np.ndarray, dt: int) -> np.ndarray:
    want = _NP_STORAGE[dt]
    if a.dtype != want:
        raise TypeError(f"storage type {dt} needs numpy {want.__name__}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise ValueError(f"{what} rejected its arguments (code {rc})")
    return rc


# ---------------------------------------------------------------------------------------------
# storage conversions
# ---------------------------------------------------------------------------------------------
def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return lib().orc_bf16_to_f64(bits)


def f64_to_f16_bits(v: float) -> int:
    return lib().orc_f64_to_f16(v)


def f64_to_bf16_bits(v: float) -> int:
    return lib().orc_f64_to_bf16(v)


def widen(a: np.ndarray, dt: int) -> np.ndarray:
    """Exact float64 value of every element (bf16 arrays are raw uint16 bit patterns)."""
    a = _storage(a, dt)
    if dt == F32:
        return a.astype(np.float64)
    f = f16_to_f64 if dt == F16 else bf16_to_f64
    flat = a.reshape(-1).view(np.uint16)
    return np.array([f(int(b)) for b in flat], dtype=np.float64).reshape(a.shape)


# ---------------------------------------------------------------------------------------------
# O1/O2 predictor, O3 selection, O4/O5 FFN  (C primitives)
# ---------------------------------------------------------------------------------------------
def predict(x, V, U, dt):
    """[DV] "The Prediction Problem": s = sigmoid(U relu(V x)).  Returns (a, z, s)."""
    x, V, U = _storage(x, dt), _storage(V, dt), _storage(U, dt)
    r, d = V.shape
    f = U.shape[0]
    assert x.shape == (d,) and U.shape == (f, r)
    a = np.empty(r, np.float64)
    z = np.empty(f, np.float64)
    s = np.empty(f, np.float32)
    _check(lib().orc_predict(_ptr(x), d, _ptr(V), r, _ptr(U), f, dt, _ptr(a), _ptr(z), _ptr(s)),
           "orc_predict")
    return a, z, s


def select_topk(s, k):
    """[DV] "The Prediction Problem": the k best scores, lower index first on ties, ascending."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(max(k, 1), np.int32)
    m = _check(lib().orc_select_topk(_ptr(s), s.shape[0], int(k), _ptr(out)), "orc_select_topk")
    return out[:m].copy()


def select_threshold(s, tau):
    """[AS] "Implementation sketch": {j : s_j >= tau} in ascending order."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(max(s.shape[0], 1), np.int32)
    m = _check(lib().orc_select_threshold(_ptr(s), s.shape[0], float(np.float32(tau)), _ptr(out)),
               "orc_select_threshold")
    return out[:m].copy()


def sparse_ffn(x, W1, b1, Wup, W2T, idx, act, dt):
    """[DV] sparse_mlp_forward over the active list idx.  Returns (h, y) in float64."""
    x, W1, W2T = _storage(x, dt), _storage(W1, dt), _storage(W2T, dt)
    Wup = None if Wup is None else _storage(Wup, dt)
    f, d = W1.shape
    b1 = None if b1 is None else np.ascontiguousarray(b1, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    h = np.empty(max(idx.shape[0], 1), np.float64)
    y = np.empty(d, np.float64)
    _check(lib().orc_sparse_ffn(_ptr(x), d, f, act, dt, _ptr(W1), _ptr(b1), _ptr(Wup), _ptr(W2T),
                                _ptr(idx), idx.shape[0], _ptr(h), _ptr(y)), "orc_sparse_ffn")
    return h[:idx.shape[0]].copy(), y


def dense_ffn(x, W1, b1, Wup, W2T, act, dt):
    x, W1, W2T = _storage(x, dt), _storage(W1, dt), _storage(W2T, dt)
    Wup = None if Wup is None else _storage(Wup, dt)
    f, d = W1.shape
    b1 = None if b1 is None else np.ascontiguousarray(b1, dtype=np.float32)
    h = np.empty(max(f, 1), np.float64)
    y = np.empty(d, np.float64)
    _check(lib().orc_dense_ffn(_ptr(x), d, f, act, dt, _ptr(W1), _ptr(b1), _ptr(Wup), _ptr(W2T),
                               _ptr(h), _ptr(y)), "orc_dense_ffn")
    return h[:f].copy(), y


def preact(x, W1, b1, dt):
    """Gate pre-activation of every neuron, W1 x + b1, in float64."""
    x, W1 = _storage(x, dt), _storage(W1, dt)
    f, d = W1.shape
    b1 = None if b1 is None else np.ascontiguousarray(b1, dtype=np.float32)
    p = np.empty(max(f, 1), np.float64)
    _check(lib().orc_preact(_ptr(x), d, f, dt, _ptr(W1), _ptr(b1), _ptr(p)), "orc_preact")
    return p[:f].copy()


def rms_normalize(x, dt, eps=1e-6):
    """x / sqrt(mean(x^2) + eps), rounded once to storage type dt (float32 stream in)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape[0], _NP_STORAGE[dt])
    _check(lib().orc_rms_normalize(_ptr(x), x.shape[0], float(eps), dt, _ptr(out)),
           "orc_rms_normalize")
    return out


# ---------------------------------------------------------------------------------------------
# O6 quality of a predicted set against the true set
# ---------------------------------------------------------------------------------------------
def true_set(x, W1, b1, dt):
    """Neurons whose ReLU (or gate ReLU) output is non-zero: pre-activation strictly > 0."""
    return np.nonzero(preact(x, W1, b1, dt) > 0.0)[0].astype(np.int32)


def silu(p: float) -> float:
    """silu(p) = p / (1 + e^-p), as the C oracle computes it."""
    return lib().orc_silu(float(p))


def functional_set(x, W1, b1, dt, tau=0.1):
    """[DV] "The Empirical Foundation" (measure_mlp_sparsity, SiLU form): the neurons whose gate
    activation is large in magnitude, |silu(W1 x + b1)| > tau, in ascending order.  SiLU is never
    exactly zero, so this is the set that matters to the output, not the set that is non-zero."""
    p = preact(x, W1, b1, dt)
    return np.array([j for j in range(p.shape[0]) if abs(silu(p[j])) > tau], dtype=np.int32)


def recall_precision(pred, true):
    """[CP] "Precision, recall, and which error hurts".  Empty denominators give 1."""
    P, T = set(int(j) for j in pred), set(int(j) for j in true)
    hit = len(P & T)
    recall = hit / len(T) if T else 1.0
    precision = hit / len(P) if P else 1.0
    return recall, precision


# ---------------------------------------------------------------------------------------------
# O7 batched: per-token sets, the union of a batch
# ---------------------------------------------------------------------------------------------
def union_of(sets, f):
    """[CP] "When it breaks": a batch must read the union of its tokens' sets (ascending)."""
    seen = [False] * f
    for s in sets:
        for j in s:
            seen[int(j)] = True
    return np.array([j for j in range(f) if seen[j]], dtype=np.int32)


def batched_ffn(X, sets, W1, b1, Wup, W2T, act, dt, union=False):
    """Token t uses its own set (union=False) or the batch union (union=True).  Returns Y [B, d]."""
    f = W1.shape[0]
    U = union_of(sets, f) if union else None
    Y = []
    for t in range(X.shape[0]):
        idx = U if union else sets[t]
        Y.append(sparse_ffn(X[t], W1, b1, Wup, W2T, idx, act, dt)[1])
    return np.stack(Y) if Y else np.zeros((0, W1.shape[1]))


def to_bitmap(idx, f):
    """Bit j of word j // 32 set for every j in idx (the packed form of an active mask)."""
    words = np.zeros((f + 31) // 32, np.uint32)
    for j in idx:
        words[int(j) // 32] |= np.uint32(1) << np.uint32(int(j) % 32)
    return words


def hot_layer_set(x, V, U_cold, hot, dt, k=None, tau=None):
    """[CP] "Static locality: hot and cold neurons": the neurons 0 .. hot-1 (ordered hot first) are
    always active; the predictor (up rows U_cold: row i scores neuron hot + i) picks among the
    rest by top-k or threshold.  Returns (ascending list, cold scores)."""
    _, _, s = predict(x, V, U_cold, dt)
    cold = select_topk(s, k) if k is not None else select_threshold(s, tau)
    return np.concatenate([np.arange(hot, dtype=np.int32), cold.astype(np.int32) + hot]), s


def round_to_storage(x, dt):
    """Round float values to storage type dt, nearest-even (bf16 as raw uint16 bits)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    if dt == F32:
        return x.astype(np.float32)
    f = f64_to_f16_bits if dt == F16 else f64_to_bf16_bits
    bits = np.array([f(float(v)) for v in x], dtype=np.uint16)
    return bits.view(np.float16) if dt == F16 else bits


# ---------------------------------------------------------------------------------------------
# O8 stack with optional look-ahead
# ---------------------------------------------------------------------------------------------
def stack_forward(x0, layers, dt, k=None, tau=None, lookahead=False, eps=1e-6, norm=True):
    """Residual stack x_{l+1} = x_l + FFN_l(xhat_l) in float32 ([CP] "The predictor and its budget").

    ``layers`` is a list of dicts with keys V, U, W1, b1, Wup, W2T, act.  Layer l's active set is
    predicted from its own normalised input (``lookahead=False``) or from the previous layer's
    normalised input (``lookahead=True``; layer 0 is always predicted from its own input).
    Returns (x_final float32, per-layer active sets, per-layer normalised inputs).
    """
    x = np.asarray(x0, dtype=np.float32).copy()
    sets, xhats = [], []
    prev_xhat = None
    for l, L in enumerate(layers):
        xhat = rms_normalize(x, dt, eps) if norm else round_to_storage(x, dt)
        src = prev_xhat if (lookahead and l > 0) else xhat
        _, _, s = predict(src, L["V"], L["U"], dt)
        idx = select_topk(s, k) if k is not None else select_threshold(s, tau)
        _, y = sparse_ffn(xhat, L["W1"], L["b1"], L.get("Wup"), L["W2T"], idx, L["act"], dt)
        x = (x.astype(np.float64) + y).astype(np.float32)
        sets.append(idx)
        xhats.append(xhat)
        prev_xhat = xhat
    return x, sets, xhats


# ---------------------------------------------------------------------------------------------
# O9 attention-head sparsity: one decode step over a set of heads  (C primitive)
# ---------------------------------------------------------------------------------------------
def attention_decode(x, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, lens, heads, dt, kv_all=False):
    """[DV] (opening section; The Empirical Foundation; Implications for System Design): one new
    token through the heads in `heads` (ascending): q, k, v projections, k and v appended to the
    storing heads' caches (rounded to the storage type), softmax(q.K / sqrt(dh)) over the cache,
    o_h = p.V, y = sum of WoT_h^T o_h.  Kc, Vc [H, Tmax, dh] (storage type) and lens [H] int32 are
    updated in place.  Returns (o [count, dh], y [d]) in float64."""
    x, Wq, Wk, Wv, WoT = (_storage(a, dt) for a in (x, Wq, Wk, Wv, WoT))
    HD, d = Wq.shape
    H, Tmax, dh = Kc.shape
    assert HD == H * dh and Vc.shape == Kc.shape and lens.shape == (H,)
    for a in (Kc, Vc):
        assert a.dtype == _NP_STORAGE[dt] and a.flags.c_contiguous
    assert lens.dtype == np.int32 and lens.flags.c_contiguous
    bq, bk, bv = (None if b is None else np.ascontiguousarray(b, dtype=np.float32)
                  for b in (bq, bk, bv))
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    n = heads.shape[0]
    o = np.empty((max(n, 1), dh), np.float64)
    y = np.empty(d, np.float64)
    _check(lib().orc_attention_decode(_ptr(x), d, H, dh, dt, _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(bq),
                                      _ptr(bk), _ptr(bv), _ptr(WoT), _ptr(Kc), _ptr(Vc), Tmax,
                                      _ptr(lens), _ptr(heads), n, int(bool(kv_all)), _ptr(o), _ptr(y)),
           "orc_attention_decode")
    return o[:n].copy(), y

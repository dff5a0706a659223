"""Thin ctypes binding of ``libcsf.so`` (the C ABI in ``include/csf.h``).

Argument marshalling only: each function checks the tensors it is given (device, dtype, shape,
contiguity), sizes and allocates the workspace with torch, passes raw device pointers and the
current HIP stream to the library, and raises on a non-zero status.  Every step of the path runs
in the library's HIP kernels; there is no fallback of any kind.  If ``libcsf.so`` has not been
built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsf.so")

F32, F16, BF16 = 0, 1, 2
RELU, REGLU, SILU, SWIGLU = 0, 1, 2, 3
GATED_ACTS = (REGLU, SWIGLU)
OP_PREDICT, OP_SELECT_TOPK, OP_SELECT_THRESHOLD, OP_SPARSE_FFN, OP_DENSE_FFN, OP_LAYER, \
    OP_BATCHED_UNION, OP_BATCHED_LAYER, OP_STACK, OP_ATTN_DECODE, OP_ATTN_LAYER = range(11)
STACK_SYNC, STACK_LOOKAHEAD, STACK_GRAPH = 0, 1, 0x100
FFN_SKIP_ZERO_H = 1
SEM_PER_TOKEN, SEM_UNION = 0, 1
PATH_AUTO, PATH_GATHER, PATH_MFMA = 0, 1, 2
MAX_UNION_BATCH = 32

_STATUS = {0: "CSF_OK", 1: "CSF_ERR_INVALID_ARG", 2: "CSF_ERR_UNSUPPORTED",
           3: "CSF_ERR_MISALIGNED", 4: "CSF_ERR_WORKSPACE_TOO_SMALL", 5: "CSF_ERR_HIP"}

EXPORTS = ("csf_abi_version", "csf_status_string", "csf_last_error", "csf_workspace_size",
           "csf_create", "csf_destroy", "csf_get_device_info", "csf_predict_active", "csf_select_topk", "csf_select_threshold", "csf_sparse_ffn",
           "csf_dense_ffn", "csf_sparse_ffn_layer", "csf_sparse_ffn_layer_hot",
           "csf_sparse_ffn_batched_union",
           "csf_sparse_ffn_batched_layer", "csf_stack_forward", "csf_set_ffn_flags",
           "csf_set_ffn_gate_threshold", "csf_set_trace_events", "csf_sparse_attention_decode",
           "csf_sparse_attention_layer", "csf_attention_workspace_size",
           "csf_sparse_ffn_layer_noalloc")


class LayerWeights(ctypes.Structure):
    """csf_layer_weights: one block's device pointers."""
    _fields_ = [("V", ctypes.c_void_p), ("U", ctypes.c_void_p), ("W1", ctypes.c_void_p),
                ("Wup", ctypes.c_void_p), ("W2T", ctypes.c_void_p), ("b1", ctypes.c_void_p)]


class CsfError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python contextual_sparsity_ffn_amd/build.py` "
            "(hipcc, gfx950).  The library has no non-HIP fallback.")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, flt = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.csf_abi_version.restype = i32
    L.csf_abi_version.argtypes = []
    L.csf_status_string.restype = ctypes.c_char_p
    L.csf_status_string.argtypes = [i32]
    L.csf_last_error.restype = ctypes.c_char_p
    L.csf_last_error.argtypes = []
    L.csf_workspace_size.restype = sz
    L.csf_workspace_size.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32]
    L.csf_create.argtypes = [ctypes.POINTER(vp), i32]
    L.csf_destroy.argtypes = [vp]
    L.csf_get_device_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    # every entry point below takes the handle first
    L.csf_predict_active.argtypes = [vp, vp, i32, i32, vp, i32, vp, i32, i32, vp, vp, sz, vp]
    L.csf_select_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.csf_select_threshold.argtypes = [vp, vp, i32, i32, flt, vp, vp, vp, vp, sz, vp]
    L.csf_sparse_ffn.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, i32,
                                 vp, vp, vp, sz, vp]
    L.csf_dense_ffn.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz,
                                vp]
    L.csf_set_trace_events.argtypes = [vp, ctypes.POINTER(ctypes.c_void_p), i32]
    L.csf_set_ffn_flags.argtypes = [vp, i32]
    L.csf_set_ffn_gate_threshold.argtypes = [vp, flt]
    L.csf_sparse_ffn_layer.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                       i32, flt, vp, vp, vp, vp, vp, sz, vp]
    L.csf_sparse_ffn_layer_hot.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                           i32, i32, flt, vp, vp, vp, vp, vp, sz, vp]
    L.csf_sparse_ffn_batched_union.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                               vp, i32, i32, vp, vp, ctypes.POINTER(i32), vp, sz,
                                               vp]
    L.csf_sparse_ffn_batched_layer.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                               vp, vp, vp, i32, flt, i32, i32, vp, vp, vp,
                                               ctypes.POINTER(i32), vp, sz, vp]
    L.csf_stack_forward.argtypes = [vp, ctypes.POINTER(LayerWeights), i32, i32, i32, i32, i32,
                                    i32, vp, i32, i32, i32, flt, i32, flt, vp, vp, vp, vp, vp, sz,
                                    vp, vp]
    L.csf_sparse_attention_decode.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                              vp, vp, vp, i32, vp, vp, vp, i32, i32, vp, vp, vp,
                                              sz, vp]
    L.csf_sparse_attention_layer.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, i32, vp, i32, flt, i32, vp,
                                             vp, vp, vp, vp, vp, sz, vp]
    L.csf_attention_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.csf_sparse_ffn_layer_noalloc.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                               vp, vp, i32, flt, vp, vp, vp, vp, vp]
    for name in EXPORTS[4:]:
        getattr(L, name).restype = i32
    L.csf_attention_workspace_size.restype = sz
    return L


lib = _load()


# ------------------------------------------------------------------------------------------------
# handles
# ------------------------------------------------------------------------------------------------
class Context:
    """A library handle (csf_create) for one HIP device: it holds the device's facts, the
    gathered FFN's options, the per-kernel timing hook and the stack's events and graph.  Use it
    from one thread at a time; `close()` (or garbage collection) destroys it."""

    def __init__(self, device=0):
        index = device.index if isinstance(device, torch.device) else int(device)
        if index is None:
            index = torch.cuda.current_device()
        h = ctypes.c_void_p()
        with torch.cuda.device(index):
            _check(lib.csf_create(ctypes.byref(h), index))
        self.handle = h
        self.device = torch.device("cuda", index)
        cus = ctypes.c_int(0)
        _check(lib.csf_get_device_info(h, None, ctypes.byref(cus)))
        self.compute_units = cus.value

    def close(self):
        if self.handle is not None and self.handle.value:
            lib.csf_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_ffn_flags(self, flags):
        _check(lib.csf_set_ffn_flags(self.handle, int(flags)))

    def set_ffn_gate_threshold(self, tau):
        _check(lib.csf_set_ffn_gate_threshold(self.handle, float(tau)))

    def set_trace_events(self, events):
        n = len(events)
        arr = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(e.cuda_event) for e in events])
        _check(lib.csf_set_trace_events(self.handle, arr, n))


_default_contexts = {}


def context(device=None) -> Context:
    """The default handle of a device (created on first use): the one the functions below use
    when no ctx is given."""
    if device is None:
        index = torch.cuda.current_device()
    elif isinstance(device, torch.device):
        index = device.index if device.index is not None else torch.cuda.current_device()
    else:
        index = int(device)
    ctx = _default_contexts.get(index)
    if ctx is None:
        ctx = Context(index)
        _default_contexts[index] = ctx
    return ctx


def _h(ctx, dev):
    """The handle for a call on device `dev`; that device is made current if it is not."""
    c = ctx if ctx is not None else context(dev)
    if torch.cuda.current_device() != c.device.index:
        torch.cuda.set_device(c.device)
    return c.handle


# ------------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------------
def dtype_code(dt: torch.dtype) -> int:
    try:
        return {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[dt]
    except KeyError:
        raise ValueError(f"unsupported weight dtype {dt}; use float32, float16 or bfloat16") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int):
    if status != 0:
        raise CsfError(status, lib.csf_last_error().decode())


def _tensor(t, name, dtype=None, shape=None, device=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def workspace_size(op, B, d, f, r=0, max_count=0, dtype=F16, ctx=None) -> int:
    """Workspace bytes of an operation; with ctx (a Context, or a device for its default
    context) sized for that handle's device, else for any device."""
    if ctx is not None and not isinstance(ctx, Context):
        ctx = context(ctx)
    return int(lib.csf_workspace_size(ctx.handle if ctx is not None else None, op, B, d, f, r,
                                      max_count, dtype))


def _workspace(nbytes, device, ws=None):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        _tensor(ws, "ws", dtype=torch.uint8, device=device)
        if ws.numel() < nbytes:
            raise ValueError(f"workspace has {ws.numel()} bytes, needs {nbytes}")
        return ws, ws.numel()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def k_from_ratio(f: int, ratio: float) -> int:
    """Active-set size for a fraction of f neurons: nearest integer, halves rounded up."""
    import math
    return int(math.floor(f * ratio + 0.5))


# ------------------------------------------------------------------------------------------------
# entry points (same names as the C ABI without the csf_ prefix)
# ------------------------------------------------------------------------------------------------
def predict_active(x, V, U, scores=None, ws=None, ctx=None):
    """Sigmoid scores [B, f] (float32) of the low-rank predictor for x [B, d] (or [d])."""
    squeeze = x.dim() == 1
    X = x.unsqueeze(0) if squeeze else x
    _tensor(X, "x")
    dev, dt = X.device, X.dtype
    B, d = X.shape
    _tensor(V, "V", dtype=dt, device=dev)
    r = V.shape[0]
    _tensor(V, "V", shape=(r, d))
    f = U.shape[0]
    _tensor(U, "U", dtype=dt, shape=(f, r), device=dev)
    if scores is None:
        scores = torch.empty(B, f, dtype=torch.float32, device=dev)
    _tensor(scores, "scores", dtype=torch.float32, device=dev)
    if scores.numel() != B * f:
        raise ValueError(f"scores must hold {B}x{f} values")
    code = dtype_code(dt)
    w, wb = _workspace(workspace_size(OP_PREDICT, B, d, f, r, 0, code), dev, ws)
    _check(lib.csf_predict_active(_h(ctx, dev), _ptr(X), B, d, _ptr(V), r, _ptr(U), f, code,
                                  _ptr(scores), _ptr(w), wb, _stream(dev)))
    return scores.view(f) if squeeze else scores.view(B, f)


def select_topk(scores, k, idx=None, count=None, bitmap=None, ctx=None):
    """Ascending top-k neuron lists [B, k] (int32); lower index wins ties."""
    squeeze = scores.dim() == 1
    S = scores.unsqueeze(0) if squeeze else scores
    _tensor(S, "scores", dtype=torch.float32)
    dev = S.device
    B, f = S.shape
    k = int(k)
    if idx is None:
        idx = torch.empty(B, max(k, 1), dtype=torch.int32, device=dev)
    _tensor(idx, "idx", dtype=torch.int32, device=dev)
    if idx.numel() < B * max(k, 1):
        raise ValueError("idx is too small")
    _tensor(count, "count", dtype=torch.int32, device=dev, optional=True)
    _tensor(bitmap, "bitmap", dtype=torch.int32, device=dev, optional=True)
    w, wb = _workspace(workspace_size(OP_SELECT_TOPK, B, 1, f, 0, k), dev)
    _check(lib.csf_select_topk(_h(ctx, dev), _ptr(S), B, f, k, _ptr(idx), _ptr(count),
                               _ptr(bitmap), _ptr(w), wb, _stream(dev)))
    out = idx.view(B, -1)[:, :k]
    return out[0] if squeeze else out


def select_threshold(scores, tau, idx=None, count=None, bitmap=None, ctx=None):
    """Every neuron with score >= tau: returns (idx [B, f] int32, count [B] int32), both on device."""
    squeeze = scores.dim() == 1
    S = scores.unsqueeze(0) if squeeze else scores
    _tensor(S, "scores", dtype=torch.float32)
    dev = S.device
    B, f = S.shape
    if idx is None:
        idx = torch.empty(B, f, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(B, dtype=torch.int32, device=dev)
    _tensor(idx, "idx", dtype=torch.int32, shape=(B, f), device=dev)
    _tensor(count, "count", dtype=torch.int32, shape=(B,), device=dev)
    _tensor(bitmap, "bitmap", dtype=torch.int32, device=dev, optional=True)
    _check(lib.csf_select_threshold(_h(ctx, dev), _ptr(S), B, f, float(tau), _ptr(idx),
                                    _ptr(count), _ptr(bitmap), None, 0, _stream(dev)))
    return (idx[0], count[0:1]) if squeeze else (idx, count)


def _ffn_weights(x, W1, b1, Wup, W2T, act):
    dev, dt = x.device, x.dtype
    f, d = W1.shape
    _tensor(W1, "W1", dtype=dt, device=dev)
    _tensor(W2T, "W2T", dtype=dt, shape=(f, d), device=dev)
    _tensor(b1, "b1", dtype=torch.float32, shape=(f,), device=dev, optional=True)
    if act in GATED_ACTS:
        _tensor(Wup, "Wup", dtype=dt, shape=(f, d), device=dev)
    elif Wup is not None:
        raise ValueError("Wup is only used with the gated activations (REGLU, SWIGLU)")
    return dev, dt, f, d


def sparse_ffn(x, W1, b1, Wup, W2T, idx, act=RELU, count=None, max_count=None, h=None, y=None,
               ws=None, ctx=None):
    """y [B, d] float32 over each token's active list idx [B, stride] (int32, ascending)."""
    squeeze = x.dim() == 1
    X = x.unsqueeze(0) if squeeze else x
    I = idx.unsqueeze(0) if idx.dim() == 1 else idx
    _tensor(X, "x")
    dev, dt, f, d = _ffn_weights(X, W1, b1, Wup, W2T, act)
    B = X.shape[0]
    _tensor(X, "x", shape=(B, d))
    _tensor(I, "idx", dtype=torch.int32, device=dev)
    if I.shape[0] != B:
        raise ValueError("idx must have one row per token")
    stride = I.shape[1]
    max_count = stride if max_count is None else int(max_count)
    _tensor(count, "count", dtype=torch.int32, shape=(B,), device=dev, optional=True)
    if h is not None:
        _tensor(h, "h", dtype=torch.float32, shape=(B, stride), device=dev)
    if y is None:
        y = torch.empty(B, d, dtype=torch.float32, device=dev)
    _tensor(y, "y", dtype=torch.float32, device=dev)
    code = dtype_code(dt)
    w, wb = _workspace(workspace_size(OP_SPARSE_FFN, B, d, f, 0, max_count, code), dev, ws)
    _check(lib.csf_sparse_ffn(_h(ctx, dev), _ptr(X), B, d, f, act, code, _ptr(W1), _ptr(b1),
                              _ptr(Wup), _ptr(W2T), _ptr(I), stride, _ptr(count), max_count,
                              _ptr(h), _ptr(y), _ptr(w), wb, _stream(dev)))
    return y.view(d) if squeeze else y.view(B, d)


def dense_ffn(x, W1, b1, Wup, W2T, act=RELU, y=None, h=None, ws=None, ctx=None):
    """y [B, d] float32 over every neuron; h [B, f] (optional) receives every activation."""
    squeeze = x.dim() == 1
    X = x.unsqueeze(0) if squeeze else x
    _tensor(X, "x")
    dev, dt, f, d = _ffn_weights(X, W1, b1, Wup, W2T, act)
    B = X.shape[0]
    _tensor(X, "x", shape=(B, d))
    if y is None:
        y = torch.empty(B, d, dtype=torch.float32, device=dev)
    _tensor(y, "y", dtype=torch.float32, device=dev)
    if h is not None:
        _tensor(h, "h", dtype=torch.float32, device=dev)
        if h.numel() != B * f:
            raise ValueError(f"h must hold {B}x{f} values")
    code = dtype_code(dt)
    w, wb = _workspace(workspace_size(OP_DENSE_FFN, B, d, f, 0, f, code), dev, ws)
    _check(lib.csf_dense_ffn(_h(ctx, dev), _ptr(X), B, d, f, act, code, _ptr(W1), _ptr(b1),
                             _ptr(Wup), _ptr(W2T), _ptr(h), _ptr(y), _ptr(w), wb, _stream(dev)))
    return y.view(d) if squeeze else y.view(B, d)


def set_ffn_flags(flags, ctx=None):
    """Options of the gathered FFN for later calls with the handle (default: the current device's
    default context): FFN_SKIP_ZERO_H or 0."""
    (ctx or context()).set_ffn_flags(flags)


def set_ffn_gate_threshold(tau, ctx=None):
    """gate_tau of the post-gate skip for later calls with the handle (0 = exact zero-skip)."""
    (ctx or context()).set_ffn_gate_threshold(tau)


def set_trace_events(events, ctx=None):
    """Per-kernel timing hook of a handle: a list of up to 16 torch.cuda.Event(enable_timing=True)
    (or [] to switch off); the i-th kernel of csf_sparse_ffn_layer gets events 2i (start) and
    2i+1 (end), recorded by the runtime at the kernel's own start and end.  torch creates the
    underlying HIP event on its first record(), so record each event once beforehand."""
    (ctx or context()).set_trace_events(events)


def sparse_ffn_layer(x, V, U, W1, b1, Wup, W2T, k=None, tau=None, act=RELU, y=None, scores=None,
                     idx=None, count=None, ws=None, ctx=None):
    """Predict, select (top-k if k is given, else threshold tau) and the sparse FFN for one token."""
    if (k is None) == (tau is None):
        raise ValueError("give exactly one of k (top-k) or tau (threshold)")
    _tensor(x, "x")
    if x.dim() != 1:
        raise ValueError("x must be one token, shape [d]")
    dev, dt, f, d = _ffn_weights(x, W1, b1, Wup, W2T, act)
    _tensor(x, "x", shape=(d,))
    r = V.shape[0]
    _tensor(V, "V", dtype=dt, shape=(r, d), device=dev)
    _tensor(U, "U", dtype=dt, shape=(f, r), device=dev)
    kk = -1 if k is None else int(k)
    if y is None:
        y = torch.empty(d, dtype=torch.float32, device=dev)
    _tensor(y, "y", dtype=torch.float32, shape=(d,), device=dev)
    _tensor(scores, "scores", dtype=torch.float32, shape=(f,), device=dev, optional=True)
    if idx is not None:
        _tensor(idx, "idx", dtype=torch.int32, device=dev)
        if idx.numel() < (f if kk < 0 else max(kk, 1)):
            raise ValueError("idx is too small")
    _tensor(count, "count", dtype=torch.int32, shape=(1,), device=dev, optional=True)
    code = dtype_code(dt)
    max_count = f if kk < 0 else kk
    w, wb = _workspace(workspace_size(OP_LAYER, 1, d, f, r, max_count, code), dev, ws)
    _check(lib.csf_sparse_ffn_layer(_h(ctx, dev), _ptr(x), d, f, r, act, code, _ptr(V), _ptr(U),
                                    _ptr(W1),
                                    _ptr(b1), _ptr(Wup), _ptr(W2T), kk,
                                    float(tau if tau is not None else 0.0), _ptr(y), _ptr(scores),
                                    _ptr(idx), _ptr(count), _ptr(w), wb, _stream(dev)))
    return y


def sparse_ffn_batched_union(X, W1, b1, Wup, W2T, bitmaps, act=RELU, semantics=SEM_PER_TOKEN,
                             path=PATH_AUTO, Y=None, union_count=None, ws=None, ctx=None):
    """Sparse FFN of the B tokens X [B, d] reading the union of their sets once.

    bitmaps [B, ceil(f/32)] int32 (the bit patterns of csf_select_*'s bitmap output).  Returns
    (Y [B, d] float32, path taken: PATH_GATHER or PATH_MFMA); union_count ([1] int32, optional)
    receives the union size on the device."""
    _tensor(X, "X")
    if X.dim() != 2:
        raise ValueError("X must be [B, d]")
    dev, dt, f, d = _ffn_weights(X, W1, b1, Wup, W2T, act)
    B = X.shape[0]
    _tensor(X, "X", shape=(B, d))
    _tensor(bitmaps, "bitmaps", dtype=torch.int32, shape=(B, (f + 31) // 32), device=dev)
    if Y is None:
        Y = torch.empty(B, d, dtype=torch.float32, device=dev)
    _tensor(Y, "Y", dtype=torch.float32, shape=(B, d), device=dev)
    _tensor(union_count, "union_count", dtype=torch.int32, shape=(1,), device=dev, optional=True)
    code = dtype_code(dt)
    c = ctx if ctx is not None else context(dev)
    w, wb = _workspace(workspace_size(OP_BATCHED_UNION, B, d, f, 0, 0, code, ctx=c), dev, ws)
    taken = ctypes.c_int(0)
    _check(lib.csf_sparse_ffn_batched_union(_h(c, dev), _ptr(X), B, d, f, act, code, _ptr(W1),
                                            _ptr(b1),
                                            _ptr(Wup), _ptr(W2T), _ptr(bitmaps), int(semantics),
                                            int(path), _ptr(Y), _ptr(union_count),
                                            ctypes.byref(taken), _ptr(w), wb, _stream(dev)))
    return Y, taken.value


def sparse_ffn_batched_layer(X, V, U, W1, b1, Wup, W2T, k=None, tau=None, act=RELU,
                             semantics=SEM_PER_TOKEN, path=PATH_AUTO, Y=None, bitmaps=None,
                             union_count=None, ws=None, ctx=None):
    """Predict, select (top-k if k is given, else threshold tau) and the batched union FFN for
    the B tokens X [B, d].  Returns (Y [B, d] float32, path taken)."""
    if (k is None) == (tau is None):
        raise ValueError("give exactly one of k (top-k) or tau (threshold)")
    _tensor(X, "X")
    if X.dim() != 2:
        raise ValueError("X must be [B, d]")
    dev, dt, f, d = _ffn_weights(X, W1, b1, Wup, W2T, act)
    B = X.shape[0]
    _tensor(X, "X", shape=(B, d))
    r = V.shape[0]
    _tensor(V, "V", dtype=dt, shape=(r, d), device=dev)
    _tensor(U, "U", dtype=dt, shape=(f, r), device=dev)
    kk = -1 if k is None else int(k)
    if Y is None:
        Y = torch.empty(B, d, dtype=torch.float32, device=dev)
    _tensor(Y, "Y", dtype=torch.float32, shape=(B, d), device=dev)
    _tensor(bitmaps, "bitmaps", dtype=torch.int32, shape=(B, (f + 31) // 32), device=dev,
            optional=True)
    _tensor(union_count, "union_count", dtype=torch.int32, shape=(1,), device=dev, optional=True)
    code = dtype_code(dt)
    max_count = f if kk < 0 else kk
    c = ctx if ctx is not None else context(dev)
    w, wb = _workspace(workspace_size(OP_BATCHED_LAYER, B, d, f, r, max_count, code, ctx=c), dev,
                       ws)
    taken = ctypes.c_int(0)
    _check(lib.csf_sparse_ffn_batched_layer(
        _h(c, dev), _ptr(X), B, d, f, r, act, code, _ptr(V), _ptr(U), _ptr(W1), _ptr(b1), _ptr(Wup), _ptr(W2T),
        kk, float(tau if tau is not None else 0.0), int(semantics), int(path), _ptr(Y),
        _ptr(bitmaps), _ptr(union_count), ctypes.byref(taken), _ptr(w), wb, _stream(dev)))
    return Y, taken.value


class StackLayers:
    """The blocks of a stack (objects with V, U, W1, b1, Wup, W2T device tensors), checked once and
    packed into the C ABI's array of weight pointers, for repeated stack_forward calls: checking
    and packing every block's tensors on each call costs the host about as much as enqueueing the
    stack.  Keeps references to the tensors; they must not be resized or moved while it is used."""

    def __init__(self, layers, act=RELU):
        self.layers = list(layers)
        self.act = act
        nl = len(self.layers)
        self.n = nl
        self.arr = (LayerWeights * max(nl, 1))()
        if nl == 0:
            self.device = self.dtype = None
            self.d = self.f = self.r = 0
            return
        L0 = self.layers[0]
        _tensor(L0.W1, "W1")
        dev, dt = L0.W1.device, L0.W1.dtype
        f, d = L0.W1.shape
        r = L0.V.shape[0]
        for i, Lw in enumerate(self.layers):
            _ffn_weights(torch.empty(0, dtype=dt, device=dev), Lw.W1, Lw.b1, Lw.Wup, Lw.W2T, act)
            _tensor(Lw.W1, "W1", shape=(f, d))
            _tensor(Lw.V, "V", dtype=dt, shape=(r, d), device=dev)
            _tensor(Lw.U, "U", dtype=dt, shape=(f, r), device=dev)
            self.arr[i] = LayerWeights(Lw.V.data_ptr(), Lw.U.data_ptr(), Lw.W1.data_ptr(),
                                       None if Lw.Wup is None else Lw.Wup.data_ptr(),
                                       Lw.W2T.data_ptr(), None if Lw.b1 is None else Lw.b1.data_ptr())
        self.device, self.dtype, self.d, self.f, self.r = dev, dt, d, f, r

    def __len__(self):
        return self.n


def stack_forward(x, layers, k=None, tau=None, act=RELU, lookahead=False, norm=True, eps=1e-6,
                  x_log=None, xhat_log=None, idx_log=None, count_log=None, side_stream=None,
                  ws=None, graph=False, ctx=None):
    """Run x [B, d] (float32, updated in place) through the residual blocks `layers` (a list of
    objects with V, U, W1, b1, Wup, W2T device tensors, or a StackLayers made from one with the
    same act).  lookahead: each layer's set is predicted from the previous layer's input on
    `side_stream` (a torch.cuda.Stream; required).  graph: enqueue the stack as one replayed HIP
    graph (captured when the arguments change; pass the same `ws` and tensors to reuse it).
    Returns x."""
    if (k is None) == (tau is None):
        raise ValueError("give exactly one of k (top-k) or tau (threshold)")
    _tensor(x, "x", dtype=torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [B, d]")
    B, d = x.shape
    dev = x.device
    if not isinstance(layers, StackLayers):
        layers = StackLayers(layers, act)
    elif layers.act != act:
        raise ValueError("the StackLayers were checked for another activation")
    nl = len(layers)
    if nl == 0:
        return x
    if layers.device != dev or layers.d != d:
        raise ValueError(f"the layers ({layers.device}, d = {layers.d}) do not match x "
                         f"({dev}, d = {d})")
    dt, f, r, arr = layers.dtype, layers.f, layers.r, layers.arr
    kk = -1 if k is None else int(k)
    stride = f if kk < 0 else max(kk, 1)
    _tensor(x_log, "x_log", dtype=torch.float32, shape=(nl, B, d), device=dev, optional=True)
    _tensor(xhat_log, "xhat_log", dtype=dt, shape=(nl, B, d), device=dev, optional=True)
    _tensor(idx_log, "idx_log", dtype=torch.int32, shape=(nl, B, stride), device=dev, optional=True)
    _tensor(count_log, "count_log", dtype=torch.int32, shape=(nl, B), device=dev, optional=True)
    if lookahead and side_stream is None:
        raise ValueError("look-ahead needs a side stream")
    code = dtype_code(dt)
    max_count = f if kk < 0 else kk
    w, wb = _workspace(workspace_size(OP_STACK, B, d, f, r, max_count, code), dev, ws)
    side = None if side_stream is None else ctypes.c_void_p(side_stream.cuda_stream)
    _check(lib.csf_stack_forward(_h(ctx, dev), arr, nl, d, f, r, act, code, _ptr(x), B,
                                 (STACK_LOOKAHEAD if lookahead else STACK_SYNC) |
                                 (STACK_GRAPH if graph else 0), kk,
                                 float(tau if tau is not None else 0.0), 1 if norm else 0,
                                 float(eps), _ptr(x_log), _ptr(xhat_log), _ptr(idx_log),
                                 _ptr(count_log), _ptr(w), wb, _stream(dev), side))
    return x


def sparse_ffn_layer_hot(x, V, U_cold, W1, b1, Wup, W2T, hot, k=None, tau=None, act=RELU, y=None,
                         scores=None, idx=None, count=None, ws=None, ctx=None):
    """One token through a hot-first layer: neurons 0 .. hot-1 always, plus the top-k (or >= tau)
    of the cold neurons scored by the predictor with up rows U_cold [f - hot, r]."""
    if (k is None) == (tau is None):
        raise ValueError("give exactly one of k (top-k) or tau (threshold)")
    _tensor(x, "x")
    if x.dim() != 1:
        raise ValueError("x must be one token, shape [d]")
    dev, dt, f, d = _ffn_weights(x, W1, b1, Wup, W2T, act)
    _tensor(x, "x", shape=(d,))
    r = V.shape[0]
    hot = int(hot)
    _tensor(V, "V", dtype=dt, shape=(r, d), device=dev)
    _tensor(U_cold, "U_cold", dtype=dt, shape=(f - hot, r), device=dev)
    kk = -1 if k is None else int(k)
    if y is None:
        y = torch.empty(d, dtype=torch.float32, device=dev)
    _tensor(y, "y", dtype=torch.float32, shape=(d,), device=dev)
    _tensor(scores, "scores", dtype=torch.float32, shape=(f - hot,), device=dev, optional=True)
    max_count = hot + (f - hot if kk < 0 else kk)
    if idx is not None:
        _tensor(idx, "idx", dtype=torch.int32, device=dev)
        if idx.numel() < max(max_count, 1):
            raise ValueError("idx is too small")
    _tensor(count, "count", dtype=torch.int32, shape=(1,), device=dev, optional=True)
    code = dtype_code(dt)
    w, wb = _workspace(workspace_size(OP_LAYER, 1, d, f, r, max_count, code), dev, ws)
    _check(lib.csf_sparse_ffn_layer_hot(_h(ctx, dev), _ptr(x), d, f, r, act, code, _ptr(V),
                                        _ptr(U_cold),
                                        _ptr(W1), _ptr(b1), _ptr(Wup), _ptr(W2T), hot, kk,
                                        float(tau if tau is not None else 0.0), _ptr(y),
                                        _ptr(scores), _ptr(idx), _ptr(count), _ptr(w), wb,
                                        _stream(dev)))
    return y


# ------------------------------------------------------------------------------------------------
# attention-head sparsity
# ------------------------------------------------------------------------------------------------
def attention_workspace_size(op, d, H, dh, r, Tmax, max_heads, dtype=F16) -> int:
    return int(lib.csf_attention_workspace_size(op, d, H, dh, r, Tmax, max_heads, dtype))


def _attn_weights(x, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, lens):
    _tensor(x, "x")
    if x.dim() != 1:
        raise ValueError("x must be one token, shape [d]")
    dev, dt = x.device, x.dtype
    H, Tmax, dh = Kc.shape
    d = x.shape[0]
    for name, W in (("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("WoT", WoT)):
        _tensor(W, name, dtype=dt, shape=(H * dh, d), device=dev)
    for name, b in (("bq", bq), ("bk", bk), ("bv", bv)):
        _tensor(b, name, dtype=torch.float32, shape=(H * dh,), device=dev, optional=True)
    _tensor(Kc, "Kc", dtype=dt, shape=(H, Tmax, dh), device=dev)
    _tensor(Vc, "Vc", dtype=dt, shape=(H, Tmax, dh), device=dev)
    _tensor(lens, "lens", dtype=torch.int32, shape=(H,), device=dev)
    return dev, dt, d, H, dh, Tmax


def sparse_attention_decode(x, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, lens, heads=None, count=None,
                            kv_all=False, o=None, y=None, ws=None, ctx=None):
    """One decode step of multi-head attention over the heads in `heads` (int32 device list;
    None = every head, the dense step).  Kc, Vc [H, Tmax, dh] and lens [H] are updated in place.
    Returns y [d] float32."""
    dev, dt, d, H, dh, Tmax = _attn_weights(x, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, lens)
    if heads is None:
        max_heads = H
        if count is not None:
            raise ValueError("count needs a head list")
    else:
        _tensor(heads, "heads", dtype=torch.int32, device=dev)
        max_heads = heads.numel()
    _tensor(count, "count", dtype=torch.int32, shape=(1,), device=dev, optional=True)
    _tensor(o, "o", dtype=torch.float32, shape=(max_heads, dh), device=dev, optional=True)
    if y is None:
        y = torch.empty(d, dtype=torch.float32, device=dev)
    _tensor(y, "y", dtype=torch.float32, shape=(d,), device=dev)
    code = dtype_code(dt)
    w, wb = _workspace(attention_workspace_size(OP_ATTN_DECODE, d, H, dh, 0, Tmax, max_heads, code),
                       dev, ws)
    _check(lib.csf_sparse_attention_decode(_h(ctx, dev), _ptr(x), d, H, dh, code, _ptr(Wq),
                                           _ptr(Wk), _ptr(Wv),
                                           _ptr(bq), _ptr(bk), _ptr(bv), _ptr(WoT), _ptr(Kc),
                                           _ptr(Vc), Tmax, _ptr(lens), _ptr(heads), _ptr(count),
                                           max_heads, 1 if kv_all else 0, _ptr(o), _ptr(y), _ptr(w),
                                           wb, _stream(dev)))
    return y


def sparse_attention_layer(x, Vp, Up, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, lens, k=None, tau=None,
                           kv_all=False, scores=None, heads=None, count=None, o=None, y=None,
                           ws=None, ctx=None):
    """Head predictor, top-k (or >= tau) head selection and the decode step over the selected
    heads, for one token.  Returns y [d] float32."""
    if (k is None) == (tau is None):
        raise ValueError("give exactly one of k (top-k) or tau (threshold)")
    dev, dt, d, H, dh, Tmax = _attn_weights(x, Wq, Wk, Wv, bq, bk, bv, WoT, Kc, Vc, lens)
    r = Vp.shape[0]
    _tensor(Vp, "Vp", dtype=dt, shape=(r, d), device=dev)
    _tensor(Up, "Up", dtype=dt, shape=(H, r), device=dev)
    kk = -1 if k is None else int(k)
    max_heads = H if kk < 0 else kk
    _tensor(scores, "scores", dtype=torch.float32, shape=(H,), device=dev, optional=True)
    if heads is not None:
        _tensor(heads, "heads", dtype=torch.int32, device=dev)
        if heads.numel() < max(max_heads, 1):
            raise ValueError("heads is too small")
    _tensor(count, "count", dtype=torch.int32, shape=(1,), device=dev, optional=True)
    _tensor(o, "o", dtype=torch.float32, shape=(max_heads, dh), device=dev, optional=True)
    if y is None:
        y = torch.empty(d, dtype=torch.float32, device=dev)
    _tensor(y, "y", dtype=torch.float32, shape=(d,), device=dev)
    code = dtype_code(dt)
    w, wb = _workspace(attention_workspace_size(OP_ATTN_LAYER, d, H, dh, r, Tmax, max_heads, code),
                       dev, ws)
    _check(lib.csf_sparse_attention_layer(_h(ctx, dev), _ptr(x), d, H, dh, r, code, _ptr(Vp),
                                          _ptr(Up), _ptr(Wq),
                                          _ptr(Wk), _ptr(Wv), _ptr(bq), _ptr(bk), _ptr(bv),
                                          _ptr(WoT), _ptr(Kc), _ptr(Vc), Tmax, _ptr(lens), kk,
                                          float(tau if tau is not None else 0.0),
                                          1 if kv_all else 0, _ptr(scores), _ptr(heads),
                                          _ptr(count), _ptr(o), _ptr(y), _ptr(w), wb, _stream(dev)))
    return y

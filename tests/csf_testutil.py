"""Helpers shared by the GPU parity tests: tensor <-> oracle storage and the FFN tolerance.

FFN tolerance.  The stated bar is a normwise max relative error of 1e-5 (float32 weights) and
2e-2 (binary16 / bfloat16 weights), ||y_gpu - y_oracle||_inf / ||y_oracle||_inf.  Both sides read
identical weight bytes, so the only difference is float32 versus double accumulation: each h_j is
a d-term float32 dot product and each y_c a count-term float32 sum, with relative error of order
sqrt(n) * 2^-24 per sum against the sum of magnitudes.  At the largest shapes here (d = 12288,
counts up to 49152) that is below 1e-5 of ||y||_inf with a wide margin, so a second, tighter bound
of 1e-4 is also asserted for the 16-bit types: it catches a dropped or doubled neuron, which the
2e-2 bar alone would not at counts in the thousands.
"""
import sys

import numpy as np
import torch

from oracle import oracle as orc

TOL_STATED = {torch.float32: 1e-5, torch.float16: 2e-2, torch.bfloat16: 2e-2}
TOL_TIGHT = {torch.float32: 1e-5, torch.float16: 1e-4, torch.bfloat16: 1e-4}
ORC_DT = {torch.float32: orc.F32, torch.float16: orc.F16, torch.bfloat16: orc.BF16}


def announce(what: str):
    """Name the case on the real stderr before a GPU step, so a crash still says which one."""
    sys.__stderr__.write(f"[gpu-case] {what}\n")
    sys.__stderr__.flush()


def to_orc(t: torch.Tensor) -> np.ndarray:
    """Tensor -> numpy array in the oracle's storage convention (bfloat16 as raw uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def normwise_err(y_gpu: torch.Tensor, y_ref: np.ndarray) -> float:
    g = y_gpu.detach().double().cpu().numpy().reshape(y_ref.shape)
    scale = np.abs(y_ref).max()
    if scale == 0.0:
        return 0.0 if not np.any(g) else float("inf")
    return float(np.abs(g - y_ref).max() / scale)


def assert_ffn_close(y_gpu: torch.Tensor, y_ref: np.ndarray, dtype: torch.dtype, what=""):
    err = normwise_err(y_gpu, y_ref)
    assert err <= TOL_STATED[dtype], f"{what}: normwise error {err:.3g} > {TOL_STATED[dtype]}"
    assert err <= TOL_TIGHT[dtype], f"{what}: normwise error {err:.3g} > {TOL_TIGHT[dtype]}"
    return err


def layer_to_orc(L):
    """Oracle-side copies of a workloads.Layer."""
    return dict(V=to_orc(L.V), U=to_orc(L.U), W1=to_orc(L.W1), b1=to_orc(L.b1),
                Wup=None if L.Wup is None else to_orc(L.Wup), W2T=to_orc(L.W2T),
                act=L.cfg.act, dt=ORC_DT[L.cfg.dtype])

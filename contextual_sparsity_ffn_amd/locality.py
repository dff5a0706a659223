"""Static locality: per-neuron firing frequency, hot-first neuron order, the cold predictor rows.

"Contextual Sparsity and Activation Predictors", section "Static locality: hot and cold neurons":
neuron activation across inputs follows a power law -- a small set fires for almost every token,
the long tail only for particular inputs -- and the static split (which neurons are always
computed) composes with the predictor (which of the rest this token needs).  "Activation
sparsity", section "Hot and cold neuron split with per-layer predictors": neurons are ranked by how
often they fire on profiling inputs.

Offline preparation of a layer for csf_sparse_ffn_layer_hot, run once per layer:
  freq = firing_frequency(layer, profile_tokens)      # the library's dense kernel, on the GPU
  order = hot_first_order(freq)                       # most frequent first, ties by index
  hot_layer = reorder(layer, order)                   # rows of U, W1, Wup, W2T and b1 permuted
  hot = hot_count(freq, threshold)                    # neurons that fire at least that often
  U_cold = hot_layer.U[hot:]                          # the predictor's rows of the cold neurons
Reordering permutes neurons, so the layer computes the same function; only the set chosen for a
token changes (the hot block is always in it).
"""
from __future__ import annotations

import torch

from . import _lib
from .workloads import Layer


def firing_frequency(layer: Layer, tokens: torch.Tensor, batch: int = 64) -> torch.Tensor:
    """Fraction of `tokens` [n, d] for which each neuron's activation is non-zero (float32 [f])."""
    f = layer.W1.shape[0]
    counts = torch.zeros(f, dtype=torch.float64, device=tokens.device)
    h = torch.empty(batch, f, dtype=torch.float32, device=tokens.device)
    for i in range(0, tokens.shape[0], batch):
        X = tokens[i:i + batch].contiguous()
        hb = h[:X.shape[0]]
        _lib.dense_ffn(X, layer.W1, layer.b1, layer.Wup, layer.W2T, act=layer.cfg.act, h=hb)
        counts += (hb != 0).sum(0, dtype=torch.float64)
    return (counts / tokens.shape[0]).float()


def hot_first_order(freq: torch.Tensor) -> torch.Tensor:
    """Neuron order, most frequently firing first; equal frequencies keep index order."""
    return torch.sort(-freq.double(), stable=True).indices


def hot_count(freq: torch.Tensor, threshold: float = 0.5, cap: int | None = None) -> int:
    """Neurons that fire for at least `threshold` of the profiling tokens (at most `cap`)."""
    n = int((freq >= threshold).sum())
    return n if cap is None else min(n, int(cap))


def reorder(layer: Layer, order: torch.Tensor) -> Layer:
    """The layer with its neurons in `order`: rows of U, W1, Wup, W2T and entries of b1 permuted
    (V is unchanged: it feeds the predictor's hidden layer, not the neurons)."""
    o = order.to(layer.W1.device)
    pick = lambda t: None if t is None else t.index_select(0, o).contiguous()
    return Layer(layer.cfg, layer.V, pick(layer.U), pick(layer.W1), pick(layer.b1), pick(layer.Wup),
                 pick(layer.W2T))

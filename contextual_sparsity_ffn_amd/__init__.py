"""contextual_sparsity_ffn_amd -- the contextual-sparsity sparse FFN step on AMD MI355X (gfx950).

The compute path is the HIP library ``libcsf.so`` (C ABI: ``include/csf.h``).  This package holds
its sources (``csrc/``), the in-tree build (``build.py``), a thin ctypes binding (``_lib``) whose
functions carry the C entry points' names, and the seeded synthetic workloads (``workloads``).
"""
from ._lib import (BF16, F16, F32, FFN_SKIP_ZERO_H, PATH_AUTO, PATH_GATHER, PATH_MFMA, REGLU, RELU,
                   SEM_PER_TOKEN, SEM_UNION, SILU, SWIGLU, Context, CsfError, context, dense_ffn, k_from_ratio, lib, predict_active,
                   select_threshold, select_topk, set_ffn_flags, set_ffn_gate_threshold, set_trace_events, sparse_ffn,
                   sparse_ffn_batched_layer, sparse_ffn_batched_union, sparse_ffn_layer,
                   sparse_ffn_layer_hot, stack_forward, StackLayers, workspace_size,
                   attention_workspace_size, sparse_attention_decode, sparse_attention_layer)

__all__ = ["BF16", "F16", "F32", "FFN_SKIP_ZERO_H", "PATH_AUTO", "PATH_GATHER", "PATH_MFMA", "REGLU", "RELU",
           "SEM_PER_TOKEN", "SEM_UNION", "SILU", "SWIGLU", "Context", "CsfError", "context", "dense_ffn", "k_from_ratio", "lib",
           "predict_active", "select_threshold", "select_topk", "set_ffn_flags",
           "set_ffn_gate_threshold", "set_trace_events",
           "sparse_ffn",
           "sparse_ffn_batched_layer", "sparse_ffn_batched_union", "sparse_ffn_layer",
           "sparse_ffn_layer_hot", "stack_forward", "StackLayers", "workspace_size",
           "attention_workspace_size", "sparse_attention_decode", "sparse_attention_layer"]

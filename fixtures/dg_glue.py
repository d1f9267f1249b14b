"""Feeding the synthetic workloads into the GPU library's binding.

The binding module is passed in (this module imports nothing of the product),
so tests and bench share one recipe for building a handle from a Workload.
"""
from __future__ import annotations

import numpy as np

from . import Workload, model_tensor, prompt_ids, tensor_shape

KIND_NAMES = ("embed", "wq", "wk", "wv", "wo", "wr", "wg", "wu", "wd", "sc_wg", "sc_wu", "sc_wd")


def make_cfg(dg, w: Workload, capture_mask: int = 0, max_ctx: int | None = None,
             max_batch: int = 1):
    act = dg.DG_F32 if w.act == "f32" else dg.DG_BF16
    exp = {"f32": dg.DG_F32, "bf16": dg.DG_BF16, "fp8": dg.DG_FP8_E4M3,
           "mxfp4": getattr(dg, "DG_MXFP4", None)}[w.experts]
    return dg.make_cfg(w.n_layers, w.d_model, w.n_q_heads, w.n_kv_heads, w.head_dim,
                       w.n_experts, w.top_k, w.d_ff, w.vocab, w.canvas,
                       max_ctx if max_ctx is not None else w.max_ctx, w.rope_base, w.rms_eps,
                       w.temperature, act, exp, capture_mask, max_batch, int(w.self_cond),
                       w.sc_ff)


def tensor_fn(w: Workload):
    def fn(kind: int, layer: int, expert):
        name = KIND_NAMES[kind]
        if expert is None:
            return model_tensor(w, name, layer)
        if expert == -1 and w.experts in ("fp8", "mxfp4") and name in ("wg", "wu", "wd"):
            parts = [model_tensor(w, name, layer, expert=e) for e in range(w.n_experts)]
            codes = np.ascontiguousarray(np.stack([p[0] for p in parts]))
            scales = np.ascontiguousarray(np.stack([p[1] for p in parts]))
            return codes, scales
        if expert == -1:
            return model_tensor(w, name, layer)
        return model_tensor(w, name, layer, expert=expert)
    return fn


def build_handle(dg, w: Workload, capture_mask: int = 0, max_ctx: int | None = None,
                 max_batch: int = 1):
    h = dg.dg_create(make_cfg(dg, w, capture_mask, max_ctx, max_batch))
    try:
        dg.load_weights(h, w.n_layers, w.n_experts, tensor_fn(w), self_cond=w.self_cond)
    except Exception:
        dg.dg_destroy(h)
        raise
    return h

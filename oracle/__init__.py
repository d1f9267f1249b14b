"""CPU oracle for the DiffusionGemma canvas-denoising step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or calls this package; only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` do.

It is a plain, slow, fp64 implementation of what one denoise pass computes,
written from the pages' description of the method: every function cites the
passage it follows.  Library primitives (numpy matmul, sort, exp/log) serve
as single steps; there is no blocking, fusion or reordering beyond what each
definition states.

Pages cited (titles as published):
  [TR]  "DiffusionGemma" technical-report summary (hyper.ai paper page),
        sections Dataset / Method / Experiment, with its display equations:
        forward process, Step map, decoder logits, update equations.
  [AS]  "Google's DiffusionGemma Generates 256 Tokens at Once, 4x Faster Than
        Any LLM" (alphasignal), sections "The problem it's solving", "How text
        diffusion actually works" (steps 1-3) and the paragraph on
        bidirectional attention.

Readings of points the pages leave open are listed in the module docstrings
where they are used (e.g. RMSNorm epsilon, RoPE variant, GQA grouping, tied
LM head, sampler schedule, Philox counter layout).

Pinning: every function here is checked by ``tests/test_oracle_*.py`` against
brute force, closed forms, invariants or library routines.  The whole-model
output has no value printed on any page for any input, so at the model level
the oracle is "parity unpinned" against the pages; it is pinned piece by piece.
"""
from .numerics import (round_bf16, e4m3_round, e4m3_value_of_code, rmsnorm, rope,
                       softmax, silu)
from .philox import philox4x32_10, init_canvas, gumbel_uniforms, renoise_tokens
from . import eb_sampler
from .model import (OracleModel, attention, route_topk, moe_ffn, lm_head_stats,
                    sampler_update, lock_count, gumbel_noise)

__all__ = [
    "round_bf16", "e4m3_round", "e4m3_value_of_code", "rmsnorm", "rope", "softmax", "silu",
    "philox4x32_10", "init_canvas", "gumbel_uniforms", "OracleModel", "attention",
    "route_topk", "moe_ffn", "lm_head_stats", "sampler_update", "lock_count", "gumbel_noise",
    "renoise_tokens", "eb_sampler",
]

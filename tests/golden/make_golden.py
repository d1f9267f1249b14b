"""Write the oracle's expected values for the full-width parity tests.

Calls only the CPU oracle (``oracle/``) on inputs from the seeded generator
(``fixtures/``); nothing here touches the GPU library.  Outputs are small
.npz files next to this script: per-position statistics and decisions with
their margins, routing with margins, sampled logits and sampled K/V rows.

    python tests/golden/make_golden.py moe26b_2layer
    python tests/golden/make_golden.py moe26b_fp8_long_2layer
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import fixtures as fx  # noqa: E402
from oracle.model import OracleModel  # noqa: E402
from oracle.philox import init_canvas  # noqa: E402
from oracle.weights import FixtureWeights  # noqa: E402

N_LOGIT_SAMPLES = 16384
N_KV_SAMPLES = 64


def _step_record(prefix, res, logits_rng, V):
    z = res.logits
    C = z.shape[0]
    rows = logits_rng.integers(0, C, N_LOGIT_SAMPLES)
    cols = logits_rng.integers(0, V, N_LOGIT_SAMPLES)
    # also every row's argmax and a near-max column, where relative error matters most
    rows = np.concatenate([rows, np.arange(C)])
    cols = np.concatenate([cols, res.stats.argmax])
    out = {
        f"{prefix}_m": res.stats.m, f"{prefix}_argmax": res.stats.argmax,
        f"{prefix}_lse": res.stats.lse, f"{prefix}_conf": res.stats.conf,
        f"{prefix}_top2_gap": res.stats.top2_gap, f"{prefix}_redraw": res.redraw,
        f"{prefix}_redraw_gap": res.redraw_gap, f"{prefix}_canvas_out": res.canvas,
        f"{prefix}_mask_out": res.mask, f"{prefix}_cut": np.array([res.sampler.cut_low, res.sampler.cut_high]),
        f"{prefix}_logit_rows": rows.astype(np.int32), f"{prefix}_logit_cols": cols.astype(np.int32),
        f"{prefix}_logit_vals": z[rows, cols],
    }
    for l, (idx, g, mg) in enumerate(zip(res.route_idx, res.route_gates, res.route_margin)):
        out[f"{prefix}_route_idx_{l}"] = idx
        out[f"{prefix}_route_gates_{l}"] = g
        out[f"{prefix}_route_margin_{l}"] = mg
    return out


def _kv_samples(m, rng, n_ctx):
    pos = np.sort(rng.choice(n_ctx, size=min(N_KV_SAMPLES, n_ctx), replace=False))
    out = {"kv_pos": pos.astype(np.int64)}
    for l in range(m.L):
        out[f"k_{l}"] = m.K[l][:, pos, :]
        out[f"v_{l}"] = m.V[l][:, pos, :]
    return out


def moe26b_2layer():
    """The 26B-class MoE denoiser truncated to layers 0-1, at full widths, P = 8192:
    prefill, canvas init, pass 0, and pass 1 teacher-forced from the oracle's state."""
    w = fx.MOE26B.with_(name="moe26b_2layer", n_layers=2)
    t0 = time.time()
    m = OracleModel(w, FixtureWeights(w))
    m.prefill(fx.prompt_ids(w))
    print(f"prefill {time.time() - t0:.1f}s", flush=True)
    rng = np.random.default_rng(20260)
    out = {"seed": np.array(w.seed), "T": np.array(w.T)}
    out.update(_kv_samples(m, rng, m.n_ctx))
    # layer-0 routing margins of the prompt tokens: a layer-1 K/V row can only be trusted
    # to match when its token's layer-0 routing is not a near tie
    out["kv_margin0"] = m.enc_route_margin[0][out["kv_pos"]]
    canvas = init_canvas(w.seed, 0, w.canvas, w.vocab)
    mask = np.zeros(w.canvas, np.uint8)
    out["canvas_in_0"], out["mask_in_0"] = canvas, mask
    for s in range(2):
        res = m.denoise_step(canvas, mask, s, w.T, w.seed, keep_logits=True)
        out.update(_step_record(f"s{s}", res, rng, w.vocab))
        print(f"pass {s} {time.time() - t0:.1f}s", flush=True)
        canvas, mask = res.canvas, res.mask
        if s == 0:
            out["canvas_in_1"], out["mask_in_1"] = canvas, mask
    np.savez_compressed(os.path.join(HERE, "moe26b_2layer.npz"), **out)


def moe26b_fp8_long_2layer():
    """The long-context fp8-expert variant truncated to layers 0-1, P = 131072.

    A whole prefill of two layers over 131072 tokens is out of the oracle's reach (its
    causal attention alone is ~70 TFLOP), so this stores what the oracle can compute
    exactly: the layer-0 cache (the projection of the embedded prompt), sampled at 64
    positions; the layer-1 cache at the same positions, from layer 0 run at those rows
    against the whole layer-0 cache; the canvas inits of blocks 0 and 1; and the cache rows
    a commit of block 0's initial canvas appends at both layers (sampled at 64 rows), with
    the layer-0 routing margins that gate the layer-1 rows."""
    from oracle.numerics import rmsnorm

    w = fx.MOE26B_FP8_LONG.with_(name="moe26b_fp8_long_2layer", n_layers=2)
    t0 = time.time()
    m = OracleModel(w, FixtureWeights(w, cache_experts=False))
    E = m.W.embed()
    ids = fx.prompt_ids(w)
    P, C = w.prompt_len, w.canvas
    n_tot = P + C
    K0 = np.empty((w.n_kv_heads, n_tot, w.head_dim))
    V0 = np.empty_like(K0)
    step = 8192
    for c0 in range(0, P, step):
        pos = np.arange(c0, min(P, c0 + step))
        K0[:, pos], V0[:, pos] = m.kv_rows(0, m._act(rmsnorm(E[ids[pos]], w.rms_eps)), pos)
    print(f"layer-0 prompt cache {time.time() - t0:.1f}s", flush=True)
    rng = np.random.default_rng(20263)
    out = {"seed": np.array(w.seed), "T": np.array(w.T)}
    kv_pos = np.sort(rng.choice(P, size=N_KV_SAMPLES, replace=False))
    out["kv_pos"] = kv_pos.astype(np.int64)
    out["k_0"], out["v_0"] = K0[:, kv_pos], V0[:, kv_pos]
    m.K[0], m.V[0] = K0[:, :P], V0[:, :P]
    h1, margin0 = m.encoder_layer_rows(0, E[ids[kv_pos]], kv_pos)
    out["k_1"], out["v_1"] = m.kv_rows(1, m._act(rmsnorm(h1, w.rms_eps)), kv_pos)
    out["kv_margin0"] = margin0
    print(f"layer-1 prompt cache samples {time.time() - t0:.1f}s", flush=True)
    for blk in range(2):
        out[f"b{blk}_canvas_in"] = init_canvas(w.seed, blk, C, w.vocab)
    # commit of block 0's initial canvas at positions P..P+C-1
    tokens = out["b0_canvas_in"]
    cpos = np.arange(P, P + C)
    K0[:, cpos], V0[:, cpos] = m.kv_rows(0, m._act(rmsnorm(E[tokens], w.rms_eps)), cpos)
    m.K[0], m.V[0] = K0, V0
    h1, cmargin0 = m.encoder_layer_rows(0, E[tokens], cpos)
    k1, v1 = m.kv_rows(1, m._act(rmsnorm(h1, w.rms_eps)), cpos)
    rows = np.sort(rng.choice(C, size=N_KV_SAMPLES, replace=False))
    out["commit_tokens"] = tokens
    out["commit_rows"] = rows.astype(np.int64)
    out["commit_k_0"], out["commit_v_0"] = K0[:, P + rows], V0[:, P + rows]
    out["commit_k_1"], out["commit_v_1"] = k1[:, rows], v1[:, rows]
    out["commit_margin0"] = cmargin0[rows]
    print(f"commit rows {time.time() - t0:.1f}s", flush=True)
    np.savez_compressed(os.path.join(HERE, "moe26b_fp8_long_2layer.npz"), **out)


if __name__ == "__main__":
    for name in sys.argv[1:]:
        globals()[name]()

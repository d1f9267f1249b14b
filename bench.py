"""Throughput of the canvas denoising step on one MI355X.

Workload: the 26B-class synthetic MoE denoiser in bf16 (30 layers, d=2816,
16/8 heads of dim 128, 128 experts top-8 with FFN width 704, vocabulary
262144), random-init N(0, 0.02) weights from the seeded generator, a prompt of
8192 uniform-random ids prefilled once, one 256-token canvas.

A step is one denoise pass over the canvas (embedding, 30 x [RMSNorm, QKV +
RoPE + cache write, attention over the 8448 keys, output projection, RMSNorm,
router, permutation, expert GEMMs, combine], final norm, LM head with the
streaming vocabulary statistics, lock / redraw sampler), cycling through the
12-pass block schedule; the canvas initialisation is part of the first pass
of every block.  value = canvas tokens per second of denoise passes (256 per
pass).  Also reported: output tokens per second of whole 256-token blocks
(12 passes, with and without the commit), per-kernel-class times from HIP
events recorded on the stream inside the timed region, the roofline of the
dominant kernel (the expert gate/up GEMM), and the CPU oracle timed on a
bounded sample of the same pass.  Further lines in the same JSON object: the
entropy-bounded sampler, batches of 1-16 canvases, the same model with the
self-conditioning block, the attention entry point alone (4096 + 256 keys),
one MoE layer alone (256 tokens, all 128 experts; bf16 and MX FP4 experts), the
same model with MX FP4 experts, and the long-context fp8 model (prompt 131072,
four canvases with commits), each with its roofline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def moe1_algorithmic_bytes(w, n_active_experts):
    """Expert gate/up weights of every expert hit, the normed activations once, H written."""
    weights = n_active_experts * w.d_model * 2 * w.d_ff * 2
    act = w.canvas * w.d_model * 2
    hid = w.canvas * w.top_k * w.d_ff * 2
    return weights + act + hid


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "denoise_pass_moe26b_hbm_traffic.txt")


def measured_traffic(label):
    """HBM bytes per launch of a kernel class from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, copy-calibrated), or None if the kernel's source file has
    changed since the counters were taken (its hash differs from the recorded one)."""
    import hashlib
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        parts = ln.split()
        if len(parts) != 5 or parts[0] != "traffic" or parts[1] != label:
            continue
        kv = dict(p.split("=", 1) for p in parts[2:])
        src = os.path.join(ROOT, "discrete_diffusion_decoding_canvas_amd", "csrc", kv["source"])
        try:
            digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        except OSError:
            return None
        return int(kv["bytes_per_launch"]) if digest == kv["sha256"] else None
    return None


def pass_flops(w, S):
    d, D, Hq, Hkv, E, k, F, V, C = (w.d_model, w.head_dim, w.n_q_heads, w.n_kv_heads,
                                    w.n_experts, w.top_k, w.d_ff, w.vocab, w.canvas)
    per_layer = 2 * C * d * (Hq + 2 * Hkv) * D + 4 * C * S * D * Hq + 2 * C * Hq * D * d \
        + 2 * C * d * E + 2 * C * k * 3 * d * F
    return w.n_layers * per_layer + 2 * C * d * V


def cpu_baseline(w, deep=None, seconds_budget=30.0):
    """Time the CPU oracle on a bounded sample of one denoise pass: decoder layer 0 of the
    canvas over the 8192-token prompt context, a deep decoder layer, and the LM head and
    sampler.  The deep layer (deep = (layer, its input [C, d], its prompt K and V, the GPU
    pass's expert ids there), taken from the GPU's pass since the oracle cannot run the
    30-layer prefill within the budget) stands for layers 1..n-1: past the first layers
    most tokens route to 10-20 experts, and the oracle's MoE cost follows the experts hit.  The pass time is estimated
    as layer 0 + (n_layers - 1) x (deep layer) + head; without a deep sample, n_layers x
    (layer 0) + head."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import fixtures as fx
    from oracle.model import OracleModel, lm_head_stats, gumbel_draw, sampler_update
    from oracle.numerics import rmsnorm, round_bf16
    from oracle.philox import init_canvas, gumbel_uniforms
    from oracle.weights import FixtureWeights

    w1 = w.with_(n_layers=1)
    W = FixtureWeights(w1)
    m = OracleModel(w1, W)
    m.prefill(fx.prompt_ids(w1))              # layer-0 K/V of the prompt (untimed set-up)
    for e in range(w.n_experts):              # generate weights outside the timed region
        for kind in ("wg", "wu", "wd"):
            W.expert(kind, 0, e)
    E = W.embed()
    canvas = init_canvas(w.seed, 0, w.canvas, w.vocab)
    h = E[canvas]
    t0 = time.perf_counter()
    hl, _ = m.decoder_layer(0, h)
    t_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    hn = round_bf16(rmsnorm(hl, w.rms_eps))
    z = (hn @ E.T) / w.temperature
    st = lm_head_stats(z)
    red = np.empty(w.canvas, np.int32)
    for c0 in range(0, w.canvas, 16):
        rows = np.arange(c0, c0 + 16)
        red[rows], _ = gumbel_draw(z[rows], gumbel_uniforms(w.seed, 0, 0, rows, w.vocab))
    sampler_update(canvas, np.zeros(w.canvas, np.uint8), st.conf, st.argmax, red, 0, w.T)
    t_head = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    if deep is None:
        t_pass = w.n_layers * t_layer + t_head
        sample = (f"decoder layer 0 of one pass ({t_layer:.2f} s, 256 canvas queries over "
                  f"{m.n_ctx + w.canvas} keys + MoE) and the LM head + sampler "
                  f"({t_head:.2f} s); pass = {w.n_layers} x layer + head = {t_pass:.1f} s")
    else:
        L, x_in, k_ctx, v_ctx, route = deep
        del m, W, E, h, hl, hn, z                     # layer 0's weights and the head's logits
        Wd = FixtureWeights(w)
        md = OracleModel(w, Wd)
        md.n_ctx = w.prompt_len
        md.K[L], md.V[L] = k_ctx, v_ctx
        for kind in ("wq", "wk", "wv", "wo", "wr"):   # weights outside the timed region
            Wd.dense(kind, L)
        hit = np.unique(route)                        # the experts the GPU pass hit there
        for e in hit:
            for kind in ("wg", "wu", "wd"):
                Wd.expert(kind, L, int(e))
        t0 = time.perf_counter()
        md.decoder_layer(L, x_in)
        t_deep = time.perf_counter() - t0
        t_pass = t_layer + (w.n_layers - 1) * t_deep + t_head
        sample = (f"decoder layer 0 ({t_layer:.2f} s), decoder layer {L} on the GPU pass's input "
                  f"to it ({t_deep:.2f} s, {len(hit)} experts hit), each with 256 canvas queries over "
                  f"{w.prompt_len + w.canvas} keys, and the LM head + sampler ({t_head:.2f} s); "
                  f"pass = layer 0 + {w.n_layers - 1} x layer {L} + head = {t_pass:.1f} s")
    return {"value": round(w.canvas / t_pass, 3), "unit": "canvas tok/s", "cores": threads,
            "kind": "oracle", "extrapolated": True, "sample": sample}


COPY_BYTES = 1 << 30


def copy_calibration(torch):
    """A plain device-to-device copy of COPY_BYTES, five times: the counters of a
    --pmc run over this command give the bytes each counter reports per byte moved."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}), flush=True)


def _grid_key(row):
    return f"{row.get('Grid_Size_X', row.get('Grid_Size', '?'))}x{row.get('Grid_Size_Y', '')}" \
           f"x{row.get('Grid_Size_Z', '')}"


def _phase_of(rows):
    """Phase of each dispatch: "load" (weight packing) before the first embedding
    launch, "prefill" from it up to the embedding launch that opens the first denoise
    pass (the last one before the first LM-head launch), "pass" from there on (the
    passes, and the commits between blocks, which run the encoder on a canvas).  The
    persistent kernels launch one grid for every batch size, so the grid alone does
    not tell the prefill launches from the pass launches."""
    def ids(word):
        return sorted(int(r["Dispatch_Id"]) for r in rows if word in r["Kernel_Name"])
    heads, embeds = ids("k_head"), ids("k_embed_rmsnorm")
    first_embed = embeds[0] if embeds else None
    pass_start = None
    if heads and embeds:
        before = [d for d in embeds if d < heads[0]]
        pass_start = before[-1] if before else heads[0]
    out = []
    for r in rows:
        d = int(r["Dispatch_Id"])
        if pass_start is not None and d >= pass_start:
            out.append("pass")
        elif first_embed is not None and d >= first_embed:
            out.append("prefill")
        else:
            out.append("load")
    return out


def summarize_trace(path):
    """Per (kernel, grid, phase) launch count and mean / min / max duration of a
    rocprofv3 --kernel-trace CSV."""
    import csv
    with open(path) as f:
        rows = list(csv.DictReader(f))
    groups = {}
    for row, ph in zip(rows, _phase_of(rows)):
        dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
        key = (row["Kernel_Name"].split("(")[0][:60], _grid_key(row), ph)
        groups.setdefault(key, []).append(dur)
    total = sum(sum(v) for v in groups.values())
    print(f"{'kernel':60s} {'grid':>18s} {'phase':>8s} {'calls':>6s} {'mean_us':>9s} {'min_us':>9s} "
          f"{'max_us':>9s} {'pct':>6s}")
    for (name, grid, ph), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"{name:60s} {grid:>18s} {ph:>8s} {len(v):6d} {sum(v) / len(v):9.2f} {min(v):9.2f} "
              f"{max(v):9.2f} {100 * sum(v) / total:6.2f}")


SIMDS = 1024        # 256 CUs x 4 SIMDs
XCDS = 8            # accelerator complex dies, one GRBM each


def summarize_pmc(path):
    """Per (kernel, grid, phase, counter) dispatch count and mean value of a rocprofv3
    --pmc CSV (each dispatch's value summed over the counter's instances).  When both
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE were collected it also prints the MFMA
    utilisation of every kernel, rocprofv3's MfmaUtil: busy cycles summed over all SIMDs
    over (active cycles x SIMDs), the active cycles being the largest GRBM_GUI_ACTIVE
    instance (one per XCD).  rocprofv3 writes GRBM_GUI_ACTIVE as one value summed over
    the 8 XCDs, which is then divided by 8 (each XCD counts the same active time; the
    quotient matches the traced durations at the shader clock within a few per cent)."""
    import csv
    with open(path) as f:
        rows = list(csv.DictReader(f))
    groups, peak = {}, {}
    for row, ph in zip(rows, _phase_of(rows)):
        key = (row["Kernel_Name"].split("(")[0][:60], _grid_key(row), ph, row["Counter_Name"])
        v = float(row["Counter_Value"])
        groups.setdefault(key, {}).setdefault(row["Dispatch_Id"], 0.0)
        groups[key][row["Dispatch_Id"]] += v
        peak.setdefault(key, {}).setdefault(row["Dispatch_Id"], []).append(v)
    print(f"{'kernel':60s} {'grid':>18s} {'phase':>8s} {'counter':>12s} {'dispatches':>10s} {'mean':>14s}")
    for (name, grid, ph, ctr), d in sorted(groups.items()):
        vals = list(d.values())
        print(f"{name:60s} {grid:>18s} {ph:>8s} {ctr:>12s} {len(vals):10d} {sum(vals) / len(vals):14.1f}")
    util = []
    for (name, grid, ph, ctr), d in groups.items():
        if ctr != "SQ_VALU_MFMA_BUSY_CYCLES":
            continue
        gk = (name, grid, ph, "GRBM_GUI_ACTIVE")
        if gk not in groups:
            continue
        busy = sum(d.values())
        active = sum(max(vs) if len(vs) > 1 else vs[0] / XCDS for vs in peak[gk].values())
        if busy > 0 and active > 0:
            util.append((name, grid, ph, len(d), busy / (active * SIMDS)))
    if util:
        print(f"\n{'kernel':60s} {'grid':>18s} {'phase':>8s} {'dispatches':>10s} {'mfma_util_pct':>14s}")
        for name, grid, ph, n, u in sorted(util, key=lambda t: -t[4]):
            print(f"{name:60s} {grid:>18s} {ph:>8s} {n:10d} {100 * u:14.2f}")


# canvases per batched pass measured beside the single-canvas pass
BATCHES = (1, 2, 4, 8, 16)


def ATTN_LONG(fx):
    """The attention shape of the long-context model: 131072 prompt + 256 canvas keys."""
    return fx.ATTN.__class__(name="attn_gqa16x8_D128_S131072p256_bf16", prompt_len=131072)


def _timed(torch, fn, n):
    """Mean milliseconds of n calls of fn on the current stream (HIP events)."""
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def attention_bench(dg, torch, fx, a=None):
    """The attention entry point alone: 16 query / 8 KV heads of dim 128, 256 canvas queries
    over the prompt's + 256 canvas keys (4096 + 256 by default), bidirectional, bf16, N(0, 1)
    inputs."""
    import numpy as np
    a = a or fx.ATTN
    q, k, v = fx.attn_inputs(a)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.empty(a.canvas, a.n_q_heads * a.head_dim, dtype=torch.bfloat16, device="cuda")
    S = a.seq
    ws = dg.dg_attention_workspace_size(a.n_q_heads, a.n_kv_heads, a.canvas, S, a.head_dim, False,
                                        0, dg.DG_BF16)
    wsd = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    scale = 1.0 / np.sqrt(a.head_dim)
    n = 50 if S <= 16384 else 10
    ms = _timed(torch, lambda: dg.dg_attention(qd, kd, vd, o, a.n_q_heads, a.n_kv_heads, a.canvas, S,
                                               a.head_dim, scale, False, 0, dg.DG_BF16, wsd), n)
    flops = 4 * a.canvas * S * a.head_dim * a.n_q_heads
    tf = flops / (ms * 1e-3) / 1e12
    log(f"attention {a.name}: {ms * 1e3:.1f} us per call, {tf:.0f} TFLOP/s")
    return {"workload": a.name, "us_per_call": round(ms * 1e3, 2), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4)},
            "note": "includes the per-call transposed pack of V into the caller's workspace"}


def moe_layer_bench(dg, torch, fx, experts="bf16"):
    """One MoE layer alone: 256 tokens of N(0, 1) hidden states, d = 2816, 128 experts top-8,
    SwiGLU width 704, router and experts N(0, 0.02); experts in bf16, or in MX FP4 (E2M1 codes
    with an E8M0 scale per 32 along the contraction, quantized from the same bf16 weights)
    with e4m3 inputs to the expert GEMMs."""
    import numpy as np
    m = fx.MOE_LAYER
    x, wr, wg, wu, wd = fx.moe_inputs(m)
    mx = experts == "mxfp4"
    cfg = dg.make_cfg(1, m.d_model, 16, 8, 128, m.n_experts, m.top_k, m.d_ff, 128, 256, 256,
                      act_dtype=dg.DG_BF16, expert_dtype=dg.DG_MXFP4 if mx else dg.DG_BF16)
    h = dg.dg_create(cfg)
    try:
        dg.dg_load_tensor(h, dg.DG_T_WR, 0, 0, wr)
        for kind, t in ((dg.DG_T_WG, wg), (dg.DG_T_WU, wu), (dg.DG_T_WD, wd)):
            if mx:
                f32 = (t.astype(np.uint32) << 16).view(np.float32)
                parts = [fx.quant_mxfp4(f32[e]) for e in range(m.n_experts)]
                dg.dg_load_tensor(h, kind, 0, -1, np.ascontiguousarray(np.stack([p[0] for p in parts])),
                                  np.ascontiguousarray(np.stack([p[1] for p in parts])))
            else:
                dg.dg_load_tensor(h, kind, 0, -1, np.ascontiguousarray(t))
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.empty_like(xd)
        idx = torch.empty(m.tokens, m.top_k, dtype=torch.int32, device="cuda")
        dg.dg_moe_layer(h, 0, xd, m.tokens, y, idx)
        torch.cuda.synchronize()
        cnt = np.bincount(idx.cpu().numpy().ravel(), minlength=m.n_experts)
        hit = int((cnt > 0).sum())
        ms = _timed(torch, lambda: dg.dg_moe_layer(h, 0, xd, m.tokens, y), 50)
    finally:
        dg.dg_destroy(h)
    # expert weights of every expert hit (MX: half a byte per element plus one scale byte per
    # 32), the router once, the hidden states in and out (bf16)
    per_weight = (0.5 + 1.0 / 32) if mx else 2
    nbytes = int(hit * 3 * m.d_model * m.d_ff * per_weight + m.d_model * m.n_experts * 2
                 + 2 * m.tokens * m.d_model * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    flops = 2 * m.tokens * m.top_k * 3 * m.d_model * m.d_ff
    log(f"MoE layer {m.name} ({experts} experts): {ms * 1e3:.1f} us per call, {hit} experts hit "
        f"(largest load {int(cnt.max())}), {gbs:.0f} GB/s algorithmic")
    return {"workload": m.name if not mx else m.name.replace("_bf16", "_mxfp4experts"),
            "experts": experts, "us_per_call": round(ms * 1e3, 2), "experts_hit": hit,
            "largest_expert_load": int(cnt.max()), "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 1)}


def mxfp4_model_bench(dg, torch, fx, build_handle, args, plain_ms):
    """The benched model with MX FP4 experts (E2M1 codes, an E8M0 scale per 32 along the
    contraction, e4m3 inputs to the expert GEMMs on the block-scaled MFMA); everything else as
    in the headline passes.  Timed like them, then once more with kernel timing; the roofline
    is that of the expert gate/up GEMM at MX bytes."""
    import numpy as np
    w = fx.MOE26B_MX
    if args.layers:
        w = w.with_(n_layers=args.layers)
    log(f"building {w.name}")
    h = build_handle(dg, w, max_ctx=w.prompt_len + w.canvas)
    try:
        dg.dg_prefill_prompt_kv(h, torch.from_numpy(fx.prompt_ids(w)).cuda(), w.prompt_len)
        C, T, seed = w.canvas, w.T, w.seed
        canvas = torch.empty(C, dtype=torch.int32, device="cuda")
        mask = torch.empty(C, dtype=torch.uint8, device="cuda")

        def step(i):
            s = i % T
            if s == 0:
                dg.dg_init_canvas(h, canvas, mask, seed + i // T)
            dg.dg_denoise_step(h, canvas, mask, s, T, seed + i // T)

        for i in range(args.warmup):
            step(i)
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            step(i)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        dg.dg_profile_begin(h, args.steps * (w.n_layers * 7 + 4))
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        prof_ms, prof_n = dg.dg_profile_end(h)
        dg.dg_set_capture(h, dg.DG_CAP_ROUTING)
        dg.dg_init_canvas(h, canvas, mask, seed)
        dg.dg_denoise_step(h, canvas, mask, 0, T, seed)
        rbuf = torch.empty(2 * C * w.top_k, dtype=torch.int32, device="cuda")
        active = []
        for l in range(w.n_layers):
            dg.dg_get_capture(h, dg.DG_CAP_ROUTING, l, rbuf)
            torch.cuda.synchronize()
            active.append(int((np.bincount(rbuf[:C * w.top_k].cpu().numpy(),
                                           minlength=w.n_experts) > 0).sum()))
        dg.dg_set_capture(h, 0)
        dg.dg_check_finite(h)
    finally:
        dg.dg_destroy(h)
        torch.cuda.synchronize()
    names = ["moe_gemm1", "moe_gemm2", "attention", "lm_head", "dense_gemm"]
    us = {n: prof_ms[i] / prof_n[i] * 1e3 if prof_n[i] else None for i, n in enumerate(names)}
    hit = float(np.mean(active))
    Fp = (w.d_ff + 127) // 128 * 128
    # gate/up codes and scales of every expert hit, the e4m3 inputs once, H written (e4m3)
    moe1_bytes = int(hit * w.d_model * 2 * w.d_ff * (0.5 + 1.0 / 32) + C * w.d_model
                     + C * w.top_k * Fp)
    moe1_gbs = moe1_bytes / (us["moe_gemm1"] * 1e-6) / 1e9
    res = {"workload": w.name, "ms_per_pass": round(ms, 4), "canvas_tok_s": round(C / (ms / 1e3), 1),
           "vs_bf16_experts": round(plain_ms / ms, 3) if plain_ms else None,
           "kernel_us_per_pass": {n: round(prof_ms[i] / args.steps * 1e3, 1)
                                  for i, n in enumerate(names)},
           "experts_hit_per_layer": round(hit, 2),
           "roofline": {"bound": "hbm", "kernel": "moe_gemm1 (MX FP4 expert gate/up GEMM + SwiGLU)",
                        "achieved": round(moe1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(moe1_gbs / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_launch": moe1_bytes,
                        "avg_launch_us": round(us["moe_gemm1"], 2)}}
    log(f"MX FP4 experts: {ms:.3f} ms per pass (bf16 experts {plain_ms or float('nan'):.3f}); "
        f"gate/up GEMM {us['moe_gemm1']:.1f} us ({moe1_gbs:.0f} GB/s algorithmic), down GEMM "
        f"{us['moe_gemm2']:.1f} us")
    return res


def long_context_bench(dg, torch, fx, build_handle, args):
    """The long-context variant: fp8 (e4m3) experts with per-column scales, a prompt of 131072
    uniform-random ids prefilled by the causal encoder, and four canvases of 256 generated one
    after another, each committed before the next (later canvases attend to the prompt and to
    every committed canvas).  Timed: the prefill, every pass (HIP events per pass) and every
    commit."""
    import numpy as np
    w = fx.MOE26B_FP8_LONG
    if args.layers:
        w = w.with_(n_layers=args.layers)
    log(f"building {w.name}")
    t0 = time.time()
    h = build_handle(dg, w)
    log(f"weights loaded in {time.time() - t0:.1f} s; prefilling {w.prompt_len} tokens")
    try:
        ids = torch.from_numpy(fx.prompt_ids(w)).cuda()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dg.dg_prefill_prompt_kv(h, ids, w.prompt_len)
        torch.cuda.synchronize()
        prefill_ms = (time.perf_counter() - t0) * 1e3
        log(f"prefill {prefill_ms:.0f} ms")
        C, T, K = w.canvas, w.T, w.n_canvases
        canvas = torch.empty(C, dtype=torch.int32, device="cuda")
        mask = torch.empty(C, dtype=torch.uint8, device="cuda")
        # one untimed block with kernel timing (warm-up, graph capture at this context)
        dg.dg_profile_begin(h, T * (w.n_layers * 7 + 4))
        dg.dg_init_canvas(h, canvas, mask, w.seed + 99)
        for s in range(T):
            dg.dg_denoise_step(h, canvas, mask, s, T, w.seed + 99)
        torch.cuda.synchronize()
        prof_ms, prof_n = dg.dg_profile_end(h)
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K * (T + 2) + 1)]
        i = 0
        ev[i].record(stream)
        for kk in range(K):
            dg.dg_init_canvas(h, canvas, mask, w.seed + kk)
            for s in range(T):
                dg.dg_denoise_step(h, canvas, mask, s, T, w.seed + kk)
                i += 1
                ev[i].record(stream)
            dg.dg_commit_canvas(h, canvas)
            i += 1
            ev[i].record(stream)
            i += 1
            ev[i].record(stream)
        torch.cuda.synchronize()
        dg.dg_check_finite(h)
    finally:
        dg.dg_destroy(h)
        torch.cuda.synchronize()
    per_pass, commits, first = [], [], []
    i = 0
    for kk in range(K):
        for s in range(T):
            d = ev[i].elapsed_time(ev[i + 1])
            (first if s == 0 else per_pass).append(d)
            i += 1
        commits.append(ev[i].elapsed_time(ev[i + 1]))
        i += 2
    total_ms = ev[0].elapsed_time(ev[i - 1])
    ms_pass = float(np.mean(per_pass))
    names = ["moe_gemm1", "moe_gemm2", "attention", "lm_head", "dense_gemm"]
    cls_us = {n: round(prof_ms[j] / T * 1e3, 1) for j, n in enumerate(names)}
    attn_us = prof_ms[2] / prof_n[2] * 1e3 if prof_n[2] else None
    S = w.prompt_len + C
    attn_tf = 4 * C * S * w.head_dim * w.n_q_heads / (attn_us * 1e-6) / 1e12 if attn_us else None
    res = {"workload": w.name, "canvases": K, "passes_per_canvas": T,
           "prefill_ms": round(prefill_ms, 1),
           "ms_per_pass": round(ms_pass, 3), "canvas_tok_s": round(C / (ms_pass / 1e3), 1),
           "first_pass_of_canvas_ms": [round(x, 2) for x in first],
           "commit_ms": [round(x, 2) for x in commits],
           "output_tok_s_with_commits": round(K * C / (total_ms / 1e3), 1),
           "kernel_us_per_pass": cls_us,
           "roofline": {"bound": "mfma", "kernel": "attention over the prompt's 131328 keys",
                        "achieved": round(attn_tf, 1) if attn_tf else None,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(attn_tf / BF16_PEAK_TFLOPS, 4) if attn_tf else None,
                        "avg_launch_us": round(attn_us, 2) if attn_us else None},
           }
    log(f"long context: {ms_pass:.3f} ms per pass, {res['output_tok_s_with_commits']:.0f} output "
        f"tok/s over {K} canvases with commits; attention {attn_us:.0f} us per layer")
    return res


def self_cond_bench(dg, torch, fx, build_handle, args, plain_ms):
    """The same model with the self-conditioning block (Fsc = d): every pass but the last of a
    block forms z = FFW(p0 E) for the next one.  Timed like the headline passes (steps cycle
    through blocks of T), then once more with kernel timing for the vocabulary contraction."""
    w = fx.MOE26B_SC
    if args.layers:
        w = w.with_(n_layers=args.layers)
    log(f"building {w.name}")
    h = build_handle(dg, w, max_ctx=w.prompt_len + w.canvas)
    try:
        dg.dg_prefill_prompt_kv(h, torch.from_numpy(fx.prompt_ids(w)).cuda(), w.prompt_len)
        C, T, seed = w.canvas, w.T, w.seed
        canvas = torch.empty(C, dtype=torch.int32, device="cuda")
        mask = torch.empty(C, dtype=torch.uint8, device="cuda")

        def step(i):
            s = i % T
            if s == 0:
                dg.dg_init_canvas(h, canvas, mask, seed + i // T)
            dg.dg_denoise_step(h, canvas, mask, s, T, seed + i // T)

        for i in range(args.warmup):
            step(i)
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            step(i)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        dg.dg_profile_begin(h, args.steps * (w.n_layers * 7 + 6))
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        prof_ms, prof_n = dg.dg_profile_end(h)
        i_sc = dg.DG_PROF_SELF_COND
        sc_us = prof_ms[i_sc] / prof_n[i_sc] * 1e3 if prof_n[i_sc] else None
        # algorithmic bytes of one contraction: E once, the bf16 posterior rows once
        sc_bytes = w.vocab * w.d_model * 2 + C * w.vocab * 2
        sc_gbs = sc_bytes / (sc_us * 1e-6) / 1e9 if sc_us else None
        out = torch.empty(C, dtype=torch.int32, device="cuda")
        dg.dg_generate_block(h, out, T, seed, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dg.dg_generate_block(h, out, T, seed + 1, False)
        torch.cuda.synchronize()
        block_ms = (time.perf_counter() - t0) * 1e3
        dg.dg_check_finite(h)
        n_sig = sum(1 for i in range(args.steps) if i % T < T - 1)
        res = {"workload": w.name, "sc_ff": w.sc_width, "ms_per_pass": round(ms, 4),
               "canvas_tok_s": round(C / (ms / 1e3), 1),
               "signal_us_per_forming_pass":
                   round((ms - plain_ms) * 1e3 * args.steps / n_sig, 1) if plain_ms else None,
               "contraction_us_per_launch": round(sc_us, 2) if sc_us else None,
               "contraction_algorithmic_bytes": sc_bytes,
               "contraction_gbs": round(sc_gbs, 1) if sc_gbs else None,
               "contraction_hbm_frac": round(sc_gbs / HBM_PEAK_GBS, 4) if sc_gbs else None,
               "contraction_traffic": measured_traffic("sc_contraction"),
               "block_ms": round(block_ms, 2)}
        log(f"self-conditioned: {ms:.3f} ms per pass (plain {plain_ms or float('nan'):.3f}); contraction "
            f"{sc_us:.1f} us ({sc_gbs:.0f} GB/s algorithmic); block {block_ms:.1f} ms")
        return res
    finally:
        dg.dg_destroy(h)
        torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-blocks", action="store_true",
                    help="skip the whole-block timing (short runs under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel, per-grid durations of a rocprofv3 kernel trace")
    ap.add_argument("--summarize-pmc", metavar="COUNTER_CSV",
                    help="print per-kernel, per-grid counter means of a rocprofv3 --pmc run")
    ap.add_argument("--no-batches", action="store_true",
                    help="skip the batched-canvas passes (profiler runs of the single pass)")
    ap.add_argument("--no-kernels", action="store_true",
                    help="skip the attention and MoE-layer kernel lines")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context fp8 model (P = 131072, four canvases)")
    ap.add_argument("--no-self-cond", action="store_true",
                    help="skip the self-conditioned model (a second handle of the same size)")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the MX FP4 expert lines (model and MoE layer)")
    ap.add_argument("--only", choices=("self_cond", "kernels", "attn_long", "long", "mx", "mx_layer"),
                    help="run one further line alone and print its JSON (for profiler runs)")
    ap.add_argument("--layers", type=int, default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the denoise pass is "
              "measured on a single MI355X; sharding across GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import discrete_diffusion_decoding_canvas_amd as dg
    import fixtures as fx
    from fixtures.dg_glue import build_handle

    w = fx.MOE26B
    if args.layers:
        w = w.with_(n_layers=args.layers)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.only:
        if args.only == "self_cond":
            out = self_cond_bench(dg, torch, fx, build_handle, args, None)
        elif args.only == "kernels":
            out = {"attention_kernel": attention_bench(dg, torch, fx),
                   "moe_layer": moe_layer_bench(dg, torch, fx)}
        elif args.only == "attn_long":
            out = attention_bench(dg, torch, fx, ATTN_LONG(fx))
        elif args.only == "mx":
            out = mxfp4_model_bench(dg, torch, fx, build_handle, args, None)
        elif args.only == "mx_layer":
            out = moe_layer_bench(dg, torch, fx, "mxfp4")
        else:
            out = long_context_bench(dg, torch, fx, build_handle, args)
        print(json.dumps(out), flush=True)
        return
    log(f"building {w.name} (weights from the seeded generator)")
    t0 = time.time()
    # room for a committed canvas (the block timing) and the largest batch after it
    h = build_handle(dg, w, max_ctx=w.prompt_len + (BATCHES[-1] + 1) * w.canvas,
                     max_batch=BATCHES[-1])
    log(f"weights loaded in {time.time() - t0:.1f} s; prefilling {w.prompt_len} tokens")
    ids = torch.from_numpy(fx.prompt_ids(w)).cuda()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dg.dg_prefill_prompt_kv(h, ids, w.prompt_len)
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - t0) * 1e3
    log(f"prefill {prefill_ms:.1f} ms")

    C, T, seed = w.canvas, w.T, w.seed
    canvas = torch.empty(C, dtype=torch.int32, device="cuda")
    mask = torch.empty(C, dtype=torch.uint8, device="cuda")

    def step(i):
        s = i % T
        if s == 0:
            dg.dg_init_canvas(h, canvas, mask, seed + i // T)
        dg.dg_denoise_step(h, canvas, mask, s, T, seed + i // T)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} passes done; timing {args.steps} passes")

    # timed passes: the decoder-layer stack replays as a HIP graph (the library default)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)
    dg.dg_check_finite(h)
    ms_per_pass = ms_total / args.steps
    canvas_tok_s = C * args.steps / (ms_total / 1e3)
    log(f"{ms_per_pass:.3f} ms per pass ({canvas_tok_s:.0f} canvas tok/s; wall {wall:.2f} s)")

    # the same passes again with per-kernel event timing (launched one by one)
    dg.dg_profile_begin(h, args.steps * (w.n_layers * 7 + 4))
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    prof_ms, prof_n = dg.dg_profile_end(h)
    ms_per_pass_eager = start.elapsed_time(end) / args.steps
    log(f"{ms_per_pass_eager:.3f} ms per pass with kernel timing (kernels launched one by one)")

    # routing of one more (untimed) pass: experts actually hit per layer set the
    # algorithmic weight bytes of the expert GEMMs
    # (the residual stream entering a deep layer and that layer's prompt K/V feed the CPU
    # oracle's timed sample of a deep layer)
    deep_layer = w.n_layers // 2
    dg.dg_set_capture(h, dg.DG_CAP_ROUTING | (0 if args.no_cpu_baseline else dg.DG_CAP_HIDDEN))
    dg.dg_init_canvas(h, canvas, mask, seed)
    dg.dg_denoise_step(h, canvas, mask, 0, T, seed)
    active, max_load, deep = [], [], None
    rbuf = torch.empty(2 * C * w.top_k, dtype=torch.int32, device="cuda")
    for l in range(w.n_layers):
        dg.dg_get_capture(h, dg.DG_CAP_ROUTING, l, rbuf)
        torch.cuda.synchronize()
        ids = rbuf[:C * w.top_k].cpu().numpy()
        cnt = np.bincount(ids, minlength=w.n_experts)
        active.append(int((cnt > 0).sum()))
        max_load.append(int(cnt.max()))
        if l == deep_layer:
            deep_route = ids
    if not args.no_cpu_baseline:
        hid = torch.empty(C, w.d_model, dtype=torch.float32, device="cuda")
        dg.dg_get_capture(h, dg.DG_CAP_HIDDEN, deep_layer - 1, hid)   # after layer L - 1
        kv = []
        for which in (0, 1):
            t = torch.empty(w.n_kv_heads, w.prompt_len, w.head_dim, dtype=torch.bfloat16, device="cuda")
            dg.dg_get_kv(h, deep_layer, which, 0, w.prompt_len, t)
            kv.append(t.float().cpu().numpy().astype(np.float64))
        torch.cuda.synchronize()
        deep = (deep_layer, hid.cpu().numpy().astype(np.float64), kv[0], kv[1], deep_route)
    dg.dg_set_capture(h, 0)
    mean_active = float(np.mean(active))
    log(f"experts hit per layer: mean {mean_active:.1f}, min {min(active)}, max {max(active)}; "
        f"largest per-expert load {max(max_load)} tokens")

    # whole blocks: 12 passes (+ the commit of the final canvas)
    block_ms = commit_ms = None
    if not args.no_blocks:
        out = torch.empty(C, dtype=torch.int32, device="cuda")
        dg.dg_generate_block(h, out, T, seed, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_blocks = 2
        for b in range(n_blocks):
            dg.dg_generate_block(h, out, T, seed + b, False)
        torch.cuda.synchronize()
        block_ms = (time.perf_counter() - t0) * 1e3 / n_blocks
        t0 = time.perf_counter()
        dg.dg_commit_canvas(h, out)
        torch.cuda.synchronize()
        commit_ms = (time.perf_counter() - t0) * 1e3
        log(f"block {block_ms:.2f} ms, commit {commit_ms:.2f} ms")

    # the entropy-bounded sampler on the same model: same decoder, the LM head with its
    # entropy term, the one-workgroup sampler.  Per-pass time (no stop: theta = 0), the
    # head's time with the entropy term, and one block with the pages' schedule
    # (tau 0.8 -> 0.4, at most 48 passes).
    ebr = None
    if not args.no_blocks:
        p_run = dg.eb_params(theta=0.0)
        info = torch.zeros(4, dtype=torch.int32, device="cuda")

        def eb_step(i):
            s = i % T
            if s == 0:
                dg.dg_init_canvas(h, canvas, mask, seed + 100 + i // T)
            dg.dg_denoise_step_eb(h, canvas, mask, s, p_run, seed, info)

        for i in range(args.warmup):
            eb_step(i)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            eb_step(i)
        end.record(stream)
        torch.cuda.synchronize()
        eb_ms = start.elapsed_time(end) / args.steps
        dg.dg_profile_begin(h, args.steps * (w.n_layers * 7 + 4))
        for i in range(args.steps):
            eb_step(i)
        torch.cuda.synchronize()
        eb_prof_ms, eb_prof_n = dg.dg_profile_end(h)
        head_i = dg.DG_PROF_LM_HEAD
        eb_head_us = eb_prof_ms[head_i] / eb_prof_n[head_i] * 1e3 if eb_prof_n[head_i] else None
        p_block = dg.eb_params()
        out = torch.empty(C, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_eb = dg.dg_generate_block_eb(h, out, p_block, seed + 7, False)
        eb_block_ms = (time.perf_counter() - t0) * 1e3
        ebr = {"ms_per_pass": round(eb_ms, 4), "lm_head_us_with_entropy": round(eb_head_us, 2),
               "block_passes": n_eb, "block_ms": round(eb_block_ms, 2),
               "params": {"tau_max": p_block.tau_max, "tau_min": round(p_block.tau_min, 6),
                          "gamma": p_block.gamma, "theta": round(p_block.theta, 6),
                          "max_steps": p_block.max_steps}}
        log(f"entropy-bounded: {eb_ms:.3f} ms per pass (head {eb_head_us:.1f} us); "
            f"block of {n_eb} passes {eb_block_ms:.1f} ms")

    # batched canvases: B canvases over the same context in one pass (one graph per B)
    batched = {}
    for B in (() if args.no_batches else BATCHES):
        bc = torch.empty(B * C, dtype=torch.int32, device="cuda")
        bm = torch.empty(B * C, dtype=torch.uint8, device="cuda")

        def bstep(i, B=B, bc=bc, bm=bm):
            s = i % T
            if s == 0:
                dg.dg_init_canvas_batch(h, bc, bm, B, seed + 200 + i // T)
            dg.dg_denoise_step_batch(h, bc, bm, B, s, T, seed + 200 + i // T)

        for i in range(2):
            bstep(i)
        n_b = max(4, args.steps // 4)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(n_b):
            bstep(i)
        end.record(stream)
        torch.cuda.synchronize()
        b_ms = start.elapsed_time(end) / n_b
        batched[str(B)] = {"ms_per_pass": round(b_ms, 4),
                           "canvas_tok_s": round(B * C / (b_ms / 1e3), 1)}
        log(f"batch of {B} canvases: {b_ms:.3f} ms per pass, {B * C / (b_ms / 1e3):.0f} canvas tok/s")
        if B == BATCHES[-1]:
            # the largest batch once more with per-kernel events: every token reaches k
            # experts, so the expert GEMMs' FLOPs are exact whatever the routing
            dg.dg_profile_begin(h, n_b * (w.n_layers * 7 + 4))
            for i in range(n_b):
                bstep(i)
            torch.cuda.synchronize()
            b_prof_ms, b_prof_n = dg.dg_profile_end(h)
            rows = B * C * w.top_k
            flops = {"moe_gemm1": rows * w.d_model * 2 * w.d_ff * 2,
                     "moe_gemm2": rows * w.d_ff * w.d_model * 2,
                     "attention": B * 4 * C * (w.prompt_len + C) * w.head_dim * w.n_q_heads}
            mfma = {}
            for i, n in enumerate(["moe_gemm1", "moe_gemm2", "attention"]):
                if b_prof_n[i]:
                    us = b_prof_ms[i] / b_prof_n[i] * 1e3
                    tf = flops[n] / (us * 1e-6) / 1e12
                    mfma[n] = {"us_per_launch": round(us, 2), "tflops": round(tf, 1),
                               "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
            batched[str(B)]["mfma"] = mfma
            log(f"batch of {B}: " + ", ".join(f"{n} {v['us_per_launch']:.1f} us = {v['tflops']:.0f} "
                                              f"TFLOP/s ({100 * v['frac_bf16_peak']:.1f} % of bf16 peak)"
                                              for n, v in mfma.items()))
    dg.dg_check_finite(h)

    # roofline of the dominant kernel (expert gate/up GEMM + SwiGLU)
    names = ["moe_gemm1", "moe_gemm2", "attention", "lm_head", "dense_gemm"]
    per_class_us = {n: (prof_ms[i] / prof_n[i] * 1e3 if prof_n[i] else None)
                    for i, n in enumerate(names)}
    per_pass_us = {n: prof_ms[i] / args.steps * 1e3 for i, n in enumerate(names)}
    moe1_us = per_class_us["moe_gemm1"]
    moe1_bytes = int(moe1_algorithmic_bytes(w, mean_active))
    moe1_gbs = moe1_bytes / (moe1_us * 1e-6) / 1e9
    moe2_bytes = int(mean_active * w.d_ff * w.d_model * 2 + C * w.top_k * (w.d_ff * 2 + w.d_model * 2))
    moe2_gbs = moe2_bytes / (per_class_us["moe_gemm2"] * 1e-6) / 1e9
    S = w.prompt_len + C
    attn_flops = 4 * C * S * w.head_dim * w.n_q_heads
    attn_tflops = attn_flops / (per_class_us["attention"] * 1e-6) / 1e12
    head_flops = 2 * C * w.d_model * w.vocab
    head_tflops = head_flops / (per_class_us["lm_head"] * 1e-6) / 1e12
    head_gbs = w.vocab * w.d_model * 2 / (per_class_us["lm_head"] * 1e-6) / 1e9
    moe_flops = 2 * C * w.top_k * 3 * w.d_model * w.d_ff
    moe_tflops = moe_flops / ((per_class_us["moe_gemm1"] + per_class_us["moe_gemm2"]) * 1e-6) / 1e12
    flops = pass_flops(w, S)

    result = {
        "metric": "canvas tok/s per denoise pass",
        "value": round(canvas_tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_pass, 4),
        "ms_per_step_kernels_one_by_one": round(ms_per_pass_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init N(0,0.02) weights, uniform-random prompt ids)",
        "config": {"workload": w.name, "layers": w.n_layers, "d_model": w.d_model,
                   "experts": w.n_experts, "top_k": w.top_k, "d_ff": w.d_ff,
                   "vocab": w.vocab, "prompt": w.prompt_len, "canvas": C,
                   "passes_per_block": T},
        "output_tok_s_per_block": round(C / (block_ms / 1e3), 1) if block_ms else None,
        "output_tok_s_per_block_with_commit":
            round(C / ((block_ms + commit_ms) / 1e3), 1) if block_ms else None,
        "block_ms": round(block_ms, 3) if block_ms else None,
        "commit_ms": round(commit_ms, 3) if block_ms else None,
        "prefill_ms": round(prefill_ms, 2),
        "entropy_bounded_sampler": ebr,
        "batched_canvases": batched,
        "pass_tflops": round(flops / (ms_per_pass * 1e-3) / 1e12, 2),
        "mfma_util_pct": {
            "moe_grouped_gemm": round(100 * moe_tflops / BF16_PEAK_TFLOPS, 2),
            "attention": round(100 * attn_tflops / BF16_PEAK_TFLOPS, 2),
            "lm_head": round(100 * head_tflops / BF16_PEAK_TFLOPS, 2),
        },
        "hbm_util_pct": {
            "moe_gemm1": round(100 * moe1_gbs / HBM_PEAK_GBS, 2),
            "moe_gemm2": round(100 * moe2_gbs / HBM_PEAK_GBS, 2),
            "lm_head": round(100 * head_gbs / HBM_PEAK_GBS, 2),
        },
        "kernel_us_per_launch": {k: (round(v, 2) if v else None) for k, v in per_class_us.items()},
        "experts_hit_per_layer": {"mean": round(mean_active, 2), "min": min(active),
                                  "max": max(active), "largest_expert_load": max(max_load)},
        "kernel_us_per_pass": {k: round(v, 1) for k, v in per_pass_us.items()},
        "roofline": {"bound": "hbm", "kernel": "moe_gemm1 (expert gate/up GEMM + SwiGLU)",
                     "achieved": round(moe1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(moe1_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": moe1_bytes,
                     "avg_launch_us": round(moe1_us, 2),
                     "traffic": measured_traffic("moe_gemm1")},
    }
    dg.dg_destroy(h)
    torch.cuda.synchronize()
    if not args.no_self_cond:
        result["self_conditioning"] = self_cond_bench(dg, torch, fx, build_handle, args,
                                                      ms_per_pass)
    if not args.no_kernels:
        result["attention_kernel"] = attention_bench(dg, torch, fx)
        result["attention_kernel_long"] = attention_bench(dg, torch, fx, ATTN_LONG(fx))
        result["moe_layer"] = moe_layer_bench(dg, torch, fx)
        if not args.no_mx:
            result["moe_layer_mxfp4"] = moe_layer_bench(dg, torch, fx, "mxfp4")
    if not args.no_mx:
        result["mxfp4_experts"] = mxfp4_model_bench(dg, torch, fx, build_handle, args, ms_per_pass)
    if not args.no_long:
        result["long_context_fp8"] = long_context_bench(dg, torch, fx, build_handle, args)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, deep)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Device-side helpers shared by the GPU tests (test infrastructure)."""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import discrete_diffusion_decoding_canvas_amd as dg   # fails loudly if libdg.so is missing
    return dg


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.uint8))).cuda()


def stats_capture(dg, h, C):
    buf = torch.empty(5 * C, dtype=torch.int32, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_STATS, 0, buf)
    torch.cuda.synchronize()
    raw = buf.cpu().numpy()
    f = raw.view(np.float32)
    return {"m": f[0:C].astype(np.float64), "argmax": raw[C:2 * C].copy(),
            "lse": f[2 * C:3 * C].astype(np.float64), "conf": f[3 * C:4 * C].astype(np.float64),
            "redraw": raw[4 * C:5 * C].copy()}


def routing_capture(dg, h, layer, C, k):
    buf = torch.empty(2 * C * k, dtype=torch.int32, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_ROUTING, layer, buf)
    torch.cuda.synchronize()
    raw = buf.cpu().numpy()
    return raw[:C * k].reshape(C, k).copy(), raw[C * k:].view(np.float32).reshape(C, k).astype(np.float64)


def logits_capture(dg, h, C, V):
    buf = torch.empty(C, V, dtype=torch.float32, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_LOGITS, 0, buf)
    torch.cuda.synchronize()
    return buf


def kv_read(dg, h, layer, which, row0, n, Hkv, D, dtype):
    t = torch.empty(Hkv, n, D, dtype=dtype, device="cuda")
    dg.dg_get_kv(h, layer, which, row0, n, t)
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def record(name: str, data: dict) -> None:
    """Write a parity record (counts of in-band decisions, per-layer statistics) as JSON to
    the directory named by DG_PARITY_RECORD_DIR, when it is set."""
    out = os.environ.get("DG_PARITY_RECORD_DIR")
    if not out:
        return
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, f"{name}.json"), "w") as f:
        json.dump(data, f, indent=1, sort_keys=True, default=float)
    log(f"parity record {name} written")

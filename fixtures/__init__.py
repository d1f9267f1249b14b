"""Seeded synthetic inputs for the canvas denoiser, shared by the CPU oracle
and by the callers of the GPU library (tests and bench).

This module holds no arithmetic of the method itself: it only produces the
random-init weights, prompt ids and kernel-level test tensors that both sides
consume, as the same bytes.  The recipe (hash, Box-Muller, bf16 / e4m3
storage) is in ``gen.c``; every value is a pure function of
(seed, tensor id, flat index).

Weights follow the "random-init N(0, 0.02)" recipe of the synthetic
configurations; logical layouts are ``[in, out]`` row-major:
E [V, d], Wq [d, Hq*D], Wk/Wv [d, Hkv*D], Wo [Hq*D, d], Wr [d, E],
Wg/Wu [E, d, F], Wd [E, F, d], and for self-conditioning workloads the one
feed-forward block of the signal, sc_wg/sc_wu [d, Fsc], sc_wd [Fsc, d], drawn
N(0, sc_sigma).  RMSNorm gains are 1 and are not stored.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfixtures.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gen.c into libfixtures.so (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
             os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p
        lib.fx_normal_f32.argtypes = [u64, u32, u64, u64, ctypes.c_float, vp]
        lib.fx_normal_bf16.argtypes = [u64, u32, u64, u64, ctypes.c_float, vp]
        lib.fx_uniform_ids.argtypes = [u64, u32, u64, u64, u32, vp]
        lib.fx_quant_e4m3_cols.argtypes = [vp, i64, i64, vp, vp]
        lib.fx_e4m3_encode.argtypes = [ctypes.c_float]
        lib.fx_e4m3_encode.restype = ctypes.c_uint8
        lib.fx_bf16_encode.argtypes = [ctypes.c_float]
        lib.fx_bf16_encode.restype = ctypes.c_uint16
        lib.fx_quant_mxfp4.argtypes = [vp, i64, i64, vp, vp]
        lib.fx_e2m1_encode.argtypes = [ctypes.c_float]
        lib.fx_e2m1_encode.restype = ctypes.c_uint8
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# --------------------------------------------------------------------------- raw streams
def normal(seed: int, tid: int, shape, sigma: float, dtype: str = "f32", start: int = 0,
           out: np.ndarray | None = None) -> np.ndarray:
    """sigma * N(0,1) for flat indices [start, start + prod(shape)).

    dtype "f32" returns float32; "bf16" returns the bf16 bit patterns as uint16.
    """
    n = int(np.prod(shape))
    lib = _load()
    if dtype == "f32":
        a = out if out is not None else np.empty(shape, np.float32)
        lib.fx_normal_f32(seed, tid, start, n, sigma, _ptr(a))
    elif dtype == "bf16":
        a = out if out is not None else np.empty(shape, np.uint16)
        lib.fx_normal_bf16(seed, tid, start, n, sigma, _ptr(a))
    else:
        raise ValueError(dtype)
    return a


def uniform_ids(seed: int, tid: int, n: int, vocab: int, start: int = 0) -> np.ndarray:
    a = np.empty(n, np.int32)
    _load().fx_uniform_ids(seed, tid, start, n, vocab, _ptr(a))
    return a


def quant_e4m3_cols(w: np.ndarray):
    """Per-output-column e4m3 quantisation of a [rows, cols] float32 matrix.

    Returns (codes uint8 [rows, cols], scales float32 [cols]).
    """
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(cols, np.float32)
    _load().fx_quant_e4m3_cols(_ptr(w), rows, cols, _ptr(q), _ptr(s))
    return q, s


def quant_mxfp4(w: np.ndarray):
    """OCP MX FP4 storage of a [rows, cols] float32 matrix whose rows are the contraction
    dimension (rows % 32 == 0, cols even): E2M1 codes two per byte along the columns (even
    column in the low nibble), [rows, cols / 2] uint8, and one E8M0 scale per 32 rows of a
    column, [rows / 32, cols] uint8 (value 2^(s - 127))."""
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.shape
    if rows % 32 or cols % 2:
        raise ValueError("MX FP4 needs rows % 32 == 0 and an even column count")
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows // 32, cols), np.uint8)
    _load().fx_quant_mxfp4(_ptr(w), rows, cols, _ptr(codes), _ptr(scales))
    return codes, scales


def e2m1_encode_scalar(x: float) -> int:
    return int(_load().fx_e2m1_encode(float(x)))


def e4m3_encode_scalar(x: float) -> int:
    return int(_load().fx_e4m3_encode(float(x)))


def bf16_encode_scalar(x: float) -> int:
    return int(_load().fx_bf16_encode(float(x)))


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly (a storage view)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def e4m3_decode_table() -> np.ndarray:
    """All 256 OCP e4m3 code values as float64 (NaN for the two NaN codes)."""
    t = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 0xF and m == 7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** -9
        else:
            t[c] = s * (1 + m / 8.0) * 2.0 ** (e - 7)
    return t


# --------------------------------------------------------------------------- tensor ids
TID_EMBED = 1
TID_PROMPT = 2
TID_ATTN_Q, TID_ATTN_K, TID_ATTN_V = 3, 4, 5
TID_MOE_X = 6
TID_SC = {"sc_wg": 7, "sc_wu": 8, "sc_wd": 9}   # self-conditioning block (one per model)
KINDS = ("wq", "wk", "wv", "wo", "wr", "wg", "wu", "wd")


def layer_tid(kind: str, layer: int) -> int:
    return 64 + 16 * layer + KINDS.index(kind)


# --------------------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    """Sizes and storage types of one synthetic denoiser configuration."""
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    d_ff: int
    vocab: int
    prompt_len: int
    canvas: int = 256
    T: int = 12
    n_canvases: int = 1
    act: str = "bf16"          # "f32" | "bf16"
    experts: str = "bf16"      # "f32" | "bf16" | "fp8" | "mxfp4"
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    temperature: float = 1.0
    sigma: float = 0.02
    seed: int = 0
    self_cond: bool = False    # z = FFW(p0 E) fed into the next pass
    sc_ff: int = 0             # width of that feed-forward block (0: d_model)
    sc_sigma: float = 0.02

    @property
    def sc_width(self) -> int:
        return self.sc_ff if self.sc_ff > 0 else self.d_model

    @property
    def max_ctx(self) -> int:
        return self.prompt_len + self.n_canvases * self.canvas

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY_FP32 = Workload("tiny_fp32_2L_d256_V1024", n_layers=2, d_model=256, n_q_heads=4,
                     n_kv_heads=2, head_dim=64, n_experts=8, top_k=2, d_ff=512, vocab=1024,
                     prompt_len=64, act="f32", experts="f32")
# Small bf16 model through the same MFMA kernels as the large ones; the prompt spans two
# prefill chunks with a ragged tail.
SMALL_BF16 = Workload("small_bf16_2L_d256_E64k4_V1024_P4296", n_layers=2, d_model=256,
                      n_q_heads=4, n_kv_heads=2, head_dim=128, n_experts=64, top_k=4, d_ff=128,
                      vocab=1024, prompt_len=4296)
MOE26B = Workload("moe26b_30L_d2816_E128k8_V262144_P8192", n_layers=30, d_model=2816,
                  n_q_heads=16, n_kv_heads=8, head_dim=128, n_experts=128, top_k=8, d_ff=704,
                  vocab=262144, prompt_len=8192)
MOE26B_FP8_LONG = MOE26B.with_(name="moe26b_fp8experts_P131072_K4", experts="fp8",
                               prompt_len=131072, n_canvases=4)
# Self-conditioning.  The small configurations run at tau = 0.5 with N(0, 1) weights in the
# signal's feed-forward block, so that the posterior is spread (largest p0 ~0.1 on average)
# and z has the size of an embedding row: the signal then moves later logits by O(1).
# The large one is the benched model with the block added (Fsc = d, N(0, 0.02)), one layer
# and a short prompt, for checks of the signal's kernels at their full size.
TINY_FP32_SC = TINY_FP32.with_(name="tiny_fp32_2L_d256_V1024_selfcond", self_cond=True,
                               temperature=0.5, sc_sigma=1.0)
SMALL_BF16_SC = SMALL_BF16.with_(name="small_bf16_2L_d256_E64k4_V1024_P300_selfcond",
                                 prompt_len=300, self_cond=True, temperature=0.5, sc_sigma=1.0)
MOE26B_SC = MOE26B.with_(name="moe26b_30L_d2816_E128k8_V262144_P8192_selfcond", self_cond=True)
# MX FP4 experts (OCP microscaling: E2M1 elements, an E8M0 scale per 32 along the contraction),
# activations into the experts in e4m3.
SMALL_BF16_MX = SMALL_BF16.with_(name="small_bf16_2L_d256_E64k4_V1024_P4296_mxfp4experts",
                                 experts="mxfp4")
MOE26B_MX = MOE26B.with_(name="moe26b_mxfp4experts_30L_d2816_E128k8_V262144_P8192",
                         experts="mxfp4")
MOE26B_SC_1L = MOE26B_SC.with_(name="moe26b_1L_d2816_E128k8_V262144_P64_selfcond", n_layers=1,
                               prompt_len=64, n_canvases=2)


@dataclass(frozen=True)
class AttnWorkload:
    name: str = "attn_gqa16x8_D128_S4096p256_bf16"
    n_q_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    prompt_len: int = 4096
    canvas: int = 256
    seed: int = 0

    @property
    def seq(self) -> int:
        return self.prompt_len + self.canvas


@dataclass(frozen=True)
class MoeWorkload:
    name: str = "moe_layer_T256_d2816_E128k8_F704_bf16"
    tokens: int = 256
    d_model: int = 2816
    n_experts: int = 128
    top_k: int = 8
    d_ff: int = 704
    sigma: float = 0.02
    seed: int = 0


ATTN = AttnWorkload()
MOE_LAYER = MoeWorkload()


# --------------------------------------------------------------------------- model tensors
def tensor_shape(w: Workload, kind: str) -> tuple:
    d, hq, hkv, D, E, F, V = (w.d_model, w.n_q_heads, w.n_kv_heads, w.head_dim,
                              w.n_experts, w.d_ff, w.vocab)
    return {"embed": (V, d), "wq": (d, hq * D), "wk": (d, hkv * D), "wv": (d, hkv * D),
            "wo": (hq * D, d), "wr": (d, E), "wg": (E, d, F), "wu": (E, d, F),
            "wd": (E, F, d), "sc_wg": (d, w.sc_width), "sc_wu": (d, w.sc_width),
            "sc_wd": (w.sc_width, d)}[kind]


def is_expert(kind: str) -> bool:
    return kind in ("wg", "wu", "wd")


def storage_dtype(w: Workload, kind: str) -> str:
    if is_expert(kind):
        return w.experts
    return w.act


def model_tensor(w: Workload, kind: str, layer: int = 0, expert: int | None = None):
    """One logical weight tensor in the workload's storage type.

    f32  -> float32 array
    bf16 -> uint16 array of bf16 bit patterns
    fp8  -> (uint8 codes, float32 per-output-column scales); experts only,
            one expert at a time (``expert`` required)
    """
    shape = tensor_shape(w, kind)
    if kind in TID_SC:
        return normal(w.seed, TID_SC[kind], shape, w.sc_sigma, storage_dtype(w, kind))
    tid = TID_EMBED if kind == "embed" else layer_tid(kind, layer)
    dt = storage_dtype(w, kind)
    start = 0
    if is_expert(kind) and expert is not None:
        shape = shape[1:]
        start = expert * int(np.prod(shape))
    if dt == "fp8":
        if expert is None:
            raise ValueError("fp8 experts are produced one expert at a time")
        vals = normal(w.seed, tid, shape, w.sigma, "f32", start=start)
        return quant_e4m3_cols(vals)
    if dt == "mxfp4":
        if expert is None:
            raise ValueError("MX FP4 experts are produced one expert at a time")
        vals = normal(w.seed, tid, shape, w.sigma, "f32", start=start)
        return quant_mxfp4(vals)
    return normal(w.seed, tid, shape, w.sigma, dt, start=start)


def prompt_ids(w: Workload) -> np.ndarray:
    return uniform_ids(w.seed, TID_PROMPT, w.prompt_len, w.vocab)


def attn_inputs(a: AttnWorkload = ATTN):
    """Q [Hq, C, D], K and V [Hkv, S, D] as bf16 bit patterns, each N(0, 1)."""
    q = normal(a.seed, TID_ATTN_Q, (a.n_q_heads, a.canvas, a.head_dim), 1.0, "bf16")
    k = normal(a.seed, TID_ATTN_K, (a.n_kv_heads, a.seq, a.head_dim), 1.0, "bf16")
    v = normal(a.seed, TID_ATTN_V, (a.n_kv_heads, a.seq, a.head_dim), 1.0, "bf16")
    return q, k, v


def moe_inputs(m: MoeWorkload = MOE_LAYER):
    """Hidden states X [T, d] ~ N(0,1) and the layer-0 router / expert weights (bf16 bits)."""
    x = normal(m.seed, TID_MOE_X, (m.tokens, m.d_model), 1.0, "bf16")
    wr = normal(m.seed, layer_tid("wr", 0), (m.d_model, m.n_experts), m.sigma, "bf16")
    wg = normal(m.seed, layer_tid("wg", 0), (m.n_experts, m.d_model, m.d_ff), m.sigma, "bf16")
    wu = normal(m.seed, layer_tid("wu", 0), (m.n_experts, m.d_model, m.d_ff), m.sigma, "bf16")
    wd = normal(m.seed, layer_tid("wd", 0), (m.n_experts, m.d_ff, m.d_model), m.sigma, "bf16")
    return x, wr, wg, wu, wd


def eb_sampler_inputs(seed: int, C: int, V: int, locked_frac: float = 0.3,
                      prev_diff: int = 0, nan_at: int | None = None):
    """Per-position statistics for one pass of the entropy-bounded sampler, seeded.

    Entropies: a mix of near-certain positions (multiples of 2^-12 in [0, 2^-6],
    many tied) and uncertain ones (exponential, mean 2, capped at log V), as
    float32.  argmax, draw and canvas uniform over [0, V); prev = argmax with
    prev_diff positions changed; mask: locked_frac of positions locked.
    Returns dict of numpy arrays."""
    rng = np.random.default_rng([seed, C, V])
    sure = rng.random(C) < 0.4
    h = np.where(sure, rng.integers(0, 65, C) / 4096.0,
                 np.minimum(rng.exponential(2.0, C), np.log(V))).astype(np.float32)
    if nan_at is not None:
        h[nan_at] = np.nan
    argmax = rng.integers(0, V, C).astype(np.int32)
    prev = argmax.copy()
    if prev_diff:
        at = rng.choice(C, size=prev_diff, replace=False)
        prev[at] = (prev[at] + 1) % V
    return {
        "entropy": h,
        "argmax": argmax,
        "draw": rng.integers(0, V, C).astype(np.int32),
        "prev": prev,
        "canvas": rng.integers(0, V, C).astype(np.int32),
        "mask": (rng.random(C) < locked_frac).astype(np.uint8),
    }

"""Python binding of libdg.so, the gfx950 canvas-denoising library.

Argument marshalling only: every step of the denoise pass runs in the HIP
kernels behind the C ABI declared in include/dg.h.  Device buffers are torch
tensors (torch provides device memory and streams); their data pointers and
the current HIP stream are passed through unchanged.  Importing this module
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg.so")

DG_OK, DG_EINVAL, DG_ENOMEM, DG_EHIP, DG_ECAPACITY, DG_ESTATE, DG_ENONFINITE = 0, -1, -2, -3, -4, -5, -6
DG_ETOKEN = -7
DG_F32, DG_BF16, DG_FP8_E4M3, DG_MXFP4 = 0, 1, 2, 3
DG_T_EMBED, DG_T_WQ, DG_T_WK, DG_T_WV, DG_T_WO, DG_T_WR, DG_T_WG, DG_T_WU, DG_T_WD = range(9)
DG_T_SC_WG, DG_T_SC_WU, DG_T_SC_WD = 9, 10, 11
DG_CAP_LOGITS, DG_CAP_STATS, DG_CAP_ROUTING, DG_CAP_HIDDEN, DG_CAP_ATTN, DG_CAP_ROUTER_LOGITS = 1, 2, 4, 8, 16, 32
DG_CAP_ENTROPY = 64
DG_CAP_SELFCOND = 128

EXPORTED = (
    "dg_create", "dg_destroy", "dg_last_error", "dg_load_tensor", "dg_prefill_prompt_kv",
    "dg_denoise_step", "dg_generate_block", "dg_commit_canvas", "dg_check_finite",
    "dg_reset_context", "dg_get_state", "dg_get_capture", "dg_get_kv", "dg_attention",
    "dg_moe_layer", "dg_init_canvas", "dg_profile_begin", "dg_profile_end", "dg_set_kv",
    "dg_set_capture", "dg_set_graphs", "dg_eb_sample", "dg_denoise_step_eb",
    "dg_generate_block_eb", "dg_attention_workspace_size", "dg_attention_noalloc",
    "dg_denoise_step_batch", "dg_init_canvas_batch", "dg_generate_block_batch",
    "dg_set_self_cond", "dg_set_state",
)
DG_PROF_MOE_GEMM1, DG_PROF_MOE_GEMM2, DG_PROF_ATTENTION, DG_PROF_LM_HEAD, DG_PROF_DENSE = range(5)
DG_PROF_SELF_COND = 5
DG_PROF_N = 6


class DGError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dg error {code}: {msg}")
        self.code = code


class dg_model_cfg(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("canvas", ctypes.c_int32), ("max_ctx", ctypes.c_int64), ("rope_base", ctypes.c_double),
        ("rms_eps", ctypes.c_float), ("temperature", ctypes.c_float),
        ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
        ("capture_mask", ctypes.c_uint32), ("max_batch", ctypes.c_int32),
        ("self_cond", ctypes.c_int32), ("sc_ff", ctypes.c_int32),
    ]


class dg_eb_params(ctypes.Structure):
    _fields_ = [
        ("tau_max", ctypes.c_float), ("tau_min", ctypes.c_float), ("gamma", ctypes.c_float),
        ("theta", ctypes.c_float), ("max_steps", ctypes.c_int32),
    ]


def eb_params(tau_max=0.8, tau_min=0.4, gamma=0.5, theta=0.1, max_steps=48) -> dg_eb_params:
    return dg_eb_params(tau_max, tau_min, gamma, theta, max_steps)


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t)
    sig = {
        "dg_create": ([ctypes.POINTER(dg_model_cfg), ctypes.POINTER(vp)], i32),
        "dg_destroy": ([vp], None),
        "dg_last_error": ([], ctypes.c_char_p),
        "dg_load_tensor": ([vp, i32, i32, i32, vp, sz, vp], i32),
        "dg_prefill_prompt_kv": ([vp, vp, i32, vp], i32),
        "dg_denoise_step": ([vp, vp, vp, i32, i32, u64, vp], i32),
        "dg_generate_block": ([vp, vp, i32, u64, i32, vp], i32),
        "dg_commit_canvas": ([vp, vp, vp], i32),
        "dg_check_finite": ([vp, vp], i32),
        "dg_reset_context": ([vp], i32),
        "dg_get_state": ([vp, ctypes.POINTER(i64), ctypes.POINTER(i32)], i32),
        "dg_get_capture": ([vp, u32, i32, vp, sz, vp], i32),
        "dg_get_kv": ([vp, i32, i32, i64, i64, vp, vp], i32),
        "dg_set_kv": ([vp, i32, i32, i64, i64, vp, vp], i32),
        "dg_set_capture": ([vp, u32], i32),
        "dg_set_graphs": ([vp, i32], i32),
        "dg_attention": ([vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float, i32, i32,
                          i32, vp, sz, vp], i32),
        "dg_attention_workspace_size": ([i32, i32, i32, i32, i32, i32, i32, i32,
                                         ctypes.POINTER(sz)], i32),
        "dg_attention_noalloc": ([vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float,
                                  i32, i32, i32, vp], i32),
        "dg_denoise_step_batch": ([vp, vp, vp, i32, i32, i32, u64, vp], i32),
        "dg_init_canvas_batch": ([vp, vp, vp, i32, u64, vp], i32),
        "dg_generate_block_batch": ([vp, vp, i32, i32, u64, vp], i32),
        "dg_set_self_cond": ([vp, vp, i32, vp], i32),
        "dg_set_state": ([vp, i64, i32], i32),
        "dg_moe_layer": ([vp, i32, vp, i32, vp, vp, vp, vp], i32),
        "dg_init_canvas": ([vp, vp, vp, u64, vp], i32),
        "dg_profile_begin": ([vp, i32], i32),
        "dg_profile_end": ([vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)], i32),
        "dg_eb_sample": ([vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                          ctypes.POINTER(dg_eb_params), u64, i32, vp], i32),
        "dg_denoise_step_eb": ([vp, vp, vp, i32, ctypes.POINTER(dg_eb_params), u64, vp, vp], i32),
        "dg_generate_block_eb": ([vp, vp, ctypes.POINTER(dg_eb_params), u64, i32,
                                  ctypes.POINTER(i32), vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load_library()


def _check(code: int) -> int:
    if code != DG_OK:
        raise DGError(code, _lib.dg_last_error().decode())
    return code


def _ptr(t) -> int | None:
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    return int(t)


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------------ C ABI, same names
def dg_create(cfg: dg_model_cfg) -> int:
    h = ctypes.c_void_p()
    _check(_lib.dg_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def dg_destroy(h) -> None:
    _lib.dg_destroy(h)


def dg_last_error() -> str:
    return _lib.dg_last_error().decode()


def dg_load_tensor(h, kind: int, layer: int, expert: int, host_array, scales=None) -> None:
    """host_array: C-contiguous numpy array in the tensor's storage type."""
    if not host_array.flags["C_CONTIGUOUS"]:
        raise ValueError("host_array must be C-contiguous")
    if scales is not None and (scales.dtype.itemsize not in (1, 4) or not scales.flags["C_CONTIGUOUS"]):
        raise ValueError("scales must be contiguous float32 (e4m3) or uint8 (MX FP4 E8M0)")
    _check(_lib.dg_load_tensor(h, kind, layer, expert, host_array.ctypes.data,
                               host_array.nbytes, _ptr(scales)))


def dg_prefill_prompt_kv(h, d_prompt_ids, P: int, stream=None) -> None:
    _check(_lib.dg_prefill_prompt_kv(h, _ptr(d_prompt_ids), P, _stream(stream)))


def dg_denoise_step(h, d_canvas, d_locked_mask, step: int, T: int, seed: int,
                    stream=None) -> None:
    _check(_lib.dg_denoise_step(h, _ptr(d_canvas), _ptr(d_locked_mask), step, T, seed,
                                _stream(stream)))


def dg_denoise_step_batch(h, d_canvas, d_locked_mask, B: int, step: int, T: int, seed: int,
                          stream=None) -> None:
    _check(_lib.dg_denoise_step_batch(h, _ptr(d_canvas), _ptr(d_locked_mask), B, step, T, seed,
                                      _stream(stream)))


def dg_init_canvas_batch(h, d_canvas, d_locked_mask, B: int, seed: int, stream=None) -> None:
    _check(_lib.dg_init_canvas_batch(h, _ptr(d_canvas), _ptr(d_locked_mask), B, seed,
                                     _stream(stream)))


def dg_generate_block_batch(h, d_out_tokens, B: int, T: int, seed: int, stream=None) -> None:
    _check(_lib.dg_generate_block_batch(h, _ptr(d_out_tokens), B, T, seed, _stream(stream)))


def dg_set_self_cond(h, d_z, rows: int, stream=None) -> None:
    _check(_lib.dg_set_self_cond(h, _ptr(d_z), rows, _stream(stream)))


def dg_init_canvas(h, d_canvas, d_locked_mask, seed: int, stream=None) -> None:
    _check(_lib.dg_init_canvas(h, _ptr(d_canvas), _ptr(d_locked_mask), seed, _stream(stream)))


def dg_generate_block(h, d_out_tokens, T: int, seed: int, commit: bool = True,
                      stream=None) -> None:
    _check(_lib.dg_generate_block(h, _ptr(d_out_tokens), T, seed, int(bool(commit)),
                                  _stream(stream)))


def dg_eb_sample(d_entropy, d_argmax, d_draw, d_prev_argmax, d_canvas, d_locked_mask, d_info,
                 C: int, V: int, step: int, params: dg_eb_params, seed: int, k_blk: int,
                 stream=None) -> None:
    _check(_lib.dg_eb_sample(_ptr(d_entropy), _ptr(d_argmax), _ptr(d_draw), _ptr(d_prev_argmax),
                             _ptr(d_canvas), _ptr(d_locked_mask), _ptr(d_info), C, V, step,
                             ctypes.byref(params), seed, k_blk, _stream(stream)))


def dg_denoise_step_eb(h, d_canvas, d_locked_mask, step: int, params: dg_eb_params, seed: int,
                       d_info=None, stream=None) -> None:
    _check(_lib.dg_denoise_step_eb(h, _ptr(d_canvas), _ptr(d_locked_mask), step,
                                   ctypes.byref(params), seed, _ptr(d_info), _stream(stream)))


def dg_generate_block_eb(h, d_out_tokens, params: dg_eb_params, seed: int, commit: bool = True,
                         stream=None) -> int:
    """Returns the number of passes run."""
    n = ctypes.c_int32()
    _check(_lib.dg_generate_block_eb(h, _ptr(d_out_tokens), ctypes.byref(params), seed,
                                     int(bool(commit)), ctypes.byref(n), _stream(stream)))
    return n.value


def dg_commit_canvas(h, d_canvas, stream=None) -> None:
    _check(_lib.dg_commit_canvas(h, _ptr(d_canvas), _stream(stream)))


def dg_check_finite(h, stream=None) -> None:
    _check(_lib.dg_check_finite(h, _stream(stream)))


def dg_reset_context(h) -> None:
    _check(_lib.dg_reset_context(h))


def dg_set_state(h, n_ctx: int, k_blk: int) -> None:
    _check(_lib.dg_set_state(h, n_ctx, k_blk))


def dg_get_state(h):
    n = ctypes.c_int64()
    k = ctypes.c_int32()
    _check(_lib.dg_get_state(h, ctypes.byref(n), ctypes.byref(k)))
    return n.value, k.value


def dg_set_capture(h, capture_mask: int) -> None:
    _check(_lib.dg_set_capture(h, capture_mask))


def dg_set_graphs(h, enable: bool) -> None:
    _check(_lib.dg_set_graphs(h, 1 if enable else 0))


def dg_get_capture(h, what: int, layer: int, d_dst, stream=None) -> None:
    nbytes = d_dst.numel() * d_dst.element_size()
    _check(_lib.dg_get_capture(h, what, layer, _ptr(d_dst), nbytes, _stream(stream)))


def dg_get_kv(h, layer: int, which: int, row0: int, n: int, d_dst, stream=None) -> None:
    _check(_lib.dg_get_kv(h, layer, which, row0, n, _ptr(d_dst), _stream(stream)))


def dg_set_kv(h, layer: int, which: int, row0: int, n: int, d_src, stream=None) -> None:
    _check(_lib.dg_set_kv(h, layer, which, row0, n, _ptr(d_src), _stream(stream)))


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def dg_attention_workspace_size(Hq: int, Hkv: int, M: int, S: int, D: int, causal: bool,
                                q_pos0: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.dg_attention_workspace_size(Hq, Hkv, M, S, D, int(bool(causal)), q_pos0, dtype,
                                            ctypes.byref(n)))
    return n.value


def dg_attention(d_q, d_k, d_v, d_o, Hq: int, Hkv: int, M: int, S: int, D: int, scale: float,
                 causal: bool, q_pos0: int, dtype: int, d_workspace=None, stream=None) -> None:
    """d_workspace: device tensor of at least dg_attention_workspace_size bytes (or None
    when that is 0)."""
    _check(_lib.dg_attention(_ptr(d_q), _ptr(d_k), _ptr(d_v), _ptr(d_o), Hq, Hkv, M, S, D,
                             scale, int(bool(causal)), q_pos0, dtype, _ptr(d_workspace),
                             _nbytes(d_workspace), _stream(stream)))


def dg_attention_noalloc(d_q, d_k, d_v, d_o, Hq: int, Hkv: int, M: int, S: int, D: int,
                         scale: float, causal: bool, q_pos0: int, dtype: int,
                         stream=None) -> None:
    _check(_lib.dg_attention_noalloc(_ptr(d_q), _ptr(d_k), _ptr(d_v), _ptr(d_o), Hq, Hkv, M, S,
                                     D, scale, int(bool(causal)), q_pos0, dtype,
                                     _stream(stream)))


def dg_moe_layer(h, layer: int, d_x, n_tokens: int, d_y, d_idx=None, d_gates=None,
                 stream=None) -> None:
    _check(_lib.dg_moe_layer(h, layer, _ptr(d_x), n_tokens, _ptr(d_y), _ptr(d_idx),
                             _ptr(d_gates), _stream(stream)))


def dg_profile_begin(h, max_launches: int) -> None:
    _check(_lib.dg_profile_begin(h, max_launches))


def dg_profile_end(h):
    """Returns (summed ms, launch counts), one entry per DG_PROF_* class."""
    ms = (ctypes.c_double * DG_PROF_N)()
    n = (ctypes.c_int32 * DG_PROF_N)()
    _check(_lib.dg_profile_end(h, ms, n))
    return list(ms), list(n)


# ------------------------------------------------------------------ convenience
def make_cfg(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, n_experts, top_k, d_ff, vocab,
             canvas, max_ctx, rope_base=10000.0, rms_eps=1e-6, temperature=1.0,
             act_dtype=DG_BF16, expert_dtype=DG_BF16, capture_mask=0,
             max_batch=1, self_cond=0, sc_ff=0) -> dg_model_cfg:
    return dg_model_cfg(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, n_experts, top_k,
                        d_ff, vocab, canvas, max_ctx, rope_base, rms_eps, temperature,
                        act_dtype, expert_dtype, capture_mask, max_batch, int(self_cond),
                        sc_ff)


def load_weights(h, n_layers: int, n_experts: int, tensor_fn, experts_at_once: bool = True,
                 self_cond: bool = False):
    """Load every tensor of a model.

    tensor_fn(kind, layer, expert) returns a numpy array in storage type, or
    (codes, scales) for e4m3 expert tensors; expert is None for dense tensors
    and -1 for "all experts at once" ([E, in, out]).  With self_cond the three
    DG_T_SC_* tensors are loaded too (layer 0).
    """
    def put(kind, layer, expert, val):
        if isinstance(val, tuple):
            dg_load_tensor(h, kind, layer, expert, val[0], val[1])
        else:
            dg_load_tensor(h, kind, layer, expert, val)

    put(DG_T_EMBED, 0, 0, tensor_fn(DG_T_EMBED, 0, None))
    for l in range(n_layers):
        for kind in (DG_T_WQ, DG_T_WK, DG_T_WV, DG_T_WO, DG_T_WR):
            put(kind, l, 0, tensor_fn(kind, l, None))
        for kind in (DG_T_WG, DG_T_WU, DG_T_WD):
            if experts_at_once:
                put(kind, l, -1, tensor_fn(kind, l, -1))
            else:
                for e in range(n_experts):
                    put(kind, l, e, tensor_fn(kind, l, e))
    if self_cond:
        for kind in (DG_T_SC_WG, DG_T_SC_WU, DG_T_SC_WD):
            put(kind, 0, 0, tensor_fn(kind, 0, None))

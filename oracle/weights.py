"""Widening of the shared synthetic weights to float64 for the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The weights themselves come from the seeded input generator (``fixtures``);
this adapter only turns their storage form into exact float64 values:
bf16 bit patterns are widened exactly, e4m3 codes decode to their value times
the per-output-column scale (the fp8 expert storage of the long-context
configuration), MX FP4 codes to their E2M1 value times their block's E8M0 scale.
"""
from __future__ import annotations

import numpy as np

import fixtures as fx

from .numerics import e4m3_value_of_code, mxfp4_dequant


def _bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class FixtureWeights:
    """Lazily generated, cached storage-form weights of one workload."""

    def __init__(self, w: "fx.Workload", cache_experts: bool = True):
        self.w = w
        self._cache: dict = {}
        self.cache_experts = cache_experts

    def _widen(self, kind: str, raw) -> np.ndarray:
        dt = fx.storage_dtype(self.w, kind)
        if dt == "f32":
            return np.asarray(raw, dtype=np.float64)
        if dt == "bf16":
            return _bits_to_f64(raw)
        codes, scales = raw
        if dt == "mxfp4":
            return mxfp4_dequant(codes, scales)
        return e4m3_value_of_code(codes) * scales.astype(np.float64)[None, :]

    def dense(self, kind: str, layer: int = 0) -> np.ndarray:
        key = (kind, layer)
        if key not in self._cache:
            self._cache[key] = self._widen(kind, fx.model_tensor(self.w, kind, layer))
        return self._cache[key]

    def expert(self, kind: str, layer: int, e: int) -> np.ndarray:
        key = (kind, layer, e)
        raw = self._cache.get(key)
        if raw is None:
            raw = fx.model_tensor(self.w, kind, layer, expert=e)
            if self.cache_experts:
                self._cache[key] = raw
        return self._widen(kind, raw)

    def embed(self) -> np.ndarray:
        return self.dense("embed", 0)

    def forget_layer(self, layer: int) -> None:
        """Drop the cached tensors of one layer (memory only; they are regenerated on use)."""
        for key in [k for k in self._cache if k[0] != "embed" and k[1] == layer]:
            del self._cache[key]


class ArrayWeights:
    """Weights given directly as float64 arrays (tiny hand-built test models).

    ``tensors`` maps "embed" to [V, d] and (kind, layer) to the dense layer
    tensors; expert tensors are [E, in, out].
    """

    def __init__(self, tensors: dict):
        self.t = tensors

    def dense(self, kind: str, layer: int = 0) -> np.ndarray:
        return np.asarray(self.t[(kind, layer)], dtype=np.float64)

    def expert(self, kind: str, layer: int, e: int) -> np.ndarray:
        return np.asarray(self.t[(kind, layer)][e], dtype=np.float64)

    def embed(self) -> np.ndarray:
        return np.asarray(self.t["embed"], dtype=np.float64)

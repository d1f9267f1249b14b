"""Philox4x32-10 and the random streams the samplers draw.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Philox4x32-10 follows its published definition (Salmon, Moraes, Dror & Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11): a 4x32-bit counter and a
2x32-bit key; each of the 10 rounds multiplies counter words 0 and 2 by the two
round constants, keeps high and low halves, XORs the high halves with the
other counter words and the round key, and bumps the key by the two Weyl
constants between rounds.

The entropy-bounded sampler renoises the positions it does not accept
"uniformly at random" ([TR] Method, the paragraph after the update equations),
which is the third stream.

The pages ask for canvas tokens "initialised with random placeholder tokens"
([AS] "How text diffusion actually works", step 1; [TR] Method, forward
process at kappa = 0, i.e. uniform over the vocabulary) and for unlocked
positions to be redrawn from the tempered posterior.  The counter layout below
is this implementation's reading (the pages fix none):

  canvas init : counter (i >> 2, k_blk, 0, 0x494E4954), output word i & 3;
                token = (word * V) >> 32           (multiply-high)
  redraw      : counter (v, i >> 2, s | k_blk << 16, 0x47554D42), word i & 3;
                u = (2 * (word >> 9) + 1) * 2^-24    (exact float in (0, 1))
  renoise     : counter (i >> 2, k_blk, s, 0x524E5345), output word i & 3;
                token = (word * V) >> 32           (multiply-high)
key = (seed & 0xffffffff, seed >> 32).  i = canvas position, v = vocabulary
id, s = pass index, k_blk = index of the canvas within the generation.
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)

INIT_TAG = 0x494E4954
GUMBEL_TAG = 0x47554D42
RENOISE_TAG = 0x524E5345


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on broadcastable uint32 counter words; returns 4 uint32 arrays."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for r in range(10):
        p0 = M0 * x0
        p1 = M1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(k0), lo1, hi0 ^ x3 ^ np.uint64(k1), lo0)
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return tuple(a.astype(np.uint32) for a in (x0, x1, x2, x3))


def _word(words, lane):
    out = np.empty(np.shape(lane), np.uint32)
    for j in range(4):
        sel = lane == j
        out[sel] = words[j][sel]
    return out


def init_canvas(seed: int, k_blk: int, C: int, V: int) -> np.ndarray:
    """Uniform-random canvas over [0, V): the kappa = 0 end of the forward process."""
    i = np.arange(C, dtype=np.uint64)
    w = philox4x32_10(i >> np.uint64(2), k_blk, 0, INIT_TAG, seed & 0xFFFFFFFF, seed >> 32)
    word = _word(w, (i & np.uint64(3)).astype(np.int64))
    return ((word.astype(np.uint64) * np.uint64(V)) >> np.uint64(32)).astype(np.int32)


def gumbel_uniforms(seed: int, k_blk: int, s: int, positions, V: int, v0: int = 0,
                    v1: int | None = None) -> np.ndarray:
    """u[i, v] in (0, 1) for the given positions and vocabulary ids [v0, v1), float64."""
    v1 = V if v1 is None else v1
    pos = np.asarray(positions, dtype=np.uint64)[:, None]
    v = np.arange(v0, v1, dtype=np.uint64)[None, :]
    w = philox4x32_10(v, pos >> np.uint64(2), (s | (k_blk << 16)) & 0xFFFFFFFF, GUMBEL_TAG,
                      seed & 0xFFFFFFFF, seed >> 32)
    lane = np.broadcast_to((pos & np.uint64(3)).astype(np.int64), w[0].shape)
    word = _word(w, lane)
    return ((word >> np.uint32(9)).astype(np.float64) * 2.0 + 1.0) * 2.0 ** -24


def renoise_tokens(seed: int, k_blk: int, s: int, C: int, V: int) -> np.ndarray:
    """Uniform token over [0, V) for every canvas position at pass s (entropy-bounded sampler)."""
    i = np.arange(C, dtype=np.uint64)
    w = philox4x32_10(i >> np.uint64(2), k_blk, s, RENOISE_TAG, seed & 0xFFFFFFFF, seed >> 32)
    word = _word(w, (i & np.uint64(3)).astype(np.int64))
    return ((word.astype(np.uint64) * np.uint64(V)) >> np.uint64(32)).astype(np.int32)

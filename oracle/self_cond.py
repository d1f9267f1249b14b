"""Self-conditioning signal of the decoder, plainly, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ([TR] Method, decoder equation and the update equations
after it; Dataset, "How the data is used"; Experiment, architecture
paragraph):
  * the decoder takes, besides the noisy canvas x_t and the context cache H, a
    continuous signal z_t with one model-width row per canvas position, which
    feeds the model's previous predictions back into it;
  * after a pass, p0 = Softmax(L_t / tau_t) over the vocabulary, and the next
    pass's signal is z = FFW(p0 E), E in R^{V x d} the token embedding and FFW a
    standard feed-forward network;
  * in training the signal is zero for half of the examples; the block adds
    few parameters next to the embedder.

Readings where the pages are silent (each listed with the others in the
design notes):
  * FFW shape: the gated form of the model's own feed-forward blocks, one
    hidden layer of width Fsc with no biases and no norm:
    FFW(u) = (silu(u Wg) * (u Wu)) Wd, Wg/Wu [d, Fsc], Wd [Fsc, d];
  * injection point: z is added to the canvas token embedding, x_i = E[x_i] +
    z_i, before the first block (the one place a per-position d-vector enters
    a pre-norm stack without a new weight);
  * the first pass of a block has no previous prediction and takes z = 0 (the
    zero state the training recipe also uses);
  * tau_t is the temperature of the pass that produced the logits (1 / the
    sampler's inverse temperature; tau_s of the entropy-bounded sampler);
  * precision plan (bf16 configurations): p0, u = p0 E and the SwiGLU output
    are rounded to bf16 where the product stores them as GEMM operands; z stays
    in full precision.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import round_bf16, silu, softmax


def posterior(z) -> np.ndarray:
    """p0 = Softmax(z) per row, z = L_t / tau_t the tempered logits [rows, V]
    ([TR] Method, first update equation)."""
    return softmax(np.asarray(z, np.float64), axis=-1)


def expected_embedding(p0, E) -> np.ndarray:
    """u = p0 E: each row is the embedding averaged under that row's posterior
    ([TR] Method, second update equation, the argument of FFW)."""
    return np.asarray(p0, np.float64) @ np.asarray(E, np.float64)


def ffw(u, wg, wu, wd, hidden_round=None) -> np.ndarray:
    """The feed-forward block (reading above): (silu(u Wg) * (u Wu)) Wd."""
    u = np.asarray(u, np.float64)
    h = silu(u @ wg) * (u @ wu)
    if hidden_round is not None:
        h = hidden_round(h)
    return h @ wd


@dataclass
class SelfCond:
    p0: np.ndarray   # [rows, V] posterior (as rounded for the bf16 plan)
    u: np.ndarray    # [rows, d] p0 E (before the bf16 rounding of the FFW input)
    z: np.ndarray    # [rows, d] the next pass's signal


def next_signal(z_tempered, E, wg, wu, wd, bf16: bool) -> SelfCond:
    """z_{t - dt} = FFW(Softmax(L_t / tau_t) E) for the rows of one pass."""
    rnd = round_bf16 if bf16 else (lambda a: np.asarray(a, np.float64))
    p0 = rnd(posterior(z_tempered))
    u = expected_embedding(p0, E)
    z = ffw(rnd(u), wg, wu, wd, hidden_round=round_bf16 if bf16 else None)
    return SelfCond(p0=p0, u=u, z=z)

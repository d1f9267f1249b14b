"""The entropy-bounded sampler with temperature annealing and adaptive stopping, plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ([TR] Method, the paragraphs after the update equations on
the sampler and on adaptive stopping; Experiment, the paragraph on the
recommended sampler):
  * tokens are accepted in rank order of their predictive entropy, lowest
    first, while a mutual-information bound of the accepted set stays strictly
    below an error tolerance; every other token is renoised uniformly at
    random;
  * the probabilities are tempered with tau < 1, annealed linearly from
    tau_max = 0.8 down to tau_min = 0.4 across the denoising time;
  * denoising halts early when the mean predictive entropy across the whole
    canvas is below a threshold and the deterministic predictions of two
    consecutive steps are identical; at most 48 steps; the thresholds for
    stopping and for selection are separate (no values are given).

Readings where the pages are silent:
  * predictive entropy of position i at pass s: H_i = -sum_v p_v log p_v with
    p = Softmax(L_i / tau_s), in nats;
  * the bound: for the n lowest-entropy candidates H_(1) <= ... <= H_(n),
    B(n) = sum_{j<=n} H_(j) - max_{j<=n} H_(j), the sum of the marginal
    entropies minus the largest one, which bounds the total correlation of
    the n tokens (sum of marginal entropies minus the joint entropy, and the
    joint entropy is at least the largest marginal one).  Candidates are
    accepted in rank order while B stays below gamma; the first one that would
    bring it to gamma or above ends acceptance.  B(1) = 0, so every pass
    accepts at least one position (ties in entropy go to the lower position);
  * candidates are the unlocked positions; an accepted position takes its
    Gumbel-max draw from p (the draw of the fixed-schedule sampler, at tau_s)
    and is locked; unaccepted unlocked positions are renoised uniformly
    (``philox.renoise_tokens``); locked positions are never written;
  * tau_s = tau_min + (tau_max - tau_min) * (S - 1 - s) / (S - 1) for pass s of
    at most S passes (tau_min when S = 1);
  * stop test at pass s >= 1: mean_i H_i over all C positions (locked ones
    included) below theta and argmax_i identical to pass s - 1 at every
    position; it is taken before acceptance.  When it holds, or at the last
    pass s = S - 1, every unlocked position takes its argmax and is locked.
    A pass that leaves no position unlocked also ends the block;
  * sums (the mean, the prefix sums of the bound) are float64, accumulated in
    order: positions in index order for the mean, candidates in rank order for
    the bound.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import renoise_tokens


@dataclass(frozen=True)
class EbParams:
    tau_max: float = 0.8
    tau_min: float = 0.4
    gamma: float = 0.5        # tolerance on the bound B(n), nats
    theta: float = 0.1        # stop threshold on the mean entropy, nats
    max_steps: int = 48


def tau_at(s: int, p: EbParams) -> float:
    """Linear annealing from tau_max at the first pass to tau_min at the last."""
    S = p.max_steps
    if S <= 1:
        return float(p.tau_min)
    t = (S - 1 - s) / (S - 1)
    return float(p.tau_min) + (float(p.tau_max) - float(p.tau_min)) * t


def entropy(z) -> np.ndarray:
    """Entropy of Softmax(z) per row of the tempered logits z [C, V] (materialised)."""
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=-1, keepdims=True)
    logp = (z - m) - np.log(e.sum(axis=-1, keepdims=True))
    return -np.sum(np.where(p > 0, p * logp, 0.0), axis=-1)


def entropy_partial(z) -> tuple:
    """(m, s, q) of one vocabulary slice of one row: m = max z, s = sum e^(z - m),
    q = sum e^(z - m) (z - m).  Then H = log s - q / s."""
    z = np.asarray(z, np.float64)
    m = z.max()
    d = z - m
    e = np.exp(d)
    return m, e.sum(), np.sum(e * d)


def entropy_merge(a, b) -> tuple:
    """Combine two slices' (m, s, q) into those of their union."""
    m = max(a[0], b[0])
    out_s = 0.0
    out_q = 0.0
    for (mi, si, qi) in (a, b):
        f = np.exp(mi - m)
        out_s += f * si
        out_q += f * (qi + (mi - m) * si)
    return m, out_s, out_q


def entropy_of_partial(t) -> float:
    return float(np.log(t[1]) - t[2] / t[1])


def mi_bound(h_prefix) -> float:
    """B(n) of an accepted set given its entropies: sum minus the largest."""
    h = np.asarray(h_prefix, np.float64)
    return float(h.sum() - h.max()) if h.size else 0.0


def rank_order(H, mask) -> np.ndarray:
    """Unlocked positions sorted by entropy ascending, ties to the lower position."""
    H = np.asarray(H, np.float64)
    unl = np.flatnonzero(np.asarray(mask) == 0)
    return unl[np.lexsort((unl, H[unl]))]


def accept_count(h_sorted, gamma: float) -> int:
    """Number of sorted candidates accepted: in rank order while B(n) < gamma (0 if none).

    B is evaluated one prefix at a time: the running sum in rank order (float64)
    minus the prefix's largest entropy, which is its last one."""
    h = np.asarray(h_sorted, np.float64)
    if h.size == 0:
        return 0
    n = 1
    run = h[0]
    for k in range(1, h.size):
        run = run + h[k]
        if run - h[k] < gamma:     # B(k + 1) with the prefix's largest entropy h[k]
            n = k + 1
        else:
            break
    return n


def mean_entropy(H) -> float:
    acc = 0.0
    for x in np.asarray(H, np.float64):
        acc = acc + x
    return acc / len(H)


@dataclass
class EbResult:
    canvas: np.ndarray
    mask: np.ndarray
    done: bool
    stopped: bool             # the adaptive stop test held
    accepted: np.ndarray      # positions accepted at this pass (rank order); all newly locked if done
    order: np.ndarray         # candidates in rank order
    n_accept: int
    mean_h: float
    prefix: np.ndarray        # running sums of the sorted candidate entropies


def eb_update(canvas, mask, H, argmax, draw, prev_argmax, s: int, p: EbParams, seed: int,
              k_blk: int, V: int) -> EbResult:
    """One pass of the sampler given the pass's entropies, argmax and Gumbel draws.

    prev_argmax is the previous pass's argmax (ignored at s = 0)."""
    canvas = np.array(canvas, dtype=np.int32, copy=True)
    mask = np.array(mask, dtype=np.uint8, copy=True)
    H = np.asarray(H, np.float64)
    argmax = np.asarray(argmax, np.int32)
    C = canvas.shape[0]
    mh = mean_entropy(H)
    stopped = (s >= 1 and mh < p.theta and prev_argmax is not None
               and np.array_equal(np.asarray(prev_argmax, np.int32), argmax))
    order = rank_order(H, mask)
    prefix = np.cumsum(H[order]) if order.size else np.zeros(0)
    if stopped or s == p.max_steps - 1:
        canvas[order] = argmax[order]
        mask[order] = 1
        return EbResult(canvas, mask, True, stopped, order, order, order.size, mh, prefix)
    n = accept_count(H[order], p.gamma)
    acc = order[:n]
    rest = order[n:]
    canvas[acc] = np.asarray(draw, np.int32)[acc]
    mask[acc] = 1
    canvas[rest] = renoise_tokens(seed, k_blk, s, C, V)[rest]
    done = bool(np.all(mask != 0))
    return EbResult(canvas, mask, done, False, acc, order, n, mh, prefix)

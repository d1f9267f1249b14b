"""Pins of the oracle's attention, routing, MoE, LM-head statistics and sampler (CPU only)."""
import math

import numpy as np
import pytest
import torch
from scipy import special, stats

from oracle import model as om
from oracle import philox as ph
from oracle.numerics import silu, softmax


# ------------------------------------------------------------------ attention
def _sdpa(q, k, v, group, mask=None):
    kk = torch.tensor(k).repeat_interleave(group, dim=0)
    vv = torch.tensor(v).repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), kk, vv, attn_mask=mask).numpy()


def test_attention_matches_torch_sdpa_noncausal_gqa():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 9, 16))
    k = rng.standard_normal((2, 23, 16))
    v = rng.standard_normal((2, 23, 16))
    assert np.allclose(om.attention(q, k, v), _sdpa(q, k, v, 2), atol=1e-12)


def test_attention_matches_torch_sdpa_causal_with_prefix():
    rng = np.random.default_rng(1)
    n_ctx, M = 11, 7
    q = rng.standard_normal((4, M, 8))
    k = rng.standard_normal((1, n_ctx + M, 8))
    v = rng.standard_normal((1, n_ctx + M, 8))
    qp = np.arange(n_ctx, n_ctx + M)
    kp = np.arange(n_ctx + M)
    mask = torch.tensor(kp[None, :] <= qp[:, None])
    got = om.attention(q, k, v, causal=True, q_pos=qp, k_pos=kp)
    assert np.allclose(got, _sdpa(q, k, v, 4, mask), atol=1e-12)


def test_attention_brute_force_loops():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 3, 4))
    k = rng.standard_normal((1, 5, 4))
    v = rng.standard_normal((1, 5, 4))
    got = om.attention(q, k, v)
    for h in range(2):
        for i in range(3):
            w = [math.exp(sum(q[h, i, t] * k[0, j, t] for t in range(4)) / 2.0) for j in range(5)]
            z = sum(w)
            for t in range(4):
                assert abs(got[h, i, t] - sum(w[j] * v[0, j, t] for j in range(5)) / z) < 1e-12


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 6, 4))
    # all keys equal => uniform weights => mean of V
    k = np.tile(rng.standard_normal((1, 1, 4)), (1, 6, 1))
    q = rng.standard_normal((1, 2, 4))
    assert np.allclose(om.attention(q, k, v)[0], v[0].mean(0), atol=1e-14)
    # permuting (key, value) rows jointly leaves the non-causal output unchanged
    k = rng.standard_normal((1, 6, 4))
    perm = rng.permutation(6)
    assert np.allclose(om.attention(q, k, v), om.attention(q, k[:, perm], v[:, perm]), atol=1e-13)


# ------------------------------------------------------------------ routing / MoE
def test_route_topk_brute_force_and_ties():
    rng = np.random.default_rng(4)
    r = rng.standard_normal((20, 8))
    idx, g, margin = om.route_topk(r, 3)
    for t in range(20):
        p = softmax(r[t])
        order = sorted(range(8), key=lambda e: (-p[e], e))[:3]
        assert list(idx[t]) == order
        assert np.isclose(g[t].sum(), 1.0)
        assert np.allclose(g[t], p[order] / p[order].sum())
        srt = sorted(r[t], reverse=True)
        assert np.isclose(margin[t], srt[2] - srt[3])
    idx, g, _ = om.route_topk(np.zeros((2, 8)), 3)
    assert idx.tolist() == [[0, 1, 2], [0, 1, 2]] and np.allclose(g, 1 / 3)


def _rand_experts(rng, E, d, F):
    return (rng.standard_normal((E, d, F)) * 0.3, rng.standard_normal((E, d, F)) * 0.3,
            rng.standard_normal((E, F, d)) * 0.3)


def test_moe_sparse_equals_dense_over_all_experts():
    rng = np.random.default_rng(5)
    M, d, F, E, k = 10, 6, 5, 5, 2
    b = rng.standard_normal((M, d))
    wg, wu, wd = _rand_experts(rng, E, d, F)
    idx, g, _ = om.route_topk(rng.standard_normal((M, E)), k)
    y = om.moe_ffn(b, idx, g, lambda e: (wg[e], wu[e], wd[e]))
    dense_gate = np.zeros((M, E))
    np.put_along_axis(dense_gate, idx, g, axis=1)
    ref = np.zeros((M, d))
    for e in range(E):
        ref += dense_gate[:, e:e + 1] * ((silu(b @ wg[e]) * (b @ wu[e])) @ wd[e])
    assert np.allclose(y, ref, atol=1e-12)


def test_moe_single_expert_is_dense_swiglu_ffn():
    rng = np.random.default_rng(6)
    b = rng.standard_normal((4, 6))
    wg, wu, wd = _rand_experts(rng, 1, 6, 3)
    idx, g, _ = om.route_topk(rng.standard_normal((4, 1)), 1)
    y = om.moe_ffn(b, idx, g, lambda e: (wg[e], wu[e], wd[e]))
    tb = torch.tensor(b)
    ref = (torch.nn.functional.silu(tb @ torch.tensor(wg[0])) * (tb @ torch.tensor(wu[0]))) \
        @ torch.tensor(wd[0])
    assert np.allclose(y, ref.numpy(), atol=1e-12)


def test_moe_all_experts_is_full_softmax_mixture():
    rng = np.random.default_rng(7)
    M, d, F, E = 3, 4, 3, 4
    b = rng.standard_normal((M, d))
    wg, wu, wd = _rand_experts(rng, E, d, F)
    r = rng.standard_normal((M, E))
    idx, g, _ = om.route_topk(r, E)
    y = om.moe_ffn(b, idx, g, lambda e: (wg[e], wu[e], wd[e]))
    p = softmax(r)
    ref = sum(p[:, e:e + 1] * ((silu(b @ wg[e]) * (b @ wu[e])) @ wd[e]) for e in range(E))
    assert np.allclose(y, ref, atol=1e-12)


# ------------------------------------------------------------------ LM-head statistics
def test_lm_head_stats_brute_force_and_bounds():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((6, 50)) * 3
    z[2, 7] = z[2, 9] = z[2].max() + 1.0      # tie: lower id wins
    st = om.lm_head_stats(z)
    assert st.argmax[2] == 7 and st.top2_gap[2] == 0.0
    assert np.allclose(st.lse, special.logsumexp(z, axis=-1), atol=1e-12)
    assert np.all(st.m <= st.lse) and np.all(st.lse <= st.m + math.log(50) + 1e-12)
    assert np.allclose(np.exp(z - st.lse[:, None]).sum(-1), 1.0)
    c = om.lm_head_stats(np.full((2, 1024), 0.37))
    assert np.all(c.conf == -math.log(1024)) or np.allclose(c.conf, -math.log(1024), atol=1e-15)


# ------------------------------------------------------------------ Gumbel redraw
def test_gumbel_max_draws_follow_softmax():
    V = 8
    z = np.array([0.5, -1.0, 2.0, 0.0, 1.0, -0.5, 0.3, 1.5])
    draws = []
    for s in range(40):
        u = ph.gumbel_uniforms(11, 0, s, np.arange(4096), V)
        w, _ = om.gumbel_draw(np.tile(z, (4096, 1)), u)
        draws.append(w)
    cnt = np.bincount(np.concatenate(draws), minlength=V)
    p = stats.chisquare(cnt, softmax(z) * cnt.sum()).pvalue
    assert p > 1e-4


def test_gumbel_dominant_logit_always_wins():
    u = ph.gumbel_uniforms(1, 0, 0, np.arange(64), 100)
    z = np.zeros((64, 100))
    z[:, 42] = 50.0
    w, gap = om.gumbel_draw(z, u)
    assert np.all(w == 42) and np.all(gap > 10)


# ------------------------------------------------------------------ sampler schedule
def test_lock_schedule_totals():
    counts = []
    unlocked = 256
    for s in range(12):
        n = om.lock_count(s, 12, 256, unlocked)
        counts.append(n)
        unlocked -= n
    assert counts == [22] * 11 + [14] and unlocked == 0


def test_sampler_invariants_over_a_trajectory():
    rng = np.random.default_rng(9)
    C, T = 256, 12
    canvas = rng.integers(0, 1000, C).astype(np.int32)
    mask = np.zeros(C, np.uint8)
    for s in range(T):
        conf = np.round(rng.standard_normal(C), 1)     # many ties
        a = rng.integers(0, 1000, C)
        red = rng.integers(0, 1000, C)
        r = om.sampler_update(canvas, mask, conf, a, red, s, T)
        locked_before = mask == 1
        assert np.array_equal(r.canvas[locked_before], canvas[locked_before])
        assert int(r.mask.sum() - mask.sum()) == om.lock_count(s, T, C, int((mask == 0).sum()))
        unl = [i for i in range(C) if mask[i] == 0]
        top = sorted(unl, key=lambda i: (-conf[i], i))[:len(r.new_locks)]
        assert sorted(top) == sorted(r.new_locks.tolist())
        assert np.array_equal(r.canvas[r.new_locks], a[r.new_locks])
        assert np.array_equal(r.canvas[r.redrawn], red[r.redrawn])
        canvas, mask = r.canvas, r.mask
    assert mask.sum() == C


def test_sampler_all_locked_is_noop():
    c = np.arange(16, dtype=np.int32)
    m = np.ones(16, np.uint8)
    r = om.sampler_update(c, m, np.zeros(16), np.zeros(16), np.zeros(16), 3, 12)
    assert np.array_equal(r.canvas, c) and np.array_equal(r.mask, m) and r.new_locks.size == 0

"""Pins of the oracle's self-conditioning signal z = FFW(Softmax(L/tau) E): closed forms at a
one-hot and a uniform posterior, linearity in p0, the feed-forward block against an elementwise
closed form with permutation weights (a transposed or swapped operand moves the indices), the
injection point (a signal E[y] - E[x] turns canvas x into canvas y), and the chaining of the
signal over a block."""
import numpy as np
import pytest
from scipy.special import expit, softmax as sp_softmax

import fixtures as fx
from oracle import model as om
from oracle import self_cond as sc
from oracle.numerics import round_bf16
from oracle.weights import ArrayWeights, FixtureWeights


def _tiny_sc(rng, d=32, F=48, V=64, act="f32", zero_down=False, sc_scale=0.4):
    w = fx.Workload("tiny_sc", n_layers=2, d_model=d, n_q_heads=4, n_kv_heads=2, head_dim=8,
                    n_experts=4, top_k=2, d_ff=16, vocab=V, prompt_len=10, canvas=12, T=4,
                    act=act, experts=act, self_cond=True, sc_ff=F, temperature=0.5)
    t = {"embed": rng.standard_normal((V, d)) * 0.5}
    for l in range(2):
        t[("wq", l)] = rng.standard_normal((d, 32)) * 0.3
        t[("wk", l)] = rng.standard_normal((d, 16)) * 0.3
        t[("wv", l)] = rng.standard_normal((d, 16)) * 0.3
        t[("wo", l)] = rng.standard_normal((32, d)) * 0.3
        t[("wr", l)] = rng.standard_normal((d, 4)) * 0.3
        t[("wg", l)] = rng.standard_normal((4, d, 16)) * 0.3
        t[("wu", l)] = rng.standard_normal((4, d, 16)) * 0.3
        t[("wd", l)] = rng.standard_normal((4, 16, d)) * 0.3
    t[("sc_wg", 0)] = rng.standard_normal((d, F)) * sc_scale
    t[("sc_wu", 0)] = rng.standard_normal((d, F)) * sc_scale
    t[("sc_wd", 0)] = rng.standard_normal((F, d)) * sc_scale * (not zero_down)
    if act == "bf16":
        t = {key: round_bf16(v) for key, v in t.items()}
    return w, ArrayWeights(t)


def test_posterior_is_the_softmax_of_the_tempered_logits():
    rng = np.random.default_rng(0)
    L = rng.standard_normal((5, 300)) * 4
    for tau in (1.0, 0.4, 2.5):
        p = sc.posterior(L / tau)
        assert np.allclose(p, sp_softmax(L / tau, axis=1), rtol=1e-13, atol=0)
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
    # a constant shift of a row leaves it unchanged
    assert np.allclose(sc.posterior(L + 7.0), sc.posterior(L), rtol=1e-12, atol=0)


def test_one_hot_posterior_gives_the_embedding_row():
    rng = np.random.default_rng(1)
    V, d = 200, 24
    E = rng.standard_normal((V, d))
    ids = np.array([0, 17, 199, 17])
    z = rng.standard_normal((4, V))
    z[np.arange(4), ids] += 5000.0           # exp(-5000) is 0 in float64: p0 is exactly one-hot
    p0 = sc.posterior(z)
    assert np.array_equal(p0, np.eye(V)[ids])
    assert np.array_equal(sc.expected_embedding(p0, E), E[ids])


def test_uniform_posterior_gives_the_mean_embedding():
    rng = np.random.default_rng(2)
    V, d = 333, 20
    E = rng.standard_normal((V, d))
    p0 = sc.posterior(np.full((3, V), -1.25))
    u = sc.expected_embedding(p0, E)
    assert np.allclose(u, np.broadcast_to(E.mean(axis=0), (3, d)), rtol=0, atol=1e-14)


def test_expected_embedding_is_linear_in_the_posterior():
    rng = np.random.default_rng(3)
    V, d = 150, 16
    E = rng.standard_normal((V, d))
    p1 = sc.posterior(rng.standard_normal((2, V)))
    p2 = sc.posterior(3 * rng.standard_normal((2, V)))
    for a in (0.0, 0.3, 1.0):
        mix = sc.expected_embedding(a * p1 + (1 - a) * p2, E)
        assert np.allclose(mix, a * sc.expected_embedding(p1, E) +
                           (1 - a) * sc.expected_embedding(p2, E), rtol=0, atol=1e-13)


def test_ffw_closed_form_with_permutation_weights():
    """Wg = a P1, Wu = b P2, Wd = c P3 (permutations, (u P)[j] = u[perm[j]]):
    z[j] = c * silu(a u[p1[q]]) * b u[p2[q]] with q = p3[j], elementwise."""
    rng = np.random.default_rng(4)
    d = 10
    u = rng.standard_normal((3, d))
    p1, p2, p3 = rng.permutation(d), rng.permutation(d), rng.permutation(d)

    def perm_matrix(p):
        m = np.zeros((d, d))
        m[p, np.arange(d)] = 1.0        # column j picks row p[j]
        return m

    a, b, c = 1.7, -0.6, 2.5
    z = sc.ffw(u, a * perm_matrix(p1), b * perm_matrix(p2), c * perm_matrix(p3))
    q = p3
    g = a * u[:, p1[q]]
    ref = c * g * expit(g) * (b * u[:, p2[q]])
    assert np.allclose(z, ref, rtol=1e-13, atol=1e-15)
    # the gate and the up projection are not interchangeable
    z_sw = sc.ffw(u, b * perm_matrix(p2), a * perm_matrix(p1), c * perm_matrix(p3))
    assert not np.allclose(z_sw, z, atol=1e-3)


def test_ffw_of_zero_is_zero_and_down_projection_scales():
    rng = np.random.default_rng(5)
    d, F = 8, 12
    wg, wu, wd = (rng.standard_normal(s) for s in ((d, F), (d, F), (F, d)))
    assert np.array_equal(sc.ffw(np.zeros((2, d)), wg, wu, wd), np.zeros((2, d)))
    u = rng.standard_normal((2, d))
    assert np.allclose(sc.ffw(u, wg, wu, 3 * wd), 3 * sc.ffw(u, wg, wu, wd), rtol=1e-13)


def test_signal_enters_at_the_token_embedding():
    """A signal E[y] - E[x] on canvas x gives the logits of canvas y with no signal, which
    holds only if z is added to the embedding ahead of every block."""
    rng = np.random.default_rng(6)
    w, W = _tiny_sc(rng)
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    x = rng.integers(0, w.vocab, w.canvas)
    y = rng.integers(0, w.vocab, w.canvas)
    E = W.embed()
    lx, _, _ = m.decoder_logits(x, E[y] - E[x])
    ly, _, _ = m.decoder_logits(y)
    assert np.allclose(lx, ly, rtol=0, atol=1e-12)
    l0, _, _ = m.decoder_logits(x, np.zeros((w.canvas, w.d_model)))
    ln, _, _ = m.decoder_logits(x)
    assert np.array_equal(l0, ln)
    assert np.abs(lx - ln).max() > 1e-3


def test_step_signal_is_ffw_of_the_tempered_posterior():
    rng = np.random.default_rng(7)
    w, W = _tiny_sc(rng)
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    canvas = rng.integers(0, w.vocab, w.canvas)
    mask = np.zeros(w.canvas, np.uint8)
    res = m.denoise_step(canvas, mask, 0, w.T, 3, keep_logits=True)
    p0 = sp_softmax(res.logits, axis=1)       # res.logits are already divided by tau
    assert np.allclose(res.sc.p0, p0, rtol=1e-12, atol=0)
    assert np.allclose(res.sc.u, p0 @ W.embed(), rtol=1e-12, atol=1e-14)
    ref = sc.ffw(p0 @ W.embed(), W.dense("sc_wg"), W.dense("sc_wu"), W.dense("sc_wd"))
    assert np.allclose(res.sc.z, ref, rtol=1e-12, atol=1e-14)
    # a one-hot tempered posterior gives FFW(E[v])
    zt = np.zeros((2, w.vocab))
    zt[0, 5] = zt[1, 60] = 1e4
    s1 = m.next_signal(zt)
    E = W.embed()
    assert np.array_equal(s1.u, E[[5, 60]])
    assert np.allclose(s1.z, sc.ffw(E[[5, 60]], W.dense("sc_wg"), W.dense("sc_wu"),
                                    W.dense("sc_wd")), rtol=1e-13, atol=0)


def test_block_chains_the_signal_and_starts_from_zero():
    rng = np.random.default_rng(8)
    w, W = _tiny_sc(rng)
    prompt = rng.integers(0, w.vocab, 10)
    m = om.OracleModel(w, W)
    m.prefill(prompt)
    seen = []
    m.generate_block(w.T, 11, commit=False, on_step=lambda s, c, k, r: seen.append((c, k, r)))
    assert [r.sc is not None for _, _, r in seen] == [True] * (w.T - 1) + [False]
    ref = om.OracleModel(w, W)
    ref.prefill(prompt)
    z = None
    for s, (c, k, r) in enumerate(seen):
        again = ref.denoise_step(c, k, s, w.T, 11, z_in=z, want_signal=s < w.T - 1)
        assert np.array_equal(again.canvas, r.canvas) and np.array_equal(again.mask, r.mask)
        z = r.sc.z if r.sc is not None else None
    # pass 0 of a self-conditioned block is the pass of the same model without the block
    plain = om.OracleModel(w.with_(self_cond=False), W)
    plain.prefill(prompt)
    c0, k0, r0 = seen[0]
    p0 = plain.denoise_step(c0, k0, 0, w.T, 11)
    assert np.array_equal(p0.canvas, r0.canvas) and p0.sc is None
    # a zero down projection makes every signal zero: the block is the plain block
    w2, W2 = _tiny_sc(np.random.default_rng(8), zero_down=True)
    a = om.OracleModel(w2, W2)
    a.prefill(prompt)
    b = om.OracleModel(w2.with_(self_cond=False), W2)
    b.prefill(prompt)
    assert np.array_equal(a.generate_block(w2.T, 11, commit=False),
                          b.generate_block(w2.T, 11, commit=False))


def test_signal_changes_later_passes():
    rng = np.random.default_rng(9)
    w, W = _tiny_sc(rng, sc_scale=1.0)
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    canvas = rng.integers(0, w.vocab, w.canvas)
    mask = np.zeros(w.canvas, np.uint8)
    r0 = m.denoise_step(canvas, mask, 0, w.T, 2, keep_logits=True)
    with_z = m.denoise_step(r0.canvas, r0.mask, 1, w.T, 2, keep_logits=True, z_in=r0.sc.z)
    without = m.denoise_step(r0.canvas, r0.mask, 1, w.T, 2, keep_logits=True)
    assert np.abs(with_z.logits - without.logits).max() > 1e-2


def test_bf16_plan_rounds_the_stored_operands():
    rng = np.random.default_rng(10)
    w, W = _tiny_sc(rng, act="bf16")
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    res = m.denoise_step(rng.integers(0, w.vocab, w.canvas), np.zeros(w.canvas, np.uint8), 0,
                         w.T, 1)
    assert np.array_equal(round_bf16(res.sc.p0), res.sc.p0)
    assert not np.array_equal(round_bf16(res.sc.z), res.sc.z)   # z stays in full precision


def test_fixture_weights_of_the_block():
    w = fx.TINY_FP32.with_(self_cond=True, sc_ff=128, sc_sigma=0.5)
    W = FixtureWeights(w)
    assert W.dense("sc_wg").shape == (256, 128) and W.dense("sc_wd").shape == (128, 256)
    assert abs(W.dense("sc_wu").std() - 0.5) < 0.01
    assert not np.array_equal(W.dense("sc_wg"), W.dense("sc_wu"))


def test_batch_takes_one_signal_per_canvas():
    rng = np.random.default_rng(11)
    w, W = _tiny_sc(rng)
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    cs = [rng.integers(0, w.vocab, w.canvas) for _ in range(2)]
    ks = [np.zeros(w.canvas, np.uint8)] * 2
    zs = [rng.standard_normal((w.canvas, w.d_model)) * 0.1 for _ in range(2)]
    batch = m.denoise_step_batch(cs, ks, 1, w.T, 5, z_ins=zs)
    for b in range(2):
        one = m.denoise_step(cs[b], ks[b], 1, w.T, 5, row0=b * w.canvas, z_in=zs[b])
        assert np.array_equal(one.canvas, batch[b].canvas)
        assert np.array_equal(one.sc.z, batch[b].sc.z)

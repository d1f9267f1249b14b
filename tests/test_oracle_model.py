"""Whole-model pins of the oracle: closed forms, causality, commit and schedule invariants."""
import numpy as np
import torch

import fixtures as fx
from oracle import model as om
from oracle.numerics import round_bf16
from oracle.weights import ArrayWeights, FixtureWeights


def _tiny(rng, L=2, d=32, hq=4, hkv=2, D=8, E=4, k=2, F=16, V=64, zero_updates=False,
          act="f32"):
    w = fx.Workload("tiny", n_layers=L, d_model=d, n_q_heads=hq, n_kv_heads=hkv, head_dim=D,
                    n_experts=E, top_k=k, d_ff=F, vocab=V, prompt_len=10, canvas=12, T=4,
                    act=act, experts=act)
    t = {"embed": rng.standard_normal((V, d)) * 0.5}
    for l in range(L):
        t[("wq", l)] = rng.standard_normal((d, hq * D)) * 0.3
        t[("wk", l)] = rng.standard_normal((d, hkv * D)) * 0.3
        t[("wv", l)] = rng.standard_normal((d, hkv * D)) * 0.3
        t[("wo", l)] = rng.standard_normal((hq * D, d)) * 0.3 * (not zero_updates)
        t[("wr", l)] = rng.standard_normal((d, E)) * 0.3
        t[("wg", l)] = rng.standard_normal((E, d, F)) * 0.3
        t[("wu", l)] = rng.standard_normal((E, d, F)) * 0.3
        t[("wd", l)] = rng.standard_normal((E, F, d)) * 0.3 * (not zero_updates)
    if act == "bf16":
        t = {key: round_bf16(v) for key, v in t.items()}
    return w, ArrayWeights(t)


def test_zero_updates_reduce_to_tied_head_closed_form():
    rng = np.random.default_rng(0)
    w, W = _tiny(rng, zero_updates=True)
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    canvas = rng.integers(0, w.vocab, w.canvas)
    logits, _, _ = m.decoder_logits(canvas)
    E = torch.tensor(W.embed())
    x = E[torch.tensor(canvas)]
    ref = torch.nn.functional.rms_norm(x, (w.d_model,), eps=w.rms_eps) @ E.T
    assert np.allclose(logits, ref.numpy(), atol=1e-12)


def test_prefill_is_causal():
    rng = np.random.default_rng(1)
    w, W = _tiny(rng)
    ids = rng.integers(0, w.vocab, 10)
    a = om.OracleModel(w, W)
    a.prefill(ids)
    b = om.OracleModel(w, W)
    b.prefill(ids[:6])
    for l in range(w.n_layers):
        assert np.allclose(a.K[l][:, :6], b.K[l], atol=1e-12)
        assert np.allclose(a.V[l][:, :6], b.V[l], atol=1e-12)


def test_commit_equals_prefill_of_the_concatenation():
    rng = np.random.default_rng(2)
    w, W = _tiny(rng)
    prompt = rng.integers(0, w.vocab, 10)
    canvas = rng.integers(0, w.vocab, w.canvas)
    a = om.OracleModel(w, W)
    a.prefill(prompt)
    a.commit(canvas)
    b = om.OracleModel(w, W)
    b.prefill(np.concatenate([prompt, canvas]))
    assert a.n_ctx == b.n_ctx == 10 + w.canvas and a.k_blk == 1
    for l in range(w.n_layers):
        assert np.allclose(a.K[l], b.K[l], atol=1e-12)
        assert np.allclose(a.V[l], b.V[l], atol=1e-12)


def test_decoder_is_bidirectional():
    rng = np.random.default_rng(3)
    w, W = _tiny(rng)
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    canvas = rng.integers(0, w.vocab, w.canvas)
    l1, _, _ = m.decoder_logits(canvas)
    canvas2 = canvas.copy()
    canvas2[-1] = (canvas2[-1] + 1) % w.vocab
    l2, _, _ = m.decoder_logits(canvas2)
    assert np.abs(l1[0] - l2[0]).max() > 1e-6      # position 0 sees the last position


def test_bf16_plan_stores_bf16_values():
    rng = np.random.default_rng(4)
    w, W = _tiny(rng, act="bf16")
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    for l in range(w.n_layers):
        assert np.array_equal(round_bf16(m.K[l]), m.K[l])
        assert np.array_equal(round_bf16(m.V[l]), m.V[l])


def test_block_schedule_invariants_tiny_fp32_workload():
    w = fx.TINY_FP32
    m = om.OracleModel(w, FixtureWeights(w))
    m.prefill(fx.prompt_ids(w))
    seen = []

    def cb(s, canvas, mask, res):
        locked = mask == 1
        assert np.array_equal(res.canvas[locked], canvas[locked])
        n_new = int(res.mask.sum() - mask.sum())
        assert n_new == om.lock_count(s, w.T, w.canvas, int((mask == 0).sum()))
        assert np.all((res.canvas >= 0) & (res.canvas < w.vocab))
        assert np.allclose(np.exp(res.stats.conf), np.exp(res.stats.m - res.stats.lse))
        seen.append(n_new)

    out = m.generate_block(w.T, w.seed, commit=True, on_step=cb)
    assert seen == [22] * 11 + [14]
    assert m.n_ctx == w.prompt_len + w.canvas and m.k_blk == 1
    # mean tokens fixed per pass 256/12 ~ 21.3, close to the reported ~20 per forward
    assert abs(np.mean(seen) - 256 / 12) < 1e-9
    assert out.shape == (w.canvas,)


def test_entropy_bounded_block_invariants_tiny_fp32_workload():
    from oracle import eb_sampler as eb
    from oracle.philox import renoise_tokens
    w = fx.TINY_FP32
    m = om.OracleModel(w, FixtureWeights(w))
    m.prefill(fx.prompt_ids(w))
    p = eb.EbParams(gamma=30.0, theta=0.0, max_steps=12)
    seen = []

    def cb(s, canvas, mask, res, er, H):
        locked = mask == 1
        assert np.array_equal(er.canvas[locked], canvas[locked])
        assert np.all((H >= 0) & (H <= np.log(w.vocab) + 1e-9))
        new = er.mask.astype(bool) & ~locked
        if not er.done:
            assert er.n_accept >= 1 and set(np.flatnonzero(new)) == set(er.accepted.tolist())
            assert np.array_equal(er.canvas[new], res.redraw[new])
            rest = ~er.mask.astype(bool)
            assert np.array_equal(er.canvas[rest], renoise_tokens(w.seed, 0, s, w.canvas,
                                                                  w.vocab)[rest])
            # the accepted set is a prefix of the entropy order whose bound stays below gamma
            assert eb.mi_bound(H[er.accepted]) < p.gamma
            if er.n_accept < er.order.size:
                assert eb.mi_bound(H[er.order[:er.n_accept + 1]]) >= p.gamma
        seen.append(int(new.sum()))

    out, n = m.generate_block_eb(p, w.seed, commit=False, on_step=cb)
    assert n == len(seen) <= p.max_steps and sum(seen) == w.canvas
    assert np.all((out >= 0) & (out < w.vocab))


def test_encoder_rows_give_the_prefill_cache_of_the_next_layer():
    """Layer 0 of the causal encoder evaluated at a few prompt rows only (against the full
    layer-0 cache) gives exactly the layer-1 cache rows a whole prefill writes there."""
    from oracle.numerics import rmsnorm
    rng = np.random.default_rng(7)
    w, W = _tiny(rng)
    ids = rng.integers(0, w.vocab, 10)
    full = om.OracleModel(w, W)
    full.prefill(ids)
    m = om.OracleModel(w, W)
    positions = np.arange(10)
    m.K[0], m.V[0] = m.kv_rows(0, m._act(rmsnorm(W.embed()[ids], w.rms_eps)), positions)
    assert np.allclose(m.K[0], full.K[0], atol=1e-12) and np.allclose(m.V[0], full.V[0], atol=1e-12)
    pos = np.array([0, 3, 9])
    h1, margin = m.encoder_layer_rows(0, W.embed()[ids[pos]], pos)
    k1, v1 = m.kv_rows(1, m._act(rmsnorm(h1, w.rms_eps)), pos)
    assert np.allclose(k1, full.K[1][:, pos], atol=1e-12)
    assert np.allclose(v1, full.V[1][:, pos], atol=1e-12)
    assert np.allclose(margin, full.enc_route_margin[0][pos], atol=1e-12)


def test_batched_canvases_are_independent_passes_on_long_canvas_streams():
    """A batch of canvases: a batch of one is the single pass; canvas b's pass equals a
    single pass whose Gumbel uniforms are drawn at rows b C + i; identical canvases in a
    batch get identical logits and statistics but independent redraws; the initial
    canvases are the first B C positions of one long canvas."""
    from oracle.philox import init_canvas, gumbel_uniforms
    rng = np.random.default_rng(11)
    w, W = _tiny(rng)
    m = om.OracleModel(w, W)
    m.prefill(rng.integers(0, w.vocab, 10))
    C, seed = w.canvas, 5
    inits = m.init_canvas_batch(seed, 3)
    assert np.array_equal(inits.ravel(), init_canvas(seed, 0, 3 * C, w.vocab))
    assert np.array_equal(inits[0], init_canvas(seed, 0, C, w.vocab))
    masks = np.zeros((3, C), np.uint8)
    canv = np.stack([inits[0], inits[1], inits[0]])
    out = m.denoise_step_batch(canv, masks, 0, w.T, seed)
    single = m.denoise_step(inits[0], masks[0], 0, w.T, seed)
    assert np.array_equal(out[0].canvas, single.canvas) and np.array_equal(out[0].mask, single.mask)
    # canvas 2 equals canvas 0 in everything but its redraw stream
    assert np.allclose(out[2].stats.conf, out[0].stats.conf, atol=0, rtol=0)
    assert np.array_equal(out[2].stats.argmax, out[0].stats.argmax)
    assert np.array_equal(out[2].mask, out[0].mask)          # the lock set follows conf
    unl = out[0].mask == 0
    assert not np.array_equal(out[2].redraw[unl], out[0].redraw[unl])
    # its redraws are the Gumbel-max draws at rows 2 C + i
    logits, _, _ = m.decoder_logits(inits[0])
    pos = np.flatnonzero(unl)[:5]
    u = gumbel_uniforms(seed, 0, 0, pos + 2 * C, w.vocab)
    draws, _ = om.gumbel_draw(logits[pos] / w.temperature, u)
    assert np.array_equal(out[2].redraw[pos], draws)

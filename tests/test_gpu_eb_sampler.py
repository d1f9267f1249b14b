"""GPU parity of the entropy-bounded sampler, through the C ABI.

dg_eb_sample (one sampler pass) against the oracle's eb_update on seeded
per-position statistics, bit for bit: ranking, acceptance and the stop test
are taken from the same float32 entropies, in float64 sums of the same order,
on both sides.  Cases: first pass, stop test held / broken by one changed
argmax / mean above theta, last pass, ragged C = 1000, C = 1, C = 1024 fully
locked, acceptance of exactly one and of all, a NaN entropy, max_steps = 1.

Whole passes (dg_denoise_step_eb) on the fp32 tiny model and the small bf16
model, teacher-forced on the oracle's canvas: tempered logits within the stated
logit tolerance, each entropy within 1e-4 nats of the entropy of the GPU's own
logits (the streaming fp32 arithmetic) and within the tolerance that the logit
tolerance implies of the oracle's (parity.entropy_tolerance, pinned on the CPU),
argmax and Gumbel draws gated by their margins, the accepted set equal to the
oracle's where its margins clear the entropy error (and a valid entropy-bounded
prefix of the pass's own entropies everywhere), renoised tokens bit-exact; a
pass repeated on the same canvas meets the stop test on both sides.  A
free-running block ends with every position locked."""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from oracle import eb_sampler as eb
from oracle.model import OracleModel
from oracle.philox import init_canvas, renoise_tokens
from oracle.weights import FixtureWeights
from parity import E2E_GATE, TOL, assert_close, entropy_tolerance, gated_mismatches, routing_sets
from gpu_util import i32_dev, log, logits_capture, need_gpu, routing_capture, stats_capture, u8_dev

pytestmark = pytest.mark.gpu

F32 = np.float32

# name, C, V, step, (gamma, theta, max_steps), fixture options
KERNEL_CASES = [
    ("first_pass", 256, 262144, 0, (0.75, 0.5, 48), {}),
    ("stop_test_holds", 256, 262144, 5, (0.75, 100.0, 48), {}),
    ("one_argmax_changed", 256, 262144, 5, (0.75, 100.0, 48), {"prev_diff": 1}),
    ("mean_above_theta", 256, 262144, 5, (0.75, 0.001, 48), {}),
    ("last_pass", 256, 1024, 47, (0.75, 0.0, 48), {}),
    ("ragged_1000", 1000, 50000, 3, (2.0, 0.0, 48), {"locked_frac": 0.5}),
    ("single_position", 1, 17, 2, (0.5, 0.0, 48), {"locked_frac": 0.0}),
    ("max_canvas_all_locked", 1024, 1024, 4, (0.5, 0.0, 48), {"locked_frac": 1.0}),
    ("accept_exactly_one", 256, 1024, 1, (-1.0, 0.0, 48), {}),
    ("accept_all", 256, 1024, 1, (1e30, 0.0, 48), {}),
    ("nan_entropy", 256, 1024, 2, (1.5, 0.0, 48), {"nan_at": 17}),
    ("single_pass_budget", 256, 1024, 0, (0.75, 0.0, 1), {}),
]


@pytest.fixture(scope="module")
def dg():
    return need_gpu()


def _oracle_params(gamma, theta, max_steps, tau_max=0.8, tau_min=0.4):
    # the C ABI takes float32 parameters: the oracle sees the same values
    return eb.EbParams(tau_max=float(F32(tau_max)), tau_min=float(F32(tau_min)),
                       gamma=float(F32(gamma)), theta=float(F32(theta)), max_steps=max_steps)


def _info_of(mask_in, er):
    locked_now = int(er.mask.sum()) - int(np.asarray(mask_in).sum())
    return [int(er.done), locked_now, int((er.mask == 0).sum()), int(er.stopped)]


@pytest.mark.parametrize("name,C,V,step,pp,kw", KERNEL_CASES, ids=[c[0] for c in KERNEL_CASES])
def test_eb_sample_matches_oracle_bit_exact(dg, name, C, V, step, pp, kw):
    seed, k_blk = 0x1234_5678_9ABC, 3
    gamma, theta, max_steps = pp
    x = fx.eb_sampler_inputs(seed, C, V, **kw)
    ref = eb.eb_update(x["canvas"], x["mask"], x["entropy"].astype(np.float64), x["argmax"],
                       x["draw"], x["prev"] if step > 0 else None, step,
                       _oracle_params(gamma, theta, max_steps), seed, k_blk, V)
    dev = {k: torch.from_numpy(v.copy()).cuda() for k, v in x.items()}
    info = torch.full((4,), -5, dtype=torch.int32, device="cuda")
    log(f"eb_sample case {name}: C={C} V={V} step={step}")
    dg.dg_eb_sample(dev["entropy"], dev["argmax"], dev["draw"], dev["prev"], dev["canvas"],
                    dev["mask"], info, C, V, step,
                    dg.eb_params(gamma=gamma, theta=theta, max_steps=max_steps), seed, k_blk)
    torch.cuda.synchronize()
    assert np.array_equal(dev["canvas"].cpu().numpy(), ref.canvas)
    assert np.array_equal(dev["mask"].cpu().numpy(), ref.mask)
    assert np.array_equal(dev["prev"].cpu().numpy(), x["argmax"])
    assert info.cpu().tolist() == _info_of(x["mask"], ref)
    log(f"  info {info.cpu().tolist()} (accepted {ref.n_accept}, stopped {ref.stopped})")


def test_eb_sample_chained_passes(dg):
    """Five passes on one canvas, each fed the oracle's previous outcome; the device keeps
    its own previous-argmax buffer across the calls."""
    C, V, seed, k_blk = 256, 4096, 77, 0
    p = (1.0, 0.0, 48)
    canvas = fx.eb_sampler_inputs(seed, C, V)["canvas"]
    mask = np.zeros(C, np.uint8)
    prev_dev = torch.zeros(C, dtype=torch.int32, device="cuda")
    prev = None
    for s in range(5):
        x = fx.eb_sampler_inputs(seed + s, C, V)
        ref = eb.eb_update(canvas, mask, x["entropy"].astype(np.float64), x["argmax"], x["draw"],
                           prev, s, _oracle_params(*p), seed, k_blk, V)
        cd, md = i32_dev(canvas), u8_dev(mask)
        info = torch.zeros(4, dtype=torch.int32, device="cuda")
        dg.dg_eb_sample(torch.from_numpy(x["entropy"]).cuda(), i32_dev(x["argmax"]),
                        i32_dev(x["draw"]), prev_dev, cd, md, info, C, V, s,
                        dg.eb_params(gamma=p[0], theta=p[1], max_steps=p[2]), seed, k_blk)
        torch.cuda.synchronize()
        assert np.array_equal(cd.cpu().numpy(), ref.canvas), f"pass {s}"
        assert np.array_equal(md.cpu().numpy(), ref.mask), f"pass {s}"
        assert info.cpu().tolist() == _info_of(mask, ref)
        canvas, mask, prev = ref.canvas, ref.mask, x["argmax"]
    log(f"5 chained passes: {int(mask.sum())} of {C} locked")


# --------------------------------------------------------------------------- whole passes
# Entropy of the GPU's own tempered logits against its streaming entropy: fp32 sums of
# e^(z - m) and e^(z - m)(z - m) over at most 1024 ids, merged per slice (~1e-6 nats).
H_SELF_TOL = 1e-4


def _model_env(dg, W):
    h = build_handle(dg, W, capture_mask=dg.DG_CAP_STATS | dg.DG_CAP_ROUTING | dg.DG_CAP_LOGITS)
    oracle = OracleModel(W, FixtureWeights(W))
    ids = fx.prompt_ids(W)
    oracle.prefill(ids)
    dg.dg_prefill_prompt_kv(h, i32_dev(ids), W.prompt_len)
    torch.cuda.synchronize()
    return h, oracle


def _check_pass(dg, h, W, s, res, er, H, canvas_in, mask_in, cd, md, info, p, seed, kind):
    """Compare one pass; returns True when the accepted set was compared exactly."""
    tag = f"{kind} pass {s}"
    C = W.canvas
    ok = np.ones(C, bool)          # rows whose routing matched in every layer
    for l in range(W.n_layers):
        gi, _ = routing_capture(dg, h, l, C, W.top_k)
        ok &= ~np.any(routing_sets(gi) != routing_sets(res.route_idx[l]), axis=1)
    Hd = torch.empty(C, dtype=torch.float32, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_ENTROPY, 0, Hd)
    st = stats_capture(dg, h, C)
    zg = logits_capture(dg, h, C, W.vocab).cpu().numpy().astype(np.float64)
    Hg = Hd.cpu().numpy().astype(np.float64)
    # the streaming entropy against the entropy of the same (GPU) logits, every row
    self_err = np.abs(Hg - eb.entropy(zg))
    assert self_err.max() <= H_SELF_TOL, f"{tag}: streaming entropy off by {self_err.max():.3g}"
    # logits L = tau z within the stated tolerance; it bounds the entropy's distance
    # from the oracle's through entropy_tolerance
    tau = eb.tau_at(s, p)
    atol, rtol = TOL[kind]
    zo = res.logits
    assert_close(f"{tag} logits", zg[ok] * tau, zo[ok] * tau, atol, rtol)
    h_tol = H_SELF_TOL + entropy_tolerance(zo[ok], atol / tau + rtol * np.abs(zo[ok]))
    err = np.abs(Hg - H)[ok]
    assert np.all(err <= h_tol), f"{tag}: entropy off by {np.max(err - h_tol):.3g} past its bound"
    tol = float(h_tol.max(initial=H_SELF_TOL))
    bad, n, _ = gated_mismatches(st["argmax"][ok], res.stats.argmax[ok], res.stats.top2_gap[ok],
                                 E2E_GATE[kind])
    assert bad == 0, f"{tag}: {bad}/{n} gated argmax differ"
    unl = (mask_in == 0) & ok
    bad, n, _ = gated_mismatches(st["redraw"][unl], res.redraw[unl], res.redraw_gap[unl], E2E_GATE[kind])
    assert bad == 0, f"{tag}: {bad}/{n} gated draws differ"

    cg, mg, ig = cd.cpu().numpy(), md.cpu().numpy().astype(bool), info.cpu().tolist()
    locked_in = mask_in.astype(bool)
    new, rest = mg & ~locked_in, ~mg
    assert np.array_equal(cg[locked_in], canvas_in[locked_in]), f"{tag}: a locked token changed"
    assert ig[1] == int(new.sum()) and ig[2] == int(rest.sum())
    assert ig[0] == int(bool(ig[3]) or not rest.any())
    assert bool(ig[3]) == er.stopped, f"{tag}: stop test differs"
    if ig[3]:
        assert mg.all() and np.array_equal(cg[new], st["argmax"][new])
        return False
    # a prefix of this pass's own entropy order whose bound stays below gamma; the rest renoised
    assert np.array_equal(cg[new], st["redraw"][new])
    assert np.array_equal(cg[rest], renoise_tokens(seed, 0, s, C, W.vocab)[rest])
    hs = np.sort(Hg[new])
    assert hs.size >= 1 and eb.mi_bound(hs) < p.gamma
    if rest.any():
        assert hs[-1] <= Hg[rest].min()
        assert eb.mi_bound(np.append(hs, Hg[rest].min())) >= p.gamma * (1 - 1e-12)
    # the oracle's accepted set, where its margins clear the entropy error
    n = er.n_accept
    h_ord = H[er.order]
    b = np.concatenate([[0.0], np.cumsum(h_ord)[:-1]])       # B(k) = sum of the first k - 1
    clear = bool(ok[er.order].all()) and (n == h_ord.size or h_ord[n] - h_ord[n - 1] > 2 * tol)
    clear = clear and abs(b[n - 1] - p.gamma) > n * tol
    if n < h_ord.size:
        clear = clear and abs(b[n] - p.gamma) > (n + 1) * tol
    if clear:
        assert set(np.flatnonzero(new)) == set(er.accepted.tolist()), f"{tag}: accepted set"
    return clear


def _teacher_forced(dg, W, kind, gamma, n_passes):
    h, oracle = _model_env(dg, W)
    try:
        seed = 21
        p_run = _oracle_params(gamma, 0.0, 48)
        p_stop = _oracle_params(gamma, 100.0, 48)
        canvas = init_canvas(seed, 0, W.canvas, W.vocab)
        mask = np.zeros(W.canvas, np.uint8)
        prev = None
        clear = 0
        for s in range(n_passes + 1):
            last = s == n_passes
            if last:                      # the previous pass's input again: the argmax repeats
                canvas, mask = c_prev, m_prev
            p = p_stop if last else p_run
            res, er, H = oracle.denoise_step_eb(canvas, mask, prev, s, p, seed, keep_logits=True)
            cd, md = i32_dev(canvas), u8_dev(mask)
            info = torch.zeros(4, dtype=torch.int32, device="cuda")
            log(f"{kind} entropy-bounded pass {s}{' (repeat)' if last else ''}")
            dg.dg_denoise_step_eb(h, cd, md, s, dg.eb_params(gamma=p.gamma, theta=p.theta,
                                                            max_steps=p.max_steps), seed, info)
            torch.cuda.synchronize()
            clear += _check_pass(dg, h, W, s, res, er, H, canvas, mask, cd, md, info, p, seed, kind)
            if last:
                assert er.stopped and info.cpu().tolist()[3] == 1
                assert md.cpu().numpy().all()
            c_prev, m_prev = canvas, mask
            canvas, mask, prev = er.canvas, er.mask, res.stats.argmax
        log(f"{kind}: {n_passes} passes + repeat, accepted set compared exactly on {clear}")
    finally:
        dg.dg_destroy(h)


def test_passes_teacher_forced_tiny_fp32(dg):
    _teacher_forced(dg, fx.TINY_FP32, "f32", gamma=30.0, n_passes=4)


def test_passes_teacher_forced_small_bf16(dg):
    _teacher_forced(dg, fx.SMALL_BF16, "bf16", gamma=30.0, n_passes=3)


def test_free_running_block_tiny_fp32(dg):
    W = fx.TINY_FP32
    h, _ = _model_env(dg, W)
    try:
        out = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
        p = dg.eb_params(gamma=30.0, theta=0.0, max_steps=12)
        n = dg.dg_generate_block_eb(h, out, p, 5, commit=True)
        o = out.cpu().numpy()
        assert 1 <= n <= 12 and o.min() >= 0 and o.max() < W.vocab
        n_ctx, k_blk = dg.dg_get_state(h)
        assert n_ctx == W.prompt_len + W.canvas and k_blk == 1
        log(f"free-running entropy-bounded block: {n} passes")
    finally:
        dg.dg_destroy(h)

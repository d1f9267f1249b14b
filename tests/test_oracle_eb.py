"""Pins of the entropy-bounded sampler's oracle (CPU only).

Entropy: closed forms (uniform, two-point, one-hot), scipy's entropy routine, and
the streaming (max, sum, weighted sum) form against the materialised one by
brute force over random slice splits.  The bound B(n) = sum - max: it dominates
the total correlation of any joint distribution with those marginals (brute
force over small alphabets) and equals it when every variable is a function of
the one with the largest entropy.  Acceptance, ranking, the stop test, the
temperature schedule and the renoise stream: hand-worked cases and invariants.
"""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import eb_sampler as eb
from oracle import philox as ph


# ----------------------------------------------------------------------------- entropy
@pytest.mark.parametrize("V", [1, 2, 7, 1024, 262144])
def test_entropy_uniform_is_log_v(V):
    z = np.full((1, V), 3.25)
    assert abs(eb.entropy(z)[0] - math.log(V)) < 1e-12 * max(1.0, math.log(V))


@pytest.mark.parametrize("a", [0.0, 0.3, -2.0, 7.5])
def test_entropy_two_point_binary_entropy(a):
    p = 1.0 / (1.0 + math.exp(-a))
    h = -(p * math.log(p) + (1 - p) * math.log(1 - p))
    assert abs(eb.entropy(np.array([[a, 0.0]]))[0] - h) < 1e-13


def test_entropy_one_hot_and_shift():
    z = np.zeros((2, 50))
    z[0, 7] = 1e4
    z[1] = np.linspace(-1, 1, 50)
    H = eb.entropy(z)
    assert H[0] == 0.0
    assert abs(eb.entropy(z + 123.0)[1] - H[1]) < 1e-12


def test_entropy_matches_scipy():
    rng = np.random.default_rng(0)
    z = rng.normal(0, 2.0, (16, 3000))
    p = np.exp(z - z.max(axis=1, keepdims=True))
    ref = stats.entropy(p, axis=1)             # normalises p itself
    assert np.allclose(eb.entropy(z), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_streaming_entropy_merge_matches_direct(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 5000))
    z = rng.normal(0, rng.uniform(0.1, 8.0), V)
    cuts = np.sort(rng.choice(np.arange(1, V), size=min(V - 1, int(rng.integers(1, 40))),
                              replace=False))
    parts = [eb.entropy_partial(c) for c in np.split(z, cuts)]
    while len(parts) > 1:                          # merge in a random tree
        i = int(rng.integers(0, len(parts) - 1))
        parts[i:i + 2] = [eb.entropy_merge(parts[i], parts[i + 1])]
    assert abs(eb.entropy_of_partial(parts[0]) - eb.entropy(z[None])[0]) < 1e-10


def test_entropy_partial_single_element():
    m, s, q = eb.entropy_partial(np.array([2.5]))
    assert (m, s, q) == (2.5, 1.0, 0.0)


# ----------------------------------------------------------------------------- the bound
def _h(p):
    p = np.asarray(p, np.float64).ravel()
    p = p[p > 0]
    return float(-(p * np.log(p)).sum())


@pytest.mark.parametrize("seed", range(20))
def test_bound_dominates_total_correlation(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 5))
    shape = tuple(int(x) for x in rng.integers(2, 5, n))
    joint = rng.dirichlet(np.full(int(np.prod(shape)), rng.uniform(0.05, 2.0))).reshape(shape)
    marg = [_h(joint.sum(axis=tuple(j for j in range(n) if j != i))) for i in range(n)]
    tc = sum(marg) - _h(joint)
    assert tc <= eb.mi_bound(marg) + 1e-12


def test_bound_equality_for_functions_of_one_variable():
    # X1 uniform over 6 values; X2 = X1 mod 3, X3 = X1 mod 2: the joint entropy is H(X1).
    joint = np.zeros((6, 3, 2))
    for x in range(6):
        joint[x, x % 3, x % 2] = 1 / 6
    marg = [_h(joint.sum(axis=(1, 2))), _h(joint.sum(axis=(0, 2))), _h(joint.sum(axis=(0, 1)))]
    tc = sum(marg) - _h(joint)
    assert abs(tc - (math.log(3) + math.log(2))) < 1e-12
    assert abs(eb.mi_bound(marg) - tc) < 1e-12
    assert abs(eb.mi_bound([0.2]) - 0.0) == 0.0


@pytest.mark.parametrize("gamma,n", [(0.1, 4), (0.079, 3), (0.081, 4), (0.0, 1), (-1.0, 1), (0.0300001, 3),
                                     (0.029, 2), (1e9, 5)])
def test_accept_count_hand_cases(gamma, n):
    h = [0.01, 0.02, 0.05, 0.5, 1.0]
    # B(1..5) = 0, 0.01, 0.03, 0.08, 0.58
    assert eb.accept_count(h, gamma) == n


def test_accept_count_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(200):
        h = np.sort(rng.exponential(rng.uniform(0.01, 2.0), int(rng.integers(1, 40))))
        gamma = float(rng.uniform(0, 5))
        ok = [k for k in range(1, h.size + 1) if eb.mi_bound(h[:k]) < gamma - 1e-9]
        near = [k for k in range(1, h.size + 1) if abs(eb.mi_bound(h[:k]) - gamma) <= 1e-9]
        if near:
            continue
        assert eb.accept_count(h, gamma) == max(ok + [1])
    assert eb.accept_count([], 1.0) == 0


def test_rank_order_ties_to_lower_position():
    H = np.array([0.5, 0.1, 0.1, 0.3, 0.0])
    mask = np.array([0, 0, 0, 1, 0], np.uint8)
    assert eb.rank_order(H, mask).tolist() == [4, 1, 2, 0]


# ----------------------------------------------------------------------------- schedule
def test_tau_schedule():
    p = eb.EbParams()
    assert eb.tau_at(0, p) == pytest.approx(0.8, abs=1e-15)
    assert eb.tau_at(47, p) == pytest.approx(0.4, abs=1e-15)
    taus = [eb.tau_at(s, p) for s in range(48)]
    assert np.allclose(np.diff(taus), -0.4 / 47, atol=1e-15)
    assert eb.tau_at(24, eb.EbParams(max_steps=49)) == pytest.approx(0.6, abs=1e-15)
    assert eb.tau_at(0, eb.EbParams(max_steps=1)) == 0.4


def test_mean_entropy_in_order():
    H = np.array([1e16, 1.0, -1e16, 1.0])
    # index order: (1e16 + 1) rounds to 1e16, then 0, then 1: the mean is 1/4
    assert eb.mean_entropy(H) == 0.25


# ----------------------------------------------------------------------------- renoise stream
def test_renoise_uniform_and_distinct_streams():
    V = 97
    t = ph.renoise_tokens(5, 1, 3, 100000, V)
    assert t.min() >= 0 and t.max() < V
    counts = np.bincount(t, minlength=V)
    assert stats.chisquare(counts).pvalue > 1e-4
    assert not np.array_equal(t[:1000], ph.renoise_tokens(5, 1, 4, 1000, V))
    assert not np.array_equal(t[:1000], ph.init_canvas(5, 1, 1000, V))
    # position i uses output word i & 3 of counter i >> 2 (same layout as the initial canvas)
    w = ph.philox4x32_10(np.array([2], np.uint32), 1, 3, ph.RENOISE_TAG, 5, 0)
    assert t[9] == (int(w[1][0]) * V) >> 32


# ----------------------------------------------------------------------------- one update
def _case(C=8, V=50):
    H = np.array([0.30, 0.01, 0.02, 2.0, 0.05, 0.01, 1.0, 0.4])[:C]
    argmax = np.arange(C, dtype=np.int32) + 10
    draw = np.arange(C, dtype=np.int32) + 20
    canvas = np.arange(C, dtype=np.int32) + 30
    mask = np.array([0, 0, 1, 0, 0, 0, 0, 0], np.uint8)[:C]
    return H, argmax, draw, canvas, mask


def test_update_accepts_lowest_entropy_prefix():
    H, am, dr, cv, mk = _case()
    p = eb.EbParams(gamma=0.1, theta=0.0, max_steps=10)
    r = eb.eb_update(cv, mk, H, am, dr, None, 2, p, seed=9, k_blk=0, V=50)
    # candidates (unlocked) by entropy: 1 (0.01), 5 (0.01), 4 (0.05), 0 (0.30), 7, 6, 3
    # B: 0, 0.01, 0.02, 0.07, 0.37 -> four accepted
    assert r.order.tolist() == [1, 5, 4, 0, 7, 6, 3]
    assert r.n_accept == 4 and r.accepted.tolist() == [1, 5, 4, 0]
    assert not r.done and not r.stopped
    noise = ph.renoise_tokens(9, 0, 2, 8, 50)
    exp = cv.copy()
    exp[[1, 5, 4, 0]] = dr[[1, 5, 4, 0]]
    exp[[7, 6, 3]] = noise[[7, 6, 3]]
    assert r.canvas.tolist() == exp.tolist()
    assert r.mask.tolist() == [1, 1, 1, 0, 1, 1, 0, 0]
    assert r.canvas[2] == cv[2]                    # locked: untouched


def test_update_stop_rule():
    H, am, dr, cv, mk = _case()
    mh = float(np.mean(H))
    p = eb.EbParams(gamma=0.1, theta=mh + 1e-6, max_steps=10)
    r = eb.eb_update(cv, mk, H, am, dr, am.copy(), 3, p, 1, 0, 50)
    assert r.stopped and r.done
    assert r.canvas.tolist() == [10, 11, 32, 13, 14, 15, 16, 17]   # unlocked take argmax
    assert r.mask.all()
    prev = am.copy()
    prev[2] += 1                                   # one differing prediction (a locked position)
    assert not eb.eb_update(cv, mk, H, am, dr, prev, 3, p, 1, 0, 50).stopped
    assert not eb.eb_update(cv, mk, H, am, dr, am.copy(), 0, p, 1, 0, 50).stopped   # no previous pass
    p2 = eb.EbParams(gamma=0.1, theta=mh - 1e-6, max_steps=10)
    assert not eb.eb_update(cv, mk, H, am, dr, am.copy(), 3, p2, 1, 0, 50).stopped  # mean too high


def test_update_last_pass_and_all_accepted():
    H, am, dr, cv, mk = _case()
    p = eb.EbParams(gamma=0.1, theta=0.0, max_steps=4)
    r = eb.eb_update(cv, mk, H, am, dr, None, 3, p, 1, 0, 50)
    assert r.done and not r.stopped and r.mask.all()
    assert r.canvas.tolist() == [10, 11, 32, 13, 14, 15, 16, 17]
    r = eb.eb_update(cv, mk, H, am, dr, None, 1, eb.EbParams(gamma=100.0, theta=0.0), 1, 0, 50)
    assert r.done and r.n_accept == 7 and r.mask.all()
    assert r.canvas.tolist() == [20, 21, 32, 23, 24, 25, 26, 27]   # all take their draws

"""Pins of the oracle's random streams and element-wise numerics (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch
from scipy import stats

import fixtures as fx
from oracle import numerics as nu
from oracle import philox as ph

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    for line in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        vals = [int(t, 16) for t in line.split()]
        rows.append((vals[:4], vals[4:6], vals[6:]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_philox_known_answers(ctr, key, expect):
    out = ph.philox4x32_10(*[np.array([c], np.uint32) for c in ctr], key[0], key[1])
    assert [int(o[0]) for o in out] == expect


def test_philox_counter_sensitivity():
    # Distinct counters give distinct, roughly uniform words (avalanche sanity).
    c = np.arange(1 << 16, dtype=np.uint32)
    w = ph.philox4x32_10(c, 0, 0, 0, 1, 2)[0]
    assert len(np.unique(w)) > (1 << 16) - 5
    bits = np.unpackbits(w.view(np.uint8))
    assert abs(bits.mean() - 0.5) < 0.01


def test_init_canvas_uniform_chi2():
    V = 64
    x = ph.init_canvas(seed=7, k_blk=0, C=1 << 16, V=V)
    assert x.min() >= 0 and x.max() < V
    cnt = np.bincount(x, minlength=V)
    p = stats.chisquare(cnt).pvalue
    assert p > 1e-4
    # forward process at kappa = 0: P(token unchanged) = 1/V for any clean token
    assert abs(np.mean(x == 5) - 1.0 / V) < 4 * math.sqrt((1 / V) * (1 - 1 / V) / x.size)


def test_init_canvas_depends_on_block_and_seed():
    a = ph.init_canvas(0, 0, 256, 1024)
    b = ph.init_canvas(0, 1, 256, 1024)
    c = ph.init_canvas(1, 0, 256, 1024)
    assert (a != b).mean() > 0.9 and (a != c).mean() > 0.9


def test_gumbel_uniforms_open_interval_and_exact_f32():
    u = ph.gumbel_uniforms(3, 0, 5, np.arange(8), 4096)
    assert u.min() > 0 and u.max() < 1
    assert np.all(u.astype(np.float32).astype(np.float64) == u)
    assert abs(u.mean() - 0.5) < 0.01


# ------------------------------------------------------------------ bf16 / e4m3
def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # add exact ties: bf16 value + half an ulp
    base = torch.tensor(x).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    for v in (x, ties, np.array([0.0, -0.0, 1e-40, -3e-39, 3.0e38], np.float32)):
        ref = torch.tensor(v).to(torch.bfloat16).double().numpy()
        got = nu.round_bf16(v.astype(np.float64))
        assert np.array_equal(ref, got)


def test_round_bf16_matches_fixture_encoder():
    rng = np.random.default_rng(1)
    for x in rng.standard_normal(2000).astype(np.float32):
        bits = fx.bf16_encode_scalar(float(x))
        assert fx.bf16_bits_to_f32(np.array([bits], np.uint16))[0] == nu.round_bf16(float(x))


def test_e4m3_exhaustive_codes_roundtrip():
    codes = np.arange(256)
    vals = nu.e4m3_value_of_code(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    assert np.nanmax(vals) == 448.0 and np.nanmin(vals) == -448.0
    assert np.array_equal(nu.e4m3_round(vals[finite]), vals[finite])


def test_e4m3_ties_to_even_and_saturation():
    vals = np.unique(nu.e4m3_value_of_code(np.arange(0, 127)))
    vals = vals[~np.isnan(vals)]
    mids = (vals[:-1] + vals[1:]) / 2
    got = nu.e4m3_round(mids)
    # the even code (mantissa LSB 0) wins each tie
    codes = {v: c for c, v in enumerate(nu.e4m3_value_of_code(np.arange(127)))}
    for m, g in zip(mids, got):
        assert g in codes and codes[g] % 2 == 0, (m, g)
    assert nu.e4m3_round(np.array([449.0, 1e6, -500.0])).tolist() == [448.0, 448.0, -448.0]


def test_e4m3_matches_torch_and_fixture_encoder():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(20000) * 40).astype(np.float32)
    x = x[np.abs(x) < 440]
    ref = torch.tensor(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(nu.e4m3_round(x.astype(np.float64)), ref)
    table = nu.e4m3_value_of_code(np.arange(256))
    for v in x[:2000]:
        assert table[fx.e4m3_encode_scalar(float(v))] == nu.e4m3_round(float(v))


# ------------------------------------------------------------------ norms / rope / silu
def test_rmsnorm_invariants():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)) * 7
    y = nu.rmsnorm(x, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-13)
    assert np.allclose(nu.rmsnorm(3.5 * x, 0.0), y, atol=1e-13)
    # eps keeps a zero row finite
    assert np.all(nu.rmsnorm(np.zeros((1, 8)), 1e-6) == 0)


def test_rope_invariants_and_complex_form():
    rng = np.random.default_rng(4)
    D = 64
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    # position 0 is the identity; norms preserved
    assert np.allclose(nu.rope(q, [0])[0, 0], q[0, 0])
    assert np.isclose(np.linalg.norm(nu.rope(q, [1234])), np.linalg.norm(q))
    # the score depends only on the position difference
    s1 = np.dot(nu.rope(q, [100])[0, 0], nu.rope(k, [40])[0, 0])
    s2 = np.dot(nu.rope(q, [1060])[0, 0], nu.rope(k, [1000])[0, 0])
    assert np.isclose(s1, s2, rtol=1e-10)
    # rotate-half pairs (j, j + D/2) as complex numbers times e^{i pos theta_j}
    pos = 77
    z = q[0, 0, :D // 2] + 1j * q[0, 0, D // 2:]
    th = 10000.0 ** (-np.arange(D // 2) * 2.0 / D)
    zr = z * np.exp(1j * pos * th)
    assert np.allclose(nu.rope(q, [pos])[0, 0], np.concatenate([zr.real, zr.imag]), atol=1e-12)


def test_silu_and_softmax_closed_forms():
    x = np.linspace(-6, 6, 101)
    s = nu.silu(x)
    assert np.allclose(s - nu.silu(-x), x)
    assert nu.silu(np.array([0.0]))[0] == 0.0
    p = nu.softmax(np.random.default_rng(5).standard_normal((4, 33)) * 10)
    assert np.allclose(p.sum(-1), 1.0)
    assert np.allclose(nu.softmax(np.zeros(8)), 1 / 8)

"""Pins of the MX FP4 expert storage (OCP Microscaling formats: E2M1 elements, one E8M0 scale per
32 elements along the contraction dimension): the oracle's decode against the format's value
table, the scale's power of two, and the seeded generator's quantizer against the block rule
recomputed by brute force (scale exponent floor(log2 amax) - 2, nearest E2M1 value with ties to
the even mantissa, saturation at 6), its nibble order, exact round trips of representable values
and the rounding error bound."""
import numpy as np
import pytest

import fixtures as fx
from oracle.numerics import e2m1_value_of_code, mxfp4_dequant
from oracle.weights import FixtureWeights

# the 8 non-negative E2M1 values by code (sign in bit 3)
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_table():
    got = e2m1_value_of_code(np.arange(16))
    assert np.array_equal(got[:8], E2M1)
    assert np.array_equal(got[8:], [-v for v in E2M1])
    assert np.signbit(got[8])                      # code 8 is -0


def test_scale_is_a_power_of_two():
    codes = np.full((32, 1), 0x22, np.uint8)      # 1.0 in both nibbles
    for s, f in ((127, 1.0), (128, 2.0), (120, 2.0 ** -7), (0, 2.0 ** -127), (254, 2.0 ** 127)):
        v = mxfp4_dequant(codes, np.array([[s, s]], np.uint8))
        assert np.all(v == f)


def _nearest_e2m1(x):
    """Brute force: the E2M1 magnitude nearest |x|, ties to the even code, saturating."""
    a = min(abs(x), 6.0)
    best = min(range(8), key=lambda c: (abs(a - E2M1[c]), c & 1))
    return np.copysign(E2M1[best], x)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantizer_follows_the_block_rule(seed):
    rng = np.random.default_rng(seed)
    K, N = 96, 10
    w = (rng.standard_normal((K, N)) * rng.choice([0.02, 1.0, 300.0], (K, N))).astype(np.float32)
    w[:32, 3] = 0.0                                # an all-zero block
    codes, scales = fx.quant_mxfp4(w)
    deq = mxfp4_dequant(codes, scales)
    for b in range(K // 32):
        for c in range(N):
            blk = w[32 * b:32 * b + 32, c].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                assert scales[b, c] == 0 and np.all(deq[32 * b:32 * b + 32, c] == 0)
                continue
            e = int(np.floor(np.log2(amax))) - 2
            assert scales[b, c] == e + 127
            X = 2.0 ** e
            ref = np.array([_nearest_e2m1(v / X) * X for v in blk])
            assert np.array_equal(deq[32 * b:32 * b + 32, c], ref), (b, c)


def test_ties_saturation_and_nibble_order():
    X = 2.0 ** -5
    col0 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0] * 4) * X   # amax 5: e = floor(log2 5X) - 2
    col1 = -np.array([6.0, 7.9, 3.0, 0.5, 0.0, 1.0, 2.0, 4.0] * 4) * X
    w = np.stack([col0, col1], axis=1).astype(np.float32)
    codes, scales = fx.quant_mxfp4(w)
    # both blocks: floor(log2 amax) - 2 = -5 (amax 5X and 7.9X are below 8X), scale X
    assert scales[0, 0] == -5 + 127 and scales[0, 1] == -5 + 127
    lo, hi = codes[:, 0] & 0xF, codes[:, 0] >> 4
    # ties to the even mantissa: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
    # 5 -> 4
    assert list(e2m1_value_of_code(lo[:8])) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 4.0]
    # the odd column in the high nibble; 7.9 saturates at 6
    assert list(e2m1_value_of_code(hi[:8])) == [-6.0, -6.0, -3.0, -0.5, -0.0, -1.0, -2.0, -4.0]


def test_representable_values_round_trip_and_error_bound():
    rng = np.random.default_rng(7)
    K, N = 64, 8
    X = 2.0 ** rng.integers(-10, 3, (K // 32, N))
    vals = rng.choice([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], (K, N))
    vals[0] = 6.0                                   # every block holds its maximum 6 X
    vals[32] = -6.0
    w = (vals * np.repeat(X, 32, axis=0)).astype(np.float32)
    codes, scales = fx.quant_mxfp4(w)
    assert np.array_equal(mxfp4_dequant(codes, scales), w.astype(np.float64))
    # error bound: half the E2M1 step at the element's magnitude, in units of its block scale
    w2 = rng.standard_normal((K, N)).astype(np.float32)
    codes, scales = fx.quant_mxfp4(w2)
    deq = mxfp4_dequant(codes, scales)
    Xb = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=0)
    r = np.abs(w2) / Xb                             # in [0, 8) by the scale rule
    half_step = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, 1.0))
    bound = np.where(r > 6, r - 6, half_step) * Xb
    assert np.all(np.abs(deq - w2) <= bound + 1e-12)


def test_fixture_weights_of_mxfp4_experts():
    w = fx.SMALL_BF16.with_(experts="mxfp4")
    W = FixtureWeights(w)
    wg = W.expert("wg", 0, 3)
    assert wg.shape == (w.d_model, w.d_ff)
    raw = fx.normal(w.seed, fx.layer_tid("wg", 0), (w.d_model, w.d_ff), w.sigma, "f32",
                    start=3 * w.d_model * w.d_ff)
    assert np.abs(wg - raw).max() <= 0.25 * np.abs(raw).max()      # within the coarse step
    assert np.abs(wg - raw).mean() < 0.1 * np.abs(raw).mean() + 1e-3

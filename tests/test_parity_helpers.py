"""CPU checks of the parity helpers' own arithmetic (test infrastructure).

entropy_tolerance turns the logit tolerance into a tolerance on per-position
entropies (the entropy-bounded sampler ranks positions by them).  It is checked
here against the entropy evaluated at perturbed logits, by brute force: the
first-order worst case (every logit moved by its full tolerance against or along
the gradient), random corners of the tolerance box and random points inside it,
on flat, unit-scale, wide and peaked rows and on tolerances from 1e-4 to 0.3.
The bound must hold everywhere and be nearly attained for small tolerances."""
import numpy as np

from oracle.eb_sampler import entropy
from parity import entropy_tolerance


def _rows(rng, V=257):
    peaked = rng.normal(0.0, 1.0, V)
    peaked[3] += 9.0
    two = np.full(V, -40.0)
    two[[5, 11]] = [0.0, -0.7]
    return {
        "flat": rng.normal(0.0, 0.05, V),
        "unit": rng.normal(0.0, 1.0, V),
        "wide": rng.normal(0.0, 5.0, V),
        "peaked": peaked,
        "two_point": two,
    }


def _tolerances(z, rng):
    tau = 0.8
    return {
        "bf16_logit_bound": 2e-2 / tau + 1e-2 * np.abs(z),
        "fp32_logit_bound": 1e-4 / tau + 1e-4 * np.abs(z),
        "tiny_const": np.full_like(z, 1e-4),
        "ragged": rng.uniform(0.0, 5e-2, z.shape),
        "large_const": np.full_like(z, 0.3),
    }


def test_entropy_tolerance_bounds_every_perturbation():
    rng = np.random.default_rng(7)
    for rname, z in _rows(rng).items():
        H0 = entropy(z[None])[0]
        e = np.exp(z - z.max())
        p = e / e.sum()
        grad = -p * (z - np.sum(p * z))
        for tname, tol in _tolerances(z, rng).items():
            bound = entropy_tolerance(z, tol)
            dirs = [np.sign(grad) * tol, -np.sign(grad) * tol]
            dirs += [rng.choice([-1.0, 1.0], z.shape) * tol for _ in range(64)]
            dirs += [rng.uniform(-1.0, 1.0, z.shape) * tol for _ in range(64)]
            worst = max(abs(entropy((z + d)[None])[0] - H0) for d in dirs)
            assert worst <= bound * (1 + 1e-9) + 1e-12, (rname, tname, worst, bound)


def test_entropy_tolerance_is_nearly_attained_for_small_tolerances():
    rng = np.random.default_rng(8)
    for rname, z in _rows(rng).items():
        tol = np.full_like(z, 1e-5)
        e = np.exp(z - z.max())
        p = e / e.sum()
        grad = -p * (z - np.sum(p * z))
        d = np.sign(grad) * tol                  # first-order worst case
        dh = abs(entropy((z + d)[None])[0] - entropy(z[None])[0])
        bound = entropy_tolerance(z, tol)
        assert dh <= bound and dh >= 0.99 * bound, (rname, dh, bound)


def test_entropy_tolerance_special_cases():
    z = np.random.default_rng(9).normal(size=(3, 64))
    assert np.all(entropy_tolerance(z, 0.0) == 0.0)
    # a constant row: every softmax weight equal, the centred logits zero -> first order 0
    flat = np.zeros(64)
    assert entropy_tolerance(flat, 1e-3) <= 8e-6
    # rows are independent: the batched call equals row-by-row calls
    tol = 1e-2 * np.abs(z) + 1e-3
    one = np.array([entropy_tolerance(z[i], tol[i]) for i in range(3)])
    assert np.allclose(entropy_tolerance(z, tol), one, rtol=1e-14, atol=0)

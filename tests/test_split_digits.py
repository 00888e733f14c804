"""CPU checks of the split-integer distance specification (tests/_digits.py)
that the library's distance kernels implement: digits reconstruct the
integers exactly and stay in int8, the int32 pair sums stay far below 2^31,
the error bound eps holds on exact rationals, and the result equals the
oracle's once-rounded distance (at every feature dimension of the
workloads, on random rows and on rows built to stress cancellation and
dynamic range)."""
from fractions import Fraction

import numpy as np
import pytest

import _digits as G
from sdtw_inputs import pair_batch


def test_digits_reconstruct_integers():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((50, 37)) * np.exp(rng.uniform(-20, 20, (50, 1)))).astype(np.float32)
    v[3] = 0.0
    v[4, :] = 0.0
    v[4, 5] = -1.5
    e = G.row_exponent(v)
    Z = G.integers(v, e)
    g = G.digits(Z)
    assert g.min() >= -128 and g.max() <= 127
    assert (np.abs(g[..., 0]) <= 64).all()        # |Z| < 2^46: the top digit is small
    back = sum(g[..., k] * (256 ** (5 - k)) for k in range(6))
    np.testing.assert_array_equal(back, Z)
    # Z is the correctly rounded v 2^(48-e)
    for r in range(0, 50, 7):
        for d in range(0, 37, 5):
            q = Fraction(float(v[r, d])) * Fraction(2) ** int(48 - e[r])
            assert abs(q - int(Z[r, d])) <= Fraction(1, 2)


def _exact_sq(a, b):
    return sum((Fraction(float(p)) - Fraction(float(q))) ** 2 for p, q in zip(a, b))


@pytest.mark.parametrize("D", [1, 2, 3, 4, 7, 16, 33, 64, 65, 128, 200, 256])
def test_bound_and_rounding_random_rows(O, D):
    x, y = pair_batch(1, 120, 130, D, seed=D)
    d, P = G.sqdist(x[0].numpy(), y[0].numpy(), return_parts=True)
    ref = O.sqeuclid(x.numpy(), y.numpy(), round_f32=True)[0]
    assert P["cmax"] < 2 ** 28
    assert (d.astype(np.float64) == ref).mean() > 1 - 1e-4
    rng = np.random.default_rng(D)
    for _ in range(25):
        i, j = int(rng.integers(120)), int(rng.integers(130))
        exact = _exact_sq(x[0, i].numpy(), y[0, j].numpy())
        assert abs(Fraction(float(P["v"][i, j])) - exact) <= Fraction(float(P["eps"][i, j]))


def test_cancellation_and_dynamic_range(O):
    """y rows close to x rows (tiny distances against large norms), rows
    with one large entry among tiny ones, zero rows and powers of two: the
    result is the oracle's once-rounded value everywhere."""
    rng = np.random.default_rng(3)
    D = 64
    x = rng.standard_normal((40, D)).astype(np.float32)
    y = np.concatenate([
        x + (rng.standard_normal((40, D)) * 1e-5).astype(np.float32),
        x[:, ::-1].copy(),
        np.zeros((5, D), np.float32),
    ]).astype(np.float32)
    x[7] = 0.0
    x[8] *= 1e-30
    x[9, :] = 1e-6
    x[9, 3] = 1e4
    x[10] = np.ldexp(1.0, rng.integers(-10, 10, D)).astype(np.float32)
    d, P = G.sqdist(x, y, return_parts=True)
    ref = O.sqeuclid(x[None], y[None], round_f32=True)[0]
    np.testing.assert_array_equal(d.astype(np.float64), ref)
    assert P["ambiguous"].any()          # the direct fallback is exercised

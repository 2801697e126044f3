"""The FP8 h quantisation of the GEMM epilogue forms each code from h / scale rounded to fp32
(the same correctly rounded fp32 quotient as the activation quantiser and the oracle) as the
fp32 rounding of the fp64 product h * RN64(1 / scale): the product is within 2^-52 (relative)
of the quotient, and a quotient of two fp32 numbers never lies closer than about 2^-49 to an fp32
rounding midpoint, so both round alike.  This checks that identity on the CPU, in numpy's IEEE
arithmetic, on random pairs and on pairs built to put the quotient next to a midpoint."""
import numpy as np


def _crq(v, s):
    # correctly rounded fp32 quotient: fp64 division then fp32 rounding (53 >= 2 * 24 + 2)
    return (v.astype(np.float64) / s.astype(np.float64)).astype(np.float32)


def _via_reciprocal(v, s):
    return (v.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)


def test_random_pairs():
    rng = np.random.default_rng(7)
    n = 2_000_000
    s = (np.abs(rng.standard_normal(n)) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1.0))
    v = (rng.standard_normal(n) * s * 448 / 4).astype(np.float32)
    assert np.array_equal(_crq(v, s).view(np.uint32), _via_reciprocal(v, s).view(np.uint32))


def test_quotients_next_to_rounding_midpoints():
    rng = np.random.default_rng(8)
    n = 2_000_000
    s = (1.0 + rng.random(n)).astype(np.float32) * np.float32(2.0) ** rng.integers(-10, 10, n)
    s = s.astype(np.float32)
    # a midpoint between two fp32 neighbours of magnitude up to 448, and v = RN32(mid * s), so
    # v / s sits within a few fp32 ulps of that midpoint
    q = (rng.random(n) * 448).astype(np.float32)
    mid = q.astype(np.float64) + np.spacing(q).astype(np.float64) / 2
    for k in (-2, -1, 0, 1, 2):
        v = (mid * s.astype(np.float64)).astype(np.float32)
        v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(-np.inf)) if k else v
        if abs(k) == 2:
            v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(-np.inf))
        a, b = _crq(v, s), _via_reciprocal(v, s)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), k
    # negative values and zeros keep their sign
    v = np.array([-0.0, 0.0, -3.5, 3.5], np.float32)
    s = np.array([0.25, 0.25, 0.3, 0.3], np.float32)
    assert np.array_equal(_crq(v, s).view(np.uint32), _via_reciprocal(v, s).view(np.uint32))

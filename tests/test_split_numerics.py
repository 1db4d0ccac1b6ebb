"""The two-term FP8 (E4M3) activation split, emulated on the CPU from its
definition: a 32-value block v becomes q1*2^e1 + q2*2^e2, where the shared
exponent puts the block maximum in [128, 256), q1 rounds v/2^e1 to E4M3
(nearest, ties to even) and q2 rounds the exact residual the same way with
the residual block's own exponent.  Pins the exactness bound the kernels'
comments state: every bf16 element of at least 2^-12 of the block maximum is
reproduced exactly; a smaller one is off by at most 2^-21 of the block
maximum; and a concrete element below the bound that is not exact.
"""
import numpy as np


def e4m3_rne(x):
    """Nearest E4M3 value of x (ties to even; subnormal step 2^-9; saturating at 448), fp64."""
    a = np.abs(x)
    e = np.clip(np.floor(np.log2(np.maximum(a, 1e-300))), -6, 8)
    step = 2.0 ** (e - 3)
    return np.sign(x) * np.minimum(np.round(a / step) * step, 448.0)


def split_exponent(amax):
    if amax <= 0:
        return 0
    return int(np.clip(np.frexp(amax)[1] - 8, -127, 127))  # amax / 2^e in [128, 256)


def split(v):
    e1 = split_exponent(np.abs(v).max())
    q1 = e4m3_rne(v / 2.0 ** e1) * 2.0 ** e1
    r = v - q1
    e2 = split_exponent(np.abs(r).max())
    return q1 + e4m3_rne(r / 2.0 ** e2) * 2.0 ** e2


def bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_e4m3_rounding_reference():
    # E4M3: 3 mantissa bits; 1.0625 is halfway between 1 and 1.125 and goes to the even 1.0
    assert e4m3_rne(np.array([1.0625, 1.1875, 448.0, 500.0, 2.0 ** -9, 3 * 2.0 ** -10])).tolist() == \
        [1.0, 1.25, 448.0, 448.0, 2.0 ** -9, 2.0 ** -8]


def test_split_exactness_bound():
    rng = np.random.default_rng(7)
    n_small = 0
    for _ in range(4000):
        v = bf16(rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20))
        # a few elements far below the block maximum
        v[:3] = bf16(v[:3] * 2.0 ** -rng.integers(8, 20, size=3))
        s = split(v)
        amax = np.abs(v).max()
        big = np.abs(v) >= 2.0 ** -12 * amax
        assert np.array_equal(s[big], v[big])
        assert np.all(np.abs(s - v) <= 2.0 ** -21 * amax)
        n_small += int((~big).sum())
    assert n_small > 1000


def test_split_counterexample_below_the_bound():
    v = np.zeros(32)
    v[0] = 1.7265625                 # q1 = 1.75: residual -0.0234375 sets the second term's grid
    v[1] = bf16(1.6 * 2.0 ** -16)    # 1.6e-5 of the block maximum
    s = split(v)
    assert s[0] == v[0] and s[1] != v[1]
    assert abs(s[1] - v[1]) <= 2.0 ** -21 * 1.7265625

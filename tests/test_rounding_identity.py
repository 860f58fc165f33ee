"""The exact-rounding identity the GroupNorm statistics kernels use.

For a power of two f and |x| = |d * f| <= 2^51 (x exact in fp64), the single
rounding of x + 1.5 * 2^52 lands on 1.5 * 2^52 + rint(x) (ties to even), and
the bit pattern of the result exceeds that of 1.5 * 2^52 by exactly rint(x)
when read as a 64-bit integer, also across the exponent step at 2^53.  The
kernels sum those patterns as integers and subtract count * bits(1.5 * 2^52).
Checked here on the host (numpy fp64 adds of exact products round like the
kernel's fused multiply-add) against numpy's rint.
"""
import numpy as np

M = np.float64(1.5 * 2.0 ** 52)
MB = np.int64(0x4338000000000000)


def bits(a):
    return np.asarray(a, dtype=np.float64).view(np.int64)


def test_magic_bits_equal_rint():
    rng = np.random.default_rng(11)
    d = rng.standard_normal(200_000).astype(np.float32).astype(np.float64)
    for e in (0, 5, 19, 30, 40, 47):
        f = np.float64(2.0 ** e)
        x = d * f                                  # exact: scaling by a power of two
        x = x[np.abs(x) <= 2.0 ** 51]
        t = x + M                                  # one rounding, as fl(fma(d, f, M))
        assert np.array_equal(bits(t) - MB, np.rint(x).astype(np.int64))


def test_ties_and_range_ends():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 2.0 ** 51, -(2.0 ** 51), 2.0 ** 51 - 0.5,
                  -(2.0 ** 51) + 0.5, 0.0, -0.0, 1e-300, -1e-300, 3.5, 4.5])
    t = x + M
    assert np.array_equal(bits(t) - MB, np.rint(x).astype(np.int64))


def test_square_terms_and_integer_sums():
    # q2 = rint(d * (d * 2^e2)): the product of two fp32 values is exact in fp64
    rng = np.random.default_rng(12)
    d = (rng.standard_normal(100_000) * 3).astype(np.float32).astype(np.float64)
    e2 = 52 - 17 - 2 * 4                           # a 2^17-element group with max |d| < 16
    x = d * (d * 2.0 ** e2)
    assert np.all(np.abs(x) <= 2.0 ** 51)
    t = x + M
    acc = int(np.sum(bits(t).astype(np.uint64), dtype=np.uint64))    # wraps mod 2^64
    total = (acc - len(x) * int(MB)) % 2 ** 64
    total = total - 2 ** 64 if total >= 2 ** 63 else total
    assert total == int(np.sum(np.rint(x).astype(np.int64)))

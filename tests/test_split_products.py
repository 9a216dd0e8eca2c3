"""Arithmetic of the Gram's split products, checked on the CPU.

The large-batch Gram kernels take every product x*y of two fp32 operands as
the six bf16 products of weight <= 2 of exact three-piece splits
x = h + m + l (h = bf16(x), m = bf16(x - h), l = bf16(x - h - m), rounding to
nearest even, differences in fp32).  These tests restate that arithmetic in
NumPy (bf16 rounding emulated on the float32 bit patterns, products summed in
float64, where products of bf16 values are exact) and check the claims the
kernels rely on: both differences are exact in fp32, the pieces give x back
to 2^-24 |x|, and the six products give x*y back to 2^-22 |x*y|.  They pin the
reading, not the kernel; the GPU value-solve tests hold the kernel's solves to
the float64 oracle.
"""
import numpy as np
import pytest


def bf16_rne(x):
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def split3(x):
    x = np.asarray(x, dtype=np.float32)
    h = bf16_rne(x)
    r1 = (x - h).astype(np.float32)
    m = bf16_rne(r1)
    r2 = (r1 - m).astype(np.float32)
    lo = bf16_rne(r2)
    return h, m, lo, r1, r2


def six_products(x, y):
    hx, mx, lx, _, _ = (a.astype(np.float64) for a in split3(x))
    hy, my, ly, _, _ = (a.astype(np.float64) for a in split3(y))
    return hx * hy + hx * my + mx * hy + hx * ly + lx * hy + mx * my


def operands(rng, n):
    """Softmax-weight-like values over a wide range, values of either sign,
    powers of two and values on bf16 rounding ties."""
    w = np.exp(rng.uniform(-60.0, 0.0, n)).astype(np.float32)
    v = (rng.standard_normal(n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32)
    p2 = np.ldexp(np.ones(64, np.float32), np.arange(-40, 24))
    tie = (np.float32(1.0) + np.float32(2.0 ** -8) * (2 * np.arange(64) + 1)).astype(np.float32)
    return np.concatenate([w, v, p2, -p2, tie, -tie]).astype(np.float32)


def test_bf16_rounding_emulation():
    # exact bf16 values are fixed points; halfway cases go to the even neighbour
    assert bf16_rne(np.float32(1.0)) == 1.0
    assert bf16_rne(np.float32(1.0 + 2 ** -8)) == 1.0            # tie -> even (1.0)
    assert bf16_rne(np.float32(1.0 + 3 * 2 ** -8)) == np.float32(1.0 + 2 ** -6)   # tie -> even
    assert bf16_rne(np.float32(1.0 + 2 ** -8 + 2 ** -20)) == np.float32(1.0 + 2 ** -7)
    x = np.float32(3.14159265)
    assert abs(float(bf16_rne(x)) - float(x)) <= 2 ** -8 * abs(float(x))


def test_split_differences_are_exact_and_reconstruct_x():
    rng = np.random.default_rng(7)
    x = operands(rng, 200000)
    h, m, lo, r1, r2 = split3(x)
    x64 = x.astype(np.float64)
    # the fp32 differences equal the exact ones
    assert np.array_equal(r1.astype(np.float64), x64 - h.astype(np.float64))
    assert np.array_equal(r2.astype(np.float64), r1.astype(np.float64) - m.astype(np.float64))
    # |x - h - m - l| <= 2^-24 |x| where l does not underflow
    err = np.abs(x64 - h.astype(np.float64) - m.astype(np.float64) - lo.astype(np.float64))
    ok = np.abs(x64) > 2.0 ** -100
    assert np.all(err[ok] <= 2.0 ** -24 * np.abs(x64[ok]))


@pytest.mark.parametrize("seed", [1, 2])
def test_six_products_within_two_to_minus_22(seed):
    rng = np.random.default_rng(seed)
    x = operands(rng, 100000)
    y = rng.permutation(operands(rng, 100000))[: x.size]
    exact = x.astype(np.float64) * y.astype(np.float64)
    got = six_products(x, y)
    ok = np.abs(exact) > 2.0 ** -90
    rel = np.abs(got[ok] - exact[ok]) / np.abs(exact[ok])
    assert rel.max() <= 2.0 ** -22
    # the dropped terms ml + lm are at most about 2^-23 |x y|; measured here
    # the worst case is near 2^-24.3
    assert rel.max() <= 2.0 ** -23
    # one fp32 rounding of the product is 2^-24; the six-product form stays
    # within a few of those
    assert np.median(rel) <= 2.0 ** -24


def test_dropping_the_l_pieces_is_not_enough():
    """With h and m only (four products) the error reaches about 2^-16: the
    l pieces are needed for fp32-level products."""
    rng = np.random.default_rng(3)
    x = operands(rng, 100000)
    y = rng.permutation(x)
    hx, mx, _, _, _ = (a.astype(np.float64) for a in split3(x))
    hy, my, _, _, _ = (a.astype(np.float64) for a in split3(y))
    four = hx * hy + hx * my + mx * hy + mx * my
    exact = x.astype(np.float64) * y.astype(np.float64)
    ok = np.abs(exact) > 2.0 ** -90
    rel = np.abs(four[ok] - exact[ok]) / np.abs(exact[ok])
    assert rel.max() > 2.0 ** -20

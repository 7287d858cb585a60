"""Pins of the orbit-patch oracle (mean deficit over the orders of a cached set).

[K] Kamera, gist.science/pt/paper/2606.23581, §3 ("Tres Operacoes de Janela Baratas",
item 1, "Reordenacao"): one patch averaged over permutations serves every order of the
set.  The mean is pinned to exact rational arithmetic with an independent
round-to-nearest-even, and to hand-worked ties; the orbit patch to the least-squares
property that makes the mean the right thing to factor: among rank-m matrices, the
top-m factorization of the mean minimizes the squared error summed over the orbit.
"""
from fractions import Fraction

import numpy as np

from oracle import patch_form as pf


def _bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 pattern, from the format's definition."""
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0:
        return s * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    v = Fraction(128 + f, 128)
    return s * (v * (1 << (e - 127)) if e >= 127 else v / (1 << (127 - e)))


def _rne_bf16(x: Fraction) -> int:
    """Exact rational -> bf16 bits, nearest with ties to even, by search over patterns
    (finite magnitudes only; the tests stay far from overflow)."""
    s = 0x8000 if x < 0 else 0
    a = abs(x)
    lo, hi = 0, 0x7F7F  # magnitudes are monotone in the pattern
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if _bf16_value(mid) <= a:
            lo = mid
        else:
            hi = mid
    if _bf16_value(hi) <= a:
        lo = hi
    up = min(lo + 1, 0x7F7F)
    dl, du = a - _bf16_value(lo), _bf16_value(up) - a
    if du < dl or (du == dl and up % 2 == 0 and up != lo):
        lo = up
    return s | lo


def test_worked_ties():
    # 1 and 1 + 2^-7 (adjacent bf16 values): the mean 1 + 2^-8 is halfway; the even
    # neighbour is 1 (0x3F80).  1 + 2^-7 and 1 + 2^-6: the mean 1 + 3 * 2^-8 is halfway
    # between 0x3F81 and 0x3F82; the even one is 0x3F82.
    got = pf.orbit_mean(np.array([[0x3F80, 0x3F81, 0xBF80], [0x3F81, 0x3F82, 0xBF81]], np.uint16))
    assert got.tolist() == [0x3F80, 0x3F82, 0xBF80]
    # three orders: (1 + 1 + 2) / 3 = 4/3 = 1.0101..b -> 1.0101011b (0x3FAB)
    got = pf.orbit_mean(np.array([[0x3F80], [0x3F80], [0x4000]], np.uint16))
    assert got.tolist() == [0x3FAB]
    # (2 + 2^-6) + 2 + 2^-28 + 0 over four: 1 + 2^-8 + 2^-30, just above the tie between
    # 1 and 1 + 2^-7, so it rounds up (0x3F81).  A sum kept in fp32 would lose the 2^-28
    # and land on the tie, which goes to the even 1.
    got = pf.orbit_mean(np.array([[0x4001, 0xC001], [0x4000, 0xC000], [0x3180, 0xB180],
                                  [0x0000, 0x8000]], np.uint16))
    assert got.tolist() == [0x3F81, 0xBF81]


def test_mean_matches_exact_rational_rounding():
    rng = np.random.default_rng(7)
    for P in (1, 2, 3, 5, 7, 8):
        # finite values whose exponents span at most 30 binades (normal and subnormal
        # bf16 included), so the fp64 sum and quotient sit far from any bf16 tie they
        # do not equal exactly
        base = int(rng.integers(1, 200))
        e = rng.integers(max(0, base - 30), base + 1, size=(P, 400))
        bits = ((e << 7) | rng.integers(0, 128, size=(P, 400)) |
                (rng.integers(0, 2, size=(P, 400)) << 15)).astype(np.uint16)
        got = pf.orbit_mean(bits)
        for i in range(bits.shape[1]):
            exact = sum(_bf16_value(int(b)) for b in bits[:, i]) / P
            want = _rne_bf16(exact)
            assert got[i] == want or (exact == 0 and got[i] & 0x7FFF == 0), (P, i, hex(got[i]), hex(want))


def test_single_order_and_sign_symmetry():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x7F80, size=(1, 1000)).astype(np.uint16)  # finite, positive
    assert np.array_equal(pf.orbit_mean(bits), bits[0])
    two = rng.integers(0, 0x7F00, size=(4, 1000)).astype(np.uint16)
    assert np.array_equal(pf.orbit_mean(two ^ 0x8000), pf.orbit_mean(two) ^ 0x8000)


def test_orbit_patch_minimizes_error_over_the_orbit():
    rng = np.random.default_rng(11)
    P, T, F, m = 5, 30, 20, 4
    common = rng.standard_normal((T, 6)) @ rng.standard_normal((6, F))
    deltas = [common + 0.3 * rng.standard_normal((T, F)) for _ in range(P)]
    mean = sum(deltas) / P
    U, V, s = pf.top_m_factors(mean, m)
    best = U @ V.T

    def J(X):
        return sum(np.linalg.norm(d - X) ** 2 for d in deltas)

    # the split of the orbit error into spread and distance to the mean
    for X in (best, np.zeros((T, F)), rng.standard_normal((T, F))):
        spread = sum(np.linalg.norm(d - mean) ** 2 for d in deltas)
        np.testing.assert_allclose(J(X), spread + P * np.linalg.norm(mean - X) ** 2, rtol=1e-12)
    # no other rank-m candidate does better: the per-order patches, perturbations of
    # the optimum, and the best product for random token factors
    for d in deltas:
        Ud, Vd, _ = pf.top_m_factors(d, m)
        assert J(Ud @ Vd.T) >= J(best) - 1e-9
    for _ in range(30):
        Q = (U + 1e-3 * rng.standard_normal(U.shape)) @ (V + 1e-3 * rng.standard_normal(V.shape)).T
        assert J(Q) >= J(best) - 1e-12
        A = rng.standard_normal((T, m))
        B = np.linalg.lstsq(A, mean, rcond=None)[0]
        assert J(A @ B) >= J(best) - 1e-9


def test_orbit_patch_factors_the_rounded_mean():
    rng = np.random.default_rng(5)
    P, L, T, F, m = 3, 2, 40, 16, 3
    x = rng.standard_normal((P, L, T, F)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    offsets = [0, 25, 40]
    U, V, S = pf.orbit_patch(bits, offsets, m)
    mean = pf._orc.bf16_to_f64(pf.orbit_mean(bits))
    U2, V2, S2 = pf.form_patch(mean, offsets, m)
    for l in range(L):
        for j in range(2):
            a, b = offsets[j], offsets[j + 1]
            np.testing.assert_allclose(U[l, a:b] @ V[l, j].T, U2[l, a:b] @ V2[l, j].T, atol=1e-12)

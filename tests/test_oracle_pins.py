"""Pins of the CPU oracle to facts outside itself.

Sources (web summaries):
  [K] Kamera, gist.science/pt/paper/2606.23581 (and the Korean twin).
  [N] "Modelos Tomam Notas no Prefill", gist.science/pt/paper/2606.17107.

Each pin is chosen so that a plausible mistake in the oracle fails at least one of
them; test_planted_mistakes_fail_a_pin plants such mistakes and checks that.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def taylor_cos_sin(x: Fraction, terms: int = 40):
    c, s = Fraction(0), Fraction(0)
    for n in range(terms):
        c += (-1) ** n * x ** (2 * n) / math.factorial(2 * n)
        s += (-1) ** n * x ** (2 * n + 1) / math.factorial(2 * n + 1)
    return c, s


def load_worked_example():
    rows = []
    with open(os.path.join(GOLDEN, "rotation_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, c = [p.split() for p in line.split("|")]
            rows.append((float(a[0]), int(a[1]), int(a[2]),
                         np.array([float(v) for v in b]), np.array([float(v) for v in c])))
    return rows


def rope_complex(x, p, theta, r):
    """Textbook RoPE at absolute position p: pair (x_i, x_{i+r/2}) read as the complex
    number x_i + i x_{i+r/2} and multiplied by exp(i p theta^(-2i/r))."""
    half = r // 2
    w = theta ** (-2.0 * np.arange(half) / r)
    z = (x[:half] + 1j * x[half:r]) * np.exp(1j * p * w)
    out = x.copy()
    out[:half], out[half:r] = z.real, z.imag
    return out


# ----------------------------------------------------------------- worked example

def test_golden_constants_are_the_closed_forms():
    # cos 1, sin 1, cos 0.01, sin 0.01 written in the fixture equal their Taylor series
    # (exact rational arithmetic) to within the rounding of a double.
    c1, s1 = taylor_cos_sin(Fraction(1))
    c2, s2 = taylor_cos_sin(Fraction(1, 100))
    for got, exact in [(0.5403023058681398, c1), (0.8414709848078965, s1),
                       (0.9999500004166653, c2), (0.009999833334166664, s2)]:
        assert abs(Fraction(got) - exact) <= Fraction(1, 2 ** 53) * abs(exact) * 2


@pytest.mark.parametrize("case", range(5))
def test_worked_example(case):
    theta, r, delta, x, y = load_worked_example()[case]
    got = orc.rotate_head_f64(x, r, theta, delta)
    np.testing.assert_allclose(got, y, rtol=0, atol=4e-16)


def test_frequency_formula_points():
    # theta^(-2i/r): i = 0 gives 1; i = r/4 gives theta^(-1/2); exact powers of two.
    assert orc.freq(1e4, 4, 0) == 1.0
    assert orc.freq(1e4, 4, 1) == pytest.approx(0.01, rel=1e-15)
    assert orc.freq(256.0, 8, 2) == 1.0 / 16.0
    assert orc.freq(1e6, 128, 32) == pytest.approx(1e-3, rel=1e-15)


# ----------------------------------------------------------------- rotation algebra

def test_composition_group_law():
    # R(d1) R(d2) = R(d1 + d2) ([K §2]: relocation is an exact rotation; rotations by
    # angles linear in delta compose additively).
    rng = np.random.default_rng(1)
    for theta, r, D, big in [(1e4, 64, 64, 1e5), (1e6, 128, 128, 1e5), (5e5, 32, 64, 300)]:
        for _ in range(20):
            x = rng.standard_normal(D)
            d1, d2 = (int(v) for v in rng.integers(-big, big + 1, size=2))
            a = orc.rotate_head_f64(orc.rotate_head_f64(x, r, theta, d2), r, theta, d1)
            b = orc.rotate_head_f64(x, r, theta, d1 + d2)
            # angle error of fp64 delta*omega is ~|delta| 2^-52 per product
            tol = 1e-13 + 4 * (abs(d1) + abs(d2)) * 2.0 ** -52
            assert np.max(np.abs(a - b)) <= tol * np.linalg.norm(x)


def test_shift_equivalence_with_textbook_rope():
    # Relocating keys rotated at position p by delta equals rotating the pre-RoPE keys
    # at p + delta ([K §2] "Relocacao" and [N §3B]: keys move to their new absolute
    # positions by re-rotation).
    rng = np.random.default_rng(2)
    for theta, r in [(1e4, 64), (1e6, 128), (5e5, 128)]:
        for _ in range(20):
            x = rng.standard_normal(r)
            p, d = (int(v) for v in rng.integers(-100000, 100001, size=2))
            got = orc.rotate_head_f64(rope_complex(x, p, theta, r), r, theta, d)
            want = rope_complex(x, p + d, theta, r)
            assert np.max(np.abs(got - want)) <= 1e-10 * np.linalg.norm(x)


def test_pair_norms_preserved():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128)
    y = orc.rotate_head_f64(x, 128, 1e6, -1536)
    n0 = x[:64] ** 2 + x[64:] ** 2
    n1 = y[:64] ** 2 + y[64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-14)


def test_partial_rotary_leaves_tail():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(128)
    y = orc.rotate_head_f64(x, 64, 1e4, 12345)
    assert np.array_equal(y[64:], x[64:])
    assert not np.array_equal(y[:64], x[:64])


# ----------------------------------------------------------------- identity / pass-through

def _all_bf16_patterns():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _problem(data, T, H, D, r, delta, rank=0, U=None, V=None, offsets=None):
    ch = dict(data=data, heads=H, dim=D, rope_dim=r, layer_stride=T * H * D,
              slot_stride=H * D, head_stride=D, page_stride=0)
    if rank:
        ch["U"], ch["V"] = U, V
    offs = np.array([0, T], dtype=np.int64) if offsets is None else offsets
    dl = np.array([delta], dtype=np.int64) if np.isscalar(delta) else np.asarray(delta, np.int64)
    orc.relocate_patch([ch], num_layers=1, theta=1e4, offsets=offs, delta=dl, rank=rank)


def test_identity_every_bit_pattern():
    # delta = 0 with no patch: every element keeps its bits (NaN payloads, -0,
    # subnormals and infinities included).
    x = _all_bf16_patterns()
    y = x.copy()
    _problem(y, T=1024, H=1, D=64, r=64, delta=0)
    assert np.array_equal(x, y)


def test_unrotated_channel_and_tail_pass_through():
    # No patch: a channel with rope_dim 0 (V, c_KV) and dims >= rope_dim keep their
    # bits whatever delta is ([K §2] c_KV reused byte for byte; [K §3] survivors need
    # only the rotation; [N §3B] values carried over unchanged).
    x = _all_bf16_patterns()
    y = x.copy()
    _problem(y, T=1024, H=1, D=64, r=0, delta=777)
    assert np.array_equal(x, y)
    y = x.copy()
    _problem(y, T=1024, H=1, D=64, r=32, delta=777)
    xv, yv = x.reshape(1024, 64), y.reshape(1024, 64)
    assert np.array_equal(xv[:, 32:], yv[:, 32:])


# ----------------------------------------------------------------- patch

def test_patch_is_added_after_rotation():
    # out(m) - out(0) = U V^T exactly in fp64, whatever delta is ([K §2], reuse
    # equation: the rank-m product is added to the relocated KV, not rotated with it).
    rng = np.random.default_rng(5)
    H, D, m, T = 2, 64, 8, 12
    F = H * D
    V = rng.standard_normal((F, m))
    for delta in (0, 37, -100000):
        for t in range(T):
            x = rng.standard_normal(F)
            u = rng.standard_normal(m)
            y0 = orc.row_f64(x, H, D, D, 1e4, delta)
            ym = orc.row_f64(x, H, D, D, 1e4, delta, u, V)
            np.testing.assert_allclose(ym - y0, np.matmul(V, u), rtol=0,
                                       atol=1e-13 * (1 + np.abs(np.matmul(V, u)).max()))


def test_svd_patch_eckart_young():
    # [K §2]: the patch is the top-m SVD factors of the deficit Delta (T x F).  With
    # m = rank(Delta) the patched KV equals KV + Delta; with m < rank the residual's
    # Frobenius norm is sqrt(sum of the dropped sigma_i^2) (Eckart-Young).
    rng = np.random.default_rng(6)
    T, F = 16, 8
    Delta = rng.standard_normal((T, F))
    x = rng.standard_normal((T, F))
    Uf, S, Vt = np.linalg.svd(Delta, full_matrices=False)
    for m in range(0, F + 1):
        U_m = Uf[:, :m] * S[:m]
        V_m = Vt[:m].T
        out = np.stack([orc.row_f64(x[t], 1, F, 0, 1e4, 0, U_m[t] if m else None,
                                    V_m if m else None) for t in range(T)])
        resid = np.linalg.norm(out - (x + Delta))
        want = math.sqrt(float(np.sum(S[m:] ** 2)))
        assert resid == pytest.approx(want, rel=1e-12, abs=1e-12)
    # brute-force check of the optimality on a 3 x 2 case: no rank-1 matrix from a
    # grid of directions beats the SVD residual.
    D3 = rng.standard_normal((3, 2))
    s3 = np.linalg.svd(D3, compute_uv=False)
    best = min(np.linalg.norm(D3 - np.outer(D3 @ v, v))
               for a in np.linspace(0, np.pi, 2001) for v in [np.array([np.cos(a), np.sin(a)])])
    assert best >= s3[1] - 1e-12 and best == pytest.approx(s3[1], rel=1e-5)


# ----------------------------------------------------------------- rounding

def _exact_rne_bf16(v: float) -> int:
    """bf16 bits of the exact rational RNE of a finite double."""
    if v == 0:
        return 0x8000 if math.copysign(1, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)
    scaled = a / Fraction(2) ** q
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** q
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = int(np.array([float(val)], dtype=np.float32).view(np.uint32)[0]) >> 16
    return sign | bits


def test_round_bf16_ties_and_boundaries_exact_rational():
    vals = []
    for b in list(range(0, 0x7F80, 97)) + [0, 1, 2, 0x7F, 0x80, 0x81, 0x7F7E, 0x7F7F]:
        lo = float(orc.bf16_to_f64(np.array([b], np.uint16))[0])
        hi = 2.0 ** 128 if b == 0x7F7F else float(orc.bf16_to_f64(np.array([b + 1], np.uint16))[0])
        mid = (lo + hi) / 2  # exact in fp64
        vals += [lo, mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), hi]
    vals += [3.3895313892515355e38, 3.402823669209385e38, 1e-45, 2.0 ** -134, 3 * 2.0 ** -135]
    vals = np.array(vals + [-v for v in vals], dtype=np.float64)
    got = orc.round_bf16(vals)
    want = np.array([_exact_rne_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_matches_torch_on_fp32_values():
    # For a value already in fp32 one rounding to bf16 is the same from fp32 or fp64:
    # torch's fp32 -> bf16 conversion (round to nearest even) must agree.
    torch = pytest.importorskip("torch")
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(7)
    bits = np.concatenate([bits, rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)])
    f32 = bits.view(np.float32)
    with np.errstate(invalid="ignore"):
        got = orc.round_bf16(f32.astype(np.float64))
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f32)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_fp32_storage_rounds_once():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(64).astype(np.float32)
    u = rng.standard_normal(4).astype(np.float32)
    V = rng.standard_normal((64, 4)).astype(np.float32)
    got = orc.row(x, 1, 64, 64, 1e4, 99, u, V)
    want = orc.row_f64(x.astype(np.float64), 1, 64, 64, 1e4, 99, u.astype(np.float64),
                       V.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ----------------------------------------------------------------- layouts

def test_paged_layout_matches_contiguous():
    # A paged cache holding the same logical tokens gives bit-identical results:
    # identity table and a random permutation, spare pool pages untouched.
    rng = np.random.default_rng(9)
    L, T, H, D, P, m = 2, 45, 2, 64, 8, 3
    n_pages_needed = -(-T // P)
    x = rng.standard_normal((L, T, H, D)).astype(np.float32)
    xb = orc.round_bf16(x.astype(np.float64)).reshape(L, T, H, D)
    U = orc.round_bf16(0.3 * rng.standard_normal((L, T, m))).reshape(L, T, m)
    V = orc.round_bf16(0.3 * rng.standard_normal((2, L, 2, H * D, m))).reshape(2, L, 2, H * D, m)
    offs = np.array([0, 20, T], np.int64)
    delta = np.array([5, -70000], np.int64)

    def chans(data, paged, pool):
        out = []
        for c in range(2):
            d = dict(data=data[c], heads=H, dim=D, rope_dim=D if c == 0 else 0,
                     slot_stride=H * D, head_stride=D, U=U, V=V[c])
            if paged:
                d.update(layer_stride=pool * P * H * D, page_stride=P * H * D)
            else:
                d.update(layer_stride=T * H * D, page_stride=0)
            out.append(d)
        return out

    cont = [xb.copy().ravel(), xb.copy().ravel()]
    orc.relocate_patch(chans(cont, False, 0), num_layers=L, theta=1e4, offsets=offs,
                       delta=delta, rank=m)
    for table in (np.arange(n_pages_needed), rng.permutation(n_pages_needed + 5)[:n_pages_needed]):
        pool = int(table.max()) + 1 + 2
        pools = []
        for c in range(2):
            pl = np.full((L, pool, P, H, D), 0x7FC1, dtype=np.uint16)  # sentinel NaN payload
            for t in range(T):
                pl[:, table[t // P], t % P] = xb[:, t]
            pools.append(pl.ravel())
        snap = [p.copy() for p in pools]
        orc.relocate_patch(chans(pools, True, pool), num_layers=L, theta=1e4, offsets=offs,
                           delta=delta, rank=m, page_size=P, block_table=table.astype(np.int32))
        for c in range(2):
            pl = pools[c].reshape(L, pool, P, H, D)
            got = np.stack([pl[:, table[t // P], t % P] for t in range(T)], axis=1)
            assert np.array_equal(got, cont[c].reshape(L, T, H, D))
            used = np.zeros((pool, P), bool)
            for t in range(T):
                used[table[t // P], t % P] = True
            assert np.array_equal(pl[:, ~used], snap[c].reshape(L, pool, P, H, D)[:, ~used])


def test_chunks_use_their_own_delta_and_factors():
    # Batched call over several chunks equals one call per chunk.
    rng = np.random.default_rng(10)
    T, H, D, m = 30, 1, 64, 2
    offs = np.array([0, 7, 7, 19, 30], np.int64)   # includes an empty chunk
    delta = np.array([3, 99, -4000, 0], np.int64)
    x = orc.round_bf16(rng.standard_normal(T * H * D))
    U = orc.round_bf16(rng.standard_normal(T * m))
    V = orc.round_bf16(rng.standard_normal(4 * H * D * m))
    batched = x.copy()
    orc.relocate_patch([dict(data=batched, heads=H, dim=D, rope_dim=D, layer_stride=T * H * D,
                             slot_stride=H * D, head_stride=D, U=U, V=V)],
                       num_layers=1, theta=1e4, offsets=offs, delta=delta, rank=m)
    for j in range(4):
        a, b = int(offs[j]), int(offs[j + 1])
        if a == b:
            continue
        part = x[a * D:b * D].copy()
        orc.relocate_patch([dict(data=part, heads=H, dim=D, rope_dim=D, layer_stride=(b - a) * D,
                                 slot_stride=D, head_stride=D, U=U[a * m:b * m].copy(),
                                 V=V[j * D * m:(j + 1) * D * m].copy())],
                           num_layers=1, theta=1e4, offsets=np.array([0, b - a], np.int64),
                           delta=delta[j:j + 1], rank=m)
        assert np.array_equal(part, batched[a * D:b * D])


# ----------------------------------------------------------------- planted mistakes

def _pins_pass(rotate, row):
    """The pins above, phrased over replaceable rotate/row functions."""
    ok = True
    for theta, r, delta, x, y in load_worked_example():
        ok &= bool(np.max(np.abs(rotate(x, r, theta, delta) - y)) <= 4e-16)
    rng = np.random.default_rng(11)
    x = rng.standard_normal(64)
    ok &= bool(np.max(np.abs(rotate(rope_complex(x, 1000, 1e4, 64), 64, 1e4, 2345)
                             - rope_complex(x, 3345, 1e4, 64))) <= 1e-10 * np.linalg.norm(x))
    T, F = 16, 8
    Delta = rng.standard_normal((T, F))
    xx = rng.standard_normal((T, F))
    Uf, S, Vt = np.linalg.svd(Delta, full_matrices=False)
    out = np.stack([row(xx[t], 1, F, 0, 1e4, 0, Uf[t] * S, Vt.T) for t in range(T)])
    ok &= bool(np.linalg.norm(out - (xx + Delta)) <= 1e-12)
    xr = rng.standard_normal(64)
    u = rng.standard_normal(3)
    V = rng.standard_normal((64, 3))
    ok &= bool(np.allclose(row(xr, 1, 64, 64, 1e4, 55, u, V) - row(xr, 1, 64, 64, 1e4, 55),
                           V @ u, rtol=0, atol=1e-12))
    return ok


def test_planted_mistakes_fail_a_pin():
    assert _pins_pass(orc.rotate_head_f64, orc.row_f64)

    def interleaved(x, r, theta, delta):  # pairs (2i, 2i+1) instead of (i, i + r/2)
        perm = np.concatenate([np.arange(0, r, 2), np.arange(1, r, 2), np.arange(r, x.size)])
        y = orc.rotate_head_f64(x[perm], r, theta, delta)
        out = np.empty_like(y)
        out[perm] = y
        return out

    mutants = {
        "sign of delta": (lambda x, r, th, d: orc.rotate_head_f64(x, r, th, -d), orc.row_f64),
        "frequency theta^(-i/r)": (lambda x, r, th, d: orc.rotate_head_f64(x, r, th ** 0.5, d),
                                   orc.row_f64),
        "interleaved pairing": (interleaved, orc.row_f64),
        "patch dropped": (orc.rotate_head_f64,
                          lambda x, H, D, r, th, d, u=None, V=None: orc.row_f64(x, H, D, r, th, d)),
        "V transposed": (orc.rotate_head_f64,
                         lambda x, H, D, r, th, d, u=None, V=None: orc.row_f64(
                             x, H, D, r, th, d, u,
                             None if V is None else np.ascontiguousarray(V.T).reshape(V.shape))),
        "patch rotated with the key": (
            orc.rotate_head_f64,
            lambda x, H, D, r, th, d, u=None, V=None: orc.row_f64(
                np.asarray(x) + (0 if V is None else V @ u), H, D, r, th, d)),
    }
    for name, (rot, row) in mutants.items():
        assert not _pins_pass(rot, row), f"planted mistake '{name}' passed every pin"

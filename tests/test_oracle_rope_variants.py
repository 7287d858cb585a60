"""Pins of the oracle's positional variants: interleaved pairing and M-RoPE sections.

[N] "Modelos Tomam Notas no Prefill", gist.science/pt/paper/2606.17107, §4 (composition,
generality): image KV is transplanted with M-RoPE re-rotation.  [K] Kamera §2 fixes the
operation (re-rotation by the phase shift of the new position); the pages print no
formula, so the references here are the textbook forms, written out independently of
the oracle:
  - interleaved (RoFormer) RoPE: pair i is the complex number x[2i] + i x[2i+1], turned
    by e^{i p w_i}, w_i = theta^(-2i/r);
  - multimodal RoPE: a position is a vector (one component per section), frequency i
    takes the component of the section it falls in (sections cut the r/2 frequencies in
    order), and each frequency turns both dims of its NeoX pair (i, i + r/2).
Relocating a key rotated at position p by delta must give the key rotated at p + delta.
"""
import numpy as np
import pytest

from oracle import oracle as orc

SECTIONS = (16, 24, 24)   # a three-section split of the 64 pairs of a 128-dim head


def freqs(theta, r):
    return theta ** (-2.0 * np.arange(r // 2) / r)


def rope_interleaved_at(x, p, theta, r):
    z = x[0:r:2] + 1j * x[1:r:2]
    z = z * np.exp(1j * p * freqs(theta, r))
    y = x.astype(np.float64).copy()
    y[0:r:2], y[1:r:2] = z.real, z.imag
    return y


def mrope_at(x, pos, theta, r, sections):
    """Textbook M-RoPE on a NeoX-paired head: cos/sin tables per position component,
    picked per frequency by section, applied as x cos + rotate_half(x) sin."""
    half = r // 2
    comp = np.repeat(np.arange(len(sections)), sections)      # component of frequency i
    ang = np.asarray(pos, dtype=np.float64)[comp] * freqs(theta, r)
    cos = np.concatenate([np.cos(ang), np.cos(ang)])
    sin = np.concatenate([np.sin(ang), np.sin(ang)])
    xr = x[:r].astype(np.float64)
    rot_half = np.concatenate([-xr[half:], xr[:half]])
    y = x.astype(np.float64).copy()
    y[:r] = xr * cos + rot_half * sin
    return y


def test_interleaved_shift_equivalence_with_textbook():
    rng = np.random.default_rng(1)
    for theta, r, D in ((1e4, 64, 64), (1e6, 128, 128), (5e5, 32, 64)):
        for p, d in ((0, 37), (1000, -1536), (70000, 65536)):
            x = rng.standard_normal(D)
            got = orc.rotate_head_f64(rope_interleaved_at(x, p, theta, r), r, theta, d,
                                      pairing=orc.INTERLEAVED)
            want = rope_interleaved_at(x, p + d, theta, r)
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-9 * (1 + abs(p + d)) ** 0.5)


def test_interleaved_is_neox_under_the_pair_permutation():
    # Interleaved pair i = dims (2i, 2i+1); NeoX pair i = dims (i, i + r/2).  With
    # perm[2i] = i and perm[2i+1] = i + r/2, an interleaved head is x_neox[perm], and
    # the two rotations commute with that move exactly (same arithmetic per pair).
    rng = np.random.default_rng(2)
    r, D = 64, 96
    perm = np.arange(D)
    perm[:r] = np.stack([np.arange(r // 2), np.arange(r // 2) + r // 2], axis=1).ravel()
    for d in (3, -99991):
        xn = rng.standard_normal(D)
        il = orc.rotate_head_f64(xn[perm], r, 1e4, d, pairing=orc.INTERLEAVED)
        assert np.array_equal(il, orc.rotate_head_f64(xn, r, 1e4, d)[perm])


@pytest.mark.parametrize("pairing", [orc.NEOX, orc.INTERLEAVED])
def test_mrope_shift_equivalence_with_textbook(pairing):
    rng = np.random.default_rng(3)
    r, D, theta = 128, 128, 1e6
    for pos, dl in (((0, 0, 0), (37, 37, 37)), ((100, 12, 30), (-1536, 5, -7)),
                    ((5000, 40, 2), (65536, 0, 17))):
        x = rng.standard_normal(D)
        if pairing == orc.NEOX:
            start = mrope_at(x, pos, theta, r, SECTIONS)
            want = mrope_at(x, np.add(pos, dl), theta, r, SECTIONS)
        else:  # same tables on the interleaved layout (head = x_neox[perm])
            perm = np.stack([np.arange(r // 2), np.arange(r // 2) + r // 2], axis=1).ravel()
            start = mrope_at(x, pos, theta, r, SECTIONS)[perm]
            want = mrope_at(x, np.add(pos, dl), theta, r, SECTIONS)[perm]
        got = orc.rotate_head_f64(start, r, theta, dl, pairing=pairing, sections=SECTIONS)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-8)


def test_equal_section_deltas_are_plain_rope():
    rng = np.random.default_rng(4)
    x = orc.round_bf16(rng.standard_normal((5, 2 * 128)))
    for d in (1, -1536, 65536):
        a = np.stack([orc.row(x[t], 2, 128, 128, 1e6, (d, d, d), sections=SECTIONS)
                      for t in range(5)])
        b = np.stack([orc.row(x[t], 2, 128, 128, 1e6, d) for t in range(5)])
        assert np.array_equal(a, b)


def test_section_with_zero_delta_keeps_every_bit():
    # Rank 0: the pairs of a section whose delta is 0 do not move (R(0) is the identity),
    # whatever the partner holds (NaN payloads, infinities, -0).
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(-1, 128)
    half = 64
    comp = np.repeat(np.arange(3), SECTIONS)
    for dl in ((0, 5, 0), (7, 0, 0), (0, 0, -3)):
        out = np.stack([orc.row(x[t], 1, 128, 128, 1e6, dl, sections=SECTIONS)
                        for t in range(x.shape[0])])
        still = np.concatenate([np.asarray(dl)[comp] == 0] * 2)
        assert np.array_equal(out[:, still], x[:, still])
        assert not np.array_equal(out[:, ~still], x[:, ~still])
        assert still.sum() < 128 and half > 0


def test_relocate_patch_with_sections_matches_rows():
    # The whole operator over chunks with per-section deltas equals the row function.
    rng = np.random.default_rng(5)
    T, H, D, m = 12, 2, 128, 4
    offs = np.array([0, 5, 12], np.int64)
    delta = np.array([[3, -2, 0], [0, 0, 0]], np.int64)
    x = orc.round_bf16(rng.standard_normal(T * H * D))
    U = orc.round_bf16(0.3 * rng.standard_normal(T * m))
    V = orc.round_bf16(0.3 * rng.standard_normal(2 * H * D * m))
    for rank in (0, m):
        y = x.copy()
        ch = dict(data=y, heads=H, dim=D, rope_dim=D, layer_stride=T * H * D, slot_stride=H * D,
                  head_stride=D)
        if rank:
            ch.update(U=U, V=V)
        orc.relocate_patch([ch], num_layers=1, theta=1e6, offsets=offs, delta=delta, rank=rank,
                           sections=SECTIONS)
        for t in range(T):
            j = 0 if t < 5 else 1
            want = orc.row(x[t * H * D:(t + 1) * H * D], H, D, D, 1e6, delta[j],
                           U[t * m:(t + 1) * m] if rank else None,
                           V[j * H * D * m:(j + 1) * H * D * m].reshape(H * D, m) if rank else None,
                           sections=SECTIONS)
            assert np.array_equal(y[t * H * D:(t + 1) * H * D], want)


def test_planted_section_mistakes_fail():
    # Sections in the wrong order, or deltas matched to the wrong section, fail the
    # textbook pin.
    rng = np.random.default_rng(6)
    r, theta = 128, 1e6
    x = rng.standard_normal(r)
    pos, dl = (100, 12, 30), (-1536, 5, -7)
    start = mrope_at(x, pos, theta, r, SECTIONS)
    want = mrope_at(x, np.add(pos, dl), theta, r, SECTIONS)
    good = orc.rotate_head_f64(start, r, theta, dl, sections=SECTIONS)
    assert np.abs(good - want).max() < 1e-8
    for bad in (orc.rotate_head_f64(start, r, theta, dl, sections=SECTIONS[::-1]),
                orc.rotate_head_f64(start, r, theta, dl[::-1], sections=SECTIONS),
                orc.rotate_head_f64(start, r, theta, dl, pairing=orc.INTERLEAVED,
                                    sections=SECTIONS)):
        assert np.abs(bad - want).max() > 1e-3

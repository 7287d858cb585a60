"""Pins of the oracle's 8-bit KV form.

[N] "Modelos Tomam Notas no Prefill", gist.science/pt/paper/2606.17107, closing summary:
the method is validated on FP8-quantised models.  Reading: KV elements are OCP FP8 E4M3
codes with one dequantisation scale per (layer, channel); the operator acts on the
values scale * code and the result is divided by the scale and rounded to the nearest
code (ties to even), saturating at +-448.  The factors stay bf16.

The codec is pinned to the OCP E4M3 definition (spot values and structure) and to
PyTorch's own E4M3 conversions, a library routine independent of the oracle; the
operator's fp8 form is pinned to its fp32 form (pinned elsewhere) followed by
PyTorch's encoder, and to exact scale invariances.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(vals_f32):
    t = torch.from_numpy(np.asarray(vals_f32, np.float32).copy()).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_spot_values_from_the_format_definition():
    # Bias 7, 3 mantissa bits, subnormals m * 2^-9, one NaN pattern per sign.
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x48: 4.0,
             0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    got = orc.fp8_to_f64(list(table))
    assert np.array_equal(got, np.array(list(table.values())))
    assert np.signbit(orc.fp8_to_f64([0x80]))[0] and orc.fp8_to_f64([0x80])[0] == 0.0
    nan = np.isnan(orc.fp8_to_f64(np.arange(256)))
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    pos = orc.fp8_to_f64(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)  # codes 0..0x7E are the magnitudes in order
    assert np.array_equal(orc.fp8_to_f64(np.arange(0x80, 0xFF)), -pos)


def test_decode_matches_pytorch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    a, b = orc.fp8_to_f64(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok])
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


def test_encode_matches_pytorch_inside_the_range():
    # Every magnitude, every midpoint (a tie) and the fp32 neighbours of each midpoint,
    # both signs, plus random values: PyTorch rounds fp32 to nearest, ties to even.
    mags = orc.fp8_to_f64(np.arange(0x7F))
    mids = (mags[:-1] + mags[1:]) / 2
    m32 = mids.astype(np.float32)
    pts = np.concatenate([mags.astype(np.float32), m32,
                          np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))])
    rng = np.random.default_rng(3)
    pts = np.concatenate([pts, rng.normal(0, 60, 4000).astype(np.float32),
                          rng.normal(0, 0.01, 2000).astype(np.float32)])
    pts = pts[np.abs(pts) <= 448]
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(orc.round_fp8(pts.astype(np.float64)), _torch_encode(pts))


def test_encode_saturates_and_keeps_nan_and_signed_zero():
    y = np.array([448.0, 460.0, 464.0, 465.0, 1e4, np.inf, -500.0, -np.inf, 0.0, -0.0,
                  -1e-30, 2.0 ** -10, 3 * 2.0 ** -11])
    got = orc.round_fp8(y)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x80,
                         0x00, 0x01]
    assert orc.round_fp8([np.nan])[0] & 0x7F == 0x7F


def _codes(rng, shape, amax=200.0):
    """Random E4M3 codes of values spread over +-amax (PyTorch's encoder)."""
    v = np.clip(rng.standard_normal(shape) * amax / 3, -amax, amax).astype(np.float32)
    return _torch_encode(v.ravel()).reshape(shape)


def _chan(data, H, D, r, L, T, U=None, V=None, scale=None):
    d = dict(data=data, heads=H, dim=D, rope_dim=r, layer_stride=T * H * D, slot_stride=H * D,
             head_stride=D, page_stride=0)
    if U is not None:
        d.update(U=U, V=V)
    if scale is not None:
        d["scale"] = scale
    return d


@pytest.mark.parametrize("m", [0, 5])
def test_fp8_operator_equals_fp32_operator_then_pytorch_encode(m):
    # The fp8 form is the fp32 form run on the values scale * code, divided by the
    # scale, then encoded.  Scales are powers of two times 1.5 so that scale * code is
    # exact in fp32 (the fp32 form's input).  Only the final fp32 -> fp8 step differs
    # (the fp8 form rounds once, from fp64), so values whose fp32 rounding lands on an
    # fp8 tie would differ; the seeds used have none.
    L, T, H, D, r = 2, 37, 2, 32, 16
    rng = np.random.default_rng(40 + m)
    q = _codes(rng, (L, T, H, D))
    scale = np.array([1.5 * 2.0 ** -6, 1.5 * 2.0 ** -9], np.float32)
    Ub = orc.round_bf16(0.5 * rng.standard_normal((L, T, max(m, 1))))[:, :, :m]
    Vb = orc.round_bf16(0.5 * rng.standard_normal((L, 2, H * D, max(m, 1))))[..., :m]
    U = np.ascontiguousarray(Ub) if m else None
    V = np.ascontiguousarray(Vb) if m else None
    offs = np.array([0, 20, T], np.int64)
    delta = np.array([777, -3], np.int64)

    got = q.copy().ravel()
    orc.relocate_patch([_chan(got, H, D, r, L, T, U, V, scale)], num_layers=L, theta=1e4,
                       offsets=offs, delta=delta, rank=m)

    x32 = (orc.fp8_to_f64(q) * scale[:, None, None, None]).astype(np.float32).ravel()
    assert np.array_equal(x32.astype(np.float64),
                          orc.fp8_to_f64(q).ravel() * np.repeat(scale, T * H * D))
    U32 = None if U is None else orc.bf16_to_f64(U).astype(np.float32)
    V32 = None if V is None else orc.bf16_to_f64(V).astype(np.float32)
    ys = np.zeros(x32.size)
    ss = np.zeros(x32.size)
    orc.relocate_patch([_chan(x32, H, D, r, L, T, U32, V32)], num_layers=L, theta=1e4,
                       offsets=offs, delta=delta, rank=m, y_out=[ys], s_out=[ss])
    y = (ys.reshape(L, -1) / scale[:, None].astype(np.float64)).ravel()
    moved = np.ones(x32.size, bool)
    if m == 0:  # only the rotated dims move; the rest keeps its codes
        moved = np.zeros((L, T, H, D), bool)
        moved[..., :r] = True
        moved = moved.ravel()
    exp = q.ravel().copy()
    # PyTorch's encoder turns overflow into NaN; the saturation is pinned on its own
    exp[moved] = _torch_encode(np.clip(y[moved], -448.0, 448.0).astype(np.float32))
    assert np.array_equal(got, exp)


def test_fp8_scale_invariance():
    # Doubling the scale and doubling U (exact in bf16) leaves every code unchanged: the
    # values double, and so does the patch.
    L, T, H, D, r, m = 2, 29, 1, 64, 64, 4
    rng = np.random.default_rng(7)
    q = _codes(rng, (L, T, H, D))
    U = orc.round_bf16(0.3 * rng.standard_normal((L, T, m)))
    V = orc.round_bf16(0.3 * rng.standard_normal((L, 1, H * D, m)))
    U2 = orc.round_bf16(2.0 * orc.bf16_to_f64(U))
    assert np.array_equal(orc.bf16_to_f64(U2), 2.0 * orc.bf16_to_f64(U))
    offs = np.array([0, T], np.int64)
    delta = np.array([12345], np.int64)
    s1 = np.array([0.01, 0.02], np.float32)
    s2 = 2 * s1
    a, b = q.copy().ravel(), q.copy().ravel()
    orc.relocate_patch([_chan(a, H, D, r, L, T, U, V, s1)], num_layers=L, theta=1e6,
                       offsets=offs, delta=delta, rank=m)
    orc.relocate_patch([_chan(b, H, D, r, L, T, U2, V, s2)], num_layers=L, theta=1e6,
                       offsets=offs, delta=delta, rank=m)
    assert np.array_equal(a, b)
    # rotation only: the scale cancels, any scale gives the same codes
    c, d = q.copy().ravel(), q.copy().ravel()
    orc.relocate_patch([_chan(c, H, D, r, L, T, scale=s1)], num_layers=L, theta=1e6,
                       offsets=offs, delta=delta)
    orc.relocate_patch([_chan(d, H, D, r, L, T, scale=np.float32([3.7, 0.11]))],
                       num_layers=L, theta=1e6, offsets=offs, delta=delta)
    assert np.array_equal(c, d)


def test_fp8_delta_zero_rank_zero_keeps_codes_and_patch_saturates():
    L, T, H, D = 1, 8, 1, 16
    rng = np.random.default_rng(9)
    q = _codes(rng, (L, T, H, D))
    a = q.copy().ravel()
    orc.relocate_patch([_chan(a, H, D, D, L, T, scale=np.float32([0.5]))], num_layers=L,
                       theta=1e4, offsets=np.array([0, T], np.int64), delta=np.array([0]))
    assert np.array_equal(a, q.ravel())
    # a patch far beyond the range pins every element at +-448
    U = orc.round_bf16(np.full((L, T, 1), 64.0))
    V = orc.round_bf16(np.concatenate([np.full((L, 1, 8, 1), 64.0),
                                       np.full((L, 1, 8, 1), -64.0)], axis=2))
    b = q.copy().ravel()
    orc.relocate_patch([_chan(b, H, D, 0, L, T, U, V, np.float32([1.0]))], num_layers=L,
                       theta=1e4, offsets=np.array([0, T], np.int64), delta=np.array([0]),
                       rank=1)
    b = b.reshape(T, D)
    assert np.all(b[:, :8] == 0x7E) and np.all(b[:, 8:] == 0xFE)


def test_fp8_recall_equals_in_place():
    L, T, H, D, r, m = 2, 33, 2, 32, 32, 8
    rng = np.random.default_rng(12)
    q = _codes(rng, (L, T, H, D))
    U = orc.round_bf16(0.3 * rng.standard_normal((L, T, m)))
    V = orc.round_bf16(0.3 * rng.standard_normal((L, 2, H * D, m)))
    sc = np.float32([0.03, 0.07])
    offs = np.array([0, 9, T], np.int64)
    delta = np.array([-40, 900], np.int64)
    ref = q.copy().ravel()
    orc.relocate_patch([_chan(ref, H, D, r, L, T, U, V, sc)], num_layers=L, theta=1e4,
                       offsets=offs, delta=delta, rank=m)
    src = q.copy().ravel()
    dst = np.zeros_like(src)
    orc.recall_patch([_chan(src, H, D, r, L, T, U, V, sc)], [_chan(dst, H, D, r, L, T)],
                     num_layers=L, theta=1e4, offsets=offs, delta=delta, rank=m)
    assert np.array_equal(dst, ref)
    assert np.array_equal(src, q.ravel())

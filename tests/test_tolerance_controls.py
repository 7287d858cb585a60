"""The parity criterion has teeth: CPU models of plausible kernel mistakes fail it, a
CPU model of a correct fp32 kernel passes it.  All models run in numpy on the CPU and
compare against the fp64 oracle with the same criterion the GPU tests use.

Workload parameters are those of the 72B-shaped long-video cache (theta 1e6,
delta +65536, rank 64), the MLA cache (theta 1e4, delta +100000) and the reorder
batch (theta 5e5, |delta| up to 32768).
"""
import numpy as np
import pytest

from oracle import oracle as orc

import parity

torch = pytest.importorskip("torch")


def to_bf16_bits(y32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def model_kernel(xb, ub, Vb, D, r, theta, delta, *, fp32_angles=False, drop_patch=False,
                 rotate_patch=False):
    """fp32 model of one token row of the operator (single head-major row, bf16 in/out)."""
    x = parity.bf16_value(xb).astype(np.float32)
    u = parity.bf16_value(ub).astype(np.float32)
    V = parity.bf16_value(Vb).astype(np.float32).reshape(-1, u.size)
    half = r // 2
    i = np.arange(half)
    if fp32_angles:
        w = np.float32(theta) ** (np.float32(-2.0) * i.astype(np.float32) / np.float32(r))
        phi = np.float32(delta) * w.astype(np.float32)
        c, s = np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)
    else:
        phi = float(delta) * theta ** (-2.0 * i / r)
        c, s = np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)
    H = x.size // D
    y = x.copy()
    p = (V @ u).astype(np.float32) if not drop_patch else np.zeros_like(x)
    if rotate_patch:
        y = y + p
        p = np.zeros_like(p)
    for h in range(H):
        a, b = y[h * D:h * D + half].copy(), y[h * D + half:h * D + r].copy()
        y[h * D:h * D + half] = a * c - b * s
        y[h * D + half:h * D + r] = b * c + a * s
    return to_bf16_bits(y + p)


def run_model(rows=600, D=128, H=8, m=64, theta=1e6, delta=65536, r=None, seed=0, **kw):
    rng = np.random.default_rng(seed)
    r = D if r is None else r
    F = H * D
    rep = parity.Report()
    sd = np.sqrt(0.1 / np.sqrt(m))
    V = orc.round_bf16(sd * rng.standard_normal(F * m))
    for _ in range(rows):
        x = orc.round_bf16(rng.standard_normal(F))
        u = orc.round_bf16(sd * rng.standard_normal(m))
        g = model_kernel(x, u, V, D, r, theta, delta, **kw)
        o = orc.row(x, H, D, r, theta, delta, u, V.reshape(F, m))
        xv, uv, Vv = (parity.bf16_value(a) for a in (x, u, V))
        y = orc.row_f64(xv, H, D, r, theta, delta, uv, Vv.reshape(F, m))
        s = orc.row_magnitude_f64(xv, H, D, r, theta, delta, uv, Vv.reshape(F, m))
        parity.compare(g, o, y, s, m, rep)
    return rep


@pytest.mark.parametrize("theta,delta,m", [(1e6, 65536, 64), (1e4, 100000, 64),
                                           (5e5, -32768, 16), (1e6, -1536, 32)])
def test_correct_fp32_model_passes(theta, delta, m):
    rep = run_model(theta=theta, delta=delta, m=m)
    assert rep.ok(), str(rep)
    assert rep.band_only <= max(2, rep.computed // 100000)


@pytest.mark.parametrize("theta,delta", [(1e6, 65536), (1e4, 100000)])
def test_fp32_angles_fail(theta, delta):
    rep = run_model(theta=theta, delta=delta, m=64, fp32_angles=True)
    assert rep.failures > 0.001 * rep.computed, str(rep)


def test_dropped_patch_fails():
    rep = run_model(rows=100, drop_patch=True)
    assert rep.failures > 0.9 * rep.computed, str(rep)


def test_rotated_patch_fails():
    rep = run_model(rows=100, rotate_patch=True)
    assert rep.failures > 0.5 * rep.computed, str(rep)


def test_patch_is_visible_at_bf16():
    # Factor variance 0.1/sqrt(m) makes each patch entry ~0.1: the patched and unpatched
    # outputs differ on nearly every element, so a kernel that skipped the patch cannot
    # pass.  (With a standard deviation of 0.1/sqrt(m) instead, the rank-64 patch would
    # be ~0.001, under half a bf16 ulp for most |x| ~ 1, and skipping it would pass.)
    rng = np.random.default_rng(1)
    for m in (4, 16, 32, 64):
        sd = np.sqrt(0.1 / np.sqrt(m))
        x = orc.round_bf16(rng.standard_normal(1024))
        u = orc.round_bf16(sd * rng.standard_normal(m))
        V = orc.round_bf16(sd * rng.standard_normal((1024, m)))
        a = orc.row(x, 8, 128, 128, 1e6, 7, u, V)
        b = orc.row(x, 8, 128, 128, 1e6, 7)
        assert np.mean(a != b) > 0.9
        sd_std = 0.1 / np.sqrt(m)
        us = orc.round_bf16(sd_std * rng.standard_normal(m))
        Vs = orc.round_bf16(sd_std * rng.standard_normal((1024, m)))
        c = orc.row(x, 8, 128, 128, 1e6, 7, us, Vs)
        if m == 64:
            assert np.mean(c != b) < 0.5

"""GPU parity of the orbit deficit (kamera_orbit_mean) and of the orbit patch.

[K] Kamera, gist.science/pt/paper/2606.23581, §3 ("Tres Operacoes de Janela Baratas",
item 1, "Reordenacao"): one patch averaged over permutations serves every order of a
cached set.  The mean is an fp64 sum in order, one fp64 division and one rounding to
bf16 on both sides, so the comparison is bit for bit (NaN compared as a class: its sign
after fp64 arithmetic is not specified).  The orbit patch is kamera_form_patch on that
mean, checked against the oracle's factors of the same mean with the patch-formation
criteria.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, synth  # noqa: E402

import parity  # noqa: E402
from test_gpu_form import _check, _w  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _random_bf16(rng, shape, special=True):
    """bf16 patterns over the whole exponent range (subnormals included), a few
    infinities and NaNs when `special`."""
    e = rng.integers(0, 255, size=shape)
    bits = (e << 7) | rng.integers(0, 128, size=shape) | (rng.integers(0, 2, size=shape) << 15)
    if special:
        flat = bits.reshape(-1)
        k = flat.size // 500 + 1
        idx = rng.choice(flat.size, size=2 * k, replace=False)
        flat[idx[:k]] = rng.choice([0x7F80, 0xFF80], size=k)
        flat[idx[k:]] = rng.choice([0x7FC0, 0x7F81, 0xFFC0, 0xFFFF], size=k)
    return bits.astype(np.uint16)


def _ties(rng, P, n):
    """Orders whose mean lands exactly on (or one fp64 step off) a bf16 tie: order 0 and
    order 1 are adjacent bf16 values of one binade, the rest repeat their mean's
    neighbours so that the sum stays exact."""
    lo = (rng.integers(1, 250, size=n) << 7) | rng.integers(0, 127, size=n)
    lo = lo | (rng.integers(0, 2, size=n) << 15)
    out = np.empty((P, n), dtype=np.uint16)
    for p in range(P):
        out[p] = lo + (p % 2)  # alternate x and its neighbour: pairs average to ties
    return out


def _compare(got, want):
    gn = (got & 0x7FFF) > 0x7F80
    wn = (want & 0x7FFF) > 0x7F80
    assert np.array_equal(gn, wn), np.flatnonzero(gn != wn)[:10]
    bad = np.flatnonzero((got != want) & ~gn)
    assert bad.size == 0, [(int(i), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("P,n,stride", [(1, 1000, 1000), (2, 4099, 4104), (3, 100003, 100008),
                                        (4, 8, 8), (5, 7, 8), (9, 65536, 65536),
                                        (16, 2048 * 1024 + 5, 2048 * 1024 + 8)])
def test_orbit_mean_bit_exact(P, n, stride):
    from oracle import patch_form as pf
    rng = np.random.default_rng(P * 1000 + n % 997)
    bits = _random_bf16(rng, (P, stride))
    if P % 2 == 0:  # ties in the first quarter
        q = n // 4
        bits[:, :q] = _ties(rng, P, q)
    print(f"\n[orbit] P={P} n={n} stride={stride}", flush=True)
    d = torch.from_numpy(bits.view(np.int16)).to(DEV)
    out = torch.full((n,), 0x5555, dtype=torch.int16, device=DEV)
    kamera.orbit_mean(d.view(torch.bfloat16), out.view(torch.bfloat16))
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = pf.orbit_mean(bits[:, :n])
    _compare(got, want)


def test_orbit_mean_large_sampled():
    # 4 orders of 64M values (a 72B-shaped layer group), checked on 200k sampled indices.
    from oracle import patch_form as pf
    P, n = 4, 64 << 20
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    d = (torch.randn((P, n), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    print(f"\n[orbit] large P={P} n={n}", flush=True)
    kamera.orbit_mean(d, out)
    torch.cuda.synchronize()
    idx = torch.randint(0, n, (200_000,), generator=g, device=DEV)
    got = out[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    want = pf.orbit_mean(d[:, idx].view(torch.int16).cpu().numpy().view(np.uint16))
    _compare(got, want)


def test_orbit_mean_empty_and_single():
    d = torch.zeros((3, 16), dtype=torch.bfloat16, device=DEV)
    out = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    kamera.orbit_mean(d, out)  # nothing to do
    x = (torch.randn((1, 1008), device=DEV)).to(torch.bfloat16)  # stride a multiple of 8
    o = torch.empty(1001, dtype=torch.bfloat16, device=DEV)
    kamera.orbit_mean(x, o)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), x[0, :1001].view(torch.int16))
    with pytest.raises(kamera.KameraError):  # stride 1001: not a multiple of 8
        kamera.orbit_mean(x[:, :1001].contiguous(), o)


def test_orbit_patch():
    # Three orders of a two-chunk, two-channel problem: a shared deficit plus an
    # order-specific part; the orbit patch is the form of their mean.
    from oracle import patch_form as pf
    w = _w(lens=(400, 200))
    base = synth.make_deficit(w, device=DEV)
    orders = [synth.make_deficit(w.with_(wid=w.wid + 1 + p), device=DEV) for p in range(3)]
    means = []
    for c in range(2):
        stack = torch.stack([(base[c].float() + 0.5 * o[c].float()).to(torch.bfloat16)
                             for o in orders])
        out = torch.empty_like(base[c])
        kamera.orbit_mean(stack, out)
        torch.cuda.synchronize()
        want = pf.orbit_mean(stack.view(torch.int16).cpu().numpy().view(np.uint16))
        _compare(out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1), want.reshape(-1))
        means.append(out)
    _check(w, 32, label="orbit patch", deficits=means)

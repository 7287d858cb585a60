"""Parity helpers: run the CPU oracle on host copies of a problem and compare a GPU
result with it element by element.

Acceptance for bf16 output (the operator is defined to round once to bf16; the
Kamera summary, §3 production deployment, states the rebuilt KV is reproduced
within bf16 rounding):
  - elements the call must not touch: bit-identical;
  - every other element: at most 1 bf16 ulp (ordinal distance) from the oracle's
    rounded value, or, near cancellation, |g - y| <= ulp_bf16(y) + (m + 4) 2^-23 S,
    where y is the oracle's unrounded fp64 value and S the sum of |terms| that
    make it.  fp32 evaluation of the same terms in any order is off by at most
    about (m + 3) 2^-24 S, so when |y| is far below S that bound, not the ulp of
    y, limits any fp32 kernel.
Acceptance for fp32 output: |g - y| <= 1e-5 max(|y|, S).
NaN matches NaN.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def host_bits(t) -> np.ndarray:
    """torch tensor -> flat numpy storage view (uint16 bf16 bits or float32)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16).ravel().copy()
    return t.detach().cpu().numpy().ravel().copy()


def bf16_ordinal(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


@dataclass
class Report:
    elements: int = 0
    computed: int = 0
    bit_equal: int = 0
    within_1ulp: int = 0
    band_only: int = 0
    failures: int = 0
    untouched_changed: int = 0
    max_ulp: int = 0
    max_rel: float = 0.0

    def ok(self) -> bool:
        return self.failures == 0 and self.untouched_changed == 0

    def __str__(self) -> str:
        return (f"elements={self.elements} computed={self.computed} bit_equal={self.bit_equal} "
                f"1ulp={self.within_1ulp} band_only={self.band_only} failures={self.failures} "
                f"untouched_changed={self.untouched_changed} max_ulp={self.max_ulp} "
                f"max_rel={self.max_rel:.3g}")


def compare(g: np.ndarray, o: np.ndarray, y: np.ndarray, s: np.ndarray, rank: int,
            report: Report | None = None) -> Report:
    """g: GPU storage, o: oracle storage, y: unrounded oracle values, s: magnitude sums
    (s < 0 marks elements the call must leave untouched)."""
    rep = report or Report()
    rep.elements += g.size
    touched = s >= 0
    rep.computed += int(touched.sum())
    if g.dtype == np.uint16:
        eq = g == o
        gv = bf16_value(g)
        nan_g, nan_o = np.isnan(gv), np.isnan(bf16_value(o))
        eq |= nan_g & nan_o
        rep.untouched_changed += int((~eq & ~touched).sum())
        rep.bit_equal += int((eq & touched).sum())
        idx = np.nonzero(~eq & touched)[0]
        if idx.size:
            d = np.abs(bf16_ordinal(g[idx]) - bf16_ordinal(o[idx]))
            near = (d <= 1) & ~nan_g[idx] & ~nan_o[idx]
            rep.within_1ulp += int(near.sum())
            rep.max_ulp = max(rep.max_ulp, int(d.max()))
            rest = idx[~near]
            if rest.size:
                tol = bf16_ulp(y[rest]) + (rank + 4) * 2.0 ** -23 * s[rest]
                band = np.abs(gv[rest] - y[rest]) <= tol
                rep.band_only += int(band.sum())
                rep.failures += int((~band).sum())
    else:
        gv, ov = g.astype(np.float64), o.astype(np.float64)
        eq = (g.view(np.uint32) == o.view(np.uint32)) | (np.isnan(gv) & np.isnan(ov))
        rep.untouched_changed += int((~eq & ~touched).sum())
        rep.bit_equal += int((eq & touched).sum())
        idx = np.nonzero(~eq & touched)[0]
        if idx.size:
            err = np.abs(gv[idx] - y[idx])
            scale = np.maximum(np.abs(y[idx]), s[idx])
            rel = np.where(scale > 0, err / np.where(scale > 0, scale, 1), err)
            rep.max_rel = max(rep.max_rel, float(np.nan_to_num(rel, nan=np.inf).max()))
            okm = rel <= 1e-5
            rep.within_1ulp += int(okm.sum())
            rep.failures += int((~okm).sum())
    return rep


def oracle_on_host(inp, before: list, factors: tuple | None = None):
    """Run the oracle on host copies `before` (flat storage arrays, one per buffer);
    returns (out, y, s) lists shaped like `before`."""
    from oracle import oracle as orc
    w = inp.workload
    out = [b.copy() for b in before]
    if before[0].dtype == np.uint16:
        y = [bf16_value(b) for b in before]
    else:
        y = [b.astype(np.float64) for b in before]
    s = [np.full(b.size, -1.0) for b in before]
    if factors is None:
        factors = ([host_bits(u) for u in inp.U], [host_bits(v) for v in inp.V])
    chans = []
    for c, lay in enumerate(inp.layouts):
        d = dict(lay)
        d["data"] = out[lay["buffer"]]
        if inp.rank > 0:
            d["U"], d["V"] = factors[0][c], factors[1][c]
        chans.append(d)
    orc.relocate_patch(chans, num_layers=w.layers, theta=w.theta, offsets=inp.struct.offsets,
                       delta=inp.struct.delta, rank=inp.rank, page_size=w.page_size,
                       block_table=inp.struct.block_table,
                       y_out=[y[lay["buffer"]] for lay in inp.layouts],
                       s_out=[s[lay["buffer"]] for lay in inp.layouts])
    return out, y, s


def check_problem(inp, run, flags: int = 0) -> Report:
    """Copy inputs to host, run `run(inp)` on the GPU, compare with the oracle."""
    import torch
    before = [host_bits(b) for b in inp.buffers]
    factors = ([host_bits(u) for u in inp.U], [host_bits(v) for v in inp.V])
    run(inp)
    torch.cuda.synchronize()
    after = [host_bits(b) for b in inp.buffers]
    out, y, s = oracle_on_host(inp, before, factors)
    rep = Report()
    for g, o, yy, ss in zip(after, out, y, s):
        compare(g, o, yy, ss, inp.rank, rep)
    return rep

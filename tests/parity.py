"""Parity helpers: run the CPU oracle on host copies of a problem and compare a GPU
result with it element by element.

Acceptance for bf16 output (the operator is defined to round once to bf16; the
Kamera summary, §3 production deployment, states the rebuilt KV is reproduced
within bf16 rounding):
  - elements the call must not touch: bit-identical;
  - every other element: at most 1 bf16 ulp (ordinal distance) from the oracle's
    rounded value, or, near cancellation (|y| < 2^-16 S), |g - y| <= ulp_bf16(g) +
    (m + 3) 2^-23 S, where y is the oracle's unrounded fp64 value and S the sum of
    |terms| that make it.  fp32 evaluation of the same terms in any order is off by
    at most about (m + 3) 2^-24 S (the rounded cos and sin, the partner product, the
    fused multiply-add and m accumulations), so where |y| is far below S that bound,
    not the ulp of y, limits any fp32 kernel.
Acceptance for fp8 E4M3 output: the same two tests on the E4M3 grid, in code units
(y and S divided by the layer's scale): at most 1 code (ordinal distance) from the
oracle's code, or (|y| < 2^-16 S) |g - y| <= ulp_fp8(g) + (m + 4) 2^-23 S.  The
kernel forms (s x' + patch) / s in fp32: two more fp32 roundings than bf16 (the scale
and its reciprocal), hence m + 4.
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
    with np.errstate(invalid="ignore"):  # signalling NaN patterns widen quietly
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def fp8_ordinal(codes: np.ndarray) -> np.ndarray:
    b = codes.astype(np.int64)
    mag = b & 0x7F
    return np.where(b & 0x80, -mag, mag)


def fp8_value(codes: np.ndarray) -> np.ndarray:
    from oracle import oracle as orc
    return orc.fp8_to_f64(codes)


def fp8_ulp(y: np.ndarray) -> np.ndarray:
    """Spacing of E4M3 codes around y: 2^(e - 3) for normal |y| >= 2^-6, else 2^-9."""
    a = np.abs(y)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.exp2(e - 3)


def storage_value(bits: np.ndarray) -> np.ndarray:
    """Storage array -> fp64 values (fp8: code values, before the scale)."""
    if bits.dtype == np.uint16:
        return bf16_value(bits)
    if bits.dtype == np.uint8:
        return fp8_value(bits)
    return bits.astype(np.float64)


@dataclass
class Report:
    elements: int = 0
    computed: int = 0
    bit_equal: int = 0
    within_1ulp: int = 0
    band_only: int = 0          # pass only through the cancellation band
    band_gated_out: int = 0     # inside the band's bound but |y| >= 2^-16 S (failures)
    failures: int = 0
    untouched_changed: int = 0
    max_ulp: int = 0
    max_rel: float = 0.0

    def ok(self) -> bool:
        return self.failures == 0 and self.untouched_changed == 0

    def __str__(self) -> str:
        return (f"elements={self.elements} computed={self.computed} bit_equal={self.bit_equal} "
                f"1ulp={self.within_1ulp} band_only={self.band_only} "
                f"band_gated_out={self.band_gated_out} failures={self.failures} "
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
    if g.dtype in (np.uint16, np.uint8):
        q8 = g.dtype == np.uint8
        ordinal, value, ulp = ((fp8_ordinal, fp8_value, fp8_ulp) if q8
                               else (bf16_ordinal, bf16_value, bf16_ulp))
        eq = g == o
        gv = value(g)
        nan_g, nan_o = np.isnan(gv), np.isnan(value(o))
        eq |= nan_g & nan_o
        rep.untouched_changed += int((~eq & ~touched).sum())
        rep.bit_equal += int((eq & touched).sum())
        idx = np.nonzero(~eq & touched)[0]
        if idx.size:
            d = np.abs(ordinal(g[idx]) - ordinal(o[idx]))
            near = (d <= 1) & ~nan_g[idx] & ~nan_o[idx]
            rep.within_1ulp += int(near.sum())
            rep.max_ulp = max(rep.max_ulp, int(d.max()))
            rest = idx[~near]
            if rest.size:
                # near cancellation only (R11): |y| < 2^-16 S
                tol = ulp(gv[rest]) + (rank + (4 if q8 else 3)) * 2.0 ** -23 * s[rest]
                within = np.abs(gv[rest] - y[rest]) <= tol
                gate = np.abs(y[rest]) < 2.0 ** -16 * s[rest]
                band = within & gate
                rep.band_only += int(band.sum())
                rep.band_gated_out += int((within & ~gate).sum())
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
    y = [storage_value(b) for b in before]
    s = [np.full(b.size, -1.0) for b in before]
    if factors is None:
        factors = ([host_bits(u) for u in inp.U], [host_bits(v) for v in inp.V])
    chans = []
    for c, lay in enumerate(inp.layouts):
        d = dict(lay)
        d["data"] = out[lay["buffer"]]
        if inp.rank > 0:
            d["U"], d["V"] = factors[0][c], factors[1][c]
        if inp.scales:
            d["scale"] = host_bits(inp.scales[c])
        chans.append(d)
    orc.relocate_patch(chans, num_layers=w.layers, theta=w.theta, offsets=inp.struct.offsets,
                       delta=inp.struct.delta, rank=inp.rank, page_size=w.page_size,
                       block_table=inp.struct.block_table, pairing=w.pairing,
                       sections=w.sections,
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


def _element_index(inp, c, layer, t, h):
    """Flat element index of (layer, token t, head h, dim 0) of channel c in its buffer,
    from the oracle's addressing."""
    from oracle import oracle as orc
    lay = inp.layouts[c]
    w = inp.workload
    return int(lay.get("offset", 0)) + orc.row_offset(lay, w.page_size, inp.struct.block_table,
                                                      layer, t, h)


def sample_rows(inp, n, seed=0):
    """(layer, token) pairs: random ones plus the first and last tokens, chunk edges and
    the last layer."""
    rng = np.random.default_rng(seed)
    w, st = inp.workload, inp.struct
    T, L = st.total_tokens, w.layers
    rows = {(0, 0), (L - 1, T - 1), (L - 1, 0), (0, T - 1)}
    for j in range(min(st.num_chunks, 16)):
        a, b = int(st.offsets[j]), int(st.offsets[j + 1])
        if b > a:
            rows.add((int(rng.integers(L)), a))
            rows.add((int(rng.integers(L)), b - 1))
    while len(rows) < n:
        rows.add((int(rng.integers(L)), int(rng.integers(T))))
    return sorted(rows)


def sampled_check(inp, run, n=1024, seed=0) -> Report:
    """Run `run(inp)` at full size and check sampled rows of every computed channel
    against the oracle, row by row."""
    import torch
    from oracle import oracle as orc
    w, st = inp.workload, inp.struct
    rows = sample_rows(inp, n, seed)
    chans = [c for c, lay in enumerate(inp.layouts) if inp.rank > 0 or lay["rope_dim"] > 0]
    idx = {}
    for c in chans:
        lay = inp.layouts[c]
        D, H = lay["dim"], lay["heads"]
        ii = np.empty((len(rows), H * D), dtype=np.int64)
        for k, (l, t) in enumerate(rows):
            for h in range(H):
                ii[k, h * D:(h + 1) * D] = _element_index(inp, c, l, t, h) + np.arange(D)
        idx[c] = ii

    def gather(c):
        buf = inp.buffers[inp.layouts[c]["buffer"]].view(-1)
        g = buf[torch.as_tensor(idx[c].ravel(), device=buf.device)].view(len(rows), -1)
        return host_bits(g).reshape(len(rows), -1)

    before = {c: gather(c) for c in chans}
    us, vs = {}, {}
    if inp.rank > 0:
        li = torch.as_tensor([l for l, _ in rows], device=inp.U[0].device)
        ti = torch.as_tensor([t for _, t in rows], device=inp.U[0].device)
        for c in chans:
            us[c] = host_bits(inp.U[c][li, ti]).reshape(len(rows), -1)
            vs[c] = host_bits(inp.V[c]).reshape(w.layers, st.num_chunks, -1, inp.rank)
    scales = {c: host_bits(inp.scales[c]) for c in chans} if inp.scales else {}
    run(inp)
    torch.cuda.synchronize()
    after = {c: gather(c) for c in chans}
    rep = Report()
    for c in chans:
        lay = inp.layouts[c]
        for k, (l, t) in enumerate(rows):
            j = int(np.searchsorted(st.offsets, t, side="right") - 1)
            compare(after[c][k], *_row_expect(w, lay, st.delta[j], before[c][k],
                                              us[c][k] if inp.rank > 0 else None,
                                              vs[c][l, j] if inp.rank > 0 else None,
                                              float(scales[c][l]) if scales else 1.0),
                    inp.rank, rep)
    return rep


def moved_dims(lay, d, pairing=0, sections=()) -> np.ndarray:
    """Elements of one row that the rotation moves (rank 0): rotated dims of pairs
    whose (section) delta is nonzero."""
    H, D, r = lay["heads"], lay["dim"], lay["rope_dim"]
    d = np.atleast_1d(np.asarray(d, dtype=np.int64))
    half = r // 2
    pair_sec = (np.repeat(np.arange(len(sections)), sections) if len(sections) > 1
                else np.zeros(half, np.int64))
    moves = d[pair_sec] != 0 if half else np.zeros(0, bool)
    head = np.zeros(D, bool)
    for i in range(half):
        a, b = (2 * i, 2 * i + 1) if pairing == 1 else (i, i + half)
        head[a] = head[b] = moves[i]
    return np.tile(head, H)


def _row_expect(w, lay, d, x, u, V, scale=1.0):
    """(oracle storage, fp64 value, magnitude or -1 where bits must match) of one row;
    fp8 rows (values scale * code) give value and magnitude in code units."""
    from oracle import oracle as orc
    kw = dict(pairing=w.pairing, sections=w.sections)
    o = orc.row(x, lay["heads"], lay["dim"], lay["rope_dim"], w.theta, d, u, V, scale=scale,
                **kw)
    xf = storage_value(x) * scale
    uf = None if u is None else bf16_value(u)
    Vf = None if V is None else bf16_value(V)
    y = orc.row_f64(xf, lay["heads"], lay["dim"], lay["rope_dim"], w.theta, d, uf, Vf,
                    **kw) / scale
    s = orc.row_magnitude_f64(xf, lay["heads"], lay["dim"], lay["rope_dim"], w.theta, d, uf,
                              Vf, **kw) / scale
    if u is None:  # rank 0: only moved dims are computed
        s = np.where(moved_dims(lay, d, w.pairing, w.sections), s, -1.0)
    return o, y, s


# ----------------------------------------------------------------- recall (out of place)

def _dicts(layouts, bufs, factors=None, rank=0, scales=()):
    out = []
    for c, lay in enumerate(layouts):
        d = dict(lay)
        d["data"] = bufs[lay["buffer"]]
        if factors is not None and rank > 0:
            d["U"], d["V"] = factors[0][c], factors[1][c]
        if scales:
            d["scale"] = host_bits(scales[c])
        out.append(d)
    return out


def check_recall(rinp, run) -> tuple:
    """Run the recall `run(rinp)` on the GPU and compare the whole destination with the
    oracle's recall (and the source with its state before).  Returns (report, src_ok)."""
    import torch
    from oracle import oracle as orc
    src = rinp.src
    w = rinp.workload
    s_before = [host_bits(b) for b in src.buffers]
    d_before = [host_bits(b) for b in rinp.dst_buffers]
    factors = ([host_bits(u) for u in src.U], [host_bits(v) for v in src.V])
    run(rinp)
    torch.cuda.synchronize()
    s_after = [host_bits(b) for b in src.buffers]
    d_after = [host_bits(b) for b in rinp.dst_buffers]
    out = [b.copy() for b in d_before]
    y = [storage_value(b) for b in d_before]
    s = [np.full(b.size, -1.0) for b in d_before]
    orc.recall_patch(_dicts(src.layouts, [b.copy() for b in s_before], factors, src.rank,
                            src.scales),
                     _dicts(rinp.dst_layouts, out), num_layers=w.layers, theta=w.theta,
                     offsets=src.struct.offsets, delta=src.struct.delta, rank=src.rank,
                     src_page_size=w.page_size, src_block_table=src.struct.block_table,
                     dst_page_size=rinp.dst_page_size, dst_block_table=rinp.dst_block_table,
                     pairing=w.pairing, sections=w.sections,
                     y_out=[y[lay["buffer"]] for lay in rinp.dst_layouts],
                     s_out=[s[lay["buffer"]] for lay in rinp.dst_layouts])
    rep = Report()
    for g, o, yy, ss in zip(d_after, out, y, s):
        compare(g, o, yy, ss, src.rank, rep)
    src_ok = all(np.array_equal(a, b) for a, b in zip(s_after, s_before))
    return rep, src_ok


def sampled_check_recall(rinp, run, n=1024, seed=0) -> Report:
    """Run a full-size recall and check sampled destination rows against the oracle's
    row function applied to the source rows."""
    import torch
    from oracle import oracle as orc
    src = rinp.src
    w, st = src.workload, src.struct
    rows = sample_rows(src, n, seed)

    def idx_for(layouts, page_size, table, c):
        lay = layouts[c]
        D, H = lay["dim"], lay["heads"]
        ii = np.empty((len(rows), H * D), dtype=np.int64)
        for k, (l, t) in enumerate(rows):
            for h in range(H):
                ii[k, h * D:(h + 1) * D] = (int(lay.get("offset", 0)) +
                                            orc.row_offset(lay, page_size, table, l, t, h) +
                                            np.arange(D))
        return ii

    def gather(bufs, layouts, ii, c):
        buf = bufs[layouts[c]["buffer"]].view(-1)
        g = buf[torch.as_tensor(ii.ravel(), device=buf.device)].view(len(rows), -1)
        return host_bits(g).reshape(len(rows), -1)

    chans = range(len(src.layouts))
    sidx = {c: idx_for(src.layouts, w.page_size, st.block_table, c) for c in chans}
    didx = {c: idx_for(rinp.dst_layouts, rinp.dst_page_size, rinp.dst_block_table, c)
            for c in chans}
    before = {c: gather(src.buffers, src.layouts, sidx[c], c) for c in chans}
    us, vs = {}, {}
    if src.rank > 0:
        li = torch.as_tensor([l for l, _ in rows], device=src.U[0].device)
        ti = torch.as_tensor([t for _, t in rows], device=src.U[0].device)
        for c in chans:
            us[c] = host_bits(src.U[c][li, ti]).reshape(len(rows), -1)
            vs[c] = host_bits(src.V[c]).reshape(w.layers, st.num_chunks, -1, src.rank)
    scales = {c: host_bits(src.scales[c]) for c in chans} if src.scales else {}
    run(rinp)
    torch.cuda.synchronize()
    rep = Report()
    for c in chans:
        lay = src.layouts[c]
        got = gather(rinp.dst_buffers, rinp.dst_layouts, didx[c], c)
        src_after = gather(src.buffers, src.layouts, sidx[c], c)
        assert np.array_equal(src_after, before[c]), "recall wrote its source"
        for k, (l, t) in enumerate(rows):
            j = int(np.searchsorted(st.offsets, t, side="right") - 1)
            compare(got[k], *_row_expect(w, lay, st.delta[j], before[c][k],
                                         us[c][k] if src.rank > 0 else None,
                                         vs[c][l, j] if src.rank > 0 else None,
                                         float(scales[c][l]) if scales else 1.0),
                    src.rank, rep)
    return rep


# ----------------------------------------------------------------- relocate-on-read attention

@dataclass
class AttendReport:
    elements: int = 0
    failures: int = 0
    lse_failures: int = 0
    max_err: float = 0.0     # max |g - y| / tol
    max_rel: float = 0.0     # max |g - y| / mag

    def ok(self) -> bool:
        return self.failures == 0 and self.lse_failures == 0

    def __str__(self) -> str:
        return (f"elements={self.elements} failures={self.failures} "
                f"lse_failures={self.lse_failures} max_err/tol={self.max_err:.3g} "
                f"max_err/mag={self.max_rel:.3g}")


def _channel_rows(inp, c, layer):
    """Values [T][heads * dim] of channel c at one layer, through its layout."""
    lay = inp.layouts[c]
    w, st = inp.workload, inp.struct
    T = st.total_tokens
    t = np.arange(T)
    if w.page_size > 0:
        slot = (st.block_table[t // w.page_size].astype(np.int64) * lay["page_stride"] +
                (t % w.page_size) * lay["slot_stride"])
    else:
        slot = t * lay["slot_stride"]
    H, D = lay["heads"], lay["dim"]
    cols = (np.arange(H)[:, None] * lay["head_stride"] + np.arange(D)[None, :]).ravel()
    idx = lay.get("offset", 0) + layer * lay["layer_stride"] + slot[:, None] + cols[None, :]
    vals = storage_value(host_bits(inp.buffers[lay["buffer"]]))
    return vals[idx]


def attend_bounds(inp, q, scale):
    """Bound sm[l][h] on the summed magnitudes of the terms of any score, for an fp32
    evaluation of the re-associated attention: sm = scale * max_t (sum_d (|q_d| +
    |q_partner(d)|) |K_t,d| + sum_k |u_t,k| sum_d |q_d| |V_K[d][k]|), where the rotated
    query's components are bounded by |q_d| + |q of d's rotary partner|."""
    w, st = inp.workload, inp.struct
    L, Hq, D = q.shape
    H = w.heads
    G = Hq // H
    m = inp.rank
    qa = np.abs(q.astype(np.float64))
    r = inp.layouts[0]["rope_dim"]
    qb = qa.copy()
    if r:
        half = r // 2
        if w.pairing == 1:
            qb[..., :r] += qa[..., :r].reshape(L, Hq, half, 2)[..., ::-1].reshape(L, Hq, r)
        else:
            qb[..., :half] += qa[..., half:r]
            qb[..., half:r] += qa[..., :half]
    sm = np.zeros((L, Hq))
    T = st.total_tokens
    if T == 0:
        return sm
    j_of_t = np.searchsorted(st.offsets, np.arange(T), side="right") - 1
    U0 = V0 = None
    if m > 0:
        U0 = np.abs(bf16_value(host_bits(inp.U[0]))).reshape(L, T, m)
        V0 = np.abs(bf16_value(host_bits(inp.V[0]))).reshape(L, st.num_chunks, H, D, m)
    ks = host_bits(inp.scales[0]).astype(np.float64) if inp.scales else None
    for l in range(L):
        rows = np.abs(_channel_rows(inp, 0, l)).reshape(T, H, D)
        if ks is not None:  # fp8: values are scale * code
            rows = rows * abs(ks[l])
        for h in range(Hq):
            g = h // G
            s = rows[:, g, :] @ qb[l, h]
            if m > 0:
                wv = np.einsum("d,jdk->jk", qa[l, h], V0[l, :, g])  # [chunks][m]
                s = s + (U0[l] * wv[j_of_t]).sum(axis=1)
            sm[l, h] = s.max()
    return sm * abs(scale)


def check_attend(inp, q, scale, run) -> AttendReport:
    """Run `run(inp, q, scale)` -> (out, lse) on the GPU and compare with the oracle's
    attention element by element, within attend_tolerance."""
    import torch
    from oracle import oracle as orc
    w = inp.workload
    bufs = [host_bits(b) for b in inp.buffers]
    chans = _dicts(inp.layouts, [b.copy() for b in bufs],
                   ([host_bits(u) for u in inp.U], [host_bits(v) for v in inp.V]), inp.rank,
                   inp.scales)
    qh = q.detach().cpu().numpy().astype(np.float64)
    out, lse = run(inp, q, scale)
    if out.is_cuda:
        torch.cuda.synchronize()
    g = out.detach().cpu().numpy().astype(np.float64)
    gl = lse.detach().cpu().numpy().astype(np.float64)
    y, yl, mag = orc.attend(chans, num_layers=w.layers, theta=w.theta, offsets=inp.struct.offsets,
                            delta=inp.struct.delta, q=qh, scale=scale, rank=inp.rank,
                            page_size=w.page_size, block_table=inp.struct.block_table,
                            pairing=w.pairing, sections=w.sections, with_mag=True)
    # A score's fp32 error is below (D + m + 8) 2^-24 sm; each weight's relative error is
    # below twice that (numerator and normaliser), and the sums over T tokens and m
    # patch terms add (T + m + 32) 2^-24 relative, all scaling mag = sum_t p_t |V'_t|.
    # lse carries the score error plus the normaliser's summation error.
    eps = 2.0 ** -24
    D, m, T = q.shape[2], inp.rank, inp.struct.total_tokens
    sm = attend_bounds(inp, qh, scale)
    ds = (D + m + 8) * eps * sm
    rel = 2 * ds + (T + m + 32) * eps
    tol = rel[..., None] * mag + 1e-30
    err = np.abs(g - y)
    rep = AttendReport(elements=int(g.size))
    rep.failures = int((~(err <= tol)).sum())
    rep.max_err = float(np.nan_to_num(err / tol, nan=np.inf).max()) if g.size else 0.0
    rep.max_rel = float(np.nan_to_num(err / np.maximum(mag, 1e-30), nan=np.inf).max()) if g.size else 0.0
    finite = np.isfinite(yl)
    lse_tol = 2 * ds + (T + 32) * eps + 1e-6
    rep.lse_failures = int((finite & ~(np.abs(gl - yl) <= lse_tol)).sum() +
                           (~finite & ~(gl == yl)).sum())
    return rep


def layer_slice(inp, layer):
    """A one-layer view of a synth.Inputs (same chunks, layout and table), on the same
    device: buffers, factors and workload cut to `layer`."""
    from rope_relocation_rank_amd import synth
    w = inp.workload.with_(layers=1)
    sub = synth.Inputs(w, inp.rank, inp.struct, inp.pool_pages,
                       [b[layer:layer + 1].contiguous() for b in inp.buffers], inp.layouts,
                       [u[layer:layer + 1].contiguous() for u in inp.U],
                       [v[layer:layer + 1].contiguous() for v in inp.V],
                       inp.offsets_t, inp.delta_t, inp.block_table_t,
                       scales=[s[layer:layer + 1].contiguous() for s in inp.scales])
    return sub

"""The attention parity criterion has teeth (CPU).

A plain fp32 numpy model of the re-associated attention (rotated query, V_K^T q, the V_V
term applied to the weighted U_V sum) must pass parity.check_attend against the fp64
oracle; the same model with a planted mistake (patch dropped, query rotated the wrong
way, scale applied twice) must fail it.
"""
import numpy as np
import pytest
import torch

import parity
from rope_relocation_rank_amd import synth


def _model(inp, q, scale, mistake=None):
    """fp32 re-associated attention over a synth.Inputs on the CPU."""
    w, st = inp.workload, inp.struct
    L, Hq, D = q.shape
    H = w.heads
    G = Hq // H
    m = inp.rank if mistake != "no_patch" else 0
    r = inp.layouts[0]["rope_dim"]
    half = r // 2
    T = st.total_tokens
    qn = q.numpy().astype(np.float32)
    out = np.zeros((L, Hq, D), np.float32)
    lse = np.zeros((L, Hq), np.float32)
    j_of_t = np.searchsorted(st.offsets, np.arange(T), side="right") - 1
    omega = w.theta ** (-2.0 * np.arange(half) / r) if r else np.zeros(0)
    for l in range(L):
        Kr = parity._channel_rows(inp, 0, l).astype(np.float32).reshape(T, H, D)
        Vr = parity._channel_rows(inp, 1, l).astype(np.float32).reshape(T, H, D)
        if m:
            U0 = parity.bf16_value(parity.host_bits(inp.U[0])).astype(np.float32).reshape(L, T, m)[l]
            U1 = parity.bf16_value(parity.host_bits(inp.U[1])).astype(np.float32).reshape(L, T, m)[l]
            VK = parity.bf16_value(parity.host_bits(inp.V[0])).astype(np.float32).reshape(
                L, st.num_chunks, H, D, m)[l]
            VV = parity.bf16_value(parity.host_bits(inp.V[1])).astype(np.float32).reshape(
                L, st.num_chunks, H, D, m)[l]
        for h in range(Hq):
            g = h // G
            s = np.zeros(T, np.float32)
            for j in range(st.num_chunks):
                sel = j_of_t == j
                if not sel.any():
                    continue
                qt = qn[l, h].copy()
                dl = int(st.delta[j])
                sign = 1.0 if mistake == "wrong_way" else -1.0
                if r and dl:
                    phi = sign * dl * omega
                    c, sn = np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)
                    a, b = qn[l, h, :half], qn[l, h, half:r]
                    qt[:half] = a * c - b * sn
                    qt[half:r] = b * c + a * sn
                sc = scale * (1.0 if mistake != "double_scale" else scale)
                s[sel] = (Kr[sel, g] @ qt) * np.float32(sc)
                if m:
                    wv = (qn[l, h] @ VK[j, g]) * np.float32(sc)
                    s[sel] += U0[sel] @ wv
            M = s.max()
            p = np.exp(s - M)
            den = p.sum()
            o = p @ Vr[:, g]
            if m:
                for j in range(st.num_chunks):
                    sel = j_of_t == j
                    if sel.any():
                        o = o + VV[j, g] @ (p[sel] @ U1[sel])
            out[l, h] = o / den
            lse[l, h] = M + np.log(den)
    return torch.from_numpy(out), torch.from_numpy(lse)


def _inputs(rank):
    w = synth.get("qwen25vl7b_segment").with_(layers=2, tokens=300, n_chunks=2, lens=(120, 180),
                                              deltas=(-1536, 777))
    inp = synth.make_inputs(w, rank)
    q = synth.make_query(w)
    return inp, q


@pytest.mark.parametrize("rank", [0, 32])
def test_fp32_model_passes(rank):
    inp, q = _inputs(rank)
    rep = parity.check_attend(inp, q, 128 ** -0.5, lambda i, qq, sc: _model(i, qq, sc))
    assert rep.ok(), str(rep)


@pytest.mark.parametrize("mistake", ["no_patch", "wrong_way", "double_scale"])
def test_planted_mistakes_fail(mistake):
    inp, q = _inputs(32)
    rep = parity.check_attend(inp, q, 128 ** -0.5,
                              lambda i, qq, sc: _model(i, qq, sc, mistake=mistake))
    assert rep.failures > rep.elements // 10, str(rep)

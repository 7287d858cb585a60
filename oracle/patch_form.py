"""Patch formation oracle: the top-m factors of the reuse deficit, by exact SVD.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this module; it shares no code with the
GPU library.

[K] "Kamera: KV Cache Multimodal Unificado e Invariante a Posicao para Reuso sem
Treinamento", gist.science/pt/paper/2606.23581, §2 ("Aplicacao de Patch"): the patch
is computed once, from one conditioned forward pass over [A, B], followed by an SVD
that keeps the top-m factors.  The deficit is Delta = KV(B|A) - KV(B|empty) (§1), one
[T_j, F] matrix per layer, channel and chunk; §3 reports its energy concentrated in
about 32 feature directions.  The forward pass is not part of this operator: Delta is
an input.

Reading (stated, not printed on the pages): Sigma is folded into the token factor,
U_m = U[:, :m] diag(s[:m]) and V_m = V[:, :m], so that U_m V_m^T is the best rank-m
approximation of Delta (Eckart-Young) and the reuse operator adds exactly that product.
numpy's LAPACK SVD in fp64 is the library step.

[K] §3, "Tres Operacoes de Janela Baratas", item 1 ("Reordenacao"): one orbit patch,
averaged over permutations, serves every order of a cached set.  Reading (stated, not
printed on the pages): the caller supplies the deficit of the chunk under each of P
orders of the set (each measured in the chunk's canonical frame), the orbit deficit is
their mean, rounded once to bf16 (the deficits' own type) so that it enters patch
formation like any deficit, and the orbit patch is its top-m factorization.  The
factorization of the exact mean is the rank-m P that minimizes the summed squared error
over the orbit, sum_p ||Delta_p - P||^2 = sum_p ||Delta_p - mean||^2 + P ||mean - P||^2.
"""
from __future__ import annotations

import numpy as np

from . import oracle as _orc


def top_m_factors(delta: np.ndarray, m: int):
    """Delta [T, F] (any float dtype) -> (U_m [T, m], V_m [F, m], s [min(T, F)]) in fp64.
    Columns past min(T, F) are zero."""
    d = np.asarray(delta, dtype=np.float64)
    T, F = d.shape
    U, s, Vt = np.linalg.svd(d, full_matrices=False)
    k = min(m, s.size)
    Um = np.zeros((T, m))
    Vm = np.zeros((F, m))
    Um[:, :k] = U[:, :k] * s[:k]
    Vm[:, :k] = Vt[:k].T
    return Um, Vm, s


def form_patch(delta, offsets, m: int):
    """Delta [L][T][F] with chunks [offsets[j], offsets[j+1]) -> U [L][T][m], V [L][n][F][m]
    and the singular values s [L][n][min(T_j, F)] (lists per chunk)."""
    d = np.asarray(delta, dtype=np.float64)
    L, T, F = d.shape
    n = len(offsets) - 1
    U = np.zeros((L, T, m))
    V = np.zeros((L, n, F, m))
    S = [[None] * n for _ in range(L)]
    for l in range(L):
        for j in range(n):
            a, b = int(offsets[j]), int(offsets[j + 1])
            if b == a:
                S[l][j] = np.zeros(0)
                continue
            Uj, Vj, s = top_m_factors(d[l, a:b], m)
            U[l, a:b] = Uj
            V[l, j] = Vj
            S[l][j] = s
    return U, V, S


def orbit_mean(deltas) -> np.ndarray:
    """Deficits [P][...] as bf16 bit patterns -> their mean as bf16 bits: the fp64 sum in
    order p = 0 .. P-1, divided by P in fp64, rounded once to bf16 (ties to even)."""
    d = np.asarray(deltas, dtype=np.uint16)
    acc = np.zeros(d.shape[1:], dtype=np.float64)
    for p in range(d.shape[0]):
        acc = acc + _orc.bf16_to_f64(d[p])
    return _orc.round_bf16(acc / d.shape[0])


def orbit_patch(deltas, offsets, m: int):
    """The orbit patch: form_patch of the rounded mean deficit (deltas [P][L][T][F] bf16
    bits)."""
    return form_patch(_orc.bf16_to_f64(orbit_mean(deltas)), offsets, m)

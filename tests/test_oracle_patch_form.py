"""Pins of the patch-formation oracle (top-m SVD factors of the deficit).

[K] Kamera, gist.science/pt/paper/2606.23581, §2 ("Aplicacao de Patch"): SVD, top-m
factors.  Pinned to Eckart-Young (no rank-m matrix is closer to Delta in Frobenius norm;
the optimum's error is the root of the dropped squared singular values), to closed forms
on hand-built matrices, and to brute force on a tiny case.
"""
import numpy as np

from oracle import patch_form as pf


def test_closed_form_rank_one_and_diagonal():
    # Delta = a b^T: the rank-1 patch is Delta itself; U_1 = |a||b| a_hat, V_1 = b_hat.
    a = np.array([3.0, 0.0, 4.0])
    b = np.array([0.0, 2.0, 0.0, 0.0])
    U, V, s = pf.top_m_factors(np.outer(a, b), 1)
    np.testing.assert_allclose(s[0], 10.0)
    np.testing.assert_allclose(U @ V.T, np.outer(a, b), atol=1e-12)
    np.testing.assert_allclose(abs(V[:, 0]), [0, 1, 0, 0], atol=1e-12)
    # Diagonal: singular values are the sorted magnitudes, factors the axes.
    D = np.diag([1.0, -7.0, 3.0])
    U, V, s = pf.top_m_factors(D, 2)
    np.testing.assert_allclose(s, [7, 3, 1])
    np.testing.assert_allclose(U @ V.T, np.diag([0.0, -7.0, 3.0]), atol=1e-12)


def test_eckart_young_error_and_optimality():
    rng = np.random.default_rng(1)
    T, F, m = 40, 24, 5
    d = rng.standard_normal((T, F)) @ np.diag(0.8 ** np.arange(F))
    U, V, s = pf.top_m_factors(d, m)
    err = np.linalg.norm(d - U @ V.T)
    np.testing.assert_allclose(err, np.sqrt((s[m:] ** 2).sum()), rtol=1e-12)
    # no random rank-m matrix (nor a perturbation of the optimum) does better
    for _ in range(50):
        A = rng.standard_normal((T, m))
        B = np.linalg.lstsq(A, d, rcond=None)[0]      # best B for this A
        assert np.linalg.norm(d - A @ B) >= err - 1e-9
        P = (U + 1e-3 * rng.standard_normal(U.shape)) @ (V + 1e-3 * rng.standard_normal(V.shape)).T
        assert np.linalg.norm(d - P) >= err - 1e-12
    # V orthonormal, U orthogonal with column norms s
    np.testing.assert_allclose(V.T @ V, np.eye(m), atol=1e-12)
    np.testing.assert_allclose(U.T @ U, np.diag(s[:m] ** 2), atol=1e-9)


def test_brute_force_rank_one_tiny():
    # 3 x 2: the best rank-1 approximation by a grid search over unit vectors v
    # (u = d v is then optimal) matches the SVD factor.
    d = np.array([[2.0, 1.0], [0.0, 1.0], [1.0, -1.0]])
    U, V, s = pf.top_m_factors(d, 1)
    best = min(np.linalg.norm(d - np.outer(d @ v, v))
               for v in (np.array([np.cos(a), np.sin(a)]) for a in np.linspace(0, np.pi, 20001)))
    np.testing.assert_allclose(np.linalg.norm(d - U @ V.T), best, rtol=1e-6)


def test_full_rank_reconstructs_and_chunks_are_separate():
    rng = np.random.default_rng(2)
    L, T, F = 2, 30, 8
    d = rng.standard_normal((L, T, F))
    offs = np.array([0, 10, 10, 30])
    U, V, S = pf.form_patch(d, offs, F)
    for l in range(L):
        np.testing.assert_allclose(U[l, 0:10] @ V[l, 0].T, d[l, 0:10], atol=1e-12)
        np.testing.assert_allclose(U[l, 10:30] @ V[l, 2].T, d[l, 10:30], atol=1e-12)
        assert S[l][1].size == 0 and not V[l, 1].any()

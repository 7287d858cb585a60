"""GPU parity of patch formation (top-m SVD factors of the deficit) against the oracle.

[K] Kamera, gist.science/pt/paper/2606.23581, §2 ("Aplicacao de Patch"): SVD, top-m
factors.  Singular vectors are unique only up to sign and within clusters of equal
singular values, so the comparison is on what is unique, and the rest is checked for
validity:
  - singular values: |s_gpu^2 - s^2| <= 1e-5 s_1^2 (fp32 Gram and fp32 eigensolver:
    eigenvalue errors are a few units of fp32 rounding of the largest eigenvalue);
  - Eckart-Young: the GPU patch is rank m, so its error ||Delta - U V^T||_F is at least
    the optimum; it may exceed it by the bf16 rounding of the factors, at most
    2^-8 ||U_m V_m^T||_F, plus 1e-3 of the optimum for the subspace iteration;
  - validity: V_m^T V_m = I and U_m^T U_m = diag(s^2) within bf16 rounding (columns with
    s > 0), U_m = Delta V_m within bf16 rounding, empty chunks give zeros.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _form(w, m, iterations=0, deficits=None):
    st = synth.structure(w)
    T, n, L = st.total_tokens, st.num_chunks, w.layers
    deltas = deficits if deficits is not None else synth.make_deficit(w, device=DEV)
    Fs = [d.shape[-1] for d in deltas]
    U = [torch.zeros((L, T, m), dtype=torch.bfloat16, device=DEV) for _ in Fs]
    V = [torch.zeros((L, n, F, m), dtype=torch.bfloat16, device=DEV) for F in Fs]
    S = [torch.zeros((L, n, m), dtype=torch.float32, device=DEV) for _ in Fs]
    offs = torch.as_tensor(st.offsets, device=DEV)
    dl = torch.zeros(n, dtype=torch.int64, device=DEV)
    ch = kamera.chunks_desc(offs, dl, T)
    d = kamera.form_desc(deltas, U, V, num_layers=L, rank=m, sigma=S, iterations=iterations)
    st_, nbytes = kamera.kamera_form_workspace(d, ch)
    kamera.check(st_)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    kamera.form_patch(d, ch, ws)
    torch.cuda.synchronize()
    host = lambda t: parity.host_bits(t)  # noqa: E731
    return st, deltas, [host(x) for x in U], [host(x) for x in V], [x.cpu().numpy() for x in S]


def _check(w, m, iterations=0, label="", deficits=None, sig_tol=1e-5, it_slack=1e-3):
    from oracle import patch_form as pf
    print(f"\n[case] form {label} m={m}", flush=True)
    st, deltas, U, V, S = _form(w, m, iterations, deficits)
    L, n = w.layers, st.num_chunks
    worst = dict(sig=0.0, ey=0.0, orth=0.0, u=0.0)
    for c, dlt in enumerate(deltas):
        F = dlt.shape[-1]
        D = parity.bf16_value(parity.host_bits(dlt)).reshape(L, -1, F)
        Ug = parity.bf16_value(U[c]).reshape(L, -1, m)
        Vg = parity.bf16_value(V[c]).reshape(L, n, F, m)
        for l in range(L):
            for j in range(n):
                a, b = int(st.offsets[j]), int(st.offsets[j + 1])
                if a == b:
                    assert not Vg[l, j].any() and not S[c][l, j].any()
                    continue
                d = D[l, a:b]
                Uo, Vo, s = pf.top_m_factors(d, m)
                r = min(m, s.size)
                # singular values
                sg = S[c][l, j][:r].astype(np.float64)
                err = np.abs(sg ** 2 - s[:r] ** 2).max() / s[0] ** 2
                worst["sig"] = max(worst["sig"], err)
                assert err <= sig_tol, (c, l, j, err)
                # Eckart-Young
                P = Ug[l, a:b] @ Vg[l, j].T
                opt = np.sqrt((s[m:] ** 2).sum())
                got = np.linalg.norm(d - P)
                assert got >= opt * (1 - 1e-9) - 1e-12
                excess = got - opt
                bound = 2.0 ** -8 * np.linalg.norm(Uo @ Vo.T) + it_slack * opt
                worst["ey"] = max(worst["ey"], excess / bound if bound else 0.0)
                assert excess <= bound, (c, l, j, excess, bound)
                # validity: orthonormal V, orthogonal U with norms s, U = Delta V
                live = sg > 1e-3 * s[0]
                vv = Vg[l, j][:, :r][:, live]
                o = np.abs(vv.T @ vv - np.eye(vv.shape[1])).max() if vv.size else 0.0
                worst["orth"] = max(worst["orth"], o)
                assert o <= 2.0 ** -6, (c, l, j, o)
                ug = Ug[l, a:b][:, :r]
                dv = d @ Vg[l, j][:, :r]
                tol = 2.0 ** -7 * (np.abs(d) @ np.abs(Vg[l, j][:, :r])) + 1e-30
                worst["u"] = max(worst["u"], (np.abs(ug - dv) / tol).max())
                assert (np.abs(ug - dv) <= tol).all()
    print(f"[case] worst: sigma {worst['sig']:.2e} ey/bound {worst['ey']:.3f} "
          f"orth {worst['orth']:.2e} u/tol {worst['u']:.3f}", flush=True)


def _w(**kw):
    base = dict(key="form", wid=80, family="gqa", layers=2, heads=4, head_dim=128, theta=1e6,
                rank=32, tokens=600)
    base.update(kw)
    return synth.Workload(**base)


@pytest.mark.parametrize("m", [1, 16, 32, 64, 112])
def test_form_qwen_shaped(m):
    _check(_w(lens=(400, 200)), m, label="F=512")


def test_form_chunks_short_and_empty():
    # Chunks shorter than the rank, a one-token chunk, an empty chunk, F = 1024.
    _check(_w(heads=8, lens=(300, 0, 10, 1, 257)), 32, label="short chunks F=1024")


def test_form_mla_widths():
    # c_KV (512) and k_rope (64): with m = 64 the k_rope patch is exact (k = F = 64).
    w = synth.get("deepseek_v3_mla").with_(layers=2, tokens=300)
    _check(w, 64, label="mla")


def test_form_rank_above_width():
    # m = 100 > F = 64 on k_rope: k = F, so only 64 columns can be nonzero; the rest of
    # U_m and V_m must be exactly zero, and the first 64 columns are the exact SVD.
    w = synth.get("deepseek_v3_mla").with_(layers=2, tokens=300)
    _check(w, 100, label="mla m=100")
    st, deltas, U, V, S = _form(w, 100)
    c = [d.shape[-1] for d in deltas].index(64)
    Ug = U[c].reshape(w.layers, -1, 100)
    Vg = V[c].reshape(w.layers, st.num_chunks, 64, 100)
    assert not Ug[..., 64:].any() and not Vg[..., 64:].any()


def test_form_many_problems():
    # 2 layers x 16 chunks = 32 problems per channel at F = 512: the workspace GEMMs run
    # with 8 x 32 = 256 workgroups of 64 rows, the form used at or above one per CU (the
    # smaller batches of the other cases take the form with K split over the waves).
    lens = tuple(24 + 5 * i for i in range(16))
    _check(_w(lens=lens, tokens=sum(lens)), 16, label="32 problems per channel")


def test_form_iterations_converge():
    # Fewer iterations leave the trailing singular values less converged (the error
    # falls like (lambda_{k+1} / lambda_i)^iterations); more meet the tight bounds.
    _check(_w(lens=(500,)), 32, iterations=2, label="2 iterations", sig_tol=1e-4,
           it_slack=1e-2)
    _check(_w(lens=(500,)), 32, iterations=16, label="16 iterations")


def test_form_rank_deficient_and_exact():
    # Delta of exact rank 5: every m >= 5 reproduces it (to bf16 rounding), with
    # singular values past 5 at zero.
    st = synth.structure(_w(lens=(200,)))
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    A = torch.randn((2, 200, 5), generator=g, device=DEV)
    B = torch.randn((2, 512, 5), generator=g, device=DEV)
    d = (A @ B.transpose(1, 2) * 0.1).to(torch.bfloat16)
    _check(_w(lens=(200,)), 16, label="rank 5", deficits=[d, d.clone()])
    assert st.total_tokens == 200


def test_form_full_size_qwen():
    # The Qwen2.5-VL-7B-shaped segment at full size (28 layers, T = 4096, F = 512, two
    # channels), rank 32, checked on a sample of layers.
    w = synth.get("qwen25vl7b_segment")
    from oracle import patch_form as pf
    st, deltas, U, V, S = _form(w, 32)
    for c in range(2):
        D = parity.bf16_value(parity.host_bits(deltas[c])).reshape(w.layers, -1, 512)
        Ug = parity.bf16_value(U[c]).reshape(w.layers, -1, 32)
        Vg = parity.bf16_value(V[c]).reshape(w.layers, 1, 512, 32)
        for l in (0, 13, 27):
            Uo, Vo, s = pf.top_m_factors(D[l], 32)
            assert np.abs(S[c][l, 0].astype(np.float64) ** 2 - s[:32] ** 2).max() <= 1e-5 * s[0] ** 2
            got = np.linalg.norm(D[l] - Ug[l] @ Vg[l, 0].T)
            opt = np.sqrt((s[32:] ** 2).sum())
            assert opt * (1 - 1e-9) <= got <= opt + 2.0 ** -8 * np.linalg.norm(Uo @ Vo.T) + 1e-3 * opt
    print(f"\n[case] form full size qwen ok", flush=True)


@pytest.mark.parametrize("heads,lens", [(2, (100, 0, 37, 300)), (8, (700, 5, 0, 1300))])
def test_form_gram_stage(heads, lens):
    # G_j = Delta_j^T Delta_j on MFMA: bf16 products are exact in fp32, so every entry is
    # within the fp32 summation bound T_j 2^-24 sum_t |Delta_ti Delta_tj| of the exact sum.
    # Chunks of many 64-token steps cycle through every LDS stage; F = 1024 has 36 tiles.
    w = _w(lens=lens, heads=heads)
    st = synth.structure(w)
    deltas = synth.make_deficit(w, device=DEV)
    L, n = w.layers, st.num_chunks
    Fs = [d.shape[-1] for d in deltas]
    G = [torch.full((L, n, F, F), float("nan"), dtype=torch.float32, device=DEV) for F in Fs]
    offs = torch.as_tensor(st.offsets, device=DEV)
    ch = kamera.chunks_desc(offs, torch.zeros(n, dtype=torch.int64, device=DEV), st.total_tokens)
    d = kamera.form_desc(deltas, [torch.empty(0, device=DEV)] * 2, [torch.empty(0, device=DEV)] * 2,
                         num_layers=L, rank=1)
    kamera.form_gram(d, ch, G)
    torch.cuda.synchronize()
    for c, F in enumerate(Fs):
        D = parity.bf16_value(parity.host_bits(deltas[c])).reshape(L, -1, F)
        g = G[c].cpu().numpy().astype(np.float64)
        for l in range(L):
            for j in range(n):
                a, b = int(st.offsets[j]), int(st.offsets[j + 1])
                x = D[l, a:b]
                exact = x.T @ x
                bound = max(b - a, 1) * 2.0 ** -24 * (np.abs(x).T @ np.abs(x)) + 1e-30
                assert (np.abs(g[l, j] - exact) <= bound).all(), (c, l, j)

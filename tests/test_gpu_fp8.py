"""GPU parity of the fp8 E4M3 KV form against the oracle's fp8 form.

8-bit KV ("Modelos Tomam Notas no Prefill", closing summary: the method holds on
FP8-quantised models): elements are OCP E4M3 codes with a per-(layer, channel) scale,
factors are bf16, and results are rounded to the nearest code, ties to even,
saturating at +-448.  Whole problems are compared element by element (1 code or the
cancellation band; untouched elements bit for bit), the encoder is checked bit for
bit on exact inputs, and the full-size fp8 workloads are checked on sampled rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _q(key, **kw):
    return synth.get(key).with_(dtype="fp8", **kw)


def _gqa(**kw):
    base = dict(key="fp8", wid=70, family="gqa", layers=2, heads=2, head_dim=128, theta=1e4,
                rank=8, tokens=100, dtype="fp8")
    base.update(kw)
    return synth.Workload(**base)


def _run_case(w, rank, flags=0, expect=None, label=""):
    print(f"\n[case] fp8 {label or w.key} rank={rank} flags={flags}", flush=True)
    inp = synth.make_inputs(w, rank, device=DEV)
    assert inp.buffers[0].dtype == torch.uint8 and len(inp.scales) == 2
    info = ops.plan(inp, flags)
    names = [kamera.KERNEL_NAMES[k] for k in info.kernel]
    if expect is not None:
        assert names == expect
    rep = parity.check_problem(inp, lambda i: ops.run(i, flags=flags))
    print(f"[case] kernels={names} {rep}", flush=True)
    assert rep.ok(), str(rep)
    assert rep.band_only <= max(2, rep.computed // 100000), str(rep)
    return rep


@pytest.mark.parametrize("rank", [0, 32])
def test_qwen_segment_reduced(rank):
    w = _q("qwen25vl7b_segment", layers=3, tokens=1000)
    _run_case(w, rank, expect=["rotate", "none"] if rank == 0 else ["rotate+patch mfma"] * 2)


def test_paged_reduced_with_spare_pages():
    w = _q("long_video_72b_paged", layers=2, tokens=1000, pool_pages=100)
    _run_case(w, w.rank, expect=["rotate+patch mfma"] * 2)


def test_paged_rotation_only():
    w = _q("long_video_72b_paged", layers=2, tokens=777, pool_pages=64)
    _run_case(w, 0, expect=["rotate", "none"])


def test_llama_reorder_reduced():
    # many chunks: boundary units cover the token groups chunk boundaries cut
    w = _q("llama3_8b_reorder", layers=2, n_chunks=9, chunk_len=(1, 300))
    _run_case(w, w.rank, expect=["rotate+patch mfma"] * 2)


def test_mla_reduced():
    w = _q("deepseek_v3_mla", layers=2, tokens=777)
    _run_case(w, w.rank, expect=["rotate+patch mfma"] * 2)


def test_mla_rotation_only():
    w = _q("deepseek_v3_mla", layers=2, tokens=300)
    rep = _run_case(w, 0, expect=["none", "rotate"])
    assert rep.computed == 2 * 300 * 64


@pytest.mark.parametrize("D,r,H,m,T", [
    (128, 32, 2, 8, 100),     # partial rotary
    (64, 16, 4, 5, 77),       # rank not a multiple of 8: generic kernel
    (128, 64, 3, 96, 130),    # rank padded to 128
    (32, 32, 4, 128, 41),     # four heads per feature block, largest tuned rank
    (96, 32, 2, 8, 40),       # dim 96: generic kernel
])
def test_shapes(D, r, H, m, T):
    w = _gqa(head_dim=D, rope_dim=r, heads=H, tokens=T, rank=m)
    _run_case(w, m, label=f"D={D} r={r} H={H} m={m} T={T}")
    if r in (16, 32, 64, 128):
        _run_case(w, 0, label=f"rotation D={D} r={r} H={H} T={T}")


@pytest.mark.parametrize("rank", [0, 16])
def test_chunk_edges(rank):
    w = _gqa(lens=(1, 0, 17, 1, 64, 0, 33, 1, 200),
             deltas=(5, 7, 0, -1, 1 << 20, 3, -(1 << 20), 0, 1), rank=16)
    _run_case(w, rank, label=f"chunk edges rank={rank}")


@pytest.mark.parametrize("rank", [0, 8])
def test_generic_kernel(rank):
    _run_case(_gqa(tokens=150), rank, flags=kamera.KAMERA_FLAG_GENERIC,
              expect=["generic", "generic" if rank else "none"])


@pytest.mark.parametrize("pairing,sections,delta_vec", [
    (1, (), None),                      # interleaved pairs
    (0, (16, 24, 24), (100, 0, -7)),    # M-RoPE sections, one of them still
])
@pytest.mark.parametrize("rank", [0, 16])
def test_positional_variants(pairing, sections, delta_vec, rank):
    kw = dict(pairing=pairing, sections=sections)
    if delta_vec is not None:
        kw["delta_vec"] = delta_vec
    w = _gqa(tokens=300, **kw)
    _run_case(w, rank, label=f"pairing={pairing} sections={sections} rank={rank}")


def test_encoder_bit_exact_on_exact_inputs():
    # Zero codes, scale 1, delta 0 and a patch with one nonzero product per element:
    # the value to encode is exact in fp32 (a product of two bf16 values), so the
    # kernel's code must equal the oracle's bit for bit: every E4M3 value, every tie
    # between neighbours, values past 448 and below the smallest subnormal, both signs.
    from oracle import oracle as orc
    mags = orc.fp8_to_f64(np.arange(0x7F))
    mids = (mags[:-1] + mags[1:]) / 2
    a = np.concatenate([mags, mids, [450.0, 464.0, 470.0, 1000.0, 2.0 ** -10, 2.0 ** -11]])
    bvals = np.array([1.0, -1.0, 0.5, -0.25, 2.0 ** -3, 3.0, -1.5, 0.75])
    assert np.array_equal(parity.bf16_value(orc.round_bf16(a)), a)  # exact in bf16
    T = -(-a.size // 16) * 16
    F = 128
    w = _gqa(heads=1, head_dim=F, tokens=T, rank=8, layers=1, deltas=(0,), lens=(T,))
    inp = synth.make_inputs(w, 8, device=DEV)
    for b in inp.buffers:
        b.zero_()
    for sc in inp.scales:
        sc.fill_(1.0)
    U = np.zeros((1, T, 8))
    U[0, :a.size, 0] = a
    V = np.zeros((1, 1, F, 8))
    V[0, 0, :, 0] = np.resize(bvals, F)
    for c in range(2):
        inp.U[c].copy_(torch.from_numpy(U).to(torch.bfloat16))
        inp.V[c].copy_(torch.from_numpy(V).to(torch.bfloat16))
    assert [kamera.KERNEL_NAMES[k] for k in ops.plan(inp).kernel] == ["rotate+patch mfma"] * 2
    before = [parity.host_bits(b) for b in inp.buffers]
    ops.run(inp)
    torch.cuda.synchronize()
    after = [parity.host_bits(b) for b in inp.buffers]
    out, _, _ = parity.oracle_on_host(inp, before)
    for g, o in zip(after, out):
        g, o = g.reshape(T, F), o.reshape(T, F)
        gv, ov = parity.fp8_value(g), parity.fp8_value(o)
        both_nan = np.isnan(gv) & np.isnan(ov)
        assert not np.isnan(ov).any()
        bad = (g != o) & ~both_nan
        assert not bad.any(), f"{int(bad.sum())} codes differ, first at {np.argwhere(bad)[:4]}"


@pytest.mark.parametrize("rank", [0, 8, 64])
def test_nan_codes_and_saturation(rank):
    # NaN codes (0x7F, 0xFF) must come out NaN, rotated together with their partner;
    # codes at +-448 and a patch far past the range must saturate to +-448, not NaN.
    w = _gqa(tokens=200, rank=max(rank, 8))
    inp = synth.make_inputs(w, rank, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(5)
    for b in inp.buffers:
        flat = b.view(-1)
        n = flat.numel()
        idx = torch.randperm(n, generator=g)[: n // 50].to(DEV)
        vals = torch.tensor([0x7F, 0xFF, 0x7E, 0xFE], dtype=torch.uint8, device=DEV)
        flat[idx] = vals[torch.arange(idx.numel(), device=DEV) % 4]
    if rank:
        for c in range(2):
            inp.U[c][:, 50:60] *= 4000.0  # these tokens' patch overflows the E4M3 range
    rep = parity.check_problem(inp, lambda i: ops.run(i))
    print(f"[case] fp8 nan/saturation rank={rank} {rep}", flush=True)
    assert rep.ok(), str(rep)


# ----------------------------------------------------------------- recall (out of place)

def _rw(**kw):
    base = dict(key="recall_fp8", wid=71, family="gqa", layers=2, heads=4, head_dim=128,
                theta=1e6, rank=32, tokens=300, delta=-1536, recall=True, dst_page_size=16,
                dst_pool_pages=40, dtype="fp8")
    base.update(kw)
    return synth.Workload(**base)


@pytest.mark.parametrize("rank,dst_page", [(32, 16), (0, 16), (64, 0)])
def test_recall(rank, dst_page):
    w = _rw(dst_page_size=dst_page, rank=rank)
    print(f"\n[case] fp8 recall rank={rank} dst_page={dst_page}", flush=True)
    r = synth.make_recall_inputs(w, rank, device=DEV)
    info = ops.recall_plan(r)
    assert [kamera.KERNEL_NAMES[k] for k in info.kernel] == ["rotate+patch mfma"] * 2
    rep, src_ok = parity.check_recall(r, lambda i: ops.run_recall(i))
    print(f"[case] {rep}", flush=True)
    assert src_ok
    assert rep.ok(), str(rep)


def test_recall_mla_generic():
    w = _rw(family="mla", heads=1, head_dim=512, rank=8, tokens=100, dst_page_size=0)
    r = synth.make_recall_inputs(w, 8, device=DEV)
    rep, src_ok = parity.check_recall(
        r, lambda i: ops.run_recall(i, flags=kamera.KAMERA_FLAG_GENERIC))
    assert src_ok and rep.ok(), str(rep)


# ----------------------------------------------------------------- full size, sampled

@pytest.mark.parametrize("key", ["qwen25vl7b_segment_fp8", "long_video_72b_paged_fp8"])
def test_full_size_sampled(key):
    w = synth.get(key)
    for rank in w.rank_passes:
        print(f"\n[case] fp8 full size {key} rank={rank}", flush=True)
        inp = synth.make_inputs(w, rank, device=DEV)
        rep = parity.sampled_check(inp, lambda i: ops.run(i), n=512)
        print(f"[case] {rep}", flush=True)
        assert rep.ok(), str(rep)
        del inp
        torch.cuda.empty_cache()

"""GPU parity of the positional variants against the oracle: interleaved pairing and
M-RoPE sections (one delta per section and chunk), in place and out of place (recall),
through the tuned and the generic kernels.

[N] "Modelos Tomam Notas no Prefill", gist.science/pt/paper/2606.17107, §4: image KV
is transplanted with M-RoPE re-rotation.  A pair whose section delta is 0 keeps its
bits when no patch is added.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SECTIONS = (16, 24, 24)


def _w(**kw):
    base = dict(key="variant", wid=70, family="gqa", layers=2, heads=2, head_dim=128, theta=1e6,
                rank=32, tokens=200, delta=-1536)
    base.update(kw)
    return synth.Workload(**base)


def _check(w, rank, flags=0, expect=None, label=""):
    print(f"\n[case] {label} rank={rank} flags={flags}", flush=True)
    inp = synth.make_inputs(w, rank, device=DEV)
    info = ops.plan(inp, flags)
    names = [kamera.KERNEL_NAMES[k] for k in info.kernel]
    if expect is not None:
        assert names == expect, names
    rep = parity.check_problem(inp, lambda i: ops.run(i, flags=flags))
    print(f"[case] kernels={names} {rep}", flush=True)
    assert rep.ok(), str(rep)
    assert rep.band_only <= max(2, rep.computed // 100000), str(rep)


def _check_recall(w, rank, flags=0, label=""):
    print(f"\n[case] recall {label} rank={rank} flags={flags}", flush=True)
    r = synth.make_recall_inputs(w, rank, device=DEV)
    rep, src_ok = parity.check_recall(r, lambda i: ops.run_recall(i, flags=flags))
    print(f"[case] {rep} src_unchanged={src_ok}", flush=True)
    assert src_ok and rep.ok(), str(rep)


MFMA2 = ["rotate+patch mfma"] * 2


@pytest.mark.parametrize("D,r,H,m", [(128, 128, 2, 32), (128, 64, 2, 8), (64, 16, 4, 64),
                                     (32, 32, 4, 0), (128, 128, 2, 0), (256, 128, 1, 16)])
def test_interleaved(D, r, H, m):
    w = _w(head_dim=D, rope_dim=r, heads=H, pairing=1, tokens=150)
    expect = (["rotate", "none"] if m == 0 else MFMA2)
    _check(w, m, expect=expect, label=f"interleaved D={D} r={r} H={H}")


def test_interleaved_chunks_paged_and_generic():
    w = _w(pairing=1, lens=(3, 0, 130, 1, 90), deltas=(5, -7, 0, 1 << 18, 65536), page_size=16,
           pool_pages=20)
    for m in (0, 16):
        _check(w, m, label="interleaved chunks paged")
        _check(w, m, flags=kamera.KAMERA_FLAG_GENERIC, expect=["generic"] * (2 if m else 1) +
               ([] if m else ["none"]), label="interleaved generic")


@pytest.mark.parametrize("m", [0, 8, 32, 64])
def test_mrope_sections(m):
    # Per-chunk section deltas, some of them 0, over several chunks and token groups.
    deltas = ((37, 37, 37), (-1536, 0, 12), (0, 0, 0), (0, 5, 0), (65536, -3, 1 << 20))
    w = _w(sections=SECTIONS, lens=(40, 100, 3, 160, 77), deltas=deltas)
    _check(w, m, label=f"mrope m={m}")


def test_mrope_paged_interleaved_and_generic():
    deltas = ((1, 2, 3), (0, -9, 0))
    for pairing in (0, 1):
        w = _w(sections=SECTIONS, lens=(70, 90), deltas=deltas, pairing=pairing, page_size=16,
               pool_pages=14)
        for m in (0, 32):
            _check(w, m, label=f"mrope paged pairing={pairing}")
            _check(w, m, flags=kamera.KAMERA_FLAG_GENERIC, label=f"mrope generic pairing={pairing}")


def test_mrope_zero_sections_keep_every_bit():
    # Rank 0: pairs of sections whose delta is 0 keep their bits, NaN payloads included.
    pats = torch.arange(65536, dtype=torch.int32, device=DEV).to(torch.int16)
    w = _w(layers=4, heads=1, sections=SECTIONS, lens=(64, 64), deltas=((0, 7, 0), (3, 0, 0)))
    for flags in (0, kamera.KAMERA_FLAG_GENERIC):
        inp = synth.make_inputs(w, 0, device=DEV)
        for b in inp.buffers:
            flat = b.view(torch.int16).view(-1)
            flat.copy_(pats[:flat.numel()])
        rep = parity.check_problem(inp, lambda i: ops.run(i, flags=flags))
        print(f"[case] mrope bit patterns flags={flags} {rep}", flush=True)
        assert rep.ok(), str(rep)


def test_mrope_mla_k_rope():
    # MLA: only the 64-dim k_rope rotates; its 32 pairs cut into sections 8 | 12 | 12.
    w = synth.get("deepseek_v3_mla").with_(layers=2, tokens=150, sections=(8, 12, 12),
                                           delta_vec=(100000, 0, -5))
    _check(w, 64, expect=MFMA2, label="mla mrope")
    _check(w, 0, label="mla mrope rotation")


def test_recall_variants():
    for pairing, sections, dl in ((1, (), None), (0, SECTIONS, ((9, 0, -4), (0, 0, 0))),
                                  (1, SECTIONS, ((1, 2, 0), (7, 7, 7)))):
        kw = dict(pairing=pairing, recall=True, dst_page_size=16, dst_pool_pages=30)
        if sections:
            kw.update(sections=sections, lens=(100, 120), deltas=dl)
        w = _w(**kw)
        for m in (0, 32):
            _check_recall(w, m, label=f"pairing={pairing} sections={sections}")
        _check_recall(w, 16, flags=kamera.KAMERA_FLAG_GENERIC, label="generic")


def test_full_size_qwen_mrope_sampled():
    # The Qwen2.5-VL-7B-shaped segment with three M-RoPE sections, at full size, in the
    # launch configuration of the benchmark, checked on sampled rows.
    w = synth.get("qwen25vl7b_segment").with_(sections=SECTIONS, delta_vec=(-1536, 4, -9))
    for m in (0, 32):
        inp = synth.make_inputs(w, m, device=DEV)
        rep = parity.sampled_check(inp, lambda i: ops.run(i), n=512)
        print(f"[case] qwen mrope full size m={m} {rep}", flush=True)
        assert rep.ok(), str(rep)
        del inp
        torch.cuda.empty_cache()

"""GPU parity of the VALU form of the rotate+patch kernel (the patch summed with
v_dot2_f32_bf16 instead of MFMA), which the library takes for bf16 in-place head
launches at rank <= 64 when KAMERA_PATCH_VALU=1.  Same oracle and bar as the MFMA
form; the switch is read on every call, so it is set and cleared around each case."""
import os

import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_valu(w, rank):
    print(f"\n[case] VALU patch {w.key} rank={rank}", flush=True)
    inp = synth.make_inputs(w, rank, device=DEV)
    os.environ["KAMERA_PATCH_VALU"] = "1"
    try:
        info = ops.plan(inp)
        rep = parity.check_problem(inp, ops.run)
    finally:
        del os.environ["KAMERA_PATCH_VALU"]
    print(f"[case] kernels={[kamera.KERNEL_NAMES[k] for k in info.kernel]} {rep}", flush=True)
    assert [kamera.KERNEL_NAMES[k] for k in info.kernel] == ["rotate+patch mfma"] * 2
    assert rep.ok(), str(rep)
    assert rep.band_only <= max(2, rep.computed // 100000), str(rep)


@pytest.mark.parametrize("rank", [8, 16, 32, 40, 64])
def test_valu_patch_contiguous(rank):
    w = synth.get("qwen25vl7b_segment").with_(layers=2, tokens=777)
    _run_valu(w, rank)


def test_valu_patch_chunks():
    w = synth.get("llama3_8b_reorder").with_(layers=2, n_chunks=9, chunk_len=(1, 300))
    _run_valu(w, w.rank)


def test_valu_patch_paged():
    w = synth.get("long_video_72b_paged").with_(layers=2, tokens=1000, pool_pages=100)
    _run_valu(w, w.rank)


def test_valu_patch_mla():
    w = synth.get("deepseek_v3_mla").with_(layers=2, tokens=777)
    _run_valu(w, w.rank)

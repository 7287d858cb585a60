"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Element-by-element comparisons at sizes the oracle finishes in seconds (several
tiles, ragged tails), plus the five workloads at their full sizes in the launch
configuration bench.py times, checked on sampled rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_case(w, rank, flags=0, expect=None, label=""):
    print(f"\n[case] {label or w.key} rank={rank} flags={flags}", flush=True)
    inp = synth.make_inputs(w, rank, device=DEV)
    info = ops.plan(inp, flags)
    if expect is not None:
        assert [kamera.KERNEL_NAMES[k] for k in info.kernel] == expect
    rep = parity.check_problem(inp, lambda i: ops.run(i, flags=flags))
    print(f"[case] kernels={[kamera.KERNEL_NAMES[k] for k in info.kernel]} {rep}", flush=True)
    assert rep.ok(), str(rep)
    assert rep.band_only <= max(2, rep.computed // 10000), str(rep)
    return rep


# ----------------------------------------------------------------- the five workloads, reduced

def test_tiny_mha_full():
    w = synth.get("tiny_mha")
    _run_case(w, w.rank, expect=["rotate+patch mfma"] * 2)


def test_tiny_mha_rotation_only():
    w = synth.get("tiny_mha")
    rep = _run_case(w, 0, expect=["rotate", "none"])
    assert rep.computed == 256 * 8 * 64  # K only: V is never touched


@pytest.mark.parametrize("rank", [0, 32])
def test_qwen_segment_reduced(rank):
    w = synth.get("qwen25vl7b_segment").with_(layers=3, tokens=1000)
    _run_case(w, rank)


def test_llama_reorder_reduced():
    w = synth.get("llama3_8b_reorder").with_(layers=2, n_chunks=9, chunk_len=(1, 300))
    _run_case(w, w.rank)


def test_mla_reduced():
    w = synth.get("deepseek_v3_mla").with_(layers=2, tokens=777)
    _run_case(w, w.rank, expect=["rotate+patch mfma"] * 2)


def test_mla_rotation_only():
    w = synth.get("deepseek_v3_mla").with_(layers=2, tokens=300)
    rep = _run_case(w, 0, expect=["none", "rotate"])
    assert rep.computed == 2 * 300 * 64  # k_rope only; c_KV byte for byte


def test_paged_reduced_with_spare_pages():
    # 1000 tokens need 63 pages; the pool has 100, so 37 spare pages must stay untouched.
    w = synth.get("long_video_72b_paged").with_(layers=2, tokens=1000, pool_pages=100)
    _run_case(w, w.rank, expect=["rotate+patch mfma"] * 2)


def test_paged_rotation_only():
    w = synth.get("long_video_72b_paged").with_(layers=2, tokens=777, pool_pages=64)
    _run_case(w, 0, expect=["rotate", "none"])


# ----------------------------------------------------------------- generic kernel

@pytest.mark.parametrize("key,rank", [("tiny_mha", 4), ("tiny_mha", 0),
                                      ("deepseek_v3_mla", 64)])
def test_generic_kernel(key, rank):
    w = synth.get(key)
    if w.family == "mla":
        w = w.with_(layers=1, tokens=200)
    _run_case(w, rank, flags=kamera.KAMERA_FLAG_GENERIC,
              expect=[kamera.KERNEL_NAMES[3] if (rank > 0 or lay_r > 0) else "none"
                      for lay_r in ([64, 0] if w.family != "mla" else [0, 64])])


def test_fp32_mode():
    w = synth.get("tiny_mha").with_(dtype="fp32")
    _run_case(w, w.rank, expect=["generic", "generic"])

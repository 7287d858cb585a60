"""GPU parity of relocate-on-read decode attention against the oracle's attention.

Kamera summary, §3 (production deployment): the rebuild runs as a hook in front of the
attention kernel.  kamera_attend consumes the relocated, patched keys and values inside
decode attention and writes nothing back; the oracle forms K' and V' in fp64 and
attends over them.  Outputs are compared element by element within the fp32 bound of
parity.check_attend (the bound's teeth are checked on the CPU).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 128 ** -0.5


def _run(inp, q, scale):
    return ops.attend(inp, q, scale)


def _case(w, rank, label="", q_heads=None):
    print(f"\n[case] attend {label or w.key} rank={rank}", flush=True)
    if q_heads is not None:
        w = w.with_(q_heads=q_heads)
    inp = synth.make_inputs(w, rank, device=DEV)
    q = synth.make_query(w, device=DEV)
    before = [parity.host_bits(b) for b in inp.buffers]
    rep = parity.check_attend(inp, q, SCALE, _run)
    print(f"[case] {rep}", flush=True)
    assert rep.ok(), str(rep)
    after = [parity.host_bits(b) for b in inp.buffers]
    assert all(np.array_equal(a, b) for a, b in zip(before, after)), "attention wrote the cache"
    return rep


@pytest.mark.parametrize("rank", [0, 32])
def test_qwen_segment_reduced(rank):
    # 28 query heads over 4 KV heads: a group of 7 in a kernel built for 8
    _case(synth.get("qwen25vl7b_segment").with_(layers=3, tokens=1000), rank)


def test_llama_reorder_reduced():
    # many chunks of ragged length: splits cut at chunk boundaries, group of 4, rank 16
    _case(synth.get("llama3_8b_reorder").with_(layers=2, n_chunks=9, chunk_len=(1, 300)), 16)


def test_paged_reduced_with_spare_pages():
    _case(synth.get("long_video_72b_paged").with_(layers=2, tokens=1000, pool_pages=100), 64)


@pytest.mark.parametrize("hq,rank", [(2, 0), (4, 48), (6, 96), (16, 128)])
def test_groups_and_ranks(hq, rank):
    # group sizes 1, 2, 3 and 8 (KV heads 2), ranks across the U-per-lane variants
    w = synth.Workload(key="att", wid=80, family="gqa", layers=2, heads=2, head_dim=128,
                       theta=1e4, rank=max(rank, 8), tokens=333, delta=-77)
    _case(w, rank, label=f"hq={hq} m={rank}", q_heads=hq)


@pytest.mark.parametrize("heads,rank,pages", [(4, 32, 0), (5, 16, 0), (6, 64, 60), (7, 8, 0),
                                               (8, 48, 60)])
def test_kv_head_counts(heads, rank, pages):
    # 4 to 8 KV heads at ranks up to 64 take one wave per KV head by default, any count
    # of them per workgroup; groups of 2 query heads, contiguous and paged caches, three
    # chunks so that splits cut at chunk boundaries too.
    w = synth.Workload(key="att", wid=82, family="gqa", layers=2, heads=heads, head_dim=128,
                       theta=1e4, rank=max(rank, 8), lens=(300, 5, 395), deltas=(11, -3, 700),
                       q_heads=2 * heads, page_size=16 if pages else 0, pool_pages=pages)
    _case(w, rank, label=f"kv heads={heads} m={rank} pages={pages}")


@pytest.mark.parametrize("rank", [0, 16])
def test_chunk_edges(rank):
    w = synth.Workload(key="att", wid=81, family="gqa", layers=2, heads=2, head_dim=128,
                       theta=1e4, rank=16, lens=(1, 0, 17, 1, 64, 0, 33, 1, 200),
                       deltas=(5, 7, 0, -1, 1 << 20, 3, -(1 << 20), 0, 1), q_heads=8)
    _case(w, rank, label=f"chunk edges rank={rank}")


@pytest.mark.parametrize("pairing,sections,delta_vec", [
    (1, (), None),
    (0, (16, 24, 24), (100, 0, -7)),
])
def test_positional_variants(pairing, sections, delta_vec):
    kw = dict(pairing=pairing, sections=sections)
    if delta_vec is not None:
        kw["delta_vec"] = delta_vec
    w = synth.Workload(key="att", wid=82, family="gqa", layers=2, heads=2, head_dim=128,
                       theta=1e6, rank=32, tokens=300, delta=300, q_heads=4, **kw)
    _case(w, 32, label=f"pairing={pairing} sections={sections}")


def test_partial_rotary():
    w = synth.Workload(key="att", wid=83, family="gqa", layers=1, heads=4, head_dim=128,
                       rope_dim=64, theta=1e4, rank=32, tokens=200, delta=9999, q_heads=8)
    _case(w, 32, label="rope_dim 64")


def test_masked_pages():
    # block-table entries outside [0, num_pages) are not attended
    w = synth.get("long_video_72b_paged").with_(layers=1, tokens=100, pool_pages=20)
    inp = synth.make_inputs(w, 64, device=DEV)
    bt = inp.struct.block_table.copy()
    bt[1] = -1
    bt[3] = 20
    inp.struct.block_table[:] = bt
    inp.block_table_t.copy_(torch.as_tensor(bt, device=DEV))
    q = synth.make_query(w, device=DEV)
    # the oracle drops negative entries; entry 20 (= num_pages) must be dropped too
    bt_oracle = bt.copy()
    bt_oracle[3] = -1
    out, lse = ops.attend(inp, q, SCALE)
    inp.struct.block_table[:] = bt_oracle
    rep = parity.check_attend(inp, q, SCALE, lambda i, qq, sc: (out, lse))
    print(f"[case] masked pages {rep}", flush=True)
    assert rep.ok(), str(rep)


def test_single_and_empty():
    w = synth.Workload(key="att", wid=84, family="gqa", layers=2, heads=2, head_dim=128,
                       theta=1e4, rank=16, tokens=1, delta=5, q_heads=4)
    _case(w, 16, label="one token")
    # no tokens: out = 0, lse = -inf
    w0 = w.with_(lens=(0,), deltas=(3,))
    inp = synth.make_inputs(w0, 0, device=DEV)
    q = synth.make_query(w0, device=DEV)
    out, lse = ops.attend(inp, q, SCALE)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_cache_untouched_and_matches_relocate_then_attend():
    # The fused result equals attention over the operator's output when that output is
    # kept unrounded: checked through the oracle; here the two GPU routes are compared
    # at bf16 rounding: relocate + patch in place, then plain attention (rank 0, delta 0).
    w = synth.get("qwen25vl7b_segment").with_(layers=2, tokens=777)
    inp = synth.make_inputs(w, 32, device=DEV)
    q = synth.make_query(w, device=DEV)
    fused, lf = ops.attend(inp, q, SCALE)
    ops.run(inp)  # K' and V' rounded to bf16, in place
    plain = synth.Inputs(inp.workload, 0, inp.struct.__class__(
        inp.struct.offsets, np.zeros_like(inp.struct.delta), inp.struct.block_table,
        inp.struct.outlier_features), inp.pool_pages, inp.buffers, inp.layouts)
    plain.offsets_t = inp.offsets_t
    plain.delta_t = torch.zeros_like(inp.delta_t)
    plain.block_table_t = inp.block_table_t
    unfused, lu = ops.attend(plain, q, SCALE)
    torch.cuda.synchronize()
    # bf16 rounding of K' and V' (2^-9 relative) bounds the difference
    diff = (fused - unfused).abs().max().item()
    ref = unfused.abs().max().item()
    print(f"[case] fused vs relocate-then-attend: max diff {diff:.3g} (max |out| {ref:.3g})")
    assert diff <= 2e-2 * ref


@pytest.mark.parametrize("P", [1, 4, 8, 32, 64])
def test_page_sizes(P):
    # pages of 16 slots or more: a tile's two block-table entries by scalar reads; below
    # 16, each lane reads its token's entry
    w = synth.get("long_video_72b_paged").with_(layers=2, tokens=333, page_size=P,
                                                pool_pages=-(-333 // P) + 5)
    _case(w, 32, label=f"pages of {P}")


# ----------------------------------------------------------------- fp8 E4M3 caches

@pytest.mark.parametrize("rank", [0, 32])
def test_fp8_qwen_segment_reduced(rank):
    # codes with per-layer scales of K and V; a group of 7 query heads per KV head
    _case(synth.get("qwen25vl7b_segment_fp8").with_(layers=3, tokens=1000), rank)


def test_fp8_paged_reduced_with_spare_pages():
    _case(synth.get("long_video_72b_paged_fp8").with_(layers=2, tokens=1000, pool_pages=100), 64)


def test_fp8_chunks_and_variants():
    # many ragged chunks (splits cut at chunk boundaries), interleaved pairing, rank 16
    w = synth.get("qwen25vl7b_segment_fp8").with_(layers=2, n_chunks=7, chunk_len=(1, 200),
                                                  pairing=1)
    _case(w, 16, label="fp8 chunks interleaved")


def test_fp8_small_pages():
    # pages of 4 slots: each lane reads its token's block-table entry
    w = synth.get("long_video_72b_paged_fp8").with_(layers=2, tokens=300, page_size=4,
                                                    pool_pages=90)
    _case(w, 32, label="fp8 pages of 4")


@pytest.mark.parametrize("key,layers", [("qwen25vl7b_segment", (0, 13, 27)),
                                        ("long_video_72b_paged", (0, 79)),
                                        ("llama3_8b_reorder", (0, 31)),
                                        ("long_video_72b_paged_fp8", (0, 79))])
def test_full_size_sampled_layers(key, layers):
    w = synth.get(key)
    rank = w.rank
    print(f"\n[case] attend full size {key} rank={rank}", flush=True)
    inp = synth.make_inputs(w, rank, device=DEV)
    q = synth.make_query(w, device=DEV)
    out, lse = ops.attend(inp, q, SCALE)
    torch.cuda.synchronize()
    for l in layers:
        sub = parity.layer_slice(inp, l)
        rep = parity.check_attend(sub, q[l:l + 1].contiguous(), SCALE,
                                  lambda i, qq, sc: (out[l:l + 1], lse[l:l + 1]))
        print(f"[case] layer {l}: {rep}", flush=True)
        assert rep.ok(), str(rep)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("hm", ["0", "1"])
@pytest.mark.parametrize("key,rank", [("llama3_8b_reorder", 16), ("long_video_72b_paged", 64),
                                      ("long_video_72b_paged_fp8", 64)])
def test_both_work_mappings(monkeypatch, hm, key, rank):
    # The tile kernel's two mappings (a 4-wave workgroup per KV head and range, or one
    # wave per KV head in a workgroup per range), each forced on a reduced shape.
    monkeypatch.setenv("KAMERA_ATTEND_HM", hm)
    w = synth.get(key).with_(layers=2)
    w = w.with_(n_chunks=5, chunk_len=(1, 400)) if w.n_chunks > 1 else w.with_(tokens=900, pool_pages=80 if w.page_size else 0)
    _case(w, rank, label=f"{key} mapping hm={hm}")

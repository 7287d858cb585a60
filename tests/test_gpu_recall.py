"""GPU parity of the recall (out-of-place) entry point against the oracle's recall.

Recall rebuilds chunks from a canonical store into other cache slots (Kamera summary,
§3, the three window operations: recall / reversible eviction).  Whole destinations
are compared element by element (slots the call must not write keep their NaN
sentinel bit for bit), the source is checked unchanged, and the full-size 72B-shaped
recall is checked on sampled rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _w(**kw):
    base = dict(key="recall", wid=60, family="gqa", layers=2, heads=4, head_dim=128, theta=1e6,
                rank=32, tokens=300, delta=-1536, recall=True, dst_page_size=16,
                dst_pool_pages=40)
    base.update(kw)
    return synth.Workload(**base)


def _run(w, rank, flags=0, expect=None, label="", prepare=None):
    print(f"\n[case] recall {label or w.key} rank={rank} flags={flags}", flush=True)
    r = synth.make_recall_inputs(w, rank, device=DEV)
    if prepare is not None:
        prepare(r)
    info = ops.recall_plan(r, flags)
    names = [kamera.KERNEL_NAMES[k] for k in info.kernel]
    if expect is not None:
        assert names == expect
    rep, src_ok = parity.check_recall(r, lambda i: ops.run_recall(i, flags=flags))
    print(f"[case] kernels={names} {rep} src_unchanged={src_ok}", flush=True)
    assert src_ok
    assert rep.ok(), str(rep)
    assert rep.band_only <= max(2, rep.computed // 100000), str(rep)
    return r, rep


MFMA2 = ["rotate+patch mfma"] * 2


@pytest.mark.parametrize("rank", [0, 8, 32, 64, 128])
def test_recall_contiguous_store_to_paged_cache(rank):
    _run(_w(), rank, expect=MFMA2, label="contiguous -> paged")


@pytest.mark.parametrize("rank", [0, 32])
def test_recall_chunks_and_tail(rank):
    # Several chunks (a delta-0 chunk, an empty chunk, boundaries inside token groups).
    w = _w(lens=(5, 0, 250, 1, 130, 300), deltas=(7, 3, 0, -9, 1 << 18, 65536))
    _run(w, rank, expect=MFMA2, label="chunks")


def test_recall_paged_store_to_contiguous_cache():
    w = _w(page_size=16, pool_pages=30, dst_page_size=0)
    _run(w, 64, expect=MFMA2, label="paged -> contiguous")
    _run(w, 0, expect=MFMA2, label="paged -> contiguous, rank 0")


def test_recall_paged_to_paged_other_page_size():
    w = _w(page_size=16, pool_pages=25, dst_page_size=32, dst_pool_pages=15)
    _run(w, 16, expect=MFMA2, label="paged 16 -> paged 32")


def test_recall_mla():
    w = synth.get("deepseek_v3_mla").with_(layers=2, tokens=200, recall=True, dst_page_size=16,
                                          dst_pool_pages=20)
    _run(w, 64, expect=MFMA2, label="mla -> paged")
    _run(w, 0, expect=MFMA2, label="mla -> paged, rank 0")


@pytest.mark.parametrize("case", ["rank12", "fp32", "dim96", "flag"])
def test_recall_generic_kernel(case):
    if case == "rank12":
        _run(_w(), 12, expect=["generic"] * 2, label=case)
    elif case == "fp32":
        _run(_w(dtype="f32"), 8, expect=["generic"] * 2, label=case)
        _run(_w(dtype="f32"), 0, expect=["generic"] * 2, label=case + " rank 0")
    elif case == "dim96":
        _run(_w(head_dim=96), 8, expect=["generic"] * 2, label=case)
    else:
        _run(_w(), 32, flags=kamera.KAMERA_FLAG_GENERIC, expect=["generic"] * 2, label=case)
        _run(_w(), 0, flags=kamera.KAMERA_FLAG_GENERIC, expect=["generic"] * 2,
             label=case + " rank 0")


@pytest.mark.parametrize("flags", [0, 1])
def test_recall_copies_every_bit_pattern(flags):
    # Rank 0: V (rope_dim 0), chunks with delta 0 and dims past rope_dim are copied bit for
    # bit, NaN payloads, -0, subnormals and infinities included.
    pats = torch.arange(65536, dtype=torch.int32, device=DEV).to(torch.int16)
    w = _w(layers=4, lens=(64, 64), deltas=(0, 12345), heads=1, rope_dim=64, dst_pool_pages=10)

    def fill(r):
        for b in r.src.buffers:
            flat = b.view(torch.int16).view(-1)
            flat.copy_(pats[:flat.numel()])
    _run(w, 0, flags=flags, label=f"bit patterns flags={flags}", prepare=fill)


def test_recall_skips_invalid_destination_pages():
    # Destination tokens whose page id is out of range are not written: the pool pages
    # the valid table would have given them keep the sentinel, bit for bit.
    from oracle import oracle as orc
    w = _w(tokens=100, dst_pool_pages=9)
    r = synth.make_recall_inputs(w, 8, device=DEV)
    valid = r.dst_block_table.copy()
    bad = valid.copy()
    bad[1], bad[4] = -1, 1 << 20
    r.dst_block_table_t = torch.as_tensor(bad, device=DEV)
    d_before = [parity.host_bits(b) for b in r.dst_buffers]
    s_host = [parity.host_bits(b) for b in r.src.buffers]
    factors = ([parity.host_bits(u) for u in r.src.U], [parity.host_bits(v) for v in r.src.V])
    ops.run_recall(r)
    torch.cuda.synchronize()
    got = [parity.host_bits(b) for b in r.dst_buffers]
    expect = [b.copy() for b in d_before]
    y = [parity.bf16_value(b) for b in d_before]
    s = [np.full(b.size, -1.0) for b in d_before]
    orc.recall_patch(parity._dicts(r.src.layouts, s_host, factors, 8),
                     parity._dicts(r.dst_layouts, expect), num_layers=w.layers, theta=w.theta,
                     offsets=r.src.struct.offsets, delta=r.src.struct.delta, rank=8,
                     dst_page_size=16, dst_block_table=valid, y_out=y, s_out=s)
    shape = (w.layers, 9, 16, w.heads, w.head_dim)
    for c in range(2):
        for pg in (valid[1], valid[4]):  # never written: sentinel, compared bit for bit
            expect[c].reshape(shape)[:, pg] = d_before[c].reshape(shape)[:, pg]
            s[c].reshape(shape)[:, pg] = -1.0
        rep = parity.compare(got[c], expect[c], y[c], s[c], 8)
        assert rep.ok(), str(rep)
        assert (got[c].reshape(shape)[:, valid[1]] == synth.DST_SENTINEL).all()


def test_recall_full_size_sampled():
    # The bench workload at full size (80 layers, T = 32768, rank 64, paged destination).
    w = synth.get("recall_72b_paged")
    print(f"\n[case] recall full size {w.key}", flush=True)
    r = synth.make_recall_inputs(w, w.rank, device=DEV)
    info = ops.recall_plan(r)
    assert [kamera.KERNEL_NAMES[k] for k in info.kernel] == MFMA2
    rep = parity.sampled_check_recall(r, lambda i: ops.run_recall(i), n=512)
    print(f"[case] {rep}", flush=True)
    assert rep.ok(), str(rep)
    del r
    torch.cuda.empty_cache()

"""GPU parity of kamera_relocate_patch_ws: one chunk over a paged cache swept in pool
order through the inverse of the block table, against the fp64 CPU oracle element by
element, and against kamera_relocate_patch bit for bit (the two differ only in the order
of the work)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _paged(**kw):
    base = synth.get("long_video_72b_paged").with_(layers=2, tokens=1000, pool_pages=0)
    return base.with_(**kw)


def _case(w, rank, label):
    print(f"\n[pool] {label} rank={rank}", flush=True)
    inp = synth.make_inputs(w, rank, device=DEV)
    ws = ops.workspace_for(inp)
    assert ws is not None, "this problem should run in pool order"
    rep = parity.check_problem(inp, lambda i: ops.run_ws(i, ws))
    print(f"[pool] {rep}", flush=True)
    assert rep.ok(), str(rep)
    assert rep.band_only <= max(2, rep.computed // 100000), str(rep)
    return inp


@pytest.mark.parametrize("rank", [64, 32, 8, 3, 100])
def test_pool_order_ranks(rank):
    # 1000 tokens in 63 pages (the last one partial); pool of exactly 63 pages.
    _case(_paged(), rank, "exact pool")


def test_pool_order_spare_pages():
    # 100 pool pages for 63 used: the 37 others keep their bits (checked by parity:
    # elements the call must not touch are compared bit for bit).
    _case(_paged(pool_pages=100), 64, "spare pages")


@pytest.mark.parametrize("P", [32, 64, 256])
def test_pool_order_page_sizes(P):
    _case(_paged(page_size=P, tokens=1500, pool_pages=-(-1500 // P) + 3), 64, f"page {P}")


def test_pool_order_fp8():
    _case(_paged(dtype="fp8"), 64, "fp8")


def test_pool_order_partial_rotary_and_variants():
    _case(_paged(rope_dim=64), 32, "partial rotary")
    _case(_paged(pairing=1), 32, "interleaved")
    _case(_paged(sections=(16, 24, 24), delta_vec=(5, 0, -300)), 32, "M-RoPE sections")


def test_pool_order_delta_zero():
    _case(_paged(delta=0), 16, "delta 0")


def test_pool_order_invalid_page_ids():
    # Entries outside [0, num_pages) leave their tokens alone; the pool pages the valid
    # table gives those tokens keep their input bits.
    w = _paged(tokens=300, pool_pages=40)
    print("\n[pool] invalid page ids", flush=True)
    inp = synth.make_inputs(w, 64, device=DEV)
    valid = np.asarray(inp.struct.block_table).copy()
    bad = valid.copy()
    bad[1], bad[4] = -1, 1 << 20
    before = [parity.host_bits(b) for b in inp.buffers]
    factors = ([parity.host_bits(u) for u in inp.U], [parity.host_bits(v) for v in inp.V])
    inp.block_table_t = torch.as_tensor(bad, dtype=torch.int32, device=DEV)
    ws = ops.workspace_for(inp)
    assert ws is not None
    ops.run_ws(inp, ws)
    torch.cuda.synchronize()
    got = [parity.host_bits(b) for b in inp.buffers]
    out, y, s = parity.oracle_on_host(inp, before, factors)
    rep = parity.Report()
    for c, lay in enumerate(inp.layouts):
        b = lay["buffer"]
        shape = (w.layers, 40, w.page_size, lay["heads"], lay["dim"])
        for pg in (valid[1], valid[4]):
            out[b].reshape(shape)[:, pg] = before[b].reshape(shape)[:, pg]
            s[b].reshape(shape)[:, pg] = -1.0
            assert (got[b].reshape(shape)[:, pg] == before[b].reshape(shape)[:, pg]).all()
    for g, o, yy, ss in zip(got, out, y, s):
        parity.compare(g, o, yy, ss, inp.rank, rep)
    print(f"[pool] {rep}", flush=True)
    assert rep.ok(), str(rep)


def test_pool_order_reused_workspace_stale_entries():
    # The same workspace serves a second call whose table maps fewer pages: the inverse
    # is rebuilt from scratch, so pool pages the first table used and the second does not
    # are left alone.
    w1 = _paged(tokens=1000, pool_pages=100)
    inp1 = synth.make_inputs(w1, 32, device=DEV)
    ws = ops.workspace_for(inp1)
    ops.run_ws(inp1, ws)
    w2 = _paged(tokens=200, pool_pages=50)
    inp2 = synth.make_inputs(w2, 32, device=DEV)
    ws2 = ops.workspace_for(inp2)
    assert ws2 is not None and ws2.numel() <= ws.numel()
    print("\n[pool] reused workspace", flush=True)
    rep = parity.check_problem(inp2, lambda i: ops.run_ws(i, ws))
    print(f"[pool] {rep}", flush=True)
    assert rep.ok(), str(rep)


def test_pool_order_matches_logical_order_full_size():
    # The 72B-shaped paged workload at full size: the pool-order call and the plain call
    # on copies of the same input give the same bits everywhere (10.7 GB compared on
    # the device), and sampled rows match the oracle.
    w = synth.get("long_video_72b_paged")
    print(f"\n[pool] full size: {w.note}", flush=True)
    inp = synth.make_inputs(w, w.rank, device=DEV)
    ref = [b.clone() for b in inp.buffers]
    twin = synth.Inputs(inp.workload, inp.rank, inp.struct, inp.pool_pages, ref, inp.layouts,
                        inp.U, inp.V, inp.offsets_t, inp.delta_t, inp.block_table_t)
    ops.run(twin)
    ws = ops.workspace_for(inp)
    assert ws is not None
    rep = parity.sampled_check(inp, lambda i: ops.run_ws(i, ws), n=1024)
    print(f"[pool] sampled {rep}", flush=True)
    assert rep.ok(), str(rep)
    for a, b in zip(inp.buffers, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    print("[pool] pool order == logical order, bit for bit", flush=True)

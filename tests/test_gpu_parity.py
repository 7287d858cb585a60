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
    assert rep.band_only <= max(2, rep.computed // 100000), str(rep)
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


# ----------------------------------------------------------------- shapes and edge cases

def _gqa(**kw):
    base = dict(key="shape", wid=50, family="gqa", layers=2, heads=2, head_dim=128, theta=1e4,
                rank=8, tokens=100)
    base.update(kw)
    return synth.Workload(**base)


@pytest.mark.parametrize("D,r,H,m,T", [
    (128, 32, 2, 8, 100),     # partial rotary, partner 2 lanes away
    (64, 16, 4, 3, 77),       # partner 1 lane away, odd rank (element loads)
    (256, 128, 2, 24, 50),    # head spans two feature blocks
    (128, 64, 3, 96, 130),    # rank padded to 128 (4 k-steps)
    (32, 32, 4, 128, 41),     # four heads per feature block, largest tuned rank
    (128, 128, 1, 1, 17),     # rank 1
    (64, 64, 3, 5, 1),        # one token; F = 192 leaves half a block idle
    (96, 32, 2, 8, 40),       # dim 96: generic kernel
])
def test_shapes(D, r, H, m, T):
    w = _gqa(head_dim=D, rope_dim=r, heads=H, tokens=T, rank=m)
    _run_case(w, m, label=f"D={D} r={r} H={H} m={m} T={T}")
    if r in (16, 32, 64, 128):
        _run_case(w, 0, label=f"rotation D={D} r={r} H={H} T={T}")


@pytest.mark.parametrize("rank", [0, 16])
def test_chunk_edges(rank):
    # empty chunks, one-token chunks, delta 0 / +-1 / +-2^20, chunks not aligned to tiles
    w = _gqa(lens=(1, 0, 17, 1, 64, 0, 33, 1, 200),
             deltas=(5, 7, 0, -1, 1 << 20, 3, -(1 << 20), 0, 1), rank=16)
    _run_case(w, rank, label=f"chunk edges rank={rank}")


@pytest.mark.parametrize("rank", [8, 64, 100])
def test_chunk_boundary_groups(rank):
    # Token groups that chunk boundaries cut: one unit per boundary in the head launch,
    # or a second launch when boundaries outnumber groups.  Boundaries here: one on a
    # group start (512 is a multiple of every group size), several inside one group, an
    # empty chunk; then many tiny chunks, so that boundaries outnumber groups.
    lens = (512, 3, 0, 250, 1, 1, 700, 40)
    deltas = (3, -5, 9, 0, 1 << 16, -7, 11, 2)
    _run_case(_gqa(lens=lens, deltas=deltas, rank=rank), rank,
              label=f"boundaries by boundary rank={rank}")
    _run_case(_gqa(lens=lens, deltas=deltas, rank=rank, page_size=16, pool_pages=110), rank,
              label=f"boundaries by boundary, paged, rank={rank}")
    rng = np.random.default_rng(rank)
    lens2 = tuple(int(x) for x in rng.integers(0, 10, size=40))
    deltas2 = tuple(int(x) for x in rng.integers(-1000, 1000, size=40))
    _run_case(_gqa(lens=lens2, deltas=deltas2, rank=rank), rank,
              label=f"boundaries by group rank={rank}")


def test_paged_chunk_edges():
    w = _gqa(lens=(5, 0, 40, 1, 70), deltas=(1, 2, -3, 0, 99999), page_size=16, pool_pages=20,
             heads=4)
    _run_case(w, 32, label="paged chunk edges")
    _run_case(w, 0, label="paged chunk edges rotation")


def test_delta_zero_rotation_only_is_untouched():
    w = _gqa(lens=(50, 30), deltas=(0, 0))
    inp = synth.make_inputs(w, 0, device=DEV)
    before = [parity.host_bits(b) for b in inp.buffers]
    ops.run(inp)
    torch.cuda.synchronize()
    after = [parity.host_bits(b) for b in inp.buffers]
    for a, b in zip(after, before):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("rank", [0, 64])
def test_paged_skips_invalid_pages(rank):
    # Tokens whose block-table entry is out of range (-1, or past the pool) are left
    # untouched: the rows are skipped through the out-of-range buffer offset, so the
    # pool pages the valid table gives those tokens keep their input bits, and every
    # other token matches the oracle run with the valid table.
    w = synth.get("long_video_72b_paged").with_(layers=2, tokens=300, pool_pages=40)
    print(f"\n[case] paged, invalid page ids, rank={rank}", flush=True)
    inp = synth.make_inputs(w, rank, device=DEV)
    valid = np.asarray(inp.struct.block_table).copy()
    bad = valid.copy()
    bad[1], bad[4] = -1, 1 << 20
    before = [parity.host_bits(b) for b in inp.buffers]
    factors = ([parity.host_bits(u) for u in inp.U], [parity.host_bits(v) for v in inp.V])
    inp.block_table_t = torch.as_tensor(bad, dtype=torch.int32, device=DEV)
    ops.run(inp)
    torch.cuda.synchronize()
    got = [parity.host_bits(b) for b in inp.buffers]
    out, y, s = parity.oracle_on_host(inp, before, factors)  # struct keeps the valid table
    rep = parity.Report()
    for c, lay in enumerate(inp.layouts):
        b = lay["buffer"]
        shape = (w.layers, 40, w.page_size, lay["heads"], lay["dim"])
        for pg in (valid[1], valid[4]):  # skipped: input bits, compared bit for bit
            out[b].reshape(shape)[:, pg] = before[b].reshape(shape)[:, pg]
            s[b].reshape(shape)[:, pg] = -1.0
            assert (got[b].reshape(shape)[:, pg] == before[b].reshape(shape)[:, pg]).all()
    for g, o, yy, ss in zip(got, out, y, s):
        parity.compare(g, o, yy, ss, inp.rank, rep)
    print(f"[case] {rep}", flush=True)
    assert rep.ok(), str(rep)

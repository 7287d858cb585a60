"""kamera_relocate_patch_noalloc through the C ABI against kamera_relocate_patch_ws, the
entry point it varies: the same bits, on two calls in a row (the second with a smaller
input, so the library-held array still holds the first call's entries), and on a
problem that needs no inverse table."""
import pytest

torch = pytest.importorskip("torch")

from rope_relocation_rank_amd import kamera as K  # noqa: E402
from rope_relocation_rank_amd import ops, synth  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _twins(w, rank):
    a = synth.make_inputs(w, rank, device=DEV)
    b = synth.Inputs(a.workload, a.rank, a.struct, a.pool_pages, [x.clone() for x in a.buffers],
                     a.layouts, a.U, a.V, a.offsets_t, a.delta_t, a.block_table_t,
                     scales=list(a.scales))
    return a, b


def _noalloc(inp):
    kv, ch, p = ops.descriptors_for(inp)
    st = K.kamera_relocate_patch_noalloc(kv, ch, p, K.current_stream())
    assert st == K.KAMERA_OK, K.kamera_last_error()


def _same(a, b):
    for x, y in zip(a.buffers, b.buffers):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_noalloc_matches_workspace_entry_point_twice():
    big = synth.get("long_video_72b_paged").with_(layers=3, tokens=4000, pool_pages=300)
    small = big.with_(layers=2, tokens=700, pool_pages=60)
    for label, w in (("first call", big), ("second call, smaller", small)):
        print(f"\n[noalloc] {label}: {w.layers} layers, {w.tokens} tokens, "
              f"{w.pool_pages} pool pages", flush=True)
        a, b = _twins(w, 64)
        ws = ops.workspace_for(a)
        assert ws is not None, "the problem should take the pool-order path"
        ops.run_ws(a, ws)
        _noalloc(b)
        torch.cuda.synchronize()
        _same(a, b)
        # and both differ from the input (the call did something)
        inp = synth.make_inputs(w, 64, device=DEV)
        assert not torch.equal(inp.buffers[0].view(torch.uint8), b.buffers[0].view(torch.uint8))


def test_noalloc_fp8_and_without_inverse_table():
    w = synth.get("long_video_72b_paged_fp8").with_(layers=2, tokens=900, pool_pages=70)
    print("\n[noalloc] fp8 paged", flush=True)
    a, b = _twins(w, 64)
    ops.run_ws(a, ops.workspace_for(a))
    _noalloc(b)
    torch.cuda.synchronize()
    _same(a, b)
    # several chunks: no inverse table; runs as kamera_relocate_patch
    w = synth.get("llama3_8b_reorder").with_(layers=2, n_chunks=5, chunk_len=(10, 300))
    print("[noalloc] several chunks, contiguous", flush=True)
    a, b = _twins(w, 16)
    assert ops.workspace_for(a) is None
    ops.run(a)
    _noalloc(b)
    torch.cuda.synchronize()
    _same(a, b)

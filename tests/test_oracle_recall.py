"""Pins of the oracle's recall (out-of-place rehydration) form.

[K] Kamera, gist.science/pt/paper/2606.23581, §3 (the three cheap window operations,
recall / reversible eviction): an evicted chunk is rebuilt from its canonical store with
a patch for its new context.  Recall writes the same rows the in-place operator would
produce, into other slots, and carries every element the operator leaves alone over
bit for bit.  The in-place oracle is pinned elsewhere (test_oracle_pins.py); these
tests tie recall to it and to the exact-copy facts ([K §2]: R(0) is the identity and
c_KV is reused as stored; [K §3]: without a patch only the keys move).
"""
import numpy as np
import pytest

from oracle import oracle as orc


def _chans(data, H, D, rope, L, slots, paged, P=0, U=None, V=None):
    out = []
    for c in range(len(data)):
        d = dict(data=data[c], heads=H, dim=D, rope_dim=rope[c], slot_stride=H * D, head_stride=D)
        if paged:
            d.update(layer_stride=slots * P * H * D, page_stride=P * H * D)
        else:
            d.update(layer_stride=slots * H * D, page_stride=0)
        if U is not None:
            d.update(U=U, V=V[c])
        out.append(d)
    return out


def _case(seed, L=2, T=45, H=2, D=64, m=3):
    rng = np.random.default_rng(seed)
    xb = orc.round_bf16(rng.standard_normal((L, T, H, D))).reshape(L, T, H, D)
    U = orc.round_bf16(0.3 * rng.standard_normal((L, T, m))).reshape(L, T, m) if m else None
    V = (orc.round_bf16(0.3 * rng.standard_normal((2, L, 3, H * D, m))).reshape(2, L, 3, H * D, m)
         if m else None)
    offs = np.array([0, 20, 20, T], np.int64)
    delta = np.array([5, 8, -70000], np.int64)
    return rng, xb, U, V, offs, delta


@pytest.mark.parametrize("m", [0, 3])
def test_recall_into_paged_slots_equals_in_place(m):
    # Contiguous canonical store -> paged cache under a random block table: every token
    # row lands in its table slot with the in-place result; spare slots and the source
    # are left alone.
    L, T, H, D, P = 2, 45, 2, 64, 8
    rng, xb, U, V, offs, delta = _case(11 + m, L, T, H, D, m)
    rope = (D, 0)
    ref = [xb.copy().ravel(), xb.copy().ravel()]
    orc.relocate_patch(_chans(ref, H, D, rope, L, T, False, U=U, V=V), num_layers=L, theta=1e4,
                       offsets=offs, delta=delta, rank=m)
    need = -(-T // P)
    table = rng.permutation(need + 4)[:need].astype(np.int32)
    pool = int(table.max()) + 2
    src = [xb.copy().ravel(), xb.copy().ravel()]
    dst = [np.full(L * pool * P * H * D, 0x7FC1, np.uint16) for _ in range(2)]
    snap = [d.copy() for d in dst]
    orc.recall_patch(_chans(src, H, D, rope, L, T, False, U=U, V=V),
                     _chans(dst, H, D, rope, L, pool, True, P), num_layers=L, theta=1e4,
                     offsets=offs, delta=delta, rank=m, dst_page_size=P, dst_block_table=table)
    used = np.zeros((pool, P), bool)
    for t in range(T):
        used[table[t // P], t % P] = True
    for c in range(2):
        assert np.array_equal(src[c], xb.ravel())
        pl = dst[c].reshape(L, pool, P, H, D)
        got = np.stack([pl[:, table[t // P], t % P] for t in range(T)], axis=1)
        assert np.array_equal(got, ref[c].reshape(L, T, H, D))
        assert np.array_equal(pl[:, ~used], snap[c].reshape(L, pool, P, H, D)[:, ~used])


def test_recall_from_paged_store_to_contiguous():
    # Paged source, contiguous destination: the source table decides where rows are
    # read, the destination takes them in token order.
    L, T, H, D, P, m = 2, 45, 2, 64, 16, 3
    rng, xb, U, V, offs, delta = _case(21, L, T, H, D, m)
    rope = (D, 0)
    ref = [xb.copy().ravel(), xb.copy().ravel()]
    orc.relocate_patch(_chans(ref, H, D, rope, L, T, False, U=U, V=V), num_layers=L, theta=1e4,
                       offsets=offs, delta=delta, rank=m)
    need = -(-T // P)
    table = rng.permutation(need + 2)[:need].astype(np.int32)
    pool = need + 2
    src = []
    for c in range(2):
        pl = np.zeros((L, pool, P, H, D), np.uint16)
        for t in range(T):
            pl[:, table[t // P], t % P] = xb[:, t]
        src.append(pl.ravel())
    dst = [np.zeros(L * T * H * D, np.uint16) for _ in range(2)]
    orc.recall_patch(_chans(src, H, D, rope, L, pool, True, P, U=U, V=V),
                     _chans(dst, H, D, rope, L, T, False), num_layers=L, theta=1e4,
                     offsets=offs, delta=delta, rank=m, src_page_size=P, src_block_table=table)
    for c in range(2):
        assert np.array_equal(dst[c], ref[c])


def test_recall_copies_every_bit_pattern():
    # No patch: a chunk with delta 0, a channel with rope_dim 0 and dims >= rope_dim are
    # copied bit for bit (NaN payloads, -0, subnormals, infinities).
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    T, H, D = 1024, 1, 64
    for delta, rope in ((0, 64), (777, 0), (777, 32)):
        src = [x.copy()]
        dst = [np.zeros_like(x)]
        orc.recall_patch(_chans(src, H, D, (rope,), 1, T, False),
                         _chans(dst, H, D, (rope,), 1, T, False), num_layers=1, theta=1e4,
                         offsets=np.array([0, T], np.int64), delta=np.array([delta], np.int64))
        if rope == 32:
            assert np.array_equal(dst[0].reshape(T, D)[:, 32:], x.reshape(T, D)[:, 32:])
            assert not np.array_equal(dst[0].reshape(T, D)[:, :32], x.reshape(T, D)[:, :32])
        else:
            assert np.array_equal(dst[0], x)
        assert np.array_equal(src[0], x)


def test_recall_reports_computed_elements():
    # y_out / s_out (destination layout) hold the fp64 value and magnitude of exactly the
    # elements the rotation or the patch changes.
    L, T, H, D, m = 1, 12, 1, 64, 0
    rng, xb, U, V, offs, delta = _case(31, L, T, H, D, m)
    delta = np.array([0, 0, 9], np.int64)
    offs = np.array([0, 4, 4, T], np.int64)
    src = [xb.copy().ravel()]
    dst = [np.zeros(T * D, np.uint16)]
    y = [np.full(T * D, np.nan)]
    s = [np.full(T * D, -1.0)]
    orc.recall_patch(_chans(src, H, D, (32,), L, T, False), _chans(dst, H, D, (32,), L, T, False),
                     num_layers=L, theta=1e4, offsets=offs, delta=delta, y_out=y, s_out=s)
    computed = s[0].reshape(T, D) >= 0
    expect = np.zeros((T, D), bool)
    expect[4:, :32] = True
    assert np.array_equal(computed, expect)
    xf = orc.bf16_to_f64(xb.reshape(T, D))
    for t in range(4, T):
        np.testing.assert_array_equal(y[0].reshape(T, D)[t, :32],
                                      orc.row_f64(xf[t], 1, D, 32, 1e4, 9)[:32])

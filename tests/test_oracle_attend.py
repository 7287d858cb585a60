"""Pins of the oracle's relocate-on-read decode attention.

[K] Kamera, gist.science/pt/paper/2606.23581, §3 (production deployment: the rebuild
runs as a hook in front of the attention kernel): attention reads the relocated and
patched keys and values, K' = R(delta) K + U V_K^T and V' = V + U V_V^T, without
storing them.  The row values K', V' come from the operator's row function, pinned
elsewhere; these tests pin what attention adds on top: the score, the softmax over
tokens, the grouped-query head mapping, masking, and the log-sum-exp, through closed
forms, special cases and invariances.
"""
import math

import numpy as np
import pytest

from oracle import oracle as orc


def _chans(K, V, r, U=None, VK=None, VV=None):
    L, T, H, D = K.shape
    out = []
    for c, data in enumerate((K, V)):
        d = dict(data=data.ravel().copy(), heads=H, dim=D, rope_dim=r if c == 0 else 0,
                 layer_stride=T * H * D, slot_stride=H * D, head_stride=D, page_stride=0)
        if U is not None:
            d.update(U=U[c], V=(VK, VV)[c])
        out.append(d)
    return out


def _rand(seed, L=2, T=37, H=2, D=16, m=0, n=2):
    rng = np.random.default_rng(seed)
    K = np.ascontiguousarray(rng.standard_normal((L, T, H, D)), np.float32)
    V = np.ascontiguousarray(rng.standard_normal((L, T, H, D)), np.float32)
    U = VK = VV = None
    if m:
        U = [np.ascontiguousarray(0.3 * rng.standard_normal((L, T, m)), np.float32)
             for _ in range(2)]
        VK = np.ascontiguousarray(0.3 * rng.standard_normal((L, n, H * D, m)), np.float32)
        VV = np.ascontiguousarray(0.3 * rng.standard_normal((L, n, H * D, m)), np.float32)
    return rng, K, V, U, VK, VV


def _relocated(chans, L, theta, offs, delta, m):
    """fp64 K', V' from the (pinned) in-place operator's unrounded values; elements it
    does not move keep their input values."""
    cs = [dict(c, data=c["data"].copy()) for c in chans]
    ys = [c["data"].astype(np.float64) for c in cs]
    ss = [np.zeros(c["data"].size) for c in cs]
    orc.relocate_patch(cs, num_layers=L, theta=theta, offsets=offs, delta=delta, rank=m,
                       y_out=ys, s_out=ss)
    return ys


def test_single_token_returns_its_relocated_value():
    # softmax over one token is 1 whatever the score: out = V'_0 of the query's KV head
    L, H, D, m = 2, 3, 8, 4
    rng, K, V, U, VK, VV = _rand(1, L=L, T=1, H=H, D=D, m=m, n=1)
    ch = _chans(K, V, D, U, VK, VV)
    offs, delta = np.array([0, 1]), np.array([12345])
    q = rng.standard_normal((L, 2 * H, D))
    out, lse = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta, q=q,
                          scale=0.3, rank=m)
    _, vprime = _relocated(ch, L, 1e4, offs, delta, m)
    vprime = vprime.reshape(L, 1, H, D)
    for h in range(2 * H):
        assert np.array_equal(out[:, h], vprime[:, 0, h // 2])


def test_zero_query_averages_values_and_lse_is_log_t():
    # q = 0 gives equal weights: out is the mean of V' over tokens, lse = log T
    L, T, H, D, m = 2, 29, 2, 16, 3
    rng, K, V, U, VK, VV = _rand(2, L=L, T=T, H=H, D=D, m=m)
    ch = _chans(K, V, D, U, VK, VV)
    offs, delta = np.array([0, 11, T]), np.array([5, -700])
    q = np.zeros((L, 4, D))
    out, lse = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta, q=q,
                          scale=1.0, rank=m)
    _, vprime = _relocated(ch, L, 1e4, offs, delta, m)
    mean = vprime.reshape(L, T, H, D).mean(axis=1)
    for h in range(4):
        np.testing.assert_allclose(out[:, h], mean[:, h // 2], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(T), rtol=1e-15)


def test_two_token_closed_form():
    # D = 2, no rotation, no patch; K rows give scores 0 and ln 3 exactly in weight:
    # p = (1/4, 3/4), out = V0 / 4 + 3 V1 / 4, lse = log 4.
    K = np.zeros((1, 2, 1, 2), np.float32)
    K[0, 1, 0, 0] = 1.0
    V = np.array([[[[4.0, -8.0]], [[8.0, 4.0]]]], np.float32)
    ch = _chans(K, V, 0)
    q = np.array([[[math.log(3.0), 7.0]]])
    out, lse = orc.attend(ch, num_layers=1, theta=1e4, offsets=np.array([0, 2]),
                          delta=np.array([0]), q=q, scale=1.0)
    np.testing.assert_allclose(out[0, 0], [4.0 / 4 + 3 * 8.0 / 4, -8.0 / 4 + 3 * 4.0 / 4],
                               rtol=1e-15)
    np.testing.assert_allclose(lse[0, 0], math.log(4.0), rtol=1e-15)


def test_grouped_query_head_mapping():
    # Query head h reads KV head h // (Hq / Hkv): each KV head's keys single out a
    # different token, and each token's value names the (head, token) it came from.
    L, T, H, D = 1, 4, 2, 4
    K = np.zeros((L, T, H, D), np.float32)
    V = np.zeros((L, T, H, D), np.float32)
    K[0, 1, 0, 0] = 1.0  # KV head 0: token 1 stands out along dim 0
    K[0, 3, 1, 0] = 1.0  # KV head 1: token 3
    for t in range(T):
        for g in range(H):
            V[0, t, g, :] = 10 * g + t
    ch = _chans(K, V, 0)
    q = np.zeros((L, 6, D))
    q[..., 0] = 60.0  # e^60 dwarfs every other weight
    out, _ = orc.attend(ch, num_layers=L, theta=1e4, offsets=np.array([0, T]),
                        delta=np.array([0]), q=q, scale=1.0)
    for h in range(6):
        np.testing.assert_allclose(out[0, h], 1.0 if h < 3 else 13.0, rtol=1e-12)


def test_relative_position_invariance():
    # Moving every chunk by the same extra Delta and the query by Delta (its own RoPE
    # rotation) leaves every score, hence every output, unchanged.
    L, T, H, D, m = 2, 40, 2, 16, 4
    rng, K, V, U, VK, VV = _rand(4, L=L, T=T, H=H, D=D, m=m)
    offs, delta = np.array([0, 15, 22, T]), np.array([3, -900, 77777])
    q = rng.standard_normal((L, 2, D))
    # the patch is not rotated, so the invariance holds for m = 0 only
    ch = _chans(K, V, D)
    a, la = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta, q=q, scale=0.25)
    shift = 1234
    qs = np.stack([[orc.rotate_head_f64(q[l, h], D, 1e4, shift) for h in range(2)]
                   for l in range(L)])
    b, lb = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta + shift, q=qs,
                       scale=0.25)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=1e-12)
    # a wrong rotation direction breaks it
    qw = np.stack([[orc.rotate_head_f64(q[l, h], D, 1e4, -shift) for h in range(2)]
                   for l in range(L)])
    c, _ = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta + shift, q=qw,
                      scale=0.25)
    assert np.abs(c - a).max() > 1e-3


def test_scale_and_shift_invariance():
    # scale multiplies the scores (scale 2 == query doubled); a query component that
    # is orthogonal to every key changes nothing
    L, T, H, D = 1, 30, 1, 8
    rng, K, V, _, _, _ = _rand(5, L=L, T=T, H=H, D=D)
    K[..., -1] = 0.0
    ch = _chans(K, V, 0)
    offs, delta = np.array([0, T]), np.array([0])
    q = rng.standard_normal((L, 1, D))
    a, _ = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta, q=q, scale=2.0)
    b, _ = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta, q=2 * q, scale=1.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    q2 = q.copy()
    q2[..., -1] += 100.0
    c, _ = orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta, q=q2, scale=2.0)
    np.testing.assert_allclose(a, c, rtol=1e-13)


def test_masked_tokens_equal_removed_tokens_and_large_scores_stay_finite():
    # Paged: tokens whose block-table entry is negative are not attended, which equals
    # attending over the cache without them.
    L, H, D, P = 1, 2, 8, 4
    rng = np.random.default_rng(6)
    T = 12
    K = rng.standard_normal((L, 4, P, H, D)).astype(np.float32)
    V = rng.standard_normal((L, 4, P, H, D)).astype(np.float32)
    table = np.array([2, -1, 0], np.int32)  # tokens 4..7 have no slot
    chans = []
    for c, data in enumerate((K, V)):
        chans.append(dict(data=data.ravel().copy(), heads=H, dim=D, rope_dim=D if c == 0 else 0,
                          layer_stride=4 * P * H * D, slot_stride=H * D, head_stride=D,
                          page_stride=P * H * D))
    q = 30 * rng.standard_normal((L, 2, D))  # scores in the hundreds
    out, lse = orc.attend(chans, num_layers=L, theta=1e4, offsets=np.array([0, T]),
                          delta=np.array([9]), q=q, scale=1.0, page_size=P, block_table=table)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    Kc = np.concatenate([K[:, 2], K[:, 0]], axis=1)  # the 8 attended tokens, in order
    Vc = np.concatenate([V[:, 2], V[:, 0]], axis=1)
    # token positions matter only through delta, which is the same for all tokens
    ref, lref = orc.attend(_chans(Kc, Vc, D), num_layers=L, theta=1e4, offsets=np.array([0, 8]),
                           delta=np.array([9]), q=q, scale=1.0)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lref, rtol=1e-13)


def test_token_order_does_not_matter():
    # attention is a function of the set of (key, value) pairs: reversing the tokens,
    # their chunk deltas and their U rows together gives the same output
    L, T, H, D, m = 1, 20, 1, 8, 2
    rng, K, V, U, VK, VV = _rand(7, L=L, T=T, H=H, D=D, m=m, n=2)
    offs, delta = np.array([0, 8, T]), np.array([40, -3])
    q = rng.standard_normal((L, 1, D))
    a, la = orc.attend(_chans(K, V, D, U, VK, VV), num_layers=L, theta=1e4, offsets=offs,
                       delta=delta, q=q, scale=0.5, rank=m)
    r = slice(None, None, -1)
    Ur = [np.ascontiguousarray(u[:, r]) for u in U]
    b, lb = orc.attend(_chans(np.ascontiguousarray(K[:, r]), np.ascontiguousarray(V[:, r]), D,
                              Ur, np.ascontiguousarray(VK[:, ::-1]),
                              np.ascontiguousarray(VV[:, ::-1])),
                       num_layers=L, theta=1e4, offsets=np.array([0, 12, T]),
                       delta=delta[::-1].copy(), q=q, scale=0.5, rank=m)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_fp8_cache_matches_the_same_values_in_bf16():
    # An fp8 E4M3 cache (codes and per-layer scales of each channel) and a bf16 cache
    # holding exactly the same values attend to the same result, bit for bit: with
    # power-of-two scales every scale * code is a bf16 value.  The scales differ per
    # layer and per channel, so a scale taken from the wrong layer or channel, or left
    # out, changes the result.
    L, T, H, D, m, n = 3, 29, 2, 16, 8, 2
    rng = np.random.default_rng(9)
    codes = []
    for _ in range(2):
        c = rng.integers(0, 0x7F, size=(L, T, H, D)) | (rng.integers(0, 2, size=(L, T, H, D)) << 7)
        codes.append(np.ascontiguousarray(c, dtype=np.uint8))
    scales = [np.array([2.0 ** -3, 2.0, 2.0 ** 4], np.float32),
              np.array([4.0, 2.0 ** -5, 1.0], np.float32)]
    bf = [orc.round_bf16(orc.fp8_to_f64(codes[c]) * scales[c].astype(np.float64)[:, None, None, None])
          for c in range(2)]
    for c in range(2):  # exact: the values are bf16 numbers
        assert np.array_equal(orc.bf16_to_f64(bf[c]),
                              orc.fp8_to_f64(codes[c]) * scales[c].astype(np.float64)[:, None, None, None])
    f = lambda x: orc.round_bf16(x)  # noqa: E731  bf16 factors
    U = [f(0.3 * rng.standard_normal((L, T, m))) for _ in range(2)]
    VK, VV = f(0.3 * rng.standard_normal((L, n, H * D, m))), f(0.3 * rng.standard_normal((L, n, H * D, m)))
    offs, delta = np.array([0, 11, T]), np.array([7, -300])
    q = rng.standard_normal((L, 2 * H, D))

    def run(data, with_scales):
        ch = _chans(data[0], data[1], D, U, VK, VV)
        if with_scales is not None:
            for c in range(2):
                ch[c]["scale"] = with_scales[c]
        return orc.attend(ch, num_layers=L, theta=1e4, offsets=offs, delta=delta, q=q,
                          scale=0.25, rank=m)

    out8, lse8 = run(codes, scales)
    out16, lse16 = run(bf, None)
    assert np.array_equal(out8, out16) and np.array_equal(lse8, lse16)
    swapped, _ = run(codes, scales[::-1])
    assert not np.allclose(swapped, out16)

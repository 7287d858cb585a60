"""GPU numerics through the real kernels: round-to-nearest-even ties, NaN / Inf /
overflow, HIP-graph capture and replay, and a non-default stream."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as orc  # noqa: E402
from rope_relocation_rank_amd import kamera, ops, synth  # noqa: E402

import parity  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits_to_bf16_tensor(bits, shape):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(
        torch.bfloat16).reshape(shape).to(DEV)


def _tie_problem(x_bits, p_bits, D=128, H=1, delta=0, flags=0):
    """One layer, T tokens of one head: out = round(R(delta) x + 1.0 * p) with rank 1."""
    T = x_bits.size // (H * D)
    K = _bits_to_bf16_tensor(x_bits, (1, T, H, D))
    Vc = K.clone()
    U = torch.ones((1, T, 1), dtype=torch.bfloat16, device=DEV)
    Vf = _bits_to_bf16_tensor(p_bits, (1, 1, H * D, 1))
    lay = [dict(buffer=0, offset=0, heads=H, dim=D, rope_dim=D, layer_stride=T * H * D,
                slot_stride=H * D, head_stride=D),
           dict(buffer=1, offset=0, heads=H, dim=D, rope_dim=0, layer_stride=T * H * D,
                slot_stride=H * D, head_stride=D)]
    offs = torch.tensor([0, T], dtype=torch.int64, device=DEV)
    dl = torch.tensor([delta], dtype=torch.int64, device=DEV)
    kv, ch, p = ops.descriptors(
        [K, Vc], lay, dtype_code=kamera.KAMERA_BF16, num_layers=1, theta=1e4, offsets_t=offs,
        delta_t=dl, total_tokens=T, rank=1, U=(U, U), V=(Vf, Vf), flags=flags)
    return K, Vc, (kv, ch, p)


@pytest.mark.parametrize("flags", [0, kamera.KAMERA_FLAG_GENERIC])
def test_ties_round_to_even(flags):
    # x + p lands exactly half-way between two bf16 values (x has 8 significant bits,
    # p is half of x's ulp, both exact in fp32): the result must round to even.
    rng = np.random.default_rng(0)
    D, T = 128, 64
    expo = rng.integers(-20, 20, size=D)            # one exponent per feature
    mant = rng.integers(0, 128, size=(T, D))
    sign = rng.integers(0, 2, size=(T, D))
    x = ((1 + mant / 128.0) * 2.0 ** expo[None, :] * (1 - 2 * sign)).ravel()
    half_ulp = 2.0 ** (expo - 8) * np.where(rng.integers(0, 2, size=D) == 1, 1, -1)
    xb = orc.round_bf16(x)
    pb = orc.round_bf16(half_ulp)
    K, Vc, (kv, ch, p) = _tie_problem(xb, pb, D=D, flags=flags)
    kamera.relocate_patch_(kv, ch, p)
    torch.cuda.synchronize()
    got = parity.host_bits(K)
    # the oracle rounds the exact fp64 sum; every element here is exactly representable
    # in fp32 before the final rounding, so the GPU must be bit-exact.
    want = np.concatenate([orc.row(xb[t * D:(t + 1) * D], 1, D, D, 1e4, 0,
                                   np.array([0x3F80], np.uint16), pb.reshape(D, 1))
                           for t in range(T)])
    assert np.array_equal(got, want)
    # and ties really occurred (all but the values at a power of two) and went to even
    xv = parity.bf16_value(xb).reshape(T, D)
    pv = parity.bf16_value(pb)[None, :]
    ties = np.abs(pv) == np.abs(parity.bf16_ulp(xv)) / 2
    ties &= ~((np.abs(xv) == 2.0 ** np.floor(np.log2(np.abs(xv)))) & (np.sign(pv) != np.sign(xv)))
    assert ties.sum() > T * D // 2
    assert np.all((got.reshape(T, D)[ties] & 1) == 0)


def test_rne_large_seeded_sample():
    # A million fp32 values the kernel forms exactly, then rounds to bf16 itself: with
    # delta = 0 and a rank-8 patch whose U row is (2^e, 2^e, 0, ...) and whose V row holds
    # two 8-bit integers scaled by 2^-15 and 2^-23, element (t, f) is x + mid + low with
    # x the bf16 input (exponent e) and mid, low filling the next 16 mantissa bits, so
    # every partial sum is exact in fp32 whatever the accumulation order.  The kernel's
    # round to nearest even must give the oracle's rounding of the exact value, bit for
    # bit: random patterns, exact ties (mid = 0x80, low = 0) either way, one unit either
    # side of a tie, a carry into the exponent, and NaN rows.
    rng = np.random.default_rng(2024)
    D, T, m = 128, 8192, 8
    e = rng.integers(-60, 60, size=T)
    sign = np.where(rng.integers(0, 2, size=(T, D)) == 1, -1.0, 1.0)
    mant = rng.integers(128, 256, size=(T, D))           # 8 significant bits
    # features 0, 1 hold exact ties: keep |y| in x's binade for negative x too
    mant[:, :2] = rng.integers(129, 256, size=(T, 2))
    mant[:, 8] = 255  # feature 8: all-ones mantissa, so rounding up carries into e + 1
    x = sign * mant * 2.0 ** (e[:, None] - 7)
    mid = rng.integers(0, 256, size=D).astype(np.float64)
    low = rng.integers(0, 256, size=D).astype(np.float64)
    special = [(128, 0), (128, 0), (128, 1), (127, 255), (0, 0), (255, 255), (128, 255), (0, 1),
               (200, 0)]
    for k, (a, b) in enumerate(special):  # ties, near-ties and the carry feature
        mid[k], low[k] = a, b
    nan_rows = rng.choice(T, size=16, replace=False)
    x[nan_rows, 9] = np.nan
    xb = orc.round_bf16(x.ravel())
    assert np.array_equal(parity.bf16_value(xb)[~np.isnan(x.ravel())], x.ravel()[~np.isnan(x.ravel())])
    U = np.zeros((T, m))
    U[:, 0] = U[:, 1] = 2.0 ** e
    Vm = np.zeros((D, m))
    Vm[:, 0], Vm[:, 1] = mid * 2.0 ** -15, low * 2.0 ** -23
    ub, vb = orc.round_bf16(U.ravel()), orc.round_bf16(Vm.ravel())
    assert np.array_equal(parity.bf16_value(ub), U.ravel())
    assert np.array_equal(parity.bf16_value(vb), Vm.ravel())
    K = _bits_to_bf16_tensor(xb, (1, T, 1, D))
    Vc = K.clone()
    Ut = _bits_to_bf16_tensor(ub, (1, T, m))
    Vt = _bits_to_bf16_tensor(vb, (1, 1, D, m))
    lay = [dict(buffer=0, offset=0, heads=1, dim=D, rope_dim=D, layer_stride=T * D,
                slot_stride=D, head_stride=D),
           dict(buffer=1, offset=0, heads=1, dim=D, rope_dim=0, layer_stride=T * D,
                slot_stride=D, head_stride=D)]
    offs = torch.tensor([0, T], dtype=torch.int64, device=DEV)
    dl = torch.tensor([0], dtype=torch.int64, device=DEV)
    kv, ch, p = ops.descriptors([K, Vc], lay, dtype_code=kamera.KAMERA_BF16, num_layers=1,
                                theta=1e4, offsets_t=offs, delta_t=dl, total_tokens=T, rank=m,
                                U=(Ut, Ut), V=(Vt, Vt))
    st, info = kamera.kamera_plan(kv, ch, p)
    assert st == 0 and info.kernel[0] == 2  # the tuned rotate+patch kernel
    kamera.relocate_patch_(kv, ch, p)
    torch.cuda.synchronize()
    got = parity.host_bits(K)
    yv = x + (mid * 2.0 ** -15)[None, :] * 2.0 ** e[:, None] + (low * 2.0 ** -23)[None, :] * 2.0 ** e[:, None]
    want = orc.round_bf16(yv.ravel())  # RNE of the exact value (exact in fp32 as well)
    nan = np.isnan(yv.ravel())
    assert np.array_equal(np.isnan(parity.bf16_value(got)), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # the sample holds the cases it claims: exact ties, both resolutions, and carries
    ties = (mid == 128) & (low == 0)
    assert ties.sum() == 2
    tie_bits = got.reshape(T, D)[:, ties]
    assert np.all((tie_bits & 1) == 0)  # ties went to the even neighbour
    carried = np.abs(parity.bf16_value(got.reshape(T, D)[:, 8])) == 2.0 ** (e + 1)
    assert carried.mean() > 0.4  # positive rows round 255 + 0.78 up to the next binade
    print(f"[rne] {T * D} values, {int(ties.sum()) * T} exact ties, {len(nan_rows)} NaN",
          flush=True)


def test_nan_inf_overflow():
    D = 128
    vals = np.array([np.inf, -np.inf, np.nan, 3.38e38, -3.38e38, 0.0, -0.0, 1e-40] * 16)[:D]
    xb = orc.round_bf16(vals)
    pb = orc.round_bf16(np.array([1.0, 1.0, 1.0, 3.0e38, -3.0e38, 0.0, -0.0, 1e-40] * 16)[:D])
    K, Vc, (kv, ch, p) = _tie_problem(xb, pb, D=D)
    kamera.relocate_patch_(kv, ch, p)
    torch.cuda.synchronize()
    got = parity.bf16_value(parity.host_bits(K))
    want = parity.bf16_value(orc.row(xb, 1, D, D, 1e4, 0, np.array([0x3F80], np.uint16),
                                     pb.reshape(D, 1)))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.isinf(got[3]) and got[3] > 0 and np.isinf(got[4]) and got[4] < 0


def test_rotation_propagates_nan_inf():
    # Rotation with delta != 0: an Inf or NaN in one dim of a pair reaches both outputs as
    # IEEE arithmetic does (inf * 0 may give NaN); elements of other pairs are unaffected.
    w = synth.Workload(key="naninf", wid=60, family="gqa", layers=1, heads=1, head_dim=128,
                       theta=1e4, rank=0, tokens=16, delta=3)
    inp = synth.make_inputs(w, 0, device=DEV)
    flat = inp.buffers[0].view(-1)
    flat[5] = float("inf")
    flat[128 + 70] = float("nan")
    rep = parity.check_problem(inp, ops.run)
    assert rep.ok(), str(rep)


def test_graph_capture_and_replay():
    # The call is stream-ordered and allocates nothing, so it can be captured; replays
    # interleaved with eager work and synchronisations must all match eager execution.
    w = synth.get("llama3_8b_reorder").with_(layers=2, n_chunks=5, chunk_len=(40, 300))
    a = synth.make_inputs(w, w.rank, device=DEV)
    b = synth.make_inputs(w, w.rank, device=DEV)
    kv_a, ch_a, p_a = ops.descriptors_for(a)
    s = torch.cuda.Stream()
    ref = [x.clone() for x in b.buffers]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kamera.relocate_patch_(kv_a, ch_a, p_a, kamera.current_stream())
    start = [x.clone() for x in a.buffers]
    for rep in range(3):
        for x, x0 in zip(a.buffers, start):
            x.copy_(x0)
        for x, x0 in zip(ref, start):
            x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        kv_r, ch_r, p_r = ops.descriptors([*ref], a.layouts, dtype_code=kamera.KAMERA_BF16,
                                          num_layers=w.layers, theta=w.theta,
                                          offsets_t=a.offsets_t, delta_t=a.delta_t,
                                          total_tokens=a.struct.total_tokens, rank=a.rank,
                                          U=a.U, V=a.V)
        kamera.relocate_patch_(kv_r, ch_r, p_r)
        torch.cuda.synchronize()
        for x, y in zip(a.buffers, ref):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"replay {rep}"


def test_non_default_stream():
    w = synth.get("tiny_mha")
    inp = synth.make_inputs(w, w.rank, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()

    def run(i):
        with torch.cuda.stream(s):
            ops.run(i)
        s.synchronize()

    rep = parity.check_problem(inp, run)
    assert rep.ok(), str(rep)

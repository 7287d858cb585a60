"""Seeded synthetic workloads: shapes, layouts, chunk structure and input values.

This module holds no step of the operator.  It draws the inputs that both the HIP
path and the CPU oracle consume, describes where every element lives (strides,
block table), and counts the bytes an ideal in-place pass moves.

Inputs stand in for real model KV of the named shapes (no weights or datasets are
used).  Values: KV ~ N(0, 1); patch factors ~ N(0, s^2) with s^2 = 0.1 / sqrt(m),
so every entry of U V^T has standard deviation 0.1 whatever m is; all drawn in fp32
and rounded to the storage dtype.  Seeds derive from (workload id, kind, layer,
channel) through numpy's SeedSequence; kind 0 = KV, 1 = U, 2 = V, 3 = structure,
4 = recall destination.  The structure stream draws chunk lengths, then deltas, then
the block-table permutation, then outlier feature indices; the destination stream
draws the destination block-table permutation.

8-bit workloads (dtype "fp8") hold OCP FP8 E4M3 codes: the KV values are drawn as
above in fp32, each (layer, channel) gets the scale s = max |value| / 224 (half the
code range, so rotation and patch keep headroom), and the codes are PyTorch's E4M3
encoding of value / s.  Their factors are bf16.

Recall workloads (out of place) read a canonical store laid out as the workload says
and write into a destination cache, paged with its own random block table or
contiguous; destination slots are pre-filled with a NaN sentinel so that any slot the
call must not write is checked bit for bit.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

KIND_KV, KIND_U, KIND_V, KIND_STRUCT, KIND_DST = 0, 1, 2, 3, 4
KIND_QUERY = 6
DST_SENTINEL = 0x7FC1  # bf16 NaN with a payload the operator never produces
DST_SENTINEL_FP8 = 0x7F  # E4M3 NaN: the operator never produces it from finite inputs


@dataclass(frozen=True)
class Workload:
    key: str
    wid: int
    family: str                 # "mha", "gqa" or "mla"
    layers: int
    heads: int                  # KV heads (1 for MLA)
    head_dim: int               # GQA/MHA head dim; MLA latent width (c_KV)
    theta: float
    rank: int                   # patch rank of the patched pass
    passes: tuple = (None,)     # ranks run per step; None = `rank`
    tokens: int = 0             # fixed chunk length (single chunk) when chunk_len is None
    n_chunks: int = 1
    chunk_len: tuple | None = None   # (lo, hi) inclusive, drawn per chunk
    delta: int = 0
    delta_range: tuple | None = None  # (lo, hi) inclusive, drawn per chunk
    rope_mla: int = 64          # MLA decoupled k_rope width
    rope_dim: int = 0           # GQA/MHA rotated dims per key head (0 = the whole head)
    lens: tuple | None = None   # explicit chunk lengths (overrides tokens / chunk_len)
    deltas: tuple | None = None  # explicit per-chunk deltas (overrides delta / delta_range)
    page_size: int = 0
    pool_pages: int = 0         # pages per layer in the pool (paged only)
    outliers: int = 0           # feature indices scaled by outlier_scale in K and V
    outlier_scale: float = 8.0
    dtype: str = "bf16"
    note: str = ""
    pairing: int = 0            # 0 NeoX half-split, 1 interleaved
    sections: tuple = ()        # M-RoPE rotary pairs per section (empty: plain RoPE)
    delta_vec: tuple | None = None  # M-RoPE: the same per-section delta for every chunk
    recall: bool = False        # out of place: canonical store -> destination cache
    dst_page_size: int = 0      # recall destination: 0 contiguous, > 0 paged
    dst_pool_pages: int = 0     # recall destination pool pages per layer (paged)
    q_heads: int = 0            # decode attention: query heads (0 = the KV heads)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def rank_passes(self) -> tuple:
        return tuple(self.rank if r is None else r for r in self.passes)

    @property
    def elem_size(self) -> int:
        return {"bf16": 2, "fp8": 1}.get(self.dtype, 4)

    @property
    def factor_size(self) -> int:
        """Bytes of a patch-factor element (bf16 for fp8 KV)."""
        return 2 if self.dtype == "fp8" else self.elem_size


WORKLOADS = {
    "tiny_mha": Workload(
        key="tiny_mha", wid=0, family="mha", layers=1, heads=8, head_dim=64, theta=1e4,
        rank=4, tokens=256, delta=37,
        note="tiny MHA, 1 layer, T=256, 8 heads x 64, delta +37, rank-4 patch on K and V"),
    "qwen25vl7b_segment": Workload(
        key="qwen25vl7b_segment", wid=1, family="gqa", layers=28, heads=4, head_dim=128,
        theta=1e6, rank=32, passes=(0, 32), tokens=4096, delta=-1536, outliers=4, q_heads=28,
        note="Qwen2.5-VL-7B-shaped video segment: 28 layers, 4 KV heads x 128, T=4096, "
             "delta -1536; rotation-only pass then rank-32 patch pass"),
    "llama3_8b_reorder": Workload(
        key="llama3_8b_reorder", wid=2, family="gqa", layers=32, heads=8, head_dim=128,
        theta=5e5, rank=16, n_chunks=64, chunk_len=(256, 2048), delta_range=(-32768, 32768),
        q_heads=32,
        note="Llama-3-8B-shaped reorder batch: 32 layers, 8 KV heads x 128, 64 chunks of "
             "256..2048 tokens, per-chunk delta in [-32768, 32768], rank-16 per chunk"),
    "deepseek_v3_mla": Workload(
        key="deepseek_v3_mla", wid=3, family="mla", layers=61, heads=1, head_dim=512,
        theta=1e4, rank=64, tokens=8192, delta=100000,
        note="DeepSeek-V3-shaped MLA: 61 layers, rows c_KV(512) | k_rope(64), T=8192, "
             "delta +100000, rank-64 on both channels"),
    "long_video_72b_paged": Workload(
        key="long_video_72b_paged", wid=4, family="gqa", layers=80, heads=8, head_dim=128,
        theta=1e6, rank=64, tokens=32768, delta=65536, page_size=16, pool_pages=2048, q_heads=64,
        note="72B-shaped long-video paged cache: 80 layers, 8 KV heads x 128, T=32768 in "
             "16-token pages scattered by a random block table, delta +65536, rank-64"),
    "qwen25vl7b_segment_fp8": Workload(
        key="qwen25vl7b_segment_fp8", wid=6, family="gqa", layers=28, heads=4, head_dim=128,
        theta=1e6, rank=32, passes=(0, 32), tokens=4096, delta=-1536, outliers=4, dtype="fp8",
        q_heads=28,
        note="Qwen2.5-VL-7B-shaped video segment in an fp8 E4M3 cache (per-layer scales): "
             "28 layers, 4 KV heads x 128, T=4096, delta -1536; rotation-only pass then "
             "rank-32 patch pass"),
    "long_video_72b_paged_fp8": Workload(
        key="long_video_72b_paged_fp8", wid=7, family="gqa", layers=80, heads=8, head_dim=128,
        theta=1e6, rank=64, tokens=32768, delta=65536, page_size=16, pool_pages=2048,
        dtype="fp8", q_heads=64,
        note="72B-shaped long-video paged cache in fp8 E4M3 (per-layer scales): 80 layers, "
             "8 KV heads x 128, T=32768 in 16-token pages under a random block table, "
             "delta +65536, rank-64"),
    "recall_72b_paged": Workload(
        key="recall_72b_paged", wid=5, family="gqa", layers=80, heads=8, head_dim=128,
        theta=1e6, rank=64, tokens=32768, delta=65536, recall=True, dst_page_size=16,
        dst_pool_pages=2048,
        note="recall of a 72B-shaped long-video segment: canonical contiguous store "
             "(80 layers, 8 KV heads x 128, T=32768) rebuilt with delta +65536 and a rank-64 "
             "patch into a paged cache of 16-token pages under a random block table"),
}


def get(key: str) -> Workload:
    return WORKLOADS[key]


def seed_of(wid: int, kind: int, layer: int = 0, channel: int = 0) -> int:
    ss = np.random.SeedSequence([wid, kind, layer, channel])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def factor_std(m: int) -> float:
    return math.sqrt(0.1 / math.sqrt(m)) if m > 0 else 0.0


# ------------------------------------------------------------------ structure

@dataclass
class Structure:
    offsets: np.ndarray            # int64 [n+1]
    delta: np.ndarray              # int64 [n]
    block_table: np.ndarray | None  # int32 [ceil(T / P)]
    outlier_features: np.ndarray   # int64 [k]

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def num_chunks(self) -> int:
        return int(self.delta.shape[0])


def structure(w: Workload) -> Structure:
    rng = np.random.default_rng(np.random.SeedSequence([w.wid, KIND_STRUCT]))
    if w.lens is not None:
        lens = np.asarray(w.lens, dtype=np.int64)
    elif w.chunk_len is not None:
        lens = rng.integers(w.chunk_len[0], w.chunk_len[1] + 1, size=w.n_chunks)
    else:
        lens = np.full(w.n_chunks, w.tokens, dtype=np.int64)
    n = len(lens)
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    S = len(w.sections) if len(w.sections) > 1 else 1
    shape = (n, S) if S > 1 else (n,)
    if w.deltas is not None:
        delta = np.asarray(w.deltas, dtype=np.int64).reshape(shape)
    elif w.delta_range is not None:
        delta = rng.integers(w.delta_range[0], w.delta_range[1] + 1, size=shape).astype(np.int64)
    elif w.delta_vec is not None:
        delta = np.tile(np.asarray(w.delta_vec, dtype=np.int64), (n, 1)).reshape(shape)
    else:
        delta = np.full(shape, w.delta, dtype=np.int64)
    T = int(offsets[-1])
    bt = None
    if w.page_size > 0:
        need = -(-T // w.page_size)
        pool = max(w.pool_pages, need)
        bt = rng.permutation(pool)[:need].astype(np.int32)
    F = feature_width(w)[0]
    outl = np.sort(rng.choice(F, size=w.outliers, replace=False)) if w.outliers else np.zeros(0, np.int64)
    return Structure(offsets, delta, bt, outl.astype(np.int64))


# ------------------------------------------------------------------ layouts

def feature_width(w: Workload) -> list:
    """Feature width F = heads * dim of each channel."""
    if w.family == "mla":
        return [w.head_dim, w.rope_mla]
    return [w.heads * w.head_dim, w.heads * w.head_dim]


def channel_layouts(w: Workload, total_tokens: int, pool_pages: int = 0) -> list:
    """Per channel: buffer index, element offset, heads, dim, rope_dim and strides."""
    if w.family == "mla":
        row = w.head_dim + w.rope_mla
        ls = total_tokens * row
        return [
            dict(buffer=0, offset=0, heads=1, dim=w.head_dim, rope_dim=0, layer_stride=ls,
                 slot_stride=row, head_stride=w.head_dim, page_stride=0),
            dict(buffer=0, offset=w.head_dim, heads=1, dim=w.rope_mla, rope_dim=w.rope_mla,
                 layer_stride=ls, slot_stride=row, head_stride=w.rope_mla, page_stride=0),
        ]
    H, D = w.heads, w.head_dim
    rk = w.rope_dim or D
    if w.page_size > 0:
        P = w.page_size
        ps = P * H * D
        return [dict(buffer=b, offset=0, heads=H, dim=D, rope_dim=rk if b == 0 else 0,
                     layer_stride=pool_pages * ps, slot_stride=H * D, head_stride=D,
                     page_stride=ps) for b in (0, 1)]
    return [dict(buffer=b, offset=0, heads=H, dim=D, rope_dim=rk if b == 0 else 0,
                 layer_stride=total_tokens * H * D, slot_stride=H * D, head_stride=D,
                 page_stride=0) for b in (0, 1)]


def dst_geometry(w: Workload, total_tokens: int):
    """Recall destination: (page_size, pool pages per layer, block table or None)."""
    P = w.dst_page_size
    if P <= 0:
        return 0, 0, None
    need = -(-total_tokens // P)
    pool = max(w.dst_pool_pages, need)
    rng = np.random.default_rng(np.random.SeedSequence([w.wid, KIND_DST]))
    return P, pool, rng.permutation(pool)[:need].astype(np.int32)


def dst_layouts(w: Workload, total_tokens: int) -> list:
    """Recall destination layout per channel (same keys as channel_layouts)."""
    P, pool, _ = dst_geometry(w, total_tokens)
    if w.family == "mla":
        row = w.head_dim + w.rope_mla
        slots = pool * P if P else total_tokens
        ps = P * row if P else 0
        return [dict(buffer=0, offset=0, heads=1, dim=w.head_dim, rope_dim=0,
                     layer_stride=slots * row, slot_stride=row, head_stride=w.head_dim,
                     page_stride=ps),
                dict(buffer=0, offset=w.head_dim, heads=1, dim=w.rope_mla, rope_dim=w.rope_mla,
                     layer_stride=slots * row, slot_stride=row, head_stride=w.rope_mla,
                     page_stride=ps)]
    return channel_layouts(w.with_(page_size=P), total_tokens, pool)


def dst_buffer_shapes(w: Workload, total_tokens: int) -> list:
    P, pool, _ = dst_geometry(w, total_tokens)
    if w.family == "mla":
        return [(w.layers, (pool * P) if P else total_tokens, w.head_dim + w.rope_mla)]
    return buffer_shapes(w.with_(page_size=P), total_tokens, pool)


def buffer_shapes(w: Workload, total_tokens: int, pool_pages: int = 0) -> list:
    """Shape of each KV buffer (MLA: one combined buffer; GQA/MHA: K and V)."""
    if w.family == "mla":
        return [(w.layers, total_tokens, w.head_dim + w.rope_mla)]
    if w.page_size > 0:
        return [(w.layers, pool_pages, w.page_size, w.heads, w.head_dim)] * 2
    return [(w.layers, total_tokens, w.heads, w.head_dim)] * 2


# ------------------------------------------------------------------ values

@dataclass
class Inputs:
    """One problem instance.  All tensors live on `device`."""
    workload: Workload
    rank: int
    struct: Structure
    pool_pages: int
    buffers: list                  # KV buffers (torch)
    layouts: list                  # per channel layout dicts
    U: list = field(default_factory=list)   # per channel [L][T][m] (torch) or []
    V: list = field(default_factory=list)   # per channel [L][n][F][m]
    offsets_t: object = None
    delta_t: object = None
    block_table_t: object = None
    scales: list = field(default_factory=list)  # fp8: per channel float32 [L]; else []


def _torch_dtype(w: Workload):
    """Storage dtype of the KV buffers (fp8 codes travel as uint8)."""
    import torch
    return {"bf16": torch.bfloat16, "fp8": torch.uint8}.get(w.dtype, torch.float32)


def _factor_dtype(w: Workload):
    import torch
    return torch.bfloat16 if w.dtype in ("bf16", "fp8") else torch.float32


def _quantize_fp8(buffers, layouts, layers: int):
    """fp32 value buffers -> (uint8 E4M3 code buffers, per channel [L] scales):
    s = max |value| / 224 over each (layer, channel), codes = E4M3(value / s)."""
    import torch
    codes = [torch.empty(b.shape, dtype=torch.uint8, device=b.device) for b in buffers]
    scales = []
    for lay in layouts:
        src = buffers[lay["buffer"]]
        dst = codes[lay["buffer"]]
        sl = slice(None)
        if src.dim() == 3 and src.shape[-1] != lay["dim"] * lay["heads"]:  # MLA row slice
            sl = slice(lay["offset"], lay["offset"] + lay["dim"])
        sc = torch.empty(layers, dtype=torch.float32, device=src.device)
        for l in range(layers):
            v = src[l][..., sl] if sl != slice(None) else src[l]
            amax = float(v.abs().max())
            sc[l] = (amax if amax > 0 else 1.0) / 224.0
            q = (v / sc[l]).to(torch.float8_e4m3fn).view(torch.uint8)
            if sl != slice(None):
                dst[l][..., sl] = q
            else:
                dst[l].copy_(q)
        scales.append(sc)
    return codes, scales


def _normal(shape, seed: int, std: float, device, dtype):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_inputs(w: Workload, rank: int, device="cpu", pass_id: int = 0) -> Inputs:
    """Draw every input of one call.  `pass_id` shifts the seeds so that a second
    pass of the same workload gets fresh values."""
    import torch
    st = structure(w)
    T = st.total_tokens
    pool = 0
    if w.page_size > 0:
        pool = max(w.pool_pages, -(-T // w.page_size))
    q8 = w.dtype == "fp8"
    dt = torch.float32 if q8 else _torch_dtype(w)
    ft = _factor_dtype(w)
    wid = w.wid + 1000 * pass_id
    shapes = buffer_shapes(w, T, pool)
    buffers = []
    for b, shp in enumerate(shapes):
        buf = torch.empty(shp, dtype=dt, device=device)
        for l in range(w.layers):
            buf[l] = _normal(shp[1:], seed_of(wid, KIND_KV, l, b), 1.0, device, dt)
        buffers.append(buf)
    layouts = channel_layouts(w, T, pool)
    if st.outlier_features.size and w.family != "mla":
        idx = torch.as_tensor(st.outlier_features, device=device)
        for buf in buffers:
            flat = buf.view(w.layers, -1, w.heads * w.head_dim)
            flat[:, :, idx] = flat[:, :, idx] * w.outlier_scale
    scales = []
    if q8:
        buffers, scales = _quantize_fp8(buffers, layouts, w.layers)
    U, V = [], []
    if rank > 0:
        s = factor_std(rank)
        for c, F in enumerate(feature_width(w)):
            u = torch.empty((w.layers, T, rank), dtype=ft, device=device)
            v = torch.empty((w.layers, st.num_chunks, F, rank), dtype=ft, device=device)
            for l in range(w.layers):
                u[l] = _normal((T, rank), seed_of(wid, KIND_U, l, c), s, device, ft)
                v[l] = _normal((st.num_chunks, F, rank), seed_of(wid, KIND_V, l, c), s, device, ft)
            U.append(u)
            V.append(v)
    inp = Inputs(w, rank, st, pool, buffers, layouts, U, V, scales=scales)
    inp.offsets_t = torch.as_tensor(st.offsets, device=device)
    inp.delta_t = torch.as_tensor(st.delta, device=device)
    if st.block_table is not None:
        inp.block_table_t = torch.as_tensor(st.block_table, device=device)
    return inp


@dataclass
class RecallInputs:
    """A recall problem: the canonical store (with chunks and factors) and the
    destination cache."""
    src: Inputs
    dst_buffers: list
    dst_layouts: list
    dst_page_size: int
    dst_pool_pages: int
    dst_block_table: np.ndarray | None
    dst_block_table_t: object = None

    @property
    def workload(self) -> Workload:
        return self.src.workload

    @property
    def rank(self) -> int:
        return self.src.rank


def make_recall_inputs(w: Workload, rank: int, device="cpu", pass_id: int = 0) -> RecallInputs:
    """Canonical store as make_inputs draws it, and a destination pre-filled with
    DST_SENTINEL (or 0x7FC00001 for fp32)."""
    import torch
    src = make_inputs(w, rank, device, pass_id)
    T = src.struct.total_tokens
    P, pool, table = dst_geometry(w, T)
    dt = _torch_dtype(w)
    bufs = []
    for shp in dst_buffer_shapes(w, T):
        if dt == torch.bfloat16:
            b = torch.full(shp, DST_SENTINEL, dtype=torch.int16, device=device).view(torch.bfloat16)
        elif dt == torch.uint8:
            b = torch.full(shp, DST_SENTINEL_FP8, dtype=torch.uint8, device=device)
        else:
            b = torch.full(shp, 0x7FC00001, dtype=torch.int32, device=device).view(torch.float32)
        bufs.append(b)
    r = RecallInputs(src, bufs, dst_layouts(w, T), P, pool, table)
    if table is not None:
        r.dst_block_table_t = torch.as_tensor(table, device=device)
    return r


# ------------------------------------------------------------------ decode attention input

def make_query(w: Workload, device="cpu", pass_id: int = 0):
    """Decode queries [L][Hq][head_dim] fp32 ~ N(0, 1), Hq = w.q_heads (or the KV
    heads): one new token's query per layer, already rotated to its own position."""
    import torch
    hq = w.q_heads or w.heads
    q = torch.empty((w.layers, hq, w.head_dim), dtype=torch.float32, device=device)
    for l in range(w.layers):
        q[l] = _normal((hq, w.head_dim), seed_of(w.wid + 1000 * pass_id, KIND_QUERY, l), 1.0,
                       device, torch.float32)
    return q


# ------------------------------------------------------------------ patch formation input

KIND_DEFICIT = 5


def make_deficit(w: Workload, device="cpu", directions: int = 32, decay: float = 0.85,
                 rms: float = 0.1, noise: float = 0.005) -> list:
    """Synthetic reuse deficits Delta [L][T][F] (one bf16 tensor per channel): per layer
    and chunk, sum_k s_k a_k b_k^T over `directions` feature directions plus N(0, noise^2)
    entries, with s_k falling geometrically by `decay` and the signal scaled to `rms`
    per entry.  The Kamera summary (section 3) reports the deficit's energy concentrated
    in about 32 feature directions; a_k and b_k are Gaussian columns scaled to unit
    expected norm (nearly orthonormal for T, F >> directions)."""
    import torch
    st = structure(w)
    T = st.total_tokens
    out = []
    for c, F in enumerate(feature_width(w)):
        buf = torch.zeros((w.layers, T, F), dtype=torch.bfloat16, device=device)
        for l in range(w.layers):
            g = torch.Generator(device=device)
            g.manual_seed(seed_of(w.wid, KIND_DEFICIT, l, c))
            for j in range(st.num_chunks):
                a, b = int(st.offsets[j]), int(st.offsets[j + 1])
                Tj = b - a
                if Tj == 0:
                    continue
                r = min(directions, Tj, F)
                s = decay ** torch.arange(r, dtype=torch.float32, device=device)
                s *= rms * math.sqrt(Tj * F) / float(torch.linalg.vector_norm(s))
                A = torch.randn((Tj, r), generator=g, device=device) / math.sqrt(Tj)
                B = torch.randn((F, r), generator=g, device=device) / math.sqrt(F)
                d = (A * s) @ B.T + noise * torch.randn((Tj, F), generator=g, device=device)
                buf[l, a:b] = d.to(torch.bfloat16)
        out.append(buf)
    return out


# ------------------------------------------------------------------ accounting

def algorithmic_bytes(w: Workload, rank: int, total_tokens: int | None = None,
                      num_chunks: int | None = None) -> int:
    """Bytes an ideal pass moves: every touched KV element read once and written once,
    every factor element read once.  In place with rank 0 only the rotated dims of
    rotating channels move (chunks with delta 0 would move nothing; no workload here
    has one); a recall reads every source row and writes every destination row whole.
    Block tables, offsets and deltas are not counted."""
    if total_tokens is None or num_chunks is None:
        st = structure(w)
        total_tokens, num_chunks = st.total_tokens, st.num_chunks
    es, fs = w.elem_size, w.factor_size
    T, L, n = total_tokens, w.layers, num_chunks
    lay = channel_layouts(w, T, 0)
    total = 0
    for c in lay:
        F = c["heads"] * c["dim"]
        if rank == 0 and w.recall:  # recall copies every row whole
            total += 2 * es * F * T * L
        elif rank == 0:
            total += 2 * es * c["heads"] * c["rope_dim"] * T * L
        else:
            total += L * (2 * es * F * T + fs * rank * T + fs * F * rank * n)
    return total


def patch_flops(w: Workload, rank: int) -> int:
    st = structure(w)
    return sum(2 * rank * F * st.total_tokens * w.layers for F in feature_width(w))


def patch_to_kv_ratio(w: Workload, rank: int) -> float:
    """Bytes of the stored patch (U and V) over bytes of the segment's KV."""
    st = structure(w)
    es, fs, T, n = w.elem_size, w.factor_size, st.total_tokens, st.num_chunks
    kv = sum(F * T * es for F in feature_width(w))
    pat = sum(fs * rank * (T + F * n) for F in feature_width(w))
    return pat / kv

"""Torch front end: builds the C descriptors for a problem held in torch tensors and
enqueues the library call.  Argument marshalling only; the HIP kernels do all work."""
from __future__ import annotations

from . import kamera as K


def descriptors(buffers, layouts, *, dtype_code: int, num_layers: int, theta: float,
                offsets_t, delta_t, total_tokens: int, rank: int = 0, U=(), V=(),
                page_size: int = 0, num_pages: int = 0, block_table_t=None, flags: int = 0,
                pairing: int = 0, sections=(), scales=()):
    """Descriptors for channels laid out as `layouts` (dicts with buffer, offset,
    heads, dim, rope_dim and element strides) over the KV tensors in `buffers`;
    `scales`: fp8 per-channel [layers] float32 device tensors."""
    chans = []
    for c, lay in enumerate(layouts):
        chans.append(K.channel(buffers[lay["buffer"]], heads=lay["heads"], dim=lay["dim"],
                               rope_dim=lay["rope_dim"], layer_stride=lay["layer_stride"],
                               slot_stride=lay["slot_stride"], head_stride=lay["head_stride"],
                               page_stride=lay.get("page_stride", 0),
                               element_offset=lay.get("offset", 0),
                               scale=scales[c] if c < len(scales) else None))
    kv = K.kv_desc(chans, dtype=dtype_code, num_layers=num_layers, rope_theta=theta,
                   page_size=page_size, num_pages=num_pages, block_table=block_table_t,
                   flags=flags, pairing=pairing, sections=sections)
    ch = K.chunks_desc(offsets_t, delta_t, total_tokens)
    Us = list(U) + [None] * (2 - len(U))
    Vs = list(V) + [None] * (2 - len(V))
    patch = K.patch_desc(rank, Us, Vs) if rank > 0 else None
    return kv, ch, patch


def descriptors_for(inp, flags: int = 0):
    """Descriptors for a synth.Inputs instance."""
    w = inp.workload
    code = K._dtype_code(inp.buffers[0])
    return descriptors(inp.buffers, inp.layouts, dtype_code=code, num_layers=w.layers,
                       theta=w.theta, offsets_t=inp.offsets_t, delta_t=inp.delta_t,
                       total_tokens=inp.struct.total_tokens, rank=inp.rank, U=inp.U, V=inp.V,
                       page_size=w.page_size, num_pages=inp.pool_pages,
                       block_table_t=inp.block_table_t, flags=flags, pairing=w.pairing,
                       sections=w.sections, scales=inp.scales)


def run(inp, stream=None, flags: int = 0) -> None:
    """Apply the operator in place to the tensors of `inp` on `stream`."""
    kv, ch, patch = descriptors_for(inp, flags)
    K.relocate_patch_(kv, ch, patch, stream)


def workspace_for(inp, flags: int = 0):
    """Workspace tensor for kamera_relocate_patch_ws on `inp` (None when it needs none)."""
    import torch
    kv, ch, patch = descriptors_for(inp, flags)
    st, nbytes = K.kamera_relocate_workspace(kv, ch, patch)
    K.check(st)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=inp.buffers[0].device)


def run_ws(inp, workspace=None, stream=None, flags: int = 0) -> None:
    """Apply the operator in place through kamera_relocate_patch_ws (pool order when the
    problem takes it); `workspace` from workspace_for, or None to size one here."""
    kv, ch, patch = descriptors_for(inp, flags)
    if workspace is None:
        workspace = workspace_for(inp, flags)
    K.relocate_patch_ws_(kv, ch, patch, workspace, stream)


def plan(inp, flags: int = 0):
    kv, ch, patch = descriptors_for(inp, flags)
    st, info = K.kamera_plan(kv, ch, patch)
    K.check(st)
    return info


def recall_descriptors(rinp, flags: int = 0):
    """(src, dst, chunks, patch) descriptors for a synth.RecallInputs instance."""
    src, ch, patch = descriptors_for(rinp.src, flags)
    w = rinp.workload
    code = K._dtype_code(rinp.dst_buffers[0])
    chans = []
    for lay in rinp.dst_layouts:
        chans.append(K.channel(rinp.dst_buffers[lay["buffer"]], heads=lay["heads"], dim=lay["dim"],
                               rope_dim=lay["rope_dim"], layer_stride=lay["layer_stride"],
                               slot_stride=lay["slot_stride"], head_stride=lay["head_stride"],
                               page_stride=lay.get("page_stride", 0),
                               element_offset=lay.get("offset", 0)))
    dst = K.kv_desc(chans, dtype=code, num_layers=w.layers, rope_theta=w.theta,
                    page_size=rinp.dst_page_size, num_pages=rinp.dst_pool_pages,
                    block_table=rinp.dst_block_table_t, flags=flags)
    return src, dst, ch, patch


def run_recall(rinp, stream=None, flags: int = 0) -> None:
    """Recall: rebuild the chunks of `rinp.src` into `rinp`'s destination on `stream`."""
    src, dst, ch, patch = recall_descriptors(rinp, flags)
    K.recall_patch(src, dst, ch, patch, stream)


def recall_plan(rinp, flags: int = 0):
    src, dst, ch, patch = recall_descriptors(rinp, flags)
    st, info = K.kamera_recall_plan(src, dst, ch, patch)
    K.check(st)
    return info


def attend_buffers(inp, q, scale: float, flags: int = 0):
    """(descriptors, out, lse, workspace) for relocate-on-read attention of query `q`
    [L][Hq][128] fp32 over the cache of a synth.Inputs instance."""
    import torch
    kv, ch, patch = descriptors_for(inp, flags)
    L, Hq, D = q.shape
    out = torch.empty((L, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((L, Hq), dtype=torch.float32, device=q.device)
    desc = K.attend_desc(q, out, scale=scale, lse=lse)
    st, nbytes = K.kamera_attend_workspace(kv, ch, patch, desc)
    K.check(st)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device) if nbytes else None
    return (kv, ch, patch, desc), out, lse, ws


def attend(inp, q, scale: float, stream=None, flags: int = 0):
    """Relocate-on-read decode attention: returns (out [L][Hq][128], lse [L][Hq])."""
    (kv, ch, patch, desc), out, lse, ws = attend_buffers(inp, q, scale, flags)
    K.attend(kv, ch, patch, desc, ws, stream)
    return out, lse

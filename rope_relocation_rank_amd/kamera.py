"""ctypes binding of libkamera.so (include/kamera.h): argument marshalling only.

The entry points keep their C names: ``kamera_relocate``, ``kamera_relocate_patch``,
``kamera_plan``, ``kamera_status_str``, ``kamera_last_error``, ``kamera_abi_version``.
Descriptors are the ctypes mirrors of the C structs.  ``desc_from_tensors`` and the
``relocate_`` / ``relocate_patch_`` helpers fill them from torch tensors (device
memory and streams are all torch is used for); every step of the operator runs in
the library's HIP kernels.  A missing library raises: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkamera.so")

KAMERA_OK, KAMERA_E_NULL, KAMERA_E_SHAPE, KAMERA_E_UNSUPPORTED = 0, 1, 2, 3
KAMERA_E_ALIGN, KAMERA_E_ALIAS, KAMERA_E_HIP = 4, 5, 6
KAMERA_BF16, KAMERA_F32, KAMERA_FP8_E4M3 = 0, 1, 2
KAMERA_ABI_VERSION = 5
KAMERA_NEOX_HALF = 0
KAMERA_INTERLEAVED = 1
KAMERA_FLAG_GENERIC = 1
KAMERA_MAX_RANK = 256
KERNEL_NAMES = {0: "none", 1: "rotate", 2: "rotate+patch mfma", 3: "generic"}

EXPORTED = ["kamera_relocate", "kamera_relocate_patch", "kamera_relocate_patch_ws",
            "kamera_relocate_patch_noalloc",
            "kamera_relocate_workspace", "kamera_recall_patch", "kamera_plan",
            "kamera_recall_plan", "kamera_form_workspace", "kamera_form_patch", "kamera_form_gram",
            "kamera_orbit_mean", "kamera_attend_workspace", "kamera_attend",
            "kamera_status_str", "kamera_last_error", "kamera_abi_version"]
KAMERA_FORM_MAX_RANK = 112


class kamera_channel(C.Structure):
    _fields_ = [("data", C.c_void_p), ("heads", C.c_int32), ("dim", C.c_int32),
                ("rope_dim", C.c_int32), ("reserved0", C.c_int32),
                ("layer_stride", C.c_int64), ("slot_stride", C.c_int64),
                ("head_stride", C.c_int64), ("page_stride", C.c_int64),
                ("scale", C.c_void_p)]


class kamera_kv_desc(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("num_layers", C.c_int32), ("num_channels", C.c_int32),
                ("pairing", C.c_int32), ("ch", kamera_channel * 2), ("rope_theta", C.c_double),
                ("page_size", C.c_int32), ("flags", C.c_uint32), ("num_pages", C.c_int64),
                ("block_table", C.c_void_p), ("num_sections", C.c_int32),
                ("section_pairs", C.c_int32 * 4), ("reserved1", C.c_int32)]


class kamera_chunks(C.Structure):
    _fields_ = [("num_chunks", C.c_int32), ("reserved0", C.c_int32),
                ("total_tokens", C.c_int64), ("token_offsets", C.c_void_p),
                ("delta", C.c_void_p)]


class kamera_patch(C.Structure):
    _fields_ = [("rank", C.c_int32), ("reserved0", C.c_int32),
                ("U", C.c_void_p * 2), ("V", C.c_void_p * 2)]


class kamera_form_desc(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("num_layers", C.c_int32), ("num_channels", C.c_int32),
                ("rank", C.c_int32), ("width", C.c_int32 * 2), ("iterations", C.c_int32),
                ("reserved0", C.c_int32), ("delta", C.c_void_p * 2), ("U", C.c_void_p * 2),
                ("V", C.c_void_p * 2), ("sigma", C.c_void_p * 2)]


class kamera_attend_desc(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("reserved0", C.c_int32), ("scale", C.c_float),
                ("reserved1", C.c_int32), ("q", C.c_void_p), ("out", C.c_void_p),
                ("lse", C.c_void_p)]


class kamera_plan_info(C.Structure):
    _fields_ = [("kernel", C.c_int32 * 2), ("launches", C.c_int32),
                ("tokens_per_unit", C.c_int32), ("units", C.c_int64)]


class KameraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kamera status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def lib():
    """Load libkamera.so from the package directory (built by build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        L.kamera_relocate.restype = C.c_int
        L.kamera_relocate.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_chunks), C.c_void_p]
        L.kamera_relocate_patch.restype = C.c_int
        L.kamera_relocate_patch.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_chunks),
                                            C.POINTER(kamera_patch), C.c_void_p]
        L.kamera_relocate_patch_ws.restype = C.c_int
        L.kamera_relocate_patch_ws.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_chunks),
                                               C.POINTER(kamera_patch), C.c_void_p, C.c_int64,
                                               C.c_void_p]
        L.kamera_relocate_patch_noalloc.restype = C.c_int
        L.kamera_relocate_patch_noalloc.argtypes = [C.POINTER(kamera_kv_desc),
                                                    C.POINTER(kamera_chunks),
                                                    C.POINTER(kamera_patch), C.c_void_p]
        L.kamera_relocate_workspace.restype = C.c_int
        L.kamera_relocate_workspace.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_chunks),
                                                C.POINTER(kamera_patch), C.POINTER(C.c_int64)]
        L.kamera_plan.restype = C.c_int
        L.kamera_plan.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_chunks),
                                  C.POINTER(kamera_patch), C.POINTER(kamera_plan_info)]
        L.kamera_recall_patch.restype = C.c_int
        L.kamera_recall_patch.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_kv_desc),
                                          C.POINTER(kamera_chunks), C.POINTER(kamera_patch),
                                          C.c_void_p]
        L.kamera_recall_plan.restype = C.c_int
        L.kamera_recall_plan.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_kv_desc),
                                         C.POINTER(kamera_chunks), C.POINTER(kamera_patch),
                                         C.POINTER(kamera_plan_info)]
        L.kamera_form_workspace.restype = C.c_int
        L.kamera_form_workspace.argtypes = [C.POINTER(kamera_form_desc), C.POINTER(kamera_chunks),
                                            C.POINTER(C.c_int64)]
        L.kamera_form_patch.restype = C.c_int
        L.kamera_form_patch.argtypes = [C.POINTER(kamera_form_desc), C.POINTER(kamera_chunks),
                                        C.c_void_p, C.c_int64, C.c_void_p]
        L.kamera_form_gram.restype = C.c_int
        L.kamera_form_gram.argtypes = [C.POINTER(kamera_form_desc), C.POINTER(kamera_chunks),
                                       C.POINTER(C.c_void_p), C.c_void_p]
        L.kamera_orbit_mean.restype = C.c_int
        L.kamera_orbit_mean.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int64, C.c_void_p,
                                        C.c_void_p]
        L.kamera_attend_workspace.restype = C.c_int
        L.kamera_attend_workspace.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_chunks),
                                              C.POINTER(kamera_patch), C.POINTER(kamera_attend_desc),
                                              C.POINTER(C.c_int64)]
        L.kamera_attend.restype = C.c_int
        L.kamera_attend.argtypes = [C.POINTER(kamera_kv_desc), C.POINTER(kamera_chunks),
                                    C.POINTER(kamera_patch), C.POINTER(kamera_attend_desc),
                                    C.c_void_p, C.c_int64, C.c_void_p]
        L.kamera_status_str.restype = C.c_char_p
        L.kamera_status_str.argtypes = [C.c_int]
        L.kamera_last_error.restype = C.c_char_p
        L.kamera_last_error.argtypes = []
        L.kamera_abi_version.restype = C.c_int
        L.kamera_abi_version.argtypes = []
        _lib = L
    return _lib


# ------------------------------------------------------------- C entry points

def kamera_relocate(kv: kamera_kv_desc, chunks: kamera_chunks, stream) -> int:
    return lib().kamera_relocate(C.byref(kv), C.byref(chunks), stream)


def kamera_relocate_patch(kv: kamera_kv_desc, chunks: kamera_chunks, patch, stream) -> int:
    return lib().kamera_relocate_patch(C.byref(kv), C.byref(chunks),
                                       None if patch is None else C.byref(patch), stream)


def kamera_relocate_patch_ws(kv: kamera_kv_desc, chunks: kamera_chunks, patch, workspace,
                             workspace_bytes: int, stream) -> int:
    return lib().kamera_relocate_patch_ws(_ref(kv), _ref(chunks), _ref(patch), workspace,
                                          workspace_bytes, stream)


def kamera_relocate_patch_noalloc(kv: kamera_kv_desc, chunks: kamera_chunks, patch,
                                  stream) -> int:
    return lib().kamera_relocate_patch_noalloc(_ref(kv), _ref(chunks), _ref(patch), stream)


def kamera_relocate_workspace(kv, chunks, patch=None):
    n = C.c_int64(0)
    st = lib().kamera_relocate_workspace(_ref(kv), _ref(chunks), _ref(patch), C.byref(n))
    return st, n.value


def kamera_plan(kv, chunks, patch=None):
    info = kamera_plan_info()
    st = lib().kamera_plan(None if kv is None else C.byref(kv),
                           None if chunks is None else C.byref(chunks),
                           None if patch is None else C.byref(patch), C.byref(info))
    return st, info


def _ref(x):
    return None if x is None else C.byref(x)


def kamera_recall_patch(src: kamera_kv_desc, dst: kamera_kv_desc, chunks: kamera_chunks, patch,
                        stream) -> int:
    return lib().kamera_recall_patch(_ref(src), _ref(dst), _ref(chunks), _ref(patch), stream)


def kamera_recall_plan(src, dst, chunks, patch=None):
    info = kamera_plan_info()
    st = lib().kamera_recall_plan(_ref(src), _ref(dst), _ref(chunks), _ref(patch), C.byref(info))
    return st, info


def kamera_status_str(status: int) -> str:
    return lib().kamera_status_str(status).decode()


def kamera_last_error() -> str:
    return lib().kamera_last_error().decode()


def kamera_abi_version() -> int:
    return lib().kamera_abi_version()


def check(status: int) -> None:
    if status != KAMERA_OK:
        raise KameraError(status, kamera_last_error() or kamera_status_str(status))


# ------------------------------------------------------------- torch helpers

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KAMERA_BF16
    if t.dtype == torch.float32:
        return KAMERA_F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return KAMERA_FP8_E4M3
    raise TypeError(f"unsupported KV dtype {t.dtype}")


def channel(data, *, heads: int, dim: int, rope_dim: int, layer_stride: int,
            slot_stride: int, head_stride: int, page_stride: int = 0,
            element_offset: int = 0, scale=None) -> kamera_channel:
    """Channel view over a tensor's storage; strides in elements.  `scale`: fp8 KV's
    float32 [num_layers] dequantisation scales (a device tensor)."""
    c = kamera_channel()
    c.data = data.data_ptr() + element_offset * data.element_size()
    c.heads, c.dim, c.rope_dim, c.reserved0 = heads, dim, rope_dim, 0
    c.layer_stride, c.slot_stride = layer_stride, slot_stride
    c.head_stride, c.page_stride = head_stride, page_stride
    c.scale = None if scale is None else scale.data_ptr()
    return c


def kv_desc(channels, *, dtype: int, num_layers: int, rope_theta: float, page_size: int = 0,
            num_pages: int = 0, block_table=None, flags: int = 0,
            pairing: int = 0, sections=()) -> kamera_kv_desc:
    """KV descriptor.  `pairing`: KAMERA_NEOX_HALF or KAMERA_INTERLEAVED; `sections`:
    M-RoPE rotary pairs per section (then the chunk deltas are [chunks][sections])."""
    d = kamera_kv_desc()
    d.dtype, d.num_layers, d.num_channels = dtype, num_layers, len(channels)
    d.pairing = pairing
    sec = list(sections)
    if len(sec) > 4:
        raise ValueError("at most 4 M-RoPE sections")
    d.num_sections = len(sec) if len(sec) > 1 else 0
    for k, v in enumerate(sec):
        d.section_pairs[k] = v
    for i, c in enumerate(channels):
        d.ch[i] = c
    d.rope_theta = rope_theta
    d.page_size, d.flags, d.num_pages = page_size, flags, num_pages
    d.block_table = None if block_table is None else block_table.data_ptr()
    return d


def chunks_desc(offsets, delta, total_tokens: int) -> kamera_chunks:
    """offsets: int64 device tensor [n+1]; delta: int64 device tensor [n], or [n][S]
    with M-RoPE sections (contiguous)."""
    c = kamera_chunks()
    c.num_chunks = int(delta.shape[0]) if delta.dim() else 1
    c.reserved0 = 0
    c.total_tokens = int(total_tokens)
    c.token_offsets = offsets.data_ptr() if offsets.numel() else None
    c.delta = delta.data_ptr() if delta.numel() else None
    return c


def patch_desc(rank: int, U=(None, None), V=(None, None)) -> kamera_patch:
    p = kamera_patch()
    p.rank, p.reserved0 = rank, 0
    for i in range(2):
        p.U[i] = None if U[i] is None else U[i].data_ptr()
        p.V[i] = None if V[i] is None else V[i].data_ptr()
    return p


def current_stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def relocate_patch_(kv: kamera_kv_desc, chunks: kamera_chunks, patch=None, stream=None) -> None:
    """Enqueue the operator on `stream` (default: torch's current stream); raise on error."""
    s = current_stream() if stream is None else stream
    if patch is None or patch.rank == 0:
        check(kamera_relocate(kv, chunks, s))
    else:
        check(kamera_relocate_patch(kv, chunks, patch, s))


def relocate_patch_ws_(kv: kamera_kv_desc, chunks: kamera_chunks, patch, workspace,
                       stream=None) -> None:
    """Enqueue kamera_relocate_patch_ws; `workspace` is a torch uint8 tensor (or None)."""
    s = current_stream() if stream is None else stream
    ws = None if workspace is None else workspace.data_ptr()
    nb = 0 if workspace is None else workspace.numel()
    check(kamera_relocate_patch_ws(kv, chunks, patch, ws, nb, s))


def recall_patch(src: kamera_kv_desc, dst: kamera_kv_desc, chunks: kamera_chunks, patch=None,
                 stream=None) -> None:
    """Enqueue a recall (out of place) on `stream` (default: torch's current stream)."""
    s = current_stream() if stream is None else stream
    check(kamera_recall_patch(src, dst, chunks, patch, s))


def form_desc(deltas, U, V, *, num_layers: int, rank: int, sigma=None,
              iterations: int = 0) -> kamera_form_desc:
    """Patch-formation descriptor over torch tensors: deltas [L][T][F] bf16 per channel,
    U [L][T][m], V [L][n][F][m] (bf16) and optional sigma [L][n][m] (fp32) outputs."""
    d = kamera_form_desc()
    d.dtype, d.num_layers, d.num_channels, d.rank = KAMERA_BF16, num_layers, len(deltas), rank
    d.iterations, d.reserved0 = iterations, 0
    for c, t in enumerate(deltas):
        d.width[c] = int(t.shape[-1])
        d.delta[c] = t.data_ptr()
        d.U[c] = U[c].data_ptr()
        d.V[c] = V[c].data_ptr()
        d.sigma[c] = None if sigma is None else sigma[c].data_ptr()
    return d


def kamera_form_workspace(desc, chunks):
    n = C.c_int64(0)
    st = lib().kamera_form_workspace(_ref(desc), _ref(chunks), C.byref(n))
    return st, n.value


def form_patch(desc: kamera_form_desc, chunks: kamera_chunks, workspace, stream=None) -> None:
    """Enqueue patch formation; `workspace` is a torch uint8 tensor (256-byte aligned)."""
    s = current_stream() if stream is None else stream
    check(lib().kamera_form_patch(C.byref(desc), C.byref(chunks), workspace.data_ptr(),
                                  workspace.numel(), s))


def form_gram(desc: kamera_form_desc, chunks: kamera_chunks, G, stream=None) -> None:
    """Enqueue the Gram stage: G[c] fp32 tensors [L][n][F][F]."""
    s = current_stream() if stream is None else stream
    arr = (C.c_void_p * 2)(*[g.data_ptr() for g in G] + [None] * (2 - len(G)))
    check(lib().kamera_form_gram(C.byref(desc), C.byref(chunks), arr, s))


def orbit_mean(deltas, out, stream=None) -> None:
    """Enqueue the orbit mean: deltas a torch bf16 tensor [P][...] (contiguous), out a
    bf16 tensor with deltas[0]'s elements."""
    s = current_stream() if stream is None else stream
    P = deltas.shape[0]
    n = out.numel()
    stride = deltas[0].numel() if P > 0 else 0
    check(lib().kamera_orbit_mean(deltas.data_ptr(), P, n, stride, out.data_ptr(), s))


# ------------------------------------------------------------- relocate-on-read attention

def attend_desc(q, out, *, scale: float, lse=None) -> kamera_attend_desc:
    """Attention descriptor over torch tensors: q and out [L][Hq][128] fp32, lse [L][Hq]."""
    d = kamera_attend_desc()
    d.num_q_heads = q.shape[1]
    d.reserved0 = d.reserved1 = 0
    d.scale = float(scale)
    d.q = q.data_ptr()
    d.out = out.data_ptr()
    d.lse = None if lse is None else lse.data_ptr()
    return d


def kamera_attend_workspace(kv, chunks, patch, attend):
    n = C.c_int64(0)
    st = lib().kamera_attend_workspace(_ref(kv), _ref(chunks), _ref(patch), _ref(attend),
                                       C.byref(n))
    return st, n.value


def attend(kv: kamera_kv_desc, chunks: kamera_chunks, patch, desc: kamera_attend_desc,
           workspace, stream=None) -> None:
    """Enqueue relocate-on-read decode attention; `workspace` is a torch uint8 tensor of
    at least kamera_attend_workspace bytes (or None when that is 0)."""
    s = current_stream() if stream is None else stream
    ws = None if workspace is None else workspace.data_ptr()
    nb = 0 if workspace is None else workspace.numel()
    check(lib().kamera_attend(C.byref(kv), C.byref(chunks), _ref(patch), C.byref(desc), ws, nb, s))

"""ctypes front end of the fp64 CPU oracle (kamera_oracle.c).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this module.  It shares no code with
the GPU library: it has its own C source, its own structs and its own loader.

Every array argument is a numpy array in storage format: bf16 values travel as
``uint16`` bit patterns, fp32 values as ``float32``, fp8 E4M3 codes as ``uint8``
(with bf16 factors and a per-layer float32 scale per channel).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kamera_oracle.c")
LIB = os.path.join(HERE, "libkamera_oracle.so")

BF16 = 0
F32 = 1
FP8 = 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE fp64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-shared", "-fPIC", "-Wall", SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class _Channel(C.Structure):
    _fields_ = [("data", C.c_void_p), ("heads", C.c_int32), ("dim", C.c_int32),
                ("rope_dim", C.c_int32), ("pad_", C.c_int32),
                ("layer_stride", C.c_int64), ("slot_stride", C.c_int64),
                ("head_stride", C.c_int64), ("page_stride", C.c_int64),
                ("U", C.c_void_p), ("V", C.c_void_p), ("scale", C.c_void_p)]


class _Rope(C.Structure):
    _fields_ = [("pairing", C.c_int32), ("num_sections", C.c_int32),
                ("section_pairs", C.c_int32 * 4)]


class _Problem(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("num_layers", C.c_int32),
                ("num_channels", C.c_int32), ("page_size", C.c_int32),
                ("ch", _Channel * 2), ("theta", C.c_double),
                ("block_table", C.c_void_p), ("total_tokens", C.c_int64),
                ("offsets", C.c_void_p), ("delta", C.c_void_p),
                ("num_chunks", C.c_int32), ("rank", C.c_int32),
                ("rope", _Rope)]


NEOX = 0
INTERLEAVED = 1


def _rope(pairing: int = NEOX, sections=()) -> _Rope:
    """Pairing (0 NeoX half-split, 1 interleaved) and M-RoPE sections (pairs per
    section, in pair order; empty or one entry = plain RoPE)."""
    q = _Rope()
    q.pairing = pairing
    sec = list(sections)
    assert len(sec) <= 4
    q.num_sections = len(sec) if len(sec) > 1 else 0
    for k, v in enumerate(sec):
        q.section_pairs[k] = v
    return q


def _delta_vec(delta) -> np.ndarray:
    return np.ascontiguousarray(np.atleast_1d(np.asarray(delta, dtype=np.int64)))


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()  # rebuilds when the source is newer than the library
        L = C.CDLL(LIB)
        L.orc_bf16_from_double.restype = C.c_uint16
        L.orc_bf16_from_double.argtypes = [C.c_double]
        L.orc_bf16_to_double.restype = C.c_double
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_round_bf16_array.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        L.orc_fp8_to_double.restype = C.c_double
        L.orc_fp8_to_double.argtypes = [C.c_uint8]
        L.orc_fp8_from_double.restype = C.c_uint8
        L.orc_fp8_from_double.argtypes = [C.c_double]
        L.orc_fp8_from_double_array.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        L.orc_row_spec_scaled.restype = C.c_int
        L.orc_row_spec_scaled.argtypes = [C.c_int, C.c_double, C.c_void_p, C.c_void_p, C.c_int,
                                          C.c_int, C.c_int, C.c_double, C.c_void_p,
                                          C.POINTER(_Rope), C.c_int, C.c_void_p, C.c_void_p]
        L.orc_freq.restype = C.c_double
        L.orc_freq.argtypes = [C.c_double, C.c_int, C.c_int]
        L.orc_rotate_head_f64.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                          C.c_double, C.c_int64]
        L.orc_row_f64.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                  C.c_double, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
        L.orc_row.restype = C.c_int
        L.orc_row.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                              C.c_double, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
        L.orc_relocate_patch.restype = C.c_int
        L.orc_relocate_patch.argtypes = [C.POINTER(_Problem)]
        L.orc_relocate_patch_ex.restype = C.c_int
        L.orc_relocate_patch_ex.argtypes = [C.POINTER(_Problem), C.POINTER(C.c_void_p),
                                            C.POINTER(C.c_void_p)]
        L.orc_recall_patch_ex.restype = C.c_int
        L.orc_recall_patch_ex.argtypes = [C.POINTER(_Problem), C.POINTER(_Problem),
                                          C.POINTER(C.c_void_p), C.POINTER(C.c_void_p)]
        L.orc_rotate_head_spec_f64.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                               C.c_double, C.c_void_p, C.POINTER(_Rope)]
        L.orc_row_spec_f64.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                       C.c_double, C.c_void_p, C.POINTER(_Rope), C.c_int,
                                       C.c_void_p, C.c_void_p]
        L.orc_row_spec.restype = C.c_int
        L.orc_row_spec.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                   C.c_double, C.c_void_p, C.POINTER(_Rope), C.c_int,
                                   C.c_void_p, C.c_void_p]
        L.orc_row_magnitude_spec_f64.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                                 C.c_int, C.c_double, C.c_void_p,
                                                 C.POINTER(_Rope), C.c_int, C.c_void_p,
                                                 C.c_void_p]
        L.orc_row_magnitude_f64.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                            C.c_double, C.c_int64, C.c_int, C.c_void_p,
                                            C.c_void_p]
        L.orc_row_offset.restype = C.c_int64
        L.orc_row_offset.argtypes = [C.POINTER(_Channel), C.c_int32, C.c_void_p,
                                     C.c_int64, C.c_int64, C.c_int64]
        L.orc_attend.restype = C.c_int
        L.orc_attend.argtypes = [C.POINTER(_Problem), C.c_int, C.c_double, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_void_p]
        L.orc_num_threads.restype = C.c_int
        L.orc_set_num_threads.restype = None
        L.orc_set_num_threads.argtypes = [C.c_int]
        L.orc_struct_sizes.restype = C.c_int
        L.orc_struct_sizes.argtypes = [C.c_int]
        assert L.orc_struct_sizes(0) == C.sizeof(_Channel)
        assert L.orc_struct_sizes(1) == C.sizeof(_Problem)
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint8:
        return FP8
    raise TypeError("storage arrays are uint16 (bf16 bits), float32 or uint8 (fp8 codes)")


def _factor_dtype(a: np.ndarray):
    """numpy dtype of the patch factors for KV stored like `a` (bf16 bits for fp8)."""
    return np.uint16 if a.dtype == np.uint8 else a.dtype


# ----------------------------------------------------------------- numbers

def round_bf16(y) -> np.ndarray:
    """fp64 -> bf16 bits, round to nearest even, in one step."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint16)
    lib().orc_round_bf16_array(_ptr(y), _ptr(out), y.size)
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bits -> exact fp64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_fp8(y) -> np.ndarray:
    """fp64 -> E4M3 codes: nearest, ties to even, saturating at +-448."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().orc_fp8_from_double_array(_ptr(y), _ptr(out), y.size)
    return out


_fp8_table = None


def fp8_to_f64(codes) -> np.ndarray:
    """E4M3 codes -> exact fp64 values (NaN for the two NaN codes)."""
    global _fp8_table
    if _fp8_table is None:
        _fp8_table = np.array([lib().orc_fp8_to_double(c) for c in range(256)])
    return _fp8_table[np.asarray(codes, dtype=np.uint8)]


def freq(theta: float, r: int, i: int) -> float:
    return lib().orc_freq(theta, r, i)


# ------------------------------------------------------------- fp64 forms

def rotate_head_f64(x, r: int, theta: float, delta, pairing: int = NEOX,
                    sections=()) -> np.ndarray:
    """One head in fp64; `delta` is one value, or one per M-RoPE section."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    if pairing == NEOX and not len(sections) > 1 and np.ndim(delta) == 0:
        lib().orc_rotate_head_f64(_ptr(x), _ptr(y), x.size, r, theta, int(delta))
    else:
        dv = _delta_vec(delta)
        q = _rope(pairing, sections)
        lib().orc_rotate_head_spec_f64(_ptr(x), _ptr(y), x.size, r, theta, _ptr(dv), C.byref(q))
    return y


def row_f64(x, heads: int, dim: int, r: int, theta: float, delta,
            u=None, V=None, pairing: int = NEOX, sections=()) -> np.ndarray:
    """One token row (heads*dim values) in fp64: rotation, then the patch row."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.size == heads * dim
    y = np.empty_like(x)
    m = 0 if u is None else int(np.asarray(u).size)
    uu = None if u is None else np.ascontiguousarray(u, dtype=np.float64)
    vv = None if V is None else np.ascontiguousarray(V, dtype=np.float64)
    if m:
        assert vv.shape == (heads * dim, m)
    dv = _delta_vec(delta)
    q = _rope(pairing, sections)
    lib().orc_row_spec_f64(_ptr(x), _ptr(y), heads, dim, r, theta, _ptr(dv), C.byref(q), m,
                           _ptr(uu), _ptr(vv))
    return y


def row_magnitude_f64(x, heads: int, dim: int, r: int, theta: float, delta,
                      u=None, V=None, pairing: int = NEOX, sections=()) -> np.ndarray:
    """Per element, the sum of |terms| that make the fp64 row value."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    s = np.empty_like(x)
    m = 0 if u is None else int(np.asarray(u).size)
    uu = None if u is None else np.ascontiguousarray(u, dtype=np.float64)
    vv = None if V is None else np.ascontiguousarray(V, dtype=np.float64)
    dv = _delta_vec(delta)
    q = _rope(pairing, sections)
    lib().orc_row_magnitude_spec_f64(_ptr(x), _ptr(s), heads, dim, r, theta, _ptr(dv),
                                     C.byref(q), m, _ptr(uu), _ptr(vv))
    return s


def row(x, heads: int, dim: int, r: int, theta: float, delta,
        u=None, V=None, pairing: int = NEOX, sections=(), scale: float = 1.0) -> np.ndarray:
    """One token row in storage format (uint16 bf16 bits, float32, or uint8 fp8 codes
    whose values are `scale` * code value; fp8 factors are bf16 bits)."""
    x = np.ascontiguousarray(x)
    code = _dtype_code(x)
    out = np.empty_like(x)
    m = 0 if u is None else int(np.asarray(u).size)
    fd = _factor_dtype(x)
    uu = None if u is None else np.ascontiguousarray(u, dtype=fd)
    vv = None if V is None else np.ascontiguousarray(V, dtype=fd)
    dv = _delta_vec(delta)
    q = _rope(pairing, sections)
    rc = lib().orc_row_spec_scaled(code, float(scale), _ptr(x), _ptr(out), heads, dim, r, theta,
                                   _ptr(dv), C.byref(q), m, _ptr(uu), _ptr(vv))
    if rc != 0:
        raise ValueError("oracle rejected the row arguments")
    return out


# ---------------------------------------------------------- whole operator

def row_offset(ch: dict, page_size: int, block_table, layer: int, t: int, h: int) -> int:
    c = _Channel()
    c.layer_stride, c.slot_stride = ch["layer_stride"], ch["slot_stride"]
    c.head_stride, c.page_stride = ch["head_stride"], ch.get("page_stride", 0)
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    return lib().orc_row_offset(C.byref(c), page_size, _ptr(bt), layer, t, h)


def _problem(channels, *, num_layers, theta, offsets, delta, rank, page_size, block_table,
             shape_from=None, pairing=NEOX, sections=()):
    """Fills an orc_problem from channel dicts; returns (problem, arrays to keep alive).
    `delta` is [chunks] or, with M-RoPE sections, [chunks][sections]."""
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    delta = np.ascontiguousarray(delta, dtype=np.int64)
    nsec = len(sections) if len(sections) > 1 else 1
    if delta.ndim == 2:
        assert delta.shape[1] == nsec
    else:
        assert nsec == 1
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    p = _Problem()
    keep = [offsets, delta, bt]
    code = None
    for i, ch in enumerate(channels):
        data = ch["data"]
        assert data.flags["C_CONTIGUOUS"] and data.flags["WRITEABLE"]
        c = _dtype_code(data)
        if code is None:
            code = c
        assert code == c
        es = data.itemsize
        shape = shape_from[i] if shape_from is not None else ch
        p.ch[i].data = data.ctypes.data + es * int(ch.get("offset", 0))
        p.ch[i].heads, p.ch[i].dim = shape["heads"], shape["dim"]
        p.ch[i].rope_dim = shape["rope_dim"]
        p.ch[i].layer_stride = ch["layer_stride"]
        p.ch[i].slot_stride = ch["slot_stride"]
        p.ch[i].head_stride = ch["head_stride"]
        p.ch[i].page_stride = ch.get("page_stride", 0)
        if rank > 0 and shape_from is None:
            U = np.ascontiguousarray(ch["U"])
            V = np.ascontiguousarray(ch["V"])
            assert U.dtype == _factor_dtype(data) and V.dtype == _factor_dtype(data)
            keep += [U, V]
            p.ch[i].U, p.ch[i].V = U.ctypes.data, V.ctypes.data
        if c == FP8 and shape_from is None:
            sc = np.ascontiguousarray(ch["scale"], dtype=np.float32)
            assert sc.size >= num_layers and np.all(sc[:num_layers] > 0)
            keep.append(sc)
            p.ch[i].scale = sc.ctypes.data
    p.dtype = code
    p.num_layers = num_layers
    p.num_channels = len(channels)
    p.page_size = page_size
    p.theta = theta
    p.block_table = _ptr(bt)
    p.total_tokens = int(offsets[-1]) if offsets.size else 0
    p.offsets = _ptr(offsets)
    p.delta = _ptr(delta)
    p.num_chunks = int(delta.shape[0]) if delta.ndim else 1
    p.rank = rank
    p.rope = _rope(pairing, sections)
    return p, keep


def _out_arrays(channels, y_out, s_out):
    ys = (C.c_void_p * 2)()
    ss = (C.c_void_p * 2)()
    for i, ch in enumerate(channels):
        yb, sb = y_out[i], s_out[i]
        assert yb.dtype == np.float64 and sb.dtype == np.float64
        assert yb.size == ch["data"].size and sb.size == ch["data"].size
        ys[i] = yb.ctypes.data + 8 * int(ch.get("offset", 0))
        ss[i] = sb.ctypes.data + 8 * int(ch.get("offset", 0))
    return ys, ss


def relocate_patch(channels, *, num_layers: int, theta: float, offsets, delta,
                   rank: int = 0, page_size: int = 0, block_table=None,
                   y_out=None, s_out=None, pairing: int = NEOX, sections=()) -> None:
    """The reuse operator over host arrays, in place.

    ``channels`` is a list of one or two dicts with keys ``data`` (a flat numpy
    buffer, uint16 or float32, element 0 = layer 0 slot 0 head 0 dim 0),
    ``offset`` (element offset of that first element inside ``data``, default
    0), ``heads``, ``dim``, ``rope_dim``, ``layer_stride``, ``slot_stride``,
    ``head_stride``, ``page_stride`` (elements) and, when ``rank > 0``, ``U``
    ([layers][tokens][rank]) and ``V`` ([layers][chunks][heads*dim][rank]).  With
    fp8 codes (uint8 ``data``) the factors are bf16 bits and ``scale`` holds the
    channel's per-layer float32 dequantisation scales.

    ``y_out`` / ``s_out``: optional lists (one per channel) of float64 buffers shaped
    like that channel's ``data``; every element the call computes receives its
    unrounded fp64 value / its sum of term magnitudes, at the same element offset
    (fp8: divided by the layer's scale).

    ``pairing`` (NEOX or INTERLEAVED) and ``sections`` (M-RoPE pairs per section;
    then ``delta`` is [chunks][sections]) select the positional variant.
    """
    p, keep = _problem(channels, num_layers=num_layers, theta=theta, offsets=offsets,
                       delta=delta, rank=rank, page_size=page_size, block_table=block_table,
                       pairing=pairing, sections=sections)
    if y_out is not None:
        ys, ss = _out_arrays(channels, y_out, s_out)
        rc = lib().orc_relocate_patch_ex(C.byref(p), ys, ss)
    else:
        rc = lib().orc_relocate_patch(C.byref(p))
    del keep
    if rc != 0:
        raise ValueError("oracle rejected the problem")


def recall_patch(src_channels, dst_channels, *, num_layers: int, theta: float, offsets, delta,
                 rank: int = 0, src_page_size: int = 0, src_block_table=None,
                 dst_page_size: int = 0, dst_block_table=None, y_out=None, s_out=None,
                 pairing: int = NEOX, sections=()) -> None:
    """Recall (out of place): rows read through ``src_channels`` (dicts as in
    ``relocate_patch``, with the factors), whole result rows written through
    ``dst_channels`` (dicts with ``data``, ``offset`` and the four strides; heads,
    dim and rope_dim come from the source).  ``y_out`` / ``s_out`` are shaped like
    the destination buffers."""
    sp, keep = _problem(src_channels, num_layers=num_layers, theta=theta, offsets=offsets,
                        delta=delta, rank=rank, page_size=src_page_size,
                        block_table=src_block_table, pairing=pairing, sections=sections)
    dp, keep2 = _problem(dst_channels, num_layers=num_layers, theta=theta, offsets=offsets,
                         delta=delta, rank=rank, page_size=dst_page_size,
                         block_table=dst_block_table, shape_from=src_channels,
                         pairing=pairing, sections=sections)
    ys = ss = None
    if y_out is not None:
        ys, ss = _out_arrays(dst_channels, y_out, s_out)
    rc = lib().orc_recall_patch_ex(C.byref(sp), C.byref(dp), ys, ss)
    del keep, keep2
    if rc != 0:
        raise ValueError("oracle rejected the problem")


def attend(channels, *, num_layers: int, theta: float, offsets, delta, q, scale: float,
           rank: int = 0, page_size: int = 0, block_table=None, pairing: int = NEOX,
           sections=(), with_mag: bool = False):
    """Relocate-on-read decode attention over host arrays: ``channels`` = [K, V] dicts
    as in ``relocate_patch`` (never written); ``q`` [L][Hq][D] float64.  Returns
    (out [L][Hq][D], lse [L][Hq]) in float64, plus mag (sum_t p_t |V'_t|) when
    ``with_mag``.  Tokens whose block-table entry is negative are not attended."""
    p, keep = _problem(channels, num_layers=num_layers, theta=theta, offsets=offsets,
                       delta=delta, rank=rank, page_size=page_size, block_table=block_table,
                       pairing=pairing, sections=sections)
    q = np.ascontiguousarray(q, dtype=np.float64)
    L, Hq, D = q.shape
    assert L == num_layers and D == channels[0]["dim"]
    out = np.empty_like(q)
    lse = np.empty((L, Hq))
    mag = np.empty_like(q) if with_mag else None
    rc = lib().orc_attend(C.byref(p), Hq, float(scale), _ptr(q), _ptr(out), _ptr(lse),
                          _ptr(mag))
    del keep
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return (out, lse, mag) if with_mag else (out, lse)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Host threads of the oracle's loops from now on (the results do not change)."""
    lib().orc_set_num_threads(int(n))

"""Host-side tests of the C ABI: load, exported symbols, struct layout, argument
checks and kernel choice.  No kernel is launched: every call into an entry point
that could launch is made with arguments the host checks reject (asserted first
through kamera_plan), or with an empty problem."""
import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

from rope_relocation_rank_amd import kamera as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kamera.h")

FAKE = 0x7F0000000000  # 4 KiB-aligned address that is never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"KAMERA_API\s+[\w\s\*]+?\b(kamera_\w+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_function():
    L = K.lib()
    names = header_functions()
    assert set(names) == set(K.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported
    assert not [e for e in exported if "launch" in e], "internal symbols leak"
    assert K.kamera_abi_version() == 5


def test_struct_layout_matches_header():
    fields = {
        "kamera_channel": [f[0] for f in K.kamera_channel._fields_],
        "kamera_kv_desc": [f[0] for f in K.kamera_kv_desc._fields_],
        "kamera_chunks": [f[0] for f in K.kamera_chunks._fields_],
        "kamera_patch": [f[0] for f in K.kamera_patch._fields_],
        "kamera_plan_info": [f[0] for f in K.kamera_plan_info._fields_],
        "kamera_form_desc": [f[0] for f in K.kamera_form_desc._fields_],
        "kamera_attend_desc": [f[0] for f in K.kamera_attend_desc._fields_],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kamera.h"', "int main(void){"]
    for s, fs in fields.items():
        lines.append(f'printf("{s} %zu\\n", sizeof({s}));')
        for f in fs:
            lines.append(f'printf("{s}.{f} %zu\\n", offsetof({s}, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(l.rsplit(" ", 1) for l in out.splitlines())
    for s, fs in fields.items():
        cls = getattr(K, s)
        assert int(got[s]) == C.sizeof(cls), s
        for f in fs:
            assert int(got[f"{s}.{f}"]) == getattr(cls, f).offset, f"{s}.{f}"


# ----------------------------------------------------------------- descriptors

class FakeTensor:
    def __init__(self, addr, es=2):
        self.addr, self.es = addr, es

    def data_ptr(self):
        return self.addr

    def element_size(self):
        return self.es

    def numel(self):
        return 1


def gqa(T=4096, L=28, H=4, D=128, r=128, m=32, dtype=K.KAMERA_BF16, kv_addr=FAKE,
        paged=False, pages=0, flags=0, n=1):
    es = {K.KAMERA_BF16: 2, K.KAMERA_FP8_E4M3: 1}.get(dtype, 4)
    chans = []
    for c in range(2):
        base = kv_addr + c * (1 << 36)
        scale = FakeTensor(FAKE + (7 << 40) + c * 4096) if dtype == K.KAMERA_FP8_E4M3 else None
        chans.append(K.channel(FakeTensor(base, es), heads=H, dim=D, rope_dim=r if c == 0 else 0,
                               layer_stride=(pages * 16 if paged else T) * H * D,
                               slot_stride=H * D, head_stride=D,
                               page_stride=16 * H * D if paged else 0, scale=scale))
    kv = K.kv_desc(chans, dtype=dtype, num_layers=L, rope_theta=1e6,
                   page_size=16 if paged else 0, num_pages=pages,
                   block_table=FakeTensor(FAKE + (1 << 40)) if paged else None, flags=flags)
    ch = K.kamera_chunks()
    ch.num_chunks, ch.total_tokens = n, T
    ch.token_offsets, ch.delta = FAKE + (3 << 38), FAKE + (3 << 38) + 4096
    p = K.patch_desc(m) if m else None
    if m:
        for c in range(2):
            p.U[c] = FAKE + (1 << 39) + c * (1 << 34)
            p.V[c] = FAKE + (1 << 39) + (1 << 33) + c * (1 << 34)
    return kv, ch, p


def plan_names(kv, ch, p):
    st, info = K.kamera_plan(kv, ch, p)
    assert st == K.KAMERA_OK, K.kamera_last_error()
    return [K.KERNEL_NAMES[k] for k in info.kernel], info


def expect_status(status, kv, ch, p=None):
    st, _ = K.kamera_plan(kv, ch, p)
    assert st == status, (st, K.kamera_last_error())
    assert K.kamera_last_error()
    # The entry points reject the same arguments before any HIP call.
    assert K.kamera_relocate_patch(kv, ch, p, None) == status
    if p is None or p.rank == 0:
        assert K.kamera_relocate(kv, ch, None) == status


# ----------------------------------------------------------------- argument checks

def test_null_descriptors():
    kv, ch, p = gqa()
    st, _ = K.kamera_plan(None, ch, p)
    assert st == K.KAMERA_E_NULL
    st, _ = K.kamera_plan(kv, None, p)
    assert st == K.KAMERA_E_NULL
    assert K.lib().kamera_relocate(None, None, None) == K.KAMERA_E_NULL
    assert "NULL" in K.kamera_last_error()


def test_bad_dtype_and_pairing():
    kv, ch, p = gqa()
    kv.dtype = 7
    expect_status(K.KAMERA_E_UNSUPPORTED, kv, ch, p)
    kv.dtype = 3
    expect_status(K.KAMERA_E_UNSUPPORTED, kv, ch, p)
    kv, ch, p = gqa()
    kv.pairing = 2
    expect_status(K.KAMERA_E_UNSUPPORTED, kv, ch, p)


def test_positional_variants():
    # Interleaved pairing and M-RoPE sections take the same kernels.
    kv, ch, p = gqa(m=32)
    kv.pairing = K.KAMERA_INTERLEAVED
    names, _ = plan_names(kv, ch, p)
    assert names == ["rotate+patch mfma"] * 2
    kv, ch, p = gqa(m=0)
    kv.pairing = K.KAMERA_INTERLEAVED
    names, _ = plan_names(kv, ch, p)
    assert names == ["rotate", "none"]
    for m in (0, 16):
        kv, ch, p = gqa(m=m)
        kv.num_sections = 3
        kv.section_pairs[0], kv.section_pairs[1], kv.section_pairs[2] = 16, 24, 24
        names, _ = plan_names(kv, ch, p)
        assert names[0] in ("rotate", "rotate+patch mfma")
    # sections must cover the rotary pairs of every rotating channel
    kv, ch, p = gqa(m=16)
    kv.num_sections = 3
    kv.section_pairs[0], kv.section_pairs[1], kv.section_pairs[2] = 16, 24, 23
    expect_status(K.KAMERA_E_SHAPE, kv, ch, p)
    kv.section_pairs[2] = 24
    kv.section_pairs[1] = -1
    expect_status(K.KAMERA_E_SHAPE, kv, ch, p)
    kv, ch, p = gqa(m=16)
    kv.num_sections = 5
    expect_status(K.KAMERA_E_SHAPE, kv, ch, p)
    kv, ch, p = gqa(m=16)
    kv.reserved1 = 1
    expect_status(K.KAMERA_E_SHAPE, kv, ch, p)


@pytest.mark.parametrize("mutate", [
    lambda kv, ch, p: setattr(kv, "num_channels", 0),
    lambda kv, ch, p: setattr(kv, "num_channels", 3),
    lambda kv, ch, p: setattr(kv, "num_layers", -1),
    lambda kv, ch, p: setattr(kv.ch[0], "heads", 0),
    lambda kv, ch, p: setattr(kv.ch[1], "dim", 0),
    lambda kv, ch, p: setattr(kv.ch[0], "rope_dim", 127),
    lambda kv, ch, p: setattr(kv.ch[0], "rope_dim", 130),
    lambda kv, ch, p: setattr(kv.ch[0], "rope_dim", -2),
    lambda kv, ch, p: setattr(kv.ch[1], "slot_stride", -8),
    lambda kv, ch, p: setattr(kv.ch[0], "reserved0", 1),
    lambda kv, ch, p: setattr(kv, "flags", 2),
    lambda kv, ch, p: setattr(kv, "rope_theta", 0.0),
    lambda kv, ch, p: setattr(kv, "rope_theta", float("nan")),
    lambda kv, ch, p: setattr(kv, "page_size", -1),
    lambda kv, ch, p: setattr(p, "rank", 257),
    lambda kv, ch, p: setattr(p, "rank", -1),
    lambda kv, ch, p: setattr(p, "reserved0", 3),
    lambda kv, ch, p: setattr(ch, "num_chunks", 0),
    lambda kv, ch, p: setattr(ch, "num_chunks", -1),
    lambda kv, ch, p: setattr(ch, "total_tokens", -5),
    lambda kv, ch, p: setattr(ch, "reserved0", 1),
])
def test_shape_errors(mutate):
    kv, ch, p = gqa()
    mutate(kv, ch, p)
    expect_status(K.KAMERA_E_SHAPE, kv, ch, p)


@pytest.mark.parametrize("mutate", [
    lambda kv, ch, p: setattr(kv.ch[0], "data", None),
    lambda kv, ch, p: p.U.__setitem__(1, None),
    lambda kv, ch, p: p.V.__setitem__(0, None),
    lambda kv, ch, p: setattr(ch, "token_offsets", None),
    lambda kv, ch, p: setattr(ch, "delta", None),
])
def test_null_pointers(mutate):
    kv, ch, p = gqa()
    mutate(kv, ch, p)
    expect_status(K.KAMERA_E_NULL, kv, ch, p)


def test_paged_without_table_or_pages():
    kv, ch, p = gqa(paged=True, pages=256)
    kv.block_table = None
    expect_status(K.KAMERA_E_NULL, kv, ch, p)
    kv, ch, p = gqa(paged=True, pages=256)
    kv.num_pages = 0
    expect_status(K.KAMERA_E_SHAPE, kv, ch, p)


def test_misaligned_pointers():
    kv, ch, p = gqa()
    kv.ch[0].data = FAKE + 1
    expect_status(K.KAMERA_E_ALIGN, kv, ch, p)
    kv, ch, p = gqa(dtype=K.KAMERA_F32)
    kv.ch[1].data = FAKE + (1 << 36) + 2
    expect_status(K.KAMERA_E_ALIGN, kv, ch, p)
    kv, ch, p = gqa()
    p.U[0] = p.U[0] + 1
    expect_status(K.KAMERA_E_ALIGN, kv, ch, p)
    kv, ch, p = gqa()
    ch.delta = ch.delta + 4
    expect_status(K.KAMERA_E_ALIGN, kv, ch, p)


def test_factors_overlapping_kv():
    kv, ch, p = gqa(T=4096, L=2)
    p.U[0] = kv.ch[1].data + 1024  # inside V's KV range
    expect_status(K.KAMERA_E_ALIAS, kv, ch, p)
    kv, ch, p = gqa(T=4096, L=2)
    p.V[1] = kv.ch[0].data + 2 * (2 * 4096 * 4 * 128) - 64  # tail of K's last layer
    expect_status(K.KAMERA_E_ALIAS, kv, ch, p)


def test_empty_problems_are_ok_without_launch():
    for L, T, n in [(0, 4096, 1), (28, 0, 0), (28, 0, 3)]:
        kv, ch, p = gqa(L=L, T=T, n=n)
        ch.total_tokens = T
        st, info = K.kamera_plan(kv, ch, p)
        assert st == K.KAMERA_OK and info.launches == 0
        assert K.kamera_relocate_patch(kv, ch, p, None) == K.KAMERA_OK
        assert K.kamera_relocate(kv, ch, None) == K.KAMERA_OK


def test_status_strings():
    for s in range(7):
        assert K.kamera_status_str(s)
    assert K.kamera_status_str(99) == "unknown status"


# ----------------------------------------------------------------- kernel choice

def test_kernel_choice():
    names, info = plan_names(*gqa(m=32))
    assert names == ["rotate+patch mfma"] * 2 and info.launches == 1
    names, info = plan_names(*gqa(m=0))
    assert names == ["rotate", "none"] and info.launches == 1
    names, _ = plan_names(*gqa(D=96, r=96, m=8))
    assert names == ["generic", "generic"]
    names, _ = plan_names(*gqa(D=128, r=32, m=8))
    assert names == ["rotate+patch mfma"] * 2
    names, _ = plan_names(*gqa(D=128, r=48, m=8))
    assert names == ["generic", "rotate+patch mfma"]
    names, _ = plan_names(*gqa(D=256, r=256, m=8))
    assert names == ["generic", "rotate+patch mfma"]
    names, _ = plan_names(*gqa(D=256, r=128, m=8))
    assert names == ["rotate+patch mfma"] * 2
    names, _ = plan_names(*gqa(D=256, r=256, m=0))
    assert names == ["generic", "none"]
    names, _ = plan_names(*gqa(D=128, r=32, m=0))
    assert names == ["rotate", "none"]
    names, _ = plan_names(*gqa(D=128, r=48, m=0))
    assert names == ["generic", "none"]
    names, _ = plan_names(*gqa(dtype=K.KAMERA_F32, m=8))
    assert names == ["generic", "generic"]
    names, _ = plan_names(*gqa(flags=K.KAMERA_FLAG_GENERIC, m=8))
    assert names == ["generic", "generic"]
    names, _ = plan_names(*gqa(m=129))
    assert names == ["generic", "generic"]
    names, _ = plan_names(*gqa(m=128))
    assert names == ["rotate+patch mfma"] * 2
    kv, ch, p = gqa(m=8)
    kv.ch[0].data = FAKE + 2  # element-aligned but not 16-byte aligned
    names, info = plan_names(kv, ch, p)
    assert names == ["generic", "rotate+patch mfma"] and info.launches == 2
    names, _ = plan_names(*gqa(paged=True, pages=256, m=64))
    assert names == ["rotate+patch mfma"] * 2


def test_buffer_range_limits():
    # The tuned kernels reach one layer of a channel, and one layer of U, through a
    # buffer resource with 32-bit byte offsets: each may span at most 2^31 - 64 bytes.
    # One head of 128 bf16 per token: a layer spans 256 * T bytes.
    t_max = ((1 << 31) - 64) // 256
    for m, tuned in ((32, "rotate+patch mfma"), (0, "rotate")):
        names, _ = plan_names(*gqa(T=t_max, L=1, H=1, D=128, r=128, m=m))
        assert names[0] == tuned
        names, _ = plan_names(*gqa(T=t_max + 1, L=1, H=1, D=128, r=128, m=m))
        assert names[0] == "generic"
    # Small rows, large U: 2^25 tokens of 16 bf16 (1 GiB per layer) fit, but U fits only
    # while 2^25 * m * 2 <= 2^31 - 64.
    names, _ = plan_names(*gqa(T=1 << 25, L=1, H=1, D=16, r=16, m=8))
    assert names == ["rotate+patch mfma"] * 2
    names, _ = plan_names(*gqa(T=1 << 25, L=1, H=1, D=16, r=16, m=32))
    assert names == ["generic", "generic"]


def test_mfma_workgroup_count():
    # One workgroup = one 128-feature block of one channel and layer over
    # tokens_per_unit tokens (a multiple of the 64 tokens four 16-token tiles cover).
    kv, ch, p = gqa(T=32768, L=80, H=8, D=128, m=64, paged=True, pages=2048)
    names, info = plan_names(kv, ch, p)
    bt = info.tokens_per_unit
    assert bt % 64 == 0
    assert info.units == 80 * 2 * (8 * 128 // 128) * (-(-32768 // bt))


def test_chunk_boundary_tail_launch():
    # Token groups that chunk boundaries cut: one more unit per boundary in the same
    # launch, or a second launch over the token groups when boundaries outnumber them.
    _, info1 = plan_names(*gqa(T=4096, m=32, n=1))
    assert info1.launches == 1
    bt = info1.tokens_per_unit
    groups = -(-4096 // bt)
    fb = 4 * 128 // 128
    _, info = plan_names(*gqa(T=4096, m=32, n=5))
    assert info.launches == 1
    assert info.units == 28 * 2 * fb * (groups + 4)
    _, info = plan_names(*gqa(T=4096, m=32, n=groups + 1))  # as many boundaries as groups
    assert info.launches == 1
    assert info.units == 28 * 2 * fb * (2 * groups)
    _, info = plan_names(*gqa(T=4096, m=32, n=groups + 100))
    assert info.launches == 2
    assert info.units == 28 * 2 * fb * (2 * groups)
    _, info = plan_names(*gqa(T=4096, m=0, n=5))  # rotation only: one kernel, no tail
    assert info.launches == 1


# ----------------------------------------------------------------- pool order (workspace)

def ws_bytes(kv, ch, p):
    st, n = K.kamera_relocate_workspace(kv, ch, p)
    assert st == K.KAMERA_OK, K.kamera_last_error()
    return n


def test_relocate_workspace_size():
    # One chunk over a paged cache (pages of 16 slots): 4 bytes per pool page, rounded up
    # to 256; the same problem contiguous, with several chunks, at rank 0 or with a pool
    # far larger than the chunk's pages needs none.
    assert ws_bytes(*gqa(T=32768, L=80, H=8, m=64, paged=True, pages=2048)) == 2048 * 4
    assert ws_bytes(*gqa(T=1000, L=2, m=64, paged=True, pages=100)) == 512
    assert ws_bytes(*gqa(T=1000, L=2, m=64, paged=True, pages=63 * 4)) == 1024
    assert ws_bytes(*gqa(T=1000, L=2, m=64, paged=True, pages=63 * 4 + 1)) == 0
    assert ws_bytes(*gqa(T=32768, m=64)) == 0
    assert ws_bytes(*gqa(T=32768, L=2, m=64, paged=True, pages=2048, n=3)) == 0
    assert ws_bytes(*gqa(T=32768, L=2, m=0, paged=True, pages=2048)) == 0
    assert ws_bytes(*gqa(T=0, L=2, m=64, paged=True, pages=2048)) == 0
    assert ws_bytes(*gqa(T=32768, L=2, m=64, paged=True, pages=2048,
                         dtype=K.KAMERA_FP8_E4M3)) == 2048 * 4
    kv, ch, p = gqa(T=32768, L=2, m=64, paged=True, pages=2048)
    kv.page_size = 8  # a 16-token tile would span two pages
    kv.ch[0].page_stride = kv.ch[1].page_stride = 8 * 4 * 128
    assert ws_bytes(kv, ch, p) == 0
    # the size query checks the arguments like the call
    kv, ch, p = gqa(T=4096, m=64, paged=True, pages=256)
    kv.ch[0].rope_dim = 3
    st, n = K.kamera_relocate_workspace(kv, ch, p)
    assert st == K.KAMERA_E_SHAPE and n == 0
    assert K.lib().kamera_relocate_workspace(C.byref(kv), C.byref(ch), C.byref(p), None) == \
        K.KAMERA_E_NULL


def test_relocate_patch_ws_checks_before_launch():
    kv, ch, p = gqa(T=4096, L=2, m=64, paged=True, pages=256)
    need = ws_bytes(kv, ch, p)
    assert need == 1024
    ws = FAKE + (9 << 40)
    # too small, misaligned, negative size: rejected before any HIP call
    assert K.kamera_relocate_patch_ws(kv, ch, p, ws, need - 1, None) == K.KAMERA_E_SHAPE
    assert "workspace" in K.kamera_last_error()
    assert K.kamera_relocate_patch_ws(kv, ch, p, ws + 4, need, None) == K.KAMERA_E_ALIGN
    assert K.kamera_relocate_patch_ws(kv, ch, p, ws, -1, None) == K.KAMERA_E_SHAPE
    # overlapping the cache, the factors or the block table
    for addr in (kv.ch[1].data + 64, p.U[0] + 256, p.V[1], kv.block_table):
        assert K.kamera_relocate_patch_ws(kv, ch, p, addr, need, None) == K.KAMERA_E_ALIAS, addr
    # argument errors of the operator itself come first
    kv.ch[0].rope_dim = 3
    assert K.kamera_relocate_patch_ws(kv, ch, p, ws, need, None) == K.KAMERA_E_SHAPE
    # an empty problem with a workspace is fine and launches nothing
    kv, ch, p = gqa(T=0, L=2, m=64, paged=True, pages=256)
    assert K.kamera_relocate_patch_ws(kv, ch, p, ws, 1024, None) == K.KAMERA_OK


def test_relocate_patch_noalloc_size_limit():
    # The library-held inverse table has room for 2^20 pool pages; a pool-order problem
    # with more is rejected before any HIP call, one that fits reports 4 MiB of workspace.
    T = (1 << 20) * 4  # tokens of 16-slot pages: a pool of 2^20 pages is within 4x
    kv, ch, p = gqa(T=T, L=1, H=1, D=16, r=16, m=8, paged=True, pages=1 << 20)
    assert ws_bytes(kv, ch, p) == (1 << 20) * 4
    kv, ch, p = gqa(T=T + 1024, L=1, H=1, D=16, r=16, m=8, paged=True, pages=(1 << 20) + 16)
    assert ws_bytes(kv, ch, p) > (1 << 20) * 4
    assert K.kamera_relocate_patch_noalloc(kv, ch, p, None) == K.KAMERA_E_SHAPE
    assert "scratch" in K.kamera_last_error()
    # argument errors come first, as for the other entry points
    kv.ch[0].rope_dim = 3
    assert K.kamera_relocate_patch_noalloc(kv, ch, p, None) == K.KAMERA_E_SHAPE
    assert "rope_dim" in K.kamera_last_error()
    # an empty problem launches nothing
    kv, ch, p = gqa(T=0, L=1, m=8, paged=True, pages=4)
    assert K.kamera_relocate_patch_noalloc(kv, ch, p, None) == K.KAMERA_OK


# ----------------------------------------------------------------- recall (out of place)

def recall_dst(T=4096, L=28, H=4, D=128, r=128, pages=300, addr=FAKE + (5 << 40), dtype=None):
    """A paged destination cache matching gqa()'s source shape."""
    es = {None: 2, K.KAMERA_BF16: 2, K.KAMERA_FP8_E4M3: 1}.get(dtype, 4)
    chans = [K.channel(FakeTensor(addr + c * (1 << 36), es), heads=H, dim=D,
                       rope_dim=r if c == 0 else 0, layer_stride=pages * 16 * H * D,
                       slot_stride=H * D, head_stride=D, page_stride=16 * H * D)
             for c in range(2)]
    return K.kv_desc(chans, dtype=K.KAMERA_BF16 if dtype is None else dtype, num_layers=L,
                     rope_theta=0.0, page_size=16, num_pages=pages,
                     block_table=FakeTensor(FAKE + (6 << 40)))


def recall_plan_names(src, dst, ch, p):
    st, info = K.kamera_recall_plan(src, dst, ch, p)
    assert st == K.KAMERA_OK, K.kamera_last_error()
    return [K.KERNEL_NAMES[k] for k in info.kernel], info


def test_recall_kernel_choice():
    # Every channel is written whole, so both launch, rank 0 included.
    for m in (0, 8, 32, 64, 128):
        src, ch, p = gqa(m=m)
        names, info = recall_plan_names(src, recall_dst(), ch, p)
        assert names == ["rotate+patch mfma"] * 2 and info.launches == 1, m
    src, ch, p = gqa(m=32, n=3)  # out of place, boundaries take a second launch
    _, info = recall_plan_names(src, recall_dst(), ch, p)
    assert info.launches == 2
    src, ch, p = gqa(m=12)  # rank not a multiple of 8
    names, _ = recall_plan_names(src, recall_dst(), ch, p)
    assert names == ["generic", "generic"]
    src, ch, p = gqa(m=8, dtype=K.KAMERA_F32)
    names, _ = recall_plan_names(src, recall_dst(dtype=K.KAMERA_F32), ch, p)
    assert names == ["generic", "generic"]
    src, ch, p = gqa(m=8)
    dst = recall_dst()
    dst.ch[1].data = FAKE + (5 << 40) + (1 << 36) + 2  # element-aligned only
    names, info = recall_plan_names(src, dst, ch, p)
    assert names == ["rotate+patch mfma", "generic"] and info.launches == 2


def test_fp8_kernel_choice_and_checks():
    Q = K.KAMERA_FP8_E4M3
    names, info = plan_names(*gqa(m=32, dtype=Q))
    assert names == ["rotate+patch mfma"] * 2 and info.launches == 1
    names, info = plan_names(*gqa(m=0, dtype=Q))
    assert names == ["rotate", "none"]
    names, _ = plan_names(*gqa(m=5, dtype=Q))  # the tuned fp8 kernel takes ranks % 8 == 0
    assert names == ["generic", "generic"]
    names, _ = plan_names(*gqa(m=128, dtype=Q, paged=True, pages=300))
    assert names == ["rotate+patch mfma"] * 2
    names, _ = plan_names(*gqa(m=8, dtype=Q, flags=K.KAMERA_FLAG_GENERIC))
    assert names == ["generic", "generic"]
    # 8-byte vector accesses: a row base on an 8-byte boundary is enough
    kv, ch, p = gqa(m=8, dtype=Q)
    kv.ch[0].data = FAKE + 8
    assert plan_names(kv, ch, p)[0] == ["rotate+patch mfma"] * 2
    kv.ch[0].data = FAKE + 4
    assert plan_names(kv, ch, p)[0] == ["generic", "rotate+patch mfma"]
    # scales are required and 4-byte aligned; factors are bf16 (2-byte aligned)
    kv, ch, p = gqa(m=8, dtype=Q)
    kv.ch[1].scale = None
    expect_status(K.KAMERA_E_NULL, kv, ch, p)
    kv, ch, p = gqa(m=8, dtype=Q)
    kv.ch[0].scale = FAKE + (7 << 40) + 2
    expect_status(K.KAMERA_E_ALIGN, kv, ch, p)
    kv, ch, p = gqa(m=8, dtype=Q)
    p.U[0] = FAKE + (1 << 39) + 1
    expect_status(K.KAMERA_E_ALIGN, kv, ch, p)
    # factor extents are counted in bf16 bytes: U right after the KV of channel 0
    kv, ch, p = gqa(T=64, L=2, m=8, dtype=Q)
    kv_bytes = 2 * 64 * 4 * 128  # layers * tokens * F, one byte each
    p.U[0] = FAKE + kv_bytes
    assert plan_names(kv, ch, p)[0] == ["rotate+patch mfma"] * 2
    p.U[0] = FAKE + kv_bytes - 2
    expect_status(K.KAMERA_E_ALIAS, kv, ch, p)
    # recall: fp8 to fp8 only; the destination's scales are not read
    src, ch, p = gqa(m=32, dtype=Q)
    names, _ = recall_plan_names(src, recall_dst(dtype=Q), ch, p)
    assert names == ["rotate+patch mfma"] * 2
    st, _ = K.kamera_recall_plan(src, recall_dst(), ch, p)
    assert st == K.KAMERA_E_SHAPE


def test_recall_argument_errors():
    src, ch, p = gqa(m=8)
    st, _ = K.kamera_recall_plan(src, None, ch, p)
    assert st == K.KAMERA_E_NULL
    st, _ = K.kamera_recall_plan(src, recall_dst(dtype=K.KAMERA_F32), ch, p)
    assert st == K.KAMERA_E_SHAPE
    st, _ = K.kamera_recall_plan(src, recall_dst(H=8), ch, p)
    assert st == K.KAMERA_E_SHAPE
    st, _ = K.kamera_recall_plan(src, recall_dst(r=64), ch, p)
    assert st == K.KAMERA_E_SHAPE
    st, _ = K.kamera_recall_plan(src, recall_dst(L=27), ch, p)
    assert st == K.KAMERA_E_SHAPE
    dst = recall_dst()
    dst.block_table = None
    st, _ = K.kamera_recall_plan(src, dst, ch, p)
    assert st == K.KAMERA_E_NULL
    dst = recall_dst()
    dst.ch[0].data = None
    st, _ = K.kamera_recall_plan(src, dst, ch, p)
    assert st == K.KAMERA_E_NULL
    # destination overlapping the source, or a factor
    st, _ = K.kamera_recall_plan(src, recall_dst(addr=FAKE + 4096), ch, p)
    assert st == K.KAMERA_E_ALIAS
    st, _ = K.kamera_recall_plan(src, recall_dst(addr=p.U[1] - 4096), ch, p)
    assert st == K.KAMERA_E_ALIAS
    # source-side errors are the in-place call's
    src2, ch2, p2 = gqa(m=8)
    src2.ch[0].rope_dim = 3
    st, _ = K.kamera_recall_plan(src2, recall_dst(), ch2, p2)
    assert st == K.KAMERA_E_SHAPE
    # empty problem: nothing to launch, but still checked
    src, ch, p = gqa(m=8, T=0, n=0)
    names, info = recall_plan_names(src, recall_dst(), ch, p)
    assert info.launches == 0


# ----------------------------------------------------------------- patch formation

def form(L=28, T=4096, F=(512, 512), m=32, n=1, iters=0):
    d = K.kamera_form_desc()
    d.dtype, d.num_layers, d.num_channels, d.rank = K.KAMERA_BF16, L, len(F), m
    d.iterations = iters
    for c, f in enumerate(F):
        d.width[c] = f
        d.delta[c] = FAKE + c * (1 << 36)
        d.U[c] = FAKE + (1 << 39) + c * (1 << 34)
        d.V[c] = FAKE + (1 << 39) + (1 << 33) + c * (1 << 34)
    ch = K.kamera_chunks()
    ch.num_chunks, ch.total_tokens = n, T
    ch.token_offsets, ch.delta = FAKE + (3 << 38), 0
    return d, ch


def test_form_workspace_and_errors():
    d, ch = form()
    st, nb = K.kamera_form_workspace(d, ch)
    assert st == K.KAMERA_OK
    k = 48  # m + 16
    per = 512 * 512 + 2 * 512 * k + 2 * k * k + k
    per = -(-per // 64) * 64 * 4
    assert nb == per * 28  # 28 problems (< 64 per batch)
    for mutate, status in [
        (lambda d, ch: setattr(d, "rank", 0), K.KAMERA_E_SHAPE),
        (lambda d, ch: setattr(d, "rank", K.KAMERA_FORM_MAX_RANK + 1), K.KAMERA_E_SHAPE),
        (lambda d, ch: d.width.__setitem__(0, 100), K.KAMERA_E_SHAPE),
        (lambda d, ch: d.width.__setitem__(1, 2048), K.KAMERA_E_SHAPE),
        (lambda d, ch: setattr(d, "dtype", K.KAMERA_F32), K.KAMERA_E_UNSUPPORTED),
        (lambda d, ch: d.delta.__setitem__(0, None), K.KAMERA_E_NULL),
        (lambda d, ch: d.delta.__setitem__(0, FAKE + 8), K.KAMERA_E_ALIGN),
        (lambda d, ch: setattr(d, "iterations", 65), K.KAMERA_E_SHAPE),
        (lambda d, ch: setattr(d, "num_channels", 3), K.KAMERA_E_SHAPE),
    ]:
        d, ch = form()
        mutate(d, ch)
        st, _ = K.kamera_form_workspace(d, ch)
        assert st == status, (status, K.kamera_last_error())


def test_form_patch_checks_before_launch():
    # Host-checkable errors come back before any HIP call (the pointers are fake).
    import ctypes as C
    L_ = K.lib()
    d, ch = form()
    # outputs overlapping the deficit
    d.U[0] = d.delta[0] + 4096
    st = L_.kamera_form_patch(C.byref(d), C.byref(ch), C.c_void_p(FAKE + (7 << 40)), 1 << 30, None)
    assert st == K.KAMERA_E_ALIAS
    d, ch = form()
    st = L_.kamera_form_patch(C.byref(d), C.byref(ch), None, 1 << 30, None)
    assert st == K.KAMERA_E_NULL
    st = L_.kamera_form_patch(C.byref(d), C.byref(ch), C.c_void_p(FAKE + (7 << 40) + 8), 1 << 30, None)
    assert st == K.KAMERA_E_ALIGN
    st = L_.kamera_form_patch(C.byref(d), C.byref(ch), C.c_void_p(FAKE + (7 << 40)), 1024, None)
    assert st == K.KAMERA_E_SHAPE  # workspace too small for one problem


# ----------------------------------------------------------------- relocate-on-read attention

def attend(Hq=28, L=28, T=4096, H=4, m=32, **kw):
    kv, ch, p = gqa(T=T, L=L, H=H, m=m, **kw)
    d = K.kamera_attend_desc()
    d.num_q_heads, d.scale = Hq, 0.088
    d.q = FAKE + (9 << 40)
    d.out = FAKE + (10 << 40)
    d.lse = FAKE + (11 << 40)
    return kv, ch, p, d


def attend_status(kv, ch, p, d):
    st, _ = K.kamera_attend_workspace(kv, ch, p, d)
    if st == K.KAMERA_OK:
        # the launch call rejects before any HIP call too, through its workspace check
        st2 = K.lib().kamera_attend(C.byref(kv), C.byref(ch), None if p is None else C.byref(p),
                                    C.byref(d), None, 0, None)
        return st, st2
    return st, None


@pytest.mark.parametrize("H,L,T,m,splits", [(8, 80, 32768, 64, 3), (8, 32, 73728, 16, 8),
                                             (8, 2, 4096, 32, 32), (8, 300, 8192, 8, 1),
                                             (4, 28, 4096, 32, 9), (4, 2, 1000, 32, 8)])
def test_attend_one_wave_per_head_splits(H, L, T, m, splits):
    # 4 to 8 KV heads at ranks up to 64 take one workgroup per (layer, split) with a
    # wave per head, bf16 one workgroup per CU: as many splits as one round of 256
    # workgroups holds (floor(256 / L), at least 1), at most one per 128 tokens.  The
    # slots per query head are the splits (one chunk): workspace = prepared queries +
    # slots.
    kv, ch, p, d = attend(Hq=8 * H, L=L, T=T, H=H, m=m)
    st, nbytes = K.kamera_attend_workspace(kv, ch, p, d)
    assert st == K.KAMERA_OK, K.kamera_last_error()
    Hq = 8 * H
    qw = -(-(L * 1 * Hq * (128 + m) * 4) // 256) * 256
    slot_floats = (4 + 128 + m + 3) & ~3
    assert nbytes == qw + L * Hq * splits * slot_floats * 4


def test_attend_workspace_and_checks():
    kv, ch, p, d = attend()
    st, nbytes = K.kamera_attend_workspace(kv, ch, p, d)
    assert st == K.KAMERA_OK and nbytes > 0
    # prepared queries [L][chunks][Hq][128 + m], then partial slots [L][Hq][slots][164]
    # (max, sum, chunk, one unused float, 128 + m sums); 4 KV heads: a workgroup per
    # (layer, split) with a wave per head, floor(256 / 28) = 9 splits
    assert nbytes == 28 * 1 * 28 * (128 + 32) * 4 + 28 * 28 * 9 * 164 * 4
    # 2 KV heads: one 4-wave workgroup per (layer, KV head, split): 4096 workgroups would
    # take 74 splits, capped at 4 splits of 1024 tokens
    kv2, ch2, p2, d2 = attend(Hq=14, H=2)
    st, nb2 = K.kamera_attend_workspace(kv2, ch2, p2, d2)
    assert st == K.KAMERA_OK and nb2 == 28 * 1 * 14 * (128 + 32) * 4 + 28 * 14 * 4 * 164 * 4
    st, st2 = attend_status(kv, ch, p, d)
    assert st2 == K.KAMERA_E_NULL  # no workspace given
    for mutate, status in [
        (lambda kv, ch, p, d: setattr(d, "num_q_heads", 30), K.KAMERA_E_SHAPE),
        (lambda kv, ch, p, d: setattr(d, "num_q_heads", 36), K.KAMERA_E_UNSUPPORTED),
        (lambda kv, ch, p, d: setattr(d, "reserved0", 1), K.KAMERA_E_SHAPE),
        (lambda kv, ch, p, d: setattr(d, "scale", float("inf")), K.KAMERA_E_SHAPE),
        (lambda kv, ch, p, d: setattr(d, "q", None), K.KAMERA_E_NULL),
        (lambda kv, ch, p, d: setattr(d, "out", FAKE + (10 << 40) + 2), K.KAMERA_E_ALIGN),
        (lambda kv, ch, p, d: setattr(kv, "dtype", K.KAMERA_F32), K.KAMERA_E_UNSUPPORTED),
        (lambda kv, ch, p, d: setattr(kv, "num_channels", 1), K.KAMERA_E_UNSUPPORTED),
        (lambda kv, ch, p, d: setattr(kv.ch[1], "rope_dim", 128), K.KAMERA_E_SHAPE),
    ]:
        kv, ch, p, d = attend()
        mutate(kv, ch, p, d)
        st, _ = K.kamera_attend_workspace(kv, ch, p, d)
        assert st == status, (st, K.kamera_last_error())
    kv, ch, p, d = attend()
    kv.ch[0].dim = kv.ch[1].dim = 64
    kv.ch[0].rope_dim = 64
    st, _ = K.kamera_attend_workspace(kv, ch, p, d)
    assert st == K.KAMERA_E_UNSUPPORTED
    # ranks above 128 or not a multiple of 8 are refused
    for m in (136, 12):
        kv, ch, p, d = attend(m=m)
        assert K.kamera_attend_workspace(kv, ch, p, d)[0] == K.KAMERA_E_UNSUPPORTED


def test_attend_aliasing():
    kv, ch, p, d = attend(T=64, L=2)
    _, nbytes = K.kamera_attend_workspace(kv, ch, p, d)
    ws = FAKE + (12 << 40)
    def call():
        return K.lib().kamera_attend(C.byref(kv), C.byref(ch), C.byref(p), C.byref(d), ws,
                                     nbytes, None)
    d.out = d.q  # output on top of the query
    assert call() == K.KAMERA_E_ALIAS
    d.out = FAKE + (10 << 40)
    d.lse = FAKE + (10 << 40) + 16  # lse inside out
    assert call() == K.KAMERA_E_ALIAS
    d.lse = FAKE + (11 << 40)
    ws = FAKE  # workspace on the K cache
    assert call() == K.KAMERA_E_ALIAS


# ----------------------------------------------------------------- orbit mean

def test_orbit_mean_checks_before_launch():
    # Every argument error returns before any HIP call (fake addresses, no GPU); an
    # empty problem returns OK without a launch.
    L = K.lib()
    A, O = FAKE, FAKE + (1 << 36)
    assert L.kamera_orbit_mean(A, 3, 0, 0, O, None) == K.KAMERA_OK
    assert L.kamera_orbit_mean(A, 0, 64, 64, O, None) == K.KAMERA_E_SHAPE
    assert L.kamera_orbit_mean(A, 3, -1, 64, O, None) == K.KAMERA_E_SHAPE
    assert L.kamera_orbit_mean(A, 3, 64, 32, O, None) == K.KAMERA_E_SHAPE
    assert L.kamera_orbit_mean(A, (1 << 20) + 1, 64, 64, O, None) == K.KAMERA_E_SHAPE
    assert L.kamera_orbit_mean(None, 3, 64, 64, O, None) == K.KAMERA_E_NULL
    assert L.kamera_orbit_mean(A, 3, 64, 64, None, None) == K.KAMERA_E_NULL
    assert L.kamera_orbit_mean(A + 2, 3, 64, 64, O, None) == K.KAMERA_E_ALIGN
    assert L.kamera_orbit_mean(A, 3, 64, 68, O, None) == K.KAMERA_E_ALIGN
    assert L.kamera_orbit_mean(A, 3, 64, 64, O + 8, None) == K.KAMERA_E_ALIGN
    # out overlapping an order's deficit (order p holds bytes [2 p stride, 2 p stride + 128))
    assert L.kamera_orbit_mean(A, 3, 64, 64, A + 128 + 16, None) == K.KAMERA_E_ALIAS
    assert L.kamera_orbit_mean(A, 3, 64, 128, A + 256 - 64, None) == K.KAMERA_E_ALIAS
    assert L.kamera_orbit_mean(A, 3, 64, 128, A + 2 * 256 + 64, None) == K.KAMERA_E_ALIAS

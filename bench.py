"""Throughput of the Kamera relocate + patch operator on one MI355X.

One step = one pass of the whole operator over one batch of synthetic input.  The
default workload is the Qwen2.5-VL-7B-shaped video segment (28 layers, 4 KV heads x
128, 4096 tokens, delta -1536, theta 1e6): a rotation-only pass (m = 0, keys only)
followed by a rank-32 relocate+patch pass on K and V.  Inputs are resident in HBM
before the timed region; steps cycle through `--copies` independent input copies
(about 2 GB) so that no step finds its data in the 256 MB last-level cache.

Prints one JSON line.  value = algorithmic bytes moved per step (every touched KV
element read once and written once, every factor element read once) x steps / wall
time of the timed steps, in GB/s (1e9); no event is recorded between those launches.
roofline = the dominant kernel (the relocate+patch launch): its launches of the timed
steps, run again back to back between two HIP events on its stream, give its average
launch time.
cpu_baseline = the fp64 CPU oracle on the host cores over a bounded sample of the same
workload.

`--workload recall_72b_paged` measures the out-of-place recall entry point instead:
a canonical contiguous store rebuilt into a paged cache (same metric, same roofline
kernel template in its out-of-place form).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "relocate+patch GB/s (read+write) and % HBM peak; tokens relocated/s"
KERNEL_SRC = os.path.join(ROOT, "rope_relocation_rank_amd", "csrc", "kernels.hip")


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str, bytes_per_launch: int):
    """Measured HBM bytes per launch of the dominant kernel from committed counter
    summaries (FETCH_SIZE and WRITE_SIZE, scaled by a copy-kernel calibration); None
    when absent or when the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(round((d["fetch_kib"] * d["fetch_scale"] + d["write_kib"] * d["write_scale"]) * 1024))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="long_video_72b_paged")
    ap.add_argument("--no-workspace", action="store_true",
                    help="call kamera_relocate_patch (logical order) even where "
                         "kamera_relocate_patch_ws would sweep a paged pool in pool order")
    ap.add_argument("--copies", type=int, default=0, help="input copies (0 = enough for >= 2 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=1024)
    ap.add_argument("--form", action="store_true",
                    help="measure patch formation (kamera_form_patch) on the workload's shape")
    ap.add_argument("--orbit", type=int, default=0,
                    help="measure the orbit deficit (kamera_orbit_mean) over this many orders "
                         "of the workload's first-channel deficit")
    ap.add_argument("--attend", action="store_true",
                    help="measure relocate-on-read decode attention (kamera_attend) on the "
                         "workload's cache, beside relocate + patch followed by attention")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the operator "
              "needs no collective, and every run here uses a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch

    from rope_relocation_rank_amd import kamera as K
    from rope_relocation_rank_amd import ops, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    K.lib()
    dev = torch.device("cuda:0")
    w = synth.get(args.workload)
    if args.orbit:
        return bench_orbit(args, w, dev)
    if args.form:
        return bench_form(args, w, dev)
    if args.attend:
        return bench_attend(args, w, dev)
    ranks = w.rank_passes
    dominant = max(range(len(ranks)), key=lambda i: synth.algorithmic_bytes(w, ranks[i]))
    bytes_pass = [synth.algorithmic_bytes(w, r) for r in ranks]
    bytes_step = sum(bytes_pass)
    per_copy = max(bytes_pass)
    copies = args.copies or max(1, min(16, -(-2_000_000_000 // per_copy)))
    print(f"[bench] workload {w.key}: {w.note}", file=sys.stderr, flush=True)
    print(f"[bench] passes m={list(ranks)} bytes/step={bytes_step} copies={copies}",
          file=sys.stderr, flush=True)

    # Inputs: one instance per (pass, copy); copies share values (the traffic does not
    # depend on them) but live at distinct addresses.
    def clone(base):
        c = synth.Inputs(base.workload, base.rank, base.struct, base.pool_pages,
                         [b.clone() for b in base.buffers], base.layouts,
                         [u.clone() for u in base.U], [v.clone() for v in base.V],
                         base.offsets_t, base.delta_t, base.block_table_t,
                         scales=list(base.scales))
        return c

    insts = []
    for pi, r in enumerate(ranks):
        if w.recall:
            base = synth.make_recall_inputs(w, r, device=dev, pass_id=pi)
            row = [base]
            for _ in range(copies - 1):
                row.append(synth.RecallInputs(clone(base.src), [b.clone() for b in base.dst_buffers],
                                              base.dst_layouts, base.dst_page_size,
                                              base.dst_pool_pages, base.dst_block_table,
                                              base.dst_block_table_t))
        else:
            base = synth.make_inputs(w, r, device=dev, pass_id=pi)
            row = [base] + [clone(base) for _ in range(copies - 1)]
        insts.append(row)
    if w.recall:
        descs = [[ops.recall_descriptors(c) for c in row] for row in insts]
        plan_info = [ops.recall_plan(row[0]) for row in insts]
        wss = [[None] * copies for _ in insts]
    else:
        descs = [[ops.descriptors_for(c) for c in row] for row in insts]
        plan_info = [ops.plan(row[0]) for row in insts]
        # Workspace of kamera_relocate_patch_ws (pool order), one per input copy,
        # allocated before the timed region.
        wss = [[None if args.no_workspace else ops.workspace_for(c) for c in row]
               for row in insts]
    entry = []
    for pi, r in enumerate(ranks):
        if w.recall:
            entry.append("kamera_recall_patch")
        elif r == 0:
            entry.append("kamera_relocate")
        else:
            entry.append("kamera_relocate_patch_ws" if wss[pi][0] is not None
                         else "kamera_relocate_patch")
    lib = K.lib()
    import ctypes as C

    stream = torch.cuda.current_stream(dev)
    s_ptr = C.c_void_p(stream.cuda_stream)

    def launch(pi, ci):
        if w.recall:
            src, dst, ch, p = descs[pi][ci]
            st = lib.kamera_recall_patch(C.byref(src), C.byref(dst), C.byref(ch),
                                         None if p is None else C.byref(p), s_ptr)
        else:
            kv, ch, p = descs[pi][ci]
            ws = wss[pi][ci]
            if p is None:
                st = lib.kamera_relocate(C.byref(kv), C.byref(ch), s_ptr)
            elif ws is not None:
                st = lib.kamera_relocate_patch_ws(C.byref(kv), C.byref(ch), C.byref(p),
                                                  ws.data_ptr(), ws.numel(), s_ptr)
            else:
                st = lib.kamera_relocate_patch(C.byref(kv), C.byref(ch), C.byref(p), s_ptr)
        if st != 0:
            raise K.KameraError(st, K.kamera_last_error())

    # Copy-kernel reference of known size (also the counter calibration point).
    nb = args.copy_calibration_mib << 20
    src = torch.empty(nb, dtype=torch.uint8, device=dev).random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    # In-place elementwise reference of the same size: a framework kernel that reads and
    # writes the same bytes, as the relocate kernels do.
    x = torch.ones(nb // 2, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        x.mul_(1.0)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(10):
        x.mul_(1.0)
    e1.record(stream)
    torch.cuda.synchronize()
    inplace_gbps = 2 * nb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x

    # Warmup.
    for s in range(args.warmup):
        for pi in range(len(ranks)):
            launch(pi, s % copies)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, launches back to back, bracketed by device
    # synchronisation.  No event is recorded inside it: an event pair around every
    # launch adds about 14 us to a 127 us step on this stack.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for pi in range(len(ranks)):
            launch(pi, s % copies)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Average launch time of each pass (the roofline's): the same launches again, each
    # pass's `steps` launches back to back between one pair of HIP events on the launch
    # stream.
    pass_ms = []
    for pi in range(len(ranks)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for s in range(args.steps):
            launch(pi, s % copies)
        b.record(stream)
        torch.cuda.synchronize()
        pass_ms.append(a.elapsed_time(b) / args.steps)

    ms_step = wall * 1e3 / args.steps
    value = bytes_step * args.steps / wall / 1e9
    dom_ms = pass_ms[dominant]
    achieved = bytes_pass[dominant] / (dom_ms * 1e-3) / 1e9
    traffic = load_traffic(w.key, bytes_pass[dominant])
    st = synth.structure(w)
    tokens_step = st.total_tokens * len(ranks)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, ranks, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3"}.get(w.dtype, "f32"),
        "data": "synthetic",
        "config": {
            "workload": w.key,
            "description": w.note,
            "layers": w.layers, "kv_heads": w.heads, "head_dim": w.head_dim,
            "tokens": st.total_tokens, "chunks": st.num_chunks,
            "theta": w.theta, "passes_rank": list(ranks), "page_size": w.page_size,
            "entry_point": entry[dominant],
            "dst_page_size": w.dst_page_size if w.recall else None,
            "bytes_per_step": bytes_step, "input_copies": copies,
            "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_relocated_per_s": round(tokens_step * args.steps / wall, 1),
        "pass_kernel_ms": [round(x, 5) for x in pass_ms],
        "pass_gbps": [round(bytes_pass[i] / (pass_ms[i] * 1e-3) / 1e9, 1) for i in range(len(ranks))],
        "kernels": [[K.KERNEL_NAMES[k] for k in pi.kernel] for pi in plan_info],
        "copy_kernel_gbps": round(copy_gbps, 1),
        "inplace_kernel_gbps": round(inplace_gbps, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "relocate_patch_rows" if ranks[dominant] > 0 else "rotate_rows",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_pass[dominant],
            "avg_launch_ms": round(dom_ms, 5),
            "timing": "HIP events around the pass's launches of the timed steps, rerun back to back",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_form(args, w, dev):
    """Patch formation on the workload's shape: synthetic deficits (32 dominant feature
    directions), rank = the workload's patch rank.  value = (layer, chunk, channel)
    problems formed per second over whole kamera_form_patch calls; roofline = the Gram
    stage (kamera_form_gram) on MFMA, timed with HIP events around each launch."""
    import torch

    from rope_relocation_rank_amd import kamera as K
    from rope_relocation_rank_amd import synth

    m = w.rank
    st = synth.structure(w)
    T, n, L = st.total_tokens, st.num_chunks, w.layers
    print(f"[bench] form {w.key}: rank {m}, {L} layers x {n} chunks", file=sys.stderr, flush=True)
    deltas = synth.make_deficit(w, device=dev)
    Fs = [d.shape[-1] for d in deltas]
    U = [torch.zeros((L, T, m), dtype=torch.bfloat16, device=dev) for _ in Fs]
    V = [torch.zeros((L, n, F, m), dtype=torch.bfloat16, device=dev) for F in Fs]
    offs = torch.as_tensor(st.offsets, device=dev)
    ch = K.chunks_desc(offs, torch.zeros(n, dtype=torch.int64, device=dev), T)
    d = K.form_desc(deltas, U, V, num_layers=L, rank=m)
    K.check(K.kamera_form_workspace(d, ch)[0])
    ws = torch.empty(K.kamera_form_workspace(d, ch)[1], dtype=torch.uint8, device=dev)
    G = [torch.empty((L, n, F, F), dtype=torch.float32, device=dev) for F in Fs]
    stream = torch.cuda.current_stream(dev)
    steps, warm = max(1, min(args.steps, 50)), max(1, min(args.warmup, 5))
    for _ in range(warm):
        K.form_patch(d, ch, ws)
        K.form_gram(d, ch, G)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    gv = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        K.form_patch(d, ch, ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        gv[i][0].record(stream)
        K.form_gram(d, ch, G)
        gv[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    gram_ms = sum(a.elapsed_time(b) for a, b in gv) / steps
    problems = L * n * len(Fs)
    # Algorithmic Gram flops: 2 T_j per entry of the upper triangle (the matrix is
    # symmetric), over every layer, chunk and channel.
    lens = np.diff(st.offsets)
    gram_flops = sum(int(L * (2 * lens * F * (F + 1) // 2).sum()) for F in Fs)
    achieved = gram_flops / (gram_ms * 1e-3) / 1e12
    cpu = None if args.no_cpu_baseline else cpu_baseline_form(w, m, args.cpu_seconds)
    line = {
        "metric": "patch formation (top-m SVD factors of the deficit): problems per second",
        "value": round(problems * steps / wall, 3),
        "unit": "problems/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp32 compute",
        "data": "synthetic",
        "config": {"workload": w.key + " (patch formation)", "rank": m, "layers": L,
                   "chunks": n, "tokens": T, "widths": Fs, "problems_per_step": problems,
                   "parallelism": "single GPU"},
        "call_ms_events": round(call_ms, 4),
        "roofline": {"bound": "mfma", "kernel": "gram_tiles", "achieved": round(achieved, 2),
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": round(achieved / 2500.0, 5),
                     "traffic": None, "algorithmic_flops_per_launch": gram_flops,
                     "avg_launch_ms": round(gram_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_orbit(args, w, dev):
    """The orbit deficit on the workload's first channel: `args.orbit` orders of its
    [L][T][F] deficit (seeded Gaussian bf16 values), averaged into one.  value = GB/s of
    algorithmic traffic (every order read once, the mean written once) over whole
    kamera_orbit_mean calls; the kernel is HBM-bound."""
    import torch

    from rope_relocation_rank_amd import kamera as K
    from rope_relocation_rank_amd import synth

    P = args.orbit
    st = synth.structure(w)
    L, T = w.layers, st.total_tokens
    F = synth.feature_width(w)[0]
    n = L * T * F
    print(f"[bench] orbit {w.key}: {P} orders of {L} x {T} x {F}", file=sys.stderr, flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    d = torch.empty((P, n), dtype=torch.bfloat16, device=dev)
    for p in range(P):
        d[p] = (torch.randn(n, generator=g, device=dev) * 0.05).to(torch.bfloat16)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps, warm = max(1, min(args.steps, 50)), max(1, min(args.warmup, 5))
    for _ in range(warm):
        K.orbit_mean(d, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        K.orbit_mean(d, out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        K.orbit_mean(d, out)
    b.record(stream)
    torch.cuda.synchronize()
    launch_ms = a.elapsed_time(b) / steps
    nbytes = (P + 1) * n * 2
    gbps = nbytes / (launch_ms * 1e-3) / 1e9
    line = {
        "metric": "orbit deficit (mean over orders): GB/s of algorithmic traffic",
        "value": round(nbytes * steps / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, f64 sum",
        "data": "synthetic",
        "config": {"workload": w.key + " (orbit deficit)", "orders": P, "layers": L,
                   "tokens": T, "width": F, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "orbit_mean_bf16", "achieved": round(gbps, 1),
                     "peak": 8000.0, "unit": "GB/s", "frac": round(gbps / 8000.0, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_ms": round(launch_ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def attend_bytes(w, rank: int) -> int:
    """Algorithmic bytes of one decode-attention call over the whole cache: K and V rows
    read once, both U factors and both feature factors read once, queries read and
    outputs (and lse) written.  The partial sums the split kernel exchanges with the
    merge kernel are not counted."""
    from rope_relocation_rank_amd import synth
    st = synth.structure(w)
    T, n, L = st.total_tokens, st.num_chunks, w.layers
    F = w.heads * w.head_dim
    hq = w.q_heads or w.heads
    kv = 2 * L * T * F * w.elem_size
    fac = 2 * L * (T * rank + n * F * rank) * 2
    qo = L * hq * (2 * w.head_dim + 1) * 4
    return kv + fac + qo


def bench_attend(args, w, dev):
    """Relocate-on-read decode attention (kamera_attend) over the workload's cache at
    its patch rank, one query per layer and query head.  value = algorithmic GB/s over
    whole calls (inputs cycled through copies so no call finds its cache in the MALL);
    beside it, the same attention done the other way: relocate + patch in place
    (kamera_relocate_patch), then plain attention over the rewritten cache."""
    import ctypes as C

    import torch

    from rope_relocation_rank_amd import kamera as K
    from rope_relocation_rank_amd import ops, synth

    m = w.rank
    st = synth.structure(w)
    per = attend_bytes(w, m)
    copies = args.copies or max(1, min(8, -(-2_000_000_000 // per)))
    print(f"[bench] attend {w.key}: rank {m}, {w.q_heads or w.heads} query heads, "
          f"{per} B per call, {copies} copies", file=sys.stderr, flush=True)
    scale = w.head_dim ** -0.5
    base = synth.make_inputs(w, m, device=dev)
    q = synth.make_query(w, device=dev)
    insts = [base]
    for _ in range(copies - 1):
        insts.append(synth.Inputs(base.workload, base.rank, base.struct, base.pool_pages,
                                  [b.clone() for b in base.buffers], base.layouts,
                                  [u.clone() for u in base.U], [v.clone() for v in base.V],
                                  base.offsets_t, base.delta_t, base.block_table_t,
                                  scales=base.scales))
    descs = [ops.attend_buffers(c, q, scale) for c in insts]
    lib = K.lib()
    stream = torch.cuda.current_stream(dev)
    s_ptr = C.c_void_p(stream.cuda_stream)

    def fused(i):
        (kv, ch, p, d), _, _, ws = descs[i]
        st_ = lib.kamera_attend(C.byref(kv), C.byref(ch), None if p is None else C.byref(p),
                                C.byref(d), None if ws is None else ws.data_ptr(),
                                0 if ws is None else ws.numel(), s_ptr)
        if st_ != 0:
            raise K.KameraError(st_, K.kamera_last_error())

    # the other way: operator in place, then attention with no motion and no patch
    zero = torch.zeros_like(base.delta_t)
    plain = []
    for c in insts:
        kv, ch, p = ops.descriptors_for(c)
        pc = K.chunks_desc(c.offsets_t, zero, st.total_tokens)
        # out2 and lse2 stay referenced: the descriptor d2 holds their raw pointers
        (kv2, _, _, d2), out2, lse2, _ = ops.attend_buffers(c, q, scale)
        # sized for this call: with no patch the planner may pick another mapping
        st2, nb2 = K.kamera_attend_workspace(kv2, pc, None, d2)
        K.check(st2)
        ws2 = torch.empty(max(nb2, 16), dtype=torch.uint8, device=dev) if nb2 else None
        plain.append((kv, ch, p, kv2, pc, d2, ws2, out2, lse2))

    def unfused(i):
        kv, ch, p, kv2, pc, d2, ws2 = plain[i][:7]
        K.check(lib.kamera_relocate_patch(C.byref(kv), C.byref(ch), C.byref(p), s_ptr))
        K.check(lib.kamera_attend(C.byref(kv2), C.byref(pc), None, C.byref(d2),
                                  None if ws2 is None else ws2.data_ptr(),
                                  0 if ws2 is None else ws2.numel(), s_ptr))

    steps, warm = max(1, args.steps), max(1, args.warmup)
    for i in range(warm):
        fused(i % copies)
    torch.cuda.synchronize()
    # Timed calls back to back (value), then the same calls with an event pair around
    # each (per-call time, and the comparison with relocate-then-attend).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fused(i % copies)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        fused(i % copies)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    for i in range(min(warm, copies)):
        unfused(i % copies)
    torch.cuda.synchronize()
    uv = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        uv[i][0].record(stream)
        unfused(i % copies)
        uv[i][1].record(stream)
    torch.cuda.synchronize()
    unfused_ms = sum(a.elapsed_time(b) for a, b in uv) / steps
    achieved = per / (call_ms * 1e-3) / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline_attend(w, m, args.cpu_seconds)
    line = {
        "metric": "relocate-on-read decode attention: algorithmic GB/s (K, V and factors read once)",
        "value": round(per * steps / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(wall * 1e3 / steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 e4m3" if w.dtype == "fp8" else "bf16") + " in, fp32 compute",
        "data": "synthetic",
        "config": {"workload": w.key + " (decode attention)", "rank": m, "layers": w.layers,
                   "kv_heads": w.heads, "q_heads": w.q_heads or w.heads,
                   "head_dim": w.head_dim, "tokens": st.total_tokens, "chunks": st.num_chunks,
                   "page_size": w.page_size, "bytes_per_call": per, "input_copies": copies,
                   "parallelism": "single GPU"},
        "call_ms_events": round(call_ms, 5),
        "relocate_then_attend_ms": round(unfused_ms, 5),
        "speedup_vs_relocate_then_attend": round(unfused_ms / call_ms, 3),
        "roofline": {"bound": "hbm", "kernel": "attend_prep + attend_tiles + attend_merge (one call)",
                     "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / 8000.0, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": per, "avg_launch_ms": round(call_ms, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_attend(w, m, seconds: float):
    """The oracle's attention (fp64: K', V' formed, then softmax) on the host, over the
    leading layers of the same workload (the oracle spreads layers over host threads),
    repeated until `seconds` have passed."""
    import torch

    from oracle import oracle as orc
    from rope_relocation_rank_amd import synth

    ww = w.with_(layers=min(w.layers, orc.num_threads()))
    inp = synth.make_inputs(ww, m, device="cpu")
    q = synth.make_query(ww, device="cpu").numpy().astype(np.float64)

    def host(t):
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    chans = []
    for c, lay in enumerate(inp.layouts):
        d = dict(lay)
        d["data"] = host(inp.buffers[lay["buffer"]]).ravel()
        if m > 0:
            d["U"], d["V"] = host(inp.U[c]), host(inp.V[c])
        if inp.scales:  # fp8: each channel's per-layer scales
            d["scale"] = inp.scales[c].numpy()
        chans.append(d)
    done, t = 0, 0.0
    while t < seconds and done < 1000:
        t0 = time.perf_counter()
        orc.attend(chans, num_layers=ww.layers, theta=w.theta, offsets=inp.struct.offsets,
                   delta=inp.struct.delta, q=q, scale=w.head_dim ** -0.5, rank=m,
                   page_size=w.page_size, block_table=inp.struct.block_table,
                   pairing=w.pairing, sections=w.sections)
        t += time.perf_counter() - t0
        done += 1
    b = done * attend_bytes(ww, m)
    return {"value": round(b / t / 1e9, 4), "unit": "GB/s",
            "cores": min(orc.num_threads(), ww.layers), "kind": "oracle",
            "sample": f"{done} x {ww.layers} of {w.layers} layers, every token; {t:.1f} s "
                      "of compute, input generation excluded"}


def cpu_baseline_form(w, m, seconds: float):
    """The oracle's exact SVD (numpy LAPACK, fp64) on the host, over as many (layer,
    chunk, channel) problems of the same deficits as fit in `seconds`."""
    import torch

    from oracle import patch_form as pf
    from rope_relocation_rank_amd import synth

    ww = w.with_(layers=1)
    deltas = synth.make_deficit(ww, device="cpu")
    st = synth.structure(ww)
    done, t = 0, 0.0
    while t < seconds and done < 10000:
        for d in deltas:
            x = d[0].float().numpy().astype(np.float64)
            for j in range(st.num_chunks):
                a, b = int(st.offsets[j]), int(st.offsets[j + 1])
                t0 = time.perf_counter()
                pf.top_m_factors(x[a:b], m)
                t += time.perf_counter() - t0
                done += 1
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = int(torch.get_num_threads())
    return {"value": round(done / t, 3), "unit": "problems/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{done} (layer, chunk, channel) problems of layer 0, exact fp64 SVD; "
                      f"{t:.1f} s of compute"}


def cpu_baseline(w, ranks, seconds: float):
    """The fp64 oracle on the host cores over a bounded sample of the same workload:
    whole steps (every pass, every layer, every token) repeated until `seconds` of
    compute have passed; for workloads too large for that, leading layers only."""
    import numpy as np
    import torch

    from oracle import oracle as orc
    from rope_relocation_rank_amd import synth

    print("[bench] cpu baseline: oracle on host cores", file=sys.stderr, flush=True)

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    def prepare(ww):
        probs = []
        for pi, r in enumerate(ranks):
            rinp = synth.make_recall_inputs(ww, r, device="cpu", pass_id=pi) if w.recall else None
            inp = rinp.src if w.recall else synth.make_inputs(ww, r, device="cpu", pass_id=pi)
            bufs = [host(b).ravel() for b in inp.buffers]
            chans = []
            for c, lay in enumerate(inp.layouts):
                d = dict(lay)
                d["data"] = bufs[lay["buffer"]]
                if r > 0:
                    d["U"] = host(inp.U[c])
                    d["V"] = host(inp.V[c])
                if inp.scales:
                    d["scale"] = host(inp.scales[c])
                chans.append(d)
            dchans = None
            if w.recall:
                dbufs = [host(b).ravel() for b in rinp.dst_buffers]
                dchans = [dict(lay, data=dbufs[lay["buffer"]]) for lay in rinp.dst_layouts]
            probs.append((r, inp, chans, rinp, dchans))
        return probs

    def step(ww, probs):
        t0 = time.perf_counter()
        for r, inp, chans, rinp, dchans in probs:
            if w.recall:
                orc.recall_patch(chans, dchans, num_layers=ww.layers, theta=w.theta,
                                 offsets=inp.struct.offsets, delta=inp.struct.delta, rank=r,
                                 src_page_size=w.page_size, src_block_table=inp.struct.block_table,
                                 dst_page_size=rinp.dst_page_size,
                                 dst_block_table=rinp.dst_block_table)
            else:
                orc.relocate_patch(chans, num_layers=ww.layers, theta=w.theta,
                                   offsets=inp.struct.offsets, delta=inp.struct.delta, rank=r,
                                   page_size=w.page_size, block_table=inp.struct.block_table)
        return time.perf_counter() - t0

    # One layer first, to size the sample.
    w1 = w.with_(layers=1)
    t1 = step(w1, prepare(w1))
    layers = int(max(1, min(w.layers, seconds / max(t1, 1e-6))))
    ww = w.with_(layers=layers)
    probs = prepare(ww)
    reps, t = 0, 0.0
    while reps < 40 and (reps == 0 or t < seconds):
        t += step(ww, probs)
        reps += 1
    b = reps * sum(synth.algorithmic_bytes(ww, r) for r in ranks)
    out = {
        "value": round(b / t / 1e9, 4),
        "unit": "GB/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{reps} x ({layers} of {w.layers} layers of every pass m={list(ranks)}, all "
                  f"tokens); {t:.1f} s of compute, input generation excluded",
    }
    out["single_thread"] = cpu_single_thread(seconds / 3)
    return out


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (the first one listed)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_single_thread(seconds: float):
    """The oracle on one host thread, as a scale reference: the Qwen2.5-VL-7B-shaped
    segment's rotation-only pass (keys only, m = 0), leading layers sized to about
    `seconds` of compute, GB/s over the same algorithmic bytes."""
    from oracle import oracle as orc
    from rope_relocation_rank_amd import synth

    w = synth.get("qwen25vl7b_segment")
    threads = orc.num_threads()
    orc.set_num_threads(1)
    try:
        def run(layers):
            ww = w.with_(layers=layers)
            inp = synth.make_inputs(ww, 0, device="cpu")
            bufs = [b.view(__import__("torch").int16).numpy().view(np.uint16).ravel()
                    for b in inp.buffers]
            chans = [dict(lay, data=bufs[lay["buffer"]]) for lay in inp.layouts]
            t0 = time.perf_counter()
            orc.relocate_patch(chans, num_layers=layers, theta=w.theta,
                               offsets=inp.struct.offsets, delta=inp.struct.delta, rank=0,
                               page_size=0, block_table=None)
            return ww, time.perf_counter() - t0

        ww, t1 = run(1)
        layers = int(max(1, min(w.layers, seconds / max(t1, 1e-6))))
        ww, t = run(layers)
        return {"value": round(synth.algorithmic_bytes(ww, 0) / t / 1e9, 4), "unit": "GB/s",
                "cores": 1, "sample": f"{w.key} rotation-only pass, {layers} of {w.layers} "
                                      f"layers; {t:.1f} s of compute"}
    finally:
        orc.set_num_threads(threads)


if __name__ == "__main__":
    main()

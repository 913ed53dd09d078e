#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 hot path on one MI355X.

One step is one pass of the whole hot path over one batch of the Llama-7B
attention-projection workload (W 4096 x 4096 bf16 N(0, 0.02), X [4 x 1024
tokens, 4096] bf16 N(0, 1), dY N(0, 1), LoRA r = 64, alpha = 16, s = 0.25):

    quantize W to NF4 + DQ  ->  dequantize to bf16  ->  fused forward  ->  backward (dX, dA, dB)

Inputs are resident in HBM before the timed region. ``value`` is the
algorithmic forward + backward flops of the step divided by the step time
(quantize and dequantize carry no flops but their time counts).

The JSON line also carries
  roofline      the dominant kernel's achieved rate against the MI355X peak,
                timed live with HIP events recorded by the library on the
                launch stream;
  rows          per-kernel figures of the step (quantize and dequantize in
                GB/s with buffer rotation past the 256 MB last-level cache);
  decode        the skinny-M forward (GEMV) at the 7B MLP shapes in GB/s,
                with rotation over > 512 MB of distinct weights;
  mlp65b        forward and backward at the 65B MLP shapes (M = 2048);
  formats       per weight format (NF4 / FP4, with / without double
                quantization): quantize, dequantize, forward, backward at the
                step's shape and the decode GEMV at the 7B gate shape;
  merge         adapter merge + requantize at the step's shape;
  adamw         one AdamW step over the 7B model's adapter parameters, state
                in HBM and paged from pinned host memory;
  layer7b_projections
                the seven QLoRA projections of a 7B decoder layer, fwd + bwd;
  dequant_solo  dequantize alone at 65B shapes, bf16 and fp32 out;
  whole_model_roundtrip
                quantize + dequantize of every tensor of a 65B-shaped
                80-layer stack (tensors generated on the GPU per layer);
  cpu_baseline  the CPU oracle timed on this host for whole steps of the
                same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-decode] [--no-large] [--no-formats] [--wm-layers L] [--no-graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s & NF4 dequant/GEMV GB/s vs roofline, 7B/65B"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
FP64_PEAK_TFLOPS = 78.6        # MI355X fp64 vector, vendor figure
ROTATE_BYTES = 640 << 20       # > 2 x (256 MB last-level cache + L2)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Sources that define each timed kernel: stored traffic counters are reported
# only while these files are unchanged.
KERNEL_SOURCES = {
    "fwd_gemm": ("linear.hip", "gemm_big.h", "gemm_core.h", "internal.h"),
    "bwd_dx_gemm": ("linear.hip", "gemm_big.h", "gemm_core.h", "internal.h"),
}


def _code_only(text: str) -> str:
    """Source text without comments and blank space (a comment edit does not
    change the kernel)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments and spacing removed) of the sources a kernel
    is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_nf4_quantized_03_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def _counter_per_dispatch(folder: str, counter: str):
    """{(kernel name, grid work-items): [counter value summed per dispatch]}
    from a rocprofv3 --pmc run."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = {}
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                key = (path, row["Dispatch_Id"])
                name = (row["Kernel_Name"], int(float(row.get("Grid_Size") or 0)))
                val = float(row["Counter_Value"])
                per[key] = (name, per[key][1] + val) if key in per else (name, val)
    out = {}
    for name, val in per.values():
        out.setdefault(name, []).append(val)
    return out


# Kernels whose HBM traffic is summarized from the counter runs of the step
# (--no-large --no-formats): key -> (kernel name fragment, grid work-items or
# None for any, algorithmic read bytes, algorithmic write bytes). Step shape:
# M = N = K = 4096, r = 64; decode shapes: gate/up 11008 x 4096 and down
# 4096 x 11008 at M = 1 and 4 (one launch shape), r = 64.
def _traffic_kernels():
    M = N = K = 4096
    r = rp = 64

    def nf4_bytes(n, k):
        nb = n * k // 64
        return n * k // 2 + nb + 4 * ((nb + 255) // 256) + 4

    def gemv(n, k):   # weight, X (M = 1), fp32 A and B; Y
        return (nf4_bytes(n, k) + k * 2 + r * k * 4 + n * r * 4, n * 2)

    return {
        "fwd_gemm": ("k_fwd_big", None, M * K * 2 + nf4_bytes(N, K) + 2 * M * rp * 2, M * N * 2),
        "bwd_dx_gemm": ("k_dx_big", None, M * N * 2 + nf4_bytes(N, K) + 2 * M * rp * 2, M * K * 2),
        "dequant_bf16": ("k_dequant<true, true>", None, nf4_bytes(N, K), N * K * 2),
        "adapter_down": ("k_adapter_down", None, None, None),
        "adapter_finish": ("k_adapter_finish", None, None, None),
        "grad": ("k_grad(", None, M * K * 2 + M * N * 2 + 2 * M * rp * 2, r * K * 4 + N * r * 4),
        "grad_finish": ("k_grad_finish", None, None, r * K * 4 + N * r * 4),
    }


def _gemv_alg_bytes():
    """Algorithmic bytes of one decode GEMV call at M = 1, r = 64: the NF4 +
    DQ weight, X, the fp32 adapter factors, and Y (the 7B gate / up and down
    shapes have the same totals up to X and Y, 8 or 22 KB)."""
    n, k, r = 11008, 4096, 64
    nb = n * k // 64
    return n * k // 2 + nb + 4 * ((nb + 255) // 256) + 4 + k * 2 + r * (n + k) * 4, n * 2


def write_traffic(fetch_dir: str, write_dir: str, cal_fetch_dir: str, cal_write_dir: str, path: str = None):
    """Calibrated HBM bytes per launch of the step's kernels (the Llama-7B
    attention shape, M = N = K = 4096, r = 64) and of the decode GEMV at the
    7B MLP shapes.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch; each is scaled by
    the factor that makes the 1 GiB copy of --calib-copy read (write) exactly
    1 GiB (the largest dispatch of the calibration run is the copy). Writes
    `path` (default profiles/traffic.json)."""
    gib = 1 << 30
    cal_f = max(v for vals in _counter_per_dispatch(cal_fetch_dir, "FETCH_SIZE").values() for v in vals)
    cal_w = max(v for vals in _counter_per_dispatch(cal_write_dir, "WRITE_SIZE").values() for v in vals)
    ff, fw = gib / (cal_f * 1024), gib / (cal_w * 1024)
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    data = {"calibration": {"copy_bytes_each_way": gib, "fetch_kib_read": cal_f, "write_kib_read": cal_w,
                            "fetch_factor": ff, "write_factor": fw}}

    def pick(table, frag, grid):
        return [v for (n, g), vals in table.items() if frag in n and (grid is None or g == grid) for v in vals]

    kernels = _traffic_kernels()
    # one entry per launch shape of the decode GEMV (grid work-items)
    for (n, g) in sorted(set(fetch) | set(write)):
        for frag in ("k_gemv_rows<", "k_gemv<"):
            if frag in n:
                tmpl = n[n.index(frag):n.index(">", n.index(frag)) + 1]
                kernels[f"gemv {tmpl} grid {g}"] = (tmpl, g) + _gemv_alg_bytes()
                break
    for key, (kname, grid, alg_r, alg_w) in kernels.items():
        fv, wv = pick(fetch, kname, grid), pick(write, kname, grid)
        if not fv or not wv:
            print(f"{kname} (grid {grid}) missing from the counter runs", file=sys.stderr)
            continue
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        ent = {
            "kernel": kname if grid is None else f"{kname} grid {grid}",
            "fetch_kib_per_dispatch": f_kib,
            "write_kib_per_dispatch": w_kib,
            "dispatches": [len(fv), len(wv)],
            "read_bytes": f_kib * 1024 * ff,
            "write_bytes": w_kib * 1024 * fw,
            "bytes_per_launch": f_kib * 1024 * ff + w_kib * 1024 * fw,
            "algorithmic_read_bytes": alg_r,
            "algorithmic_write_bytes": alg_w,
        }
        if key in KERNEL_SOURCES:
            ent["source_hash"] = kernel_source_hash(key)
        data[key] = ent
    if path is None:
        path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    for k, v in data.items():
        if "bytes_per_launch" in v:
            ar = v["algorithmic_read_bytes"]
            print(f"{k:16s} read {v['read_bytes'] / 1e6:9.2f} MB (alg {ar / 1e6 if ar else float('nan'):8.2f})  "
                  f"write {v['write_bytes'] / 1e6:8.2f} MB  dispatches {v['dispatches']}")


def decoder_layer_row(qb, dev, ev_time):
    """A Llama-7B decoder layer (d 4096, MLP 11008, 32 heads, r = 64) on 4
    sequences of 1024 tokens: the seven QLoRA projections on the library's
    kernels through the autograd wrapper, RMSNorm, causal attention and the
    SwiGLU gating as fp32 torch glue. Forward + backward time, plain and with
    the layer's forward recomputed in the backward, and the peak of device
    memory above the inputs for one layer and for a stack of four."""
    import torch
    import torch.utils.checkpoint as ckpt
    from tests import decoder_layer as dl
    spec = dl.LayerSpec(d=4096, f=11008, heads=32, r=64, alpha=16.0)
    layer = dl.GpuLayer(qb, spec, dl.make_params(spec, seed=77), dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(78)
    x = torch.randn((4, 1024, spec.d), generator=gen, device=dev)
    dy = torch.randn((4, 1024, spec.d), generator=gen, device=dev)

    def run(checkpoint, depth=1):
        layer.zero_grad()
        xi = x.detach().requires_grad_(True)
        y = xi
        for _ in range(depth):
            y = ckpt.checkpoint(layer.forward, y, use_reentrant=False) if checkpoint else layer.forward(y)
        y.backward(dy)

    row = {"tokens": 4096, "sequences": 4, "d": spec.d, "f": spec.f, "heads": spec.heads, "r": spec.r,
           "weight_bytes_nf4": sum(qb.qlora_weight_storage_bytes(*spec.shape(n), 0) for n in dl.NAMES)}
    for name, ck in (("plain", False), ("checkpointed", True)):
        run(ck)
        row[f"ms_{name}"] = ev_time(lambda: run(ck), 3)
        for depth in (1, 4):
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            base = torch.cuda.memory_allocated()
            run(ck, depth)
            torch.cuda.synchronize()
            row[f"peak_mib_{name}_depth{depth}"] = (torch.cuda.max_memory_allocated() - base) / 2**20
    log(f"decoder layer 7B (4 x 1024 tokens, fwd + bwd): {row['ms_plain']:.2f} ms plain, "
        f"{row['ms_checkpointed']:.2f} ms checkpointed; peak above inputs, stack of 4: "
        f"{row['peak_mib_plain_depth4']:.0f} MiB plain, {row['peak_mib_checkpointed_depth4']:.0f} MiB checkpointed")
    del layer
    torch.cuda.empty_cache()
    return row


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the 65B MLP, 65B dequantize and whole-model rows")
    ap.add_argument("--wm-layers", type=int, default=80,
                    help="layers of the 65B-shaped stack in the whole-model round trip")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the comparison formats (NF4 without DQ, FP4 with and without)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="no GPU: turn four rocprofv3 --pmc output folders (FETCH_SIZE and "
                         "WRITE_SIZE of a short bench run, then of --calib-copy) into "
                         "profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X; see the design notes on sharding).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import bit_nf4_quantized_03_amd as qb
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_each_way": src.numel() * 4, "launches": 3}))
        return

    def d_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def d_f32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    # ------------------------------------------------------------ workload
    wl = synth.workload("attn7b")
    M, N, K, r, s = wl.M, wl.N, wl.K, wl.r, wl.s
    log(f"workload attn7b M={M} N={N} K={K} r={r} s={s}")
    W, X, A, B, dY = d_bf16(wl.W), d_bf16(wl.X), d_f32(wl.A), d_f32(wl.B), d_bf16(wl.dY)
    q = qb.NF4Weight.empty(N, K, dev)
    ws_q = torch.empty(qb.qlora_nf4_quantize_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    ws_l = qb.linear_workspace(M, N, K, r, dev)
    Wdq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    Hs = torch.empty((M, r), dtype=torch.bfloat16, device=dev)

    # The forward keeps the adapter activations bf16(s X A^T) for the
    # backward, as a training step keeps its activations.
    def step():
        qb.qlora_nf4_quantize(W, out=q, ws=ws_q)
        qb.qlora_nf4_dequantize(q, torch.bfloat16, out=Wdq)
        qb.qlora_linear_fwd_save(X, q, A, B, s, ws=ws_l, out=Y, hs=Hs)
        qb.qlora_linear_bwd_saved(dY, X, Hs, q, A, B, s, ws=ws_l, outs=(dX, dA, dB))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Eager steps with the library's kernel timing hooks (HIP events recorded
    # on the launch stream around the dominant kernels).
    qb.qlora_profile_reset()
    qb.qlora_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    qb.qlora_profile_enable(False)
    ms_step_eager = (t1 - t0) * 1e3 / args.steps
    eager_out = [t.clone() for t in (q.codes, q.absmax_q, q.dq_scale, q.dq_mean, Wdq, Y, Hs, dX, dA, dB)]

    # The same step captured once as a HIP graph and replayed: one launch per
    # step instead of one per kernel. Every replay must reproduce the eager
    # outputs bit for bit, else the eager timing is reported.
    graph_ok = False
    ms_step = ms_step_eager
    if not args.no_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            graph_ok = True
            for _ in range(3):
                for t in (Y, Hs, dX, dA, dB, Wdq):
                    t.zero_()
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                outs = (q.codes, q.absmax_q, q.dq_scale, q.dq_mean, Wdq, Y, Hs, dX, dA, dB)
                graph_ok = graph_ok and all(torch.equal(a, b) for a, b in zip(outs, eager_out))
            if graph_ok:
                for _ in range(args.warmup):
                    graph.replay()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(args.steps):
                    graph.replay()
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                ms_step = (t1 - t0) * 1e3 / args.steps
            else:
                log("graph replay differs from the eager step: reporting eager timing")
            del graph
        except Exception as e:  # noqa: BLE001 - capture unsupported: keep eager timing
            log(f"graph capture failed ({e}); reporting eager timing")
            graph_ok = False

    fwd_flops = 2.0 * M * N * K + 2.0 * M * r * (K + N)
    bwd_flops = 2.0 * M * N * K + 4.0 * M * r * (N + K)
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms (eager {ms_step_eager:.3f} ms, graph {'on' if graph_ok else 'off'}) "
        f"-> {value:.1f} TFLOP/s (fwd+bwd algorithmic)")

    kinds = {"fwd_gemm": qb.QLORA_PROF_FWD_GEMM, "bwd_dx_gemm": qb.QLORA_PROF_BWD_DX,
             "quantize_codes": qb.QLORA_PROF_QUANTIZE, "dequantize": qb.QLORA_PROF_DEQUANTIZE}
    kt = {}
    for name, kind in kinds.items():
        tot, cnt = qb.qlora_profile_read(kind)
        kt[name] = tot / cnt if cnt else None
    qb.qlora_profile_reset()

    n = N * K
    nb, nd = n // 64, n // 64 // 256
    stored = n // 2 + nb + 4 * nd + 4
    # Algorithmic work of the two GEMM kernels (the adapter's up projection is
    # folded into the forward kernel, the dH A term into the dX kernel).
    fwd_kernel_flops = 2.0 * M * N * (K + r)
    dx_kernel_flops = 2.0 * M * K * (N + r)
    rows = {
        "fwd_gemm": {"us": kt["fwd_gemm"] * 1e3, "flops": fwd_kernel_flops,
                     "tflops": fwd_kernel_flops / (kt["fwd_gemm"] * 1e-3) / 1e12},
        "bwd_dx_gemm": {"us": kt["bwd_dx_gemm"] * 1e3, "flops": dx_kernel_flops,
                        "tflops": dx_kernel_flops / (kt["bwd_dx_gemm"] * 1e-3) / 1e12},
    }
    for k in rows:
        rows[k]["frac_of_bf16_peak"] = rows[k]["tflops"] / BF16_PEAK_TFLOPS
    dom = max(("fwd_gemm", "bwd_dx_gemm"), key=lambda k: rows[k]["us"])

    # ------------------------------- quantize / dequantize with rotation
    # enough distinct weights that the data each call reads (the bf16 weight
    # for quantize, the codes for dequantize) exceeds the rotation bound
    R = max(2, ROTATE_BYTES // (2 * n + stored) + 1, ROTATE_BYTES // stored + 1)
    Ws = [W] + [W.clone() for _ in range(R - 1)]
    qs = [qb.NF4Weight.empty(N, K, dev) for _ in range(R)]
    outs = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(R)]

    def timed(fn, reps=3):
        """Per-call time of fn(0..R-1) (distinct buffers, so every call streams
        from HBM): eager launches, and the same R calls captured as one HIP
        graph and replayed (no host launch overhead). Returns (graph, eager)
        in ms; graph is None if capture fails."""
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(R):
            fn(i)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            for i in range(R):
                fn(i)
        ev1.record()
        torch.cuda.synchronize()
        eager = ev0.elapsed_time(ev1) / (reps * R)
        if args.no_graph:
            return None, eager
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(R):
                    fn(i)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(reps):
                g.replay()
            ev1.record()
            torch.cuda.synchronize()
            del g
            return ev0.elapsed_time(ev1) / (reps * R), eager
        except Exception as e:  # noqa: BLE001 - capture unsupported: eager only
            log(f"graph capture failed ({e}); eager timing only")
            return None, eager

    qg, qe = timed(lambda i: qb.qlora_nf4_quantize(Ws[i], out=qs[i], ws=ws_q))
    dg, de = timed(lambda i: qb.qlora_nf4_dequantize(qs[i], torch.bfloat16, out=outs[i]))
    qms, dms = (qg if qg is not None else qe), (dg if dg is not None else de)
    q_bytes = 2 * n + stored
    d_bytes = stored + 2 * n
    rows["quantize"] = {"us": qms * 1e3, "us_eager": qe * 1e3, "bytes": q_bytes,
                        "gbs": q_bytes / (qms * 1e-3) / 1e9}
    rows["dequantize_bf16"] = {"us": dms * 1e3, "us_eager": de * 1e3, "bytes": d_bytes,
                               "gbs": d_bytes / (dms * 1e-3) / 1e9}
    for k in ("quantize", "dequantize_bf16"):
        rows[k]["frac_of_hbm_peak"] = rows[k]["gbs"] / HBM_PEAK_GBS
    rows["quantize"]["rotation"] = R
    rows["dequantize_bf16"]["rotation"] = R
    del Ws, qs, outs
    torch.cuda.empty_cache()

    # Context, not part of the path: the dense bf16 library GEMM (torch.matmul,
    # hipBLASLt) on the dequantized weight at the same shapes, i.e. what an
    # unfused "dequantize, then GEMM" forward and dX would cost.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    library = {}
    for key, fn, fl in (("fwd_x_wt", lambda: torch.matmul(X, Wdq.t()), 2.0 * M * N * K),
                        ("dx_dy_w", lambda: torch.matmul(dY, Wdq), 2.0 * M * N * K)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(10):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / 10
        library[key] = {"us": us, "tflops": fl / (us * 1e-6) / 1e12,
                        "plus_dequantize_us": us + rows["dequantize_bf16"]["us"]}
        log(f"library bf16 GEMM {key}: {us:.1f} us ({library[key]['tflops']:.0f} TFLOP/s); "
            f"+ dequantize {library[key]['plus_dequantize_us']:.1f} us")

    # ---------------------------------------------- decode (skinny M) GEMV
    decode = {}
    if not args.no_decode:
        for name in ("gate7b_m1", "gate7b_m4", "gate7b_m16", "down7b_m1", "down7b_m4", "down7b_m16"):
            w2 = synth.workload(name)
            Mx, Nx, Kx = w2.M, w2.N, w2.K
            st = qb.qlora_nf4_storage_bytes(Nx, Kx)
            per_set = st + 4 * r * (Kx + Nx)
            Rd = max(2, ROTATE_BYTES // per_set + 1)
            Wd = d_bf16(w2.W)
            qd = [qb.qlora_nf4_quantize(Wd) for _ in range(Rd)]
            Ad = [d_f32(w2.A) for _ in range(Rd)]
            Bd = [d_f32(w2.B) for _ in range(Rd)]
            Xd = d_bf16(w2.X)
            Yd = torch.empty((Mx, Nx), dtype=torch.bfloat16, device=dev)
            wsd = qb.linear_workspace(Mx, Nx, Kx, r, dev)
            R_saved, R = R, Rd
            # one untimed call first: a kernel's first launch also loads its code
            qb.qlora_linear_fwd(Xd, qd[0], Ad[0], Bd[0], w2.s, ws=wsd, out=Yd)
            torch.cuda.synchronize()
            qb.qlora_profile_reset()
            qb.qlora_profile_enable(True)
            for i in range(Rd):
                qb.qlora_linear_fwd(Xd, qd[i], Ad[i], Bd[i], w2.s, ws=wsd, out=Yd)
            torch.cuda.synchronize()
            qb.qlora_profile_enable(False)
            ktot, kcnt = qb.qlora_profile_read(qb.QLORA_PROF_FWD_GEMM)
            qb.qlora_profile_reset()
            g_ms, e_ms = timed(lambda i: qb.qlora_linear_fwd(Xd, qd[i], Ad[i], Bd[i], w2.s, ws=wsd, out=Yd),
                               reps=5)
            R = R_saved
            ms = g_ms if g_ms is not None else e_ms
            byts = st + 4 * r * (Kx + Nx) + 2 * Mx * Kx + 2 * Mx * Nx
            kus = ktot / kcnt * 1e3 if kcnt else None
            # the streaming kernel alone moves the NF4+DQ stream, X, A and its partials
            decode[name] = {"M": Mx, "N": Nx, "K": Kx, "us": ms * 1e3, "us_eager": e_ms * 1e3,
                            "bytes": byts, "gbs": byts / (ms * 1e-3) / 1e9,
                            "frac_of_hbm_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "stream_kernel_us": kus, "rotation": Rd}
            log(f"decode {name}: {ms * 1e3:.2f} us/call ({decode[name]['gbs']:.0f} GB/s), "
                f"eager {e_ms * 1e3:.2f} us, streaming kernel {kus:.2f} us")
            del qd, Ad, Bd, Wd
            torch.cuda.empty_cache()

    # ------------------------------------- large shapes, generated on device
    # Timing-only inputs with the same distributions as the parity workloads
    # (N(0, 0.02) weights, 1 % outliers x10 for the 65B MLP, N(0, 1)
    # activations), drawn on the GPU from seeded generators.
    def dev_normal(shape, std, seed, outlier_frac=0.0):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std
        if outlier_frac > 0:
            mask = torch.rand(shape, generator=gen, device=dev) < outlier_frac
            x = torch.where(mask, x * 10.0, x)
        return x.to(torch.bfloat16)

    def ev_time(fn, reps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    # ---------------- the weight formats at the step's shape (and decode M = 1)
    # Per format: quantize (bf16 W in), dequantize (bf16 out), the fused
    # forward and backward at M = 4096, and the decode GEMV at the 7B gate
    # shape with rotating weights, as in the decode rows above.
    formats = {}
    if not args.no_formats:
        wg = synth.workload("gate7b_m1")
        Wg = d_bf16(wg.W)
        Xg = d_bf16(wg.X)
        Yg = torch.empty((wg.M, wg.N), dtype=torch.bfloat16, device=dev)
        wsg = qb.linear_workspace(wg.M, wg.N, wg.K, r, dev)
        for fmt, fname in ((qb.QLORA_FMT_NF4_DQ, "nf4_dq"), (qb.QLORA_FMT_NF4, "nf4"),
                           (qb.QLORA_FMT_FP4_DQ, "fp4_dq"), (qb.QLORA_FMT_FP4, "fp4")):
            qf = qb.NF4Weight.empty(N, K, dev, fmt)
            st = qb.qlora_weight_storage_bytes(N, K, fmt)
            qz_ms = ev_time(lambda: qb.qlora_nf4_quantize(W, out=qf, ws=ws_q), 10)
            dq_ms = ev_time(lambda: qb.qlora_nf4_dequantize(qf, torch.bfloat16, out=Wdq), 10)
            f_ms = ev_time(lambda: qb.qlora_linear_fwd(X, qf, A, B, s, ws=ws_l, out=Y), 10)
            b_ms = ev_time(lambda: qb.qlora_linear_bwd(dY, X, qf, A, B, s, ws=ws_l, outs=(dX, dA, dB)), 10)
            stg = qb.qlora_weight_storage_bytes(wg.N, wg.K, fmt)
            per_set = stg + 4 * r * (wg.K + wg.N)
            Rd = max(2, ROTATE_BYTES // per_set + 1)
            qg = [qb.qlora_nf4_quantize(Wg, fmt=fmt) for _ in range(Rd)]
            Ag = [d_f32(wg.A) for _ in range(Rd)]
            Bg = [d_f32(wg.B) for _ in range(Rd)]
            qb.qlora_linear_fwd(Xg, qg[0], Ag[0], Bg[0], wg.s, ws=wsg, out=Yg)
            torch.cuda.synchronize()
            R_saved, R = R, Rd
            g_ms, e_ms = timed(lambda i: qb.qlora_linear_fwd(Xg, qg[i], Ag[i], Bg[i], wg.s, ws=wsg, out=Yg), reps=5)
            R = R_saved
            d_ms = g_ms if g_ms is not None else e_ms
            d_bytes = per_set + 2 * wg.M * wg.K + 2 * wg.M * wg.N
            formats[fname] = {
                "format": fmt, "storage_bytes": st, "bits_per_param": 8.0 * st / (N * K),
                "quantize_us": qz_ms * 1e3, "quantize_gbs": (2 * N * K + st) / (qz_ms * 1e-3) / 1e9,
                "dequant_bf16_us": dq_ms * 1e3, "dequant_gbs": (st + 2 * N * K) / (dq_ms * 1e-3) / 1e9,
                "fwd_us": f_ms * 1e3, "fwd_tflops": fwd_flops / (f_ms * 1e-3) / 1e12,
                "bwd_us": b_ms * 1e3, "bwd_tflops": bwd_flops / (b_ms * 1e-3) / 1e12,
                "decode_gate7b_m1_us": d_ms * 1e3, "decode_gbs": d_bytes / (d_ms * 1e-3) / 1e9,
            }
            log(f"format {fname}: {8.0 * st / (N * K):.3f} bit/param; quantize {qz_ms * 1e3:.1f} us, "
                f"dequantize {dq_ms * 1e3:.1f} us, fwd {f_ms * 1e3:.1f} us "
                f"({formats[fname]['fwd_tflops']:.0f} TFLOP/s), bwd {b_ms * 1e3:.1f} us, "
                f"decode gate7b M=1 {d_ms * 1e3:.2f} us ({formats[fname]['decode_gbs']:.0f} GB/s)")
            del qf, qg, Ag, Bg
            torch.cuda.empty_cache()
        del Wg, Xg, Yg, wsg

    # -------------- adapter merge + requantize at the step's shape (r = 64)
    merge_row = None
    if not args.no_formats:
        wsm = torch.empty(qb.qlora_nf4_merge_workspace_bytes(N, K, r), dtype=torch.uint8, device=dev)
        qbase = qb.qlora_nf4_quantize(W)
        qout = qb.NF4Weight.empty(N, K, dev)
        m_ms = ev_time(lambda: qb.qlora_nf4_merge(qbase, A, B, s, out=qout, ws=wsm), 10)
        m_flops = 2.0 * N * K * r
        merge_row = {"N": N, "K": K, "r": r, "us": m_ms * 1e3,
                     "rank_sum_fp64_tflops": m_flops / (m_ms * 1e-3) / 1e12,
                     "frac_of_fp64_peak": m_flops / (m_ms * 1e-3) / 1e12 / FP64_PEAK_TFLOPS}
        log(f"merge attn7b r={r}: {m_ms * 1e3:.1f} us per call (merge + requantize), rank sum "
            f"{merge_row['rank_sum_fp64_tflops']:.1f} fp64 TFLOP/s over the whole call")
        del wsm, qbase, qout
        torch.cuda.empty_cache()

    # ---------- AdamW on the adapter parameters of a 7B model (32 layers x
    # q, k, v, o, gate, up, down at r = 64: 159.9 M parameters), state in
    # device memory, then paged from pinned host memory
    opt = None
    if not args.no_formats:
        n_opt = 32 * (4 * r * (4096 + 4096) + 3 * r * (4096 + 11008))
        gen = torch.Generator(device=dev)
        gen.manual_seed(77)
        Po = torch.randn(n_opt, generator=gen, device=dev) * 0.02
        Go = torch.randn(n_opt, generator=gen, device=dev) * 1e-3
        Mo, Vo = torch.zeros_like(Po), torch.zeros_like(Po)
        d_ms = ev_time(lambda: qb.qlora_adamw_step(Po, Go, Mo, Vo, 1, 1e-4, weight_decay=0.01), 5)
        Mh = torch.zeros(n_opt, dtype=torch.float32, pin_memory=True)
        Vh = torch.zeros(n_opt, dtype=torch.float32, pin_memory=True)
        wso = torch.empty(qb.qlora_adamw_workspace_bytes(n_opt, True), dtype=torch.uint8, device=dev)
        h_ms = ev_time(lambda: qb.qlora_adamw_step(Po, Go, Mh, Vh, 1, 1e-4, weight_decay=0.01, ws=wso), 3)
        hbm = 28.0 * n_opt
        opt = {"params": n_opt, "device_state_us": d_ms * 1e3, "device_state_gbs": hbm / (d_ms * 1e-3) / 1e9,
               "device_state_frac_of_hbm_peak": hbm / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               "paged_state_ms": h_ms, "paged_state_pcie_gbs": 16.0 * n_opt / (h_ms * 1e-3) / 1e9}
        log(f"adamw {n_opt / 1e6:.1f} M params: device state {d_ms * 1e3:.0f} us "
            f"({opt['device_state_gbs']:.0f} GB/s HBM); paged state {h_ms:.1f} ms "
            f"({opt['paged_state_pcie_gbs']:.1f} GB/s over PCIe, both ways)")
        del Po, Go, Mo, Vo, Mh, Vh, wso
        torch.cuda.empty_cache()

    # ---------- the seven QLoRA projections of one Llama-7B decoder layer
    # (q, k, v, o: 4096 x 4096; gate, up: 11008 x 4096; down: 4096 x 11008),
    # forward and backward at 4096 tokens, r = 64, one after another on the
    # stream (attention and the activations are not part of the library)
    layer_row = None
    if not args.no_formats:
        shapes = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                  ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
        Ml = 4096
        projs = []
        for i, (nm, Nl, Kl) in enumerate(shapes):
            ql = qb.qlora_nf4_quantize(dev_normal((Nl, Kl), 0.02, 900 + i))
            projs.append((ql, dev_normal((Ml, Kl), 1.0, 950 + i), dev_normal((r, Kl), 0.01, 970 + i).float(),
                          dev_normal((Nl, r), 0.01, 990 + i).float(), dev_normal((Ml, Nl), 1.0, 1010 + i),
                          torch.empty((Ml, Nl), dtype=torch.bfloat16, device=dev),
                          torch.empty((Ml, Kl), dtype=torch.bfloat16, device=dev),
                          torch.empty((r, Kl), dtype=torch.float32, device=dev),
                          torch.empty((Nl, r), dtype=torch.float32, device=dev),
                          qb.linear_workspace(Ml, Nl, Kl, r, dev)))

        def layer_step():
            for (ql, Xl, Al, Bl, dYl, Yl, dXl, dAl, dBl, wsl) in projs:
                qb.qlora_linear_fwd(Xl, ql, Al, Bl, s, ws=wsl, out=Yl)
            for (ql, Xl, Al, Bl, dYl, Yl, dXl, dAl, dBl, wsl) in reversed(projs):
                qb.qlora_linear_bwd(dYl, Xl, ql, Al, Bl, s, ws=wsl, outs=(dXl, dAl, dBl))
        l_ms = ev_time(layer_step, 5)
        l_flops = sum(2.0 * Ml * Nl * Kl * 2 + 2.0 * Ml * r * (Kl + Nl) + 4.0 * Ml * r * (Nl + Kl)
                      for _, Nl, Kl in shapes)
        layer_row = {"tokens": Ml, "r": r, "ms": l_ms, "tflops": l_flops / (l_ms * 1e-3) / 1e12,
                 "frac_of_bf16_peak": l_flops / (l_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                 "weight_bytes_nf4": sum(qb.qlora_nf4_storage_bytes(Nl, Kl) for _, Nl, Kl in shapes)}
        log(f"layer7b projections (7 x fwd + bwd, 4096 tokens): {l_ms:.2f} ms, "
            f"{layer_row['tflops']:.0f} TFLOP/s")
        del projs
        torch.cuda.empty_cache()
        dec_row = decoder_layer_row(qb, dev, ev_time)
    else:
        dec_row = None

    mlp = {}
    if not args.no_large:
        for name, (Nm, Km) in (("up65b", (22016, 8192)), ("down65b", (8192, 22016))):
            Mm = 2048
            seed = 65 if name == "up65b" else 66
            Wm = dev_normal((Nm, Km), 0.02, seed, 0.01)
            qm = qb.qlora_nf4_quantize(Wm)
            del Wm
            Xm = dev_normal((Mm, Km), 1.0, seed + 1000)
            dYm = dev_normal((Mm, Nm), 1.0, seed + 2000)
            Am = dev_normal((r, Km), 0.01, seed + 3000).float()
            Bm = dev_normal((Nm, r), 0.01, seed + 4000).float()
            wsm = qb.linear_workspace(Mm, Nm, Km, r, dev)
            Ym = torch.empty((Mm, Nm), dtype=torch.bfloat16, device=dev)
            dXm = torch.empty((Mm, Km), dtype=torch.bfloat16, device=dev)
            dAm = torch.empty((r, Km), dtype=torch.float32, device=dev)
            dBm = torch.empty((Nm, r), dtype=torch.float32, device=dev)
            fwd_ms = ev_time(lambda: qb.qlora_linear_fwd(Xm, qm, Am, Bm, s, ws=wsm, out=Ym), 5)
            bwd_ms = ev_time(lambda: qb.qlora_linear_bwd(dYm, Xm, qm, Am, Bm, s, ws=wsm, outs=(dXm, dAm, dBm)), 5)
            qb.qlora_profile_reset()
            qb.qlora_profile_enable(True)
            for _ in range(3):
                qb.qlora_linear_fwd(Xm, qm, Am, Bm, s, ws=wsm, out=Ym)
                qb.qlora_linear_bwd(dYm, Xm, qm, Am, Bm, s, ws=wsm, outs=(dXm, dAm, dBm))
            torch.cuda.synchronize()
            qb.qlora_profile_enable(False)
            kf = qb.qlora_profile_read(qb.QLORA_PROF_FWD_GEMM)
            kd = qb.qlora_profile_read(qb.QLORA_PROF_BWD_DX)
            qb.qlora_profile_reset()
            ff = 2.0 * Mm * Nm * Km + 2.0 * Mm * r * (Km + Nm)
            bf = 2.0 * Mm * Nm * Km + 4.0 * Mm * r * (Nm + Km)
            kf_us, kd_us = kf[0] / kf[1] * 1e3, kd[0] / kd[1] * 1e3
            mlp[name] = {"M": Mm, "N": Nm, "K": Km, "r": r,
                         "fwd_us": fwd_ms * 1e3, "fwd_tflops": ff / (fwd_ms * 1e-3) / 1e12,
                         "bwd_us": bwd_ms * 1e3, "bwd_tflops": bf / (bwd_ms * 1e-3) / 1e12,
                         "fwd_gemm_kernel_us": kf_us,
                         "fwd_gemm_kernel_tflops": 2.0 * Mm * Nm * (Km + r) / (kf_us * 1e-6) / 1e12,
                         "bwd_dx_kernel_us": kd_us,
                         "bwd_dx_kernel_tflops": 2.0 * Mm * Km * (Nm + r) / (kd_us * 1e-6) / 1e12}
            for k in ("fwd_tflops", "bwd_tflops", "fwd_gemm_kernel_tflops", "bwd_dx_kernel_tflops"):
                mlp[name][k.replace("tflops", "frac_of_bf16_peak")] = mlp[name][k] / BF16_PEAK_TFLOPS
            log(f"{name}: fwd {fwd_ms * 1e3:.1f} us ({mlp[name]['fwd_tflops']:.0f} TFLOP/s), "
                f"bwd {bwd_ms * 1e3:.1f} us ({mlp[name]['bwd_tflops']:.0f} TFLOP/s)")
            del qm, Xm, dYm, Am, Bm, wsm, Ym, dXm, dAm, dBm
            torch.cuda.empty_cache()

    # dequantize alone at the 65B shapes (bf16 and fp32 out), rotating over
    # enough weights that the codes read exceed the rotation bound (the
    # streaming output stores leave the codes in the last-level cache otherwise)
    dq_solo = {}
    if not args.no_large:
        for name, (Nq, Kq) in (("up65b", (22016, 8192)), ("attn65b", (8192, 8192))):
            st = qb.qlora_nf4_storage_bytes(Nq, Kq)
            Rq = max(2, ROTATE_BYTES // st + 1)
            qs2 = [qb.qlora_nf4_quantize(dev_normal((Nq, Kq), 0.02, 500 + i)) for i in range(Rq)]
            for dt, esz in ((torch.bfloat16, 2), (torch.float32, 4)):
                outs2 = [torch.empty((Nq, Kq), dtype=dt, device=dev) for _ in range(Rq)]
                ms = ev_time(lambda: [qb.qlora_nf4_dequantize(qs2[i], dt, out=outs2[i]) for i in range(Rq)], 3) / Rq
                byts = st + esz * Nq * Kq
                key = f"{name}_{'bf16' if esz == 2 else 'f32'}"
                dq_solo[key] = {"N": Nq, "K": Kq, "us": ms * 1e3, "bytes": byts, "rotation": Rq,
                                "gbs": byts / (ms * 1e-3) / 1e9,
                                "frac_of_hbm_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
                log(f"dequantize {key}: {ms * 1e3:.1f} us, {dq_solo[key]['gbs']:.0f} GB/s")
                del outs2
            del qs2
            torch.cuda.empty_cache()

    # whole 65B-shaped stack: per layer, 4 x 8192^2 + 3 x 8192x22016 bf16
    # tensors generated on the device, then quantize + dequantize (bf16) of
    # all seven timed back to back
    wm = None
    if not args.no_large:
        shapes = [(8192, 8192)] * 4 + [(22016, 8192), (22016, 8192), (8192, 22016)]
        layers = args.wm_layers
        qs7 = [qb.NF4Weight.empty(a, b, dev) for a, b in shapes]
        outs7 = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in shapes]
        wsq = torch.empty(max(qb.qlora_nf4_quantize_workspace_bytes(a, b) for a, b in shapes),
                          dtype=torch.uint8, device=dev)
        total_ms = 0.0
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for layer in range(layers):
            ws7 = [dev_normal(sh, 0.02, 1000 * layer + t) for t, sh in enumerate(shapes)]
            torch.cuda.synchronize()
            ev0.record()
            for t in range(7):
                qb.qlora_nf4_quantize(ws7[t], out=qs7[t], ws=wsq)
                qb.qlora_nf4_dequantize(qs7[t], torch.bfloat16, out=outs7[t])
            ev1.record()
            torch.cuda.synchronize()
            total_ms += ev0.elapsed_time(ev1)
            del ws7
        n_layer = sum(a * b for a, b in shapes)
        st_layer = sum(qb.qlora_nf4_storage_bytes(a, b) for a, b in shapes)
        byts = layers * 2 * (2 * n_layer + st_layer)
        wm = {"layers": layers, "params_per_layer": n_layer, "total_ms": total_ms,
              "ms_per_layer": total_ms / layers, "ms_80_layers": total_ms / layers * 80,
              "bytes": byts, "gbs": byts / (total_ms * 1e-3) / 1e9,
              "frac_of_hbm_peak": byts / (total_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"whole-model round trip: {layers} layers in {total_ms:.1f} ms "
            f"({total_ms / layers:.3f} ms/layer, {wm['gbs']:.0f} GB/s)")
        del qs7, outs7, wsq
        torch.cuda.empty_cache()

    # ------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, fwd_flops + bwd_flops, args.cpu_seconds)

    dom_row = rows[dom]
    roofline = {
        "kernel": "k_fwd_big (fused NF4 dequant-GEMM + LoRA fold)" if dom == "fwd_gemm"
        else "k_dx_big (transposed NF4 dequant-GEMM + dH A fold)",
        "bound": "mfma",
        "achieved": dom_row["tflops"],
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": dom_row["tflops"] / BF16_PEAK_TFLOPS,
        "traffic": load_traffic(dom),
        "launch_us": dom_row["us"],
        "flops_per_launch": dom_row["flops"],
    }
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_eager": ms_step_eager,
        "hip_graph": graph_ok,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations and gradients)",
        "config": {"workload": "Llama-7B attention projection: W 4096x4096 NF4+DQ, "
                               "X [4x1024 tokens, 4096] bf16, LoRA r=64 alpha=16; step = "
                               "quantize + dequantize + fused forward + backward",
                   "M": M, "N": N, "K": K, "r": r, "scale": s,
                   "step_flops": fwd_flops + bwd_flops},
        "roofline": roofline,
        "rows": rows,
        "library_gemm_context": library,
        "decode": decode,
        "formats": formats,
        "merge": merge_row,
        "adamw": opt,
        "layer7b_projections": layer_row,
        "decoder_layer7b": dec_row,
        "mlp65b": mlp,
        "dequant_solo": dq_solo,
        "whole_model_roundtrip": wm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def _cpu_model() -> str:
    """The host CPU's model name (the first processor of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, step_flops, seconds):
    """Time the oracle (as it stands) for whole steps of the same workload on
    this host: quantize + dequantize (NumPy, one thread) and the fp64
    forward / backward matmuls (BLAS thread pool)."""
    import numpy as np
    import synth
    from oracle import linear, nf4
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001 - threadpoolctl is optional
        threads = os.cpu_count() or 1
    cb = nf4.nf4_codebook()
    w32 = wl.W_f32()
    X32, dY32 = synth.bf16_to_f32(wl.X), synth.bf16_to_f32(wl.dY)
    t0 = time.perf_counter()
    nsteps = 0
    while True:
        q = nf4.quantize(w32, cb)
        What = nf4.dequantize(q, cb)
        linear.forward(X32, What, wl.A, wl.B, wl.s)
        linear.backward(dY32, X32, What, wl.A, wl.B, wl.s)
        nsteps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / nsteps
    cpu_model = _cpu_model()
    log(f"cpu oracle: {dt:.2f} s per step on {threads} BLAS threads ({cpu_model})")
    return {"value": step_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model, "host_logical_cpus": os.cpu_count(),
            "sample": f"{nsteps} whole oracle step(s) of the same workload (quantize, dequantize, "
                      f"fp64 fwd+bwd at M=4096), {dt:.2f} s per step",
            "s_per_step": dt}


if __name__ == "__main__":
    main()

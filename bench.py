"""Benchmark: one MI355X, a stack of 30 Gemma-4-26B-A4B-shaped MoE layers with
128 int4 experts each (11.3 GiB of packed experts resident in HBM, each layer's
experts found through its own expert -> slot table in shuffled slot order).

A step is one pass of the whole path -- router top-k, permutation, gated w13
(gate+up) + activation, w2 down, weighted combine -- over all 30 layers for a
decode batch of T = 16 tokens (fresh synthetic logits and activations per
layer).  The step is captured once in a HIP graph and replayed; the timed
region brackets K replays with a device synchronisation on both sides.

Printed: one JSON line with tokens/s (value), ms per step, the achieved HBM
GB/s of the step, the roofline of the dominant kernel (the gate/up half of the
expert FFN, timed with HIP events on its own stream in an instrumented pass of
the same steps), the 1024-token prefill chunk through the same stack (MFMA
utilisation), and the CPU oracle timed on a bounded sample on this host.

Other measurements, each instead of the step and printing its own JSON line:
  --configs        single-layer timings of the other workloads (bf16 / int8 /
                   int4, decode and prefill, uniform and Zipf routing)
  --slot-fill      int4 expert slot fill: pinned DMA, unpack, and both
  --miss-step      decode with 15 of 128 experts resident, misses copied in,
                   at min_weight 1.0 / 0.6 / 0.4
  --refresh-step   the same with a residency refresh every 4 tokens
  --router         router GEMV + top-k against matmul + top-k
  --residency      the residency refresh kernel alone
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

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
# the kernel moe_ffn_gate_up launches for int4 at H = 2816, T <= 16 (the whole call)
GATE_UP_KERNEL = "gate_up_int4_dec_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_int4_T16.json")
CALIB_BYTES = 512 << 20
MFMA_BF16_PEAK_TFLOPS = 2500.0
G = synth.GEMMA
L_LAYERS = 30


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_stack(lib, seed, L, E, H, FF, fmt, device):
    """Pool of L*E slots; expert e of layer l at slot pi[l*E + e]."""
    import torch
    sb = lib.expert_bytes(fmt, H, FF)
    slots = synth.slot_table(seed, L, E)
    pool = torch.empty(L * E * sb, dtype=torch.uint8, device=device)
    for l in range(L):
        w13, w2 = synth.layer_weights_cuda(seed, l, E, H, FF, device)
        w13i, w2i = w13.view(torch.int16), w2.view(torch.int16)
        for e in range(E):
            s = int(slots[l, e])
            lib.pack_expert(fmt, w13i[e], w2i[e], pool[s * sb:(s + 1) * sb])
        del w13, w2, w13i, w2i
    torch.cuda.synchronize()
    return pool, sb, slots


def layer_inputs(seed, L, T, E, H, device, zipf=None):
    import torch
    logits = [torch.from_numpy(synth.logits(seed, l, T, E, zipf)).to(device) for l in range(L)]
    xs = [torch.from_numpy(synth.x_bf16(seed, l, T, H).view(np.int16)).to(device).view(torch.bfloat16)
          for l in range(L)]
    return logits, xs


class StackRunner:
    """Raw C calls with every argument prepared once (no per-call marshalling).

    Each layer keeps its own routing results (ids, weights, offsets, sorted
    routes, route positions, dropped count) and its own output y, as the
    layers of a model would; the per-route outputs and the workspace are
    shared, since each layer is done with them before the next starts."""

    def __init__(self, lib, pool, sb, slots, T, E, k, H, FF, fmt, logits, xs, stream):
        import ctypes
        import torch
        from expert_ffn_amd.layer import MoeLayer
        self.L = len(logits)
        self.T = T
        self.sb = sb
        dev = pool.device
        # per-route outputs in bf16: half the bytes of the down write and the combine read
        self.ml = MoeLayer(E, k, H, FF, fmt, T, device=dev, out_dtype=torch.bfloat16)
        ml = self.ml
        self.slot_d = [torch.from_numpy(slots[l].copy()).to(dev) for l in range(self.L)]
        i32 = torch.int32
        self.rt = [dict(ids=torch.empty((T, k), dtype=i32, device=dev),
                        w=torch.empty((T, k), dtype=torch.float32, device=dev),
                        offsets=torch.empty(E + 1, dtype=i32, device=dev),
                        sorted_route=torch.empty(T * k, dtype=i32, device=dev),
                        route_pos=torch.empty(T * k, dtype=i32, device=dev),
                        n_dropped=torch.empty(1, dtype=i32, device=dev),
                        y=torch.empty((T, H), dtype=torch.bfloat16, device=dev))
                   for _ in range(self.L)]
        c = lib.lib()
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        s = ctypes.c_void_p(stream.cuda_stream)
        ws = ml.ws.numel()
        self.calls = []
        for l in range(self.L):
            slot, r = P(self.slot_d[l]), self.rt[l]
            # router top-k and grouping in one call (one launch for T k <= 1024)
            route = (c.moe_route_permute, (P(logits[l]), T, E, k, 1, slot, P(r["ids"]), P(r["w"]),
                                           P(r["offsets"]), P(r["sorted_route"]), P(r["route_pos"]),
                                           P(r["n_dropped"]), s))
            ffn_args = (P(pool), sb, slot, E, H, FF, fmt, 0, P(xs[l]), 1, T, k, P(r["offsets"]),
                        P(r["sorted_route"]), P(ml.out_routes), 1, P(ml.ws), ws, s)
            gu = (c.moe_ffn_gate_up, ffn_args)
            dn = (c.moe_ffn_down, ffn_args)
            comb = (c.moe_combine, (P(ml.out_routes), 1, P(r["w"]), P(r["route_pos"]), T, k, H,
                                    P(r["y"]), 1, s))
            self.calls.append((route, gu, dn, comb))

    @staticmethod
    def _call(fa):
        if fa[0](*fa[1]):
            raise RuntimeError("launch failed")

    def step(self, events=None):
        for l, (route, gu, dn, comb) in enumerate(self.calls):
            self._call(route)
            if events is not None:
                events[l][0].record()
            self._call(gu)
            if events is not None:
                events[l][1].record()
            self._call(dn)
            self._call(comb)

    def gate_up_only(self):
        """The gate/up half of every layer, back to back, on the routing the
        last step left (for timing that kernel alone)."""
        for _, gu, _, _ in self.calls:
            self._call(gu)

    def capture(self, stream, body=None):
        """A HIP graph of one step (or of body()), captured on stream."""
        import torch
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            (body or self.step)()
        return graph


def call_times(run, stream, reps, graphs=True):
    """Microseconds per launch of each call of the step -- route_permute,
    gate_up, down, combine -- from a HIP graph of that call for every layer
    (on the routing the last step left; eager calls with graphs=False),
    replayed `reps` times between two HIP events recorded on the stream the
    calls run on."""
    import torch
    out = {}
    for name, idx in (("route_permute", 0), ("gate_up", 1), ("down", 2), ("combine", 3)):
        body = lambda idx=idx: [run._call(c[idx]) for c in run.calls]
        g = run.capture(stream, body=body) if graphs else None
        fn = g.replay if graphs else body
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        out[name] = round(e0.elapsed_time(e1) * 1e3 / (reps * run.L), 2)
        del g
    return out


def trace_avg_us(kernel, summary=os.path.join(ROOT, "profiles", "kernels_int4_stack_decode_T16_prefill_T1024.md")):
    """Average duration of a kernel in the committed rocprofv3 trace summary
    (None if absent)."""
    try:
        with open(summary) as f:
            for line in f:
                if line.startswith(f"| `moe::{kernel}") and "(idle)" not in line and "(beside" not in line:
                    return float(line.split("|")[4])
    except OSError:
        pass
    return None


def measure_peaks(lib, dev, pool, run, stream, reps=5):
    """Achieved peaks on this GPU (the measurement library's kernels):
    streaming read of 8 GiB of the slot pool (best over grid sizes), the decode
    gate/up kernel's weight loads alone over the stack's layers, and
    back-to-back bf16 MFMA 32x32x16."""
    import ctypes

    import torch
    from expert_ffn_amd import _build
    P = ctypes.c_void_p
    pk = ctypes.CDLL(_build.PEAKS_LIB)
    pk.peak_stream_read.argtypes = [P, ctypes.c_uint64, ctypes.c_int, P, P]
    pk.peak_tile_loads.argtypes = [P, ctypes.c_uint64, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    pk.peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    s = P(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def timed(fn, n):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n   # s per call

    out = {}
    nbytes = min(pool.numel(), 8 << 30)
    best = (0.0, 0)
    for blocks in (cus * 4, cus * 8, cus * 16, cus * 32):
        t = timed(lambda: pk.peak_stream_read(P(pool.data_ptr()), nbytes, blocks, P(sink.data_ptr()), s), reps)
        best = max(best, (nbytes / t / 1e9, blocks))
    out["hbm_stream_read_gbs"] = round(best[0], 1)
    out["hbm_stream_read_blocks"] = best[1]
    E, H, FF = G["E"], G["H"], G["FF"]
    w13_codes = 2 * FF * H // 2
    dist = [int((np.diff(r["offsets"].cpu().numpy()) > 0).sum()) for r in run.rt]

    def tiles():
        for l in range(run.L):
            pk.peak_tile_loads(P(pool.data_ptr()), run.sb, P(run.slot_d[l].data_ptr()),
                               P(run.rt[l]["offsets"].data_ptr()), E, H, FF, P(sink.data_ptr()), s)
    t = timed(tiles, reps)
    out["decode_tile_loads_gbs"] = round(sum(dist) * w13_codes / t / 1e9, 1)
    iters, blocks = 4000, cus * 2
    fsink = sink.view(torch.float32)
    t = timed(lambda: pk.peak_mfma_bf16(blocks, iters, P(fsink.data_ptr()), s), reps)
    out["mfma_bf16_tflops"] = round(blocks * 4 * iters * 4 * 32768 / t / 1e12, 1)
    out["note"] = ("stream read: 16-byte loads, 8 in flight per thread, over 8 GiB; tile loads: the "
                   "decode gate/up kernel's weight fragments only (w13 codes of the routed experts, "
                   "no compute); mfma: 4 independent 32x32x16 bf16 chains per wave, 8 waves per CU")
    return out


def realised_routing(lib, runner, logits):
    """Distinct experts and routes per layer (read once, outside any timing)."""
    import torch
    out = []
    for l, (route, _, _, _) in enumerate(runner.calls):
        runner._call(route)
        torch.cuda.synchronize()
        off = runner.rt[l]["offsets"].cpu().numpy()
        counts = np.diff(off)
        out.append((int((counts > 0).sum()), int(off[-1])))
    return out


def kernel_source_hash():
    """Hash of the sources the gate/up decode kernel is compiled from: the
    headers it includes and the int4 section of its file (the int4 helpers
    and kernels up to the down decode kernel; the launch code after it is not
    part of the kernel).  Counter figures taken on other sources are not used."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "expert_ffn_amd", "csrc")
    for name in ("common.h", "kernels.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    with open(os.path.join(csrc, "ffn.hip"), "rb") as f:
        text = f.read()
    a = text.index(b"// ------------------------------------------------------------ int4 paths --")
    b = text.index(b"// ------------------------------------------------------ int4 down, decode --")
    h.update(b"ffn.hip" + text[a:b])
    return h.hexdigest()[:16]


def measured_traffic(kernel_hash):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter runs,
    if they were taken on the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    return d.get("bytes_per_launch") if d.get("kernel_hash") == kernel_hash else None


def calibration_copies(device, reps=3):
    """Plain copies of known size for scaling the HBM byte counters: a
    device-to-device copy (the runtime's copy kernel) and a torch elementwise
    copy (neg), CALIB_BYTES read and CALIB_BYTES written each."""
    import torch
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _counter_rows(d):
    """(kernel name, counter, value) of every dispatch in a rocprofv3 --pmc
    run written with -f csv under directory d."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def summarize_pmc(fetch_dir, write_dir, commands):
    """HBM bytes per gate/up launch from a FETCH_SIZE run and a WRITE_SIZE run
    (KiB per dispatch), each scaled by the reading of the same counter for the
    calibration copy of CALIB_BYTES; written to TRAFFIC_FILE."""
    out = dict(kernel=GATE_UP_KERNEL, kernel_hash=kernel_source_hash(), calib_bytes=CALIB_BYTES,
               commands=commands)
    for key, d, cname in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = [(k, v) for k, c, v in _counter_rows(d) if c == cname]
        gate = [v for k, v in rows if GATE_UP_KERNEL in k]
        # launches that streamed weights (at T = 1024 the kernel runs with no group of its own)
        gate = [v for v in gate if v >= 0.5 * max(gate)] if gate else gate
        for calib_name in ("copyBuffer", "neg_kernel"):
            cal = [v for k, v in rows if calib_name in k and v * 1024 > CALIB_BYTES / 4]
            if cal:
                break
        if not gate or not cal:
            raise SystemExit(f"{cname}: {len(gate)} gate/up and {len(cal)} calibration dispatches")
        factor = CALIB_BYTES / (float(np.median(cal)) * 1024.0)
        out[key] = dict(counter=cname, kib_per_launch=float(np.mean(gate)), launches=len(gate),
                        calib_kernel=calib_name, calib_kib=float(np.median(cal)), scale=factor,
                        bytes_per_launch=float(np.mean(gate)) * 1024.0 * factor)
    out["bytes_per_launch"] = round(out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"])
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def summarize_counters(dirs, dest, command, kernels):
    """Per kernel (names containing one of `kernels`), the mean per dispatch of
    every counter collected by the rocprofv3 --pmc runs under dirs, and the
    ratios derived from them, as markdown.  Dispatches shorter than a quarter
    of the kernel's 90th-percentile duration (launches that found no work)
    are left out."""
    import csv
    import glob
    disp = {}   # (kernel, run dir, dispatch id) -> {counter: value, "_us": duration}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as f:
                for r in csv.DictReader(f):
                    base = r["Kernel_Name"].split("(")[0].replace("void ", "")
                    if not any(kk in base for kk in kernels):
                        continue
                    rec = disp.setdefault((base, d, r["Dispatch_Id"]), {})
                    rec[r["Counter_Name"]] = float(r["Counter_Value"])
                    rec["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    table = {}
    for (base, _, _), rec in disp.items():
        table.setdefault(base, []).append(rec)
    for base, recs in table.items():
        p90 = np.percentile([r["_us"] for r in recs], 90)
        table[base] = [r for r in recs if r["_us"] >= 0.25 * p90]

    def mean(recs, c):
        v = [r[c] for r in recs if c in r]
        return float(np.mean(v)) if v else float("nan")

    cols = sorted({c for recs in table.values() for r in recs for c in r if c != "_us"})
    lines = ["# rocprofv3 counters per dispatch", "", "Commands (from the repository root):", "", "```",
             command, "```", "",
             "Raw means per dispatch (launches that found no work left out):", "",
             "| kernel | dispatches | avg us | " + " | ".join(cols) + " |",
             "|---|---|---|" + "---|" * len(cols)]
    for name, recs in sorted(table.items()):
        vals = [f"{mean(recs, c):.4g}" for c in cols]
        lines.append(f"| `{name[:60]}` | {len(recs)} | {mean(recs, '_us'):.2f} | " + " | ".join(vals) + " |")
    lines += ["", "Derived (per dispatch; MI355X has 8 XCDs, 256 CUs, 1024 SIMDs):", "",
              "- cycles = the smaller of GRBM_GUI_ACTIVE / 8 (it counts on every XCD, over a window a few us",
              "  longer than a short kernel) and duration x 2.4 GHz; window GHz = GRBM_GUI_ACTIVE / 8 / duration;",
              "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles);",
              "- VALU issue = 4 x SQ_ACTIVE_INST_VALU (quad-cycles, MFMA issue included) / (1024 x cycles);",
              "- waves/SIMD = 4 x SQ_WAVE_CYCLES (quad-cycles) / (1024 x cycles), the mean resident waves;",
              "- s_waitcnt share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, wave time spent waiting on a counter;",
              "- issued TFLOP/s = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 / duration (padding included);",
              "- VALU/MFMA = non-MFMA VALU instructions per MFMA instruction;",
              "- LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS;",
              "- L2 hit = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum).", "",
              "| kernel | window GHz | MFMA busy | VALU issue | waves/SIMD | s_waitcnt share | issued TFLOP/s | "
              "VALU/MFMA | LDS conflict | L2 hit |", "|---|---|---|---|---|---|---|---|---|---|"]
    for name, recs in sorted(table.items()):
        us = mean(recs, "_us")
        win = mean(recs, "GRBM_GUI_ACTIVE") / 8
        cyc = min(win, us * 2.4e3)
        simd = 1024 * cyc
        mf = mean(recs, "SQ_INSTS_MFMA")
        row = [win / (us * 1e3), mean(recs, "SQ_VALU_MFMA_BUSY_CYCLES") / simd,
               4 * mean(recs, "SQ_ACTIVE_INST_VALU") / simd, 4 * mean(recs, "SQ_WAVE_CYCLES") / simd,
               mean(recs, "SQ_WAIT_INST_ANY") / mean(recs, "SQ_WAVE_CYCLES"),
               512 * mean(recs, "SQ_INSTS_VALU_MFMA_MOPS_BF16") / (us * 1e6),
               (mean(recs, "SQ_INSTS_VALU") - mf) / mf if mf else float("nan"),
               mean(recs, "SQ_LDS_BANK_CONFLICT") / mean(recs, "SQ_ACTIVE_INST_LDS")
               if mean(recs, "SQ_ACTIVE_INST_LDS") else float("nan"),
               mean(recs, "TCC_HIT_sum") / (mean(recs, "TCC_HIT_sum") + mean(recs, "TCC_MISS_sum"))]
        lines.append(f"| `{name[:60]}` | " + " | ".join(f"{v:.3g}" for v in row) + " |")
    with open(dest, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_dir, dest, command):
    """Per-kernel count / average / median duration from a rocprofv3
    --kernel-trace --stats run written with -f csv, as a markdown table."""
    import csv
    import glob
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    launches = []
    for path in paths:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"].split("(")[0].replace("void ", "")
                launches.append((name, r.get("Grid_Size_Y") or r.get("Grid_Size", ""),
                                 int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    # launches that overlap a grouped-GEMM launch in time (the two kernel
    # families of one call run side by side on two streams)
    gemm = sorted((a, b) for n, _, a, b in launches if "ffn_int4_gemm_kernel" in n)
    starts = [a for a, _ in gemm]
    import bisect

    def beside_gemm(a, b):
        i = bisect.bisect_left(starts, b)   # GEMM launches starting before b
        return any(gemm[j][1] > a for j in range(max(0, i - 4), i))
    by = {}
    for name, grid, a, b in launches:
        if "ffn_int4_gemm_kernel" not in name and gemm and beside_gemm(a, b):
            name += " (beside the GEMM)"
        by.setdefault((name, grid), []).append((b - a) / 1e3)
    tot = sum(sum(v) for v in by.values())
    lines = ["# rocprofv3 kernel trace summary", "", "Command (from the repository root):", "",
             "```", command, "```", "",
             "Launches that overlap a grouped-GEMM launch in time are listed apart (beside the GEMM):",
             "at T > 32 the streaming kernels run on the caller's stream while the GEMM runs on a",
             "second one, and at T = 1024 they find almost no group of their own.  Other launches of",
             "a kernel shorter than a quarter of its 90th-percentile duration are listed apart as idle.", "",
             "| kernel | grid y | launches | avg us | median us | min us | max us | share |",
             "|---|---|---|---|---|---|---|---|"]
    rows = []
    for (name, grid), v in by.items():
        a = np.array(v)
        idle = a < 0.25 * np.percentile(a, 90)
        if idle.any() and (~idle).any():
            rows.append((name, grid, a[~idle]))
            rows.append((name + " (idle)", grid, a[idle]))
        else:
            rows.append((name, grid, a))
    for name, grid, a in sorted(rows, key=lambda r: -r[2].sum()):
        lines.append(f"| `{name[:78]}` | {grid} | {len(a)} | {a.mean():.2f} | {np.median(a):.2f} | "
                     f"{a.min():.2f} | {a.max():.2f} | {100 * a.sum() / tot:.1f} % |")
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        lines += ["", "rocprofv3 --stats (kernel_stats.csv):", "", "```"]
        with open(stats[0]) as f:
            lines += [l.rstrip("\n") for l in f]
        lines += ["```"]
    with open(dest, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:40]))


def _oracle_layer_setup(seed_w, seed_x, layer, T):
    """Inputs of one stack layer for the oracle: logits, fp32 x, and a pool
    with the experts those logits route to, packed by the oracle from the
    layer's bf16 weights (drawn as the stack draws them).  Not timed."""
    import torch

    import oracle as ora
    E, k, H, FF = G["E"], G["k"], G["H"], G["FF"]
    logits = synth.logits(seed_x, layer, T, E)
    x = ora.bf16_to_f32(synth.x_bf16(seed_x, layer, T, H))
    ids, _ = ora.route_topk(logits, k)
    need = sorted(set(int(e) for e in ids.reshape(-1)))
    w13, w2 = synth.layer_weights_cuda(seed_w, layer, E, H, FF, "cuda")
    w13 = w13.view(torch.int16).cpu().numpy().view(np.uint16)
    w2 = w2.view(torch.int16).cpu().numpy().view(np.uint16)
    sb = ora.expert_bytes(2, H, FF)
    pool = np.zeros(E * sb, np.uint8)
    for e in need:
        pool[e * sb:(e + 1) * sb] = ora.pack_expert(2, w13[e], w2[e], H, FF)
    del w13, w2
    return logits, x, pool, sb, np.arange(E, dtype=np.int32), len(need)


def cpu_baseline(seed, T, layers=L_LAYERS):
    """The oracle as it stands (plain C, fp64 accumulation, OpenMP over routes)
    on bounded samples of the benchmark's own inputs, route + permute + FFN +
    combine per layer (packing and input generation not timed):
      decode  layer 0 at T tokens, all host threads (median of 3 runs) and one
              thread (one run), scaled to the step of `layers` layers;
      prefill layers 0 and 15 at T = 1024 (one run each, all threads), the
              mean extrapolated to the chunk of `layers` layers.
    value = the all-thread decode rate, in the headline's unit."""
    import oracle as ora
    E, k, H, FF = G["E"], G["k"], G["H"], G["FF"]
    threads = ora.set_threads(0)
    legs = []

    def run(setup, reps):
        logits, x, pool, sb, slot_of, _ = setup
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            ora.moe_layer(logits, x, pool, sb, slot_of, H, FF, 2, 0, k)
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    dec = _oracle_layer_setup(seed, seed, 0, T)
    t_all = run(dec, 3)
    legs.append(dict(leg="decode", T=T, threads=threads, s_per_layer=round(t_all, 4),
                     tokens_per_s=round(T / (t_all * layers), 3)))
    ora.set_threads(1)
    t_one = run(dec, 1)
    ora.set_threads(threads)
    legs.append(dict(leg="decode", T=T, threads=1, s_per_layer=round(t_one, 4),
                     tokens_per_s=round(T / (t_one * layers), 4)))
    del dec
    tp = []
    for l in (0, 15):
        pre = _oracle_layer_setup(seed, seed + 1, l, 1024)
        tp.append(run(pre, 1))
        del pre
    t_pre = float(np.mean(tp))
    legs.append(dict(leg="prefill", T=1024, threads=threads, layers_sampled=[0, 15],
                     s_per_layer=[round(v, 3) for v in tp],
                     tokens_per_s=round(1024 / (t_pre * layers), 3),
                     note=f"extrapolated from 2 sampled layers to {layers}"))
    return dict(value=legs[0]["tokens_per_s"], unit="tokens/s", cores=threads, kind="oracle",
                sample=f"decode: layer 0 of {layers} at T={T} ({dec_need_note(seed, T)}), median of 3 runs of "
                       f"route+permute+FFN+combine on {threads} threads, {t_all * 1e3:.1f} ms per layer, "
                       f"scaled x{layers} to the stack step; also 1 thread and a T=1024 prefill leg (legs)",
                legs=legs)


def dec_need_note(seed, T):
    import oracle as ora
    ids, _ = ora.route_topk(synth.logits(seed, 0, T, G["E"]), G["k"])
    return f"int4, {len(set(ids.reshape(-1).tolist()))} distinct experts"


def measure_configs(lib, dev, seed, copies=4, reps=20):
    """Single-layer timings of the other Gemma-shaped workloads (bf16 decode
    T = 1, 4, 16, 64; int8 decode T = 16 with Zipf routing; int4 at T = 128
    with Zipf routing and T = 256 uniform, where the streaming kernels and the
    grouped GEMM share a call; int4 prefill T = 1024, uniform and Zipf).  Each runs over `copies` independently packed
    copies of the layer, in turn, so that the weights come from HBM and not
    from the 256 MB last-level cache; a replay of one graph per copy round."""
    import torch
    E, k, H, FF = G["E"], G["k"], G["H"], G["FF"]
    cases = [("bf16_decode", lib.W_BF16, T, None) for T in (1, 4, 16, 64)]
    cases += [("int8_decode_zipf", lib.W_INT8_ROW, 16, 1.1),
              ("int4_mid_zipf", lib.W_INT4_G64, 128, 1.1), ("int4_mid", lib.W_INT4_G64, 256, None),
              ("int4_prefill", lib.W_INT4_G64, 1024, None), ("int4_prefill_zipf", lib.W_INT4_G64, 1024, 1.1)]
    out, built = [], {}
    stream = torch.cuda.Stream()
    for name, fmt, T, zipf in cases:
        if fmt not in built:
            built.clear()
            torch.cuda.empty_cache()
            log(f"packing {copies} copies of the layer as format {fmt} ...")
            built[fmt] = build_stack(lib, seed + 11, copies, E, H, FF, fmt, dev)
        pool, sb, slots = built[fmt]
        logits, xs = layer_inputs(seed + 13, copies, T, E, H, dev, zipf)
        with torch.cuda.stream(stream):
            run = StackRunner(lib, pool, sb, slots, T, E, k, H, FF, fmt, logits, xs, stream)
            routing = realised_routing(lib, run, logits)
            for _ in range(3):
                run.step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                run.step()
            graph.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                graph.replay()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) / (reps * copies) * 1e6
            calls = call_times(run, stream, max(3, reps // 4))
            del graph, run
        distinct = float(np.mean([d for d, _ in routing]))
        kept = float(np.mean([r for _, r in routing]))
        byts = distinct * sb + 2 * T * H * 2 + T * E * 4 + T * k * 16
        flops = kept * 6.0 * H * FF
        out.append(dict(config=name, weights=["bf16", "int8_row", "int4_g64"][fmt], T=T, zipf=zipf,
                        us_per_layer=round(us, 2), tokens_per_s=round(T / (us * 1e-6), 1),
                        distinct_experts=round(distinct, 1), hbm_gbs=round(byts / (us * 1e-6) / 1e9, 1),
                        hbm_frac=round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        mfma_tflops=round(flops / (us * 1e-6) / 1e12, 1),
                        mfma_frac=round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                        calls_us=calls))
        log(json.dumps(out[-1]))
    return out


def measure_slot_fill(lib, dev, seed, n=64, reps=7):
    """Slot fill of Gemma-shaped int4 experts (prain README, "int4 experts on
    RDNA2": one DMA through a pinned buffer, then one unpack kernel).  n
    distinct canonical blobs (random bytes: the fill moves bytes, their values
    do not matter) in pinned host memory and in device memory; timed with
    events on one stream: the plain pinned host -> device copy, the unpack
    kernel alone (device source), and the whole fill from host (copy into a
    staging buffer, then the kernel)."""
    import torch
    H, FF, fmt = G["H"], G["FF"], lib.W_INT4_G64
    sb = lib.expert_bytes(fmt, H, FF)
    g = torch.Generator().manual_seed(seed + 17)
    host = torch.randint(0, 256, (n, sb), dtype=torch.uint8, generator=g).pin_memory()
    src = host.to(dev)
    slots = torch.empty((n, sb), dtype=torch.uint8, device=dev)
    staging = torch.empty((2, sb), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def timed(body):   # median over passes of us per expert
        with torch.cuda.stream(stream):
            body()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                body()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3 / n)
        return float(np.median(ts))

    def copy_only():
        for i in range(n):
            staging[i & 1].copy_(host[i], non_blocking=True)

    def unpack_only():
        for i in range(n):
            lib.fill_slot(fmt, src[i], H, FF, slots[i], stream=stream)

    def fill_from_host():
        for i in range(n):
            lib.fill_slot(fmt, host[i], H, FF, slots[i], staging=staging[i & 1], stream=stream)

    def fill_direct():
        for i in range(n):
            lib.fill_slot(fmt, host[i], H, FF, slots[i], stream=stream, direct=True)

    # interleaved rounds, median of the round medians (the bus is shared and noisy)
    runs = {f: [] for f in (copy_only, unpack_only, fill_from_host, fill_direct)}
    for _ in range(3):
        for f in runs:
            runs[f].append(timed(f))
    t_copy, t_unpack, t_fill, t_direct = (float(np.median(v)) for v in runs.values())
    # every fill must reproduce the device-source result byte for byte
    check = slots.clone()
    with torch.cuda.stream(stream):
        unpack_only()
    torch.cuda.synchronize()
    same = bool(torch.equal(check, slots))
    return dict(metric="int4 expert slot fill", unit="GB/s", config=dict(
                    workload=f"Gemma-4-26B-A4B int4 expert (H={H}, FF={FF}), {n} experts per pass"),
                expert_bytes=sb, h2d_GBps=round(sb / (t_copy * 1e-6) / 1e9, 2),
                unpack_hbm_GBps=round(2 * sb / (t_unpack * 1e-6) / 1e9, 1),
                unpack_us_per_expert=round(t_unpack, 2), h2d_us_per_expert=round(t_copy, 2),
                fill_from_host_us_per_expert=round(t_fill, 2),
                fill_from_host_GBps=round(sb / (t_fill * 1e-6) / 1e9, 2),
                fill_direct_us_per_expert=round(t_direct, 2),
                fill_direct_GBps=round(sb / (t_direct * 1e-6) / 1e9, 2),
                fills_agree=same)


def measure_router(lib, dev, seed, reps=200):
    """Router GEMV + top-k at the Gemma shape (E = 128, H = 2816, top-8, bf16
    hidden states, fp32 router weight): moe_router_topk (partial GEMV, then
    slice sums + top-k) against torch's fp32 matmul of the widened x followed
    by moe_route_topk.
    Each variant is captured once in a HIP graph of `reps` calls over
    different token blocks of a larger x (the weight stays in cache either
    way: it is 1.44 MB) and replayed; time per call."""
    import torch
    E, k, H = G["E"], G["k"], G["H"]
    wr = torch.from_numpy(synth.router_weight(seed, 0, E, H)).to(dev)
    stream = torch.cuda.Stream()
    rows = []
    for T in (1, 16, 64, 1024):
        copies = max(1, min(64, (64 << 20) // (T * H * 2)))
        x = torch.from_numpy(synth.x_bf16(seed, 0, T * copies, H).view(np.int16)).to(dev).view(torch.bfloat16)
        xs = [x[i * T:(i + 1) * T] for i in range(copies)]
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        ws = torch.empty(lib.router_ws_bytes(T, H, E), dtype=torch.uint8, device=dev)

        def fused(i):
            lib.router_topk(xs[i % copies], wr, k, logits, ws, ids, w, stream=stream)

        def split(i):
            torch.mm(xs[i % copies].float(), wr.t(), out=logits)
            lib.route_topk(logits, k, ids, w, 1, stream)

        out = dict(T=T)
        for name, f in (("fused", fused), ("split", split)):
            with torch.cuda.stream(stream):
                for i in range(3):
                    f(i)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(reps):
                        f(i)
                g.replay()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(5):
                    g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                out[f"{name}_us"] = round(a.elapsed_time(b) * 1e3 / (5 * reps), 2)
                del g
        flops = 2.0 * T * E * H
        out["fused_tflops"] = round(flops / (out["fused_us"] * 1e-6) / 1e12, 2)
        out["fused_frac_fp32"] = round(out["fused_tflops"] / 157.3, 4)
        rows.append(out)
        log(json.dumps(out))
    return dict(metric="router GEMV + top-k", unit="us per call",
                config=dict(workload=f"Gemma-4-26B-A4B router: E={E}, H={H}, top-{k}, bf16 x, fp32 weight"),
                rows=rows)


def measure_residency(lib, dev, seed, reps=200):
    """The residency refresh kernel at the Gemma shape (E = 128, 15 resident
    slots, budget 15) on one step's routes: decode (16 tokens x top-8) and a
    prefill chunk (1024 x 8); uniform and Zipf(1.1) routing.  Graph replays of
    `reps` calls, each starting from the same table (a copy back precedes the
    refresh inside the graph; its time is measured alone and subtracted)."""
    import torch
    E, k = G["E"], G["k"]
    budget = S = 15
    rows = []
    stream = torch.cuda.Stream()
    base = torch.full((E,), -1, dtype=torch.int32, device=dev)
    base[:S] = torch.arange(S, dtype=torch.int32, device=dev)
    slot = base.clone()
    outs = [torch.empty(n, dtype=torch.int32, device=dev) for n in (E, budget, E, E, E, 3)]
    for T, zipf in ((16, None), (1024, None), (16, 1.1), (1024, 1.1)):
        ids_h, _ = _oracle_free_topk(synth.logits(seed, 0, T, E, zipf), k)
        ids = torch.from_numpy(ids_h).to(dev)

        def one(with_refresh):
            slot.copy_(base)
            if with_refresh:
                lib.residency_refresh(ids, E, budget, S, slot, *outs, stream=stream)

        t = {}
        for name, flag in (("copy_only", False), ("refresh", True)):
            with torch.cuda.stream(stream):
                one(flag)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for _ in range(reps):
                        one(flag)
                g.replay()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(5):
                    g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                t[name] = a.elapsed_time(b) * 1e3 / (5 * reps)
                del g
        one(True)
        torch.cuda.synchronize()
        c = outs[5].tolist()
        rows.append(dict(T=T, routes=T * k, zipf=zipf, us_per_refresh=round(t["refresh"] - t["copy_only"], 2),
                         promotions=c[1], demotions=c[2], MB_to_copy=round(c[1] * lib.expert_bytes(
                             lib.W_INT4_G64, G["H"], G["FF"]) / 1e6, 2)))
        log(json.dumps(rows[-1]))
    return dict(metric="residency refresh", unit="us per call",
                config=dict(workload=f"Gemma-4-26B-A4B layer: E={E}, top-{k}, {S} resident slots, budget {budget}"),
                rows=rows)


def _oracle_free_topk(logits, k):
    """Top-k ids of host logits with numpy (larger first, equal: lower id) --
    inputs for the refresh timing only."""
    return np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32), None


def measure_miss_step(lib, dev, seed, tokens=16, n_res=15, shares=(1.0, 0.6, 0.4)):
    """Decode (one token per step) through the 30-layer int4 stack when only
    n_res of each layer's 128 experts are resident (450 slots over 30 layers,
    as in prain's agent setup), for several min_weight shares (prain README,
    "Trading quality for speed").  Per layer: top-k and min_weight on the
    device, the miss counts back to the host, one slot fill per missed expert
    from pinned host memory (DMA + unpack), then grouping, the expert FFN and
    the combine; the filled slots are released again after the layer (a
    fixed resident set).  The host copies are layer 0's blobs for every
    layer: the fill moves bytes, and a copy's cost does not depend on them."""
    import ctypes
    import torch
    from expert_ffn_amd.layer import MoeLayer
    E, k, H, FF, Lyr = G["E"], G["k"], G["H"], G["FF"], synth.CONFIGS["int4_stack"]["L"]
    fmt = lib.W_INT4_G64
    log(f"packing the {Lyr}-layer int4 stack ...")
    pool, sb, slots = build_stack(lib, seed, Lyr, E, H, FF, fmt, dev)
    logits, xs = layer_inputs(seed + 1, Lyr, tokens, E, H, dev)
    r = np.random.default_rng(seed + 23)
    host = torch.empty((E, sb), dtype=torch.uint8).pin_memory()
    for e in range(E):
        host[e].copy_(pool[int(slots[0, e]) * sb:(int(slots[0, e]) + 1) * sb])
    staging = torch.empty((E, sb), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    c = lib.lib()
    P = ctypes.c_void_p
    s = P(stream.cuda_stream)
    ml = MoeLayer(E, k, H, FF, fmt, 1, device=dev, out_dtype=torch.bfloat16)
    miss_h = torch.zeros(E, dtype=torch.int32).pin_memory()

    def run(share, resident):
        base = []
        for l in range(Lyr):
            t = torch.full((E,), -1, dtype=torch.int32)
            keep = np.arange(E) if resident >= E else r.choice(E, resident, replace=False)
            t[torch.from_numpy(keep)] = torch.from_numpy(slots[l][keep].astype(np.int32))
            base.append(t.pin_memory())
        tab = [b.clone().pin_memory() for b in base]
        slot_d = [b.to(dev) for b in base]
        ws = ml.ws.numel()
        copies = 0

        def token(i):
            nonlocal copies
            for l in range(Lyr):
                sd = P(slot_d[l].data_ptr())
                lg, x = logits[l][i:i + 1], xs[l][i:i + 1]
                assert not c.moe_route_topk(P(lg.data_ptr()), 1, E, k, 1, P(ml.topk_ids.data_ptr()),
                                            P(ml.topk_w.data_ptr()), s)
                assert not c.moe_min_weight(P(ml.topk_ids.data_ptr()), P(ml.topk_w.data_ptr()), 1, k, E, sd,
                                            ctypes.c_float(share), P(ml.topk_ids.data_ptr()),
                                            P(ml.topk_w.data_ptr()), P(ml.miss_count.data_ptr()), s)
                miss_h.copy_(ml.miss_count, non_blocking=True)
                stream.synchronize()
                missed = np.flatnonzero(miss_h.numpy())
                if missed.size:
                    tab[l].copy_(base[l])
                    # the layer's copies back to back on the copy engine, then one
                    # unpack launch for all of them (moe_fill_slots)
                    n = missed.size
                    srcs = (P * n)(*[host[e].data_ptr() for e in missed])
                    dsts = (P * n)(*[pool.data_ptr() + int(slots[l, e]) * sb for e in missed])
                    assert not c.moe_fill_slots(fmt, n, srcs, H, FF, P(staging.data_ptr()), dsts, s)
                    for e in missed:
                        tab[l][e] = int(slots[l, e])
                    slot_d[l].copy_(tab[l], non_blocking=True)
                    copies += missed.size
                assert not c.moe_permute(P(ml.topk_ids.data_ptr()), 1, k, E, sd, P(ml.offsets.data_ptr()),
                                         P(ml.sorted_route.data_ptr()), P(ml.route_pos.data_ptr()),
                                         P(ml.n_dropped.data_ptr()), s)
                assert not c.moe_expert_ffn(P(pool.data_ptr()), sb, sd, E, H, FF, fmt, 0, P(x.data_ptr()), 1, 1,
                                            k, P(ml.offsets.data_ptr()), P(ml.sorted_route.data_ptr()),
                                            P(ml.out_routes.data_ptr()), 1, P(ml.ws.data_ptr()), ws, s)
                assert not c.moe_combine(P(ml.out_routes.data_ptr()), 1, P(ml.topk_w.data_ptr()),
                                         P(ml.route_pos.data_ptr()), 1, k, H, P(ml.y.data_ptr()), 1, s)
                if missed.size:
                    slot_d[l].copy_(base[l], non_blocking=True)     # release the filled slots

        with torch.cuda.stream(stream):
            token(0)
            stream.synchronize()
            copies = 0
            t0 = time.perf_counter()
            for i in range(1, tokens):
                token(i)
            stream.synchronize()
            dt = time.perf_counter() - t0
        n = tokens - 1
        return dict(min_weight=share, resident_per_layer=int(min(resident, E)),
                    tokens_per_s=round(n / dt, 2), ms_per_token=round(dt / n * 1e3, 2),
                    experts_copied_per_token=round(copies / n, 1),
                    GB_copied_per_token=round(copies / n * sb / 1e9, 3))

    rows = [run(sh, n_res) for sh in shares]
    ref = run(1.0, E)
    return dict(metric="decode tokens/s with expert misses", unit="tokens/s",
                config=dict(workload=f"Gemma-4-26B-A4B int4 stack, {Lyr} layers, one token per step, "
                                     f"{n_res} of {E} experts resident per layer, misses copied from pinned "
                                     f"host memory", tokens=tokens - 1),
                rows=rows, all_resident=ref)


def measure_refresh_step(lib, dev, seed, tokens=33, S=15, every=4, share=1.0):
    """Decode (one token per step) through 30 int4 layers with S = 15 resident
    slots per layer, misses copied in as in the miss step, with and without a
    residency refresh (rlx_runtime expert_pool.rs, TIDE-style: the budget
    most-hit experts, paired promote/demote) every `every` tokens from the
    hit counts of the last `every` tokens' routes; promoted experts are
    copied into their slots (one DMA + unpack each).  Uniform and Zipf(1.1)
    routing.  Each layer has its own region of S resident slots plus k miss
    slots; the resident set starts as experts 0 .. S-1 (the crate's initial
    pool).  The host copies are one layer's packed blobs, as in the miss
    step: a copy's cost does not depend on the bytes."""
    import ctypes
    import torch
    E, k, H, FF, Lyr = G["E"], G["k"], G["H"], G["FF"], synth.CONFIGS["int4_stack"]["L"]
    fmt = lib.W_INT4_G64
    sb = lib.expert_bytes(fmt, H, FF)
    NS = S + k                                  # slots per layer region
    log("packing one layer's experts for the host copies ...")
    one = torch.empty(E * sb, dtype=torch.uint8, device=dev)
    w13, w2 = synth.layer_weights_cuda(seed, 0, E, H, FF, dev)
    for e in range(E):
        lib.pack_expert(fmt, w13[e].view(torch.int16), w2[e].view(torch.int16), one[e * sb:(e + 1) * sb])
    host = one.view(E, sb).cpu().pin_memory()
    del one, w13, w2
    pool = torch.empty(Lyr * NS * sb, dtype=torch.uint8, device=dev)
    staging = torch.empty((E, sb), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    c = lib.lib()
    P = ctypes.c_void_p
    s = P(stream.cuda_stream)
    from expert_ffn_amd.layer import MoeLayer
    ml = MoeLayer(E, k, H, FF, fmt, 1, device=dev, out_dtype=torch.bfloat16)
    ws = ml.ws.numel()
    miss_h = torch.zeros(E, dtype=torch.int32).pin_memory()
    cnt_h = torch.zeros(3, dtype=torch.int32).pin_memory()
    prom_h = torch.zeros(2 * E, dtype=torch.int32).pin_memory()
    outs = [torch.empty(n, dtype=torch.int32, device=dev) for n in (E, S, E, E, E, 3)]
    hits, target, promote, promote_slot, demote, counts = outs
    rows = []
    for zipf in (None, 1.1):
        logits, xs = layer_inputs(seed + 5, Lyr, tokens, E, H, dev, zipf)
        for refresh in (False, True):
            # resident experts 0 .. S-1 in slots 0 .. S-1 of every layer's region
            for l in range(Lyr):
                for e in range(S):
                    lib.fill_slot(fmt, host[e], H, FF, pool[(l * NS + e) * sb:(l * NS + e + 1) * sb],
                                  staging=staging[e], stream=stream)
            stream.synchronize()
            base = []
            for l in range(Lyr):
                t = torch.full((E,), -1, dtype=torch.int32)
                t[:S] = torch.arange(S, dtype=torch.int32)
                base.append(t.to(dev))
            tab = torch.full((E,), -1, dtype=torch.int32).pin_memory()
            tmp_d = torch.empty(E, dtype=torch.int32, device=dev)
            ring = [torch.full((every * k,), -1, dtype=torch.int32, device=dev) for _ in range(Lyr)]
            copies = [0, 0]   # miss copies, promotion copies

            def token(i):
                for l in range(Lyr):
                    pl = pool.data_ptr() + l * NS * sb
                    lg, x = logits[l][i:i + 1], xs[l][i:i + 1]
                    ids_p, w_p = P(ml.topk_ids.data_ptr()), P(ml.topk_w.data_ptr())
                    assert not c.moe_route_topk(P(lg.data_ptr()), 1, E, k, 1, ids_p, w_p, s)
                    ring[l][(i % every) * k:(i % every + 1) * k].copy_(ml.topk_ids[0], non_blocking=True)
                    if refresh and i % every == every - 1:
                        assert not c.moe_residency_refresh(P(ring[l].data_ptr()), every * k, E, S, S,
                                                           P(base[l].data_ptr()), *(P(t.data_ptr()) for t in outs), s)
                        cnt_h.copy_(counts, non_blocking=True)
                        prom_h[:E].copy_(promote, non_blocking=True)
                        prom_h[E:].copy_(promote_slot, non_blocking=True)
                        stream.synchronize()
                        npro = int(cnt_h[1])
                        if npro:
                            srcs = (P * npro)(*[host[int(prom_h[j])].data_ptr() for j in range(npro)])
                            dsts = (P * npro)(*[pl + int(prom_h[E + j]) * sb for j in range(npro)])
                            assert not c.moe_fill_slots(fmt, npro, srcs, H, FF, P(staging.data_ptr()), dsts, s)
                        copies[1] += npro
                    sd = P(base[l].data_ptr())
                    assert not c.moe_min_weight(ids_p, w_p, 1, k, E, sd, ctypes.c_float(share), ids_p, w_p,
                                                P(ml.miss_count.data_ptr()), s)
                    miss_h.copy_(ml.miss_count, non_blocking=True)
                    stream.synchronize()
                    missed = np.flatnonzero(miss_h.numpy())
                    if missed.size:
                        tab.copy_(base[l])
                        n = missed.size
                        srcs = (P * n)(*[host[e].data_ptr() for e in missed])
                        dsts = (P * n)(*[pl + (S + j) * sb for j in range(n)])
                        assert not c.moe_fill_slots(fmt, n, srcs, H, FF, P(staging.data_ptr()), dsts, s)
                        for j, e in enumerate(missed):
                            tab[e] = S + j
                        tmp_d.copy_(tab, non_blocking=True)
                        sd = P(tmp_d.data_ptr())
                        copies[0] += missed.size
                    assert not c.moe_permute(ids_p, 1, k, E, sd, P(ml.offsets.data_ptr()),
                                             P(ml.sorted_route.data_ptr()), P(ml.route_pos.data_ptr()),
                                             P(ml.n_dropped.data_ptr()), s)
                    assert not c.moe_expert_ffn(P(pl), sb, sd, E, H, FF, fmt, 0, P(x.data_ptr()), 1, 1, k,
                                                P(ml.offsets.data_ptr()), P(ml.sorted_route.data_ptr()),
                                                P(ml.out_routes.data_ptr()), 1, P(ml.ws.data_ptr()), ws, s)
                    assert not c.moe_combine(P(ml.out_routes.data_ptr()), 1, w_p, P(ml.route_pos.data_ptr()), 1, k,
                                             H, P(ml.y.data_ptr()), 1, s)
                    if missed.size:
                        stream.synchronize()   # tab and the miss slots are reused by the next layer

            with torch.cuda.stream(stream):
                for i in range(every):          # warm-up: one refresh interval
                    token(i)
                stream.synchronize()
                copies[0] = copies[1] = 0
                t0 = time.perf_counter()
                for i in range(every, tokens):
                    token(i)
                stream.synchronize()
                dt = time.perf_counter() - t0
            n = tokens - every
            rows.append(dict(zipf=zipf, refresh_every=every if refresh else None, tokens_per_s=round(n / dt, 2),
                             ms_per_token=round(dt / n * 1e3, 2), miss_copies_per_token=round(copies[0] / n, 1),
                             promotion_copies_per_token=round(copies[1] / n, 1)))
            log(json.dumps(rows[-1]))
    return dict(metric="decode tokens/s with expert misses and residency refresh", unit="tokens/s",
                config=dict(workload=f"Gemma-4-26B-A4B int4, {Lyr} layers, one token per step, {S} of {E} experts "
                                     f"resident per layer, misses copied from pinned host memory, min_weight {share}",
                            tokens=tokens - every), rows=rows)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=16)
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--layers", type=int, default=L_LAYERS, help="stack depth (30; fewer for profiling runs)")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the achieved-peak microbenchmarks")
    ap.add_argument("--no-configs", dest="configs_summary", action="store_false",
                    help="skip the single-layer figures of the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run the plain copies that scale the HBM byte counters")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the gate/up traffic file from two rocprofv3 --pmc runs (no GPU)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "DEST"),
                    help="write a kernel-trace summary from a rocprofv3 run (no GPU)")
    ap.add_argument("--command", default="", help="the profiled command, recorded in summaries")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="counter table of --kernels from rocprofv3 --pmc runs, written to --dest")
    ap.add_argument("--kernels", nargs="+", default=["ffn_int4_gemm_kernel", "gate_up_int4_dec_kernel",
                                                     "down_int4_dec_kernel"])
    ap.add_argument("--dest", default="")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the stack step: single-layer timings of the other workloads "
                         "(one JSON object per line)")
    ap.add_argument("--refresh-step", action="store_true",
                    help="instead of the stack step: decode with misses, with and without a residency refresh "
                         "every 4 tokens, uniform and Zipf routing (one JSON line)")
    ap.add_argument("--residency", action="store_true",
                    help="instead of the stack step: residency refresh timings (one JSON line)")
    ap.add_argument("--router", action="store_true",
                    help="instead of the stack step: router GEMV + top-k timings, fused and split (one JSON line)")
    ap.add_argument("--miss-step", action="store_true",
                    help="instead of the stack step: decode with 15 of 128 experts resident per layer and "
                         "misses copied in, at min_weight 1.0 / 0.6 / 0.4 (one JSON line)")
    ap.add_argument("--slot-fill", action="store_true",
                    help="instead of the stack step: int4 expert slot fill rates (one JSON line)")
    args = ap.parse_args()
    if (args.summarize_pmc or args.summarize_trace or args.summarize_counters) and not args.command.strip():
        raise SystemExit("--command: the profiled command is recorded in the summary and must be given")
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, commands=args.command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, command=args.command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.dest, args.command, args.kernels)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the expert FFN here runs on one GPU and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import expert_ffn_amd as lib
    lib.lib()
    dev = torch.device("cuda:0")
    if args.refresh_step:
        print(json.dumps(measure_refresh_step(lib, dev, args.seed)), flush=True)
        return
    if args.residency:
        print(json.dumps(measure_residency(lib, dev, args.seed)), flush=True)
        return
    if args.router:
        print(json.dumps(measure_router(lib, dev, args.seed)), flush=True)
        return
    if args.miss_step:
        print(json.dumps(measure_miss_step(lib, dev, args.seed)), flush=True)
        return
    if args.slot_fill:
        print(json.dumps(measure_slot_fill(lib, dev, args.seed)), flush=True)
        return
    if args.configs:
        for r in measure_configs(lib, dev, args.seed):
            print(json.dumps(r), flush=True)
        return
    E, k, H, FF = G["E"], G["k"], G["H"], G["FF"]
    fmt = lib.W_INT4_G64
    T = args.tokens
    Ls = args.layers

    t0 = time.time()
    log(f"building the {Ls}-layer int4 stack ...")
    pool, sb, slots = build_stack(lib, args.seed, Ls, E, H, FF, fmt, dev)
    log(f"  pool {pool.numel() / 2**30:.2f} GiB, slot {sb} B, built in {time.time() - t0:.1f} s")

    if args.calib_copy:
        calibration_copies(dev)
    stream = torch.cuda.Stream()
    logits, xs = layer_inputs(args.seed, Ls, T, E, H, dev)
    with torch.cuda.stream(stream):
        run = StackRunner(lib, pool, sb, slots, T, E, k, H, FF, fmt, logits, xs, stream)
        routing = realised_routing(lib, run, logits)
        for _ in range(args.warmup):
            run.step()
        torch.cuda.synchronize()
        graph = None
        use_graph = not args.no_graph
        if use_graph:
            # the warmup steps again as replays of the graph the timed region
            # replays (its first replays after capture run slower)
            graph = run.capture(stream)
            for _ in range(max(3, args.warmup)):
                graph.replay()
        torch.cuda.synchronize()
        # timed region: K steps
        t_start = time.perf_counter()
        for _ in range(args.steps):
            graph.replay() if graph is not None else run.step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        # per-call times (HIP events around graphs of one call kind)
        calls = call_times(run, stream, max(5, min(args.steps, 20)), graphs=graph is not None)
        t_e = time.perf_counter()
        for _ in range(args.steps):
            run.step()
        torch.cuda.synchronize()
        eager_ms = (time.perf_counter() - t_e) / args.steps * 1e3
        peaks = measure_peaks(lib, dev, pool, run, stream) if args.peaks else None
    ms_per_step = elapsed / args.steps * 1e3
    tok_s = T * args.steps / elapsed

    # algorithmic bytes: each distinct expert's packed bytes once, plus x, y, logits and the route indices
    off = lib.blob_layout(fmt, H, FF)
    w13_bytes, w2_bytes = off[2], sb - off[2]   # w13 codes + scales; w2 codes + scales
    per_layer_io = T * H * 2 * 2 + T * E * 4 + T * k * 4 * 4 + (E + 1) * 4
    step_bytes = sum(d * sb + per_layer_io for d, _ in routing)
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    dist = float(np.mean([d for d, _ in routing]))
    gu_bytes = dist * w13_bytes + T * H * 2
    dn_bytes = dist * w2_bytes + T * k * FF * 2 + T * k * H * 2
    achieved = gu_bytes / (calls["gate_up"] * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = measured_traffic(khash)
    tr_us = trace_avg_us(GATE_UP_KERNEL)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel=GATE_UP_KERNEL + " (moe_ffn_gate_up)",
                    avg_launch_us=calls["gate_up"], bytes_per_launch=round(gu_bytes),
                    trace_avg_us=tr_us,
                    trace_frac=round(gu_bytes / (tr_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if tr_us else None)
    if peaks:
        roofline["frac_of_measured_stream"] = round(achieved / peaks["hbm_stream_read_gbs"], 4)
    kernels = {name: dict(us=us) for name, us in calls.items()}
    for name, b in (("gate_up", gu_bytes), ("down", dn_bytes)):
        kernels[name]["gbs"] = round(b / (calls[name] * 1e-6) / 1e9, 1)
        kernels[name]["hbm_frac"] = round(b / (calls[name] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    ffn_us = calls["gate_up"] + calls["down"]
    kernels["expert_ffn_hbm_frac"] = round((gu_bytes + dn_bytes) / (ffn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)

    # prefill chunk through the same stack
    prefill = None
    if args.prefill_steps > 0:
        Tp = 1024
        lp, xp = layer_inputs(args.seed + 1, Ls, Tp, E, H, dev)
        with torch.cuda.stream(stream):
            runp = StackRunner(lib, pool, sb, slots, Tp, E, k, H, FF, fmt, lp, xp, stream)
            rp = realised_routing(lib, runp, lp)
            runp.step()
            gp = runp.capture(stream) if use_graph else None
            stepp = gp.replay if gp is not None else runp.step
            for _ in range(3):   # warm replays before the timed ones
                stepp()
            torch.cuda.synchronize()
            tp = time.perf_counter()
            for _ in range(args.prefill_steps):
                stepp()
            torch.cuda.synchronize()
            pms = (time.perf_counter() - tp) / args.prefill_steps * 1e3
            callp = call_times(runp, stream, 3, graphs=gp is not None)
            del gp, stepp
        kept = sum(r for _, r in rp)
        flops = kept * 6.0 * H * FF
        pbytes = sum(d * sb for d, _ in rp) + Ls * (Tp * H * 2 * 2 + Tp * E * 4 + Tp * k * 16)
        gu_fl, dn_fl = kept / Ls * 4.0 * H * FF, kept / Ls * 2.0 * H * FF
        tf = lambda fl, us: fl / (us * 1e-6) / 1e12
        prefill = dict(T=Tp, ms_per_chunk=round(pms, 3), tokens_per_s=round(Tp / (pms * 1e-3), 1),
                       mfma_tflops=round(flops / (pms * 1e-3) / 1e12, 1),
                       mfma_frac=round(flops / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                       hbm_gbs=round(pbytes / (pms * 1e-3) / 1e9, 1),
                       hbm_frac=round(pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       calls_us=callp,
                       roofline=dict(bound="mfma", kernel="ffn_int4_gemm_kernel (moe_ffn_gate_up: prep + GEMM)",
                                     achieved=round(tf(gu_fl, callp["gate_up"]), 1), peak=MFMA_BF16_PEAK_TFLOPS,
                                     unit="TFLOP/s",
                                     frac=round(tf(gu_fl, callp["gate_up"]) / MFMA_BF16_PEAK_TFLOPS, 4),
                                     down_tflops=round(tf(dn_fl, callp["down"]), 1),
                                     down_frac=round(tf(dn_fl, callp["down"]) / MFMA_BF16_PEAK_TFLOPS, 4)))
        if peaks:
            prefill["mfma_frac_of_measured"] = round(prefill["mfma_tflops"] / peaks["mfma_bf16_tflops"], 4)
        del runp

    configs = None
    if args.configs_summary:
        log("single-layer timings of the other workloads ...")
        del graph, run
        torch.cuda.empty_cache()
        configs = [{k2: r[k2] for k2 in ("config", "T", "us_per_layer", "tokens_per_s", "hbm_frac", "mfma_frac", "calls_us")}
                   for r in measure_configs(lib, dev, args.seed)]

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on samples ...")
        tc = time.time()
        cpu = cpu_baseline(args.seed, T, Ls)
        log(f"  oracle legs took {time.time() - tc:.1f} s")

    out = {
        "metric": "expert-FFN tokens/s + HBM GB/s (int4 decode T=16) and MFMA util (T=1024 prefill)",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) logits and activations, N(0,0.02) weights; "
                "random-init Gemma-4-26B-A4B expert shapes)",
        "config": {"workload": f"int4_stack_decode: {Ls} MoE layers x 128 int4 experts (w4a16, bf16 scale "
                               "per 64, MSE clip), H=2816, FF=704, top-8 renormalised, T=16 decode, "
                               "shuffled per-layer slot tables, 11.3 GiB resident",
                   "layers": Ls, "experts": E, "top_k": k, "hidden": H, "ffn": FF,
                   "tokens": T, "weights": "int4_g64", "graph": use_graph},
        "hbm_gbs": round(step_gbs, 1), "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "distinct_experts_per_layer": round(dist, 2),
        "roofline": roofline,
        "kernels": kernels,
        "prefill": prefill,
        "peaks": peaks,
        "configs": configs,
        "cpu_baseline": cpu,
        "kernel_hash": khash,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the routed-MoE expert layer (2-bit routed experts) on one MI355X.

A step is one full pass of the layer's hot path on one batch: router
(logits, top-k, grouping), shared expert, routed expert FFN (gate/up +
SwiGLU + down) and the weighted combine.  The headline workload is decode of
one token through one DeepSeek-V3-class layer (H=7168, I=2048, 256 experts,
top-8, bf16 shared expert); the reported value is whole-step algorithmic
bytes / step time in GB/s.  The weights of the timed steps rotate over
several copies at distinct addresses, as a model cycles through its layers,
so they do not stay in the on-chip caches.

Prints one JSON line (rank 0, one GPU).  Every other workload of the layer
(batched decode, prefill, the Q4_K variants) is measured the same way and
reported inside it under "workloads": ms per step (mean, and median / p10 /
p90 of single steps), throughput, the dominant kernel's roofline and the
oracle's time on the host over a bounded sample.
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
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode GB/s (% HBM peak) + prefill tokens/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
CACHE = os.environ.get("MOE_CACHE_DIR", "/tmp/moe_layer_cache")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# sources that define each timed kernel (plus the shared headers)
_KERNEL_SOURCES = {"dec_": ["decode.hip", "decode.h", "route_dev.h"], "route_": ["route.hip", "route_dev.h"],
                   "ffn_prefill_": ["prefill.hip", "ffn.hip"], "ffn_decode_": ["prefill.hip", "ffn.hip"],
                   "bd_": ["prefill.hip", "ffn.hip"],
                   "ffn_schedule": ["ffn.hip"], "sh_finalize": ["ffn.hip"], "combine": ["ffn.hip"]}

# the library's launch names (moe_profile.name) and the GPU kernel symbols each one runs
LAUNCH_SYMBOLS = [
    ("dec_stage1", r"dec1_gateup_kernel<(?:true|false), [13],"),
    ("dec_stage2", r"dec1_gateup_kernel<(?:true|false), 2,"),
    ("dec_hform", r"dec1_hform_kernel"),
    ("dec_down_fused", r"dec1_down_fused_kernel"),
    ("bd_gateup", r"bd_kernel<[17], "),
    ("bd_down", r"bd_kernel<2, "),
    ("ffn_decode_gateup", r"np_kernel<\d+, true, true,"),
    ("ffn_decode_down", r"np_kernel<\d+, false, true,"),
    ("ffn_prefill_gateup", r"np_kernel<\d+, true, false,"),
    ("ffn_prefill_down", r"np_kernel<\d+, false, false,"),
    ("ffn_schedule", r"moe::ffn_schedule\("),
    ("sh_finalize", r"sh_finalize_kernel"),
    ("combine", r"moe::combine_kernel"),
    ("route_logits", r"route_logits_(?:small|tiled|mfma)"),
    ("route_partial", r"route_partial<"),
    ("route_select", r"route_select_(?:one|tok)[<(]"),
    ("route_select_small", r"route_select_small"),
    ("route_topk", r"route_topk<"),
    ("route_rank", r"route_rank\("),
    ("route_scan", r"route_scan\("),
    ("route_scatter", r"route_scatter\("),
]


def kernel_source_hash(kernel: str | None = None) -> str:
    """Hash of the sources of one kernel (all of csrc/ when kernel is None)."""
    h = hashlib.sha1()
    d = os.path.join(ROOT, "bit_quantized_routed_amd", "csrc")
    files = sorted(f for f in os.listdir(d) if f.endswith((".hip", ".h")))
    if kernel is not None:
        for prefix, own in _KERNEL_SOURCES.items():
            if kernel.startswith(prefix):
                files = sorted(own + ["common.h", "kernels.h"])
                break
    for f in files:
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:12]


def machine_ceilings():
    """What this machine sustains, measured with the library's probe kernels: the
    best streaming-read rate over a few launch shapes (1 GiB, read 5 times)
    and a bf16 MFMA loop filling every CU."""
    import torch
    import bit_quantized_routed_amd as M
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    best_gbs, best_grid = 0.0, None
    for nt in (False, True):
        for grid in (256, 512, 1024, 2048):
            sink = torch.empty(grid * 512 * 4, dtype=torch.int32, device="cuda")
            M.probe_stream_read(buf, grid, sink, nt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                M.probe_stream_read(buf, grid, sink, nt)
            e1.record()
            e1.synchronize()
            gbs = 5 * buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbs > best_gbs:
                best_gbs, best_grid = gbs, "%d%s" % (grid, " nontemporal" if nt else "")
    del buf
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    grid, iters = 4 * n_cu, 4000
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    # the 32x32x16 loop: the 16x16x32 probe loop carries compiler-inserted
    # accumulator moves (about 7 VALU instructions per MFMA) and reads half the
    # rate that shape reaches in the kernels
    tf = {}
    for shape, name, fl in ((1, "32x32x16", 32768),):
        M.probe_mfma_loop(shape, grid, 10, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.probe_mfma_loop(shape, grid, iters, sink)
        e1.record()
        e1.synchronize()
        tf[name] = round(grid * 4 * iters * 8 * fl / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    return {"stream_read_GBps": round(best_gbs, 1), "stream_read_grid": best_grid,
            "mfma_bf16_TFLOPs": tf["32x32x16"], "mfma_probe_shape": "v_mfma_f32_32x32x16_bf16",
            "probe": "moe_probe_stream_read / moe_probe_mfma_loop"}


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 5):
    """Plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) taken under rocprofv3."""
    import torch
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps, "read_bytes_per_copy": nbytes,
                      "write_bytes_per_copy": nbytes}), flush=True)


# ------------------------------------------------------------------ algorithmic work
def layer_bytes(cfg, n_active, T):
    """Bytes the method must move for one step: weights of the active experts,
    the shared expert and the router, plus x in and y out."""
    import bit_quantized_routed_amd as M
    H, I, E, sh = cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["sh_inter"]
    per_expert = 2 * M.q2_packed_bytes(cfg["fmt_gate_up"], I, H) + M.q2_packed_bytes(cfg["fmt_down"], H, I)
    xb = 2 if cfg["x_dtype"] == "bf16" else 4
    return n_active * per_expert + 3 * sh * H * 2 + E * H * 4 + T * H * xb + T * H * 4


def kernel_bytes(cfg, n_active, T, name):
    """Algorithmic bytes of one launch of the named FFN kernel."""
    import bit_quantized_routed_amd as M
    H, I, k, sh = cfg["hidden"], cfg["inter"], cfg["top_k"], cfg["sh_inter"]
    xb = 2 if cfg["x_dtype"] == "bf16" else 4
    rows = T * k + (T if sh else 0)
    if name == "dec_down_fused":
        # every selected expert's down, h in (fp32), the shared down's partial rows and y out
        return n_active * M.q2_packed_bytes(cfg["fmt_down"], H, I) + T * k * I * 4 + (sh // 512) * H * 4 + T * H * 4
    if name == "dec_stage1":
        # the shared gate/up and the router weights, x in, the shared K-part sums out
        return 2 * sh * H * 2 + cfg["n_experts"] * H * 4 + T * H * xb + 8 * 2 * sh * 4
    if name == "dec_stage2":
        # every selected expert's gate/up and the shared down, the per-chunk sums out
        return (n_active * 2 * M.q2_packed_bytes(cfg["fmt_gate_up"], I, H) + sh * H * 2 + T * H * xb
                + (H // 1024) * k * 2 * I * 4 + (sh // 512) * H * 4)
    if name == "bd_gateup":
        # the routed experts' gate/up (the shared expert runs in the grouped GEMM beside it), x in, h out
        return n_active * 2 * M.q2_packed_bytes(cfg["fmt_gate_up"], I, H) + T * H * xb + T * k * I * 4
    if name == "bd_down":
        return n_active * M.q2_packed_bytes(cfg["fmt_down"], H, I) + T * k * I * 4 + T * k * H * 4
    if name.endswith("gateup"):
        hb = 4 if "decode" in name else 2
        return n_active * 2 * M.q2_packed_bytes(cfg["fmt_gate_up"], I, H) + 2 * sh * H * 2 + T * H * xb + rows * I * hb
    if name.endswith("down"):
        hb = 4 if "decode" in name else 2
        return n_active * M.q2_packed_bytes(cfg["fmt_down"], H, I) + sh * H * 2 + rows * I * hb + rows * H * 4
    return None


def layer_flops(cfg, T):
    H, I, E, k, sh = cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["top_k"], cfg["sh_inter"]
    return 6.0 * H * I * T * k + 6.0 * H * sh * T + 2.0 * T * E * H


def kernel_flops(cfg, T, name):
    H, I, k, sh = cfg["hidden"], cfg["inter"], cfg["top_k"], cfg["sh_inter"]
    if name.endswith("gateup"):
        return 4.0 * H * (I * T * k + sh * T)
    if name.endswith("down"):
        return 2.0 * H * (I * T * k + sh * T)
    return None


# ------------------------------------------------------------------ GPU timing
class Stepper:
    def __init__(self, wl, cfg, decode):
        import torch
        import bit_quantized_routed_amd as M
        self.M, self.torch = M, torch
        self.wl, self.cfg, self.decode = wl, cfg, decode
        self.x, self.act = wl.tokens(cfg)
        self.T = self.x.shape[0]
        self.bias = wl.bias(cfg)
        c = wl.cfg
        self.r = M.Routing(self.T, c["top_k"], c["n_experts"])
        self.y = torch.empty((self.T, c["hidden"]), device="cuda")
        self.ws_route = wl.layer.workspace(self.T, M.PATH_ROUTE)
        # decode steps are one moe_layer_decode call (router and FFN; the
        # single-token layer runs the router inside the FFN's launches)
        self.ws_ffn = wl.layer.workspace(self.T, M.PATH_LAYER_DECODE if decode else M.PATH_PREFILL)
        self.stream = torch.cuda.current_stream()
        self.i = 0

    def step(self, prof_route=None, prof_ffn=None):
        M = self.M
        layer = self.wl.layers[self.i % len(self.wl.layers)]
        self.i += 1
        if self.decode:
            M.layer_decode(layer, self.x, self.act, self.T, self.bias, self.r, self.y, self.ws_ffn, self.stream,
                           prof_ffn)
            return
        M.route(layer, self.x, self.act, self.T, self.bias, self.r, self.ws_route, self.stream, prof_route)
        M.ffn_prefill(layer, self.x, self.act, self.T, self.r, self.y, self.ws_ffn, self.stream, prof_ffn)

    def n_active(self):
        import numpy as np
        off = self.r.offsets.cpu().numpy()
        return int((np.diff(off) > 0).sum())

    def kernel_times(self, reps=5):
        """Average duration (ms) of every launch of one step, by name."""
        torch, M = self.torch, self.M
        out = {}
        for which in ("route", "ffn"):
            k = 0
            while True:
                times = []
                name = None
                for _ in range(reps):
                    p = M.Profile(k, 0, None, None, None)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(); e1.record()
                    p.ev_start, p.ev_stop = e0.cuda_event, e1.cuda_event
                    self.step(p if which == "route" else None, p if which == "ffn" else None)
                    torch.cuda.synchronize()
                    n = p.n_launches
                    if k >= n:
                        break
                    name = p.name.decode()
                    times.append(e0.elapsed_time(e1))
                if name is None:
                    break
                out[name] = (which, k, sum(times) / len(times))
                k += 1
        return out

    def timed(self, steps, warmup, dominant=None):
        """ms per step over `steps` steps with nothing but the layer's launches on
        the stream; with `dominant` = (which, index), a second run of `steps` steps
        brackets that launch with HIP events on the layer's stream and returns its
        average duration (the events themselves slow the step a little, so that
        run does not give ms per step)."""
        torch, M = self.torch, self.M
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for _ in range(steps):
            self.step()
        stop.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        ms = start.elapsed_time(stop) / steps
        if not dominant:
            return ms, None, wall
        kms = self.dominant_ms(steps, dominant)
        return ms, kms, wall

    def step_percentiles(self, steps):
        """Median, p10 and p90 of single-step times (ms), each step bracketed by
        its own pair of events on the layer's stream."""
        import numpy as np
        torch = self.torch
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in pairs:
            a.record()
            self.step()
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in pairs])
        return {"median": round(float(np.median(t)), 5), "p10": round(float(np.percentile(t, 10)), 5),
                "p90": round(float(np.percentile(t, 90)), 5)}

    def dominant_ms(self, steps, dominant):
        """Average duration (ms) of launch `dominant` = (which, index) over `steps`
        steps, bracketed by HIP events the library records on its stream."""
        torch, M = self.torch, self.M
        pairs, profs = [], []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(); e1.record()              # materialise the events
            pairs.append((e0, e1))
            profs.append(M.Profile(dominant[1], 0, e0.cuda_event, e1.cuda_event, None))
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(profs[i] if dominant[0] == "route" else None, profs[i] if dominant[0] == "ffn" else None)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in pairs) / steps


# ------------------------------------------------------------------ CPU baseline
def _blas():
    from threadpoolctl import threadpool_info
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    vendor = ",".join(sorted({str(i.get("internal_api", i.get("user_api", "?"))) for i in info})) or "none"
    return int(threads), vendor


def cpu_baseline(cfg, n_tok):
    """The oracle, untuned, on the host cores, over the first n_tok tokens of
    the workload (the whole step when n_tok >= T): route + dequantize the
    experts those tokens select + fp64 FFN + combine.  Quantizing the experts
    beforehand (the oracle's own quantizer) is excluded.  Decode workloads
    report the sample's algorithmic bytes (its experts, the shared expert and
    the router, x and y) per second, prefill workloads tokens per second."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import synthetic as S
    from oracle import formats as F
    from oracle import moe_ref as R
    import bit_quantized_routed_amd as M

    n_tok = min(n_tok, cfg["T"])
    x, kind = S.tokens(cfg)
    x = x[:n_tok]
    xf = S.bf16_to_f32(x) if kind == "bf16" else x
    wr, b = S.router_weight(cfg), S.logit_bias(cfg)
    idx0, _, _ = R.route(xf, wr, cfg["top_k"], b)
    cb = S.codebook_for(cfg["fmt_gate_up"])
    H, I = cfg["hidden"], cfg["inter"]

    def pack(e):
        return e, [F.pack(fmt, S.expert_weight(cfg, which, e), cb)
                   for which, fmt in (("gate", cfg["fmt_gate_up"]), ("up", cfg["fmt_gate_up"]),
                                      ("down", cfg["fmt_down"]))]

    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        packed = dict(ex.map(pack, [int(e) for e in np.unique(idx0)]))
    sh = tuple(S.bf16_to_f32(S.shared_weight_bf16(cfg, n)) for n in ("gate", "up", "down")) if cfg["sh_inter"] else None
    t0 = time.perf_counter()
    idx, w, _ = R.route(xf, wr, cfg["top_k"], b)
    R.group(idx, cfg["n_experts"])
    ex = {}
    for e in np.unique(idx):
        p = packed[int(e)]
        ex[int(e)] = (F.unpack(cfg["fmt_gate_up"], p[0], I, H, cb), F.unpack(cfg["fmt_gate_up"], p[1], I, H, cb),
                      F.unpack(cfg["fmt_down"], p[2], H, I, cb))
    R.moe_layer(xf, idx, w, ex, sh)
    dt = time.perf_counter() - t0
    threads, vendor = _blas()
    decode = cfg["name"].startswith("decode")
    what = ("%d of %d tokens" % (n_tok, cfg["T"])) if n_tok < cfg["T"] else "the whole step (T=%d)" % cfg["T"]
    sample = ("%s of %s: fp64 route, numpy dequant of the %d experts they select, fp64 FFN and combine; "
              "%.2f s; BLAS %s" % (what, cfg["name"], len(ex), dt, vendor))
    if decode:
        per_expert = 2 * M.q2_packed_bytes(cfg["fmt_gate_up"], I, H) + M.q2_packed_bytes(cfg["fmt_down"], H, I)
        xb = 2 if cfg["x_dtype"] == "bf16" else 4
        nbytes = (len(ex) * per_expert + 3 * cfg["sh_inter"] * H * 2 + cfg["n_experts"] * H * 4
                  + n_tok * H * (xb + 4))
        return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
                "blas": vendor, "sample": sample}
    return {"value": round(n_tok / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "blas": vendor, "sample": sample}


# ------------------------------------------------------------------ traffic (rocprofv3 --pmc)
def _profile_value(path, key, kernel):
    """`key <kernel>: <value> sources <hash>` from a committed profile summary,
    if that hash is the one of the kernel's current sources."""
    if not os.path.exists(path):
        return None
    m = re.search(r"^%s %s:\s*([0-9.eE+]+)\s+sources\s+(\w+)" % (key, re.escape(kernel)), open(path).read(), re.M)
    if not m or m.group(2) != kernel_source_hash(kernel):
        return None
    return float(m.group(1))


def read_traffic(kernel, workload):
    """Per-launch HBM bytes (read + write) from the committed counter summary."""
    return _profile_value(os.path.join(ROOT, "profiles", "%s_traffic.md" % workload), "traffic_bytes_per_launch", kernel)


def read_trace_avg(kernel, workload):
    """Average kernel execution time (ms) from the committed rocprofv3 kernel trace."""
    us = _profile_value(os.path.join(ROOT, "profiles", "%s_kernel_trace.md" % workload), "trace_avg_us", kernel)
    return us * 1e-3 if us is not None else None


# ------------------------------------------------------------------ rocprofv3 summaries
def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, d))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _launch_of(symbol):
    for launch, pat in LAUNCH_SYMBOLS:
        if re.search(pat, symbol):
            return launch
    return None


def _command_text(cmd):
    """The command with the repository root (wherever it was run) written as $R."""
    return re.sub(r"(?:/[^\s/]+)*/repo(?=/(?:gpurun_out|bench\.py))", "$R", cmd.replace(ROOT, "$R"))


def summarize_trace(workload, d, cmd):
    """Markdown summary of a `rocprofv3 --kernel-trace --output-format csv` run:
    per-kernel count / mean / median / min / max of the dispatch durations and,
    per library launch, the mean in the form `bench.py` reads back."""
    import statistics as st
    by = {}
    for r in _csv_rows(d, "kernel_trace.csv"):
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in by.values())
    out = ["# Kernel trace: %s" % workload, "",
           "Command (from the repository root R on the MI355X; the summary below is the second line's output):", "",
           "```", _command_text(cmd), "python3 $R/bench.py --summarize-trace %s <the -d folder> '<the first line>'" % workload,
           "```", "",
           "| kernel | launch | calls | total (us) | mean (us) | median (us) | min (us) | max (us) | share |",
           "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    per_launch = {}
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        launch = _launch_of(name)
        if launch:
            per_launch.setdefault(launch, []).extend(v)
        out.append("| `%s` | %s | %d | %.1f | %.2f | %.2f | %.2f | %.2f | %.1f%% |" % (
            name[:150], launch or "", len(v), sum(v), st.mean(v), st.median(v), min(v), max(v), 100 * sum(v) / total))
    out += ["", "Per library launch (mean over its dispatches; the hash is that of the kernel's sources):", ""]
    for launch, v in per_launch.items():
        out.append("trace_avg_us %s: %.3f sources %s" % (launch, st.mean(v), kernel_source_hash(launch)))
    print("\n".join(out))


def summarize_counters(workload, copy_fetch, copy_write, fetch, write, cmds):
    """Markdown summary of two `rocprofv3 --pmc` runs of a workload (FETCH_SIZE,
    then WRITE_SIZE, in KiB per dispatch) scaled by what the same counters read
    for a device copy of known size, per library launch."""
    import statistics as st

    def per_kernel(d, counter):
        acc = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        by = {}
        for (_, name), v in acc.items():
            by.setdefault(name, []).append(v)
        return by

    def copy_kib(d, counter):
        by = per_kernel(d, counter)
        big = max(by, key=lambda n: st.mean(by[n]))          # the 1 GiB copy is the largest dispatch
        return st.mean(by[big]), big

    cf, cname = copy_kib(copy_fetch, "FETCH_SIZE")
    cw, _ = copy_kib(copy_write, "WRITE_SIZE")
    gib = float(1 << 30)
    fscale, wscale = gib / (cf * 1024), gib / (cw * 1024)
    fb, wb = per_kernel(fetch, "FETCH_SIZE"), per_kernel(write, "WRITE_SIZE")
    out = ["# HBM traffic per launch: %s" % workload, "",
           "Counters from two `rocprofv3 --pmc` runs of the workload (one counter per run) and two of a",
           "1 GiB device copy, each counter's KiB per dispatch scaled by copy bytes / counted bytes.",
           "Commands (from the repository root R on the MI355X; the summary is the last line's output):", "",
           "```"] + [_command_text(c) for c in cmds] + [
           "python3 $R/bench.py --summarize-counters %s <the four -d folders, in this order>" % workload, "```", "",
           "| quantity | value |", "|---|---:|",
           "| copy kernel | `%s` |" % cname[:80],
           "| copy: FETCH_SIZE KiB per 1 GiB read | %.1f |" % cf,
           "| copy: WRITE_SIZE KiB per 1 GiB written | %.1f |" % cw,
           "| fetch scale (bytes per counted byte) | %.4f |" % fscale,
           "| write scale | %.4f |" % wscale, "",
           "| kernel | launch | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | write bytes (scaled) |",
           "|---|---|---:|---:|---:|---:|---:|"]
    per_launch = {}
    for name in sorted(set(fb) | set(wb), key=lambda n: -st.mean(fb.get(n, [0.0]))):
        f = st.mean(fb[name]) if name in fb else 0.0
        w = st.mean(wb[name]) if name in wb else 0.0
        launch = _launch_of(name)
        rb, wbytes = f * 1024 * fscale, w * 1024 * wscale
        if launch:
            per_launch.setdefault(launch, []).append((rb, wbytes, len(fb.get(name, []))))
        out.append("| `%s` | %s | %d | %.1f | %.1f | %.0f | %.0f |" % (
            name[:120], launch or "", len(fb.get(name, [])), f, w, rb, wbytes))
    out += ["", "Per library launch (read + write bytes; the hash is that of the kernel's sources):", ""]
    for launch, v in per_launch.items():
        n = sum(c for _, _, c in v) or 1
        tot = sum((r + w) * c for r, w, c in v) / n
        out.append("traffic_bytes_per_launch %s: %.0f sources %s" % (launch, tot, kernel_source_hash(launch)))
    print("\n".join(out))


# counters of one `rocprofv3 --pmc` pass over the compute pipeline (8 SQ and 1 GRBM
# counter: within one pass's limits)
SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
               "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")


def summarize_sq(workload, d, cmd):
    """Markdown summary of one `rocprofv3 --pmc` run of SQ_COUNTERS: per kernel and
    dispatch, each counter summed over its instances; derived per kernel: the
    MFMA busy share (SQ_VALU_MFMA_BUSY_CYCLES, one count per busy SIMD cycle,
    over the GPU-active cycles of the dispatch -- GRBM_GUI_ACTIVE summed over the
    8 XCDs, divided by 8 -- times the chip's SIMDs), the bf16 MFMA flops executed
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts them in units of 512) against the
    kernel's algorithmic flops where defined, VALU instructions per MFMA
    instruction, LDS bank-conflict cycles per LDS instruction and the share of
    wave cycles spent waiting on LDS results."""
    import statistics as st
    import synthetic as S
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        acc.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
        acc[key][r["Counter_Name"]] += float(r["Counter_Value"])
    by = {}
    for (_, name), v in acc.items():
        by.setdefault(name, []).append(v)
    simds = 256 * 4
    cfg = S.config(workload)
    T = cfg["T"]
    out = ["# Compute-pipeline counters: %s" % workload, "",
           "One `rocprofv3 --pmc` run of %s (per dispatch, summed over" % ", ".join("`%s`" % c for c in SQ_COUNTERS),
           "instances, averaged over the kernel's dispatches). Command (from the repository root R on the",
           "MI355X; the summary is the second line's output):", "",
           "```", _command_text(cmd), "python3 $R/bench.py --summarize-sq %s <the -d folder> '<the first line>'" % workload,
           "```", "",
           "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x %d SIMDs); MFMA flops = 512 x" % simds,
           "SQ_INSTS_VALU_MFMA_MOPS_BF16 (executed, padding and the second bf16 term of fp32 operands",
           "included); algorithmic flops as the bench defines them for the grouped-GEMM launches.", "",
           "| kernel | launch | dispatches | MFMA busy | MFMA flops executed | / algorithmic | VALU per MFMA | "
           "LDS conflict cycles per LDS instr | LDS wait share |",
           "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for name, runs in sorted(by.items(), key=lambda kv: -st.mean(x.get("SQ_WAVE_CYCLES", 0.0) for x in kv[1])):
        m = {c: st.mean(x.get(c, 0.0) for x in runs) for c in SQ_COUNTERS}
        launch = _launch_of(name)
        cyc = m["GRBM_GUI_ACTIVE"] / 8
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds) if cyc else 0.0
        flops = 512 * m["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
        alg = kernel_flops(cfg, T, launch) if launch and launch.startswith("ffn_prefill_") else None
        vpm = m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"] if m["SQ_INSTS_MFMA"] else float("nan")
        cpl = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_INSTS_LDS"] if m["SQ_INSTS_LDS"] else float("nan")
        wait = m["SQ_WAIT_INST_LDS"] / m["SQ_WAVE_CYCLES"] if m["SQ_WAVE_CYCLES"] else float("nan")
        out.append("| `%s` | %s | %d | %.1f%% | %.3g | %s | %.1f | %.2f | %.1f%% |" % (
            name[:110], launch or "", len(runs), 100 * busy, flops, "%.2f" % (flops / alg) if alg else "",
            vpm, cpl, 100 * wait))
    print("\n".join(out))


SWEEP_T = (1, 2, 4, 8, 16, 24, 32, 48, 64)


def sweep(args):
    """Decode (fp32-accurate) and prefill (bf16 MFMA) paths on the full layer at
    T = SWEEP_T tokens, Zipf-skewed routing as in decode32: time per step of each,
    the decode path's algorithmic GB/s, the first T at which prefill is faster,
    and how far each token's decode output in the batch is from the same token
    decoded alone (max |difference| relative to max |y|; 0 means bit-identical);
    the same for decode with the layer's token-by-token flag, whose outputs must
    be bit-identical to decoding each token alone."""
    import torch
    import synthetic as S
    import workload as W
    import bit_quantized_routed_amd as M
    base = S.config("decode32")
    wl = W.Workload(base, cache_dir=CACHE, progress=True, replicas=args.replicas)
    rows = []
    for T in SWEEP_T:
        c = S.config("decode32", T=T)
        row = {"T": T}
        ys = {}
        for mode in ("decode", "prefill"):
            st = Stepper(wl, c, mode == "decode")
            st.step()
            torch.cuda.synchronize()
            if mode == "decode":
                ys["batch"] = st.y.clone()
                row["active_experts"] = st.n_active()
            ms, _, _ = st.timed(args.steps, args.warmup)
            row[mode + "_ms"] = round(ms, 5)
        # token 0 alone, on replica 0 as in the batch's first step
        one = Stepper(wl, S.config("decode32", T=1), True)
        xb, _ = wl.tokens(c)
        one.x = xb[:1].contiguous()
        one.step()
        torch.cuda.synchronize()
        d = (one.y[0] - ys["batch"][0]).abs().max().item()
        row["token0_alone_vs_batch"] = d / max(ys["batch"][0].abs().max().item(), 1e-30)
        # token by token (the layer flag), on every replica
        for lay in wl.layers:
            lay.c.flags = M.LAYER_TOKENWISE_DECODE
        try:
            st = Stepper(wl, c, True)
            st.step()
            torch.cuda.synchronize()
            dt = (one.y[0] - st.y[0]).abs().max().item()
            row["tokenwise_token0_vs_alone"] = dt / max(one.y[0].abs().max().item(), 1e-30)
            ms, _, _ = st.timed(args.steps, args.warmup)
            row["tokenwise_ms"] = round(ms, 5)
        finally:
            for lay in wl.layers:
                lay.c.flags = 0
        row["decode_GBps"] = round(layer_bytes(c, row["active_experts"], T) / (row["decode_ms"] * 1e-3) / 1e9, 1)
        row["faster"] = "prefill" if row["prefill_ms"] < row["decode_ms"] else "decode"
        log("sweep T=%d: %s" % (T, row))
        rows.append(row)
    cross = next((r["T"] for r in rows if r["faster"] == "prefill"), None)
    if args.sweep_md:
        print("| T | active experts | decode path (ms) | decode GB/s | token-by-token (ms) | prefill path (ms) | "
              "faster | token0 alone vs batch | token-by-token vs alone |")
        print("|---:|---:|---:|---:|---:|---:|---|---:|---:|")
        for r in rows:
            print("| %d | %d | %.4f | %.1f | %.4f | %.4f | %s | %.2e | %.2e |" % (
                r["T"], r["active_experts"], r["decode_ms"], r["decode_GBps"], r["tokenwise_ms"], r["prefill_ms"],
                r["faster"], r["token0_alone_vs_batch"], r["tokenwise_token0_vs_alone"]))
        print("\ncrossover_T (first T where the prefill path is faster): %s" % cross)
        return
    print(json.dumps({"sweep": "decode vs prefill path, full layer (H=7168, I=2048, E=256, k=8, bf16 shared), "
                               "Zipf-skewed routing", "steps": args.steps, "warmup": args.warmup,
                      "rows": rows, "crossover_T": cross}), flush=True)


DEFAULT_EXTRA = "decode32,prefill2048,prefill8192,prefill8192_q4k,decode32_q4k,prefill2048_cb2s,decode32_cb2s"
# tokens of each workload the oracle baseline evaluates (the whole step at T = 1)
CPU_SAMPLE = {"decode1": 1, "decode32": 2, "decode32_q4k": 2, "prefill2048": 2, "prefill8192": 2,
              "prefill8192_q4k": 2, "prefill2048_cb2s": 1, "decode32_cb2s": 1}
FMT_NAMES = {1: "CB2", 2: "Q2_K", 3: "Q4_K", 5: "Q5_K", 6: "Q6_K", 7: "CB2S"}


def measure(wl, cfg, name, steps, warmup, with_cpu):
    """One workload on its layer: per-kernel times, the dominant kernel's
    roofline, ms per step (mean over `steps`, and median / p10 / p90 of single
    steps), throughput in the metric's unit and the oracle baseline."""
    import torch
    decode = name.startswith("decode")
    st = Stepper(wl, cfg, decode)
    st.step()
    torch.cuda.synchronize()
    n_active = st.n_active()
    kt = st.kernel_times()
    # with the routed batched-decode kernels, the shared expert's launches run
    # on the library's second stream beside them: their event spans include
    # the routed kernels' time, so the dominant kernel is one of the others
    side = ("ffn_decode_gateup", "sh_finalize", "ffn_decode_down") if "bd_gateup" in kt else ()
    dom_name = max((n for n in kt if n not in side), key=lambda n: kt[n][2])
    which, kidx, _ = kt[dom_name]
    log("%s per-kernel ms: %s" % (name, ", ".join("%s=%.4f" % (n, v[2]) for n, v in kt.items())))
    ms, kms, wall = st.timed(steps, warmup, (which, kidx))
    pct = st.step_percentiles(steps)
    T = st.T
    trace_ms = read_trace_avg(dom_name, name)
    if decode:
        nbytes = layer_bytes(cfg, n_active, T)
        value = nbytes / (ms * 1e-3) / 1e9
        kb = kernel_bytes(cfg, n_active, T, dom_name)
        ach = kb / (kms * 1e-3) / 1e9 if kb else None
        roof = {"bound": "hbm", "kernel": dom_name, "achieved": round(ach, 1) if ach else None,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4) if ach else None,
                "traffic": read_traffic(dom_name, name), "algorithmic_bytes": kb, "avg_launch_ms": round(kms, 5)}
        if roof["traffic"] and kb:
            roof["traffic_ratio"] = round(roof["traffic"] / kb, 3)
        if trace_ms and kb:
            roof["trace_avg_ms"] = trace_ms
            roof["achieved_trace"] = round(kb / (trace_ms * 1e-3) / 1e9, 1)
            roof["frac_trace"] = round(roof["achieved_trace"] / HBM_PEAK_GBS, 4)
        out = {"ms_per_step": round(ms, 5), "GB/s": round(value, 1), "hbm_frac": round(value / HBM_PEAK_GBS, 4),
               "algorithmic_bytes": nbytes}
    else:
        fl = layer_flops(cfg, T)
        tf = fl / (ms * 1e-3) / 1e12
        kf = kernel_flops(cfg, T, dom_name)
        ach = kf / (kms * 1e-3) / 1e12 if kf else None
        roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(ach, 1) if ach else None,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4) if ach else None,
                "traffic": read_traffic(dom_name, name), "algorithmic_flops": kf, "avg_launch_ms": round(kms, 5)}
        if trace_ms and kf:
            roof["trace_avg_ms"] = trace_ms
            roof["achieved_trace"] = round(kf / (trace_ms * 1e-3) / 1e12, 1)
            roof["frac_trace"] = round(roof["achieved_trace"] / BF16_PEAK_TFLOPS, 4)
        value = T / (ms * 1e-3)
        out = {"ms_per_step": round(ms, 5), "tokens/s": round(value, 1), "TFLOP/s": round(tf, 1),
               "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": fl}
    out.update({"T": T, "formats": "gate/up %s, down %s" % (FMT_NAMES[cfg["fmt_gate_up"]], FMT_NAMES[cfg["fmt_down"]]),
                "active_experts": n_active, "steps": steps, "step_ms": pct, "wall_ms_per_step": round(wall, 5),
                "roofline": roof, "kernels_ms": {n: round(v[2], 5) for n, v in kt.items()}})
    if with_cpu:
        log("%s: timing the oracle on the host (cpu_baseline)" % name)
        out["cpu_baseline"] = cpu_baseline(cfg, CPU_SAMPLE.get(name, 4))
    log("%s: %s" % (name, {k: v for k, v in out.items() if k not in ("kernels_ms",)}))
    return value, out


HOST_LINK_PEAK_GBS = 64.0     # PCIe 5.0 x16, one direction


def measure_stream(wl, steps, warmup, n_slots):
    """Expert streaming on the full layer: its routed experts in pinned host
    memory, an HBM cache of n_slots slots.  Decode: single-token steps over a
    stream of distinct tokens (route, cache map -- resolve plus the copy of the
    misses -- and the decode FFN on the cache view), with the hit rate and the
    copy kernel's rate from host memory.  Prefill: a 2048-token layer call
    while the next layer's experts are loaded into a second cache on another
    stream, against the same two steps one after the other."""
    import numpy as np
    import torch
    import synthetic as S
    import bit_quantized_routed_amd as M
    base = wl.layer
    host = M.HostLayer(base)
    cache = M.ExpertCache(base.c, 1, n_slots)
    cfg1 = S.config("decode1")
    xs, act = wl.tokens(S.config("prefill2048"))          # 2048 distinct tokens, one per step
    T1 = 1
    r = M.Routing(T1, cfg1["top_k"], cfg1["n_experts"])
    ws_r = base.workspace(T1, M.PATH_ROUTE)
    y = torch.empty((T1, cfg1["hidden"]), device="cuda")
    ws_f = None
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        nonlocal ws_f
        x = xs[i % xs.shape[0]:i % xs.shape[0] + 1]
        M.route(base, x, act, T1, None, r, ws_r)
        if ev:
            ev[0].record()
        view = cache.map(0, host, r.topk_idx, T1)
        if ev:
            ev[1].record()
        if ws_f is None:
            ws_f = view.workspace(T1, M.PATH_DECODE)
        M.ffn_decode(view, x, act, T1, r, y, ws_f)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    h0, m0, b0, _ = cache.stats()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    maps = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        pairs[i][0].record()
        step(warmup + i, maps[i])
        pairs[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in pairs])
    tm = np.array([a.elapsed_time(b) for a, b in maps])
    h1, m1, b1, _ = cache.stats()
    hits, misses, nbytes = h1 - h0, m1 - m0, b1 - b0
    fetch_gbs = nbytes / (tm.sum() * 1e-3) / 1e9 if tm.sum() > 0 else None
    dec = {"n_slots": n_slots, "experts": cfg1["n_experts"], "steps": steps,
           "ms_per_step": {"median": round(float(np.median(t)), 4), "p10": round(float(np.percentile(t, 10)), 4),
                           "p90": round(float(np.percentile(t, 90)), 4)},
           "hit_rate": round(hits / max(hits + misses, 1), 4), "misses_per_step": round(misses / steps, 3),
           "copied_bytes_per_step": int(nbytes / steps),
           "map_ms_per_step": round(float(tm.mean()), 4),
           "roofline": {"bound": "host-link", "kernel": "cache map (resolve + copy of the misses)",
                        "achieved": round(fetch_gbs, 2) if fetch_gbs else None, "peak": HOST_LINK_PEAK_GBS,
                        "unit": "GB/s", "frac": round(fetch_gbs / HOST_LINK_PEAK_GBS, 4) if fetch_gbs else None}}
    # the same bytes by the copy engines (pinned host -> device), for context
    src = host.tensors[0]
    dst = torch.empty_like(src, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    dec["copy_engine_GBps"] = round(3 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2)
    del dst
    log("decode1_stream: %s" % dec)

    # prefill: the next layer's experts load on a second stream during this layer's call
    cfgp = S.config("prefill2048")
    xp, actp = wl.tokens(cfgp)
    T = xp.shape[0]
    rp = M.Routing(T, cfgp["top_k"], cfgp["n_experts"])
    ws_rp = base.workspace(T, M.PATH_ROUTE)
    yp = torch.empty((T, cfgp["hidden"]), device="cuda")
    E = cfgp["n_experts"]
    full = [M.ExpertCache(base.c, 1, E), M.ExpertCache(base.c, 1, E)]
    experts = torch.arange(E, dtype=torch.int32, device="cuda")
    copy_stream = torch.cuda.Stream()
    M.route(base, xp, actp, T, None, rp, ws_rp)
    full[0].prefetch(0, host, experts, E)
    view = full[0].map(0, host, rp.topk_idx, T)
    ws_p = view.workspace(T, M.PATH_PREFILL)
    torch.cuda.synchronize()

    def layer_call():
        M.route(base, xp, actp, T, None, rp, ws_rp)
        v = full[0].map(0, host, rp.topk_idx, T)           # all hits: loaded before
        M.ffn_prefill(v, xp, actp, T, rp, yp, ws_p)

    def timed(fn, reps=3):
        out = []
        for _ in range(reps):
            full[1] = M.ExpertCache(base.c, 1, E)              # empty: the next layer's experts all miss
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            out.append((time.perf_counter() - t0) * 1e3)
        return float(np.median(out))

    def serial():
        full[1].prefetch(0, host, experts, E)
        layer_call()

    def overlapped():
        ready = torch.cuda.Event()
        with torch.cuda.stream(copy_stream):
            full[1].prefetch(0, host, experts, E, stream=copy_stream)
            ready.record(copy_stream)
        layer_call()
        stream.wait_event(ready)

    t_layer = timed(layer_call)
    t_fetch = timed(lambda: full[1].prefetch(0, host, experts, E))
    t_serial, t_over = timed(serial), timed(overlapped)
    per_expert = 2 * base_bytes(wl.cfg)[0] + base_bytes(wl.cfg)[1]
    pre = {"T": T, "layer_ms": round(t_layer, 3), "next_layer_fetch_ms": round(t_fetch, 3),
           "next_layer_fetch_GBps": round(E * per_expert / (t_fetch * 1e-3) / 1e9, 2),
           "serial_ms": round(t_serial, 3), "overlapped_ms": round(t_over, 3),
           "hidden_fraction_of_layer": round((t_serial - t_over) / t_layer, 3) if t_layer > 0 else None}
    log("prefill2048_stream: %s" % pre)
    return {"decode1_stream": dec, "prefill2048_stream": pre}


def base_bytes(cfg):
    import bit_quantized_routed_amd as M
    H, I = cfg["hidden"], cfg["inter"]
    return M.q2_packed_bytes(cfg["fmt_gate_up"], I, H), M.q2_packed_bytes(cfg["fmt_down"], H, I)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode1")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma-separated extra workloads, each measured like the headline one ('' for none)")
    ap.add_argument("--extra-steps", type=int, default=20, help="minimum timed steps of each extra workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the machine-ceiling probes")
    ap.add_argument("--one-stream", action="store_true",
                    help="layers flagged MOE_LAYER_ONE_STREAM: every launch on the caller's stream (batched decode "
                         "otherwise runs the shared expert beside the routed kernels on a second stream)")
    ap.add_argument("--stream-slots", type=int, default=128,
                    help="HBM slots of the expert-streaming measurement (0: skip it)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the micro-batch sweep: decode and prefill paths at T = 1..64 on the full layer "
                         "(Zipf-skewed routing), with the crossover T; one JSON line")
    ap.add_argument("--sweep-md", action="store_true", help="with --sweep: print the table as markdown")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy 5 times (counter calibration under rocprofv3)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("WORKLOAD", "DIR", "COMMAND"),
                    help="only print the markdown summary of a rocprofv3 --kernel-trace csv run (no GPU)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="only print the markdown traffic summary: WORKLOAD COPY_FETCH_DIR COPY_WRITE_DIR "
                         "FETCH_DIR WRITE_DIR COMMAND... (no GPU)")
    ap.add_argument("--summarize-sq", nargs=3, metavar=("WORKLOAD", "DIR", "COMMAND"),
                    help="only print the markdown summary of a rocprofv3 --pmc run of the compute-pipeline "
                         "counters (no GPU)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        a = args.summarize_counters
        summarize_counters(a[0], a[1], a[2], a[3], a[4], a[5:])
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the layer's multi-GPU sharding is a design, not "
              "built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_routed_amd as M
    import synthetic as S
    import workload as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.sweep:
        sweep(args)
        return
    cfg = S.config(args.workload)
    layers = {}

    def layer_for(c, replicas):
        key = (c["fmt_gate_up"], c["fmt_down"])
        if key not in layers:
            log("building layer (%s formats), %d replicas" % (c["name"], replicas))
            t0 = time.time()
            layers[key] = W.Workload(c, cache_dir=CACHE, progress=True, replicas=replicas)
            if args.one_stream:
                for lay in layers[key].layers:
                    lay.c.flags |= M.LAYER_ONE_STREAM
            log("layer ready in %.0f s" % (time.time() - t0))
        return layers[key]

    wl = layer_for(cfg, args.replicas)
    value, head = measure(wl, cfg, args.workload, args.steps, args.warmup, not args.no_cpu_baseline)
    decode = args.workload.startswith("decode")

    workloads = {}
    for name in [w for w in args.extra.split(",") if w and w != args.workload]:
        c2 = S.config(name)
        # a layer of other formats is built once, with fewer copies (its
        # workloads stream more bytes per step than the on-chip caches hold)
        wl2 = layer_for(c2, min(args.replicas, 2))
        _, workloads[name] = measure(wl2, c2, name, max(args.extra_steps, args.steps // 10),
                                     max(2, args.warmup // 4), not args.no_cpu_baseline)
    if args.stream_slots > 0 and args.extra:
        workloads.update(measure_stream(layer_for(S.config("decode1"), args.replicas), max(args.extra_steps, 50),
                                        10, args.stream_slots))

    ceil = None
    roof = head["roofline"]
    if not args.no_ceilings:
        ceil = machine_ceilings()
        log("machine ceilings: %s" % ceil)
        meas = ceil["stream_read_GBps"] if decode else ceil["mfma_bf16_TFLOPs"]
        roof["measured_peak"] = meas
        roof["frac_of_measured"] = round(roof["achieved"] / meas, 4) if roof["achieved"] and meas else None

    out = {
        "metric": METRIC, "value": round(value, 2) if decode else round(value, 1),
        "unit": "GB/s" if decode else "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "T": head["T"], "hidden": cfg["hidden"], "inter": cfg["inter"],
                   "experts": cfg["n_experts"], "top_k": cfg["top_k"], "shared_inter": cfg["sh_inter"],
                   "formats": "gate/up %s, down %s, shared bf16" % (
                       FMT_NAMES[cfg["fmt_gate_up"]], FMT_NAMES[cfg["fmt_down"]]),
                   "active_experts": head["active_experts"], "weight_replicas": args.replicas},
        "hbm_frac": head.get("hbm_frac"), "mfma_frac": head.get("mfma_frac"),
        "step_ms": head["step_ms"],
        "wall_ms_per_step": head["wall_ms_per_step"],
        "roofline": roof,
        "cpu_baseline": head.get("cpu_baseline"),
        "kernels_ms": head["kernels_ms"],
        "machine_ceilings": ceil,
        "kernel_source_hash": kernel_source_hash(),
        "workloads": workloads,
    }
    if decode:
        out["config"]["algorithmic_bytes"] = head["algorithmic_bytes"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

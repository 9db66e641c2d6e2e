"""Benchmark of the int8 quantized linear hot path on one MI355X.

The headline step is one W8A8 prefill pass of the dense 8B decoder layer (hidden 4096,
intermediate 12288) over 16384 tokens: per-token int8 quantization of the layer's four
distinct inputs, then the int8 MFMA GEMMs with the fused scale + bias epilogue to bf16.
Projections that read the same input run as one GEMM over their concatenated weights
(q/k/v: N = 6144; gate/up: N = 24576), as a serving engine launches them: four GEMMs with
exactly the products of the seven projections.  ``value`` is the step's int8 throughput
(2*M*N*K ops summed over the seven projections, over the whole step time, quantization
included), with every input resident in HBM.  Weight copies are rotated so every GEMM reads
weights that are not in the 256 MB Infinity Cache.  After W eager warm-up steps, exactly K
steps are captured in one HIP graph and replayed between two HIP events (after one untimed
replay), as an inference engine would launch them; the graph holds the same kernels on the
same stream, so host launch overhead does not enter the kernel timings.

The same JSON line also carries ``roofline`` (the W8A8 kernel over the step's launches, each
repeated on its own between HIP events on the kernels' stream, classified MFMA- or HBM-bound
by its algorithmic work), ``cpu_baseline`` (the CPU oracle on a bounded sample of the step),
and the other rows of the path, each timed on its own workload: the same layer at 4096
tokens, the dense 4B layer at 128/512/2048 tokens, W8A16 decode on 8B shapes (M = 1, 4, 8)
next to a measured copy floor, the grouped MoE W8A16 GEMM and block (T = 1..64 tokens), and
the per-channel weight quantizer.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sections a,b,...]
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

METRIC = "int8 GEMM TOPS (prefill) + decode GB/s, % of MI355X roofline"
PEAK_INT8_TOPS = 5000.0     # dense int8 MFMA, MI355X
PEAK_HBM_GBS = 8000.0       # HBM3E, MI355X
PEAK_GFX_MHZ = 2400.0       # graphics clock the int8 peak is quoted at
MALL_BYTES = 256 << 20
ROTATE_BYTES = 1 << 30      # rotate weight copies over at least this much memory

KERNEL_SOURCES = {
    "w8a8_kernel": "int8_quantized_linear_amd/csrc/w8a8_gemm.hip",
    "w8a16_kernel": "int8_quantized_linear_amd/csrc/w8a16_gemm.hip",
    "grouped_w8a16_kernel": "int8_quantized_linear_amd/csrc/grouped_w8a16.hip",
    "quantize_rows_vec_kernel": "int8_quantized_linear_amd/csrc/quantize_rows.hip",
    "rmsnorm_rows_kernel": "int8_quantized_linear_amd/csrc/quantize_rows.hip",
}


CALIB_BYTES = 256 << 20  # calibration copy for the traffic counters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    paths = [KERNEL_SOURCES[kernel], "int8_quantized_linear_amd/csrc/sync.hpp"]
    if "w8a16" in kernel:
        paths.append("int8_quantized_linear_amd/csrc/dequant_mma.hpp")
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------------------
# algorithmic work (what the method must move or compute)

def w8a8_ops(m, n, k):
    return 2.0 * m * n * k


def w8a8_bytes(m, n, k, out_bytes=2, bias=False):
    return n * k + m * k + 4 * n + 4 * m + m * n * out_bytes + (4 * n if bias else 0)


def w8a16_bytes(m, n, k, out_bytes=2, bias=False):
    return n * k + 4 * n + 2 * m * k + m * n * out_bytes + (4 * n if bias else 0)


def quant_bytes(r, k, in_bytes=2):
    return r * k * in_bytes + r * k + 4 * r


def grouped_bytes(distinct, n, k, x_rows, assignments, out_bytes=2):
    return distinct * (n * k + 4 * n) + x_rows * k * 2 + assignments * n * out_bytes


# ---------------------------------------------------------------------------------------

def gfx_clock_mhz():
    """Mean current graphics clock over the GPU's XCDs as amd-smi reports it, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"],
                           capture_output=True, text=True, timeout=60)
        clk = json.loads(r.stdout)["gpu_data"][0]["clock"]
        vals = [v["clk"]["value"] for name, v in clk.items() if name.startswith("gfx")]
        return sum(vals) / len(vals) if vals else None
    except Exception:  # tool missing or output format changed: report no reading
        return None


def graph_time(torch, body, iters, warmup=1, clock=None, passes=1, reduce=min):
    """Seconds for body(0 .. iters-1), launched from one captured HIP graph and timed with
    two HIP events around its replay (no host launch overhead between kernels).  body(0) runs
    once eagerly first so that one-time setup never happens under capture, and the graph is
    replayed `warmup` times untimed before the timed replay (the fastest of `passes` timed
    replays when passes > 1).  With a `clock` dict, the graph is then queued again for about
    three seconds (untimed) while a thread reads the graphics clock over and over; amd-smi's
    reading trails the load by up to a second, so readings from the first second and the
    last 0.2 s are dropped and clock["mhz"] is the median of the rest (clock["samples"] of
    them)."""
    body(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            body(i)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    # a short graph is replayed untimed for about 20 ms more: right after idle time (or after
    # the clock sampling below) a few replays of microsecond kernels do not bring the GPU back
    # to its working clock, and the first timed replays ran up to twice as slow
    t_one = time.time()
    g.replay()
    torch.cuda.synchronize()
    t_one = time.time() - t_one
    for _ in range(min(2000, int(0.02 / max(t_one, 1e-6)))):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(passes):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) * 1e-3)
    secs = reduce(times)
    if clock is not None:
        import statistics
        import threading
        samples, stop = [], threading.Event()

        def sample():
            while not stop.is_set():
                t = time.time() - t0
                v = gfx_clock_mhz()
                if v is None:
                    return
                samples.append((t, v))

        t0 = time.time()
        th = threading.Thread(target=sample)  # started first: queueing a large graph takes a while
        th.start()
        for _ in range(max(1, int(3.0 / max(secs, 1e-6)))):
            g.replay()
        torch.cuda.synchronize()
        busy = time.time() - t0
        stop.set()
        th.join()
        keep = [v for t, v in samples if 1.0 <= t <= busy - 0.2]
        clock["mhz"] = statistics.median(keep) if keep else None
        clock["samples"] = len(keep)
    del g
    return secs


def per_call(torch, fn, reps, warmup=1):
    """Average seconds per call of fn(i), from a graph of `reps` calls: the fastest of five
    timed replays (a short graph replayed once right after host-side work can run while the
    clock is still ramping up from idle).  Used for the per-launch breakdowns only."""
    return graph_time(torch, fn, reps, warmup, passes=5) / reps


def mean_call(torch, fn, reps):
    """Average seconds per call of fn(i): a graph of `reps` calls, replayed three times
    untimed (the first graph timed after a long run of other work can run slow), then the
    mean of three timed replays (an average over launches, as a kernel trace reports)."""
    return graph_time(torch, fn, reps, 3, passes=3, reduce=lambda t: sum(t) / len(t)) / reps


def time_loop(torch, body, steps, warmup, clock=None):
    """W eager warm-up steps, then exactly `steps` steps replayed from one HIP graph."""
    for i in range(warmup):
        body(i)
    torch.cuda.synchronize()
    return graph_time(torch, lambda i: body(warmup + i), steps, 1, clock)


# ---------------------------------------------------------------------------------------
# sections

def launch_bound(ops, nbytes, secs):
    """Which roofline bounds one launch (the larger of its MFMA time at 5.0 POP/s and its
    HBM time at 8 TB/s for the algorithmic work), and the fraction of that bound reached."""
    t_mfma = ops / (PEAK_INT8_TOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    return ("mfma" if t_mfma >= t_hbm else "hbm"), max(t_mfma, t_hbm) / secs


class PrefillWorkload:
    """One W8A8 prefill layer: per-token quantization of its four distinct inputs (attention
    in/out, MLP in/mid), then one GEMM per group of projections that read the same input
    (q/k/v and gate/up over concatenated weights), with the fused scale (+bias) epilogue to
    bf16.  Weight copies rotate over at least ROTATE_BYTES so that no timed GEMM reads its
    weights from the Infinity Cache."""

    INPUTS = ("attn_in", "attn_out", "mlp_in", "mlp_mid")
    SRC = {"qkv": "attn_in", "o": "attn_out", "gate_up": "mlp_in", "down": "mlp_mid"}

    def __init__(self, torch, i8, wl, dev, shapes, fused, tokens, frac, bias, seed,
                 group_scales=False):
        self.torch, self.i8, self.wl = torch, i8, wl
        self.tokens, self.shapes = tokens, shapes
        self.group_scales = group_scales  # weight scales per group of 128 input channels
        g = wl.rng(seed)
        pq, ps, pb = {}, {}, {}
        layer_bytes = 0
        quant = i8.quantize_per_group_int8 if group_scales else i8.quantize_per_channel_int8
        for nm, (n, k) in shapes.items():
            w = wl.to_bf16(wl.weight(g, n, k)).to(dev)
            pq[nm], ps[nm] = quant(w)
            layer_bytes += n * k
            del w
            if bias:
                pb[nm] = torch.from_numpy(g.standard_normal(n, dtype=np.float32)
                                          * np.float32(0.02)).to(dev)
        self.names = list(fused)
        # per-channel quantization is row-wise, so concatenated codes and scales are exactly
        # those of the separate projections
        q0 = {f: torch.cat([pq[p] for p in parts]).contiguous() for f, parts in fused.items()}
        self.s = {f: torch.cat([ps[p] for p in parts]).contiguous() for f, parts in fused.items()}
        self.b = ({f: torch.cat([pb[p] for p in parts]).contiguous() for f, parts in fused.items()}
                  if bias else {f: None for f in fused})
        del pq, ps, pb
        self.copies = max(2, -(-ROTATE_BYTES // layer_bytes))
        self.qs = [q0] + [{nm: q0[nm].clone() for nm in self.names}
                          for _ in range(self.copies - 1)]
        self.shape = {f: (q0[f].shape[0], q0[f].shape[1]) for f in self.names}
        kin = {"attn_in": self.shape["qkv"][1], "attn_out": self.shape["o"][1],
               "mlp_in": self.shape["gate_up"][1], "mlp_mid": self.shape["down"][1]}
        self.kin = kin
        self.xs, self.qx, self.outs = {}, {}, {}
        for m in tokens:
            self.xs[m] = {key: wl.to_bf16(wl.activations(g, m, kin[key], frac)).to(dev)
                          for key in self.INPUTS}
            self.qx[m] = {key: (torch.empty((m, kin[key]), dtype=torch.int8, device=dev),
                                torch.empty((m,), dtype=torch.float32, device=dev))
                          for key in self.INPUTS}
            self.outs[m] = {nm: torch.empty((m, self.shape[nm][0]), dtype=torch.bfloat16,
                                            device=dev) for nm in self.names}
        self.bias = bias

    def ops(self):
        return sum(w8a8_ops(m, n, k) for m in self.tokens for (n, k) in self.shape.values())

    def quantize(self, m, key):
        q, s = self.qx[m][key]
        self.i8.quantize_per_token_int8(self.xs[m][key], q, s)

    # below this many tokens the four inputs of a token count are quantized in one launch
    # (the launches are latency-bound); from it on one launch each (bandwidth-bound: at
    # 16384 tokens the single launch took 229 us against 220 us for four)
    MULTI_BELOW = 4096

    def quantize_all(self, m):
        """The four inputs of one token count, quantized per token."""
        if m < self.MULTI_BELOW:
            self.i8.quantize_per_token_int8_multi([self.xs[m][key] for key in self.INPUTS],
                                                  [self.qx[m][key] for key in self.INPUTS])
        else:
            for key in self.INPUTS:
                self.quantize(m, key)

    def gemm(self, m, nm, copy):
        q, s = self.qx[m][self.SRC[nm]]
        f = self.i8.w8a8_gemm_g128 if self.group_scales else self.i8.w8a8_gemm
        f(q, s, self.qs[copy % self.copies][nm], self.s[nm], self.b[nm], out=self.outs[m][nm])

    def step(self, i):
        for mi, m in enumerate(self.tokens):
            self.quantize_all(m)
            for nm in self.names:
                self.gemm(m, nm, i * len(self.tokens) + mi)


def measure_prefill(torch, wl, wk, args, label, clock=True):
    """Time `args.steps` steps from one HIP graph after `args.warmup` eager ones, then every
    launch of the step on its own (repeated back to back in a graph between two HIP events on
    the kernels' stream, weight copies rotating as in the step)."""
    ops = wk.ops()
    log(f"[{label}] {wk.copies} weight copies; warmup {args.warmup}, steps {args.steps}")
    clk = {} if clock else None
    secs = time_loop(torch, wk.step, args.steps, args.warmup, clk)
    out = {"ms_per_step": secs / args.steps * 1e3, "TOPS": ops / (secs / args.steps) / 1e12}
    if clock:
        out["gfx_clock_mhz_during_step"] = clk.get("mhz")
        out["gfx_clock_samples"] = clk.get("samples")
    log(f"[{label}] {out['ms_per_step']:.4f} ms/step, {out['TOPS']:.1f} TOPS")
    reps = max(5, args.steps // 5)
    per, quant, multi = [], [], []
    for m in wk.tokens:
        sec = mean_call(torch, lambda i, m=m: wk.quantize_all(m), reps)
        qb = sum(quant_bytes(m, wk.kin[key]) for key in wk.INPUTS)
        multi.append({"m": m, "us": sec * 1e6, "GBs": qb / sec / 1e9})
        for key in wk.INPUTS:
            sec = mean_call(torch, lambda i, m=m, key=key: wk.quantize(m, key), reps)
            quant.append({"m": m, "k": wk.kin[key], "input": key, "us": sec * 1e6,
                          "GBs": quant_bytes(m, wk.kin[key]) / sec / 1e9})
        for nm in wk.names:
            sec = mean_call(torch, lambda i, m=m, nm=nm: wk.gemm(m, nm, i), reps)
            n, k = wk.shape[nm]
            o, b = w8a8_ops(m, n, k), w8a8_bytes(m, n, k, bias=wk.bias)
            if wk.group_scales:
                b += n * (k // 128 - 1) * 4  # a scale per group instead of one per channel
            bound, frac = launch_bound(o, b, sec)
            per.append({"m": m, "n": n, "k": k, "proj": nm, "us": sec * 1e6, "ops": o,
                        "bytes": b, "TOPS": o / sec / 1e12, "GBs": b / sec / 1e9,
                        "bound": bound, "frac_of_bound": frac,
                        "frac_mfma": o / sec / 1e12 / PEAK_INT8_TOPS,
                        "frac_hbm": b / sec / 1e9 / PEAK_HBM_GBS})
    # the step's GEMMs alone, in step order with the step's weight rotation: the W8A8
    # kernel's launches as the timed step runs them (back to back with other launches, not
    # each repeated on its own), which the roofline's average launch duration is taken from
    seq = mean_call(torch, lambda i: [wk.gemm(m, nm, i) for m in wk.tokens for nm in wk.names],
                    reps)
    out["w8a8_gemm_sequence_us_per_step"] = seq * 1e6
    t_gemm = sum(p["us"] for p in per) * 1e-6
    t_quant = sum(q["us"] for q in multi) * 1e-6
    t_sep = sum(q["us"] for q in quant) * 1e-6
    qbytes = sum(quant_bytes(q["m"], q["k"]) for q in quant)
    out["per_launch"] = per
    out["quantize_per_token"] = {
        "per_token_count": multi, "us_per_step": t_quant * 1e6,
        "GBs": qbytes / t_quant / 1e9,
        "frac_hbm": qbytes / t_quant / 1e9 / PEAK_HBM_GBS,
        "what": "the step's four inputs of each token count, timed together: one "
                "quantize_per_token_int8_multi launch below 4096 tokens, else one "
                "quantize_per_token_int8 launch each",
        "separate": {"what": "one quantize_per_token_int8 launch per input", "launches": quant,
                     "us_per_step": t_sep * 1e6, "GBs": qbytes / t_sep / 1e9}}
    out["w8a8_gemm_us_per_step"] = t_gemm * 1e6
    return out


def w8a8_roofline(per, traffic, seq_us):
    """The roofline entry of the W8A8 kernel over a step's GEMM launches: the bound that
    holds for most of the kernel time (by each launch's own classification), achieved =
    algorithmic work / the launches' durations in step order (seq_us per step: int8 TOPS
    against 5.0 POP/s, or GB/s against 8 TB/s)."""
    t_own = sum(p["us"] for p in per) * 1e-6
    t_mfma = sum(p["us"] for p in per if p["bound"] == "mfma") * 1e-6
    bound = "mfma" if t_mfma >= t_own / 2 else "hbm"
    t = seq_us * 1e-6
    n = len(per)
    if bound == "mfma":
        ach, peak, unit = sum(p["ops"] for p in per) / t / 1e12, PEAK_INT8_TOPS, "TOPS"
    else:
        ach, peak, unit = sum(p["bytes"] for p in per) / t / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"kernel": "w8a8_kernel (all tile instantiations)", "bound": bound,
            "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
            "traffic": traffic, "avg_launch_us": t / n * 1e6, "launches_per_step": n,
            "avg_launch_us_each_on_its_own": t_own / n * 1e6,
            "ops_per_launch": sum(p["ops"] for p in per) / n,
            "algorithmic_bytes_per_launch": sum(p["bytes"] for p in per) / n,
            "launches_by_bound": {b: sum(1 for p in per if p["bound"] == b)
                                  for b in ("mfma", "hbm")}}


HEADLINE = "dense 8B W8A8 prefill step M=16384"


def prefill_8b(torch, i8, wl, dev, tokens):
    return PrefillWorkload(torch, i8, wl, dev, wl.DENSE_8B, wl.DENSE_8B_FUSED, tokens, 0.01,
                           True, seed=3)


def prefill_4b(torch, i8, wl, dev):
    return PrefillWorkload(torch, i8, wl, dev, wl.DENSE_4B, wl.DENSE_4B_FUSED,
                           wl.PREFILL_4B_TOKENS, 0.001, False, seed=0)


def section_step(torch, i8, wl, dev, args, result):
    """The headline: the dense 8B decoder layer's W8A8 prefill at 16384 tokens."""
    wk = prefill_8b(torch, i8, wl, dev, (16384,))
    out = measure_prefill(torch, wl, wk, args, "step")
    result.update(value=out["TOPS"], ms_per_step=out["ms_per_step"])
    result["gfx_clock_mhz_during_step"] = out["gfx_clock_mhz_during_step"]
    result["gfx_clock_samples"] = out["gfx_clock_samples"]
    mhz = out["gfx_clock_mhz_during_step"]
    result["frac_mfma_step"] = out["TOPS"] / PEAK_INT8_TOPS
    result["frac_mfma_step_at_sustained_clock"] = (
        out["TOPS"] / (PEAK_INT8_TOPS * mhz / PEAK_GFX_MHZ) if mhz else None)
    result["roofline"] = w8a8_roofline(out["per_launch"], traffic_for("w8a8_kernel", HEADLINE),
                                       out["w8a8_gemm_sequence_us_per_step"])
    result["per_launch"] = out["per_launch"]
    result["quantize_per_token"] = out["quantize_per_token"]
    result["parts_us_per_step"] = {"w8a8_gemm": out["w8a8_gemm_us_per_step"],
                                   "quantize_per_token": out["quantize_per_token"]["us_per_step"]}
    rf = result["roofline"]
    log(f"[step] roofline {rf['bound']}: {rf['achieved']:.0f} {rf['unit']} = "
        f"{100 * rf['frac']:.1f}% (avg launch {rf['avg_launch_us']:.2f} us)")
    del wk
    torch.cuda.empty_cache()


def section_prefill_8b_m4096(torch, i8, wl, dev, args, result):
    wk = prefill_8b(torch, i8, wl, dev, (4096,))
    out = measure_prefill(torch, wl, wk, args, "prefill_8b_m4096")
    out["roofline"] = w8a8_roofline(out["per_launch"], None,
                                    out["w8a8_gemm_sequence_us_per_step"])
    result["prefill_8b_m4096"] = {
        "workload": "dense 8B decoder layer, W8A8 prefill at 4096 tokens (the same step as the "
                    "headline at its other token count)", "unit": "TOPS", **out}
    del wk
    torch.cuda.empty_cache()


def section_prefill_8b_g128(torch, i8, wl, dev, args, result):
    """The headline layer with weight scales per group of 128 input channels (W8A8-g128),
    next to the per-channel numbers of the headline when both ran."""
    wk = PrefillWorkload(torch, i8, wl, dev, wl.DENSE_8B, wl.DENSE_8B_FUSED, (16384,), 0.01,
                         True, seed=3, group_scales=True)
    out = measure_prefill(torch, wl, wk, args, "prefill_8b_g128", clock=False)
    out["roofline"] = w8a8_roofline(out["per_launch"], None,
                                    out["w8a8_gemm_sequence_us_per_step"])
    if result.get("per_launch"):
        pc = {(p["m"], p["proj"]): p["us"] for p in result["per_launch"]}
        for p in out["per_launch"]:
            p["vs_per_channel"] = p["us"] / pc[(p["m"], p["proj"])]
        out["vs_per_channel_step"] = out["ms_per_step"] / result["ms_per_step"]
    result["prefill_8b_g128"] = {
        "workload": "the headline step (dense 8B layer, 16384 tokens, bias) with weight scales "
                    "per group of 128 input channels: w8a8_gemm_g128", "unit": "TOPS", **out}
    del wk
    torch.cuda.empty_cache()


def section_prefill_4b(torch, i8, wl, dev, args, result):
    wk = prefill_4b(torch, i8, wl, dev)
    out = measure_prefill(torch, wl, wk, args, "prefill_4b", clock=False)
    out["roofline"] = w8a8_roofline(out["per_launch"],
                                    traffic_for("w8a8_kernel", "dense 4B W8A8 prefill step"),
                                    out["w8a8_gemm_sequence_us_per_step"])
    result["prefill_4b"] = {
        "workload": "dense 4B decoder layer (q 2560->4096, k/v 2560->1024, o 4096->2560, "
                    "gate/up 2560->9728, down 9728->2560), W8A8 prefill at M in {128, 512, "
                    "2048} per step, no bias, 0.1% outlier dims x100", "unit": "TOPS", **out}
    del wk
    torch.cuda.empty_cache()


def traffic_entry(kernel, workload):
    """The committed rocprofv3 counter summary of a kernel on a workload (profiles/
    traffic.json), if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    ent = data.get(kernel, {}).get(workload)
    if not ent or ent.get("source_sha") != source_sha(kernel):
        return None
    return ent


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None."""
    ent = traffic_entry(kernel, workload)
    return None if ent is None else ent["bytes_per_launch"]


CPU_SAMPLE_ROWS = 2048  # token rows of the headline step the oracle is timed on


def section_cpu_baseline(i8, wl, args, result):
    """The oracle as it stands, on a bounded sample of the headline workload: the first
    CPU_SAMPLE_ROWS of the 16384 token rows through all seven projections of the 8B layer
    (per-token quantization, exact int32 GEMM, float64 epilogue with bias), on every host
    thread; rows are independent, so the rate is the step's rate."""
    import oracle
    ref = oracle.load()
    threads = len(os.sched_getaffinity(0))
    ref.set_threads(threads)
    g = wl.rng(5)
    shapes = wl.DENSE_8B
    ws = {nm: ref.quantize_rows(wl.bits16(wl.to_bf16(wl.weight(g, n, k))), "bf16")
          for nm, (n, k) in shapes.items()}
    bias = {nm: (g.standard_normal(n, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
            for nm, (n, k) in shapes.items()}
    src = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "attn_out", "gate": "mlp_in",
           "up": "mlp_in", "down": "mlp_mid"}
    kin = {"attn_in": 4096, "attn_out": 4096, "mlp_in": 4096, "mlp_mid": 12288}
    r = CPU_SAMPLE_ROWS
    xs = {key: wl.bits16(wl.to_bf16(wl.activations(g, r, k, 0.01))) for key, k in kin.items()}
    ops = 0.0
    t0 = time.perf_counter()
    qx = {key: ref.quantize_rows(x, "bf16") for key, x in xs.items()}
    for nm, (n, k) in shapes.items():
        q, s_ = qx[src[nm]]
        ref.w8a8(q, s_, ws[nm][0], ws[nm][1], bias[nm])
        ops += w8a8_ops(r, n, k)
    dt = time.perf_counter() - t0
    single = {}
    ref.set_threads(1)
    t = wl.tiny_w8a8(0)
    t0 = time.perf_counter()
    qw, sw = ref.quantize_rows(t["w"], "f32")
    qxt, sxt = ref.quantize_rows(t["x"], "f32")
    ref.w8a8(qxt, sxt, qw, sw)
    single["tiny 4x256x512 (quantize both + GEMM)"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    q, s_ = ref.quantize_rows(xs["attn_in"][:128], "bf16")
    ref.w8a8(q, s_, ws["q"][0], ws["q"][1], bias["q"])
    single["q 128x4096x4096 (quantize tokens + GEMM)"] = time.perf_counter() - t0
    ref.set_threads(threads)
    result["cpu_baseline"] = {
        "value": ops / dt / 1e12, "unit": "TOPS", "cores": ref.threads(), "kind": "oracle",
        "sample": f"the headline step's first {r} of 16384 token rows through all 7 "
                  f"projections of the 8B layer: per-token quantization + int32 GEMM + "
                  f"float64 epilogue with bias; {dt:.1f} s",
        "seconds": dt, "single_thread_seconds": single}
    log(f"[cpu_baseline] {ops/dt/1e12*1e3:.2f} GOP/s on {ref.threads()} threads, {dt:.1f} s; "
        f"1 thread: {single}")


def copy_floor(torch, dev, nbytes, reps):
    """Seconds per device-to-device copy of nbytes / 2 bytes (nbytes through HBM: half read,
    half written), graph-replayed with the sources rotating over at least ROTATE_BYTES."""
    half = max(16, int(nbytes) // 2 // 16 * 16)
    copies = max(2, -(-ROTATE_BYTES // half))
    src = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(copies)]
    dst = torch.empty(half, dtype=torch.uint8, device=dev)
    t = per_call(torch, lambda i: dst.copy_(src[i % copies]), reps)
    del src, dst
    return t


def section_decode(torch, i8, wl, dev, args, result):
    g = wl.rng(1)
    # per-channel quantization per projection, then the projections that share an input
    # concatenated along N (q/k/v: 6144 x 4096, gate/up: 24576 x 4096), as for the step
    pq, ps = {}, {}
    for nm, (n, k) in wl.DENSE_8B.items():
        pq[nm], ps[nm] = i8.quantize_per_channel_int8(wl.to_bf16(wl.weight(g, n, k)).to(dev))
    names = list(wl.DENSE_8B_FUSED)
    q0 = {f: torch.cat([pq[p] for p in parts]).contiguous()
          for f, parts in wl.DENSE_8B_FUSED.items()}
    s0 = {f: torch.cat([ps[p] for p in parts]).contiguous()
          for f, parts in wl.DENSE_8B_FUSED.items()}
    del pq, ps
    shapes = {f: (q0[f].shape[0], q0[f].shape[1]) for f in names}
    layer = sum(n * k for n, k in shapes.values())
    copies = max(2, -(-ROTATE_BYTES // layer))
    qs = [q0] + [{nm: q0[nm].clone() for nm in names} for _ in range(copies - 1)]
    out = {"copies": copies, "per_m": {}}
    floors = {nm: copy_floor(torch, dev, w8a16_bytes(1, *shapes[nm]), max(5, args.steps // 5))
              for nm in names}
    out["floor_copy"] = {
        "what": "a device-to-device copy (torch copy_, graph-replayed, sources rotating over "
                ">= 1 GiB) that moves as many bytes through HBM as the projection's M=1 "
                "algorithmic bytes: half of them read, half written",
        "per_proj": {nm: {"us": t * 1e6, "GBs": w8a16_bytes(1, *shapes[nm]) / t / 1e9}
                     for nm, t in floors.items()}}
    for m in wl.DECODE_8B_BATCH:
        xs = {k: wl.to_bf16(wl.activations(g, m, k)).to(dev) for k in (4096, 12288)}
        ys = {nm: torch.empty((m, shapes[nm][0]), dtype=torch.bfloat16, device=dev) for nm in names}
        def body(i):
            wq = qs[i % copies]
            for nm in names:
                n, k = shapes[nm]
                i8.w8a16_gemm(xs[k], wq[nm], s0[nm], out=ys[nm])
        secs = time_loop(torch, body, args.steps, args.warmup)
        reps = max(5, args.steps // 5)
        durs = {nm: per_call(torch, lambda i, nm=nm: i8.w8a16_gemm(
            xs[shapes[nm][1]], qs[i % copies][nm], s0[nm], out=ys[nm]), reps) for nm in names}
        nbytes = sum(w8a16_bytes(m, n, k) for n, k in shapes.values())
        per = {}
        for nm in names:
            n, k = shapes[nm]
            t = durs[nm]
            per[nm] = {"n": n, "k": k, "us": t * 1e6,
                       "GBs": w8a16_bytes(m, n, k) / t / 1e9,
                       "frac_hbm": w8a16_bytes(m, n, k) / t / 1e9 / PEAK_HBM_GBS,
                       "vs_copy_floor": t / floors[nm]}
        gbs_kernels = nbytes / sum(durs.values()) / 1e9
        out["per_m"][m] = {"layer_us": secs / args.steps * 1e6,
                           "GBs_layer": nbytes / (secs / args.steps) / 1e9,
                           "GBs_kernels": gbs_kernels,
                           "frac_hbm_kernels": gbs_kernels / PEAK_HBM_GBS,
                           "per_proj": per}
        log(f"[decode] M={m}: {secs/args.steps*1e6:.1f} us/layer, kernels {gbs_kernels:.0f} GB/s")
    # The same layer with one scale per group of 128 input channels (w8a16_gemm_g128).
    gq, gs = {}, {}
    for nm, (n, k) in wl.DENSE_8B.items():
        gq[nm], gs[nm] = i8.quantize_per_group_int8(wl.to_bf16(wl.weight(g, n, k)).to(dev))
    g0 = {f: torch.cat([gq[p] for p in parts]).contiguous()
          for f, parts in wl.DENSE_8B_FUSED.items()}
    gs0 = {f: torch.cat([gs[p] for p in parts]).contiguous()
           for f, parts in wl.DENSE_8B_FUSED.items()}
    del gq, gs
    gqs = [g0] + [{nm: g0[nm].clone() for nm in names} for _ in range(copies - 1)]
    out["g128"] = {"per_m": {}}
    for m in wl.DECODE_8B_BATCH:
        xs = {k: wl.to_bf16(wl.activations(g, m, k)).to(dev) for k in (4096, 12288)}
        ys = {nm: torch.empty((m, shapes[nm][0]), dtype=torch.bfloat16, device=dev) for nm in names}
        def body_g(i):
            wq = gqs[i % copies]
            for nm in names:
                n, k = shapes[nm]
                i8.w8a16_gemm_g128(xs[k], wq[nm], gs0[nm], out=ys[nm])
        secs = time_loop(torch, body_g, args.steps, args.warmup)
        nbytes = sum(w8a16_bytes(m, n, k) + n * (k // 128 - 1) * 4 for n, k in shapes.values())
        out["g128"]["per_m"][m] = {"layer_us": secs / args.steps * 1e6,
                                   "GBs_layer": nbytes / (secs / args.steps) / 1e9}
        log(f"[decode] g128 M={m}: {secs/args.steps*1e6:.1f} us/layer, "
            f"{nbytes / (secs / args.steps) / 1e9:.0f} GB/s")
    out["traffic_m1"] = traffic_for("w8a16_kernel", "dense 8B decode layer M=1")
    m1 = out["per_m"][1]
    result["decode"] = {"workload": "dense 8B decoder projections, W8A16 decode, M in {1,4,8}; "
                                    "q/k/v and gate/up as fused GEMMs (N 6144 and 24576); "
                                    "'g128': the same layer with one scale per 128 input "
                                    "channels",
                        "value": m1["GBs_kernels"], "unit": "GB/s",
                        "frac_hbm": m1["frac_hbm_kernels"], **out}


def section_moe(torch, i8, wl, dev, args, result):
    g = wl.rng(2)
    e = wl.MOE_ROUTED + wl.MOE_SHARED
    stacks = {}
    for proj, (n, k) in wl.MOE_16B.items():
        w = wl.to_bf16(wl.moe_weights(g, n, k).reshape(e * n, k)).to(dev)
        q, s = i8.quantize_per_channel_int8(w)
        del w
        stacks[proj] = (q.view(e, n, k), s.view(e, n))
    per_layer = sum(e * n * k for n, k in wl.MOE_16B.values())
    copies = max(2, -(-ROTATE_BYTES // per_layer))
    rot = [stacks] + [{p: (q.clone(), s) for p, (q, s) in stacks.items()} for _ in range(copies - 1)]
    out = {"copies": copies, "per_t": {}}
    for t in wl.MOE_TOKENS:
        ids = wl.moe_expert_ids(g, t)
        distinct = len(np.unique(ids))
        ids_d = torch.from_numpy(ids).to(dev)
        topk = ids.shape[1]
        x_in = wl.to_bf16(wl.activations(g, t, 2048)).to(dev)
        x_mid = wl.to_bf16(wl.activations(g, t * topk, 1408)).to(dev)
        ys = {p: torch.empty((t * topk, wl.MOE_16B[p][0]), dtype=torch.bfloat16, device=dev)
              for p in wl.MOE_16B}
        def call(p, i):
            q, s_ = rot[i % copies][p]
            x, pa = (x_mid, True) if p == "down" else (x_in, False)
            i8.grouped_w8a16_gemm(x, q, s_, ids_d, x_per_assignment=pa, out=ys[p])

        secs = time_loop(torch, lambda i: [call(p, i) for p in ("gate", "up", "down")],
                         args.steps, args.warmup)
        reps = max(5, args.steps // 5)
        durs = {p: per_call(torch, lambda i, p=p: call(p, i), reps) for p in wl.MOE_16B}
        nbytes = 0.0
        per = {}
        for p, (n, k) in wl.MOE_16B.items():
            xr = t * topk if p == "down" else t
            b = grouped_bytes(distinct, n, k, xr, t * topk)
            nbytes += b
            d = durs[p]
            per[p] = {"us": d * 1e6, "GBs": b / d / 1e9, "frac_hbm": b / d / 1e9 / PEAK_HBM_GBS}
        allk = sum(durs.values())
        out["per_t"][t] = {"distinct_experts": distinct, "layer_us": secs / args.steps * 1e6,
                           "GBs_kernels": nbytes / allk / 1e9,
                           "frac_hbm_kernels": nbytes / allk / 1e9 / PEAK_HBM_GBS,
                           "per_proj": per}
        ent = traffic_entry("grouped_w8a16_kernel", moe_traffic_workload(t))
        if ent is not None:  # HBM bytes per launch (FETCH_SIZE + WRITE_SIZE) vs algorithmic
            out["per_t"][t]["traffic"] = {
                "hbm_bytes_per_launch": ent["bytes_per_launch"],
                "algorithmic_bytes_per_launch": ent["algorithmic_bytes_per_launch"],
                "ratio": ent["bytes_per_launch"] / ent["algorithmic_bytes_per_launch"]}
        log(f"[moe] T={t}: {distinct} experts, {secs/args.steps*1e6:.1f} us/layer, "
            f"{out['per_t'][t]['GBs_kernels']:.0f} GB/s")
    # The whole block: routing from router logits, gate and up as one grouped GEMM over
    # weights stacked [E, 2 * 1408, 2048] with SiLU·mul fused, down, weighted combine.
    gu = [(torch.cat([r["gate"][0], r["up"][0]], dim=1).contiguous(),
           torch.cat([r["gate"][1], r["up"][1]], dim=1).contiguous()) for r in rot]
    n_i, hid = wl.MOE_16B["gate"]
    out["block"] = {}
    for t in wl.MOE_TOKENS:
        logits = torch.from_numpy(wl.router_logits(g, t)).to(dev)
        x_in = wl.to_bf16(wl.activations(g, t, hid)).to(dev)
        kk = wl.MOE_TOP + wl.MOE_SHARED
        ids_d = torch.empty((t, kk), dtype=torch.int32, device=dev)
        w_d = torch.empty((t, kk), dtype=torch.float32, device=dev)
        h = torch.empty((t * kk, n_i), dtype=torch.bfloat16, device=dev)
        dn = torch.empty((t * kk, hid), dtype=torch.bfloat16, device=dev)
        y = torch.empty((t, hid), dtype=torch.bfloat16, device=dev)
        steps_of = {
            "route": lambda i: i8.moe_route_topk(logits, wl.MOE_TOP, wl.MOE_SHARED,
                                                 ids_out=ids_d, weights_out=w_d),
            "gate_up_silu": lambda i: i8.grouped_w8a16_silu_gemm(
                x_in, gu[i % copies][0], gu[i % copies][1], ids_d, out=h),
            "down": lambda i: i8.grouped_w8a16_gemm(
                h, rot[i % copies]["down"][0], rot[i % copies]["down"][1], ids_d,
                x_per_assignment=True, out=dn),
            "combine": lambda i: i8.moe_combine(dn, w_d, out=y),
        }
        steps_of["route"](0)
        torch.cuda.synchronize()
        distinct = len(np.unique(ids_d.cpu().numpy()))
        secs = time_loop(torch, lambda i: [f(i) for f in steps_of.values()], args.steps,
                         args.warmup)
        reps = max(5, args.steps // 5)
        durs = {nm: per_call(torch, f, reps) for nm, f in steps_of.items()}
        nbytes = (grouped_bytes(distinct, 2 * n_i, hid, t, t * kk)
                  + grouped_bytes(distinct, hid, n_i, t * kk, t * kk)
                  + t * wl.MOE_ROUTED * 4 + t * kk * 8            # logits in, ids + weights out
                  + t * kk * hid * 2 + t * kk * 4 + t * hid * 2)  # combine
        us = secs / args.steps * 1e6
        out["block"][t] = {"distinct_experts": distinct, "block_us": us,
                           "GBs_block": nbytes / (secs / args.steps) / 1e9,
                           "frac_hbm_block": nbytes / (secs / args.steps) / 1e9 / PEAK_HBM_GBS,
                           "per_step_us": {nm: d * 1e6 for nm, d in durs.items()}}
        log(f"[moe] block T={t}: {distinct} experts, {us:.1f} us "
            f"(route {durs['route']*1e6:.1f}, gate/up+SiLU {durs['gate_up_silu']*1e6:.1f}, "
            f"down {durs['down']*1e6:.1f}, combine {durs['combine']*1e6:.1f}), "
            f"{out['block'][t]['GBs_block']:.0f} GB/s")
    result["moe"] = {"workload": "16B MoE block (64 routed + 2 shared experts, top-6), grouped "
                     "W8A16 gate/up/down, T in {1,4,16,64}; 'block': routing + gate/up with "
                     "SiLU·mul + down + combine", "unit": "GB/s", **out}


def calibration_copy(torch, dev):
    """A device-to-device copy of CALIB_BYTES, whose counter readings calibrate FETCH_SIZE
    and WRITE_SIZE (it moves exactly CALIB_BYTES each way)."""
    a = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def section_counters(torch, i8, wl, dev, args, result):
    """Eager launches for the hardware-counter runs of the headline step (rocprofv3 --pmc
    FETCH_SIZE, then WRITE_SIZE): the calibration copy, then two steps of the workload with
    its weight rotation, each kernel launched on its own."""
    wk = prefill_8b(torch, i8, wl, dev, (16384,))
    calibration_copy(torch, dev)
    for step in range(2):
        wk.step(step)
    torch.cuda.synchronize()
    result["counters"] = {"workload": HEADLINE, "calibration_copy_bytes": CALIB_BYTES,
                          "steps": 2}


def section_counters_4b(torch, i8, wl, dev, args, result):
    """As `counters`, for the dense 4B prefill step."""
    wk = prefill_4b(torch, i8, wl, dev)
    calibration_copy(torch, dev)
    for step in range(2):
        wk.step(step)
    torch.cuda.synchronize()
    result["counters_4b"] = {"calibration_copy_bytes": CALIB_BYTES, "steps": 2}


def section_counters_w8a8_large(torch, i8, wl, dev, args, result):
    """Eager launches for stall-counter runs of the W8A8 main loop: three 8192 x 8192 x 8192
    GEMMs with 256 x 256 tiles (configuration 0), bf16 output, random codes."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    m = n = k = 8192
    xq = torch.randint(-127, 128, (m, k), dtype=torch.int8, device=dev, generator=g)
    wq = torch.randint(-127, 128, (n, k), dtype=torch.int8, device=dev, generator=g)
    sx = torch.rand(m, device=dev, generator=g)
    sw = torch.rand(n, device=dev, generator=g)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        i8.w8a8_gemm_with_config(0, xq, sx, wq, sw, out=y)
    torch.cuda.synchronize()
    result["counters_w8a8_large"] = {"shape": [m, n, k], "config": 0, "launches": 3}


def section_counters_decode(torch, i8, wl, dev, args, result):
    """Like `counters`, for the W8A16 decode layer: the calibration copy, then two passes of
    the fused 8B decode projections at M = 1 with rotating weight copies, kernel by kernel."""
    g = wl.rng(1)
    pq, ps = {}, {}
    for nm, (n, k) in wl.DENSE_8B.items():
        pq[nm], ps[nm] = i8.quantize_per_channel_int8(wl.to_bf16(wl.weight(g, n, k)).to(dev))
    q0 = {f: torch.cat([pq[p] for p in parts]).contiguous()
          for f, parts in wl.DENSE_8B_FUSED.items()}
    s0 = {f: torch.cat([ps[p] for p in parts]).contiguous()
          for f, parts in wl.DENSE_8B_FUSED.items()}
    del pq, ps
    layer = sum(q.numel() for q in q0.values())
    copies = max(2, -(-ROTATE_BYTES // layer))
    qs = [q0] + [{nm: q.clone() for nm, q in q0.items()} for _ in range(copies - 1)]
    xs = {k: wl.to_bf16(wl.activations(g, 1, k)).to(dev) for k in (4096, 12288)}
    a = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    for rep in range(2):
        for nm, q in qs[rep % copies].items():
            i8.w8a16_gemm(xs[q.shape[1]], q, s0[nm])
    torch.cuda.synchronize()
    result["counters_decode"] = {"calibration_copy_bytes": CALIB_BYTES, "passes": 2}


MOE_COUNTER_TOKENS = (1, 4, 16, 64)


def moe_traffic_workload(t):
    return f"16B MoE grouped W8A16 gate/up/down T={t}"


def section_counters_moe(torch, i8, wl, dev, args, result):
    """Like `counters`, for the grouped W8A16 GEMMs of the 16B MoE block: the calibration
    copy, then for T in MOE_COUNTER_TOKENS two passes of gate, up and down (each launched on
    its own, weight copies rotating over >= 1 GiB), with each launch's algorithmic bytes."""
    g = wl.rng(2)
    e = wl.MOE_ROUTED + wl.MOE_SHARED
    stacks = {}
    for proj, (n, k) in wl.MOE_16B.items():
        w = wl.to_bf16(wl.moe_weights(g, n, k).reshape(e * n, k)).to(dev)
        q, s = i8.quantize_per_channel_int8(w)
        del w
        stacks[proj] = (q.view(e, n, k), s.view(e, n))
    per_layer = sum(e * n * k for n, k in wl.MOE_16B.values())
    copies = max(2, -(-ROTATE_BYTES // per_layer))
    rot = [stacks] + [{p: (q.clone(), s) for p, (q, s) in stacks.items()} for _ in range(copies - 1)]
    inputs = {}
    for t in MOE_COUNTER_TOKENS:
        ids = wl.moe_expert_ids(g, t)
        topk = ids.shape[1]
        inputs[t] = (torch.from_numpy(ids).to(dev), len(np.unique(ids)), topk,
                     wl.to_bf16(wl.activations(g, t, 2048)).to(dev),
                     wl.to_bf16(wl.activations(g, t * topk, 1408)).to(dev))
    calibration_copy(torch, dev)
    launches = []
    i = 0
    for t in MOE_COUNTER_TOKENS:
        ids_d, distinct, topk, x_in, x_mid = inputs[t]
        for rep in range(2):
            for p in ("gate", "up", "down"):
                n, k = wl.MOE_16B[p]
                q, s_ = rot[i % copies][p]
                x, pa = (x_mid, True) if p == "down" else (x_in, False)
                i8.grouped_w8a16_gemm(x, q, s_, ids_d, x_per_assignment=pa)
                xr = t * topk if p == "down" else t
                launches.append({"tokens": t, "proj": p,
                                 "algorithmic_bytes": grouped_bytes(distinct, n, k, xr,
                                                                    t * topk)})
            i += 1
    torch.cuda.synchronize()
    result["counters_moe"] = {"calibration_copy_bytes": CALIB_BYTES, "launches": launches}


def section_weight_quant(torch, i8, wl, dev, args, result):
    g = wl.rng(4)
    ws = {nm: wl.to_bf16(wl.weight(g, n, k)).to(dev) for nm, (n, k) in wl.DENSE_8B.items()}
    outs = {nm: (torch.empty(w.shape, dtype=torch.int8, device=dev),
                 torch.empty((w.shape[0],), dtype=torch.float32, device=dev)) for nm, w in ws.items()}
    steps = max(3, args.steps // 10)
    secs = time_loop(torch, lambda i: [i8.quantize_per_channel_int8(w, *outs[nm]) for nm, w in ws.items()],
                     steps, 2)
    nbytes = sum(quant_bytes(*w.shape) for w in ws.values())
    gbs = nbytes / (secs / steps) / 1e9
    result["weight_quant"] = {"workload": "per-channel quantization of the dense 8B layer's bf16 "
                              "weights", "GBs": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    log(f"[weight_quant] {gbs:.0f} GB/s")


def section_norm_quant(torch, i8, wl, dev, args, result):
    """The per-token quantizer fused into the RMS norm that produces a projection's input
    (with the residual add), against the same norm writing bf16 followed by the quantizer,
    at the decoder layers' normed inputs: hidden 4096 at 4096 and 16384 tokens (8B), hidden
    2560 at 128, 512 and 2048 tokens (4B).  Inputs rotate over >= ROTATE_BYTES."""
    out = {"what": "rmsnorm_quantize_per_token_int8 (norm + residual add + per-token int8 in "
                   "one pass) vs rmsnorm_bf16 then quantize_per_token_int8; algorithmic bytes: "
                   "x, residual read and written, gamma, codes and scales (the unfused pair "
                   "also writes and reads the bf16 norm output)", "per_shape": []}
    g = wl.rng(77)
    for label, m, k in (("8B", 16384, 4096), ("8B", 4096, 4096), ("4B", 2048, 2560),
                        ("4B", 512, 2560), ("4B", 128, 2560)):
        copies = int(min(1024, max(1, -(-ROTATE_BYTES // (m * k * 4)))))
        x0 = wl.to_bf16(wl.activations(g, m, k, outlier_frac=0.01)).to(dev)
        r0 = wl.to_bf16(wl.activations(g, m, k)).to(dev)
        xs = [x0.clone() for _ in range(copies)]
        rs = [r0.clone() for _ in range(copies)]
        gamma = wl.to_bf16(wl.norm_weight(g, k)).to(dev)
        q = torch.empty((m, k), dtype=torch.int8, device=dev)
        sc = torch.empty((m,), dtype=torch.float32, device=dev)
        h = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
        reps = max(copies, 20)

        def fused(i):
            i8.rmsnorm_quantize_per_token_int8(xs[i % copies], gamma, 1e-6, rs[i % copies],
                                               q_out=q, scale_out=sc)

        def unfused(i):
            i8.rmsnorm_bf16(xs[i % copies], gamma, 1e-6, rs[i % copies], y_out=h)
            i8.quantize_per_token_int8(h, q_out=q, scale_out=sc)

        t_f = per_call(torch, fused, reps)
        t_u = per_call(torch, unfused, reps)
        b_f = m * k * (2 + 2 + 2 + 1) + 4 * m + 2 * k
        b_u = b_f + m * k * (2 + 2)
        out["per_shape"].append({"model": label, "m": m, "k": k, "fused_us": t_f * 1e6,
                                 "unfused_us": t_u * 1e6, "fused_GBs": b_f / t_f / 1e9,
                                 "fused_frac_hbm": b_f / t_f / 1e9 / PEAK_HBM_GBS,
                                 "unfused_GBs": b_u / t_u / 1e9, "saved_us": (t_u - t_f) * 1e6})
        if (m, k) == (16384, 4096):
            tr = traffic_for("rmsnorm_rows_kernel", NORM_TRAFFIC)
            out["per_shape"][-1]["traffic_fused_bytes"] = tr
            out["per_shape"][-1]["algorithmic_fused_bytes"] = b_f
        log(f"[norm_quant] {label} {m}x{k}: fused {t_f * 1e6:.1f} us "
            f"({b_f / t_f / 1e9:.0f} GB/s), norm + quantizer {t_u * 1e6:.1f} us")
        del xs, rs, x0, r0
    result["norm_quant"] = out


def section_silu_quant(torch, i8, wl, dev, args, result):
    """The per-token quantizer fused into the SiLU·mul that produces a down projection's input
    from the gate/up output, against SiLU·mul writing bf16 followed by the quantizer, at the
    decoder MLPs' shapes: intermediate 12288 at 4096 and 16384 tokens (8B), 9728 at 128, 512
    and 2048 tokens (4B).  Inputs rotate over >= ROTATE_BYTES."""
    out = {"what": "silu_mul_quantize_per_token_int8 (SiLU·mul + per-token int8 in one pass) vs "
                   "silu_mul_bf16 then quantize_per_token_int8; algorithmic bytes: the gate/up "
                   "rows read, codes and scales written (the unfused pair also writes and reads "
                   "the bf16 activation)", "per_shape": []}
    g = wl.rng(79)
    for label, m, n in (("8B", 16384, 12288), ("8B", 4096, 12288), ("4B", 2048, 9728),
                        ("4B", 512, 9728), ("4B", 128, 9728)):
        copies = int(min(1024, max(1, -(-ROTATE_BYTES // (m * n * 4)))))
        gate = g.standard_normal((m, n), dtype=np.float32) * np.float32(4.0)
        up = g.standard_normal((m, n), dtype=np.float32) * np.float32(3.0)
        g0 = wl.to_bf16(np.concatenate([gate, up], axis=1)).to(dev)
        del gate, up
        gus = [g0.clone() for _ in range(copies)]
        q = torch.empty((m, n), dtype=torch.int8, device=dev)
        sc = torch.empty((m,), dtype=torch.float32, device=dev)
        h = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        reps = max(copies, 20)

        def fused(i):
            i8.silu_mul_quantize_per_token_int8(gus[i % copies], q_out=q, scale_out=sc)

        def unfused(i):
            i8.silu_mul_bf16(gus[i % copies], h_out=h)
            i8.quantize_per_token_int8(h, q_out=q, scale_out=sc)

        t_f = per_call(torch, fused, reps)
        t_u = per_call(torch, unfused, reps)
        b_f = m * n * (2 + 2 + 1) + 4 * m
        b_u = b_f + m * n * (2 + 2)
        out["per_shape"].append({"model": label, "m": m, "n": n, "fused_us": t_f * 1e6,
                                 "unfused_us": t_u * 1e6, "fused_GBs": b_f / t_f / 1e9,
                                 "fused_frac_hbm": b_f / t_f / 1e9 / PEAK_HBM_GBS,
                                 "unfused_GBs": b_u / t_u / 1e9, "saved_us": (t_u - t_f) * 1e6})
        log(f"[silu_quant] {label} {m}x{n}: fused {t_f * 1e6:.1f} us "
            f"({b_f / t_f / 1e9:.0f} GB/s), SiLU·mul + quantizer {t_u * 1e6:.1f} us")
        del gus, g0
    result["silu_quant"] = out


def section_layer_8b(torch, i8, wl, dev, args, result):
    """The dense 8B decoder layer's W8A8 projections in their data flow, attention left out:
    the RMS norm (with the residual add) produces q/k/v's input, a synthetic attention output
    is quantized for o, the second norm adds o's output to the residual stream and produces
    gate/up's input, and SiLU·mul of the gate/up output produces down's input.  Once with
    the quantizer fused into the norms and the SiLU·mul, once with them writing bf16 and the
    quantizer apart.  4096 and 16384 tokens, bias, weights rotating as in the step."""
    out = {"what": "norm+quant -> q/k/v GEMM; quant(attention output, synthetic) -> o GEMM; "
                   "norm(residual + o)+quant -> gate/up GEMM; SiLU·mul+quant -> down GEMM; "
                   "fused producers vs the same producers writing bf16 + quantize_per_token_int8",
           "per_tokens": {}}
    g = wl.rng(83)
    eps = 1e-6
    for m in (4096, 16384):
        wk = prefill_8b(torch, i8, wl, dev, (m,))
        hid = wk.kin["attn_in"]
        inter = wk.kin["mlp_mid"]
        x = wl.to_bf16(wl.activations(g, m, hid, 0.01)).to(dev)       # previous layer's output
        res = wl.to_bf16(wl.activations(g, m, hid)).to(dev)          # residual stream
        attn = wk.xs[m]["attn_out"]                                  # stands in for attention
        g1 = wl.to_bf16(wl.norm_weight(g, hid)).to(dev)
        g2 = wl.to_bf16(wl.norm_weight(g, hid)).to(dev)
        hb = torch.empty((m, hid), dtype=torch.bfloat16, device=dev)
        hm = torch.empty((m, inter), dtype=torch.bfloat16, device=dev)
        qx = wk.qx[m]
        outs = wk.outs[m]

        def gemm(nm, src, i):
            q, sx = qx[src]
            i8.w8a8_gemm(q, sx, wk.qs[i % wk.copies][nm], wk.s[nm], wk.b[nm], out=outs[nm])

        def layer(i, fused):
            if fused:
                i8.rmsnorm_quantize_per_token_int8(x, g1, eps, res, *qx["attn_in"])
            else:
                i8.rmsnorm_bf16(x, g1, eps, res, y_out=hb)
                i8.quantize_per_token_int8(hb, *qx["attn_in"])
            gemm("qkv", "attn_in", i)
            i8.quantize_per_token_int8(attn, *qx["attn_out"])
            gemm("o", "attn_out", i)
            if fused:
                i8.rmsnorm_quantize_per_token_int8(outs["o"], g2, eps, res, *qx["mlp_in"])
            else:
                i8.rmsnorm_bf16(outs["o"], g2, eps, res, y_out=hb)
                i8.quantize_per_token_int8(hb, *qx["mlp_in"])
            gemm("gate_up", "mlp_in", i)
            if fused:
                i8.silu_mul_quantize_per_token_int8(outs["gate_up"], *qx["mlp_mid"])
            else:
                i8.silu_mul_bf16(outs["gate_up"], h_out=hm)
                i8.quantize_per_token_int8(hm, *qx["mlp_mid"])
            gemm("down", "mlp_mid", i)

        steps = max(5, args.steps // 5)
        t_f = time_loop(torch, lambda i: layer(i, True), steps, 2) / steps
        t_u = time_loop(torch, lambda i: layer(i, False), steps, 2) / steps
        ops = wk.ops()
        out["per_tokens"][str(m)] = {"fused_ms": t_f * 1e3, "unfused_ms": t_u * 1e3,
                                     "fused_TOPS": ops / t_f / 1e12,
                                     "unfused_TOPS": ops / t_u / 1e12,
                                     "saved_us": (t_u - t_f) * 1e6}
        log(f"[layer_8b] {m} tokens: fused producers {t_f * 1e3:.3f} ms "
            f"({ops / t_f / 1e12:.0f} TOPS over the GEMMs' ops), unfused {t_u * 1e3:.3f} ms")
        del wk, x, res, hb, hm
        torch.cuda.empty_cache()
    result["layer_8b"] = out


NORM_TRAFFIC = "RMS norm + residual + per-token int8, 16384x4096"


def section_counters_norm(torch, i8, wl, dev, args, result):
    """Like `counters`, for the RMS norm fused with the per-token quantizer at 16384 x 4096
    with the residual add: the calibration copy, then four fused launches over rotating
    inputs, then two of the unfused pair (the norm writing bf16, then the quantizer)."""
    g = wl.rng(77)
    m, k = 16384, 4096
    copies = 4
    x0 = wl.to_bf16(wl.activations(g, m, k, outlier_frac=0.01)).to(dev)
    r0 = wl.to_bf16(wl.activations(g, m, k)).to(dev)
    xs = [x0.clone() for _ in range(copies)]
    rs = [r0.clone() for _ in range(copies)]
    gamma = wl.to_bf16(wl.norm_weight(g, k)).to(dev)
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    sc = torch.empty((m,), dtype=torch.float32, device=dev)
    h = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    calibration_copy(torch, dev)
    for i in range(copies):
        i8.rmsnorm_quantize_per_token_int8(xs[i], gamma, 1e-6, rs[i], q_out=q, scale_out=sc)
    for i in range(2):
        i8.rmsnorm_bf16(xs[i], gamma, 1e-6, rs[i], y_out=h)
        i8.quantize_per_token_int8(h, q_out=q, scale_out=sc)
    torch.cuda.synchronize()
    result["counters_norm"] = {"workload": NORM_TRAFFIC, "calibration_copy_bytes": CALIB_BYTES,
                               "fused_launches": copies,
                               "algorithmic_bytes_fused": m * k * 7 + 4 * m + 2 * k}


SECTIONS = {  # name -> (function, needs the GPU objects); the default run is DEFAULT
    "step": section_step, "prefill_8b_m4096": section_prefill_8b_m4096,
    "prefill_8b_g128": section_prefill_8b_g128,
    "prefill_4b": section_prefill_4b, "decode": section_decode, "moe": section_moe,
    "weight_quant": section_weight_quant, "norm_quant": section_norm_quant,
    "silu_quant": section_silu_quant, "layer_8b": section_layer_8b,
    # hardware-counter runs only (eager launches, nothing timed)
    "counters": section_counters, "counters_4b": section_counters_4b,
    "counters_decode": section_counters_decode,
    "counters_w8a8_large": section_counters_w8a8_large,
    "counters_moe": section_counters_moe, "counters_norm": section_counters_norm,
}
DEFAULT = ("step,cpu_baseline,prefill_8b_m4096,prefill_8b_g128,prefill_4b,decode,moe,"
           "weight_quant,norm_quant,silu_quant,layer_8b")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sections", default=DEFAULT)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(only the single-GPU path is built: column-parallel projections would shard N, "
              "row-parallel ones K with an all-reduce, the MoE block its experts)",
              file=sys.stderr)
        sys.exit(2)
    sections = args.sections.split(",")
    unknown = [x for x in sections if x not in SECTIONS and x != "cpu_baseline"]
    if unknown:
        print(f"unknown sections {unknown}; known: cpu_baseline, {', '.join(SECTIONS)}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_quantized_linear_amd as i8
    from int8_quantized_linear_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    i8.load_library()
    dev = torch.device("cuda:0")
    result = {"metric": METRIC, "value": None, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
              "config": {"workload": "W8A8 prefill at scale on the dense 8B decoder layer "
                         "(hidden 4096, intermediate 12288: q/o 4096->4096, k/v 4096->1024, "
                         "gate/up 4096->12288, down 12288->4096), 16384 tokens per step: "
                         "per-token int8 quantization of the layer's 4 inputs + int8 MFMA "
                         "GEMMs with the fused scale + bias epilogue to bf16",
                         "launches": "q/k/v and gate/up each run as one GEMM over their "
                                     "concatenated weights (N 6144 and 24576): 4 quantizer + "
                                     "4 GEMM launches per step, the same products as 7 "
                                     "separate projections",
                         "tokens_per_step": 16384,
                         "weights": "bf16 N(0,0.02) -> per-channel int8; bias fp32 N(0,0.02)",
                         "activations": "bf16 N(0,1), 1% outlier dims x100",
                         "also_measured": "the same layer at 4096 tokens (prefill_8b_m4096), "
                                          "the dense 4B layer at 128/512/2048 tokens "
                                          "(prefill_4b), W8A16 decode, the grouped MoE "
                                          "GEMM and block, the weight quantizer"},
              "device": torch.cuda.get_device_name(0)}
    for name in sections:
        if name == "cpu_baseline":
            section_cpu_baseline(i8, wl, args, result)
        else:
            SECTIONS[name](torch, i8, wl, dev, args, result)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

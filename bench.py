"""Benchmark: Llama-3-8B W4A16 decode step (129 quantized linears) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B]
                    [--workload decode|large-batch|fp8|int8|70b|pack-mse|moe|moe-w4a8]

One step is one pass of the whole hot path over one batch: the 129 W4A16
GEMMs of a Llama-3-8B decode step (32 layers of qkv 4096->6144, o 4096->4096,
gate_up 4096->28672, down 14336->4096, plus the LM head 4096->128256), each with
its own INT4 g128 weight (3.87 GB in total, far beyond every cache) and its own
bf16 activations, all resident in HBM before timing starts.  The step is
captured once in a HIP graph and replayed; HIP events on the launch stream
bracket exactly `--steps` replays after `--warmup` untimed ones.

Default workload "decode": B in {1, 2, 4, 8, 16}; the JSON line's value is
the algorithmic HBM throughput at --batch (default 16), the other batches are
listed under "by_batch".  The same line carries "single_gemm" (a[4, 4096] x
W[4096, 4096] over 64 rotating weight copies) and "large_batch" (the stack at
B in {32 .. 1024} against the dense bf16 stack in both weight layouts: MFMA
utilisation with its roofline at B = 512, the crossover, the oracle's CPU
baseline); --no-large-batch leaves the latter out.  Other workloads (one line
each):
  large-batch  only the large-batch half
  fp8          the W8A8-FP8 stack (per-token activation quantization + fp8 GEMM)
  int8         the W8A8-INT8 stack (per-token activation quantization + int8 GEMM)
  70b          the Llama-3-70B W4A16 stack on one GPU
  pack-mse     offline INT4 g128 packing of the Llama-3-8B weights with
               MSE-optimal clipping (100-point grid), against abs-max packing
  moe          the routed-expert GEMMs of a Qwen3-30B-A3B decode step (48
               layers x {gate_up, down} over 128 experts, top-8 routing),
               expert-grouped W4A16
  moe-w4a8     the same expert GEMMs as W4A8-FP8: per-token e4m3 quantization
               of each GEMM's rows, then the grouped INT4 x e4m3 GEMM

Algorithmic bytes of one W4A16 GEMM: K*N/2 (codes) + 2*N*K/128 (scales) +
2*M*K (activations) + 2*M*N (outputs); flops: 2*M*N*K.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
# Vector ALU rates per lane and clock from the published peaks: fp32 157.3 TFLOP/s
# = 256 CUs x 64 lanes x 2.4 GHz x 2 FMA x 2 flops, fp64 78.6 = the same x 1 FMA
VALU_LANE_CLOCKS = 256 * 64 * 2.4e9
VALU_FP32_PER_CLK, VALU_FP64_PER_CLK = 2.0, 1.0
# Instructions per (weight, grid point) in the clipping search's inner loop,
# counted in the AMD assembly of this build: 32-bit ones (the IEEE fp32 division
# sequence, rint, clamp, select) and 64-bit ones (convert, product, difference,
# square, sum)
MSE_FP32_OPS_PER_POINT = 14.05
MSE_FP64_OPS_PER_POINT = 5.58
MSE_GRID = 100
DOMINANT_SRC = os.path.join(ROOT, "weight_only_quantized_w4a16_amd", "csrc", "w4a16.hip")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(B):
    return os.path.join(PROFILES, f"w4a16_decode_kernel_llama3_8b_decode_B{B}_traffic.txt")


def w4a16_bytes(M, K, N):
    return K * N // 2 + 2 * N * (K // 128) + 2 * M * K + 2 * M * N


def fp8_bytes(M, K, N):
    # weights + channel scales + fp8 activations + row scales + bf16 outputs
    return K * N + 4 * N + M * K + 4 * M + 2 * M * N


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--batch", type=int, default=16)
    p.add_argument("--workload", default="decode", choices=["decode", "large-batch", "fp8", "int8", "70b", "pack-mse", "moe",
                                                     "moe-w4a8"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--batches", default="",
                   help="large-batch workload: extra batch sizes to time, comma separated")
    p.add_argument("--no-large-batch", action="store_true",
                   help="decode workload: skip the large-batch half (B = 32 .. 1024 against dense bf16)")
    p.add_argument("--lb-steps", type=int, default=20,
                   help="timed replays per large-batch step (B = 32 .. 1024)")
    p.add_argument("--only-batch", action="store_true",
                   help="decode workload: time only --batch (short profiled runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (counter calibration) and exit")
    p.add_argument("--summarize-stats", metavar="CSV",
                   help="print a text summary of a rocprofv3 *_kernel_stats.csv and exit")
    p.add_argument("--summarize-mfma", metavar="DIR",
                   help="print the MFMA busy share per kernel from a rocprofv3 --pmc run of "
                        "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE and exit")
    p.add_argument("--profile-step", action="store_true",
                   help="run --steps eager decode steps at --batch (no graphs, no timing) for counter runs")
    p.add_argument("--summarize-counters", nargs=5,
                   metavar=("FETCH_DIR", "WRITE_DIR", "VALU_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                   help="per-GEMM HBM traffic and VALU lane-ops per weight of a --profile-step run at "
                        "--batch; writes the dominant kernel's traffic summary under profiles/, then exits")
    p.add_argument("--command", default="", help="command line recorded in summaries")
    return p.parse_args()


# ----------------------------------------------------------------------------- GPU side

class Stack:
    """The packed weights, activations and outputs of one decode step."""

    def __init__(self, ops, synth, torch, model, batches, fp8=False, int8=False):
        self.torch = torch
        self.ops = ops
        self.shapes = synth.stack_shapes(model)
        self.batches = batches
        self.fp8 = fp8
        self.int8 = int8
        dev = torch.device("cuda:0")
        self.layers = []
        maxb = max(batches)
        for idx, (name, K, N) in enumerate(self.shapes):
            layer, j = divmod(idx, 4)
            seed = synth.weight_seed(layer, j)
            w = synth.normal_bf16_device((K, N), seed, synth.WEIGHT_STD, dev)
            if fp8:
                wt = ops.Fp8Weight.from_bf16(w)
            elif int8:
                wt = ops.Int8Weight.from_bf16(w)
            else:
                wt = ops.Int4G128Weight.from_bf16(w)
            del w
            a = synth.normal_bf16_device((maxb, K), synth.activation_seed(layer, j), 1.0, dev)
            y = torch.empty((maxb, N), dtype=torch.bfloat16, device=dev)
            if fp8:
                lin = ops.W8A8Fp8Linear(wt)
            elif int8:
                lin = ops.W8A8Int8Linear(wt)
            else:
                lin = ops.W4A16Linear(wt)
            rec = {"name": name, "K": K, "N": N, "w": wt, "a": a, "y": y, "lin": lin}
            if fp8 or int8:
                rec["qa"] = torch.empty((maxb, K), dtype=torch.int8 if int8 else torch.uint8, device=dev)
                rec["sa"] = torch.empty(maxb, dtype=torch.float32, device=dev)
            # allocate the largest workspace up front
            for b in batches:
                lin.workspace(b)
                if fp8 or int8:
                    lin.workspace(b, dynamic=True)
            self.layers.append(rec)
        torch.cuda.synchronize()

    def step(self, B, only=None, two_call=False):
        """One pass over the stack at batch B.  8-bit: the per-token activation
        quantization inside each GEMM call (qgemm_w8a8_*_dynamic), or with
        two_call the separate quantization kernel before each GEMM."""
        ops = self.ops
        for r in self.layers:
            if only is not None and not only(r):
                continue
            a = r["a"][:B]
            y = r["y"][:B]
            if (self.int8 or self.fp8) and not two_call:
                ws, nb = r["lin"].workspace(B, dynamic=True)
                dyn = ops.qgemm_w8a8_int8_dynamic if self.int8 else ops.qgemm_w8a8_fp8_dynamic
                dyn(a, r["w"].codes, r["w"].scales, y, B, r["N"], r["K"], ws, nb)
            elif self.int8:
                ops.quant_act_per_token_int8(a, B, r["K"], r["qa"][:B], r["sa"][:B])
                ws, nb = r["lin"].workspace(B)
                ops.qgemm_w8a8_int8(r["qa"][:B], r["sa"][:B], r["w"].codes, r["w"].scales, y,
                                    B, r["N"], r["K"], ws, nb)
            elif self.fp8:
                ops.quant_act_per_token(a, B, r["K"], r["qa"][:B], r["sa"][:B])
                ws, nb = r["lin"].workspace(B)
                ops.qgemm_w8a8_fp8(r["qa"][:B], r["sa"][:B], r["w"].codes, r["w"].scales, y,
                                   B, r["N"], r["K"], ws, nb)
            else:
                ws, nb = r["lin"].workspace(B)
                ops.qgemm_w4a16(a, r["w"].packed, r["w"].scales, y, B, r["N"], r["K"], ws, nb)

    def check_outputs(self, B, g, **step_args):
        return check_replay(self.torch, g, lambda: self.step(B, **step_args),
                            [r["y"][:B] for r in self.layers], f"B={B}")

    def bytes(self, B, only=None):
        f = fp8_bytes if (self.fp8 or self.int8) else w4a16_bytes
        return sum(f(B, r["K"], r["N"]) for r in self.layers if only is None or only(r))

    def flops(self, B):
        return sum(2 * B * r["K"] * r["N"] for r in self.layers)


def check_replay(torch, g, step, outputs, what):
    """Replays the timed step's graph once, then runs the same step eagerly:
    every output must be finite and the two runs identical bit for bit (a
    split-K slot read before its write, or any other race between the step's
    launches, would show here).  Returns True when both hold."""
    g.replay()
    torch.cuda.synchronize()
    first = [y.clone() for y in outputs]
    step()
    torch.cuda.synchronize()
    finite = all(bool(torch.isfinite(f).all()) for f in first)
    same = all(torch.equal(f, y) for f, y in zip(first, outputs))
    del first
    if not (finite and same):
        print(f"[bench] {what}: output check failed (finite {finite}, replay == eager {same})",
              file=sys.stderr, flush=True)
    return finite and same


def graph_of(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, steps, warmup):
    """Replay `warmup` times untimed, then time exactly `steps` replays with HIP
    events on the replay stream; returns ms per replay."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def replay_percentiles(torch, g, n=50):
    """p10 / median / p90 of single replays, each bracketed by its own HIP events
    (a pass of its own after the timed region)."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    return [round(float(np.percentile(t, q)), 4) for q in (10, 50, 90)]


DOMINANT_KERNEL = "w4a16_decode_kernel"


def dominant_rule(ops, M, K, N):
    """Launches that run the dominant kernel (the library reports which kernel it
    selects for a shape): at B <= 16 the decode kernel runs every GEMM."""
    return ops.w4a16_kernel_for(M, N, K).startswith(DOMINANT_KERNEL + "<")


def read_traffic(kernel_sha, B):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary at this batch, if it was taken on the current kernel source; else None."""
    path = traffic_file(B)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(B):
    """The oracle (numpy fp32 dequant + fp64 matmul) on the host cores, on a bounded
    sample of the decode step: one decoder layer's four GEMMs plus 1/8 of the LM
    head's columns, each timed REPS times, scaled to the full 129-GEMM step."""
    REPS = 24
    from oracle import int4_g128 as q4
    from weight_only_quantized_w4a16_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    total = 0.0
    parts = []
    for j, (name, K, N) in enumerate(synth.LLAMA3_8B_LAYER):
        w = synth.weights(K, N, seed=synth.weight_seed(0, j))
        a = synth.activations(B, K, seed=synth.activation_seed(0, j))
        codes, s = q4.quantize(w)                   # offline: not timed
        del w
        t = time.perf_counter()
        for _ in range(REPS):
            q4.gemm_ref(a, codes, s)
        dt = (time.perf_counter() - t) / REPS
        total += 32 * dt
        parts.append(f"{name} {dt:.2f}s")
        del codes, s
    K, N = synth.LLAMA3_8B_HEAD[1:]
    cols = N // 8
    w = synth.weights(K, cols, seed=synth.weight_seed(32, 0))
    a = synth.activations(B, K, seed=synth.activation_seed(32, 0))
    codes, s = q4.quantize(w)
    del w
    t = time.perf_counter()
    for _ in range(REPS):
        q4.gemm_ref(a, codes, s)
    dt = (time.perf_counter() - t) / REPS
    total += 8 * dt
    parts.append(f"lm_head[:, :{cols}] {dt:.2f}s")
    return total, threads, parts


# ----------------------------------------------------------------------------- main

COPY_BYTES = 1 << 30


def copy_calibration(torch):
    """A plain device-to-device copy of 1 GiB, run 3 times: the counters of these
    dispatches read COPY_BYTES fetched and COPY_BYTES written per dispatch."""
    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "dispatches": 3}))


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def _gemm_dispatches(d, counter):
    """(kernel name, value) of every GEMM dispatch carrying `counter`, in dispatch order."""
    rows = [r for r in _pmc_rows(d) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    out = []
    for r in rows:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        if any(k in name for k in ("w4a16_decode_kernel", "w4a16_small_m_kernel", "w4a16_large_m_kernel")):
            out.append((name, float(r["Counter_Value"])))
    return out


def _copy_kib(d, counter):
    vals = [float(r["Counter_Value"]) for r in _pmc_rows(d)
            if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower() and "qg::" not in r["Kernel_Name"]]
    return sum(vals) / len(vals), len(vals)


def summarize_counters(dirs, B, command):
    """Per-GEMM HBM traffic (FETCH_SIZE + WRITE_SIZE, each scaled by what the
    counter reads for a 1 GiB device copy) and VALU lane-ops per streamed weight
    (SQ_INSTS_VALU x 64 / K N) of a --profile-step run: its GEMM dispatches come
    in the step's order, so dispatch i is GEMM i mod 129 of the stack."""
    from weight_only_quantized_w4a16_amd import synth
    fetch_dir, write_dir, valu_dir, cf_dir, cw_dir = dirs
    shapes = synth.stack_shapes("8b")
    n = len(shapes)
    fetch = _gemm_dispatches(fetch_dir, "FETCH_SIZE")
    write = _gemm_dispatches(write_dir, "WRITE_SIZE")
    valu = _gemm_dispatches(valu_dir, "SQ_INSTS_VALU")
    mfma = _gemm_dispatches(valu_dir, "SQ_INSTS_MFMA")
    cf_kib, ncf = _copy_kib(cf_dir, "FETCH_SIZE")
    cw_kib, ncw = _copy_kib(cw_dir, "WRITE_SIZE")
    f_scale = (COPY_BYTES / 1024) / cf_kib
    w_scale = (COPY_BYTES / 1024) / cw_kib
    for lst in (fetch, write, valu, mfma):
        assert len(lst) % n == 0 and len(lst) > 0, f"{len(lst)} GEMM dispatches is not a whole number of steps"
    groups = {}                                  # (layer-shape name, kernel) -> accumulators
    for i, (name, K, N) in enumerate(shapes):
        base = name.split(".")[-1]
        kern = fetch[i][0]
        key = (base, kern)
        g = groups.setdefault(key, {"K": K, "N": N, "n": 0, "f": 0.0, "w": 0.0, "v": 0.0, "m": 0.0})
        steps = len(fetch) // n
        for st in range(steps):
            j = st * n + i
            assert fetch[j][0] == kern and write[j][0] == kern and valu[j][0] == kern
            g["f"] += fetch[j][1] * 1024 * f_scale
            g["w"] += write[j][1] * 1024 * w_scale
            g["v"] += valu[j][1]
            g["m"] += mfma[j][1]
            g["n"] += 1
    sha = hashlib.sha256(open(DOMINANT_SRC, "rb").read()).hexdigest()
    lines = [f"# HBM traffic and VALU work per W4A16 GEMM, Llama-3-8B decode step, B={B}",
             f"# command: {command}",
             "# FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by copy bytes / counter of a 1 GiB device",
             "# copy; c = SQ_INSTS_VALU x 64 lanes / weights of the GEMM (VALU lane-ops per weight, budget",
             "# D*b/beta = 2.53 at which vector work takes as long as the weight stream).",
             f"copy_fetch_kib_raw: {cf_kib:.1f}  (dispatches {ncf})   fetch_scale: {f_scale:.4f}",
             f"copy_write_kib_raw: {cw_kib:.1f}  (dispatches {ncw})   write_scale: {w_scale:.4f}",
             f"{'gemm':8s} {'kernel':44s} {'disp':>5s} {'alg_MB':>8s} {'fetch_MB':>9s} {'write_MB':>9s} "
             f"{'hbm/alg':>8s} {'c':>6s} {'mfma':>8s}"]
    dom_bytes = dom_hbm = 0.0
    dom_n = 0
    for (base, kern), g in groups.items():
        K, N = g["K"], g["N"]
        alg = w4a16_bytes(B, K, N)
        f, w, v, m = (g[k] / g["n"] for k in ("f", "w", "v", "m"))
        lines.append(f"{base:8s} {kern[:44]:44s} {g['n']:5d} {alg / 1e6:8.2f} {f / 1e6:9.2f} {w / 1e6:9.3f} "
                     f"{(f + w) / alg:8.3f} {v * 64 / (K * N):6.3f} {m:8.0f}")
        if DOMINANT_KERNEL in kern:
            dom_bytes += alg * g["n"]
            dom_hbm += (f + w) * g["n"]
            dom_n += g["n"]
    if dom_n:
        lines += [f"kernel: {DOMINANT_KERNEL}",
                  f"dominant_dispatches: {dom_n}",
                  f"algorithmic_bytes_per_launch: {dom_bytes / dom_n:.0f}",
                  f"hbm_bytes_per_launch: {dom_hbm / dom_n:.0f}",
                  f"hbm_over_algorithmic: {dom_hbm / dom_bytes:.4f}"]
    lines.append(f"kernel_source_sha256: {sha}")
    with open(traffic_file(B), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def run_profile_step(args, torch, ops, synth):
    """--steps eager decode steps at --batch, nothing else on the GPU (counter runs)."""
    stack = Stack(ops, synth, torch, "8b", [args.batch])
    torch.cuda.synchronize()
    for _ in range(args.steps):
        stack.step(args.batch)
    torch.cuda.synchronize()
    print(json.dumps({"profile_step": args.batch, "steps": args.steps, "gemms_per_step": len(stack.layers)}))


def summarize_mfma(dirname, command):
    """MFMA busy share of the library's kernels from one rocprofv3 --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA and GRBM_GUI_ACTIVE: busy cycles over
    the SIMD cycles of each dispatch (GRBM_GUI_ACTIVE counts every XCD's cycles,
    so one XCD's clock count is GRBM_GUI_ACTIVE / 8; the GPU has 256 CUs x 4
    SIMDs), and the clock that implies."""
    import collections
    rows = _pmc_rows(dirname)
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for r in rows:
        name = r["Kernel_Name"]
        if "qg::" not in name or "pack_" in name:   # the offline weight packing is setup
            continue
        d = per[name.split("(")[0].replace("void ", "")][r["Dispatch_Id"]]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    simds, xcds = 256 * 4, 8
    print("# MFMA busy share per kernel, rocprofv3 counters")
    print(f"# command: {command}")
    print("# busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8); clock = GRBM_GUI_ACTIVE / 8 / duration")
    print("# (the counter window is longer than a dispatch's timestamps: short dispatches read a high clock")
    print("# and a low busy share; the long GEMM dispatches give the step's figures)")
    print(f"{'kernel':60s} {'disp':>5s} {'avg_us':>8s} {'busy':>6s} {'GHz':>5s} {'share_of_time':>13s}")
    tot_busy = tot_cyc = tot_ns = 0.0
    summary = []
    for k, ds in per.items():
        ds = [d for d in ds.values() if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d]
        if not ds:
            continue
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds)
        cyc = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / xcds * simds
        ns = sum(d["ns"] for d in ds)
        tot_busy += busy
        tot_cyc += cyc
        tot_ns += ns
        summary.append((ns, k, len(ds), ns / len(ds) / 1e3, busy / cyc,
                        sum(d["GRBM_GUI_ACTIVE"] for d in ds) / xcds / ns))
    if not summary:
        print("no dispatch carries all three counters")
        return
    for ns, k, n, us, b, ghz in sorted(summary, reverse=True):
        print(f"{k[:60]:60s} {n:5d} {us:8.2f} {b:6.3f} {ghz:5.2f} {ns / tot_ns:13.3f}")
    print(f"{'all library kernels':60s} {'':5s} {'':8s} {tot_busy / tot_cyc:6.3f}")


def summarize_stats(csv_path, command):
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print(f"# rocprofv3 --kernel-trace --stats summary")
    print(f"# command: {command}")
    print(f"{'kernel':70s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_ms':>9s} {'pct':>6s}")
    for r in rows:
        name = r["Name"].split("(")[0][:70]
        print(f"{name:70s} {int(r['Calls']):7d} {float(r['AverageNs'])/1e3:9.2f} "
              f"{float(r['MinNs'])/1e3:9.2f} {float(r['MaxNs'])/1e3:9.2f} "
              f"{float(r['TotalDurationNs'])/1e6:9.2f} {float(r['Percentage']):6.2f}")
    # a large-M GEMM call is two launches (offset-term pre-pass + GEMM kernel):
    # their summed time per call, the figure bench.py's large-batch roofline times
    pre = [r for r in rows if "w4a16_group_rowsum_kernel" in r["Name"]]
    lm = [r for r in rows if "w4a16_large_m_kernel" in r["Name"]]
    if pre and lm:
        calls = sum(int(r["Calls"]) for r in pre)
        ns = sum(float(r["TotalDurationNs"]) for r in pre + lm)
        print(f"# large-M GEMM calls (pre-pass + w4a16_large_m_kernel): {calls} calls, "
              f"{ns / calls / 1e3:.2f} us of kernel time per call")


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.batch, args.command)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the quantized "
                          "linear layer is measured on one GPU's share (see the sharding notes); "
                          "--gpus N > 1 is not supported"}))
        sys.exit(2)

    import torch
    from weight_only_quantized_w4a16_amd import ops, synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.profile_step:
        run_profile_step(args, torch, ops, synth)
        return

    if args.workload == "decode":
        run_decode(args, torch, ops, synth)
    elif args.workload == "large-batch":
        run_large_batch(args, torch, ops, synth)
    elif args.workload in ("fp8", "int8"):
        run_fp8(args, torch, ops, synth, int8=args.workload == "int8")
    elif args.workload == "pack-mse":
        run_pack_mse(args, torch, ops, synth)
    elif args.workload in ("moe", "moe-w4a8"):
        run_moe(args, torch, ops, synth, w4a8=args.workload == "moe-w4a8")
    else:
        run_70b(args, torch, ops, synth)


LARGE_BATCHES = [32, 64, 128, 256, 384, 512, 576, 640, 768, 1024]
LARGE_ROOFLINE_B = 512         # the large-batch roofline and CPU baseline are quoted here


def run_decode(args, torch, ops, synth):
    """The default run: the decode step at B in {1, 2, 4, 8, 16} (the headline
    value, at --batch), the single-GEMM configuration, and the large-batch half
    of the metric (MFMA utilisation at B >= 512, the crossover against dense
    bf16), all in one JSON line."""
    decode_batches = [args.batch] if args.only_batch else sorted({1, 2, 4, 8, 16, args.batch})
    large = [] if (args.only_batch or args.no_large_batch) else LARGE_BATCHES
    stack = Stack(ops, synth, torch, "8b", decode_batches)
    print(f"[bench] packed {len(stack.layers)} GEMMs, {stack.bytes(0) / 1e9:.3f} GB of weights+scales",
          file=sys.stderr, flush=True)
    by_batch = {}
    for B in decode_batches:
        nbytes = stack.bytes(B)
        rec = {}
        g = graph_of(torch, lambda: stack.step(B))
        ms_g = time_graph(torch, g, args.steps, args.warmup)
        rec["step_ms_p10_p50_p90"] = replay_percentiles(torch, g)
        rec["outputs_checked"] = stack.check_outputs(B, g)
        del g
        ms = ms_g
        rec.update({"ms_per_step": round(ms, 5), "TB_s": round(nbytes / (ms * 1e-3) / 1e12, 3),
                    "hbm_frac": round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)})
        by_batch[str(B)] = rec
        print(f"[bench] B={B}: {rec}", file=sys.stderr, flush=True)
    B = args.batch
    ms = by_batch[str(B)]["ms_per_step"]
    nbytes = stack.bytes(B)

    # dominant kernel and its average launch duration, measured with HIP events
    # on the stream it runs on
    dom = lambda r: dominant_rule(ops, B, r["K"], r["N"])
    launches = sum(1 for r in stack.layers if dom(r))
    kernel = f"{DOMINANT_KERNEL} ({launches} launches per step)"
    g = graph_of(torch, lambda: stack.step(B, only=dom))
    dom_ms = time_graph(torch, g, args.steps, args.warmup)
    del g
    dom_bytes_per_launch = stack.bytes(B, only=dom) / launches
    dom_avg_us = dom_ms * 1e3 / launches
    achieved = dom_bytes_per_launch / (dom_avg_us * 1e-6) / 1e9
    sha = hashlib.sha256(open(DOMINANT_SRC, "rb").read()).hexdigest()
    traffic = read_traffic(sha, B)

    out = {
        "metric": "Llama-3-8B W4A16 decode-step ms & HBM TB/s vs batch; MFMA util at B>=512",
        "value": round(nbytes / (ms * 1e-3) / 1e12, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-g128 x bf16 -> fp32 acc (bf16 MFMA)",
        "data": "synthetic: weights N(0, 0.02^2) bf16 RTN-quantized on the GPU, activations N(0,1) bf16",
        "config": {"workload": "Llama-3-8B decode linear stack, W4A16 g128, 129 GEMMs "
                               "(32 x qkv/o/gate_up/down + LM head) in stream order, one HIP graph "
                               "per step",
                   "batch": B, "streamed_params": synth.stack_params("8b"),
                   "algorithmic_bytes_per_step": nbytes, "parallelism": "single GPU"},
        "by_batch": by_batch,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": kernel,
                     "launches_per_step": launches,
                     "algorithmic_bytes_per_launch": round(dom_bytes_per_launch),
                     "avg_launch_us": round(dom_avg_us, 3)},
    }
    if not args.no_cpu_baseline:
        sec, threads, parts = cpu_baseline(B)
        out["cpu_baseline"] = {
            "value": round(nbytes / sec / 1e12, 6), "unit": "TB/s", "cores": threads,
            "kind": "oracle", "seconds_per_step": round(sec, 2),
            "sample": (f"B={B}: layer-0 qkv/o/gate_up/down (each x32) + LM head columns "
                       f"[0, 16032) (x8), mean of 24 timed runs each; numpy fp32 dequant + fp64 matmul; "
                       + ", ".join(parts))}
    if not args.only_batch:
        del stack
        torch.cuda.empty_cache()
        out["single_gemm"] = single_gemm_part(args, torch, ops, synth)
    if large:
        out["large_batch"] = large_batch_part(args, torch, ops, synth, large)
    print(json.dumps(out), flush=True)


def single_gemm_part(args, torch, ops, synth):
    """The single-GEMM configuration: a[4, 4096] x W[4096, 4096] (weight seed 0,
    activation seed 1), timed over 64 copies of the packed weight (each copy
    quantized from its own draw), called in turn inside one HIP graph, so every
    call streams its weight from HBM (64 x 8.65 MB = 554 MB, beyond the 256 MB
    memory-side cache)."""
    M, K, N, COPIES = 4, 4096, 4096, 64
    dev = torch.device("cuda:0")
    ws = []
    for c in range(COPIES):
        w = synth.normal_bf16_device((K, N), 7000 + c, synth.WEIGHT_STD, dev)
        ws.append(ops.Int4G128Weight.from_bf16(w))
        del w
    w0 = synth.weights(K, N, seed=0)                       # copy 0 is the configuration's own draw
    ws[0] = ops.Int4G128Weight.from_bf16(torch.from_numpy(w0.view(np.int16)).view(torch.bfloat16).to(dev))
    a = torch.from_numpy(synth.activations(M, K, seed=1).view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert ops.w4a16_workspace_bytes(M, N, K) == 0

    def calls():
        for wt in ws:
            ops.qgemm_w4a16(a, wt.packed, wt.scales, y, M, N, K)
    g = graph_of(torch, calls)
    ms = time_graph(torch, g, args.steps, args.warmup)
    del g
    us = ms * 1e3 / COPIES
    nbytes = w4a16_bytes(M, K, N)
    rec = {"workload": "single W4A16 GEMM a[4, 4096] x W[4096, 4096], 64 rotating weight copies in one "
                       "HIP graph (HBM-resident weights)",
           "kernel": ops.w4a16_kernel_for(M, N, K), "us_per_gemm": round(us, 3),
           "algorithmic_bytes": nbytes, "TB_s": round(nbytes / (us * 1e-6) / 1e12, 3),
           "hbm_frac": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_single_gemm()
    print(f"[bench] single GEMM: {rec}", file=sys.stderr, flush=True)
    return rec


def cpu_baseline_single_gemm(reps=5):
    """The oracle on the single-GEMM configuration, the fp32 dequantization and the
    fp64 product timed separately, on every host core and on one core."""
    from oracle import int4_g128 as q4
    from oracle.bf16 import bf16_bits_to_f32
    from threadpoolctl import threadpool_info, threadpool_limits
    from weight_only_quantized_w4a16_amd import synth
    w = synth.weights(4096, 4096, seed=0)
    a = synth.activations(4, 4096, seed=1)
    codes, s = q4.quantize(w)                     # offline: not timed
    out = {"unit": "us per GEMM", "kind": "oracle"}
    for label, limit in (("all_cores", None), ("one_core", 1)):
        with threadpool_limits(limits=limit):
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            t_deq = t_mm = 0.0
            for _ in range(reps):
                t0 = time.perf_counter()
                wd = q4.dequant_f32(codes, s).astype(np.float64)
                t1 = time.perf_counter()
                bf16_bits_to_f32(a).astype(np.float64) @ wd
                t2 = time.perf_counter()
                t_deq += t1 - t0
                t_mm += t2 - t1
        out[label] = {"cores": threads, "dequant_us": round(t_deq / reps * 1e6, 1),
                      "matmul_us": round(t_mm / reps * 1e6, 1),
                      "value": round((t_deq + t_mm) / reps * 1e6, 1)}
    out["value"] = out["all_cores"]["value"]
    out["cores"] = out["all_cores"]["cores"]
    out["sample"] = f"the whole GEMM, mean of {reps} runs (dequant and fp64 matmul timed separately)"
    return out


def cpu_baseline_large(B):
    """The oracle on a bounded sample of the large-batch step: layer 0's four
    GEMMs at B rows and 1/16 of the LM head's columns, each timed 8 times,
    scaled to the 129-GEMM step (x32 and x16)."""
    from oracle import int4_g128 as q4
    from threadpoolctl import threadpool_info
    from weight_only_quantized_w4a16_amd import synth
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    total, parts = 0.0, []
    shapes = [(name, K, N, 32, j) for j, (name, K, N) in enumerate(synth.LLAMA3_8B_LAYER)]
    shapes.append(("lm_head/16", synth.LLAMA3_8B_HEAD[1], synth.LLAMA3_8B_HEAD[2] // 16, 16, None))
    REPS = 8
    for name, K, N, mult, j in shapes:
        seed = synth.weight_seed(0, j) if j is not None else synth.weight_seed(32, 0)
        w = synth.weights(K, N, seed=seed)
        a = synth.activations(B, K, seed=seed + 1000)
        codes, s = q4.quantize(w)                 # offline: not timed
        del w
        t0 = time.perf_counter()
        for _ in range(REPS):
            q4.gemm_ref(a, codes, s)
        dt = (time.perf_counter() - t0) / REPS
        total += mult * dt
        parts.append(f"{name} {dt:.2f}s")
        del codes, s
    return total, threads, parts


def large_batch_part(args, torch, ops, synth, batches):
    """The same W4A16 stack at large batches against the dense bf16 stack of the
    same weights, stored both as [K, N] (torch.matmul(a, w)) and in the
    checkpoint layout [N, K] (a @ w.T, what a linear layer computes);
    the crossover is located against the faster dense layout at each batch.
    Each step is a HIP graph, `steps` replays timed with HIP events."""
    steps, warmup = args.lb_steps, max(2, min(args.warmup, 5))
    stack = Stack(ops, synth, torch, "8b", batches)
    dev = torch.device("cuda:0")
    dense_kn, dense_nk = [], []
    for idx, (name, K, N) in enumerate(stack.shapes):
        layer, j = divmod(idx, 4)
        w = synth.normal_bf16_device((K, N), synth.weight_seed(layer, j), synth.WEIGHT_STD, dev)
        dense_kn.append(w)
        dense_nk.append(w.t().contiguous())
    torch.cuda.synchronize()
    res = {}
    for B in batches:
        g = graph_of(torch, lambda: stack.step(B))
        ms4 = time_graph(torch, g, steps, warmup)
        checked = stack.check_outputs(B, g)
        del g

        def kn_step():
            for r, w in zip(stack.layers, dense_kn):
                torch.matmul(r["a"][:B], w, out=r["y"][:B])

        def nk_step():
            for r, w in zip(stack.layers, dense_nk):
                torch.matmul(r["a"][:B], w.t(), out=r["y"][:B])      # a @ w.T, as a linear layer runs
        g = graph_of(torch, kn_step)
        ms_kn = time_graph(torch, g, steps, warmup)
        del g
        g = graph_of(torch, nk_step)
        ms_nk = time_graph(torch, g, steps, warmup)
        del g
        fl = stack.flops(B)
        frac = lambda t: round(fl / (t * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)
        res[str(B)] = {"w4a16_ms": round(ms4, 4), "bf16_kn_ms": round(ms_kn, 4), "bf16_nk_ms": round(ms_nk, 4),
                       "w4a16_mfma_frac": frac(ms4), "bf16_kn_mfma_frac": frac(ms_kn),
                       "bf16_nk_mfma_frac": frac(ms_nk),
                       "w4a16_TB_s": round(stack.bytes(B) / (ms4 * 1e-3) / 1e12, 3),
                       "outputs_checked": checked}
        print(f"[bench] large B={B}: {res[str(B)]}", file=sys.stderr, flush=True)
    # the smallest measured batch from which W4A16 is not faster than the faster
    # dense layout at every larger measured batch
    cross = None
    for b in sorted(res, key=int, reverse=True):
        r = res[b]
        if r["w4a16_ms"] < min(r["bf16_kn_ms"], r["bf16_nk_ms"]):
            break
        cross = int(b)
    B = LARGE_ROOFLINE_B if str(LARGE_ROOFLINE_B) in res else max(batches)
    fl = stack.flops(B)
    ms4 = res[str(B)]["w4a16_ms"]
    launches = len(stack.layers)
    avg_us = ms4 * 1e3 / launches
    achieved = fl / launches / (avg_us * 1e-6) / 1e12
    kernels = sorted({ops.w4a16_kernel_for(B, r["N"], r["K"]) for r in stack.layers})
    out = {"batches": batches, "steps": steps, "warmup": warmup, "by_batch": res,
           "crossover_batch_w4a16_not_faster": cross,
           "crossover_rule": "smallest measured B from which W4A16 is not faster than the faster dense "
                             "bf16 layout at every larger measured B",
           "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": f"w4a16_large_m_kernel with its offset-term pre-pass "
                                  f"(w4a16_group_rowsum_kernel), one GEMM call = both launches; "
                                  f"{launches} calls per step at B={B}: " + "; ".join(kernels),
                        "batch": B, "calls_per_step": launches,
                        "algorithmic_flops_per_call": round(fl / launches),
                        "avg_call_us": round(avg_us, 3)}}
    if not args.no_cpu_baseline:
        sec, threads, parts = cpu_baseline_large(B)
        out["cpu_baseline"] = {
            "value": round(fl / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds_per_step": round(sec, 2),
            "sample": f"B={B}: layer-0 qkv/o/gate_up/down (x32) + LM head columns [0, 8016) (x16), "
                      f"mean of 8 timed runs each; numpy fp32 dequant + fp64 matmul; " + ", ".join(parts)}
    del dense_kn, dense_nk, stack
    torch.cuda.empty_cache()
    return out


def run_large_batch(args, torch, ops, synth):
    """Only the large-batch half (with --batches: extra batch sizes)."""
    batches = LARGE_BATCHES
    if args.batches:
        extra = {int(x) for x in args.batches.split(",")}
        batches = sorted(extra if args.only_batch else set(batches) | extra)
    lb = large_batch_part(args, torch, ops, synth, batches)
    B = LARGE_ROOFLINE_B if str(LARGE_ROOFLINE_B) in lb["by_batch"] else batches[-1]
    out = {"metric": "Llama-3-8B W4A16 decode-step ms & HBM TB/s vs batch; MFMA util at B>=512",
           "value": lb["by_batch"][str(B)]["w4a16_mfma_frac"], "unit": f"fraction of bf16 MFMA peak at B={B}",
           "n_gpus": 1, "steps": lb["steps"], "warmup": lb["warmup"],
           "ms_per_step": lb["by_batch"][str(B)]["w4a16_ms"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int4-g128 x bf16 -> fp32 acc (bf16 MFMA)",
           "data": "synthetic", "config": {"workload": "Llama-3-8B W4A16 stack vs dense bf16 stack "
                                                       "([K, N] and [N, K] weights, hipBLASLt via torch)",
                                           "batch": B},
           "large_batch": lb}
    print(json.dumps(out), flush=True)


INT8_PEAK_TOPS = 5000.0        # dense int8 MFMA


def run_fp8(args, torch, ops, synth, int8=False):
    batches = [1, 16, 128, 512, 1024]
    stack = Stack(ops, synth, torch, "8b", batches, fp8=not int8, int8=int8)
    fmt = "int8" if int8 else "fp8"
    peak = INT8_PEAK_TOPS if int8 else FP8_PEAK_TFLOPS
    res = {}
    for B in batches:
        g = graph_of(torch, lambda: stack.step(B))
        ms = time_graph(torch, g, args.steps, args.warmup)
        checked = stack.check_outputs(B, g)
        del g
        g = graph_of(torch, lambda: stack.step(B, two_call=True))
        ms_two = time_graph(torch, g, args.steps, args.warmup)
        checked = stack.check_outputs(B, g, two_call=True) and checked
        del g
        res[str(B)] = {"ms_per_step": round(ms, 4),
                       "TB_s": round(stack.bytes(B) / (ms * 1e-3) / 1e12, 3),
                       f"{fmt}_mfma_frac": round(stack.flops(B) / (ms * 1e-3) / (peak * 1e12), 4),
                       "two_call_ms_per_step": round(ms_two, 4),
                       "outputs_checked": checked,
                       "gemms_quantizing_inside": sum(
                           1 for r in stack.layers
                           if ops.w8a8_dynamic_kernel_for(B, r["N"], r["K"]).startswith("w8a8_small_m_dyn"))}
        print(f"[bench] {fmt} B={B}: {res[str(B)]}", file=sys.stderr, flush=True)
    FMT = fmt.upper()
    out = {"metric": f"Llama-3-8B W8A8-{FMT} decode-step ms vs batch", "value": res["16"]["TB_s"],
           "unit": "TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": res["16"]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None,
           "dtype": ("int8 x int8 -> int32 acc (int8 MFMA)" if int8 else "e4m3 x e4m3 -> fp32 acc (fp8 MFMA)"),
           "data": "synthetic",
           "config": {"workload": f"Llama-3-8B W8A8-{FMT} stack incl. per-token activation quantization "
                                  f"(inside the GEMM call, qgemm_w8a8_{fmt}_dynamic; two_call: the separate "
                                  f"quantization kernel first)",
                      "batch": 16}, "by_batch": res}
    print(json.dumps(out), flush=True)


def cpu_baseline_pack_mse():
    """The oracle's MSE-clipping quantizer on gate_up columns [0, 1536) of layer 0
    (4096 x 1536 weights), one run.  Its work is numpy element-wise arithmetic,
    which runs on one thread."""
    from oracle import int4_g128 as q4
    from weight_only_quantized_w4a16_amd import synth
    threads = 1
    K, cols = 4096, 1536
    w = synth.weights(K, 28672, seed=synth.weight_seed(0, 2))[:, :cols]
    t = time.perf_counter()
    q4.quantize_mse(w, n_alpha=MSE_GRID)
    sec = time.perf_counter() - t
    return K * cols / sec, threads, f"layer-0 gate_up columns [0, {cols}) ({K * cols} weights), one run"


def run_pack_mse(args, torch, ops, synth):
    dev = torch.device("cuda:0")
    reps = max(3, min(args.steps, 10))
    stream = torch.cuda.current_stream()
    shapes = [(name, K, N, synth.LLAMA3_8B_LAYERS, j) for j, (name, K, N) in enumerate(synth.LLAMA3_8B_LAYER)]
    shapes.append((synth.LLAMA3_8B_HEAD[0], *synth.LLAMA3_8B_HEAD[1:], 1, 0))
    res = {}
    total_w = total_mse_s = total_abs_s = 0.0
    for name, K, N, count, j in shapes:
        w = synth.normal_bf16_device((K, N), synth.weight_seed(0 if count > 1 else 32, j),
                                     synth.WEIGHT_STD, dev)
        packed = torch.empty(K * N // 8, dtype=torch.int32, device=dev)
        scales = torch.empty(K // 128 * N, dtype=torch.int16, device=dev)

        def timed(fn, n):
            for _ in range(args.warmup if n > 3 else 1):
                fn()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(n):
                fn()
            t1.record(stream)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / n

        ms_abs = timed(lambda: ops.pack_int4_g128(w, K, N, packed, scales), args.steps)
        ms_mse = timed(lambda: ops.pack_int4_g128_mse(w, K, N, MSE_GRID, packed, scales), reps)
        # summed squared error of both packings (exact fp32 reconstruction on the GPU)
        errs = []
        for grid in (0, MSE_GRID):
            wt = ops.Int4G128Weight.from_bf16(w, mse_grid=grid)
            _, codes = wt.dequant(with_codes=True)
            G = K // 128
            s = wt.scales.view(torch.bfloat16).float().view(N // 16, G, 16).permute(1, 0, 2).reshape(G, N)
            what = (codes.float() - 8.0).view(G, 128, N) * s[:, None, :]
            errs.append(float(((w.float().view(G, 128, N) - what) ** 2).double().sum()))
            del wt, codes, what
        res[name] = {"K": K, "N": N, "count": count, "abs_max_ms": round(ms_abs, 4),
                     "abs_max_GB_s": round((2.5 + 1 / 64) * K * N / (ms_abs * 1e-3) / 1e9, 1),
                     "mse_ms": round(ms_mse, 3),
                     "mse_Gweights_s": round(K * N / (ms_mse * 1e-3) / 1e9, 2),
                     "sq_error_mse_over_abs_max": round(errs[1] / errs[0], 4)}
        print(f"[bench] pack {name}: {res[name]}", file=sys.stderr, flush=True)
        total_w += count * K * N
        total_mse_s += count * ms_mse * 1e-3
        total_abs_s += count * ms_abs * 1e-3
        del w, packed, scales
    gw = total_w / total_mse_s / 1e9
    achieved = gw * 1e9 * MSE_GRID / 1e12                        # T (weight, grid point) pairs / s
    peak = VALU_LANE_CLOCKS / (MSE_FP32_OPS_PER_POINT / VALU_FP32_PER_CLK
                               + MSE_FP64_OPS_PER_POINT / VALU_FP64_PER_CLK) / 1e12
    out = {"metric": "Llama-3-8B INT4 g128 packing with MSE-optimal clipping: weights per second",
           "value": round(gw, 3), "unit": "Gweights/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
           "ms_per_step": round(total_mse_s * 1e3, 2), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16 in, fp32 search, fp64 error sums", "data": "synthetic N(0, 0.02^2)",
           "config": {"workload": f"Llama-3-8B linear weights (32 x qkv/o/gate_up/down + LM head, "
                                  f"{int(total_w)} weights), {MSE_GRID}-point clipping grid",
                      "abs_max_pack_ms": round(total_abs_s * 1e3, 2)},
           "by_shape": res,
           "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(peak, 3),
                        "unit": "T weight-grid-points/s", "frac": round(achieved / peak, 4),
                        "traffic": None, "kernel": "int4_mse_scale_kernel (+ the packer, about 1 %)",
                        "fp32_ops_per_point": MSE_FP32_OPS_PER_POINT,
                        "fp64_ops_per_point": MSE_FP64_OPS_PER_POINT}}
    if not args.no_cpu_baseline:
        rate, threads, sample = cpu_baseline_pack_mse()
        out["cpu_baseline"] = {"value": round(rate / 1e9, 6), "unit": "Gweights/s", "cores": threads,
                               "kind": "oracle", "sample": sample}
    print(json.dumps(out), flush=True)


def moe_bytes(offsets, K, N, w4a8=False):
    """Algorithmic bytes of one grouped GEMM: the weights of the experts that
    receive rows, their activations (bf16, or e4m3 codes + row scales) and
    outputs."""
    active = int(np.sum(np.diff(offsets) > 0))
    T = int(offsets[-1])
    act = T * K + 4 * T if w4a8 else 2 * T * K
    return active * (K * N // 2 + 2 * N * (K // 128)) + act + 2 * T * N


def cpu_baseline_moe(B, w4a8=False):
    """The oracle on layer 0 of the expert stack at batch B: both grouped GEMMs
    over the first 16 experts that receive rows (quantization untimed), scaled
    by the number of experts with rows and by 48 layers."""
    from oracle import int4_g128 as q4
    from oracle import fp8_e4m3 as f8
    from oracle import w4a8 as o_w4a8
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    from weight_only_quantized_w4a16_amd import synth
    E, k = synth.QWEN3_MOE_EXPERTS, synth.QWEN3_MOE_TOPK
    token, offsets = synth.moe_routing(B, E, k, seed=B)
    total = 0.0
    for j, (name, K, N) in enumerate(synth.QWEN3_MOE_SHAPES):
        a = synth.activations(B, K, seed=synth.activation_seed(0, j))[token]
        active = [e for e in range(E) if offsets[e + 1] > offsets[e]]
        ex = {e: q4.quantize(synth.weights(K, N, seed=synth.weight_seed(0, j) * 1000 + e))
              for e in active[:16]}
        t = time.perf_counter()
        if w4a8:
            qa, sa = f8.quant_act_per_token(a)
            o_w4a8.grouped_gemm_ref(qa, sa, offsets, ex)
        else:
            q4.grouped_gemm_ref(a, offsets, ex)
        total += (time.perf_counter() - t) * len(active) / len(ex)
    return total * synth.QWEN3_MOE_LAYERS, threads


def run_moe(args, torch, ops, synth, w4a8=False):
    dev = torch.device("cuda:0")
    E, k, L = synth.QWEN3_MOE_EXPERTS, synth.QWEN3_MOE_TOPK, synth.QWEN3_MOE_LAYERS
    batches = [1, 16, 64, 256, 1024]
    maxT = max(batches) * k
    gemms = []
    for layer in range(L):
        for j, (name, K, N) in enumerate(synth.QWEN3_MOE_SHAPES):
            w = synth.normal_bf16_device((E, K, N), synth.weight_seed(layer, j), synth.WEIGHT_STD, dev)
            gw = ops.GroupedInt4Weight.from_bf16(w)
            del w
            a = synth.normal_bf16_device((maxT, K), synth.activation_seed(layer, j), 1.0, dev)
            y = torch.empty((maxT, N), dtype=torch.bfloat16, device=dev)
            q = (torch.empty((maxT, K), dtype=torch.uint8, device=dev),
                 torch.empty(maxT, dtype=torch.float32, device=dev)) if w4a8 else None
            gemms.append((name, K, N, gw, a, y, q))
    torch.cuda.synchronize()
    res = {}
    for B in batches:
        token, offsets = synth.moe_routing(B, E, k, seed=B)
        T = B * k
        off = torch.from_numpy(offsets).to(dev)
        nbytes = sum(moe_bytes(offsets, K, N, w4a8) for (_, K, N, *_r) in gemms)

        def step(two_call=False):
            for (_, K, N, gw, a, y, q) in gemms:
                if w4a8 and two_call:
                    ops.quant_act_per_token(a[:T], T, K, q[0][:T], q[1][:T])
                    gw.w4a8(q[0][:T], q[1][:T], off, out=y[:T])
                elif w4a8:
                    gw.w4a8_dynamic(a[:T], off, out=y[:T])
                else:
                    gw(a[:T], off, out=y[:T])
        outs = [y[:T] for (_, _, _, _, _, y, _) in gemms]
        g = graph_of(torch, step)
        ms = time_graph(torch, g, args.steps, args.warmup)
        checked = check_replay(torch, g, step, outs, f"moe B={B}")
        del g
        res[str(B)] = {"ms_per_step": round(ms, 4), "rows": T,
                       "active_experts": int(np.sum(np.diff(offsets) > 0)),
                       "TB_s": round(nbytes / (ms * 1e-3) / 1e12, 3), "bytes": nbytes}
        if w4a8:
            # the same step with the separate quantization kernel before each GEMM
            g = graph_of(torch, lambda: step(two_call=True))
            res[str(B)]["two_call_ms_per_step"] = round(time_graph(torch, g, args.steps, args.warmup), 4)
            checked = check_replay(torch, g, lambda: step(two_call=True), outs, f"moe two-call B={B}") and checked
            del g
            res[str(B)]["gemms_quantizing_inside"] = sum(
                1 for (_, K, N, gw, *_r) in gemms
                if ops.w4a8_grouped_dynamic_kernel_for(gw.E, T, N, K) == "w4a8_grouped_dyn_kernel")
        res[str(B)]["outputs_checked"] = checked
        print(f"[bench] moe B={B}: {res[str(B)]}", file=sys.stderr, flush=True)
    B = 16
    r = res[str(B)]
    _, K0, N0 = synth.QWEN3_MOE_SHAPES[0]
    per_launch_us = r["ms_per_step"] * 1e3 / len(gemms)
    achieved = r["bytes"] / len(gemms) / (per_launch_us * 1e-6) / 1e9
    fmt = "W4A8-FP8" if w4a8 else "W4A16"
    out = {"metric": f"Qwen3-30B-A3B routed-expert {fmt} decode step: HBM TB/s", "value": r["TB_s"],
           "unit": "TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None,
           "dtype": ("int4-g128 x e4m3 -> fp32 acc (fp8 MFMA)" if w4a8
                     else "int4-g128 x bf16 -> fp32 acc (bf16 MFMA)"),
           "data": "synthetic: weights N(0, 0.02^2), activations N(0, 1), seeded uniform top-8 routing",
           "config": {"workload": "Qwen3-30B-A3B routed experts: 48 layers x {gate_up 2048->1536, "
                                  f"down 768->2048}} x 128 experts, top-8, expert-grouped {fmt}"
                                  + (" incl. per-token e4m3 quantization of each GEMM's rows" if w4a8 else "")
                                  + " (attention, router and shared layers excluded)", "batch": B},
           "by_batch": res,
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": (ops.w4a8_grouped_dynamic_kernel_for(E, B * k, N0, K0) if w4a8
                                   else "w4a16_grouped_kernel") + " per GEMM (96 per step)",
                        "avg_launch_us": round(per_launch_us, 3)}}
    if not args.no_cpu_baseline:
        sec, threads = cpu_baseline_moe(B, w4a8)
        out["cpu_baseline"] = {"value": round(r["bytes"] / sec / 1e12, 6), "unit": "TB/s", "cores": threads,
                               "kind": "oracle", "seconds_per_step": round(sec, 2),
                               "sample": f"B={B}: layer 0, both grouped GEMMs over the first 16 experts "
                                         f"with rows (" + ("per-token e4m3 quantization, " if w4a8 else "")
                                         + "fp32 dequant + fp64 matmul per expert), scaled to all "
                                         f"experts with rows and x48 layers"}
    print(json.dumps(out), flush=True)


def run_70b(args, torch, ops, synth):
    batches = [1, 8, 64, 256]
    stack = Stack(ops, synth, torch, "70b", batches)
    res = {}
    for B in batches:
        g = graph_of(torch, lambda: stack.step(B))
        ms = time_graph(torch, g, args.steps, args.warmup)
        checked = stack.check_outputs(B, g)
        del g
        res[str(B)] = {"ms_per_step": round(ms, 4),
                       "TB_s": round(stack.bytes(B) / (ms * 1e-3) / 1e12, 3),
                       "mfma_frac": round(stack.flops(B) / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
                       "outputs_checked": checked}
        print(f"[bench] 70b B={B}: {res[str(B)]}", file=sys.stderr, flush=True)
    out = {"metric": "Llama-3-70B W4A16 decode-step ms vs batch (one GPU)", "value": res["1"]["TB_s"],
           "unit": "TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": res["1"]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int4-g128 x bf16 -> fp32 acc (bf16 MFMA)", "data": "synthetic",
           "config": {"workload": "Llama-3-70B decode linear stack, W4A16 g128, 321 GEMMs", "batch": 1},
           "by_batch": res}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the fused dequantize-and-multiply path on one MI355X.

Headline (one JSON line): decode (M = 1) weight GB/s over Llama-3-70B-shaped
decoder layers -- q, k, v, o, gate, up, down at 64x128 blocks with bitwidths
from {1,2,3,4,6,8} (mean 2.1) -- against the 8 TB/s HBM peak.  Projections
that read the same input are packed as one matrix, as serving stacks do:
q|k|v (10240 x 8192) and gate|up (57344 x 8192), so a layer is four dependent
launches (qkv, o, gate_up, down).  One step is one token through a stack of
three distinct layer copies whose packed weights (756 MB) exceed the 256 MiB
Infinity Cache, so every weight byte comes from HBM.  The step is replayed
from a HIP graph of its 12 launches.

Also reported: p10/p50/p90 of single step replays, each launch group alone
(a graph of that group's launches), the same step as one library graph, the
70B layer at M = 8 and 32, the Llama-3-8B layer at M = 1 and 8, the same 8B
shapes with uniform 3- and 4-bit bitmaps (the cost of mixing bitwidths), one
4096 x 4096 matrix at M = 1, the M = 2048 prefill GEMM (TFLOP/s against the
2.5 PFLOP/s fp16 dense peak) with an fp16 library GEMM on the dequantized
weights for context, the same matrices at M = 64 ... 1024 (K split), the
W4.4A8 layer (M = 32 ... 4096) and its down-projection shape 8192 x 28672
at M = 1 ... 256 (K split), and the oracle timed on the host cores over one
copy of the headline layer (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--extras a,b,...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
LAYER_COPIES_8B = 8       # 8 x 91.5 MB > 512 MiB
LAYER_COPIES_70B = 3      # 3 x 252 MB > 512 MiB


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode1_llama3_70b_layer_m1.md")
DECODE_SOURCES = [os.path.join(ROOT, "gemm_block_bit_amd", "csrc", f) for f in ("decode.hip", "decode_common.h")]


def decode_source_digest():
    """sha256 over the decode kernel's sources (decode.hip, then decode_common.h)."""
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed FETCH_SIZE / WRITE_SIZE
    profile, or None when the decode kernel's sources have changed since."""
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if ":" in line and line.startswith(("traffic_bytes_per_launch", "decode_source_sha256")):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("decode_source_sha256") != decode_source_digest():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# extra workloads after the headline, in run order
EXTRAS = ("llama3_70b_batch", "llama3_8b", "mixed_vs_uniform", "blocks_64x64", "linear_4096", "prefill", "w44a8")


def gpu_max_clock_mhz():
    """The GPU agent's maximum engine clock as rocminfo reports it (None if
    rocminfo is unavailable); the peaks used here are the published figures,
    which assume 2400 MHz on 256 CUs."""
    import subprocess
    if any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ):
        return None   # under a profiler, whose library has already opened the GPU in this process
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    gpu = False
    for line in out.splitlines():
        line = line.strip()
        if line.startswith("Name:") and "gfx" in line:
            gpu = True
        elif gpu and line.startswith("Max Clock Freq. (MHz):"):
            try:
                return int(line.split(":")[1].split()[0])
            except (IndexError, ValueError):
                return None
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_bytes(bits: np.ndarray, block_cols: int = 128) -> int:
    """Algorithmic bytes of one packed matrix: codes (1024 b per 64x128
    block, 512 b per 64x64 block), 256 B of fp16 scale/zero per block, 1 B
    bitwidth and 4 B offset per block (+4)."""
    nblk = bits.size
    return 8 * block_cols * int(bits.astype(np.int64).sum()) + 256 * nblk + nblk + 4 * (nblk + 1)


class DecodeLayerSet:
    """R copies of one decoder layer's packed launch groups on the GPU, with
    their activations, outputs and one shared split-K workspace."""

    def __init__(self, torch, gbb, synth, gen, copies, M, dev, keep_host=False, block_cols=128):
        self.torch, self.gbb = torch, gbb
        self.M = M
        self.block_cols = block_cols
        host = []
        for name, idx in synth.LAYER_LAUNCH_GROUPS:
            N, K, W, bits = synth.stacked_group(gen, idx)
            img, _, _ = gbb.pack_blocks(W, bits, block_cols=block_cols)
            host.append((name, (N, K), img, bits))
            del W
        self.images = [[torch.from_numpy(img).to(dev) for (_, _, img, _) in host] for _ in range(copies)]
        self.shapes = [shape for (_, shape, _, _) in host]
        self.names = [name for (name, _, _, _) in host]
        self.bytes = [weight_bytes(b, block_cols) for (_, _, _, b) in host]
        self.layer_bytes = sum(self.bytes)
        nblk = sum(b.size for (_, _, _, b) in host)
        self.mean_bits = float(sum(int(b.astype(np.int64).sum()) for (_, _, _, b) in host)) / nblk
        self.copies = copies
        self.host = host if keep_host else None
        g = np.random.default_rng(7)
        self.x = [torch.from_numpy(g.standard_normal((M, K)).astype(np.float16)).to(dev) for (_, K) in self.shapes]
        self.y = [torch.empty((M, N), dtype=torch.float16, device=dev) for (N, _) in self.shapes]
        ws = max(self._workspace(N, K, M) for (N, K) in self.shapes)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        # raw arguments for direct C calls (no per-call Python marshalling)
        self.fn = gbb.lib().gbb_gemm_mixed_w if block_cols == 128 else gbb.lib().gbb_gemm_mixed_w_64x64

    def _workspace(self, N, K, M):
        if self.block_cols == 128:
            return self.gbb.gemm_mixed_w_workspace(N, K, M)
        return self.gbb.gemm_mixed_w_64x64_workspace(N, K, M)

    def with_batch(self, M, seed):
        """The same packed layers with new activations, outputs and workspace
        for a batch of M tokens (the images are shared, not copied)."""
        torch, gbb = self.torch, self.gbb
        other = DecodeLayerSet.__new__(DecodeLayerSet)
        other.__dict__.update(self.__dict__)
        other.M = M
        dev = self.images[0][0].device
        g = np.random.default_rng(seed)
        other.x = [torch.from_numpy(g.standard_normal((M, K)).astype(np.float16)).to(dev) for (_, K) in self.shapes]
        other.y = [torch.empty((M, N), dtype=torch.float16, device=dev) for (N, _) in self.shapes]
        ws = max(self._workspace(N, K, M) for (N, K) in self.shapes)
        other.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        return other

    def launches(self):
        for r in range(self.copies):
            for i, (N, K) in enumerate(self.shapes):
                yield r, i, N, K

    def launch(self, r, i, stream_handle):
        N, K = self.shapes[i]
        st = self.fn(self.images[r][i].data_ptr(), N, K, self.x[i].data_ptr(), self.y[i].data_ptr(), self.M,
                     self.ws.data_ptr(), self.ws.numel(), stream_handle)
        if st:
            raise RuntimeError(self.gbb.lib().gbb_last_error().decode())

    def step(self, stream_handle):
        for r, i, _, _ in self.launches():
            self.launch(r, i, stream_handle)

    def group_step(self, i, stream_handle):
        """Launch group i of every copy."""
        for r in range(self.copies):
            self.launch(r, i, stream_handle)


GRAPH_MAX_STEPS = 64    # steps captured in one graph
SETTLE_S = 0.25         # seconds of untimed replays before the warmup steps


def time_graph(torch, fn, steps, warmup):
    """Seconds per call of fn() (one step) in HIP graphs: consecutive steps
    are captured into one graph (up to GRAPH_MAX_STEPS of them), as a
    decoder's whole forward pass would be, so the timed region pays the
    graph-launch boundary once per graph instead of once per step.  The
    graphs are first replayed untimed for SETTLE_S seconds (the GPU clock
    ramps up under load), then exactly `warmup` untimed steps, then exactly
    `steps` timed steps between two events.  Returns (seconds per step, host
    wall seconds per step, a graph of one step)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()          # eager warm run outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    cache = {}

    def graph_of(n):
        if n not in cache:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(n):
                    fn()
            cache[n] = g
        return cache[n]

    def plan(n):   # graphs whose step counts add up to exactly n
        full, rest = divmod(n, GRAPH_MAX_STEPS)
        return [graph_of(GRAPH_MAX_STEPS)] * full + ([graph_of(rest)] if rest else [])

    one = graph_of(1)
    timed = plan(steps)
    warm = plan(warmup)
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        timed[0].replay()
        torch.cuda.synchronize()
    for g in warm:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for g in timed:
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for n in [k for k in cache if k != 1]:
        del cache[n]
    return e0.elapsed_time(e1) / 1e3 / steps, wall / steps, one


def replay_percentiles(torch, graph, n):
    """p10 / p50 / p90 (microseconds) of n single replays of a captured graph,
    each between its own pair of events."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return [round(float(v), 1) for v in np.percentile(t, [10, 50, 90])]


class Rotation:
    """Cycles through equal copies of a device image, one per call."""

    def __init__(self, items):
        self.items, self.i = items, 0

    def next(self):
        self.i = (self.i + 1) % len(self.items)
        return self.items[self.i]


def time_eager(torch, fn, reps, warmup):
    """Seconds per call of fn() from events around reps back-to-back calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def group_graph_times(torch, L, steps, warmup, h):
    """Each launch group alone: a graph of that group's launch in every copy,
    replayed; microseconds and weight GB/s per launch."""
    out = {}
    for i, name in enumerate(L.names):
        sec, _, g = time_graph(torch, lambda i=i: L.group_step(i, h()), steps, warmup)
        del g
        us = sec * 1e6 / L.copies
        out[name] = {"N": L.shapes[i][0], "K": L.shapes[i][1], "us": round(us, 2), "MB": round(L.bytes[i] / 1e6, 2),
                     "GBps": round(L.bytes[i] / us / 1e3, 1),
                     "frac_hbm": round(L.bytes[i] / us / 1e3 / HBM_PEAK_GBS, 3)}
    return out


def library_graph_us(torch, gbb, L, steps, warmup):
    """The step as library graphs (gbb_graph_create over its launches, up to
    GRAPH_MAX_STEPS steps per graph, as in time_graph): microseconds per
    step."""
    reps = min(steps, GRAPH_MAX_STEPS)
    lg = gbb.Graph([(L.images[r][i], N, K, L.x[i], L.y[i]) for r, i, N, K in L.launches()] * reps)
    n = max(1, steps // reps)
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        lg.launch()
        torch.cuda.synchronize()
    for _ in range(max(1, warmup // reps)):
        lg.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        lg.launch()
    e1.record()
    torch.cuda.synchronize()
    lg.close()
    return e0.elapsed_time(e1) * 1e3 / (n * reps)


def grouped_step(torch, gbb, L, steps, warmup):
    """The step's products as independent problems in ONE grouped launch
    (gbb_gemm_mixed_w_batched; every product gets its own output): weight
    GB/s of a graph replaying it.  This ignores the dependencies between a
    layer's products, so it is a measure of the grouped launch, not of a
    decoder step."""
    ys = [torch.empty((L.M, N), dtype=torch.float16, device=L.x[i].device) for _, i, N, _ in L.launches()]
    b = gbb.Batched([(L.images[r][i], N, K, L.x[i], y) for (r, i, N, K), y in zip(L.launches(), ys)])
    sec, _, g = time_graph(torch, b.launch, steps, warmup)
    del g
    return L.layer_bytes * L.copies / sec / 1e9, sec * 1e6


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline only (no extra workloads, no cpu baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated extra workloads to run after the headline (default: all of "
                         + ", ".join(EXTRAS) + ")")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB elementwise copy (read 256 MiB, write 256 MiB) five times, "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters of a profiled run")
    args = ap.parse_args()
    want = set(w for w in args.extras.split(",") if w)
    if want - set(EXTRAS):
        ap.error("unknown extra workload(s): " + ", ".join(sorted(want - set(EXTRAS))))
    if args.quick:
        want = set()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the fused dequant-GEMM path has no multi-GPU component here "
              "(the path would shard by output rows or by K; that is not built here); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    max_clock = gpu_max_clock_mhz()   # before this process opens the GPU

    import torch

    import gemm_block_bit_amd as gbb
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} CUs={props.multi_processor_count}")

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("calibration copy: 5 x (read 268435456 B, write 268435456 B)")
        del src, dst

    device_info = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count,
                   "memory_GiB": round(props.total_memory / 2**30, 1),
                   "max_clock_MHz": max_clock}
    h = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731

    # ---------------- headline: Llama-3-70B layers, decode M = 1 ----------------
    log("packing Llama-3-70B-shaped layer (qkv, o, gate_up, down)")
    L70 = DecodeLayerSet(torch, gbb, synth, synth.llama3_70b_proj, LAYER_COPIES_70B, 1, dev,
                         keep_host=not args.quick and not args.no_cpu_baseline)
    log(f"layer weight bytes {L70.layer_bytes / 1e6:.1f} MB x {L70.copies} copies, mean {L70.mean_bits:.3f} bits")
    sec, wall, g70 = time_graph(torch, lambda: L70.step(h()), args.steps, args.warmup)
    total_bytes = L70.layer_bytes * L70.copies
    value = total_bytes / sec / 1e9
    log(f"decode M=1: {sec * 1e6:.1f} us/step, {value:.0f} GB/s")
    step_pct = replay_percentiles(torch, g70, args.steps)
    del g70
    # each launch group on its own, and the step as one library graph
    per_group = group_graph_times(torch, L70, args.steps, args.warmup, h)
    log(f"per launch group: {per_group}")
    lib_us = library_graph_us(torch, gbb, L70, args.steps, args.warmup)
    log(f"the same step as one library graph: {lib_us:.1f} us")
    grp_gbs, grp_us = grouped_step(torch, gbb, L70, args.steps, args.warmup)
    log(f"the step's 12 products as one grouped launch (independent): {grp_us:.1f} us, {grp_gbs:.0f} GB/s")

    # The graph replays the step's launches back to back on this stream, so
    # step time / launches is the mean duration per launch (gaps included)
    n_launch = L70.copies * len(L70.shapes)
    mean_us = sec * 1e6 / n_launch
    mean_bytes = float(np.mean(L70.bytes))
    achieved = mean_bytes / mean_us / 1e3
    extra = {"per_launch_group_m1_graph": per_group, "graph_step_us": round(sec * 1e6, 1),
             "one_step_graph_replay_us_p10_p50_p90": step_pct, "library_graph_step_us": round(lib_us, 1),
             "grouped_launch_independent_products": {"us": round(grp_us, 1), "GBps": round(grp_gbs, 1),
                                                     "frac_hbm": round(grp_gbs / HBM_PEAK_GBS, 3)},
             "host_wall_us_per_step": round(wall * 1e6, 1), "layer_MB": round(L70.layer_bytes / 1e6, 1),
             "mean_bits": round(L70.mean_bits, 3), "device": device_info}

    if not args.quick:
        # context: a plain device-to-device copy of 1 GiB (read + write bytes)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        extra["copy_1GiB_GBps"] = round(2 * 10 * (1 << 30) / (c0.elapsed_time(c1) / 1e3) / 1e9, 1)
        log(f"device copy of 1 GiB: {extra['copy_1GiB_GBps']} GB/s (read + write)")
        del src, dst
        torch.cuda.empty_cache()

    if "llama3_70b_batch" in want:
        # ---------------- the same 70B layers at M = 8 and 32 ----------------
        for M in (8, 32):
            Lm = L70.with_batch(M, M)
            sm, _, _ = time_graph(torch, lambda: Lm.step(h()), max(10, args.steps // 2), args.warmup)
            extra[f"llama3_70b_decode_m{M}_GBps"] = round(total_bytes / sm / 1e9, 1)
            log(f"70B decode M={M}: {total_bytes / sm / 1e9:.0f} GB/s")
            del Lm
    host70 = L70.host
    want_cpu = not args.quick and not args.no_cpu_baseline
    oracle_inputs = {}   # host inputs of the extras, for the oracle timed beside them
    del L70
    torch.cuda.empty_cache()

    if "llama3_8b" in want:
        # ---------------- Llama-3-8B layers, decode M = 1 and 8 ----------------
        log("packing Llama-3-8B-shaped layer (qkv, o, gate_up, down)")
        L8 = DecodeLayerSet(torch, gbb, synth, synth.llama3_8b_proj, LAYER_COPIES_8B, 1, dev, keep_host=want_cpu)
        b8 = L8.layer_bytes * L8.copies
        s8, _, _ = time_graph(torch, lambda: L8.step(h()), args.steps, args.warmup)
        v8 = b8 / s8 / 1e9
        e8 = {"GBps": round(v8, 1), "frac_hbm": round(v8 / HBM_PEAK_GBS, 3), "graph_step_us": round(s8 * 1e6, 1),
              "layers_per_step": L8.copies, "layer_MB": round(L8.layer_bytes / 1e6, 1),
              "mean_bits": round(L8.mean_bits, 3),
              "per_launch_group_m1_graph": group_graph_times(torch, L8, args.steps, args.warmup, h),
              "library_graph_step_us": round(library_graph_us(torch, gbb, L8, args.steps, args.warmup), 1)}
        g8, g8us = grouped_step(torch, gbb, L8, args.steps, args.warmup)
        e8["grouped_launch_independent_products"] = {"us": round(g8us, 1), "GBps": round(g8, 1),
                                                     "frac_hbm": round(g8 / HBM_PEAK_GBS, 3)}
        log(f"8B: the step's 32 products as one grouped launch: {g8us:.1f} us, {g8:.0f} GB/s")
        log(f"8B decode M=1: {v8:.0f} GB/s; per group {e8['per_launch_group_m1_graph']}")
        L8b = L8.with_batch(8, 8)
        s8b, _, _ = time_graph(torch, lambda: L8b.step(h()), args.steps, args.warmup)
        e8["decode_m8_GBps"] = round(b8 / s8b / 1e9, 1)
        log(f"8B decode M=8: {b8 / s8b / 1e9:.0f} GB/s")
        del L8b
        extra["llama3_8b_layer_m1"] = e8
        if want_cpu:
            oracle_inputs["llama3_8b_layer"] = (L8.host, {1: s8 / L8.copies, 8: s8b / L8.copies})

        if "mixed_vs_uniform" in want:
            # ------- the same shapes with uniform 3- and 4-bit bitmaps, M = 1 -------
            # The mixed layers' GB/s against uniform layers' GB/s interpolated to
            # the same mean bitwidth: the cost of mixing bitwidths in one launch.
            uni = {}
            for b in (3, 4):
                def gen_uniform(i, b=b):
                    p, W, _ = synth.llama3_8b_proj(i)
                    return p, W, synth.uniform_bitmap(p.N, p.K, b)
                log(f"packing Llama-3-8B-shaped layer with uniform {b}-bit blocks")
                Lu = DecodeLayerSet(torch, gbb, synth, gen_uniform, LAYER_COPIES_8B, 1, dev)
                su, _, _ = time_graph(torch, lambda: Lu.step(h()), args.steps, args.warmup)
                uni[b] = Lu.layer_bytes * Lu.copies / su / 1e9
                log(f"uniform {b}-bit decode M=1: {uni[b]:.0f} GB/s")
                del Lu
                torch.cuda.empty_cache()
            ref = uni[3] + (L8.mean_bits - 3.0) * (uni[4] - uni[3])
            extra["mixed_vs_uniform_8b_m1"] = {
                "uniform3_GBps": round(uni[3], 1), "uniform4_GBps": round(uni[4], 1),
                "mixed_GBps": round(v8, 1), "mixed_mean_bits": round(L8.mean_bits, 3),
                "mixed_over_uniform_at_same_bits": round(v8 / ref, 3)}
            log(f"mixed / uniform at {L8.mean_bits:.2f} bits: {v8 / ref:.3f}")

        if "blocks_64x64" in want:
            # ------- the same layer with 64x64 blocks at the same mean bits -------
            # Same weights and bit quotas over twice the blocks: a 64x64 block
            # carries the same 256 B of scales and zeros for half the codes,
            # so the step reads more bytes; the comparison is step time and
            # GB/s at M = 1 and 8.
            log("packing Llama-3-8B-shaped layer with 64x64 blocks")
            L64 = DecodeLayerSet(torch, gbb, synth, synth.llama3_8b_proj64, LAYER_COPIES_8B, 1, dev, block_cols=64)
            b64 = L64.layer_bytes * L64.copies
            s64, _, _ = time_graph(torch, lambda: L64.step(h()), args.steps, args.warmup)
            L64b = L64.with_batch(8, 8)
            s64b, _, _ = time_graph(torch, lambda: L64b.step(h()), args.steps, args.warmup)
            extra["blocks_64x64_8b"] = {
                "mean_bits": round(L64.mean_bits, 3), "layer_MB": round(L64.layer_bytes / 1e6, 1),
                "m1": {"GBps": round(b64 / s64 / 1e9, 1), "graph_step_us": round(s64 * 1e6, 1),
                       "frac_hbm": round(b64 / s64 / 1e9 / HBM_PEAK_GBS, 3)},
                "m8": {"GBps": round(b64 / s64b / 1e9, 1), "graph_step_us": round(s64b * 1e6, 1)},
                "blocks_64x128_same_layer": {"mean_bits": round(L8.mean_bits, 3),
                                             "layer_MB": round(L8.layer_bytes / 1e6, 1),
                                             "m1": {"GBps": round(v8, 1), "graph_step_us": round(s8 * 1e6, 1)},
                                             "m8": {"GBps": e8["decode_m8_GBps"],
                                                    "graph_step_us": round(s8b * 1e6, 1)}}}
            log(f"8B 64x64 blocks: M=1 {b64 / s64 / 1e9:.0f} GB/s ({s64 * 1e6:.1f} us/step), "
                f"M=8 {b64 / s64b / 1e9:.0f} GB/s ({s64b * 1e6:.1f} us/step)")
            del L64, L64b
            torch.cuda.empty_cache()
            # prefill, M = 2048, on the gate projection (14336 x 4096) in both formats
            pf = {}
            for bc, gen in ((128, synth.llama3_8b_proj), (64, synth.llama3_8b_proj64)):
                p, W, bits = gen(4)
                img, _, _ = gbb.pack_blocks(W, bits, block_cols=bc)
                del W
                imgd = torch.from_numpy(img).to(dev)
                rot = Rotation([imgd] + [imgd.clone() for _ in range(11)])   # 12 copies > 256 MiB
                x = torch.from_numpy(synth.prefill_x(2048, p.K, 4)).to(dev)
                y = torch.empty((2048, p.N), dtype=torch.float16, device=dev)
                call = gbb.gemm_mixed_w if bc == 128 else gbb.gemm_mixed_w_64x64
                sp = time_eager(torch, lambda: call(rot.next(), p.N, p.K, x, out=y), 30, 30)
                pf[f"blocks_64x{bc}"] = {"ms": round(sp * 1e3, 3),
                                         "TFLOPs": round(2.0 * 2048 * p.N * p.K / sp / 1e12, 1)}
                del rot, imgd, x, y
                torch.cuda.empty_cache()
            extra["blocks_64x64_8b"]["prefill_m2048_gate_14336x4096"] = pf
            log(f"8B gate prefill M=2048: {pf}")
        del L8
        torch.cuda.empty_cache()

    if "linear_4096" in want:
        # ---------------- one 4096 x 4096 matrix, M = 1 ----------------
        W, bits, x1 = synth.linear_4096()
        img, _, _ = gbb.pack_blocks(W, bits)
        del W
        d = torch.from_numpy(img).to(dev)
        lin = [d] + [d.clone() for _ in range(79)]   # 80 x 7.0 MB > 512 MiB
        xd = torch.from_numpy(x1).to(dev)
        yd = torch.empty((1, 4096), dtype=torch.float16, device=dev)
        wsl = torch.zeros(max(gbb.gemm_mixed_w_workspace(4096, 4096, 1), 256), dtype=torch.uint8, device=dev)
        fn = gbb.lib().gbb_gemm_mixed_w

        def lin_step():
            for im in lin:
                if fn(im.data_ptr(), 4096, 4096, xd.data_ptr(), yd.data_ptr(), 1, wsl.data_ptr(), wsl.numel(), h()):
                    raise RuntimeError(gbb.lib().gbb_last_error().decode())
        sl1, _, _ = time_graph(torch, lin_step, max(10, args.steps // 2), args.warmup)
        lb = weight_bytes(bits) * len(lin)
        extra["linear_4096_m1"] = {"us_per_launch": round(sl1 * 1e6 / len(lin), 2), "GBps": round(lb / sl1 / 1e9, 1),
                                   "weight_MB": round(weight_bytes(bits) / 1e6, 2)}
        log(f"4096x4096 M=1: {sl1 * 1e6 / len(lin):.2f} us/launch, {lb / sl1 / 1e9:.0f} GB/s")
        if want_cpu:
            oracle_inputs["linear_4096_m1"] = (img, bits, x1, sl1 / len(lin))
        del lin, d
        torch.cuda.empty_cache()

    roof2048 = None
    if "prefill" in want:
        # ---------------- prefill M = 2048 on the 70B MLP ----------------
        pre = {}
        for i in range(2):
            p, W, bits = synth.prefill_70b_mlp(i)
            img, _, _ = gbb.pack_blocks(W, bits)
            del W
            imgd = torch.from_numpy(img).to(dev)
            # Six rotating copies (~590 MB) keep the weights out of the
            # 256 MiB last-level cache between calls.
            rot = Rotation([imgd] + [imgd.clone() for _ in range(5)])
            x = torch.from_numpy(synth.prefill_x(2048, p.K, i)).to(dev)
            y = torch.empty((2048, p.N), dtype=torch.float16, device=dev)
            fl = 2.0 * 2048 * p.N * p.K
            # matrix-core-bound launches reach steady clocks only after some
            # tens of milliseconds of such work: warm up for ~30 launches
            sp = time_eager(torch, lambda: gbb.gemm_mixed_w(rot.next(), p.N, p.K, x, out=y), 30, 30)
            # moderate batches: the library's own choice (the K-split prefill
            # kernel, or 32-token decode chunks where even the split grid
            # would leave most compute units idle), against the prefill
            # kernel with no K split (a workspace too small for one)
            mid = {}
            no_split_ws = torch.zeros(256, dtype=torch.uint8, device=dev)
            for Mm in (64, 128, 256, 512, 1024):
                xm = x[:Mm].contiguous()
                ym = y[:Mm]
                sa = time_eager(torch, lambda: gbb.gemm_mixed_w(rot.next(), p.N, p.K, xm, out=ym), 30, 12)
                sf = time_eager(torch, lambda: gbb.gemm_mixed_w_path(rot.next(), p.N, p.K, xm, 2, out=ym,
                                                                     workspace=no_split_ws), 30, 12)
                flm = 2.0 * Mm * p.N * p.K
                mid[f"M{Mm}"] = {"us": round(sa * 1e6, 1), "TFLOPs": round(flm / sa / 1e12, 1),
                                 "prefill_kernel_no_k_split_us": round(sf * 1e6, 1),
                                 "workspace_MB": round(gbb.gemm_mixed_w_workspace(p.N, p.K, Mm) / 1e6, 1)}
                log(f"prefill {p.name} M={Mm}: {sa * 1e6:.1f} us, {flm / sa / 1e12:.0f} TFLOP/s "
                    f"(no K split {sf * 1e6:.1f} us)")
            del no_split_ws
            del rot
            w32, w16 = gbb.dequant(imgd, p.N, p.K)
            del w32
            sl = time_eager(torch, lambda: torch.matmul(x, w16.t(), out=y), 30, 30)
            pre[p.name] = {"N": p.N, "K": p.K, "ms": round(sp * 1e3, 3), "TFLOPs": round(fl / sp / 1e12, 1),
                           "frac_fp16_peak": round(fl / sp / 1e12 / FP16_PEAK_TFLOPS, 3),
                           "fp16_library_gemm_on_dequantized_TFLOPs": round(fl / sl / 1e12, 1),
                           "moderate_batches": mid}
            log(f"prefill {p.name}: {fl / sp / 1e12:.0f} TFLOP/s (library fp16 GEMM {fl / sl / 1e12:.0f})")
            if want_cpu:
                oracle_inputs.setdefault("prefill_m2048", []).append(
                    (p.name, p.N, p.K, img, synth.prefill_x(ORACLE_PREFILL_TOKENS, p.K, i), sp))
            del imgd, x, y, w16
            torch.cuda.empty_cache()
        extra["prefill_m2048_70b_mlp"] = pre
        fl_all = sum(2.0 * 2048 * v["N"] * v["K"] for v in pre.values())
        ms_all = sum(v["ms"] for v in pre.values())
        roof2048 = {"bound": "mfma", "achieved": round(fl_all / (ms_all * 1e-3) / 1e12, 1), "peak": FP16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(fl_all / (ms_all * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 3),
                    "traffic": None, "kernel": "prefill_kernel",
                    "workload": "M=2048 x Llama-3-70B MLP (28672x8192 gate and 8192x28672 down), 2*M*N*K flops "
                                "over both launches"}

    if "w44a8" in want:
        # ---------------- W4.4A8 28672 x 8192 ----------------
        W, rows8 = synth.w44a8_28672x8192()
        img, _, _ = gbb.pack_w48(W, rows8)
        del W
        imgd = torch.from_numpy(img).to(dev)
        # Four rotating copies (535 MB) keep the weights out of the 256 MiB
        # last-level cache between calls.
        rot = Rotation([imgd] + [imgd.clone() for _ in range(3)])
        w48 = {}
        for M in (32, 96, 512, 4096):
            x = torch.from_numpy(synth.activations(M, 8192, synth.WL_W44A8, 0)).to(dev)
            xq, xs = gbb.quant_act_i8(x)
            y = torch.empty((M, 28672), dtype=torch.float16, device=dev)
            # warm up for ~30 ms of launches (at least 4, at most 200)
            sw = time_eager(torch, lambda: gbb.gemm_w48a8(rot.next(), 28672, 8192, rows8.size, xq, xs, out=y), 30,
                            min(200, max(4, int(30e-3 / (2.0 * M * 28672 * 8192 / 1e15)))))
            ops = 2.0 * M * 28672 * 8192
            w48[f"M{M}"] = {"us": round(sw * 1e6, 1), "TOPs": round(ops / sw / 1e12, 1),
                            "frac_int8_peak": round(ops / sw / 1e12 / INT8_PEAK_TOPS, 3),
                            "weight_GBps": round(img.size / sw / 1e9, 1)}
            log(f"w44a8 M={M}: {w48[f'M{M}']}")
            if want_cpu:
                oracle_inputs.setdefault("w44a8", {"img": img})[M] = sw
        extra["w44a8_28672x8192"] = w48
        # the same layer with activation scales per group of 128 columns (the
        # granularity the MixLLM page benchmarks)
        w48g = {}
        for M in (1, 32, 512):
            x = torch.from_numpy(synth.activations(M, 8192, synth.WL_W44A8, 0)).to(dev)
            xq, xs = gbb.quant_act_i8(x, 128)
            y = torch.empty((M, 28672), dtype=torch.float16, device=dev)
            sw = time_eager(torch, lambda: gbb.gemm_w48a8(rot.next(), 28672, 8192, rows8.size, xq, xs, 128, out=y), 30,
                            min(200, max(4, int(30e-3 / (2.0 * M * 28672 * 8192 / 1e15)))))
            ops = 2.0 * M * 28672 * 8192
            w48g[f"M{M}"] = {"us": round(sw * 1e6, 1), "TOPs": round(ops / sw / 1e12, 1),
                             "weight_GBps": round(img.size / sw / 1e9, 1)}
            log(f"w44a8 group-128 activation scales M={M}: {w48g[f'M{M}']}")
        extra["w44a8_28672x8192_group128_act_scales"] = w48g
        del imgd, rot
        torch.cuda.empty_cache()

        # ---------------- W4.4A8 8192 x 28672 (down projection), small batches ----------------
        # 129 row blocks for 256 CUs: the stream kernel splits K (6 segments
        # for the 8-bit row blocks, 3 for the 4-bit ones), and at M = 256 the
        # tile kernel (2 and 4 segments), against the same kernels unsplit
        W, rows8 = synth.w44a8_8192x28672()
        img, _, _ = gbb.pack_w48(W, rows8)
        del W
        imgd = torch.from_numpy(img).to(dev)
        rot = Rotation([imgd] + [imgd.clone() for _ in range(3)])
        down = {}
        for M in (1, 16, 32, 64, 96, 256):
            x = torch.from_numpy(synth.activations(M, 28672, synth.WL_W44A8, 2)).to(dev)
            xq, xs = gbb.quant_act_i8(x)
            y = torch.empty((M, 8192), dtype=torch.float16, device=dev)
            ss = time_eager(torch, lambda: gbb.gemm_w48a8(rot.next(), 8192, 28672, rows8.size, xq, xs, out=y), 30, 30)
            su = time_eager(torch, lambda: gbb.gemm_w48a8(rot.next(), 8192, 28672, rows8.size, xq, xs, out=y,
                                                          split=False), 30, 30)
            down[f"M{M}"] = {"us": round(ss * 1e6, 1), "weight_GBps": round(img.size / ss / 1e9, 1),
                             "frac_hbm": round(img.size / ss / 1e9 / HBM_PEAK_GBS, 3),
                             "no_k_split_us": round(su * 1e6, 1),
                             "workspace_MB": round(gbb.gemm_w48a8_workspace(8192, 28672, rows8.size, M) / 1e6, 2)}
            log(f"w44a8 8192x28672 M={M}: {down[f'M{M}']}")
        extra["w44a8_8192x28672"] = down
        del imgd, rot
        torch.cuda.empty_cache()

    cpu = None
    if want_cpu:
        cpu = cpu_baseline(host70)
        extra["cpu_baseline_one_thread_o_proj_GBps"] = cpu_baseline_one_thread(host70)
        extra["oracle_beside_extras"] = oracle_beside(oracle_inputs)

    out = {
        "metric": "fused dequant-GEMM: weight GB/s (%HBM peak) at M=1; TFLOP/s (%MFMA) at M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded random weights and activations of Llama-3-70B layer shapes)",
        "config": {"workload": "llama3_70b_layer_decode_m1", "layers_per_step": LAYER_COPIES_70B,
                   "projections": "q,k,v,o,gate,up,down", "launches_per_layer": "qkv,o,gate_up,down",
                   "M": 1, "block": "64x128", "bits": "{1,2,3,4,6,8} mean 2.10", "group": 128,
                   "weight_MB_per_step": round(total_bytes / 1e6, 1), "parallelism": "single GPU"},
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 3), "traffic": measured_traffic(),
                     "kernel": "decode1_kernel<4>", "mean_launch_us": round(mean_us, 3),
                     "mean_algorithmic_bytes_per_launch": round(mean_bytes)},
        "roofline_m2048": roof2048,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(host):
    """The oracle as it stands -- its own unpacker, exact fp32 dequant and an
    fp64 product -- over one copy of the headline layer (its four packed
    launch groups, M = 1), on the host's cores."""
    from threadpoolctl import threadpool_info

    from oracle import blockquant as bq
    from oracle import image as oimg

    log("cpu baseline: oracle over one Llama-3-70B-shaped layer at M=1")
    total_bytes = 0
    t = 0.0
    for (name, (N, K), img, bits) in host:
        x = np.random.default_rng(7).standard_normal((1, K)).astype(np.float16)
        t0 = time.perf_counter()
        d = oimg.read_block_image(img)
        w = bq.dequant_fp32(d["q"], d["s16"], d["z16"])
        bq.gemm_fp64(x, w)
        t += time.perf_counter() - t0
        total_bytes += weight_bytes(bits)
        del d, w
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    return {"value": round(total_bytes / t / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one copy of the headline layer (q|k|v, o, gate|up, down; {total_bytes / 1e6:.1f} MB "
                      f"packed) at M=1: oracle unpack + fp32 dequant + fp64 GEMV, {t:.1f} s"}


def cpu_baseline_one_thread(host):
    """The same oracle on one thread (BLAS limited to one), over the o
    projection only, for context next to the multi-thread figure."""
    from threadpoolctl import threadpool_limits

    from oracle import blockquant as bq
    from oracle import image as oimg

    name, (N, K), img, bits = [hh for hh in host if hh[0] == "o"][0]
    x = np.random.default_rng(7).standard_normal((1, K)).astype(np.float16)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        d = oimg.read_block_image(img)
        w = bq.dequant_fp32(d["q"], d["s16"], d["z16"])
        bq.gemm_fp64(x, w)
        t = time.perf_counter() - t0
    return round(weight_bytes(bits) / t / 1e9, 3)


ORACLE_PREFILL_TOKENS = 256      # prefill: the oracle's product runs on this many of the 2048 tokens
ORACLE_W48_SAMPLE = (256, 2048)  # W4.4A8: at most this many tokens x rows in the oracle's products


def oracle_beside(inputs):
    """The oracle timed beside each extra on its own inputs (host cores):
    its unpack of the packed image and exact fp32 dequant (or, for W4.4A8,
    its image reader and activation quantization) always in full, and its
    fp64 / exact-integer products in full or on a stated sample scaled to
    the whole call.  Each entry gives the oracle's seconds per call, the
    GPU's, and their ratio."""
    from oracle import blockquant as bq
    from oracle import image as oimg
    from oracle import w48 as ow

    out = {}

    def entry(t_oracle, t_gpu, sample):
        return {"oracle_s": round(t_oracle, 3), "gpu_s": float(f"{t_gpu:.4g}"),
                "gpu_speedup": round(t_oracle / t_gpu, 1), "sample": sample}

    if "linear_4096_m1" in inputs:
        img, bits, x1, t_gpu = inputs["linear_4096_m1"]
        t0 = time.perf_counter()
        d = oimg.read_block_image(img)
        bq.gemm_fp64(x1, bq.dequant_fp32(d["q"], d["s16"], d["z16"]))
        out["linear_4096_m1"] = entry(time.perf_counter() - t0, t_gpu, "the whole call")
        log(f"oracle beside 4096x4096 M=1: {out['linear_4096_m1']}")
    if "llama3_8b_layer" in inputs:
        host, t_gpu = inputs["llama3_8b_layer"]
        t_deq, t_mm = 0.0, {1: 0.0, 8: 0.0}
        g = np.random.default_rng(7)
        for (name, (N, K), img, bits) in host:
            t0 = time.perf_counter()
            d = oimg.read_block_image(img)
            w = bq.dequant_fp32(d["q"], d["s16"], d["z16"])
            t_deq += time.perf_counter() - t0
            for M in (1, 8):
                x = g.standard_normal((M, K)).astype(np.float16)
                t0 = time.perf_counter()
                bq.gemm_fp64(x, w)
                t_mm[M] += time.perf_counter() - t0
            del d, w
        for M in (1, 8):
            out[f"llama3_8b_layer_m{M}"] = entry(t_deq + t_mm[M], t_gpu[M],
                                                 "one layer (q|k|v, o, gate|up, down), the whole call")
            log(f"oracle beside 8B layer M={M}: {out[f'llama3_8b_layer_m{M}']}")
    for (name, N, K, img, xs, t_gpu) in inputs.get("prefill_m2048", []):
        t0 = time.perf_counter()
        d = oimg.read_block_image(img)
        w = bq.dequant_fp32(d["q"], d["s16"], d["z16"])
        t_deq = time.perf_counter() - t0
        del d
        t0 = time.perf_counter()
        bq.gemm_fp64(xs, w)
        t_mm = (time.perf_counter() - t0) * (2048 / xs.shape[0])
        del w
        out[f"prefill_m2048_{name}"] = entry(t_deq + t_mm, t_gpu,
                                             f"unpack + dequant in full; the fp64 product on {xs.shape[0]} of "
                                             f"the 2048 tokens, scaled x{2048 // xs.shape[0]}")
        log(f"oracle beside prefill {name}: {out[f'prefill_m2048_{name}']}")
    if "w44a8" in inputs:
        rec = inputs["w44a8"]
        t0 = time.perf_counter()
        qd = oimg.read_w48_image(rec["img"])
        t_read = time.perf_counter() - t0
        N, K = qd["N"], qd["K"]
        Wz4 = qd["q4"].astype(np.int64) - np.repeat(qd["z4"].astype(np.int64), 128, axis=1)
        for M in sorted(k for k in rec if isinstance(k, int)):
            m_s, n_s = min(M, ORACLE_W48_SAMPLE[0]), ORACLE_W48_SAMPLE[1]
            x = synth_activations(M, K)
            t0 = time.perf_counter()
            A_q, s_a = ow.quant_act(x)
            t_q = time.perf_counter() - t0
            n8s = max(1, n_s * qd["n8"] // N)
            t0 = time.perf_counter()
            ow.two_step(A_q[:m_s], s_a[:m_s], qd["q8"][:n8s].astype(np.int64), qd["s8"][:n8s])
            ow.two_step(A_q[:m_s], s_a[:m_s], Wz4[:n_s - n8s], qd["s4"][:n_s - n8s])
            t_mm = (time.perf_counter() - t0) * (M / m_s) * (N / n_s)
            out[f"w44a8_m{M}"] = entry(t_read + t_q + t_mm, rec[M],
                                       f"image read and activation quantization in full; the exact group products "
                                       f"and scaling on {m_s} tokens x {n_s} rows, scaled to {M} x {N}")
            log(f"oracle beside w44a8 M={M}: {out[f'w44a8_m{M}']}")
    return out


def synth_activations(M, K):
    import synth
    return synth.activations(M, K, synth.WL_W44A8, 0)


if __name__ == "__main__":
    main()

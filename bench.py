"""Benchmark of the fused dequantize-and-multiply path on one MI355X.

Headline (one JSON line): decode (M = 1) weight GB/s over Llama-3-8B-shaped
decoder layers -- q, k, v, o, gate, up, down at 64x128 blocks with bitwidths
from {1,2,3,4,6,8} (mean 3.1) -- against the 8 TB/s HBM peak.  Projections
that read the same input are packed as one matrix, as serving stacks do:
q|k|v (6144 x 4096) and gate|up (28672 x 4096), so a layer is four launches
(qkv, o, gate_up, down).  One step is one token through a stack of distinct
layer copies whose packed weights (732 MB) exceed the 256 MiB Infinity
Cache, so every weight byte comes from HBM.  The step is replayed from a HIP
graph of its 32 launches.

Also reported: p10/p50/p90 of single step replays, M = 8 on the same
layers, the same shapes with uniform 3- and 4-bit bitmaps (the cost of
mixing bitwidths), one 4096 x 4096 matrix at M = 1, the 70B-shaped layer at
M = 1, 8 and 32, the M = 2048 prefill GEMM (TFLOP/s against the 2.5 PFLOP/s fp16 dense peak) with
an fp16 library GEMM on the dequantized weights for context, the W4.4A8 layer
(M = 32, 512, 4096) and the oracle timed on the host cores (cpu_baseline).

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
LAYER_COPIES_70B = 3      # 3 x 252 MB


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode1_llama3_8b_layer_m1.md")
DECODE_SOURCE = os.path.join(ROOT, "gemm_block_bit_amd", "csrc", "decode.hip")


def measured_traffic():
    """HBM bytes per decode launch from the committed FETCH_SIZE / WRITE_SIZE
    profile, or None when the decode kernel source has changed since."""
    import hashlib
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if ":" in line and line.startswith(("traffic_bytes_per_launch", "decode_hip_sha256")):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        with open(DECODE_SOURCE, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
        if fields.get("decode_hip_sha256") != digest:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# extra workloads after the headline, in run order
EXTRAS = ("llama3_8b_m8", "mixed_vs_uniform", "linear_4096", "llama3_70b", "prefill", "w44a8")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_bytes(bits: np.ndarray) -> int:
    """Algorithmic bytes of one packed matrix: codes (1024 b per 64x128
    block), 256 B of fp16 scale/zero per block, 1 B bitwidth and 4 B offset
    per block (+4)."""
    nblk = bits.size
    return 1024 * int(bits.astype(np.int64).sum()) + 256 * nblk + nblk + 4 * (nblk + 1)


# launch groups of a decoder layer: projections that share their input are
# stacked along the output rows into one packed matrix
GROUPS = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))


class DecodeLayerSet:
    """R copies of one decoder layer's packed launch groups on the GPU, with
    their activations, outputs and one shared split-K workspace."""

    def __init__(self, torch, gbb, synth, gen, copies, M, dev):
        self.torch, self.gbb = torch, gbb
        self.M = M
        host = []
        for name, idx in GROUPS:
            parts = [gen(i) for i in idx]
            W = np.concatenate([W for (_, W, _) in parts])
            bits = np.concatenate([b for (_, _, b) in parts])
            img, _, _ = gbb.pack_blocks(W, bits)
            host.append((name, W.shape, img, bits))
            del W, parts
        self.images = [[torch.from_numpy(img).to(dev) for (_, _, img, _) in host] for _ in range(copies)]
        self.shapes = [shape for (_, shape, _, _) in host]
        self.names = [name for (name, _, _, _) in host]
        self.bytes = [weight_bytes(b) for (_, _, _, b) in host]
        self.layer_bytes = sum(self.bytes)
        nblk = sum(b.size for (_, _, _, b) in host)
        self.mean_bits = float(sum(int(b.astype(np.int64).sum()) for (_, _, _, b) in host)) / nblk
        self.copies = copies
        g = np.random.default_rng(7)
        self.x = [torch.from_numpy(g.standard_normal((M, K)).astype(np.float16)).to(dev) for (_, K) in self.shapes]
        self.y = [torch.empty((M, N), dtype=torch.float16, device=dev) for (N, _) in self.shapes]
        ws = max(gbb.gemm_mixed_w_workspace(N, K, M) for (N, K) in self.shapes)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        # raw arguments for direct C calls (no per-call Python marshalling)
        self.fn = gbb.lib().gbb_gemm_mixed_w

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
        ws = max(gbb.gemm_mixed_w_workspace(N, K, M) for (N, K) in self.shapes)
        other.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        return other

    def launches(self):
        for r in range(self.copies):
            for i, (N, K) in enumerate(self.shapes):
                yield r, i, N, K

    def step(self, stream_handle, events=None):
        fn, ws = self.fn, self.ws
        for r, i, N, K in self.launches():
            if events is not None:
                events[r][i][0].record()
            st = fn(self.images[r][i].data_ptr(), N, K, self.x[i].data_ptr(), self.y[i].data_ptr(), self.M,
                    ws.data_ptr(), ws.numel(), stream_handle)
            if st:
                raise RuntimeError(self.gbb.lib().gbb_last_error().decode())
            if events is not None:
                events[r][i][1].record()


def time_graph(torch, fn, steps, warmup):
    """Capture fn() in a HIP graph, replay warmup + steps times, return
    seconds per step over the timed replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()          # eager warm run outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3 / steps, wall / steps, graph


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
                   "memory_GiB": round(props.total_memory / 2**30, 1)}

    # ---------------- headline: Llama-3-8B layers, decode M = 1 ----------------
    log("packing Llama-3-8B-shaped layer (qkv, o, gate_up, down)")
    L8 = DecodeLayerSet(torch, gbb, synth, synth.llama3_8b_proj, LAYER_COPIES_8B, 1, dev)
    log(f"layer weight bytes {L8.layer_bytes / 1e6:.1f} MB x {L8.copies} copies")
    h = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731

    sec, wall, g8 = time_graph(torch, lambda: L8.step(h()), args.steps, args.warmup)
    total_bytes = L8.layer_bytes * L8.copies
    value = total_bytes / sec / 1e9
    log(f"decode M=1: {sec * 1e6:.1f} us/step, {value:.0f} GB/s")
    step_pct = replay_percentiles(torch, g8, args.steps)
    del g8

    # the same step as one library graph (gbb_graph_create over the 32 calls)
    lg = gbb.Graph([(L8.images[r][i], N, K, L8.x[i], L8.y[i]) for r, i, N, K in L8.launches()])
    for _ in range(args.warmup):
        lg.launch()
    torch.cuda.synchronize()
    le0, le1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    le0.record()
    for _ in range(args.steps):
        lg.launch()
    le1.record()
    torch.cuda.synchronize()
    lib_graph_us = le0.elapsed_time(le1) * 1e3 / args.steps
    lg.close()
    log(f"the same step as one library graph: {lib_graph_us:.1f} us")

    # per-launch events over the same timed work (eager launches, one stream)
    ng = len(L8.shapes)
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(ng)] for _ in range(L8.copies)]
    durs = np.zeros((args.steps, L8.copies, ng))
    for _ in range(args.warmup):
        L8.step(h())
    torch.cuda.synchronize()
    for s in range(args.steps):
        L8.step(h(), ev)
        torch.cuda.synchronize()
        for r in range(L8.copies):
            for i in range(ng):
                durs[s, r, i] = ev[r][i][0].elapsed_time(ev[r][i][1]) * 1e3   # us
    # average launch: the graph replays the step's launches back to back on
    # this stream, so step time / launches is the mean duration per launch
    n_launch = L8.copies * ng
    mean_us = sec * 1e6 / n_launch
    eager_mean_us = float(durs.mean())
    mean_bytes = float(np.mean(L8.bytes))
    per_proj = {}
    for i, n in enumerate(L8.names):
        d = float(durs[:, :, i].mean())
        per_proj[n] = {"us": round(d, 2), "MB": round(L8.bytes[i] / 1e6, 2),
                       "GBps": round(L8.bytes[i] / d / 1e3, 1),
                       "frac_hbm": round(L8.bytes[i] / d / 1e3 / HBM_PEAK_GBS, 3)}
    achieved = mean_bytes / mean_us / 1e3
    log(f"decode kernel: mean {mean_us:.2f} us/launch in the graph ({eager_mean_us:.2f} between eager events), "
        f"{achieved:.0f} GB/s; per launch group {per_proj}")

    extra = {"per_launch_group_m1_eager_events": per_proj,
             "kernel_sum_us_per_step": round(float(durs.sum(axis=(1, 2)).mean()), 1),
             "graph_step_us": round(sec * 1e6, 1), "graph_step_us_p10_p50_p90": step_pct,
             "library_graph_step_us": round(lib_graph_us, 1),
             "host_wall_us_per_step": round(wall * 1e6, 1)}

    extra["device"] = device_info
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

    if "llama3_8b_m8" in want:
        # ---------------- same layers at M = 8 ----------------
        L8b = L8.with_batch(8, 8)
        s8, _, _ = time_graph(torch, lambda: L8b.step(h()), args.steps, args.warmup)
        extra["llama3_8b_decode_m8_GBps"] = round(total_bytes / s8 / 1e9, 1)
        log(f"decode M=8: {total_bytes / s8 / 1e9:.0f} GB/s")
        del L8b

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
            "mixed_GBps": round(value, 1), "mixed_mean_bits": round(L8.mean_bits, 3),
            "mixed_over_uniform_at_same_bits": round(value / ref, 3)}
        log(f"mixed / uniform at {L8.mean_bits:.2f} bits: {value / ref:.3f}")

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
        del lin, d
        torch.cuda.empty_cache()

    if "llama3_70b" in want:
        # ---------------- Llama-3-70B layer, decode M = 1 ----------------
        log("packing Llama-3-70B-shaped layer")
        L70 = DecodeLayerSet(torch, gbb, synth, synth.llama3_70b_proj, LAYER_COPIES_70B, 1, dev)
        s70, _, _ = time_graph(torch, lambda: L70.step(h()), max(10, args.steps // 2), args.warmup)
        b70 = L70.layer_bytes * L70.copies
        extra["llama3_70b_decode_m1_GBps"] = round(b70 / s70 / 1e9, 1)
        extra["llama3_70b_layer_MB"] = round(L70.layer_bytes / 1e6, 1)
        log(f"70B decode M=1: {b70 / s70 / 1e9:.0f} GB/s")
        for M in (8, 32):
            Lm = L70.with_batch(M, M)
            sm, _, _ = time_graph(torch, lambda: Lm.step(h()), max(10, args.steps // 2), args.warmup)
            extra[f"llama3_70b_decode_m{M}_GBps"] = round(b70 / sm / 1e9, 1)
            log(f"70B decode M={M}: {b70 / sm / 1e9:.0f} GB/s")
            del Lm
        del L70
        torch.cuda.empty_cache()

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
            # moderate batches: the library's own choice between the prefill
            # kernel and 32-token decode chunks, against the prefill kernel forced
            mid = {}
            for Mm in (64, 256):
                xm = x[:Mm].contiguous()
                ym = y[:Mm]
                sa = time_eager(torch, lambda: gbb.gemm_mixed_w(rot.next(), p.N, p.K, xm, out=ym), 30, 12)
                sf = time_eager(torch, lambda: gbb.gemm_mixed_w_path(rot.next(), p.N, p.K, xm, 2, out=ym), 30, 12)
                mid[f"M{Mm}"] = {"us": round(sa * 1e6, 1), "prefill_kernel_us": round(sf * 1e6, 1)}
                log(f"prefill {p.name} M={Mm}: {sa * 1e6:.1f} us (prefill kernel alone {sf * 1e6:.1f} us)")
            del rot
            w32, w16 = gbb.dequant(imgd, p.N, p.K)
            del w32
            sl = time_eager(torch, lambda: torch.matmul(x, w16.t(), out=y), 30, 30)
            pre[p.name] = {"N": p.N, "K": p.K, "ms": round(sp * 1e3, 3), "TFLOPs": round(fl / sp / 1e12, 1),
                           "frac_fp16_peak": round(fl / sp / 1e12 / FP16_PEAK_TFLOPS, 3),
                           "fp16_library_gemm_on_dequantized_TFLOPs": round(fl / sl / 1e12, 1),
                           "moderate_batches": mid}
            log(f"prefill {p.name}: {fl / sp / 1e12:.0f} TFLOP/s (library fp16 GEMM {fl / sl / 1e12:.0f})")
            del imgd, x, y, w16
            torch.cuda.empty_cache()
        extra["prefill_m2048_70b_mlp"] = pre

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
        extra["w44a8_28672x8192"] = w48
        del imgd, rot
        torch.cuda.empty_cache()

    cpu = None
    if not args.quick and not args.no_cpu_baseline:
        cpu = cpu_baseline(gbb, synth)
        extra["cpu_baseline_one_thread_o_proj_GBps"] = cpu_baseline_one_thread(gbb, synth)

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
        "data": "synthetic (seeded random weights and activations of Llama-3 layer shapes)",
        "config": {"workload": "llama3_8b_layer_decode_m1", "layers_per_step": LAYER_COPIES_8B,
                   "projections": "q,k,v,o,gate,up,down", "launches_per_layer": "qkv,o,gate_up,down",
                   "M": 1, "block": "64x128",
                   "bits": "{1,2,3,4,6,8} mean 3.10", "group": 128,
                   "weight_MB_per_step": round(total_bytes / 1e6, 1), "parallelism": "single GPU"},
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 3), "traffic": measured_traffic(),
                     "kernel": "decode1_kernel<4>", "mean_launch_us": round(mean_us, 3),
                     "mean_algorithmic_bytes_per_launch": round(mean_bytes)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(gbb, synth):
    """The oracle as it stands -- its own unpacker, exact fp32 dequant and an
    fp64 product -- over one copy of the headline layer (7 projections, M=1)."""
    from threadpoolctl import threadpool_info

    from oracle import blockquant as bq
    from oracle import image as oimg

    log("cpu baseline: oracle over one Llama-3-8B-shaped layer at M=1")
    total_bytes = 0
    t = 0.0
    for i in range(7):
        p, W, bits = synth.llama3_8b_proj(i)
        img, _, _ = gbb.pack_blocks(W, bits)
        del W
        x = np.random.default_rng(7).standard_normal((1, p.K)).astype(np.float16)
        t0 = time.perf_counter()
        d = oimg.read_block_image(img)
        w = bq.dequant_fp32(d["q"], d["s16"], d["z16"])
        bq.gemm_fp64(x, w)
        t += time.perf_counter() - t0
        total_bytes += weight_bytes(bits)
        del d, w
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    return {"value": round(total_bytes / t / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one layer copy (7 projections, {total_bytes / 1e6:.1f} MB packed) at M=1: oracle unpack + "
                      f"fp32 dequant + fp64 GEMV, {t:.1f} s"}


def cpu_baseline_one_thread(gbb, synth):
    """The same oracle on one thread (BLAS limited to one), over the o
    projection only, for context next to the multi-thread figure."""
    from threadpoolctl import threadpool_limits

    from oracle import blockquant as bq
    from oracle import image as oimg

    p, W, bits = synth.llama3_8b_proj(3)
    img, _, _ = gbb.pack_blocks(W, bits)
    del W
    x = np.random.default_rng(7).standard_normal((1, p.K)).astype(np.float16)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        d = oimg.read_block_image(img)
        w = bq.dequant_fp32(d["q"], d["s16"], d["z16"])
        bq.gemm_fp64(x, w)
        t = time.perf_counter() - t0
    return round(weight_bytes(bits) / t / 1e9, 3)


if __name__ == "__main__":
    main()

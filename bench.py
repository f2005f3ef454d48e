#!/usr/bin/env python3
"""Benchmark of the block-wise int4 matmul hot path on one MI355X.

One step = one pass of the whole hot path over the measured workloads, each
launched on R rotating copies of its operands (weights, activations, outputs)
so the working set (> 1 GiB per workload) defeats the 256 MB Infinity Cache:

  prefill GEMM     M=2048 K=4096 N=14336 g=128 fp16, asymmetric zero points
  (+ the same with an fp16 bias, with act order, and with int8 activations)
  small-M GEMM     M=2,4,8,16 K=4096 N=14336 g=64 fp16, asymmetric zero points
  down projection  M=1 K=11008 N=4096 g=128 fp16
  gate/up SwiGLU   M=1 K=4096 N=11008 g=128 fp16 (two weights, fused)
  (decode GEMV with act order, with int8 activations, with a bias)
  tiny GEMV        M=1 K=256 N=256 g=32 fp32 (256 copies: launch-bound)
  decode GEMV      M=1 K=4096 N=4096 g=32 fp16, asymmetric zero points

The compute-bound GEMMs run first and the decode GEMV last: right after the
prefill's milliseconds of matrix work the chip runs memory-bound kernels about
0.8 us slower per launch (its clocks recover over the next milliseconds), so
the memory-bound kernels that measure the headline run furthest from it.

Each workload's R launches are recorded once into a HIP graph; every step
replays the graphs, timed with HIP events on the replay stream, so the figures
are back-to-back GPU time (kernel plus dispatch gap), not the host's launch
rate.  The headline value is the decode GEMV's effective bandwidth:
algorithmic bytes (ONNX-layout codes + scales + zero points + A + Y) per
launch over the average launch duration.  The prefill GEMM is reported in
TFLOP/s (2MNK).

After the timed steps, outside them: every memory-bound workload's graph is
replayed alone ("isolated_us"), and a plain streaming read of the same number
of bytes over as many rotating buffers ("floor_us", the yardstick library) is
timed the same way; frac_of_floor = floor_us / isolated_us.  Each
compute-bound GEMM's graph is replayed back to back until the clock has
settled ("sustained_us", its last 6 of 18 replays): in the step the prefill
follows milliseconds of memory-bound work and runs its first launches at a
higher clock than sustained matrix work holds.  The CPU baseline
leg times the oracle on a bounded sample of each measured configuration and
checks the GPU's outputs of the timed run on that sample (max |err| / bound,
pass).  Prints one JSON line.
"""
import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix
COLD_BYTES = 1 << 30           # rotation working set per workload
TINY_COPIES = 256              # the 43 KB tiny GEMV is launch-bound
SETTLE_REPLAYS = 12            # untimed graph replays before the sustained GEMM figure


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-isolated", action="store_true",
                   help="skip the isolated replays and the streaming-read floors")
    p.add_argument("--cpu-seconds", type=float, default=8.0)
    p.add_argument("--only", default="",
                   help="comma list of: prefill,small_m,down,gate_up,gemv,tiny,bias,act_order,accuracy4 "
                        "(default all); copy adds a plain 256 MiB device copy, the reference kernel "
                        "for scaling the HBM byte counters; gidx adds the general group-index route at "
                        "M = 1, 16 and 256, prefill_groups the prefill GEMM at g = 64, 32 and 16 (neither "
                        "is part of the default step)")
    return p.parse_args()


def onnx_bytes(M, K, N, g, scale_bytes, zp, act_bytes, n_weights=1, out_n=None):
    kb = K // g
    w = N * K // 2 + N * kb * scale_bytes + (N * ((kb + 1) // 2) if zp else 0)
    out_n = N if out_n is None else out_n
    return n_weights * w + M * K * act_bytes + M * out_n * act_bytes


def _graph_of(launch):
    """A HIP graph of launch() recorded on a side stream (first-call setup
    outside the capture)."""
    import torch
    launch()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            launch()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return graph


def _time_isolated(graph, R, reps=6, warm=2):
    """us per launch of a graph of R launches replayed alone, back to back,
    after warm untimed replays."""
    import torch
    for _ in range(warm):
        graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * R)


class CopyWorkload:
    """A plain streaming kernel of known size: torch's elementwise negation
    of a 256 MiB fp16 tensor into another, which reads 256 MiB and writes
    256 MiB.  The FETCH_SIZE / WRITE_SIZE counters of the other kernels are
    scaled by what the same counters read for it (its kernel name is unique
    in the run, unlike the runtime's blit copies)."""

    config = "copy"
    memory_bound = False

    def __init__(self, nbytes=256 << 20):
        import torch
        self.name, self.variant = "plain copy %d MiB" % (nbytes >> 20), "torch neg (copy)"
        self.src = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda:0")
        self.dst = torch.empty_like(self.src)
        self.bytes, self.flops, self.R = 2 * nbytes, 0, 1
        self.events = []

    def capture(self):
        pass

    def run(self, timed):
        import torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.neg(self.src, out=self.dst)
        e1.record()
        if timed:
            self.events.append((e0, e1))

    def keep_output(self):
        pass


class Workload:
    """R rotating device copies of one workload's operands, plus the host
    operands of copy 0 and, after the run, its output (for the parity check
    of the CPU baseline leg)."""

    def __init__(self, name, config, M, weights, K, N, g, act="f16", sigma=1.0, seed=(0,), bias=None,
                 act_order=False, accuracy4=False, copies=None, group_indices=False):
        import numpy as np
        import torch
        from block_wise_int4_amd import mnb, synth
        self.name, self.config, self.M, self.K, self.N, self.g = name, config, M, K, N, g
        self.weights = weights
        dev = torch.device("cuda:0")
        qs = []
        self.perm = None
        self.g_idx = None
        self.g_idx_dev = None
        for w in weights:
            args = (torch.from_numpy(w.packed.reshape(-1)).to(dev), torch.from_numpy(w.scales.reshape(-1)).to(dev),
                    None if w.zero_points is None else torch.from_numpy(w.zero_points.reshape(-1)).to(dev))
            if act_order:
                # a seeded act order: every group gets exactly g positions
                rng = np.random.default_rng(seed + (7,))
                g_idx = np.empty(K, np.int32)
                g_idx[rng.permutation(K)] = np.arange(K) // g
                self.g_idx = g_idx
                d = mnb.desc(N, K, g, w.zero_points is not None, mnb._dtype_code(args[1]))
                self.perm = torch.from_numpy(mnb.mnb_act_order_permutation(d, g_idx)).to(dev)
                out = torch.empty(mnb.mnb_repacked_bytes(d), dtype=torch.uint8, device=dev)
                mnb.mnb_repack_act_order(d, *args, self.perm, out)
                q = mnb.QuantWeight(d, out)
            else:
                q = mnb.repack(*args, N, K, g)
                if group_indices:
                    # a seeded g_idx whose groups have random sizes (the
                    # general route's input)
                    rng = np.random.default_rng(seed + (9,))
                    self.g_idx = rng.integers(0, K // g, K).astype(np.int32)
                    self.g_idx_dev = torch.from_numpy(self.g_idx).to(dev)
            qs.append(q)
        self.A_host = synth.activation(M, K, act, sigma, seed)
        A = torch.from_numpy(self.A_host).to(dev)
        zp = weights[0].zero_points is not None
        sb = 2 if weights[0].scales.dtype.itemsize == 2 else 4
        ab = 2 if act == "f16" else 4
        self.bytes = onnx_bytes(M, K, N, g, sb, zp, ab, len(weights))
        # optional bias epilogue: ("vector" | "rows", mode); its fp16 elements
        # count as algorithmic bytes
        self.bias = bias
        bias_rows = 0
        if bias is not None:
            bias_rows = M if bias[0] == "rows" else 1
            self.bias_stride = N if bias[0] == "rows" else 0
            self.bias_mode = bias[1]
            self.bytes += bias_rows * N * 2
        if act_order or group_indices:
            self.bytes += K * 4                       # the group indices
        self.accuracy4 = accuracy4
        if accuracy4:
            self.bytes += N * 4                       # the fp32 bias
        self.flops = 2 * M * N * K * len(weights)
        per_copy = (sum(q.repacked.numel() for q in qs) + A.numel() * A.element_size() * 2
                    + M * N * A.element_size() + bias_rows * N * 2)
        self.R = copies if copies is not None else max(2, -(-COLD_BYTES // per_copy))
        self.desc = qs[0].desc
        self.copies = []
        self.bias_host = None
        for r in range(self.R):
            ws = [q.repacked.clone() for q in qs]
            a = A.clone()
            y = torch.empty((M, N), dtype=A.dtype, device=dev)
            b = None
            if bias_rows or accuracy4:
                gen = torch.Generator().manual_seed(1000 + r)
                bh = torch.randn(max(bias_rows, 1) * N, generator=gen).to(A.dtype)
                if r == 0:
                    self.bias_host = bh.numpy()
                b = bh.to(dev)
            self.copies.append((ws, a, y, b))
        self.ws_bytes = mnb.mnb_gemm_workspace_bytes(self.desc, M) if len(qs) == 1 else 0
        if act_order:
            self.ws_bytes = mnb.mnb_gemm_act_order_workspace_bytes(self.desc, M)
        if accuracy4:
            # the decode call keeps the codes on chip (no workspace)
            self.ws_bytes = mnb.mnb_gemm_accuracy4_workspace_bytes(self.desc, M) if M > 1 else 0
        self.workspaces = [torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
                           for _ in range(self.R)]
        torch.cuda.synchronize()
        self.fused = len(qs) == 2
        self.memory_bound = M <= 16
        self.events = []
        self.variant = ""
        self.y_host = None

    def launch_all(self):
        from block_wise_int4_amd import mnb
        for r, (ws, a, y, b) in enumerate(self.copies):
            if self.fused:
                mnb.mnb_gemv_gate_up_swiglu(self.desc, ws[0], ws[1], a, y)
            elif self.accuracy4:
                mnb.mnb_gemm_accuracy4(self.desc, ws[0], a, self.M, b, y,
                                       self.workspaces[r] if self.ws_bytes else None, self.ws_bytes)
            elif self.g_idx_dev is not None:
                mnb.mnb_gemm_group_indices(self.desc, ws[0], a, self.M, self.g_idx_dev, y)
            elif self.perm is not None:
                mnb.mnb_gemm_act_order(self.desc, ws[0], a, self.M, self.perm, y, self.workspaces[r],
                                       self.ws_bytes)
            elif b is not None:
                mnb.mnb_gemm_bias(self.desc, ws[0], a, self.M, b, self.bias_stride, self.bias_mode, y,
                                  self.workspaces[r], self.ws_bytes)
            else:
                mnb.mnb_gemm(self.desc, ws[0], a, self.M, y, self.workspaces[r], self.ws_bytes)
        self.variant = mnb.mnb_last_variant()

    def capture(self):
        """Record the R launches into one HIP graph, so a replay measures the
        GPU (back-to-back kernels) rather than the host's launch rate."""
        self.graph = _graph_of(self.launch_all)

    def run(self, timed):
        import torch
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        self.graph.replay()
        if timed:
            e1.record()
            self.events.append((e0, e1))

    def keep_output(self):
        import torch
        torch.cuda.synchronize()
        self.y_host = self.copies[0][2].float().cpu().numpy().astype("float64")


def finish(w):
    total = sum(a.elapsed_time(b) for a, b in w.events)
    s = total / (len(w.events) * w.R) * 1e-3
    out = {"workload": w.name, "config": w.config, "variant": w.variant, "avg_launch_us": round(s * 1e6, 3),
           "kernel_source": kernel_source_sha(w.variant), "rotating_copies": w.R,
           "algorithmic_bytes": w.bytes, "flops": w.flops,
           "GBps": round(w.bytes / s / 1e9, 1), "hbm_frac": round(w.bytes / s / 1e9 / HBM_PEAK_GBS, 4),
           "TFLOPs": round(w.flops / s / 1e12, 2),
           "mfma_frac": round(w.flops / s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
    kt = kernel_trace(w.name, w.variant)
    if kt is not None:
        out["kernel_trace_us"] = kt
    return out


# Source files each variant's kernel is compiled from (its own file plus the
# shared headers): a profile summary applies only while these are unchanged.
CSRC = os.path.join(ROOT, "block_wise_int4_amd", "csrc")
SHARED_HEADERS = ["mnb_device.hpp", "mnb_layout.hpp", "mnb_internal.hpp", "mnb_acc4.hpp"]
VARIANT_SOURCE = {"gemv_accuracy4": "acc4.hip", "gemv": "gemv.hip", "gemm_small": "gemm_small.hip",
                  "gemm_mfma": "gemm_mfma.hip", "gemm_gidx": "gidx.hip"}


def kernel_source_sha(variant):
    import hashlib
    src = next((f for p, f in VARIANT_SOURCE.items() if variant.startswith(p)), None)
    if src is None:
        return None
    h = hashlib.sha256()
    for f in [src] + SHARED_HEADERS:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_lines(tag):
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith(tag + "|"):
                    yield [x.strip() for x in line.split("|")[1:]]


def counted_traffic(workload, variant):
    """HBM bytes per launch of `workload`, from the committed counter summaries
    profiles/*.txt (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter
    reads for the plain copy).  None when no summary covers this workload or
    its kernel source has changed since the counters were taken."""
    sha = kernel_source_sha(variant)
    for f in _profile_lines("traffic"):
        if f[0] == workload and f[1] == sha:
            return int(f[2])
    return None


def kernel_trace(workload, variant):
    """The rocprofv3 kernel-trace figures (us per dispatch: median, mean) of
    `workload` from the committed summaries, while its kernel source is
    unchanged; else None."""
    sha = kernel_source_sha(variant)
    for f in _profile_lines("ktrace"):
        if f[0] == workload and f[1] == sha:
            return {"median": float(f[2]) / 1e3, "mean": float(f[3]) / 1e3, "dispatches": int(f[4])}
    return None


def build_workloads(only):
    from block_wise_int4_amd import mnb
    from block_wise_int4_amd import synth as S
    sel = set(x for x in only.split(",") if x) or {"prefill", "small_m", "down", "gate_up", "gemv", "tiny",
                                                   "bias", "act_order", "accuracy4"}
    wl = [CopyWorkload()] if "copy" in sel else []
    # compute-bound GEMMs first ...
    if "prefill" in sel:
        c = S.PREFILL_GEMM
        wl.append(Workload(c.name, "c5", c.M, [S.workload_weights(c)], c.K, c.N, c.group, sigma=c.sigma,
                           seed=c.seed + (c.M,)))
    if "bias" in sel:
        c = S.PREFILL_GEMM
        wl.append(Workload(c.name + " + bias [N] fp16(fp16(acc)+b)", "N2", c.M, [S.workload_weights(c)],
                           c.K, c.N, c.group, sigma=c.sigma, seed=c.seed + (c.M,),
                           bias=("vector", mnb.MNB_BIAS_AFTER_ROUND)))
    if "act_order" in sel:
        c = S.PREFILL_GEMM
        wl.append(Workload(c.name + " act-order", "N3", c.M, [S.workload_weights(c)], c.K, c.N, c.group,
                           sigma=c.sigma, seed=c.seed + (c.M,), act_order=True))
    if "accuracy4" in sel:
        c = S.ACC4_PREFILL
        wl.append(Workload(c.name + " + bias", "N4", c.M, [S.workload_weights(c)], c.K, c.N, c.group,
                           act="f32", seed=c.seed + (c.M,), accuracy4=True))
    # ... then the memory-bound ones, the decode GEMV last
    if "small_m" in sel:
        c = S.SMALL_M_GEMM
        w = S.workload_weights(c)
        for M in S.SMALL_M_VALUES:
            wl.append(Workload(c.name.replace("small-M", "small-M M=%d" % M), "c4", M, [w], c.K, c.N,
                               c.group, seed=c.seed + (M,)))
    if "down" in sel:
        c = S.DOWN_PROJ_GEMV
        wl.append(Workload(c.name, "N1", 1, [S.workload_weights(c)], c.K, c.N, c.group, seed=c.seed + (1,)))
    if "gate_up" in sel:
        c = S.GATE_UP_SWIGLU
        g, u = S.workload_weights(c)
        wl.append(Workload(c.name, "c3", 1, [g, u], c.K, c.N, c.group, seed=c.seed + (1,)))
    if "act_order" in sel:
        c = S.DECODE_GEMV
        wl.append(Workload(c.name + " act-order", "N3", 1, [S.workload_weights(c)], c.K, c.N, c.group,
                           seed=c.seed + (1,), act_order=True))
    if "accuracy4" in sel:
        c = S.ACC4_DECODE
        wl.append(Workload(c.name + " + bias", "N4", c.M, [S.workload_weights(c)], c.K, c.N, c.group,
                           act="f32", seed=c.seed + (c.M,), accuracy4=True))
    if "bias" in sel:
        c = S.DECODE_GEMV
        wl.append(Workload(c.name + " + bias [N] fp16(acc+b)", "N2", 1, [S.workload_weights(c)], c.K, c.N,
                           c.group, seed=c.seed + (1,), bias=("vector", mnb.MNB_BIAS_FUSED)))
    if "tiny" in sel:
        c = S.TINY_GEMV
        wl.append(Workload(c.name, "c1", 1, [S.workload_weights(c)], c.K, c.N, c.group, act="f32",
                           seed=c.seed + (1,), copies=TINY_COPIES))
    if "gemv" in sel:
        c = S.DECODE_GEMV
        wl.append(Workload(c.name, "c2", 1, [S.workload_weights(c)], c.K, c.N, c.group, seed=c.seed + (1,)))
    # the prefill at the other group sizes, only on request (not part of a step)
    if "prefill_groups" in sel:
        import dataclasses
        c0 = S.PREFILL_GEMM
        for g in (64, 32, 16):
            c = dataclasses.replace(c0, name=c0.name.replace("g=128", "g=%d" % g), group=g, seed=c0.seed + (g,))
            wl.append(Workload(c.name, "c5-g%d" % g, c.M, [S.workload_weights(c)], c.K, c.N, c.group,
                               sigma=c.sigma, seed=c.seed + (c.M,)))
    # the general group-index route, only on request (not part of a step)
    if "gidx" in sel:
        c = S.DECODE_GEMV
        for M in (1, 16, 256):
            wl.append(Workload(c.name.replace("decode GEMV M=1", "group-index route M=%d" % M) + ", g_idx of random group sizes", "N3", M,
                               [S.workload_weights(c)], c.K, c.N, c.group, seed=c.seed + (M,),
                               group_indices=True))
    return wl


class Yardstick:
    """bench's streaming-read floor: the plain read kernel of
    libmnb_yardstick.so over R rotating buffers of a workload's byte count,
    recorded into a HIP graph and replayed alone, at a few grid shapes (the
    best counts)."""

    GRIDS = ((512, 512), (1024, 512), (2048, 512), (2048, 1024))

    def __init__(self):
        import torch
        from block_wise_int4_amd import build as B
        if not os.path.exists(B.YARDSTICK_LIB):
            raise ImportError("libmnb_yardstick.so is not built; run `python -m block_wise_int4_amd.build`")
        self.lib = ctypes.CDLL(B.YARDSTICK_LIB)
        self.lib.mnb_yardstick_read.restype = ctypes.c_int
        self.lib.mnb_yardstick_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_void_p]
        self.sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
        self.cache = {}

    def floor_us(self, nbytes):
        import torch
        nbytes = nbytes // 16 * 16
        if nbytes in self.cache:
            return self.cache[nbytes]
        R = max(2, -(-COLD_BYTES // nbytes)) if nbytes >= (1 << 20) else TINY_COPIES
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0") for _ in range(R)]
        best = None
        for blocks, threads in self.GRIDS:
            def launch():
                s = torch.cuda.current_stream().cuda_stream
                for b in bufs:
                    rc = self.lib.mnb_yardstick_read(ctypes.c_void_p(b.data_ptr()), nbytes,
                                                     ctypes.c_void_p(self.sink.data_ptr()), blocks, threads,
                                                     ctypes.c_void_p(s))
                    if rc != 0:
                        raise RuntimeError("yardstick launch failed (%d)" % rc)
            us = _time_isolated(_graph_of(launch), R)
            best = us if best is None or us < best else best
        del bufs
        torch.cuda.empty_cache()
        self.cache[nbytes] = round(best, 3)
        return self.cache[nbytes]


def time_repack():
    """The offline repack (ONNX bytes to the device layout), timed once per
    weight apart from the metric: HIP events around 5 calls after one warm-up
    call, on the current stream."""
    import torch
    from block_wise_int4_amd import mnb, synth as S
    out = []
    dev = torch.device("cuda:0")
    for c in (S.DECODE_GEMV, S.PREFILL_GEMM):
        w = S.workload_weights(c)
        packed = torch.from_numpy(w.packed.reshape(-1)).to(dev)
        scales = torch.from_numpy(w.scales.reshape(-1)).to(dev)
        zp = None if w.zero_points is None else torch.from_numpy(w.zero_points.reshape(-1)).to(dev)
        q = mnb.repack(packed, scales, zp, c.N, c.K, c.group)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            mnb.mnb_repack(q.desc, packed, scales, zp, q.repacked)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 5 * 1e3
        nbytes = packed.numel() + scales.numel() * scales.element_size() + (0 if zp is None else zp.numel()) \
            + q.repacked.numel()
        out.append({"weight": "%s (N=%d K=%d g=%d)" % (c.name.split(" M=")[0], c.N, c.K, c.group),
                    "us": round(us, 2), "GBps_read_plus_written": round(nbytes / (us * 1e-6) / 1e9, 1)})
    return out


def _cpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds, workloads):
    """The oracle as it stands (C, fp64, OpenMP over outputs) on the host
    cores: the decode GEMV in full, repeated for about `seconds` (and on one
    thread), then a bounded sample of each measured configuration, each timed
    and compared with the GPU's outputs of the timed run on the same outputs
    (max |err| / bound and pass, under the tests' bounds)."""
    import numpy as np
    from block_wise_int4_amd import synth as S
    from oracle import oracle as o
    threads = len(os.sched_getaffinity(0))
    c = S.DECODE_GEMV
    w = S.workload_weights(c)
    A = S.activation(1, c.K, "f16", 1.0, c.seed + (1,))
    t0 = time.perf_counter()
    reps = 0
    while True:
        o.matmul_nbits(A, w.packed, w.scales, w.zero_points, c.N, c.K, c.group, threads=threads)
        reps += 1
        if time.perf_counter() - t0 > seconds * 0.5:
            break
    gemv_s = (time.perf_counter() - t0) / reps
    bytes_ = onnx_bytes(1, c.K, c.N, c.group, 2, True, 2)
    t0 = time.perf_counter()
    reps1 = 0
    while True:
        o.matmul_nbits(A, w.packed, w.scales, w.zero_points, c.N, c.K, c.group, threads=1)
        reps1 += 1
        if time.perf_counter() - t0 > seconds * 0.2:
            break
    gemv1_s = (time.perf_counter() - t0) / reps1

    rng = np.random.default_rng(99)
    per_config = []
    gemm_rate = None
    for wk in workloads:
        if not isinstance(wk, Workload) or wk.y_host is None or wk.config not in ("c1", "c2", "c3", "c4", "c5", "N1"):
            continue
        ws = wk.weights
        t0 = time.perf_counter()
        if wk.fused:
            Yg, Bg = o.matmul_nbits(wk.A_host, ws[0].packed, ws[0].scales, ws[0].zero_points, wk.N, wk.K, wk.g,
                                    threads=threads)
            Yu, Bu = o.matmul_nbits(wk.A_host, ws[1].packed, ws[1].scales, ws[1].zero_points, wk.N, wk.K, wk.g,
                                    threads=threads)
            Y = o.swiglu(Yg, Yu)
            tol = o.swiglu_bound(Yg, Bg, Yu, Bu)
            got, sample = wk.y_host, "every output"
        elif wk.M > 16:
            # the first 8 rows in full and 4096 outputs drawn from the rest
            rows = 8
            ms = np.concatenate([np.repeat(np.arange(rows), wk.N), rng.integers(rows, wk.M, 4096)])
            ns = np.concatenate([np.tile(np.arange(wk.N), rows), rng.integers(0, wk.N, 4096)])
            Y, B = o.matmul_nbits_at(wk.A_host, ws[0].packed, ws[0].scales, ws[0].zero_points, wk.N, wk.K, wk.g,
                                     ms, ns, threads=threads)
            tol = o.REL_TOL * B + o.ABS_TOL
            got, sample = wk.y_host[ms, ns], "rows 0..%d in full and 4096 random outputs" % (rows - 1)
            gemm_rate = 2.0 * ms.size * wk.K / (time.perf_counter() - t0) / 1e12
        else:
            Y, B = o.matmul_nbits(wk.A_host, ws[0].packed, ws[0].scales, ws[0].zero_points, wk.N, wk.K, wk.g,
                                  threads=threads)
            tol = o.REL_TOL * B + o.ABS_TOL
            got, sample = wk.y_host, "every output"
        secs = time.perf_counter() - t0
        got = np.asarray(got, np.float64).reshape(np.shape(Y))
        ok = o.within_bound(got, Y, None, tol=tol)
        fin = np.isfinite(Y) & (tol > 0)
        r = float(np.max(np.abs(got[fin] - Y[fin]) / tol[fin])) if fin.any() else 0.0
        per_config.append({"workload": wk.name, "config": wk.config, "oracle_s": round(secs, 3),
                           "sample": sample, "outputs": int(np.size(Y)), "of": wk.M * wk.N,
                           "max_err_over_bound": round(r, 4), "pass": bool(ok.all())})
    return {"value": round(bytes_ / gemv_s / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": "decode GEMV M=1 K=4096 N=4096 g=32 in full, %d repetitions (%.2f ms each)"
                      % (reps, gemv_s * 1e3),
            "one_thread": {"value": round(bytes_ / gemv1_s / 1e9, 3), "unit": "GB/s",
                           "sample": "the same call on 1 thread, %d repetitions (%.2f ms each)"
                                     % (reps1, gemv1_s * 1e3)},
            "gemm": None if gemm_rate is None else
            {"value": round(gemm_rate, 5), "unit": "TFLOP/s",
             "sample": "the prefill GEMM's parity sample below (2K FLOPs per output)"},
            "configs": per_config}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU; --gpus %d is not supported "
              "(multi-GPU sharding is a design note, not a measured path)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    from block_wise_int4_amd import mnb  # noqa: F401  (loads libmnb.so; fails loudly if absent)
    torch.cuda.set_device(0)
    wls = build_workloads(args.only)
    for w in wls:
        w.capture()
    for _ in range(args.warmup):
        for w in wls:
            w.run(timed=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for w in wls:
            w.run(timed=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for w in wls:
        w.keep_output()
    res = {w.name: finish(w) if isinstance(w, Workload) else finish_copy(w) for w in wls}

    # outside the timed steps: each memory-bound workload alone, and its floor
    if not args.no_isolated:
        yard = Yardstick()
        for w in wls:
            if isinstance(w, Workload) and w.memory_bound:
                r = res[w.name]
                r["isolated_us"] = round(_time_isolated(w.graph, w.R), 3)
                r["floor_us"] = yard.floor_us(w.bytes)
                r["frac_of_floor"] = round(r["floor_us"] / r["isolated_us"], 4)
        # the compute-bound GEMMs alone, back to back, once the clock has
        # settled: the chip's power management lowers the clock over the
        # first milliseconds of sustained matrix work, and in the step each
        # of these runs for only about 2 ms
        for w in wls:
            if isinstance(w, Workload) and not w.memory_bound:
                r = res[w.name]
                us = _time_isolated(w.graph, w.R, reps=6, warm=SETTLE_REPLAYS)
                r["sustained_us"] = round(us, 3)
                r["sustained_TFLOPs"] = round(r["flops"] / us / 1e6, 2)
                r["sustained_mfma_frac"] = round(r["flops"] / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)

    head = next((r for r in res.values() if r["config"] == "c2"), None)
    gemm = next((r for r in res.values() if r["config"] == "c5"), None)

    def roof(r, bound):
        if r is None:
            return None
        s = r["avg_launch_us"] * 1e-6
        if bound == "hbm":
            a = r["algorithmic_bytes"] / s / 1e9
            return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(a / HBM_PEAK_GBS, 4),
                    "traffic": counted_traffic(r["workload"], r["variant"]),
                    "kernel": r["variant"], "avg_launch_us": r["avg_launch_us"]}
        a = r["flops"] / s / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": counted_traffic(r["workload"], r["variant"]),
                "kernel": r["variant"], "avg_launch_us": r["avg_launch_us"],
                "sustained_us": r.get("sustained_us"), "sustained_frac": r.get("sustained_mfma_frac")}

    out = {
        "metric": "M=1 int4 GEMV effective HBM GB/s (% peak); M=2048 GEMM TFLOP/s (% MFMA)",
        "value": head["GBps"] if head else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded uniform codes, zero points and scales; normal activations)",
        "config": {"workload": "decode GEMV M=1 K=4096 N=4096 g=32 fp16 asym-zp (cold cache)",
                   "step": [w.name for w in wls]},
        "roofline": roof(head, "hbm"),
        "roofline_gemm": roof(gemm, "mfma"),
        "gemm_TFLOPs": gemm["TFLOPs"] if gemm else None,
        "workloads": list(res.values()),
    }
    out["repack"] = time_repack()
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args.cpu_seconds, wls)
        out["cpu_baseline"] = cb
        by_name = {c["workload"]: c for c in cb["configs"]}
        for r in out["workloads"]:
            c = by_name.get(r["workload"])
            if c is not None:
                r["parity"] = {k: c[k] for k in ("outputs", "of", "max_err_over_bound", "pass")}
    print(json.dumps(out))


def finish_copy(w):
    total = sum(a.elapsed_time(b) for a, b in w.events)
    s = total / len(w.events) * 1e-3
    return {"workload": w.name, "config": w.config, "variant": w.variant, "avg_launch_us": round(s * 1e6, 3),
            "algorithmic_bytes": w.bytes, "GBps": round(w.bytes / s / 1e9, 1)}


if __name__ == "__main__":
    main()

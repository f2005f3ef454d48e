#!/usr/bin/env python3
"""Benchmark of the block-wise int4 matmul hot path on one MI355X.

One step = one pass of the whole hot path over the measured workloads, each
launched on R rotating copies of its operands (weights, activations, outputs)
so the working set (> 1 GiB per workload) defeats the 256 MB Infinity Cache:
  decode GEMV      M=1  K=4096 N=4096  g=32  fp16, asymmetric zero points
  gate/up SwiGLU   M=1  K=4096 N=11008 g=128 fp16 (two weights, fused)
  small-M GEMM     M=2,4,8,16 K=4096 N=14336 g=64 fp16, asymmetric zero points
  prefill GEMM     M=2048 K=4096 N=14336 g=128 fp16, asymmetric zero points
Each workload's R launches are recorded once into a HIP graph; every step
replays the graphs, timed with HIP events on the replay stream, so the
figures are back-to-back GPU time (kernel plus dispatch gap), not the host's
launch rate.  The headline value is the decode GEMV's effective bandwidth: algorithmic bytes
(ONNX-layout codes + scales + zero points + A + Y) per launch over the
average launch duration.  The prefill GEMM is reported in TFLOP/s (2MNK).
Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix
COLD_BYTES = 1 << 30           # rotation working set per workload


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--only", default="",
                   help="comma list of: gemv,gate_up,down,small_m,prefill,bias,act_order,accuracy4 (default all); "
                        "copy adds a plain 256 MiB device copy, the reference kernel "
                        "for scaling the HBM byte counters")
    return p.parse_args()


def onnx_bytes(M, K, N, g, scale_bytes, zp, act_bytes, n_weights=1, out_n=None):
    kb = K // g
    w = N * K // 2 + N * kb * scale_bytes + (N * ((kb + 1) // 2) if zp else 0)
    out_n = N if out_n is None else out_n
    return n_weights * w + M * K * act_bytes + M * out_n * act_bytes


class CopyWorkload:
    """A plain streaming kernel of known size: torch's elementwise negation
    of a 256 MiB fp16 tensor into another, which reads 256 MiB and writes
    256 MiB.  The FETCH_SIZE / WRITE_SIZE counters of the other kernels are
    scaled by what the same counters read for it (its kernel name is unique
    in the run, unlike the runtime's blit copies)."""

    def __init__(self, nbytes=256 << 20):
        import torch
        self.name, self.variant = "plain copy %d MiB" % (nbytes >> 20), "torch neg (copy)"
        self.src = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda:0")
        self.dst = torch.empty_like(self.src)
        self.bytes, self.flops, self.R = 2 * nbytes, 0, 1
        self.times_ms, self.events = [], []

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

    finish = None  # set below (shares Workload.finish)


class Workload:
    """R rotating device copies of one workload's operands."""

    def __init__(self, name, M, weights, K, N, g, act_fp16=True, sigma=1.0, seed=(0,), bias=None,
                 act_order=False, accuracy4=False):
        import torch
        from block_wise_int4_amd import mnb, synth
        self.name, self.M, self.K, self.N, self.g = name, M, K, N, g
        dev = torch.device("cuda:0")
        qs = []
        self.perm = None
        for w in weights:
            args = (torch.from_numpy(w.packed.reshape(-1)).to(dev), torch.from_numpy(w.scales.reshape(-1)).to(dev),
                    None if w.zero_points is None else torch.from_numpy(w.zero_points.reshape(-1)).to(dev))
            if act_order:
                # a seeded act order: every group gets exactly g positions
                import numpy as np
                rng = np.random.default_rng(seed + (7,))
                g_idx = np.empty(K, np.int32)
                g_idx[rng.permutation(K)] = np.arange(K) // g
                d = mnb.desc(N, K, g, w.zero_points is not None, mnb._dtype_code(args[1]))
                self.perm = torch.from_numpy(mnb.mnb_act_order_permutation(d, g_idx)).to(dev)
                out = torch.empty(mnb.mnb_repacked_bytes(d), dtype=torch.uint8, device=dev)
                mnb.mnb_repack_act_order(d, *args, self.perm, out)
                q = mnb.QuantWeight(d, out)
            else:
                q = mnb.repack(*args, N, K, g)
            qs.append(q)
        A = torch.from_numpy(synth.activation(M, K, "f16" if act_fp16 else "f32", sigma, seed)).to(dev)
        zp = weights[0].zero_points is not None
        sb = 2 if weights[0].scales.dtype.itemsize == 2 else 4
        self.bytes = onnx_bytes(M, K, N, g, sb, zp, 2 if act_fp16 else 4, len(weights))
        # optional bias epilogue: ("vector" | "rows", mode); its fp16 elements
        # count as algorithmic bytes
        self.bias = bias
        bias_rows = 0
        if bias is not None:
            bias_rows = M if bias[0] == "rows" else 1
            self.bias_stride = N if bias[0] == "rows" else 0
            self.bias_mode = bias[1]
            self.bytes += bias_rows * N * 2
        if act_order:
            self.bytes += K * 4                       # the group indices
        self.accuracy4 = accuracy4
        if accuracy4:
            self.bytes += N * 4                       # the fp32 bias
        self.flops = 2 * M * N * K * len(weights)
        per_copy = (sum(q.repacked.numel() for q in qs) + A.numel() * A.element_size() * 2
                    + M * N * A.element_size() + bias_rows * N * 2)
        self.R = max(2, -(-COLD_BYTES // per_copy))
        self.desc = qs[0].desc
        self.copies = []
        for r in range(self.R):
            ws = [q.repacked.clone() for q in qs]
            a = A.clone()
            y = torch.empty((M, N), dtype=A.dtype, device=dev)
            b = None
            if bias_rows or accuracy4:
                gen = torch.Generator().manual_seed(1000 + r)
                b = torch.randn(max(bias_rows, 1) * N, generator=gen).to(A.dtype).to(dev)
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
        self.times_ms = []
        self.variant = ""

    def launch_all(self):
        from block_wise_int4_amd import mnb
        for r, (ws, a, y, b) in enumerate(self.copies):
            if self.fused:
                mnb.mnb_gemv_gate_up_swiglu(self.desc, ws[0], ws[1], a, y)
            elif self.accuracy4:
                mnb.mnb_gemm_accuracy4(self.desc, ws[0], a, self.M, b, y,
                                       self.workspaces[r] if self.ws_bytes else None, self.ws_bytes)
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
        import torch
        self.launch_all()                      # first-call setup outside capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(self.graph, stream=s):
                self.launch_all()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    def run(self, timed):
        import torch
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        self.graph.replay()
        if timed:
            e1.record()
            self.events = getattr(self, "events", []) + [(e0, e1)]

    def finish(self):
        from block_wise_int4_amd import mnb
        total = sum(a.elapsed_time(b) for a, b in self.events)
        self.avg_launch_ms = total / (len(self.events) * self.R)
        s = self.avg_launch_ms * 1e-3
        return {"workload": self.name, "variant": self.variant, "avg_launch_us": round(s * 1e6, 3),
                "kernel_source": kernel_source_sha(self.variant),
                "rotating_copies": self.R, "algorithmic_bytes": self.bytes, "flops": self.flops,
                "GBps": round(self.bytes / s / 1e9, 1),
                "hbm_frac": round(self.bytes / s / 1e9 / HBM_PEAK_GBS, 4),
                "TFLOPs": round(self.flops / s / 1e12, 2),
                "mfma_frac": round(self.flops / s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}


CopyWorkload.finish = Workload.finish

# Source files each variant's kernel is compiled from (its own file plus the
# shared headers): a counter summary applies only while these are unchanged.
CSRC = os.path.join(ROOT, "block_wise_int4_amd", "csrc")
SHARED_HEADERS = ["mnb_device.hpp", "mnb_layout.hpp", "mnb_internal.hpp"]
VARIANT_SOURCE = {"gemv_accuracy4": "acc4.hip", "gemv": "gemv.hip", "gemm_small": "gemm_small.hip",
                  "gemm_mfma": "gemm_mfma.hip"}


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


def counted_traffic(workload, variant):
    """HBM bytes per launch of `workload`, from the committed counter summaries
    profiles/*.txt (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter
    reads for the plain copy).  None when no summary covers this workload or
    its kernel source has changed since the counters were taken."""
    import glob
    sha = kernel_source_sha(variant)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        with open(path) as fh:
            for line in fh:
                if not line.startswith("traffic|"):
                    continue
                _, name, src_sha, nbytes = [x.strip() for x in line.split("|")[:4]]
                if name == workload and src_sha == sha:
                    return int(nbytes)
    return None


def build_workloads(only):
    from block_wise_int4_amd import synth as S
    sel = set(x for x in only.split(",") if x) or {"gemv", "gate_up", "down", "small_m", "prefill", "bias",
                                                   "act_order", "accuracy4"}
    wl = [CopyWorkload()] if "copy" in sel else []
    if "gemv" in sel:
        c = S.DECODE_GEMV
        wl.append(Workload(c.name, 1, [S.workload_weights(c)], c.K, c.N, c.group, seed=c.seed + (1,)))
    if "gate_up" in sel:
        c = S.GATE_UP_SWIGLU
        g, u = S.workload_weights(c)
        wl.append(Workload(c.name, 1, [g, u], c.K, c.N, c.group, seed=c.seed + (1,)))
    if "down" in sel:
        c = S.DOWN_PROJ_GEMV
        wl.append(Workload(c.name, 1, [S.workload_weights(c)], c.K, c.N, c.group, seed=c.seed + (1,)))
    if "small_m" in sel:
        c = S.SMALL_M_GEMM
        w = S.workload_weights(c)
        for M in S.SMALL_M_VALUES:
            wl.append(Workload(c.name.replace("small-M", "small-M M=%d" % M), M, [w], c.K, c.N,
                               c.group, seed=c.seed + (M,)))
    if "prefill" in sel:
        c = S.PREFILL_GEMM
        wl.append(Workload(c.name, c.M, [S.workload_weights(c)], c.K, c.N, c.group, sigma=c.sigma,
                           seed=c.seed + (c.M,)))
    if "bias" in sel:
        from block_wise_int4_amd import mnb
        c = S.DECODE_GEMV
        wl.append(Workload(c.name + " + bias [N] fp16(acc+b)", 1, [S.workload_weights(c)], c.K, c.N,
                           c.group, seed=c.seed + (1,), bias=("vector", mnb.MNB_BIAS_FUSED)))
        c = S.PREFILL_GEMM
        wl.append(Workload(c.name + " + bias [N] fp16(fp16(acc)+b)", c.M, [S.workload_weights(c)],
                           c.K, c.N, c.group, sigma=c.sigma, seed=c.seed + (c.M,),
                           bias=("vector", mnb.MNB_BIAS_AFTER_ROUND)))
    if "accuracy4" in sel:
        for c in (S.ACC4_DECODE, S.ACC4_PREFILL):
            wl.append(Workload(c.name + " + bias", c.M, [S.workload_weights(c)], c.K, c.N, c.group,
                               act_fp16=False, seed=c.seed + (c.M,), accuracy4=True))
    if "act_order" in sel:
        c = S.DECODE_GEMV
        wl.append(Workload(c.name + " act-order", 1, [S.workload_weights(c)], c.K, c.N, c.group,
                           seed=c.seed + (1,), act_order=True))
        c = S.PREFILL_GEMM
        wl.append(Workload(c.name + " act-order", c.M, [S.workload_weights(c)], c.K, c.N, c.group,
                           sigma=c.sigma, seed=c.seed + (c.M,), act_order=True))
    return wl


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


def cpu_baseline(seconds):
    """The oracle as it stands (C, fp64, OpenMP over outputs) on the host
    cores: the decode GEMV workload in full, repeated for about `seconds`,
    and a bounded row sample of the prefill GEMM."""
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
    # the same call on one thread
    t0 = time.perf_counter()
    reps1 = 0
    while True:
        o.matmul_nbits(A, w.packed, w.scales, w.zero_points, c.N, c.K, c.group, threads=1)
        reps1 += 1
        if time.perf_counter() - t0 > seconds * 0.2:
            break
    gemv1_s = (time.perf_counter() - t0) / reps1
    p = S.PREFILL_GEMM
    wp = S.workload_weights(p)
    rows = 8
    Ap = S.activation(rows, p.K, "f16", p.sigma, p.seed + (rows,))
    t0 = time.perf_counter()
    o.matmul_nbits(Ap, wp.packed, wp.scales, wp.zero_points, p.N, p.K, p.group, threads=threads)
    gemm_s = time.perf_counter() - t0
    return {"value": round(bytes_ / gemv_s / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "decode GEMV M=1 K=4096 N=4096 g=32 in full, %d repetitions (%.2f ms each)"
                      % (reps, gemv_s * 1e3),
            "one_thread": {"value": round(bytes_ / gemv1_s / 1e9, 3), "unit": "GB/s",
                           "sample": "the same call on 1 thread, %d repetitions (%.2f ms each)"
                                     % (reps1, gemv1_s * 1e3)},
            "gemm": {"value": round(2 * rows * p.N * p.K / gemm_s / 1e12, 5), "unit": "TFLOP/s",
                     "sample": "prefill GEMM rows 0..%d of M=2048 (K=4096 N=14336 g=128), %.2f s"
                               % (rows - 1, gemm_s)}}


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
    res = {w.name: w.finish() for w in wls}

    head = next((r for r in res.values() if r["workload"].startswith("decode GEMV")), None)
    gemm = next((r for r in res.values() if r["workload"].startswith("prefill GEMM")), None)

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
                "kernel": r["variant"], "avg_launch_us": r["avg_launch_us"]}

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
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the block-scaled quantization + grouped expert GEMM hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input.  The
default workload is the DeepSeek-V3-shaped MoE layer on one GPU (4096 tokens,
hidden 7168, 256 routed + 1 shared expert, top-8, expert projections
7168 x 2048, uniform-plus-Zipf router load), all MXFP8 with rowwise and
columnwise copies: per step the expert weights and the activations are
quantized (row + column copies), then the forward (gate/up, SwiGLU + quantize,
down), data-gradient and weight-gradient grouped GEMMs run.  Other workloads
(--workload) time the Qwen3-30B-A3B-shaped NVFP4 forward, its BF16 backward
GEMMs in the high-precision and the dequantized mode, its 4-bit backward on
stochastically requantized operands, the MXFP8
quantization of 8192 x 2048 activations plus 128 expert weights, the
16384 x 2048 requant with stochastic rounding, and the 256 x 2048 round trip.

Prints one JSON line: value = whole-step throughput (GEMM TFLOP/s for the MoE
workloads, GB/s for the quantization workloads), the roofline of the dominant
kernel (its algorithmic bytes or flops per launch over its mean duration,
timed with HIP events on the launch stream), the CPU oracle timed on a
bounded sample of the same workload, and a per-op breakdown.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp16": 2500.0, "bf16": 2500.0, "fp4": 10100.0}
# VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, in lane-operations per
# second (a quarter-rate instruction counts 4)
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
SEED = 20261201
GRAPH_REPLAYS = 5


class Op:
    """One library call of the step with its algorithmic bytes and flops per launch."""

    def __init__(self, name, fn, nbytes, flops=0.0, mfma=None, valu=0.0):
        self.name = name
        self.fn = fn
        self.nbytes = float(nbytes)
        self.flops = float(flops)
        self.mfma = mfma          # MFMA input type of a GEMM ("fp8", "fp16"), None for memory-bound ops
        self.valu = float(valu)   # algorithmic VALU lane-operations per launch (0: not counted)
        self.times = []

    def bound(self):
        t_mem = self.nbytes / (HBM_PEAK_GBS * 1e9)
        t_valu = self.valu / (VALU_PEAK_TOPS * 1e12)
        if self.mfma:
            t_mfma = self.flops / (MFMA_PEAK_TFLOPS[self.mfma] * 1e12)
            return "mfma" if t_mfma >= t_mem else "hbm"
        return "alu" if t_valu > t_mem else "hbm"


def timed_until(unit_fn, min_seconds=10.0, max_reps=10000):
    """Run unit_fn() (returning the work it did) until min_seconds have elapsed."""
    work, reps = 0.0, 0
    t0 = time.perf_counter()
    while reps < max_reps:
        work += unit_fn()
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    return work, time.perf_counter() - t0, reps


def percentiles(times):
    """Median, 10th and 90th percentile of per-launch times (ms)."""
    import numpy as np
    t = np.asarray(times, np.float64)
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def host_facts():
    """The CPU the oracle baseline ran on: logical CPUs, the affinity set this
    process may use, the model name and the OpenMP setting."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "model": model,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline_both(wl, budget_s=8.0):
    """The oracle leg at one thread and at all the threads OpenMP uses, each on
    its own bounded sample (about budget_s of CPU work)."""
    import oracle
    n_all = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        one = wl.cpu_baseline(budget_s)
    finally:
        oracle.set_num_threads(n_all)
    res = wl.cpu_baseline(budget_s)
    if res is None:
        return None
    res = dict(res)
    if one is not None:
        res["one_thread"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}
    res["host"] = host_facts()
    return res


def requant_size_sweep(dev, sizes=(16384, 65536, 262144), K=2048, launches=20):
    """Requant + SR at growing M (K = 2048): mean per launch over HIP-graph
    replays, input copies rotated so that at least 600 MB are cycled (beyond the
    256 MB MALL).  Returns one entry per size with GB/s and fractions of the
    HBM peak and of the VALU issue rate (14 lane-operations per element)."""
    import torch
    from block_scaled_precision_token_amd import ops, synth
    stream = torch.cuda.current_stream(dev)
    out = []
    for M in sizes:
        nbytes = M * K * (0.5 + 1 / 16) * 2 + M * 4 + 4
        copies = max(1, min(8, int(-(-600e6 // nbytes))))
        x = synth.device_activations(SEED + 90 + M // 16384, M, K, dev)
        ins = [ops.quantize_nvfp4_per_token(x)]
        for _ in range(copies - 1):
            ins.append(tuple(t.clone() for t in ins[0]))
        del x
        outs = [(torch.empty((K, M // 2), dtype=torch.uint8, device=dev),
                 torch.empty((K, M // 16), dtype=torch.uint8, device=dev),
                 torch.empty((4,), dtype=torch.float32, device=dev)) for _ in range(copies)]
        ws = torch.empty((max(ops.requant_workspace_size(M), 16),), dtype=torch.uint8, device=dev)
        for i in range(copies):
            ops.requant_transpose_sr(*ins[i], seed=i, workspace=ws, out=outs[i])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(launches):
                i = j % copies
                ops.requant_transpose_sr(*ins[i], seed=0x5EED + j, workspace=ws, out=outs[i])
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(GRAPH_REPLAYS):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / launches)
        med, p10, p90 = percentiles(times)
        gbs = nbytes / (med * 1e-3) / 1e9
        valu = M * K * (96 / 8 + 2)
        out.append({"M": M, "K": K, "us_median": round(med * 1e3, 2), "us_p10": round(p10 * 1e3, 2),
                    "us_p90": round(p90 * 1e3, 2), "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "alu_frac": round(valu / (med * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4), "input_copies": copies})
        del g, ins, outs, ws
        torch.cuda.empty_cache()
    return out


def bf16_dev(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class Dsv3MoeMxfp8:
    """DeepSeek-V3-shaped MoE layer, MXFP8 forward + dgrad + wgrad.  SwiGLU runs
    as its own kernel on the gate/up GEMM's bf16 output, fused with h's rowwise
    MXFP8 quantization; a second pass makes h's grouped columnwise copy."""
    name = "dsv3_moe_mxfp8"
    unit = "TFLOP/s"
    dtype = "fp8_e4m3"

    def __init__(self, dev):
        import numpy as np
        import torch
        from block_scaled_precision_token_amd import ops, synth
        self.ops_mod = ops
        T, H, I, E, k = 4096, 7168, 2048, 256, 8
        G = E + 1
        N13 = 2 * I
        self.shape = dict(T=T, H=H, I=I, E=E, k=k, G=G)
        bias = synth.zipf_bias(SEED + 5, E, 1.1, uniform_mix=0.5)
        off, src = synth.route_topk(SEED + 6, T, E, k, bias, shared_expert=True)
        R = int(off[-1])
        self.R = R
        self.counts = np.diff(off)
        self.off_h, self.src_h = off, src
        off_d = torch.from_numpy(off).to(dev)
        src_d = torch.from_numpy(src).to(dev)
        X = synth.device_activations(SEED + 7, T, H, dev)
        W13 = synth.device_weights(SEED + 8, G, N13, H, dev)
        W2 = synth.device_weights(SEED + 9, G, H, I, dev)
        dY = synth.device_activations(SEED + 10, R, H, dev)
        dH13 = synth.device_activations(SEED + 11, R, N13, dev)
        self.X, self.W13, self.W2, self.dH13 = X, W13, W2, dH13
        u8, bf = torch.uint8, torch.bfloat16
        ld = ops.mxfp8_grouped_cols(R, G)
        emp = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)
        w13q = {"codes_row": emp(G, N13, H), "scales_row": emp(G, N13, H // 32),
                "codes_colT": emp(G, H, N13), "scales_colT": emp(G, H, N13 // 32)}
        w2q = {"codes_row": emp(G, H, I), "scales_row": emp(G, H, I // 32),
               "codes_colT": emp(G, I, H), "scales_colT": emp(G, I, H // 32)}
        xq = {"codes_row": emp(T, H), "scales_row": emp(T, H // 32)}
        xgq = {"codes_colT": emp(H, ld), "scales_colT": emp(H, ld // 32)}
        h13 = emp(R, N13, dt=bf)
        hq = (emp(R, I, dt=bf), emp(R, I), emp(R, I // 32), None)
        hcq = {"codes_colT": emp(I, ld), "scales_colT": emp(I, ld // 32)}
        y = emp(R, H, dt=bf)
        dyq = {"codes_row": emp(R, H), "scales_row": emp(R, H // 32), "codes_colT": emp(H, ld),
               "scales_colT": emp(H, ld // 32)}
        dh = emp(R, I, dt=bf)
        dh13q = {"codes_row": emp(R, N13), "scales_row": emp(R, N13 // 32), "codes_colT": emp(N13, ld),
                 "scales_colT": emp(N13, ld // 32)}
        dxg = emp(R, H, dt=bf)
        dw2 = emp(G, H, I, dt=bf)
        dw13 = emp(G, N13, H, dt=bf)
        # (mode, M, N, K) of the six GEMMs below; one workspace serves them in turn
        shapes = [(0, R, N13, H), (0, R, H, I), (1, R, I, H), (1, R, H, N13), (2, H, I, ld), (2, N13, H, ld)]
        ws = emp(max(ops.gemm_workspace_size(ops.FMT_MXFP8, m, a, b, c, G) for m, a, b, c in shapes))
        q, gm = ops.quantize_mxfp8, ops.moe_grouped_gemm_blockscaled
        F, D, W, M8 = ops.GEMM_FPROP, ops.GEMM_DGRAD, ops.GEMM_WGRAD, ops.FMT_MXFP8
        s8 = 1 + 1 / 32                                 # MXFP8 bytes per value (code + scale share)
        self.ops = [
            Op("quant_w13_row_col", lambda: q(W13.view(G, N13, H), True, True, out=w13q),
               G * N13 * H * (2 + 2 * s8)),
            Op("quant_w2_row_col", lambda: q(W2.view(G, H, I), True, True, out=w2q), G * H * I * (2 + 2 * s8)),
            Op("quant_x_row", lambda: q(X, True, False, out=xq), T * H * (2 + s8)),
            Op("quant_xg_col_grouped", lambda: q(X, False, True, group_offsets=off_d, row_gather=src_d, out=xgq),
               T * H * 2 + R * H * s8),
            Op("gemm_fprop_gate_up", lambda: gm(M8, F, xq["codes_row"], xq["scales_row"], w13q["codes_row"],
                                                 w13q["scales_row"], off_d, N13, H, M=R, a_gather=src_d, out=h13,
                                                 workspace=ws),
               G * N13 * H * s8 + T * H * s8 + R * N13 * 2, 2.0 * R * N13 * H, "fp8"),
            Op("swiglu_quant_h", lambda: ops.swiglu_quantize(h13, ops.FMT_MXFP8, out=hq), R * N13 * 2 + R * I * (2 + s8)),
            Op("quant_h_col_grouped", lambda: q(hq[0], False, True, group_offsets=off_d, out=hcq), R * I * (2 + s8)),
            Op("gemm_fprop_down", lambda: gm(M8, F, hq[1], hq[2], w2q["codes_row"], w2q["scales_row"], off_d, H, I,
                                              M=R, out=y, workspace=ws),
               G * H * I * s8 + R * I * s8 + R * H * 2, 2.0 * R * H * I, "fp8"),
            Op("quant_dy_row_col", lambda: q(dY, True, True, group_offsets=off_d, out=dyq), R * H * (2 + 2 * s8)),
            Op("gemm_dgrad_down", lambda: gm(M8, D, dyq["codes_row"], dyq["scales_row"], w2q["codes_colT"],
                                              w2q["scales_colT"], off_d, I, H, M=R, out=dh, workspace=ws),
               G * H * I * s8 + R * H * s8 + R * I * 2, 2.0 * R * I * H, "fp8"),
            Op("quant_dh13_row_col", lambda: q(dH13, True, True, group_offsets=off_d, out=dh13q),
               R * N13 * (2 + 2 * s8)),
            Op("gemm_dgrad_gate_up", lambda: gm(M8, D, dh13q["codes_row"], dh13q["scales_row"], w13q["codes_colT"],
                                                 w13q["scales_colT"], off_d, H, N13, M=R, out=dxg, workspace=ws),
               G * N13 * H * s8 + R * N13 * s8 + R * H * 2, 2.0 * R * H * N13, "fp8"),
            Op("gemm_wgrad_down", lambda: gm(M8, W, dyq["codes_colT"], dyq["scales_colT"], hcq["codes_colT"],
                                              hcq["scales_colT"], off_d, I, ld, M=H, out=dw2, workspace=ws),
               R * H * s8 + R * I * s8 + G * H * I * 2, 2.0 * R * H * I, "fp8"),
            Op("gemm_wgrad_gate_up", lambda: gm(M8, W, dh13q["codes_colT"], dh13q["scales_colT"], xgq["codes_colT"],
                                                 xgq["scales_colT"], off_d, H, ld, M=N13, out=dw13, workspace=ws),
               R * N13 * s8 + R * H * s8 + G * N13 * H * 2, 2.0 * R * N13 * H, "fp8"),
        ]
        self.gemm_flops = sum(o.flops for o in self.ops)

    def config(self):
        c = self.counts[:-1]
        return {"workload": "dsv3_moe_layer_mxfp8_fwd_dgrad_wgrad", "tokens": self.shape["T"],
                "hidden": self.shape["H"], "expert_intermediate": self.shape["I"],
                "experts": self.shape["E"], "shared_experts": 1, "topk": self.shape["k"], "routed_rows": self.R,
                "group_rows": {"max": int(c.max()), "mean": float(c.mean()), "median": float(__import__("numpy").median(c)),
                               "min": int(c.min()), "empty": int((c == 0).sum()), "shared": int(self.counts[-1])},
                "weights_quantized_per_step": True, "swiglu": "kernel_fused_with_h_quantization",
                "gemm_flops_per_step": self.gemm_flops}

    def value(self, ms_per_step):
        return self.gemm_flops / (ms_per_step * 1e-3) / 1e12

    def cpu_baseline(self, budget_s=10.0):
        """The oracle on a bounded sample of the same step, op kind by op kind, and
        the whole step extrapolated from those rates.  Samples (about a quarter
        of the budget each): the rowwise + columnwise MXFP8 quantization of
        experts' gate/up weights; and the three GEMM directions in fp64 on the
        experts with the largest, median and smallest routed loads and the
        shared expert -- forward gate/up and data gradient on at most 8 evenly
        spaced rows of each, weight gradient on 64 output rows over at most 256
        of the expert's tokens.  The step's quantization bytes and each
        GEMM's flops are divided by the matching rate."""
        import numpy as np
        import torch
        import oracle
        H, N13 = self.shape["H"], 2 * self.shape["I"]
        routed = self.counts[:-1]
        order = np.argsort(routed)
        subset = [int(order[-1]), int(order[len(order) // 2]), int(order[0]), len(routed)]   # largest, median, smallest, shared
        host = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        share = budget_s / 4

        def rows_of(e, cap=8):
            lo, hi = int(self.off_h[e]), int(self.off_h[e + 1])
            n = hi - lo
            return lo + (np.arange(min(n, cap)) * n) // min(n, cap)

        qi = iter(subset * 4)

        def quant_unit():
            e = next(qi)
            w = host(self.W13[e * N13:(e + 1) * N13])
            oracle.quantize_mxfp8_rowwise(w)
            oracle.quantize_mxfp8_colwise(w)
            return w.size * (2 + 2 * (1 + 1 / 32))

        qb, qt, qn = timed_until(quant_unit, share, max_reps=len(subset) * 4)
        w13 = {e: host(self.W13[e * N13:(e + 1) * N13]) for e in subset}
        fi = iter(subset)

        def fprop_unit():
            e = next(fi)
            r = rows_of(e)
            x = host(self.X[torch.from_numpy(self.src_h[r].astype(np.int64)).to(self.X.device)])
            ac, as_ = oracle.quantize_mxfp8_rowwise(x)
            bc, bs = oracle.quantize_mxfp8_rowwise(w13[e])
            t0 = time.perf_counter()
            oracle.gemm_rowgroup(oracle.FMT_MXFP8, ac, as_, None, None, np.array([0, len(r)]), N13, H, bc, bs, None)
            fprop_unit.gemm_s += time.perf_counter() - t0
            return 2.0 * len(r) * N13 * H
        fprop_unit.gemm_s = 0.0
        ff, _, fn = timed_until(fprop_unit, share, max_reps=len(subset))
        di = iter(subset)

        def dgrad_unit():
            e = next(di)
            r = rows_of(e)
            dh = host(self.dH13[torch.from_numpy(r.astype(np.int64)).to(self.dH13.device)])
            ac, as_ = oracle.quantize_mxfp8_rowwise(dh)
            bc, bs = oracle.quantize_mxfp8_colwise(w13[e])
            t0 = time.perf_counter()
            oracle.gemm_rowgroup(oracle.FMT_MXFP8, ac, as_, None, None, np.array([0, len(r)]), H, N13, bc, bs, None)
            dgrad_unit.gemm_s += time.perf_counter() - t0
            return 2.0 * len(r) * N13 * H
        dgrad_unit.gemm_s = 0.0
        df, _, dn = timed_until(dgrad_unit, share, max_reps=len(subset))
        wi = iter([subset[2], subset[1], subset[0], subset[3]])   # by increasing load, the shared expert last

        def wgrad_unit():
            e = next(wi)
            lo = int(self.off_h[e])
            hi = min(int(self.off_h[e + 1]), lo + 256)
            one = np.array([0, hi - lo], np.int64)
            dh = host(self.dH13[lo:hi])
            x = host(self.X[torch.from_numpy(self.src_h[lo:hi].astype(np.int64)).to(self.X.device)])
            ac, as_ = oracle.quantize_mxfp8_colwise(dh, one)
            bc, bs = oracle.quantize_mxfp8_colwise(x, one)
            sel = np.stack([np.zeros(64, np.int64), (np.arange(64) * N13) // 64], 1)
            t0 = time.perf_counter()
            oracle.gemm_wgrad(ac, as_, bc, bs, one, sel)
            wgrad_unit.gemm_s += time.perf_counter() - t0
            return 2.0 * (hi - lo) * 64 * H
        wgrad_unit.gemm_s = 0.0
        wf, _, wn = timed_until(wgrad_unit, share, max_reps=len(subset))
        rate = {"quant_GB_s": qb / qt / 1e9, "fprop_GFLOP_s": ff / fprop_unit.gemm_s / 1e9,
                "dgrad_GFLOP_s": df / dgrad_unit.gemm_s / 1e9, "wgrad_GFLOP_s": wf / wgrad_unit.gemm_s / 1e9}
        step_s = 0.0
        for op in self.ops:
            if op.flops:
                kind = "wgrad" if "wgrad" in op.name else "dgrad" if "dgrad" in op.name else "fprop"
                step_s += op.flops / (rate[f"{kind}_GFLOP_s"] * 1e9)
            else:
                step_s += op.nbytes / (rate["quant_GB_s"] * 1e9)
        qbytes = sum(o.nbytes for o in self.ops if not o.flops)
        return {"value": self.gemm_flops / step_s / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
                "kind": "oracle", "rates": {k: round(v, 4) for k, v in rate.items()},
                "extrapolated_step_s": round(step_s, 1),
                "sample": f"quantization of {qn} experts' 4096x7168 gate/up weights (row + column); GEMMs in fp64 "
                          f"on the largest/median/smallest-load and shared experts ({fn} forward, {dn} data-gradient "
                          f"on at most 8 evenly spaced rows each; {wn} weight-gradient, 64 output rows over at most "
                          f"256 tokens); the step extrapolated from the four rates: GEMM flops x"
                          f"{self.gemm_flops / (ff + df + wf):.0f} and quantization bytes x{qbytes / qb:.0f} "
                          f"of the sampled ones"}


class Qwen3MoeNvfp4:
    """Qwen3-30B-A3B-shaped MoE layer forward in NVFP4 (8192 tokens, top-8 of
    128 experts): per-token 4/6 quantization of X, gate/up GEMM (bf16 output),
    SwiGLU fused with the per-token 4/6 quantization of h in one kernel, down
    GEMM."""
    name = "qwen3_moe_nvfp4"
    unit = "TFLOP/s"
    dtype = "fp16"

    def __init__(self, dev):
        import numpy as np
        import torch
        from block_scaled_precision_token_amd import ops, synth
        T, H, I, E, k = 8192, 2048, 768, 128, 8
        N13 = 2 * I
        self.shape = dict(T=T, H=H, I=I, E=E, k=k)
        bias = synth.zipf_bias(SEED + 4, E, 1.1)
        off, src = synth.route_topk(SEED + 5, T, E, k, bias)
        R = int(off[-1])
        self.R, self.counts, self.off_h, self.src_h = R, np.diff(off), off, src
        off_d = torch.from_numpy(off).to(dev)
        src_d = torch.from_numpy(src).to(dev)
        X = synth.device_activations(SEED + 6, T, H, dev)
        W13 = synth.device_weights(SEED + 7, E, N13, H, dev)
        W2 = synth.device_weights(SEED + 8, E, H, I, dev)
        self.X, self.W13 = X, W13
        # weights are quantized once (rollout weights), per expert: gate and up share one outer scale
        w13 = ops.quantize_nvfp4_per_token(W13, rows_per_scale=N13)
        w2 = ops.quantize_nvfp4_per_token(W2, rows_per_scale=H)
        u8, bf, f32 = torch.uint8, torch.bfloat16, torch.float32
        emp = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)
        xq = (emp(T, H // 2), emp(T, H // 16), emp(T, dt=f32))
        h13 = emp(R, N13, dt=bf)
        hq = (None, emp(R, I // 2), emp(R, I // 16), emp(R, dt=f32))
        y = emp(R, H, dt=bf)
        ws = emp(max(ops.gemm_workspace_size(ops.FMT_NVFP4, 0, R, n, k, E) for n, k in ((N13, H), (H, I))))
        gm, F, NV = ops.moe_grouped_gemm_blockscaled, ops.GEMM_FPROP, ops.FMT_NVFP4
        s4 = 0.5 + 1 / 16
        self.ops = [
            Op("quant_x_nvfp4_46", lambda: ops.quantize_nvfp4_per_token(X, mode46=True, out=xq), T * H * (2 + s4) + T * 4),
            Op("gemm_fprop_gate_up", lambda: gm(NV, F, xq[0], xq[1], w13[0], w13[1], off_d, N13, H, M=R,
                                                 a_outer=xq[2], b_outer=w13[2], a_gather=src_d, out=h13, workspace=ws),
               E * N13 * H * s4 + T * H * s4 + R * N13 * 2, 2.0 * R * N13 * H, "fp16"),
            Op("swiglu_quant_h_nvfp4_46", lambda: ops.swiglu_quantize(h13, ops.FMT_NVFP4, mode46=True, return_h=False,
                                                                        out=hq),
               R * N13 * 2 + R * I * s4 + R * 4),
            Op("gemm_fprop_down", lambda: gm(NV, F, hq[1], hq[2], w2[0], w2[1], off_d, H, I, M=R, a_outer=hq[3],
                                              b_outer=w2[2], out=y, workspace=ws),
               E * H * I * s4 + R * I * s4 + R * H * 2, 2.0 * R * H * I, "fp16"),
        ]
        self.gemm_flops = sum(o.flops for o in self.ops)

    def config(self):
        import numpy as np
        c = self.counts
        return {"workload": "qwen3_30b_a3b_moe_layer_nvfp4_forward", "tokens": self.shape["T"],
                "hidden": self.shape["H"], "expert_intermediate": self.shape["I"], "experts": self.shape["E"],
                "topk": self.shape["k"], "routed_rows": self.R, "activation_46": True,
                "swiglu": "kernel_fused_with_h_quantization",
                "group_rows": {"max": int(c.max()), "mean": float(c.mean()), "median": float(np.median(c)),
                               "min": int(c.min()), "empty": int((c == 0).sum())},
                "gemm_flops_per_step": self.gemm_flops}

    def value(self, ms_per_step):
        return self.gemm_flops / (ms_per_step * 1e-3) / 1e12

    def cpu_baseline(self, budget_s=10.0):
        """Oracle on a sample: experts from the median load up, NVFP4 quantize of the expert's
        gate/up weights and up to 128 token rows (4/6), then their fp64 forward GEMM."""
        import numpy as np
        import torch
        import oracle
        H, N13 = self.shape["H"], 2 * self.shape["I"]
        order = np.argsort(self.counts)
        order = np.concatenate([order[len(order) // 2:], order[:len(order) // 2]])
        it = iter(order.tolist())

        def unit():
            e = next(it)
            w = self.W13[e * N13:(e + 1) * N13].view(torch.int16).cpu().numpy().view(np.uint16)
            rows = self.src_h[self.off_h[e]:self.off_h[e + 1]][:128]
            x = self.X[rows.tolist()].view(torch.int16).cpu().numpy().view(np.uint16)
            off = np.array([0, len(rows)], np.int64)
            bc, bs, bg = oracle.quantize_nvfp4(w, rows_per_scale=N13)
            ac, as_, ag = oracle.quantize_nvfp4(x, mode46=True)
            oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, None, off, N13, H, bc, bs, bg)
            return 2.0 * len(rows) * N13 * H

        flops, dt, reps = timed_until(unit, budget_s, max_reps=len(order))
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{reps} experts from the median load up: NVFP4 quantize of each expert's 1536x2048 "
                          f"gate/up weights and up to 128 of its token rows (4/6), then their forward GEMM in fp64 "
                          f"({flops / 1e9:.1f} GFLOP in {dt:.1f} s)"}


class Qwen3MoeNvfp4Bwd:
    """Qwen3-30B-A3B-shaped NVFP4 MoE layer, backward GEMMs in BF16 (the forward
    workload's shapes): data- and weight-gradient GEMMs of the down and gate/up
    projections, on the original bf16 operands (high-precision mode) or on
    dequantized copies of the forward's NVFP4 operands (dequantized mode, the
    four dequantizations timed inside the step).  The upstream gradients dY
    [routed rows, hidden] and dH13 [routed rows, 2 x intermediate] are
    synthetic N(0,1) with outliers (the SwiGLU backward between them is not on
    the path)."""
    unit = "TFLOP/s"
    dtype = "bf16"
    mode = "hp"

    def __init__(self, dev):
        import numpy as np
        import torch
        from block_scaled_precision_token_amd import ops, synth
        T, H, I, E, k = 8192, 2048, 768, 128, 8
        N13 = 2 * I
        self.shape = dict(T=T, H=H, I=I, E=E, k=k)
        bias = synth.zipf_bias(SEED + 4, E, 1.1)
        off, src = synth.route_topk(SEED + 5, T, E, k, bias)
        R = int(off[-1])
        self.R, self.counts, self.off_h, self.src_h = R, np.diff(off), off, src
        off_d = torch.from_numpy(off).to(dev)
        src_d = torch.from_numpy(src).to(dev)
        X = synth.device_activations(SEED + 6, T, H, dev)
        W13 = synth.device_weights(SEED + 7, E, N13, H, dev)
        W2 = synth.device_weights(SEED + 8, E, H, I, dev)
        h = synth.device_activations(SEED + 9, R, I, dev, std=0.5)          # SwiGLU output of the forward
        dY = synth.device_activations(SEED + 10, R, H, dev)
        dH13 = synth.device_activations(SEED + 11, R, N13, dev)
        self.X, self.W13, self.dH13 = X, W13, dH13
        bf = torch.bfloat16
        emp = lambda *s_, dt=bf: torch.empty(s_, dtype=dt, device=dev)
        dh, dX = emp(R, I), emp(R, H)
        dW2, dW13 = emp(E, H, I), emp(E, N13, H)
        ws = emp(max(ops.gemm_bf16_workspace_size(md, m, n, kk, E)
                     for md, m, n, kk in ((ops.GEMM_DGRAD, R, I, H), (ops.GEMM_DGRAD, R, H, N13),
                                          (ops.GEMM_WGRAD, H, I, R), (ops.GEMM_WGRAD, N13, H, R))), dt=torch.uint8)
        gm, DG, WG = ops.moe_grouped_gemm_bf16, ops.GEMM_DGRAD, ops.GEMM_WGRAD
        self.ops = []
        if self.mode == "deq":
            # the forward's NVFP4 operands (quantized once here, as the forward would have)
            xq = ops.quantize_nvfp4_per_token(X, mode46=True)
            hq = ops.quantize_nvfp4_per_token(h, mode46=True)
            w13q = ops.quantize_nvfp4_per_token(W13, rows_per_scale=N13)
            w2q = ops.quantize_nvfp4_per_token(W2, rows_per_scale=H)
            X, h, W13, W2 = emp(T, H), emp(R, I), emp(E * N13, H), emp(E * H, I)
            s4 = 0.5 + 1 / 16
            NV = ops.FMT_NVFP4
            self.ops += [
                Op("dequant_x", lambda: ops.dequantize(NV, *xq, out=X), T * H * (s4 + 2) + T * 4),
                Op("dequant_h", lambda: ops.dequantize(NV, *hq, out=h), R * I * (s4 + 2) + R * 4),
                Op("dequant_w13", lambda: ops.dequantize(NV, *w13q, rows_per_scale=N13, out=W13),
                   E * N13 * H * (s4 + 2) + E * 4),
                Op("dequant_w2", lambda: ops.dequantize(NV, *w2q, rows_per_scale=H, out=W2),
                   E * H * I * (s4 + 2) + E * 4),
            ]
        self.ops += [
            Op("gemm_dgrad_down", lambda: gm(DG, dY, W2, off_d, I, H, out=dh, workspace=ws),
               R * H * 2 + E * H * I * 2 + R * I * 2, 2.0 * R * I * H, "bf16"),
            Op("gemm_wgrad_down", lambda: gm(WG, dY, h, off_d, I, R, out=dW2, workspace=ws),
               R * H * 2 + R * I * 2 + E * H * I * 2, 2.0 * R * H * I, "bf16"),
            Op("gemm_dgrad_gate_up", lambda: gm(DG, dH13, W13, off_d, H, N13, out=dX, workspace=ws),
               R * N13 * 2 + E * N13 * H * 2 + R * H * 2, 2.0 * R * H * N13, "bf16"),
            Op("gemm_wgrad_gate_up", lambda: gm(WG, dH13, X, off_d, H, R, gather=src_d, out=dW13, workspace=ws),
               R * N13 * 2 + T * H * 2 + E * N13 * H * 2, 2.0 * R * N13 * H, "bf16"),
        ]
        self.gemm_flops = sum(o.flops for o in self.ops)

    def config(self):
        import numpy as np
        c = self.counts
        name = {"hp": "high_precision", "deq": "dequantized"}[self.mode]
        return {"workload": f"qwen3_30b_a3b_moe_layer_nvfp4_backward_bf16_{name}", "tokens": self.shape["T"],
                "hidden": self.shape["H"], "expert_intermediate": self.shape["I"], "experts": self.shape["E"],
                "topk": self.shape["k"], "routed_rows": self.R, "backward_mode": name,
                "gradient_dtype": "bf16",
                "group_rows": {"max": int(c.max()), "mean": float(c.mean()), "median": float(np.median(c)),
                               "min": int(c.min()), "empty": int((c == 0).sum())},
                "gemm_flops_per_step": self.gemm_flops}

    def value(self, ms_per_step):
        return self.gemm_flops / (ms_per_step * 1e-3) / 1e12

    def cpu_baseline(self, budget_s=10.0):
        """Oracle on a sample: experts from the median load up, the data-gradient GEMM of up
        to 128 of the expert's rows against its gate/up weight in fp64 (dequantized mode:
        after the oracle's NVFP4 quantize + dequantize of those operands)."""
        import numpy as np
        import torch
        import oracle
        H, N13 = self.shape["H"], 2 * self.shape["I"]
        order = np.argsort(self.counts)
        order = np.concatenate([order[len(order) // 2:], order[:len(order) // 2]])
        it = iter(order.tolist())
        deq = self.mode == "deq"

        def unit():
            e = next(it)
            w = self.W13[e * N13:(e + 1) * N13].view(torch.int16).cpu().numpy().view(np.uint16)
            lo = int(self.off_h[e])
            n = min(int(self.off_h[e + 1]) - lo, 128)
            a = self.dH13[lo:lo + n].view(torch.int16).cpu().numpy().view(np.uint16)
            if deq:
                w = oracle.dequantize_nvfp4(*oracle.quantize_nvfp4(w, rows_per_scale=N13), rows_per_scale=N13)[1]
            off = np.array([0, n], np.int64)
            oracle.gemm_bf16_rowgroup(oracle.GEMM_DGRAD, a, w, None, off, H, N13)
            return 2.0 * n * N13 * H

        flops, dt, reps = timed_until(unit, budget_s, max_reps=len(order))
        what = "NVFP4 quantize + dequantize of each expert's 1536x2048 gate/up weight, then " if deq else ""
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{reps} experts from the median load up: {what}the data-gradient GEMM of up to 128 of "
                          f"its rows (dH13 x W13_e) in fp64 ({flops / 1e9:.1f} GFLOP in {dt:.1f} s)"}


class Qwen3MoeNvfp4BwdHp(Qwen3MoeNvfp4Bwd):
    name = "qwen3_moe_nvfp4_bwd_hp"
    mode = "hp"


class Qwen3MoeNvfp4BwdDeq(Qwen3MoeNvfp4Bwd):
    name = "qwen3_moe_nvfp4_bwd_deq"
    mode = "deq"


class Qwen3MoeNvfp4BwdFp4:
    """Qwen3-30B-A3B-shaped NVFP4 MoE layer, backward in 4 bits (the forward
    workload's shapes): the gradients dY and dH13 are quantized per token, the forward's
    NVFP4 weights and activations are dequantized, transposed and requantized
    with stochastic rounding (per expert for the weights, per expert group of
    routed tokens for the activations and gradients), and the four data- and
    weight-gradient GEMMs run on NVFP4 operands."""
    name = "qwen3_moe_nvfp4_bwd_fp4"
    unit = "TFLOP/s"
    dtype = "fp16"

    def __init__(self, dev):
        import numpy as np
        import torch
        from block_scaled_precision_token_amd import ops, synth
        T, H, I, E, k = 8192, 2048, 768, 128, 8
        N13 = 2 * I
        self.shape = dict(T=T, H=H, I=I, E=E, k=k)
        bias = synth.zipf_bias(SEED + 4, E, 1.1)
        off, src = synth.route_topk(SEED + 5, T, E, k, bias)
        R = int(off[-1])
        self.R, self.counts, self.off_h, self.src_h = R, np.diff(off), off, src
        off_d = torch.from_numpy(off).to(dev)
        src_d = torch.from_numpy(src).to(dev)
        X = synth.device_activations(SEED + 6, T, H, dev)
        W13 = synth.device_weights(SEED + 7, E, N13, H, dev)
        W2 = synth.device_weights(SEED + 8, E, H, I, dev)
        h = synth.device_activations(SEED + 9, R, I, dev, std=0.5)
        dY = synth.device_activations(SEED + 10, R, H, dev)
        dH13 = synth.device_activations(SEED + 11, R, N13, dev)
        self.dH13, self.W13 = dH13, W13
        # the forward's NVFP4 operands
        xq = ops.quantize_nvfp4_per_token(X, mode46=True)
        hq = ops.quantize_nvfp4_per_token(h, mode46=True)
        w13q = ops.quantize_nvfp4_per_token(W13, rows_per_scale=N13)
        w2q = ops.quantize_nvfp4_per_token(W2, rows_per_scale=H)
        u8, bf, f32 = torch.uint8, torch.bfloat16, torch.float32
        emp = lambda *s_, dt=u8: torch.empty(s_, dtype=dt, device=dev)
        G = E
        ld = ops.mxfp8_grouped_cols(R, G)
        nvq = lambda M, K: (emp(M, K // 2), emp(M, K // 16), emp(M, dt=f32))
        dyq, dhq = nvq(R, H), nvq(R, N13)
        w2t = (emp(E * I, H // 2), emp(E * I, H // 16), emp(max(E, 4), dt=f32))
        w13t = (emp(E * H, N13 // 2), emp(E * H, N13 // 16), emp(max(E, 4), dt=f32))
        gq = lambda K: (torch.zeros((K, ld // 2), dtype=u8, device=dev), torch.zeros((K, ld // 16), dtype=u8, device=dev),
                        emp(max(G, 4), dt=f32))
        dyT, hT, dhT, xT = gq(H), gq(I), gq(N13), gq(H)
        rq_ws = emp(max(ops.requant_batched_workspace_size(E, n, n) for n in (H, N13)))
        dh, dX = emp(R, I, dt=bf), emp(R, H, dt=bf)
        dW2, dW13 = emp(E, H, I, dt=bf), emp(E, N13, H, dt=bf)
        gm, NV = ops.moe_grouped_gemm_blockscaled, ops.FMT_NVFP4
        ws = emp(max(ops.gemm_workspace_size(NV, md, m, n, kk, E)
                     for md, m, n, kk in ((ops.GEMM_DGRAD, R, I, H), (ops.GEMM_DGRAD, R, H, N13),
                                          (ops.GEMM_WGRAD, H, I, ld), (ops.GEMM_WGRAD, N13, H, ld))))
        s4 = 0.5 + 1 / 16
        rqg = ops.requant_transpose_sr_grouped
        self.ops = [
            Op("quant_dy", lambda: ops.quantize_nvfp4_per_token(dY, out=dyq), R * H * (2 + s4) + R * 4),
            Op("quant_dh13", lambda: ops.quantize_nvfp4_per_token(dH13, out=dhq), R * N13 * (2 + s4) + R * 4),
            Op("requant_w2", lambda: ops.requant_transpose_sr_batched(*w2q, E, H, seed=1, workspace=rq_ws, out=w2t),
               2 * E * H * I * s4),
            Op("requant_w13", lambda: ops.requant_transpose_sr_batched(*w13q, E, N13, seed=2, workspace=rq_ws,
                                                                       out=w13t),
               2 * E * N13 * H * s4),
            Op("requant_dy_grouped", lambda: rqg(*dyq, off_d, R, ldT=ld, seed=3, out=dyT), 2 * R * H * s4),
            Op("requant_h_grouped", lambda: rqg(*hq, off_d, R, ldT=ld, seed=4, out=hT), 2 * R * I * s4),
            Op("requant_dh13_grouped", lambda: rqg(*dhq, off_d, R, ldT=ld, seed=5, out=dhT), 2 * R * N13 * s4),
            Op("requant_x_grouped", lambda: rqg(*xq, off_d, R, ldT=ld, gather=src_d, seed=6, out=xT),
               T * H * s4 + R * H * s4),
            Op("gemm_dgrad_down", lambda: gm(NV, ops.GEMM_DGRAD, dyq[0], dyq[1], w2t[0], w2t[1], off_d, I, H,
                                             a_outer=dyq[2], b_outer=w2t[2], out=dh, workspace=ws),
               R * H * s4 + E * H * I * s4 + R * I * 2, 2.0 * R * I * H, "fp16"),
            Op("gemm_wgrad_down", lambda: gm(NV, ops.GEMM_WGRAD, dyT[0], dyT[1], hT[0], hT[1], off_d, I, ld, M=H,
                                             a_outer=dyT[2], b_outer=hT[2], out=dW2, workspace=ws),
               R * H * s4 + R * I * s4 + E * H * I * 2, 2.0 * R * H * I, "fp16"),
            Op("gemm_dgrad_gate_up", lambda: gm(NV, ops.GEMM_DGRAD, dhq[0], dhq[1], w13t[0], w13t[1], off_d, H, N13,
                                                a_outer=dhq[2], b_outer=w13t[2], out=dX, workspace=ws),
               R * N13 * s4 + E * N13 * H * s4 + R * H * 2, 2.0 * R * H * N13, "fp16"),
            Op("gemm_wgrad_gate_up", lambda: gm(NV, ops.GEMM_WGRAD, dhT[0], dhT[1], xT[0], xT[1], off_d, H, ld,
                                                M=N13, a_outer=dhT[2], b_outer=xT[2], out=dW13, workspace=ws),
               R * N13 * s4 + R * H * s4 + E * N13 * H * 2, 2.0 * R * N13 * H, "fp16"),
        ]
        self.gemm_flops = sum(o.flops for o in self.ops)

    def config(self):
        import numpy as np
        c = self.counts
        return {"workload": "qwen3_30b_a3b_moe_layer_nvfp4_backward_fp4_requant_sr", "tokens": self.shape["T"],
                "hidden": self.shape["H"], "expert_intermediate": self.shape["I"], "experts": self.shape["E"],
                "topk": self.shape["k"], "routed_rows": self.R, "backward_mode": "nvfp4_requant_sr",
                "gradient_dtype": "bf16",
                "group_rows": {"max": int(c.max()), "mean": float(c.mean()), "median": float(np.median(c)),
                               "min": int(c.min()), "empty": int((c == 0).sum())},
                "gemm_flops_per_step": self.gemm_flops}

    def value(self, ms_per_step):
        return self.gemm_flops / (ms_per_step * 1e-3) / 1e12

    def cpu_baseline(self, budget_s=10.0):
        """Oracle on a sample: experts from the median load up, the NVFP4 quantize of up to 128
        of the expert's dH13 rows, the requant (SR) of its gate/up weight, and their data-gradient
        GEMM in fp64."""
        import numpy as np
        import torch
        import oracle
        H, N13 = self.shape["H"], 2 * self.shape["I"]
        order = np.argsort(self.counts)
        order = np.concatenate([order[len(order) // 2:], order[:len(order) // 2]])
        it = iter(order.tolist())

        def unit():
            e = next(it)
            w = self.W13[e * N13:(e + 1) * N13].view(torch.int16).cpu().numpy().view(np.uint16)
            lo = int(self.off_h[e])
            n = min(int(self.off_h[e + 1]) - lo, 128)
            a = self.dH13[lo:lo + n].view(torch.int16).cpu().numpy().view(np.uint16)
            wc, wsc, wg = oracle.quantize_nvfp4(w, rows_per_scale=N13)
            bc, bs, bg = oracle.requant_transpose_sr_batched(wc, wsc, wg, 1, N13, seed=2)
            ac, as_, ag = oracle.quantize_nvfp4(a)
            off = np.array([0, n], np.int64)
            oracle.gemm_rowgroup(oracle.FMT_NVFP4, ac, as_, ag, None, off, H, N13, bc, bs, bg)
            return 2.0 * n * N13 * H

        flops, dt, reps = timed_until(unit, budget_s, max_reps=len(order))
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{reps} experts from the median load up: NVFP4 quantize of the expert's 1536x2048 gate/up "
                          f"weight and its requant with SR, NVFP4 quantize of up to 128 of its dH13 rows, then their "
                          f"data-gradient GEMM in fp64 ({flops / 1e9:.1f} GFLOP in {dt:.1f} s)"}


class Mxfp8Quant:
    """MXFP8 rowwise + columnwise quantization of 8192 x 2048 activations and rowwise
    quantization of 128 expert weights 2048 x 768."""
    name = "mxfp8_quant"
    unit = "GB/s"
    dtype = "f32"
    graph = True

    def __init__(self, dev):
        import torch
        from block_scaled_precision_token_amd import ops, synth
        M, K, E, N, KW = 8192, 2048, 128, 2048, 768
        self.copies = 16     # rotate activation buffers so they do not stay resident in the 256 MB MALL
        xs = [synth.device_activations(SEED + 20 + i, M, K, dev, row_log10_range=(-3, 2)) for i in range(self.copies)]
        W = synth.device_weights(SEED + 40, E, N, KW, dev)
        u8 = torch.uint8
        emp = lambda *s: torch.empty(s, dtype=u8, device=dev)
        outs = [{"codes_row": emp(M, K), "scales_row": emp(M, K // 32), "codes_colT": emp(K, M),
                 "scales_colT": emp(K, M // 32)} for _ in range(self.copies)]
        wq = {"codes_row": emp(E * N, KW), "scales_row": emp(E * N, KW // 32)}
        self.step_i = 0
        s8 = 1 + 1 / 32

        def quant_x():
            i = self.step_i % self.copies
            ops.quantize_mxfp8(xs[i], True, True, out=outs[i])
            self.step_i += 1

        def quant_w():
            ops.quantize_mxfp8(W, True, False, out=wq)

        self.ops = [Op("quant_x_row_col", quant_x, M * K * (2 + 2 * s8)),
                    Op("quant_weights_row", quant_w, E * N * KW * (2 + s8))]
        self.total_bytes = sum(o.nbytes for o in self.ops)
        self.x_host = None
        self.X0 = xs[0]

    def config(self):
        return {"workload": "mxfp8_quant_activations_8192x2048_row_col_plus_128_weights_2048x768",
                "bytes_per_step": self.total_bytes, "activation_copies_rotated": self.copies}

    def value(self, ms_per_step):
        return self.total_bytes / (ms_per_step * 1e-3) / 1e9

    def cpu_baseline(self, budget_s=10.0):
        import numpy as np
        import torch
        import oracle
        x = self.X0.view(torch.int16).cpu().numpy().view(np.uint16)

        def unit():
            oracle.quantize_mxfp8_rowwise(x)
            oracle.quantize_mxfp8_colwise(x)
            return x.size * (2 + 2 * (1 + 1 / 32))

        b, dt, reps = timed_until(unit, budget_s)
        return {"value": b / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"rowwise + columnwise MXFP8 of one 8192x2048 activation tensor, {reps} times "
                          f"({dt:.1f} s)"}


class RequantSr:
    """Dequantize -> transpose -> requantize with SR of a 16384 x 2048 NVFP4 tensor."""
    name = "requant_sr"
    unit = "GB/s"
    dtype = "f32"
    graph = True

    def __init__(self, dev):
        import torch
        from block_scaled_precision_token_amd import ops, synth
        M, K = 16384, 2048
        self.M, self.K = M, K
        self.copies = 32     # 32 x 37.8 MB rotated: larger than the MALL
        ins, outs = [], []
        for i in range(self.copies):
            x = synth.device_activations(SEED + 60 + i, M, K, dev)
            ins.append(ops.quantize_nvfp4_per_token(x))
            outs.append((torch.empty((K, M // 2), dtype=torch.uint8, device=dev),
                         torch.empty((K, M // 16), dtype=torch.uint8, device=dev),
                         torch.empty((4,), dtype=torch.float32, device=dev)))
            if i == 0:
                self.x0 = x
            del x
        ws = torch.empty((ops.requant_workspace_size(M),), dtype=torch.uint8, device=dev)
        self.step_i = 0

        def run():
            i = self.step_i % self.copies
            c, s, g = ins[i]
            ops.requant_transpose_sr(c, s, g, seed=0x5EED + self.step_i, sr=True, workspace=ws, out=outs[i])
            self.step_i += 1

        nbytes = M * K * (0.5 + 1 / 16) * 2 + M * 4 + 4
        # The generator alone fixes the VALU floor: Philox4x32-10 gives 8 elements
        # their 16 bits with 19 32x32->64 products (V_MAD_U64_U32, quarter rate: 4
        # each; the first Philox round has one, two counter words being zero) and 20 three-input
        # xors (1 each), 96 lane-operations; plus the dequantizing and the rescaling
        # multiply of every element: 14 per element.
        valu = M * K * (96 / 8 + 2)
        self.ops = [Op("requant_transpose_sr", run, nbytes, valu=valu)]
        self.total_bytes = nbytes

    def config(self):
        return {"workload": "nvfp4_requant_transpose_sr_16384x2048", "bytes_per_step": self.total_bytes,
                "input_copies_rotated": self.copies, "rng": "philox4x32-10"}

    def value(self, ms_per_step):
        return self.total_bytes / (ms_per_step * 1e-3) / 1e9

    def cpu_baseline(self, budget_s=10.0):
        import numpy as np
        import torch
        import oracle
        x = self.x0[:4096].view(torch.int16).cpu().numpy().view(np.uint16)
        c, s, g = oracle.quantize_nvfp4(x)
        seeds = iter(range(1, 1 << 30))

        def unit():
            oracle.requant_transpose_sr(c, s, g, seed=next(seeds), use_sr=True)
            return x.size * (0.5 + 1 / 16) * 2 + x.shape[0] * 4

        b, dt, reps = timed_until(unit, budget_s)
        return {"value": b / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"requant + SR of the first 4096 of the 16384 rows, {reps} seeds ({dt:.1f} s)"}


class RoundTrip:
    """256 x 2048 activation round trip + small GEMM against a 2048 x 768 weight."""
    name = "roundtrip"
    unit = "us"
    dtype = "f32"

    def __init__(self, dev):
        import numpy as np
        import torch
        from block_scaled_precision_token_amd import ops, synth
        M, K, N = 256, 2048, 768
        x = bf16_dev(synth.activations(SEED, M, K), dev)
        w = bf16_dev(synth.weights(SEED + 1, 1, N, K), dev)
        off = torch.tensor([0, M], dtype=torch.int64, device=dev)
        st = {}

        def nv():
            st["xn"] = ops.quantize_nvfp4_per_token(x)
            st["wn"] = ops.quantize_nvfp4_per_token(w, rows_per_scale=N)

        def mx():
            st["xm"] = ops.quantize_mxfp8(x)
            st["wm"] = ops.quantize_mxfp8(w)

        def dq():
            ops.dequantize(ops.FMT_NVFP4, *st["xn"])
            ops.dequantize(ops.FMT_MXFP8, st["xm"]["codes_row"], st["xm"]["scales_row"])

        def gemm():
            ops.moe_grouped_gemm_blockscaled(ops.FMT_NVFP4, ops.GEMM_FPROP, st["xn"][0], st["xn"][1], st["wn"][0],
                                             st["wn"][1], off, N, K, a_outer=st["xn"][2], b_outer=st["wn"][2])
            ops.moe_grouped_gemm_blockscaled(ops.FMT_MXFP8, ops.GEMM_FPROP, st["xm"]["codes_row"],
                                             st["xm"]["scales_row"], st["wm"]["codes_row"], st["wm"]["scales_row"],
                                             off, N, K)

        self.ops = [Op("quant_nvfp4_x_w", nv, (M + N) * K * 2.56), Op("quant_mxfp8_x_w", mx, (M + N) * K * 3.03),
                    Op("dequant_both", dq, M * K * (0.56 + 4 + 1.03 + 4)),
                    Op("gemm_nvfp4_and_mxfp8", gemm, (M + N) * K * 1.6 + M * N * 8, 4.0 * M * N * K, "fp16")]

    def config(self):
        return {"workload": "roundtrip_256x2048_and_gemm_768", "launch_bound": True}

    def value(self, ms_per_step):
        return ms_per_step * 1e3

    def cpu_baseline(self, budget_s=10.0):
        import numpy as np
        import oracle
        from block_scaled_precision_token_amd import synth
        x = synth.activations(SEED, 256, 2048)
        w = synth.weights(SEED + 1, 1, 768, 2048)
        t0 = time.perf_counter()
        c, s, g = oracle.quantize_nvfp4(x)
        wc, ws_, wg = oracle.quantize_nvfp4(w, rows_per_scale=768)
        mc, ms = oracle.quantize_mxfp8_rowwise(x)
        oracle.dequantize_nvfp4(c, s, g)
        oracle.dequantize_mxfp8(mc, ms)
        off = np.array([0, 256], np.int64)
        oracle.gemm_rowgroup(oracle.FMT_NVFP4, c, s, g, None, off, 768, 2048, wc, ws_, wg)
        dt = time.perf_counter() - t0
        return {"value": dt * 1e6, "unit": "us", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": "the whole round trip: NVFP4 quantize of x and w, MXFP8 quantize of x, both dequantizes "
                          "and the 256x768x2048 NVFP4 GEMM in fp64"}


class HbmCopy:
    """A plain 1 GiB device-to-device copy: the achievable HBM rate, and the kernel of
    known size that calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    name = "hbm_copy"
    unit = "GB/s"
    dtype = "u8"

    def __init__(self, dev):
        import torch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        self.ops = [Op("copy_1GiB", lambda: dst.copy_(src), 2.0 * n)]
        self.total_bytes = 2.0 * n

    def config(self):
        return {"workload": "device_copy_1GiB", "bytes_per_step": self.total_bytes}

    def value(self, ms_per_step):
        return self.total_bytes / (ms_per_step * 1e-3) / 1e9

    def cpu_baseline(self, budget_s=10.0):
        return None


WORKLOADS = {c.name: c for c in (Dsv3MoeMxfp8, Qwen3MoeNvfp4, Qwen3MoeNvfp4BwdHp, Qwen3MoeNvfp4BwdDeq,
                                  Qwen3MoeNvfp4BwdFp4, Mxfp8Quant, RequantSr, RoundTrip, HbmCopy)}


# ---------------------------------------------------------------------------

# The source files an op's kernels are compiled from (the shared device and
# launch headers included): the grouped GEMMs, and everything else.
KERNEL_SOURCES = {"gemm": ("bsp_gemm.hip", "bsp_device.hpp", "bsp_internal.hpp"),
                  "other": ("bsp_quant.hip", "bsp_device.hpp", "bsp_internal.hpp")}


def kernel_sources_of(op):
    return KERNEL_SOURCES["gemm" if op.startswith("gemm") else "other"]


def kernel_source_digest(files=None):
    """sha256 over HIP sources the library is built from (all of them, or the
    given files): file names and code with comments and whitespace runs
    removed, so that documentation edits keep the measurements valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_precision_token_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if files is not None and name not in files:
            continue
        if name.endswith((".hip", ".hpp", ".cpp", ".h")):
            with open(os.path.join(csrc, name)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            text = " ".join(text.split())
            h.update(name.encode())
            h.update(text.encode())
    return h.hexdigest()


def measured_traffic(workload, op):
    """HBM bytes per launch of `op` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    ent = table.get("ops", {}).get(f"{workload}/{op}")
    if not ent or ent.get("source_sha256") != kernel_source_digest(kernel_sources_of(op)):
        return None
    return ent.get("bytes_per_launch")


def time_eager(wl, steps, dev):
    """Launch `steps` steps from Python, with HIP events around every op on the
    launch stream; returns (wall ms per step, event ms per step)."""
    import torch
    stream = torch.cuda.current_stream(dev)
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for _ in range(steps):
        for op in wl.ops:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            op.fn()
            b.record(stream)
            events.append((op, a, b))
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for op, a, b in events:
        op.times.append(a.elapsed_time(b))
    return wall * 1e3 / steps, e_start.elapsed_time(e_end) / steps


def time_graphed(wl, steps, dev):
    """Short steps are bound by the Python launch rate, not by the GPU: capture the
    launches in HIP graphs and time their replay.  Each op is timed alone (a graph
    of `steps` launches of it, replayed GRAPH_REPLAYS times: one mean per replay),
    then the whole step (a graph of `steps` steps); every graph is replayed once
    untimed first.  Returns (wall ms per step of the
    step graph's timed replay, event ms per step of it)."""
    import torch
    stream = torch.cuda.current_stream(dev)

    def capture(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                for fn in fns:
                    fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        return g

    for op in wl.ops:
        g = capture([op.fn])
        for _ in range(GRAPH_REPLAYS):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            op.times.append(a.elapsed_time(b) / steps)
        del g
    g = capture([op.fn for op in wl.ops])
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    g.replay()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, e_start.elapsed_time(e_end) / steps


def measure(wl, steps, warmup, use_graph, dev):
    """Warm up, time `steps` steps of workload `wl` and summarize: (ms per
    step, per-op components, roofline object of the dominant op)."""
    import torch
    torch.cuda.synchronize()
    print(f"[bench] workload {wl.name} ready; {len(wl.ops)} ops per step", file=sys.stderr, flush=True)
    for _ in range(warmup):
        for op in wl.ops:
            op.fn()
    torch.cuda.synchronize()
    if use_graph:
        ms_per_step, ev_ms_per_step = time_graphed(wl, steps, dev)
    else:
        ms_per_step, ev_ms_per_step = time_eager(wl, steps, dev)
    print(f"[bench] timed {steps} steps{' (HIP graph replay)' if use_graph else ''}: "
          f"{ms_per_step:.3f} ms/step (events {ev_ms_per_step:.3f})", file=sys.stderr, flush=True)

    comps = {}
    for op in wl.ops:
        ms = sum(op.times) / len(op.times)
        med, p10, p90 = percentiles(op.times)
        d = {"ms": round(ms, 4), "ms_median": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
             "samples": len(op.times), "GB_s": round(op.nbytes / (ms * 1e-3) / 1e9, 1),
             "hbm_frac": round(op.nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bound": op.bound()}
        if op.flops:
            tf = op.flops / (ms * 1e-3) / 1e12
            d["TFLOP_s"] = round(tf, 1)
            d["mfma_frac"] = round(tf / MFMA_PEAK_TFLOPS[op.mfma], 4)
        if op.valu:
            to = op.valu / (ms * 1e-3) / 1e12
            d["TOP_s"] = round(to, 2)
            d["alu_frac"] = round(to / VALU_PEAK_TOPS, 4)
        comps[op.name] = d
    dom = max(wl.ops, key=lambda o: sum(o.times))
    dom_ms = sum(dom.times) / len(dom.times)
    traffic = measured_traffic(wl.name, dom.name)
    if dom.bound() == "mfma":
        ach = dom.flops / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFLOPS[dom.mfma], "unit": "TFLOP/s",
                "frac": round(ach / MFMA_PEAK_TFLOPS[dom.mfma], 4), "traffic": traffic, "kernel": dom.name}
    elif dom.bound() == "alu":
        ach = dom.valu / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(ach, 2), "peak": round(VALU_PEAK_TOPS, 2), "unit": "TOP/s",
                "frac": round(ach / VALU_PEAK_TOPS, 4), "traffic": traffic, "kernel": dom.name,
                "hbm_GB_s": round(dom.nbytes / (dom_ms * 1e-3) / 1e9, 1)}
    else:
        ach = dom.nbytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom.name}
    return ms_per_step, comps, roof


# Workloads the default run measures after the headline one, each in a few
# steps on the same GPU, so that every configuration's figures come from the
# same run (reported beside the headline, never folded into it).
SECONDARY = ("qwen3_moe_nvfp4", "qwen3_moe_nvfp4_bwd_fp4", "qwen3_moe_nvfp4_bwd_hp", "mxfp8_quant", "requant_sr")


def secondary_workloads(dev, steps=5, warmup=2):
    import torch
    out = {}
    for name in SECONDARY:
        wl = WORKLOADS[name](dev)
        ms, comps, roof = measure(wl, steps, warmup, getattr(wl, "graph", False), dev)
        out[name] = {"ms_per_step": round(ms, 4), "value": round(wl.value(ms), 3), "unit": wl.unit,
                     "config": wl.config(), "roofline": {k: roof[k] for k in ("kernel", "bound", "achieved",
                                                                               "unit", "frac")},
                     "steps": steps, "warmup": warmup}
        del wl, comps
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3_moe_mxfp8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the requant size sweep")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads the default run measures after the headline one")
    ap.add_argument("--only", default=None, help="time just this op of the workload (for profiler runs)")
    ap.add_argument("--graph", default="auto", choices=["auto", "on", "off"],
                    help="time HIP-graph replays instead of Python launches (auto: for the short-step workloads)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    from block_scaled_precision_token_amd import ops
    ops.lib()      # fails loudly when the HIP library is missing

    wl = WORKLOADS[args.workload](dev)
    if args.only:
        sel = [op for op in wl.ops if op.name == args.only]
        if not sel:
            print(f"bench.py: no op {args.only!r} in {wl.name}; ops: {[op.name for op in wl.ops]}", file=sys.stderr)
            sys.exit(2)
        wl.ops = sel
    use_graph = {"auto": getattr(wl, "graph", False), "on": True, "off": False}[args.graph]
    ms_per_step, comps, roof = measure(wl, args.steps, args.warmup, use_graph, dev)

    sweep = None
    if not args.no_sweep and not args.only and wl.name in ("dsv3_moe_mxfp8", "requant_sr"):
        print("[bench] requant size sweep", file=sys.stderr, flush=True)
        sweep = requant_size_sweep(dev)

    secondary = None
    if not args.no_secondary and not args.only and wl.name == "dsv3_moe_mxfp8":
        print("[bench] other workloads, a few steps each", file=sys.stderr, flush=True)
        secondary = secondary_workloads(dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample (one thread, then all)", file=sys.stderr, flush=True)
        try:
            cpu = cpu_baseline_both(wl)
        except Exception as exc:  # the baseline is reported, never required
            cpu = {"error": repr(exc)}

    value = wl.value(ms_per_step)
    line = {
        "metric": "quantize/requant GB/s (% HBM peak); MoE block-scaled GEMM TFLOPS (% MFMA)",
        "value": round(value, 3), "unit": wl.unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": wl.unit != "us", "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": dict(wl.config(), **({"only_op": args.only} if args.only else {}),
                       **({"timing": "hip_graph_replay"} if use_graph else {})), "roofline": roof,
        "cpu_baseline": cpu, "components": comps,
    }
    if sweep is not None:
        line["requant_size_sweep"] = sweep
    if secondary is not None:
        line["other_workloads"] = secondary
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

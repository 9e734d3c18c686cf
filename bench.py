#!/usr/bin/env python3
"""Benchmark of the fused NF4 double-quantized QLoRA linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole hot path over one batch: forward and backward
(dX, dA, dB; never dW) of all seven linears of a 7B-class decoder layer
(q/k/v/o 4096->4096, gate/up 4096->11008, down 11008->4096) at 2048 tokens,
rank 16, alpha 32, with every weight stored as NF4 with double-quantized
block scales and dequantized to bf16 inside the GEMMs.  Inputs are seeded
synthetic tensors already resident in HBM; the one-time quantization runs
before the timed region.

Prints one JSON line: whole-step TFLOP/s (algorithmic flops
4MNK + 6Mr(N+K) per linear), the roofline of the dominant kernel (measured
per launch with HIP events recorded around that kernel inside the timed
region), the CPU oracle timed on a bounded sample, and secondary HBM-bound
figures (standalone dequant and few-token forward on 70B shapes).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused NF4-QLoRA linear fwd+bwd TFLOP/s, % bf16 MFMA peak, 7B shapes"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PACKED_B_PER_W = (4 + 8 / 64 + 32 / 16384) / 8  # 0.51587 bytes per weight
PMC_COPY_BYTES = 256 << 20  # calibration copy of the counter runs


def flops_linear(m, n, k, r):
    return 4 * m * n * k + 6 * m * r * (n + k)


class HipEvents:
    """Raw HIP events (the library records them on the stream it launches on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    # hipEventDisableSystemFence: the marker takes its timestamp without the
    # system-scope release (an L2 write-back) that a default event adds after
    # the kernel; with default events the timed layer step runs 3-4 % slower.
    EVENT_FLAGS = 0x20000000

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), ctypes.c_uint(self.EVENT_FLAGS)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def load_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (profiles/pmc_traffic.json, written by bit_nf4_quantized_double_amd.pmc),
    if they were taken on the kernel's current sources; else None."""
    from bit_nf4_quantized_double_amd import pmc
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path) or kernel_key not in pmc.KERNELS:
        return None
    with open(path) as f:
        d = json.load(f)
    ent = d.get(kernel_key)
    if not ent or ent.get("source_hash") != pmc.source_hash(pmc.KERNELS[kernel_key][1]):
        return None
    return ent.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="for rocprofv3 --pmc runs: warmup + steps of the layer, then a "
                         "device-to-device copy of PMC_COPY_BYTES for counter calibration; no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the path runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path is single-GPU: no sharding, no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_nf4_quantized_double_amd import qlora, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    qlora.lib()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------------------------------------------------- inputs ----
    wl = "7b"
    M, r, alpha = synth.TOKENS[wl], synth.RANK[wl], synth.ALPHA[wl]
    lins = []
    host = []
    for i, lin in enumerate(synth.LAYERS[wl]):
        d = synth.workload_linear(wl, i)
        host.append(d)
        w = qlora.quantize(torch.from_numpy(d["W"]).to(dev))
        e = dict(name=lin.name, n=lin.n_out, k=lin.k_in, w=w,
                 X=to_dev(d["X"]), A=to_dev(d["A"]), B=to_dev(d["B"]), dY=to_dev(d["dY"]))
        e["Y"] = torch.empty((M, lin.n_out), dtype=torch.bfloat16, device=dev)
        e["U"] = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        e["dX"] = torch.empty((M, lin.k_in), dtype=torch.bfloat16, device=dev)
        e["dA"] = torch.empty((r, lin.k_in), dtype=torch.float32, device=dev)
        e["dB"] = torch.empty((lin.n_out, r), dtype=torch.float32, device=dev)
        e["ws"] = qlora.new_workspace(qlora.QLORA_OP_BWD, M, lin.n_out, lin.k_in, r, dev)
        e["ws_fwd"] = qlora.new_workspace(qlora.QLORA_OP_FWD, M, lin.n_out, lin.k_in, r, dev)
        lins.append(e)
    torch.cuda.synchronize()
    step_flops = sum(flops_linear(M, e["n"], e["k"], r) for e in lins)
    L = qlora.lib()
    evs = HipEvents()

    # events for every GEMM launch of the timed region, created up front
    pool = [evs.create() for _ in range(4 * len(lins) * args.steps)]

    def step(timing=None):
        for e in lins:
            if timing is not None:
                a, b = pool.pop(), pool.pop()
                timing["fwd"].append((a, b, e))
                L.qlora_time_next_gemm(a, b)
            qlora.linear_fwd(e["w"], e["X"], e["A"], e["B"], r, alpha, Y=e["Y"], U=e["U"], ws=e["ws_fwd"])
            if timing is not None:
                a, b = pool.pop(), pool.pop()
                timing["dx"].append((a, b, e))
                L.qlora_time_next_gemm(a, b)
            qlora.linear_bwd(e["w"], e["X"], e["dY"], e["A"], e["B"], r, alpha, e["U"],
                             dX=e["dX"], dA=e["dA"], dB=e["dB"], ws=e["ws"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.pmc_pass:
        for _ in range(args.steps):
            step()
        # plain elementwise copy kernel (reads and writes PMC_COPY_BYTES once)
        src = torch.ones(PMC_COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"pmc pass done: {args.steps} steps, elementwise copy of {PMC_COPY_BYTES} bytes")
        return
    timing = {"fwd": [], "dx": []}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step(timing)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / max(1, args.steps)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # ---- per-kernel roofline from the events recorded inside the timed region
    per = {}
    for kind, lst in timing.items():
        tot_ms, tot_fl, n = 0.0, 0.0, 0
        for a, b, e in lst:
            tot_ms += evs.ms(a, b)
            c = e["n"] if kind == "fwd" else e["k"]
            tot_fl += 2.0 * M * e["n"] * e["k"] + 2.0 * M * r * c
            n += 1
            evs.destroy(a)
            evs.destroy(b)
        per[kind] = dict(avg_us=1e3 * tot_ms / max(1, n), launches=n,
                         avg_flops=tot_fl / max(1, n), total_ms=tot_ms)
    dom = max(per, key=lambda k: per[k]["total_ms"])
    dk = per[dom]
    achieved = dk["avg_flops"] / (dk["avg_us"] * 1e-6) / 1e12
    kname = {"fwd": "k_gemm_nf4<false, Bf16> (fused forward GEMM, 256x128 tiles, wave-specialised)",
             "dx": "k_gemm_nf4<true, Bf16> (fused dX GEMM, 256x128 tiles, wave-specialised)"}[dom]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic("gemm_" + dom + "_7b"),
                "kernel": kname, "avg_launch_us": round(dk["avg_us"], 2),
                "flops_per_launch": dk["avg_flops"]}
    other = {k: {"avg_launch_us": round(v["avg_us"], 2),
                 "tflops": round(v["avg_flops"] / (v["avg_us"] * 1e-6) / 1e12, 2)}
             for k, v in per.items()}

    # ------------------------------------------------------- secondary ----
    secondary = None
    if not args.no_secondary:
        secondary = bench_secondary(torch, qlora, synth, dev, evs)
        # the same layer step with LoRA dropout p = 0.05 on every adapter
        # input (the pages' setting), a fresh mask per step and linear
        p_drop = 0.05

        def step_drop(k):
            for i, e in enumerate(lins):
                sd = (k << 8) | i
                qlora.linear_fwd(e["w"], e["X"], e["A"], e["B"], r, alpha, Y=e["Y"], U=e["U"], ws=e["ws_fwd"],
                                 dropout_p=p_drop, seed=sd)
                qlora.linear_bwd(e["w"], e["X"], e["dY"], e["A"], e["B"], r, alpha, e["U"],
                                 dX=e["dX"], dA=e["dA"], dB=e["dB"], ws=e["ws"], dropout_p=p_drop, seed=sd)

        for k in range(2):
            step_drop(k)
        torch.cuda.synchronize()
        t0.record()
        for k in range(args.steps):
            step_drop(100 + k)
        t1.record()
        torch.cuda.synchronize()
        ms_d = t0.elapsed_time(t1) / max(1, args.steps)
        secondary["layer_7b_dropout_0.05"] = {
            "ms_per_step": round(ms_d, 4), "TFLOP/s": round(step_flops / (ms_d * 1e-3) / 1e12, 2),
            "slowdown_vs_no_dropout": round(ms_d / ms_per_step, 4)}

        # the same layer step in the fp16 instance (the bf16 inputs converted
        # exactly to fp16; outputs fp16)
        h = []
        for e in lins:
            f = {k: e[k].to(torch.float16) for k in ("X", "A", "B", "dY")}
            f["Y"] = torch.empty_like(e["Y"], dtype=torch.float16)
            f["U"] = torch.empty_like(e["U"], dtype=torch.float16)
            f["dX"] = torch.empty_like(e["dX"], dtype=torch.float16)
            h.append(f)

        def step_f16():
            for e, f in zip(lins, h):
                qlora.linear_fwd(e["w"], f["X"], f["A"], f["B"], r, alpha, Y=f["Y"], U=f["U"], ws=e["ws_fwd"])
                qlora.linear_bwd(e["w"], f["X"], f["dY"], f["A"], f["B"], r, alpha, f["U"],
                                 dX=f["dX"], dA=e["dA"], dB=e["dB"], ws=e["ws"])

        for _ in range(2):
            step_f16()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            step_f16()
        t1.record()
        torch.cuda.synchronize()
        ms_h = t0.elapsed_time(t1) / max(1, args.steps)
        secondary["layer_7b_fp16"] = {
            "ms_per_step": round(ms_h, 4), "TFLOP/s": round(step_flops / (ms_h * 1e-3) / 1e12, 2),
            "frac_fp16_mfma_peak": round(step_flops / (ms_h * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del h

        # each linear alone: fwd + bwd call pairs timed one by one (10 warmup,
        # 50 timed), median and p10 / p90; the layer figure from the sum of
        # the medians, beside the back-to-back step above
        secondary["per_linear_7b"] = bench_per_linear(lins, qlora, r, alpha, M, evs)

        # the 3B layer (2048 tokens) and the 8B layer (8192 tokens): the same
        # path at the pages' other training shapes
        for wl in ("3b", "8b"):
            secondary[f"layer_{wl}"] = bench_layer(torch, qlora, synth, dev, wl, max(3, args.steps // 4))
        # the 7B layer at 512 tokens: grids of 64-176 tiles, where the fused
        # GEMMs split their reduction
        secondary["layer_7b_512_tokens"] = bench_layer(torch, qlora, synth, dev, "7b", max(3, args.steps // 2),
                                                       tokens=512)

        # context, not a product path: the same layer's 14 products as plain
        # dense bf16 GEMMs in torch.matmul (hipBLASLt) on a bf16 copy of each
        # weight -- what the fused kernels are measured against
        d = []
        for e in lins:
            W = (torch.randn((e["n"], e["k"]), device=dev) * 0.02).to(torch.bfloat16)
            d.append(dict(W=W, Wt=W.t().contiguous(), Y=torch.empty_like(e["Y"]), dX=torch.empty_like(e["dX"])))

        def step_dense():
            for e, f in zip(lins, d):
                torch.matmul(e["X"], f["Wt"], out=f["Y"])
                torch.matmul(e["dY"], f["W"], out=f["dX"])

        for _ in range(2):
            step_dense()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            step_dense()
        t1.record()
        torch.cuda.synchronize()
        ms_dn = t0.elapsed_time(t1) / max(1, args.steps)
        dense_flops = sum(4.0 * M * e["n"] * e["k"] for e in lins)
        secondary["context_dense_bf16_matmul_7b"] = {
            "what": "the 7B layer's 14 GEMMs (Y = X W^T, dX = dY W) as dense bf16 torch.matmul "
                    "(hipBLASLt) on a bf16 weight copy, no adapter and no NF4 decode",
            "ms_per_step": round(ms_dn, 4), "TFLOP/s": round(dense_flops / (ms_dn * 1e-3) / 1e12, 2),
            "frac_bf16_mfma_peak": round(dense_flops / (ms_dn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del d

    # ---------------------------------------------------- cpu baseline ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = bench_cpu(host, r, alpha)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "7B-class decoder layer, 7 NF4-DQ QLoRA linears fwd+bwd "
                               "(q/k/v/o 4096->4096, gate/up 4096->11008, down 11008->4096)",
                   "tokens": M, "rank": r, "alpha": alpha, "block": 64, "dq_group": 256,
                   "parallelism": "single GPU"},
        "pct_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "step_gflop": round(step_flops / 1e9, 2),
        "roofline": roofline,
        "gemm_kernels": other,
        "cpu_baseline": cpu,
        "device": device_info(torch, dev),
        "secondary": secondary,
    }
    print(json.dumps(out))


def bench_per_linear(lins, qlora, r, alpha, M, evs, warmup=10, reps=50):
    """fwd + bwd of each linear of the layer timed per call with HIP events
    on the launch stream: median, p10 and p90 in microseconds."""
    import torch
    out = {}
    tot_fl, tot_ms = 0.0, 0.0
    for e in lins:
        def call():
            qlora.linear_fwd(e["w"], e["X"], e["A"], e["B"], r, alpha, Y=e["Y"], U=e["U"], ws=e["ws_fwd"])
            qlora.linear_bwd(e["w"], e["X"], e["dY"], e["A"], e["B"], r, alpha, e["U"],
                             dX=e["dX"], dA=e["dA"], dB=e["dB"], ws=e["ws"])
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        stream = ctypes.c_void_p(qlora._stream())  # the stream the calls launch on
        ev = [(evs.create(), evs.create()) for _ in range(reps)]
        for a, b in ev:
            if evs.hip.hipEventRecord(a, stream) != 0:
                raise RuntimeError("hipEventRecord failed")
            call()
            if evs.hip.hipEventRecord(b, stream) != 0:
                raise RuntimeError("hipEventRecord failed")
        us = np.array([1e3 * evs.ms(a, b) for a, b in ev])
        for a, b in ev:
            evs.destroy(a)
            evs.destroy(b)
        med = float(np.median(us))
        fl = flops_linear(M, e["n"], e["k"], r)
        out[e["name"]] = {"shape": f"{M}x{e['n']}x{e['k']}", "median_us": round(med, 2),
                          "p10_us": round(float(np.percentile(us, 10)), 2),
                          "p90_us": round(float(np.percentile(us, 90)), 2),
                          "TFLOP/s": round(fl / (med * 1e-6) / 1e12, 2)}
        tot_fl += fl
        tot_ms += med * 1e-3
    out["layer_sum_of_medians"] = {"ms": round(tot_ms, 4), "TFLOP/s": round(tot_fl / (tot_ms * 1e-3) / 1e12, 2),
                                   "frac_bf16_mfma_peak": round(tot_fl / (tot_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


def bench_secondary(torch, qlora, synth, dev, evs, reps=10):
    """70B bandwidth-bound shapes: standalone dequant and few-token forward.
    Three copies of each packed weight are rotated so the 256 MB on-die cache
    cannot hold the weight between calls."""
    res = {}
    for idx in (0, 1):
        lin = synth.LAYERS["70b"][idx]
        rng = synth.rng_for("70b", idx)
        W = torch.from_numpy(synth.draw(rng, (lin.n_out, lin.k_in), 0.02)).to(dev)
        w0 = qlora.quantize(W)
        if idx == 0:
            res["formats_70b_gate"] = bench_formats(torch, qlora, W, reps)
        del W
        copies = [w0] + [qlora.NF4Weight(w0.codes.clone(), w0.absmax_q8.clone(), w0.absmax_scale.clone(),
                                          w0.n_out, w0.k_in) for _ in range(2)]
        out = torch.empty((lin.n_out, lin.k_in), dtype=torch.bfloat16, device=dev)
        nw = lin.n_out * lin.k_in
        if idx == 0:
            res["hbm_ceiling_70b_gate"] = bench_hbm_ceiling(torch, out, reps)
        for c in copies:
            qlora.dequant(c, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps * 3):
            qlora.dequant(copies[i % 3], out)
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / (reps * 3)
        gbs = (PACKED_B_PER_W + 2.0) * nw / (us * 1e-6) / 1e9
        res[f"dequant_70b_{lin.name}"] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                                          "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        if idx == 0:
            # merge the adapter into the weight (bf16 out) and re-quantize it
            rr, alpha = synth.RANK["70b"], synth.ALPHA["70b"]
            dm = synth.linear_inputs(lin.n_out, lin.k_in, 1, rr, synth.rng_for("70b", 30), with_grad=False)
            Am = torch.from_numpy(dm["A"].view(np.int16)).view(torch.bfloat16).to(dev)
            Bm = torch.from_numpy(dm["B"].view(np.int16)).view(torch.bfloat16).to(dev)
            for c in copies:
                qlora.merge(c, Am, Bm, rr, alpha, out)
            torch.cuda.synchronize()
            a.record()
            for i in range(reps * 3):
                qlora.merge(copies[i % 3], Am, Bm, rr, alpha, out)
            b.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / (reps * 3)
            gbs = (PACKED_B_PER_W + 2.0) * nw / (us * 1e-6) / 1e9
            res["merge_70b_gate"] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
            qlora.quantize(out)
            torch.cuda.synchronize()
            a.record()
            for i in range(reps):
                qlora.quantize(out)
            b.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / reps
            gbs = (PACKED_B_PER_W + 2.0) * nw / (us * 1e-6) / 1e9
            res["requantize_70b_gate"] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                                          "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
            del Am, Bm
        del out
        # few-token forward on both weights
        rr, alpha = synth.RANK["70b"], synth.ALPHA["70b"]
        for m in (1, 4, 16):
            d = synth.linear_inputs(lin.n_out, lin.k_in, m, rr, synth.rng_for("70b", 10 + m),
                                    with_grad=False)
            X = torch.from_numpy(d["X"].view(np.int16)).view(torch.bfloat16).to(dev)
            A = torch.from_numpy(d["A"].view(np.int16)).view(torch.bfloat16).to(dev)
            B = torch.from_numpy(d["B"].view(np.int16)).view(torch.bfloat16).to(dev)
            Y = torch.empty((m, lin.n_out), dtype=torch.bfloat16, device=dev)
            U = torch.empty((m, rr), dtype=torch.bfloat16, device=dev)
            ws = qlora.new_workspace(qlora.QLORA_OP_FWD, m, lin.n_out, lin.k_in, rr, dev)
            for c in copies:
                qlora.linear_fwd(c, X, A, B, rr, alpha, Y=Y, U=U, ws=ws)
            torch.cuda.synchronize()
            a.record()
            for i in range(reps * 3):
                qlora.linear_fwd(copies[i % 3], X, A, B, rr, alpha, Y=Y, U=U, ws=ws)
            b.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / (reps * 3)
            byts = (nw * PACKED_B_PER_W + 2 * m * (lin.k_in + lin.n_out)
                    + 2 * rr * (lin.k_in + lin.n_out) + 2 * m * rr)
            gbs = byts / (us * 1e-6) / 1e9
            res[f"fwd_70b_{lin.name}_M{m}"] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                                               "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        del copies, w0
        torch.cuda.empty_cache()
    # the 2-byte-per-weight output alone, written at the measured plain-write
    # rate, bounds each of these kernels' time from below (gate and down hold
    # the same number of weights)
    t_floor = res["hbm_ceiling_70b_gate"]["write_us"]
    for key in [k for k in res if k.startswith(("dequant_70b", "merge_70b", "requantize_70b"))]:
        res[key]["frac_plain_write_ceiling"] = round(t_floor / res[key]["us"], 4)
    return res


def bench_hbm_ceiling(torch, out, reps):
    """Plain-write and plain-copy rates of this GPU on a 16-bit buffer of the
    70B gate's size (the dequantized weight, 2 bytes per weight), with torch's
    own fill and copy kernels: what any kernel that writes these bytes can
    approach.  The copy source is a second buffer of the same size."""
    src = torch.empty_like(out)
    src.fill_(0.5)
    nbytes = out.numel() * out.element_size()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"bytes": nbytes}
    for name, fn, moved in (("write", lambda: out.fill_(1.0), nbytes), ("copy", lambda: out.copy_(src), 2 * nbytes)):
        fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps * 3):
            fn()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / (reps * 3)
        res[f"{name}_us"] = round(us, 2)
        res[f"{name}_GB/s"] = round(moved / (us * 1e-6) / 1e9, 1)
        res[f"{name}_frac_hbm"] = round(moved / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    del src
    return res


def bench_layer(torch, qlora, synth, dev, wl, steps, tokens=None):
    """fwd+bwd of the 7 linears of a decoder layer at its token count (or
    `tokens`) on device-generated N(0, 0.02^2) weights and N(0, 1) inputs."""
    M, r, alpha = tokens or synth.TOKENS[wl], synth.RANK[wl], synth.ALPHA[wl]
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    lins = []
    for lin in synth.LAYERS[wl]:
        n, k = lin.n_out, lin.k_in
        W = torch.randn((n, k), device=dev, generator=g) * 0.02
        e = dict(n=n, k=k, w=qlora.quantize(W))
        del W
        bf = lambda *shape, sd=1.0: (torch.randn(shape, device=dev, generator=g) * sd).to(torch.bfloat16)
        e.update(X=bf(M, k), A=bf(r, k, sd=k ** -0.5), B=bf(n, r, sd=0.01), dY=bf(M, n))
        e.update(Y=torch.empty((M, n), dtype=torch.bfloat16, device=dev),
                 U=torch.empty((M, r), dtype=torch.bfloat16, device=dev),
                 dX=torch.empty((M, k), dtype=torch.bfloat16, device=dev),
                 dA=torch.empty((r, k), dtype=torch.float32, device=dev),
                 dB=torch.empty((n, r), dtype=torch.float32, device=dev),
                 ws=qlora.new_workspace(qlora.QLORA_OP_BWD, M, n, k, r, dev),
                 ws_fwd=qlora.new_workspace(qlora.QLORA_OP_FWD, M, n, k, r, dev))
        lins.append(e)

    def step():
        for e in lins:
            qlora.linear_fwd(e["w"], e["X"], e["A"], e["B"], r, alpha, Y=e["Y"], U=e["U"], ws=e["ws_fwd"])
            qlora.linear_bwd(e["w"], e["X"], e["dY"], e["A"], e["B"], r, alpha, e["U"],
                             dX=e["dX"], dA=e["dA"], dB=e["dB"], ws=e["ws"])

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    fl = sum(flops_linear(M, e["n"], e["k"], r) for e in lins)
    del lins
    torch.cuda.empty_cache()
    return {"tokens": M, "steps": steps, "ms_per_step": round(ms, 4), "step_gflop": round(fl / 1e9, 2),
            "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def bench_formats(torch, qlora, W, reps):
    """The storage formats the pages weigh NF4-DQ against, on one weight:
    bits per weight, relative Frobenius error of the decoded bf16 weight, and
    standalone dequant time (3 rotated copies) and bandwidth."""
    out = {}
    n, k = W.shape
    nw = n * k
    Wd = W.double()
    wnorm = float(torch.linalg.vector_norm(Wd))
    dst = torch.empty((n, k), dtype=torch.bfloat16, device=W.device)
    for fmt in ("nf4_dq", "nf4", "int4_dq", "int4"):
        copies = [qlora.quantize_format(W, fmt) for _ in range(3)]
        qlora.dequant_format(copies[0], dst)
        torch.cuda.synchronize()
        err = float(torch.linalg.vector_norm(dst.double() - Wd)) / wnorm
        packed = copies[0].nbytes()
        for c in copies:
            qlora.dequant_format(c, dst)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(3 * reps):
            qlora.dequant_format(copies[i % 3], dst)
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / (3 * reps)
        gbs = (packed + 2 * nw) / (us * 1e-6) / 1e9
        out[fmt] = {"bits_per_weight": round(8 * packed / nw, 4), "rel_error": round(err, 5),
                    "dequant_us": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        del copies
    del Wd, dst
    return out


def bench_cpu(host, r, alpha, m_sample=2048, min_seconds=10.0):
    """The CPU oracle as it stands on a bounded sample of the same step:
    dequant + forward + backward of all seven linears for the first
    `m_sample` tokens.  The oracle quantizes each weight itself first
    (untimed, like the GPU's one-time quantization)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    qs = [oracle.quantize_nf4_dq(d["W"]) for d in host]
    t = time.perf_counter()
    fl = 0
    passes = 0
    # whole passes until about 10 s of CPU work (at most 8 passes)
    while passes < 8 and (passes == 0 or time.perf_counter() - t < min_seconds):
        for d, q in zip(host, qs):
            n, k = d["n_out"], d["k_in"]
            _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], n, k)
            oracle.linear_fwd(wb, d["X"][:m_sample], d["A"], d["B"], alpha, r)
            oracle.linear_bwd(wb, d["X"][:m_sample], d["dY"][:m_sample], d["A"], d["B"], alpha, r)
            fl += flops_linear(m_sample, n, k, r)
        passes += 1
    sec = time.perf_counter() - t
    return {"value": round(fl / sec / 1e12, 4), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"all 7 linears of the 7B layer at {m_sample} of 2048 tokens: oracle dequant + "
                      f"fwd + bwd in fp64 numpy, {passes} pass(es) in {sec:.1f} s",
            "seconds": round(sec, 2), "cpu": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def device_info(torch, dev):
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1)}


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-NF4 linear hot path on one MI355X.

One step = one pass of the whole path over one batch, for every linear of the
workload: NF4 quantisation with double quantisation of the fp32 weight,
dequantisation to bf16, the fused forward, and the backward (dX, dA, dB).
Inputs are drawn once and stay resident in HBM; the weight is rotated over
several copies (> 256 MB in total) so the quantiser does not read it from the
Infinity Cache.

Prints one JSON line.  `value` is the step's algorithmic fwd+bwd flops
(4MNK + 6Mr(K+N) per linear) over the measured step time, in TFLOP/s.
`roofline` describes the dominant kernel, timed with HIP events recorded on
its launch stream around every launch inside the timed region.
`cpu_baseline` times the CPU oracle on the same workload (rank 0, N = 1).

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload 2]
"""

import argparse
import json
import os
import sys
import time

METRIC = "QLoRA linear fwd+bwd TFLOP/s and quantize GB/s (fraction of roofline), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

# Algorithmic bytes per weight: packed codes 0.5 + FP8 constant 1/64 +
# fp32 second-level scale 4/16384 (the 4-byte mean is per tensor).
STORED_BYTES_PER_PARAM = 0.5 + 1.0 / 64 + 4.0 / 16384
QUANT_BYTES_PER_PARAM = 4.0 + STORED_BYTES_PER_PARAM      # fp32 in
DEQUANT_BYTES_PER_PARAM = STORED_BYTES_PER_PARAM + 2.0    # bf16 out

WORKLOAD_NAMES = {
    1: "tiny: W 256x256 NF4+DQ, X 16x256 bf16, r=8, alpha=16",
    2: "7B attention projection: W 4096x4096 NF4+DQ, X 4096x4096 bf16 (4 x 1024 tokens), r=64, alpha=16",
    3: "7B MLP block: gate/up 11008x4096 + down 4096x11008 NF4+DQ, 2048 tokens, r=64, alpha=16",
    4: "65B-shaped MLP: gate/up 22016x8192 + down 8192x22016 NF4+DQ (Student-t), 8192 tokens, r=64, alpha=16",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--rotate", type=int, default=0, help="weight copies (0: enough for > 256 MB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded, so the
    library can record them on its launch stream (torch.cuda.Event objects
    are created lazily and track their own recording state)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def create(self):
        h = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.pool.append(h)
        return h

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed (event not recorded?)")
        return ms.value

    def close(self):
        for h in self.pool:
            self.hip.hipEventDestroy(h)
        self.pool = []


def linear_flops(lin):
    return 4 * lin.M * lin.N * lin.K + 6 * lin.M * lin.r * (lin.K + lin.N)


def cpu_baseline(lin, tensors):
    """Time the CPU oracle on one full step of one linear: quantise with double
    quantisation, dequantise, forward and backward in fp64."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import blockwise, linear

    W = tensors["W"].cpu().numpy()
    X, A, Bm, dY = (tensors[k].float().cpu().numpy() for k in ("X", "A", "B", "dY"))
    t0 = time.perf_counter()
    st = blockwise.quantize(W, double_quant=True)
    Wb = blockwise.bf16_round(st.dequantize())
    Y, XA = linear.forward(X, Wb, A, Bm, lin.s)
    dX, dA, dB = linear.backward(dY, X, Wb, A, Bm, lin.s)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    del Y, XA, dX, dA, dB, np
    return {
        "value": linear_flops(lin) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"one full step of the {lin.name} linear ({lin.N}x{lin.K} weight, {lin.M} tokens, r={lin.r}): "
                   f"oracle quantise+DQ, dequantise, fwd and bwd in fp64 numpy; {dt:.2f} s; "
                   f"BLAS threads {threads}, os.cpu_count() {os.cpu_count()}"),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_nf4_quantized_quantize_amd import binding as B
    from bit_nf4_quantized_quantize_amd import synth

    B.lib()  # raises if the HIP library is missing: there is no fallback
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bf = torch.bfloat16

    lins = synth.workload(args.workload)
    wbytes = sum(l.N * l.K * 4 for l in lins)
    rotate = args.rotate or max(1, -(-(300 << 20) // wbytes))
    layers = []
    for lin in lins:
        t = lin.draw(dev)
        st = {
            "lin": lin, "t": t,
            "W": [t["W"]] + [t["W"].clone() for _ in range(rotate - 1)],
            "qw": B.NF4Weight(lin.N, lin.K, True, dev),
            "Wd": torch.empty(lin.N, lin.K, dtype=bf, device=dev),
            "Y": torch.empty(lin.M, lin.N, dtype=bf, device=dev),
            "XA": torch.empty(lin.M, lin.r, dtype=bf, device=dev),
            "dX": torch.empty(lin.M, lin.K, dtype=bf, device=dev),
            "dA": torch.empty(lin.K, lin.r, dtype=bf, device=dev),
            "dB": torch.empty(lin.r, lin.N, dtype=bf, device=dev),
            "ws": B.Workspace(),
            "qws": torch.empty(max(B.qlora_nf4_quantize_workspace(lin.N * lin.K, True), 16),
                               dtype=torch.uint8, device=dev),
        }
        layers.append(st)

    kernels = ("quantize", "dequantize", "fwd_main", "bwd_dx")
    phases = ("quantize", "dequantize", "fwd", "bwd")
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    hev = HipEvents()
    # one event pair per (timed step, linear, kernel), created before timing
    kpool = [[{k: (hev.create(), hev.create()) for k in kernels} for _ in layers] for _ in range(args.steps)]

    def step(i, rec):
        for li, L in enumerate(layers):
            lin, t = L["lin"], L["t"]
            kev = kpool[i][li] if rec is not None else None
            if kev:
                for k in kernels:
                    B.lib().qlora_profile_events(B.QLORA_KERNEL[k], kev[k][0], kev[k][1])
            pe = [ev() for _ in range(5)] if rec is not None else None
            if pe:
                pe[0].record()
            B.qlora_nf4_quantize(L["W"][i % rotate], double_quant=True, out=L["qw"], workspace=L["qws"])
            if pe:
                pe[1].record()
            B.qlora_nf4_dequantize(L["qw"], bf, out=L["Wd"])
            if pe:
                pe[2].record()
            B.qlora_linear_fwd(t["X"], L["qw"], t["A"], t["B"], lin.s, Y=L["Y"], XA=L["XA"], workspace=L["ws"])
            if pe:
                pe[3].record()
            B.qlora_linear_bwd(t["dY"], t["X"], L["XA"], L["qw"], t["A"], t["B"], lin.s,
                               dX=L["dX"], dA=L["dA"], dB=L["dB"], workspace=L["ws"])
            if pe:
                pe[4].record()
                rec.append((li, kev, pe))
        if rec is not None:
            for k in kernels:
                B.lib().qlora_profile_events(B.QLORA_KERNEL[k], None, None)

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    rec = []
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i, rec)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(stop) / args.steps

    # per-kernel and per-phase averages (microseconds), per linear
    per = []
    for li, L in enumerate(layers):
        kt = {k: [] for k in kernels}
        pt = {p: [] for p in phases}
        for (lj, kev, pe) in rec:
            if lj != li:
                continue
            for k in kernels:
                kt[k].append(hev.elapsed_ms(kev[k][0], kev[k][1]) * 1e3)
            for j, p in enumerate(phases):
                pt[p].append(pe[j].elapsed_time(pe[j + 1]) * 1e3)
        per.append(({k: sum(v) / len(v) for k, v in kt.items()}, {p: sum(v) / len(v) for p, v in pt.items()}))

    hev.close()
    breakdown = []
    dominant = None
    for (kt, pt), L in zip(per, layers):
        lin = L["lin"]
        p = lin.N * lin.K
        fwd_main_flops = 2 * lin.M * lin.N * lin.K + 2 * lin.M * lin.r * lin.N
        bwd_dx_flops = 2 * lin.M * lin.N * lin.K + 2 * lin.M * lin.r * lin.K
        rows = {
            "linear": lin.name, "M": lin.M, "N": lin.N, "K": lin.K, "r": lin.r,
            "quantize_call_us": pt["quantize"], "quantize_kernel_us": kt["quantize"],
            "quantize_GBps": QUANT_BYTES_PER_PARAM * p / pt["quantize"] / 1e3,
            "dequantize_us": kt["dequantize"],
            "dequantize_GBps": DEQUANT_BYTES_PER_PARAM * p / kt["dequantize"] / 1e3,
            "fwd_us": pt["fwd"], "fwd_main_kernel_us": kt["fwd_main"],
            "fwd_TFLOPs": (2 * lin.M * lin.N * lin.K + 2 * lin.M * lin.r * (lin.K + lin.N)) / pt["fwd"] / 1e6,
            "bwd_us": pt["bwd"], "bwd_dx_kernel_us": kt["bwd_dx"],
            "bwd_TFLOPs": (2 * lin.M * lin.N * lin.K + 4 * lin.M * lin.r * (lin.K + lin.N)) / pt["bwd"] / 1e6,
        }
        breakdown.append(rows)
        cands = [
            ("fwd_main", "mfma", fwd_main_flops, kt["fwd_main"]),
            ("bwd_dx", "mfma", bwd_dx_flops, kt["bwd_dx"]),
            ("quantize", "hbm", (4.0 + 0.5) * p + 4.0 * (p // 64), kt["quantize"]),
            ("dequantize", "hbm", DEQUANT_BYTES_PER_PARAM * p, kt["dequantize"]),
        ]
        for c in cands:
            if dominant is None or c[3] > dominant[3]:
                dominant = c + (lin.name,)

    name, bound, work, us, lname = dominant
    if bound == "mfma":
        achieved = work / us / 1e6
        roof = {"kernel": name, "linear": lname, "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                "algorithmic_per_launch": work, "avg_launch_us": us}
    else:
        achieved = work / us / 1e3
        roof = {"kernel": name, "linear": lname, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "algorithmic_per_launch": work, "avg_launch_us": us}

    flops = sum(linear_flops(L["lin"]) for L in layers)
    value = flops / (ms_per_step / 1e3) / 1e12
    q_bytes = sum(QUANT_BYTES_PER_PARAM * L["lin"].N * L["lin"].K for L in layers)
    q_us = sum(b["quantize_call_us"] for b in breakdown)

    cpu = None
    if not args.no_cpu_baseline:
        L0 = layers[0]
        cpu = cpu_baseline(L0["lin"], L0["t"])

    lin0 = layers[0]["lin"]
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.workload],
            "linears": [{"name": L["lin"].name, "M": L["lin"].M, "N": L["lin"].N, "K": L["lin"].K,
                         "r": L["lin"].r, "alpha": L["lin"].alpha} for L in layers],
            "global_batch": lin0.M, "weight_copies_rotated": rotate,
            "step": "quantize+DQ, dequantize->bf16, fwd, bwd (dX, dA, dB) per linear",
        },
        "quantize": {"GB/s": q_bytes / q_us / 1e3, "frac_hbm": q_bytes / q_us / 1e3 / HBM_PEAK_GBS,
                     "bytes_per_param": QUANT_BYTES_PER_PARAM},
        "roofline": roof,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

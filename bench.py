#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-NF4 linear hot path on one MI355X.

One step = one pass of the whole path over one batch, for every linear of the
workload: NF4 quantisation with double quantisation of the fp32 weight,
dequantisation to bf16, the fused forward, and the backward (dX, dA, dB),
taken phase by phase over the linears.  The default workload is the largest
that fits one GPU, the 65B-shaped MLP layer (gate and up 22016x8192, down
8192x22016, 8192 tokens, Student-t weights); its line also carries the 7B
attention projection (4096x4096, 4096 tokens) under "attn_4096" and the
small-batch forward (1, 4 and 16 tokens against the 8192x22016 weight, GB/s,
with the 32-layer 7B quantise/dequantise sweep) under "small_batch".
Inputs are drawn once and stay resident in HBM; the fp32 weights are rotated
over more than 1 GB of copies and the quantise and dequantise phases are
timed one call at a time after a 1 GiB cache scrub, so no input comes from
the 256 MB Infinity Cache.

Measurement:
  1. W untimed warm-up steps;
  2. a breakdown pass: a few steps with HIP events around every library
     kernel of interest (each event costs the stream a few us, so this pass
     is not used for `value`), then each phase timed per call;
  3. the timed region: K steps bracketed by synchronisation, with events
     only around the dominant kernel (found in pass 2), recorded by the
     library on the kernel's own launch stream; its mean duration over the
     K launches gives `roofline.achieved`.
"achievable" is what the device streams in a plain copy and a plain read.

Prints one JSON line.  `value` is the step's algorithmic fwd+bwd flops
(4MNK + 6Mr(K+N) per linear) over the measured step time, in TFLOP/s (GB/s
of algorithmic bytes for workload 5).  `cpu_baseline` times the CPU oracle
on a bounded sample of the same workload (rank 0, N = 1), scaled to it.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload 4]
"""

import argparse
import json
import os
import sys
import time

METRIC = "QLoRA linear fwd+bwd TFLOP/s and quantize GB/s (fraction of roofline), 1 GPU"
SMALL_METRIC = "QLoRA small-batch forward GB/s (fraction of HBM roofline), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

# Algorithmic bytes per weight: packed codes 0.5 + FP8 constant 1/64 +
# fp32 second-level scale 4/16384 (the 4-byte mean is per tensor).
STORED_BYTES_PER_PARAM = 0.5 + 1.0 / 64 + 4.0 / 16384
QUANT_BYTES_PER_PARAM = 4.0 + STORED_BYTES_PER_PARAM      # fp32 in
DEQUANT_BYTES_PER_PARAM = STORED_BYTES_PER_PARAM + 2.0    # bf16 out

# HBM bytes per launch of the dominant kernels, from two rocprofv3 counter
# runs (FETCH_SIZE, WRITE_SIZE; each scaled by what it reads for a plain copy
# of known size; profiles/*_hbm_bytes.md give the commands and tables).  Valid
# only for the kernel sources they were taken on: `traffic` is null when the
# digest of those sources differs.
KERNEL_SOURCES = ("csrc/linear.hip", "csrc/quantize.hip", "csrc/device.h", "csrc/codebooks.h")
TRAFFIC_DIGEST = "831fb0751b08e428"
TRAFFIC_BYTES = {
    (4, "fwd_main"): 4202.1e6 + 323.3e6,
    (4, "bwd_dx"): 3458.2e6 + 217.9e6,
    (4, "quantize"): 721.5e6 + 103.6e6,
    (4, "dequantize"): 93.6e6 + 360.7e6,
    (2, "bwd_dx"): 108.1e6 + 35.6e6,
    (2, "fwd_main"): 112.4e6 + 38.0e6,
    (2, "quantize"): 67.3e6 + 9.5e6,
    (2, "dequantize"): 8.7e6 + 33.6e6,
    (5, "fwd_main"): 99.2e6 + 2.0e6,
}


def kernel_digest():
    import hashlib
    from bit_nf4_quantized_quantize_amd import binding
    root = os.path.dirname(os.path.abspath(binding.__file__))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


WORKLOAD_NAMES = {
    1: "tiny: W 256x256 NF4+DQ, X 16x256 bf16, r=8, alpha=16",
    2: "7B attention projection: W 4096x4096 NF4+DQ, X 4096x4096 bf16 (4 x 1024 tokens), r=64, alpha=16",
    3: "7B MLP block: gate/up 11008x4096 + down 4096x11008 NF4+DQ, 2048 tokens, r=64, alpha=16",
    4: "65B-shaped MLP: gate/up 22016x8192 + down 8192x22016 NF4+DQ (Student-t), 8192 tokens, r=64, alpha=16",
    5: "small batch: 1, 4 and 16 tokens against the 8192x22016 NF4+DQ weight (Student-t), r=64, alpha=16, fwd only",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=4, choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--rotate", type=int, default=0, help="weight copies (0: enough for > 256 MB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="measure only the chosen workload (no achievable-bandwidth probe; for workload 4 no "
                        "7B-attention and small-batch keys)")
    p.add_argument("--no-sweep", action="store_true", help="workload 5: skip the 32-layer 7B quantise/dequantise sweep")
    p.add_argument("--no-code-types", action="store_true",
                   help="workload 2: skip the extra measurements (storage types, LoRA dropout, optimizer "
                        "step, decoder block)")
    p.add_argument("--no-block", action="store_true",
                   help="workload 2: skip the decoder-block measurement (its linears have other shapes, so "
                        "per-kernel counter averages of a profiled run stay those of the workload)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="first run a plain device copy of this many MiB three times (a known-size kernel that "
                        "calibrates hardware byte counters taken over the same run)")
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


def _blas_threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def cpu_baseline(lin, tensors, min_s=10.0, max_steps=20):
    """Time the CPU oracle on full steps of one linear (quantise with double
    quantisation, dequantise, forward and backward in fp64), repeated until
    about min_s seconds of CPU work have run."""
    from oracle import blockwise, linear

    W = tensors["W"].cpu().numpy()
    X, A, Bm, dY = (tensors[k].float().cpu().numpy() for k in ("X", "A", "B", "dY"))
    t0 = time.perf_counter()
    n = 0
    while n < max_steps and (n == 0 or time.perf_counter() - t0 < min_s):
        st = blockwise.quantize(W, double_quant=True)
        Wb = blockwise.bf16_round(st.dequantize())
        Y, XA = linear.forward(X, Wb, A, Bm, lin.s)
        dX, dA, dB = linear.backward(dY, X, Wb, A, Bm, lin.s)
        del st, Wb, Y, XA, dX, dA, dB
        n += 1
    dt = (time.perf_counter() - t0) / n
    threads = _blas_threads()
    return {
        "value": linear_flops(lin) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n} full steps of the {lin.name} linear ({lin.N}x{lin.K} weight, {lin.M} tokens, r={lin.r}): "
                   f"oracle quantise+DQ, dequantise, fwd and bwd in fp64 numpy; {dt:.2f} s per step; "
                   f"BLAS threads {threads}, os.cpu_count() {os.cpu_count()}"),
    }


def cpu_baseline_scaled(lins, tensors, rows=5504, tokens=1024):
    """The CPU oracle on a bounded sample of the 65B-shaped step, scaled to
    the whole step (the whole step is 18 TFLOP of fp64 products plus the
    quantisation of 541M weights, minutes of CPU time): quantise+DQ and
    dequantise a `rows`-row slice of the first linear's fp32 weight, scaled
    by parameter count to all three weights; forward and backward of the first
    linear over `tokens` tokens (fp64 products against that slice's bf16
    weight, completed to the full weight by flop count), scaled by flops to
    every linear at its full token count."""
    from oracle import blockwise, linear

    lin0 = lins[0]
    W = tensors["W"][:rows].cpu().numpy()
    X = tensors["X"][:tokens].float().cpu().numpy()
    A, Bm = tensors["A"].float().cpu().numpy(), tensors["B"].float().cpu().numpy()[:, :rows]
    dY = tensors["dY"][:tokens, :rows].float().cpu().numpy()
    t0 = time.perf_counter()
    st = blockwise.quantize(W, double_quant=True)
    Wb = blockwise.bf16_round(st.dequantize())
    t_q = time.perf_counter() - t0
    t0 = time.perf_counter()
    Y, XA = linear.forward(X, Wb, A, Bm, lin0.s)
    dX, dA, dB = linear.backward(dY, X, Wb, A, Bm, lin0.s)
    t_g = time.perf_counter() - t0
    del st, Wb, Y, XA, dX, dA, dB
    sample_params = rows * lin0.K
    sample_flops = 4 * tokens * rows * lin0.K + 6 * tokens * lin0.r * (lin0.K + rows)
    params = sum(l.N * l.K for l in lins)
    flops = sum(linear_flops(l) for l in lins)
    t_step = t_q * params / sample_params + t_g * flops / sample_flops
    threads = _blas_threads()
    return {
        "value": flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"oracle quantise+DQ and dequantise of a {rows}x{lin0.K} slice of the {lin0.name} weight "
                   f"({t_q:.2f} s, scaled by parameters to the 3 weights), fwd+bwd in fp64 numpy over {tokens} "
                   f"tokens against that slice ({t_g:.2f} s, scaled by flops to the 3 linears at {lin0.M} tokens); "
                   f"{t_step:.1f} s per step estimated; BLAS threads {threads}, os.cpu_count() {os.cpu_count()}"),
    }


def cpu_baseline_small(L, rows=1024, min_s=10.0, max_reps=50):
    """Time the CPU oracle's forward at the largest token count on a slice of
    the weight's rows (dequantise the slice from its stored state, then the
    fp64 product), repeated for about min_s seconds; GB/s over the same
    algorithmic bytes per weight as the GPU figure."""
    import torch

    from oracle import blockwise, linear

    lin = L["lin"]
    g = torch.Generator().manual_seed(1234)
    Wr = (torch.randn(rows, lin.K, generator=g) * 0.02).numpy()
    st = blockwise.quantize(Wr, double_quant=True)
    X = L["X"].float().cpu().numpy()
    A = L["A"].float().cpu().numpy()
    Bm = L["B"].float().cpu().numpy()[:, :rows]
    t0 = time.perf_counter()
    n = 0
    while n < max_reps and (n == 0 or time.perf_counter() - t0 < min_s):
        Wb = blockwise.bf16_round(st.dequantize())
        Y, XA = linear.forward(X, Wb, A, Bm, lin.s)
        del Wb, Y, XA
        n += 1
    dt = (time.perf_counter() - t0) / n
    gb = STORED_BYTES_PER_PARAM * rows * lin.K + 2 * lin.M * (lin.K + rows) + 2 * lin.r * (lin.K + rows)
    threads = _blas_threads()
    return {
        "value": gb / dt / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n} forwards of {lin.M} tokens against a {rows}x{lin.K} slice of the weight (oracle "
                   f"dequantise from the stored NF4+DQ state, fp64 product); {dt * 1e3:.1f} ms each; "
                   f"BLAS threads {threads}, os.cpu_count() {os.cpu_count()}"),
    }


def run_sweep(B, synth, dev, reps=3):
    """The 32-layer 7B-shaped sweep: every fp32 weight (224 matrices, 6.48e9
    parameters, each drawn with its own seed and resident in HBM) is quantised
    with double quantisation (one batched call, and as 224 single calls), then
    every stored weight is dequantised to its own bf16 output.  Each pass (224 back-to-back calls) is timed between two
    events, `reps` times after a warm-up pass; the median pass is reported,
    with the host time to enqueue a pass (the GPU time is only meaningful
    while that stays below it)."""
    import torch

    shapes = synth.sweep_7b_shapes()
    ws_bytes = max(B.qlora_nf4_quantize_workspace(n * k, True) for n, k in shapes)
    qws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    W, Q, D = [], [], []
    for i, (n, k) in enumerate(shapes):
        W.append(synth.sweep_weight(i, dev))
        Q.append(B.NF4Weight(n, k, True, dev))
        D.append(torch.empty(n, k, dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()

    def timed(fn):
        times, enq = [], 0.0
        for p in range(reps + 1):                 # the first pass is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record()
            for i in range(len(shapes)):
                fn(i)
            e1.record()
            t1 = time.perf_counter()
            torch.cuda.synchronize()
            if p > 0:
                times.append(e0.elapsed_time(e1))
                enq = max(enq, (t1 - t0) * 1e3)
        return sorted(times)[len(times) // 2], enq

    q1_ms, q1_enq = timed(lambda i: B.qlora_nf4_quantize(W[i], double_quant=True, out=Q[i], workspace=qws))
    del qws
    nbw = ctypes_workspace_bytes(B, Q)
    bws = torch.empty(max(nbw, 16), dtype=torch.uint8, device=dev)

    def batched(i):  # the whole sweep in one batched call (issued at i == 0)
        if i == 0:
            B.qlora_nf4_quantize_batched(W, Q, workspace=bws)
    q_ms, q_enq = timed(batched)
    d_ms, d_enq = timed(lambda i: B.qlora_nf4_dequantize(Q[i], torch.bfloat16, out=D[i]))
    params = sum(n * k for n, k in shapes)
    qb, db = QUANT_BYTES_PER_PARAM * params, DEQUANT_BYTES_PER_PARAM * params
    del W, Q, D, bws
    torch.cuda.empty_cache()
    return {
        "matrices": len(shapes), "params": params, "passes": reps,
        "quantize_ms": q_ms, "quantize_GBps": qb / q_ms / 1e6, "quantize_frac_hbm": qb / q_ms / 1e6 / HBM_PEAK_GBS,
        "quantize_how": "one qlora_nf4_quantize_batched call for all 224 matrices",
        "quantize_single_calls_ms": q1_ms, "quantize_single_calls_GBps": qb / q1_ms / 1e6,
        "dequantize_ms": d_ms, "dequantize_GBps": db / d_ms / 1e6,
        "dequantize_frac_hbm": db / d_ms / 1e6 / HBM_PEAK_GBS,
        "host_enqueue_ms": {"quantize": q_enq, "quantize_single_calls": q1_enq, "dequantize": d_enq},
        "bytes_per_param": {"quantize": QUANT_BYTES_PER_PARAM, "dequantize": DEQUANT_BYTES_PER_PARAM},
    }


def ctypes_workspace_bytes(B, weights):
    """Workspace bytes of one batched quantisation of `weights`."""
    import ctypes
    descs = (B.qlora_nf4_t * len(weights))(*[q.desc() for q in weights])
    n = ctypes.c_int64(0)
    B._check(B.lib().qlora_nf4_quantize_batched_workspace(descs, len(weights), ctypes.byref(n)),
             "qlora_nf4_quantize_batched_workspace")
    return n.value


def run_code_types(B, L, dev, reps=10):
    """Section 3's data-type comparison on the same kernels: the layer's
    N(0, 0.02^2) fp32 weight stored as NF4, FP4 E2M1, FP4 E3M0 and Int4, and
    as blockwise Int8 (Eq. 1; all with double quantisation).  Per type: the
    reconstruction error of the dequantised weight (||W_hat - W|| / ||W||,
    fp32 on the device), and the median over `reps` calls of the quantise
    call, the bf16 dequantise call and one forward + backward (Int8 on the
    generic GEMM tiles), each between two events."""
    import torch

    lin, t = L["lin"], L["t"]
    W = L["W"][0]
    bf = torch.bfloat16
    res = {}

    def med(fn):
        ts = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    for name, ct in list(B.CODE_TYPES.items()) + [("int8", B.QLORA_CODE_INT8)]:
        qw = B.NF4Weight(lin.N, lin.K, True, dev, ct)
        q_us = med(lambda: B.qlora_nf4_quantize(W, double_quant=True, out=qw, workspace=L["qws"]))
        d_us = med(lambda: B.qlora_nf4_dequantize(qw, bf, out=L["Wd"]))
        Wd32 = B.qlora_nf4_dequantize(qw, torch.float32)
        err = float(torch.linalg.vector_norm((Wd32 - W).double()) / torch.linalg.vector_norm(W.double()))
        del Wd32

        def fb():
            B.qlora_linear_fwd(t["X"], qw, t["A"], t["B"], lin.s, Y=L["Y"], XA=L["XA"], workspace=L["ws"])
            B.qlora_linear_bwd(t["dY"], t["X"], L["XA"], qw, t["A"], t["B"], lin.s,
                               dX=L["dX"], dA=L["dA"], dB=L["dB"], workspace=L["ws"])
        fb_us = med(fb)
        p = lin.N * lin.K
        code_bytes = 1.0 if ct == B.QLORA_CODE_INT8 else 0.5  # Int8 stores a byte per weight, not a nibble
        res[name] = {"rel_rms_error": err,
                     "quantize_us": q_us,
                     "quantize_GBps": (QUANT_BYTES_PER_PARAM + code_bytes - 0.5) * p / q_us / 1e3,
                     "dequantize_us": d_us,
                     "dequantize_GBps": (DEQUANT_BYTES_PER_PARAM + code_bytes - 0.5) * p / d_us / 1e3,
                     "fwd_bwd_us": fb_us, "fwd_bwd_TFLOPs": linear_flops(lin) / fb_us / 1e6}
        del qw
    return res


def run_block(dev, reps=5):
    """The whole-layer workload behind the memory discussion (QLoRA section
    2, "Memory Requirement of Parameter-Efficient Finetuning", and Appendix
    G, Figure 6: batch 1, sequence 512, gradient checkpointing): a
    LLaMA-7B-shaped decoder block (hidden 4096, MLP 11008, 32 heads) with
    r = 64, alpha = 16 adapters on all seven linears, fwd + bwd with and
    without checkpointing.  Per batch size: the activation bytes the forward
    leaves for the backward, the peak bytes above the resident state during
    fwd + bwd (adapter gradients included), and the median fwd + bwd time.
    Resident state: the NF4+DQ weights, the bf16 adapters, and (computed,
    not allocated here) their bf16 gradients and the optimizer's fp32
    master weights and Adam moments."""
    import torch
    from bit_nf4_quantized_quantize_amd import block as BLK
    from bit_nf4_quantized_quantize_amd import synth

    hidden, mlp, heads, r, alpha, seq = 4096, 11008, 32, 64, 16, 512
    W, A, Bm = {}, {}, {}
    for i, (n, sh) in enumerate(BLK.linear_shapes(hidden, mlp).items()):
        W[n] = synth.weight(sh, "normal", synth.seed_of(6, i, "W"), dev)
        A[n] = synth.normal((sh[1], r), 0.01, synth.seed_of(6, i, "A"), dev)
        Bm[n] = synth.normal((r, sh[0]), 0.01, synth.seed_of(6, i, "B"), dev)
    ones = torch.ones(hidden, device=dev)
    blk = BLK.QLoraBlock(W, A, Bm, ones, ones, alpha / r, heads)
    del W, A, Bm
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    nparam = sum(p.numel() for p in blk.parameters())
    res = {"config": {"hidden": hidden, "mlp": mlp, "heads": heads, "r": r, "alpha": alpha, "seq": seq,
                      "linears": list(BLK.LINEARS)},
           "weight_bytes": blk.weight_bytes(), "adapter_bytes": blk.adapter_bytes(),
           "adapter_grad_bytes": 2 * nparam, "optimizer_state_bytes": 12 * nparam, "runs": []}

    def fwd_bwd(xg, dy, ck):
        for p in blk.parameters():
            p.grad = None
        y = blk(xg, checkpoint=ck)
        y.backward(dy)
        return y

    for batch in (1, 4):
        x = synth.normal((batch, seq, hidden), 1.0, synth.seed_of(6, 8, "X"), dev)
        dy = synth.normal((batch, seq, hidden), 1.0, synth.seed_of(6, 8, "dY"), dev)
        for ck in (False, True):
            xg = x.clone().requires_grad_(True)
            fwd_bwd(xg, dy, ck)  # warm-up: workspaces, allocator pools
            for p in blk.parameters():
                p.grad = None
            xg.grad = None
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            base = torch.cuda.memory_allocated()
            y = blk(xg, checkpoint=ck)
            torch.cuda.synchronize()
            held = torch.cuda.memory_allocated() - base - y.numel() * y.element_size()
            y.backward(dy)
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated() - base
            del y
            ts = []
            for _ in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                xg.grad = None
                e0.record()
                fwd_bwd(xg, dy, ck)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ts = sorted(ts[1:])
            # saved_activation_bytes: held between forward and backward beyond
            # the block input itself (which the caller keeps either way)
            res["runs"].append({"batch": batch, "checkpoint": ck, "saved_activation_bytes": held,
                                "saved_per_sequence_bytes": held / batch,
                                "block_input_bytes": x.numel() * x.element_size(),
                                "peak_fwd_bwd_bytes": peak, "fwd_bwd_ms": ts[len(ts) // 2]})
    del blk
    torch.cuda.empty_cache()
    return res


def run_dropout(B, L, dev, p=0.1, reps=10):
    """LoRA dropout on the adapter input (QLoRA Appendix B.2 uses p = 0.1 up
    to 13B): the keep mask drawn on the device (qlora_dropout_mask,
    Philox4x64-10), then forward + backward of the layer with it, against the
    same calls without dropout.  Median over `reps` calls between two
    events."""
    import torch

    lin, t = L["lin"], L["t"]
    keep = B.qlora_dropout_mask(11, 0, lin.M, lin.K, p, device=dev)
    qw = L["qw"]
    ts = []
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.qlora_dropout_mask(11, i, lin.M, lin.K, p, out=keep)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    mask_us = sorted(ts[1:])[len(ts) // 2]

    def fb(kw):
        B.qlora_linear_fwd(t["X"], qw, t["A"], t["B"], lin.s, Y=L["Y"], XA=L["XA"], workspace=L["ws"], **kw)
        B.qlora_linear_bwd(t["dY"], t["X"], L["XA"], qw, t["A"], t["B"], lin.s,
                           dX=L["dX"], dA=L["dA"], dB=L["dB"], workspace=L["ws"], **kw)

    out = {"p": p, "mask_us": mask_us, "mask_bytes": lin.M * lin.K // 8}
    for name, kw in (("dropout", {"keep": keep, "p": p}), ("plain", {})):
        ts = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fb(kw)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts = sorted(ts[1:])
        us = ts[len(ts) // 2]
        out[name] = {"fwd_bwd_us": us, "fwd_bwd_TFLOPs": linear_flops(lin) / us / 1e6}
    return out


OPT_BYTES_PER_PARAM = 30.0  # clip: bf16 grad read; step: grad, fp32 p/m/v read+write, bf16 p written


def run_optimizer(B, L, dev, reps=20):
    """The LoRA-only optimizer step (QLoRA Appendix B.2: beta2 0.999, max
    grad norm 0.3) over the layer's adapters A and B in one flat buffer:
    clip scale + AdamW, with the fp32 states on the device, in pinned host
    memory updated in place over the link, and paged through a device
    staging buffer (QLoRA section 3 "Paged Optimizers").  Median of `reps`
    steps between two events each."""
    import torch

    lin = L["lin"]
    n = lin.r * (lin.K + lin.N)
    g = torch.Generator(device=dev).manual_seed(21)
    grad = (torch.randn(n, generator=g, device=dev) * 1e-3).to(torch.bfloat16)
    out = {"params": n, "bytes_per_param": OPT_BYTES_PER_PARAM}
    staging = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream(device=dev)
    for where in ("device", "pinned_host_in_place", "paged", "paged_one_stream"):
        p = torch.randn(n, generator=g, device=dev) * 0.01
        pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
        if where == "device":
            m, v = torch.zeros(n, device=dev), torch.zeros(n, device=dev)
        else:
            m, v = torch.zeros(n).pin_memory(), torch.zeros(n).pin_memory()
        sc = torch.empty(4, dtype=torch.float32, device=dev)
        ts = []
        for t in range(1, reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.qlora_clip_scale(grad, 0.3, scale=sc)
            if where.startswith("paged"):
                B.qlora_adamw_step_paged(p, grad, m, v, t, 2e-4, staging, (0.9, 0.999), 1e-8, 0.0, grad_scale=sc,
                                         param_bf16=pb, copy_stream=copy_stream if where == "paged" else None)
            else:
                B.qlora_adamw_step(p, grad, m, v, t, 2e-4, (0.9, 0.999), 1e-8, 0.0, grad_scale=sc, param_bf16=pb)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts = sorted(ts[1:])
        us = ts[len(ts) // 2]
        out[where] = {"step_us": us, "GB/s": OPT_BYTES_PER_PARAM * n / us / 1e3}
    out["paged_staging_bytes"] = staging.numel()
    out["how"] = ("device: states in HBM; pinned_host_in_place: the update kernel reads and writes the pinned host "
                  "states over the link; paged: states paged through a 1 MiB device staging buffer in chunks, copies "
                  "on a second stream overlapping the updates (paged_one_stream: all on one stream)")
    return out


def _dominant(per, layers, small):
    """(kernel, bound, algorithmic work, mean us, linear index) of the kernel
    with the largest share of the step, from a per-linear kernel breakdown.
    The small-token forward kernel streams the packed weight (HBM-bound)."""
    best = None
    for li, (kt, _) in enumerate(per):
        lin = layers[li]["lin"]
        p = lin.N * lin.K
        cands = [
            ("fwd_main", "hbm", STORED_BYTES_PER_PARAM * p) if small else
            ("fwd_main", "mfma", 2 * lin.M * lin.N * lin.K + 2 * lin.M * lin.r * lin.N),
            ("bwd_dx", "mfma", 2 * lin.M * lin.N * lin.K + 2 * lin.M * lin.r * lin.K),
            ("quantize", "hbm", QUANT_BYTES_PER_PARAM * p),
            ("dequantize", "hbm", DEQUANT_BYTES_PER_PARAM * p),
        ]
        for name, bound, work in cands:
            if name in kt and (best is None or kt[name] > best[3]):
                best = (name, bound, work, kt[name], li)
    return best


def achievable_bandwidth(dev, mib=1024, reps=5):
    """What this device streams, as the roofline's "achievable" companion to
    the datasheet figure: a plain device copy (torch copy_, read + write
    bytes) and a plain read (the library's streaming-read probe, 16-byte
    loads, four in flight per thread) of `mib` MiB, median of `reps` after a
    warm-up."""
    import torch

    from bit_nf4_quantized_quantize_amd import binding as B

    n = mib << 18
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def med(fn):
        ts = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    copy_ms = med(lambda: dst.copy_(src))
    read_ms = med(lambda: B.qlora_probe_read(src, sink))
    del src, dst
    torch.cuda.empty_cache()
    nbytes = 4 * n
    return {"copy_GBps": 2 * nbytes / copy_ms / 1e6, "read_GBps": nbytes / read_ms / 1e6, "buffer_MiB": mib,
            "how": "torch copy_ (read + write bytes) and the library's streaming-read probe qlora_probe_read "
                   f"(read bytes) of one fp32 buffer, median of {reps}"}


class Scrub:
    """A 1 GiB device buffer read between timed calls, so that a timed call
    finds none of its inputs in the 256 MB Infinity Cache.  The buffer is
    written once and read once more at construction; after that every scrub
    only reads it, so the caches it leaves behind hold clean lines and the
    timed call pays no write-back of the scrub's own data."""

    def __init__(self, dev, mib=1024):
        import torch
        self.buf = torch.full((mib << 18,), 0.5, dtype=torch.float32, device=dev)
        self()
        torch.cuda.synchronize(dev)

    def __call__(self):
        self.buf.sum()


def measure(args, workload, steps, warmup, with_cpu, dev):
    """The measurement of one workload (see the module docstring); returns
    the JSON object of its line."""
    import torch

    from bit_nf4_quantized_quantize_amd import binding as B
    from bit_nf4_quantized_quantize_amd import synth

    bf = torch.bfloat16
    small = workload == 5
    lins = synth.workload(workload)
    if small:
        # the three token counts share one weight (rows drawn for the largest)
        base = lins[-1]
        t0 = base.draw(dev, with_grad=False)
        wbytes = base.N * base.K * 0.516
        rotate = args.rotate or max(1, -(-(1200 << 20) // int(wbytes)))
        qws = [B.qlora_nf4_quantize(t0["W"] * (1.0 + 1e-3 * i)) for i in range(rotate)]
        del t0["W"]
        layers = []
        for lin in lins:
            layers.append({"lin": lin, "X": t0["X"][:lin.M].contiguous(), "A": t0["A"], "B": t0["B"],
                           "Y": torch.empty(lin.M, lin.N, dtype=bf, device=dev),
                           "XA": torch.empty(lin.M, lin.r, dtype=bf, device=dev), "ws": B.Workspace()})
        kernels = ("fwd_main",)
        phases = ("fwd",)
    else:
        # fp32 weights rotated over more than 1 GB (the 65B-shaped layer's
        # three weights are 2.2 GB already)
        wbytes = sum(l.N * l.K * 4 for l in lins)
        rotate = args.rotate or max(1, -(-(1200 << 20) // wbytes))
        layers = []
        for lin in lins:
            t = lin.draw(dev)
            layers.append({
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
            })
        kernels = ("quantize", "dequantize", "fwd_main", "bwd_dx")
        phases = ("quantize", "dequantize", "fwd", "bwd")

    hev = HipEvents()
    tev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    scrub = Scrub(dev)

    def run_phase(li, p, i):
        """One call of phase p for linear li (rotation index i)."""
        L = layers[li]
        lin = L["lin"]
        if small:
            B.qlora_linear_fwd(L["X"], qws[i % rotate], L["A"], L["B"], lin.s, Y=L["Y"], XA=L["XA"],
                               workspace=L["ws"])
            return
        t = L["t"]
        if p == "quantize":
            B.qlora_nf4_quantize(L["W"][i % rotate], double_quant=True, out=L["qw"], workspace=L["qws"])
        elif p == "dequantize":
            B.qlora_nf4_dequantize(L["qw"], bf, out=L["Wd"])
        elif p == "fwd":
            B.qlora_linear_fwd(t["X"], L["qw"], t["A"], t["B"], lin.s, Y=L["Y"], XA=L["XA"], workspace=L["ws"])
        else:
            B.qlora_linear_bwd(t["dY"], t["X"], L["XA"], L["qw"], t["A"], t["B"], lin.s,
                               dX=L["dX"], dA=L["dA"], dB=L["dB"], workspace=L["ws"])

    def run_step(i, kev=None):
        """One step, phase by phase over all linears (so a linear's codes are
        dequantised after the other linears' weights have streamed through
        the cache); kev[li][kernel] = (start, stop) hipEvents the library
        records around its kernels."""
        for p in phases:
            for li in range(len(layers)):
                if kev is not None:
                    for k, (e0, e1) in kev[li].items():
                        B.lib().qlora_profile_events(B.QLORA_KERNEL[k], e0, e1)
                run_phase(li, p, i)
        if kev is not None:
            for k in kernels:
                B.lib().qlora_profile_events(B.QLORA_KERNEL[k], None, None)

    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()

    # 1) breakdown (untimed for `value`): kernel durations from events around
    # each library kernel; call durations of each phase: HBM-bound phases
    # (quantise, dequantise, the small-token forward) one call at a time after
    # a 1 GiB cache scrub (median), the GEMM phases as nprof back-to-back calls
    nprof = max(3, min(steps, 10))
    kev_all = [[{k: (hev.create(), hev.create()) for k in kernels} for _ in layers] for _ in range(nprof)]
    for i in range(nprof):
        run_step(warmup + i, kev_all[i])
    torch.cuda.synchronize()
    per = []
    for li in range(len(layers)):
        kt = {k: sum(hev.elapsed_ms(*kev_all[i][li][k]) for i in range(nprof)) * 1e3 / nprof for k in kernels}
        pt = {}
        for p in phases:
            if small or p in ("quantize", "dequantize"):
                ts = []
                for i in range(nprof):
                    scrub()
                    e0, e1 = tev(), tev()
                    e0.record()
                    run_phase(li, p, warmup + i)
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3)
                pt[p] = sorted(ts)[len(ts) // 2]
            else:
                e0, e1 = tev(), tev()
                e0.record()
                for i in range(nprof):
                    run_phase(li, p, warmup + i)
                e1.record()
                torch.cuda.synchronize()
                pt[p] = e0.elapsed_time(e1) * 1e3 / nprof
        per.append((kt, pt))
    name, bound, work, _, dli = _dominant(per, layers, small)

    # 2) timed region: K steps, events only around the dominant kernel
    kev_t = [[{name: (hev.create(), hev.create())} if li == dli else {} for li in range(len(layers))]
             for _ in range(steps)]
    start, stop = tev(), tev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(steps):
        run_step(warmup + nprof + i, kev_t[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(stop) / steps
    us = sum(hev.elapsed_ms(*kev_t[i][dli][name]) for i in range(steps)) * 1e3 / steps
    hev.close()
    del scrub

    if bound == "mfma":
        achieved = work / us / 1e6
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None}
    else:
        achieved = work / us / 1e3
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    roof.update({"kernel": name, "linear": layers[dli]["lin"].name, "algorithmic_per_launch": work,
                 "avg_launch_us": us})
    if kernel_digest() == TRAFFIC_DIGEST and (workload, name) in TRAFFIC_BYTES:
        roof["traffic"] = TRAFFIC_BYTES[(workload, name)]
        roof["traffic_unit"] = "bytes per launch (HBM read + write)"

    breakdown = []
    for (kt, pt), L in zip(per, layers):
        lin = L["lin"]
        p = lin.N * lin.K
        row = {"linear": lin.name, "M": lin.M, "N": lin.N, "K": lin.K, "r": lin.r}
        if small:
            gb = STORED_BYTES_PER_PARAM * p + 2 * lin.M * (lin.K + lin.N) + 2 * lin.r * (lin.K + lin.N)
            row.update({"fwd_us": pt["fwd"], "fwd_GBps": gb / pt["fwd"] / 1e3,
                        "weight_kernel_us": kt["fwd_main"],
                        "weight_kernel_GBps": STORED_BYTES_PER_PARAM * p / kt["fwd_main"] / 1e3})
        else:
            row.update({
                "quantize_call_us": pt["quantize"], "quantize_kernel_us": kt["quantize"],
                "quantize_GBps": QUANT_BYTES_PER_PARAM * p / pt["quantize"] / 1e3,
                "dequantize_call_us": pt["dequantize"], "dequantize_kernel_us": kt["dequantize"],
                "dequantize_GBps": DEQUANT_BYTES_PER_PARAM * p / pt["dequantize"] / 1e3,
                "fwd_us": pt["fwd"], "fwd_main_kernel_us": kt["fwd_main"],
                "fwd_TFLOPs": (2 * lin.M * lin.N * lin.K + 2 * lin.M * lin.r * (lin.K + lin.N)) / pt["fwd"] / 1e6,
                "bwd_us": pt["bwd"], "bwd_dx_kernel_us": kt["bwd_dx"],
                "bwd_TFLOPs": (2 * lin.M * lin.N * lin.K + 4 * lin.M * lin.r * (lin.K + lin.N)) / pt["bwd"] / 1e6,
                "fwd_bwd_TFLOPs": linear_flops(lin) / (pt["fwd"] + pt["bwd"]) / 1e6,
            })
        breakdown.append(row)

    cpu = None
    if with_cpu:
        if small:
            cpu = cpu_baseline_small(layers[-1])
        elif workload == 4:
            cpu = cpu_baseline_scaled([L["lin"] for L in layers], layers[0]["t"])
        else:
            cpu = cpu_baseline(layers[0]["lin"], layers[0]["t"])

    lin0 = layers[0]["lin"]
    if small:
        total_bytes = sum(STORED_BYTES_PER_PARAM * L["lin"].N * L["lin"].K
                          + 2 * L["lin"].M * (L["lin"].K + L["lin"].N) + 2 * L["lin"].r * (L["lin"].K + L["lin"].N)
                          for L in layers)
        metric, unit = SMALL_METRIC, "GB/s"
        value = total_bytes / (ms_per_step / 1e3) / 1e9
        step_desc = "forward (fused small-token path) at 1, 4 and 16 tokens against one rotated NF4+DQ weight"
    else:
        metric, unit = METRIC, "TFLOP/s"
        value = sum(linear_flops(L["lin"]) for L in layers) / (ms_per_step / 1e3) / 1e12
        step_desc = ("quantize+DQ, dequantize->bf16, fwd, bwd (dX, dA, dB) of every linear, phase by phase over "
                     "the linears")
    out = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[workload],
            "linears": [{"name": L["lin"].name, "M": L["lin"].M, "N": L["lin"].N, "K": L["lin"].K,
                         "r": L["lin"].r, "alpha": L["lin"].alpha} for L in layers],
            "global_batch": lin0.M, "weight_copies_rotated": rotate, "step": step_desc,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
        "breakdown_steps": nprof,
        "wall_s_timed": wall,
    }
    if not small:
        q_us = sum(b["quantize_call_us"] for b in breakdown)
        q_bytes = sum(QUANT_BYTES_PER_PARAM * L["lin"].N * L["lin"].K for L in layers)
        d_us = sum(b["dequantize_call_us"] for b in breakdown)
        d_bytes = sum(DEQUANT_BYTES_PER_PARAM * L["lin"].N * L["lin"].K for L in layers)
        out["quantize"] = {"GB/s": q_bytes / q_us / 1e3, "frac_hbm": q_bytes / q_us / 1e3 / HBM_PEAK_GBS,
                           "bytes_per_param": QUANT_BYTES_PER_PARAM, "cold_cache": True}
        out["dequantize"] = {"GB/s": d_bytes / d_us / 1e3, "frac_hbm": d_bytes / d_us / 1e3 / HBM_PEAK_GBS,
                             "bytes_per_param": DEQUANT_BYTES_PER_PARAM, "cold_cache": True}
        fb_us = sum(b["fwd_us"] + b["bwd_us"] for b in breakdown)
        fb = sum(linear_flops(L["lin"]) for L in layers) / fb_us / 1e6
        out["fwd_bwd"] = {"TFLOP/s": fb, "frac_mfma": fb / BF16_PEAK_TFLOPS}
        if workload == 2 and not args.no_code_types:
            out["code_types"] = run_code_types(B, layers[0], dev)
            out["lora_dropout"] = run_dropout(B, layers[0], dev)
            out["optimizer"] = run_optimizer(B, layers[0], dev)
            if not args.no_block:
                out["qlora_block"] = run_block(dev)
        del layers
        torch.cuda.empty_cache()
    else:
        del layers, qws
        torch.cuda.empty_cache()
        if not args.no_sweep:
            out["sweep"] = run_sweep(B, synth, dev)
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_nf4_quantized_quantize_amd import binding as B

    B.lib()  # raises if the HIP library is missing: there is no fallback
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_probe_mib > 0:
        src = torch.empty(args.copy_probe_mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ach = achievable_bandwidth(dev) if not args.no_extras else None
    out = measure(args, args.workload, args.steps, args.warmup, not args.no_cpu_baseline, dev)
    if ach is not None:
        out["achievable"] = ach
        if out["roofline"]["unit"] == "GB/s":
            out["roofline"]["achievable"] = ach["read_GBps"]
            out["roofline"]["frac_of_achievable"] = out["roofline"]["achieved"] / ach["read_GBps"]
        for key in ("quantize", "dequantize"):
            if key in out:
                out[key]["frac_of_achievable_copy"] = out[key]["GB/s"] / ach["copy_GBps"]
    if args.workload == 4 and not args.no_extras:
        # the other two headline shapes, as extra keys of the same line
        print("bench: 65B-shaped layer done; 7B attention projection next", file=sys.stderr, flush=True)
        sub = argparse.Namespace(**vars(args))
        sub.rotate = 0
        out["attn_4096"] = measure(sub, 2, 20, 3, False, dev)
        print("bench: 7B attention done; small batch next", file=sys.stderr, flush=True)
        out["small_batch"] = measure(sub, 5, 20, 3, False, dev)
        if ach is not None:
            sb = out["small_batch"]["roofline"]
            sb["achievable"] = ach["read_GBps"]
            sb["frac_of_achievable"] = sb["achieved"] / ach["read_GBps"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

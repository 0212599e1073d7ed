#!/usr/bin/env python3
"""Throughput of the NF4 QLoRA linear layer on one MI355X.

One step = one forward + one backward pass (dX, dL1, dL2) of the frozen NF4 linear layer with its
LoRA branch over one batch, through the C ABI (qlora_linear_fwd + qlora_linear_bwd), inputs
already resident in HBM.  The default workload is the LLaMA-7B attention projection
(W 4096x4096 NF4, block 64, double quantization block 256; 8 x 512 = 4096 tokens; r = 64,
alpha = 16).  The headline value is algorithmic TFLOP/s (2MNK per dense product, LoRA at rank r),
timed over 100 steps after 200 untimed ones (the clocks of sustained load; every other timed
region below follows at least 150 ms of the same work).

Also reported on the same JSON line:
  roofline     the dominant kernel (the larger of the two bf16 GEMM launches), timed live with
               HIP events recorded by the library around each of its launches in the timed
               region; step_frac is the whole step's fraction of the bf16 peak
  cpu_baseline the CPU oracle on a bounded sample of the same workload
  gemv         decode-size forward (W 28672x8192, M = 1, 4, 16) in GB/s, weights rotated over
               three replicas so the 256 MB last-level cache cannot hold them
  c3           the LLaMA-7B SwiGLU MLP (gate/up 11008x4096, down 4096x11008, 4096 tokens, r = 64):
               forward + backward TFLOP/s, every GEMM launch timed, the dominant one as roofline
  c4           the LLaMA-65B-shaped MLP (22016x8192 / 8192x22016, 2048 tokens, heavy-tailed
               weights): the same, plus quantize + double quant of its three weights in GB/s
  qkv          the LLaMA-7B q, k, v projections (three 4096x4096 linears sharing X) as one product
               against three linear calls (forward), at 4096 and 1024 tokens
  mid          the 7B attention projection forward + backward at 1, 16, 32, 256, 512 and 1536
               tokens (the GEMVs, the fused dequant GEMMs and the under-filled expanded GEMM, their
               reductions split where tiles leave CUs idle)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-gemv] [--no-mlp]
                       [--no-mid]
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
TIMING_EVERY = 4               # timed steps whose GEMM launches carry HIP events
# Sustained work before each timed region: the GPU's clocks climb over the first ~10-50 ms of
# load after an idle spell (the 7B projection step read 0.304-0.310 ms after 5 warm-up steps,
# 0.275 after 50 and 0.271 after 200; 2000 steps, the default, read 0.278-0.279 against
# 0.280-0.281 after 200 on one box), so every timed region follows at least this much.
WARM_MS = 150.0


def warm(torch, fn, min_ms=WARM_MS, min_calls=3):
    """Call fn(i) until the calls have kept the GPU busy for min_ms (timed with events, in batches
    that double), at least min_calls times; returns the number of calls."""
    done, calls, batch = 0.0, 0, 1
    while done < min_ms or calls < min_calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(batch):
            fn(calls + i)
        e1.record()
        torch.cuda.synchronize()
        done += e0.elapsed_time(e1)
        calls += batch
        batch = min(2 * batch, 4096)
    return calls
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "NF4 dequant-GEMM+LoRA fwd/bwd TFLOP/s (7B shapes); M=1 GEMV GB/s"

# HBM traffic of the GEMMs at the llama7b_attn workload, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
#   python bench.py --steps 3 --warmup 1 --no-gemv --no-cpu-baseline
# scaled by what the same counters read for a plain copy of exactly 1 GiB
# (python bench.py --copy-calibration: FETCH_SIZE 524301 KiB, WRITE_SIZE 1048576 KiB), i.e.
# FETCH_SIZE counts half the bytes read on this GPU.  Valid only for the kernel sources they were
# taken on: if the hashed sources differ, traffic is reported as null.
FETCH_SCALE = 1048576.0 / 524301.3
WRITE_SCALE = 1048576.0 / 1048576.0
GEMM_TRAFFIC_KIB = {0: (99996.0, 33116.0), 1: (99984.0, 32922.0)}   # kind -> (FETCH_SIZE, WRITE_SIZE)
GEMM_TRAFFIC_SOURCES = {
    "csrc/gemm_bf16.hip": "8d4c622103c4179b729e2f2b1d8fa91ead1c5985e53e4327c52d5db59c5225d5",
    "csrc/common.h": "1cf2a1ddbbf0b49703ce638ad570d618aa6e5700ecdf039bf1c982405beaf8f7",
    "csrc/dqtile.h": "5e5858351a391c0bf4b3b0eb26d1438c822fbee72afe0766f9790cb36c7179b7",
}


def gemm_traffic_bytes(kind):
    """Calibrated HBM bytes per launch of the GEMM of this kind, or None if stale or unmeasured."""
    import hashlib
    if kind not in GEMM_TRAFFIC_KIB:
        return None
    pkg = os.path.join(ROOT, "bit_nf4_quantized_codebook_amd")
    for rel, digest in GEMM_TRAFFIC_SOURCES.items():
        try:
            with open(os.path.join(pkg, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        except OSError:
            return None
    fetch, write = GEMM_TRAFFIC_KIB[kind]
    return int(round((fetch * FETCH_SCALE + write * WRITE_SCALE) * 1024))


def linear_flops(M, N, K, r):
    """Algorithmic flops of one forward + backward of the layer (2 per multiply-add)."""
    fwd = 2 * M * N * K + 2 * M * K * r + 2 * M * r * N
    bwd = 2 * M * N * K + 2 * M * N * r + 2 * r * M * N + 2 * K * M * r + 2 * M * r * K
    return fwd, bwd


def gemm_launch_flops(kind, M, N, K, r):
    """Algorithmic flops of one GEMM launch (main product + LoRA extension)."""
    return 2 * M * N * K + (2 * M * r * N if kind == 0 else 2 * M * r * K)


def gemv_bytes(M, N, K, r):
    """Algorithmic HBM bytes of one decode-size forward."""
    nb = N * K // 64
    return (N * K // 2 + nb + (nb + 255) // 256 * 4 + 4 + K * r * 2 + r * N * 2 + M * K * 2 + M * N * 2)


def make_linear(torch, nf4, synth, wl, lin, M, dev, replicas=1):
    import numpy as np
    cb = nf4.nf4_build_codebook()
    W = torch.from_numpy(synth.weight_f32(wl, lin)).to(dev)
    w0 = nf4.NF4Weight.from_float(W, cb)
    del W
    ws = [w0]
    for _ in range(replicas - 1):
        ws.append(nf4.NF4Weight(w0.packed.clone(), w0.absmax_q.clone(), w0.absmax_scale.clone(),
                                w0.absmax_mean.clone(), w0.rows, w0.cols, cb))
    l1, l2 = synth.lora_f32(wl, lin)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    st = {
        "w": ws, "L1": bf(l1), "L2": bf(l2),
        "X": bf(synth.x_f32(wl, M=M, K=lin.K)),
        "dY": bf(synth.dy_f32(wl, M, lin.N)),
        "Y": torch.empty((M, lin.N), dtype=torch.bfloat16, device=dev),
        "T": torch.empty((M, wl.r), dtype=torch.bfloat16, device=dev),
        "dX": torch.empty((M, lin.K), dtype=torch.bfloat16, device=dev),
        "dL1": torch.empty((lin.K, wl.r), dtype=torch.bfloat16, device=dev),
        "dL2": torch.empty((wl.r, lin.N), dtype=torch.bfloat16, device=dev),
        "ws": torch.empty(nf4.qlora_linear_workspace_size(M, lin.N, lin.K, wl.r), dtype=torch.uint8,
                          device=dev),
        "s": wl.scale, "M": M, "N": lin.N, "K": lin.K, "r": wl.r,
    }
    return st


def step_linear(nf4, st, i=0):
    w = st["w"][i % len(st["w"])]
    nf4.qlora_linear_fwd(w, st["X"], st["L1"], st["L2"], st["s"], Y=st["Y"], T=st["T"], workspace=st["ws"])
    nf4.qlora_linear_bwd(w, st["dY"], st["X"], st["L1"], st["L2"], st["T"], st["s"], dX=st["dX"],
                         dL1=st["dL1"], dL2=st["dL2"], workspace=st["ws"])


def cpu_baseline(synth, wl, lin, budget_s=10.0, sample_tokens=512):
    """The oracle as it stands, on a bounded token sample of the same workload."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    W = synth.weight_f32(wl, lin)
    l1, l2 = synth.lora_f32(wl, lin)
    L1, L2 = synth.to_bf16_bits(l1), synth.to_bf16_bits(l2)
    X = synth.to_bf16_bits(synth.x_f32(wl, M=sample_tokens, K=lin.K))
    dY = synth.to_bf16_bits(synth.dy_f32(wl, sample_tokens, lin.N))
    q = oracle.quantize_dq(W)
    fwd, bwd = linear_flops(sample_tokens, lin.N, lin.K, wl.r)
    reps, t_total = 0, 0.0
    while reps < 1 or (t_total < budget_s and reps < 20):
        t0 = time.perf_counter()
        Wd = oracle.dequant_weight(q)
        oracle.forward(X, Wd, L1, L2, wl.scale)
        oracle.backward(dY, X, Wd, L1, L2, wl.scale)
        t_total += time.perf_counter() - t0
        reps += 1
    threads = 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 1)))
    return {
        "value": round((fwd + bwd) * reps / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": (f"{reps} oracle fwd+bwd passes over {sample_tokens} of the {wl.M} tokens "
                   f"({lin.N}x{lin.K} weight double-dequantized by the oracle each pass, float64 "
                   f"numpy products), {t_total:.1f} s"),
    }


def bench_gemv(torch, nf4, synth, dev, reps=60, warmup=10):
    """Decode-size forward, weights rotated over 3 replicas (378 MB > 256 MB last-level cache)."""
    wl = synth.WORKLOADS["gemv"]
    lin = wl.linears[0]
    out = {}
    for M in (1, 4, 16):
        st = make_linear(torch, nf4, synth, wl, lin, M, dev, replicas=3)

        def call(i):
            nf4.qlora_linear_fwd(st["w"][i % 3], st["X"], st["L1"], st["L2"], st["s"], Y=st["Y"], T=st["T"],
                                 workspace=st["ws"])
        warm(torch, call, min_calls=warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            w = st["w"][i % 3]
            nf4.qlora_linear_fwd(w, st["X"], st["L1"], st["L2"], st["s"], Y=st["Y"], T=st["T"],
                                 workspace=st["ws"])
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        b = gemv_bytes(M, lin.N, lin.K, wl.r)
        out[f"M{M}"] = {"us_per_call": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                        "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": b}
        del st
        torch.cuda.empty_cache()
    return out


def mlp_launches(M, F, K, r):
    """GEMM launches of one MLP step in launch order: (name, kind recorded by the library,
    algorithmic flops).  F = hidden size of the MLP (gate/up rows, down's reduction), K = model
    width.  From 1024 tokens with F a multiple of 256, gate and up run as one product."""
    fwd_gu = 2 * M * F * K + 2 * M * r * F
    if M >= 1024 and F % 256 == 0:
        first = [("gate+up fwd (one product over both weights)", 0, 2 * fwd_gu)]
    else:
        first = [("gate fwd", 0, fwd_gu), ("up fwd", 0, fwd_gu)]
    return first + [("down fwd", 0, 2 * M * K * F + 2 * M * r * K), ("down bwd (dH)", 1, 2 * M * K * F + 2 * M * r * F),
                    ("gate+up bwd (dX over both weights)", 4, 2 * (2 * M * F * K) + 2 * (2 * M * r * K))]


def mlp_flops(M, F, K, r):
    """Algorithmic flops of one MLP forward + backward: three linears, LoRA at rank r (the glue's
    elementwise work is not counted)."""
    gu = linear_flops(M, F, K, r)
    dn = linear_flops(M, K, F, r)
    return 2 * sum(gu) + sum(dn)


def make_mlp(torch, nf4, synth, wl, dev):
    """The three QLoRA linears of a SwiGLU MLP workload, their adapters, X, dY and the buffers of one
    step; the weights are quantized on the GPU from the seeded float32 draws."""
    import numpy as np
    cb = nf4.nf4_build_codebook()
    gate, up, down = wl.linears
    M, r, F, K = wl.M, wl.r, gate.N, gate.K
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)  # noqa: E731
    st = {"M": M, "r": r, "F": F, "K": K, "s": wl.scale, "w": [], "L1": [], "L2": []}
    for lin in wl.linears:
        W = torch.from_numpy(synth.weight_f32(wl, lin)).to(dev)
        st["w"].append(nf4.NF4Weight.from_float(W, cb))
        del W
        l1, l2 = synth.lora_f32(wl, lin)
        st["L1"].append(bf(l1))
        st["L2"].append(bf(l2))
    st["X"] = bf(synth.x_f32(wl, M=M, K=K))
    st["dY"] = bf(synth.dy_f32(wl, M, down.N))
    e = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=dev)  # noqa: E731
    st.update(Y=e(M, K), Td=e(M, r), dH=e(M, F), dX=e(M, K), dL1d=e(F, r), dL2d=e(r, K))
    wsb = max(nf4.lib.qlora_gated_workspace_size(M, F, K, r), nf4.qlora_linear_workspace_size(M, K, F, r))
    st["ws"] = torch.empty(wsb, dtype=torch.uint8, device=dev)
    return st


def step_mlp(nf4, st):
    """One forward + backward of the MLP: gate and up (two linears, then the glue), down; down's
    backward, the glue's backward and both linears' backward with dX as one product over the two
    weights (the library's faster form of each)."""
    wg, wu, wd = st["w"]
    (L1g, L1u, L1d), (L2g, L2u, L2d) = st["L1"], st["L2"]
    s, ws = st["s"], st["ws"]
    G, U, H, Tg, Tu = nf4.qlora_gated_fwd(wg, wu, st["X"], L1g, L2g, L1u, L2u, s, workspace=ws)
    nf4.qlora_linear_fwd(wd, H, L1d, L2d, s, Y=st["Y"], T=st["Td"], workspace=ws)
    nf4.qlora_linear_bwd(wd, st["dY"], H, L1d, L2d, st["Td"], s, dX=st["dH"], dL1=st["dL1d"], dL2=st["dL2d"],
                         workspace=ws)
    nf4.qlora_gated_bwd(wg, wu, st["dH"], st["X"], G, U, L1g, L2g, L1u, L2u, Tg, Tu, s, dX=st["dX"],
                        workspace=ws, fuse=True)


def bench_mlp(torch, nf4, synth, dev, wl, steps=10, warmup=3):
    """Forward + backward TFLOP/s of a SwiGLU MLP workload (three QLoRA linears and the glue), with
    every GEMM launch of one step in four timed with HIP events on its stream."""
    st = make_mlp(torch, nf4, synth, wl, dev)
    M, F, K, r = st["M"], st["F"], st["K"], st["r"]
    warm(torch, lambda i: step_mlp(nf4, st), min_calls=warmup)
    launches = mlp_launches(M, F, K, r)
    nl = len(launches)
    nsampled = (steps + TIMING_EVERY - 1) // TIMING_EVERY
    timer = nf4.GemmTimer(nl * nsampled)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cnt = 0
    e0.record()
    for i in range(steps):
        sampled = i % TIMING_EVERY == 0
        if sampled:
            timer.arm_at(cnt, nl)
        step_mlp(nf4, st)
        if sampled:
            cnt += timer.disarm()
    e1.record()
    torch.cuda.synchronize()
    durs = timer.durations_ms(cnt)
    timer.close()
    if cnt != nl * nsampled or any(k != launches[i % nl][1] for i, (k, _) in enumerate(durs)):
        raise RuntimeError(f"unexpected GEMM launch sequence: {[k for k, _ in durs]}")
    ms = e0.elapsed_time(e1) / steps
    flops = mlp_flops(M, F, K, r)
    kernels = {}
    for i, (name, _, lf) in enumerate(launches):
        us = sum(d for j, (_, d) in enumerate(durs) if j % nl == i) / nsampled * 1e3
        kernels[name] = {"us": round(us, 2), "TFLOP/s": round(lf / us / 1e6, 1),
                         "frac": round(lf / us / 1e6 / BF16_PEAK_TFLOPS, 4), "flops": lf}
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    value = flops / (ms * 1e-3) / 1e12
    del st
    torch.cuda.empty_cache()
    return {
        "workload": f"{wl.name}: {wl.notes}; gate/up W {F}x{K}, down W {K}x{F}, NF4 (block 64, double-quant "
                    f"block 256), {M} tokens, LoRA r={r} alpha={wl.alpha:g} on all three, forward + backward",
        "value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4), "steps": steps,
        "flops_per_step": flops, "step_frac": round(value / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": kernels[dom]["TFLOP/s"], "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": kernels[dom]["frac"], "traffic": None,
                     "kernel": dom, "avg_launch_us": kernels[dom]["us"], "launches_timed": nsampled},
        "gemm_launches": kernels,
    }


def quantize_bytes(numel):
    """Algorithmic HBM bytes of quantize + double quant of one float32 weight: W read (4 B), codes
    (0.5 B) and block constants (4/64 B) written; the constants read back (4/64 B), their 8-bit codes
    (1/64 B), second-level scales and the mean written."""
    nb = numel // 64
    return 4 * numel + numel // 2 + 4 * nb + 4 * nb + nb + 4 * ((nb + 255) // 256) + 4


def bench_quantize(torch, nf4, synth, dev, wl, reps=5):
    """Quantize + double-quantize every weight of a workload from float32 in HBM, GB/s."""
    import ctypes
    import numpy as np
    cb = nf4.nf4_build_codebook()
    cbp = ctypes.c_void_p(cb.ctypes.data)
    bufs = []
    for lin in wl.linears:
        n = lin.N * lin.K
        nb = n // 64
        wsb = nf4.lib.nf4_double_quant_workspace_size(nb, 256)
        bufs.append({
            "W": torch.from_numpy(synth.weight_f32(wl, lin)).to(dev).reshape(-1), "n": n, "nb": nb,
            "packed": torch.empty(n // 2, dtype=torch.uint8, device=dev),
            "absmax": torch.empty(nb, dtype=torch.float32, device=dev),
            "q": torch.empty(nb, dtype=torch.uint8, device=dev),
            "sc": torch.empty((nb + 255) // 256, dtype=torch.float32, device=dev),
            "mean": torch.empty(1, dtype=torch.float32, device=dev),
            "ws": torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev), "wsb": wsb})
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def run():
        for b in bufs:
            nf4._check(nf4.lib.nf4_quantize(p(b["W"]), b["n"], 64, cbp, p(b["packed"]), p(b["absmax"]), stream),
                       "nf4_quantize")
            nf4._check(nf4.lib.nf4_double_quant(p(b["absmax"]), b["nb"], 256, p(b["q"]), p(b["sc"]), p(b["mean"]),
                                                p(b["ws"]), b["wsb"], stream), "nf4_double_quant")

    warm(torch, lambda i: run())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = sum(quantize_bytes(b["n"]) for b in bufs)
    del bufs
    torch.cuda.empty_cache()
    return {"workload": f"quantize + double quant of the {len(wl.linears)} float32 weights of {wl.name} "
                        f"({' + '.join(f'{l.N}x{l.K}' for l in wl.linears)})",
            "us": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
            "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def qerror_gpu(torch, nf4, W, cb, dq=True, dq_format="e4m3"):
    """Quantization error of the float32 device weight W [rows, cols] under the 16-entry table cb,
    from the library's own quantize / double quant / dequant (eq. 6, or eq. 2 at one level without
    DQ): mse and max_abs of (deq - W) in float64, the element count per code, its entropy in bits,
    and the stored bits per weight (codes, block constants and, with DQ, the mean)."""
    n = W.numel()
    if dq:
        w = nf4.NF4Weight.from_float(W, cb, dq_format=dq_format)
        packed = w.packed
        deq = nf4.nf4_dequant(w).reshape(-1)
        stored = packed.numel() + w.absmax_q.numel() + 4 * w.absmax_scale.numel() + 4 * w.absmax_mean.numel()
    else:
        packed, absmax = nf4.nf4_quantize(W.reshape(-1), cb)
        deq = nf4.nf4_dequant_single(packed, absmax, n, cb)
        stored = packed.numel() + 4 * absmax.numel()
    err = deq.double() - W.reshape(-1).double()
    codes = torch.stack([packed & 15, packed >> 4], dim=1).reshape(-1)[:n]
    occ = torch.bincount(codes.long(), minlength=16).cpu().numpy()
    import numpy as np
    p = occ[occ > 0] / float(n)
    return {"mse": float((err * err).mean()), "max_abs": float(err.abs().max()), "occupancy": occ,
            "entropy_bits": float(-(p * np.log2(p)).sum()), "bits_per_param": 8.0 * stored / n}


def bench_qerror(torch, nf4, synth, dev):
    """NF4 against Int4 and FP4, with DQ (8-bit float or 8-bit integer second level) and without,
    on a 4096 x 4096 weight drawn N(0, 0.02) and with 1 % of entries from N(0, 0.2) (heavy tail);
    times quantize + dequant per weight."""
    import numpy as np
    tables = {"nf4": nf4.nf4_build_codebook(), "int4": nf4.nf4_build_int4_codebook(),
              "fp4": nf4.nf4_build_fp4_codebook()}
    dists = {"normal": synth.normal_f32(1000, (4096, 4096), 0.02),
             "heavy_tail": synth.heavy_tail_f32(1000, 6000, (4096, 4096), 0.02, 0.2, 0.01)}
    rows = []
    for dname, Wh in dists.items():
        W = torch.from_numpy(Wh).to(dev)
        var = float((W.double() ** 2).mean())
        for cname, cb in tables.items():
            for dqname in ("e4m3", "int8", "none"):
                dq = dqname != "none"
                fmt = dqname if dq else "e4m3"
                st = qerror_gpu(torch, nf4, W, cb, dq, fmt)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(5):
                    if dq:
                        nf4.nf4_dequant(nf4.NF4Weight.from_float(W, cb, dq_format=fmt))
                    else:
                        pk, am = nf4.nf4_quantize(W.reshape(-1), cb)
                        nf4.nf4_dequant_single(pk, am, W.numel(), cb)
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) * 1e3 / 5
                rows.append({"weights": dname, "type": cname, "dq": dqname, "mse": st["mse"],
                             "snr_db": round(10 * np.log10(var / st["mse"]), 3),
                             "max_abs": st["max_abs"], "entropy_bits": round(st["entropy_bits"], 4),
                             "bits_per_param": round(st["bits_per_param"], 4),
                             "occupancy": [int(v) for v in st["occupancy"]],
                             "quantize_dequant_ms": round(ms, 3)})
        del W
    return rows


def bench_gated(torch, nf4, synth, dev, reps=10):
    """Gated MLP at the LLaMA-7B MLP shape (4096 tokens, gate and up 11008 x 4096, r = 64): the
    gated forward (gate and up as one product over both weights, then the glue) against two linear
    forwards and the glue, and the fused backward (dX as one product over both weights) against the
    linears' backward."""
    wl = synth.WORKLOADS["llama7b_mlp"]
    gate, up = wl.linears[0], wl.linears[1]
    M, F, K, r = wl.M, gate.N, gate.K, wl.r
    ws = [nf4.NF4Weight.from_float(torch.from_numpy(synth.weight_f32(wl, lin)).to(dev)) for lin in (gate, up)]
    ad = [tuple(torch.from_numpy(synth.to_bf16_bits(a).view("int16")).to(dev).view(torch.bfloat16)
                for a in synth.lora_f32(wl, lin)) for lin in (gate, up)]
    X = torch.from_numpy(synth.to_bf16_bits(synth.x_f32(wl, M=M, K=K)).view("int16")).to(dev).view(torch.bfloat16)
    s = wl.scale
    wsb = max(nf4.lib.qlora_gated_workspace_size(M, F, K, r), nf4.lib.qlora_linear_workspace_size(M, F, K, r))
    wbuf = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def gated():
        nf4.qlora_gated_fwd(ws[0], ws[1], X, ad[0][0], ad[0][1], ad[1][0], ad[1][1], s, workspace=wbuf)

    def separate():
        G, _ = nf4.qlora_linear_fwd(ws[0], X, ad[0][0], ad[0][1], s, workspace=wbuf)
        U, _ = nf4.qlora_linear_fwd(ws[1], X, ad[1][0], ad[1][1], s, workspace=wbuf)
        nf4.qlora_swiglu_fwd(G, U)

    G, U, _, Tg, Tu = nf4.qlora_gated_fwd(ws[0], ws[1], X, ad[0][0], ad[0][1], ad[1][0], ad[1][1], s, workspace=wbuf)
    dH = torch.randn_like(G)
    dX = torch.empty_like(X)

    def bwd(fuse):
        return lambda: nf4.qlora_gated_bwd(ws[0], ws[1], dH, X, G, U, ad[0][0], ad[0][1], ad[1][0], ad[1][1],
                                           Tg, Tu, s, dX=dX, workspace=wbuf, fuse=fuse)

    out = {"workload": f"gated MLP forward and backward, M={M} F={F} K={K} r={r}"}
    flops = 2 * (2 * M * F * K + 2 * M * K * r + 2 * M * r * F)
    for name, fn in (("fwd_gated", gated), ("fwd_separate", separate), ("bwd_fused", bwd(True)),
                     ("bwd_separate", bwd(False))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4)}
        if name.startswith("fwd"):
            out[name]["TFLOP/s"] = round(flops / ms / 1e9, 1)
    return out


def bench_mid(torch, nf4, synth, dev, Ms=(1, 16, 32, 256, 512, 1536), steps=20, warmup=5):
    """The LLaMA-7B attention projection (W 4096 x 4096, r = 64) forward + backward at token counts
    between the decode GEMVs and the training shapes: the wide GEMV forward (up to 64 tokens), the
    fused dequant GEMMs (the backward, and the forward from 65 tokens) and the expanded-weight GEMM
    below a full wave of output tiles, each with its reduction split over several workgroups where
    the output tiles leave CUs idle (qlora_linear_route gives the paths and splits)."""
    wl = synth.WORKLOADS["llama7b_attn"]
    lin = wl.linears[0]
    out = {"workload": f"W {lin.N}x{lin.K} NF4, LoRA r={wl.r}, forward + backward, by token count"}
    for M in Ms:
        st = make_linear(torch, nf4, synth, wl, lin, M, dev)
        warm(torch, lambda i: step_linear(nf4, st, i), min_calls=warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step_linear(nf4, st, i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        fwd, bwd = linear_flops(M, lin.N, lin.K, wl.r)
        out[f"M{M}"] = {"ms_per_step": round(ms, 4), "TFLOP/s": round((fwd + bwd) / ms / 1e9, 1),
                        "route": nf4.qlora_linear_route(M, lin.N, lin.K, wl.r)}
        del st
    torch.cuda.empty_cache()
    return out


def bench_qkv(torch, nf4, synth, dev, reps=10, rounds=3):
    """The q, k and v projections of the LLaMA-7B attention block (three 4096 x 4096 QLoRA linears
    sharing X, r = 64, forward): qlora_multi_fwd (one product over the concatenated weights)
    against three qlora_linear_fwd calls, at 4096 tokens and at 1024 (where one linear's 64 output
    tiles leave most CUs idle).  The two forms alternate, first one then the other, over `rounds`
    rounds of `reps` calls each; the median round is reported."""
    import numpy as np
    wl = synth.WORKLOADS["llama7b_attn"]
    base = wl.linears[0]
    lins = [synth.Linear(n, base.N, base.K, 1000 + i, 3000 + i, 4000 + i) for i, n in enumerate(("q", "k", "v"))]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)  # noqa: E731
    ws = [nf4.NF4Weight.from_float(torch.from_numpy(synth.weight_f32(wl, l)).to(dev)) for l in lins]
    ad = [tuple(bf(a) for a in synth.lora_f32(wl, l)) for l in lins]
    X_full = bf(synth.x_f32(wl, M=wl.M, K=base.K))
    N, K, r, s = base.N, base.K, wl.r, wl.scale
    out = {"workload": f"q, k, v projections: 3 x W {N}x{K} NF4 sharing X, LoRA r={r}, forward"}
    for M in (wl.M, 1024):
        X = X_full[:M].contiguous()
        wsb = max(nf4.qlora_multi_workspace_size([N] * 3, K, M, r), nf4.qlora_linear_workspace_size(M, N, K, r))
        wbuf = torch.empty(wsb, dtype=torch.uint8, device=dev)
        Ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        Ts = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in range(3)]

        def multi():
            nf4.qlora_multi_fwd(ws, X, [a[0] for a in ad], [a[1] for a in ad], s, workspace=wbuf)

        def separate():
            for w, a, Y, T in zip(ws, ad, Ys, Ts):
                nf4.qlora_linear_fwd(w, X, a[0], a[1], s, Y=Y, T=T, workspace=wbuf)

        flops = 3 * (2 * M * N * K + 2 * M * K * r + 2 * M * r * N)
        times = {"one_product": [], "three_calls": []}
        for rnd in range(rounds):
            order = (("one_product", multi), ("three_calls", separate))
            for name, fn in (order if rnd % 2 == 0 else order[::-1]):
                warm(torch, lambda i: fn(), min_ms=50.0, min_calls=2)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1) / reps)
        res = {}
        for name, t in times.items():
            ms = float(np.median(t))
            res[name] = {"ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 1)}
        out[f"M{M}"] = res
        del wbuf, Ys, Ts
    del ws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="llama7b_attn")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mlp", action="store_true", help="skip the two MLP workloads (c3, c4 keys)")
    ap.add_argument("--no-mid", action="store_true", help="skip the mid-size token counts (mid key)")
    ap.add_argument("--mid", action="store_true", help="time only the mid-size token counts")
    ap.add_argument("--quantize", action="store_true",
                    help="time only quantization + double quantization of the 65B-shaped MLP's weights")
    ap.add_argument("--gemv-only", action="store_true", help="time only the decode-size forward")
    ap.add_argument("--qerror", action="store_true",
                    help="quantization error of NF4, Int4 and FP4, with and without DQ, on synthetic "
                         "normal and heavy-tail 4096 x 4096 weights (one JSON line)")
    ap.add_argument("--gated", action="store_true",
                    help="time the gated MLP forward and backward against separate calls")
    ap.add_argument("--qkv", action="store_true",
                    help="time the q/k/v projections as one product against three linear calls")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of exactly 1 GiB, 5 times (the reference kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the layer would shard "
              "data-parallel with one all-reduce of the LoRA gradients); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_nf4_quantized_codebook_amd as nf4
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return
    if args.gemv_only:
        print(json.dumps({"gemv": bench_gemv(torch, nf4, synth, dev)}), flush=True)
        return
    if args.gated:
        print(json.dumps(bench_gated(torch, nf4, synth, dev)), flush=True)
        return
    if args.qkv:
        print(json.dumps(bench_qkv(torch, nf4, synth, dev)), flush=True)
        return
    if args.mid:
        print(json.dumps(bench_mid(torch, nf4, synth, dev)), flush=True)
        return
    if args.quantize:
        print(json.dumps(bench_quantize(torch, nf4, synth, dev, synth.WORKLOADS["llama65b_mlp"])), flush=True)
        return
    if args.qerror:
        print(json.dumps({"workload": "qerror: 4-bit types on synthetic 4096x4096 weights",
                          "rows": bench_qerror(torch, nf4, synth, dev)}), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    if wl.swiglu:
        # an MLP workload on its own line (the default run carries both MLP workloads as extra keys)
        line = bench_mlp(torch, nf4, synth, dev, wl, steps=args.steps, warmup=args.warmup)
        if wl.name == "llama65b_mlp":
            line["quantize"] = bench_quantize(torch, nf4, synth, dev, wl)
        print(json.dumps({"metric": METRIC, "n_gpus": 1, "dtype": "bf16", "data": "synthetic", **line}),
              flush=True)
        return
    lin = wl.linears[0]
    M, N, K, r = wl.M, lin.N, lin.K, wl.r
    print(f"[bench] workload {wl.name}: M={M} N={N} K={K} r={r}", file=sys.stderr, flush=True)
    st = make_linear(torch, nf4, synth, wl, lin, M, dev)
    for i in range(args.warmup):
        step_linear(nf4, st, i)
    torch.cuda.synchronize()

    # The GEMM launches of every TIMING_EVERY-th timed step are bracketed by HIP events on their
    # stream (recorded by the library); the other steps run uninstrumented, since each event
    # record costs the step about 2.5 us of dispatch.
    nsampled = (args.steps + TIMING_EVERY - 1) // TIMING_EVERY
    timer = nf4.GemmTimer(2 * nsampled)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    cnt = 0
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        sampled = i % TIMING_EVERY == 0
        if sampled:
            timer.arm_at(cnt, 2)
        step_linear(nf4, st, i)
        if sampled:
            cnt += timer.disarm()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = timer.durations_ms(cnt)
    timer.close()
    ms = e0.elapsed_time(e1) / args.steps
    fwd, bwd = linear_flops(M, N, K, r)
    value = (fwd + bwd) / (ms * 1e-3) / 1e12
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}), "
          f"{value:.1f} TFLOP/s", file=sys.stderr, flush=True)

    per_kind = {}
    for kind, d in durs:
        per_kind.setdefault(kind, []).append(d)
    means = {k: sum(v) / len(v) for k, v in per_kind.items()}
    dom = max(means, key=lambda k: means[k])
    flops_launch = gemm_launch_flops(dom, M, N, K, r)
    achieved = flops_launch / (means[dom] * 1e-3) / 1e12
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": gemm_traffic_bytes(dom),
        # operand reads + output write of one launch (bwd: dY, W^T bf16, dT, L1 -> dX; fwd: X, W bf16,
        # sT, L2 -> Y); at this token count the weight is expanded to bf16 by a pass of its own
        "traffic_algorithmic": ((M * N * 2 if dom == 1 else M * K * 2) + N * K * 2 + M * r * 2 +
                                (K * r * 2 + M * K * 2 if dom == 1 else r * N * 2 + M * N * 2)),
        "kernel": "gemm_bf16_kernel<" + ("true" if dom == 1 else "false") + "> (" +
                  ("backward dX" if dom == 1 else "forward Y") + ", bf16-expanded weight)",
        "avg_launch_us": round(means[dom] * 1e3, 2),
        "flops_per_launch": flops_launch,
        "launches_timed": len(per_kind[dom]),
        "step_frac": round(value / BF16_PEAK_TFLOPS, 4),
        "other_gemm_avg_us": {("bwd" if k == 1 else "fwd"): round(v * 1e3, 2) for k, v in means.items()},
    }
    print(f"[bench] dominant kernel: {roofline['kernel']} {roofline['avg_launch_us']} us, "
          f"{roofline['achieved']} TFLOP/s ({roofline['frac'] * 100:.1f}% of peak)", file=sys.stderr,
          flush=True)

    del st
    torch.cuda.empty_cache()
    gemv = None
    if not args.no_gemv:
        gemv = bench_gemv(torch, nf4, synth, dev)
        print(f"[bench] gemv {gemv}", file=sys.stderr, flush=True)

    mlp = {}
    if not args.no_mlp:
        for key, name in (("c3", "llama7b_mlp"), ("c4", "llama65b_mlp")):
            mlp[key] = bench_mlp(torch, nf4, synth, dev, synth.WORKLOADS[name])
            print(f"[bench] {key} {name}: {mlp[key]['value']} TFLOP/s, {mlp[key]['ms_per_step']} ms/step; "
                  f"dominant {mlp[key]['roofline']['kernel']} {mlp[key]['roofline']['avg_launch_us']} us",
                  file=sys.stderr, flush=True)
        mlp["c4"]["quantize"] = bench_quantize(torch, nf4, synth, dev, synth.WORKLOADS["llama65b_mlp"])
        print(f"[bench] c4 quantize {mlp['c4']['quantize']}", file=sys.stderr, flush=True)
        mlp["qkv"] = bench_qkv(torch, nf4, synth, dev)
        print(f"[bench] qkv {mlp['qkv']}", file=sys.stderr, flush=True)
    if not args.no_mid:
        mlp["mid"] = bench_mid(torch, nf4, synth, dev)
        print(f"[bench] mid {mlp['mid']}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(synth, wl, lin)
        print(f"[bench] cpu baseline {cpu}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.notes}; W {N}x{K} NF4 (block 64, double-quant block 256), "
                               f"{M} tokens, LoRA r={r} alpha={wl.alpha:g}, forward + backward (dX, dL1, dL2)",
                   "M": M, "N": N, "K": K, "r": r, "flops_per_step": fwd + bwd},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if gemv is not None:
        line["gemv"] = {"workload": "W 28672x8192 NF4 forward with LoRA r=64, weights rotated over 3 replicas",
                        **gemv}
    line.update(mlp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

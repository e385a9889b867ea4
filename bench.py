"""Benchmark: Direct-P FP4 attention forward on one MI355X.

One step = the whole Direct-P path on one batch of synthetic input already resident in HBM:
MX-quantize Q and K along D and V along the sequence (MXFP4), then the Direct-P forward
(S = QK^T, running max, score-to-code classification, consistent normalizer, P.V, epilogue).
Workload: B=1, H=16, N=4096, D=128, noncausal (the configuration the pages' headline metric
is reported on). FLOPs per step = 4*B*H*N^2*D.

Printed: one JSON line with the driver's fields plus
  roofline     -- the attention kernel against the MXFP4 dense MFMA peak (10.1 PFLOP/s)
  cpu_baseline -- the CPU oracle timed on a bounded sample of the same workload
  extra        -- kernel-only TFLOP/s, the FP4/BF16 ratio against the BF16-MFMA variant of the
                  same kernel design (its V transposed once, outside the timed launches; both
                  kernels timed back to back), quantizer GB/s, the causal FP8 forward and FP8 backward at the
                  8B training shape (B=1, H=32, Hkv=8, N=8192, D=128), and Direct-P with its
                  FP4/BF16 ratio at the DiT shape with outlier channels (B=1, H=24, N=32768, D=128),
                  and the QKV projection with the quantization in its epilogue
                  (fp4attn_project_qkv) against a GEMM, a layout copy and the quantizer.

roofline.clock_ghz_measured is the shader clock measured live right after the timed kernels
(fp4attn_clock_probe: s_memtime over s_memrealtime under an MFMA + VALU load on every CU), and
roofline.frac_at_measured_clock the fraction of the peak scaled to that clock.

Untimed warm-up: at least W steps, and more until about 150 ms have passed (the GPU's clocks rise
over the first tens of milliseconds of work); extra.warmup_steps_run gives the count.

The timed region is K steps with plain launches (value, ms_per_step). The attention kernel's
duration for roofline.achieved comes from a second run of max(K, 100) identical steps right after
it, in which each step's attention kernel carries a pair of HIP events bound to its own dispatch
(fp4attn_fwd_ex): the median of those kernel durations. The events are kept out of the timed
region because they lengthen each step by a few microseconds (the runtime adds a marker for the
start event); extra.ms_per_step_with_kernel_events reports that run's step time.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--only-kernel] [--only-bwd]
       [--only-quant] [--only-project] [--only-project-train] [--only-nvfp4] [--only-causal] [--only-fp8route]
       [--only-bf16] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Direct-P fwd TFLOP/s at H16 N4096 D128; % of MXFP4 MFMA peak; FP4/BF16 x"
PEAK_MXFP4_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA, published
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5030.0  # MI355X dense FP8 MFMA, published
# FP8-route forward: half of its FLOPs on FP4 (QK^T), half on FP8 (P.V)
PEAK_FWD_FP4_FP8_TFLOPS = 2.0 / (1.0 / PEAK_MXFP4_TFLOPS + 1.0 / PEAK_FP8_TFLOPS)
# backward: 1 FP4 product (S) and 4 FP8 products (dP, dV, dQ, dK) of equal size
PEAK_BWD_TFLOPS = 5.0 / (1.0 / PEAK_MXFP4_TFLOPS + 4.0 / PEAK_FP8_TFLOPS)
# NVFP4-style Q/K route: QK^T on the BF16 MFMA, P.V on the FP4 MFMA
PEAK_NVFP4_ROUTE_TFLOPS = 2.0 / (1.0 / PEAK_BF16_TFLOPS + 1.0 / PEAK_MXFP4_TFLOPS)
HBM_GBPS = 8000.0
# HBM bytes per launch of the Direct-P kernel from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE,
# each scaled by what the counter reads for a plain 256 MiB copy; valid only for the kernel
# sources it was measured on (profiles/attn_fwd_directp_h16_n4096_d128.md), else null.
MEASURED_TRAFFIC = {"sources_sha256_prefix": "67825b45f20c8592", "bytes": (6631.0 * 2.0 + 16642.0 * 1.0) * 1024}
TRAFFIC_SOURCES = ("attn_fwd_directp.hip", "fwd_common.h", "device_common.h")
# the clock the Direct-P kernel ran at in the counter harness's clock pass (GRBM_GUI_ACTIVE per XCC
# over a sustained launch of the same kernel, profiles/attn_fwd_directp_h16_n4096_d128.md); the
# JSON line carries the clock measured live on the GPU that ran it (fp4attn_clock_probe)
COUNTER_PASS_CLOCK_GHZ = 2.300
DATASHEET_CLOCK_GHZ = 2.4


def sources_sha():
    import hashlib

    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, "precision_attention_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    ok = MEASURED_TRAFFIC["sources_sha256_prefix"] == sources_sha()
    return MEASURED_TRAFFIC["bytes"] if ok else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-kernel", action="store_true", help="time the attention kernel only (for profiling)")
    ap.add_argument("--anchored", action="store_true",
                    help="with --only-kernel: the Direct-P kernel on the integer-log2 anchor")
    ap.add_argument("--n", type=int, default=4096,
                    help="with --only-kernel: the sequence length (B=1, H=16, D=128); the counters' clock pass "
                         "uses a long kernel")
    ap.add_argument("--only-bwd", action="store_true",
                    help="time the causal FP8 backward at B=1 H=32 Hkv=8 N=8192 D=128 only (for profiling)")
    ap.add_argument("--only-quant", action="store_true",
                    help="time the one-launch MX quantization of Q, K and V only (for profiling)")
    ap.add_argument("--only-project", action="store_true",
                    help="time the fused QKV projection at B=1 N=4096 Dm=2048 H=16 D=128 only (for profiling)")
    ap.add_argument("--only-project-train", action="store_true",
                    help="time the fused QKV projection at B=1 N=8192 Dm=4096 H=32 Hkv=8 D=128 with the FP8 "
                         "views only (for profiling)")
    ap.add_argument("--only-nvfp4", action="store_true",
                    help="time the NVFP4-style Q/K forward at B=1 H=16 N=4096 D=128 only (for profiling)")
    ap.add_argument("--only-causal", action="store_true",
                    help="time the causal FP8 forward at B=1 Hq=32 Hkv=8 N=8192 D=128 only (for profiling)")
    ap.add_argument("--only-fp8route", action="store_true",
                    help="time the noncausal FP8 P/V route at B=1 H=16 N=4096 D=128 only (for profiling)")
    ap.add_argument("--only-bf16", action="store_true",
                    help="time the BF16-MFMA forward at B=1 H=16 N=4096 D=128 only (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def to_dev(bits, dev):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def warm(fn, ms=200.0, batch=5):
    """Run fn() until about ms of wall time has passed: the GPU's clocks rise over the first tens
    of milliseconds of sustained work, and the heavy kernels keep speeding up for longer."""
    import torch

    t0 = time.perf_counter()
    while ms > 0 and (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()


def time_region(fn, steps, warmup, warm_ms=200.0):
    """Average ms per call of fn() on the current stream, bracketed by synchronizations, after a
    warm-up of warmup calls and about warm_ms of wall time."""
    import torch

    for _ in range(warmup):
        fn()
    warm(fn, warm_ms)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def projection_bench(B, N, Dm, H, Hkv, D, v_fmt, views, steps=20):
    """The QKV projection with the MX quantization in its epilogue (one launch) against the
    separate path: a GEMM into bf16 (torch.mm, hipBLASLt), the copy of Q, K, V into per-head
    [B, heads, N, D] layout, and the quantizer launches. Returns a dict of times (ms)."""
    import torch

    import precision_attention_amd as pa
    from precision_attention_amd.inputs import projection_inputs

    dev = torch.device("cuda:0")
    F = (H + 2 * Hkv) * D
    xin = projection_inputs(B, N, Dm, H, Hkv, D, seed=1)
    x, w = to_dev(xin["x"], dev), to_dev(xin["w"], dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    fused = pa.ProjectCall(x, w, H, Hkv, D, v_fmt=v_fmt, fp8_views=views)
    f_ms = time_region(lambda: fused(stream), steps, 3)
    wt = w.t().contiguous()  # [Dm, F]: the GEMM's right operand as a plain row-major matrix
    x2 = x.view(B * N, Dm)
    y = torch.empty((B * N, F), dtype=torch.bfloat16, device=dev)
    qh = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    kh = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    vh = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    calls = [pa.QuantizeBatchCall((qh, kh, vh), (pa.MXFP4, pa.MXFP4, v_fmt), (pa.ALONG_D, pa.ALONG_D, pa.ALONG_SEQ))]
    if views:
        calls.append(pa.QuantizeBatchCall((qh, kh, vh), (pa.MXFP8,) * 3, (pa.ALONG_SEQ, pa.ALONG_SEQ, pa.ALONG_D)))

    def gemm():
        torch.mm(x2, wt, out=y)

    def split():
        t = y.view(B, N, H + 2 * Hkv, D).permute(0, 2, 1, 3)
        qh.copy_(t[:, :H])
        kh.copy_(t[:, H:H + Hkv])
        vh.copy_(t[:, H + Hkv:])

    def quant():
        for c in calls:
            c(stream)

    g_ms = time_region(gemm, steps, 3)
    s_ms = time_region(split, steps, 3)
    q_ms = time_region(quant, steps, 3)
    t_ms = time_region(lambda: (gemm(), split(), quant()), steps, 3)
    flops = 2.0 * B * N * Dm * F
    return {"fused_ms": f_ms, "fused_tflops": flops / f_ms / 1e9,
            "fused_pct_of_bf16_peak": 100.0 * flops / f_ms / 1e9 / PEAK_BF16_TFLOPS,
            "separate_ms": t_ms, "separate_gemm_ms": g_ms, "separate_gemm_tflops": flops / g_ms / 1e9,
            "separate_layout_copy_ms": s_ms, "separate_quantize_ms": q_ms, "separate_over_fused": t_ms / f_ms}


def cpu_baseline(x, B, H, N, D, KB, budget_s=10.0, max_passes=10):
    """The oracle, as it stands, on the same workload: whole passes of its Direct-P forward
    (MX quantization of Q, K, V and attention over every query row), repeated until about
    budget_s of CPU time has been spent (the oracle finishes one pass in seconds)."""
    import oracle

    times = []
    while (not times or sum(times) < budget_s) and len(times) < max_passes:
        t0 = time.perf_counter()
        oracle.directp_forward(x["q"], x["k"], x["v"], KB=KB)
        times.append(time.perf_counter() - t0)
    t = sum(times) / len(times)
    return {
        "value": 4.0 * B * H * N * N * D / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "the whole workload (all %d query rows, quantization included), %d passes, %.2f s per pass" % (
            B * H * N, len(times), t),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import precision_attention_amd as pa
    from precision_attention_amd.inputs import attention_inputs

    dev = torch.device("cuda:0")
    B, H, Hkv, N, D = 1, 16, 16, (args.n if args.only_kernel else 4096), 128
    x = attention_inputs(B, H, Hkv, N, D, seed=0)
    q, k, v = (to_dev(x[n], dev) for n in ("q", "k", "v"))
    qm = pa.mx_empty(B, H, N, D, pa.MXFP4, pa.ALONG_D, dev)
    km = pa.mx_empty(B, Hkv, N, D, pa.MXFP4, pa.ALONG_D, dev)
    vm = pa.mx_empty(B, Hkv, N, D, pa.MXFP4, pa.ALONG_SEQ, dev)
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    flops = 4.0 * B * H * N * N * D

    # prepared calls: validated once, so a call costs the host only the C call itself
    quantize = pa.QuantizeBatchCall((q, k, v), (pa.MXFP4, pa.MXFP4, pa.MXFP4),
                                    (pa.ALONG_D, pa.ALONG_D, pa.ALONG_SEQ), outs=(qm, km, vm))
    attn = pa.FwdCall(qm, km, vm, causal=False, out=o, lse=lse)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms = time_region(lambda: dst.copy_(src), args.steps, args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "copy_256MiB", "bytes_read": 256 << 20, "bytes_written": 256 << 20, "ms": ms,
                          "gbps": 2 * (256 << 20) / ms / 1e6}), flush=True)
        return

    if args.only_bwd:
        xb = attention_inputs(1, 32, 8, 8192, 128, seed=0, with_do=True)
        qb, kb, vb, dob = (to_dev(xb[n], dev) for n in ("q", "k", "v", "do"))
        qbm = pa.quantize_mx(qb, pa.MXFP4, pa.ALONG_D)
        kbm = pa.quantize_mx(kb, pa.MXFP4, pa.ALONG_D)
        vbm = pa.quantize_mx(vb, pa.MXFP8, pa.ALONG_SEQ)
        ob, lb = pa.fwd(qbm, kbm, vbm, causal=True)
        q8 = pa.quantize_mx(qb, pa.MXFP8, pa.ALONG_SEQ)
        k8 = pa.quantize_mx(kb, pa.MXFP8, pa.ALONG_SEQ)
        v8 = pa.quantize_mx(vb, pa.MXFP8, pa.ALONG_D)
        ws = torch.empty(pa.bwd_workspace_bytes(1, 32, 8, 8192, 128), dtype=torch.uint8, device=dev)
        ms = time_region(lambda: pa.bwd(qbm, kbm, q8, k8, v8, ob, dob, lb, causal=True, workspace=ws), args.steps,
                         args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "attn_bwd_causal_h32kv8_n8192_d128", "ms": ms,
                          "tflops": 10.0 * 32 * 8192 * 8192 * 128 / 2 / ms / 1e9}), flush=True)
        return

    if args.only_quant:
        ms = time_region(quantize, args.steps, args.warmup, warm_ms=0.0)
        nbytes = 3 * B * H * N * D * (2 + 0.5 + 1.0 / 32)
        print(json.dumps({"kernel": "quant_kernel<128> (Q, K along D; V along the sequence; MXFP4)", "ms": ms,
                          "gbps": nbytes / ms / 1e6}), flush=True)
        return

    if args.only_project:
        from precision_attention_amd.inputs import projection_inputs

        xin = projection_inputs(1, 4096, 2048, 16, 16, 128, seed=1)
        call = pa.ProjectCall(to_dev(xin["x"], dev), to_dev(xin["w"], dev), 16, 16, 128)
        ms = time_region(call, args.steps, args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "proj_qkv_kernel<128> (B1 N4096 Dm2048 H16 D128, MXFP4 Q, K, V)", "ms": ms,
                          "tflops": 2.0 * 4096 * 2048 * 6144 / ms / 1e9}), flush=True)
        return

    if args.only_project_train:
        from precision_attention_amd.inputs import projection_inputs

        xin = projection_inputs(1, 8192, 4096, 32, 8, 128, seed=1)
        call = pa.ProjectCall(to_dev(xin["x"], dev), to_dev(xin["w"], dev), 32, 8, 128, pa.MXFP8, True)
        ms = time_region(call, args.steps, args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "proj_qkv_wide_kernel<128> (B1 N8192 Dm4096 H32 Hkv8 D128, MXFP8 V, FP8 views)",
                          "ms": ms, "tflops": 2.0 * 8192 * 4096 * 6144 / ms / 1e9}), flush=True)
        return

    if args.only_nvfp4:
        quantize()
        qn, kn = pa.quantize_nvfp4(q), pa.quantize_nvfp4(k)
        call = pa.FwdNvCall(qn, kn, vm, out=o, lse=lse)
        ms = time_region(call, args.steps, args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "attn_fwd_nvfp4 (B1 H16 N4096 D128)", "ms": ms, "tflops": flops / ms / 1e9}),
              flush=True)
        return

    if args.only_causal:
        xc = attention_inputs(1, 32, 8, 8192, 128, seed=0)
        qc, kc, vc = (to_dev(xc[n], dev) for n in ("q", "k", "v"))
        qcm = pa.quantize_mx(qc, pa.MXFP4, pa.ALONG_D)
        kcm = pa.quantize_mx(kc, pa.MXFP4, pa.ALONG_D)
        vcm = pa.quantize_mx(vc, pa.MXFP8, pa.ALONG_SEQ)
        call = pa.FwdCall(qcm, kcm, vcm, causal=True)
        ms = time_region(call, args.steps, args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "attn_fwd_kernel<128, true, true> (B1 Hq32 Hkv8 N8192 D128, causal, FP8 P and V)",
                          "ms": ms, "tflops": 4.0 * 32 * 8192 * 8192 * 128 / 2 / ms / 1e9}), flush=True)
        return

    if args.only_fp8route:
        quantize()
        v8m = pa.quantize_mx(v, pa.MXFP8, pa.ALONG_SEQ)
        call = pa.FwdCall(qm, km, v8m, causal=False, out=o, lse=lse)
        ms = time_region(call, args.steps, args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "attn_fwd_kernel<128, false, true> (B1 H16 N4096 D128, FP8 P and V)", "ms": ms,
                          "tflops": flops / ms / 1e9}), flush=True)
        return

    if args.only_bf16:
        vt = v.transpose(-1, -2).contiguous()
        ms = time_region(lambda: pa.fwd_bf16(q, k, vt, causal=False, out=o, lse=lse), args.steps, args.warmup,
                         warm_ms=0.0)
        print(json.dumps({"kernel": "attn_fwd_bf16 (B1 H16 N4096 D128)", "ms": ms, "tflops": flops / ms / 1e9}),
              flush=True)
        return

    if args.only_kernel:
        quantize()
        fn = pa.FwdCall(qm, km, vm, causal=False, out=o, lse=lse, anchored=True) if args.anchored else attn
        ms = time_region(fn, args.steps, args.warmup, warm_ms=0.0)
        print(json.dumps({"kernel": "attn_fwd_directp" + ("_anchored" if args.anchored else ""), "ms": ms,
                          "tflops": flops / ms / 1e9}), flush=True)
        return

    # ---- timed region: K whole steps with plain launches ----
    # untimed warm-up: the W steps asked for, and more until about 150 ms have passed, so that the
    # timed steps do not run while the GPU's clocks are still rising (a short W would time a cold
    # GPU); the number of warm-up steps run is reported
    warm_steps = 0
    t_w0 = time.perf_counter()
    while warm_steps < args.warmup or (time.perf_counter() - t_w0) < 0.15:
        quantize()
        attn()
        warm_steps += 1
        if warm_steps % 50 == 0 or warm_steps == args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream
    t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record()
    for i in range(args.steps):
        quantize(stream)
        attn(stream)
    t_all1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_all0.elapsed_time(t_all1) / args.steps
    value = flops / ms_step / 1e9  # TFLOP/s

    # ---- the attention kernel's own duration: the same steps again, each attention kernel with a
    # pair of events bound to its dispatch ----
    n_ev = max(args.steps, 100)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in starts + ends:
        e.record()  # torch creates an event at its first record; the steps below re-bind it
    torch.cuda.synchronize()
    t_all0.record()
    for i in range(n_ev):
        quantize(stream)
        attn(stream, events=(starts[i], ends[i]))
    t_all1.record()
    torch.cuda.synchronize()
    ev_step_ms = t_all0.elapsed_time(t_all1) / n_ev
    attn_samples = np.array([starts[i].elapsed_time(ends[i]) for i in range(n_ev)])
    attn_ms = float(np.median(attn_samples))

    # ---- the shader clock, measured live right after the timed kernels: s_memtime over
    # s_memrealtime in every workgroup of a load of FP4 MFMAs and VALU work in the Direct-P loop's
    # proportion on every CU (fp4attn_clock_probe); the median of three probes ----
    probes = [pa.clock_probe() for _ in range(3)]
    clock_ghz = float(np.median([p["ghz_median"] for p in probes]))

    # ---- other measurements (outside the timed region) ----
    quant_ms = time_region(quantize, 20, 3)
    quant_bytes = 3 * B * H * N * D * (2 + 0.5 + 1.0 / 32)
    extra = {
        "attn_kernel_ms": attn_ms,
        "attn_kernel_ms_mean": float(attn_samples.mean()),
        "attn_kernel_ms_min": float(attn_samples.min()),
        "attn_kernel_ms_max": float(attn_samples.max()),
        "attn_kernel_samples": int(attn_samples.size),
        "attn_kernel_tflops": flops / attn_ms / 1e9,
        "pct_of_mxfp4_peak": 100.0 * flops / attn_ms / 1e9 / PEAK_MXFP4_TFLOPS,
        "quantize_qkv_ms": quant_ms,
        "quantize_gbps": quant_bytes / quant_ms / 1e6,
        "wall_s_timed_region": wall,
        "ms_per_step_with_kernel_events": ev_step_ms,
        "warmup_steps_run": warm_steps,
        "clock_probe_ghz_medians": [p["ghz_median"] for p in probes],
        "clock_probe_ghz_min_max": [min(p["ghz_min"] for p in probes), max(p["ghz_max"] for p in probes)],
    }
    attn_b2b_ms = time_region(attn, 20, 3)
    extra["attn_kernel_back_to_back_ms"] = attn_b2b_ms
    extra["attn_kernel_back_to_back_tflops"] = flops / attn_b2b_ms / 1e9
    ob = torch.empty_like(o)
    lb = torch.empty_like(lse)
    vt = v.transpose(-1, -2).contiguous()  # the BF16 kernel's V layout, made outside the timed region
    try:
        bf_ms = time_region(lambda: pa.fwd_bf16(q, k, vt, causal=False, out=ob, lse=lb), 20, 3)
        extra["bf16_kernel_ms"] = bf_ms
        extra["bf16_kernel_tflops"] = flops / bf_ms / 1e9
        extra["bf16_pct_of_bf16_peak"] = 100.0 * flops / bf_ms / 1e9 / PEAK_BF16_TFLOPS
        # both kernels timed the same way: back-to-back launches between two events
        extra["fp4_over_bf16"] = bf_ms / attn_b2b_ms
    except pa.Fp4AttnError as e:
        extra["bf16_kernel_ms"] = None
        extra["bf16_error"] = str(e)
    # Direct-P on the integer-log2 anchor (the range-guarded route) at the same shape: kernel time
    # from dispatch-bound events (median of 100 launches) and back to back
    attn_a = pa.FwdCall(qm, km, vm, causal=False, out=ob, lse=lb, anchored=True)
    warm(lambda: (quantize(stream), attn_a(stream)))
    # the same sequence as the headline's event loop (a quantizer launch between the kernels), so
    # the two medians compare
    ev_a = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(100)]
    for e0, e1 in ev_a:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for e in ev_a:
        quantize(stream)
        attn_a(stream, events=e)
    torch.cuda.synchronize()
    a_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev_a]))
    extra["anchored_directp_kernel_ms"] = a_ms
    extra["anchored_directp_tflops"] = flops / a_ms / 1e9
    extra["anchored_directp_pct_of_mxfp4_peak"] = 100.0 * flops / a_ms / 1e9 / PEAK_MXFP4_TFLOPS
    extra["anchored_directp_back_to_back_ms"] = time_region(lambda: attn_a(stream), 20, 3)
    extra["anchored_step_ms"] = time_region(lambda: (quantize(stream), attn_a(stream)), 20, 3)
    # NVFP4-style Q and K (E4M3 scales per 16) at the same shape: the quantizer for Q and K, and the
    # anchored Direct-P kernel with QK^T on the BF16 MFMA from their bf16 expansions
    qn, kn = pa.quantize_nvfp4(q), pa.quantize_nvfp4(k)
    nv_call = pa.FwdNvCall(qn, kn, vm, out=ob, lse=lb)
    nv_ms = time_region(lambda: nv_call(stream), 20, 3)
    extra["nvfp4_fwd_ms"] = nv_ms
    extra["nvfp4_fwd_tflops"] = flops / nv_ms / 1e9
    extra["nvfp4_fwd_pct_of_bf16_fp4_peak"] = 100.0 * flops / nv_ms / 1e9 / PEAK_NVFP4_ROUTE_TFLOPS
    extra["nvfp4_quantize_qk_ms"] = time_region(
        lambda: (pa.quantize_nvfp4(q, out=qn), pa.quantize_nvfp4(k, out=kn)), 20, 3)
    # the noncausal FP8 P/V route at the same shape (MXFP8 V, E4M3 P)
    vm8 = pa.quantize_mx(v, pa.MXFP8, pa.ALONG_SEQ)
    f8_ms = time_region(lambda: pa.fwd(qm, km, vm8, causal=False, out=ob, lse=lb), 20, 3)
    extra["fp8_route_fwd_h16_n4096_ms"] = f8_ms
    extra["fp8_route_fwd_h16_n4096_tflops"] = flops / f8_ms / 1e9
    extra["fp8_route_fwd_pct_of_fp4_fp8_peak"] = 100.0 * flops / f8_ms / 1e9 / PEAK_FWD_FP4_FP8_TFLOPS
    del vm8
    # causal FP8 forward at the 8B training shape
    xc = attention_inputs(1, 32, 8, 8192, 128, seed=0)
    qc, kc, vc = (to_dev(xc[n], dev) for n in ("q", "k", "v"))
    qcm = pa.quantize_mx(qc, pa.MXFP4, pa.ALONG_D)
    kcm = pa.quantize_mx(kc, pa.MXFP4, pa.ALONG_D)
    vcm = pa.quantize_mx(vc, pa.MXFP8, pa.ALONG_SEQ)
    oc = torch.empty((1, 32, 8192, 128), dtype=torch.bfloat16, device=dev)
    lc = torch.empty((1, 32, 8192), dtype=torch.float32, device=dev)
    c_ms = time_region(lambda: pa.fwd(qcm, kcm, vcm, causal=True, out=oc, lse=lc), 20, 3)
    c_flops = 4.0 * 32 * 8192 * 8192 * 128 / 2
    extra["causal_fwd_h32kv8_n8192_ms"] = c_ms
    extra["causal_fwd_h32kv8_n8192_tflops"] = c_flops / c_ms / 1e9
    extra["causal_fwd_pct_of_fp4_fp8_peak"] = 100.0 * c_flops / c_ms / 1e9 / PEAK_FWD_FP4_FP8_TFLOPS
    # FP8 backward at the same shape (Delta, dO views, dK/dV, dQ): 5 products of 2*N^2*D per
    # head, halved by the mask
    doc = to_dev(attention_inputs(1, 32, 8, 8192, 128, seed=0, with_do=True)["do"], dev)
    q8 = pa.quantize_mx(qc, pa.MXFP8, pa.ALONG_SEQ)
    k8 = pa.quantize_mx(kc, pa.MXFP8, pa.ALONG_SEQ)
    v8 = pa.quantize_mx(vc, pa.MXFP8, pa.ALONG_D)
    ws = torch.empty(pa.bwd_workspace_bytes(1, 32, 8, 8192, 128), dtype=torch.uint8, device=dev)
    b_ms = time_region(lambda: pa.bwd(qcm, kcm, q8, k8, v8, oc, doc, lc, causal=True, workspace=ws), 10, 2)
    b_flops = 10.0 * 32 * 8192 * 8192 * 128 / 2
    extra["causal_bwd_h32kv8_n8192_ms"] = b_ms
    extra["causal_bwd_h32kv8_n8192_tflops"] = b_flops / b_ms / 1e9
    extra["causal_bwd_pct_of_fp4_fp8_peak"] = 100.0 * b_flops / b_ms / 1e9 / PEAK_BWD_TFLOPS
    del qc, kc, vc, qcm, kcm, vcm, oc, lc, doc, q8, k8, v8, ws
    # Direct-P at the DiT/video shape with outlier channels (B=1, H=24, N=32768, D=128; the
    # shape of the pages' peak forward figure) and the BF16 variant at the same shape
    xd = attention_inputs(1, 24, 24, 32768, 128, seed=0, outlier_frac=0.01)
    qd, kd, vd = (to_dev(xd[n], dev) for n in ("q", "k", "v"))
    del xd
    qdm = pa.quantize_mx(qd, pa.MXFP4, pa.ALONG_D)
    kdm = pa.quantize_mx(kd, pa.MXFP4, pa.ALONG_D)
    vdm = pa.quantize_mx(vd, pa.MXFP4, pa.ALONG_SEQ)
    od = torch.empty((1, 24, 32768, 128), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((1, 24, 32768), dtype=torch.float32, device=dev)
    d_flops = 4.0 * 24 * 32768 * 32768 * 128
    d_ms = time_region(lambda: pa.fwd(qdm, kdm, vdm, causal=False, out=od, lse=ld), 5, 1)
    extra["dit_directp_h24_n32768_ms"] = d_ms
    extra["dit_directp_h24_n32768_tflops"] = d_flops / d_ms / 1e9
    extra["dit_directp_h24_n32768_pct_of_mxfp4_peak"] = 100.0 * d_flops / d_ms / 1e9 / PEAK_MXFP4_TFLOPS
    dqn, dkn = pa.quantize_nvfp4(qd), pa.quantize_nvfp4(kd)
    dn_ms = time_region(lambda: pa.fwd_nvfp4(dqn, dkn, vdm, out=od, lse=ld), 5, 1)
    extra["dit_nvfp4_h24_n32768_ms"] = dn_ms
    extra["dit_nvfp4_h24_n32768_pct_of_bf16_fp4_peak"] = 100.0 * d_flops / dn_ms / 1e9 / PEAK_NVFP4_ROUTE_TFLOPS
    del dqn, dkn
    da_ms = time_region(lambda: pa.fwd(qdm, kdm, vdm, causal=False, out=od, lse=ld, anchored=True), 5, 1)
    extra["dit_anchored_h24_n32768_ms"] = da_ms
    extra["dit_anchored_h24_n32768_pct_of_mxfp4_peak"] = 100.0 * d_flops / da_ms / 1e9 / PEAK_MXFP4_TFLOPS
    try:
        vdt = vd.transpose(-1, -2).contiguous()
        db_ms = time_region(lambda: pa.fwd_bf16(qd, kd, vdt, causal=False, out=od, lse=ld), 3, 1)
        del vdt
        extra["dit_bf16_h24_n32768_ms"] = db_ms
        extra["dit_fp4_over_bf16"] = db_ms / d_ms
    except pa.Fp4AttnError as e:
        extra["dit_bf16_error"] = str(e)
    del qd, kd, vd, qdm, kdm, vdm, od, ld
    # the QKV projection that feeds the headline attention (model dimension H D = 2048; MXFP4 Q,
    # K, V) and the 8B training shape's (Dm 4096, H32 Hkv8; MXFP8 V and the backward's FP8 views)
    for key, cfg in (("project_h16_n4096_dm2048", (1, 4096, 2048, 16, 16, 128, pa.MXFP4, False)),
                     ("project_train_h32kv8_n8192_dm4096", (1, 8192, 4096, 32, 8, 128, pa.MXFP8, True))):
        for name, val in projection_bench(*cfg).items():
            extra["%s_%s" % (key, name)] = val

    traffic = measured_traffic()
    roofline = {
        "bound": "mfma",
        "achieved": flops / attn_ms / 1e9,
        "peak": PEAK_MXFP4_TFLOPS,
        "unit": "TFLOP/s",
        "frac": flops / attn_ms / 1e9 / PEAK_MXFP4_TFLOPS,
        "traffic": traffic,
        "clock_ghz_measured": clock_ghz,
        "frac_at_measured_clock": flops / attn_ms / 1e9 / PEAK_MXFP4_TFLOPS * DATASHEET_CLOCK_GHZ / clock_ghz,
        "clock_measurement": "live: shader cycles (s_memtime) over real-time ticks (s_memrealtime), median "
                             "over 512 workgroups of fp4attn_clock_probe (FP4 MFMAs and VALU in the Direct-P "
                             "loop's proportion on every CU), median of 3 probes right after the timed kernels; "
                             "the counters' clock pass on a sustained Direct-P launch read %.3f GHz on the box "
                             "of the committed profile (boxes differ)" % COUNTER_PASS_CLOCK_GHZ,
        "kernel": "attn_fwd_directp_kernel<128>",
        "algorithmic_flops_per_launch": flops,
        "timing": "median kernel duration over %d steps, HIP events bound to the kernel's dispatch" % n_ev,
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, B, H, N, D, pa.key_block(D, False))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "directp_h16_n4096_d128", "B": B, "H": H, "Hkv": Hkv, "N": N, "D": D,
                   "causal": False, "key_block": pa.key_block(D, False)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

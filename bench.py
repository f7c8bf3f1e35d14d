"""Benchmark of the MXFP8 attention training hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input at the B=4, H=16,
N=4096, D=128 shape (non-causal, inputs ~ N(0,1) bf16, already resident in HBM):
  quantize Q, K (32x32 square blocks), V (32x1 along keys for the forward, 1x32 along D for the
  backward) and dO (square blocks)  ->  attention forward  ->  attention backward (FP16 dQ with a
  static scale of 1).
value = attention FLOPs of the step (forward 4 N^2 D per head, backward 2.5x forward) / step time,
in PF/s. The forward and backward calls are also timed on their own (HIP events on the stream the
kernels run on), which gives the per-call PF/s and the fraction of the MI355X dense MXFP8 MFMA
peak (5.03 PF/s = 256 CU x 4 SIMD x 2048 FLOP/clk x 2.4 GHz).

cpu_baseline: the CPU oracle, as it is, on a bounded sample of the same workload (batch element 0,
6 of the 16 heads, N = 4096, forward + backward) on this host's cores.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MXFP8 = 5.03e15  # FLOP/s
PEAK_HBM = 8.0e12     # B/s
B, H, N, D = 4, 16, 4096, 128
SEED = 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dq-mode", type=int, default=1, help="0 = FP32 dQ, 1 = FP16 static-scale dQ")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy first (reference kernel for HBM byte counters)")
    ap.add_argument("--producers", action="store_true",
                    help="time the fused RMSNorm+quantize producer at the module workload's shapes and the jagged "
                         "scale scatter instead of the attention step (one JSON line of its own)")
    ap.add_argument("--projection", action="store_true",
                    help="time the module workload's projection GEMM+quantize producers instead of the attention "
                         "step (one JSON line of its own)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bwd_B4_H16_N4096_hbm_traffic.md")
BWD_SOURCES = [os.path.join(ROOT, "precision_mxfp8_block_amd", "csrc", f) for f in ("attn_bwd.hip", "mx_device.h")]


def bwd_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in BWD_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per backward call (its three kernels) from the committed counter summary, or None
    when the backward kernel sources changed since the counters were taken (or no summary exists)."""
    import re
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", txt)
    m_bytes = re.search(r"hbm_bytes_per_call:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != bwd_source_hash():
        return None
    return float(m_bytes.group(1))


def make_inputs(torch, synth):
    T, C = B * N, H * D
    cu = synth.cu_seqlens([N] * B)
    host = {n: synth.normal_bf16(SEED, s, (T, C)) for n, s in
            (("q", synth.STREAM_Q), ("k", synth.STREAM_K), ("v", synth.STREAM_V), ("do", synth.STREAM_DO))}
    dev = {n: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for n, a in host.items()}
    cu_d = torch.from_numpy(cu).cuda()
    return host, dev, cu, cu_d


CPU_HEADS = 6  # heads of batch element 0 in the CPU sample (about 25 s of oracle work on 16 cores)


def cpu_baseline(host, cu):
    import oracle
    nthreads = max(1, min(16, os.cpu_count() or 1))
    # sample: sequence 0 (N tokens), the first CPU_HEADS heads, forward + backward (FP32 dQ)
    hs = CPU_HEADS
    xs = {n: np.ascontiguousarray(a[:N, :hs * D]) for n, a in host.items()}
    cu0 = np.array([0, N], np.int32)
    c = float(np.float32(1 / math.sqrt(D)))
    t0 = time.perf_counter()
    q = oracle.quantize(xs["q"], cu0, oracle.SQ32)
    k = oracle.quantize(xs["k"], cu0, oracle.SQ32)
    v = oracle.quantize(xs["v"], cu0, oracle.COL32)
    vd = oracle.quantize(xs["v"], cu0, oracle.ROW32)
    do = oracle.quantize(xs["do"], cu0, oracle.SQ32)
    o16, _, lse = oracle.attn_fwd_mx(q[0], q[1], 2, k[0], k[1], 2, v[0], v[1], 1, cu0, cu0, hs, D, c, False,
                                     nthreads=nthreads)
    oracle.attn_bwd_mx(q[0], q[1], k[0], k[1], vd[0], vd[1], 0, do[0], do[1], o16, xs["do"], lse, cu0, cu0, hs, D, c,
                       False, 0, 1.0, nthreads=nthreads)
    dt = time.perf_counter() - t0
    flops = 3.5 * 4.0 * N * N * D * hs
    return {"value": flops / dt / 1e15, "unit": "PF/s", "cores": nthreads, "kind": "oracle",
            "sample": f"batch element 0 of the step, heads 0-{hs - 1} of {H} (N={N}): quantize + forward + "
                      f"backward (FP32 dQ), {dt:.1f} s wall"}


MODULE_SEED, MODULE_B, MODULE_DIM = 4, 64, 1024


def bench_projection(args, torch, mx, synth):
    """The cross-attention module's projection producers (GEMM + SQ32 quantize with both scale layouts):
    X [T, 1024] (bf16 N(0,1) quantized SQ32) times W [1024, 1024] (bf16 N(0,0.02) quantized ROW32), for
    the query side (64 samples x 256 tokens) and the key/value side (64 jagged lengths uniform in
    [256, 2048]). value = FLOPs of the key/value-side call / its mean time over back-to-back calls (HIP
    events on the launch stream)."""
    stream = torch.cuda.current_stream()
    C = MODULE_DIM
    w_host = synth.normal_bf16(MODULE_SEED, synth.STREAM_WEIGHT, (C, C), std=0.02)
    w_dev = torch.from_numpy(w_host.view(np.int16)).view(torch.bfloat16).cuda()
    wd, ws, _ = mx.quantize(w_dev, np.array([0, C], np.int32), torch.tensor([0, C], dtype=torch.int32, device="cuda"),
                            mx.ROW32)
    wop = mx.MxOperand(wd, ws, mx.ROW32)
    res = {}
    for side, lens in (("q", [256] * MODULE_B), ("kv", [int(v) for v in synth.lengths(MODULE_SEED, MODULE_B, 256, 2048)])):
        cu = synth.cu_seqlens(lens)
        T = int(cu[-1])
        cu_d = torch.from_numpy(cu).cuda()
        x_host = synth.normal_bf16(MODULE_SEED, synth.STREAM_ACT, (T, C))
        x_dev = torch.from_numpy(x_host.view(np.int16)).view(torch.bfloat16).cuda()
        xd, xs, _ = mx.quantize(x_dev, cu, cu_d, mx.SQ32)
        xop = mx.MxOperand(xd, xs, mx.SQ32)
        nb = xs.shape[0]
        d = torch.empty((T, C), dtype=torch.uint8, device="cuda")
        sc = torch.empty((nb, C // 32), dtype=torch.uint8, device="cuda")
        sct = torch.empty((C // 32, nb), dtype=torch.uint8, device="cuda")

        def call():
            mx.mxfa_linear_quantize(xop, wop, T, C, C, cu_d, len(lens), max(lens), d, sc, sct, stream)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        # the calls back to back between one pair of events: per-call event pairs would add their own
        # gaps to a kernel of a few tens of microseconds
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / args.steps
        flops = 2.0 * T * C * C
        res[side] = {"T": T, "us": round(t * 1e6, 2), "pflops": round(flops / t / 1e15, 4),
                     "frac_peak": round(flops / t / PEAK_MXFP8, 4)}
        print(f"# projection {side}: T={T} {t * 1e6:.1f} us, {flops / t / 1e15:.3f} PF/s", file=sys.stderr, flush=True)
    kv = res["kv"]
    out = {
        "metric": "MXFP8 projection GEMM+quantize PF/s and % of MI355X dense MXFP8 MFMA peak",
        "value": kv["pflops"], "unit": "PF/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(kv["us"] / 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "cross-attention module projection producers, model dim 1024 -> 1024",
                   "kv_side": res["kv"], "q_side": res["q"]},
        "roofline": {"bound": "mfma", "achieved": round(kv["pflops"] * 1e3, 2), "peak": PEAK_MXFP8 / 1e12,
                     "unit": "TFLOP/s", "frac": kv["frac_peak"], "traffic": None,
                     "kernel": "linear_quantize_kernel", "launch_us": kv["us"]},
    }
    print(json.dumps(out), flush=True)


def _time_back_to_back(torch, stream, call, warmup, steps):
    """Mean time of one call over `steps` calls issued back to back between one pair of HIP events on the
    launch stream (per-call event pairs would add their own gaps to kernels of a few microseconds)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def bench_producers(args, torch, mx, synth):
    """HBM-bound producers of the path, each against the 8 TB/s HBM peak:
    * fused RMSNorm + SQ32 quantize with both scale layouts at the cross-attention module's shapes
      (model dim 1024; query side 64 x 256 tokens, key/value side 64 jagged lengths uniform in
      [256, 2048]); algorithmic bytes per element: 2 read (bf16) + 1 written (E4M3) + 2/1024 (the scale
      grid twice), plus gamma;
    * the jagged scale scatter at the 32-sequence self-attention shapes (lengths uniform in [128, 4096],
      16 heads x 128 = 2048 columns) for the ROW32, COL32 and SQ32 scale layouts; algorithmic bytes:
      the compact scale bytes read plus the padded scale bytes written.
    value = the key/value-side RMSNorm+quantize GB/s."""
    stream = torch.cuda.current_stream()
    C = MODULE_DIM
    gamma = torch.ones(C, dtype=torch.float32, device="cuda")
    res = {}
    for side, lens in (("q", [256] * MODULE_B), ("kv", [int(v) for v in synth.lengths(MODULE_SEED, MODULE_B, 256, 2048)])):
        cu = synth.cu_seqlens(lens)
        T = int(cu[-1])
        cu_d = torch.from_numpy(cu).cuda()
        x_host = synth.normal_bf16(MODULE_SEED, synth.STREAM_ACT, (T, C))
        x = torch.from_numpy(x_host.view(np.int16)).view(torch.bfloat16).cuda()
        nb = sum((L + 31) // 32 for L in lens)
        d = torch.empty((T, C), dtype=torch.uint8, device="cuda")
        sc = torch.empty((nb, C // 32), dtype=torch.uint8, device="cuda")
        sct = torch.empty((C // 32, nb), dtype=torch.uint8, device="cuda")

        def call():
            mx.mxfa_rmsnorm_quantize(x, C, T, C, gamma, 1e-6, cu_d, len(lens), max(lens), d, sc, sct, stream)
        t = _time_back_to_back(torch, stream, call, args.warmup, args.steps)
        nbytes = T * C * 3 + 2 * nb * (C // 32) + 4 * C
        res["rmsnorm_quantize_" + side] = {"T": T, "us": round(t * 1e6, 2), "gbps": round(nbytes / t / 1e9, 1),
                                           "frac_hbm": round(nbytes / t / PEAK_HBM, 4)}
        print(f"# rmsnorm_quantize {side}: T={T} {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s", file=sys.stderr,
              flush=True)
    lens = [int(v) for v in synth.lengths(4, 32, 128, 4096)]
    cu = synth.cu_seqlens(lens)
    cu_d = torch.from_numpy(cu).cuda()
    T, Cj = int(cu[-1]), 16 * D
    nb = sum((L + 31) // 32 for L in lens)
    padded = sum((L + 127) // 128 * 128 for L in lens)
    for name, mode, rows, prow, width in (("row32", mx.ROW32, T, padded, Cj // 32),
                                          ("col32", mx.COL32, nb, padded // 32, Cj),
                                          ("sq32", mx.SQ32, nb, padded // 32, Cj // 32)):
        compact = torch.randint(0, 255, (rows, width), dtype=torch.uint8, device="cuda")
        out = torch.empty((prow, width), dtype=torch.uint8, device="cuda")

        def call():
            mx.mxfa_varlen_scale_scatter(compact, cu_d, len(lens), max(lens), Cj, mode, out, prow, stream)
        t = _time_back_to_back(torch, stream, call, args.warmup, args.steps)
        nbytes = rows * width + prow * width
        res["scale_scatter_" + name] = {"bytes": nbytes, "us": round(t * 1e6, 2), "gbps": round(nbytes / t / 1e9, 1),
                                        "frac_hbm": round(nbytes / t / PEAK_HBM, 4)}
        print(f"# scale_scatter {name}: {nbytes} B {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s", file=sys.stderr,
              flush=True)
    kv = res["rmsnorm_quantize_kv"]
    out = {
        "metric": "MXFP8 fused RMSNorm+quantize producer GB/s and % of MI355X HBM peak",
        "value": kv["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(kv["us"] / 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 -> mxfp8_e4m3", "data": "synthetic",
        "config": {"workload": "cross-attention module RMSNorm+quantize (model dim 1024) and jagged scale scatter "
                               "(32 sequences, 16 heads)", **res},
        "roofline": {"bound": "hbm", "achieved": kv["gbps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": kv["frac_hbm"], "traffic": None, "kernel": "rmsnorm_quantize_kernel",
                     "launch_us": kv["us"]},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); each GPU's shard of a larger "
              "job is this single-GPU workload at its real shape", file=sys.stderr)
        sys.exit(2)
    import torch
    import precision_mxfp8_block_amd as mx
    import synth

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("# copy calibration: 536870912 bytes read and written by one copy kernel", file=sys.stderr, flush=True)
        del src, dst
    if args.projection:
        bench_projection(args, torch, mx, synth)
        return
    if args.producers:
        bench_producers(args, torch, mx, synth)
        return
    host, dev, cu, cu_d = make_inputs(torch, synth)
    T, C = B * N, H * D
    c = float(np.float32(1 / math.sqrt(D)))
    stream = torch.cuda.current_stream()
    nb = T // 32

    # outputs and workspace allocated once (the library never allocates)
    def u8(*shape):
        return torch.empty(shape, dtype=torch.uint8, device="cuda")
    qd, kd, vd_, vrd, dod = u8(T, C), u8(T, C), u8(T, C), u8(T, C), u8(T, C)
    qs, ks, dos = u8(nb, C // 32), u8(nb, C // 32), u8(nb, C // 32)
    vs, vrs = u8(nb, C), u8(T, C // 32)
    o = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    dq = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    attn = mx.AttnArgs(mx.MxOperand(qd, qs, mx.SQ32), mx.MxOperand(kd, ks, mx.SQ32), mx.MxOperand(vd_, vs, mx.COL32),
                       cu_d, cu_d, B, N, N, T, T, H, D, c, False)
    vop, doop = mx.MxOperand(vrd, vrs, mx.ROW32), mx.MxOperand(dod, dos, mx.SQ32)
    ws_bytes = mx.mxfa_bwd_workspace_size(attn, args.dq_mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    names = ("quant", "fwd", "bwd")
    ev = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)] for n in names}

    def step(i):
        record = i is not None
        if record:
            ev["quant"][i][0].record(stream)
        mx.mxfa_quantize(dev["q"], C, T, C, cu_d, B, N, mx.SQ32, qd, qs, None, stream)
        mx.mxfa_quantize(dev["k"], C, T, C, cu_d, B, N, mx.SQ32, kd, ks, None, stream)
        mx.mxfa_quantize(dev["v"], C, T, C, cu_d, B, N, mx.COL32, vd_, vs, None, stream)
        mx.mxfa_quantize(dev["v"], C, T, C, cu_d, B, N, mx.ROW32, vrd, vrs, None, stream)
        mx.mxfa_quantize(dev["do"], C, T, C, cu_d, B, N, mx.SQ32, dod, dos, None, stream)
        if record:
            ev["quant"][i][1].record(stream)
            ev["fwd"][i][0].record(stream)
        mx.mxfa_fwd(attn, o, lse, stream)
        if record:
            ev["fwd"][i][1].record(stream)
            ev["bwd"][i][0].record(stream)
        mx.mxfa_bwd(attn, vop, doop, o, dev["do"], lse, args.dq_mode, 1.0, ws, ws_bytes, dq, dk, dv, stream)
        if record:
            ev["bwd"][i][1].record(stream)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"# timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    # the backward once more with FP32 dQ, timed on the same stream
    ws32, ws32_bytes = ws, ws_bytes  # the workspace layout does not depend on the dQ mode
    n32 = 5
    e32 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n32)]
    for i in range(n32 + 1):
        if i:
            e32[i - 1][0].record(stream)
        mx.mxfa_bwd(attn, vop, doop, o, dev["do"], lse, 0, 1.0, ws32, ws32_bytes, dq, dk, dv, stream)
        if i:
            e32[i - 1][1].record(stream)
    torch.cuda.synchronize()
    bwd32_s = float(np.median([e[0].elapsed_time(e[1]) * 1e-3 for e in e32]))

    # the forward once more with the dynamic per-block P scale (same inputs and stream), for the
    # comparison of the two P scales
    edyn = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n32)]
    o_dyn = torch.empty_like(o)
    lse_dyn = torch.empty_like(lse)
    for i in range(n32 + 1):
        if i:
            edyn[i - 1][0].record(stream)
        mx.mxfa_fwd_p_scale(attn, mx.P_BLOCK_DYNAMIC, o_dyn, lse_dyn, stream)
        if i:
            edyn[i - 1][1].record(stream)
    torch.cuda.synchronize()
    fwd_dyn_s = float(np.median([e[0].elapsed_time(e[1]) * 1e-3 for e in edyn]))

    # the forward writing O as MXFP8 only (ROW32 blocks along D, for the next projection)
    emx = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n32)]
    o_mxd = torch.empty((T, C), dtype=torch.uint8, device=o.device)
    o_mxs = torch.empty((T, C // 32), dtype=torch.uint8, device=o.device)
    for i in range(n32 + 1):
        if i:
            emx[i - 1][0].record(stream)
        mx.mxfa_fwd_mx_out(attn, mx.P_STATIC, None, o_mxd, o_mxs, lse_dyn, stream)
        if i:
            emx[i - 1][1].record(stream)
    torch.cuda.synchronize()
    fwd_mx_s = float(np.median([e[0].elapsed_time(e[1]) * 1e-3 for e in emx]))

    # the backward writing the gradients as MXFP8 only (SQ32 blocks, compact codes), FP16 dQ as in the step
    nb = T // 32
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=o.device)
    gmx = (u8(T, C), u8(nb, C // 32), u8(T, C), u8(nb, C // 32), u8(T, C), u8(nb, C // 32))
    ebm = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n32)]
    for i in range(n32 + 1):
        if i:
            ebm[i - 1][0].record(stream)
        mx.mxfa_bwd_mx_out(attn, vop, doop, o, dev["do"], lse, args.dq_mode, 1.0, ws, ws_bytes, None, None, None, gmx,
                           stream)
        if i:
            ebm[i - 1][1].record(stream)
    torch.cuda.synchronize()
    bwd_mx_s = float(np.median([e[0].elapsed_time(e[1]) * 1e-3 for e in ebm]))

    times = {n: [e[0].elapsed_time(e[1]) * 1e-3 for e in ev[n]] for n in names}
    med = {n: float(np.median(v)) for n, v in times.items()}
    f_fwd = 4.0 * N * N * D * B * H
    f_bwd = 2.5 * f_fwd
    step_s = wall / args.steps
    value = (f_fwd + f_bwd) / step_s / 1e15
    quant_bytes = 5 * T * C * (2 + 1) + 3 * T * C / 1024 + T * C / 32 * 2  # bf16 in, e4m3 out, scales
    fwd_pf, bwd_pf = f_fwd / med["fwd"] / 1e15, f_bwd / med["bwd"] / 1e15
    dominant = "bwd" if med["bwd"] >= med["fwd"] else "fwd"
    flops_dom = f_bwd if dominant == "bwd" else f_fwd
    roof = {"bound": "mfma", "achieved": flops_dom / med[dominant] / 1e12, "peak": PEAK_MXFP8 / 1e12,
            "unit": "TFLOP/s", "frac": flops_dom / med[dominant] / PEAK_MXFP8,
            "traffic": measured_traffic() if dominant == "bwd" else None,
            "kernel": "mxfa_bwd call: bwd_preprocess_kernel + attn_bwd_kernel + attn_dq_kernel"
            if dominant == "bwd" else "attn_fwd_kernel",
            "launch_us": round(med[dominant] * 1e6, 2)}
    out = {
        "metric": "MXFP8 attention fwd/bwd PF/s and % of MI355X dense MXFP8 MFMA peak",
        "value": round(value, 4), "unit": "PF/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "MXFP8 attention training step (quantize + fwd + bwd), non-causal",
                   "B": B, "H": H, "N": N, "D": D, "dq_mode": "fp16_static" if args.dq_mode else "fp32",
                   "dq_static_scale": 1.0},
        "fwd_pflops": round(fwd_pf, 4), "fwd_frac_peak": round(fwd_pf * 1e15 / PEAK_MXFP8, 4),
        "bwd_pflops": round(bwd_pf, 4), "bwd_frac_peak": round(bwd_pf * 1e15 / PEAK_MXFP8, 4),
        "fwd_us": round(med["fwd"] * 1e6, 2), "bwd_us": round(med["bwd"] * 1e6, 2),
        "bwd_fp32dq_us": round(bwd32_s * 1e6, 2), "bwd_fp32dq_pflops": round(f_bwd / bwd32_s / 1e15, 4),
        "fwd_dynamic_p_us": round(fwd_dyn_s * 1e6, 2), "fwd_dynamic_p_pflops": round(f_fwd / fwd_dyn_s / 1e15, 4),
        "fwd_mx_out_us": round(fwd_mx_s * 1e6, 2), "fwd_mx_out_pflops": round(f_fwd / fwd_mx_s / 1e15, 4),
        "bwd_mx_out_us": round(bwd_mx_s * 1e6, 2), "bwd_mx_out_pflops": round(f_bwd / bwd_mx_s / 1e15, 4),
        "quant_us": round(med["quant"] * 1e6, 2),
        "quant_gbps": round(quant_bytes / med["quant"] / 1e9, 1),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(host, cu)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

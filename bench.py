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

The headline step is timed first, on a GPU that has run nothing else in the process; then one JSON
line per further workload (the headline line is printed last), each with its own
roofline entry and oracle sample (--headline-only skips them): causal B=4 H=16 N=8192 with 0.5% x64
outliers (fwd + bwd, FP16 dQ at sigma 2^-4 and FP32 dQ); the jagged batch of 32 sequences with lengths
uniform in [128, 4096] beside a uniform batch of the same total tokens; the forward-only LLM shape
(Q/K ROW32, V COL32) and the same forward with Q and K in MXFP4 (E2M1) and MXFP6 (E2M3); the cross-attention module
step (producers, scatter, attention fwd + bwd).
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
PEAK_MXFP4 = 10.1e15  # FLOP/s, dense FP4 and FP6 scaled MFMA
# forward with Q/K in MXFP4 or MXFP6: S = Q K^T (half the FLOPs) at the FP4/FP6 rate, O = P V at the FP8 rate
PEAK_FWD_QK4 = 1.0 / (0.5 / PEAK_MXFP4 + 0.5 / PEAK_MXFP8)
PEAK_HBM = 8.0e12     # B/s
synth_mod = None  # the synth module, set in main()
B, H, N, D = 4, 16, 4096, 128
SEED = 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--dq-mode", type=int, default=1, help="0 = FP32 dQ, 1 = FP16 static-scale dQ")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the per-workload lines (causal outliers, jagged vs uniform, module, forward-only) "
                         "printed before the headline line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy first (reference kernel for HBM byte counters)")
    ap.add_argument("--producers", action="store_true",
                    help="time the fused RMSNorm+quantize producer at the module workload's shapes and the jagged "
                         "scale scatter instead of the attention step (one JSON line of its own)")
    ap.add_argument("--forward-only", action="store_true",
                    help="only the forward-only LLM shape, with Q/K in MXFP8, MXFP4 and MXFP6 (three JSON lines)")
    ap.add_argument("--module", action="store_true",
                    help="time only the cross-attention module training step (the config-5 shape, then module "
                         "latency at 4k, 8k and 16k key/value tokens), one JSON line each")
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
    model, nproc, _ = host_cpu()
    return {"value": flops / dt / 1e15, "unit": "PF/s", "cores": min(nthreads, hs), "kind": "oracle",
            "cpu_model": model, "nproc": nproc,
            "sample": f"batch element 0 of the step, heads 0-{hs - 1} of {H} (N={N}): quantize + forward + "
                      f"backward (FP32 dQ), one thread per head, {dt:.1f} s wall"}


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


def host_cpu():
    """CPU model and the number of cores the oracle may use here (the box's share, at most 16)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count() or 1, max(1, min(16, os.cpu_count() or 1))


def oracle_slices(slices, backward, c, causal, qk_mode=2, qk_small=None):
    """The oracle, as it is, on (sequence, head) slices given as bf16 arrays {q, k, v, do}: each slice one
    sequence of a one-head batch, so the slices run on parallel threads. Returns wall seconds."""
    import oracle
    cq = synth_mod.cu_seqlens([x["q"].shape[0] for x in slices])
    ck = synth_mod.cu_seqlens([x["k"].shape[0] for x in slices])
    cat = {n: np.ascontiguousarray(np.concatenate([x[n] for x in slices])) for n in ("q", "k", "v", "do")}
    nthreads = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    if qk_small:  # forward with Q and K in MXFP4 ("e2m1") or MXFP6 ("e2m3")
        from oracle import mxfp4, mxfp6
        mod, fwd = (mxfp4, mxfp4.attn_fwd_qk_fp4) if qk_small == "e2m1" else (mxfp6, mxfp6.attn_fwd_qk_fp6)
        q4, k4 = mod.quantize_row32(cat["q"]), mod.quantize_row32(cat["k"])
        v = oracle.quantize(cat["v"], ck, oracle.COL32)
        fwd(q4[0], q4[1], k4[0], k4[1], v[0], v[1], cq, ck, 1, D, c, causal)
        return time.perf_counter() - t0, min(nthreads, len(slices))
    q = oracle.quantize(cat["q"], cq, qk_mode)
    k = oracle.quantize(cat["k"], ck, qk_mode)
    v = oracle.quantize(cat["v"], ck, oracle.COL32)
    o16, _, lse = oracle.attn_fwd_mx(q[0], q[1], qk_mode, k[0], k[1], qk_mode, v[0], v[1], oracle.COL32, cq, ck, 1, D,
                                     c, causal, nthreads=nthreads)
    if backward:
        vd = oracle.quantize(cat["v"], ck, oracle.ROW32)
        do = oracle.quantize(cat["do"], cq, oracle.SQ32)
        oracle.attn_bwd_mx(q[0], q[1], k[0], k[1], vd[0], vd[1], oracle.ROW32, do[0], do[1], o16, cat["do"], lse, cq,
                           ck, 1, D, c, causal, 0, 1.0, nthreads=nthreads)
    return time.perf_counter() - t0, min(nthreads, len(slices))


def attn_flops(lens_q, lens_k, H, causal):
    """Forward FLOPs (4 D per visible (query, key) pair; top-left causal: the pairs j <= i)."""
    pairs = 0
    for lq, lk in zip(lens_q, lens_k):
        pairs += (min(lq, lk) * (min(lq, lk) + 1) // 2 + max(0, lq - lk) * lk) if causal else lq * lk
    return 4.0 * D * H * pairs


def bench_attention_workload(args, torch, mx, label, workload, lens_q, lens_k, H, causal, outlier_p, seed,
                             fwd_only=False, qk_mode=None, dq_modes=((1, 1.0), (0, 1.0)), cpu_slices=4,
                             cpu_backward=False, extra_config=None, qk_small=None, keep_fwd=None, cpu_repeats=1):
    """One attention workload at its full size: quantize, forward and backward (each dQ mode) timed over
    back-to-back calls with HIP events on the launch stream. Returns the JSON dict (not printed); with
    keep_fwd (a list) the forward call on the quantized operands is appended to it."""
    stream = torch.cuda.current_stream()
    qk_mode = (mx.ROW32 if fwd_only else mx.SQ32) if qk_mode is None else qk_mode
    cu_q, cu_k = synth_mod.cu_seqlens(lens_q), synth_mod.cu_seqlens(lens_k)
    Tq, Tk, C = int(cu_q[-1]), int(cu_k[-1]), H * D
    kw = dict(outlier_p=outlier_p)
    host = {"q": synth_mod.normal_bf16(seed, synth_mod.STREAM_Q, (Tq, C), **kw),
            "k": synth_mod.normal_bf16(seed, synth_mod.STREAM_K, (Tk, C), **kw),
            "v": synth_mod.normal_bf16(seed, synth_mod.STREAM_V, (Tk, C), **kw),
            "do": synth_mod.normal_bf16(seed, synth_mod.STREAM_DO, (Tq, C), **kw)}
    dev = {n: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for n, a in host.items()}
    cq_d, ck_d = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    c = float(np.float32(1 / math.sqrt(D)))
    nbq, nbk = int(np.sum((np.array(lens_q) + 31) // 32)), int(np.sum((np.array(lens_k) + 31) // 32))
    Pq, Pk = mx.mxfa_padded_token_rows(cu_q), mx.mxfa_padded_token_rows(cu_k)
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device="cuda")
    srows = {mx.ROW32: (lambda T, nb, P: (T, C // 32), lambda T, nb, P: (P, C // 32)),
             mx.COL32: (lambda T, nb, P: (nb, C), lambda T, nb, P: (P // 32, C)),
             mx.SQ32: (lambda T, nb, P: (nb, C // 32), lambda T, nb, P: (P // 32, C // 32))}
    jag_q, jag_k = any(L % 128 for L in lens_q), any(L % 128 for L in lens_k)

    def operand(name, mode, T, nb, P, cu_d, lens, jag):
        d, sc = u8(T, C), u8(*srows[mode][0](T, nb, P))
        pad = u8(*srows[mode][1](T, nb, P)) if jag else sc

        def run():
            mx.mxfa_quantize(dev[name], C, T, C, cu_d, len(lens), max(lens), mode, d, sc, None, stream)
            if jag:
                mx.mxfa_varlen_scale_scatter(sc, cu_d, len(lens), max(lens), C, mode, pad, pad.shape[0], stream)
        return mx.MxOperand(d, pad, mode), run
    def operand_small(name, T, P, cu_d, lens, jag):
        # MXFP4 (16 B per 32 elements) or MXFP6 (24 B), ROW32 scales
        nbytes, quant, elem = {"e2m1": (16, mx.mxfa_quantize_e2m1, mx.E2M1),
                               "e2m3": (24, mx.mxfa_quantize_e2m3, mx.E2M3)}[qk_small]
        d, sc = u8(T, C // 32 * nbytes), u8(T, C // 32)
        pad = u8(P, C // 32) if jag else sc

        def run():
            quant(dev[name], C, T, C, d, sc, stream)
            if jag:
                mx.mxfa_varlen_scale_scatter(sc, cu_d, len(lens), max(lens), C, mx.ROW32, pad, pad.shape[0], stream)
        return mx.MxOperand(d, pad, mx.ROW32, elem), run
    if qk_small:
        assert fwd_only and qk_mode == mx.ROW32
        qop, rq = operand_small("q", Tq, Pq, cq_d, lens_q, jag_q)
        kop, rk = operand_small("k", Tk, Pk, ck_d, lens_k, jag_k)
    else:
        qop, rq = operand("q", qk_mode, Tq, nbq, Pq, cq_d, lens_q, jag_q)
        kop, rk = operand("k", qk_mode, Tk, nbk, Pk, ck_d, lens_k, jag_k)
    def operand_v_both(T, nb, P, cu_d, lens, jag):
        # V's COL32 payload (the forward's P V) and ROW32 payload (the backward's dP = dO V^T), one read
        dcol, scol = u8(T, C), u8(*srows[mx.COL32][0](T, nb, P))
        drow, srow = u8(T, C), u8(*srows[mx.ROW32][0](T, nb, P))
        pcol = u8(*srows[mx.COL32][1](T, nb, P)) if jag else scol
        prow = u8(*srows[mx.ROW32][1](T, nb, P)) if jag else srow

        def run():
            mx.mxfa_quantize_col32_row32(dev["v"], C, T, C, cu_d, len(lens), max(lens), dcol, scol, drow, srow, stream)
            if jag:
                mx.mxfa_varlen_scale_scatter(scol, cu_d, len(lens), max(lens), C, mx.COL32, pcol, pcol.shape[0], stream)
                mx.mxfa_varlen_scale_scatter(srow, cu_d, len(lens), max(lens), C, mx.ROW32, prow, prow.shape[0], stream)
        return mx.MxOperand(dcol, pcol, mx.COL32), mx.MxOperand(drow, prow, mx.ROW32), run
    if fwd_only:
        vop, rv = operand("v", mx.COL32, Tk, nbk, Pk, ck_d, lens_k, jag_k)
        runs = [rq, rk, rv]
    else:
        vop, vdop, rv = operand_v_both(Tk, nbk, Pk, ck_d, lens_k, jag_k)
        doop, rdo = operand("do", mx.SQ32, Tq, nbq, Pq, cq_d, lens_q, jag_q)
        runs = [rq, rk, rv, rdo]

    def quant():
        for r in runs:
            r()
    attn = mx.AttnArgs(qop, kop, vop, cq_d, ck_d, len(lens_q), max(lens_q), max(lens_k), Tq, Tk, H, D, c, causal)
    o = torch.empty((Tq, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, Tq), dtype=torch.float32, device="cuda")
    quant()
    t_quant = _time_back_to_back(torch, stream, quant, 2, max(3, args.steps // 4))
    t_fwd = _time_back_to_back(torch, stream, lambda: mx.mxfa_fwd(attn, o, lse, stream), 2, args.steps)
    if keep_fwd is not None:
        keep_fwd.append(lambda: mx.mxfa_fwd(attn, o, lse, stream))
    f_fwd = attn_flops(lens_q, lens_k, H, causal)
    res = {"fwd_us": round(t_fwd * 1e6, 2), "fwd_pflops": round(f_fwd / t_fwd / 1e15, 4),
           "quant_us": round(t_quant * 1e6, 2)}
    dom_t, dom_f, dom_name = t_fwd, f_fwd, "attn_fwd_kernel"
    if not fwd_only:
        ws_bytes = mx.mxfa_bwd_workspace_size(attn, 1)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        dq, dk, dv = (torch.empty((T, C), dtype=torch.bfloat16, device="cuda") for T in (Tq, Tk, Tk))
        for dq_mode, sigma in dq_modes:
            t = _time_back_to_back(torch, stream, lambda: mx.mxfa_bwd(attn, vdop, doop, o, dev["do"], lse, dq_mode, sigma,
                                                                     ws, ws_bytes, dq, dk, dv, stream), 2, args.steps)
            key = "bwd_fp16dq" if dq_mode == 1 else "bwd_fp32dq"
            res[key + "_us"] = round(t * 1e6, 2)
            res[key + "_pflops"] = round(2.5 * f_fwd / t / 1e15, 4)
            res[key + "_sigma"] = sigma
        t_bwd = res["bwd_fp16dq_us"] * 1e-6
        dom_t, dom_f, dom_name = (t_bwd, 2.5 * f_fwd, "mxfa_bwd call (FP16 dQ)") if t_bwd > t_fwd else (dom_t, dom_f,
                                                                                                       dom_name)
        res["step_us"] = round((t_quant + t_fwd + t_bwd) * 1e6, 2)
        value = 3.5 * f_fwd / (t_fwd + t_bwd) / 1e15
    else:
        value = f_fwd / t_fwd / 1e15
    print(f"# {label}: " + ", ".join(f"{k}={v}" for k, v in res.items()), file=sys.stderr, flush=True)
    cfg = {"workload": workload, "H": H, "D": D, "causal": bool(causal), "nseq": len(lens_q), "tokens_q": Tq,
           "tokens_k": Tk, "max_len": max(lens_k), "outlier_p": outlier_p, **(extra_config or {}), **res}
    peak = PEAK_FWD_QK4 if qk_small else PEAK_MXFP8
    small = {"e2m1": ("MXFP4", "FP4", "mxfp4_e2m1"), "e2m3": ("MXFP6", "FP6", "mxfp6_e2m3")}.get(qk_small)
    out = {
        "metric": (f"{small[0]}-QK attention forward PF/s and % of the MI355X dense MFMA peak of its mix (S in "
                   f"{small[1]}, P V in FP8)") if small else
                  "MXFP8 attention fwd/bwd PF/s and % of MI355X dense MXFP8 MFMA peak",
        "value": round(value, 4), "unit": "PF/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((res.get("step_us", res["fwd_us"])) / 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"{small[2]} Q/K, mxfp8_e4m3 V/P (fp32 accumulate)" if small else "mxfp8_e4m3 (fp32 accumulate)",
        "data": "synthetic", "config": cfg,
        "roofline": {"bound": "mfma", "achieved": round(dom_f / dom_t / 1e12, 2), "peak": round(peak / 1e12, 1),
                     "unit": "TFLOP/s", "frac": round(dom_f / dom_t / peak, 4), "traffic": None,
                     "kernel": dom_name, "launch_us": round(dom_t * 1e6, 2)},
    }
    if not args.no_cpu_baseline and cpu_slices:
        picks = [(s, (7 * s + 3) % H) for s in np.argsort(lens_k)[::-1][:cpu_slices]]
        sl = [{n: np.ascontiguousarray(host[n][int((cu_q if n in ("q", "do") else cu_k)[s]):
                                               int((cu_q if n in ("q", "do") else cu_k)[s + 1]), h * D:(h + 1) * D])
               for n in ("q", "k", "v", "do")} for s, h in picks]
        runs = [oracle_slices(sl, cpu_backward, c, causal, qk_mode, qk_small) for _ in range(cpu_repeats)]
        dt, cores = float(np.median([r[0] for r in runs])), runs[0][1]
        f = sum(attn_flops([lens_q[s]], [lens_k[s]], 1, causal) for s, _ in picks) * (3.5 if cpu_backward else 1.0)
        model, nproc, _ = host_cpu()
        out["cpu_baseline"] = {"value": round(f / dt / 1e15, 8), "unit": "PF/s", "cores": cores, "kind": "oracle",
                               "cpu_model": model, "nproc": nproc,
                               "sample": f"{len(picks)} (sequence, head) slices of the longest sequences, quantize + "
                                         f"forward{' + backward' if cpu_backward else ''}, one thread per slice, "
                                         f"{dt:.3g} s wall" + (f" (median of {cpu_repeats} runs)" if cpu_repeats > 1
                                                               else "")}
    del dev
    torch.cuda.empty_cache()
    return out


def bench_workloads(args, torch, mx):
    """The per-workload lines: the tiny B=1 H=1 N=256 case, causal N=8192 with outliers, jagged 32 sequences beside a uniform batch of
    the same total tokens, and the forward-only LLM shape (Q/K ROW32)."""
    lines = []
    # the small case: the whole problem on the oracle (one (sequence, head) slice, so one thread), median of 5
    lines.append(bench_attention_workload(
        args, torch, mx, "tiny", "tiny B=1 H=1 N=256, fwd + bwd", [256], [256], 1, False, 0.0, 1, cpu_slices=1,
        cpu_backward=True, cpu_repeats=5))
    lines.append(bench_attention_workload(
        args, torch, mx, "causal outliers", "causal B=4 H=16 N=8192, 0.5% of entries x64, fwd + bwd",
        [8192] * 4, [8192] * 4, 16, True, 0.005, 3, dq_modes=((1, 0.0625), (0, 1.0)), cpu_slices=4))
    lens = [int(v) for v in synth_mod.lengths(4, 32, 128, 4096)]
    jag = bench_attention_workload(
        args, torch, mx, "jagged", "jagged self-attention, 32 sequences with lengths uniform in [128, 4096], fwd + bwd",
        lens, lens, 16, False, 0.0, 4, cpu_slices=4)
    L = int(round(sum(lens) / len(lens) / 128.0)) * 128
    uni = bench_attention_workload(
        args, torch, mx, "uniform", f"uniform self-attention, 32 sequences of {L} tokens, fwd + bwd",
        [L] * 32, [L] * 32, 16, False, 0.0, 4, cpu_slices=0)
    jag["config"]["uniform_same_batch"] = {k: uni["config"][k] for k in uni["config"] if k.endswith(("us", "pflops"))}
    jag["config"]["uniform_same_batch"]["len"] = L
    lines.append(jag)
    lines += bench_forward_only(args, torch, mx)
    for line in lines:
        print(json.dumps(line), flush=True)


def _time_round_robin(torch, stream, calls, warmup, rounds):
    """Median time of each call when the calls take turns (each launch between its own pair of HIP
    events), so that a clock that drifts over the run weighs on all of them alike."""
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ts = [[] for _ in calls]
    for _ in range(rounds):
        for i, c in enumerate(calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            c()
            e1.record(stream)
            torch.cuda.synchronize()
            ts[i].append(e0.elapsed_time(e1) * 1e-3)
    return [float(np.median(t)) for t in ts]


def bench_forward_only(args, torch, mx):
    """The forward-only LLM shape with Q/K in MXFP8 and, on the same inputs, in MXFP4 and MXFP6. Each line
    times its own forward back to back; the three forwards are then also timed taking turns
    (`fwd_us_interleaved`), which compares them at the same clock."""
    lines, fwds = [], []
    fo = bench_attention_workload(
        args, torch, mx, "forward-only", "LLM forward B=4 H=16 N=4096, Q/K ROW32, V COL32",
        [N] * B, [N] * B, H, False, 0.0, SEED, fwd_only=True, cpu_slices=4, keep_fwd=fwds)
    lines.append(fo)
    f4 = bench_attention_workload(
        args, torch, mx, "forward-only MXFP4 Q/K", "LLM forward B=4 H=16 N=4096, Q/K MXFP4 (E2M1) ROW32, V E4M3 COL32",
        [N] * B, [N] * B, H, False, 0.0, SEED, fwd_only=True, cpu_slices=2, qk_small="e2m1", keep_fwd=fwds)
    f6 = bench_attention_workload(
        args, torch, mx, "forward-only MXFP6 Q/K", "LLM forward B=4 H=16 N=4096, Q/K MXFP6 (E2M3) ROW32, V E4M3 COL32",
        [N] * B, [N] * B, H, False, 0.0, SEED, fwd_only=True, cpu_slices=2, qk_small="e2m3", keep_fwd=fwds)
    rr = _time_round_robin(torch, torch.cuda.current_stream(), fwds, 3, max(10, args.steps))
    inter = {"mxfp8": round(rr[0] * 1e6, 2), "mxfp4": round(rr[1] * 1e6, 2), "mxfp6": round(rr[2] * 1e6, 2)}
    print("# forward-only, the three taking turns: " + ", ".join(f"{k}={v} us" for k, v in inter.items()),
          file=sys.stderr, flush=True)
    fo["config"]["fwd_us_interleaved"] = inter
    for f in (f4, f6):
        f["config"]["mxfp8_qk_same_shape"] = {k: fo["config"][k] for k in ("fwd_us", "fwd_pflops", "quant_us")}
        f["config"]["fwd_us_interleaved"] = inter
        lines.append(f)
    fwds.clear()
    torch.cuda.empty_cache()
    return lines


def module_step_setup(torch, mx, lens_k, seed, NQ=256, Hm=8, CM=None):
    """Buffers of one cross-attention module training step: query side len(lens_k) samples x NQ tokens,
    key/value side the given jagged lengths, H=Hm heads of 128, model dim CM; bf16 N(0,1) activations,
    N(0, 0.02) weights quantized once (W along C_in for the forward, W^T along C_out for the data
    gradient), dO N(0,1)."""
    CM = CM or MODULE_DIM
    Bm = len(lens_k)
    lens_q = [NQ] * Bm
    cu_q, cu_k = synth_mod.cu_seqlens(lens_q), synth_mod.cu_seqlens(lens_k)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    m = dict(Bm=Bm, NQ=NQ, Hm=Hm, CM=CM, lens_q=lens_q, lens_k=lens_k, cu_q=cu_q, cu_k=cu_k, Tq=Tq, Tk=Tk,
             cq_d=torch.from_numpy(cu_q).cuda(), ck_d=torch.from_numpy(cu_k).cuda())
    m["xq_h"] = synth_mod.normal_bf16(seed, synth_mod.STREAM_ACT, (Tq, CM))
    m["xkv_h"] = synth_mod.normal_bf16(seed, synth_mod.STREAM_ACT + 1, (Tk, CM))
    m["w_h"] = {n: synth_mod.normal_bf16(seed, synth_mod.STREAM_WEIGHT + i, (CM, CM), std=0.02) for i, n in enumerate("qkv")}
    C = Hm * D
    m["do_h"] = synth_mod.normal_bf16(seed, synth_mod.STREAM_DO, (Tq, C))
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    m["xq"], m["xkv"], m["dout"] = bf(m["xq_h"]), bf(m["xkv_h"]), bf(m["do_h"])
    m["gamma"] = torch.ones(CM, dtype=torch.float32, device="cuda")
    wcu, tcu = np.array([0, C], np.int32), np.array([0, CM], np.int32)
    w_hat = {n: mx.quantize(bf(m["w_h"][n]), wcu, torch.from_numpy(wcu).cuda(), mx.ROW32) for n in "qkv"}
    wt_hat = {n: mx.quantize(bf(m["w_h"][n].T), tcu, torch.from_numpy(tcu).cuda(), mx.ROW32) for n in "qkv"}
    m["wop"] = {n: mx.MxOperand(w_hat[n][0], w_hat[n][1], mx.ROW32) for n in "qkv"}
    m["wtop"] = {n: mx.MxOperand(wt_hat[n][0], wt_hat[n][1], mx.ROW32) for n in "qkv"}
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device="cuda")
    bf16 = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    nbq, nbk = int(np.sum((np.array(lens_q) + 31) // 32)), int(np.sum((np.array(lens_k) + 31) // 32))
    Pk = mx.mxfa_padded_token_rows(cu_k)
    sq = lambda T, nb, w: (u8(T, w), u8(nb, w // 32), u8(w // 32, nb))
    m["xqh"], m["xkvh"] = sq(Tq, nbq, CM), sq(Tk, nbk, CM)
    m["gq"], m["gk"], m["gv"] = sq(Tq, nbq, C), sq(Tk, nbk, C), sq(Tk, nbk, C)
    m["pk"], m["pv"] = u8(Pk // 32, C // 32), u8(Pk // 32, C // 32)
    m["gdo"] = (u8(Tq, C), u8(nbq, C // 32))
    c = float(np.float32(1 / math.sqrt(D)))
    m["c"] = c
    m["attn"] = mx.AttnArgs(mx.MxOperand(m["gq"][0], m["gq"][1], mx.SQ32), mx.MxOperand(m["gk"][0], m["pk"], mx.SQ32),
                            mx.MxOperand(m["gv"][0], m["pv"], mx.SQ32), m["cq_d"], m["ck_d"], Bm, NQ, max(lens_k), Tq,
                            Tk, Hm, D, c, False)
    m["o"], m["lse"] = bf16(Tq, C), f32(Hm, Tq)
    m["ws_bytes"] = mx.mxfa_bwd_workspace_size(m["attn"], 1)
    m["ws"] = u8(m["ws_bytes"])
    m["qdq"], m["qdk"], m["qdv"] = sq(Tq, nbq, C), sq(Tk, nbk, C), sq(Tk, nbk, C)
    m["dxq"], m["dxkv"] = bf16(Tq, CM), bf16(Tk, CM)
    m["dxq_in"], m["dxkv_in"] = bf16(Tq, CM), bf16(Tk, CM)
    m["dgq"], m["dgkv"] = f32(CM), f32(CM)
    m["dw"] = {n: f32(C, CM) for n in "qkv"}
    m["wg_bytes"] = max(mx.mxfa_linear_bwd_weight_workspace_size(T, Bm, C, CM) for T in (Tq, Tk))
    m["wg_ws"] = u8(m["wg_bytes"])
    m["rb_bytes"] = max(mx.mxfa_rmsnorm_bwd_workspace_size(T, CM) for T in (Tq, Tk))
    m["rb_ws"] = u8(m["rb_bytes"])
    return m


MODULE_PHASES = ["producers", "scatter", "attn_fwd", "attn_bwd", "producer_bwd"]


def module_step(mx, m, stream, ev=None):
    """One training step of the module; ev: 6 events marking the phase boundaries (or None)."""
    def mark(i):
        if ev is not None:
            ev[i].record(stream)
    Bm, NQ, CM, Tq, Tk, C = m["Bm"], m["NQ"], m["CM"], m["Tq"], m["Tk"], m["Hm"] * D
    mk = max(m["lens_k"])
    cq_d, ck_d = m["cq_d"], m["ck_d"]
    SQ = mx.SQ32
    mark(0)
    mx.mxfa_rmsnorm_quantize(m["xq"], CM, Tq, CM, m["gamma"], 1e-6, cq_d, Bm, NQ, *m["xqh"], stream)
    mx.mxfa_rmsnorm_quantize(m["xkv"], CM, Tk, CM, m["gamma"], 1e-6, ck_d, Bm, mk, *m["xkvh"], stream)
    mx.mxfa_linear_quantize(mx.MxOperand(m["xqh"][0], m["xqh"][1], SQ), m["wop"]["q"], Tq, CM, C, cq_d, Bm, NQ,
                            *m["gq"], stream)
    for n in "kv":
        mx.mxfa_linear_quantize(mx.MxOperand(m["xkvh"][0], m["xkvh"][1], SQ), m["wop"][n], Tk, CM, C, ck_d, Bm, mk,
                                *m["g" + n], stream)
    mark(1)
    mx.mxfa_varlen_scale_scatter(m["gk"][1], ck_d, Bm, mk, C, SQ, m["pk"], m["pk"].shape[0], stream)
    mx.mxfa_varlen_scale_scatter(m["gv"][1], ck_d, Bm, mk, C, SQ, m["pv"], m["pv"].shape[0], stream)
    mark(2)
    mx.mxfa_fwd(m["attn"], m["o"], m["lse"], stream)
    mark(3)
    mx.mxfa_quantize(m["dout"], C, Tq, C, cq_d, Bm, NQ, SQ, m["gdo"][0], m["gdo"][1], None, stream)
    # the gradients leave the attention backward as SQ32 MXFP8 with both code layouts (the producers'
    # format), which the projections' backward consumes directly
    qdq, qdk, qdv = m["qdq"], m["qdk"], m["qdv"]
    mx.mxfa_bwd_mx_out(m["attn"], mx.MxOperand(m["gv"][0], m["pv"], SQ), mx.MxOperand(m["gdo"][0], m["gdo"][1], SQ),
                       m["o"], m["dout"], m["lse"], 1, 1.0, m["ws"], m["ws_bytes"], None, None, None,
                       [qdq[0], qdq[1], qdk[0], qdk[1], qdv[0], qdv[1], qdq[2], qdk[2], qdv[2]], stream)
    mark(4)
    # projection data gradients (the key/value input sums its two), RMSNorm backward, weight gradients
    mx.mxfa_linear_bwd_data(mx.MxOperand(m["qdq"][0], m["qdq"][1], SQ), m["wtop"]["q"], Tq, C, CM, cq_d, Bm, NQ, 0,
                            m["dxq"], stream)
    mx.mxfa_linear_bwd_data(mx.MxOperand(m["qdk"][0], m["qdk"][1], SQ), m["wtop"]["k"], Tk, C, CM, ck_d, Bm, mk, 0,
                            m["dxkv"], stream)
    mx.mxfa_linear_bwd_data(mx.MxOperand(m["qdv"][0], m["qdv"][1], SQ), m["wtop"]["v"], Tk, C, CM, ck_d, Bm, mk, 1,
                            m["dxkv"], stream)
    mx.mxfa_rmsnorm_bwd(m["xq"], CM, Tq, CM, m["gamma"], 1e-6, m["dxq"], m["rb_ws"], m["rb_bytes"], m["dxq_in"],
                        m["dgq"], stream)
    mx.mxfa_rmsnorm_bwd(m["xkv"], CM, Tk, CM, m["gamma"], 1e-6, m["dxkv"], m["rb_ws"], m["rb_bytes"], m["dxkv_in"],
                        m["dgkv"], stream)
    for n, qg, xh, T, cu, ms in (("q", m["qdq"], m["xqh"], Tq, cq_d, NQ), ("k", m["qdk"], m["xkvh"], Tk, ck_d, mk),
                                 ("v", m["qdv"], m["xkvh"], Tk, ck_d, mk)):
        mx.mxfa_linear_bwd_weight(qg[0], qg[2], xh[0], xh[2], T, C, CM, cu, Bm, ms, m["wg_ws"], m["wg_bytes"],
                                  m["dw"][n], stream)
    mark(5)


def module_cpu_baseline(m, picks):
    """The oracle on head 3 of the picked samples: RMSNorm+quantize, the three projections (that head's 128
    columns), attention fwd + bwd, and the projections' data and weight gradients and the RMSNorm
    backward of that head's slice."""
    import oracle
    D_, CM, NQ = D, m["CM"], m["NQ"]
    c = m["c"]
    t0 = time.perf_counter()
    fl = 0.0
    h = 3
    ones = np.ones(CM, np.float32)
    for s in picks:
        Lk = m["lens_k"][s]
        rq = slice(int(m["cu_q"][s]), int(m["cu_q"][s + 1]))
        rk = slice(int(m["cu_k"][s]), int(m["cu_k"][s + 1]))
        cq1, ck1 = np.array([0, NQ], np.int32), np.array([0, Lk], np.int32)
        xq1 = oracle.rmsnorm_quantize(np.ascontiguousarray(m["xq_h"][rq]), ones, 1e-6, cq1)
        xk1 = oracle.rmsnorm_quantize(np.ascontiguousarray(m["xkv_h"][rk]), ones, 1e-6, ck1)
        outs, wts = {}, {}
        for n, x1, cu1 in (("q", xq1, cq1), ("k", xk1, ck1), ("v", xk1, ck1)):
            wslice = np.ascontiguousarray(m["w_h"][n][h * D_:(h + 1) * D_])
            wd, ws1, _ = oracle.quantize(wslice, np.array([0, D_], np.int32), oracle.ROW32)
            wts[n] = oracle.quantize(np.ascontiguousarray(wslice.T), np.array([0, CM], np.int32), oracle.ROW32)
            outs[n] = oracle.linear_quantize(x1[0], x1[1], wd, ws1, cu1)
        o16, _, lse1 = oracle.attn_fwd_mx(outs["q"][0], outs["q"][1], 2, outs["k"][0], outs["k"][1], 2, outs["v"][0],
                                          outs["v"][1], 2, cq1, ck1, 1, D_, c, False)
        do1 = np.ascontiguousarray(m["do_h"][rq, h * D_:(h + 1) * D_])
        rdo = oracle.quantize(do1, cq1, oracle.SQ32)
        g = oracle.attn_bwd_mx(outs["q"][0], outs["q"][1], outs["k"][0], outs["k"][1], outs["v"][0], outs["v"][1], 2,
                               rdo[0], rdo[1], o16, do1, lse1, cq1, ck1, 1, D_, c, False, 1, 1.0)
        for n, gname, x1, cu1, xsrc, rows in (("q", "dq", xq1, cq1, m["xq_h"], rq), ("k", "dk", xk1, ck1, m["xkv_h"], rk),
                                              ("v", "dv", xk1, ck1, m["xkv_h"], rk)):
            gq = oracle.quantize(g[gname], cu1, oracle.SQ32)
            dx, _ = oracle.linear_bwd_data(gq[0], gq[1], wts[n][0], wts[n][1], cu1)
            oracle.rmsnorm_bwd(np.ascontiguousarray(xsrc[rows]), ones, 1e-6, dx)
            oracle.linear_bwd_weight(gq[0], gq[2], x1[0], x1[2], cu1)
        fl += 3.5 * attn_flops([NQ], [Lk], 1, False) + 3 * 2.0 * CM * D_ * (NQ + 2 * Lk)
    return fl, time.perf_counter() - t0


def bench_module(args, torch, mx, lens_k=None, seed=5, label=None, cpu_picks=2):
    """One cross-attention module training step at full size: forward (RMSNorm+quantize of the query- and
    key/value-side activations, the three projection GEMM+quantize producers with SQ32 outputs in both
    scale layouts, the jagged scale scatter of K and V, attention forward), backward (quantize dO,
    attention backward with FP16 dQ writing the gradients as SQ32 MXFP8 with both code layouts, the
    projections' data gradients (W^T along C_out; the key/value input sums its two), the RMSNorm
    backward on both sides, the projections' weight gradients over all tokens through the transposed
    scale grids). The weights are quantized once, outside the step. Step and phases timed with HIP
    events (median over the timed steps)."""
    stream = torch.cuda.current_stream()
    if lens_k is None:
        lens_k = [int(v) for v in synth_mod.lengths(5, MODULE_B, 256, 2048)]
    m = module_step_setup(torch, mx, lens_k, seed)
    for _ in range(args.warmup):
        module_step(mx, m, stream)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(MODULE_PHASES) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        module_step(mx, m, stream, evs[i])
    torch.cuda.synchronize()
    ph = {n: float(np.median([e[i].elapsed_time(e[i + 1]) * 1e-3 for e in evs])) for i, n in enumerate(MODULE_PHASES)}
    t_step = float(np.median([e[0].elapsed_time(e[-1]) * 1e-3 for e in evs]))
    Tq, Tk, CM, C = m["Tq"], m["Tk"], m["CM"], m["Hm"] * D
    f_attn = attn_flops(m["lens_q"], lens_k, m["Hm"], False)
    f_proj = 2.0 * CM * C * (Tq + 2 * Tk)
    total = 3.5 * f_attn + 3 * f_proj
    res = {k + "_us": round(v * 1e6, 2) for k, v in ph.items()}
    res.update({"module_step_us": round(t_step * 1e6, 2), "fwd_us": round(sum(ph[k] for k in MODULE_PHASES[:3]) * 1e6, 2),
                "bwd_us": round(sum(ph[k] for k in MODULE_PHASES[3:]) * 1e6, 2),
                "attn_fwd_pflops": round(f_attn / ph["attn_fwd"] / 1e15, 4),
                "attn_bwd_pflops": round(2.5 * f_attn / ph["attn_bwd"] / 1e15, 4),
                "projection_pflops": round(f_proj / ph["producers"] / 1e15, 4),
                "producer_bwd_pflops": round(2 * f_proj / ph["producer_bwd"] / 1e15, 4)})
    print("# module: " + ", ".join(f"{k}={v}" for k, v in res.items()), file=sys.stderr, flush=True)
    dom = max(ph, key=ph.get)
    dom_f = {"producers": f_proj, "attn_fwd": f_attn, "attn_bwd": 2.5 * f_attn, "scatter": 0.0,
             "producer_bwd": 2 * f_proj}[dom]
    workload = label or ("cross-attention module training step: 64 samples x 256 queries, 64 key sequences with "
                         "lengths uniform in [256, 2048], H=8, model dim 1024")
    out = {
        "metric": "MXFP8 cross-attention module training step PF/s (projections, their backward, attention fwd/bwd) "
                  "and % of MI355X dense MXFP8 MFMA peak",
        "value": round(total / t_step / 1e15, 4), "unit": "PF/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": workload + "; RMSNorm+quantize -> projection+quantize -> scale scatter -> attention "
                                          "fwd -> quantize dO -> attention bwd (FP16 dQ, MXFP8 gradients) -> "
                                          "projection data/weight gradients -> RMSNorm bwd",
                   "tokens_q": Tq, "tokens_k": Tk, **res},
        "roofline": {"bound": "mfma", "achieved": round(dom_f / ph[dom] / 1e12, 2), "peak": PEAK_MXFP8 / 1e12,
                     "unit": "TFLOP/s", "frac": round(dom_f / ph[dom] / PEAK_MXFP8, 4), "traffic": None,
                     "kernel": {"producers": "rmsnorm_quantize + linear_quantize (phase)", "attn_fwd": "attn_fwd_kernel",
                                "attn_bwd": "quantize dO + mxfa_bwd_mx_out call", "scatter": "scale_scatter_kernel",
                                "producer_bwd": "linear_bwd_data x3 + rmsnorm_bwd x2 + linear_bwd_weight x3 (phase)"}[dom],
                     "launch_us": round(ph[dom] * 1e6, 2)},
    }
    if not args.no_cpu_baseline and cpu_picks:
        picks = [int(s) for s in np.argsort(lens_k)[::-1][:cpu_picks]]
        fl, dt = module_cpu_baseline(m, picks)
        model, nproc, _ = host_cpu()
        out["cpu_baseline"] = {"value": round(fl / dt / 1e15, 8), "unit": "PF/s", "cores": 16 if nproc >= 16 else nproc,
                               "kind": "oracle", "cpu_model": model, "nproc": nproc,
                               "sample": f"head 3 of the {len(picks)} samples with the longest key sequences: the whole "
                                         f"training step on that head's slice, {dt:.1f} s wall"}
    print(json.dumps(out), flush=True)
    del m
    torch.cuda.empty_cache()


def bench_module_latency(args, torch, mx):
    """Module training-step latency at 4,096, 8,192 and 16,384 key/value tokens (64 samples x 256 queries,
    key lengths uniform around total / 64), one JSON line each."""
    for total in (4096, 8192, 16384):
        L = total // MODULE_B
        lens = [int(v) for v in synth_mod.lengths(6, MODULE_B, L // 2, L + L // 2)]
        bench_module(args, torch, mx, lens_k=lens, seed=6,
                     label=f"cross-attention module training step at {total} key/value tokens (actual {sum(lens)}): "
                           f"64 samples x 256 queries, key lengths uniform in [{L // 2}, {L + L // 2}], H=8, "
                           f"model dim 1024", cpu_picks=1)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); each GPU's shard of a larger "
              "job is this single-GPU workload at its real shape", file=sys.stderr)
        sys.exit(2)
    import torch
    import precision_mxfp8_block_amd as mx
    import synth
    global synth_mod
    synth_mod = synth

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
    if args.forward_only:
        for line in bench_forward_only(args, torch, mx):
            print(json.dumps(line), flush=True)
        return
    if args.module:
        bench_module(args, torch, mx)
        bench_module_latency(args, torch, mx)
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
        mx.mxfa_quantize_col32_row32(dev["v"], C, T, C, cu_d, B, N, vd_, vs, vrd, vrs, stream)
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
    # Q, K, V, dO read once in bf16; five E4M3 payloads (V's COL32 and ROW32 from one read); scales
    quant_bytes = 4 * T * C * 2 + 5 * T * C + 3 * T * C / 1024 + T * C / 32 * 2
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
    # the headline step is measured first, on a GPU that has run nothing else; the per-workload lines
    # follow, and the headline line is printed last
    if not args.headline_only:
        bench_workloads(args, torch, mx)
        bench_module(args, torch, mx)
        bench_module_latency(args, torch, mx)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(host, cu)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

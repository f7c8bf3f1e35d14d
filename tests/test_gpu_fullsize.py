"""Full-size parity on the GPU: the HIP path runs at the benchmark workloads' full sizes and in the
launch configuration the benchmark uses (whole batch, all heads, one call per step), and sampled
(sequence, head) slices are checked against the oracle, which computes each slice alone in seconds.
Quantization, RMSNorm and attention never mix sequences or heads (the projection mixes columns
but not tokens), so a slice of the full-size result must equal the oracle's result on the slice's
inputs.

Workloads (shapes, value distributions and seeds of the five workload descriptions):
  LLM forward     B=4, H=16, N=4096: Q/K ROW32, V COL32, forward only; the same with Q/K in MXFP4
                  and in MXFP6
  training step   same shape: Q/K/dO SQ32, V COL32 (forward) + ROW32 (backward), FP16 dQ with
                  sigma = 1 (the benchmark's step) and FP32 dQ
  causal          B=4, H=16, N=8192, causal, 0.5% of entries x64, both dQ modes
  jagged          32 sequences with lengths uniform in [128, 4096], H=16, scales scattered
  cross-attention module  64 x 256 queries, 64 key sequences with lengths uniform in [256, 2048],
                  H=8, model dim 1024: RMSNorm+quantize -> projection+quantize -> scatter ->
                  forward -> backward
"""
import math

import numpy as np
import pytest
import torch

import oracle
import precision_mxfp8_block_amd as mx
import synth
from mx_cases import (Guarded, LinearCase, certify_linear, check_grads, check_o, cu_dev, gpu_quantize_padded,
                      gpu_quantize_v_both_padded, say,
                      to_dev_bf16, to_host_bf16_bits)

pytestmark = pytest.mark.gpu

D = 128
C_SCALE = float(np.float32(1.0 / math.sqrt(D)))


def block_offsets(lens):
    """Compact block-row offset of each sequence: sum over earlier sequences of ceil(L/32)."""
    return np.concatenate([[0], np.cumsum((np.asarray(lens) + 31) // 32)]).astype(np.int64)


def scale_slice(scale, mode, cu, boff, s, h, heads_cols=True):
    """Compact scales of sequence s, head h (all columns of the row when heads_cols is False)."""
    rows = slice(int(cu[s]), int(cu[s + 1])) if mode == mx.ROW32 else slice(int(boff[s]), int(boff[s + 1]))
    if not heads_cols:
        return scale[rows]
    cols = slice(h * D, (h + 1) * D) if mode == mx.COL32 else slice(h * D // 32, (h + 1) * D // 32)
    return scale[rows, cols]


def host(t):
    return t.detach().cpu().numpy()


def xcd_slices(nseq, H, n=8):
    """One (sequence, head) pair from each XCD's share of the attention kernels' grid, at a different
    position in each share: the forward's XCD x runs the pairs p = x, x + 8, x + 16, ... (p = sequence *
    H + head); for 64 pairs the picks also fall in the 8 different contiguous ranges of 8 pairs that
    the backward of a uniform batch gives the XCDs."""
    pairs = nseq * H
    per = pairs // n
    out = []
    for x in range(n):
        p = x + 8 * ((3 * x + 1) % max(per, 1))
        out.append((p // H, p % H))
    return out


def all_written(t, label):
    """Outputs are NaN-prefilled: a non-finite element anywhere in the full tensor is one the kernels
    never wrote (the inputs here produce finite outputs)."""
    bad = int((~torch.isfinite(t.float())).sum())
    assert bad == 0, f"{label}: {bad} elements not written (still NaN) or non-finite"


class FullAttn:
    """Full-size attention problem on the GPU plus oracle checks of sampled (sequence, head) slices, all
    slices in one oracle call (one sequence per slice, so they run on parallel threads)."""

    def __init__(self, seed, lens_q, lens_k, H, causal=False, outlier_p=0.0, qk_mode=mx.SQ32):
        self.outliers = outlier_p > 0
        self.lens_q, self.lens_k = list(lens_q), list(lens_k)
        self.cu_q, self.cu_k = synth.cu_seqlens(self.lens_q), synth.cu_seqlens(self.lens_k)
        self.bq, self.bk = block_offsets(self.lens_q), block_offsets(self.lens_k)
        self.Tq, self.Tk = int(self.cu_q[-1]), int(self.cu_k[-1])
        self.H, self.causal, self.qk_mode = H, causal, qk_mode
        C = H * D
        self.C = C
        kw = dict(outlier_p=outlier_p)
        say(f"  generating inputs Tq={self.Tq} Tk={self.Tk} C={C}")
        self.x = {"q": synth.normal_bf16(seed, synth.STREAM_Q, (self.Tq, C), **kw),
                  "k": synth.normal_bf16(seed, synth.STREAM_K, (self.Tk, C), **kw),
                  "v": synth.normal_bf16(seed, synth.STREAM_V, (self.Tk, C), **kw),
                  "do": synth.normal_bf16(seed, synth.STREAM_DO, (self.Tq, C), **kw)}
        self.dev = {n: to_dev_bf16(a) for n, a in self.x.items()}
        self.cu_q_d, self.cu_k_d = cu_dev(self.cu_q), cu_dev(self.cu_k)

    def gpu_fwd(self, p_scale=mx.P_STATIC):
        self.gq = gpu_quantize_padded(self.dev["q"], self.cu_q, self.cu_q_d, self.qk_mode)
        self.gk = gpu_quantize_padded(self.dev["k"], self.cu_k, self.cu_k_d, self.qk_mode)
        if self.qk_mode == mx.SQ32:
            # training: V's two payloads from one read, as the benchmark's step quantizes it
            self.gv, self.gvd = gpu_quantize_v_both_padded(self.dev["v"], self.cu_k, self.cu_k_d)
        else:
            self.gv = gpu_quantize_padded(self.dev["v"], self.cu_k, self.cu_k_d, mx.COL32)
            self.gvd = None
        self.args = mx.AttnArgs(mx.MxOperand(self.gq[0], self.gq[1], self.qk_mode),
                                mx.MxOperand(self.gk[0], self.gk[1], self.qk_mode),
                                mx.MxOperand(self.gv[0], self.gv[1], mx.COL32),
                                self.cu_q_d, self.cu_k_d, len(self.lens_q), max(self.lens_q), max(self.lens_k),
                                self.Tq, self.Tk, self.H, D, C_SCALE, self.causal)
        o, lse = Guarded((self.Tq, self.C), torch.bfloat16), Guarded((self.H, self.Tq), torch.float32)
        if p_scale == mx.P_STATIC:
            mx.mxfa_fwd(self.args, o.t, lse.t)
        else:
            mx.mxfa_fwd_p_scale(self.args, p_scale, o.t, lse.t)
        torch.cuda.synchronize()
        o.check("O"), lse.check("LSE")
        all_written(o.t, "O")
        self.o, self.lse = o.t, lse.t

    def gpu_bwd(self, dq_mode, sigma):
        if self.gvd is None:
            self.gvd = gpu_quantize_padded(self.dev["v"], self.cu_k, self.cu_k_d, mx.ROW32)
        self.gdo = gpu_quantize_padded(self.dev["do"], self.cu_q, self.cu_q_d, mx.SQ32)
        need = mx.mxfa_bwd_workspace_size(self.args, dq_mode)
        ws = Guarded((need,), torch.uint8)
        g = [Guarded((T, self.C), torch.bfloat16) for T in (self.Tq, self.Tk, self.Tk)]
        mx.mxfa_bwd(self.args, mx.MxOperand(self.gvd[0], self.gvd[1], mx.ROW32),
                    mx.MxOperand(self.gdo[0], self.gdo[1], mx.SQ32), self.o, self.dev["do"], self.lse, dq_mode, sigma,
                    ws.t, need, *(x.t for x in g))
        torch.cuda.synchronize()
        ws.check("workspace")
        for x, n in zip(g, ("dQ", "dK", "dV")):
            x.check(n)
            all_written(x.t, n)
        return tuple(x.t for x in g)

    def _stack(self, name, slices):
        """The (sequence, head) slices of one input stacked as the sequences of a one-head batch."""
        cu = self.cu_q if name in ("q", "do") else self.cu_k
        return np.ascontiguousarray(np.concatenate(
            [self.x[name][int(cu[s]):int(cu[s + 1]), h * D:(h + 1) * D] for s, h in slices]))

    def _stack_cu(self, slices, side):
        lens = self.lens_q if side == "q" else self.lens_k
        return synth.cu_seqlens([lens[s] for s, _ in slices])

    def _check_quant(self, name, gpu, mode, slices, ref):
        """The GPU's full-size quantization, sliced, equals the oracle's quantization of the slices."""
        cu, boff = (self.cu_q, self.bq) if name in ("q", "do") else (self.cu_k, self.bk)
        cs = self._stack_cu(slices, "q" if name in ("q", "do") else "k")
        bs = block_offsets(np.diff(cs))
        for i, (s, h) in enumerate(slices):
            rows = slice(int(cu[s]), int(cu[s + 1]))
            np.testing.assert_array_equal(host(gpu[0][rows, h * D:(h + 1) * D]), ref[0][int(cs[i]):int(cs[i + 1])],
                                          err_msg=f"{name} payload, slice {s, h}")
            rrows = slice(int(cs[i]), int(cs[i + 1])) if mode == mx.ROW32 else slice(int(bs[i]), int(bs[i + 1]))
            np.testing.assert_array_equal(scale_slice(host(gpu[2]), mode, cu, boff, s, h), ref[1][rrows],
                                          err_msg=f"{name} scale, slice {s, h}")

    def oracle_fwd_slices(self, slices, p_scale=oracle.P_STATIC):
        cq, ck = self._stack_cu(slices, "q"), self._stack_cu(slices, "k")
        say(f"  oracle forward on {len(slices)} slices {slices}")
        self.rq = oracle.quantize(self._stack("q", slices), cq, self.qk_mode)
        self.rk = oracle.quantize(self._stack("k", slices), ck, self.qk_mode)
        rv = oracle.quantize(self._stack("v", slices), ck, oracle.COL32)
        self._check_quant("q", self.gq, self.qk_mode, slices, self.rq)
        self._check_quant("k", self.gk, self.qk_mode, slices, self.rk)
        self._check_quant("v", self.gv, mx.COL32, slices, rv)
        o16, o32, lse = oracle.attn_fwd_mx(self.rq[0], self.rq[1], self.qk_mode, self.rk[0], self.rk[1], self.qk_mode,
                                           rv[0], rv[1], oracle.COL32, cq, ck, 1, D, C_SCALE, self.causal,
                                           p_scale=p_scale)
        for i, (s, h) in enumerate(slices):
            rows = slice(int(self.cu_q[s]), int(self.cu_q[s + 1]))
            r = slice(int(cq[i]), int(cq[i + 1]))
            o_g = to_host_bf16_bits(self.o[rows, h * D:(h + 1) * D])
            lse_g = host(self.lse[h, rows])[None, :]
            check_o(o_g, o32[r], lse_g, lse[:, r], f"seq {s} head {h}", outliers=self.outliers)
        return o16, lse

    def oracle_bwd_slices(self, slices, o16, lse, g, dq_mode, sigma):
        cq, ck = self._stack_cu(slices, "q"), self._stack_cu(slices, "k")
        say(f"  oracle backward on {len(slices)} slices, dq_mode {dq_mode}")
        rvd = oracle.quantize(self._stack("v", slices), ck, oracle.ROW32)
        rdo = oracle.quantize(self._stack("do", slices), cq, oracle.SQ32)
        self._check_quant("v", self.gvd, mx.ROW32, slices, rvd)
        self._check_quant("do", self.gdo, mx.SQ32, slices, rdo)
        ref = oracle.attn_bwd_mx(self.rq[0], self.rq[1], self.rk[0], self.rk[1], rvd[0], rvd[1], oracle.ROW32,
                                 rdo[0], rdo[1], o16, self._stack("do", slices), lse, cq, ck, 1, D, C_SCALE,
                                 self.causal, dq_mode, sigma)
        assert ref["overflow"] == 0, "oracle FP16 accumulator overflowed: sigma too large for this input"
        for i, (s, h) in enumerate(slices):
            qr = slice(int(self.cu_q[s]), int(self.cu_q[s + 1]))
            kr = slice(int(self.cu_k[s]), int(self.cu_k[s + 1]))
            rq_, rk_ = slice(int(cq[i]), int(cq[i + 1])), slice(int(ck[i]), int(ck[i + 1]))
            cols = slice(h * D, (h + 1) * D)
            gs = (to_host_bf16_bits(g[0][qr, cols]), to_host_bf16_bits(g[1][kr, cols]),
                  to_host_bf16_bits(g[2][kr, cols]))
            sub = {"dq_f": ref["dq_f"][rq_], "dk_f": ref["dk_f"][rk_], "dv_f": ref["dv_f"][rk_]}
            check_grads(gs, sub, f"seq {s} head {h} dq_mode {dq_mode}", qk_outliers=self.outliers)


def test_llm_forward_B4_H16_N4096():
    say("full-size forward: B=4 H=16 N=4096, Q/K ROW32, V COL32")
    fa = FullAttn(2, [4096] * 4, [4096] * 4, 16, qk_mode=mx.ROW32)
    fa.gpu_fwd()
    fa.oracle_fwd_slices(xcd_slices(4, 16))


@pytest.mark.parametrize("fmt", ["e2m1", "e2m3"])
def test_llm_forward_small_qk_B4_H16_N4096(fmt):
    """The forward with Q and K in MXFP4 (E2M1) or MXFP6 (E2M3), ROW32, at the benchmark's size: the GPU's
    payloads and scales of the sampled slices equal the oracle's, and the slices' O and LSE match the
    oracle's forward."""
    from oracle import mxfp4, mxfp6
    mod, fwd, quant, elem, nb = ((mxfp4, mxfp4.attn_fwd_qk_fp4, mx.quantize_e2m1, mx.E2M1, D // 2) if fmt == "e2m1"
                                 else (mxfp6, mxfp6.attn_fwd_qk_fp6, mx.quantize_e2m3, mx.E2M3, 3 * D // 4))
    say(f"full-size forward: B=4 H=16 N=4096, Q/K {fmt} ROW32, V E4M3 COL32")
    fa = FullAttn(2, [4096] * 4, [4096] * 4, 16, qk_mode=mx.ROW32)
    q4, qs = quant(fa.dev["q"])
    k4, ks = quant(fa.dev["k"])
    gv = gpu_quantize_padded(fa.dev["v"], fa.cu_k, fa.cu_k_d, mx.COL32)
    args = mx.AttnArgs(mx.MxOperand(q4, qs, mx.ROW32, elem), mx.MxOperand(k4, ks, mx.ROW32, elem),
                       mx.MxOperand(gv[0], gv[1], mx.COL32), fa.cu_q_d, fa.cu_k_d, 4, 4096, 4096, fa.Tq, fa.Tk, 16, D,
                       C_SCALE, False)
    o, lse = Guarded((fa.Tq, fa.C), torch.bfloat16), Guarded((16, fa.Tq), torch.float32)
    mx.mxfa_fwd(args, o.t, lse.t)
    torch.cuda.synchronize()
    o.check("O"), lse.check("LSE")
    all_written(o.t, "O")
    slices = xcd_slices(4, 16)
    cq, ck = fa._stack_cu(slices, "q"), fa._stack_cu(slices, "k")
    rq = mod.quantize_row32(fa._stack("q", slices))
    rk = mod.quantize_row32(fa._stack("k", slices))
    rv = oracle.quantize(fa._stack("v", slices), ck, oracle.COL32)
    for i, (s, h) in enumerate(slices):
        rows = slice(int(fa.cu_q[s]), int(fa.cu_q[s + 1]))
        r = slice(int(cq[i]), int(cq[i + 1]))
        np.testing.assert_array_equal(host(q4[rows, h * nb:(h + 1) * nb]), rq[0][r])
        np.testing.assert_array_equal(host(qs[rows, h * 4:(h + 1) * 4]), rq[1][r])
        np.testing.assert_array_equal(host(k4[rows, h * nb:(h + 1) * nb]), rk[0][r])
        np.testing.assert_array_equal(host(ks[rows, h * 4:(h + 1) * 4]), rk[1][r])
    say(f"  oracle {fmt} forward on {len(slices)} slices {slices}")
    _, o32, lse_r = fwd(rq[0], rq[1], rk[0], rk[1], rv[0], rv[1], cq, ck, 1, D, C_SCALE)
    for i, (s, h) in enumerate(slices):
        rows = slice(int(fa.cu_q[s]), int(fa.cu_q[s + 1]))
        r = slice(int(cq[i]), int(cq[i + 1]))
        check_o(to_host_bf16_bits(o.t[rows, h * D:(h + 1) * D]), o32[r], host(lse.t[h, rows])[None, :], lse_r[:, r],
                f"seq {s} head {h}")


@pytest.mark.parametrize("dq_mode,sigma", [(mx.DQ_FP16_STATIC, 1.0), (mx.DQ_FP32, 1.0)])
def test_training_step_B4_H16_N4096(dq_mode, sigma):
    say(f"full-size training step: B=4 H=16 N=4096, dq_mode={dq_mode}")
    fa = FullAttn(2, [4096] * 4, [4096] * 4, 16)
    fa.gpu_fwd()
    g = fa.gpu_bwd(dq_mode, sigma)
    slices = xcd_slices(4, 16)
    o16, lse = fa.oracle_fwd_slices(slices)
    fa.oracle_bwd_slices(slices, o16, lse, g, dq_mode, sigma)


def test_training_forward_dynamic_p_B4_H16_N4096():
    """The forward with the dynamic per-block P scale, as the benchmark times it (training modes)."""
    say("full-size forward, dynamic P scale: B=4 H=16 N=4096, Q/K SQ32, V COL32")
    fa = FullAttn(2, [4096] * 4, [4096] * 4, 16)
    fa.gpu_fwd(mx.P_BLOCK_DYNAMIC)
    fa.oracle_fwd_slices(xcd_slices(4, 16)[::2], oracle.P_DYNAMIC)


@pytest.mark.parametrize("dq_mode,sigma", [(mx.DQ_FP16_STATIC, 0.0625), (mx.DQ_FP32, 1.0)])
def test_causal_outliers_B4_H16_N8192(dq_mode, sigma):
    say(f"full-size causal: B=4 H=16 N=8192, 0.5% x64 outliers, dq_mode={dq_mode} sigma={sigma}")
    fa = FullAttn(3, [8192] * 4, [8192] * 4, 16, causal=True, outlier_p=0.005)
    fa.gpu_fwd()
    g = fa.gpu_bwd(dq_mode, sigma)
    slices = xcd_slices(4, 16)
    o16, lse = fa.oracle_fwd_slices(slices)
    fa.oracle_bwd_slices(slices, o16, lse, g, dq_mode, sigma)


def test_jagged_32_sequences_H16():
    lens = [int(v) for v in synth.lengths(4, 32, 128, 4096)]
    say(f"full-size jagged: 32 sequences (sum {sum(lens)}), H=16, scattered scales, FP16 dQ")
    fa = FullAttn(4, lens, lens, 16)
    fa.gpu_fwd()
    g = fa.gpu_bwd(mx.DQ_FP16_STATIC, 1.0)
    longest = int(np.argmax(lens))
    ragged = [i for i, L in enumerate(lens) if L % 128 and i != longest]
    slices = [(longest, 3), (ragged[0], 12), (ragged[len(ragged) // 2], 7), (ragged[-1], 0)]
    o16, lse = fa.oracle_fwd_slices(slices)
    fa.oracle_bwd_slices(slices, o16, lse, g, mx.DQ_FP16_STATIC, 1.0)


# ---------------------------------------------------------------------------------------------
# Cross-attention module: producers + attention
# ---------------------------------------------------------------------------------------------

def test_cross_attention_module():
    B, NQ, H, CM = 64, 256, 8, 1024
    eps = 1e-6
    lens_q = [NQ] * B
    lens_k = [int(v) for v in synth.lengths(5, B, 256, 2048)]
    cu_q, cu_k = synth.cu_seqlens(lens_q), synth.cu_seqlens(lens_k)
    bq, bk = block_offsets(lens_q), block_offsets(lens_k)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    say(f"module: {B} x {NQ} queries, {Tk} keys, H={H}, model dim {CM}")
    xq = synth.normal_bf16(5, synth.STREAM_ACT, (Tq, CM))
    xkv = synth.normal_bf16(5, synth.STREAM_ACT + 1, (Tk, CM))
    w = {n: synth.normal_bf16(5, synth.STREAM_WEIGHT + i, (CM, CM), std=0.02) for i, n in enumerate("qkv")}
    dout = synth.normal_bf16(5, synth.STREAM_DO, (Tq, H * D))
    cq_d, ck_d = cu_dev(cu_q), cu_dev(cu_k)
    ones = torch.ones(CM, dtype=torch.float32, device="cuda")
    wcu = np.array([0, CM], np.int32)

    # ---- GPU path ----
    xq_hat = mx.rmsnorm_quantize(to_dev_bf16(xq), ones, eps, cu_q, cq_d)
    xkv_hat = mx.rmsnorm_quantize(to_dev_bf16(xkv), ones, eps, cu_k, ck_d)
    w_hat = {n: mx.quantize(to_dev_bf16(w[n]), wcu, cu_dev(wcu), mx.ROW32) for n in "qkv"}

    def project(xh, n, cu, cu_d):
        return mx.linear_quantize(mx.MxOperand(xh[0], xh[1], mx.SQ32), mx.MxOperand(w_hat[n][0], w_hat[n][1], mx.ROW32),
                                  cu, cu_d)
    gq = project(xq_hat, "q", cu_q, cq_d)
    gk = project(xkv_hat, "k", cu_k, ck_d)
    gv = project(xkv_hat, "v", cu_k, ck_d)
    pad = {n: mx.scale_scatter(t[1], cu_k, ck_d, H * D, mx.SQ32) for n, t in (("k", gk), ("v", gv))}
    args = mx.AttnArgs(mx.MxOperand(gq[0], gq[1], mx.SQ32), mx.MxOperand(gk[0], pad["k"], mx.SQ32),
                       mx.MxOperand(gv[0], pad["v"], mx.SQ32), cq_d, ck_d, B, NQ, max(lens_k), Tq, Tk, H, D, C_SCALE,
                       False)
    o, lse = mx.fwd(args)
    do_d = to_dev_bf16(dout)
    gdo = mx.quantize(do_d, cu_q, cq_d, mx.SQ32)
    grads = {m: mx.bwd(args, mx.MxOperand(gv[0], pad["v"], mx.SQ32), mx.MxOperand(gdo[0], gdo[1], mx.SQ32), o, do_d,
                       lse, m, 1.0) for m in (mx.DQ_FP16_STATIC, mx.DQ_FP32)}
    torch.cuda.synchronize()

    # ---- oracle on sampled (sequence, head) slices ----
    longest = int(np.argmax(lens_k))
    for s, h in [(longest, 2), (7, 5)]:
        cq = np.array([0, NQ], np.int32)
        ck = np.array([0, lens_k[s]], np.int32)
        qrows, krows = slice(int(cu_q[s]), int(cu_q[s + 1])), slice(int(cu_k[s]), int(cu_k[s + 1]))
        cols = slice(h * D, (h + 1) * D)
        say(f"  module slice: seq {s} (keys {lens_k[s]}), head {h}")
        outs = {}
        for n, xsrc, rows, cu1, boff, xh_g, g in (("q", xq, qrows, cq, bq, xq_hat, gq),
                                                  ("k", xkv, krows, ck, bk, xkv_hat, gk),
                                                  ("v", xkv, krows, ck, bk, xkv_hat, gv)):
            xd, xsc, _, _ = oracle.rmsnorm_quantize(np.ascontiguousarray(xsrc[rows]), np.ones(CM, np.float32), eps,
                                                    cu1)
            np.testing.assert_array_equal(host(xh_g[0][rows]), xd)
            brows = slice(int(boff[s]), int(boff[s + 1]))
            np.testing.assert_array_equal(host(xh_g[1][brows]), xsc)
            wd, ws, _ = oracle.quantize(np.ascontiguousarray(w[n][cols]), np.array([0, D], np.int32), oracle.ROW32)
            np.testing.assert_array_equal(host(w_hat[n][0][cols]), wd)
            np.testing.assert_array_equal(host(w_hat[n][1][cols]), ws)
            d_o, s_o, st_o, y = oracle.linear_quantize(xd, xsc, wd, ws, cu1)
            yabs = np.abs(oracle.dequantize(xd, xsc, cu1, oracle.SQ32)) @ np.abs(
                oracle.dequantize(wd, ws, np.array([0, D], np.int32), oracle.ROW32)).T
            hb = slice(h * D // 32, (h + 1) * D // 32)
            certify_linear(host(g[0][rows, cols]), host(g[1][brows, hb]), host(g[2][hb, brows]), d_o, s_o,
                           y.astype(np.float64), yabs, cu1, f"{n} projection seq {s} head {h}")
            outs[n] = (d_o, s_o)
        o16, o32, lse_r = oracle.attn_fwd_mx(outs["q"][0], outs["q"][1], oracle.SQ32, outs["k"][0], outs["k"][1],
                                             oracle.SQ32, outs["v"][0], outs["v"][1], oracle.SQ32, cq, ck, 1, D,
                                             C_SCALE, False)
        check_o(to_host_bf16_bits(o[qrows, cols]), o32, host(lse[h, qrows])[None, :], lse_r, f"module seq {s} head {h}")
        rdo = oracle.quantize(np.ascontiguousarray(dout[qrows, cols]), cq, oracle.SQ32)
        for m, g in grads.items():
            ref = oracle.attn_bwd_mx(outs["q"][0], outs["q"][1], outs["k"][0], outs["k"][1], outs["v"][0],
                                     outs["v"][1], oracle.SQ32, rdo[0], rdo[1], o16,
                                     np.ascontiguousarray(dout[qrows, cols]), lse_r, cq, ck, 1, D, C_SCALE, False, m,
                                     1.0)
            gs = (to_host_bf16_bits(g[0][qrows, cols]), to_host_bf16_bits(g[1][krows, cols]),
                  to_host_bf16_bits(g[2][krows, cols]))
            check_grads(gs, ref, f"module seq {s} head {h} dq_mode {m}")

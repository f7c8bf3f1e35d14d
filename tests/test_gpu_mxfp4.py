"""MXFP4 (E2M1) and MXFP6 (E2M3) paths on the GPU against the oracle: the ROW32 quantizers bit for
bit, the forward with Q and K in MXFP4 or MXFP6 (V in E4M3 COL32) to the forward's O and LSE
tolerances, and their SQNR against exact attention next to the MXFP8 forward's on the same inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import precision_mxfp8_block_amd as mx
import synth
from oracle import mxfp4, mxfp6
from mx_cases import (O_REL_FRO, Guarded, bf16_bits_to_f64, certify_mx_output, check_o, cu_dev, gpu_quantize_padded,
                      gpu_scale_scatter, say, to_dev_bf16, to_host_bf16_bits)

pytestmark = pytest.mark.gpu


# element format -> (payload bytes per 32 elements, GPU entry point, oracle module)
FORMATS = {"e2m1": (16, mx.mxfa_quantize_e2m1, mxfp4), "e2m3": (24, mx.mxfa_quantize_e2m3, mxfp6)}


def gpu_quantize_small(x_dev, fmt="e2m1"):
    T, C = x_dev.shape
    nbytes, fn, _ = FORMATS[fmt]
    data, scale = Guarded((T, C // 32 * nbytes), torch.uint8), Guarded((T, C // 32), torch.uint8)
    fn(x_dev, x_dev.stride(0), T, C, data.t, scale.t)
    torch.cuda.synchronize()
    data.check(f"{fmt} payload"), scale.check(f"{fmt} scales")
    return data.t.cpu().numpy(), scale.t.cpu().numpy()


def bf16_bits(vals):
    a = np.asarray(vals, np.float32).view(np.uint32)
    return (a >> 16).astype(np.uint16)


def crafted_rows_e2m3():
    """Rows of 64 columns at block maximum 4 (code 127, scale 1): every E2M3 midpoint, both signs;
    saturation; subnormal range; NaN/Inf and zero blocks."""
    grid = list(np.arange(0, 1, 1 / 8)) + list(np.arange(1, 2, 1 / 8)) + list(np.arange(2, 4, 1 / 4)) + \
        list(np.arange(4, 8, 1 / 2))
    mids = [(grid[c] + grid[c + 1]) / 2 for c in range(24)]  # midpoints up to 3.875 (block max stays 4)
    rows = []
    r = np.zeros(64, np.float32)
    r[:24] = mids
    r[24] = 4.0
    r[32:56] = -np.array(mids, np.float32)
    r[56] = -4.0
    rows.append(bf16_bits(r))
    r = np.zeros(64, np.float32)
    r[:6] = [7.25, 7.5, 7.75, 7.875, -7.625, 4.25]   # block max 7.875 (code 127): saturation and ties
    r[32:38] = [4.75, 5.25, 5.75, 6.25, 6.75, 7.25]  # midpoints of the top binade
    rows.append(bf16_bits(r))
    for extra in crafted_rows()[2:]:
        rows.append(extra)
    return np.stack(rows)


def crafted_rows():
    """Rows of 64 columns: ties at every midpoint, saturation, signed zeros, bf16 subnormals, a NaN and an
    Inf block, an all-zero block."""
    rows = []
    # block maximum 4 (code 127, scale 1): the scaled values are the values themselves
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0 / 1.25]  # 4.0 (the last) keeps amax at 4
    r = np.zeros(64, np.float32)
    r[:7] = mids
    r[7:14] = -np.array(mids, np.float32)
    r[14] = 4.0
    r[15] = -0.0
    r[32:40] = [0.3, 0.7, 1.1, 1.4, 2.2, 2.9, 3.6, -3.9]
    rows.append(bf16_bits(r))
    # maxima in [6, 8) after scaling saturate: block max 7.5 (code 127), elements 6.5, 7, 7.5
    r = np.zeros(64, np.float32)
    r[:4] = [6.5, 7.0, 7.5, -7.25]
    r[32:36] = [5.0, 5.5, -5.75, 6.0]
    rows.append(bf16_bits(r))
    # bf16 subnormals (code 0) and tiny normals
    b = np.zeros(64, np.uint16)
    b[:8] = [0x0001, 0x8002, 0x0040, 0x007F, 0x0080, 0x8081, 0x00FF, 0x0100]
    rows.append(b)
    # NaN in block 0, Inf in block 1
    b = bf16_bits(np.linspace(-3, 3, 64).astype(np.float32))
    b[5] = 0x7FC0
    b[40] = 0xFF80
    rows.append(b)
    rows.append(np.zeros(64, np.uint16))
    return np.stack(rows)


@pytest.mark.parametrize("fmt", ["e2m1", "e2m3"])
@pytest.mark.parametrize("case", ["normal_300x256", "normal_77x2048_ld", "crafted", "scaled_wide"])
def test_quantize_small_formats_bit_exact(case, fmt):
    say(f"{fmt} quantize case {case}")
    if case == "normal_300x256":
        x = synth.normal_bf16(41, 1, (300, 256))
        xd = to_dev_bf16(x)
    elif case == "normal_77x2048_ld":
        full = synth.normal_bf16(42, 2, (77, 2048 + 64))
        x = np.ascontiguousarray(full[:, :2048])
        xd = to_dev_bf16(full)[:, :2048]  # row stride 2112 elements
    elif case == "crafted":
        x = crafted_rows() if fmt == "e2m1" else crafted_rows_e2m3()
        xd = to_dev_bf16(x)
    else:
        # magnitudes spread over many binades per block
        rng = np.random.default_rng(43)
        f = (rng.normal(size=(64, 512)) * np.exp2(rng.integers(-60, 60, (64, 512)))).astype(np.float32)
        x = bf16_bits(f.view(np.uint32) & 0xFFFF0000)
        xd = to_dev_bf16(x)
    d, s = gpu_quantize_small(xd, fmt)
    d_ref, s_ref = FORMATS[fmt][2].quantize_row32(x)
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(d, d_ref)


class Fp4Case:
    """Attention problem whose Q and K are quantized to MXFP4 or MXFP6 (ROW32) and V to MXFP8 COL32."""

    def __init__(self, seed, lens_q, lens_k=None, H=2, causal=False, fmt="e2m1"):
        self.H, self.causal, self.fmt = H, causal, fmt
        self.lens_q, self.lens_k = list(lens_q), list(lens_k or lens_q)
        self.cu_q, self.cu_k = synth.cu_seqlens(self.lens_q), synth.cu_seqlens(self.lens_k)
        self.Tq, self.Tk = int(self.cu_q[-1]), int(self.cu_k[-1])
        C = H * 128
        self.C = C
        self.q = synth.normal_bf16(seed, synth.STREAM_Q, (self.Tq, C))
        self.k = synth.normal_bf16(seed, synth.STREAM_K, (self.Tk, C))
        self.v = synth.normal_bf16(seed, synth.STREAM_V, (self.Tk, C))
        self.c = float(np.float32(1 / math.sqrt(128)))

    def run_gpu(self, p_scale=mx.P_STATIC):
        cq, ck = cu_dev(self.cu_q), cu_dev(self.cu_k)
        qd, kd, vd = to_dev_bf16(self.q), to_dev_bf16(self.k), to_dev_bf16(self.v)
        quant = mx.quantize_e2m1 if self.fmt == "e2m1" else mx.quantize_e2m3
        elem = mx.E2M1 if self.fmt == "e2m1" else mx.E2M3
        q4, qs = quant(qd)
        k4, ks = quant(kd)
        qsp = qs if all(L % 128 == 0 for L in self.lens_q) else gpu_scale_scatter(qs, self.cu_q, cq, self.C, mx.ROW32)
        ksp = ks if all(L % 128 == 0 for L in self.lens_k) else gpu_scale_scatter(ks, self.cu_k, ck, self.C, mx.ROW32)
        gv = gpu_quantize_padded(vd, self.cu_k, ck, mx.COL32)
        args = mx.AttnArgs(mx.MxOperand(q4, qsp, mx.ROW32, elem), mx.MxOperand(k4, ksp, mx.ROW32, elem),
                           mx.MxOperand(gv[0], gv[1], mx.COL32), cq, ck, len(self.lens_q), max(self.lens_q),
                           max(self.lens_k), self.Tq, self.Tk, self.H, 128, self.c, self.causal)
        self.args = args
        o, lse = Guarded((self.Tq, self.C), torch.bfloat16), Guarded((self.H, self.Tq), torch.float32)
        if p_scale == mx.P_STATIC:
            mx.mxfa_fwd(args, o.t, lse.t)
        else:
            mx.mxfa_fwd_p_scale(args, p_scale, o.t, lse.t)
        torch.cuda.synchronize()
        o.check("O"), lse.check("LSE")
        self.q4_gpu, self.k4_gpu = q4.cpu().numpy(), k4.cpu().numpy()
        return to_host_bf16_bits(o.t), lse.t.cpu().numpy()

    def run_oracle(self, p_scale=oracle.P_STATIC):
        mod = FORMATS[self.fmt][2]
        q4, qs = mod.quantize_row32(self.q)
        k4, ks = mod.quantize_row32(self.k)
        v8, vs, _ = oracle.quantize(self.v, self.cu_k, oracle.COL32)
        self.q4_ref, self.k4_ref = q4, k4
        fwd = mxfp4.attn_fwd_qk_fp4 if self.fmt == "e2m1" else mxfp6.attn_fwd_qk_fp6
        return fwd(q4, qs, k4, ks, v8, vs, self.cu_q, self.cu_k, self.H, 128, self.c, self.causal, p_scale=p_scale)


FWD_CASES = [
    ("uniform 2x256", 51, [256, 256], None, 2, False, mx.P_STATIC),
    ("jagged 300/1000/77", 52, [300, 1000, 77], None, 2, False, mx.P_STATIC),
    ("causal 640", 53, [640], None, 1, True, mx.P_STATIC),
    ("cross 128/200 x 1000/333", 54, [128, 200], [1000, 333], 2, False, mx.P_STATIC),
    ("jagged, dynamic P scale", 55, [300, 513], None, 2, False, mx.P_BLOCK_DYNAMIC),
]


@pytest.mark.parametrize("fmt", ["e2m1", "e2m3"])
@pytest.mark.parametrize("label,seed,lq,lk,H,causal,p_scale", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_small_qk_parity(label, seed, lq, lk, H, causal, p_scale, fmt):
    say(f"{fmt} Q/K forward case {label}: seed {seed}, lengths {lq} / {lk or lq}, H={H}, causal={causal}")
    case = Fp4Case(seed, lq, lk, H, causal, fmt)
    o_g, lse_g = case.run_gpu(p_scale)
    _, o32, lse = case.run_oracle(oracle.P_STATIC if p_scale == mx.P_STATIC else oracle.P_DYNAMIC)
    np.testing.assert_array_equal(case.q4_gpu, case.q4_ref)
    np.testing.assert_array_equal(case.k4_gpu, case.k4_ref)
    check_o(o_g, o32, lse_g, lse, label=label)


MX_OUT_SMALL_CASES = [FWD_CASES[i] for i in (1, 2)]


@pytest.mark.parametrize("fmt", ["e2m1", "e2m3"])
@pytest.mark.parametrize("label,seed,lq,lk,H,causal,p_scale", MX_OUT_SMALL_CASES, ids=[c[0] for c in MX_OUT_SMALL_CASES])
def test_fwd_small_qk_mx_out(label, seed, lq, lk, H, causal, p_scale, fmt):
    """The MXFP4 / MXFP6 Q/K forward writing O as MXFP8 (ROW32 blocks along D) with bf16 O in the same
    pass: the bf16 O and LSE equal mxfa_fwd's bit for bit, every code and byte of the MXFP8 O is
    certified against that bf16 O (mx_cases.certify_mx_output), and against the oracle's FP32 O the
    codes are within one and the dequantized O within 2^-4 + the O tolerance (relative Frobenius)."""
    say(f"{fmt} Q/K forward with MXFP8 O, case {label}")
    case = Fp4Case(seed, lq, lk, H, causal, fmt)
    o_bits, lse_g = case.run_gpu()
    T, C = case.Tq, case.C
    o16, od, osc = Guarded((T, C), torch.bfloat16), Guarded((T, C), torch.uint8), Guarded((T, C // 32), torch.uint8)
    lse2 = Guarded((case.H, T), torch.float32)
    mx.mxfa_fwd_mx_out(case.args, mx.P_STATIC, o16.t, od.t, osc.t, lse2.t)
    torch.cuda.synchronize()
    for g in (o16, od, osc, lse2):
        g.check("fwd_mx_out output")
    np.testing.assert_array_equal(to_host_bf16_bits(o16.t), o_bits)
    np.testing.assert_array_equal(lse2.t.cpu().numpy(), lse_g)
    gd, gs = od.t.cpu().numpy(), osc.t.cpu().numpy()
    certify_mx_output(gd, gs, o_bits, case.cu_q, oracle.ROW32, f"{fmt} {label} O")
    _, o32, _ = case.run_oracle()
    o32 = np.asarray(o32, np.float32)
    _, rs, _ = oracle.quantize(o32, case.cu_q, oracle.ROW32)
    assert np.abs(gs.astype(np.int64) - rs.astype(np.int64)).max() <= 1
    deq = oracle.dequantize(gd, gs, case.cu_q, oracle.ROW32)
    fro = float(np.linalg.norm(deq - o32) / np.linalg.norm(o32))
    say(f"  rel_fro of the dequantized MXFP8 O vs the oracle's FP32 O: {fro:.3e}")
    assert fro <= 2.0 ** -4 + O_REL_FRO


def sqnr_db(x, ref):
    return 10.0 * math.log10(float(np.sum(ref * ref)) / float(np.sum((x - ref) ** 2)))


def test_fwd_small_qk_sqnr_next_to_mxfp8():
    """O's SQNR against exact attention for Q/K in MXFP4, MXFP6 and MXFP8 (same inputs, V E4M3 COL32 in
    all): the GPU's value matches the oracle's replay within 0.25 dB in each format."""
    case = Fp4Case(56, [1024, 1024], None, 2, False)
    o_g, _ = case.run_gpu()
    o16_ref, _, _ = case.run_oracle()
    c6 = Fp4Case(56, [1024, 1024], None, 2, False, "e2m3")
    o6_g, _ = c6.run_gpu()
    o6_ref, _, _ = c6.run_oracle()
    f = {n: bf16_bits_to_f64(getattr(case, n)) for n in ("q", "k", "v")}
    _, ex, _ = oracle.attn_fwd_f64(f["q"], f["k"], f["v"], case.cu_q, case.cu_k, case.H, 128, case.c, False,
                                   quant_p=False)
    ex = ex.astype(np.float64)
    s4_gpu, s4_orc = sqnr_db(bf16_bits_to_f64(o_g), ex), sqnr_db(bf16_bits_to_f64(o16_ref), ex)
    s6_gpu, s6_orc = sqnr_db(bf16_bits_to_f64(o6_g), ex), sqnr_db(bf16_bits_to_f64(o6_ref), ex)
    # the MXFP8 forward on the same inputs (Q, K ROW32)
    from mx_cases import AttnCase
    c8 = AttnCase(56, [1024, 1024], H=2, fwd_modes="infer")
    o8_g, _ = c8.run_gpu_fwd()
    o8_ref, _, _ = c8.run_oracle_fwd()
    s8_gpu, s8_orc = sqnr_db(bf16_bits_to_f64(o8_g), ex), sqnr_db(bf16_bits_to_f64(o8_ref), ex)
    say(f"O SQNR vs exact: Q/K MXFP4 {s4_gpu:.2f} dB (oracle {s4_orc:.2f}), Q/K MXFP6 {s6_gpu:.2f} dB "
        f"(oracle {s6_orc:.2f}), Q/K MXFP8 {s8_gpu:.2f} dB (oracle {s8_orc:.2f})")
    assert abs(s4_gpu - s4_orc) <= 0.25 and abs(s6_gpu - s6_orc) <= 0.25 and abs(s8_gpu - s8_orc) <= 0.25
    # E2M3 keeps E4M3's three mantissa bits (only the exponent range shrinks, which a 32-element block
    # of N(0,1) values hardly uses): MXFP6 Q/K lands within 1 dB of MXFP8; E2M1's single bit costs ~9 dB
    assert abs(s6_gpu - s8_gpu) < 1.0 and min(s6_gpu, s8_gpu) > s4_gpu + 5.0

"""GPU parity of the producer backward against the oracle: the projection's data gradient
(mxfa_linear_bwd_data), its weight gradient (mxfa_linear_bwd_weight, fed by the transposed scale grids)
and the RMSNorm backward (mxfa_rmsnorm_bwd).

Bounds. The GPU's scaled MFMA adds products in groups of 8 with an adder that drops the bits of each
product below 2^(e - 14), e the exponent of the group's largest product, then accumulates in FP32
(the same bound the projection's test uses): |GPU - exact| <= LINEAR_DELTA_REL * sum |products|. dX is
then rounded to bf16 (half an ulp, 2^-9 relative, allowed as 2^-8). The RMSNorm backward runs in FP32
(sums over C and over the rows in a different order than the oracle's FP64): 1e-5 of the terms' size,
then the bf16 rounding of dx. Every output is prefilled with NaN patterns inside guard bytes, so an
element the kernels never write, or a write out of bounds, fails.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from mx_cases import LINEAR_DELTA_REL, Guarded, cu_dev, say, to_dev_bf16

pytestmark = pytest.mark.gpu

import precision_mxfp8_block_amd as mx  # noqa: E402


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _operands(seed, lens, C_out, C_in, dy_mode=oracle.SQ32):
    """dY ~ N(0,1) [T, C_out] quantized (SQ32 by default) and X ~ N(0,1) [T, C_in] SQ32, W ~ N(0, 0.02)
    [C_out, C_in] with W^T quantized ROW32 along C_out; quantization by the oracle (inputs only)."""
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    dy = synth.normal_bf16(seed, synth.STREAM_DO, (T, C_out))
    x = synth.normal_bf16(seed, synth.STREAM_ACT, (T, C_in))
    w = synth.normal_bf16(seed, synth.STREAM_WEIGHT, (C_out, C_in), std=0.02)
    q_dy = oracle.quantize(dy, cu, dy_mode)
    q_x = oracle.quantize(x, cu, oracle.SQ32)
    q_wt = oracle.quantize(np.ascontiguousarray(w.T), np.array([0, C_in], np.int32), oracle.ROW32)
    return cu, T, q_dy, q_x, q_wt


DATA_CASES = [
    # (label, seed, lens, C_out, C_in, dy mode)
    ("ragged_Cout256_Cin384", 71, [40, 300, 1, 129], 256, 384, oracle.SQ32),
    ("dense_Cout1024_Cin1024", 72, [512], 1024, 1024, oracle.SQ32),
    ("row32_dy_Cout128_Cin256", 73, [200, 33], 128, 256, oracle.ROW32),
]


@pytest.mark.parametrize("case", DATA_CASES, ids=[c[0] for c in DATA_CASES])
def test_linear_bwd_data(case):
    label, seed, lens, C_out, C_in, dy_mode = case
    say(f"linear_bwd_data {label}: lens={lens} C_out={C_out} C_in={C_in}")
    cu, T, (dyd, dys, _), _, (wtd, wts, _) = _operands(seed, lens, C_out, C_in, dy_mode)
    dx = Guarded((T, C_in), torch.bfloat16)
    mx.mxfa_linear_bwd_data(mx.MxOperand(torch.from_numpy(dyd).cuda(), torch.from_numpy(dys).cuda(), dy_mode),
                            mx.MxOperand(torch.from_numpy(wtd).cuda(), torch.from_numpy(wts).cuda(), mx.ROW32),
                            T, C_out, C_in, cu_dev(cu), len(lens), max(lens), 0, dx.t)
    torch.cuda.synchronize()
    dx.check("dx")
    g = _bf16_to_f64(dx.t.cpu().view(torch.int16).numpy().view(np.uint16))
    dy_deq = oracle.dequantize(dyd, dys, cu, dy_mode)
    wt_deq = oracle.dequantize(wtd, wts, np.array([0, C_in], np.int32), oracle.ROW32)
    if dy_mode == oracle.SQ32:
        _, ref = oracle.linear_bwd_data(dyd, dys, wtd, wts, cu)
        ref = ref.astype(np.float64)
    else:  # the oracle's data gradient takes SQ32 dY; ROW32 dY by its dequantized product
        ref = (dy_deq @ wt_deq.T).astype(np.float32).astype(np.float64)
    absum = np.abs(dy_deq) @ np.abs(wt_deq).T
    err = np.abs(g - ref)
    bound = 2.0 ** -8 * np.abs(ref) + LINEAR_DELTA_REL * absum
    say(f"  max err / bound = {np.max(err / np.maximum(bound, 1e-300)):.3f}, rel fro "
        f"{np.linalg.norm(g - ref) / np.linalg.norm(ref):.2e}")
    assert np.all(np.isfinite(g))
    assert np.all(err <= bound), np.argwhere(err > bound)[:5]


def test_linear_bwd_data_accumulate():
    """Two data gradients into one input (key and value projections): the second call adds to the bf16
    output of the first; compared with the oracle's same two-call composition."""
    lens, C_out, C_in = [300, 77, 129], 256, 384
    cu, T, (d1, s1, _), _, (w1, ws1, _) = _operands(74, lens, C_out, C_in)
    _, _, (d2, s2, _), _, (w2, ws2, _) = _operands(75, lens, C_out, C_in)
    say(f"linear_bwd_data accumulate: T={T}")
    dx = Guarded((T, C_in), torch.bfloat16)
    dev = lambda a: torch.from_numpy(a).cuda()
    for acc, (d, s, w, ws) in enumerate(((d1, s1, w1, ws1), (d2, s2, w2, ws2))):
        mx.mxfa_linear_bwd_data(mx.MxOperand(dev(d), dev(s), mx.SQ32), mx.MxOperand(dev(w), dev(ws), mx.ROW32), T, C_out,
                                C_in, cu_dev(cu), len(lens), max(lens), acc, dx.t)
    torch.cuda.synchronize()
    dx.check("dx")
    g = _bf16_to_f64(dx.t.cpu().view(torch.int16).numpy().view(np.uint16))
    ref1, ref1_f = oracle.linear_bwd_data(d1, s1, w1, ws1, cu)
    _, ref = oracle.linear_bwd_data(d2, s2, w2, ws2, cu, dx_in=ref1)
    ref = ref.astype(np.float64)
    wcu = np.array([0, C_in], np.int32)
    absum = (np.abs(oracle.dequantize(d1, s1, cu, oracle.SQ32)) @ np.abs(oracle.dequantize(w1, ws1, wcu, oracle.ROW32)).T +
             np.abs(oracle.dequantize(d2, s2, cu, oracle.SQ32)) @ np.abs(oracle.dequantize(w2, ws2, wcu, oracle.ROW32)).T)
    # the final bf16 rounding, the first call's bf16 output (which may round the other way on the GPU:
    # one ulp of the first product) and the two products' MFMA error
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -7 * np.abs(ref1_f.astype(np.float64)) + LINEAR_DELTA_REL * absum
    err = np.abs(g - ref)
    say(f"  max err / bound = {np.max(err / bound):.3f}")
    assert np.all(err <= bound), np.argwhere(err > bound)[:5]


WEIGHT_CASES = [
    # (label, seed, lens, C_out, C_in)
    ("ragged_Cout256_Cin384", 81, [40, 300, 1, 129, 7], 256, 384),
    ("odd_block_count", 82, [129], 128, 128),               # a chunk holding one token block
    ("whole_blocks_spare_chunk", 84, [32, 64, 32], 128, 128),  # the grid's last chunk has no block
    ("many_chunks_Cout256_Cin256", 83, None, 256, 256),
]


@pytest.mark.parametrize("case", WEIGHT_CASES, ids=[c[0] for c in WEIGHT_CASES])
def test_linear_bwd_weight(case):
    label, seed, lens, C_out, C_in = case
    if lens is None:  # 200 jagged sequences: many token chunks, partial blocks everywhere
        lens = [int(v) for v in synth.lengths(seed, 200, 1, 300)]
    say(f"linear_bwd_weight {label}: {len(lens)} sequences, T={sum(lens)}, C_out={C_out}, C_in={C_in}")
    cu, T, (dyd, dys, dyst), (xd, xs, xst), _ = _operands(seed, lens, C_out, C_in)
    ws = torch.empty(mx.mxfa_linear_bwd_weight_workspace_size(T, len(lens), C_out, C_in), dtype=torch.uint8,
                     device="cuda")
    dw = Guarded((C_out, C_in), torch.float32)
    dev = {n: torch.from_numpy(a).cuda() for n, a in (("dy", dyd), ("dyst", dyst), ("x", xd), ("xst", xst))}
    mx.mxfa_linear_bwd_weight(dev["dy"], dev["dyst"], dev["x"], dev["xst"], T, C_out, C_in, cu_dev(cu), len(lens),
                              max(lens), ws, ws.numel(), dw.t)
    torch.cuda.synchronize()
    dw.check("dw")
    g = dw.t.cpu().numpy().astype(np.float64)
    ref = oracle.linear_bwd_weight(dyd, dyst, xd, xst, cu).astype(np.float64)
    dyq = oracle.dequantize(dyd, dys, cu, oracle.SQ32)
    xq = oracle.dequantize(xd, xs, cu, oracle.SQ32)
    absum = np.abs(dyq).T @ np.abs(xq)
    err = np.abs(g - ref)
    bound = LINEAR_DELTA_REL * absum
    say(f"  max err / bound = {np.max(err / np.maximum(bound, 1e-300)):.3f}, rel fro "
        f"{np.linalg.norm(g - ref) / np.linalg.norm(ref):.2e}")
    assert np.all(np.isfinite(g))
    assert np.all(err <= bound), np.argwhere(err > bound)[:5]


def test_linear_bwd_weight_module_shape_sampled():
    """The module's key/value side (64 jagged lengths uniform in [256, 2048], T = 75,659, 1024 x 1024):
    sampled 64 x 64 corners and an interior block of dW against a float64 matmul of the dequantized
    operands (the oracle's dequantizer; the oracle's own dW over all tokens is checked above)."""
    lens = [int(v) for v in synth.lengths(4, 64, 256, 2048)]
    C = 1024
    cu, T, (dyd, dys, dyst), (xd, xs, xst), _ = _operands(4, lens, C, C)
    say(f"linear_bwd_weight module shape: T={T}")
    ws = torch.empty(mx.mxfa_linear_bwd_weight_workspace_size(T, len(lens), C, C), dtype=torch.uint8, device="cuda")
    dw = Guarded((C, C), torch.float32)
    dev = {n: torch.from_numpy(a).cuda() for n, a in (("dy", dyd), ("dyst", dyst), ("x", xd), ("xst", xst))}
    mx.mxfa_linear_bwd_weight(dev["dy"], dev["dyst"], dev["x"], dev["xst"], T, C, C, cu_dev(cu), len(lens), max(lens),
                              ws, ws.numel(), dw.t)
    torch.cuda.synchronize()
    dw.check("dw")
    g = dw.t.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g))
    dyq = oracle.dequantize(dyd, dys, cu, oracle.SQ32)
    xq = oracle.dequantize(xd, xs, cu, oracle.SQ32)
    for o0, i0 in [(0, 0), (960, 960), (448, 576), (0, 960)]:
        os_, is_ = slice(o0, o0 + 64), slice(i0, i0 + 64)
        ref = dyq[:, os_].T @ xq[:, is_]
        absum = np.abs(dyq[:, os_]).T @ np.abs(xq[:, is_])
        err = np.abs(g[os_, is_] - ref)
        say(f"  block ({o0}, {i0}): max err / bound {np.max(err / (LINEAR_DELTA_REL * absum)):.3f}")
        assert np.all(err <= LINEAR_DELTA_REL * absum)


RMS_CASES = [
    # (label, seed, T, C, eps)
    ("T1000_C1024", 91, 1000, 1024, 1e-6),
    ("T300_C96_partial_lanes", 92, 300, 96, 1e-6),
    ("T257_C2048", 93, 257, 2048, 1e-5),
]


@pytest.mark.parametrize("case", RMS_CASES, ids=[c[0] for c in RMS_CASES])
def test_rmsnorm_bwd(case):
    label, seed, T, C, eps = case
    say(f"rmsnorm_bwd {label}")
    x = synth.normal_bf16(seed, synth.STREAM_ACT, (T, C), std=3.0)
    dy = synth.normal_bf16(seed, synth.STREAM_DO, (T, C))
    gamma = (0.5 + synth.uniform(seed, synth.STREAM_WEIGHT, C)).astype(np.float32)
    ws = torch.empty(mx.mxfa_rmsnorm_bwd_workspace_size(T, C), dtype=torch.uint8, device="cuda")
    dx = Guarded((T, C), torch.bfloat16)
    dg = Guarded((C,), torch.float32)
    xd = to_dev_bf16(x)
    mx.mxfa_rmsnorm_bwd(xd, C, T, C, torch.from_numpy(gamma).cuda(), eps, to_dev_bf16(dy), ws, ws.numel(), dx.t, dg.t)
    torch.cuda.synchronize()
    dx.check("dx")
    dg.check("dgamma")
    _, dx_ref, dg_ref = oracle.rmsnorm_bwd(x, gamma, eps, dy)
    xf, dyf, g64 = _bf16_to_f64(x), _bf16_to_f64(dy), gamma.astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + eps)
    scale = np.abs(r * g64 * dyf) + np.abs(xf) * r ** 3 * np.sum(np.abs(g64 * dyf * xf), axis=1, keepdims=True) / C
    gx = _bf16_to_f64(dx.t.cpu().view(torch.int16).numpy().view(np.uint16))
    err = np.abs(gx - dx_ref)
    bound = 2.0 ** -8 * np.abs(dx_ref) + 1e-5 * scale
    say(f"  dx max err / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound), np.argwhere(err > bound)[:5]
    gg = dg.t.cpu().numpy().astype(np.float64)
    absum = np.sum(np.abs(dyf * xf * r), axis=0)
    say(f"  dgamma max err / bound {np.max(np.abs(gg - dg_ref) / (1e-5 * absum)):.3f}")
    assert np.all(np.abs(gg - dg_ref) <= 1e-5 * absum)

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on identical seeded inputs.

Bit-exact for the quantizer, the scale scatter and the RMSNorm+quantize producer; certified
mismatches only for the projection GEMM + quantize producer; tolerances of
tests/mx_cases.py for attention (both P scales). The MXFP8 outputs of the forward (O) and the backward
(dQ, dK, dV) are certified byte by byte against the GPU's own bf16 results of the same pass and compared
with the oracle's FP32 results through its quantizer. Every output is written into a NaN-prefilled
buffer between guard bytes (mx_cases.Guarded). Sizes here finish in seconds on the oracle and still
span several tiles and ragged tails; full-size sampled checks are in test_gpu_fullsize.py, the
structure-sensitive backward cases in test_gpu_structure.py and the exhaustive quantizer sweep in
test_gpu_quantize_sweep.py.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_mxfp8_block_amd as mx
import synth
from mx_cases import (GRAD_REL_FRO, O_MAX_ABS, O_REL_FRO, AttnCase, Guarded, LinearCase, certify_linear,
                      certify_mx_output, check_grads, check_o, cu_dev, gpu_quantize, gpu_scale_scatter, rel_fro, say,
                      to_dev_bf16, to_host_bf16_bits)

pytestmark = pytest.mark.gpu


def _special_matrix(seed, T, C):
    """N(0,1) bf16 with outliers, exact zeros, bf16 subnormals, a NaN and an Inf block, and
    values that scale onto E4M3 rounding ties."""
    x = synth.normal_bf16(seed, 1, (T, C), outlier_p=0.01)
    xf = synth.bf16_bits_to_f32(x).copy()
    xf[0, :64] = 0.0
    xf[1, 32:64] = np.float32(1e-39)  # bf16 subnormals
    xf[1, 40] = np.float32(3e-39)
    xf[2, 0:32] = np.float32([1.0625, 1.1875, 2.0, 432.0] * 8)  # ties after scaling
    if T > 40:
        xf[40, 5] = np.nan
        xf[37, 100 % C] = np.inf
    return synth.f32_to_bf16_bits(xf)


@pytest.mark.parametrize("mode", [oracle.ROW32, oracle.COL32, oracle.SQ32])
@pytest.mark.parametrize("lens", [[256], [37, 128, 1, 300, 95, 64]])
@pytest.mark.parametrize("C", [384, 160, 224, 96])  # C % 128 = 32, 96 and C < 128: partial column groups
def test_quantize_bit_exact(mode, lens, C):
    say(f"quantize mode={mode} lens={lens} C={C}")
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    x = _special_matrix(3 + mode, T, C)
    d_ref, s_ref, st_ref = oracle.quantize(x, cu, mode)
    data, scale, scale_t = gpu_quantize(to_dev_bf16(x), cu, cu_dev(cu), mode, want_scale_t=(mode == oracle.SQ32))
    np.testing.assert_array_equal(data.cpu().numpy(), d_ref)
    np.testing.assert_array_equal(scale.cpu().numpy(), s_ref)
    if mode == oracle.SQ32:
        np.testing.assert_array_equal(scale_t.cpu().numpy(), st_ref)


def gpu_quantize_col32_row32(x_dev, cu, ld=None):
    T, C = x_dev.shape
    lens = np.diff(np.asarray(cu, np.int64))
    nb = int(np.sum((lens + 31) // 32))
    dc, sc = Guarded((T, C), torch.uint8), Guarded((nb, C), torch.uint8)
    dr, sr = Guarded((T, C), torch.uint8), Guarded((T, C // 32), torch.uint8)
    mx.mxfa_quantize_col32_row32(x_dev, ld or x_dev.stride(0), T, C, cu_dev(cu), len(lens), int(lens.max()), dc.t,
                                 sc.t, dr.t, sr.t)
    torch.cuda.synchronize()
    for g, n in ((dc, "COL32 payload"), (sc, "COL32 scales"), (dr, "ROW32 payload"), (sr, "ROW32 scales")):
        g.check(n)
    return [g.t.cpu().numpy() for g in (dc, sc, dr, sr)]


@pytest.mark.parametrize("lens", [[256], [37, 128, 1, 300, 95, 64]])
@pytest.mark.parametrize("C", [384, 160, 224, 96, 2048])
def test_quantize_col32_row32_bit_exact(lens, C):
    """One read, both layouts: byte for byte the oracle's COL32 and ROW32 quantizations (NaN/Inf blocks,
    subnormals, ties, ragged sequence tails, partial column groups)."""
    say(f"quantize COL32+ROW32 lens={lens} C={C}")
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    x = _special_matrix(11, T, C)
    dc, sc, dr, sr = gpu_quantize_col32_row32(to_dev_bf16(x), cu)
    dc_ref, sc_ref, _ = oracle.quantize(x, cu, oracle.COL32)
    dr_ref, sr_ref, _ = oracle.quantize(x, cu, oracle.ROW32)
    np.testing.assert_array_equal(sc, sc_ref)
    np.testing.assert_array_equal(dc, dc_ref)
    np.testing.assert_array_equal(sr, sr_ref)
    np.testing.assert_array_equal(dr, dr_ref)


def test_quantize_col32_row32_strided_and_sweep():
    """ld_x > C, and every bf16 pattern (the exhaustive sweep matrix) through the fused quantizer."""
    from test_gpu_quantize_sweep import sweep_matrix
    say("quantize COL32+ROW32 strided")
    T, C, ld = 96, 128, 200
    full = synth.normal_bf16(5, 1, (T, ld))
    cu = synth.cu_seqlens([40, 56])
    x = np.ascontiguousarray(full[:, :C])
    dc, sc, dr, sr = gpu_quantize_col32_row32(to_dev_bf16(full)[:, :C], cu, ld=ld)
    for got, ref in zip((dc, sc), oracle.quantize(x, cu, oracle.COL32)[:2]):
        np.testing.assert_array_equal(got, ref)
    for got, ref in zip((dr, sr), oracle.quantize(x, cu, oracle.ROW32)[:2]):
        np.testing.assert_array_equal(got, ref)
    say("quantize COL32+ROW32 sweep")
    x, cu = sweep_matrix()
    dc, sc, dr, sr = gpu_quantize_col32_row32(to_dev_bf16(x), cu)
    for got, ref in zip((dc, sc), oracle.quantize(x, cu, oracle.COL32)[:2]):
        np.testing.assert_array_equal(got, ref)
    for got, ref in zip((dr, sr), oracle.quantize(x, cu, oracle.ROW32)[:2]):
        np.testing.assert_array_equal(got, ref)


def test_quantize_strided_rows():
    """ld_x > C: the quantizer reads the first C columns of each row."""
    say("quantize strided")
    T, C, ld = 64, 128, 200
    full = synth.normal_bf16(4, 1, (T, ld))
    cu = synth.cu_seqlens([T])
    d_ref, s_ref, _ = oracle.quantize(np.ascontiguousarray(full[:, :C]), cu, oracle.SQ32)
    xd = to_dev_bf16(full)
    data, scale = Guarded((T, C), torch.uint8), Guarded((2, C // 32), torch.uint8)
    mx.mxfa_quantize(xd, ld, T, C, cu_dev(cu), 1, T, mx.SQ32, data.t, scale.t)
    torch.cuda.synchronize()
    data.check("data"), scale.check("scale")
    np.testing.assert_array_equal(data.t.cpu().numpy(), d_ref)
    np.testing.assert_array_equal(scale.t.cpu().numpy(), s_ref)


@pytest.mark.parametrize("C", [256, 2048])
@pytest.mark.parametrize("mode", [oracle.ROW32, oracle.COL32, oracle.SQ32])
def test_scale_scatter_bit_exact(mode, C):
    # C = 256: ROW32/SQ32 scale rows of 8 bytes (byte copies); C = 2048: every layout in 16-byte pieces
    lens = [37, 128, 1, 300, 95, 256]
    say(f"scatter mode={mode} C={C}")
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    x = synth.normal_bf16(5, 1, (T, C))
    _, s_ref, _ = oracle.quantize(x, cu, mode)
    p_ref = oracle.scale_scatter(s_ref, cu, C, mode)
    cud = cu_dev(cu)
    _, scale, _ = gpu_quantize(to_dev_bf16(x), cu, cud, mode)
    padded = gpu_scale_scatter(scale, cu, cud, C, mode)
    np.testing.assert_array_equal(padded.cpu().numpy(), p_ref)


RMSNORM_CASES = [
    # (lens, C, NaN position or None): C = 512..2048 in steps of 512 take the register-resident
    # kernel, other multiples of 32 the general one
    ([64], 1024, None),
    ([37, 128, 1, 95], 1024, None),
    ([37, 128, 1, 95], 512, None),
    ([40, 33], 1536, None),
    ([37, 1, 70], 2048, None),
    ([37, 64, 1], 1024, (40, 100)),
    ([37, 128, 1, 95], 800, None),
    ([5, 64], 96, (6, 3)),
]


@pytest.mark.parametrize("lens,C,nan_at", RMSNORM_CASES, ids=[f"{c[1]}-{len(c[0])}seq-{'nan' if c[2] else 'fin'}"
                                                             for c in RMSNORM_CASES])
def test_rmsnorm_quantize_bit_exact(lens, C, nan_at):
    say(f"rmsnorm lens={lens} C={C} nan_at={nan_at}")
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    x = synth.normal_bf16(6, synth.STREAM_ACT, (T, C))
    if nan_at is not None:
        x[nan_at] = 0x7FC0  # a quiet bf16 NaN: its row's blocks get code 255 and payload 0x7F
    gamma = (1.0 + 0.1 * synth.normal(6, synth.STREAM_WEIGHT, C)).astype(np.float32)
    d_ref, s_ref, st_ref, _ = oracle.rmsnorm_quantize(x, gamma, 1e-6, cu)
    nb = s_ref.shape[0]
    data, scale, scale_t = Guarded((T, C), torch.uint8), Guarded((nb, C // 32), torch.uint8), Guarded((C // 32, nb),
                                                                                                      torch.uint8)
    mx.mxfa_rmsnorm_quantize(to_dev_bf16(x), C, T, C, torch.from_numpy(gamma).cuda(), 1e-6, cu_dev(cu), len(lens),
                             max(lens), data.t, scale.t, scale_t.t)
    torch.cuda.synchronize()
    for g in (data, scale, scale_t):
        g.check("rmsnorm output")
    np.testing.assert_array_equal(data.t.cpu().numpy(), d_ref)
    np.testing.assert_array_equal(scale.t.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(scale_t.t.cpu().numpy(), st_ref)


LINEAR_CASES = [
    # (label, seed, lens, C_in, C_out, x_mode, nan_at, pm_exp2)
    ("dense_T256_1024x1024", 21, [256], 1024, 1024, oracle.SQ32, None, None),
    ("jagged_ragged_256x256", 22, [40, 300, 1, 129], 256, 256, oracle.SQ32, None, None),
    ("row32_x_128x384", 23, [200], 128, 384, oracle.ROW32, None, None),
    ("nan_block", 24, [64, 96], 256, 128, oracle.SQ32, (70, 5), None),
    # products of +-2^-60 entries: Y is exact and its block codes fall below 8
    ("tiny_codes_exact", 25, [96, 200], 256, 384, oracle.SQ32, None, (-60, -60)),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=[c[0] for c in LINEAR_CASES])
def test_linear_quantize_certified(case):
    label, seed, lens, C_in, C_out, x_mode, nan_at, pm_exp2 = case
    say(f"linear {label}")
    lc = LinearCase(seed, lens, C_in, C_out, x_mode=x_mode, nan_at=nan_at, pm_exp2=pm_exp2)
    dg, sg, stg = lc.run_gpu()
    do, so, sto, y, yabs = lc.run_oracle()
    if pm_exp2 is not None:  # exact Y: bytes and codes must match exactly
        assert int(so[so != 255].max()) < 8, "the case must reach output codes below 8"
        np.testing.assert_array_equal(sg, so)
        np.testing.assert_array_equal(stg, sto)
        np.testing.assert_array_equal(dg, do)
    certify_linear(dg, sg, stg, do, so, y, yabs, lc.cu, label)


FWD_CASES = [
    # (label, seed, lens_q, lens_k, H, causal, outlier_p, modes)
    ("tiny_N256_train", 1, [256], None, 1, False, 0.0, "train"),
    ("N512_H2_fwdonly", 2, [512], None, 2, False, 0.0, "fwd"),
    ("ragged_train", 3, [200, 77, 384, 1], None, 2, False, 0.0, "train"),
    ("ragged_causal_outliers", 4, [300, 129, 512], None, 1, True, 0.005, "train"),
    ("cross_lens", 5, [256, 64], [1000, 33], 1, False, 0.0, "fwd"),
    # an empty sequence between two others (offsets of the compact and padded layouts skip it);
    # 640 keys: an odd number of key tiles, 1 and 2 tiles in the others
    ("empty_seq_middle", 6, [128, 0, 200, 640], None, 2, False, 0.0, "train"),
    ("causal_5_tiles", 10, [640, 130], None, 1, True, 0.0, "train"),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_parity(case):
    label, seed, lq, lk, H, causal, op, modes = case
    say(f"fwd {label}")
    c = AttnCase(seed, lq, lk, H=H, causal=causal, outlier_p=op, fwd_modes=modes)
    o_gpu, lse_gpu = c.run_gpu_fwd()
    _, o32, lse = c.run_oracle_fwd()
    check_o(o_gpu, o32, lse_gpu, lse, label)


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_parity_dynamic_p(case):
    """The per-block dynamic P scale against the oracle's dynamic mode on the same cases."""
    label, seed, lq, lk, H, causal, op, modes = case
    say(f"fwd dynamic P {label}")
    c = AttnCase(seed, lq, lk, H=H, causal=causal, outlier_p=op, fwd_modes=modes)
    o_gpu, lse_gpu = c.run_gpu_fwd(mx.P_BLOCK_DYNAMIC)
    _, o32, lse = c.run_oracle_fwd(oracle.P_DYNAMIC)
    check_o(o_gpu, o32, lse_gpu, lse, label)


def test_fwd_dynamic_p_peaky_softmax():
    """Softmax scale 1 (scores with standard deviation ~11): most 32-key blocks lie far below their
    row maximum, so their codes drop below 119 and, at the static scale, their P would fall among
    E4M3 subnormals or to zero. Both P scales must match the oracle's corresponding mode (under the
    peaked-softmax bound), and the dynamic scale must change the result."""
    say("fwd dynamic P peaky softmax")
    c = AttnCase(21, [384, 200, 640], None, H=2, fwd_modes="train", softmax_scale=1.0)
    o_sta, lse_sta = c.run_gpu_fwd(mx.P_STATIC)
    _, o32, lse = c.run_oracle_fwd(oracle.P_STATIC)
    check_o(o_sta, o32, lse_sta, lse, "peaky_static", peaked=True)
    o_dyn, lse_dyn = c.run_gpu_fwd(mx.P_BLOCK_DYNAMIC)
    _, o32, lse = c.run_oracle_fwd(oracle.P_DYNAMIC)
    check_o(o_dyn, o32, lse_dyn, lse, "peaky_dynamic", peaked=True)
    assert np.any(o_dyn != o_sta)
    _, o_exact, _ = c.run_oracle_fwd(oracle.P_NONE)
    err_dyn = rel_fro(synth.bf16_bits_to_f32(o_dyn), o_exact)
    err_sta = rel_fro(synth.bf16_bits_to_f32(o_sta), o_exact)
    say(f"  rel_fro vs unquantized P: dynamic {err_dyn:.3e}, static {err_sta:.3e}")


def check_mx_sq32_output(label, gd, gs, own_bits, ref_f, cu, rel_tol):
    """An SQ32 MXFP8 output, certified byte by byte against the GPU's own bf16 output written in the same
    pass (mx_cases.certify_mx_output), and against the oracle's FP32 result (codes within one, relative
    Frobenius error within 2^-4 + the stated tolerance; the fractions of equal codes and bytes with the
    oracle's quantization of its own result are printed)."""
    certify_mx_output(gd, gs, own_bits, cu, oracle.SQ32, label)
    deq = oracle.dequantize(gd, gs, cu, oracle.SQ32)
    rd, rs, _ = oracle.quantize(np.asarray(ref_f, np.float32), cu, oracle.SQ32)
    dc = gs.astype(np.int64) - rs.astype(np.int64)
    fro = rel_fro(deq, ref_f)
    say(f"  {label}: codes equal {float(np.mean(dc == 0)):.4f}, bytes equal {float(np.mean(gd == rd)):.4f}, "
        f"rel_fro vs oracle {fro:.3e}")
    assert np.abs(dc).max() <= 1, label
    assert fro <= 2.0 ** -4 + rel_tol, label


MX_OUT_CASES = [FWD_CASES[i] for i in (0, 2, 3, 4, 5)]


@pytest.mark.parametrize("case", MX_OUT_CASES, ids=[c[0] for c in MX_OUT_CASES])
def test_fwd_mx_out_parity(case):
    """O written as MXFP8 (ROW32 blocks along D) in the forward's epilogue.
    * Against the GPU's own O (the bf16 O written in the same pass rounds the FP32 O that was quantized):
      every block code and every byte certified by mx_cases.certify_mx_output.
    * Against the oracle (its FP32 O, which differs from the GPU's by the attention tolerance): codes
      within one, the dequantized output within the O tolerance plus amax / 8, and within 2^-4 + the O
      tolerance in relative Frobenius norm; the fractions of equal codes and bytes are printed.
    * The bf16 O written in the same pass equals mxfa_fwd's bit for bit, and O_data does not depend on
      whether bf16 O is written. Outputs are guarded and NaN-prefilled."""
    label, seed, lq, lk, H, causal, op, modes = case
    say(f"fwd MX O {label}")
    c = AttnCase(seed, lq, lk, H=H, causal=causal, outlier_p=op, fwd_modes=modes)
    o_bits, lse_g = c.run_gpu_fwd()
    T, C = c.Tq, c.C

    def run(with_bf16):
        o16 = Guarded((T, C), torch.bfloat16) if with_bf16 else None
        od, osc, lse2 = Guarded((T, C), torch.uint8), Guarded((T, C // 32), torch.uint8), Guarded((c.H, T), torch.float32)
        mx.mxfa_fwd_mx_out(c.args, mx.P_STATIC, o16.t if o16 else None, od.t, osc.t, lse2.t)
        torch.cuda.synchronize()
        for g in (o16, od, osc, lse2):
            if g is not None:
                g.check("fwd_mx_out output")
        return (to_host_bf16_bits(o16.t) if o16 else None), od.t.cpu().numpy(), osc.t.cpu().numpy(), lse2.t.cpu().numpy()
    o16, gd, gs, lse2 = run(True)
    _, od_only, osc_only, _ = run(False)
    np.testing.assert_array_equal(o16, o_bits)
    np.testing.assert_array_equal(lse2, lse_g)
    np.testing.assert_array_equal(od_only, gd)
    np.testing.assert_array_equal(osc_only, gs)
    certify_mx_output(gd, gs, o_bits, c.cu_q, oracle.ROW32, f"{label} O")
    _, o32, _ = c.run_oracle_fwd()
    o32 = np.asarray(o32, np.float32)
    rd, rs, _ = oracle.quantize(o32, c.cu_q, oracle.ROW32)
    dc = gs.astype(np.int64) - rs.astype(np.int64)
    same_code, same_byte = float(np.mean(dc == 0)), float(np.mean(gd == rd))
    deq = oracle.dequantize(gd, gs, c.cu_q, oracle.ROW32)
    amax = np.repeat(np.abs(o32).reshape(T, C // 32, 32).max(axis=2), 32, axis=1)
    scale = max(1.0, float(np.abs(o32).max()))
    err = np.abs(deq - o32)
    say(f"  {label} codes equal {same_code:.4f}, payload bytes equal {same_byte:.4f}, "
        f"max err / (amax/8) {float(np.max(err / np.maximum(amax / 8, 1e-30))):.3f}, rel_fro {rel_fro(deq, o32):.3e}")
    assert np.abs(dc).max() <= 1
    assert np.all(err <= O_MAX_ABS * scale + amax / 8)
    assert rel_fro(deq, o32) <= 2.0 ** -4 + O_REL_FRO


def test_fwd_empty_key_sequence():
    """A sequence with no keys gives O = 0 and LSE = -inf."""
    say("fwd empty keys")
    c = AttnCase(7, [128, 64], [256, 0], H=1, fwd_modes="fwd")
    o_gpu, lse_gpu = c.run_gpu_fwd()
    _, o32, lse = c.run_oracle_fwd()
    check_o(o_gpu, o32, lse_gpu, lse, "empty_keys")
    assert np.all(o_gpu[128:] == 0)


BWD_CASES = [
    # (label, seed, lens, H, causal, outlier_p, FP16 static scale sigma)
    ("tiny_N256", 1, [256], 1, False, 0.0, 1.0),
    ("N512_H2", 2, [512], 2, False, 0.0, 1.0),
    ("ragged", 3, [200, 77, 384, 1], 2, False, 0.0, 1.0),
    # x64 outliers make |dQ / c| reach ~1.5e5: sigma = 2^-4 keeps the FP16 accumulator finite
    ("ragged_causal_outliers", 4, [300, 129, 512], 1, True, 0.005, 0.0625),
    ("empty_seq_middle", 6, [128, 0, 200, 640], 2, False, 0.0, 1.0),
]


@pytest.mark.parametrize("dq_mode", [mx.DQ_FP32, mx.DQ_FP16_STATIC])
@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_parity(case, dq_mode):
    label, seed, lens, H, causal, op, sigma = case
    say(f"bwd {label} dq_mode={dq_mode} sigma={sigma}")
    c = AttnCase(seed, lens, None, H=H, causal=causal, outlier_p=op, fwd_modes="train")
    c.run_gpu_fwd()
    c.run_oracle_fwd()
    g = c.run_gpu_bwd(dq_mode, sigma)
    ref = c.run_oracle_bwd(dq_mode, sigma)
    assert ref["overflow"] == 0
    check_grads(g, ref, label)


def test_bwd_fp16_sigma_scaling():
    """sigma = 2^-4: FP16 accumulator holds sigma dQ; the finalize divides it out."""
    say("bwd sigma")
    c = AttnCase(8, [256], None, H=1)
    c.run_gpu_fwd()
    c.run_oracle_fwd()
    g = c.run_gpu_bwd(mx.DQ_FP16_STATIC, 0.0625)
    ref = c.run_oracle_bwd(1, 0.0625)
    check_grads(g, ref, "sigma")


def test_bwd_deterministic():
    """The dQ reduction runs over the KV tiles in a fixed order: repeated runs are bit-identical in
    both dQ modes."""
    say("bwd determinism")
    c = AttnCase(9, [512, 300], None, H=2)
    c.run_gpu_fwd()
    for mode, sigma in ((mx.DQ_FP32, 1.0), (mx.DQ_FP16_STATIC, 0.5)):
        a = c.run_gpu_bwd(mode, sigma)
        b = c.run_gpu_bwd(mode, sigma)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


MX_GRAD_CASES = [(BWD_CASES[2], mx.DQ_FP32), (BWD_CASES[3], mx.DQ_FP16_STATIC), (BWD_CASES[4], mx.DQ_FP16_STATIC)]


@pytest.mark.parametrize("case,dq_mode", MX_GRAD_CASES, ids=[f"{c[0]}-dq{m}" for c, m in MX_GRAD_CASES])
def test_bwd_mx_out_parity(case, dq_mode):
    """dQ, dK, dV written as MXFP8 (SQ32 blocks from each sequence start, compact codes) in the
    backward's epilogues; the bf16 gradients of the same pass equal mxfa_bwd's bit for bit, and the
    MXFP8 payloads do not depend on whether bf16 gradients are written."""
    label, seed, lens, H, causal, op, sigma = case
    say(f"bwd MX gradients {label} dq_mode={dq_mode}")
    c = AttnCase(seed, lens, None, H=H, causal=causal, outlier_p=op, fwd_modes="train")
    c.run_gpu_fwd()
    c.run_oracle_fwd()
    g_bits = c.run_gpu_bwd(dq_mode, sigma)
    bits, mxo = c.run_gpu_bwd_mx_out(dq_mode, sigma)
    _, mxo_only = c.run_gpu_bwd_mx_out(dq_mode, sigma, with_bf16=False)
    for a, b in zip(bits, g_bits):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(mxo, mxo_only):
        np.testing.assert_array_equal(a, b)
    ref = c.run_oracle_bwd(dq_mode, sigma)
    for i, name in enumerate(("dq", "dk", "dv")):
        cu = c.cu_q if name == "dq" else c.cu_k
        check_mx_sq32_output(f"{label} {name}", mxo[2 * i], mxo[2 * i + 1], bits[i], ref[name + "_f"], cu,
                             GRAD_REL_FRO)


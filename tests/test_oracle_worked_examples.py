"""Hand-worked pins of the oracle's quantization points that closed forms with P in {0, 1} cannot see.

Each pin is written as a function of the oracle module (`orc`) so that tests/test_oracle_mutations.py
can run the same pin against deliberately broken copies of the oracle and require it to fail. Every
expected value below is derived by hand in the docstring or comment next to it (E4M3 codes from the
bit layout, FP16 results from IEEE binary16 round-to-nearest-even), never by calling the oracle.

Passages pinned:
  * static P scale 2^-8, E8M0 code 119 [brifing.si item 4: constant scale for P because softmax
    output lies in [0, 1]; andresseo.expert "Inside the TMEM Bargain and Zero-Gather Jagged
    Pipeline": P converted to MXFP8 online] -- forward and the backward's recomputed P;
  * Delta from the bf16 O and dO (the FlashAttention backward term the pages leave implicit; the
    oracle's reading) -- not from the quantized dO;
  * dS quantized once per 32 x 32 square block [andresseo.expert, same section; brifing.si item 6];
  * the FP16 dQ accumulator with a static power-of-two scale [andresseo.expert, same section:
    dQ reduced in FP16 with static scaling, or in FP32], and the binary16 rounding it uses.
"""
import math

import numpy as np

import oracle

E = 2.0 ** -17  # 256 * E = 2^-9, the smallest E4M3 subnormal: P = m * 2^-17 has code m at scale 2^-8

# Static-P table: (target P, the value E4M3(256 P) / 256 decodes to, worked by hand).
#   m * 2^-17, m = 1..7 : 256 P = m * 2^-9, exactly the subnormal with mantissa field m
#   0.4 * 2^-17         : 256 P = 0.4 * 2^-9 < 2^-10 (half the smallest subnormal) -> 0
#   0.6 * 2^-17         : 256 P = 0.6 * 2^-9 -> nearest subnormal 1 * 2^-9
#   1.3 * 2^-14         : 256 P = 1.3 * 2^-6, binade [2^-6, 2^-5) with step 2^-9: 1.3 * 8 = 10.4 -> 10,
#                         1.25 * 2^-6 (code 0x0A)
#   0.75                : 256 P = 192 = 1.5 * 2^7 exactly (code 0x74)
#   0.3                 : 256 P = 76.8, binade [64, 128) with step 8: 9.6 -> 10, 80 (code 0x6A), 80/256
STATIC_P_TABLE = ([(1.0, 1.0)] + [(m * E, m * E) for m in range(1, 8)] +
                  [(0.4 * E, 0.0), (0.6 * E, E), (1.3 * 2.0 ** -14, 1.25 * 2.0 ** -14), (0.75, 0.75),
                   (0.3, 0.3125)])


def _static_p_problem():
    """One query row against keys whose scores make P_j = exp(s_j - 0) the table's targets: q = e_0,
    k_j = s_j e_0 with s_j = fp32(ln target_j), softmax scale 1, key 0 the row maximum (s = 0, P = 1)."""
    nk, D = len(STATIC_P_TABLE), 128
    s = np.array([np.float32(math.log(t)) for t, _ in STATIC_P_TABLE], np.float64)
    q = np.zeros((1, D)); q[0, 0] = 1.0
    k = np.zeros((nk, D)); k[:, 0] = s
    p32 = np.array([np.float32(math.exp(x)) for x in s], np.float64)  # fl32 of the exact exponential
    deq = np.array([d for _, d in STATIC_P_TABLE])
    return nk, D, q, k, p32, deq


def pin_static_p_forward(orc):
    """Forward, static P scale: with V the identity, O_d = fl32(deq(P_q)_d / l) exposes every
    quantized P, and l = fl32(sum of the FP32 P) (the row sum adds the unquantized P). The scores
    place most P in E4M3's subnormal band at scale 2^-8; at scale 1 they would all round to zero."""
    nk, D, q, k, p32, deq = _static_p_problem()
    v = np.zeros((nk, D)); v[np.arange(nk), np.arange(nk)] = 1.0
    cu_q, cu_k = np.array([0, 1], np.int32), np.array([0, nk], np.int32)
    _, o, lse = orc.attn_fwd_f64(q, k, v, cu_q, cu_k, 1, D, 1.0, quant_p=orc.P_STATIC)
    l = np.float32(np.sum(p32))  # exact in double: every P is an fp32 number within 2^-18 .. 1
    expect = np.zeros(D, np.float32)
    expect[:nk] = (deq / np.float64(l)).astype(np.float32)
    np.testing.assert_array_equal(o[0], expect)
    assert lse[0, 0] == np.float32(math.log(float(l)))


def pin_static_p_backward(orc):
    """Backward, the recomputed P = exp(c S - LSE) at the same static scale: with LSE = 0, one query
    row and dO = e_0, dV_j = deq(P_q)_j e_0 exposes every quantized P (dV sums the quantized P, not the
    FP32 P). V, O and dO in Delta are 0 here, so dS = 0 and dQ = dK = 0."""
    nk, D, q, k, p32, deq = _static_p_problem()
    zeros_q, zeros_k = np.zeros((1, D)), np.zeros((nk, D))
    do = np.zeros((1, D)); do[0, 0] = 1.0
    cu_q, cu_k = np.array([0, 1], np.int32), np.array([0, nk], np.int32)
    lse = np.zeros((1, 1), np.float32)
    out = orc.attn_bwd_f64(q, k, zeros_k, do, zeros_q, zeros_q, lse, cu_q, cu_k, 1, D, 1.0, quant=True, dq_mode=0)
    expect = np.zeros((nk, D), np.float32)
    expect[:, 0] = deq
    np.testing.assert_array_equal(out["dv_f"], expect)
    assert not out["dq_f"].any() and not out["dk_f"].any()


def _bf16(vals):
    from synth import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(vals, np.float32))


def _bwd_mx(orc, q_bf, k_bf, v_bf, do_bf, o_bf, lens_q, lens_k, D, lse, dq_mode=0, sigma=1.0, c=1.0):
    """The oracle's MX backward on bf16 inputs quantized by its own quantizer: Q, K, dO SQ32, V ROW32."""
    cu_q = np.array(np.concatenate([[0], np.cumsum(lens_q)]), np.int32)
    cu_k = np.array(np.concatenate([[0], np.cumsum(lens_k)]), np.int32)
    qq = orc.quantize(q_bf, cu_q, orc.SQ32)
    kq = orc.quantize(k_bf, cu_k, orc.SQ32)
    vq = orc.quantize(v_bf, cu_k, orc.ROW32)
    dq_ = orc.quantize(do_bf, cu_q, orc.SQ32)
    return orc.attn_bwd_mx(qq[0], qq[1], kq[0], kq[1], vq[0], vq[1], orc.ROW32, dq_[0], dq_[1], o_bf, do_bf,
                           np.asarray(lse, np.float32), cu_q, cu_k, 1, D, c, dq_mode=dq_mode, dq_sigma=sigma)


def pin_delta_from_bf16_do(orc):
    """Delta = rowsum(dO o O) uses the bf16 dO, not its MXFP8 copy. One query, one key, D = 32:
    dO = [256, 2^-12, 0...] shares one block whose code is 127 (amax 256), where 2^-12 lies below half
    the smallest subnormal (2^-10) and quantizes to 0; O = [0, 1, 0...]. So Delta = 2^-12 from the bf16
    dO (0 from the quantized one). K = 0 and LSE = 0 give P = 1; V = 0 gives dP = 0; dS = -2^-12 is one
    1 x 1 block quantized exactly (code 107, payload -256). With Q = 1 everywhere and c = 1,
    dK = dS Q = -2^-12 in every column, dQ = dS K = 0 and dV = P dO_q = [256, 0...]."""
    D = 32
    q = _bf16(np.ones((1, D)))
    k = _bf16(np.zeros((1, D)))
    v = _bf16(np.zeros((1, D)))
    do = np.zeros((1, D), np.float32); do[0, 0] = 256.0; do[0, 1] = 2.0 ** -12
    o = np.zeros((1, D), np.float32); o[0, 1] = 1.0
    out = _bwd_mx(orc, q, k, v, _bf16(do), _bf16(o), [1], [1], D, [[0.0]])
    np.testing.assert_array_equal(out["dk_f"], np.full((1, D), -2.0 ** -12, np.float32))
    assert not out["dq_f"].any()
    expect_dv = np.zeros((1, D), np.float32); expect_dv[0, 0] = 256.0
    np.testing.assert_array_equal(out["dv_f"], expect_dv)


def pin_ds_square_blocks(orc):
    """dS is quantized per 32 x 32 block of the tile, and dK/dQ use the quantized dS. 32 queries, 64 keys
    (two key blocks), D = 32, c = 1, K = 0 and LSE = 0 (P = 1), O = 0 (Delta = 0), so dS = dP = dO V^T.
    dO_i = [1, 1, 0...] for every query; V_j = [1, 1/16 if j odd else 0, 0...] for keys 0-31 and
    [2^-20, 0...] for keys 32-63 (each exact in its ROW32 block). Then:
      key block 0: dS = 1 (even j) or 1.0625 (odd j); the block maximum 1.0625 gives code 119 and
        1.0625 * 256 = 272, a tie between 256 and 288 that rounds to the even mantissa: dS_q = 1 for
        every key of the block (1.0625 would survive only if dS were used unquantized);
      key block 1: dS = 2^-20 everywhere, its own block's code 99 makes it exact; quantized together
        with block 0 (one scale for 32 x 64 or wider) it would be 2^-12 at scale 2^-8, below half the
        smallest subnormal, i.e. 0.
    With Q_i = [0, 1, 0...]: dK_j = sum_i dS_q,ij Q_i = [0, 32 dS_q,j, 0...]: 32 for keys 0-31 and
    32 * 2^-20 = 2^-15 for keys 32-63. dQ = dS_q K = 0; dV_j = sum_i P_q,ij dO_i = [32, 32, 0...]."""
    D, nq, nk = 32, 32, 64
    q = np.zeros((nq, D), np.float32); q[:, 1] = 1.0
    do = np.zeros((nq, D), np.float32); do[:, :2] = 1.0
    v = np.zeros((nk, D), np.float32)
    v[:32, 0] = 1.0
    v[1:32:2, 1] = 1.0 / 16
    v[32:, 0] = 2.0 ** -20
    out = _bwd_mx(orc, _bf16(q), _bf16(np.zeros((nk, D))), _bf16(v), _bf16(do), _bf16(np.zeros((nq, D))), [nq], [nk],
                  D, np.zeros((1, nq)))
    expect_dk = np.zeros((nk, D), np.float32)
    expect_dk[:32, 1] = 32.0
    expect_dk[32:, 1] = 2.0 ** -15
    np.testing.assert_array_equal(out["dk_f"], expect_dk)
    assert not out["dq_f"].any()
    expect_dv = np.zeros((nk, D), np.float32); expect_dv[:, :2] = 32.0
    np.testing.assert_array_equal(out["dv_f"], expect_dv)


def _dq_accumulation_problem(orc, dq_mode, sigma):
    """One query against 256 keys (two KV tiles), D = 32, c = 1. Q = e_0 and K_j = e_1 k_j are
    orthogonal (S = 0, P = 1 with LSE = 0); O = 0 (Delta = 0); dO = e_0 and V_j = [u_j, 0...], so
    dS_0j = u_j. Only key 0 (u = 1, k = 1, tile 0) and key 128 (u = 1.5 * 2^-11, k = 1, tile 1)
    contribute: the per-tile partials of dQ_0 (column 1) are exactly 1 and 1.5 * 2^-11, every value
    exact in its block."""
    D, nk = 32, 256
    q = np.zeros((1, D), np.float32); q[0, 0] = 1.0
    k = np.zeros((nk, D), np.float32); k[0, 1] = 1.0; k[128, 1] = 1.0
    v = np.zeros((nk, D), np.float32); v[0, 0] = 1.0; v[128, 0] = 1.5 * 2.0 ** -11
    do = np.zeros((1, D), np.float32); do[0, 0] = 1.0
    out = _bwd_mx(orc, _bf16(q), _bf16(k), _bf16(v), _bf16(do), _bf16(np.zeros((1, D))), [1], [nk], D, [[0.0]],
                  dq_mode=dq_mode, sigma=sigma)
    assert out["overflow"] == 0
    return out["dq_f"][0, 1]


def pin_dq_accumulators(orc):
    """The dQ reduction over KV tiles in order.
    FP32: acc = 1 + 1.5 * 2^-11, exact in fp32.
    FP16, sigma = 1: acc = fp16(1 + fp16(1.5 * 2^-11)); binary16 has step 2^-10 at 1, and 1.5 * 2^-11 is
      0.75 of that step, so RNE gives 1 + 2^-10 = 1.0009765625.
    FP16, sigma = 2^-20: sigma * 1 = 2^-20 is a binary16 subnormal (16 * 2^-24) and
      sigma * 1.5 * 2^-11 = 1.5 * 2^-31 is below half the smallest subnormal (2^-25), so it rounds to 0:
      acc = 2^-20 and dQ = acc / sigma = 1 exactly (sigma scales the partial before its rounding)."""
    assert _dq_accumulation_problem(orc, 0, 1.0) == np.float32(1.0 + 1.5 * 2.0 ** -11)
    assert _dq_accumulation_problem(orc, 1, 1.0) == np.float32(1.0 + 2.0 ** -10)
    assert _dq_accumulation_problem(orc, 1, 2.0 ** -20) == np.float32(1.0)


def _fp16_probe_values():
    """Doubles around every kind of binary16 boundary: subnormals k 2^-24 and their midpoints, ties in
    every binade, one double ulp either side of each midpoint, the top of the range (65504, the
    65520 overflow midpoint) and values beyond it; both signs."""
    vals = [0.0, 2.0 ** -26, 2.0 ** -25, 2.0 ** -25 * (1 + 2.0 ** -40), 3 * 2.0 ** -25, 2.0 ** -24]
    vals += [k * 2.0 ** -24 for k in range(0, 2048, 7)] + [(k + 0.5) * 2.0 ** -24 for k in range(0, 2048, 5)]
    for e in range(-14, 16):
        step = 2.0 ** (e - 10)
        for m in range(0, 1024, 37):
            mid = 2.0 ** e + (m + 0.5) * step
            vals += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), 2.0 ** e + m * step]
    vals += [65504.0, 65504.0 + 15.999, 65519.999999, 65520.0, 65520.0000001, 65536.0, 1e6, float("inf")]
    vals = np.array(vals, np.float64)
    rng = np.random.default_rng(5)
    vals = np.concatenate([vals, np.ldexp(rng.uniform(1, 2, 4000), rng.integers(-27, 17, 4000))])
    return np.concatenate([vals, -vals])


def pin_fp16_round(orc):
    """binary16 rounding of the FP16 dQ accumulator equals numpy's float16 conversion (an independent
    IEEE round-to-nearest-even from double, with overflow to infinity past 65520)."""
    vals = _fp16_probe_values()
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).astype(np.float64)
    got = np.array([orc.fp16_round(float(x)) for x in vals])
    bad = np.nonzero(~((got == ref) & (np.signbit(got) == np.signbit(ref))))[0]
    assert bad.size == 0, [(vals[i], got[i], ref[i]) for i in bad[:5]]


PINS = {
    "static_p_forward": pin_static_p_forward,
    "static_p_backward": pin_static_p_backward,
    "delta_from_bf16_do": pin_delta_from_bf16_do,
    "ds_square_blocks": pin_ds_square_blocks,
    "dq_accumulators": pin_dq_accumulators,
    "fp16_round": pin_fp16_round,
}


def test_static_p_forward_worked_example():
    pin_static_p_forward(oracle)


def test_static_p_backward_worked_example():
    pin_static_p_backward(oracle)


def test_delta_from_bf16_do_worked_example():
    pin_delta_from_bf16_do(oracle)


def test_ds_square_blocks_worked_example():
    pin_ds_square_blocks(oracle)


def test_dq_accumulators_worked_example():
    pin_dq_accumulators(oracle)


def test_fp16_round_equals_numpy_float16():
    pin_fp16_round(oracle)

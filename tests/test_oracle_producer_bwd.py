"""Pins of the oracle's producer backward: the projection's data and weight gradients and the RMSNorm
backward (CPU only).

Reading pinned (the module's training step past the attention backward; brifing.si item 7: the
producers write FP8 with the scale grid in two layouts so that one payload serves the forward GEMM,
which contracts over channels, and the weight-gradient GEMM, which contracts over tokens;
andresseo.expert "Inside the TMEM Bargain and Zero-Gather Jagged Pipeline": square blocks serve the
plain and the transposed product):
  dX = dY W, dW = dY^T X over the tokens of every sequence, the X and dY operands of dW read through
  their transposed scale grids; RMSNorm y = x r gamma with r = (mean x^2 + eps)^(-1/2) differentiated
  with the quantizers passed straight through.

Each pin is a function of the oracle module (`orc`) so that tests/test_oracle_mutations.py can run it
against broken copies of the oracle. Expected values come from numpy on exactly representable
operands (every product and sum exact), from central finite differences of an FP64 forward written
here, or from an identity of the mathematics; never from the oracle itself.
"""
import numpy as np

import oracle

LENS = [40, 7, 100]  # jagged: partial token blocks in every sequence


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _block_rows(lens):
    """Token block index (from each sequence start) of every token."""
    out, b = [], 0
    for L in lens:
        out += [b + i // 32 for i in range(L)]
        b += (L + 31) // 32
    return np.array(out), b


def block_scaled_ints(rng, lens, C, emin=-6, emax=6):
    """k * 2^e with k integer in [-8, 8] and e drawn per (token block, 32-channel block): every 32 x 32
    block (and every 1 x 32 row block) quantizes exactly, since |k| <= 8 has at most three significant
    bits and the block maximum lands the largest |k| in [256, 512) or below 448."""
    br, nb = _block_rows(lens)
    e = rng.integers(emin, emax + 1, size=(nb, C // 32))
    k = rng.integers(-8, 9, size=(len(br), C)).astype(np.float64)
    return k * np.exp2(e[br][:, np.repeat(np.arange(C // 32), 32)])


def row_scaled_ints(rng, R, C, emin=-6, emax=6):
    """k * 2^e with e drawn per (row, 32-column block): exact under ROW32 quantization."""
    e = rng.integers(emin, emax + 1, size=(R, C // 32))
    k = rng.integers(-8, 9, size=(R, C)).astype(np.float64)
    return k * np.exp2(e[:, np.repeat(np.arange(C // 32), 32)])


def bf16_bits(x):
    """float -> bf16 bit patterns, round to nearest even (numpy, independent of the oracle)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_values(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- projection data gradient ----------------------------------------------------------------

def pin_linear_bwd_data_exact(orc):
    """dX = dY W with exactly representable operands: dy block-scaled integers (SQ32), W^T row-block
    scaled integers (ROW32 along C_out); every sum is exact in FP32, so dX_f32 equals numpy's float64
    product exactly and dX_bf16 its RNE rounding. The operands' exponents differ per block, so reading
    a scale through the wrong block, or W instead of W^T, changes the result."""
    rng = np.random.default_rng(11)
    C_out, C_in = 64, 96
    cu = _cu(LENS)
    dy = block_scaled_ints(rng, LENS, C_out, -3, 3)
    wt = row_scaled_ints(rng, C_in, C_out, -3, 3)
    dyd, dys, _ = orc.quantize(dy.astype(np.float32), cu, orc.SQ32)
    wtd, wts, _ = orc.quantize(wt.astype(np.float32), np.array([0, C_in], np.int32), orc.ROW32)
    dx_bf, dx_f = orc.linear_bwd_data(dyd, dys, wtd, wts, cu)
    expect = (dy @ wt.T).astype(np.float32)
    np.testing.assert_array_equal(dx_f, expect)
    np.testing.assert_array_equal(dx_bf, bf16_bits(expect))


def pin_linear_bwd_data_accumulate(orc):
    """Two data gradients into one input (the key and value projections of one activation): the second
    call adds its product to the first call's bf16 output. With exactly representable operands whose
    products and sums stay exact in bf16 (integers below 2^8), the result is dY1 W1 + dY2 W2 exactly."""
    rng = np.random.default_rng(15)
    C_out, C_in = 64, 96
    cu = _cu(LENS)
    dys = [np.clip(rng.integers(-2, 3, size=(int(cu[-1]), C_out)), -2, 2).astype(np.float64) for _ in range(2)]
    wts = [rng.integers(-1, 2, size=(C_in, C_out)).astype(np.float64) for _ in range(2)]
    q = [(orc.quantize(d.astype(np.float32), cu, orc.SQ32), orc.quantize(w.astype(np.float32),
                                                                          np.array([0, C_in], np.int32), orc.ROW32))
         for d, w in zip(dys, wts)]
    dx1, _ = orc.linear_bwd_data(q[0][0][0], q[0][0][1], q[0][1][0], q[0][1][1], cu)
    dx2, dx2f = orc.linear_bwd_data(q[1][0][0], q[1][0][1], q[1][1][0], q[1][1][1], cu, dx_in=dx1)
    expect = dys[0] @ wts[0].T + dys[1] @ wts[1].T
    assert np.abs(expect).max() < 256
    np.testing.assert_array_equal(dx2f.astype(np.float64), expect)
    np.testing.assert_array_equal(dx2, bf16_bits(expect))


def pin_linear_bwd_data_identity(orc):
    """W = I (exactly representable): dX = deq(dY), bit for bit."""
    rng = np.random.default_rng(12)
    C = 64
    cu = _cu(LENS)
    dy = rng.standard_normal((int(cu[-1]), C)).astype(np.float32)
    dyd, dys, _ = orc.quantize(dy, cu, orc.SQ32)
    wtd, wts, _ = orc.quantize(np.eye(C, dtype=np.float32), np.array([0, C], np.int32), orc.ROW32)
    _, dx_f = orc.linear_bwd_data(dyd, dys, wtd, wts, cu)
    np.testing.assert_array_equal(dx_f, orc.dequantize(dyd, dys, cu, orc.SQ32).astype(np.float32))


# ---- projection weight gradient ----------------------------------------------------------------

def pin_linear_bwd_weight_scaled_blocks(orc):
    """dW = dY^T X over all tokens of a jagged batch, both operands read through their transposed scale
    grids: block-scaled integers (a different power of two per token block and channel block) make every
    sum exact, so dW equals numpy's float64 product exactly; reading the grid untransposed, or a token
    block of the wrong sequence, moves it."""
    rng = np.random.default_rng(13)
    C_out, C_in = 64, 96
    cu = _cu(LENS)
    dy = block_scaled_ints(rng, LENS, C_out, -4, 4)
    x = block_scaled_ints(rng, LENS, C_in, -4, 4)
    dyd, _, dyst = orc.quantize(dy.astype(np.float32), cu, orc.SQ32)
    xd, _, xst = orc.quantize(x.astype(np.float32), cu, orc.SQ32)
    dw = orc.linear_bwd_weight(dyd, dyst, xd, xst, cu)
    np.testing.assert_array_equal(dw, (dy.T @ x).astype(np.float32))


def pin_linear_bwd_adjoint(orc):
    """The three products of the projection agree as adjoints: <dY, X W^T> = <dY W, X> = <dY^T X, W>,
    with the forward Y from the oracle's projection (W quantized ROW32 along C_in) and the data gradient
    from W^T quantized ROW32 along C_out (W has one exponent, so both quantizations are exact)."""
    rng = np.random.default_rng(14)
    C_out, C_in = 64, 96
    cu = _cu(LENS)
    x = block_scaled_ints(rng, LENS, C_in, -2, 2)
    dy = block_scaled_ints(rng, LENS, C_out, -2, 2)
    w = rng.integers(-8, 9, size=(C_out, C_in)).astype(np.float64) * 0.25
    xd, xs, xst = orc.quantize(x.astype(np.float32), cu, orc.SQ32)
    dyd, dys, dyst = orc.quantize(dy.astype(np.float32), cu, orc.SQ32)
    wd, ws, _ = orc.quantize(w.astype(np.float32), np.array([0, C_out], np.int32), orc.ROW32)
    wtd, wts, _ = orc.quantize(np.ascontiguousarray(w.T).astype(np.float32), np.array([0, C_in], np.int32), orc.ROW32)
    *_, y = orc.linear_quantize(xd, xs, wd, ws, cu)
    _, dx = orc.linear_bwd_data(dyd, dys, wtd, wts, cu)
    dw = orc.linear_bwd_weight(dyd, dyst, xd, xst, cu)
    a = float(np.sum(dy * y.astype(np.float64)))
    b = float(np.sum(dx.astype(np.float64) * x))
    c = float(np.sum(dw.astype(np.float64) * w))
    assert a == b == c, (a, b, c)


# ---- RMSNorm backward ----------------------------------------------------------------------------

def _rms_problem(seed, T=3, C=64, xscale=3.0):
    rng = np.random.default_rng(seed)
    xb = bf16_bits(rng.standard_normal((T, C)) * xscale)
    dyb = bf16_bits(rng.standard_normal((T, C)))
    gamma = rng.uniform(0.5, 1.5, C).astype(np.float32)
    return xb, dyb, gamma


def _rms_loss(x, gamma, dy, eps):
    """sum(dy * y) for y = x r gamma, r = (mean x^2 + eps)^(-1/2), all in float64."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return float(np.sum(dy * x * r * gamma))


def pin_rmsnorm_bwd_finite_differences(orc):
    """dx and dgamma against central finite differences of the FP64 forward (x scaled so that r is
    far from 1, which separates r^3 from r^2 and r from 1)."""
    eps = 1e-3
    xb, dyb, gamma = _rms_problem(21)
    x, dy, g = bf16_values(xb), bf16_values(dyb), gamma.astype(np.float64)
    _, dx, dg = orc.rmsnorm_bwd(xb, gamma, eps, dyb)
    fd_x = np.zeros_like(x)
    for t in range(x.shape[0]):
        for c in range(x.shape[1]):
            h = 1e-5 * max(1.0, abs(x[t, c]))
            xp, xm = x.copy(), x.copy()
            xp[t, c] += h
            xm[t, c] -= h
            fd_x[t, c] = (_rms_loss(xp, g, dy, eps) - _rms_loss(xm, g, dy, eps)) / (2 * h)
    fd_g = np.zeros_like(g)
    for c in range(g.size):
        h = 1e-6
        gp, gm = g.copy(), g.copy()
        gp[c] += h
        gm[c] -= h
        fd_g[c] = (_rms_loss(x, gp, dy, eps) - _rms_loss(x, gm, dy, eps)) / (2 * h)
    np.testing.assert_allclose(dx, fd_x, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dg, fd_g, rtol=1e-5, atol=1e-6)


def pin_rmsnorm_bwd_scale_invariance(orc):
    """y is invariant to scaling x up to eps: sum_k dx_k x_k = eps r^3 sum_c gamma_c dy_c x_c per row
    (from d/ds y(s x) at s = 1). A large eps keeps the right side well above FP32 rounding."""
    eps = 0.25
    xb, dyb, gamma = _rms_problem(22, T=4)
    x, dy, g = bf16_values(xb), bf16_values(dyb), gamma.astype(np.float64)
    _, dx, _ = orc.rmsnorm_bwd(xb, gamma, eps, dyb)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    lhs = np.sum(dx.astype(np.float64) * x, axis=1)
    rhs = eps * r ** 3 * np.sum(g * dy * x, axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-4, atol=1e-6)


PINS = {
    "linear_bwd_data_exact": pin_linear_bwd_data_exact,
    "linear_bwd_data_identity": pin_linear_bwd_data_identity,
    "linear_bwd_data_accumulate": pin_linear_bwd_data_accumulate,
    "linear_bwd_weight_scaled_blocks": pin_linear_bwd_weight_scaled_blocks,
    "linear_bwd_adjoint": pin_linear_bwd_adjoint,
    "rmsnorm_bwd_finite_differences": pin_rmsnorm_bwd_finite_differences,
    "rmsnorm_bwd_scale_invariance": pin_rmsnorm_bwd_scale_invariance,
}


def test_linear_bwd_data_exact():
    pin_linear_bwd_data_exact(oracle)


def test_linear_bwd_data_accumulate():
    pin_linear_bwd_data_accumulate(oracle)


def test_linear_bwd_data_identity():
    pin_linear_bwd_data_identity(oracle)


def test_linear_bwd_weight_scaled_blocks():
    pin_linear_bwd_weight_scaled_blocks(oracle)


def test_linear_bwd_adjoint():
    pin_linear_bwd_adjoint(oracle)


def test_rmsnorm_bwd_finite_differences():
    pin_rmsnorm_bwd_finite_differences(oracle)


def test_rmsnorm_bwd_scale_invariance():
    pin_rmsnorm_bwd_scale_invariance(oracle)


def test_rmsnorm_bwd_bf16_is_rounded_f32():
    """The bf16 dx is the RNE rounding of the FP32 dx."""
    xb, dyb, gamma = _rms_problem(23)
    dxb, dx, _ = oracle.rmsnorm_bwd(xb, gamma, 1e-6, dyb)
    np.testing.assert_array_equal(dxb, bf16_bits(dx))

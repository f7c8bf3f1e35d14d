"""MXFP4 quantization for the CPU oracle: OCP microscaling blocks of 32 elements, each element an
FP4 E2M1 number, each block scaled by one E8M0 byte.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the test suite, the smoke
check and the benchmark's CPU-baseline leg, never by the product path.

The pages name MXFP6 and MXFP4 as the next, lower precisions for the attention
(brifing.si, "Future directions"; theclarity.today paragraph 1: the block-scaled matrix units run
MXFP8, MXFP6 and MXFP4). The element format and the scale rule are those of the OCP MX
specification, which the pages' MXFP8 rule instantiates for E4M3 (kongchang.com, "Why MXFP8"):
  * E2M1: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0; magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7; no infinity, no NaN.
  * Block scale: code = clamp(exponent_field(amax) - 2, 0, 254), 2 being the exponent of E2M1's
    largest magnitude (6 = 1.5 * 2^2); 255 (NaN) when the block holds a NaN or an infinity.
  * Payload: the element x * 2^(127 - code) rounded to the nearest E2M1 magnitude, ties to the even
    code, saturated at 6; the sign bit is x's sign bit (so -0.0 and negatives that round to zero give
    code 8). A NaN block's payload is 0.
Reading (stated in the design notes): only the ROW32 shape (1 x 32 along the columns) is provided,
for Q and K of the forward's S = Q K^T, whose contraction runs along D.

Layout: payload [T, C/2] bytes, element 2i in the low nibble of byte i, element 2i + 1 in the high
nibble; scales [T, C/32] (the ROW32 layout of the MXFP8 quantizer).
"""
import numpy as np

E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_EMAX = 2  # exponent of the largest magnitude


def e2m1_decode(code):
    """Value of a 4-bit E2M1 code."""
    code = int(code) & 0xF
    mag = E2M1_MAGNITUDES[code & 7]
    return -mag if code & 8 else mag


def e2m1_encode(v):
    """Nearest E2M1 code to the float v (ties to the even code, saturation at 6, sign kept)."""
    v = float(v)
    sign = 8 if np.signbit(v) else 0
    a = min(abs(v), E2M1_MAGNITUDES[-1])  # saturation: magnitudes beyond 6 become 6
    best, best_d = 0, None
    for c, m in enumerate(E2M1_MAGNITUDES):
        d = abs(a - m)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return sign | best


def e2m1_encode_array(v):
    """e2m1_encode over an array (the same nearest-magnitude rule, written with numpy)."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), E2M1_MAGNITUDES[-1])
    mags = np.array(E2M1_MAGNITUDES)
    d = np.abs(a[..., None] - mags)
    near = d == d.min(axis=-1, keepdims=True)
    # one or two nearest magnitudes; of two (a tie) take the even code
    prefer = near * (1 + (np.arange(8) % 2 == 0))
    code = np.argmax(prefer, axis=-1).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _exponent_field(a):
    """Biased binary32 exponent field of a non-negative finite float (bf16 values are exact)."""
    return int((np.array([a], np.float32).view(np.uint32)[0] >> 23) & 0xFF)


def scale_code(block):
    """E8M0 code of a block of floats (numpy float64), 255 if any element is not finite."""
    if not np.all(np.isfinite(block)):
        return 255
    amax = float(np.max(np.abs(block))) if block.size else 0.0
    return min(max(_exponent_field(amax) - E2M1_EMAX, 0), 254)


def quantize_row32(x_bf16):
    """x_bf16: uint16 bf16 bits [T, C], C a multiple of 32. Returns (payload uint8 [T, C/2],
    scale uint8 [T, C/32])."""
    x = _bf16_to_f64(x_bf16)
    T, C = x.shape
    assert C % 32 == 0
    data = np.zeros((T, C // 2), np.uint8)
    scale = np.zeros((T, C // 32), np.uint8)
    nib = np.zeros((T, C), np.uint8)
    for t in range(T):
        for b in range(C // 32):
            blk = x[t, 32 * b:32 * b + 32]
            code = scale_code(blk)
            scale[t, b] = code
            if code != 255:  # a NaN block keeps payload 0
                nib[t, 32 * b:32 * b + 32] = e2m1_encode_array(blk * 2.0 ** (127 - code))
    data[:] = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return data, scale


def dequantize_row32(data, scale):
    """Inverse of quantize_row32 up to the rounding: float64 [T, C] (NaN for NaN blocks)."""
    T, C2 = data.shape
    nib = np.empty((T, 2 * C2), np.uint8)
    nib[:, 0::2] = data & 0xF
    nib[:, 1::2] = data >> 4
    table = np.array([e2m1_decode(c) for c in range(16)])
    code = np.repeat(np.asarray(scale, np.int64), 32, axis=1)
    out = table[nib] * np.exp2(code - 127.0)
    out[code == 255] = np.nan
    return out


def attn_fwd_qk_fp4(q4, q_scale, k4, k_scale, v, v_scale, cu_q, cu_k, H, D, softmax_scale, causal=False,
                    p_scale=1):
    """The forward with Q and K in MXFP4 (ROW32, this module's layout) and V in MXFP8 COL32 (the MXFP8
    quantizer's compact layout): every operand dequantized to float64, then the oracle's forward
    (S, online softmax, P quantized to E4M3, O). Returns (o_bf16, o_f32, lse) as attn_fwd_f64."""
    from . import COL32, attn_fwd_f64, dequantize
    q = dequantize_row32(q4, q_scale)
    k = dequantize_row32(k4, k_scale)
    vd = dequantize(v, v_scale, cu_k, COL32)
    return attn_fwd_f64(q, k, vd, cu_q, cu_k, H, D, softmax_scale, causal, quant_p=p_scale)

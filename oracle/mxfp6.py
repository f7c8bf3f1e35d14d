"""MXFP6 quantization for the CPU oracle: OCP microscaling blocks of 32 elements, each element an
FP6 E2M3 number, each block scaled by one E8M0 byte.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the test suite, the smoke
check and the benchmark's CPU-baseline leg, never by the product path.

The pages name MXFP6 beside MXFP4 as the next precisions for the attention (brifing.si, "Future
directions"; theclarity.today paragraph 1). The element format and the scale rule are the OCP MX
ones, as for MXFP8 (kongchang.com, "Why MXFP8") and MXFP4 (mxfp4.py):
  * E2M3: sign bit 5, exponent bits 4-3 (bias 1), mantissa bits 2-0; magnitude f/8 for exponent
    field 0 (subnormal), 2^(e-1) (1 + f/8) otherwise: 0 .. 0.875 in steps of 1/8, 1 .. 1.875 in
    steps of 1/8, 2 .. 3.75 in steps of 1/4, 4 .. 7.5 in steps of 1/2; no infinity, no NaN.
  * Block scale: code = clamp(exponent_field(amax) - 2, 0, 254) (7.5 = 1.875 * 2^2); 255 when the
    block holds a NaN or an infinity.
  * Element: the magnitude nearest to |x| * 2^(127 - code), ties to the even code, saturated at 7.5;
    the sign bit is x's sign bit. A NaN block's payload is 0.
Layout: a block's 32 six-bit codes fill 24 bytes as one little-endian bit string (code j at bits
6j .. 6j + 5); the blocks of a row go in pairs (2p, 2p + 1), 48 bytes per pair: bytes 0-15 of block 2p,
bytes 0-15 of block 2p + 1, bytes 16-23 of block 2p, bytes 16-23 of block 2p + 1 (so that each block
is one 16-byte piece and one 8-byte piece). Payload [T, 3 C / 4] (C a multiple of 64), scales
[T, C / 32] (ROW32).
"""
import numpy as np

E2M3_EMAX = 2


def e2m3_value(code):
    """Value of a 6-bit E2M3 code, from the format's definition."""
    code = int(code) & 0x3F
    s, e, f = code >> 5, (code >> 3) & 3, code & 7
    v = f / 8.0 if e == 0 else 2.0 ** (e - 1) * (1 + f / 8.0)
    return -v if s else v


E2M3_MAGNITUDES = tuple(e2m3_value(c) for c in range(32))


def e2m3_encode(v):
    """Nearest E2M3 code to the float v (ties to the even code, saturation at 7.5, sign kept)."""
    v = float(v)
    sign = 32 if np.signbit(v) else 0
    a = min(abs(v), E2M3_MAGNITUDES[-1])
    best, best_d = 0, None
    for c, m in enumerate(E2M3_MAGNITUDES):
        d = abs(a - m)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return sign | best


def e2m3_encode_array(v):
    """e2m3_encode over an array (the same nearest-magnitude rule, written with numpy)."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), E2M3_MAGNITUDES[-1])
    mags = np.array(E2M3_MAGNITUDES)
    d = np.abs(a[..., None] - mags)
    near = d == d.min(axis=-1, keepdims=True)
    prefer = near * (1 + (np.arange(32) % 2 == 0))  # of two nearest magnitudes, the even code
    code = np.argmax(prefer, axis=-1).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 5)


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _exponent_field(a):
    return int((np.array([a], np.float32).view(np.uint32)[0] >> 23) & 0xFF)


def scale_code(block):
    if not np.all(np.isfinite(block)):
        return 255
    amax = float(np.max(np.abs(block))) if block.size else 0.0
    return min(max(_exponent_field(amax) - E2M3_EMAX, 0), 254)


def pack_block(codes):
    """32 six-bit codes -> 24 bytes, code j at bits 6j .. 6j + 5 of a little-endian bit string."""
    bits = 0
    for j, c in enumerate(codes):
        bits |= (int(c) & 0x3F) << (6 * j)
    return np.frombuffer(bits.to_bytes(24, "little"), np.uint8)


def unpack_block(b):
    bits = int.from_bytes(bytes(np.asarray(b, np.uint8)), "little")
    return [(bits >> (6 * j)) & 0x3F for j in range(32)]


def block_bytes(b):
    """Byte positions, in a row's payload, of block b's 24-byte bit string (in bit-string order)."""
    p, a = divmod(b, 2)
    return list(range(48 * p + 16 * a, 48 * p + 16 * a + 16)) + list(range(48 * p + 32 + 8 * a, 48 * p + 40 + 8 * a))


def quantize_row32(x_bf16):
    """x_bf16: uint16 bf16 bits [T, C], C a multiple of 64. Returns (payload uint8 [T, 3C/4],
    scale uint8 [T, C/32])."""
    x = _bf16_to_f64(x_bf16)
    T, C = x.shape
    assert C % 64 == 0
    data = np.zeros((T, 3 * C // 4), np.uint8)
    scale = np.zeros((T, C // 32), np.uint8)
    for t in range(T):
        for b in range(C // 32):
            blk = x[t, 32 * b:32 * b + 32]
            code = scale_code(blk)
            scale[t, b] = code
            if code != 255:  # a NaN block keeps payload 0
                data[t, block_bytes(b)] = pack_block(e2m3_encode_array(blk * 2.0 ** (127 - code)))
    return data, scale


def dequantize_row32(data, scale):
    T = data.shape[0]
    C = data.shape[1] * 4 // 3
    out = np.empty((T, C), np.float64)
    for t in range(T):
        for b in range(C // 32):
            code = int(scale[t, b])
            codes = unpack_block(data[t, block_bytes(b)])
            out[t, 32 * b:32 * b + 32] = (np.nan if code == 255 else
                                         np.array([e2m3_value(c) for c in codes]) * 2.0 ** (code - 127))
    return out


def attn_fwd_qk_fp6(q6, q_scale, k6, k_scale, v, v_scale, cu_q, cu_k, H, D, softmax_scale, causal=False,
                    p_scale=1):
    """The forward with Q and K in MXFP6 E2M3 (ROW32, this module's layout) and V in MXFP8 COL32:
    every operand dequantized to float64, then the oracle's forward. Returns (o_bf16, o_f32, lse)."""
    from . import COL32, attn_fwd_f64, dequantize
    q = dequantize_row32(q6, q_scale)
    k = dequantize_row32(k6, k_scale)
    vd = dequantize(v, v_scale, cu_k, COL32)
    return attn_fwd_f64(q, k, vd, cu_q, cu_k, H, D, softmax_scale, causal, quant_p=p_scale)

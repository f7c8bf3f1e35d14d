"""Pins of the MXFP6 (E2M3 elements, E8M0 block scales) quantizer of the oracle, against what the
format's definition fixes (OCP MX specification; the pages name MXFP6 with MXFP4 as the next
precisions: brifing.si "Future directions", theclarity.today paragraph 1): the magnitude grid written
out from the format's binades, brute-force nearest rounding with ties to even, saturation, the scale
rule, the 6-bit packing and pair layout of a hand-built row, and the round-trip bound."""
import numpy as np

import synth
from oracle import mxfp6 as m

# the 32 magnitudes, binade by binade: subnormals f/8, then [1, 2) in 1/8, [2, 4) in 1/4, [4, 7.5] in 1/2
GRID = list(np.arange(0, 1, 1 / 8)) + list(np.arange(1, 2, 1 / 8)) + list(np.arange(2, 4, 1 / 4)) + \
    list(np.arange(4, 8, 1 / 2))


def test_grid_matches_the_binades():
    assert len(GRID) == 32
    assert list(m.E2M3_MAGNITUDES) == GRID
    for c in range(64):
        assert m.e2m3_value(c) == (-GRID[c & 31] if c & 32 else GRID[c & 31])


def test_encode_round_trips_every_code():
    for c in range(64):
        v = -0.0 if c == 32 else m.e2m3_value(c)
        assert m.e2m3_encode(v) == c, c


def test_nearest_by_brute_force_and_ties_to_even():
    rng = np.random.default_rng(9)
    for v in rng.uniform(-8, 8, 3000):
        got = abs(m.e2m3_value(m.e2m3_encode(v)))
        assert all(abs(abs(v) - got) <= abs(abs(v) - g) for g in GRID if g <= 7.5), v
    for c in range(31):
        mid = (GRID[c] + GRID[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert m.e2m3_encode(mid) == even and m.e2m3_encode(-mid) == 32 | even, (mid, c)


def test_saturation_and_sign():
    for v in (7.5, 7.74, 7.76, 8.0, 1e30):
        assert m.e2m3_encode(v) == 31 and m.e2m3_encode(-v) == 63
    assert m.e2m3_encode(-0.0) == 32 and m.e2m3_encode(-0.05) == 32 and m.e2m3_encode(0.07) == 1


def test_array_encoder_matches_scalar():
    rng = np.random.default_rng(10)
    vals = np.concatenate([rng.normal(0, 3, 20000), [(GRID[c] + GRID[c + 1]) / 2 for c in range(31)], [-0.0]])
    np.testing.assert_array_equal(m.e2m3_encode_array(vals), [m.e2m3_encode(v) for v in vals])


def bf16(vals):
    a = np.asarray(vals, np.float32).view(np.uint32)
    assert np.all(a & 0xFFFF == 0), "values must be bf16-exact"
    return (a >> 16).astype(np.uint16)


def test_scale_rule():
    for amax, code in ((7.5, 127), (4.0, 127), (1.0, 125), (3.0, 126), (2.0 ** -100, 25)):
        x = np.zeros((1, 64), np.float32)
        x[0, 9] = amax
        _, s = m.quantize_row32(bf16(x))
        assert s[0, 0] == code, (amax, s[0, 0])
    for bad in (0x7FC0, 0xFF80):
        x = bf16(np.ones((1, 64), np.float32))
        x[0, 33] = bad
        d, s = m.quantize_row32(x)
        # block 1's bytes in the pair layout: 16-31 and 40-47
        assert s[0, 1] == 255 and not d[0, 16:32].any() and not d[0, 40:48].any() and s[0, 0] == 125


def test_hand_built_block_packing():
    # block 0: amax 3.75 (exponent field 128) -> code 126, scale 2^-1: x = 1 -> 2.0 (code 16), -0.1875 ->
    # -0.375 (32 | 3), 3.75 -> 7.5 (31), 0.5 -> 1.0 (8), the rest 0: bits 16 | (35 << 6) | (31 << 12) |
    # (8 << 18). Block 1: x[63] = 4 (code 127, scale 1) -> code 24 at bits 186..191 (byte 23: 24 << 2).
    # Pair layout: bytes 0-15 block 0, 16-31 block 1, 32-39 block 0's bytes 16-23, 40-47 block 1's.
    x = np.zeros((1, 64), np.float32)
    x[0, :4] = [1.0, -0.1875, 3.75, 0.5]
    x[0, 63] = 4.0
    d, s = m.quantize_row32(bf16(x))
    assert list(s[0]) == [126, 127]
    b0 = np.frombuffer((16 | (35 << 6) | (31 << 12) | (8 << 18)).to_bytes(24, "little"), np.uint8)
    b1 = np.frombuffer((24 << 186).to_bytes(24, "little"), np.uint8)
    want = np.concatenate([b0[:16], b1[:16], b0[16:], b1[16:]])
    np.testing.assert_array_equal(d[0], want)
    assert d[0, 47] == 24 << 2 and not d[0, 16:32].any()
    y = m.dequantize_row32(d, s)[0]
    np.testing.assert_array_equal(y[:4], [1.0, -0.1875, 3.75, 0.5])
    assert y[63] == 4.0 and not y[4:63].any()


def test_round_trip_error_bound():
    x = synth.normal_bf16(5, 1, (64, 256))
    d, s = m.quantize_row32(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = m.dequantize_row32(d, s)
    scale = np.exp2(np.repeat(s.astype(np.float64), 32, axis=1) - 127)
    a = np.abs(xf) / scale
    half = np.where(a < 2, 1 / 16, np.where(a < 4, 1 / 8, 1 / 4))
    bound = np.where(a > 7.5, a - 7.5, half) * scale
    assert np.all(np.abs(y - xf) <= bound + 1e-300)

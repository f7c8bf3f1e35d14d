"""Pins of the MXFP4 (E2M1 elements, E8M0 block scales) quantizer of the oracle, against what the
format's definition fixes (OCP MX specification; the pages name MXFP4 as the next precision:
brifing.si "Future directions", theclarity.today paragraph 1), not against the oracle itself:
the closed-form value of every code, brute-force nearest rounding with ties to even, saturation, the
scale rule on hand-picked blocks, a hand-worked block, the nibble order, and the error bound of the
round trip."""
import numpy as np

import synth
from oracle import mxfp4 as m


def closed_form(code):
    """E2M1: exponent field e (bias 1), mantissa bit f: 2^(e-1) (1 + f/2) for e >= 1, f/2 for e = 0."""
    s, e, f = code >> 3, (code >> 1) & 3, code & 1
    v = 2.0 ** (e - 1) * (1 + f / 2) if e else f / 2
    return -v if s else v


def test_decode_matches_closed_form():
    for c in range(16):
        assert m.e2m1_decode(c) == closed_form(c), c
    assert sorted(set(abs(closed_form(c)) for c in range(16))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_encode_round_trips_every_code():
    for c in range(16):
        assert m.e2m1_encode(closed_form(c) if c != 8 else -0.0) == c, c


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.uniform(-7, 7, 4000), rng.uniform(-1, 1, 1000)])
    grid = [closed_form(c) for c in range(8)]
    for v in vals:
        got = abs(closed_form(m.e2m1_encode(v)))
        assert all(abs(abs(v) - got) <= abs(abs(v) - g) + 0.0 for g in grid), v


def test_ties_go_to_the_even_code():
    # midpoints of consecutive magnitudes, from the closed form, and the even code of each pair
    mags = [closed_form(c) for c in range(8)]
    for c in range(7):
        mid = (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert m.e2m1_encode(mid) == even, (mid, c)
        assert m.e2m1_encode(-mid) == 8 | even, (-mid, c)


def test_saturation_and_sign():
    for v in (6.0, 6.5, 7.99, 100.0, 1e30):
        assert m.e2m1_encode(v) == 7 and m.e2m1_encode(-v) == 15
    assert m.e2m1_encode(-0.0) == 8 and m.e2m1_encode(-0.1) == 8 and m.e2m1_encode(0.1) == 0


def test_array_encoder_matches_scalar():
    rng = np.random.default_rng(8)
    vals = np.concatenate([rng.normal(0, 3, 20000), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.0]])
    want = np.array([m.e2m1_encode(v) for v in vals], np.uint8)
    np.testing.assert_array_equal(m.e2m1_encode_array(vals), want)


def bf16(vals):
    a = np.asarray(vals, np.float32).view(np.uint32)
    assert np.all(a & 0xFFFF == 0), "values must be bf16-exact"
    return (a >> 16).astype(np.uint16)


def test_scale_rule_on_chosen_blocks():
    # the largest magnitude 6 = 1.5 * 2^2: a block maximum amax = 1.5 * 2^k gets code 127 + k - 2 + 2
    # ... i.e. exponent_field(amax) - 2, which maps amax into [4, 8) (values in [6, 8) saturate)
    for amax, code in ((6.0, 127), (4.0, 127), (7.5, 127), (1.0, 125), (0.5, 124), (2.0 ** -100, 25)):
        x = np.zeros((1, 32), np.float32)
        x[0, 5] = amax
        _, s = m.quantize_row32(bf16(x))
        assert s[0, 0] == code, (amax, s[0, 0])
    # all zero: code 0, payload 0; bf16 subnormal maxima clamp at code 0
    d, s = m.quantize_row32(np.zeros((1, 32), np.uint16))
    assert s[0, 0] == 0 and not d.any()
    x = np.zeros((1, 32), np.uint16)
    x[0, 3] = 0x0001  # smallest bf16 subnormal
    _, s = m.quantize_row32(x)
    assert s[0, 0] == 0
    # NaN or Inf anywhere: code 255, payload 0 (the other block untouched)
    for bad in (0x7FC0, 0x7F80, 0xFF80):
        x = bf16(np.ones((1, 64), np.float32))
        x[0, 40] = bad
        d, s = m.quantize_row32(x)
        assert s[0, 1] == 255 and not d[0, 16:].any() and s[0, 0] == 125


def test_hand_worked_block():
    # x = [1, -0.296875, 0.703125, 2.625, 0...]: amax 2.625 (exponent field 128) -> code 126, scale 2^-1;
    # scaled 2, -0.59375, 1.40625, 5.25 -> codes 4, 8|1, 3, 7 (nearest 2, 0.5, 1.5, 6) -> values
    # 1, -0.25, 0.75, 3; bytes: (4 | 9 << 4) = 0x94, (3 | 7 << 4) = 0x73
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [1.0, -0.296875, 0.703125, 2.625]
    d, s = m.quantize_row32(bf16(x))
    assert s[0, 0] == 126
    assert d[0, 0] == 0x94 and d[0, 1] == 0x73 and not d[0, 2:].any()
    np.testing.assert_array_equal(m.dequantize_row32(d, s)[0, :4], [1.0, -0.25, 0.75, 3.0])


def test_round_trip_error_bound():
    # per element: half the E2M1 spacing at its magnitude (0.5 below 2, 1 in [2, 4), 2 in [4, 6]),
    # times the block scale; beyond 6 (scaled) the error is the excess over 6 (saturation)
    x = synth.normal_bf16(3, 1, (64, 256))
    d, s = m.quantize_row32(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = m.dequantize_row32(d, s)
    scale = np.exp2(np.repeat(s.astype(np.float64), 32, axis=1) - 127)
    a = np.abs(xf) / scale
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = np.where(a > 6, a - 6, half) * scale
    assert np.all(np.abs(y - xf) <= bound + 1e-300)
    assert np.all(a < 8)  # the scale rule puts every block maximum below 8

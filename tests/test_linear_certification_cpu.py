"""CPU checks of the certified-mismatch comparison used for the projection GEMM + quantize
producer: it accepts the oracle's own output, accepts a byte moved across a rounding midpoint
that lies inside the accumulation-error band, and rejects a byte that no value in the band
encodes to (a planted mistake, made on the CPU copy of the output)."""
import numpy as np
import pytest

import oracle
from mx_cases import LINEAR_DELTA_REL, LinearCase, certify_linear, e4m3_table


@pytest.fixture(scope="module")
def case():
    lc = LinearCase(31, [40, 90], 256, 128)
    return lc, lc.run_oracle()


def test_oracle_output_certifies_itself(case):
    lc, (d, s, st, y, yabs) = case
    n_pay, n_scale = certify_linear(d.copy(), s.copy(), st.copy(), d, s, y, yabs, lc.cu, "self")
    assert (n_pay, n_scale) == (0, 0)


def test_planted_wrong_byte_is_rejected(case):
    lc, (d, s, st, y, yabs) = case
    bad = d.copy()
    bad[3, 7] ^= 0x04  # two E4M3 steps away from the oracle's byte
    with pytest.raises(AssertionError):
        certify_linear(bad, s, st, d, s, y, yabs, lc.cu, "planted")


def test_planted_wrong_scale_is_rejected(case):
    lc, (d, s, st, y, yabs) = case
    bad = s.copy()
    bad[1, 2] += 1
    with pytest.raises(AssertionError):
        certify_linear(d, bad, bad.T.copy(), d, s, y, yabs, lc.cu, "planted scale")


def test_neighbour_byte_inside_band_is_certified(case):
    """Move the element nearest to a rounding midpoint (relative to the band) to the other side's
    code: the comparison must certify it."""
    lc, (d, s, st, y, yabs) = case
    dec = e4m3_table()
    cu = lc.cu
    # scale code of each element's block
    br_of = np.concatenate([np.arange(int(cu[i + 1] - cu[i])) // 32 + sum((int(cu[j + 1] - cu[j]) + 31) // 32
                                                                         for j in range(i))
                            for i in range(len(cu) - 1)])
    code = s[br_of][:, np.repeat(np.arange(d.shape[1] // 32), 32)].astype(np.int64)
    v = y * np.ldexp(1.0, 127 - code)
    lo = oracle.e4m3_encode_array(((y - LINEAR_DELTA_REL * yabs) * np.ldexp(1.0, 127 - code)).astype(np.float32))
    hi = oracle.e4m3_encode_array(((y + LINEAR_DELTA_REL * yabs) * np.ldexp(1.0, 127 - code)).astype(np.float32))
    lo, hi = lo.reshape(d.shape), hi.reshape(d.shape)
    cand = np.nonzero((lo != hi) & (np.abs(v) < 400))
    assert cand[0].size > 0
    t, c = cand[0][0], cand[1][0]
    moved = d.copy()
    moved[t, c] = lo[t, c] if moved[t, c] != lo[t, c] else hi[t, c]
    assert dec[moved[t, c]] != dec[d[t, c]]
    n_pay, _ = certify_linear(moved, s, st, d, s, y, yabs, cu, "moved")
    assert n_pay == 1

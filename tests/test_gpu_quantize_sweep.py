"""Exhaustive MX quantizer sweep on the GPU: every bf16 bit pattern, at several block scales, in all
three block layouts, bit-exact against the oracle.

The input is a jagged batch of 288-token sequences of 256 columns. Inside each sequence, every element
whose row (from the sequence start) or column is a multiple of 32 holds that sequence's anchor value,
so every ROW32, COL32 and SQ32 block contains the anchor; the other elements hold bf16 patterns no
larger in magnitude than the anchor, so the anchor fixes the block's scale code and each pattern is
quantized at that code. The patterns of each sequence cycle through the whole set (every finite
pattern with |p| <= |anchor|, both signs) in a seeded order. Anchors:
  3.39e38 (the largest finite bf16; code 246: nearly everything underflows, signed zeros)
  256 (code 127), 1.875 (code 119: 448 < 1.875 * 256 = 480, the saturation band),
  1.0 (code 119: ties at every binade, subnormal outputs), 2^-100 (code 19),
  2^-126 (the clamp to code 0; bf16 subnormal inputs);
plus a sequence without anchor whose patterns have magnitudes in [2^-20, 2^10) (every block's own
maximum sets its code; maxima land anywhere in [256, 512)) and a sequence whose patterns include all 256 NaN and infinity patterns (blocks -> code 255,
payload 0x7F).
"""
import numpy as np
import pytest

import oracle
import synth
from mx_cases import cu_dev, gpu_quantize, say, to_dev_bf16

pytestmark = pytest.mark.gpu

L, C = 288, 256
ANCHORS = [0x7F7F, 0x4380, 0x3FF0, 0x3F80, 0x0D80, 0x0080]


def _patterns():
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allp[(allp & 0x7F80) != 0x7F80]
    return allp, finite


def _sequence(anchor, pool, seed):
    """One L x C sequence: the anchor on rows and columns that are multiples of 32 (when given), the
    pool's patterns on the other positions, each at least once (there are more positions than
    patterns), in a seeded order."""
    x = np.zeros((L, C), np.uint16)
    free = np.ones((L, C), bool)
    if anchor is not None:
        free[np.arange(L) % 32 == 0, :] = False
        free[:, np.arange(C) % 32 == 0] = False
        x[~free] = anchor
    rng = np.random.default_rng(seed)
    npos = int(free.sum())
    assert npos >= pool.size
    x[free] = rng.permutation(np.resize(rng.permutation(pool), npos))
    return x


def sweep_matrix():
    allp, finite = _patterns()
    mag = finite & 0x7FFF
    seqs = []
    for i, a in enumerate(ANCHORS):
        seqs.append(_sequence(a, finite[mag <= a], 100 + i))
    # no anchor: patterns with magnitudes in [2^-20, 2^10), so the blocks' own maxima vary
    mid = finite[(mag >= 0x3580) & (mag < 0x4480)]
    seqs.append(_sequence(None, mid, 200))
    # the NaN and infinity patterns over the first third of a sequence's rows (the rest stays finite)
    x = _sequence(None, mid, 201)
    nonfinite = allp[(allp & 0x7F80) == 0x7F80]
    rng = np.random.default_rng(202)
    pos = rng.choice((L // 3) * C, size=nonfinite.size, replace=False)
    x.reshape(-1)[pos] = nonfinite
    seqs.append(x)
    return np.concatenate(seqs), synth.cu_seqlens([L] * len(seqs))


def test_sweep_covers_every_pattern():
    x, _ = sweep_matrix()
    assert np.unique(x).size == 1 << 16


@pytest.mark.parametrize("mode", [oracle.ROW32, oracle.COL32, oracle.SQ32])
def test_quantize_sweep_bit_exact(mode):
    x, cu = sweep_matrix()
    say(f"quantize sweep mode={mode}: {x.shape[0]} tokens x {C}, {len(cu) - 1} sequences")
    d_ref, s_ref, st_ref = oracle.quantize(x, cu, mode)
    data, scale, scale_t = gpu_quantize(to_dev_bf16(x), cu, cu_dev(cu), mode, want_scale_t=(mode == oracle.SQ32))
    np.testing.assert_array_equal(scale.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(data.cpu().numpy(), d_ref)
    if mode == oracle.SQ32:
        np.testing.assert_array_equal(scale_t.cpu().numpy(), st_ref)
    codes = np.unique(s_ref)
    say(f"  {codes.size} distinct codes from {codes.min()} to {codes.max()}, {np.unique(d_ref).size} distinct bytes")


@pytest.mark.parametrize("fmt", ["e2m1", "e2m3"])
def test_small_format_sweep_bit_exact(fmt):
    """The same matrix through the MXFP4 and MXFP6 ROW32 quantizers: every bf16 pattern at the codes the
    anchors fix for these formats (code = exponent field - 2), the saturation bands above 6 and 7.5 (the
    blocks without anchor put their maxima anywhere in [4, 8) after scaling), subnormal inputs at code 0,
    and the NaN/Inf blocks (code 255, payload 0)."""
    from test_gpu_mxfp4 import FORMATS, gpu_quantize_small
    x, _ = sweep_matrix()
    say(f"{fmt} quantize sweep: {x.shape[0]} tokens x {C}")
    d, s = gpu_quantize_small(to_dev_bf16(x), fmt)
    d_ref, s_ref = FORMATS[fmt][2].quantize_row32(x)
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(d, d_ref)
    codes = np.unique(s_ref)
    say(f"  {codes.size} distinct codes from {codes.min()} to {codes.max()}, {np.unique(d_ref).size} distinct bytes")

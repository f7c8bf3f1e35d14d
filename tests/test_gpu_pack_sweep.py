"""Every fp32 bit pattern through the device's E4M3 packs, byte-exact against the oracle's encoder.

The kernels turn fp32 values into E4M3 bytes with three routines (unscaled and saturating; x / sc
with a power-of-two sc and saturating; and the unclamped pack of values known to lie in
[-448, 448]). mxfa_e4m3_pack_patterns runs each routine over consecutive bit patterns. The oracle's
encoder (round to nearest even at every exponent, subnormals included, saturation at 448, the sign
kept on zero results; itself pinned by brute-force search over all codes) gives the expected byte.
For the scaled pack the oracle encodes x * (1 / sc) computed in fp32: for a power-of-two sc that
product is x / sc exactly, except where it overflows (to infinity, which saturates like the exact
value above 448) or falls below 2^-126 (where the exact value also encodes as a signed zero).
NaN patterns are not compared (the kernels mark NaN blocks with scale code 255), nor, for the
in-range pack, patterns of magnitude above 448.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import precision_mxfp8_block_amd as mx
from mx_cases import say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27
THREADS = max(1, min(16, os.cpu_count() or 1))


def _oracle_bytes(y, pool):
    out = np.empty(y.size, np.uint8)
    lib = oracle._load()
    step = -(-y.size // THREADS)

    def part(i):
        lo, hi = i * step, min(y.size, (i + 1) * step)
        if lo < hi:
            lib.orc_e4m3_encode_array(y[lo:].ctypes.data, hi - lo, out[lo:].ctypes.data)

    list(pool.map(part, range(THREADS)))  # ctypes releases the GIL during each call
    return out


def _sweep(variant, sc, start, count):
    dev = torch.full((CHUNK,), 0xA5, dtype=torch.uint8, device="cuda")
    checked = 0
    with ThreadPoolExecutor(THREADS) as pool:
        for off in range(0, count, CHUNK):
            n = min(CHUNK, count - off)
            first = (start + off) & 0xFFFFFFFF
            mx.mxfa_e4m3_pack_patterns(first, n, variant, sc, dev)
            got = dev[:n].cpu().numpy()
            bits = (np.arange(n, dtype=np.uint64) + first).astype(np.uint32)
            x = bits.view(np.float32)
            with np.errstate(over="ignore", under="ignore", invalid="ignore"):
                y = x * np.float32(1.0 / sc) if variant == 1 else x
            ref = _oracle_bytes(np.ascontiguousarray(y), pool)
            keep = ~np.isnan(x)
            if variant == 2:
                keep &= np.abs(x) <= 448.0
            bad = np.flatnonzero(keep & (got != ref))
            if bad.size:
                show = [(hex(int(bits[i])), float(x[i]), hex(int(got[i])), hex(int(ref[i]))) for i in bad[:8]]
                raise AssertionError(f"variant {variant} sc {sc}: {bad.size} mismatches in [{first:#x}, +{n}): {show}")
            checked += int(keep.sum())
            if (off // CHUNK) % 8 == 7:
                say(f"  ... {off + n:#x} patterns from {start:#x} checked")
            dev[:n].fill_(0xA5)
    return checked


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant,sc", [(0, 1.0), (1, 2.0 ** -8), (1, 2.0 ** 12)])
def test_pack_every_fp32_pattern(variant, sc):
    say(f"E4M3 pack sweep: variant {variant}, sc {sc}, all 2^32 patterns, {THREADS} oracle threads")
    checked = _sweep(variant, sc, 0, 1 << 32)
    say(f"  {checked} non-NaN patterns byte-exact")
    assert checked == (1 << 32) - 2 * ((1 << 23) - 1)  # every pattern but the NaNs


@pytest.mark.timeout(900)
def test_pack_inrange_every_pattern_to_448():
    # 0x43E00000 is 448.0; the sweep runs to the next multiple of 4 and masks what lies above
    n = 0x43E00004
    say(f"E4M3 in-range pack sweep: |x| <= 448, both signs, {2 * n} patterns")
    checked = _sweep(2, 1.0, 0, n) + _sweep(2, 1.0, 0x80000000, n)
    say(f"  {checked} patterns byte-exact")
    assert checked == 2 * (0x43E00000 + 1)


"""The projection producer's persistent schedule on the GPU: large jagged batches that give every
workgroup many items, so that the item list is refilled, the next item's loads are issued across
item boundaries at every ring phase (C_in = 128: one chunk, each item from its own prologue;
256: two chunks; 384: the ring base moves by two slots per item), and partial column tiles occur.

Every output byte and code is checked as written (the outputs are prefilled with 0xFF, which the
kernel writes only for a NaN block, and the inputs hold none), and sampled sequences (the first,
the last, the longest and random ones) are certified against the oracle as in the small cases.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from mx_cases import Guarded, certify_linear, cu_dev, say

pytestmark = pytest.mark.gpu

# (label, seed, number of sequences, length range, C_in, C_out)
CASES = [
    ("cin128_one_chunk", 61, 1100, (1, 600), 128, 1024),
    ("cin256_two_chunks", 62, 1100, (1, 600), 256, 1024),
    ("cin384_ring_shift_half_tile", 63, 700, (1, 900), 384, 384),
]


def _block_offsets(lens):
    return np.concatenate([[0], np.cumsum((np.asarray(lens) + 31) // 32)]).astype(np.int64)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_linear_many_items(case):
    label, seed, nseq, (lo, hi), C_in, C_out = case
    lens = [int(v) for v in synth.lengths(seed, nseq, lo, hi)]
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    items = sum((L + 255) // 256 for L in lens) * ((C_out + 255) // 256)
    say(f"linear schedule {label}: {nseq} sequences, T={T}, C_in={C_in}, C_out={C_out}, {items} items")
    x = synth.normal_bf16(seed, synth.STREAM_ACT, (T, C_in))
    w = synth.normal_bf16(seed, synth.STREAM_WEIGHT, (C_out, C_in), std=0.02)
    xd, xs, _ = oracle.quantize(x, cu, oracle.SQ32)
    wcu = np.array([0, C_out], np.int32)
    wd, ws, _ = oracle.quantize(w, wcu, oracle.ROW32)
    boff = _block_offsets(lens)
    nb = int(boff[-1])

    import precision_mxfp8_block_amd as mx
    xo = mx.MxOperand(torch.from_numpy(xd).cuda(), torch.from_numpy(xs).cuda(), mx.SQ32)
    wo = mx.MxOperand(torch.from_numpy(wd).cuda(), torch.from_numpy(ws).cuda(), mx.ROW32)
    data, scale, scale_t = (Guarded((T, C_out), torch.uint8), Guarded((nb, C_out // 32), torch.uint8),
                            Guarded((C_out // 32, nb), torch.uint8))
    mx.mxfa_linear_quantize(xo, wo, T, C_in, C_out, cu_dev(cu), nseq, max(lens), data.t, scale.t, scale_t.t)
    torch.cuda.synchronize()
    for g in (data, scale, scale_t):
        g.check(f"{label} output")
    for name, g in (("payload", data), ("scale", scale), ("transposed scale", scale_t)):
        unwritten = int((g.t == 0xFF).sum())
        assert unwritten == 0, f"{label}: {unwritten} {name} bytes never written"
    dg, sg, stg = data.t.cpu().numpy(), scale.t.cpu().numpy(), scale_t.t.cpu().numpy()

    rng = np.random.default_rng(seed)
    sample = sorted({0, nseq - 1, int(np.argmax(lens))} | set(int(v) for v in rng.choice(nseq, 9, replace=False)))
    for s in sample:
        rows = slice(int(cu[s]), int(cu[s + 1]))
        brows = slice(int(boff[s]), int(boff[s + 1]))
        cu1 = np.array([0, lens[s]], np.int32)
        d_o, s_o, st_o, y = oracle.linear_quantize(np.ascontiguousarray(xd[rows]), np.ascontiguousarray(xs[brows]),
                                                   wd, ws, cu1)
        yabs = np.abs(oracle.dequantize(np.ascontiguousarray(xd[rows]), np.ascontiguousarray(xs[brows]), cu1,
                                        oracle.SQ32)) @ np.abs(oracle.dequantize(wd, ws, wcu, oracle.ROW32)).T
        certify_linear(dg[rows], sg[brows], stg[:, brows], d_o, s_o, y.astype(np.float64), yabs, cu1,
                       f"{label} seq {s} (L={lens[s]})")

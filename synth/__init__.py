"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the attention method: it only draws numbers.

Generator: a counter-based SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the finalizer constants are the published ones). Draw i of
stream s under seed S is mix(base(S, s) + (i + 1) * GOLDEN), where base(S, s) = (S * 64 + s) << 40
and mix is the SplitMix64 output function. Uniforms take the top 53 bits; normals come from the
Box-Muller transform; values are rounded to bf16 with round-to-nearest-even.

Streams (fixed order): 0 lengths, 1 Q, 2 K, 3 V, 4 dO, 5 outlier masks (+ tensor index),
8 weights (+ index), 16 activations (+ index).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_LENGTHS, STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_OUTLIER = 0, 1, 2, 3, 4, 5
STREAM_WEIGHT, STREAM_ACT = 8, 16


def _mix(z):
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def raw_u64(seed, stream, n, offset=0):
    base = np.uint64(((seed * 64 + stream) << 40) & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
        return _mix(base + i * GOLDEN)


def uniform(seed, stream, n, offset=0):
    """Uniform doubles in (0, 1)."""
    r = raw_u64(seed, stream, n, offset)
    return ((r >> np.uint64(11)).astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed, stream, n, offset=0):
    """Standard normal doubles by Box-Muller over pairs of uniforms (draws 2*offset' onwards for
    an even element offset, so any even-aligned chunk reproduces the same values)."""
    m = (n + 1) // 2
    u = uniform(seed, stream, 2 * m, offset)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * m)
    z[0::2] = r * np.cos(2 * np.pi * u2)
    z[1::2] = r * np.sin(2 * np.pi * u2)
    return z[:n]


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK = 1 << 20  # elements per worker chunk (even, so Box-Muller pairs never straddle chunks)


def _normal_bf16_chunk(seed, stream, start, n, std, outlier_p, outlier_mult, os_):
    x = (normal(seed, stream, n, offset=start) * std).astype(np.float32)
    if outlier_p > 0:
        mask = uniform(seed, os_, n, offset=start) < outlier_p
        x[mask] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def normal_bf16(seed, stream, shape, std=1.0, outlier_p=0.0, outlier_mult=64.0, outlier_stream=None):
    """bf16 bits of N(0, std^2) values; each entry independently (probability outlier_p) is
    multiplied by outlier_mult in fp32 before the bf16 rounding. Element i always takes draws
    2*floor(i/2)+{1,2} of the value stream and draw i+1 of the outlier stream, so large tensors are
    generated in parallel chunks with identical results."""
    n = int(np.prod(shape))
    os_ = outlier_stream if outlier_stream is not None else STREAM_OUTLIER * 8 + stream
    out = np.empty(n, np.uint16)
    starts = list(range(0, n, _CHUNK))

    def work(st):
        cnt = min(_CHUNK, n - st)
        out[st:st + cnt] = _normal_bf16_chunk(seed, stream, st, cnt, std, outlier_p, outlier_mult, os_)

    if len(starts) <= 1:
        for st in starts:
            work(st)
    else:
        with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(work, starts))
    return out.reshape(shape)


def signs_bf16(seed, stream, shape, exp2):
    """bf16 bits of +-2^exp2 (a normal bf16 power of two), the sign of element i from bit 0 of
    draw i+1 of the stream."""
    n = int(np.prod(shape))
    mag = np.uint16((127 + int(exp2)) << 7)
    neg = (raw_u64(seed, stream, n) & np.uint64(1)).astype(np.uint16) << np.uint16(15)
    return (mag | neg).reshape(shape)


def lengths(seed, n, lo, hi):
    """n integer sequence lengths, uniform in [lo, hi]."""
    u = uniform(seed, STREAM_LENGTHS, n)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64).clip(lo, hi)


def cu_seqlens(lens):
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    return cu

"""Structured attention inputs whose results depend on one quantization point of the method.

Like the rest of synth/, this module only builds input tensors (bf16 bit patterns of seeded normal
values with some columns set to constants); it holds none of the method's arithmetic. Each builder
returns {"q", "k", "v", "do": bf16 bits [T, H*128]} plus the sequence lengths and softmax scale.

* delta_sensitive: in every head, V is 0 in columns 0, 32, 64, 96 and dO holds values of magnitude
  >= 2^22 there. Each 32 x 32 block of dO then has a scale at which its N(0,1) entries round to zero,
  so the quantized dO is zero outside those columns while the bf16 dO is not; with O = 0 in those
  columns, the backward's Delta = rowsum(dO o O) is carried entirely by the bf16 entries.
* ds_block_range: in every head, Q's column 0 is 12 and K's column 0 is -12 for keys in odd 32-key
  blocks of each sequence (0 elsewhere), so P in odd key blocks is ~2^-18 of P in even ones, and dS
  spans that range within each 32-query band of a 128-key tile.
* p_subnormal_band: the same with +-8, so P in odd key blocks is ~2^-8 of the even blocks' P: at the
  static P scale 2^-8 those P land among E4M3 subnormals.
* dq_fp16_rounding: one query against 256 keys with exact small values (see the builder).
"""
import numpy as np

from . import STREAM_DO, STREAM_K, STREAM_Q, STREAM_V, cu_seqlens, f32_to_bf16_bits, normal_bf16, bf16_bits_to_f32

D = 128


def _normals(seed, lens, H):
    T = int(np.sum(lens))
    C = H * D
    return {n: bf16_bits_to_f32(normal_bf16(seed, s, (T, C))).copy()
            for n, s in (("q", STREAM_Q), ("k", STREAM_K), ("v", STREAM_V), ("do", STREAM_DO))}


def _odd_key_blocks(lens):
    """Boolean per token: True for tokens in odd 32-token blocks counted from each sequence start."""
    return np.concatenate([((np.arange(L) // 32) % 2 == 1) for L in lens]) if len(lens) else np.zeros(0, bool)


def _pack(x, lens, c):
    return {"inputs": {n: f32_to_bf16_bits(a) for n, a in x.items()}, "lens": list(lens),
            "softmax_scale": c}


def delta_sensitive(seed=41, lens=(256, 130), H=2):
    x = _normals(seed, lens, H)
    big = (2.0 ** 22) * (1.0 + np.abs(x["do"]))
    for h in range(H):
        for col in (0, 32, 64, 96):
            j = h * D + col
            x["v"][:, j] = 0.0
            x["do"][:, j] = np.where(x["do"][:, j] < 0, -big[:, j], big[:, j])
    return _pack(x, lens, float(np.float32(1.0 / np.sqrt(D))))


def _key_block_offset(seed, lens, H, a):
    x = _normals(seed, lens, H)
    odd = _odd_key_blocks(lens)
    for h in range(H):
        x["q"][:, h * D] = a
        x["k"][:, h * D] = np.where(odd, -a, 0.0)
    return _pack(x, lens, float(np.float32(1.0 / np.sqrt(D))))


def ds_block_range(seed=42, lens=(512, 200), H=2):
    return _key_block_offset(seed, lens, H, 12.0)


def p_subnormal_band(seed=43, lens=(256, 384), H=2):
    return _key_block_offset(seed, lens, H, 8.0)


def dq_fp16_rounding():
    """One query, 256 keys (two 128-key tiles), one head, softmax scale 1. Q = e_0, K_0 = K_128 = e_1
    (other keys 0), V_0 = e_0, V_128 = (3/8) e_0, dO = e_0. Given O = 0 and LSE = 0 (passed directly
    to the backward), S = 0, P = 1, Delta = 0 and dS_0j = V_j0: the dQ partials of the two key tiles
    in column 1 are exactly 1 and 3/8."""
    q = np.zeros((1, D), np.float32); q[0, 0] = 1.0
    k = np.zeros((256, D), np.float32); k[0, 1] = 1.0; k[128, 1] = 1.0
    v = np.zeros((256, D), np.float32); v[0, 0] = 1.0; v[128, 0] = 0.375
    do = np.zeros((1, D), np.float32); do[0, 0] = 1.0
    return {"inputs": {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v),
                       "do": f32_to_bf16_bits(do)}, "lens_q": [1], "lens_k": [256], "softmax_scale": 1.0}


__all__ = ["delta_sensitive", "ds_block_range", "p_subnormal_band", "dq_fp16_rounding", "cu_seqlens"]

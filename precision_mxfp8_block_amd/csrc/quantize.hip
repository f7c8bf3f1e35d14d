// MX quantizer, jagged scale scatter and the fused RMSNorm + quantize producer (gfx950).
//
// All three are HBM-bound streaming kernels: every input byte is read once with 16-byte (or
// 8-byte) coalesced loads, every output byte written once. The block scale comes from the
// exponent bits of the block maximum (integer max over magnitude bit patterns, no logarithm or
// division), the payload from the hardware E4M3 converter after a saturating clamp (E2M1 and E2M3:
// the scaled FP4 / FP6 converters, which saturate by themselves).
// Pages: andresseo.expert "MXFP8 FlashAttention-4 Hits 2.85 Petaflops...", section "Inside the
// TMEM Bargain and Zero-Gather Jagged Pipeline" (32-element blocks, bit-extraction scale, fused
// RMSNorm producer, scale-only padding for jagged inputs); brifing.si items 5-7.
#include <algorithm>

#include "mx_device.h"
#include "mxfa_internal.h"

namespace {

// Row t and position j in the row of the flat lane index u (u < rows * per_row, the row length in
// lanes): a 32-bit division when the whole index space fits in 32 bits (a uniform branch on kernel
// arguments), the 64-bit one otherwise.
__device__ __forceinline__ void split_flat_index(int64_t u, int64_t per_row, int64_t total, int64_t& t, int& j) {
  if (total <= (int64_t)0xffffffffu) {
    const uint32_t q = (uint32_t)u / (uint32_t)per_row;
    t = q;
    j = (int)((uint32_t)u - q * (uint32_t)per_row);
  } else {
    t = u / per_row;
    j = (int)(u - t * per_row);
  }
}

// ---------------------------------------------------------------------------------------------
// ROW32: 1 x 32 blocks along the columns. Two lanes share a block, 16 bf16 each (two 16-byte loads).
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) quantize_row32_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int64_t T,
                                                             int C, uint8_t* __restrict__ data,
                                                             uint8_t* __restrict__ scale) {
  const int64_t chunks_per_row = C >> 4;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = T * chunks_per_row;
  if (u >= total) return;  // pairs of lanes leave together (chunks_per_row is even)
  int64_t t;
  int j;
  split_flat_index(u, chunks_per_row, total, t, j);
  const uint4* src = reinterpret_cast<const uint4*>(x + t * ld_x + (int64_t)j * 16);
  uint4 a = src[0], b = src[1];
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
    amax = max(amax, max(lo, hi));
  }
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
  const uint32_t code = mx_code_from_amax_bits(amax << 16);
  uint4 out;
  if (code == 255u) {
    out = make_uint4(0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu);
  } else {
    const float inv = mx_inv_scale(code);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t p = w[2 * i], q = w[2 * i + 1];
      o[i] = mx_pack4(bf16_to_f32(p & 0xffffu) * inv, bf16_to_f32(p >> 16) * inv, bf16_to_f32(q & 0xffffu) * inv,
                      bf16_to_f32(q >> 16) * inv);
    }
    out = make_uint4(o[0], o[1], o[2], o[3]);
  }
  *reinterpret_cast<uint4*>(data + t * C + (int64_t)j * 16) = out;
  if ((j & 1) == 0) scale[t * (C >> 5) + (j >> 1)] = (uint8_t)code;
}

// ---------------------------------------------------------------------------------------------
// ROW32 in MXFP4 and MXFP6 (OCP MX element formats E2M1 and E2M3, both with largest exponent 2): the
// scale code is clamp(exponent_field(amax) - 2, 0, 254); 255 and a zero payload for blocks holding
// NaN or Inf. The elements come from gfx950's scaled conversions, which take the E8M0 scale as the
// exponent field of a float (code << 23, so code 0 is 2^-127) and give the nearest code of x / 2^(code
// - 127): ties to the even code, saturating at the largest magnitude (6 and 7.5), the sign kept for
// values that round to zero, bf16 subnormals exact. Measured on the device at every midpoint of both
// grids, on saturating values, signed zeros and subnormal inputs with code 0.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float e8m0_as_scale(uint32_t code) { return __uint_as_float(code << 23); }

// Byte SEL of `old` <- the E2M1 codes of the two bf16 in w (low half -> low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t old, uint32_t w, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, __uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u),
                                                  sc, SEL);
}

// MXFP4: two lanes share a block, 16 bf16 each; a lane writes 8 bytes (element 2i in the low nibble of
// byte i).
__global__ void __launch_bounds__(256) quantize_row32_e2m1_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                                  int64_t T, int C, uint8_t* __restrict__ data,
                                                                  uint8_t* __restrict__ scale) {
  const int64_t chunks_per_row = C >> 4;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = T * chunks_per_row;
  if (u >= total) return;  // pairs of lanes leave together (chunks_per_row is even)
  int64_t t;
  int j;
  split_flat_index(u, chunks_per_row, total, t, j);
  const uint4* src = reinterpret_cast<const uint4*>(x + t * ld_x + (int64_t)j * 16);
  const uint4 a = src[0], b = src[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = max(amax, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
  const uint32_t e = amax >> 7;  // biased exponent field of the bf16 (= fp32) maximum
  const uint32_t code = e >= 255u ? 255u : (e > 2u ? e - 2u : 0u);
  uint2 out = make_uint2(0u, 0u);
  if (code != 255u) {
    const float sc = e8m0_as_scale(code);
    uint32_t o0 = e2m1_pair<0>(0u, w[0], sc), o1 = e2m1_pair<0>(0u, w[4], sc);
    o0 = e2m1_pair<1>(o0, w[1], sc);
    o1 = e2m1_pair<1>(o1, w[5], sc);
    o0 = e2m1_pair<2>(o0, w[2], sc);
    o1 = e2m1_pair<2>(o1, w[6], sc);
    o0 = e2m1_pair<3>(o0, w[3], sc);
    o1 = e2m1_pair<3>(o1, w[7], sc);
    out = make_uint2(o0, o1);
  }
  *reinterpret_cast<uint2*>(data + t * (C >> 1) + (int64_t)j * 8) = out;
  if ((j & 1) == 0) scale[t * (C >> 5) + (j >> 1)] = (uint8_t)code;
}

// MXFP6: a block's 32 six-bit codes form a 24-byte little-endian bit string (code j at bits 6j .. 6j +
// 5). Blocks go in pairs (2p, 2p + 1) of 48 bytes: bytes 0-15 of block 2p, bytes 0-15 of block 2p + 1,
// then the two blocks' bytes 16-23, so that a block is one 16-byte and one 8-byte piece (the forward
// reads an FP6 operand as exactly these two pieces). One lane per block: four 16-byte loads, the block
// maximum in the lane, one conversion of all 32 elements, one 16-byte and one 8-byte store.
// The conversion (v_cvt_scalef32_2xpk16_fp6_f32) takes its first source as the even elements and its
// second as the odd ones (code 2i from the first source's element i, code 2i + 1 from the second's),
// measured on the device. It is written as inline asm with an early-clobber result: when the compiler
// let the result registers start inside the first source (result at source register 2), the element in
// the overwritten register came out wrong on the device, so the result must not overlap the sources.
typedef int mx_v6i __attribute__((ext_vector_type(6)));

__global__ void __launch_bounds__(256) quantize_row32_e2m3_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                                  int64_t T, int C, uint8_t* __restrict__ data,
                                                                  uint8_t* __restrict__ scale) {
  const int64_t blocks_per_row = C >> 5;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = T * blocks_per_row;
  if (u >= total) return;
  int64_t t;
  int blk;
  split_flat_index(u, blocks_per_row, total, t, blk);
  const uint4* src = reinterpret_cast<const uint4*>(x + t * ld_x + (int64_t)blk * 32);
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = src[q];
    w[4 * q] = v.x;
    w[4 * q + 1] = v.y;
    w[4 * q + 2] = v.z;
    w[4 * q + 3] = v.w;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  const uint32_t e = amax >> 7;
  const uint32_t code = e >= 255u ? 255u : (e > 2u ? e - 2u : 0u);
  uint4 head = make_uint4(0u, 0u, 0u, 0u);
  uint2 tail = make_uint2(0u, 0u);
  if (code != 255u) {
    mx_v16f even, odd;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      even[i] = __uint_as_float(w[i] << 16);
      odd[i] = __uint_as_float(w[i] & 0xffff0000u);
    }
    mx_v6i r;
    asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(even), "v"(odd), "v"(e8m0_as_scale(code)));
    head = make_uint4((uint32_t)r[0], (uint32_t)r[1], (uint32_t)r[2], (uint32_t)r[3]);
    tail = make_uint2((uint32_t)r[4], (uint32_t)r[5]);
  }
  uint8_t* pair = data + t * (3 * (int64_t)C / 4) + 48 * (blk >> 1);
  *reinterpret_cast<uint4*>(pair + 16 * (blk & 1)) = head;
  *reinterpret_cast<uint2*>(pair + 32 + 8 * (blk & 1)) = tail;
  scale[t * blocks_per_row + blk] = (uint8_t)code;
}

// ---------------------------------------------------------------------------------------------
// COL32: 32 x 1 blocks along the tokens. A wave covers 32 rows x 128 columns: lane l owns columns
// 4 (l % 32) .. +3 (8-byte loads) of rows 16 (l / 32) + i, i = 0..15; a column's maximum joins the
// two half-waves with one lane swap. Every load instruction covers two 256-byte row segments and
// every store two whole 128-byte output row segments; four waves cover 512 columns.
// Grid: x = C / 512 (rounded up), y = block index inside the sequence, z = sequence.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) quantize_col32_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int C,
                                                             const int32_t* __restrict__ cu,
                                                             uint8_t* __restrict__ data,
                                                             uint8_t* __restrict__ scale) {
  const int s = blockIdx.z, b = blockIdx.y;
  const int64_t t0 = cu[s], L = (int64_t)cu[s + 1] - t0;
  if ((int64_t)b * 32 >= L) return;  // uniform over the workgroup
  const SeqOffsets off = seq_offsets(cu, s);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cg = blockIdx.x * 4 + wave;  // 128-column group
  if (cg * 128 >= C) return;             // whole wave leaves together
  const int col = cg * 128 + 4 * (lane & 31);
  const bool col_ok = col < C;
  const int col_ld = col_ok ? col : cg * 128;  // lanes past C re-read the group's first columns
  const int half = lane >> 5;
  const int rows = (int)min<int64_t>(32, L - (int64_t)b * 32);
  const int64_t ta = t0 + (int64_t)b * 32;
  // rows past the sequence end re-read its last row: every load is issued without a branch, and a
  // repeated row does not change the block maximum
  uint2 v[16];
  uint32_t am[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = *reinterpret_cast<const uint2*>(x + (ta + min(16 * half + i, rows - 1)) * ld_x + col_ld);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    am[0] = max(am[0], v[i].x & 0x7fffu);
    am[1] = max(am[1], (v[i].x >> 16) & 0x7fffu);
    am[2] = max(am[2], v[i].y & 0x7fffu);
    am[3] = max(am[3], (v[i].y >> 16) & 0x7fffu);
  }
  uint32_t code[4];
  float inv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    auto sw = __builtin_amdgcn_permlane32_swap(am[k], am[k], false, false);  // the other half-wave
    const uint32_t m = max((uint32_t)sw[0], (uint32_t)sw[1]);
    code[k] = mx_code_from_amax_bits(m << 16);
    inv[k] = code[k] == 255u ? 0.0f : mx_inv_scale(code[k]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * half + i;
    if (col_ok && r < rows) {
      uint32_t o = mx_pack4(bf16_to_f32(v[i].x & 0xffffu) * inv[0], bf16_to_f32(v[i].x >> 16) * inv[1],
                            bf16_to_f32(v[i].y & 0xffffu) * inv[2], bf16_to_f32(v[i].y >> 16) * inv[3]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (code[k] == 255u) o = (o & ~(0xffu << (8 * k))) | (0x7fu << (8 * k));
      *reinterpret_cast<uint32_t*>(data + (ta + r) * C + col) = o;
    }
  }
  if (half == 0 && col_ok) {
    const int64_t br = off.blocks32 + b;
    *reinterpret_cast<uint32_t*>(scale + br * C + col) = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
  }
}

// ---------------------------------------------------------------------------------------------
// COL32 and ROW32 of one matrix from one read (an operand contracted over the tokens in one GEMM and
// over the columns in another, as V is in the attention's forward and backward). The wave layout of
// the COL32 kernel; a row's 32-column ROW32 block is the 4 columns of 8 consecutive lanes (lane bits
// 0-2), whose maximum takes three DPP steps. Both payloads leave as the COL32 kernel's stores; lane
// 8 b + 0 stores the ROW32 code of its row and block. Same grid as the COL32 kernel.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
}

__global__ void __launch_bounds__(256) quantize_col32_row32_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                                   int C, const int32_t* __restrict__ cu,
                                                                   uint8_t* __restrict__ data_c,
                                                                   uint8_t* __restrict__ scale_c,
                                                                   uint8_t* __restrict__ data_r,
                                                                   uint8_t* __restrict__ scale_r) {
  const int s = blockIdx.z, b = blockIdx.y;
  const int64_t t0 = cu[s], L = (int64_t)cu[s + 1] - t0;
  if ((int64_t)b * 32 >= L) return;  // uniform over the workgroup
  const SeqOffsets off = seq_offsets(cu, s);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cg = blockIdx.x * 4 + wave;  // 128-column group
  if (cg * 128 >= C) return;             // whole wave leaves together
  const int col = cg * 128 + 4 * (lane & 31);
  // C is a multiple of 32, so the lanes past C are whole 8-lane ROW32 groups: they compute but store
  // nothing
  const bool col_ok = col < C;
  const int col_ld = col_ok ? col : cg * 128;
  const int half = lane >> 5;
  const int rows = (int)min<int64_t>(32, L - (int64_t)b * 32);
  const int64_t ta = t0 + (int64_t)b * 32;
  uint2 v[16];
  uint32_t am[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = *reinterpret_cast<const uint2*>(x + (ta + min(16 * half + i, rows - 1)) * ld_x + col_ld);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    am[0] = max(am[0], v[i].x & 0x7fffu);
    am[1] = max(am[1], (v[i].x >> 16) & 0x7fffu);
    am[2] = max(am[2], v[i].y & 0x7fffu);
    am[3] = max(am[3], (v[i].y >> 16) & 0x7fffu);
  }
  uint32_t code[4];
  float inv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    auto sw = __builtin_amdgcn_permlane32_swap(am[k], am[k], false, false);  // the other half-wave
    const uint32_t m = max((uint32_t)sw[0], (uint32_t)sw[1]);
    code[k] = mx_code_from_amax_bits(m << 16);
    inv[k] = code[k] == 255u ? 0.0f : mx_inv_scale(code[k]);
  }
  const uint32_t cnan = (code[0] == 255u ? 0xffu : 0u) | (code[1] == 255u ? 0xff00u : 0u) |
                        (code[2] == 255u ? 0xff0000u : 0u) | (code[3] == 255u ? 0xff000000u : 0u);
  const int64_t cs = C >> 5;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float f0 = bf16_to_f32(v[i].x & 0xffffu), f1 = bf16_to_f32(v[i].x >> 16);
    const float f2 = bf16_to_f32(v[i].y & 0xffffu), f3 = bf16_to_f32(v[i].y >> 16);
    const uint32_t rm = max_over_8_lanes(max(max(v[i].x & 0x7fffu, (v[i].x >> 16) & 0x7fffu),
                                             max(v[i].y & 0x7fffu, (v[i].y >> 16) & 0x7fffu)));
    const uint32_t rcode = mx_code_from_amax_bits(rm << 16);
    const int r = 16 * half + i;
    if (col_ok && r < rows) {
      uint32_t oc = mx_pack4(f0 * inv[0], f1 * inv[1], f2 * inv[2], f3 * inv[3]);
      oc = (oc & ~cnan) | (0x7f7f7f7fu & cnan);
      uint32_t orow = 0x7f7f7f7fu;
      if (rcode != 255u) {
        const float ri = mx_inv_scale(rcode);
        orow = mx_pack4(f0 * ri, f1 * ri, f2 * ri, f3 * ri);
      }
      *reinterpret_cast<uint32_t*>(data_c + (ta + r) * C + col) = oc;
      *reinterpret_cast<uint32_t*>(data_r + (ta + r) * C + col) = orow;
      if ((lane & 7) == 0) scale_r[(ta + r) * cs + (col >> 5)] = (uint8_t)rcode;
    }
  }
  if (half == 0 && col_ok) {
    const int64_t br = off.blocks32 + b;
    *reinterpret_cast<uint32_t*>(scale_c + br * C + col) =
        code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
  }
}

// ---------------------------------------------------------------------------------------------
// SQ32: 32 x 32 blocks. A wave covers 32 rows x 64 columns (two blocks): lane l reads the 16-byte
// chunk l % 8 (8 bf16) of rows l / 8 + 8 i, i = 0..3, so every load and store instruction covers
// whole 128-byte row segments. The lane's block is (l % 8) / 4; its maximum is taken over the 32
// lanes that share lane bit 2 (DPP and lane swaps, no LDS). Four waves cover 256 columns.
// Grid: x = C / 256 (rounded up), y = block row inside the sequence, z = sequence.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t max_over_block_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false));   // lane bit 0
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false));   // lane bit 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, false));  // row_ror:8, lane bit 3
  auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);                   // lane bit 4
  v = max((uint32_t)s16[0], (uint32_t)s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);                   // lane bit 5
  return max((uint32_t)s32[0], (uint32_t)s32[1]);
}

__global__ void __launch_bounds__(256) quantize_sq32_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int C,
                                                            const int32_t* __restrict__ cu, int nseq,
                                                            uint8_t* __restrict__ data, uint8_t* __restrict__ scale,
                                                            uint8_t* __restrict__ scale_t) {
  const int s = blockIdx.z, b = blockIdx.y;
  const int64_t t0 = cu[s], L = (int64_t)cu[s + 1] - t0;
  if ((int64_t)b * 32 >= L) return;
  const SeqOffsets off = seq_offsets(cu, s);
  int64_t nb_total = 0;
  if (scale_t) nb_total = seq_offsets(cu, nseq).blocks32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cg = blockIdx.x * 4 + wave;  // 64-column group
  if (cg * 64 >= C) return;              // whole wave leaves together
  const int chunk = lane & 7, rl = lane >> 3;
  const int col = cg * 64 + chunk * 8;
  const bool col_ok = col < C;  // C % 64 == 32: the group's second block does not exist
  const int rows = (int)min<int64_t>(32, L - (int64_t)b * 32);
  const int64_t tb = t0 + (int64_t)b * 32;
  // rows past the sequence end re-read its last row and a missing second block re-reads the first
  // (neither changes a stored block maximum), so every load is issued without a branch
  const int col_ld = col_ok ? col : col - 32;
  uint4 w[4];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = min(rl + 8 * i, rows - 1);
    w[i] = *reinterpret_cast<const uint4*>(x + (tb + rr) * ld_x + col_ld);
    const uint32_t q[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = max(amax, max(q[k] & 0x7fffu, (q[k] >> 16) & 0x7fffu));
  }
  amax = max_over_block_lanes(amax);
  const uint32_t code = mx_code_from_amax_bits(amax << 16);
  const float inv = code == 255u ? 0.0f : mx_inv_scale(code);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = rl + 8 * i;
    if (col_ok && rr < rows) {
      uint2 out;
      if (code == 255u) {
        out = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
      } else {
        const uint32_t q[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
        out.x = mx_pack4(bf16_to_f32(q[0] & 0xffffu) * inv, bf16_to_f32(q[0] >> 16) * inv,
                         bf16_to_f32(q[1] & 0xffffu) * inv, bf16_to_f32(q[1] >> 16) * inv);
        out.y = mx_pack4(bf16_to_f32(q[2] & 0xffffu) * inv, bf16_to_f32(q[2] >> 16) * inv,
                         bf16_to_f32(q[3] & 0xffffu) * inv, bf16_to_f32(q[3] >> 16) * inv);
      }
      *reinterpret_cast<uint2*>(data + (tb + rr) * C + col) = out;
    }
  }
  if ((lane & 3) == 0 && lane < 8 && col_ok) {  // lanes 0 and 4: the group's two blocks
    const int cb = col >> 5;
    const int64_t br = off.blocks32 + b;
    scale[br * (C >> 5) + cb] = (uint8_t)code;
    if (scale_t) scale_t[(int64_t)cb * nb_total + br] = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------------------------
// Scale scatter: compact rows -> padded rows; each workgroup moves the rows of one 128-token group
// of one sequence and zero-fills the rows of that group that lie past the sequence end.
// Grid: x = 128-token groups (max_seqlen / 128 rounded up), y = sequence.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) scale_scatter_kernel(const uint8_t* __restrict__ compact,
                                                            const int32_t* __restrict__ cu, int C, int mode,
                                                            uint8_t* __restrict__ padded, int64_t padded_rows) {
  const int s = blockIdx.y, g = blockIdx.x;
  const int64_t L = (int64_t)cu[s + 1] - cu[s];
  if ((int64_t)g * 128 >= L) return;
  const SeqOffsets off = seq_offsets(cu, s);
  const int width = (mode == 1) ? C : (C >> 5);
  const int unit = (mode == 0) ? 1 : 32;                 // tokens per layout row
  const int rows_per_group = 128 / unit;
  const int64_t valid_rows = (L + unit - 1) / unit;      // rows of this sequence in the compact tensor
  const int64_t src_row0 = (mode == 0) ? (int64_t)cu[s] : off.blocks32;
  const int64_t dst_row0 = off.padded / unit;
  const int64_t grow0 = (int64_t)g * rows_per_group;     // first row of this group inside the sequence
  // rows of the group that hold data, and rows that exist in the padded buffer
  const int nvalid = (int)max<int64_t>(0, min<int64_t>(rows_per_group, valid_rows - grow0));
  const int nrows = (int)max<int64_t>(0, min<int64_t>(rows_per_group, padded_rows - dst_row0 - grow0));
  const uint8_t* src = compact + (src_row0 + grow0) * width;
  uint8_t* dst = padded + (dst_row0 + grow0) * width;
  if ((width & 15) == 0) {
    // 16-byte pieces (the row width and both row starts are multiples of 16 bytes)
    const int wv = width >> 4;
    const int n = nrows * wv;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int rr = i / wv;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < nvalid) v = reinterpret_cast<const uint4*>(src)[i];
      reinterpret_cast<uint4*>(dst)[i] = v;
    }
  } else {
    const int n = nrows * width;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int rr = i / width;
      dst[i] = rr < nvalid ? src[i] : (uint8_t)0;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Fused RMSNorm + SQ32 quantize. One workgroup per (sequence, 32-token block), all C columns:
//   pass 1: per-row sum of squares (FP64 adds of exact bf16 squares, one rounding to fp32),
//           r = 1 / sqrtf(ss / C + eps) with IEEE division and square root;
//   pass 2: y = (x * r) * gamma, block maxima per 32-column block (integer max in LDS);
//   pass 3: y again, quantize with the block's code, store payload and both scale layouts.
// Passes 2 and 3 re-read the 32 x C tile, which the L2 holds; HBM sees one read and one write.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) rmsnorm_quantize_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int C,
                                                               const float* __restrict__ gamma, float eps,
                                                               const int32_t* __restrict__ cu, int nseq,
                                                               uint8_t* __restrict__ data,
                                                               uint8_t* __restrict__ scale,
                                                               uint8_t* __restrict__ scale_t) {
  __shared__ float rs[32];
  __shared__ uint32_t bmax[1024];  // up to C = 32768 columns
  const int s = blockIdx.y, b = blockIdx.x;
  const int64_t t0 = cu[s], L = (int64_t)cu[s + 1] - t0;
  if ((int64_t)b * 32 >= L) return;
  const SeqOffsets off = seq_offsets(cu, s);
  int64_t nb_total = 0;
  if (scale_t) nb_total = seq_offsets(cu, nseq).blocks32;
  const int rows = (int)min<int64_t>(32, L - (int64_t)b * 32);
  const int64_t ta = t0 + (int64_t)b * 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int ncb = C >> 5;
  for (int i = threadIdx.x; i < ncb; i += blockDim.x) bmax[i] = 0;
  // pass 1: one wave per row
  for (int r = wave; r < rows; r += nwaves) {
    const uint16_t* row = x + (ta + r) * ld_x;
    double ss = 0.0;
    for (int c = lane * 8; c < C; c += 64 * 8) {
      uint4 v = *reinterpret_cast<const uint4*>(row + c);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = bf16_to_f32(w[i] & 0xffffu), bb = bf16_to_f32(w[i] >> 16);
        ss += (double)(a * a) + (double)(bb * bb);  // squares of bf16 values are exact in fp32
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) {
      float ms = (float)ss / (float)C;
      rs[r] = 1.0f / __fsqrt_rn(ms + eps);
    }
  }
  __syncthreads();
  // pass 2: block maxima of y. Thread covers 8 columns of one row.
  const int chunks = C >> 3;
  for (int i = threadIdx.x; i < rows * chunks; i += blockDim.x) {
    const int r = i / chunks, ch = i % chunks;
    uint4 v = *reinterpret_cast<const uint4*>(x + (ta + r) * ld_x + (int64_t)ch * 8);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const float rr = rs[r];
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y0 = __fmul_rn(__fmul_rn(bf16_to_f32(w[k] & 0xffffu), rr), gamma[ch * 8 + 2 * k]);
      float y1 = __fmul_rn(__fmul_rn(bf16_to_f32(w[k] >> 16), rr), gamma[ch * 8 + 2 * k + 1]);
      am = max(am, max(__float_as_uint(y0) & 0x7fffffffu, __float_as_uint(y1) & 0x7fffffffu));
    }
    atomicMax(&bmax[ch >> 2], am);
  }
  __syncthreads();
  // pass 3: quantize and store
  for (int i = threadIdx.x; i < rows * chunks; i += blockDim.x) {
    const int r = i / chunks, ch = i % chunks;
    uint4 v = *reinterpret_cast<const uint4*>(x + (ta + r) * ld_x + (int64_t)ch * 8);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const float rr = rs[r];
    const uint32_t code = mx_code_from_amax_bits(bmax[ch >> 2]);
    uint2 out;
    if (code == 255u) {
      out = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
    } else {
      const float inv = mx_inv_scale(code);
      float y[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[2 * k] = __fmul_rn(__fmul_rn(bf16_to_f32(w[k] & 0xffffu), rr), gamma[ch * 8 + 2 * k]);
        y[2 * k + 1] = __fmul_rn(__fmul_rn(bf16_to_f32(w[k] >> 16), rr), gamma[ch * 8 + 2 * k + 1]);
      }
      out.x = mx_pack4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
      out.y = mx_pack4(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
    }
    *reinterpret_cast<uint2*>(data + (ta + r) * C + (int64_t)ch * 8) = out;
  }
  const int64_t br = off.blocks32 + b;
  for (int cb = threadIdx.x; cb < ncb; cb += blockDim.x) {
    const uint8_t code = (uint8_t)mx_code_from_amax_bits(bmax[cb]);
    scale[br * ncb + cb] = code;
    if (scale_t) scale_t[(int64_t)cb * nb_total + br] = code;
  }
}

// ---------------------------------------------------------------------------------------------
// Fused RMSNorm + SQ32 quantize for C = 512 SEGS (SEGS = 1..4) with the 32 x C tile held in
// registers: one read of the input, one write of the payload. Workgroup = 8 waves per (sequence,
// 32-token block); wave w owns rows 4w..4w+3, lane l columns 512 j + 8 l .. + 7 of segment j
// (16-byte loads and 8-byte stores cover whole 1 KB / 512 B row segments per instruction).
// Per row: sum of squares in FP64 (exact bf16 squares), lane sum by butterfly, one rounding to
// fp32; r = 1 / sqrtf(ss / C + eps). y = (x r) gamma; the maximum |y| of each 32 x 32 block is
// taken over the lane's 4 rows x 8 columns, the 4 lanes of the block (DPP) and the 8 waves (LDS).
// Rows past the sequence end re-read the block's last row (no branch on the loads; a repeated
// row leaves every block maximum unchanged) and are not stored.
// ---------------------------------------------------------------------------------------------
template <int SEGS>
__global__ void __launch_bounds__(512) rmsnorm_quantize_regs_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                                    const float* __restrict__ gamma, float eps,
                                                                    const int32_t* __restrict__ cu, int nseq,
                                                                    uint8_t* __restrict__ data,
                                                                    uint8_t* __restrict__ scale,
                                                                    uint8_t* __restrict__ scale_t) {
  constexpr int C = 512 * SEGS;
  constexpr int NCB = C / 32;
  __shared__ uint32_t bm[8][NCB];
  const int s = blockIdx.y, b = blockIdx.x;
  const int64_t t0 = cu[s], L = (int64_t)cu[s + 1] - t0;
  if ((int64_t)b * 32 >= L) return;  // uniform over the workgroup
  const SeqOffsets off = seq_offsets(cu, s);
  int64_t nb_total = 0;
  if (scale_t) nb_total = seq_offsets(cu, nseq).blocks32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = (int)min<int64_t>(32, L - (int64_t)b * 32);
  const int64_t tb = t0 + (int64_t)b * 32;

  uint4 v[4][SEGS];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = min(4 * wave + i, rows - 1);
#pragma unroll
    for (int j = 0; j < SEGS; ++j)
      v[i][j] = *reinterpret_cast<const uint4*>(x + (tb + rr) * ld_x + 512 * j + 8 * lane);
  }
  float g[SEGS][8];
#pragma unroll
  for (int j = 0; j < SEGS; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) g[j][e] = gamma[512 * j + 8 * lane + e];

  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < SEGS; ++j) {
      const uint32_t w[4] = {v[i][j].x, v[i][j].y, v[i][j].z, v[i][j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = bf16_to_f32(w[k] & 0xffffu), c = bf16_to_f32(w[k] >> 16);
        ss += (double)(a * a) + (double)(c * c);  // squares of bf16 values are exact in fp32
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float ms = (float)ss / (float)C;
    r[i] = 1.0f / __fsqrt_rn(ms + eps);
  }

  auto yval = [&](int i, int j, int e) {
    const uint32_t w = (e >> 1) == 0 ? v[i][j].x : (e >> 1) == 1 ? v[i][j].y : (e >> 1) == 2 ? v[i][j].z : v[i][j].w;
    const float xv = bf16_to_f32((e & 1) ? (w >> 16) : (w & 0xffffu));
    return __fmul_rn(__fmul_rn(xv, r[i]), g[j][e]);
  };
  // block maxima (magnitude bit patterns; NaN and Inf order above every finite value)
#pragma unroll
  for (int j = 0; j < SEGS; ++j) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) am = max(am, __float_as_uint(yval(i, j, e)) & 0x7fffffffu);
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0u, am, 0xB1, 0xF, 0xF, false));  // lane bit 0
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0u, am, 0x4E, 0xF, 0xF, false));  // lane bit 1
    if ((lane & 3) == 0) bm[wave][16 * j + (lane >> 2)] = am;
  }
  __syncthreads();
  uint32_t code[SEGS];
#pragma unroll
  for (int j = 0; j < SEGS; ++j) {
    uint32_t am = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) am = max(am, bm[w][16 * j + (lane >> 2)]);
    code[j] = mx_code_from_amax_bits(am);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * wave + i;
    if (rr < rows) {
#pragma unroll
      for (int j = 0; j < SEGS; ++j) {
        uint2 out;
        if (code[j] == 255u) {
          out = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
        } else {
          const float inv = mx_inv_scale(code[j]);
          out.x = mx_pack4(yval(i, j, 0) * inv, yval(i, j, 1) * inv, yval(i, j, 2) * inv, yval(i, j, 3) * inv);
          out.y = mx_pack4(yval(i, j, 4) * inv, yval(i, j, 5) * inv, yval(i, j, 6) * inv, yval(i, j, 7) * inv);
        }
        *reinterpret_cast<uint2*>(data + (tb + rr) * C + 512 * j + 8 * lane) = out;
      }
    }
  }
  if (wave == 0 && (lane & 3) == 0) {
    const int64_t br = off.blocks32 + b;
#pragma unroll
    for (int j = 0; j < SEGS; ++j) {
      const int cb = 16 * j + (lane >> 2);
      scale[br * NCB + cb] = (uint8_t)code[j];
      if (scale_t) scale_t[(int64_t)cb * nb_total + br] = (uint8_t)code[j];
    }
  }
}

}  // namespace

namespace mxfa {

hipError_t launch_quantize(const uint16_t* x, int64_t ld_x, int64_t T, int C, const int32_t* cu, int nseq,
                           int max_seqlen, int mode, uint8_t* data, uint8_t* scale, uint8_t* scale_t,
                           hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (mode == 0) {
    const int64_t units = T * (C >> 4);
    const int64_t blocks = (units + 255) / 256;
    hipLaunchKernelGGL(quantize_row32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, ld_x, T, C, data,
                       scale);
  } else if (mode == 1) {
    dim3 grid((unsigned)((C + 511) / 512), (unsigned)((max_seqlen + 31) / 32), (unsigned)nseq);
    hipLaunchKernelGGL(quantize_col32_kernel, grid, dim3(256), 0, stream, x, ld_x, C, cu, data, scale);
  } else {
    dim3 grid((unsigned)((C + 255) / 256), (unsigned)((max_seqlen + 31) / 32), (unsigned)nseq);
    hipLaunchKernelGGL(quantize_sq32_kernel, grid, dim3(256), 0, stream, x, ld_x, C, cu, nseq, data, scale,
                       scale_t);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_col32_row32(const uint16_t* x, int64_t ld_x, int C, const int32_t* cu, int nseq,
                                      int max_seqlen, uint8_t* data_col, uint8_t* scale_col, uint8_t* data_row,
                                      uint8_t* scale_row, hipStream_t stream) {
  if (max_seqlen == 0) return hipSuccess;
  dim3 grid((unsigned)((C + 511) / 512), (unsigned)((max_seqlen + 31) / 32), (unsigned)nseq);
  hipLaunchKernelGGL(quantize_col32_row32_kernel, grid, dim3(256), 0, stream, x, ld_x, C, cu, data_col, scale_col,
                     data_row, scale_row);
  return hipGetLastError();
}

hipError_t launch_quantize_e2m1(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data, uint8_t* scale,
                               hipStream_t stream) {
  const int64_t units = T * (C >> 4);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_row32_e2m1_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, x, ld_x,
                     T, C, data, scale);
  return hipGetLastError();
}

hipError_t launch_quantize_e2m3(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data, uint8_t* scale,
                               hipStream_t stream) {
  const int64_t units = T * (C >> 5);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_row32_e2m3_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, x, ld_x,
                     T, C, data, scale);
  return hipGetLastError();
}

hipError_t launch_scale_scatter(const uint8_t* compact, const int32_t* cu, int nseq, int max_seqlen, int C, int mode,
                                uint8_t* padded, int64_t padded_rows, hipStream_t stream) {
  if (max_seqlen == 0) return hipSuccess;
  dim3 grid((unsigned)((max_seqlen + 127) / 128), (unsigned)nseq);
  hipLaunchKernelGGL(scale_scatter_kernel, grid, dim3(256), 0, stream, compact, cu, C, mode, padded, padded_rows);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t ld_x, int C, const float* gamma, float eps,
                                   const int32_t* cu, int nseq, int max_seqlen, uint8_t* data, uint8_t* scale,
                                   uint8_t* scale_t, hipStream_t stream) {
  if (max_seqlen == 0) return hipSuccess;
  dim3 grid((unsigned)((max_seqlen + 31) / 32), (unsigned)nseq);
  switch (C) {
    case 512:
      hipLaunchKernelGGL(rmsnorm_quantize_regs_kernel<1>, grid, dim3(512), 0, stream, x, ld_x, gamma, eps, cu, nseq,
                         data, scale, scale_t);
      break;
    case 1024:
      hipLaunchKernelGGL(rmsnorm_quantize_regs_kernel<2>, grid, dim3(512), 0, stream, x, ld_x, gamma, eps, cu, nseq,
                         data, scale, scale_t);
      break;
    case 1536:
      hipLaunchKernelGGL(rmsnorm_quantize_regs_kernel<3>, grid, dim3(512), 0, stream, x, ld_x, gamma, eps, cu, nseq,
                         data, scale, scale_t);
      break;
    case 2048:
      hipLaunchKernelGGL(rmsnorm_quantize_regs_kernel<4>, grid, dim3(512), 0, stream, x, ld_x, gamma, eps, cu, nseq,
                         data, scale, scale_t);
      break;
    default:
      hipLaunchKernelGGL(rmsnorm_quantize_kernel, grid, dim3(256), 0, stream, x, ld_x, C, gamma, eps, cu, nseq, data,
                         scale, scale_t);
  }
  return hipGetLastError();
}

// Consecutive fp32 bit patterns through the E4M3 packs the kernels use, four patterns per thread
// (one 4-byte store): variant 0 the saturating pack of unscaled values (quantizers, O and projection
// epilogues), 1 the saturating pack of x / sc (dS and projection epilogues), 2 the pack of values
// known to lie in [-448, 448] (P * 256). Patterns wrap modulo 2^32.
__global__ void __launch_bounds__(256) e4m3_pack_patterns_kernel(uint32_t first, int64_t nwords, int variant,
                                                                 float sc, float lim, uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords; w += stride) {
    const uint32_t b = first + 4u * (uint32_t)w;
    const float a = __uint_as_float(b), c = __uint_as_float(b + 1u);
    const float d = __uint_as_float(b + 2u), e = __uint_as_float(b + 3u);
    uint32_t r;
    if (variant == 0)
      r = mx_pack4(a, c, d, e);
    else if (variant == 1)
      r = mx_pack4_scaled(a, c, d, e, sc, lim);
    else
      r = mx_pack4_inrange(a, c, d, e);
    out[w] = r;
  }
}

hipError_t launch_e4m3_pack_patterns(uint32_t first, int64_t n, int variant, float sc, uint8_t* out,
                                     hipStream_t stream) {
  const int64_t nwords = n >> 2;
  if (nwords == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((nwords + 255) / 256, 8192);
  hipLaunchKernelGGL(e4m3_pack_patterns_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, first, nwords, variant,
                     sc, 448.0f * sc, reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

}  // namespace mxfa

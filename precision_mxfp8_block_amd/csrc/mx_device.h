// Device-side MX helpers for gfx950 (CDNA4): E8M0 scale from exponent bits, saturating E4M3 pack
// on the hardware converter, wave reductions, and the operand layouts of the scaled MFMA.
//
// Lane layouts of the scaled matrix instructions, as measured on gfx950:
//   v_mfma_scale_f32_32x32x64_f8f6f4 (A: 32 x 64, B: 64 x 32, both 8 VGPRs of E4M3 per lane):
//     lane l holds row r = l % 32 of A (column r of B); with h = l / 32, bytes 0-15 are
//     k = 16h + [0,16) and bytes 16-31 are k = 32 + 16h + [0,16). The E8M0 scale of row r's
//     k-block kb (k in [32kb, 32kb+32)) is taken from lane r + 32kb, byte `opsel` of the scale VGPR.
//     Accumulator: lane l holds column l % 32, rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
//   Only two facts matter to the kernels: the contraction order inside an MFMA is free as long as
//   A and B agree on it, and the 16 bytes at the same byte offset of lanes r and r+32 form one
//   scale block.
//   ds_read_b64_tr_b8: in each group of 16 lanes, destination lane j receives byte b = byte (j & 7)
//     of the 8 bytes addressed by lane 2b + (j >> 3) of the group.
//   v_permlane32_swap(x, x): every lane receives x of lane l % 32 and of lane l % 32 + 32.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

typedef int mx_v8i __attribute__((ext_vector_type(8)));
typedef int mx_v4i __attribute__((ext_vector_type(4)));
typedef int mx_v2i __attribute__((ext_vector_type(2)));
typedef float mx_v16f __attribute__((ext_vector_type(16)));
typedef float mx_v4f __attribute__((ext_vector_type(4)));
typedef unsigned int mx_u32x4 __attribute__((ext_vector_type(4)));

#define MX_LDS __attribute__((address_space(3)))

// E8M0 code of a block from the bit pattern of its absolute maximum (sign already clear): the
// fp32 exponent field minus 8 (= floor(log2 amax) - 8 + 127, the largest E4M3 exponent being 8),
// clamped at 0; 255 when amax is Inf or NaN (bit patterns >= 0x7f800000 order above all finite
// magnitudes as integers). This is the "bit extraction instead of logarithms" scale rule.
__device__ __forceinline__ uint32_t mx_code_from_amax_bits(uint32_t amax_bits) {
  uint32_t e = amax_bits >> 23;
  if (e >= 255u) return 255u;
  return e > 8u ? e - 8u : 0u;
}

// 2^(127 - code) as an fp32 (exact for code <= 253; finite amax never gives a code above 246).
__device__ __forceinline__ float mx_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// Two floats -> two E4M3 bytes, round to nearest even, saturating at +-448. The hardware converter
// turns out-of-range values into NaN, so values are clamped with v_med3 first (NaN blocks are
// handled by the caller through code 255).
__device__ __forceinline__ uint32_t mx_pack2_lo(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}
__device__ __forceinline__ uint32_t mx_pack2_hi(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true);
}
// Four floats already known to lie in [-448, 448] (no clamp needed), e.g. P * 256 <= 256.
__device__ __forceinline__ uint32_t mx_pack4_inrange(float a, float b, float c, float d) {
  // the first conversion writes bytes 0-1 and the second bytes 2-3, so the register the first one
  // starts from is irrelevant: a's own (no zeroing move)
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)r, true);
}
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d) {
  return mx_pack2_hi(c, d, mx_pack2_lo(a, b, 0u));
}

// Four floats -> four E4M3 bytes of x / sc (sc a power of two, lim = 448 sc), round to nearest even,
// saturating: the scaled conversion does not saturate, so the inputs are clamped to +-lim first.
// Same bytes as clamping x / sc to +-448 and converting (x / sc is exact for a power-of-two sc).
__device__ __forceinline__ uint32_t mx_pack4_scaled(float a, float b, float c, float d, float sc, float lim) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  a = __builtin_amdgcn_fmed3f(a, -lim, lim);
  b = __builtin_amdgcn_fmed3f(b, -lim, lim);
  c = __builtin_amdgcn_fmed3f(c, -lim, lim);
  d = __builtin_amdgcn_fmed3f(d, -lim, lim);
  // the first conversion writes bytes 0-1, the second bytes 2-3: the initial value is irrelevant
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, a), a, b, sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, sc, true);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// max(a, b, c) in one v_max3_f32. Written as asm because the compiler, in IEEE mode, first
// quiets (canonicalizes) every input that comes from an MFMA, which costs one extra instruction
// per element; MFMA results are never signalling NaNs.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// max(acc, |a|, |b|) in one v_max3_f32 with absolute-value source modifiers (used for block maxima of
// non-negative running values). A NaN operand does not propagate (IEEE maxNum), an infinity does.
__device__ __forceinline__ float max3_abs(float acc, float a, float b) {
  float d;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(d) : "v"(acc), "v"(a), "v"(b));
  return d;
}

// max(|a|, |b|, |c|) in one v_max3_f32 with absolute-value modifiers on all three sources (no separate
// sign-clearing instruction); NaN and infinity behave as in max3_abs.
__device__ __forceinline__ float max3_abs3(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// A pointer the caller knows to be wave-uniform, moved to scalar registers (a buffer resource built
// from a value in vector registers would need a loop over its distinct values).
__device__ __forceinline__ void* mx_uniform_ptr(void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's 16 bytes at
// base + voff land at lds_dst + 16 l. Written as asm so that the compiler does not treat later LDS
// reads as dependent on it (it would wait for every outstanding vector memory operation before the
// next LDS read); the caller waits (s_waitcnt vmcnt) before reading the destination. lds_dst and base
// must be wave-uniform. M0 carries the LDS address; no other code here keeps a value in M0.
__device__ __forceinline__ void mx_lds_dma16(MX_LDS void* lds_dst, const void* base, uint32_t voff) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m), "v"(voff), "s"(mx_uniform_ptr((void*)base))
               : "memory");
}

// mx_lds_dma16 with the non-temporal hint, for data read exactly once (it is not kept in the caches
// for reuse).
__device__ __forceinline__ void mx_lds_dma16_nt(MX_LDS void* lds_dst, const void* base, uint32_t voff) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m), "v"(voff), "s"(mx_uniform_ptr((void*)base))
               : "memory");
}

// The same for 4 bytes per lane (global_load_lds_dword): lane l's word lands at lds_dst + 4 l.
__device__ __forceinline__ void mx_lds_dma4(MX_LDS void* lds_dst, const void* base, uint32_t voff) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(m), "v"(voff), "s"(mx_uniform_ptr((void*)base))
               : "memory");
}

// The same with a 64-bit per-lane address (the lanes may read from different arrays).
__device__ __forceinline__ void mx_lds_dma4_addr(MX_LDS void* lds_dst, const void* addr) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m), "v"(addr) : "memory");
}


// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS row. With 64 four-byte banks, a
// wave's 16-byte row reads (16 consecutive rows, one chunk) and the transposed 8-byte reads of
// ds_read_b64_tr_b8 (rows {0-3, 8-11} or {4-7, 12-15} of a 16-row group, two adjacent chunks) both
// touch 16 distinct (row parity, physical chunk) pairs, i.e. no bank conflicts. k = (row >> 1) & 7,
// result = k with its two low bits exchanged.
__device__ __forceinline__ int lds_swz(int row) {
  const int k = (row >> 1) & 7;
  return (k & 4) | ((k & 1) << 1) | ((k >> 1) & 1);
}

// Sum over the 64 lanes of a wave, returned in every lane: DPP within rows of 16 (after the quad
// steps each group of lanes holds one value, so the mirrors add the partner group), then the
// permlane16 and permlane32 swaps across rows. The wave must be fully active.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false);  // row_mirror
  auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = (uint32_t)s16[0] + (uint32_t)s16[1];
  auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (uint32_t)s32[0] + (uint32_t)s32[1];
}

// A 64-bit value the caller knows to be wave-uniform, moved to scalar registers (so that addresses
// derived from it stay scalar and uniform loads become scalar loads).
__device__ __forceinline__ int64_t mx_uniform_i64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Workgroup id -> work item of the attention kernels, items being (pair, tile) with pair = sequence *
// heads + head. Consecutive workgroup ids are dispatched to the 8 XCDs in turn (id % 8); XCD x takes
// the pairs x, x + 8, x + 16, ... and runs each pair's tiles back to back, so one head's K and V (or Q
// and dO) stay in one XCD's L2, and the heads of every sequence spread over all XCDs: a jagged batch
// gives each XCD the same share of long and short sequences. The grid is mx_pair_grid(pairs, tiles);
// ids that fall past the last pair give -1. reverse runs each XCD's pairs last to first.
//
// For a uniform batch (every sequence at the maximum length) every pair carries the same work, and the
// backward launcher takes the contiguous order instead (mx_item_order): XCD x runs one contiguous
// range of about total / 8 items, a pair's tiles still back to back; the grid is the item count.
// Measured on MI355X (B=4 H=16 N=4096, D=128): with both backward passes in this order the dQ pass
// takes 270 us instead of 311 us (causal: 160 instead of 193 us); the main pass and the forward do not
// change. The choice never affects results: both orders visit every item once.
__host__ __device__ __forceinline__ int64_t mx_pair_grid(int64_t pairs, int64_t tiles) {
  return (pairs + 7) / 8 * 8 * tiles;
}
__device__ __forceinline__ int mx_pair_item(int bid, int tiles, int pairs, bool reverse = false) {
  const int x = bid & 7, slot = bid >> 3;
  const int pl = slot / tiles, t = slot - pl * tiles;
  const int pair = (reverse ? (pairs + 7) / 8 - 1 - pl : pl) * 8 + x;
  return pair < pairs ? pair * tiles + t : -1;
}
__device__ __forceinline__ int mx_range_item(int bid, int total, bool reverse = false) {
  const int per = total >> 3, rem = total & 7;
  const int x = bid & 7, slot = bid >> 3;
  const int cnt = per + (x < rem ? 1 : 0);  // ids x, x + 8, ... below total
  return x * per + (x < rem ? x : rem) + (reverse ? cnt - 1 - slot : slot);
}
// Item order and grid of an attention launch: contiguous ranges for a uniform batch (every sequence at
// the maximum length: total tokens = sequences x maximum, on both sides), else pairs dealt to XCDs.
struct MxItemOrder {
  int contiguous;
  int64_t grid;
};
__host__ __forceinline__ MxItemOrder mx_item_order(int64_t total_q, int64_t total_k, int nseq, int max_q, int max_k,
                                                   int64_t pairs, int64_t tiles) {
  MxItemOrder o;
  o.contiguous = total_q == (int64_t)nseq * max_q && total_k == (int64_t)nseq * max_k;
  o.grid = o.contiguous ? pairs * tiles : mx_pair_grid(pairs, tiles);
  return o;
}
__device__ __forceinline__ int mx_item(int contiguous, int bid, int total, int tiles, int pairs, bool reverse = false) {
  return contiguous ? mx_range_item(bid, total, reverse) : mx_pair_item(bid, tiles, pairs, reverse);
}

// Offsets of sequence s in the compact and padded layouts from the device cu_seqlens, computed by
// every wave on its own (no barrier; the wave must be fully active): blocks32 = sum_{r<s}
// ceil(L_r/32), padded = sum_{r<s} round_up(L_r,128). The sums fit 32 bits for any token count
// whose data fits in device memory.
struct SeqOffsets {
  int64_t blocks32;
  int64_t padded;
};
__device__ __forceinline__ SeqOffsets seq_offsets(const int32_t* cu, int s) {
  const int lane = threadIdx.x & 63;
  uint32_t b = 0, p = 0;
  for (int r = lane; r < s; r += 64) {
    const uint32_t L = (uint32_t)(cu[r + 1] - cu[r]);
    b += (L + 31u) >> 5;
    p += (L + 127u) >> 7;
  }
  SeqOffsets o;
  o.blocks32 = mx_uniform_i64((int64_t)wave_sum_u32(b));
  o.padded = mx_uniform_i64((int64_t)wave_sum_u32(p)) << 7;
  return o;
}

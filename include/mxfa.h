/*
 * mxfa.h -- C ABI of the MXFP8 block-scaled attention library for AMD MI355X (gfx950).
 *
 * The operations follow four web pages about MXFP8 FlashAttention-4 (cited by short name):
 *   [AE] andresseo.expert, "MXFP8 FlashAttention-4 Hits 2.85 Petaflops in Meta's Production
 *        Training", section "Inside the TMEM Bargain and Zero-Gather Jagged Pipeline" (AE-TMEM).
 *   [BR] brifing.si, "Meta's FlashAttention-4 Achieves 2.85 PF/s with MXFP8 on Blackwell GPUs",
 *        numbered items.
 *   [TC] theclarity.today, "Meta's MXFP8 FlashAttention-4 kernel, tackling TMEM scale-factor
 *        constraints, hits up to 1.6x over BF16", paragraphs 1-4.
 *   [KC] kongchang.com, "Low-Precision FlashAttention-4: End-to-End Block-Scaled Attention on
 *        Blackwell", section "Why MXFP8".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer is a DEVICE pointer unless marked (host). Pointers must be 16-byte aligned;
 *    row strides (ld_x) must be multiples of 8 elements.
 *  - The caller owns every buffer (inputs, outputs, workspace). The library never allocates,
 *    frees or synchronizes; it keeps no state between calls and may be called from any thread.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default stream).
 *  - All argument checks run on the host before anything is enqueued: a call that returns an
 *    error has enqueued nothing and written nothing. The thread-local message of the last error
 *    is available from mxfa_last_error_message().
 *  - Device-resident cu_seqlens arrays (int32, nseq + 1 entries, cu[0] = 0, non-decreasing,
 *    cu[nseq] = total tokens, every length <= the host max_seqlen) are a precondition that the
 *    host cannot check without a synchronization; violating it is undefined behaviour.
 *
 * MX data (MXFP8, OCP microscaling [KC]): an E4M3 payload byte per element and one E8M0 scale
 * byte (value 2^(e-127), 255 = NaN) per block of 32 elements. A matrix X is [T, C] row-major
 * (T tokens of a jagged batch, C = heads * head_dim columns); token blocks start at each
 * sequence start, the last block of a sequence may be partial. Block shapes:
 *   MXFA_ROW32: 1 x 32 along the columns       scales [T][C/32]
 *   MXFA_COL32: 32 x 1 along the tokens        scales [NB][C]
 *   MXFA_SQ32 : 32 x 32 square blocks          scales [NB][C/32] (+ optional transpose [C/32][NB])
 * with NB = sum over sequences of ceil(L/32) ("compact" layout, written by the quantizer).
 * The attention entry points read scales in the "padded" layout written by
 * mxfa_varlen_scale_scatter: sequence s starts at token row P_s = sum_{r<s} round_up(L_r, 128)
 * (block row P_s/32), rows in the padding are 0x00 [AE-TMEM: only the scale tensors are padded
 * and aligned, the FP8 data stays compact]. When every length is a multiple of 128 the two
 * layouts coincide and no scatter is needed.
 */
#ifndef MXFA_H
#define MXFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFA_OK = 0,
  MXFA_ERR_INVALID = 1,     /* bad pointer, size, alignment, enum or workspace */
  MXFA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim != 128) */
  MXFA_ERR_HIP = 3          /* a HIP launch failed; see mxfa_last_error_message() */
} mxfa_status;

typedef enum { MXFA_ROW32 = 0, MXFA_COL32 = 1, MXFA_SQ32 = 2 } mxfa_block;

typedef enum {
  MXFA_DQ_FP32 = 0,        /* dQ partials of the KV tiles summed in FP32 [AE, Bench: FP32 dQ] */
  MXFA_DQ_FP16_STATIC = 1  /* dQ partials times a static power-of-two scale sigma, summed in FP16
                              [AE-TMEM: dQ reduction in FP16 with static scaling; BR item 6] */
} mxfa_dq_mode;

/* Element format of an MX payload. E4M3 (MXFP8) everywhere; for the forward's q and k only, in ROW32
 * blocks, also E2M1 (MXFP4: two elements per byte, element 2i in the low nibble of byte i, magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6) or E2M3 (MXFP6: a block's 32 six-bit codes in 24 bytes, code j at bits
 * 6j..6j+5 of a little-endian bit string, blocks in pairs as mxfa_quantize_e2m3 describes; magnitudes
 * f/8 below 1, then 2^e (1 + f/8) up to 7.5)
 * [brifing.si "Future directions": MXFP6 and MXFP4 as the next precisions; TC paragraph 1: the
 * block-scaled matrix units run MXFP8, MXFP6 and MXFP4]. */
typedef enum { MXFA_E4M3 = 0, MXFA_E2M1 = 1, MXFA_E2M3 = 2 } mxfa_elem;

/* One MX operand: payload [T, C] (row stride C bytes; C/2 for E2M1, 3C/4 for E2M3) and its scale tensor in
 * `mode`'s layout. A zero-initialised struct has elem = MXFA_E4M3. */
typedef struct {
  const uint8_t* data;
  const uint8_t* scale;
  mxfa_block mode;
  mxfa_elem elem;
} mxfa_mx;

/* Attention problem shared by the forward and the backward.
 * q: [T_q, H*D]; k, v: [T_k, H*D]; scales in the PADDED layout.
 * Allowed modes (scales along the MMA contraction dimension [TC paragraph 3]):
 *   q, k : ROW32 (along D) or SQ32 (square; one payload serves both GEMM directions [AE-TMEM])
 *   v    : COL32 (along the keys, for O = P V) or SQ32.
 * Element formats: E4M3 for all three, or (forward entry points only) q and k both E2M1 or both
 * E2M3 in ROW32 with v E4M3: S = Q K^T then runs on the FP4 / FP6 form of the scaled MMA; the
 * backward entry points return MXFA_ERR_UNSUPPORTED for such operands.
 * Causal masking is top-left aligned (key j visible to query i iff j <= i, positions counted
 * from each sequence start). head_dim must be 128. */
typedef struct {
  mxfa_mx q, k, v;
  const int32_t* cu_seqlens_q; /* device, nseq + 1 */
  const int32_t* cu_seqlens_k; /* device, nseq + 1 */
  int nseq;
  int max_seqlen_q;  /* (host) max length over sequences */
  int max_seqlen_k;  /* (host) */
  int64_t total_q;   /* (host) T_q = cu_seqlens_q[nseq] */
  int64_t total_k;   /* (host) T_k = cu_seqlens_k[nseq] */
  int num_heads;
  int head_dim;
  float softmax_scale; /* c in softmax(c Q K^T) */
  int causal;
} mxfa_attn_args;

/* MX quantization of a bf16 matrix [AE-TMEM: 32-element blocks, the scale from bit extraction
 * instead of logarithms or division; BR item 6: square 32x32 blocks].
 * Per block: amax = max |x|; scale code e = clamp(exponent_field(amax) - 8, 0, 254), 255 if the
 * block holds NaN or Inf; payload = E4M3(x * 2^(127-e)) with round-to-nearest-even and saturation
 * to +-448 (NaN blocks: every payload byte 0x7F).
 *   x          : bf16 bits [T, ld_x] (first C columns used)
 *   C          : columns, multiple of 32
 *   cu_seqlens : sequence boundaries (device). ROW32 does not use it (may be NULL).
 *   nseq, max_seqlen : (host) sequence count and maximum length (COL32 / SQ32)
 *   data_out   : [T, C] payload; scale_out: compact scales (see above)
 *   scale_t_out: SQ32 only, nullable: the same scales transposed, [C/32][NB] ("dual scale
 *                layouts" [BR item 7]); must be NULL for other modes. */
mxfa_status mxfa_quantize(const uint16_t* x, int64_t ld_x, int64_t T, int C, const int32_t* cu_seqlens, int nseq,
                          int max_seqlen, mxfa_block mode, uint8_t* data_out, uint8_t* scale_out,
                          uint8_t* scale_t_out, void* stream);

/* COL32 and ROW32 quantization of one bf16 matrix from a single read: the payloads and scales that
 * mxfa_quantize writes for MXFA_COL32 and for MXFA_ROW32, byte for byte, for an operand contracted
 * over the tokens in one GEMM and over its columns in another (V: P V in the forward, dP = dO V^T in
 * the backward) [BR item 7: both scale layouts from one producer pass; TC paragraph 3: the scale
 * blocks run along each GEMM's contraction dimension].
 *   x, ld_x, T, C, cu_seqlens, nseq, max_seqlen : as mxfa_quantize (cu_seqlens required; rows outside
 *                the sequences are not written)
 *   data_col, scale_col : the COL32 payload [T, C] and its compact scales
 *   data_row, scale_row : the ROW32 payload [T, C] and its scales [T][C/32]
 * All five pointers 16-byte aligned. Errors as mxfa_quantize. */
mxfa_status mxfa_quantize_col32_row32(const uint16_t* x, int64_t ld_x, int64_t T, int C, const int32_t* cu_seqlens,
                                      int nseq, int max_seqlen, uint8_t* data_col, uint8_t* scale_col,
                                      uint8_t* data_row, uint8_t* scale_row, void* stream);

/* MXFP4 quantization of a bf16 matrix in ROW32 blocks (1 x 32 along the columns), by the OCP MX rule
 * for E2M1 [brifing.si "Future directions"; the rule of mxfa_quantize with E2M1's largest exponent]:
 * scale code e = clamp(exponent_field(amax) - 2, 0, 254), 255 if the block holds NaN or Inf; element
 * = the E2M1 magnitude nearest to |x| * 2^(127-e) (ties to the even code, saturating at 6) with x's
 * sign bit (NaN blocks: payload 0).
 *   x          : bf16 bits [T, ld_x] (first C columns used); C a multiple of 32
 *   data_out   : [T, C/2] payload, element 2i in the low nibble of byte i
 *   scale_out  : [T][C/32] (the ROW32 layout; scatter it with mxfa_varlen_scale_scatter as for
 *                E4M3 payloads). x, data_out and scale_out 16-byte aligned. */
mxfa_status mxfa_quantize_e2m1(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data_out,
                               uint8_t* scale_out, void* stream);

/* MXFP6 quantization of a bf16 matrix in ROW32 blocks, by the same rule with E2M3 elements
 * [brifing.si "Future directions"]: scale code e = clamp(exponent_field(amax) - 2, 0, 254) (7.5 =
 * 1.875 * 2^2), 255 for NaN/Inf blocks; element = the E2M3 magnitude nearest to |x| * 2^(127-e), ties
 * to the even code, saturating at 7.5, with x's sign bit (NaN blocks: payload 0).
 *   C         : columns, a multiple of 64
 *   data_out  : [T, 3C/4] payload. A block's codes form a 24-byte little-endian bit string (code j at
 *               bits 6j .. 6j + 5); the blocks of a row go in pairs (2p, 2p + 1) of 48 bytes at 48p:
 *               bytes 0-15 of block 2p, bytes 0-15 of block 2p + 1, bytes 16-23 of block 2p, bytes
 *               16-23 of block 2p + 1 (each block one 16-byte and one 8-byte piece)
 *   scale_out : [T][C/32]; other arguments as mxfa_quantize_e2m1. */
mxfa_status mxfa_quantize_e2m3(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data_out,
                               uint8_t* scale_out, void* stream);

/* Jagged zero-gather scale path [AE-TMEM: split addressing; BR item 5: lightweight scatter that
 * moves scale factors without changing values]. Copies compact scales (as written by
 * mxfa_quantize) to the padded layout: sequence s starts at token row P_s (ROW32) or block row
 * P_s/32 (COL32, SQ32), P_s = sum_{r<s} round_up(L_r, 128); rows inside each sequence's padding
 * are written 0x00; rows at and beyond the total padded count are not written.
 *   padded_rows: (host) rows of padded_out in the layout's row unit (token rows for ROW32, block
 *   rows otherwise); must be >= the total padded count. */
mxfa_status mxfa_varlen_scale_scatter(const uint8_t* compact, const int32_t* cu_seqlens, int nseq, int max_seqlen,
                                      int C, mxfa_block mode, uint8_t* padded_out, int64_t padded_rows,
                                      void* stream);

/* The device's E4M3 conversion, exposed so that it can be checked against an independent encoder on
 * every fp32 bit pattern [KC "Why MXFP8": E4M3 elements, 448 the largest finite magnitude; AE-TMEM:
 * P converted online to E4M3]. Byte i of out is the E4M3 code of the fp32 whose bit pattern is
 * first + i (mod 2^32), computed by the routine the kernels use for
 *   variant 0 : unscaled values (quantizers, the MXFP8 O and gradient epilogues): round to nearest
 *               even, saturating at +-448, the sign kept on zero results
 *   variant 1 : x / sc with sc a power of two (dS_q and projection epilogues), same rounding and
 *               saturation; sc in [2^-126, 2^119]
 *   variant 2 : values already in [-448, 448] (P * 256); bytes for other patterns are unspecified
 * NaN patterns give unspecified bytes (the kernels mark NaN blocks through scale code 255).
 *   n   : (host) number of patterns, a multiple of 4 in [0, 2^32]
 *   out : device bytes [n], 4-byte aligned, written entirely (caller owns it)
 * MXFA_ERR_INVALID for a bad variant, sc, n or pointer, before any launch. */
mxfa_status mxfa_e4m3_pack_patterns(uint32_t first, int64_t n, int variant, float sc, uint8_t* out, void* stream);

/* Host helper: padded row count for given host-side sequence lengths (NULL-safe). */
int64_t mxfa_padded_token_rows(const int32_t* cu_seqlens_host, int nseq);

/* Attention forward [AE-TMEM: S = Q K^T, FP32 online softmax, P converted online to MXFP8, O = P V;
 * TC paragraph 1: softmax in FP32, then P quantized with its scales in the same step; BR item 4:
 * constant scale for P because softmax output lies in [0, 1]].
 * Per 128-row query tile and 128-row key tiles: m' = max(m, rowmax S); P = exp(c (S - m'));
 * l = exp(c (m - m')) l + rowsum P; P quantized to E4M3 with the static block scale 2^-8;
 * O = exp(c (m - m')) O + deq(P) V. Outputs O / l as bf16 and LSE = c m + ln l.
 *   o  : bf16 [T_q, H*D]
 *   lse: fp32 [H][T_q]; rows of a sequence with no keys get O = 0 and LSE = -inf. */
mxfa_status mxfa_fwd(const mxfa_attn_args* a, uint16_t* o, float* lse, void* stream);

/* How the forward scales each 32-key block of P before the E4M3 pack. */
typedef enum {
  MXFA_P_STATIC = 0,        /* 2^-8 on every block (code 119): P <= 1, so 1.0 maps to 256
                               [BR item 4: constant scale because softmax output lies in [0, 1]] */
  MXFA_P_BLOCK_DYNAMIC = 1  /* per (query row, 32-key block of the tile): the MX scale rule applied to
                               the block's largest P, code = floor(log2 max P) - 8 + 127 clamped at 0,
                               payload E4M3(P 2^(127-code)) saturated at 448; a block holding the row
                               maximum gets code 119 [AE-TMEM: per-block scales from the block maximum,
                               which the row-max pass of the online softmax already visits] */
} mxfa_p_scale;

/* Attention forward with a choice of P scale; mxfa_fwd(a, o, lse, s) is
 * mxfa_fwd_p_scale(a, MXFA_P_STATIC, o, lse, s). The dynamic scale keeps small probabilities out of
 * the E4M3 subnormal range (a block whose largest P is far below the row maximum gets a finer
 * scale); the row sum l still adds the FP32 P. Same arguments, layouts and errors as mxfa_fwd;
 * MXFA_ERR_INVALID for any other p_scale value. */
mxfa_status mxfa_fwd_p_scale(const mxfa_attn_args* a, mxfa_p_scale p_scale, uint16_t* o, float* lse, void* stream);

/* Attention forward with O written as MXFP8 for the next projection [AE-TMEM: FP8 outputs with their
 * scales, quantized in the epilogue of the kernel that produces them; TC paragraph 3: scales along the
 * next GEMM's contraction dimension, here D]. O = O_acc / l in FP32 is quantized in ROW32 blocks
 * (32 of D per token and head) by the rule of mxfa_quantize; bf16 O can be written in the same pass
 * (the backward needs it for Delta).
 *   o       : bf16 [T_q, H*D], or NULL to skip it
 *   o_data  : E4M3 [T_q, H*D], 4-byte aligned, or NULL to skip it (not both NULL)
 *   o_scale : E8M0 [T_q, H*D/32] (the ROW32 layout of mxfa_quantize), 4-byte aligned; required with o_data
 *   p_scale, lse, stream: as mxfa_fwd_p_scale. Same problem checks and errors as mxfa_fwd. */
mxfa_status mxfa_fwd_mx_out(const mxfa_attn_args* a, mxfa_p_scale p_scale, uint16_t* o, uint8_t* o_data,
                            uint8_t* o_scale, float* lse, void* stream);

/* Workspace bytes mxfa_bwd needs for problem `a` (host struct; only nseq, max_seqlen_q/k, total_q and
 * num_heads are read): one 16 KB FP8 dS tile plus 16 bytes of block codes per (head, sequence,
 * 128-query tile, 128-key tile) of the longest sequences, i.e. H * nseq * ceil(max_q/128) *
 * ceil(max_k/128) tiles, then two fp32 [H][T_q] row vectors (-Delta and the softmax exponent
 * offsets); each region 256-byte aligned. 0 if `a` is NULL or malformed. The size does not depend
 * on dq_mode. */
size_t mxfa_bwd_workspace_size(const mxfa_attn_args* a, mxfa_dq_mode dq_mode);

/* Attention backward with recomputation [AE-TMEM: five GEMMs; Q, K and dO in square 32x32 blocks
 * so one E4M3 payload serves the plain and the transposed GEMM; dS quantized once per square block
 * with a wave-wide absolute maximum; dQ reduced in FP16 with a static scale, or in FP32].
 * The dQ reduction runs over the KV tiles in order (per query tile: acc = fp16(acc + fp16(sigma
 * dS_q K_tile)) or acc = fl32(acc + dS_q K_tile)), so the result is deterministic.
 *   a        : the forward's problem; q and k must be SQ32, v is ignored here
 *   v_d      : V quantized along D (ROW32 or SQ32), padded layout, for dP = dO V^T
 *   dout     : dO quantized SQ32, padded layout
 *   o, dout_bf16 : bf16 [T_q, H*D] forward output and incoming gradient (for Delta = rowsum(dO o O))
 *   lse      : fp32 [H][T_q] from mxfa_fwd on the same inputs
 *   dq_mode, dq_static_scale : accumulator type; sigma must be a positive power of two
 *                              (FP16 holds sigma * dQ; the finalize divides by sigma)
 *   workspace, workspace_bytes : >= mxfa_bwd_workspace_size(...), 256-byte aligned
 *   dq, dk, dv : bf16 [T, H*D] outputs. */
mxfa_status mxfa_bwd(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o,
                     const uint16_t* dout_bf16, const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale,
                     void* workspace, size_t workspace_bytes, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                     void* stream);

/* mxfa_bwd without a workspace argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The workspace lives in a
 * fixed array of mxfa_bwd_no_alloc_max_workspace() bytes (64 MiB) that the library holds on each GPU
 * it runs on until the process ends; the call itself allocates and frees nothing.
 *   Arguments, layouts and results as mxfa_bwd (dq, dk, dv required).
 *   MXFA_ERR_INVALID (nothing enqueued) when mxfa_bwd_workspace_size(a, dq_mode) exceeds the array:
 *   such problems need mxfa_bwd with a caller-owned workspace.
 *   Every call on one GPU uses that GPU's array: calls that overlap in time on the same GPU (other
 *   streams, other threads) race and give wrong results. Every byte the kernels read from the array is
 *   written earlier in the same call, so nothing needs clearing between calls. */
mxfa_status mxfa_bwd_no_alloc(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o,
                              const uint16_t* dout_bf16, const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale,
                              uint16_t* dq, uint16_t* dk, uint16_t* dv, void* stream);

/* Size in bytes of the fixed workspace array behind mxfa_bwd_no_alloc (host only). */
size_t mxfa_bwd_no_alloc_max_workspace(void);

/* MXFP8 gradient outputs (E4M3 payloads with their E8M0 codes). */
typedef struct {
  uint8_t* dq;        /* [T_q, H*D] */
  uint8_t* dq_scale;  /* SQ32 codes, compact layout of mxfa_quantize: [sum_s ceil(Lq_s/32)][H*D/32] */
  uint8_t* dk;        /* [T_k, H*D] */
  uint8_t* dk_scale;  /* [sum_s ceil(Lk_s/32)][H*D/32] */
  uint8_t* dv;        /* [T_k, H*D] */
  uint8_t* dv_scale;  /* [sum_s ceil(Lk_s/32)][H*D/32] */
  /* Optional (each may be NULL): the same codes in the transposed layout [H*D/32][NB] (NB the
   * block rows above), the second layout of the producers' format [BR item 7], which the weight
   * gradient of the projection consumes (mxfa_linear_bwd_weight). */
  uint8_t* dq_scale_t;
  uint8_t* dk_scale_t;
  uint8_t* dv_scale_t;
} mxfa_grad_mx;

/* Attention backward with the gradients written as MXFP8 [BR item 8 / AE-TMEM: quantized gradients
 * exposed to the next layer, quantized in the epilogue of the kernel that produces them]. Each
 * gradient (the FP32 value whose bf16 rounding mxfa_bwd writes) is quantized in square 32 x 32
 * blocks (32 tokens from each sequence start x 32 of D) by the rule of mxfa_quantize, so one payload
 * serves the next products along D (the projection's input gradient) and along the tokens (its
 * weight gradient); a partial last block takes its maximum over the rows inside the sequence.
 *   dq, dk, dv : bf16 outputs as in mxfa_bwd, all set or all NULL
 *   mx_out     : host struct of device pointers (the six payloads and codes all set, payloads 16-byte
 *                aligned; the three transposed code grids each optional), or NULL
 *   at least one of the two sets; everything else as mxfa_bwd. */
mxfa_status mxfa_bwd_mx_out(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o,
                            const uint16_t* dout_bf16, const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale,
                            void* workspace, size_t workspace_bytes, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                            const mxfa_grad_mx* mx_out, void* stream);

/* Fused RMSNorm + quantize producer [AE-TMEM: quantization fused into RMSNorm, no separate
 * global-memory pass; BR item 7: FP8 output with dual scale layouts in one pass].
 * y = fl32(fl32(x * r) * gamma[c]), r = 1 / sqrtf(ss / C + eps), ss = sum of x^2 over the row
 * rounded once to fp32; then SQ32 quantization of y (token blocks aligned to sequence starts).
 *   x: bf16 [T, ld_x]; gamma: fp32 [C] (device); outputs as mxfa_quantize in SQ32 mode, with
 *   scale_t_out nullable. */
mxfa_status mxfa_rmsnorm_quantize(const uint16_t* x, int64_t ld_x, int64_t T, int C, const float* gamma, float eps,
                                  const int32_t* cu_seqlens, int nseq, int max_seqlen, uint8_t* data_out,
                                  uint8_t* scale_out, uint8_t* scale_t_out, void* stream);

/* Fused projection GEMM + quantize producer [AE-TMEM: quantization fused into the epilogue of the
 * projection GEMM, no separate global-memory pass; BR item 7: FP8 output with dual scale layouts in
 * one pass]. Y = deq(x) deq(w)^T accumulated in FP32, then SQ32 quantization of Y exactly as
 * mxfa_quantize does it (token blocks aligned to sequence starts). Y itself is never stored.
 *   x          : [T, C_in] payload with compact SQ32 (or ROW32) scales, e.g. from
 *                mxfa_rmsnorm_quantize
 *   w          : [C_out, C_in] payload with ROW32 scales [C_out][C_in/32] (1 x 32 along C_in)
 *   C_in, C_out: multiples of 128 (C_out = heads * head_dim: the output is [T, heads, head_dim])
 *   cu_seqlens, nseq, max_seqlen : as mxfa_quantize (device cu_seqlens, host sizes)
 *   data_out [T, C_out]; scale_out [NB][C_out/32]; scale_t_out nullable, [C_out/32][NB].
 * The FP32 accumulation order is the hardware's, so a payload byte or scale can differ from a
 * correctly rounded Y where Y lies within rounding of an E4M3 midpoint or a block maximum within
 * rounding of a power of two. */
mxfa_status mxfa_linear_quantize(mxfa_mx x, mxfa_mx w, int64_t T, int C_in, int C_out, const int32_t* cu_seqlens,
                                 int nseq, int max_seqlen, uint8_t* data_out, uint8_t* scale_out,
                                 uint8_t* scale_t_out, void* stream);

/* Backward of the projection, data gradient [BR item 7; AE-TMEM: square 32 x 32 blocks serve the
 * plain and the transposed product]: dX = dY W accumulated in FP32, written as bf16 (accumulate = 0)
 * or added in FP32 to the bf16 dx already there (accumulate = 1: an input that feeds two projections,
 * such as the key and value projections of one activation, gets the sum of both products). It is
 * the projection kernel with dY as its input and W^T as its weight.
 *   dy     : [T, C_out] payload with compact SQ32 (or ROW32) scales, e.g. the MXFP8 gradients of
 *            mxfa_bwd_mx_out
 *   wt     : W^T [C_in, C_out] payload with ROW32 scales [C_in][C_out/32] (1 x 32 along C_out, the
 *            contraction dimension), i.e. mxfa_quantize of the transposed weight
 *   C_out  : multiple of 128 in [128, 65536]; C_in: positive multiple of 128
 *   cu_seqlens, nseq, max_seqlen : as mxfa_quantize
 *   dx     : bf16 [T, C_in], 16-byte aligned. No workspace. */
mxfa_status mxfa_linear_bwd_data(mxfa_mx dy, mxfa_mx wt, int64_t T, int C_out, int C_in, const int32_t* cu_seqlens,
                                 int nseq, int max_seqlen, int accumulate, uint16_t* dx, void* stream);

/* Workspace bytes of mxfa_linear_bwd_weight (host only; 0 for invalid sizes). */
size_t mxfa_linear_bwd_weight_workspace_size(int64_t T, int nseq, int C_out, int C_in);

/* Backward of the projection, weight gradient [BR item 7: the producers' second, transposed scale
 * layout exists for this product; AE-TMEM: square blocks]: dW[o, i] = sum over every token of every
 * sequence of deq(dY)[t, o] deq(X)[t, i], FP32. Both operands are SQ32 payloads read through their
 * transposed scale grids, whose rows run along the tokens (the contraction).
 *   dy, dy_scale_t : [T, C_out] E4M3 and its transposed SQ32 codes [C_out/32][NB]
 *   x, x_scale_t   : [T, C_in] E4M3 and [C_in/32][NB] (e.g. mxfa_rmsnorm_quantize's outputs)
 *   NB = sum over sequences of ceil(L/32); C_out, C_in positive multiples of 128; T x C below 2^32
 *   workspace      : device, 16-byte aligned, >= mxfa_linear_bwd_weight_workspace_size(...) bytes
 *                    (token block table and one FP32 partial dW per token chunk, summed in order)
 *   dw             : FP32 [C_out, C_in], 16-byte aligned
 * The FP32 accumulation order is the hardware's (parity by tolerance). */
mxfa_status mxfa_linear_bwd_weight(const uint8_t* dy, const uint8_t* dy_scale_t, const uint8_t* x,
                                   const uint8_t* x_scale_t, int64_t T, int C_out, int C_in,
                                   const int32_t* cu_seqlens, int nseq, int max_seqlen, void* workspace,
                                   size_t workspace_bytes, float* dw, void* stream);

/* Workspace bytes of mxfa_rmsnorm_bwd (host only; 0 for invalid sizes). */
size_t mxfa_rmsnorm_bwd_workspace_size(int64_t T, int C);

/* RMSNorm backward (the producer mxfa_rmsnorm_quantize differentiated with its quantizer passed
 * straight through): with r = 1 / sqrt(mean_c x_c^2 + eps) per token (computed as the forward does),
 *   dx_k = r gamma_k dy_k - x_k r^3 (sum_c gamma_c dy_c x_c) / C     -> bf16 [T, C]
 *   dgamma_c = sum_t dy_tc x_tc r_t                                  -> FP32 [C]
 *   x: bf16 [T, ld_x] (16-byte aligned, ld_x >= C, multiple of 8); dy: bf16 [T, C]; gamma: FP32 [C]
 *   C: multiple of 32 in [32, 2048]
 *   workspace: device, 16-byte aligned, >= mxfa_rmsnorm_bwd_workspace_size(T, C) bytes (per-wave
 *   partial dgamma rows, summed in order) */
mxfa_status mxfa_rmsnorm_bwd(const uint16_t* x, int64_t ld_x, int64_t T, int C, const float* gamma, float eps,
                             const uint16_t* dy, void* workspace, size_t workspace_bytes, uint16_t* dx, float* dgamma,
                             void* stream);

/* Human-readable name of a status code (static string). */
const char* mxfa_status_string(mxfa_status s);

/* Thread-local message describing the last error returned on this thread ("" if none). */
const char* mxfa_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFA_H */

// Internal interface between the C ABI layer (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace mxfa {

struct MxOperand {
  const uint8_t* data;
  const uint8_t* scale;
  int mode;      // 0 ROW32, 1 COL32, 2 SQ32
  int elem = 0;  // 0 E4M3 (one byte per element), 1 E2M1 (two elements per byte), 2 E2M3 (4 per 3 bytes)
};

struct AttnProblem {
  MxOperand q, k, v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int nseq, max_seqlen_q, max_seqlen_k;
  int64_t total_q, total_k;
  int H;
  float softmax_scale;
  int causal;
};

hipError_t launch_quantize(const uint16_t* x, int64_t ld_x, int64_t T, int C, const int32_t* cu, int nseq,
                           int max_seqlen, int mode, uint8_t* data, uint8_t* scale, uint8_t* scale_t,
                           hipStream_t stream);
hipError_t launch_quantize_col32_row32(const uint16_t* x, int64_t ld_x, int C, const int32_t* cu, int nseq,
                                      int max_seqlen, uint8_t* data_col, uint8_t* scale_col, uint8_t* data_row,
                                      uint8_t* scale_row, hipStream_t stream);
// MXFP4 (E2M1) ROW32 quantization: payload [T, C/2], scales [T][C/32].
hipError_t launch_quantize_e2m1(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data, uint8_t* scale,
                               hipStream_t stream);
// MXFP6 (E2M3) ROW32 quantization: payload [T, 3C/4] (24 bytes per block), scales [T][C/32].
hipError_t launch_quantize_e2m3(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data, uint8_t* scale,
                               hipStream_t stream);
// n fp32 bit patterns first, first + 1, ... (mod 2^32) -> E4M3 bytes through pack variant 0/1/2 (n a
// multiple of 4, out 4-byte aligned).
hipError_t launch_e4m3_pack_patterns(uint32_t first, int64_t n, int variant, float sc, uint8_t* out,
                                     hipStream_t stream);
hipError_t launch_scale_scatter(const uint8_t* compact, const int32_t* cu, int nseq, int max_seqlen, int C, int mode,
                                uint8_t* padded, int64_t padded_rows, hipStream_t stream);
hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t ld_x, int C, const float* gamma, float eps,
                                   const int32_t* cu, int nseq, int max_seqlen, uint8_t* data, uint8_t* scale,
                                   uint8_t* scale_t, hipStream_t stream);
// out_bf16 set: Y written as bf16 [T, C_out] (data, scale and scale_t unused) instead of quantized,
// added to the bf16 values already there when accumulate is set.
hipError_t launch_linear_quantize(const MxOperand& x, const MxOperand& w, int64_t T, int C_in, int C_out,
                                  const int32_t* cu, int nseq, int max_seqlen, uint8_t* data, uint8_t* scale,
                                  uint8_t* scale_t, uint16_t* out_bf16, int accumulate, hipStream_t stream);
// Producer backward (linear_bwd.hip).
size_t wgrad_workspace_bytes(int64_t T, int nseq, int C_out, int C_in);
hipError_t launch_linear_wgrad(const uint8_t* dy, const uint8_t* dy_st, const uint8_t* x, const uint8_t* x_st,
                               int64_t T, int C_out, int C_in, const int32_t* cu, int nseq, int max_seqlen,
                               void* workspace, float* dw, hipStream_t stream);
size_t rmsnorm_bwd_workspace_bytes(int64_t T, int C);
hipError_t launch_rmsnorm_bwd(const uint16_t* x, int64_t ld_x, int64_t T, int C, const float* gamma, float eps,
                              const uint16_t* dy, void* workspace, uint16_t* dx, float* dgamma, hipStream_t stream);
// o and o_mx may each be null (not both): bf16 O and/or E4M3 O in ROW32 blocks with its codes.
hipError_t launch_attn_fwd(const AttnProblem& a, int p_dynamic, uint16_t* o, uint8_t* o_mx, uint8_t* o_mx_scale,
                           float* lse, hipStream_t stream);
size_t bwd_workspace_bytes(int64_t Tq, int H, int nseq, int max_q, int max_k);
// MXFP8 gradient outputs: E4M3 payloads [T, H*D] and compact SQ32 codes [blocks][H*D/32].
struct GradMxOut {
  uint8_t *dq, *dq_scale, *dk, *dk_scale, *dv, *dv_scale;
  uint8_t *dq_scale_t, *dk_scale_t, *dv_scale_t;  // transposed code grids [C/32][NB], each nullable
};
// dq, dk, dv (bf16) are all null or all set; mx_out (all six pointers set) may be null.
hipError_t launch_attn_bwd(const AttnProblem& a, const MxOperand& v_d, const MxOperand& dout, const uint16_t* o,
                           const uint16_t* dout_bf16, const float* lse, int dq_fp16, float sigma, void* workspace,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, const GradMxOut* mx_out, hipStream_t stream);

}  // namespace mxfa

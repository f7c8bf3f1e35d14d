// C ABI of the MXFP8 attention library: argument validation (host only, before any launch) and
// dispatch to the kernel launchers. Declarations and the contract of every entry point are in
// include/mxfa.h.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "mxfa.h"
#include "mxfa_internal.h"

namespace {

thread_local std::string g_last_error;

mxfa_status fail(mxfa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mxfa_status ok() {
  g_last_error.clear();
  return MXFA_OK;
}

mxfa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MXFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_mode(int m) { return m == MXFA_ROW32 || m == MXFA_COL32 || m == MXFA_SQ32; }

// Operands of every entry point but the forward's Q and K must be E4M3.
bool e4m3(const mxfa_mx& m) { return m.elem == MXFA_E4M3; }

bool is_pow2(float x) {
  if (!(x > 0.0f) || !std::isfinite(x)) return false;
  int e;
  return std::frexp(x, &e) == 0.5f;
}

constexpr int kMaxGridY = 65535;

mxfa_status check_jagged(const int32_t* cu, int nseq, int max_seqlen, int64_t T, const char* fn) {
  if (!cu) return fail(MXFA_ERR_INVALID, "%s: cu_seqlens is NULL", fn);
  if (!aligned(cu, 4)) return fail(MXFA_ERR_INVALID, "%s: cu_seqlens not 4-byte aligned", fn);
  if (nseq < 1 || nseq > kMaxGridY) return fail(MXFA_ERR_INVALID, "%s: nseq=%d out of [1, %d]", fn, nseq, kMaxGridY);
  if (max_seqlen < 0 || (int64_t)max_seqlen > T)
    return fail(MXFA_ERR_INVALID, "%s: max_seqlen=%d not in [0, T=%lld]", fn, max_seqlen, (long long)T);
  if ((max_seqlen + 31) / 32 > kMaxGridY) return fail(MXFA_ERR_INVALID, "%s: max_seqlen too large", fn);
  return MXFA_OK;
}

mxfa_status check_attn(const mxfa_attn_args* a, const char* fn) {
  if (!a) return fail(MXFA_ERR_INVALID, "%s: args is NULL", fn);
  if (a->head_dim != 128) return fail(MXFA_ERR_UNSUPPORTED, "%s: head_dim=%d (only 128 is implemented)", fn, a->head_dim);
  if (a->num_heads < 1 || a->num_heads > kMaxGridY)
    return fail(MXFA_ERR_INVALID, "%s: num_heads=%d out of [1, %d]", fn, a->num_heads, kMaxGridY);
  if (a->nseq < 1) return fail(MXFA_ERR_INVALID, "%s: nseq=%d", fn, a->nseq);
  if (a->total_q < 0 || a->total_k < 0) return fail(MXFA_ERR_INVALID, "%s: negative total tokens", fn);
  if (a->max_seqlen_q < 0 || a->max_seqlen_q > a->total_q || a->max_seqlen_k < 0 || a->max_seqlen_k > a->total_k)
    return fail(MXFA_ERR_INVALID, "%s: max_seqlen out of range", fn);
  if (!a->cu_seqlens_q || !a->cu_seqlens_k || !aligned(a->cu_seqlens_q, 4) || !aligned(a->cu_seqlens_k, 4))
    return fail(MXFA_ERR_INVALID, "%s: cu_seqlens NULL or misaligned", fn);
  if (!std::isfinite(a->softmax_scale)) return fail(MXFA_ERR_INVALID, "%s: softmax_scale not finite", fn);
  const mxfa_mx* ops[3] = {&a->q, &a->k, &a->v};
  const char* names[3] = {"q", "k", "v"};
  for (int i = 0; i < 3; ++i) {
    if (!ops[i]->data || !ops[i]->scale) return fail(MXFA_ERR_INVALID, "%s: %s data/scale is NULL", fn, names[i]);
    if (!aligned(ops[i]->data, 16) || !aligned(ops[i]->scale, 16))
      return fail(MXFA_ERR_INVALID, "%s: %s data/scale not 16-byte aligned", fn, names[i]);
  }
  for (int i = 0; i < 3; ++i)
    if (ops[i]->elem != MXFA_E4M3 && ops[i]->elem != MXFA_E2M1 && ops[i]->elem != MXFA_E2M3)
      return fail(MXFA_ERR_INVALID, "%s: %s.elem=%d is not an element format", fn, names[i], (int)ops[i]->elem);
  if (a->q.elem != a->k.elem) return fail(MXFA_ERR_INVALID, "%s: q and k must share one element format", fn);
  if (!e4m3(a->v)) return fail(MXFA_ERR_UNSUPPORTED, "%s: v must be E4M3 (MXFP4/MXFP6 are for q and k only)", fn);
  if (!e4m3(a->q) && (a->q.mode != MXFA_ROW32 || a->k.mode != MXFA_ROW32))
    return fail(MXFA_ERR_UNSUPPORTED, "%s: MXFP4/MXFP6 q and k must be ROW32", fn);
  if (a->q.mode != MXFA_ROW32 && a->q.mode != MXFA_SQ32)
    return fail(MXFA_ERR_INVALID, "%s: q.mode must be ROW32 or SQ32", fn);
  if (a->k.mode != MXFA_ROW32 && a->k.mode != MXFA_SQ32)
    return fail(MXFA_ERR_INVALID, "%s: k.mode must be ROW32 or SQ32", fn);
  const int64_t qtiles = ((int64_t)a->max_seqlen_q + 127) / 128, ktiles = ((int64_t)a->max_seqlen_k + 127) / 128;
  const int64_t pairs = (int64_t)a->num_heads * a->nseq;
  const int64_t items = (qtiles > ktiles ? qtiles : ktiles) * ((pairs + 7) / 8 * 8);  // the largest grid
  if (items >= (int64_t)1 << 31) return fail(MXFA_ERR_INVALID, "%s: problem too large for one launch", fn);
  return MXFA_OK;
}

// Workspace of mxfa_bwd_no_alloc: one fixed array per GPU, resident until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: kernels get the device address
// that hipGetSymbolAddress returns for the current device, fetched once per device and kept below.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call per device).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

mxfa::AttnProblem to_problem(const mxfa_attn_args* a) {
  mxfa::AttnProblem p;
  p.q = {a->q.data, a->q.scale, (int)a->q.mode, (int)a->q.elem};
  p.k = {a->k.data, a->k.scale, (int)a->k.mode, (int)a->k.elem};
  p.v = {a->v.data, a->v.scale, (int)a->v.mode, (int)a->v.elem};
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.nseq = a->nseq;
  p.max_seqlen_q = a->max_seqlen_q;
  p.max_seqlen_k = a->max_seqlen_k;
  p.total_q = a->total_q;
  p.total_k = a->total_k;
  p.H = a->num_heads;
  p.softmax_scale = a->softmax_scale;
  p.causal = a->causal ? 1 : 0;
  return p;
}

// Every argument check of the backward entry points (host only). workspace may be NULL only when
// `library_workspace` is set (the fixed array of mxfa_bwd_no_alloc, whose size is checked here).
mxfa_status check_bwd(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o, const uint16_t* dout_bf16,
                      const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale, const void* workspace,
                      size_t workspace_bytes, const uint16_t* dq, const uint16_t* dk, const uint16_t* dv,
                      const mxfa_grad_mx* mx_out, bool library_workspace, const char* fn) {
  mxfa_status st = check_attn(a, fn);
  if (st != MXFA_OK) return st;
  if (!e4m3(a->q) || !e4m3(v_d) || !e4m3(dout))
    return fail(MXFA_ERR_UNSUPPORTED, "%s: the backward takes E4M3 operands only", fn);
  if (a->q.mode != MXFA_SQ32 || a->k.mode != MXFA_SQ32)
    return fail(MXFA_ERR_INVALID, "%s: q and k must be SQ32 (square blocks serve both GEMM directions)", fn);
  if (v_d.mode != MXFA_ROW32 && v_d.mode != MXFA_SQ32)
    return fail(MXFA_ERR_INVALID, "%s: v_d.mode must be ROW32 or SQ32", fn);
  if (dout.mode != MXFA_SQ32) return fail(MXFA_ERR_INVALID, "%s: dout.mode must be SQ32", fn);
  if (!v_d.data || !v_d.scale || !dout.data || !dout.scale)
    return fail(MXFA_ERR_INVALID, "%s: NULL v_d/dout data or scale", fn);
  if (!aligned(v_d.data, 16) || !aligned(v_d.scale, 16) || !aligned(dout.data, 16) || !aligned(dout.scale, 16))
    return fail(MXFA_ERR_INVALID, "%s: v_d/dout not 16-byte aligned", fn);
  if (!o || !dout_bf16 || !lse) return fail(MXFA_ERR_INVALID, "%s: NULL tensor argument", fn);
  const bool bf16_out = dq || dk || dv;
  if (bf16_out && !(dq && dk && dv)) return fail(MXFA_ERR_INVALID, "%s: dq, dk, dv must be all set or all NULL", fn);
  if (!bf16_out && !mx_out) return fail(MXFA_ERR_INVALID, "%s: no gradient output", fn);
  if (!aligned(o, 16) || !aligned(dout_bf16, 16) || !aligned(lse, 4) ||
      (bf16_out && (!aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))))
    return fail(MXFA_ERR_INVALID, "%s: misaligned tensor argument", fn);
  if (mx_out) {
    const mxfa_grad_mx& g = *mx_out;
    if (!g.dq || !g.dq_scale || !g.dk || !g.dk_scale || !g.dv || !g.dv_scale)
      return fail(MXFA_ERR_INVALID, "%s: every MXFP8 gradient payload and scale pointer must be set", fn);
    if (!aligned(g.dq, 16) || !aligned(g.dk, 16) || !aligned(g.dv, 16))
      return fail(MXFA_ERR_INVALID, "%s: MXFP8 gradient payloads must be 16-byte aligned", fn);
  }
  if (dq_mode != MXFA_DQ_FP32 && dq_mode != MXFA_DQ_FP16_STATIC)
    return fail(MXFA_ERR_INVALID, "%s: bad dq_mode %d", fn, (int)dq_mode);
  if (dq_mode == MXFA_DQ_FP16_STATIC && !is_pow2(dq_static_scale))
    return fail(MXFA_ERR_INVALID, "%s: dq_static_scale=%g must be a positive power of two", fn,
                (double)dq_static_scale);
  const size_t need = mxfa_bwd_workspace_size(a, dq_mode);
  if (library_workspace) {
    if (need > kScratchBytes)
      return fail(MXFA_ERR_INVALID,
                  "%s: the problem needs %zu workspace bytes, more than the %zu of the fixed array; call mxfa_bwd "
                  "with a caller-owned workspace", fn, need, kScratchBytes);
  } else if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) {
    return fail(MXFA_ERR_INVALID, "%s: workspace NULL, misaligned or smaller than %zu bytes", fn, need);
  }
  return MXFA_OK;
}

mxfa_status launch_bwd(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o,
                       const uint16_t* dout_bf16, const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale,
                       void* workspace, uint16_t* dq, uint16_t* dk, uint16_t* dv, const mxfa_grad_mx* mx_out,
                       void* stream, const char* fn) {
  mxfa::GradMxOut gm{};
  if (mx_out)
    gm = {mx_out->dq,         mx_out->dq_scale,   mx_out->dk,        mx_out->dk_scale, mx_out->dv,
          mx_out->dv_scale,   mx_out->dq_scale_t, mx_out->dk_scale_t, mx_out->dv_scale_t};
  mxfa::MxOperand vv{v_d.data, v_d.scale, (int)v_d.mode};
  mxfa::MxOperand dd{dout.data, dout.scale, (int)dout.mode};
  return hip_status(mxfa::launch_attn_bwd(to_problem(a), vv, dd, o, dout_bf16, lse,
                                          dq_mode == MXFA_DQ_FP16_STATIC ? 1 : 0,
                                          dq_mode == MXFA_DQ_FP16_STATIC ? dq_static_scale : 1.0f, workspace, dq, dk,
                                          dv, mx_out ? &gm : nullptr, (hipStream_t)stream),
                    fn);
}

}  // namespace

extern "C" {

const char* mxfa_status_string(mxfa_status s) {
  switch (s) {
    case MXFA_OK: return "MXFA_OK";
    case MXFA_ERR_INVALID: return "MXFA_ERR_INVALID";
    case MXFA_ERR_UNSUPPORTED: return "MXFA_ERR_UNSUPPORTED";
    case MXFA_ERR_HIP: return "MXFA_ERR_HIP";
  }
  return "MXFA_UNKNOWN_STATUS";
}

const char* mxfa_last_error_message(void) { return g_last_error.c_str(); }

int64_t mxfa_padded_token_rows(const int32_t* cu_host, int nseq) {
  if (!cu_host || nseq < 1) return 0;
  int64_t p = 0;
  for (int s = 0; s < nseq; ++s) p += ((int64_t)cu_host[s + 1] - cu_host[s] + 127) / 128 * 128;
  return p;
}

mxfa_status mxfa_quantize(const uint16_t* x, int64_t ld_x, int64_t T, int C, const int32_t* cu_seqlens, int nseq,
                          int max_seqlen, mxfa_block mode, uint8_t* data_out, uint8_t* scale_out,
                          uint8_t* scale_t_out, void* stream) {
  const char* fn = "mxfa_quantize";
  if (!valid_mode(mode)) return fail(MXFA_ERR_INVALID, "%s: bad block mode %d", fn, (int)mode);
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T=%lld < 0", fn, (long long)T);
  if (C <= 0 || C % 32) return fail(MXFA_ERR_INVALID, "%s: C=%d must be a positive multiple of 32", fn, C);
  if (ld_x < C || ld_x % 8) return fail(MXFA_ERR_INVALID, "%s: ld_x=%lld must be >= C and a multiple of 8", fn, (long long)ld_x);
  if (!x || !data_out || !scale_out) return fail(MXFA_ERR_INVALID, "%s: NULL x/data_out/scale_out", fn);
  if (!aligned(x, 16) || !aligned(data_out, 16) || !aligned(scale_out, 16))
    return fail(MXFA_ERR_INVALID, "%s: x/data_out/scale_out not 16-byte aligned", fn);
  if (scale_t_out && mode != MXFA_SQ32) return fail(MXFA_ERR_INVALID, "%s: scale_t_out is for SQ32 only", fn);
  if (scale_t_out && !aligned(scale_t_out, 16)) return fail(MXFA_ERR_INVALID, "%s: scale_t_out not aligned", fn);
  if (mode != MXFA_ROW32) {
    mxfa_status st = check_jagged(cu_seqlens, nseq, max_seqlen, T, fn);
    if (st != MXFA_OK) return st;
  }
  if (mode == MXFA_ROW32 && T * (C / 16) / 256 >= ((int64_t)1 << 31))
    return fail(MXFA_ERR_INVALID, "%s: tensor too large for one launch", fn);
  return hip_status(mxfa::launch_quantize(x, ld_x, T, C, cu_seqlens, nseq, max_seqlen, (int)mode, data_out, scale_out,
                                          scale_t_out, (hipStream_t)stream),
                    fn);
}

mxfa_status mxfa_quantize_col32_row32(const uint16_t* x, int64_t ld_x, int64_t T, int C, const int32_t* cu_seqlens,
                                      int nseq, int max_seqlen, uint8_t* data_col, uint8_t* scale_col,
                                      uint8_t* data_row, uint8_t* scale_row, void* stream) {
  const char* fn = "mxfa_quantize_col32_row32";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T=%lld < 0", fn, (long long)T);
  if (C <= 0 || C % 32) return fail(MXFA_ERR_INVALID, "%s: C=%d must be a positive multiple of 32", fn, C);
  if (ld_x < C || ld_x % 8) return fail(MXFA_ERR_INVALID, "%s: ld_x=%lld must be >= C and a multiple of 8", fn, (long long)ld_x);
  if (!x || !data_col || !scale_col || !data_row || !scale_row)
    return fail(MXFA_ERR_INVALID, "%s: NULL x/data_col/scale_col/data_row/scale_row", fn);
  if (!aligned(x, 16) || !aligned(data_col, 16) || !aligned(scale_col, 16) || !aligned(data_row, 16) ||
      !aligned(scale_row, 16))
    return fail(MXFA_ERR_INVALID, "%s: x and the four outputs must be 16-byte aligned", fn);
  mxfa_status st = check_jagged(cu_seqlens, nseq, max_seqlen, T, fn);
  if (st != MXFA_OK) return st;
  return hip_status(mxfa::launch_quantize_col32_row32(x, ld_x, C, cu_seqlens, nseq, max_seqlen, data_col, scale_col,
                                                      data_row, scale_row, (hipStream_t)stream),
                    fn);
}

mxfa_status mxfa_e4m3_pack_patterns(uint32_t first, int64_t n, int variant, float sc, uint8_t* out, void* stream) {
  const char* fn = "mxfa_e4m3_pack_patterns";
  if (n < 0 || n > ((int64_t)1 << 32) || n % 4)
    return fail(MXFA_ERR_INVALID, "%s: n=%lld must be a multiple of 4 in [0, 2^32]", fn, (long long)n);
  if (variant < 0 || variant > 2) return fail(MXFA_ERR_INVALID, "%s: variant=%d not in {0, 1, 2}", fn, variant);
  if (variant == 1 && (!is_pow2(sc) || sc < 0x1p-126f || sc > 0x1p119f))
    return fail(MXFA_ERR_INVALID, "%s: sc=%g must be a power of two in [2^-126, 2^119]", fn, (double)sc);
  if (variant != 1) sc = 1.0f;
  if (n > 0 && !out) return fail(MXFA_ERR_INVALID, "%s: out is NULL", fn);
  if (!aligned(out, 4)) return fail(MXFA_ERR_INVALID, "%s: out not 4-byte aligned", fn);
  return hip_status(mxfa::launch_e4m3_pack_patterns(first, n, variant, sc, out, (hipStream_t)stream), fn);
}

mxfa_status mxfa_quantize_e2m1(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data_out,
                               uint8_t* scale_out, void* stream) {
  const char* fn = "mxfa_quantize_e2m1";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T=%lld < 0", fn, (long long)T);
  if (C <= 0 || C % 32) return fail(MXFA_ERR_INVALID, "%s: C=%d must be a positive multiple of 32", fn, C);
  if (ld_x < C || ld_x % 8) return fail(MXFA_ERR_INVALID, "%s: ld_x=%lld must be >= C and a multiple of 8", fn, (long long)ld_x);
  if (!x || !data_out || !scale_out) return fail(MXFA_ERR_INVALID, "%s: NULL x/data_out/scale_out", fn);
  if (!aligned(x, 16) || !aligned(data_out, 16) || !aligned(scale_out, 16))
    return fail(MXFA_ERR_INVALID, "%s: x/data_out/scale_out not 16-byte aligned", fn);
  if (T * (C / 16) / 256 >= ((int64_t)1 << 31)) return fail(MXFA_ERR_INVALID, "%s: tensor too large for one launch", fn);
  return hip_status(mxfa::launch_quantize_e2m1(x, ld_x, T, C, data_out, scale_out, (hipStream_t)stream), fn);
}

mxfa_status mxfa_quantize_e2m3(const uint16_t* x, int64_t ld_x, int64_t T, int C, uint8_t* data_out,
                               uint8_t* scale_out, void* stream) {
  const char* fn = "mxfa_quantize_e2m3";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T=%lld < 0", fn, (long long)T);
  if (C <= 0 || C % 64) return fail(MXFA_ERR_INVALID, "%s: C=%d must be a positive multiple of 64", fn, C);
  if (ld_x < C || ld_x % 8) return fail(MXFA_ERR_INVALID, "%s: ld_x=%lld must be >= C and a multiple of 8", fn, (long long)ld_x);
  if (!x || !data_out || !scale_out) return fail(MXFA_ERR_INVALID, "%s: NULL x/data_out/scale_out", fn);
  if (!aligned(x, 16) || !aligned(data_out, 16) || !aligned(scale_out, 16))
    return fail(MXFA_ERR_INVALID, "%s: x/data_out/scale_out not 16-byte aligned", fn);
  if (T * (C / 16) / 256 >= ((int64_t)1 << 31)) return fail(MXFA_ERR_INVALID, "%s: tensor too large for one launch", fn);
  return hip_status(mxfa::launch_quantize_e2m3(x, ld_x, T, C, data_out, scale_out, (hipStream_t)stream), fn);
}

mxfa_status mxfa_varlen_scale_scatter(const uint8_t* compact, const int32_t* cu_seqlens, int nseq, int max_seqlen,
                                      int C, mxfa_block mode, uint8_t* padded_out, int64_t padded_rows,
                                      void* stream) {
  const char* fn = "mxfa_varlen_scale_scatter";
  if (!valid_mode(mode)) return fail(MXFA_ERR_INVALID, "%s: bad block mode %d", fn, (int)mode);
  if (C <= 0 || C % 32) return fail(MXFA_ERR_INVALID, "%s: C=%d must be a positive multiple of 32", fn, C);
  if (!compact || !padded_out) return fail(MXFA_ERR_INVALID, "%s: NULL compact/padded_out", fn);
  if (padded_rows < 0) return fail(MXFA_ERR_INVALID, "%s: padded_rows < 0", fn);
  if (!cu_seqlens || !aligned(cu_seqlens, 4)) return fail(MXFA_ERR_INVALID, "%s: cu_seqlens NULL or misaligned", fn);
  if (nseq < 1 || nseq > kMaxGridY) return fail(MXFA_ERR_INVALID, "%s: nseq=%d out of range", fn, nseq);
  if (max_seqlen < 0 || (max_seqlen + 127) / 128 > (int64_t)1 << 30)
    return fail(MXFA_ERR_INVALID, "%s: max_seqlen=%d out of range", fn, max_seqlen);
  const int unit = mode == MXFA_ROW32 ? 1 : 32;
  const int64_t min_rows = ((int64_t)max_seqlen + 127) / 128 * 128 / unit;
  if (padded_rows < min_rows)
    return fail(MXFA_ERR_INVALID, "%s: padded_rows=%lld smaller than one padded sequence", fn, (long long)padded_rows);
  return hip_status(mxfa::launch_scale_scatter(compact, cu_seqlens, nseq, max_seqlen, C, (int)mode, padded_out,
                                               padded_rows, (hipStream_t)stream),
                    fn);
}

mxfa_status mxfa_fwd(const mxfa_attn_args* a, uint16_t* o, float* lse, void* stream) {
  return mxfa_fwd_p_scale(a, MXFA_P_STATIC, o, lse, stream);
}

mxfa_status mxfa_fwd_p_scale(const mxfa_attn_args* a, mxfa_p_scale p_scale, uint16_t* o, float* lse, void* stream) {
  if (!o) return fail(MXFA_ERR_INVALID, "%s: NULL o", p_scale == MXFA_P_STATIC ? "mxfa_fwd" : "mxfa_fwd_p_scale");
  return mxfa_fwd_mx_out(a, p_scale, o, nullptr, nullptr, lse, stream);
}

mxfa_status mxfa_fwd_mx_out(const mxfa_attn_args* a, mxfa_p_scale p_scale, uint16_t* o, uint8_t* o_data,
                            uint8_t* o_scale, float* lse, void* stream) {
  const char* fn = o_data ? "mxfa_fwd_mx_out" : p_scale == MXFA_P_STATIC ? "mxfa_fwd" : "mxfa_fwd_p_scale";
  if (p_scale != MXFA_P_STATIC && p_scale != MXFA_P_BLOCK_DYNAMIC)
    return fail(MXFA_ERR_INVALID, "%s: bad p_scale %d", fn, (int)p_scale);
  mxfa_status st = check_attn(a, fn);
  if (st != MXFA_OK) return st;
  if (a->v.mode != MXFA_COL32 && a->v.mode != MXFA_SQ32)
    return fail(MXFA_ERR_INVALID, "%s: v.mode must be COL32 or SQ32", fn);
  if (!lse) return fail(MXFA_ERR_INVALID, "%s: NULL lse", fn);
  if (!o && !o_data) return fail(MXFA_ERR_INVALID, "%s: neither o nor o_data given", fn);
  if (o_data && !o_scale) return fail(MXFA_ERR_INVALID, "%s: o_data without o_scale", fn);
  if ((o && !aligned(o, 16)) || !aligned(lse, 4) || (o_data && (!aligned(o_data, 4) || !aligned(o_scale, 4))))
    return fail(MXFA_ERR_INVALID, "%s: misaligned output", fn);
  return hip_status(mxfa::launch_attn_fwd(to_problem(a), p_scale == MXFA_P_BLOCK_DYNAMIC ? 1 : 0, o, o_data,
                                          o_data ? o_scale : nullptr, lse, (hipStream_t)stream),
                    fn);
}

size_t mxfa_bwd_workspace_size(const mxfa_attn_args* a, mxfa_dq_mode dq_mode) {
  (void)dq_mode;  // the layout is the same for both reductions
  if (!a || a->total_q < 0 || a->num_heads < 1 || a->nseq < 1 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0) return 0;
  return mxfa::bwd_workspace_bytes(a->total_q, a->num_heads, a->nseq, a->max_seqlen_q, a->max_seqlen_k);
}

mxfa_status mxfa_bwd(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o,
                     const uint16_t* dout_bf16, const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale,
                     void* workspace, size_t workspace_bytes, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                     void* stream) {
  if (!dq || !dk || !dv) return fail(MXFA_ERR_INVALID, "mxfa_bwd: NULL tensor argument");
  return mxfa_bwd_mx_out(a, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, workspace, workspace_bytes, dq, dk,
                         dv, nullptr, stream);
}

size_t mxfa_bwd_no_alloc_max_workspace(void) { return kScratchBytes; }

mxfa_status mxfa_bwd_no_alloc(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o,
                              const uint16_t* dout_bf16, const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale,
                              uint16_t* dq, uint16_t* dk, uint16_t* dv, void* stream) {
  const char* fn = "mxfa_bwd_no_alloc";
  if (!dq || !dk || !dv) return fail(MXFA_ERR_INVALID, "%s: NULL tensor argument", fn);
  mxfa_status st = check_bwd(a, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, nullptr, 0, dq, dk, dv,
                             nullptr, true, fn);
  if (st != MXFA_OK) return st;
  void* ws = nullptr;
  st = hip_status(scratch_address(&ws), fn);
  if (st != MXFA_OK) return st;
  return launch_bwd(a, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, ws, dq, dk, dv, nullptr, stream, fn);
}

mxfa_status mxfa_bwd_mx_out(const mxfa_attn_args* a, mxfa_mx v_d, mxfa_mx dout, const uint16_t* o,
                            const uint16_t* dout_bf16, const float* lse, mxfa_dq_mode dq_mode, float dq_static_scale,
                            void* workspace, size_t workspace_bytes, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                            const mxfa_grad_mx* mx_out, void* stream) {
  const char* fn = mx_out ? "mxfa_bwd_mx_out" : "mxfa_bwd";
  mxfa_status st = check_bwd(a, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, workspace, workspace_bytes, dq,
                             dk, dv, mx_out, false, fn);
  if (st != MXFA_OK) return st;
  return launch_bwd(a, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, workspace, dq, dk, dv, mx_out, stream, fn);
}

mxfa_status mxfa_rmsnorm_quantize(const uint16_t* x, int64_t ld_x, int64_t T, int C, const float* gamma, float eps,
                                  const int32_t* cu_seqlens, int nseq, int max_seqlen, uint8_t* data_out,
                                  uint8_t* scale_out, uint8_t* scale_t_out, void* stream) {
  const char* fn = "mxfa_rmsnorm_quantize";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T < 0", fn);
  if (C <= 0 || C % 32 || C > 32768) return fail(MXFA_ERR_INVALID, "%s: C=%d must be a multiple of 32 in [32, 32768]", fn, C);
  if (ld_x < C || ld_x % 8) return fail(MXFA_ERR_INVALID, "%s: bad ld_x", fn);
  if (!x || !gamma || !data_out || !scale_out) return fail(MXFA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(x, 16) || !aligned(gamma, 4) || !aligned(data_out, 16) || !aligned(scale_out, 16) ||
      (scale_t_out && !aligned(scale_t_out, 16)))
    return fail(MXFA_ERR_INVALID, "%s: misaligned argument", fn);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(MXFA_ERR_INVALID, "%s: eps must be finite and >= 0", fn);
  mxfa_status st = check_jagged(cu_seqlens, nseq, max_seqlen, T, fn);
  if (st != MXFA_OK) return st;
  return hip_status(mxfa::launch_rmsnorm_quantize(x, ld_x, C, gamma, eps, cu_seqlens, nseq, max_seqlen, data_out,
                                                  scale_out, scale_t_out, (hipStream_t)stream),
                    fn);
}

mxfa_status mxfa_linear_quantize(mxfa_mx x, mxfa_mx w, int64_t T, int C_in, int C_out, const int32_t* cu_seqlens,
                                 int nseq, int max_seqlen, uint8_t* data_out, uint8_t* scale_out,
                                 uint8_t* scale_t_out, void* stream) {
  const char* fn = "mxfa_linear_quantize";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T < 0", fn);
  if (C_in <= 0 || C_in % 128 || C_in > 65536)
    return fail(MXFA_ERR_INVALID, "%s: C_in=%d must be a multiple of 128 in [128, 65536]", fn, C_in);
  if (C_out <= 0 || C_out % 128) return fail(MXFA_ERR_INVALID, "%s: C_out=%d must be a positive multiple of 128", fn, C_out);
  if (!e4m3(x) || !e4m3(w)) return fail(MXFA_ERR_UNSUPPORTED, "%s: x and w must be E4M3", fn);
  if (x.mode != MXFA_SQ32 && x.mode != MXFA_ROW32) return fail(MXFA_ERR_INVALID, "%s: x.mode must be SQ32 or ROW32", fn);
  if (w.mode != MXFA_ROW32) return fail(MXFA_ERR_INVALID, "%s: w.mode must be ROW32 (scales along C_in)", fn);
  if (!x.data || !x.scale || !w.data || !w.scale || !data_out || !scale_out)
    return fail(MXFA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(x.data, 16) || !aligned(x.scale, 16) || !aligned(w.data, 16) || !aligned(w.scale, 16) ||
      !aligned(data_out, 16) || !aligned(scale_out, 16) || (scale_t_out && !aligned(scale_t_out, 16)))
    return fail(MXFA_ERR_INVALID, "%s: misaligned argument", fn);
  mxfa_status st = check_jagged(cu_seqlens, nseq, max_seqlen, T, fn);
  if (st != MXFA_OK) return st;
  if ((int64_t)nseq * ((max_seqlen + 127) / 128) * (C_out / 128) >= ((int64_t)1 << 31))
    return fail(MXFA_ERR_INVALID, "%s: problem too large for one launch", fn);
  mxfa::MxOperand xx{x.data, x.scale, (int)x.mode};
  mxfa::MxOperand ww{w.data, w.scale, (int)w.mode};
  return hip_status(mxfa::launch_linear_quantize(xx, ww, T, C_in, C_out, cu_seqlens, nseq, max_seqlen, data_out,
                                                 scale_out, scale_t_out, nullptr, 0, (hipStream_t)stream),
                    fn);
}

mxfa_status mxfa_linear_bwd_data(mxfa_mx dy, mxfa_mx wt, int64_t T, int C_out, int C_in, const int32_t* cu_seqlens,
                                 int nseq, int max_seqlen, int accumulate, uint16_t* dx, void* stream) {
  const char* fn = "mxfa_linear_bwd_data";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T < 0", fn);
  if (C_out <= 0 || C_out % 128 || C_out > 65536)
    return fail(MXFA_ERR_INVALID, "%s: C_out=%d must be a multiple of 128 in [128, 65536]", fn, C_out);
  if (C_in <= 0 || C_in % 128) return fail(MXFA_ERR_INVALID, "%s: C_in=%d must be a positive multiple of 128", fn, C_in);
  if (!e4m3(dy) || !e4m3(wt)) return fail(MXFA_ERR_UNSUPPORTED, "%s: dy and wt must be E4M3", fn);
  if (dy.mode != MXFA_SQ32 && dy.mode != MXFA_ROW32) return fail(MXFA_ERR_INVALID, "%s: dy.mode must be SQ32 or ROW32", fn);
  if (wt.mode != MXFA_ROW32) return fail(MXFA_ERR_INVALID, "%s: wt.mode must be ROW32 (scales along C_out)", fn);
  if (!dy.data || !dy.scale || !wt.data || !wt.scale || !dx) return fail(MXFA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(dy.data, 16) || !aligned(dy.scale, 16) || !aligned(wt.data, 16) || !aligned(wt.scale, 16) ||
      !aligned(dx, 16))
    return fail(MXFA_ERR_INVALID, "%s: misaligned argument", fn);
  if (accumulate != 0 && accumulate != 1) return fail(MXFA_ERR_INVALID, "%s: accumulate must be 0 or 1", fn);
  mxfa_status st = check_jagged(cu_seqlens, nseq, max_seqlen, T, fn);
  if (st != MXFA_OK) return st;
  if ((int64_t)nseq * ((max_seqlen + 127) / 128) * (C_in / 128) >= ((int64_t)1 << 31))
    return fail(MXFA_ERR_INVALID, "%s: problem too large for one launch", fn);
  // the projection kernel with dY as its input (contraction over C_out) and W^T as its weight
  mxfa::MxOperand dd{dy.data, dy.scale, (int)dy.mode};
  mxfa::MxOperand ww{wt.data, wt.scale, (int)wt.mode};
  return hip_status(mxfa::launch_linear_quantize(dd, ww, T, C_out, C_in, cu_seqlens, nseq, max_seqlen, nullptr, nullptr,
                                                 nullptr, dx, accumulate, (hipStream_t)stream),
                    fn);
}

size_t mxfa_linear_bwd_weight_workspace_size(int64_t T, int nseq, int C_out, int C_in) {
  if (T < 0 || nseq < 1 || C_out <= 0 || C_in <= 0) return 0;
  return mxfa::wgrad_workspace_bytes(T, nseq, C_out, C_in);
}

mxfa_status mxfa_linear_bwd_weight(const uint8_t* dy, const uint8_t* dy_scale_t, const uint8_t* x,
                                   const uint8_t* x_scale_t, int64_t T, int C_out, int C_in,
                                   const int32_t* cu_seqlens, int nseq, int max_seqlen, void* workspace,
                                   size_t workspace_bytes, float* dw, void* stream) {
  const char* fn = "mxfa_linear_bwd_weight";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T < 0", fn);
  if (C_out <= 0 || C_out % 128 || C_in <= 0 || C_in % 128)
    return fail(MXFA_ERR_INVALID, "%s: C_out=%d and C_in=%d must be positive multiples of 128", fn, C_out, C_in);
  if (T * (int64_t)std::max(C_out, C_in) >= ((int64_t)1 << 32))
    return fail(MXFA_ERR_UNSUPPORTED, "%s: T x C must stay below 2^32 bytes per operand", fn);
  if (!dy || !dy_scale_t || !x || !x_scale_t || !dw || !workspace) return fail(MXFA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(dw, 16) || !aligned(workspace, 16))
    return fail(MXFA_ERR_INVALID, "%s: misaligned argument", fn);
  mxfa_status st = check_jagged(cu_seqlens, nseq, max_seqlen, T, fn);
  if (st != MXFA_OK) return st;
  if (workspace_bytes < mxfa::wgrad_workspace_bytes(T, nseq, C_out, C_in))
    return fail(MXFA_ERR_INVALID, "%s: workspace too small (%zu < %zu bytes)", fn, workspace_bytes,
                mxfa::wgrad_workspace_bytes(T, nseq, C_out, C_in));
  return hip_status(mxfa::launch_linear_wgrad(dy, dy_scale_t, x, x_scale_t, T, C_out, C_in, cu_seqlens, nseq,
                                              max_seqlen, workspace, dw, (hipStream_t)stream),
                    fn);
}

size_t mxfa_rmsnorm_bwd_workspace_size(int64_t T, int C) {
  if (T < 0 || C <= 0) return 0;
  return mxfa::rmsnorm_bwd_workspace_bytes(T, C);
}

mxfa_status mxfa_rmsnorm_bwd(const uint16_t* x, int64_t ld_x, int64_t T, int C, const float* gamma, float eps,
                             const uint16_t* dy, void* workspace, size_t workspace_bytes, uint16_t* dx, float* dgamma,
                             void* stream) {
  const char* fn = "mxfa_rmsnorm_bwd";
  if (T < 0) return fail(MXFA_ERR_INVALID, "%s: T < 0", fn);
  if (C <= 0 || C % 32 || C > 2048)
    return fail(MXFA_ERR_UNSUPPORTED, "%s: C=%d must be a multiple of 32 in [32, 2048]", fn, C);
  if (ld_x < C || ld_x % 8) return fail(MXFA_ERR_INVALID, "%s: bad ld_x", fn);
  if (!x || !gamma || !dy || !dx || !dgamma || !workspace) return fail(MXFA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16) || !aligned(gamma, 4) || !aligned(dgamma, 16) ||
      !aligned(workspace, 16))
    return fail(MXFA_ERR_INVALID, "%s: misaligned argument", fn);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(MXFA_ERR_INVALID, "%s: eps must be finite and >= 0", fn);
  if (workspace_bytes < mxfa::rmsnorm_bwd_workspace_bytes(T, C))
    return fail(MXFA_ERR_INVALID, "%s: workspace too small (%zu < %zu bytes)", fn, workspace_bytes,
                mxfa::rmsnorm_bwd_workspace_bytes(T, C));
  return hip_status(mxfa::launch_rmsnorm_bwd(x, ld_x, T, C, gamma, eps, dy, workspace, dx, dgamma, (hipStream_t)stream),
                    fn);
}

}  // extern "C"

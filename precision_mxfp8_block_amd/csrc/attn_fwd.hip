// MXFP8 attention forward for gfx950: scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), K/V tiles
// staged in LDS, FP32 online softmax, P quantized online to E4M3 with a static block scale.
//
// What is computed (andresseo.expert "MXFP8 FlashAttention-4 Hits 2.85 Petaflops...", section
// "Inside the TMEM Bargain and Zero-Gather Jagged Pipeline"; theclarity.today paragraphs 1-3;
// brifing.si item 4): per (sequence, head, 128-row query tile), for 128-row key tiles in order:
//   S = Q K^T with Q, K scaled along D;  m' = max(m, rowmax S);  P = exp(c (S - m'));
//   l = exp(c (m - m')) l + rowsum P;   P -> E4M3 at the constant scale 2^-8 (P <= 1 because the
//   running row max is the reference, so no second max pass);  O = exp(c (m - m')) O + P V with V
//   scaled along the keys.  Output O / l in bf16 and LSE = c m + ln l.
//
// gfx950 design (not the pages' Blackwell design):
//  * Workgroup = 4 waves = one 128-row query tile; wave w owns query rows 32w..32w+31.
//  * The score tile is computed transposed, S^T = K Q^T (A = K from LDS, B = Q held in VGPRs), so
//    the accumulator gives each lane one query row (column l % 32) and 64 of its 128 keys; the
//    lane pair (l, l + 32) holds the whole row. Row max and row sum need one v_permlane32_swap.
//  * O is accumulated transposed too, O^T = V^T P^T, so the rescale factor exp(c (m - m')) is a
//    per-lane scalar. P's bytes go into the B operand in the accumulator's own key order (no lane
//    shuffle): the 16 bytes at one byte offset of lanes r and r+32 always cover one aligned 32-key
//    block, which is all the block scale of V requires.
//  * V^T is read from the row-major LDS tile with ds_read_b64_tr_b8 (8 keys x 1 column per lane per
//    read), in exactly that key order.
//  * LDS tiles are 128 rows x 128 bytes with the 16-byte chunk index XOR-swizzled by
//    (row & 7) ^ ((row & 8) >> 1): conflict-free for the row reads of K and the transposed reads
//    of V.
//  * Grid order is XCD-aware: consecutive workgroup IDs land on different XCDs, so IDs are remapped
//    to give each XCD a contiguous range of (sequence, head, tile) items; the query tiles of one
//    head then share one XCD's L2, which holds that head's K and V.
#include "mx_device.h"
#include "mxfa_internal.h"

namespace {

constexpr int kTile = 128;
constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;

struct FwdParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* q_scale;
  const uint8_t* k_scale;
  const uint8_t* v_scale;
  int q_row_shift;  // 0: ROW32 (one scale row per token), 5: SQ32 (one per 32 tokens)
  int k_row_shift;
  int v_col_shift;  // 0: COL32 (a scale per column), 5: SQ32 (a scale per 32 columns)
  const int32_t* cu_q;
  const int32_t* cu_k;
  int nseq, H, n_qtiles;
  int64_t total_items;
  float c;   // softmax scale
  float c2;  // softmax scale * log2(e)
  int causal;
  uint16_t* o;
  float* lse;
  int64_t Tq;
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row & 8) >> 1); }

// XCD-aware mapping of a linear workgroup id to a work item (bijective for any total).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t total) {
  const int64_t per = total / 8, rem = total % 8;
  const int64_t x = bid % 8, slot = bid / 8;
  return x * per + (x < rem ? x : rem) + slot;
}

__global__ void __launch_bounds__(256, 1) attn_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kTile * kD];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[kTile * kD];
  __shared__ int64_t red[16];

  const int64_t item = xcd_remap(blockIdx.x, p.total_items);
  const int qt = p.n_qtiles - 1 - (int)(item % p.n_qtiles);  // heavy (late) query tiles first
  const int h = (int)((item / p.n_qtiles) % p.H);
  const int s = (int)(item / ((int64_t)p.n_qtiles * p.H));
  const int64_t q_start = p.cu_q[s], k_start = p.cu_k[s];
  const int Lq = p.cu_q[s + 1] - (int)q_start;
  const int Lk = p.cu_k[s + 1] - (int)k_start;
  if (qt * kTile >= Lq) return;  // uniform over the workgroup

  const SeqOffsets qoff = seq_offsets(p.cu_q, s, red);
  const SeqOffsets koff = seq_offsets(p.cu_k, s, red);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int C = p.H * kD;
  const int Cs = C >> 5;  // scale bytes per row in the along-D layouts

  // ---- Q tile rows of this wave, held as the B operand of S^T = K Q^T ----
  const int qrow = qt * kTile + wave * 32 + r;  // position in the sequence
  mx_v8i qa[2];
  {
    const bool valid = qrow < Lq;
    const uint8_t* src = p.q + (q_start + qrow) * (int64_t)C + h * kD;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
      if (valid) {
        lo = *reinterpret_cast<const uint4*>(src + 64 * ds + 16 * hh);
        hi = *reinterpret_cast<const uint4*>(src + 64 * ds + 32 + 16 * hh);
      }
      qa[ds] = mx_v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
  // scale of d-block (2 ds + hh) of row qrow: byte 0 for ds = 0, byte 2 for ds = 1
  const uint32_t qsc =
      *reinterpret_cast<const uint32_t*>(p.q_scale + ((qoff.padded + qrow) >> p.q_row_shift) * (int64_t)Cs + h * 4) >>
      (8 * hh);

  float m = -INFINITY;  // running max of raw scores for query row qrow
  float lsum = 0.0f;    // this lane's half of the row sum of P * 256
  mx_v16f oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = mx_v16f{};

  int n_ktiles = (Lk + kTile - 1) / kTile;
  if (p.causal) {
    const int q_last = min(qt * kTile + kTile - 1, Lq - 1);
    n_ktiles = min(n_ktiles, q_last / kTile + 1);
  }

  // per-lane constants of the transposed V read (see the lane map in mx_device.h)
  const int grp = lane >> 4, gl = lane & 15;
  const int tb = gl >> 1, ts = gl & 1;
  const int tr_row = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);  // + 64 ks + 32 (c >> 1) + 16 (c & 1)
  const int tr_col = 16 * (grp & 1) + 8 * ts;                    // + 32 dblk
  const int tr_swz = swz(tr_row);

  for (int kt = 0; kt < n_ktiles; ++kt) {
    const int kv0 = kt * kTile;
    __syncthreads();
    // ---- K and V tiles: global -> LDS (16-byte chunks, swizzled) ----
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int row = i >> 3, ch = i & 7;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (kv0 + row < Lk) {
        const int64_t g = (k_start + kv0 + row) * (int64_t)C + h * kD + 16 * ch;
        kv = *reinterpret_cast<const uint4*>(p.k + g);
        vv = *reinterpret_cast<const uint4*>(p.v + g);
      }
      const int off = row * kD + 16 * (ch ^ swz(row));
      *reinterpret_cast<uint4*>(lds_k + off) = kv;
      *reinterpret_cast<uint4*>(lds_v + off) = vv;
    }
    __syncthreads();

    // ---- S^T = K Q^T : 4 key blocks of 32 x 2 D-steps of 64 ----
    mx_v16f sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = 32 * kb + r;
      const uint32_t ksc =
          *reinterpret_cast<const uint32_t*>(p.k_scale + ((koff.padded + kv0 + row) >> p.k_row_shift) * (int64_t)Cs +
                                             h * 4) >>
          (8 * hh);
      sacc[kb] = mx_v16f{};
      const uint8_t* krow = lds_k + row * kD;
      const int sw = swz(row);
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        uint4 lo = *reinterpret_cast<const uint4*>(krow + 16 * ((4 * ds + hh) ^ sw));
        uint4 hi = *reinterpret_cast<const uint4*>(krow + 16 * ((4 * ds + 2 + hh) ^ sw));
        mx_v8i ka{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if (ds == 0)
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa[0], sacc[kb], 0, 0, 0, (int)ksc, 0,
                                                                     (int)qsc);
        else
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa[1], sacc[kb], 0, 0, 2, (int)ksc, 2,
                                                                     (int)qsc);
      }
    }

    // ---- mask (ragged tail, causal diagonal) ----
    const bool need_mask = (kv0 + kTile > Lk) || (p.causal && kv0 + kTile - 1 > qt * kTile + wave * 32);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kvpos = kv0 + 32 * kb + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (kvpos >= Lk || (p.causal && kvpos > qrow)) sacc[kb][v] = -INFINITY;
        }
    }

    // ---- online softmax (FP32) ----
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    {
      auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1]));
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m - m_use) * p.c2);
    const float base = m_use * p.c2 - 8.0f;  // exp2(S c2 - base) = 256 P
    m = m_new;
    uint32_t pk[4][4];
    float ps = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 0], p.c2, -base));
        float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 1], p.c2, -base));
        float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 2], p.c2, -base));
        float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 3], p.c2, -base));
        ps += (e0 + e1) + (e2 + e3);
        pk[kb][i] = mx_pack4_inrange(e0, e1, e2, e3);
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;

    // ---- O^T += V^T P^T : 2 key steps of 64 x 4 D-blocks of 32 ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      mx_v8i pb{(int)pk[2 * ks][0], (int)pk[2 * ks][1], (int)pk[2 * ks][2], (int)pk[2 * ks][3],
                (int)pk[2 * ks + 1][0], (int)pk[2 * ks + 1][1], (int)pk[2 * ks + 1][2], (int)pk[2 * ks + 1][3]};
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        mx_v2i part[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int row = 64 * ks + 32 * (cc >> 1) + 16 * (cc & 1) + tr_row;
          const int col = 32 * db + tr_col;
          const int off = row * kD + 16 * ((col >> 4) ^ tr_swz) + (col & 15);
          part[cc] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MX_LDS mx_v2i*)(lds_v + off));
        }
        mx_v8i va{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
        // V scale of key block (2 ks + hh), column 32 db + r
        const int64_t vrow = (koff.padded + kv0 + 64 * ks + 32 * hh) >> 5;
        const int vcol = (h * kD + 32 * db + r) >> p.v_col_shift;
        const uint32_t vsc = p.v_scale[vrow * (int64_t)(C >> p.v_col_shift) + vcol];
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[db], 0, 0, 0, (int)vsc, 0, 119);
      }
    }
  }

  // ---- epilogue: O / l -> bf16, LSE ----
  {
    auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
  }
  const float l = lsum * (1.0f / 256.0f);
  if (qrow < Lq) {
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* dst = p.o + (q_start + qrow) * (int64_t)C + h * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * hh;
        uint32_t w0 = f32_to_bf16(oacc[db][4 * i + 0] * inv_l) | (f32_to_bf16(oacc[db][4 * i + 1] * inv_l) << 16);
        uint32_t w1 = f32_to_bf16(oacc[db][4 * i + 2] * inv_l) | (f32_to_bf16(oacc[db][4 * i + 3] * inv_l) << 16);
        *reinterpret_cast<uint2*>(dst + d) = make_uint2(w0, w1);
      }
    if (hh == 0) p.lse[(int64_t)h * p.Tq + q_start + qrow] = l > 0.0f ? m * p.c + logf(l) : -INFINITY;
  }
}

}  // namespace

namespace mxfa {

hipError_t launch_attn_fwd(const AttnProblem& a, uint16_t* o, float* lse, hipStream_t stream) {
  FwdParams p;
  p.q = a.q.data; p.k = a.k.data; p.v = a.v.data;
  p.q_scale = a.q.scale; p.k_scale = a.k.scale; p.v_scale = a.v.scale;
  p.q_row_shift = a.q.mode == 0 ? 0 : 5;
  p.k_row_shift = a.k.mode == 0 ? 0 : 5;
  p.v_col_shift = a.v.mode == 1 ? 0 : 5;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.nseq = a.nseq; p.H = a.H;
  p.n_qtiles = (a.max_seqlen_q + kTile - 1) / kTile;
  p.total_items = (int64_t)p.n_qtiles * a.H * a.nseq;
  p.c = a.softmax_scale;
  p.c2 = a.softmax_scale * kLog2e;
  p.causal = a.causal;
  p.o = o; p.lse = lse; p.Tq = a.total_q;
  if (p.total_items == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)p.total_items), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mxfa

// MXFP8 attention backward for gfx950: recomputation with five scaled-MFMA GEMMs on square-block
// (32 x 32) quantized Q, K and dO, online dS quantization, dQ reduced through global atomics.
//
// What is computed (andresseo.expert "MXFP8 FlashAttention-4 Hits 2.85 Petaflops...", section
// "Inside the TMEM Bargain and Zero-Gather Jagged Pipeline": five GEMMs; Q, K and dO in square
// 32 x 32 blocks so one E4M3 payload serves the plain and the transposed GEMM; dS quantized once per
// square block with a wave-wide absolute maximum; dQ reduction in FP16 with a static scale, or FP32;
// brifing.si item 6):
//   Delta_i = sum_d dO_id O_id                                   (preprocess)
//   per KV tile (workgroup), per Q tile (inner loop):
//     S = Q K^T;  P = exp(c S - LSE);  P_q = E4M3(P 2^8) at code 119
//     dV += P_q^T dO;  dP = dO V^T;  dS = P (dP - Delta);  dS_q = SQ32(dS)
//     dK += dS_q^T Q;  dQ_partial = dS_q K  -> atomically added (FP32, or FP16 holding sigma dQ)
//   dK = c dK, dQ = c acc / sigma (finalize).
//
// gfx950 layout choices:
//  * Workgroup = 4 waves = one 128-row KV tile; wave w owns key rows 32w..32w+31. Its K and V rows
//    stay in VGPRs as the B operands of S = Q K^T and dP = dO V^T, so S and dP come out with one
//    key per lane (column) and 16 queries per lane per 32-query block.
//  * That accumulator layout is exactly the A operand of dV = P^T dO and dK = dS^T Q (one key per
//    lane, contraction over queries): P_q and dS_q bytes are used in place, in the accumulator's
//    query order; dO^T and Q^T are read from LDS with ds_read_b64_tr_b8 in the same order.
//  * dQ = dS K contracts over all 128 keys of the tile (all four waves): dS_q goes to LDS key-major,
//    each wave then computes 32 query rows and adds them to the accumulator with coalesced atomics
//    (packed FP16 pairs or FP32).
//  * Q and dO tiles (and the tile's LSE and Delta) are double-buffered in LDS and fetched one tile
//    ahead with direct global -> LDS loads; all LDS tiles use the forward's XOR swizzle.
//  * P is produced as 256 P straight from exp2 (the static scale folded into the exponent); dS is
//    carried as 256 dS, which shifts its E8M0 code by exactly 8 (power-of-two scaling is exact).
#include <cmath>
#include <type_traits>

#include "mx_device.h"
#include "mxfa_internal.h"

namespace {

constexpr int kTile = 128;
constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row) { return lds_swz(row); }

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = bid & 7, slot = bid >> 3;
  return x * per + (x < rem ? x : rem) + slot;
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Per-lane constants for filling a 128 x 128-byte swizzled LDS tile with direct global -> LDS loads:
// lane piece c of wave w covers tile row trow[c], logical chunk byte offset tcol[c].
struct TileLane {
  int trow[4], tcol[4];
  uint32_t toff[4];  // trow * C + tcol (full tiles)
};

__device__ __forceinline__ TileLane tile_lane(int wave, int lane, int C) {
  TileLane t;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int p = (wave * 4 + c) * 64 + lane;
    t.trow[c] = p >> 3;
    t.tcol[c] = 16 * ((p & 7) ^ swz(p >> 3));
    t.toff[c] = (uint32_t)(t.trow[c] * C + t.tcol[c]);
  }
  return t;
}

// Asynchronous copy of a tile whose first row is at `base` (this head's columns). Rows at or past
// `valid` re-fetch the last valid row (finite data; their contributions are masked to zero).
__device__ __forceinline__ void issue_tile_load(uint8_t* lds_tile, const uint8_t* base, int valid, int C,
                                                const TileLane& t, int wave_s) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t off = valid >= kTile ? t.toff[c] : (uint32_t)(min(t.trow[c], valid - 1) * C + t.tcol[c]);
    __builtin_amdgcn_global_load_lds((const void*)(base + off), (MX_LDS void*)(lds_tile + (wave_s * 4 + c) * 1024),
                                     16, 0, 0);
  }
}

// A/B operand of a 32x32x64 MFMA from a row of a swizzled LDS tile: 16 bytes at k = 16 hh and
// 16 bytes at k = 32 + 16 hh of the 64-byte step ds.
__device__ __forceinline__ mx_v8i lds_row_operand(const uint8_t* lds, int row, int ds, int hh) {
  const uint8_t* p = lds + row * kD;
  const int sw = swz(row);
  uint4 lo = *reinterpret_cast<const uint4*>(p + 16 * ((4 * ds + hh) ^ sw));
  uint4 hi = *reinterpret_cast<const uint4*>(p + 16 * ((4 * ds + 2 + hh) ^ sw));
  return mx_v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Transposed operand from a swizzled [row][col] LDS tile: lane (column col0 + l % 32, hh) receives
// rows 64 ks + {8 i + 4 hh + t} (bytes 0-15) and 64 ks + 32 + {8 i + 4 hh + t} (bytes 16-31),
// i, t = 0..3, i.e. the key/query order of an MFMA accumulator.
__device__ __forceinline__ mx_v8i lds_tr_operand(const uint8_t* lds, int ks, int col0, int tr_row, int tr_col,
                                                 int tr_swz) {
  mx_v2i part[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int row = 64 * ks + 32 * (cc >> 1) + 16 * (cc & 1) + tr_row;
    const int col = col0 + tr_col;
    const int off = row * kD + 16 * ((col >> 4) ^ tr_swz) + (col & 15);
    part[cc] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MX_LDS mx_v2i*)(lds + off));
  }
  return mx_v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
}

// Maximum over the 64 lanes of a wave: DPP within rows of 16, one bpermute across rows, one
// permlane32 swap across the halves.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)s[0], (uint32_t)s[1]);
}

// ---------------------------------------------------------------------------------------------
// Preprocess: Delta[h][t] = sum_d dO[t, h, d] * O[t, h, d] (fp32); the exponent offset of 256 P,
// b[h][t] = 8 - LSE[h][t] log2(e) (so 256 P = exp2(c log2(e) S + b)); and zero the dQ accumulator.
// One wave per (token, head) row of 128: two bf16 pairs per lane.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_preprocess_kernel(const uint16_t* __restrict__ o,
                                                             const uint16_t* __restrict__ dout,
                                                             const float* __restrict__ lse, int64_t T, int H,
                                                             float* __restrict__ delta, float* __restrict__ pexp,
                                                             uint32_t* __restrict__ acc, int64_t acc_words) {
  const int64_t gw = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (gw < T * H) {
    const int64_t t = gw / H;
    const int h = (int)(gw % H);
    const uint32_t a = *reinterpret_cast<const uint32_t*>(o + gw * kD + 2 * lane);
    const uint32_t b = *reinterpret_cast<const uint32_t*>(dout + gw * kD + 2 * lane);
    float sum = bf16_to_f32(a & 0xffffu) * bf16_to_f32(b & 0xffffu) + bf16_to_f32(a >> 16) * bf16_to_f32(b >> 16);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) {
      delta[(int64_t)h * T + t] = sum;
      pexp[(int64_t)h * T + t] = 8.0f - lse[(int64_t)h * T + t] * kLog2e;
    }
  }
  // zero the accumulator (grid-stride over 16-byte words)
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < acc_words / 4; i += nthreads)
    reinterpret_cast<uint4*>(acc)[i] = make_uint4(0, 0, 0, 0);
}

struct BwdParams {
  const uint8_t *q, *k, *v, *dO;
  const uint8_t *q_scale, *k_scale, *v_scale, *dO_scale;
  int v_row_shift;  // V along D: 0 ROW32, 5 SQ32
  const int32_t *cu_q, *cu_k;
  int nseq, H, n_ktiles;
  int total_items;
  float c2;  // c * log2(e)
  int causal;
  const float* pexp;   // [H][Tq]: 8 - LSE log2(e)
  const float* delta;  // [H][Tq]
  int64_t Tq;
  int dq_fp16;
  int log2_sigma;  // FP16 static scale sigma = 2^log2_sigma (0 in FP32 mode)
  void* dq_acc;  // [Tq, C] fp32 or fp16
  float c;
  uint16_t *dk, *dv;
};

__global__ void __launch_bounds__(256, 1) attn_bwd_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k[kTile * kD];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_qd[2][2][kTile * kD];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(1024))) uint8_t lds_ds[kTile * kD];        // dS_q, key-major [kv][q]
  __shared__ __attribute__((aligned(512))) float lds_ld[2][2][kTile];          // [stage][8 - LSE log2e, Delta]
  __shared__ uint32_t lds_dscode[4];                                           // [kv block] -> 4 q-block codes
  __shared__ int64_t red[16];

  const int item = xcd_remap((int)blockIdx.x, p.total_items);
  const int kt = item % p.n_ktiles;
  const int h = (item / p.n_ktiles) % p.H;
  const int s = item / (p.n_ktiles * p.H);
  const int64_t q_start = p.cu_q[s], k_start = p.cu_k[s];
  const int Lq = p.cu_q[s + 1] - (int)q_start;
  const int Lk = p.cu_k[s + 1] - (int)k_start;
  if (kt * kTile >= Lk) return;

  const SeqOffsets qoff = seq_offsets(p.cu_q, s, red);
  const SeqOffsets koff = seq_offsets(p.cu_k, s, red);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int r = lane & 31, hh = lane >> 5;
  const int C = p.H * kD;
  const int Cs = C >> 5;
  const int kv0 = kt * kTile;
  const int kvrow = kv0 + 32 * wave + r;  // this lane's key row (B operands of S and dP)
  const TileLane tl = tile_lane(wave, lane, C);

  const int n_qtiles = (Lq + kTile - 1) / kTile;
  const int qt_begin = p.causal ? kt : 0;

  const uint8_t* qbase = p.q + q_start * (int64_t)C + h * kD;
  const uint8_t* dobase = p.dO + q_start * (int64_t)C + h * kD;
  const float* lse_base = p.pexp + (int64_t)h * p.Tq + q_start;
  const float* del_base = p.delta + (int64_t)h * p.Tq + q_start;
  // exponent offsets and Delta of a query tile: waves 0 and 1 each copy one 128-float vector (one
  // 4-byte element per lane, two pieces of 64 lanes).
  auto issue_ld_load = [&](int st, int q0) {
    if (wave_s < 2) {
      const float* src = wave_s == 0 ? lse_base : del_base;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = min(q0 + c * 64 + lane, Lq - 1);
        __builtin_amdgcn_global_load_lds((const void*)(src + row), (MX_LDS void*)(&lds_ld[st][wave_s][c * 64]), 4, 0,
                                         0);
      }
    }
  };

  // prologue: K tile, the first Q/dO tile and its LSE/Delta
  issue_tile_load(lds_k, p.k + (k_start + kv0) * (int64_t)C + h * kD, Lk - kv0, C, tl, wave_s);
  if (qt_begin < n_qtiles) {
    const int64_t q0 = (int64_t)qt_begin * kTile;
    issue_tile_load(lds_qd[qt_begin & 1][0], qbase + q0 * C, Lq - (int)q0, C, tl, wave_s);
    issue_tile_load(lds_qd[qt_begin & 1][1], dobase + q0 * C, Lq - (int)q0, C, tl, wave_s);
    issue_ld_load(qt_begin & 1, (int)q0);
  }

  // this wave's K and V rows in VGPRs (B operands of S = Q K^T and dP = dO V^T)
  mx_v8i kb_op[2], vb_op[2];
  {
    const bool valid = kvrow < Lk;
    const uint8_t* ks = p.k + (k_start + kvrow) * (int64_t)C + h * kD;
    const uint8_t* vs = p.v + (k_start + kvrow) * (int64_t)C + h * kD;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
      if (valid) {
        a0 = *reinterpret_cast<const uint4*>(ks + 64 * ds + 16 * hh);
        a1 = *reinterpret_cast<const uint4*>(ks + 64 * ds + 32 + 16 * hh);
        b0 = *reinterpret_cast<const uint4*>(vs + 64 * ds + 16 * hh);
        b1 = *reinterpret_cast<const uint4*>(vs + 64 * ds + 32 + 16 * hh);
      }
      kb_op[ds] = mx_v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      vb_op[ds] = mx_v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    }
  }
  // K (SQ32) and V (ROW32/SQ32) scales along D of this lane's key row: byte 0 = d-block hh, byte 2 =
  // d-block 2 + hh
  const uint32_t ksc_b =
      *reinterpret_cast<const uint32_t*>(p.k_scale + ((koff.padded + kvrow) >> 5) * (int64_t)Cs + h * 4) >> (8 * hh);
  const uint32_t vsc_b =
      *reinterpret_cast<const uint32_t*>(p.v_scale + ((koff.padded + kvrow) >> p.v_row_shift) * (int64_t)Cs + h * 4) >>
      (8 * hh);
  // K's scales for dQ = dS K (B operand: key block 2 ks + hh, d-block db): one word per key step
  uint32_t kq_sc[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    kq_sc[ks] =
        *reinterpret_cast<const uint32_t*>(p.k_scale + ((koff.padded + kv0) / 32 + 2 * ks + hh) * (int64_t)Cs + h * 4);

  // Q and dO scales of a query tile (SQ32): one word (4 d-blocks) per query block, raw
  const uint8_t* qs_base = p.q_scale + (qoff.padded >> 5) * (int64_t)Cs + h * 4;
  const uint8_t* ds_base = p.dO_scale + (qoff.padded >> 5) * (int64_t)Cs + h * 4;
  uint32_t qsc[4], dosc[4];
  auto load_q_scales = [&](int qt) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const uint32_t off = (uint32_t)((qt * 4 + qb) * Cs);
      qsc[qb] = *reinterpret_cast<const uint32_t*>(qs_base + off);
      dosc[qb] = *reinterpret_cast<const uint32_t*>(ds_base + off);
    }
  };
  if (qt_begin < n_qtiles) load_q_scales(qt_begin);

  mx_v16f dk_acc[4], dv_acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dk_acc[i] = mx_v16f{};
    dv_acc[i] = mx_v16f{};
  }

  // per-lane constants of the transposed LDS reads
  const int grp = lane >> 4, gl = lane & 15;
  const int tb = gl >> 1, ts = gl & 1;
  const int tr_row = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);
  const int tr_col = 16 * (grp & 1) + 8 * ts;
  const int tr_swz = swz(tr_row);

  // dQ accumulator addressing: element (query row, column) of this head
  float* dq32 = reinterpret_cast<float*>(p.dq_acc) + q_start * (int64_t)C + h * kD;
  __half2* dq16 = reinterpret_cast<__half2*>(reinterpret_cast<__half*>(p.dq_acc) + q_start * (int64_t)C + h * kD);
  const bool odd = r & 1;

  wait_vm();
  __syncthreads();

  for (int qt = qt_begin; qt < n_qtiles; ++qt) {
    const int q0 = qt * kTile;
    const int st = qt & 1;
    const uint8_t* lds_q = lds_qd[st][0];
    const uint8_t* lds_do = lds_qd[st][1];
    const float* pexp = lds_ld[st][0];
    const float* dlt = lds_ld[st][1];
    // prefetch the next query tile
    if (qt + 1 < n_qtiles) {
      const int64_t nq0 = (int64_t)(q0 + kTile);
      issue_tile_load(lds_qd[st ^ 1][0], qbase + nq0 * C, Lq - (int)nq0, C, tl, wave_s);
      issue_tile_load(lds_qd[st ^ 1][1], dobase + nq0 * C, Lq - (int)nq0, C, tl, wave_s);
      issue_ld_load(st ^ 1, (int)nq0);
    }

    // raw Q and dO scales for the B operands of G3 and G4 (query block 2 ks + hh, d-block db)
    uint32_t qsc_t[2], dosc_t[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qsc_t[ks] = hh ? qsc[2 * ks + 1] : qsc[2 * ks];
      dosc_t[ks] = hh ? dosc[2 * ks + 1] : dosc[2 * ks];
    }
    uint32_t qsc_c[4], dosc_c[4];  // this tile's along-D scales for G1 and G2
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      qsc_c[qb] = qsc[qb] >> (8 * hh);
      dosc_c[qb] = dosc[qb] >> (8 * hh);
    }
    if (qt + 1 < n_qtiles) load_q_scales(qt + 1);
    const bool need_mask = (q0 + kTile > Lq) || (kv0 + kTile > Lk) || (p.causal && kv0 + kTile - 1 > q0);
    uint32_t codes = 0;  // dS codes of the four query blocks, one byte each

    // Two halves of 64 queries (query blocks 2 ks, 2 ks + 1): the 64-query contraction step of G3/G4.
    // Software pipeline inside the wave: the S and dP MFMAs of half 1 are issued before the
    // elementwise work of half 0, so the matrix core runs them while the VALU works.
    auto g12 = [&](int ks, mx_v16f* sacc, mx_v16f* dpacc) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int qb = 2 * ks + j;
        const int row = 32 * qb + r;
        mx_v8i qa0 = lds_row_operand(lds_q, row, 0, hh);
        mx_v8i qa1 = lds_row_operand(lds_q, row, 1, hh);
        sacc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa0, kb_op[0], mx_v16f{}, 0, 0, 0, (int)qsc_c[qb], 0,
                                                                  (int)ksc_b);
        sacc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa1, kb_op[1], sacc[j], 0, 0, 2, (int)qsc_c[qb], 2,
                                                                  (int)ksc_b);
        mx_v8i da0 = lds_row_operand(lds_do, row, 0, hh);
        mx_v8i da1 = lds_row_operand(lds_do, row, 1, hh);
        dpacc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(da0, vb_op[0], mx_v16f{}, 0, 0, 0, (int)dosc_c[qb],
                                                                   0, (int)vsc_b);
        dpacc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(da1, vb_op[1], dpacc[j], 0, 0, 2, (int)dosc_c[qb], 2,
                                                                   (int)vsc_b);
        // issue order: these MFMAs stay here, ahead of the elementwise work that follows
        asm volatile("" : "+v"(sacc[j]), "+v"(dpacc[j])::"memory");
      }
    };
    mx_v16f sacc_h[2][2], dpacc_h[2][2];
    g12(0, sacc_h[0], dpacc_h[0]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks == 0) g12(1, sacc_h[1], dpacc_h[1]);
      mx_v16f* sacc = sacc_h[ks];
      mx_v16f* dpacc = dpacc_h[ks];

      // ---- 256 P, 256 dS (lane: key kvrow; queries 32 qb + 8 i + 4 hh + t) ----
      // Two instantiations behind one wave-uniform branch: interior tiles carry no mask code.
      uint32_t pk[2][4], dsk[2][4], dscode[2];
      auto elementwise = [&](auto masked) {
        constexpr bool MASK = decltype(masked)::value;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int qb = 2 * ks + j;
          uint32_t am = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // the lane's 4 consecutive query rows 32 qb + 8 i + 4 hh + (0..3)
            const float4 pe4 = *reinterpret_cast<const float4*>(pexp + 32 * qb + 8 * i + 4 * hh);
            const float4 dl4 = *reinterpret_cast<const float4*>(dlt + 32 * qb + 8 * i + 4 * hh);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int v = 4 * i + t;
              const float pe = (&pe4.x)[t], dl = (&dl4.x)[t];
              float e = __builtin_amdgcn_exp2f(fmaf(sacc[j][v], p.c2, pe));  // 256 P
              if (MASK) {
                const int qpos = q0 + 32 * qb + 8 * i + 4 * hh + t;
                const bool ok = (kvrow < Lk) & (qpos < Lq) & ((p.causal == 0) | (kvrow <= qpos));
                e = ok ? e : 0.0f;
              }
              const float dsv = e * (dpacc[j][v] - dl);  // 256 dS
              sacc[j][v] = e;
              dpacc[j][v] = dsv;
              am = max(am, __float_as_uint(dsv) & 0x7fffffffu);
            }
          }
          // block maximum over the wave (one 32 x 32 block), code of dS = code of 256 dS - 8
          const uint32_t c256 = mx_code_from_amax_bits(wave_max_dpp(am));
          dscode[j] = c256 == 255u ? 255u : (c256 > 8u ? c256 - 8u : 0u);
          // 256 dS * 2^(127 - (code + 8)) = dS * 2^(127 - code)
          const float inv = dscode[j] == 255u ? 0.0f : mx_inv_scale(dscode[j] + 8u);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pk[j][i] = mx_pack4_inrange(sacc[j][4 * i], sacc[j][4 * i + 1], sacc[j][4 * i + 2], sacc[j][4 * i + 3]);
            const uint32_t w = mx_pack4(dpacc[j][4 * i] * inv, dpacc[j][4 * i + 1] * inv, dpacc[j][4 * i + 2] * inv,
                                        dpacc[j][4 * i + 3] * inv);
            dsk[j][i] = dscode[j] == 255u ? 0x7f7f7f7fu : w;
          }
        }
      };
      if (need_mask)
        elementwise(std::true_type{});
      else
        elementwise(std::false_type{});
      codes |= (dscode[0] << (16 * ks)) | (dscode[1] << (16 * ks + 8));

      // ---- dS_q to LDS, key-major [kv][q], for dQ ----
      {
        const int kvl = 32 * wave + r;  // key row inside the tile
        const int sw = swz(kvl);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ql = 32 * (2 * ks + j) + 8 * i + 4 * hh;
            *reinterpret_cast<uint32_t*>(lds_ds + kvl * kD + 16 * ((ql >> 4) ^ sw) + (ql & 15)) = dsk[j][i];
          }
      }

      // ---- G3: dV += P_q^T dO  and  G4: dK += dS_q^T Q  (this 64-query step) ----
      {
        mx_v8i pa{(int)pk[0][0], (int)pk[0][1], (int)pk[0][2], (int)pk[0][3],
                  (int)pk[1][0], (int)pk[1][1], (int)pk[1][2], (int)pk[1][3]};
        mx_v8i sa{(int)dsk[0][0], (int)dsk[0][1], (int)dsk[0][2], (int)dsk[0][3],
                  (int)dsk[1][0], (int)dsk[1][1], (int)dsk[1][2], (int)dsk[1][3]};
        // A-operand scale of dS_q: k-block hh of this step is query block 2 ks + hh
        const uint32_t sa_sc = hh ? dscode[1] : dscode[0];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          mx_v8i dob = lds_tr_operand(lds_do, ks, 32 * db, tr_row, tr_col, tr_swz);
          dv_acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, dob, dv_acc[db], 0, 0, 0, 119, 0,
                                                                       (int)(dosc_t[ks] >> (8 * db)));
          mx_v8i qbt = lds_tr_operand(lds_q, ks, 32 * db, tr_row, tr_col, tr_swz);
          dk_acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(sa, qbt, dk_acc[db], 0, 0, 0, (int)sa_sc, 0,
                                                                       (int)(qsc_t[ks] >> (8 * db)));
          // Keep these MFMAs here (the compiler would otherwise sink them below the barrier and hold
          // all of their operands in registers); the accumulators stay in AGPRs.
          asm volatile("" : "+a"(dv_acc[db]), "+a"(dk_acc[db])::"memory");
        }
      }
    }
    if (lane == 0) lds_dscode[wave] = codes;
    __syncthreads();  // dS_q of all four waves is in LDS
    // This thread's part of the next query tile has landed (and the previous tile's dQ atomics,
    // which had a whole iteration to drain, are done); this tile's atomics stay in flight.
    wait_vm();

    // ---- G5: dQ rows 32 wave.. of this tile = dS_q K over the 128 keys; atomics ----
    // The FP16 static scale sigma (a power of two) is folded into dS_q's E8M0 code here, so the MFMA
    // returns sigma dQ exactly with no multiply.
    {
      uint32_t a_sc[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = (int)((lds_dscode[2 * ks + hh] >> (8 * wave)) & 0xffu);
        a_sc[ks] = c == 255 ? 255u : (uint32_t)min(max(c + p.log2_sigma, 0), 254);
      }
      mx_v8i dsa[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dsa[ks] = lds_tr_operand(lds_ds, ks, 32 * wave, tr_row, tr_col, tr_swz);
      // rows of the wave's block: 8 (v/4) + 4 hh + v%4; the v-dependent part is a scalar offset
      const int qr0 = q0 + 32 * wave;
      const bool full = qr0 + 32 <= Lq;  // wave-uniform: no row of this block is past the sequence
      const uint32_t lane_row = (uint32_t)(4 * hh);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        mx_v16f acc = mx_v16f{};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          mx_v8i kbt = lds_tr_operand(lds_k, ks, 32 * db, tr_row, tr_col, tr_swz);
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(dsa[ks], kbt, acc, 0, 0, 0, (int)a_sc[ks], 0,
                                                                (int)(kq_sc[ks] >> (8 * db)));
        }
        // acc: column d = 32 db + r, rows 8 (v/4) + 4 hh + v%4 of the wave's 32-query block
        if (!p.dq_fp16) {
          const uint32_t lane_off = lane_row * C + 32 * db + r;
#define MXFA_DQ32(V)                                                                              \
  {                                                                                               \
    const int rv = 8 * ((V) >> 2) + ((V) & 3);                                                    \
    float* rowp = dq32 + (size_t)(qr0 + rv) * C; /* wave-uniform */                               \
    if (full || qr0 + rv + (int)lane_row < Lq) unsafeAtomicAdd(rowp + lane_off, acc[V]);          \
  }
          MXFA_DQ32(0) MXFA_DQ32(1) MXFA_DQ32(2) MXFA_DQ32(3) MXFA_DQ32(4) MXFA_DQ32(5) MXFA_DQ32(6) MXFA_DQ32(7)
          MXFA_DQ32(8) MXFA_DQ32(9) MXFA_DQ32(10) MXFA_DQ32(11) MXFA_DQ32(12) MXFA_DQ32(13) MXFA_DQ32(14)
          MXFA_DQ32(15)
#undef MXFA_DQ32
        } else {
          // Pair neighbouring columns: the even lane adds (row v, columns d, d+1), the odd lane adds
          // (row v+1, columns d-1, d). One DPP swap with the neighbour lane per pair.
          const uint32_t lane_off = (lane_row + (odd ? 1u : 0u)) * (uint32_t)(C >> 1) + (uint32_t)((32 * db + r) >> 1);
#define MXFA_DQ16(V)                                                                              \
  {                                                                                               \
    const float send = odd ? acc[V] : acc[(V) + 1];                                               \
    const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false)); \
    const float lo = odd ? other : acc[V];                                                        \
    const float hi = odd ? acc[(V) + 1] : other;                                                  \
    const int rv = 8 * ((V) >> 2) + ((V) & 3);                                                    \
    __half2* rowp = dq16 + (size_t)(qr0 + rv) * (C >> 1); /* wave-uniform */                      \
    if (full || qr0 + rv + (int)lane_row + (odd ? 1 : 0) < Lq)                                    \
      unsafeAtomicAdd(rowp + lane_off, __floats2half2_rn(lo, hi));                                \
  }
          MXFA_DQ16(0) MXFA_DQ16(2) MXFA_DQ16(4) MXFA_DQ16(6) MXFA_DQ16(8) MXFA_DQ16(10) MXFA_DQ16(12)
          MXFA_DQ16(14)
#undef MXFA_DQ16
        }
        asm volatile("" ::: "memory");  // the next D-block's operand reads stay below these atomics
      }
    }
    __syncthreads();  // every thread's part of the next tile has landed; all reads of this stage,
                      // of dS_q and of the codes are done
  }

  // ---- epilogue: dK = c dK, dV -> bf16 (accumulator: column d = 32 db + r, rows kv) ----
  uint16_t* dkb = p.dk + (k_start + kv0 + 32 * wave) * (int64_t)C + h * kD;
  uint16_t* dvb = p.dv + (k_start + kv0 + 32 * wave) * (int64_t)C + h * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kr = 8 * (v >> 2) + 4 * hh + (v & 3);
      if (kv0 + 32 * wave + kr < Lk) {
        const uint32_t idx = (uint32_t)(kr * C + 32 * db + r);
        dkb[idx] = (uint16_t)f32_to_bf16(dk_acc[db][v] * p.c);
        dvb[idx] = (uint16_t)f32_to_bf16(dv_acc[db][v]);
      }
    }
}

// dQ = bf16(c * acc / sigma)
__global__ void __launch_bounds__(256) bwd_finalize_kernel(const void* __restrict__ acc, int dq_fp16, float mult,
                                                           int64_t n, uint16_t* __restrict__ dq) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4];
  if (dq_fp16) {
    const __half2* a = reinterpret_cast<const __half2*>(acc) + i / 2;
    float2 x0 = __half22float2(a[0]), x1 = __half22float2(a[1]);
    v[0] = x0.x; v[1] = x0.y; v[2] = x1.x; v[3] = x1.y;
  } else {
    float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(acc) + i);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  uint2 out;
  out.x = f32_to_bf16(v[0] * mult) | (f32_to_bf16(v[1] * mult) << 16);
  out.y = f32_to_bf16(v[2] * mult) | (f32_to_bf16(v[3] * mult) << 16);
  *reinterpret_cast<uint2*>(dq + i) = out;
}

}  // namespace

namespace mxfa {

// Workspace: dQ accumulator [Tq, H*D] (fp32 or fp16), then Delta [H][Tq] and the exponent offsets
// [H][Tq] (fp32), each 256-byte aligned.
size_t bwd_workspace_bytes(int64_t Tq, int H, int D, int dq_fp16) {
  const size_t acc = (size_t)Tq * H * D * (dq_fp16 ? 2 : 4);
  const size_t vec = ((size_t)Tq * H * 4 + 255) / 256 * 256;
  return (acc + 255) / 256 * 256 + 2 * vec;
}

hipError_t launch_attn_bwd(const AttnProblem& a, const MxOperand& v_d, const MxOperand& dout, const uint16_t* o,
                           const uint16_t* dout_bf16, const float* lse, int dq_fp16, float sigma, void* workspace,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, hipStream_t stream) {
  const int64_t Tq = a.total_q;
  const int C = a.H * kD;
  const size_t acc_bytes = (size_t)Tq * C * (dq_fp16 ? 2 : 4);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  void* acc = ws;
  float* delta = reinterpret_cast<float*>(ws + (acc_bytes + 255) / 256 * 256);
  float* pexp = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(delta) + ((size_t)Tq * a.H * 4 + 255) / 256 * 256);
  {
    const int64_t rows = Tq * a.H;  // one wave per row
    int64_t blocks = (rows + 3) / 4;
    if (blocks < 1) blocks = 1;
    const int64_t acc_words = (int64_t)((acc_bytes + 15) / 16 * 4);
    hipLaunchKernelGGL(bwd_preprocess_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o, dout_bf16, lse, Tq,
                       a.H, delta, pexp, reinterpret_cast<uint32_t*>(acc), acc_words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdParams p;
  p.q = a.q.data; p.k = a.k.data; p.v = v_d.data; p.dO = dout.data;
  p.q_scale = a.q.scale; p.k_scale = a.k.scale; p.v_scale = v_d.scale; p.dO_scale = dout.scale;
  p.v_row_shift = v_d.mode == 0 ? 0 : 5;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.nseq = a.nseq; p.H = a.H;
  p.n_ktiles = (a.max_seqlen_k + kTile - 1) / kTile;
  p.total_items = p.n_ktiles * a.H * a.nseq;  // < 2^31, checked by the caller
  p.c2 = a.softmax_scale * kLog2e;
  p.causal = a.causal;
  p.pexp = pexp; p.delta = delta; p.Tq = Tq;
  p.dq_fp16 = dq_fp16;
  {
    int e = 0;
    std::frexp(dq_fp16 ? sigma : 1.0f, &e);  // sigma = 0.5 * 2^e exactly (a power of two, checked by the caller)
    p.log2_sigma = e - 1;
  }
  p.dq_acc = acc;
  p.c = a.softmax_scale;
  p.dk = dk; p.dv = dv;
  if (p.total_items > 0) {
    hipLaunchKernelGGL(attn_bwd_kernel, dim3((unsigned)p.total_items), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = Tq * C;
  if (n > 0) {
    const float mult = a.softmax_scale / (dq_fp16 ? sigma : 1.0f);
    hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, acc, dq_fp16,
                       mult, n, dq);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mxfa

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
//  * Workgroup = 8 waves (two per SIMD) = one 128-row KV tile. Wave w owns key rows 32 (w & 3) ..
//    +31 and query half w >> 2 of every query tile (queries 64 (w >> 2) .. +63). Its K and V rows
//    (from the K and V tiles in LDS) are the B operands of S = Q K^T and dP = dO V^T, so S and dP
//    come out with one key per lane (column) and 16 queries per lane per 32-query block.
//  * That accumulator layout is exactly the A operand of dV = P^T dO and dK = dS^T Q (one key per
//    lane, contraction over queries): P_q and dS_q bytes are used in place, in the accumulator's
//    query order; dO^T and Q^T are read from LDS with ds_read_b64_tr_b8 in the same order.
//  * The two waves that share a key block split the accumulators instead of duplicating them: the
//    query-half-0 wave accumulates dV, the query-half-1 wave dK, over all 128 queries of the tile.
//    Each hands the other the packed operand it lacks (P_q or dS_q of its half, 2 KB) through LDS,
//    so a wave holds one 32 x 128 FP32 accumulator and two waves fit on each SIMD.
//  * dQ = dS K contracts over all 128 keys of the tile: dS_q goes to LDS key-major, each wave then
//    computes one 32 x 64 block of the tile's dQ and adds it to the accumulator with coalesced
//    buffer atomics (packed FP16 pairs or FP32).
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

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the
// counters not waited on are at their maximum).
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm16 = 0x4F70;
constexpr int kWaitVm32 = 0x8F70;
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(kWaitVm0); }

constexpr int kWaves = 8;
constexpr int kPieces = kTile * kD / 1024 / kWaves;  // 1 KB pieces (64 lanes x 16 B) per wave per tile

// Per-lane constants for filling a 128 x 128-byte swizzled LDS tile with direct global -> LDS loads:
// lane piece c of wave w covers tile row trow[c], logical chunk byte offset tcol[c].
struct TileLane {
  int trow[kPieces], tcol[kPieces];
  uint32_t toff[kPieces];  // trow * C + tcol (full tiles)
};

__device__ __forceinline__ TileLane tile_lane(int wave, int lane, int C) {
  TileLane t;
#pragma unroll
  for (int c = 0; c < kPieces; ++c) {
    const int p = (wave * kPieces + c) * 64 + lane;
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
  for (int c = 0; c < kPieces; ++c) {
    const uint32_t off = valid >= kTile ? t.toff[c] : (uint32_t)(min(t.trow[c], valid - 1) * C + t.tcol[c]);
    mx_lds_dma16((MX_LDS void*)(lds_tile + (wave_s * kPieces + c) * 1024), base, off);
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

__global__ void __launch_bounds__(512, 1) attn_bwd_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k[kTile * kD];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v[kTile * kD];         // V along D (for dP)
  __shared__ __attribute__((aligned(1024))) uint8_t lds_qd[2][2][kTile * kD];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(1024))) uint8_t lds_ds[kTile * kD];        // dS_q, key-major [kv][q]
  __shared__ __attribute__((aligned(1024))) uint4 lds_xchg[kWaves][2][64];     // operand handed to the partner
  __shared__ __attribute__((aligned(512))) float lds_ld[2][2][kTile];          // [stage][8 - LSE log2e, Delta]
  __shared__ __attribute__((aligned(256))) uint32_t lds_sc[2][64];             // [stage][Q, dO scale words]
  __shared__ uint8_t lds_dscode[4][4];                                         // dS codes [kv block][q block]
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
  const int kw = wave_s & 3;    // key block of this wave
  const int half = wave_s >> 2;  // query half of every tile; 0: accumulates dV, 1: accumulates dK
  const int r = lane & 31, hh = lane >> 5;
  const int C = p.H * kD;
  const int Cs = C >> 5;
  const int kv0 = kt * kTile;
  const int kvrow = kv0 + 32 * kw + r;  // this lane's key row (B operands of S and dP)
  const TileLane tl = tile_lane(wave, lane, C);

  const int n_qtiles = (Lq + kTile - 1) / kTile;
  const int qt_begin = p.causal ? kt : 0;

  // wave-uniform base pointers, kept in scalar registers
  const uint8_t* qbase = (const uint8_t*)mx_uniform_ptr((void*)(p.q + q_start * (int64_t)C + h * kD));
  const uint8_t* dobase = (const uint8_t*)mx_uniform_ptr((void*)(p.dO + q_start * (int64_t)C + h * kD));
  const float* lse_base = (const float*)mx_uniform_ptr((void*)(p.pexp + (int64_t)h * p.Tq + q_start));
  const float* del_base = (const float*)mx_uniform_ptr((void*)(p.delta + (int64_t)h * p.Tq + q_start));
  // exponent offsets and Delta of a query tile: waves 0 and 1 each copy one 128-float vector (one
  // 4-byte element per lane, two pieces of 64 lanes).
  auto issue_ld_load = [&](int st, int q0) {
    if (wave_s < 2) {
      const float* src = wave_s == 0 ? lse_base : del_base;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = min(q0 + c * 64 + lane, Lq - 1);
        mx_lds_dma4((MX_LDS void*)(&lds_ld[st][wave_s][c * 64]), src, (uint32_t)row * 4u);
      }
    }
  };

  // prologue: K and V tiles, the first Q/dO tile and its LSE/Delta
  issue_tile_load(lds_k, p.k + (k_start + kv0) * (int64_t)C + h * kD, Lk - kv0, C, tl, wave_s);
  issue_tile_load(lds_v, p.v + (k_start + kv0) * (int64_t)C + h * kD, Lk - kv0, C, tl, wave_s);
  if (qt_begin < n_qtiles) {
    const int64_t q0 = (int64_t)qt_begin * kTile;
    issue_tile_load(lds_qd[qt_begin & 1][0], qbase + q0 * C, Lq - (int)q0, C, tl, wave_s);
    issue_tile_load(lds_qd[qt_begin & 1][1], dobase + q0 * C, Lq - (int)q0, C, tl, wave_s);
    issue_ld_load(qt_begin & 1, (int)q0);
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

  // Q and dO scales of a query tile (SQ32): one word (4 d-blocks) per query block, raw. Wave 2 copies
  // them into LDS with the tile (lanes 0-3: Q blocks, lanes 4-7: dO blocks, the rest repeat lane 0).
  const uint8_t* qs_base = p.q_scale + (qoff.padded >> 5) * (int64_t)Cs + h * 4;
  const uint8_t* ds_base = p.dO_scale + (qoff.padded >> 5) * (int64_t)Cs + h * 4;
  auto issue_sc_load = [&](int st, int qt) {
    if (wave_s == 2) {
      const int i = lane < 8 ? lane : 0;
      const uint8_t* src = (i < 4 ? qs_base : ds_base) + (int64_t)((qt * 4 + (i & 3)) * Cs);
      mx_lds_dma4_addr((MX_LDS void*)&lds_sc[st][0], src);
    }
  };
  if (qt_begin < n_qtiles) issue_sc_load(qt_begin & 1, qt_begin);
  uint32_t qsc[4], dosc[4];

  // dV (query-half-0 waves) or dK (query-half-1 waves) of this wave's 32 keys
  mx_v16f kv_acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kv_acc[i] = mx_v16f{};

  // per-lane constants of the transposed LDS reads
  const int grp = lane >> 4, gl = lane & 15;
  const int tb = gl >> 1, ts = gl & 1;
  const int tr_row = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);
  const int tr_col = 16 * (grp & 1) + 8 * ts;
  const int tr_swz = swz(tr_row);
  const bool odd = r & 1;
  const uint64_t odd_lanes = 0xAAAAAAAAAAAAAAAAull;

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
    // this tile's scale words (landed with the tile)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      qsc[qb] = lds_sc[st][qb];
      dosc[qb] = lds_sc[st][4 + qb];
    }
    if (qt + 1 < n_qtiles) {
      const int64_t nq0 = (int64_t)(q0 + kTile);
      issue_sc_load(st ^ 1, qt + 1);
      issue_tile_load(lds_qd[st ^ 1][0], (const uint8_t*)mx_uniform_ptr((void*)(qbase + nq0 * C)), Lq - (int)nq0, C,
                      tl, wave_s);
      issue_tile_load(lds_qd[st ^ 1][1], (const uint8_t*)mx_uniform_ptr((void*)(dobase + nq0 * C)), Lq - (int)nq0, C,
                      tl, wave_s);
      issue_ld_load(st ^ 1, (int)nq0);
    }

    // raw Q and dO scales for the B operands of G3 and G4 (query block 2 ks + hh, d-block db)
    uint32_t qsc_t[2], dosc_t[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qsc_t[ks] = hh ? qsc[2 * ks + 1] : qsc[2 * ks];
      dosc_t[ks] = hh ? dosc[2 * ks + 1] : dosc[2 * ks];
    }
    uint32_t qsc_c[2], dosc_c[2];  // this wave's query blocks' along-D scales for G1 and G2
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      qsc_c[j] = (half ? qsc[2 + j] : qsc[j]) >> (8 * hh);
      dosc_c[j] = (half ? dosc[2 + j] : dosc[j]) >> (8 * hh);
    }
    const bool need_mask = (q0 + kTile > Lq) || (kv0 + kTile > Lk) || (p.causal && kv0 + kTile - 1 > q0);

    // ---- per query block j of this wave's half: G1, G2 (S and dP), then 256 P, 256 dS ----
    // (lane: key kvrow; queries 64 half + 32 j + 8 i + 4 hh + t). Two instantiations of the
    // elementwise part behind one wave-uniform branch: interior tiles carry no mask code.
    uint32_t pk[2][4], dsk[2][4], dscode[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ql0 = 64 * half + 32 * j;  // first query of the block inside the tile
      mx_v16f sacc, dpacc;
      {
        const int row = ql0 + r;       // query row (A operand)
        const int krow = 32 * kw + r;  // key row (B operand), from the K and V tiles in LDS
        mx_v8i qa0 = lds_row_operand(lds_q, row, 0, hh);
        mx_v8i kb0 = lds_row_operand(lds_k, krow, 0, hh);
        mx_v8i qa1 = lds_row_operand(lds_q, row, 1, hh);
        mx_v8i kb1 = lds_row_operand(lds_k, krow, 1, hh);
        sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa0, kb0, mx_v16f{}, 0, 0, 0, (int)qsc_c[j], 0,
                                                               (int)ksc_b);
        sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa1, kb1, sacc, 0, 0, 2, (int)qsc_c[j], 2, (int)ksc_b);
        mx_v8i da0 = lds_row_operand(lds_do, row, 0, hh);
        mx_v8i vb0 = lds_row_operand(lds_v, krow, 0, hh);
        mx_v8i da1 = lds_row_operand(lds_do, row, 1, hh);
        mx_v8i vb1 = lds_row_operand(lds_v, krow, 1, hh);
        dpacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(da0, vb0, mx_v16f{}, 0, 0, 0, (int)dosc_c[j], 0,
                                                                (int)vsc_b);
        dpacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(da1, vb1, dpacc, 0, 0, 2, (int)dosc_c[j], 2,
                                                                (int)vsc_b);
        asm volatile("" : "+v"(sacc), "+v"(dpacc)::"memory");
      }
      auto elementwise = [&](auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the lane's 4 consecutive query rows ql0 + 8 i + 4 hh + (0..3)
          const float4 pe4 = *reinterpret_cast<const float4*>(pexp + ql0 + 8 * i + 4 * hh);
          const float4 dl4 = *reinterpret_cast<const float4*>(dlt + ql0 + 8 * i + 4 * hh);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int v = 4 * i + t;
            const float pe = (&pe4.x)[t], dl = (&dl4.x)[t];
            float e = __builtin_amdgcn_exp2f(fmaf(sacc[v], p.c2, pe));  // 256 P
            if (MASK) {
              const int qpos = q0 + ql0 + 8 * i + 4 * hh + t;
              const bool ok = (kvrow < Lk) & (qpos < Lq) & ((p.causal == 0) | (kvrow <= qpos));
              e = ok ? e : 0.0f;
            }
            const float dsv = e * (dpacc[v] - dl);  // 256 dS
            sacc[v] = e;
            dpacc[v] = dsv;
          }
          am = max3_abs(am, dpacc[4 * i], dpacc[4 * i + 1]);
          am = max3_abs(am, dpacc[4 * i + 2], dpacc[4 * i + 3]);
        }
        // block maximum over the wave (one 32 x 32 block), code of dS = code of 256 dS - 8
        const uint32_t c256 = mx_code_from_amax_bits(wave_max_dpp(__float_as_uint(am)));
        dscode[j] = c256 == 255u ? 255u : (c256 > 8u ? c256 - 8u : 0u);
        // 256 dS * 2^(127 - (code + 8)) = dS * 2^(127 - code)
        const float inv = dscode[j] == 255u ? 0.0f : mx_inv_scale(dscode[j] + 8u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[j][i] = mx_pack4_inrange(sacc[4 * i], sacc[4 * i + 1], sacc[4 * i + 2], sacc[4 * i + 3]);
          const uint32_t w =
              mx_pack4(dpacc[4 * i] * inv, dpacc[4 * i + 1] * inv, dpacc[4 * i + 2] * inv, dpacc[4 * i + 3] * inv);
          dsk[j][i] = dscode[j] == 255u ? 0x7f7f7f7fu : w;
        }
      };
      if (need_mask)
        elementwise(std::true_type{});
      else
        elementwise(std::false_type{});
    }

    // ---- dS_q to LDS key-major [kv][q] (for dQ); the partner's operand; the block codes ----
    {
      const int kvl = 32 * kw + r;  // key row inside the tile
      const int sw = swz(kvl);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ql = 64 * half + 32 * j + 8 * i + 4 * hh;
          *reinterpret_cast<uint32_t*>(lds_ds + kvl * kD + 16 * ((ql >> 4) ^ sw) + (ql & 15)) = dsk[j][i];
        }
      // the dV wave (half 0) needs the other half's P_q, the dK wave (half 1) the other half's dS_q
#pragma unroll
      for (int j = 0; j < 2; ++j)
        lds_xchg[wave_s][j][lane] = half ? make_uint4(pk[j][0], pk[j][1], pk[j][2], pk[j][3])
                                         : make_uint4(dsk[j][0], dsk[j][1], dsk[j][2], dsk[j][3]);
      if (lane == 0) {
        lds_dscode[kw][2 * half] = (uint8_t)dscode[0];
        lds_dscode[kw][2 * half + 1] = (uint8_t)dscode[1];
      }
    }
    __syncthreads();  // dS_q, the partner operands and the codes of all eight waves are in LDS

    // ---- G3 (half-0 waves): dV += P_q^T dO;  G4 (half-1 waves): dK += dS_q^T Q; all 128 queries ----
    {
      const int partner = wave_s ^ 4;
      const uint4 x0 = lds_xchg[partner][0][lane], x1 = lds_xchg[partner][1][lane];
      const mx_v8i other{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      if (half == 0) {
        const mx_v8i own{(int)pk[0][0], (int)pk[0][1], (int)pk[0][2], (int)pk[0][3],
                         (int)pk[1][0], (int)pk[1][1], (int)pk[1][2], (int)pk[1][3]};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const mx_v8i pa = ks == 0 ? own : other;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            mx_v8i dob = lds_tr_operand(lds_do, ks, 32 * db, tr_row, tr_col, tr_swz);
            kv_acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, dob, kv_acc[db], 0, 0, 0, 119, 0,
                                                                         (int)(dosc_t[ks] >> (8 * db)));
            asm volatile("" : "+v"(kv_acc[db])::"memory");
          }
        }
      } else {
        const mx_v8i own{(int)dsk[0][0], (int)dsk[0][1], (int)dsk[0][2], (int)dsk[0][3],
                         (int)dsk[1][0], (int)dsk[1][1], (int)dsk[1][2], (int)dsk[1][3]};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const mx_v8i sa = ks == 1 ? own : other;
          // A-operand scale of dS_q: k-block hh of this step is query block 2 ks + hh
          const uint32_t sa_sc = lds_dscode[kw][2 * ks + hh];
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            mx_v8i qbt = lds_tr_operand(lds_q, ks, 32 * db, tr_row, tr_col, tr_swz);
            kv_acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(sa, qbt, kv_acc[db], 0, 0, 0, (int)sa_sc, 0,
                                                                         (int)(qsc_t[ks] >> (8 * db)));
            asm volatile("" : "+v"(kv_acc[db])::"memory");
          }
        }
      }
    }

    // ---- G5: dQ block (query block wave & 3, d-blocks 2 half, 2 half + 1) = dS_q K; atomics ----
    // The FP16 static scale sigma (a power of two) is folded into dS_q's E8M0 code here, so the MFMA
    // returns sigma dQ exactly with no multiply.
    {
      const int qb = kw;
      uint32_t a_sc[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = (int)lds_dscode[2 * ks + hh][qb];
        a_sc[ks] = c == 255 ? 255u : (uint32_t)min(max(c + p.log2_sigma, 0), 254);
      }
      mx_v8i dsa[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dsa[ks] = lds_tr_operand(lds_ds, ks, 32 * qb, tr_row, tr_col, tr_swz);
      mx_v16f acc[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int db = 2 * half + e;
        acc[e] = mx_v16f{};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          mx_v8i kbt = lds_tr_operand(lds_k, ks, 32 * db, tr_row, tr_col, tr_swz);
          acc[e] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(dsa[ks], kbt, acc[e], 0, 0, 0, (int)a_sc[ks], 0,
                                                                   (int)(kq_sc[ks] >> (8 * db)));
        }
        asm volatile("" : "+v"(acc[e])::"memory");
      }
      // rows of the block: 8 (v/4) + 4 hh + v%4; the v-dependent part is a scalar offset
      const int qr0 = q0 + 32 * qb;
      const bool full = qr0 + 32 <= Lq;  // wave-uniform: no row of this block is past the sequence
      const uint32_t lane_row = (uint32_t)(4 * hh);
      // buffer over the block's 32 accumulator rows: scalar base, per-lane byte offset, scalar row offset
      const uint32_t esize = p.dq_fp16 ? 2u : 4u;
      const __amdgpu_buffer_rsrc_t dq_rsrc = mx_buffer_rsrc(
          mx_uniform_ptr(reinterpret_cast<char*>(p.dq_acc) + ((q_start + qr0) * (int64_t)C + h * kD) * esize),
          (uint32_t)__builtin_amdgcn_readfirstlane((int)(32u * C * esize)));
      // acc[e]: column d = 32 db + r, rows 8 (v/4) + 4 hh + v%4 of the query block
      auto atomics = [&](auto all_rows) {
        constexpr bool FULL = decltype(all_rows)::value;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int db = 2 * half + e;
          if (!p.dq_fp16) {
            const int lane_boff = (int)((lane_row * C + 32 * db + r) * 4u);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rv = 8 * (v >> 2) + (v & 3);
              if (FULL || qr0 + rv + (int)lane_row < Lq)
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[e][v], dq_rsrc, lane_boff, rv * C * 4, 0);
            }
          } else {
            // Pair neighbouring columns: the even lane adds (row v, columns d, d+1), the odd lane adds
            // (row v+1, columns d-1, d). One DPP swap with the neighbour lane per pair.
            const int lane_boff =
                (int)(((lane_row + (odd ? 1u : 0u)) * (uint32_t)(C >> 1) + (uint32_t)((32 * db + r) >> 1)) * 4u);
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
              const float a0 = acc[e][v], a1 = acc[e][v + 1];
              const float send = mx_select(odd_lanes, a0, a1);
              const float other =
                  __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
              const float lo = mx_select(odd_lanes, other, a0);
              const float hi = mx_select(odd_lanes, a1, other);
              const int rv = 8 * (v >> 2) + (v & 3);
              if (FULL || qr0 + rv + (int)lane_row + (odd ? 1 : 0) < Lq) {
                const __half2 hv = __floats2half2_rn(lo, hi);
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_v2f16(__builtin_bit_cast(mx_h2, hv), dq_rsrc, lane_boff,
                                                                  rv * C * 2, 0);
              }
            }
          }
        }
      };
      // Wait for this thread's part of the next query tile (issued at the top of the iteration).
      // Vector memory operations complete in issue order, so allowing the atomics issued since then
      // (16 FP16 or 32 FP32 per wave on full blocks) to stay in flight still covers the tile loads;
      // the atomics drain behind the next tile's work instead of stalling this wave.
      if (full) {
        atomics(std::true_type{});
        if (p.dq_fp16)
          __builtin_amdgcn_s_waitcnt(kWaitVm16);
        else
          __builtin_amdgcn_s_waitcnt(kWaitVm32);
      } else {
        atomics(std::false_type{});
        wait_vm();
      }
    }
    __syncthreads();  // every thread's part of the next tile has landed; all reads of this stage,
                      // of dS_q, of the partner operands and of the codes are done
  }

  // ---- epilogue: half-0 waves store dV, half-1 waves dK = c dK (accumulator: column d = 32 db + r,
  // rows kv 8 (v/4) + 4 hh + v%4 of the wave's key block) ----
  uint16_t* outb = (half ? p.dk : p.dv) + (k_start + kv0 + 32 * kw) * (int64_t)C + h * kD;
  const float mult = half ? p.c : 1.0f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kr = 8 * (v >> 2) + 4 * hh + (v & 3);
      if (kv0 + 32 * kw + kr < Lk) outb[(uint32_t)(kr * C + 32 * db + r)] = (uint16_t)f32_to_bf16(kv_acc[db][v] * mult);
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
    hipLaunchKernelGGL(attn_bwd_kernel, dim3((unsigned)p.total_items), dim3(64 * kWaves), 0, stream, p);
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

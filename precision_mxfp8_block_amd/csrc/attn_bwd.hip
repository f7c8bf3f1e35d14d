// MXFP8 attention backward for gfx950: recomputation with five scaled-MFMA GEMMs on square-block
// (32 x 32) quantized Q, K and dO, online dS quantization, dQ reduced over the KV tiles in order.
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
//     dK += dS_q^T Q;  dS_q stored for the dQ kernel
//   dK = c dK;  per Q tile (dQ kernel): dQ = c/sigma * reduction over KV tiles, in KV-tile order, of
//   dS_q K (FP16 holding sigma dQ, or FP32).
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
//  * dQ is not reduced with atomics: device-scope atomics on gfx950 are executed beyond the XCD's
//    L2 and sustain about 1.3 TB/s of payload (measured), so 32 KV tiles x 67 MB of FP16 partials
//    bound the backward at ~1.6 ms at 4 x 16 x 4096. Instead each (Q tile, KV tile) pair writes its
//    16 KB dS_q tile (FP8, half the bytes of an FP16 partial, plain streaming stores) and the dQ
//    kernel reads them back per Q tile and reduces dS_q K over the KV tiles in order, in FP16 with
//    the static scale or in FP32, with no atomics and a deterministic result.
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

// Waits on the vector memory counter, written as asm: the direct LDS loads are asm too, so the
// compiler does not see them and would drop a builtin wait it believes to be redundant.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_vm() { wait_vmcnt<0>(); }

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
// b[h][t] = 8 - LSE[h][t] log2(e) (so 256 P = exp2(c log2(e) S + b)).
// Sixteen lanes per (token, head) row of 128: eight bf16 of O and of dO per lane.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_preprocess_kernel(const uint16_t* __restrict__ o,
                                                             const uint16_t* __restrict__ dout,
                                                             const float* __restrict__ lse, int64_t T, int H,
                                                             float* __restrict__ delta, float* __restrict__ pexp) {
  // 16 lanes per (token, head) row of 128: 8 bf16 of O and of dO per lane (16-byte loads)
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int g = threadIdx.x & 15;
  const bool valid = row < T * H;
  float sum = 0.0f;
  if (valid) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * kD + 8 * g);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + row * kD + 8 * g);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sum += bf16_to_f32(aw[i] & 0xffffu) * bf16_to_f32(bw[i] & 0xffffu) +
             bf16_to_f32(aw[i] >> 16) * bf16_to_f32(bw[i] >> 16);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 16);
  if (valid && g == 0) {
    const int64_t t = row / H;
    const int h = (int)(row % H);
    delta[(int64_t)h * T + t] = sum;
    pexp[(int64_t)h * T + t] = 8.0f - lse[(int64_t)h * T + t] * kLog2e;
  }
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
  int ntq_max, ntk_max;  // query / key tiles of the longest sequences (dS image grid)
  uint8_t* ds_img;       // [H][nseq][ntq_max][ntk_max] 16 KB dS_q images
  uint8_t* ds_codes;     // [H][nseq][ntq_max][ntk_max] 16 E8M0 codes
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

    // ---- dS_q of this (query tile, KV tile) pair to global memory for the dQ kernel: the 16 KB LDS
    // image as it is (swizzled, key-major) and the 16 block codes; 2 KB per wave, 16 B per lane ----
    {
      const int64_t tile = (((int64_t)h * p.nseq + s) * p.ntq_max + qt) * p.ntk_max + kt;
      uint8_t* img = p.ds_img + tile * (kTile * kD);
      const int o0 = wave_s * 2048 + lane * 16;
      const uint4 w0 = *reinterpret_cast<const uint4*>(lds_ds + o0);
      const uint4 w1 = *reinterpret_cast<const uint4*>(lds_ds + o0 + 1024);
      *reinterpret_cast<uint4*>(img + o0) = w0;
      *reinterpret_cast<uint4*>(img + o0 + 1024) = w1;
      if (wave_s == 0 && lane == 0)
        *reinterpret_cast<uint4*>(p.ds_codes + tile * 16) = *reinterpret_cast<const uint4*>(lds_dscode);
      // Wait for this thread's part of the next query tile (issued at the top of the iteration).
      // Vector memory operations complete in issue order, so leaving the two stores issued since then
      // in flight still covers the tile loads.
      wait_vmcnt<2>();
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

// ---------------------------------------------------------------------------------------------
// dQ = c * sum over KV tiles of dS_q K, reduced in KV-tile order: per tile, the 32 x 32 x 128 partial
// of an MFMA block is added either in FP16 holding sigma dQ (acc = fp16(acc + fp16(sigma partial)),
// the static scale folded into dS_q's E8M0 code) or in FP32 (acc = fl32(acc + partial)); then
// dQ = bf16(c acc / sigma). One workgroup of 8 waves per (sequence, head, 128-query tile); wave w
// owns query block w & 3 and d-blocks 2 (w >> 2), 2 (w >> 2) + 1. The dS_q images and the K tiles
// stream through an LDS ring with direct loads.
// ---------------------------------------------------------------------------------------------
struct DqParams {
  const uint8_t* k;
  const uint8_t* k_scale;
  const int32_t *cu_q, *cu_k;
  int nseq, H, ntq_max, ntk_max;
  int total_items;
  int causal;
  const uint8_t* ds_img;
  const uint8_t* ds_codes;
  int dq_fp16;
  int log2_sigma;  // sigma = 2^log2_sigma (0 in FP32 mode)
  float mult;      // c / sigma
  uint16_t* dq;
};

// LDS ring of (dS image, K tile) stages (a power of two). Two stages keep the LDS at 66 KB so two
// workgroups share a CU, which measured faster than deeper prefetching with one workgroup per CU.
constexpr int kDqStages = 2;

__global__ void __launch_bounds__(512, 1) attn_dq_kernel(DqParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_img[kDqStages][kTile * kD];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_kt[kDqStages][kTile * kD];
  __shared__ __attribute__((aligned(256))) uint32_t lds_codes[kDqStages][64];
  __shared__ __attribute__((aligned(256))) uint32_t lds_ksc[kDqStages][64];
  __shared__ int64_t red[16];

  const int item = xcd_remap((int)blockIdx.x, p.total_items);
  const int qt = item % p.ntq_max;
  const int h = (item / p.ntq_max) % p.H;
  const int s = item / (p.ntq_max * p.H);
  const int64_t q_start = p.cu_q[s], k_start = p.cu_k[s];
  const int Lq = p.cu_q[s + 1] - (int)q_start;
  const int Lk = p.cu_k[s + 1] - (int)k_start;
  const int q0 = qt * kTile;
  if (q0 >= Lq) return;  // uniform over the workgroup
  const SeqOffsets koff = seq_offsets(p.cu_k, s, red);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int qb = wave_s & 3, half = wave_s >> 2;
  const int r = lane & 31, hh = lane >> 5;
  const int C = p.H * kD;
  const int Cs = C >> 5;
  const TileLane tl = tile_lane(wave, lane, C);
  int ntk = (Lk + kTile - 1) / kTile;
  if (p.causal) ntk = min(ntk, qt + 1);  // key tiles past the query tile are fully masked

  const uint8_t* kbase = (const uint8_t*)mx_uniform_ptr((void*)(p.k + k_start * (int64_t)C + h * kD));
  const int64_t tile0 = (((int64_t)h * p.nseq + s) * p.ntq_max + qt) * p.ntk_max;  // image of key tile 0
  const uint8_t* img_base = (const uint8_t*)mx_uniform_ptr((void*)(p.ds_img + tile0 * (kTile * kD)));
  const uint8_t* code_base = p.ds_codes + tile0 * 16;
  const uint8_t* ksc_base = p.k_scale + (koff.padded / 32) * (int64_t)Cs + h * 4;
  auto issue_loads = [&](int kt, uint8_t* img, uint8_t* ktile, uint32_t* codes, uint32_t* kscw) {
    // the dS_q image is copied as it is (2 KB per wave, 16 B per lane)
#pragma unroll
    for (int c = 0; c < kPieces; ++c) {
      const uint32_t off = (uint32_t)((wave_s * kPieces + c) * 1024 + lane * 16);
      mx_lds_dma16((MX_LDS void*)(img + (wave_s * kPieces + c) * 1024), img_base + (int64_t)kt * (kTile * kD), off);
    }
    issue_tile_load(ktile, kbase + (int64_t)kt * kTile * C, Lk - kt * kTile, C, tl, wave_s);
    if (wave_s == 2) mx_lds_dma4_addr((MX_LDS void*)codes, code_base + (int64_t)kt * 16 + 4 * (lane & 3));
    // K's scale words along D of the tile's four key blocks (lanes 0-3; the rest repeat them)
    if (wave_s == 3) mx_lds_dma4_addr((MX_LDS void*)kscw, ksc_base + (int64_t)(4 * kt + (lane & 3)) * Cs);
  };

  // per-lane constants of the transposed LDS reads
  const int grp = lane >> 4, gl = lane & 15;
  const int tb = gl >> 1, ts = gl & 1;
  const int tr_row = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);
  const int tr_col = 16 * (grp & 1) + 8 * ts;
  const int tr_swz = swz(tr_row);

  // accumulators of the wave's two 32 x 32 blocks: FP32 values, or FP16 pairs (rows v, v + 1)
  mx_v16f acc32[2];
  uint32_t acc16[2][8];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    acc32[e] = mx_v16f{};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc16[e][i] = 0u;
  }

  // Each stage's loads are 4 vector memory operations per wave (5 for waves 2 and 3). Waiting for
  // the oldest of the tiles in flight leaves the newer ones' operations outstanding (they complete
  // in issue order). Supports up to three tiles in flight.
  static_assert(kDqStages >= 2 && kDqStages <= 4 && (kDqStages & (kDqStages - 1)) == 0, "ring size");
  const bool extra_op = wave_s == 2 || wave_s == 3;
  auto wait_tile = [&](int newer) {
    if (newer <= 0)
      wait_vmcnt<0>();
    else if (newer == 1) {
      if (extra_op)
        wait_vmcnt<5>();
      else
        wait_vmcnt<4>();
    } else {
      if (extra_op)
        wait_vmcnt<10>();
      else
        wait_vmcnt<8>();
    }
  };
#pragma unroll
  for (int i = 0; i < kDqStages - 1; ++i)
    if (i < ntk) issue_loads(i, lds_img[i], lds_kt[i], lds_codes[i], lds_ksc[i]);
  for (int kt = 0; kt < ntk; ++kt) {
    const int st = kt & (kDqStages - 1);
    wait_tile(min(kDqStages - 2, ntk - 1 - kt));
    __syncthreads();  // tile kt has landed for every wave; all reads of the stage refilled below are done
    if (kt + kDqStages - 1 < ntk) {
      const int ns = (kt + kDqStages - 1) & (kDqStages - 1);
      issue_loads(kt + kDqStages - 1, lds_img[ns], lds_kt[ns], lds_codes[ns], lds_ksc[ns]);
    }
    const uint8_t* img = lds_img[st];
    const uint8_t* ktile = lds_kt[st];
    const uint32_t* codes = lds_codes[st];
    // K's scales along D for this tile (B operand: key block 2 ks + hh, d-block db)
    uint32_t kq_sc[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) kq_sc[ks] = lds_ksc[st][2 * ks + hh];
    // dS_q scale of (key block 2 ks + hh, query block qb), sigma folded in for the FP16 reduction
    uint32_t a_sc[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = (int)((codes[2 * ks + hh] >> (8 * qb)) & 0xffu);
      a_sc[ks] = c == 255 ? 255u : (uint32_t)min(max(c + p.log2_sigma, 0), 254);
    }
    mx_v8i dsa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) dsa[ks] = lds_tr_operand(img, ks, 32 * qb, tr_row, tr_col, tr_swz);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int db = 2 * half + e;
      mx_v16f part = mx_v16f{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        mx_v8i kbt = lds_tr_operand(ktile, ks, 32 * db, tr_row, tr_col, tr_swz);
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(dsa[ks], kbt, part, 0, 0, 0, (int)a_sc[ks], 0,
                                                               (int)(kq_sc[ks] >> (8 * db)));
      }
      if (p.dq_fp16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // fp16(acc + fp16(partial)): round the partial to FP16, then one FP16 addition
          const uint32_t ph = (uint32_t)__builtin_bit_cast(uint32_t, __floats2half2_rn(part[2 * i], part[2 * i + 1]));
          const __half2 sum = __hadd2(__builtin_bit_cast(__half2, acc16[e][i]), __builtin_bit_cast(__half2, ph));
          acc16[e][i] = __builtin_bit_cast(uint32_t, sum);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc32[e][v] += part[v];
      }
    }
  }

  // ---- epilogue: dQ = bf16(c acc / sigma); block rows 8 (v/4) + 4 hh + v%4, column 32 db + r ----
  uint16_t* dqb = p.dq + (q_start + q0 + 32 * qb) * (int64_t)C + h * kD;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int db = 2 * half + e;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float x;
      if (p.dq_fp16) {
        const float2 f = __half22float2(__builtin_bit_cast(__half2, acc16[e][v >> 1]));
        x = (v & 1) ? f.y : f.x;
      } else {
        x = acc32[e][v];
      }
      const int qr = 8 * (v >> 2) + 4 * hh + (v & 3);
      if (q0 + 32 * qb + qr < Lq) dqb[(uint32_t)(qr * C + 32 * db + r)] = (uint16_t)f32_to_bf16(x * p.mult);
    }
  }
}

}  // namespace

namespace mxfa {

// Workspace: the dS_q images [H][nseq][ntq_max][ntk_max] (16 KB each), their block codes (16 B
// each), then Delta [H][Tq] and the exponent offsets [H][Tq] (fp32), each region 256-byte aligned.
struct BwdWorkspace {
  size_t img, codes, delta, pexp, total;
};
static BwdWorkspace bwd_workspace_layout(int64_t Tq, int H, int nseq, int max_q, int max_k) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t tiles = (size_t)H * nseq * ((max_q + kTile - 1) / kTile) * ((max_k + kTile - 1) / kTile);
  BwdWorkspace w;
  w.img = 0;
  w.codes = al(tiles * kTile * kD);
  w.delta = w.codes + al(tiles * 16);
  w.pexp = w.delta + al((size_t)Tq * H * 4);
  w.total = w.pexp + al((size_t)Tq * H * 4);
  return w;
}

size_t bwd_workspace_bytes(int64_t Tq, int H, int nseq, int max_q, int max_k) {
  return bwd_workspace_layout(Tq, H, nseq, max_q, max_k).total;
}

hipError_t launch_attn_bwd(const AttnProblem& a, const MxOperand& v_d, const MxOperand& dout, const uint16_t* o,
                           const uint16_t* dout_bf16, const float* lse, int dq_fp16, float sigma, void* workspace,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, hipStream_t stream) {
  const int64_t Tq = a.total_q;
  const int C = a.H * kD;
  const BwdWorkspace w = bwd_workspace_layout(Tq, a.H, a.nseq, a.max_seqlen_q, a.max_seqlen_k);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  float* delta = reinterpret_cast<float*>(ws + w.delta);
  float* pexp = reinterpret_cast<float*>(ws + w.pexp);
  const int ntq_max = (a.max_seqlen_q + kTile - 1) / kTile;
  const int ntk_max = (a.max_seqlen_k + kTile - 1) / kTile;
  if (Tq > 0) {
    const int64_t rows = Tq * a.H;  // 16 lanes per row
    const int64_t blocks = (rows + 15) / 16;
    hipLaunchKernelGGL(bwd_preprocess_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o, dout_bf16, lse, Tq,
                       a.H, delta, pexp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdParams p;
  p.q = a.q.data; p.k = a.k.data; p.v = v_d.data; p.dO = dout.data;
  p.q_scale = a.q.scale; p.k_scale = a.k.scale; p.v_scale = v_d.scale; p.dO_scale = dout.scale;
  p.v_row_shift = v_d.mode == 0 ? 0 : 5;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.nseq = a.nseq; p.H = a.H;
  p.n_ktiles = ntk_max;
  p.total_items = p.n_ktiles * a.H * a.nseq;  // < 2^31, checked by the caller
  p.c2 = a.softmax_scale * kLog2e;
  p.causal = a.causal;
  p.pexp = pexp; p.delta = delta; p.Tq = Tq;
  p.ntq_max = ntq_max; p.ntk_max = ntk_max;
  p.ds_img = ws + w.img;
  p.ds_codes = ws + w.codes;
  p.c = a.softmax_scale;
  p.dk = dk; p.dv = dv;
  if (p.total_items > 0) {
    hipLaunchKernelGGL(attn_bwd_kernel, dim3((unsigned)p.total_items), dim3(64 * kWaves), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  DqParams d;
  d.k = a.k.data; d.k_scale = a.k.scale;
  d.cu_q = a.cu_q; d.cu_k = a.cu_k;
  d.nseq = a.nseq; d.H = a.H; d.ntq_max = ntq_max; d.ntk_max = ntk_max;
  d.total_items = ntq_max * a.H * a.nseq;
  d.causal = a.causal;
  d.ds_img = ws + w.img;
  d.ds_codes = ws + w.codes;
  d.dq_fp16 = dq_fp16;
  {
    int e = 0;
    std::frexp(dq_fp16 ? sigma : 1.0f, &e);  // sigma = 0.5 * 2^e exactly (a power of two, checked by the caller)
    d.log2_sigma = e - 1;
  }
  d.mult = a.softmax_scale / (dq_fp16 ? sigma : 1.0f);
  d.dq = dq;
  if (d.total_items > 0) {
    hipLaunchKernelGGL(attn_dq_kernel, dim3((unsigned)d.total_items), dim3(64 * kWaves), 0, stream, d);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mxfa

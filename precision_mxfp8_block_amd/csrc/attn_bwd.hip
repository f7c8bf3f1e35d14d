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
//  * Workgroup = 8 waves = one 128-row KV tile; waves w and w + 4 share a SIMD (measured) and own
//    the same 32 keys (32 (w & 3) .. +31), with different roles. Producer waves (0-3) run G1 and G2
//    (their K and V rows, the B operands, stay in registers for the whole loop, so S and dP come out
//    with one key per lane and 16 queries per lane per 32-query block) and the elementwise part, and
//    write P_q and dS_q to LDS. Consumer waves (4-7) hold dV and dK (32 x 128 FP32 each) and run G3
//    and G4 one query tile behind, plus all global -> LDS copies and the dS_q image stores. The
//    SIMD's one VALU-heavy wave and one MFMA-heavy wave overlap, and both stay within 256 VGPRs, so
//    every MFMA keeps its accumulator in VGPRs.
//  * The S and dP accumulator layout (one key per lane, contraction over queries) is exactly the A
//    operand of dV = P^T dO and dK = dS^T Q: P_q and dS_q bytes are handed over in that order;
//    dO^T and Q^T are read from LDS with ds_read_b64_tr_b8 in the same order.
//  * The producer software-pipelines its four 32-query blocks: block j + 1's scaled MFMAs are in
//    flight while block j's first elementwise half (exp2, dS, P_q, wave-wide maximum) runs beside
//    block j - 1's second half (dS_q and the LDS writes); the last block's second half runs in the
//    next period beside that tile's first loads and MFMAs.
//  * dP - Delta comes out of the MFMA: the dP accumulator starts at -Delta (the preprocess stores
//    the negated row sums).
//  * dQ is not reduced with atomics: device-scope atomics on gfx950 are executed beyond the XCD's
//    L2 and sustain about 1.3 TB/s of payload (measured), so 32 KV tiles x 67 MB of FP16 partials
//    bound the backward at ~1.6 ms at 4 x 16 x 4096. Instead each (Q tile, KV tile) pair writes its
//    16 KB dS_q tile (FP8, half the bytes of an FP16 partial, plain streaming stores) and the dQ
//    kernel reads them back per Q tile and reduces dS_q K over the KV tiles in order, in FP16 with
//    the static scale or in FP32, with no atomics and a deterministic result.
//  * Q and dO tiles (and the tile's LSE and Delta) pass through three LDS stages (the producers read
//    tile k, the consumers tile k - 1, tile k + 1 lands) with direct global -> LDS loads; all LDS
//    tiles use the forward's XOR swizzle.
//  * P is produced as 256 P straight from exp2 (the static scale folded into the exponent); dS is
//    carried as 256 dS, which shifts its E8M0 code by exactly 8 (power-of-two scaling is exact), and
//    converted with the scaled FP8 conversion after clamping to +-448 times the block scale.
#include <cmath>
#include <type_traits>

#include "mx_device.h"
#include "mxfa_internal.h"

namespace {

constexpr int kTile = 128;
constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row) { return lds_swz(row); }

// Waits on the vector memory counter, written as asm: the direct LDS loads are asm too, so the
// compiler does not see them and would drop a builtin wait it believes to be redundant.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_vm() { wait_vmcnt<0>(); }

constexpr int kBwdWaves = 8;  // main kernel: two waves per SIMD (a producer and a consumer)
constexpr int kDqWaves = 8;   // dQ kernel: two waves per SIMD

// Per-lane constants for filling a 128 x 128-byte swizzled LDS tile with direct global -> LDS loads
// by W waves: lane piece c of wave w covers tile row trow[c], logical chunk byte offset tcol[c].
template <int W>
struct TileLane {
  static constexpr int kPieces = kTile * kD / 1024 / W;  // 1 KB pieces (64 lanes x 16 B) per wave
  int trow[kPieces], tcol[kPieces];
  uint32_t toff[kPieces];  // trow * C + tcol (full tiles)
};

template <int W>
__device__ __forceinline__ TileLane<W> tile_lane(int wave, int lane, int C) {
  TileLane<W> t;
#pragma unroll
  for (int c = 0; c < TileLane<W>::kPieces; ++c) {
    const int p = (wave * TileLane<W>::kPieces + c) * 64 + lane;
    t.trow[c] = p >> 3;
    t.tcol[c] = 16 * ((p & 7) ^ swz(p >> 3));
    t.toff[c] = (uint32_t)(t.trow[c] * C + t.tcol[c]);
  }
  return t;
}

// Asynchronous copy of a tile whose first row is at `base` (this head's columns). Rows at or past
// `valid` re-fetch the last valid row (finite data; their contributions are masked to zero).
template <int W>
__device__ __forceinline__ void issue_tile_load(uint8_t* lds_tile, const uint8_t* base, int valid, int C,
                                                const TileLane<W>& t, int wave_s) {
  constexpr int P = TileLane<W>::kPieces;
#pragma unroll
  for (int c = 0; c < P; ++c) {
    const uint32_t off = valid >= kTile ? t.toff[c] : (uint32_t)(min(t.trow[c], valid - 1) * C + t.tcol[c]);
    mx_lds_dma16((MX_LDS void*)(lds_tile + (wave_s * P + c) * 1024), base, off);
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

// Maximum over the 64 lanes of a wave: DPP within rows of 16, then permlane16 and permlane32 swaps
// across rows (no LDS traffic).
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false));  // row_mirror
  auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows 0 <-> 1, 2 <-> 3
  v = max((uint32_t)s16[0], (uint32_t)s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // halves
  return max((uint32_t)s32[0], (uint32_t)s32[1]);
}

// SQ32 quantization (the MX scale rule of the operand quantizer) of one 32 x 32 gradient block that
// a wave holds in the MFMA accumulator layout: lane (r, hh) holds column r and rows
// 8 (v / 4) + 4 hh + v % 4, v = 0..15. Rows at or past `valid` lie outside the sequence: they are
// left out of the block maximum and not stored. The payload goes through the wave's 1 KB of LDS
// (`stage`, [32 rows][32 bytes]) so that it leaves as 16-byte row pieces (lane l: row l / 2, bytes
// 16 (l % 2) ..), to dst + row * C (dst at the block's row 0, column 0); the E8M0 code to *code_dst
// and, when set, *code_t_dst (lane 0). Every lane of the wave must take part; LDS operations of one
// wave execute in order, so the reads see the wave's own writes.
__device__ __forceinline__ void store_grad_sq32(const float (&x)[16], int valid, uint8_t* dst, int C,
                                                uint8_t* code_dst, uint8_t* code_t_dst, uint8_t* stage, int lane,
                                                int hh) {
  uint32_t am = 0;  // largest sign-cleared bit pattern: orders NaN > Inf > finite magnitudes
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if (8 * (v >> 2) + 4 * hh + (v & 3) < valid) am = max(am, __float_as_uint(x[v]) & 0x7fffffffu);
  am = wave_max_dpp(am);
  const uint32_t code = mx_code_from_amax_bits(am);
  const float inv = mx_inv_scale(code == 255u ? 127u : code);
  const int r = lane & 31;
#pragma unroll
  for (int v = 0; v < 16; v += 2) {
    const uint32_t w = code == 255u ? 0x7f7fu : mx_pack2_lo(x[v] * inv, x[v + 1] * inv, 0u);
    const int r0 = 8 * (v >> 2) + 4 * hh + (v & 3);
    stage[r0 * 32 + r] = (uint8_t)w;
    stage[(r0 + 1) * 32 + r] = (uint8_t)(w >> 8);
  }
  const int row = lane >> 1;
  const uint4 piece = *reinterpret_cast<const uint4*>(stage + row * 32 + 16 * (lane & 1));
  if (row < valid) *reinterpret_cast<uint4*>(dst + (int64_t)row * C + 16 * (lane & 1)) = piece;
  if (lane == 0) {
    *code_dst = (uint8_t)code;
    if (code_t_dst) *code_t_dst = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------------------------
// Preprocess: the negated row sums -Delta[h][t] = -sum_d dO[t, h, d] * O[t, h, d] (fp32, the
// initial value of the dP accumulator) and the exponent offset of 256 P, b[h][t] = 8 - LSE[h][t]
// log2(e) (so 256 P = exp2(c log2(e) S + b)).
// A workgroup covers 64 consecutive tokens of one head: four lanes per (token, head) row of 128,
// lane g reading 16-byte pieces g, g + 4, g + 8, g + 12 of O and of dO (every load instruction
// covers whole 64-byte row segments), so each wave writes 16 consecutive outputs per array.
// Grid: x = tokens / 64 (rounded up), y = head.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_preprocess_kernel(const uint16_t* __restrict__ o,
                                                             const uint16_t* __restrict__ dout,
                                                             const float* __restrict__ lse, int64_t T, int H,
                                                             float* __restrict__ ndelta, float* __restrict__ pexp) {
  const int h = blockIdx.y;
  const int g = threadIdx.x & 3;
  const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const bool valid = t < T;
  const int64_t row = (valid ? t : T - 1) * H + h;  // rows past the end re-read the last one
  uint4 a[4], b[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    a[c] = *reinterpret_cast<const uint4*>(o + row * kD + 8 * (g + 4 * c));
    b[c] = *reinterpret_cast<const uint4*>(dout + row * kD + 8 * (g + 4 * c));
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t aw[4] = {a[c].x, a[c].y, a[c].z, a[c].w}, bw[4] = {b[c].x, b[c].y, b[c].z, b[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sum += bf16_to_f32(aw[i] & 0xffffu) * bf16_to_f32(bw[i] & 0xffffu) +
             bf16_to_f32(aw[i] >> 16) * bf16_to_f32(bw[i] >> 16);
  }
  sum += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(sum), 0xB1, 0xF, 0xF, false));  // lane bit 0
  sum += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(sum), 0x4E, 0xF, 0xF, false));  // lane bit 1
  if (valid && g == 0) {
    ndelta[(int64_t)h * T + t] = -sum;
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
  int contiguous;  // item order (mx_item)
  float c2;  // c * log2(e)
  int causal;
  const float* pexp;    // [H][Tq]: 8 - LSE log2(e)
  const float* ndelta;  // [H][Tq]: -Delta
  int64_t Tq;
  int ntq_max, ntk_max;  // query / key tiles of the longest sequences (dS image grid)
  uint8_t* ds_img;       // [H][nseq][ntq_max][ntk_max] 16 KB dS_q images
  uint8_t* ds_codes;     // [H][nseq][ntq_max][ntk_max] 16 E8M0 codes
  float c;
  uint16_t *dk, *dv;                  // bf16 gradients, or null
  uint8_t *dk_mx, *dk_mx_scale;       // E4M3 SQ32 gradients (compact codes [blocks][C/32]), or null
  uint8_t *dk_mx_scale_t, *dv_mx_scale_t;  // the codes transposed [C/32][blocks], each nullable
  uint8_t *dv_mx, *dv_mx_scale;
};

__global__ void __launch_bounds__(64 * kBwdWaves, 1) attn_bwd_kernel(BwdParams p) {
  // [stage][Q, dO] tiles, three stages: the producers read tile k while the consumers read tile k - 1
  // and tile k + 1 lands. The prologue parks the K and V tiles in stage 2.
  __shared__ __attribute__((aligned(1024))) uint8_t lds_qd[3][2][kTile * kD];
  __shared__ __attribute__((aligned(1024))) uint4 lds_pq[4][4][64];  // P_q, lane order [key block][q block][lane]
  __shared__ __attribute__((aligned(1024))) uint4 lds_sq[4][4][64];  // dS_q, lane order
  __shared__ __attribute__((aligned(1024))) uint8_t lds_ds[kTile * kD];  // dS_q image, key-major [kv][q], swizzled
  __shared__ __attribute__((aligned(512))) float lds_ld[3][2][kTile];   // [stage][8 - LSE log2e, -Delta]
  __shared__ __attribute__((aligned(256))) uint32_t lds_sc[3][64];      // [stage][Q, dO scale words]
  __shared__ uint32_t lds_dscode[4];                                     // dS codes [key block] (byte: q block)

  const int item = mx_item(p.contiguous, (int)blockIdx.x, p.total_items, p.n_ktiles, p.nseq * p.H);
  if (item < 0) return;
  const int kt = item % p.n_ktiles;
  const int h = (item / p.n_ktiles) % p.H;
  const int s = item / (p.n_ktiles * p.H);
  const int64_t q_start = p.cu_q[s], k_start = p.cu_k[s];
  const int Lq = p.cu_q[s + 1] - (int)q_start;
  const int Lk = p.cu_k[s + 1] - (int)k_start;
  if (kt * kTile >= Lk) return;

  const SeqOffsets qoff = seq_offsets(p.cu_q, s);
  const SeqOffsets koff = seq_offsets(p.cu_k, s);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave_s & 3;              // key block of this wave
  const bool producer = wave_s < 4;      // waves 0-3: G1/G2 and the elementwise part; 4-7: G3/G4, loads
  const int r = lane & 31, hh = lane >> 5;
  const int C = p.H * kD;
  const int Cs = C >> 5;
  const int kv0 = kt * kTile;
  const int kvrow = kv0 + 32 * kw + r;  // this lane's key row
  const TileLane<4> tl = tile_lane<4>(kw, lane, C);

  const int n_qtiles = (Lq + kTile - 1) / kTile;
  const int qt_begin = p.causal ? kt : 0;

  // wave-uniform base pointers, kept in scalar registers
  const uint8_t* qbase = (const uint8_t*)mx_uniform_ptr((void*)(p.q + q_start * (int64_t)C + h * kD));
  const uint8_t* dobase = (const uint8_t*)mx_uniform_ptr((void*)(p.dO + q_start * (int64_t)C + h * kD));
  const float* lse_base = (const float*)mx_uniform_ptr((void*)(p.pexp + (int64_t)h * p.Tq + q_start));
  const float* del_base = (const float*)mx_uniform_ptr((void*)(p.ndelta + (int64_t)h * p.Tq + q_start));
  const uint8_t* qs_base = p.q_scale + (qoff.padded >> 5) * (int64_t)Cs + h * 4;
  const uint8_t* ds_base = p.dO_scale + (qoff.padded >> 5) * (int64_t)Cs + h * 4;

  // All global -> LDS copies are issued by the consumer waves: a query tile's Q and dO (four 1 KB
  // pieces per wave each), its exponent offsets and -Delta (consumer waves 0 and 1, one 128-float
  // vector each), its Q and dO scale words (consumer wave 2; lanes 0-3: Q blocks, 4-7: dO blocks).
  auto issue_qtile = [&](int st, int qt) {
    const int64_t q0 = (int64_t)qt * kTile;
    issue_tile_load(lds_qd[st][0], (const uint8_t*)mx_uniform_ptr((void*)(qbase + q0 * C)), Lq - (int)q0, C, tl, kw);
    issue_tile_load(lds_qd[st][1], (const uint8_t*)mx_uniform_ptr((void*)(dobase + q0 * C)), Lq - (int)q0, C, tl, kw);
    if (kw < 2) {
      const float* src = kw == 0 ? lse_base : del_base;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = min((int)q0 + c * 64 + lane, Lq - 1);
        mx_lds_dma4((MX_LDS void*)(&lds_ld[st][kw][c * 64]), src, (uint32_t)row * 4u);
      }
    } else if (kw == 2) {
      const int i = lane < 8 ? lane : 0;
      const uint8_t* src = (i < 4 ? qs_base : ds_base) + (int64_t)((qt * 4 + (i & 3)) * Cs);
      mx_lds_dma4_addr((MX_LDS void*)&lds_sc[st][0], src);
    }
  };

  // prologue: K and V tiles into stage 2, the first query tile into stage 0
  if (!producer) {
    issue_tile_load(lds_qd[2][0], p.k + (k_start + kv0) * (int64_t)C + h * kD, Lk - kv0, C, tl, kw);
    issue_tile_load(lds_qd[2][1], p.v + (k_start + kv0) * (int64_t)C + h * kD, Lk - kv0, C, tl, kw);
    if (qt_begin < n_qtiles) issue_qtile(0, qt_begin);
  }

  // K (SQ32) and V (ROW32/SQ32) scales along D of this lane's key row: byte 0 = d-block hh, byte 2 =
  // d-block 2 + hh
  const uint32_t ksc_b =
      *reinterpret_cast<const uint32_t*>(p.k_scale + ((koff.padded + kvrow) >> 5) * (int64_t)Cs + h * 4) >> (8 * hh);
  const uint32_t vsc_b =
      *reinterpret_cast<const uint32_t*>(p.v_scale + ((koff.padded + kvrow) >> p.v_row_shift) * (int64_t)Cs + h * 4) >>
      (8 * hh);

  // per-lane constants of the transposed LDS reads
  const int grp = lane >> 4, gl = lane & 15;
  const int tb = gl >> 1, ts = gl & 1;
  const int tr_row = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);
  const int tr_col = 16 * (grp & 1) + 8 * ts;
  const int tr_swz = swz(tr_row);

  wait_vm();
  __syncthreads();

  // Period k: the producers turn query tile k into P_q and dS_q, the consumers run G3 and G4 of tile
  // k - 1 and fetch tile k + 1. Two workgroup barriers per period: B1 at the top (tile k has landed,
  // everything of period k - 1 is done) and B2 once the consumers hold tile k - 1's P_q, dS_q and
  // codes in registers (the producers may overwrite them). The two roles run separate loops with the
  // same periods, so neither keeps the other's registers alive.
  const int k_end = qt_begin < n_qtiles ? n_qtiles : qt_begin - 1;  // last period (none without tiles)
  if (producer) {
    // this wave's K and V rows, the B operands of S = Q K^T and dP = dO V^T, for the whole loop
    const int krow = 32 * kw + r;
    const mx_v8i kb0 = lds_row_operand(lds_qd[2][0], krow, 0, hh), kb1 = lds_row_operand(lds_qd[2][0], krow, 1, hh);
    const mx_v8i vb0 = lds_row_operand(lds_qd[2][1], krow, 0, hh), vb1 = lds_row_operand(lds_qd[2][1], krow, 1, hh);
    // The E8M0 code of a dS block from the exponent field of its |256 dS| maximum (wave-uniform, in
    // scalar registers): code of 256 dS = efield - 8 (0 below, 255 for NaN/Inf), code of dS = that - 8;
    // dS_q is E4M3 of 256 dS at scale 2^(cs - 127), cs = clamp(efield - 8, 8, 246) (the clamp only
    // keeps the unused NaN-block values finite).
    auto block_code = [](uint32_t efield, uint32_t& code, uint32_t& cs) {
      asm("s_sub_u32 %1, %2, 8\n\t"      // cs = efield - 8 (wraps below 8)
          "s_sub_u32 %0, %2, 16\n\t"     // code = efield - 16 ...
          "s_cmp_lt_u32 %2, 16\n\t"
          "s_cselect_b32 %0, 0, %0\n\t"  // ... 0 below 16
          "s_cmp_ge_u32 %2, 255\n\t"
          "s_cselect_b32 %0, 255, %0\n\t"  // NaN/Inf block
          "s_max_u32 %1, %1, 8\n\t"
          "s_cmp_lt_u32 %2, 8\n\t"
          "s_cselect_b32 %1, 8, %1\n\t"
          "s_min_u32 %1, %1, 246"
          : "=&s"(code), "=&s"(cs)
          : "s"(efield)
          : "scc");
    };
    // Second half of block j's elementwise part: dS_q from 256 dS at the block's scale, and the LDS
    // writes of P_q, dS_q (operand order) and of the dS_q image for the dQ kernel.
    auto ew_b = [&](int j, const mx_v16f& dpacc, uint32_t code, uint32_t cs, const uint32_t (&pk)[4]) {
      const float sc = __uint_as_float(cs << 23);
      const float lim = __uint_as_float(((cs + 8u) << 23) | 0x600000u);  // 448 sc
      uint32_t dsk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = mx_pack4_scaled(dpacc[4 * i], dpacc[4 * i + 1], dpacc[4 * i + 2], dpacc[4 * i + 3], sc, lim);
        dsk[i] = code == 255u ? 0x7f7f7f7fu : w;
      }
      if (j == 0) __syncthreads();  // B2: the consumers hold their operands of tile k - 1 but block 3's
      lds_pq[kw][j][lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      lds_sq[kw][j][lane] = make_uint4(dsk[0], dsk[1], dsk[2], dsk[3]);
      // the image: key row 32 kw + r. Lane (r, hh) holds the 4-query groups 32 j + 8 i + 4 hh; two
      // half-wave swaps give lane (r, 0) queries 32 j + 0..15 and lane (r, 1) queries 32 j + 16..31
      // (words: hh = 0 group i, hh = 1 group i, hh = 0 group i + 1, hh = 1 group i + 1), which it
      // writes as one 16-byte chunk
      const int kvl = 32 * kw + r;
      const auto x02 = __builtin_amdgcn_permlane32_swap(dsk[0], dsk[2], false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(dsk[1], dsk[3], false, false);
      const uint4 chunk = make_uint4(x02[0], x02[1], x13[0], x13[1]);
      *reinterpret_cast<uint4*>(lds_ds + kvl * kD + 16 * ((2 * j + hh) ^ swz(kvl))) = chunk;
    };
    // Block 3's second half is deferred into the next period, where it runs beside that tile's first
    // loads and MFMAs (the consumers read block 3's operands and image chunks after B2).
    mx_v16f ds3{};
    uint32_t pk3[4] = {0u, 0u, 0u, 0u}, code3 = 0u, cs3 = 8u;
    int st = 0;  // stage of tile k
    for (int k = qt_begin; k <= k_end; ++k) {
      __syncthreads();  // B1
      if (k < n_qtiles) {
        const int q0 = k * kTile;
        const uint8_t* lds_q = lds_qd[st][0];
        const uint8_t* lds_do = lds_qd[st][1];
        const float* pexp = lds_ld[st][0];
        const float* ndl = lds_ld[st][1];
        uint32_t qsc[4], dosc[4];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          qsc[qb] = lds_sc[st][qb];
          dosc[qb] = lds_sc[st][4 + qb];
        }
        const bool need_mask = (q0 + kTile > Lq) || (kv0 + kTile > Lk) || (p.causal && kv0 + kTile - 1 > q0);

        // Per query block j (lane: key kvrow; queries 32 j + 8 i + 4 hh + t): G1 and G2 (S and
        // dP - Delta, the dP accumulator starting at -Delta), then 256 P and 256 dS with their E4M3
        // codes. G1/G2 of block j + 1 are issued before block j's elementwise part. Two
        // instantiations behind one wave-uniform branch: interior tiles carry no mask code.
        auto tile_body = [&](auto masked) {
          constexpr bool MASK = decltype(masked)::value;
          // distinct first instructions keep the compiler from hoisting the two instantiations' common
          // prologue above the branch (where it would hold registers across both)
          if (MASK)
            asm volatile("; masked tile" ::: "memory");
          else
            asm volatile("; interior tile" ::: "memory");
          // Q and dO rows of block j (A operands of G1 and G2)
          auto load_rows = [&](int j, mx_v8i (&a)[4]) {
            const int row = 32 * j + r;
            a[0] = lds_row_operand(lds_q, row, 0, hh);
            a[1] = lds_row_operand(lds_q, row, 1, hh);
            a[2] = lds_row_operand(lds_do, row, 0, hh);
            a[3] = lds_row_operand(lds_do, row, 1, hh);
          };
          // exponent offsets of block j's 16 query rows, and -Delta as the dP accumulator's start
          auto load_pe = [&](int j, float4 (&pe)[4]) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pe[i] = *reinterpret_cast<const float4*>(pexp + 32 * j + 8 * i + 4 * hh);
          };
          auto load_nd = [&](int j, mx_v16f& dpacc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 nd4 = *reinterpret_cast<const float4*>(ndl + 32 * j + 8 * i + 4 * hh);
              dpacc[4 * i] = nd4.x;
              dpacc[4 * i + 1] = nd4.y;
              dpacc[4 * i + 2] = nd4.z;
              dpacc[4 * i + 3] = nd4.w;
            }
          };
          auto g1 = [&](int j, const mx_v8i (&a)[4], mx_v16f& sacc) {
            const uint32_t qs = qsc[j] >> (8 * hh);
            sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0], kb0, mx_v16f{}, 0, 0, 0, (int)qs, 0,
                                                                   (int)ksc_b);
            sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1], kb1, sacc, 0, 0, 2, (int)qs, 2, (int)ksc_b);
          };
          auto g2 = [&](int j, const mx_v8i (&a)[4], mx_v16f& dpacc) {
            const uint32_t dos = dosc[j] >> (8 * hh);
            dpacc =
                __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[2], vb0, dpacc, 0, 0, 0, (int)dos, 0, (int)vsc_b);
            dpacc =
                __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[3], vb1, dpacc, 0, 0, 2, (int)dos, 2, (int)vsc_b);
          };
          // first half of block j's elementwise part: 256 P (packed to pk), 256 dS (left in dpacc) and
          // the block's code and scale exponent (wave-uniform)
          uint32_t codes = 0;
          auto ew_a = [&](int j, mx_v16f& sacc, mx_v16f& dpacc, const float4 (&pe)[4], uint32_t (&pk)[4]) {
            const int ql0 = 32 * j;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int v = 4 * i + t;
                float e = __builtin_amdgcn_exp2f(fmaf(sacc[v], p.c2, (&pe[i].x)[t]));  // 256 P
                if (MASK) {
                  const int qpos = q0 + ql0 + 8 * i + 4 * hh + t;
                  const bool ok = (kvrow < Lk) & (qpos < Lq) & ((p.causal == 0) | (kvrow <= qpos));
                  e = ok ? e : 0.0f;
                }
                sacc[v] = e;
                dpacc[v] = e * dpacc[v];  // 256 dS
              }
            // |256 dS| maximum of the lane as a tree of max3, then over the wave
            float m[5];
#pragma unroll
            for (int g = 0; g < 5; ++g) m[g] = max3_abs3(dpacc[3 * g], dpacc[3 * g + 1], dpacc[3 * g + 2]);
            const float am = max3_abs(max3_abs(m[0], m[1], m[2]), m[3], m[4]);
            const float am2 = max3_abs(am, dpacc[15], dpacc[15]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pk[i] = mx_pack4_inrange(sacc[4 * i], sacc[4 * i + 1], sacc[4 * i + 2], sacc[4 * i + 3]);
            const uint32_t efield =
                (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_max_dpp(__float_as_uint(am2))) >> 23;
            uint32_t code, cs;
            block_code(efield, code, cs);
            codes |= code << (8 * j);
            return make_uint2(code, cs);
          };
          // Software pipeline over the four blocks. Stage j issues block j + 1's G1/G2 and runs block
          // j's first elementwise half beside block j - 1's second half (block 3's of the previous tile
          // in stage 0), so one block's wave-wide maximum overlaps the other's arithmetic. dP's
          // accumulator of block j + 1 (which starts at -Delta) reuses block j - 1's registers once
          // its dS values are packed.
          mx_v8i rows[4];
          mx_v16f sacc[2], dpacc[2];
          float4 pe[2][4];
          uint32_t pk[2][4];
          uint2 cc[2];
          load_rows(0, rows);
          load_pe(0, pe[0]);
          load_nd(0, dpacc[0]);
          g1(0, rows, sacc[0]);
          g2(0, rows, dpacc[0]);
          load_rows(1, rows);
          load_pe(1, pe[1]);
          load_nd(1, dpacc[1]);
          __builtin_amdgcn_sched_barrier(0);
          ew_b(3, ds3, code3, cs3, pk3);
          g1(1, rows, sacc[1]);
          g2(1, rows, dpacc[1]);
          cc[0] = ew_a(0, sacc[0], dpacc[0], pe[0], pk[0]);
          load_rows(2, rows);
          __builtin_amdgcn_sched_barrier(0);
          ew_b(0, dpacc[0], cc[0].x, cc[0].y, pk[0]);
          load_pe(2, pe[0]);
          load_nd(2, dpacc[0]);
          g1(2, rows, sacc[0]);
          g2(2, rows, dpacc[0]);
          cc[1] = ew_a(1, sacc[1], dpacc[1], pe[1], pk[1]);
          load_rows(3, rows);
          __builtin_amdgcn_sched_barrier(0);
          ew_b(1, dpacc[1], cc[1].x, cc[1].y, pk[1]);
          load_pe(3, pe[1]);
          load_nd(3, dpacc[1]);
          g1(3, rows, sacc[1]);
          g2(3, rows, dpacc[1]);
          cc[0] = ew_a(2, sacc[0], dpacc[0], pe[0], pk[0]);
          __builtin_amdgcn_sched_barrier(0);
          ew_b(2, dpacc[0], cc[0].x, cc[0].y, pk[0]);
          cc[1] = ew_a(3, sacc[1], dpacc[1], pe[1], pk[1]);
          if (lane == 0) lds_dscode[kw] = codes;
          ds3 = dpacc[1];
#pragma unroll
          for (int i = 0; i < 4; ++i) pk3[i] = pk[1][i];
          code3 = cc[1].x;
          cs3 = cc[1].y;
        };
        if (need_mask)
          tile_body(std::true_type{});
        else
          tile_body(std::false_type{});
      } else {
        ew_b(3, ds3, code3, cs3, pk3);  // the last tile's block 3
        __syncthreads();                // B2 (no tile left to produce)
      }
      st = st == 2 ? 0 : st + 1;
    }
  } else {
    // dV and dK of the wave's 32 keys
    mx_v16f dv_acc[4], dk_acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dv_acc[i] = mx_v16f{};
      dk_acc[i] = mx_v16f{};
    }
    // which of the lane's four 16-byte image chunks (rows 32 kw + 8 c + lane / 8, stored chunk lane % 8)
    // hold block 3's queries (logical chunks 6 and 7)
    bool img_blk3[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) img_blk3[c] = (((lane & 7) ^ swz(32 * kw + 8 * c + (lane >> 3))) >> 1) == 3;
    int st = 0;  // stage of tile k
    for (int k = qt_begin; k <= k_end; ++k) {
      const int st_prev = st == 0 ? 2 : st - 1, st_next = st == 2 ? 0 : st + 1;
      __syncthreads();  // B1
      // take tile k - 1's P_q, dS_q (blocks 0-2), codes and image chunks (but block 3's) to registers and
      // global memory, fetch tile k + 1; after B2: block 3's operands and image chunks
      mx_v8i pa[2], sa[2];
      uint32_t codes = 0;
      const int64_t tile = (((int64_t)h * p.nseq + s) * p.ntq_max + (k - 1)) * p.ntk_max + kt;
      uint8_t* img = p.ds_img + tile * (kTile * kD) + kw * 4096;
      // the wave's four 16-byte chunks of tile k - 1's dS_q image: taken from LDS now (blocks 0-2) and
      // after B2 (block 3), stored to global memory after this period's load wait (see below)
      uint4 imgv[4];
      if (k > qt_begin) {
        const uint4 p0 = lds_pq[kw][0][lane], p1 = lds_pq[kw][1][lane], p2 = lds_pq[kw][2][lane];
        const uint4 s0 = lds_sq[kw][0][lane], s1 = lds_sq[kw][1][lane], s2 = lds_sq[kw][2][lane];
        pa[0] = mx_v8i{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
        sa[0] = mx_v8i{(int)s0.x, (int)s0.y, (int)s0.z, (int)s0.w, (int)s1.x, (int)s1.y, (int)s1.z, (int)s1.w};
        pa[1] = mx_v8i{(int)p2.x, (int)p2.y, (int)p2.z, (int)p2.w, 0, 0, 0, 0};
        sa[1] = mx_v8i{(int)s2.x, (int)s2.y, (int)s2.z, (int)s2.w, 0, 0, 0, 0};
        codes = lds_dscode[kw];
#pragma unroll
        for (int c = 0; c < 4; ++c) imgv[c] = *reinterpret_cast<const uint4*>(lds_ds + kw * 4096 + c * 1024 + lane * 16);
      }
      if (k + 1 < n_qtiles) issue_qtile(st_next, k + 1);
      __syncthreads();  // B2
      if (k > qt_begin) {
        const uint4 p3 = lds_pq[kw][3][lane], s3 = lds_sq[kw][3][lane];
        pa[1][4] = (int)p3.x;
        pa[1][5] = (int)p3.y;
        pa[1][6] = (int)p3.z;
        pa[1][7] = (int)p3.w;
        sa[1][4] = (int)s3.x;
        sa[1][5] = (int)s3.y;
        sa[1][6] = (int)s3.z;
        sa[1][7] = (int)s3.w;
        // block 3's chunks again, now written (the others may already hold tile k's image: keep the
        // values read before B2 for them)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 v = *reinterpret_cast<const uint4*>(lds_ds + kw * 4096 + c * 1024 + lane * 16);
          imgv[c].x = img_blk3[c] ? v.x : imgv[c].x;
          imgv[c].y = img_blk3[c] ? v.y : imgv[c].y;
          imgv[c].z = img_blk3[c] ? v.z : imgv[c].z;
          imgv[c].w = img_blk3[c] ? v.w : imgv[c].w;
        }
      }
      if (k > qt_begin) {
        // G3: dV += P_q^T dO; G4: dK += dS_q^T Q over the 128 queries of tile k - 1 (k-step ks: queries
        // 64 ks .. +63; B scales: query block 2 ks + hh, d-block db; the A scale of dS_q likewise)
        const uint8_t* lds_q = lds_qd[st_prev][0];
        const uint8_t* lds_do = lds_qd[st_prev][1];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t qsc_t = lds_sc[st_prev][2 * ks + hh];
          const uint32_t dosc_t = lds_sc[st_prev][4 + 2 * ks + hh];
          const uint32_t asc = (codes >> (8 * (2 * ks + hh))) & 0xffu;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const mx_v8i dob = lds_tr_operand(lds_do, ks, 32 * db, tr_row, tr_col, tr_swz);
            dv_acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa[ks], dob, dv_acc[db], 0, 0, 0, 119, 0,
                                                                         (int)(dosc_t >> (8 * db)));
            const mx_v8i qbt = lds_tr_operand(lds_q, ks, 32 * db, tr_row, tr_col, tr_swz);
            dk_acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(sa[ks], qbt, dk_acc[db], 0, 0, 0, (int)asc,
                                                                         0, (int)(qsc_t >> (8 * db)));
          }
        }
      }
      // This wave's part of tile k + 1 has landed. The vector memory counter also counts stores, so
      // the image and code stores are issued only now: they complete during the next period instead
      // of holding up this wait.
      wait_vm();
      if (k > qt_begin) {
        if (lane == 0) *reinterpret_cast<uint32_t*>(p.ds_codes + tile * 16 + 4 * kw) = codes;
#pragma unroll
        // non-temporal: the dQ pass reads each image once, and stores that do not stay dirty in the
        // caches leave its reads without write-backs to wait behind (dQ pass 268 -> 250 us measured)
        for (int c = 0; c < 4; ++c) {
          const mx_u32x4 v4 = {imgv[c].x, imgv[c].y, imgv[c].z, imgv[c].w};
          __builtin_nontemporal_store(v4, reinterpret_cast<mx_u32x4*>(img + c * 1024 + lane * 16));
        }
      }
      st = st_next;
    }

    // ---- epilogue: dV and dK = c dK of the wave's 32 keys (accumulator: column d = 32 db + r, rows
    // kv 8 (v/4) + 4 hh + v%4 of the wave's key block) ----
    const int64_t orow = (k_start + kv0 + 32 * kw) * (int64_t)C + h * kD;
    if (p.dv) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kr = 8 * (v >> 2) + 4 * hh + (v & 3);
          if (kv0 + 32 * kw + kr < Lk) {
            const uint32_t o = (uint32_t)(kr * C + 32 * db + r);
            p.dv[orow + o] = (uint16_t)f32_to_bf16(dv_acc[db][v]);
            p.dk[orow + o] = (uint16_t)f32_to_bf16(dk_acc[db][v] * p.c);
          }
        }
    }
    // MXFP8 gradients: the wave's 32 keys x 4 blocks of 32 columns are four SQ32 blocks each (key
    // blocks start at the sequence start); block row koff.blocks32 + (kv0 + 32 kw) / 32
    const int kvalid = Lk - (kv0 + 32 * kw);
    if (p.dv_mx && kvalid > 0) {  // wave-uniform
      const int64_t brow = koff.blocks32 + ((kv0 + 32 * kw) >> 5);
      const int64_t nbk = (p.dk_mx_scale_t || p.dv_mx_scale_t) ? seq_offsets(p.cu_k, p.nseq).blocks32 : 0;
      // staging for the payload: 1 KB of this wave's own part of the dS image buffer, which nothing
      // reads after the last period (this wave read its image chunks before its last stores)
      uint8_t* stage = lds_ds + kw * 4096;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        float x[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] = dv_acc[db][v];
        store_grad_sq32(x, kvalid, p.dv_mx + orow + 32 * db, C, p.dv_mx_scale + brow * Cs + h * 4 + db,
                        p.dv_mx_scale_t ? p.dv_mx_scale_t + (int64_t)(h * 4 + db) * nbk + brow : nullptr, stage, lane,
                        hh);
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] = dk_acc[db][v] * p.c;
        store_grad_sq32(x, kvalid, p.dk_mx + orow + 32 * db, C, p.dk_mx_scale + brow * Cs + h * 4 + db,
                        p.dk_mx_scale_t ? p.dk_mx_scale_t + (int64_t)(h * 4 + db) * nbk + brow : nullptr, stage, lane,
                        hh);
      }
    }
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
  int contiguous;
  int causal;
  const uint8_t* ds_img;
  const uint8_t* ds_codes;
  int dq_fp16;
  int log2_sigma;  // sigma = 2^log2_sigma (0 in FP32 mode)
  float mult;      // c / sigma
  uint16_t* dq;    // bf16 dQ, or null
  uint8_t *dq_mx, *dq_mx_scale;  // E4M3 SQ32 dQ (compact codes [blocks][C/32]), or null
  uint8_t* dq_mx_scale_t;         // the codes transposed [C/32][blocks], or null
};

// LDS ring of (dS image, K tile) stages (a power of two). Two stages keep the LDS at 66 KB so two
// workgroups share a CU, which measured faster than deeper prefetching with one workgroup per CU.
constexpr int kDqStages = 2;

__global__ void __launch_bounds__(64 * kDqWaves, 1) attn_dq_kernel(DqParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_img[kDqStages][kTile * kD];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_kt[kDqStages][kTile * kD];
  __shared__ __attribute__((aligned(256))) uint32_t lds_codes[kDqStages][64];
  __shared__ __attribute__((aligned(256))) uint32_t lds_ksc[kDqStages][64];

  // pairs in the reverse of the main pass's order: the images it wrote last are read first
  const int item = mx_item(p.contiguous, (int)blockIdx.x, p.total_items, p.ntq_max, p.nseq * p.H, true);
  if (item < 0) return;
  const int qt = item % p.ntq_max;
  const int h = (item / p.ntq_max) % p.H;
  const int s = item / (p.ntq_max * p.H);
  const int64_t q_start = p.cu_q[s], k_start = p.cu_k[s];
  const int Lq = p.cu_q[s + 1] - (int)q_start;
  const int Lk = p.cu_k[s + 1] - (int)k_start;
  const int q0 = qt * kTile;
  if (q0 >= Lq) return;  // uniform over the workgroup
  const SeqOffsets koff = seq_offsets(p.cu_k, s);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int qb = wave_s & 3, half = wave_s >> 2;
  const int r = lane & 31, hh = lane >> 5;
  const int C = p.H * kD;
  const int Cs = C >> 5;
  const TileLane<kDqWaves> tl = tile_lane<kDqWaves>(wave, lane, C);
  int ntk = (Lk + kTile - 1) / kTile;
  if (p.causal) ntk = min(ntk, qt + 1);  // key tiles past the query tile are fully masked

  const uint8_t* kbase = (const uint8_t*)mx_uniform_ptr((void*)(p.k + k_start * (int64_t)C + h * kD));
  const int64_t tile0 = (((int64_t)h * p.nseq + s) * p.ntq_max + qt) * p.ntk_max;  // image of key tile 0
  const uint8_t* img_base = (const uint8_t*)mx_uniform_ptr((void*)(p.ds_img + tile0 * (kTile * kD)));
  const uint8_t* code_base = p.ds_codes + tile0 * 16;
  const uint8_t* ksc_base = p.k_scale + (koff.padded / 32) * (int64_t)Cs + h * 4;
  auto issue_loads = [&](int kt, uint8_t* img, uint8_t* ktile, uint32_t* codes, uint32_t* kscw) {
    // the dS_q image is copied as it is (2 KB per wave, 16 B per lane), read once: non-temporal
#pragma unroll
    for (int c = 0; c < TileLane<kDqWaves>::kPieces; ++c) {
      const int piece = wave_s * TileLane<kDqWaves>::kPieces + c;
      mx_lds_dma16_nt((MX_LDS void*)(img + piece * 1024), img_base + (int64_t)kt * (kTile * kD),
                   (uint32_t)(piece * 1024 + lane * 16));
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
  const int64_t orow = (q_start + q0 + 32 * qb) * (int64_t)C + h * kD;
  const int qvalid = Lq - (q0 + 32 * qb);
  int64_t brow = 0, nbq = 0;
  if (p.dq_mx) {
    brow = seq_offsets(p.cu_q, s).blocks32 + ((q0 + 32 * qb) >> 5);
    __syncthreads();  // every wave is done with the image stages; 1 KB of stage 0 per wave stages dQ
  }
  if (p.dq_mx_scale_t) nbq = seq_offsets(p.cu_q, p.nseq).blocks32;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int db = 2 * half + e;
    float x[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (p.dq_fp16) {
        const float2 f = __half22float2(__builtin_bit_cast(__half2, acc16[e][v >> 1]));
        x[v] = ((v & 1) ? f.y : f.x) * p.mult;
      } else {
        x[v] = acc32[e][v] * p.mult;
      }
    }
    if (p.dq) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int qr = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (qr < qvalid) p.dq[orow + (uint32_t)(qr * C + 32 * db + r)] = (uint16_t)f32_to_bf16(x[v]);
      }
    }
    // MXFP8 dQ: one SQ32 block (32 queries from the sequence start x 32 columns) per (e, wave)
    if (p.dq_mx && qvalid > 0)
      store_grad_sq32(x, qvalid, p.dq_mx + orow + 32 * db, C, p.dq_mx_scale + brow * Cs + h * 4 + db,
                      p.dq_mx_scale_t ? p.dq_mx_scale_t + (int64_t)(h * 4 + db) * nbq + brow : nullptr,
                      &lds_img[0][wave_s * 1024], lane, hh);
  }
}

}  // namespace

namespace mxfa {

// Workspace: the dS_q images [H][nseq][ntq_max][ntk_max] (16 KB each), their block codes (16 B
// each), then -Delta [H][Tq] and the exponent offsets [H][Tq] (fp32), each region 256-byte aligned.
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
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, const GradMxOut* mx_out, hipStream_t stream) {
  const int64_t Tq = a.total_q;
  const int C = a.H * kD;
  const BwdWorkspace w = bwd_workspace_layout(Tq, a.H, a.nseq, a.max_seqlen_q, a.max_seqlen_k);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  float* delta = reinterpret_cast<float*>(ws + w.delta);
  float* pexp = reinterpret_cast<float*>(ws + w.pexp);
  const int ntq_max = (a.max_seqlen_q + kTile - 1) / kTile;
  const int ntk_max = (a.max_seqlen_k + kTile - 1) / kTile;
  if (Tq > 0) {
    hipLaunchKernelGGL(bwd_preprocess_kernel, dim3((unsigned)((Tq + 63) / 64), (unsigned)a.H), dim3(256), 0, stream, o,
                       dout_bf16, lse, Tq,
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
  const MxItemOrder ord = mx_item_order(a.total_q, a.total_k, a.nseq, a.max_seqlen_q, a.max_seqlen_k,
                                       (int64_t)a.H * a.nseq, p.n_ktiles);
  p.contiguous = ord.contiguous;
  p.total_items = (int)ord.grid;  // < 2^31, checked by the caller
  p.c2 = a.softmax_scale * kLog2e;
  p.causal = a.causal;
  p.pexp = pexp; p.ndelta = delta; p.Tq = Tq;
  p.ntq_max = ntq_max; p.ntk_max = ntk_max;
  p.ds_img = ws + w.img;
  p.ds_codes = ws + w.codes;
  p.c = a.softmax_scale;
  p.dk = dk; p.dv = dv;
  p.dk_mx = mx_out ? mx_out->dk : nullptr;
  p.dk_mx_scale = mx_out ? mx_out->dk_scale : nullptr;
  p.dv_mx = mx_out ? mx_out->dv : nullptr;
  p.dv_mx_scale = mx_out ? mx_out->dv_scale : nullptr;
  p.dk_mx_scale_t = mx_out ? mx_out->dk_scale_t : nullptr;
  p.dv_mx_scale_t = mx_out ? mx_out->dv_scale_t : nullptr;
  if (p.total_items > 0) {
    hipLaunchKernelGGL(attn_bwd_kernel, dim3((unsigned)p.total_items), dim3(64 * kBwdWaves), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  DqParams d;
  d.k = a.k.data; d.k_scale = a.k.scale;
  d.cu_q = a.cu_q; d.cu_k = a.cu_k;
  d.nseq = a.nseq; d.H = a.H; d.ntq_max = ntq_max; d.ntk_max = ntk_max;
  const MxItemOrder dord = mx_item_order(a.total_q, a.total_k, a.nseq, a.max_seqlen_q, a.max_seqlen_k,
                                        (int64_t)a.H * a.nseq, ntq_max);
  d.contiguous = dord.contiguous;
  d.total_items = (int)dord.grid;
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
  d.dq_mx = mx_out ? mx_out->dq : nullptr;
  d.dq_mx_scale = mx_out ? mx_out->dq_scale : nullptr;
  d.dq_mx_scale_t = mx_out ? mx_out->dq_scale_t : nullptr;
  if (d.total_items > 0) {
    hipLaunchKernelGGL(attn_dq_kernel, dim3((unsigned)d.total_items), dim3(64 * kDqWaves), 0, stream, d);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mxfa

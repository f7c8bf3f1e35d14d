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
//  * LDS tiles are 128 rows x 128 bytes with the 16-byte chunk index XOR-swizzled (lds_swz):
//    conflict-free for the row reads of K and the transposed reads of V.
//  * Grid order is XCD-aware (mx_pair_item): the query tiles of one (sequence, head) pair run on one
//    XCD, whose L2 holds that head's K and V, and the pairs are dealt to the XCDs in turn, so every
//    XCD gets the same share of a jagged batch's long and short sequences.
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
  int total_items;
  float c;   // softmax scale
  float c2;  // softmax scale * log2(e)
  int causal;
  uint16_t* o;          // bf16 O, or null
  uint8_t* o_mx;        // E4M3 O in ROW32 blocks (32 of D per token and head), or null
  uint8_t* o_mx_scale;  // its E8M0 codes [T_q][H*D/32]
  float* lse;
  int64_t Tq;
};

__device__ __forceinline__ int swz(int row) { return lds_swz(row); }

// x if off < lim, else -inf. One compare into VCC and one select (inline asm so that the 64 compares
// of a masked tile do not each occupy a scalar register pair).
__device__ __forceinline__ float keep_below(float x, int off, int lim, float ninf) {
  float y;
  asm("v_cmp_lt_i32_e32 vcc, %2, %3\n\tv_cndmask_b32_e32 %0, %4, %1, vcc"
      : "=v"(y)
      : "v"(x), "i"(off), "v"(lim), "v"(ninf)
      : "vcc");
  return y;
}

template <int V>
struct Stage {
  static constexpr int value = V;
};

// LDS image of one workgroup: two stages x (K tile, V tile), then per stage the tile's K scale words
// (one per key row) and V scale bytes (4 key blocks x 128 columns).
constexpr int kLdsTiles = 2 * 2 * kTile * kD;
constexpr int kLdsKsc = kLdsTiles;               // 2 x 128 words
constexpr int kLdsVsc = kLdsKsc + 2 * kTile * 4; // 2 x 512 bytes
constexpr int kLdsBytes = kLdsVsc + 2 * kTile * 4;
constexpr int lds_k_off(int st) { return (2 * st) * kTile * kD; }
constexpr int lds_v_off(int st) { return (2 * st + 1) * kTile * kD; }

// Direct global -> LDS copies whose LDS destination is a per-wave base register plus a compile-time
// offset, added straight into M0 (so no per-destination scalar register stays live across the loop).
// dma16_at: lane l's 16 bytes at base + voff land at wave_lds + IMM + 16 l. dma4_at: lane l's word
// at addr lands at wave_lds + IMM + 4 l. The caller waits (s_waitcnt vmcnt) before reading them.
template <int IMM>
__device__ __forceinline__ void dma16_at(uint32_t wave_lds, const void* base, uint32_t voff) {
  asm volatile("s_add_u32 m0, %0, %3\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(wave_lds), "v"(voff), "s"(base),
               "i"(IMM)
               : "memory", "scc");
}
template <int IMM>
__device__ __forceinline__ void dma4_at(uint32_t wave_lds, const void* addr) {
  asm volatile("s_add_u32 m0, %0, %2\n\tglobal_load_lds_dword %1, off" ::"s"(wave_lds), "v"(addr), "i"(IMM)
               : "memory", "scc");
}

// Issue the asynchronous global -> LDS copy of one 128 x 128-byte tile into a swizzled LDS tile at
// byte offset TILE of the workgroup's LDS image. `base` is the wave-uniform address of the tile's
// first row (this head's columns); each wave writes four contiguous 1 KB pieces (64 lanes x 16
// bytes) starting at wave_lds = 4 KB x wave, and the swizzle is applied by choosing which logical
// chunk each lane fetches: lane piece c covers row trow[c], logical chunk offset tcol[c] (byte
// offset toff[c] in a full tile). Rows past the end of the sequence fetch the last valid row
// instead (finite data; the scores of those rows are masked and their P is exactly 0).
template <int TILE>
__device__ __forceinline__ void issue_tile_load(uint32_t wave_lds, const uint8_t* base, int valid, int C,
                                                const int* trow, const int* tcol, const uint32_t* toff) {
  uint32_t off[4];
  if (valid >= kTile) {
#pragma unroll
    for (int c = 0; c < 4; ++c) off[c] = toff[c];
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) off[c] = (uint32_t)(min(trow[c], valid - 1) * C + tcol[c]);
  }
  dma16_at<TILE + 0>(wave_lds, base, off[0]);
  dma16_at<TILE + 1024>(wave_lds, base, off[1]);
  dma16_at<TILE + 2048>(wave_lds, base, off[2]);
  dma16_at<TILE + 3072>(wave_lds, base, off[3]);
}

// The direct LDS loads are inline asm (mx_lds_dma16/4): the compiler would otherwise wait for every
// outstanding vector memory operation before the next LDS read, i.e. for the prefetch of the next
// tile right after issuing it. Their waits are asm as well.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Two floats -> two E4M3 bytes in the low or high half of a word whose other half is kept.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}
// A register with unspecified contents (no instruction): the first conversion into a word starts
// from it, and the second overwrites the other half, so no zeroing move is needed.
__device__ __forceinline__ uint32_t undef_word() {
  uint32_t u;
  asm volatile("; unspecified %0" : "=v"(u));
  return u;
}

// QKF: the element format of Q and K, as the scaled MFMA's format code: 0 E4M3; 4 E2M1 (MXFP4, two
// elements per byte); 2 E2M3 (MXFP6, a block's 32 codes in 24 bytes, the two blocks of each 64-element
// d-step stored as their two 16-byte pieces, then their two 8-byte pieces). Both low-precision forms run
// S at twice the FP8 rate with ROW32 scales; a lane's operand is then the 32 elements of one d-block
// (16 or 24 bytes). The MXFP4 K tile takes 64 bytes per key: LDS row R of the K stage holds keys 2R
// (logical chunks 0-3) and 2R + 1 (chunks 4-7). The MXFP6 K tile keeps one key per 128-byte row
// (96 bytes used; the copy of logical chunks 6 and 7 re-reads chunks 0 and 1). Both are swizzled
// like the FP8 tiles.
template <bool VCOL32, bool PDYN, int QKF>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(FwdParams p) {
  constexpr bool QK4 = QKF == 4, QK6 = QKF == 2;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[kLdsBytes];
  MX_LDS uint8_t* const lds = (MX_LDS uint8_t*)lds_raw;

  const int item = mx_pair_item((int)blockIdx.x, p.n_qtiles, p.nseq * p.H);
  if (item < 0) return;
  const int qt = p.n_qtiles - 1 - item % p.n_qtiles;  // heavy (late) query tiles first
  const int h = (item / p.n_qtiles) % p.H;
  const int s = item / (p.n_qtiles * p.H);
  const int64_t q_start = p.cu_q[s], k_start = p.cu_k[s];
  const int Lq = p.cu_q[s + 1] - (int)q_start;
  const int Lk = p.cu_k[s + 1] - (int)k_start;
  if (qt * kTile >= Lq) return;  // uniform over the workgroup

  const SeqOffsets qoff = seq_offsets(p.cu_q, s);
  const SeqOffsets koff = seq_offsets(p.cu_k, s);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int C = p.H * kD;
  const int Cs = C >> 5;

  int n_ktiles = (Lk + kTile - 1) / kTile;
  if (p.causal) {
    const int q_last = min(qt * kTile + kTile - 1, Lq - 1);
    n_ktiles = min(n_ktiles, q_last / kTile + 1);
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave index as a scalar
  int trow[4], tcol[4];
  uint32_t toff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int pchunk = (wave * 4 + c) * 64 + lane;  // physical 16-byte chunk index in the tile
    trow[c] = pchunk >> 3;
    tcol[c] = 16 * ((pchunk & 7) ^ swz(pchunk >> 3));
    toff[c] = (uint32_t)(trow[c] * C + tcol[c]);
  }
  // row stride of Q and K in bytes, and the K tile pieces of QK4 (two 1 KB pieces per wave: piece c
  // of wave w covers LDS row R = 8 (2 w + c) + l / 8, physical chunk l % 8, i.e. key 2 R + lc / 4,
  // bytes 16 (lc % 4) of its 64, lc = (l % 8) ^ swz(R) the logical chunk)
  constexpr int kQKBytes = QK4 ? kD / 2 : QK6 ? 3 * kD / 4 : kD;
  const int ldqk = QK4 ? C / 2 : QK6 ? 3 * C / 4 : C;
  int k4row[2];
  uint32_t k4col[2];
  if constexpr (QK4) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int pchunk = (wave * 2 + c) * 64 + lane;
      const int R = pchunk >> 3, lc = (pchunk & 7) ^ swz(pchunk >> 3);
      k4row[c] = 2 * R + (lc >> 2);
      k4col[c] = (uint32_t)(16 * (lc & 3));
    }
  }
  // MXFP6 K tile pieces: as the FP8 tile's, 96-byte rows (logical chunks 6 and 7 re-read 0 and 1)
  uint32_t k6col[4];
  if constexpr (QK6) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int lc = tcol[c] >> 4;
      k6col[c] = (uint32_t)(16 * (lc < 6 ? lc : lc - 6));
    }
  }
  const uint8_t* kbase = (const uint8_t*)mx_uniform_ptr((void*)(p.k + k_start * (int64_t)ldqk + h * kQKBytes));
  const uint8_t* vbase = (const uint8_t*)mx_uniform_ptr((void*)(p.v + k_start * (int64_t)C + h * kD));
  // LDS byte address of this wave's pieces of a tile, and of its part of the scale areas
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  const uint32_t wave_lds = lds_addr + (uint32_t)wave_s * 4096u;
  const uint32_t wave_lds_k4 = lds_addr + (uint32_t)wave_s * 2048u;  // QK4 K tile pieces
  // K tile of key rows kv0.. into K stage TILE: FP8 tiles as V's, FP4 tiles in 8 KB
  auto issue_k_load = [&](auto tilec, int kv0) {
    constexpr int TILE = decltype(tilec)::value;
    const uint8_t* base = kbase + (int64_t)kv0 * ldqk;
    const int valid = Lk - kv0;
    if constexpr (QK4) {
      uint32_t off[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) off[c] = (uint32_t)(min(k4row[c], valid - 1) * ldqk) + k4col[c];
      dma16_at<TILE + 0>(wave_lds_k4, base, off[0]);
      dma16_at<TILE + 1024>(wave_lds_k4, base, off[1]);
    } else if constexpr (QK6) {
      uint32_t off[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) off[c] = (uint32_t)(min(trow[c], valid - 1) * ldqk) + k6col[c];
      dma16_at<TILE + 0>(wave_lds, base, off[0]);
      dma16_at<TILE + 1024>(wave_lds, base, off[1]);
      dma16_at<TILE + 2048>(wave_lds, base, off[2]);
      dma16_at<TILE + 3072>(wave_lds, base, off[3]);
    } else {
      issue_tile_load<TILE>(wave_lds, base, valid, C, trow, tcol, toff);
    }
  };

  // ---- Q tile rows of this wave, held as the B operand of S^T = K Q^T ----
  const int qrow = qt * kTile + wave * 32 + r;  // position in the sequence
  mx_v8i qa[2];
  {
    const bool valid = qrow < Lq;
    const uint8_t* src = p.q + (q_start + qrow) * (int64_t)ldqk + h * kQKBytes;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
      if constexpr (QK4) {
        // FP4: the lane's 32 elements of d-block 2 ds + hh, 16 bytes (the upper operand half unused)
        if (valid) lo = *reinterpret_cast<const uint4*>(src + 32 * ds + 16 * hh);
      } else if constexpr (QK6) {
        // FP6: the 24 bytes of d-block 2 ds + hh (registers 0-5): its 16-byte piece, then its 8-byte one
        if (valid) {
          lo = *reinterpret_cast<const uint4*>(src + 48 * ds + 16 * hh);
          const uint2 t8 = *reinterpret_cast<const uint2*>(src + 48 * ds + 32 + 8 * hh);
          hi = make_uint4(t8.x, t8.y, 0u, 0u);
        }
      } else if (valid) {
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

  // K and V scales of a key tile, copied into LDS with the tile: word l of a K scale stage is the K
  // scale word (4 d-blocks) of key row kv0 + l (ROW32) or of its 32-row block (SQ32); a V scale
  // stage holds, for key block vb = 0..3, the 128 V scale bytes of this head's columns (COL32) or
  // its 4 d-block bytes (SQ32) at byte offset 128 vb. Waves 0-1 copy K scales, waves 2-3 V scales
  // (64 words each).
  const uint8_t* ksbase = p.k_scale + (koff.padded >> p.k_row_shift) * (int64_t)Cs + h * 4;
  const uint8_t* vsbase = p.v_scale + (koff.padded >> 5) * (int64_t)(VCOL32 ? C : Cs);
  constexpr int vcs_shift = VCOL32 ? 0 : 5;
  const uint32_t scale_lds = lds_addr + 256u * (uint32_t)(wave_s & 1);
  auto issue_kscale_load = [&](int kv0, auto stc) {  // waves 0-1
    constexpr int st = decltype(stc)::value;
    const int l = 64 * (wave_s & 1) + lane;
    dma4_at<kLdsKsc + st * 512>(scale_lds, ksbase + (int64_t)(((kv0 + l) >> p.k_row_shift) * Cs));
  };
  auto issue_vscale_load = [&](int kv0, auto stc) {  // waves 2-3
    constexpr int st = decltype(stc)::value;
    const int l = 64 * (wave_s & 1) + lane;
    const int col = VCOL32 ? h * kD + 4 * (l & 31) : h * 4;
    dma4_at<kLdsVsc + st * 512>(scale_lds, vsbase + (int64_t)(((kv0 >> 5) + (l >> 5)) * (C >> vcs_shift) + col));
  };
  // Prologue loads: K, V and their scales of tile 0 into stage 0, K and its scales of tile 1 into
  // stage 1. In the loop, the loads issued in the middle of step t bring K of tile t + 2 and V of
  // tile t + 1 (with their scales): K one step before its scores are computed, V one and a half.
  if (n_ktiles > 0) {
    issue_k_load(Stage<lds_k_off(0)>{}, 0);
    issue_tile_load<lds_v_off(0)>(wave_lds, vbase, Lk, C, trow, tcol, toff);
    if (wave_s < 2)
      issue_kscale_load(0, Stage<0>{});
    else
      issue_vscale_load(0, Stage<0>{});
  }
  if (n_ktiles > 1) {
    issue_k_load(Stage<lds_k_off(1)>{}, kTile);
    if (wave_s < 2) issue_kscale_load(kTile, Stage<1>{});
  }

  float m = -INFINITY;  // running max of raw scores for query row qrow
  float lsum = 0.0f;    // this lane's half of the row sum of P * 256
  mx_v16f oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = mx_v16f{};

  // Per-lane LDS byte offsets that do not change from tile to tile (the stage and the key/row
  // block are compile-time offsets added to them):
  //  * K rows: row 32 kb + r, d-step ds, half (lo: chunk 4 ds + hh, hi: chunk 4 ds + 2 + hh), swizzled
  //    by swz(r) (adding 32 kb leaves the swizzle unchanged);
  //  * V^T reads (see the lane map in mx_device.h): row tr_row (+ 64 ks + 32 (cc >> 1) + 16 (cc & 1),
  //    which leave the swizzle unchanged), column 32 db + tr_col;
  //  * scales: K scale word 32 kb + r; V scale byte 128 (2 ks + hh) + (COL32: 32 db + r, SQ32: db).
  //  * QK4 K rows: key 32 kb + r is in LDS row 16 kb + r / 2 (its swizzle does not depend on kb),
  //    logical chunk 4 (r % 2) + 2 ds + hh: the 32 elements of d-block 2 ds + hh;
  //  * QK6 K rows: key row r, the 24 bytes of d-block 2 ds + hh: logical chunk 3 ds + hh (16 bytes)
  //    and the half hh of logical chunk 3 ds + 2 (8 bytes) (koffs6);
  uint32_t koffs[2][2];
  uint32_t koffs6[2][2];
  if constexpr (QK6) {
    const int sw = swz(r);
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      koffs6[ds][0] = (uint32_t)(r * kD + 16 * ((3 * ds + hh) ^ sw));
      koffs6[ds][1] = (uint32_t)(r * kD + 16 * ((3 * ds + 2) ^ sw) + 8 * hh);
    }
  }
  if constexpr (QK4) {
    const int R = r >> 1, sw = swz(R);
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      koffs[ds][0] = (uint32_t)(R * kD + 16 * ((4 * (r & 1) + 2 * ds + hh) ^ sw));
      koffs[ds][1] = koffs[ds][0];
    }
  } else {
    const int sw = swz(r);
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      koffs[ds][0] = (uint32_t)(r * kD + 16 * ((4 * ds + hh) ^ sw));
      koffs[ds][1] = (uint32_t)(r * kD + 16 * ((4 * ds + 2 + hh) ^ sw));
    }
  }
  uint32_t voffs[4];
  {
    const int grp = lane >> 4, gl = lane & 15;
    const int tb = gl >> 1, ts = gl & 1;
    const int tr_row = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);
    const int tr_col = 16 * (grp & 1) + 8 * ts;
    const int tr_swz = swz(tr_row);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int col = 32 * db + tr_col;
      voffs[db] = (uint32_t)(tr_row * kD + 16 * ((col >> 4) ^ tr_swz) + (col & 15));
    }
  }
  const uint32_t ksc_off = (uint32_t)(kLdsKsc + 4 * r);
  const uint32_t vsc_off = (uint32_t)(kLdsVsc + 128 * hh + (VCOL32 ? r : 0));

  // S^T = K Q^T for key blocks [KB0, KB1) of the tile in K stage SK: 4 key blocks of 32 x 2 D-steps
  // of 64, the K scale words read from the tile's scale stage
  mx_v16f sacc[4];
  auto issue_s = [&](auto skc, auto kb0c, auto kb1c) {
    constexpr int sk = decltype(skc)::value, kb0 = decltype(kb0c)::value, kb1 = decltype(kb1c)::value;
#pragma unroll
    for (int kb = kb0; kb < kb1; ++kb) {
      const uint32_t kscb = *(const MX_LDS uint32_t*)(lds + ksc_off + sk * 512 + 128 * kb) >> (8 * hh);
      sacc[kb] = mx_v16f{};
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        // operand format: the MFMA's code (the FP4 operand fills registers 0-3, the FP6 one 0-5)
        constexpr int fmt = QKF;
        mx_v8i ka;
        if constexpr (QK6) {
          const MX_LDS uint8_t* t = lds + lds_k_off(sk) + 32 * kb * kD;
          const mx_v4i a16 = *(const MX_LDS mx_v4i*)(t + koffs6[ds][0]);
          const mx_v2i a8 = *(const MX_LDS mx_v2i*)(t + koffs6[ds][1]);
          ka = mx_v8i{a16.x, a16.y, a16.z, a16.w, a8.x, a8.y, 0, 0};
        } else {
          const MX_LDS uint8_t* t = lds + lds_k_off(sk) + 32 * kb * kQKBytes;
          const mx_v4i lo = *(const MX_LDS mx_v4i*)(t + koffs[ds][0]);
          mx_v4i hi = mx_v4i{0, 0, 0, 0};
          if constexpr (!QK4) hi = *(const MX_LDS mx_v4i*)(t + koffs[ds][1]);
          ka = mx_v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
        if (ds == 0)
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa[0], sacc[kb], fmt, fmt, 0, (int)kscb, 0,
                                                                     (int)qsc);
        else
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa[1], sacc[kb], fmt, fmt, 2, (int)kscb, 2,
                                                                     (int)qsc);
      }
    }
  };
  using KB0 = Stage<0>;
  using KB2 = Stage<2>;
  using KB4 = Stage<4>;

  wait_vm();
  __syncthreads();
  if (n_ktiles > 0) issue_s(Stage<0>{}, KB0{}, KB4{});

  // One step per key tile t (stage st = t % 2). Software pipeline: the scores of tile t + 1 are
  // computed by MFMAs issued in the middle and at the end of step t, into the registers that the
  // exponentials of tile t have just consumed, so the matrix cores work while this wave runs the
  // softmax:
  //   1. mask, row max (and, with the dynamic P scale, the block maxima and codes), exponent
  //      offsets (tile t's scores are complete)
  //   2. P of key blocks 0-1 -> E4M3
  //   3. rescale O and l where the row max moved (skipped, exactly, when none did)
  //   4. wait for the loads issued one step ago (K of t + 1, V of t, their scales), barrier; issue
  //      the loads of K of t + 2 and V of t + 1 into the stages of K of t and V of t - 1, which every
  //      wave has finished reading
  //   5. scores of tile t + 1, key blocks 0-1; O^T += V^T P^T for keys 0-63
  //   6. P of key blocks 2-3 -> E4M3 (while the MFMAs of 5 run)
  //   7. O^T += V^T P^T for keys 64-127; scores of tile t + 1, key blocks 2-3
  auto step = [&](int kt, auto stc) {
    constexpr int st = decltype(stc)::value;
    const int kv0 = kt * kTile;

    // ---- 1. mask (ragged tail, causal diagonal) ----
    const bool need_mask = (kv0 + kTile > Lk) || (p.causal && kv0 + kTile - 1 > qt * kTile + wave * 32);
    if (need_mask) {
      // key kv0 + 32 kb + 8 (v >> 2) + 4 hh + (v & 3) is masked when its offset in the tile reaches
      // lim + 4 hh: past the sequence end, or (causal) past this lane's query row
      const int lim = min(Lk - kv0, p.causal ? qrow - kv0 + 1 : kTile) - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          sacc[kb][v] = keep_below(sacc[kb][v], 32 * kb + 8 * (v >> 2) + (v & 3), lim, -INFINITY);
    }

    // online softmax (FP32)
    float m_new;
    float bmx[4];  // dynamic P scale: largest score of each 32-key block (both lane halves)
    if constexpr (!PDYN) {
      // two independent max chains (key blocks 0-1 first: their MFMAs were issued first), joined
      // at the end
      float mx0 = m, mx1 = m;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        mx0 = max3f(mx0, sacc[0][v], sacc[0][v + 1]);
        mx1 = max3f(mx1, sacc[1][v], sacc[1][v + 1]);
      }
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        mx0 = max3f(mx0, sacc[2][v], sacc[2][v + 1]);
        mx1 = max3f(mx1, sacc[3][v], sacc[3][v + 1]);
      }
      // joins by v_max3 as well (fmaxf would first canonicalize each operand with a max of itself)
      const float mx = max3f(mx0, mx1, mx1);
      auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      m_new = max3f(__uint_as_float(sw2[0]), __uint_as_float(sw2[1]), __uint_as_float(sw2[1]));
    } else {
      // one chain per key block, each joined with the other lane half (which holds the block's
      // other 16 keys); the row maximum is the largest block maximum
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float x = max3f(sacc[kb][0], sacc[kb][1], sacc[kb][2]);
#pragma unroll
        for (int v = 3; v < 15; v += 2) x = max3f(x, sacc[kb][v], sacc[kb][v + 1]);
        x = fmaxf(x, sacc[kb][15]);
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        bmx[kb] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      m_new = fmaxf(max3f(m, bmx[0], bmx[1]), fmaxf(bmx[2], bmx[3]));
    }
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float base = m_use * p.c2 - 8.0f;  // exp2(S c2 - base) = 256 P

    // Exponent offset of each key block: P_q = E4M3(exp2(S c2 - pbase)). Static scale: pbase =
    // base for every block (256 P, code 119). Dynamic scale: the MX rule on the block's largest P,
    // code = exponent field of max P - 8 (clamped at 0), so that P lands in [256, 512) relative to
    // the block scale 2^(code - 127): pbase = base + code - 119. max P is taken as
    // exp2((block max - m) c2), which is exactly 1 for the block holding the row maximum: going
    // through base instead (exp2(block max c2 - base) / 256) would put it just below 1 whenever
    // base rounds up, and give that block code 118 and a saturated largest element. The row sum
    // collects each block's exponentials with the weight 2^(code - 119).
    float pbase[4];
    uint32_t pcode[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if constexpr (PDYN) {
        const float pmax = __builtin_amdgcn_exp2f((bmx[kb] - m_use) * p.c2);
        const int code = max((int)(__float_as_uint(pmax) >> 23) - 8, 0);
        pcode[kb] = (uint32_t)code;
        pbase[kb] = base + (float)(code - 119);
      } else {
        pcode[kb] = 119u;
        pbase[kb] = base;
      }
    }


    // ---- 2. P = exp2(S c2 - pbase), packed to E4M3. Static scale: 256 P in [0, 256], no clamp
    // needed. Dynamic scale: up to 512, saturated at 448 (the converter gives NaN beyond) ----
    uint32_t pk[4][4];
    float ps = 0.0f;
    auto exp_pack = [&](int kb) {
      float psk = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 0], p.c2, -pbase[kb]));
        float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 1], p.c2, -pbase[kb]));
        float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 2], p.c2, -pbase[kb]));
        float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * i + 3], p.c2, -pbase[kb]));
        if constexpr (PDYN) {
          psk += (e0 + e1) + (e2 + e3);
          e0 = fminf(e0, 448.0f);
          e1 = fminf(e1, 448.0f);
          e2 = fminf(e2, 448.0f);
          e3 = fminf(e3, 448.0f);
        } else {
          ps += (e0 + e1) + (e2 + e3);
        }
        pk[kb][i] = cvt2<true>(e2, e3, cvt2<false>(e0, e1, undef_word()));
      }
      if constexpr (PDYN) ps = fmaf(psk, __uint_as_float((pcode[kb] + 8u) << 23), ps);
    };
    exp_pack(0);
    exp_pack(1);

    // ---- 3. rescale O and l where the row max moved (skipped, exactly, when none did); after the
    // exponentials so that the wait for the last PV products of the previous step is short ----
    if (__builtin_amdgcn_ballot_w64(m_new > m)) {
      const float alpha = __builtin_amdgcn_exp2f((m - m_use) * p.c2);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
    }
    m = m_new;
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. loads of the next stages ----
    wait_vm();
    __syncthreads();
    if (kt + 2 < n_ktiles) {
      issue_k_load(Stage<lds_k_off(st)>{}, kv0 + 2 * kTile);
      if (wave_s < 2) issue_kscale_load(kv0 + 2 * kTile, Stage<st>{});
    }
    const bool more = kt + 1 < n_ktiles;
    if (more) {
      issue_tile_load<lds_v_off(st ^ 1)>(wave_lds, vbase + (int64_t)(kv0 + kTile) * C, Lk - kv0 - kTile, C, trow,
                                         tcol, toff);
      if (wave_s >= 2) issue_vscale_load(kv0 + kTile, Stage<st ^ 1>{});
    }

    // O^T += V^T P^T for key step ks (64 keys) x 4 D-blocks of 32; the transposed V reads are issued
    // one MFMA ahead, and an empty asm statement that uses the MFMA result and clobbers memory pins
    // each MFMA and keeps later LDS reads below it
    auto read_v = [&](int ks, int db) {
      mx_v2i part[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int rowoff = (64 * ks + 32 * (cc >> 1) + 16 * (cc & 1)) * kD;
        part[cc] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MX_LDS mx_v2i*)(lds + lds_v_off(st) + rowoff + voffs[db]));
      }
      return mx_v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
    };
    auto pv = [&](int ks) {
      // P scale of this lane's K block: lane half hh supplies key block 2 ks + hh
      const uint32_t psc = PDYN ? (hh ? pcode[2 * ks + 1] : pcode[2 * ks]) : 119u;
      const mx_v8i pb{(int)pk[2 * ks][0], (int)pk[2 * ks][1], (int)pk[2 * ks][2], (int)pk[2 * ks][3],
                      (int)pk[2 * ks + 1][0], (int)pk[2 * ks + 1][1], (int)pk[2 * ks + 1][2], (int)pk[2 * ks + 1][3]};
      mx_v8i va_next = read_v(ks, 0);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t vsc = lds[vsc_off + st * 512 + 256 * ks + (VCOL32 ? 32 * db : db)];
        const mx_v8i va = va_next;
        if (db < 3) va_next = read_v(ks, db + 1);
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[db], 0, 0, 0, (int)vsc, 0, (int)psc);
        asm volatile("" : "+v"(oacc[db])::"memory");
      }
    };

    // ---- 5. ----
    // The next tile's scores are issued whether or not a next tile exists: after the last tile they
    // are computed from whatever the other stage holds and never read. A conditional issue would
    // merge two register assignments of the score accumulators after it, which the compiler
    // resolves with 32 register moves per step.
    issue_s(Stage<st ^ 1>{}, KB0{}, KB2{});
    pv(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 6. ----
    exp_pack(2);
    exp_pack(3);
    lsum += ps;
    asm volatile("" : "+v"(lsum));  // keep the row sum here (not sunk past the PV products)
    __builtin_amdgcn_sched_barrier(0);

    // ---- 7. ----
    pv(1);
    issue_s(Stage<st ^ 1>{}, KB2{}, KB4{});
  };

  // two tiles per iteration so that each stage's LDS addresses are compile-time offsets
  for (int kt = 0; kt < n_ktiles; kt += 2) {
    step(kt, Stage<0>{});
    if (kt + 1 < n_ktiles) step(kt + 1, Stage<1>{});
  }

  // ---- epilogue: O / l -> bf16, LSE ----
  {
    auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
  }
  const float l = lsum * (1.0f / 256.0f);
  const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
  // MX output: O = O_acc / l in FP32, quantized in ROW32 blocks (the MX scale rule of the operand
  // quantizer). Lane (r, hh) holds 16 of block db's 32 values (d = 32 db + 8 i + 4 hh + j), the
  // other lane half the other 16, so the block maximum is joined across the halves. Every lane
  // runs this part (the swap reads the partner lane); only rows inside the sequence store.
  uint32_t mx_words[4][4];
  uint32_t mx_codes = 0;
  if (p.o_mx) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      uint32_t amax = 0;  // largest sign-cleared bit pattern: orders NaN > Inf > finite magnitudes
#pragma unroll
      for (int v = 0; v < 16; ++v) amax = max(amax, __float_as_uint(oacc[db][v] * inv_l) & 0x7fffffffu);
      const auto sw = __builtin_amdgcn_permlane32_swap(amax, amax, false, false);
      amax = max((uint32_t)sw[0], (uint32_t)sw[1]);
      const uint32_t code = mx_code_from_amax_bits(amax);
      mx_codes |= code << (8 * db);
      const float inv = mx_inv_scale(code == 255u ? 127u : code);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mx_words[db][i] = code == 255u ? 0x7f7f7f7fu
                                       : mx_pack4(oacc[db][4 * i + 0] * inv_l * inv, oacc[db][4 * i + 1] * inv_l * inv,
                                                  oacc[db][4 * i + 2] * inv_l * inv, oacc[db][4 * i + 3] * inv_l * inv);
    }
  }
  if (qrow < Lq) {
    if (p.o) {
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
    }
    if (p.o_mx) {
      uint8_t* dst = p.o_mx + (q_start + qrow) * (int64_t)C + h * kD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(dst + 32 * db + 8 * i + 4 * hh) = mx_words[db][i];
      if (hh == 0) *reinterpret_cast<uint32_t*>(p.o_mx_scale + (q_start + qrow) * (int64_t)Cs + h * 4) = mx_codes;
    }
    if (hh == 0) p.lse[(int64_t)h * p.Tq + q_start + qrow] = l > 0.0f ? m * p.c + logf(l) : -INFINITY;
  }
}

}  // namespace

namespace mxfa {

hipError_t launch_attn_fwd(const AttnProblem& a, int p_dynamic, uint16_t* o, uint8_t* o_mx, uint8_t* o_mx_scale,
                           float* lse, hipStream_t stream) {
  FwdParams p;
  p.q = a.q.data; p.k = a.k.data; p.v = a.v.data;
  p.q_scale = a.q.scale; p.k_scale = a.k.scale; p.v_scale = a.v.scale;
  p.q_row_shift = a.q.mode == 0 ? 0 : 5;
  p.k_row_shift = a.k.mode == 0 ? 0 : 5;
  p.v_col_shift = a.v.mode == 1 ? 0 : 5;
  p.cu_q = a.cu_q; p.cu_k = a.cu_k;
  p.nseq = a.nseq; p.H = a.H;
  p.n_qtiles = (a.max_seqlen_q + kTile - 1) / kTile;
  p.total_items = (int)mx_pair_grid((int64_t)a.H * a.nseq, p.n_qtiles);  // < 2^31, checked by the caller
  p.c = a.softmax_scale;
  p.c2 = a.softmax_scale * kLog2e;
  p.causal = a.causal;
  p.o = o; p.o_mx = o_mx; p.o_mx_scale = o_mx_scale; p.lse = lse; p.Tq = a.total_q;
  if (p.total_items == 0) return hipSuccess;
  const dim3 grid((unsigned)p.total_items), block(256);
  // Q and K in MXFP4 (elem 1) or MXFP6 (elem 2): checked by the caller (both ROW32, V in E4M3)
  auto launch = [&](auto qkf) {
    constexpr int F = decltype(qkf)::value;
    if (p.v_col_shift == 0) {
      if (p_dynamic)
        hipLaunchKernelGGL((attn_fwd_kernel<true, true, F>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((attn_fwd_kernel<true, false, F>), grid, block, 0, stream, p);
    } else {
      if (p_dynamic)
        hipLaunchKernelGGL((attn_fwd_kernel<false, true, F>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((attn_fwd_kernel<false, false, F>), grid, block, 0, stream, p);
    }
  };
  if (a.q.elem == 1)
    launch(Stage<4>{});
  else if (a.q.elem == 2)
    launch(Stage<2>{});
  else
    launch(Stage<0>{});
  return hipGetLastError();
}

}  // namespace mxfa

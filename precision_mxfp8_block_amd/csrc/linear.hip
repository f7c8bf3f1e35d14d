// Fused projection GEMM + MX quantize producer for gfx950: Y = deq(X) deq(W)^T on scaled MFMA with
// FP32 accumulation, and an epilogue that quantizes Y in 32 x 32 square blocks and writes both
// scale layouts.
//
// What is computed (andresseo.expert "MXFP8 FlashAttention-4 Hits 2.85 Petaflops...", section
// "Inside the TMEM Bargain and Zero-Gather Jagged Pipeline": the quantization moves into the
// epilogue of the projection GEMM, so no separate pass over Y in global memory; brifing.si item 7:
// FP8 output with the scales in both layouts from one pass):
//   X [T, C_in] E4M3 with SQ32 (or ROW32) scales, W [C_out, C_in] E4M3 with 1 x 32 scales along
//   C_in, Y = sum_k deq(X)_tk deq(W)_nk in FP32; per 32 x 32 block of Y (token blocks start at
//   sequence starts, a sequence's last block may be partial): code = clamp(expbits(amax) - 8, 0,
//   254), payload = E4M3_RNE_sat(Y 2^(127 - code)); scales [NB][C_out/32] and [C_out/32][NB].
//
// gfx950 design:
//  * Workgroup = 8 waves = 256 tokens of one sequence x 256 output columns (the L2 traffic of X and W
//    falls with the tile edge). Wave w owns token blocks 2 (w & 3), +1 and column blocks 4 (w >> 2)
//    .. +3, so each of its eight 32 x 32 accumulators is exactly one output scale block and the block
//    maximum is a wave-wide reduction.
//  * The product is computed transposed, Y^T = W X^T (A = W rows, B = X rows, both read from LDS
//    as 16-byte row pieces): the accumulator gives each lane one token and 4 x 4 consecutive
//    output columns, i.e. four 4-byte payload stores per block.
//  * X and W chunks of 256 x 128 bytes are double-buffered in LDS (128 KB; direct global -> LDS
//    loads, XOR-swizzled chunks) and fetched one chunk of C_in ahead; the E8M0 scales of the next
//    chunk are fetched into registers at the same time.
//  * Items are (sequence, token tile, column tile) with the column tile fastest, remapped so that
//    each XCD works on a contiguous item range: the column tiles of one token tile then share one
//    L2, which serves the X tile to all of them.
#include "mx_device.h"
#include "mxfa_internal.h"

namespace {

constexpr int kTok = 256;    // tokens per workgroup
constexpr int kCol = 256;    // output columns per workgroup
constexpr int kChunk = 128;  // bytes of C_in per LDS stage
constexpr int kLinWaves = 8;

struct LinearParams {
  const uint8_t* x;
  const uint8_t* x_scale;
  int x_row_shift;  // 5: SQ32 (a scale row per 32 tokens), 0: ROW32 (a scale row per token)
  const uint8_t* w;
  const uint8_t* w_scale;
  const int32_t* cu;
  int nseq, tiles_per_seq, n_coltiles, total_items;
  int C_in, C_out;
  uint8_t* data;
  uint8_t* scale;
  uint8_t* scale_t;
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = bid & 7, slot = bid >> 3;
  return x * per + (x < rem ? x : rem) + slot;
}

// The direct LDS loads are inline asm (mx_lds_dma16) and so is their wait: with the compiler's own
// direct-load builtin it waits for every outstanding load before the next LDS read, i.e. for the
// next chunk's prefetch before the current chunk's MFMAs.
template <int N>
struct IntC {
  static constexpr int value = N;
};

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Global -> LDS copy of a 256-row x 128-byte chunk (row stride ld bytes, `base` wave-uniform) into a
// swizzled LDS tile, four 1 KB pieces per wave; rows at or past `valid` re-fetch the last valid row
// (finite data, never stored).
__device__ __forceinline__ void issue_chunk_load(uint8_t* lds_tile, const uint8_t* base, int valid, int ld,
                                                 const int* trow, const int* tcol, int wave_s) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t off = (uint32_t)(min(trow[c], valid - 1) * ld + tcol[c]);
    mx_lds_dma16((MX_LDS void*)(lds_tile + (wave_s * 4 + c) * 1024), base, off);
  }
}

// Operand of a 32x32x64 MFMA from row `row` of a swizzled LDS tile, 64-byte step ds.
__device__ __forceinline__ mx_v8i lds_row_operand(const uint8_t* lds, int row, int ds, int hh) {
  const uint8_t* p = lds + row * kChunk;
  const int sw = lds_swz(row);
  uint4 lo = *reinterpret_cast<const uint4*>(p + 16 * ((4 * ds + hh) ^ sw));
  uint4 hi = *reinterpret_cast<const uint4*>(p + 16 * ((4 * ds + 2 + hh) ^ sw));
  return mx_v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Four floats -> four E4M3 bytes of x / sc (sc a power of two) with no saturation: for callers that
// know |x| / sc <= 448.
__device__ __forceinline__ uint32_t pack4_div(float a, float b, float c, float d, float sc) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, a), a, b, sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, sc, true);
  return __builtin_bit_cast(uint32_t, r);
}

__global__ void __launch_bounds__(64 * kLinWaves, 1) linear_quantize_kernel(LinearParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][kTok * kChunk];  // stage x (X, W)

  const int item = xcd_remap((int)blockIdx.x, p.total_items);
  const int ct = item % p.n_coltiles;
  const int tt = (item / p.n_coltiles) % p.tiles_per_seq;
  const int s = item / (p.n_coltiles * p.tiles_per_seq);
  const int64_t start = p.cu[s];
  const int L = p.cu[s + 1] - (int)start;
  const int t0 = tt * kTok;
  if (t0 >= L) return;  // uniform over the workgroup
  const int valid = min(kTok, L - t0);
  const int64_t br0 = seq_offsets(p.cu, s).blocks32 + (t0 >> 5);  // first 32-token block row
  const int64_t nb_total = p.scale_t ? seq_offsets(p.cu, p.nseq).blocks32 : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tq = wave_s & 3;   // token blocks 2 tq, 2 tq + 1 of the tile
  const int cq = wave_s >> 2;  // column blocks 4 cq .. 4 cq + 3 of the tile
  const int ldw = p.C_in;      // row stride of X and W in bytes
  const int lds_s = p.C_in >> 5;  // scale row length in bytes (both X and W)
  const int wrows = min(kCol, p.C_out - ct * kCol);  // 256, or 128 for a last half tile
  const bool col_live = 128 * cq < wrows;           // wave-uniform
  int trow[4], tcol[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int pc = (wave_s * 4 + c) * 64 + lane;
    trow[c] = pc >> 3;
    tcol[c] = 16 * ((pc & 7) ^ lds_swz(pc >> 3));
  }
  const uint8_t* xbase = (const uint8_t*)mx_uniform_ptr((void*)(p.x + (start + t0) * (int64_t)ldw));
  const uint8_t* wbase = (const uint8_t*)mx_uniform_ptr((void*)(p.w + (int64_t)ct * kCol * ldw));

  // Scale rows: X of the wave's two token blocks (SQ32) or the lane's tokens (ROW32), W rows of the
  // wave's four column blocks, all clamped into range (clamped rows are never stored).
  const uint32_t* xs_ptr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b0 = 64 * tq + 32 * i;
    const int64_t row = p.x_row_shift ? br0 + (min(b0, valid - 1) >> 5) : start + t0 + min(b0 + r, valid - 1);
    xs_ptr[i] = reinterpret_cast<const uint32_t*>(p.x_scale + row * lds_s);
  }
  const uint32_t* ws_ptr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ws_ptr[j] = reinterpret_cast<const uint32_t*>(
        p.w_scale + ((int64_t)ct * kCol + min(128 * cq + 32 * j + r, wrows - 1)) * lds_s);

  const int nchunks = p.C_in / kChunk;
  uint32_t xsc[2], wsc[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) xsc[i] = xs_ptr[i][0];
#pragma unroll
  for (int j = 0; j < 4; ++j) wsc[j] = ws_ptr[j][0];
  issue_chunk_load(lds[0][0], xbase, valid, ldw, trow, tcol, wave_s);
  issue_chunk_load(lds[0][1], wbase, wrows, ldw, trow, tcol, wave_s);
  wait_vm();
#pragma unroll
  for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(xsc[i]));  // loaded: see the loop's wait below
#pragma unroll
  for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(wsc[j]));
  __syncthreads();

  // acc[i][j]: Y^T block of column block 4 cq + j and token block 2 tq + i (A = W rows, B = X rows)
  mx_v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mx_v16f{};

  for (int c = 0; c < nchunks; ++c) {
    const int st = c & 1;
    uint32_t xsn[2] = {0, 0}, wsn[4] = {0, 0, 0, 0};
    if (c + 1 < nchunks) {
#pragma unroll
      for (int i = 0; i < 2; ++i) xsn[i] = xs_ptr[i][c + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) wsn[j] = ws_ptr[j][c + 1];
      issue_chunk_load(lds[st ^ 1][0], (const uint8_t*)mx_uniform_ptr((void*)(xbase + (c + 1) * kChunk)), valid, ldw,
                       trow, tcol, wave_s);
      issue_chunk_load(lds[st ^ 1][1], (const uint8_t*)mx_uniform_ptr((void*)(wbase + (c + 1) * kChunk)), wrows, ldw,
                       trow, tcol, wave_s);
    }
    // Operands are read from LDS two MFMA steps ahead of their use (a step = one W operand times
    // both X operands, 2 MFMAs); the X operands of the second 64-byte half are read during the
    // first half. The scheduling groups keep that order: LDS latency stays behind MFMA work.
    const uint8_t* lx = lds[st][0];
    const uint8_t* lw = lds[st][1];
    mx_v8i xb[2][2], wa[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) xb[0][i] = lds_row_operand(lx, 64 * tq + 32 * i + r, 0, hh);
    wa[0] = lds_row_operand(lw, 128 * cq + r, 0, hh);
    wa[1] = lds_row_operand(lw, 128 * cq + 32 + r, 0, hh);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
    auto step = [&](auto S_) {
      constexpr int s = decltype(S_)::value;
      constexpr int ds = s >> 2, j = s & 3;
      constexpr int nreads = (s + 2 < 8 ? 2 : 0) + (s == 2 ? 4 : 0);
      if constexpr (s + 2 < 8) wa[s + 2] = lds_row_operand(lw, 128 * cq + 32 * ((s + 2) & 3) + r, (s + 2) >> 2, hh);
      if constexpr (s == 2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) xb[1][i] = lds_row_operand(lx, 64 * tq + 32 * i + r, 1, hh);
      }
      const uint32_t ws_l = wsc[j] >> (8 * hh);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t xs_l = xsc[i] >> (8 * hh);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa[s], xb[ds][i], acc[i][j], 0, 0, 2 * ds, (int)ws_l,
                                                                    2 * ds, (int)xs_l);
      }
      if constexpr (nreads > 0) __builtin_amdgcn_sched_group_barrier(0x100, nreads, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    };
    step(IntC<0>{});
    step(IntC<1>{});
    step(IntC<2>{});
    step(IntC<3>{});
    step(IntC<4>{});
    step(IntC<5>{});
    step(IntC<6>{});
    step(IntC<7>{});
    wait_vm();
    // The next chunk's scale words were loaded before the direct loads above; their first use is
    // pinned here, after the wait. Otherwise the compiler places its own wait for them among this
    // chunk's MFMAs, and because the hardware counter retires in order, that wait also waits for
    // the direct loads of the next chunk.
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(xsn[i]));
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(wsn[j]));
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) xsc[i] = xsn[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) wsc[j] = wsn[j];
  }

  // ---- epilogue: one 32 x 32 output block per accumulator ----
  // The payload goes through LDS (the chunk buffers are free after the loop's last barrier): a
  // lane's accumulator holds 4-byte pieces of 32 different token rows, which as direct stores would
  // be partial-line writes; staged as a 256-token x 256-byte tile (16-byte pieces XOR-swizzled by
  // row) it leaves as whole 256-byte row segments, 16 bytes per lane.
  uint8_t* stage = &lds[0][0][0];
  const int ncs = p.C_out >> 5;
  if (col_live) {  // wave-uniform
    // Rows past the sequence end hold finite values (their X rows re-read the last valid row): they
    // are converted and staged like the others but take no part in the block maximum and are never
    // stored, so the block loop has no lane-dependent branches.
    const bool live0 = 64 * tq + r < valid, live1 = 64 * tq + 32 + r < valid;
    // |y| maximum of each lane's 16 values per block, on the bit patterns: the unsigned maximum is
    // led by the negative value of largest magnitude (if any), the signed one by the largest
    // positive value. v[4 i + j] = block (i, j).
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t mu = 0;
        int32_t mi = 0;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const uint32_t b0 = __float_as_uint(acc[i][j][e]), b1 = __float_as_uint(acc[i][j][e + 1]);
          mu = max(max(mu, b0), b1);
          mi = max(max(mi, (int32_t)b0), (int32_t)b1);
        }
        v[4 * i + j] = (i ? live1 : live0) ? max(mu & 0x7fffffffu, (uint32_t)mi) : 0u;
      }
    // The eight wave-wide maxima in one pass: swapping lane halves pairs block k (lanes 0-31) with
    // block k + 4 (lanes 32-63) in one register, swapping 16-lane rows then packs four blocks per
    // register (v[0]: blocks 0, 1, 4, 5 in rows 0-3; v[2]: blocks 2, 3, 6, 7), and four DPP steps
    // finish each row.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      auto sw = __builtin_amdgcn_permlane32_swap(v[k], v[k + 4], false, false);
      v[k] = max((uint32_t)sw[0], (uint32_t)sw[1]);
    }
#pragma unroll
    for (int k = 0; k < 4; k += 2) {
      auto sw = __builtin_amdgcn_permlane16_swap(v[k], v[k + 1], false, false);
      uint32_t x = max((uint32_t)sw[0], (uint32_t)sw[1]);
      x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
      x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
      x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
      v[k] = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x140, 0xF, 0xF, false));  // row_mirror
    }
    uint32_t amax[8];  // wave-uniform
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int reg = (k & 2) ? 2 : 0;                    // blocks 2, 3, 6, 7 in v[2]
      const int row = (k & 1) | ((k >> 1) & 2);           // row of block k inside its register
      amax[k] = __builtin_amdgcn_readlane(v[reg], 16 * row);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int trow_l = 64 * tq + 32 * i + r;
      uint8_t* srow = stage + trow_l * kCol;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t m = amax[4 * i + j];
        const uint32_t code = mx_code_from_amax_bits(m);
        const mx_v16f& y = acc[i][j];
        uint32_t words[4];
        if (code == 255u) {  // scalar branches from here on
#pragma unroll
          for (int q = 0; q < 4; ++q) words[q] = 0x7f7f7f7fu;
        } else if (code >= 8u) {
          // y / 2^(code - 127) in the converter; no clamp is needed when the block maximum's
          // mantissa is at most 1.75 (then |y| / 2^(code - 127) <= 448)
          const float sc = __uint_as_float(code << 23);
          if ((m & 0x7fffffu) <= 0x600000u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) words[q] = pack4_div(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3], sc);
          } else {
            const float lim = __uint_as_float(((code + 8u) << 23) | 0x600000u);  // 448 sc
#pragma unroll
            for (int q = 0; q < 4; ++q)
              words[q] = mx_pack4_scaled(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3], sc, lim);
          }
        } else {
          const float inv = mx_inv_scale(code);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            words[q] = mx_pack4(y[4 * q] * inv, y[4 * q + 1] * inv, y[4 * q + 2] * inv, y[4 * q + 3] * inv);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cb = 128 * cq + 32 * j + 8 * q + 4 * hh;  // byte column inside the tile
          *reinterpret_cast<uint32_t*>(srow + (((cb >> 4) ^ (trow_l & 15)) << 4) + (cb & 15)) = words[q];
        }
      }
    }
    // lane k < 8 stores the code of block (k >> 2, k & 3) in both scale layouts
    uint32_t mine = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mine = lane == k ? mx_code_from_amax_bits(amax[k]) : mine;
    const int bi = (lane >> 2) & 1, bj = lane & 3;
    if (lane < 8 && 64 * tq + 32 * bi < valid) {
      const int64_t br = br0 + 2 * tq + bi;
      const int cb = (ct * kCol + 128 * cq) / 32 + bj;
      p.scale[br * ncs + cb] = (uint8_t)mine;
      if (p.scale_t) p.scale_t[(int64_t)cb * nb_total + br] = (uint8_t)mine;
    }
  }
  __syncthreads();
  const int kq = tid & 15;           // 16-byte piece of the row
  const bool kq_live = 16 * kq < wrows;
  uint8_t* dtile = p.data + (start + t0) * (int64_t)p.C_out + ct * kCol + 16 * kq;
#pragma unroll
  for (int pass = 0; pass < kTok / 32; ++pass) {
    const int row = pass * 32 + (tid >> 4);
    if (row < valid && kq_live)
      *reinterpret_cast<uint4*>(dtile + row * (int64_t)p.C_out) =
          *reinterpret_cast<const uint4*>(stage + row * kCol + ((kq ^ (row & 15)) << 4));
  }
}

}  // namespace

namespace mxfa {

hipError_t launch_linear_quantize(const MxOperand& x, const MxOperand& w, int64_t T, int C_in, int C_out,
                                  const int32_t* cu, int nseq, int max_seqlen, uint8_t* data,
                                  uint8_t* scale, uint8_t* scale_t, hipStream_t stream) {
  LinearParams p;
  p.x = x.data;
  p.x_scale = x.scale;
  p.x_row_shift = x.mode == 2 ? 5 : 0;
  p.w = w.data;
  p.w_scale = w.scale;
  p.cu = cu;
  p.nseq = nseq;
  p.tiles_per_seq = (max_seqlen + kTok - 1) / kTok;
  p.n_coltiles = (C_out + kCol - 1) / kCol;
  p.C_in = C_in;
  p.C_out = C_out;
  p.data = data;
  p.scale = scale;
  p.scale_t = scale_t;
  const int64_t items = (int64_t)nseq * p.tiles_per_seq * p.n_coltiles;
  if (T == 0 || items == 0) return hipSuccess;
  p.total_items = (int)items;
  hipLaunchKernelGGL(linear_quantize_kernel, dim3((unsigned)items), dim3(64 * kLinWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mxfa

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
constexpr int kHalf = 64;    // bytes of C_in per LDS stage
constexpr int kStages = 4;   // stages in the LDS ring (three loads in flight)
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

// The direct LDS loads are inline asm (mx_lds_dma16/4) and so are their waits and the stage
// barriers: the compiler's own direct-load builtin makes it wait for every outstanding load before
// the next LDS read, and its workgroup barrier waits for every outstanding load as well. The counts
// are exact per wave (see the issue order in the kernel); loads retire in order.
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Every wave's LDS reads so far have completed and its loads up to the last wait are visible.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
struct IntC {
  static constexpr int value = N;
};

// XOR swizzle of the 16-byte piece inside a 64-byte LDS row: the 16 rows that one 16-lane group of
// an operand read touches fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz64(int row) { return (row >> 2) & 3; }

// Global -> LDS copy of a 256-row x 64-byte stage tile (row stride ld bytes, `base` wave-uniform),
// two 1 KB pieces per wave; rows at or past `valid` re-fetch the last valid row (finite data, never
// stored). A dummy copy (every lane reads the first 16 bytes at `base`) keeps the number of loads per
// stage fixed past the end of C_in; its destination is a free stage.
__device__ __forceinline__ void issue_half_load(uint8_t* lds_tile, const uint8_t* base, int valid, int ld,
                                                const int* trow, const int* tcol, int wave_s, bool dummy) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t off = dummy ? 0u : (uint32_t)(min(trow[c], valid - 1) * ld + tcol[c]);
    mx_lds_dma16((MX_LDS void*)(lds_tile + (wave_s * 2 + c) * 1024), base, off);
  }
}

// Operand of a 32x32x64 MFMA from row `row` of a swizzled 64-byte-row stage tile: lanes 0-31 take
// bytes [0, 16) and [32, 48), lanes 32-63 bytes [16, 32) and [48, 64).
__device__ __forceinline__ mx_v8i stage_operand(const uint8_t* lds, int row, int hh) {
  const uint8_t* p = lds + row * kHalf;
  const int sw = swz64(row);
  uint4 lo = *reinterpret_cast<const uint4*>(p + 16 * (hh ^ sw));
  uint4 hi = *reinterpret_cast<const uint4*>(p + 16 * ((2 + hh) ^ sw));
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
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages][2][kTok * kHalf];  // stage x (X, W)
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[kStages][2 * 256 * 4];    // scale words: X, W

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
  int trow[2], tcol[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int pc = (wave_s * 2 + c) * 64 + lane;  // 16-byte piece of a 256 x 64-byte stage tile
    trow[c] = pc >> 2;
    tcol[c] = 16 * ((pc & 3) ^ swz64(pc >> 2));
  }
  const uint8_t* xbase = (const uint8_t*)mx_uniform_ptr((void*)(p.x + (start + t0) * (int64_t)ldw));
  const uint8_t* wbase = (const uint8_t*)mx_uniform_ptr((void*)(p.w + (int64_t)ct * kCol * ldw));

  // Scale words (4 codes = 128 bytes of C_in per row) reach LDS the same way as the payload: wave w
  // copies 64 entries of the X part (w < 4) or W part (w >= 4) of a 2 KB ring slot per chunk. X
  // entries are token rows (ROW32) or 32-token block rows (SQ32); rows are clamped into range
  // (clamped rows are never stored).
  const uint8_t* sbase;
  uint32_t soff;
  {
    const int e = 64 * (wave_s & 3) + lane;
    if (wave_s < 4) {
      const int64_t row0 = p.x_row_shift ? br0 : start + t0;
      sbase = p.x_scale + row0 * lds_s;
      soff = (uint32_t)((p.x_row_shift ? min(e, (valid - 1) >> 5) : min(e, valid - 1)) * lds_s);
    } else {
      sbase = p.w_scale + (int64_t)ct * kCol * lds_s;
      soff = (uint32_t)(min(e, wrows - 1) * lds_s);
    }
    sbase = (const uint8_t*)mx_uniform_ptr((void*)sbase);
  }
  const int nchunks = p.C_in >> 7;  // 128-byte chunks, two 64-byte stages each
  const int nh = 2 * nchunks;
  // Stage h of the ring holds C_in bytes [64 h, 64 h + 64) of the tile's X and W rows. Every wave
  // issues, in this order: scale(0), stage 0, stage 1, scale(1), stage 2, then per chunk c stage
  // 2c + 3 at its first barrier and scale(c + 2), stage 2c + 4 at its second. A stage is 4 direct
  // loads per wave and a scale slot 1; past the end of C_in they are dummies, so every wait below
  // leaves exactly 9 loads in flight and the loop body has no branches (the compiler could
  // otherwise sink MFMAs past a wait).
  auto issue_stage = [&](int h) {
    const int sl = h & (kStages - 1);
    const bool dummy = h >= nh;
    const int hc = dummy ? 0 : h;
    issue_half_load(lds[sl][0], (const uint8_t*)mx_uniform_ptr((void*)(xbase + hc * kHalf)), valid, ldw, trow, tcol,
                    wave_s, dummy);
    issue_half_load(lds[sl][1], (const uint8_t*)mx_uniform_ptr((void*)(wbase + hc * kHalf)), wrows, ldw, trow, tcol,
                    wave_s, dummy);
  };
  auto issue_scales = [&](int c) {
    mx_lds_dma4((MX_LDS void*)(lds_sc[c & (kStages - 1)] + 256 * wave_s), sbase,
                soff + 4u * (uint32_t)min(c, nchunks - 1));
  };
  issue_scales(0);
  issue_stage(0);
  issue_stage(1);
  issue_scales(1);
  issue_stage(2);

  // acc[i][j]: Y^T block of column block 4 cq + j and token block 2 tq + i (A = W rows, B = X rows)
  mx_v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mx_v16f{};

  // MFMAs of one stage: operands read from LDS, X rows of the wave's two token blocks, W rows of its
  // four column blocks; the scale codes of the stage's two 32-element K blocks are bytes 2 HF and
  // 2 HF + 1 of the chunk's scale words (selected per lane half, then by op_sel).
  auto stage_mfma = [&](auto HF_, int h, const uint32_t (&xsc)[2], const uint32_t (&wsc)[4]) {
    constexpr int hf = decltype(HF_)::value;
    const uint8_t* lx = lds[h & (kStages - 1)][0];
    const uint8_t* lw = lds[h & (kStages - 1)][1];
    mx_v8i xb[2], wa[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) xb[i] = stage_operand(lx, 64 * tq + 32 * i + r, hh);
#pragma unroll
    for (int j = 0; j < 4; ++j) wa[j] = stage_operand(lw, 128 * cq + 32 * j + r, hh);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ws_l = wsc[j] >> (8 * hh);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t xs_l = xsc[i] >> (8 * hh);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa[j], xb[i], acc[i][j], 0, 0, 2 * hf, (int)ws_l,
                                                                    2 * hf, (int)xs_l);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the stage's MFMAs are issued before the next wait
  };

  for (int c = 0; c < nchunks; ++c) {
    // stage 2c and scale(c) have landed (in flight behind them: stage 2c+1, scale(c+1), stage 2c+2)
    wait_vm_n<9>();
    stage_barrier();
    issue_stage(2 * c + 3);  // into the stage every wave finished reading before the barrier
    uint32_t xsc[2], wsc[4];
    {
      const uint32_t* sx = reinterpret_cast<const uint32_t*>(lds_sc[c & (kStages - 1)]);
#pragma unroll
      for (int i = 0; i < 2; ++i) xsc[i] = sx[p.x_row_shift ? 2 * tq + i : 64 * tq + 32 * i + r];
#pragma unroll
      for (int j = 0; j < 4; ++j) wsc[j] = sx[256 + 128 * cq + 32 * j + r];
    }
    stage_mfma(IntC<0>{}, 2 * c, xsc, wsc);
    // stage 2c+1 has landed (behind it: scale(c+1), stage 2c+2, stage 2c+3)
    wait_vm_n<9>();
    stage_barrier();
    issue_scales(c + 2);
    issue_stage(2 * c + 4);
    stage_mfma(IntC<1>{}, 2 * c + 1, xsc, wsc);
  }
  // the trailing dummy loads land before the epilogue reuses the ring
  wait_vm_n<0>();
  stage_barrier();

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

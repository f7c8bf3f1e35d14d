// Backward of the producers for gfx950: the projection's weight gradient dW = dY^T X (a contraction
// over tokens, fed by the transposed scale layout the producers write), the RMSNorm backward, and
// the ordered reduction of FP32 partials both use. The projection's data gradient dX = dY W is the
// projection kernel itself (linear.hip) with W^T as its weight and a bf16 epilogue.
//
// What is computed (brifing.si item 7: the producers write FP8 with the scale grid in two layouts,
// [NB][C/32] and its transpose [C/32][NB]; andresseo.expert "MXFP8 FlashAttention-4 Hits 2.85
// Petaflops...", section "Inside the TMEM Bargain and Zero-Gather Jagged Pipeline": square 32 x 32
// blocks let one payload serve the plain and the transposed product):
//   dW[o, i] = sum over every token t of every sequence of deq(dY)[t, o] deq(X)[t, i], FP32, where a
//   token block of 32 (from its sequence start) and a channel block of 32 share one E8M0 code, read
//   from [C/32][NB] so that the codes along the contraction (the token blocks) are contiguous;
//   dx = r gamma dy - x r^3 (sum_c gamma_c dy_c x_c) / C and dgamma = sum_t dy x r for the RMSNorm
//   y = x r gamma, r = 1 / sqrt(mean x^2 + eps), the quantizers passed straight through.
//
// gfx950 design of the weight gradient:
//  * Workgroup = 8 waves = a 256 (o) x 256 (i) tile of dW over one chunk of consecutive token
//    blocks; wave w owns o blocks 2 (w & 3), +1 and i blocks 4 (w >> 2) .. +3 (eight 32 x 32 FP32
//    accumulators). The chunks' partial tiles go to a workspace and one ordered pass adds them.
//  * A K step is two token blocks (64 token rows, one scaled 32x32x64 MFMA contraction, one E8M0
//    code per block). dY and X rows of the step land in LDS as [64 rows][128 B] half tiles (XOR-
//    swizzled 16-byte chunks) by direct global -> LDS loads, four slots of 32 KB, three steps in
//    flight; both operands are read transposed (ds_read_b64_tr_b8), which hands each lane 32 token
//    rows of one channel in the same order for A and B.
//  * Token blocks shorter than 32 rows (a sequence's last block) and the missing second block of an
//    odd chunk are zero-filled in LDS by the waves that loaded them, after their loads land and
//    before the step's barrier; their loads re-read the block's last row (always in bounds).
//  * The chunk's codes (16 channel blocks x up to 256 token blocks) are copied to LDS once, before
//    the first direct load is issued.
//  * The (o, i) tiles of one chunk are consecutive workgroups on one XCD (mx_pair_item), so the
//    chunk's dY and X rows come from that XCD's L2 after the first tile reads them.
#include <algorithm>

#include "mx_device.h"
#include "mxfa_internal.h"

namespace {

constexpr int kWgTile = 256;    // o and i extent of a workgroup's dW tile
constexpr int kWgWaves = 8;
constexpr int kWgSlots = 4;     // LDS ring slots (K steps)
constexpr int kWgMaxChunk = 256;  // token blocks per chunk, at most
constexpr int kRmsWaves = 8;
constexpr int kRmsMaxC = 2048;  // widest row of the RMSNorm backward

template <int N>
__device__ __forceinline__ void wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void step_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------------------------
// Token block table: for every compact token block b (32 tokens from its sequence start, the last
// one possibly shorter), its first token and its length. One thread per (sequence, block).
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) block_table_kernel(const int32_t* __restrict__ cu, int nseq, int max_blocks,
                                                          int2* __restrict__ table) {
  const int s = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int start = cu[s], L = cu[s + 1] - start;
  const SeqOffsets off = seq_offsets(cu, s);  // every wave computes it, all lanes active
  if (j * 32 >= L || j >= max_blocks) return;
  table[off.blocks32 + j] = make_int2(start + 32 * j, min(32, L - 32 * j));
}

// ---------------------------------------------------------------------------------------------
// Ordered sums of FP32 partial arrays: group g = blockIdx.y adds parts g * per_group .. (g + 1) *
// per_group - 1 (k ascending): out[g * n + e] = sum_k part[k * n + e]. One group gives the total;
// many partials are summed in two passes (groups, then the group sums) so that no thread walks a long
// chain of dependent loads.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sum_parts_kernel(const float* __restrict__ part, int n_parts, int per_group,
                                                        int64_t n, float* __restrict__ out) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  const int k0 = blockIdx.y * per_group, k1 = min(n_parts, k0 + per_group);
  float4 acc = *reinterpret_cast<const float4*>(part + (int64_t)k0 * n + e);
  for (int k = k0 + 1; k < k1; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)k * n + e);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(out + (int64_t)blockIdx.y * n + e) = acc;
}

// ---------------------------------------------------------------------------------------------
// Weight gradient
// ---------------------------------------------------------------------------------------------
struct WgradParams {
  const uint8_t* dy;     // [T, C_out] E4M3
  const uint8_t* dy_st;  // [C_out/32][NB] E8M0
  const uint8_t* x;      // [T, C_in] E4M3
  const uint8_t* x_st;   // [C_in/32][NB] E8M0
  const int2* blocks;    // [NB] first token, length
  const int32_t* cu;
  int nseq, C_out, C_in;
  int n_otiles, n_itiles, chunks, chunk;  // chunk: token blocks per chunk (even)
  float* part;           // [chunks][C_out][C_in]
};

// Transposed MFMA operand from a [64 rows][128 B] swizzled LDS half tile: lane (column col0 + l % 32,
// hh) receives 16 rows in bytes 0-15 (token block 0 of the step) and the same 16 rows + 32 in bytes
// 16-31 (token block 1), the two lane halves covering all 32 rows of each block.
__device__ __forceinline__ mx_v8i tr_operand(const uint8_t* lds, int col0, int tr_row, int tr_col, int tr_swz) {
  mx_v2i part[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int row = 32 * (cc >> 1) + 16 * (cc & 1) + tr_row;
    const int col = col0 + tr_col;
    const int off = row * 128 + 16 * ((col >> 4) ^ tr_swz) + (col & 15);
    part[cc] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MX_LDS mx_v2i*)(lds + off));
  }
  return mx_v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
}

__global__ void __launch_bounds__(64 * kWgWaves, 1) wgrad_kernel(WgradParams p) {
  // slot: four [64][128] half tiles: dY o 0-127, dY o 128-255, X i 0-127, X i 128-255
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kWgSlots][4][64 * 128];
  __shared__ uint8_t lds_codes[16][kWgMaxChunk];  // rows 0-7: dY o blocks of the tile, 8-15: X i blocks
  __shared__ int2 lds_blk[kWgMaxChunk];

  const int tiles = p.n_otiles * p.n_itiles;
  const int item = mx_pair_item((int)blockIdx.x, tiles, p.chunks);
  if (item < 0) return;
  const int ch = item / tiles, tile = item - ch * tiles;
  const int ot = tile / p.n_itiles, it = tile - ot * p.n_itiles;
  const int o0 = ot * kWgTile, i0 = it * kWgTile;
  const int orows = min(kWgTile, p.C_out - o0), irows = min(kWgTile, p.C_in - i0);  // 256 or 128
  const int nb = (int)seq_offsets(p.cu, p.nseq).blocks32;  // token blocks of the batch
  const int b_lo = ch * p.chunk, nblk = min(p.chunk, nb - b_lo);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, hh = lane >> 5;
  const int ob = wave_s & 3;   // o blocks 2 ob, 2 ob + 1 of the tile
  const int iq = wave_s >> 2;  // i blocks 4 iq .. 4 iq + 3 of the tile
  float* out = p.part + (int64_t)ch * p.C_out * p.C_in;  // this chunk's partial dW

  if (nblk <= 0) {  // a chunk past the last token block (the grid is sized from a bound): zeros
    for (int e = tid; e < orows * (irows / 4); e += 64 * kWgWaves) {
      const int o = e / (irows / 4), i4 = e - o * (irows / 4);
      *reinterpret_cast<float4*>(out + (int64_t)(o0 + o) * p.C_in + i0 + 4 * i4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const int nsteps = (nblk + 1) >> 1;

  // chunk's block table and codes (plain loads, before any direct load is in flight)
  for (int k = tid; k < nblk; k += 64 * kWgWaves) lds_blk[k] = p.blocks[b_lo + k];
  for (int k = tid; k < 16 * kWgMaxChunk; k += 64 * kWgWaves) {
    const int row = k / kWgMaxChunk, j = k - row * kWgMaxChunk;
    uint8_t c = 0;
    if (j < nblk) {
      if (row < 8) {
        const int cb = (o0 >> 5) + min(row, (orows >> 5) - 1);
        c = p.dy_st[(int64_t)cb * nb + b_lo + j];
      } else {
        const int cb = (i0 >> 5) + min(row - 8, (irows >> 5) - 1);
        c = p.x_st[(int64_t)cb * nb + b_lo + j];
      }
    }
    lds_codes[row][j] = c;
  }
  __syncthreads();

  // Direct loads of step k: wave w fills 1 KB pieces 4 w .. 4 w + 3 of the step's slot (piece q: half
  // tile q / 8, rows 8 (q % 8) .. + 7, lane l landing at row 8 (q % 8) + l / 8, physical 16-byte chunk
  // l % 8, so it fetches the logical chunk (l % 8) ^ swizzle(row)). Row j of a half tile is row j % 32
  // of token block 2 k + j / 32 of the chunk.
  const int lrow = lane >> 3;
  auto issue_step = [&](int k) {
    const int slot = k & (kWgSlots - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int q = 4 * wave_s + c;  // wave-uniform
      const int half = q >> 3;       // 0, 1: dY o halves; 2, 3: X i halves
      const int row = 8 * (q & 7) + lrow;
      const int2 bi = lds_blk[min(2 * k + (row >> 5), nblk - 1)];
      const int t = bi.x + min(row & 31, bi.y - 1);  // rows past a block's length re-read its last row
      const uint8_t* base;
      uint32_t ld;
      if (half < 2) {
        base = p.dy + min(o0 + 128 * half, p.C_out - 128);
        ld = (uint32_t)p.C_out;
      } else {
        base = p.x + min(i0 + 128 * (half - 2), p.C_in - 128);
        ld = (uint32_t)p.C_in;
      }
      const uint32_t voff = (uint32_t)t * ld + 16u * (uint32_t)((lane & 7) ^ lds_swz(row));
      mx_lds_dma16((MX_LDS void*)(&lds[slot][half][(q & 7) * 1024]), base, voff);
    }
  };
  // After its loads of step k have landed, a wave zeroes the rows of its pieces that lie past their
  // block's length (or belong to the missing second block of an odd chunk).
  auto zero_dead_rows = [&](int k) {
    const int slot = k & (kWgSlots - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int q = 4 * wave_s + c;
      const int row = 8 * (q & 7) + lrow;
      const int jb = 2 * k + (row >> 5);
      const bool dead = jb >= nblk || (row & 31) >= lds_blk[min(jb, nblk - 1)].y;
      if (dead) *reinterpret_cast<uint4*>(&lds[slot][q >> 3][(q & 7) * 1024 + 16 * lane]) = make_uint4(0, 0, 0, 0);
    }
  };
  // Per-lane constants of the transposed reads.
  const int grp = lane >> 4, gl = lane & 15;
  const int tb = gl >> 1, ts = gl & 1;
  const int tr_row = 8 * (tb >> 2) + 4 * (grp >> 1) + (tb & 3);
  const int tr_col = 16 * (grp & 1) + 8 * ts;
  const int tr_swz = lds_swz(tr_row);

  // acc[a][b]: dW block (o block 2 ob + a, i block 4 iq + b); lane: column i = r, rows
  // o = 8 (v / 4) + 4 hh + v % 4
  mx_v16f acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = mx_v16f{};

#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (k < nsteps) issue_step(k);
  for (int k = 0; k < nsteps; ++k) {
    // step k has landed (behind it: steps k + 1 and k + 2 when they exist, 4 loads each)
    if (k + 2 < nsteps)
      wait_vm_n<8>();
    else if (k + 1 < nsteps)
      wait_vm_n<4>();
    else
      wait_vm_n<0>();
    const bool partial = 2 * k + 1 >= nblk || lds_blk[2 * k].y < 32 || lds_blk[2 * k + 1].y < 32;  // uniform
    if (partial) zero_dead_rows(k);
    step_barrier();
    if (k + 3 < nsteps) issue_step(k + 3);  // into the slot of step k - 1, read before the barrier
    const int slot = k & (kWgSlots - 1);
    const int j0 = min(2 * k + hh, nblk - 1);  // the lane half's token block (scale operand)
    mx_v8i bop[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) bop[b] = tr_operand(lds[slot][2 + iq], 32 * b, tr_row, tr_col, tr_swz);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int oa = 2 * ob + a;
      const mx_v8i aop = tr_operand(lds[slot][oa >> 2], 32 * (oa & 3), tr_row, tr_col, tr_swz);
      const int sa = lds_codes[oa][j0];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[b], acc[a][b], 0, 0, 0, sa, 0,
                                                                    (int)lds_codes[8 + 4 * iq + b][j0]);
    }
    __builtin_amdgcn_sched_barrier(0);  // the step's MFMAs are issued before the next wait
  }

  // partial tile of this chunk: [chunk][o][i], 128-byte row segments per store
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int ol = 32 * (2 * ob + a);
    if (ol >= orows) continue;  // wave-uniform
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int il = 32 * (4 * iq + b);
      if (il >= irows) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int o = o0 + ol + 8 * (v >> 2) + 4 * hh + (v & 3);
        out[(int64_t)o * p.C_in + i0 + il + r] = acc[a][b][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// RMSNorm backward: one wave per token row (rows strided over all waves of the grid); lane l covers
// columns 8 l + 512 k (16-byte pieces of x and dy), K = ceil(C / 512) <= 4 pieces per lane (C <= 2048). r is
// recomputed as the forward computes it (FP64 sum of squares, one fp32 rounding, 1 / sqrt in fp32);
// each wave accumulates its rows' dy x r per column; the workgroup adds its 8 waves' sums in wave order
// (through LDS) and writes one partial row for the ordered reduction.
// ---------------------------------------------------------------------------------------------
template <int K>
__global__ void __launch_bounds__(64 * kRmsWaves) rmsnorm_bwd_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                                  int64_t T, int C, const float* __restrict__ gamma,
                                                                  float eps, const uint16_t* __restrict__ dy,
                                                                  uint16_t* __restrict__ dx, float* __restrict__ dg_part) {
  __shared__ float lds_dg[kRmsWaves][kRmsMaxC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * kRmsWaves + wave;
  const int64_t nw = (int64_t)gridDim.x * kRmsWaves;
  float g[K][8], dgacc[K][8];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 512 * k + 8 * lane + e;
      g[k][e] = c < C ? gamma[c] : 0.0f;
      dgacc[k][e] = 0.0f;
    }
  for (int64_t t = gw; t < T; t += nw) {
    float xv[K][8], dyv[K][8];
    double ss = 0.0;
    float sd = 0.0f;  // sum of gamma dy x over the lane's columns
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int c0 = 512 * k + 8 * lane;
      uint4 xa = make_uint4(0, 0, 0, 0), da = make_uint4(0, 0, 0, 0);
      if (c0 < C) {
        xa = *reinterpret_cast<const uint4*>(x + t * ld_x + c0);
        da = *reinterpret_cast<const uint4*>(dy + t * (int64_t)C + c0);
      }
      const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w}, dw[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[k][2 * e] = bf16_to_f32(xw[e] & 0xffffu);
        xv[k][2 * e + 1] = bf16_to_f32(xw[e] >> 16);
        dyv[k][2 * e] = bf16_to_f32(dw[e] & 0xffffu);
        dyv[k][2 * e + 1] = bf16_to_f32(dw[e] >> 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss += (double)(xv[k][e] * xv[k][e]);  // squares of bf16 values are exact in fp32
        sd += g[k][e] * dyv[k][e] * xv[k][e];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      ss += __shfl_xor(ss, o, 64);
      sd += __shfl_xor(sd, o, 64);
    }
    const float rr = 1.0f / __fsqrt_rn((float)ss / (float)C + eps);
    const float coef = rr * rr * rr * sd / (float)C;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int c0 = 512 * k + 8 * lane;
      if (c0 >= C) continue;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = rr * g[k][2 * e] * dyv[k][2 * e] - xv[k][2 * e] * coef;
        const float d1 = rr * g[k][2 * e + 1] * dyv[k][2 * e + 1] - xv[k][2 * e + 1] * coef;
        w[e] = f32_to_bf16(d0) | (f32_to_bf16(d1) << 16);
      }
      *reinterpret_cast<uint4*>(dx + t * (int64_t)C + c0) = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) dgacc[k][e] += dyv[k][e] * xv[k][e] * rr;
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c0 = 512 * k + 8 * lane;
    if (c0 >= C) continue;
    float* dst = &lds_dg[wave][c0];
    *reinterpret_cast<float4*>(dst) = make_float4(dgacc[k][0], dgacc[k][1], dgacc[k][2], dgacc[k][3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(dgacc[k][4], dgacc[k][5], dgacc[k][6], dgacc[k][7]);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += 64 * kRmsWaves) {
    float v = lds_dg[0][c];
#pragma unroll
    for (int w = 1; w < kRmsWaves; ++w) v += lds_dg[w][c];
    dg_part[(int64_t)blockIdx.x * C + c] = v;
  }
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// Weight-gradient work split: chunks of an even number of token blocks (at most kWgMaxChunk), enough
// chunks that the (chunk, tile) items fill about one round of the chip.
struct WgradSplit {
  int chunk, chunks;
};
WgradSplit wgrad_split(int64_t nb, int tiles) {
  WgradSplit w;
  const int64_t want = std::max<int64_t>((nb + kWgMaxChunk - 1) / kWgMaxChunk, (256 + tiles - 1) / tiles);
  int64_t chunk = (nb + want - 1) / want;
  chunk = std::min<int64_t>(kWgMaxChunk, (chunk + 1) & ~(int64_t)1);
  w.chunk = (int)std::max<int64_t>(chunk, 2);
  w.chunks = (int)((nb + w.chunk - 1) / w.chunk);
  return w;
}

constexpr int kRmsGridMax = 2048;  // workgroups of the RMSNorm backward, at most

}  // namespace

namespace mxfa {

size_t wgrad_workspace_bytes(int64_t T, int nseq, int C_out, int C_in) {
  const int64_t nb = T / 32 + nseq;  // an upper bound on the token blocks
  const int tiles = ((C_out + kWgTile - 1) / kWgTile) * ((C_in + kWgTile - 1) / kWgTile);
  const WgradSplit w = wgrad_split(nb, tiles);
  const size_t table = ((size_t)nb * sizeof(int2) + 255) / 256 * 256;
  return table + (size_t)w.chunks * C_out * C_in * sizeof(float);
}

hipError_t launch_linear_wgrad(const uint8_t* dy, const uint8_t* dy_st, const uint8_t* x, const uint8_t* x_st,
                               int64_t T, int C_out, int C_in, const int32_t* cu, int nseq, int max_seqlen,
                               void* workspace, float* dw, hipStream_t stream) {
  if (T == 0) return hipMemsetAsync(dw, 0, (size_t)C_out * C_in * sizeof(float), stream);  // no tokens: dW = 0
  const int64_t nb = T / 32 + nseq;  // a bound on the token blocks; the kernel finds the exact count
  const int n_ot = (C_out + kWgTile - 1) / kWgTile, n_it = (C_in + kWgTile - 1) / kWgTile;
  const WgradSplit w = wgrad_split(nb, n_ot * n_it);
  int2* table = (int2*)workspace;
  const size_t table_bytes = ((size_t)(T / 32 + nseq) * sizeof(int2) + 255) / 256 * 256;
  float* part = (float*)((uint8_t*)workspace + table_bytes);
  const int mb = (max_seqlen + 31) / 32;
  hipLaunchKernelGGL(block_table_kernel, dim3((unsigned)((mb + 255) / 256), (unsigned)nseq), dim3(256), 0, stream, cu,
                     nseq, mb, table);
  WgradParams p;
  p.dy = dy;
  p.dy_st = dy_st;
  p.x = x;
  p.x_st = x_st;
  p.blocks = table;
  p.cu = cu;
  p.nseq = nseq;
  p.C_out = C_out;
  p.C_in = C_in;
  p.n_otiles = n_ot;
  p.n_itiles = n_it;
  p.chunks = w.chunks;
  p.chunk = w.chunk;
  p.part = part;
  const int64_t grid = mx_pair_grid(w.chunks, n_ot * n_it);
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)grid), dim3(64 * kWgWaves), 0, stream, p);
  const int64_t n = (int64_t)C_out * C_in;
  hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, part, w.chunks,
                     w.chunks, n, dw);
  return hipGetLastError();
}

static int rms_grid(int64_t T) {
  const int64_t rows_per_round = (int64_t)cu_count() * 2 * kRmsWaves;  // two workgroups per CU
  const int64_t waves = std::min<int64_t>(T, rows_per_round);
  return (int)std::max<int64_t>(1, std::min<int64_t>(kRmsGridMax, (waves + kRmsWaves - 1) / kRmsWaves));
}

constexpr int kRmsPerGroup = 32;  // partial rows per group of the first reduction pass

size_t rmsnorm_bwd_workspace_bytes(int64_t T, int C) {
  (void)T;
  const size_t parts = kRmsGridMax;
  return (parts + (parts + kRmsPerGroup - 1) / kRmsPerGroup) * C * sizeof(float);
}

hipError_t launch_rmsnorm_bwd(const uint16_t* x, int64_t ld_x, int64_t T, int C, const float* gamma, float eps,
                              const uint16_t* dy, void* workspace, uint16_t* dx, float* dgamma, hipStream_t stream) {
  if (T == 0) return hipMemsetAsync(dgamma, 0, (size_t)C * sizeof(float), stream);
  const int grid = rms_grid(T);
  float* part = (float*)workspace;
  const int K = (C + 511) / 512;
  if (K <= 1)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<1>, dim3(grid), dim3(64 * kRmsWaves), 0, stream, x, ld_x, T, C, gamma, eps, dy,
                       dx, part);
  else if (K <= 2)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<2>, dim3(grid), dim3(64 * kRmsWaves), 0, stream, x, ld_x, T, C, gamma, eps, dy,
                       dx, part);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<4>, dim3(grid), dim3(64 * kRmsWaves), 0, stream, x, ld_x, T, C, gamma, eps, dy,
                       dx, part);
  // per-workgroup partial rows -> group sums -> dgamma, each in ascending order
  const int parts = grid, groups = (parts + kRmsPerGroup - 1) / kRmsPerGroup;
  float* level2 = part + (int64_t)kRmsGridMax * C;
  const unsigned cblocks = (unsigned)(((int64_t)C / 4 + 255) / 256);
  hipLaunchKernelGGL(sum_parts_kernel, dim3(cblocks, (unsigned)groups), dim3(256), 0, stream, part, parts, kRmsPerGroup,
                     (int64_t)C, level2);
  hipLaunchKernelGGL(sum_parts_kernel, dim3(cblocks, 1), dim3(256), 0, stream, level2, groups, groups, (int64_t)C,
                     dgamma);
  return hipGetLastError();
}

}  // namespace mxfa

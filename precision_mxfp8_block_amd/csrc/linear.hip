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
//  * Item = 256 tokens of one sequence x 256 output columns, computed by a workgroup of 8 waves (the
//    L2 traffic of X and W falls with the tile edge). Wave w owns token blocks 2 (w & 3), +1 and
//    column blocks 4 (w >> 2) .. +3, so each of its eight 32 x 32 accumulators is exactly one output
//    scale block and the block maximum is a wave-wide reduction.
//  * The product is computed transposed, Y^T = W X^T (A = W rows, B = X rows, both read from LDS
//    as 16-byte row pieces): the accumulator gives each lane one token and 4 x 4 consecutive
//    output columns, i.e. four 4-byte payload stores per block.
//  * X and W reach LDS in stages of 256 rows x 64 bytes of C_in through a four-slot ring (128 KB;
//    direct global -> LDS loads, 16-byte pieces XOR-swizzled by row) with three stages in flight; the
//    E8M0 scale words of each 128-byte chunk of C_in travel the same way through a four-slot ring.
//  * Persistent: one workgroup per compute unit runs a list of items. The non-empty token tiles are
//    dealt to the XCDs in turn and an XCD's (token tile, column tile) items to its workgroups in
//    turn, so a jagged batch loads every compute unit to within one item, and the column tiles of
//    a token tile run together on one XCD, whose L2 serves them its X tile. The loads of the next
//    item's first stages are issued during the current item's last chunk and overlap its epilogue.
#include <algorithm>

#include "mx_device.h"
#include "mxfa_internal.h"

namespace {

constexpr int kTok = 256;     // tokens per item
constexpr int kCol = 256;     // output columns per item
constexpr int kHalf = 64;     // bytes of C_in per LDS stage
constexpr int kStages = 4;    // slots of the LDS ring
constexpr int kLinWaves = 8;  // two waves per SIMD, each 64 tokens x 128 columns of the item
constexpr int kListCap = 16;  // work items of a workgroup held in LDS at a time

struct LinearParams {
  const uint8_t* x;
  const uint8_t* x_scale;
  int x_row_shift;  // 5: SQ32 (a scale row per 32 tokens), 0: ROW32 (a scale row per token)
  const uint8_t* w;
  const uint8_t* w_scale;
  const int32_t* cu;
  int nseq, n_coltiles;
  int C_in, C_out;
  uint8_t* data;
  uint8_t* scale;
  uint8_t* scale_t;
  uint16_t* out_bf16;  // set: Y is written as bf16 [T, C_out] instead of quantized
  int accumulate;      // with out_bf16: Y is added to the bf16 values already there (FP32 add)
};

// The direct LDS loads are inline asm (mx_lds_dma16/4) and so are their waits and the stage
// barriers: the compiler's own direct-load builtin makes it wait for every outstanding load before
// the next LDS read, and its workgroup barrier waits for every outstanding load as well. The counts
// are exact per wave (see the issue order in the kernel); loads retire in order.
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most n (wave-uniform) of this wave's vector memory operations are outstanding, n
// rounded down to a count the loop uses (waiting for more is always safe).
__device__ __forceinline__ void wait_vm_var(int n) {
  if (n >= 9)
    wait_vm_n<9>();
  else if (n >= 5)
    wait_vm_n<5>();
  else if (n >= 4)
    wait_vm_n<4>();
  else
    wait_vm_n<0>();
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

// Global -> LDS copy of this wave's eighth of a 256-row x 64-byte stage tile (row stride ld bytes,
// `base` wave-uniform): two 1 KB pieces, piece c covering rows 16 (2 wave + c) .. + 15; rows at or
// past `valid` re-fetch the last valid row (finite data, never stored).
__device__ __forceinline__ void issue_stage_tile(uint8_t* lds_tile, const uint8_t* base, int valid, int ld, int wave_s,
                                                 int lane) {
  const int tcol = 16 * ((lane & 3) ^ ((lane >> 4) & 3));
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int trow = 16 * (2 * wave_s + c) + (lane >> 2);
    const uint32_t off = (uint32_t)(min(trow, valid - 1) * ld + tcol);
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

// maximum(m, |a|, |b|) with NaN propagation (one v_maximum3_f32 with absolute-value modifiers).
__device__ __forceinline__ float abs_maximum3(float m, float a, float b) {
  return __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(fabsf(a), fabsf(b)));
}

// Four floats -> four E4M3 bytes of x / sc (sc a power of two) with no saturation: for callers that
// know |x| / sc <= 448.
__device__ __forceinline__ uint32_t pack4_div(float a, float b, float c, float d, float sc) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, a), a, b, sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, sc, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Wave-wide maxima of eight per-lane values v[0..7] (bit patterns of non-negative floats), every
// lane receiving all eight. Swapping lane halves pairs value k (lanes 0-31) with value k + 4 (lanes
// 32-63) in one register, swapping 16-lane rows then packs four values per register (v[0]: 0, 1, 4,
// 5 in rows 0-3; v[2]: 2, 3, 6, 7), and four DPP steps finish each row.
__device__ __forceinline__ void wave_max8(uint32_t (&v)[8], uint32_t (&amax)[8]) {
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
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int reg = (k & 2) ? 2 : 0;           // values 2, 3, 6, 7 in v[2]
    const int row = (k & 1) | ((k >> 1) & 2);  // row of value k inside its register
    amax[k] = __builtin_amdgcn_readlane(v[reg], 16 * row);
  }
}

// Inclusive prefix sum over the 64 lanes of a fully active wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    v += lane >= d ? o : 0;
  }
  return v;
}

__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }
__device__ __forceinline__ int ceil_div(int a, int b) { return -floor_div(-a, b); }

// What issuing the loads of one work item (a 256-token tile of one sequence times a 256-column tile
// of the output) takes. All fields are wave-uniform except soff.
struct LinItem {
  const uint8_t* xbase;  // X row of the tile's first token
  const uint8_t* wbase;  // W row of the tile's first output column
  const uint8_t* sbase;  // this wave's scale source: X part (waves 0-3) or W part (waves 4-7)
  uint32_t soff;         // per lane: byte offset of the lane's scale row at chunk 0
  int valid, wrows;      // tokens (1..256) and output columns (256, or 128 in a last half tile)
};

// Where an item sits in the batch.
struct LinPlace {
  int ct;             // column tile
  int valid;          // tokens in the tile
  int64_t row0, br0;  // first token row, first 32-token block row (compact scale layout)
};

__global__ void __launch_bounds__(64 * kLinWaves, 1) linear_quantize_kernel(LinearParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages][2][kTok * kHalf];  // slot x (X, W)
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[kStages][2 * 256 * 4];    // scale words: X, W
  __shared__ int lds_list[kListCap][4];  // work list: sequence start, length, token tile, blocks before
  __shared__ int lds_red[kLinWaves][2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tq = wave_s & 3;   // token blocks 2 tq, 2 tq + 1 of the item
  const int cq = wave_s >> 2;  // column blocks 4 cq .. 4 cq + 3 of the item
  const int ldw = p.C_in;      // row stride of X and W in bytes
  const int lds_s = p.C_in >> 5;    // scale row length in bytes (both X and W)
  const int nchunks = p.C_in >> 7;  // 128-byte chunks of C_in, two 64-byte stages each
  const int nh = 2 * nchunks;
  const int nct = p.n_coltiles;

  // ---- work list ----
  // Token tiles are numbered over the sequences in order (ceil(L / 256) per sequence) and dealt to
  // the XCDs in turn (tile j to XCD j mod 8; workgroup b runs on XCD b mod 8). An XCD's items are its
  // tiles' (tile, column tile) pairs in order, dealt to its workgroups in turn, so every workgroup
  // gets the same number of items to within one, and the column tiles of one token tile run at about
  // the same time on one XCD, whose L2 then serves that X tile to all of them. fill_list(n0) writes
  // this workgroup's items n0 .. n0 + kListCap - 1 to LDS (one pass over cu_seqlens, 512 sequences at
  // a time) and returns the item count; it has workgroup barriers, so every thread calls it.
  const int xcd = blockIdx.x & 7, wg = blockIdx.x >> 3, nwg = gridDim.x >> 3;
  int64_t nb_total = 0;  // 32-token blocks of the batch (rows of the transposed scale layout)
  auto fill_list = [&](int n0) -> int {
    int gbase = 0, bbase = 0;
    for (int s0 = 0; s0 < p.nseq; s0 += 64 * kLinWaves) {
      const int s = s0 + tid;
      int start = 0, L = 0;
      if (s < p.nseq) {
        start = p.cu[s];
        L = p.cu[s + 1] - start;
      }
      const int g = (L + kTok - 1) / kTok, b = (L + 31) >> 5;
      const int gi = wave_incl_scan(g), bi = wave_incl_scan(b);
      if (lane == 63) {
        lds_red[wave_s][0] = gi;
        lds_red[wave_s][1] = bi;
      }
      __syncthreads();
      int gpre = 0, bpre = 0, gtot = 0, btot = 0;
#pragma unroll
      for (int w = 0; w < kLinWaves; ++w) {
        const int gw = lds_red[w][0], bw = lds_red[w][1];
        gpre += w < wave_s ? gw : 0;
        bpre += w < wave_s ? bw : 0;
        gtot += gw;
        btot += bw;
      }
      __syncthreads();  // lds_red is free for the next pass
      if (g > 0) {
        const int G = gbase + gpre + gi - g;  // first token tile of sequence s
        const int B = bbase + bpre + bi - b;  // 32-token blocks before sequence s
        const int qlo = ceil_div(G - xcd, 8), qhi = floor_div(G + g - 1 - xcd, 8);  // the XCD's tiles in s
        if (qhi >= qlo) {
          const int nlo = max(ceil_div(qlo * nct - wg, nwg), n0);
          const int nhi = min(ceil_div((qhi + 1) * nct - wg, nwg), n0 + kListCap);
          for (int n = nlo; n < nhi; ++n) {
            const int j = ((wg + n * nwg) / nct) * 8 + xcd;
            lds_list[n - n0][0] = start;
            lds_list[n - n0][1] = L;
            lds_list[n - n0][2] = j - G;
            lds_list[n - n0][3] = B;
          }
        }
      }
      gbase += gtot;
      bbase += btot;
    }
    __syncthreads();
    nb_total = bbase;
    const int xtiles = gbase > xcd ? (gbase - xcd + 7) >> 3 : 0;
    const int nitems = xtiles * nct;  // items of this XCD
    return nitems > wg ? ceil_div(nitems - wg, nwg) : 0;
  };

  // Item n of this workgroup from the list (n0 <= n < n0 + kListCap).
  int n0 = 0;
  auto place = [&](int n) {
    LinPlace q;
    const int* e = lds_list[n - n0];
    const int start = __builtin_amdgcn_readfirstlane(e[0]);
    const int L = __builtin_amdgcn_readfirstlane(e[1]);
    const int t0 = __builtin_amdgcn_readfirstlane(e[2]) * kTok;
    const int B = __builtin_amdgcn_readfirstlane(e[3]);
    q.ct = (wg + n * nwg) % nct;
    q.valid = min(kTok, L - t0);
    q.row0 = (int64_t)start + t0;
    q.br0 = (int64_t)B + (t0 >> 5);
    return q;
  };
  // Scale words (4 codes = 128 bytes of C_in per row) reach LDS the same way as the payload: a 2 KB
  // ring slot per chunk holds 256 X entries then 256 W entries, wave w copying entries 64 w .. + 63
  // (one load). X entries are token rows (ROW32) or 32-token block rows (SQ32); rows are clamped
  // into range (clamped rows are never used for a stored value).
  auto make_item = [&](int n) {
    const LinPlace q = place(n);
    LinItem it;
    it.valid = q.valid;
    it.wrows = min(kCol, p.C_out - q.ct * kCol);
    it.xbase = (const uint8_t*)mx_uniform_ptr((void*)(p.x + q.row0 * ldw));
    it.wbase = (const uint8_t*)mx_uniform_ptr((void*)(p.w + (int64_t)q.ct * kCol * ldw));
    if (wave_s < 4) {
      const int64_t srow = p.x_row_shift ? q.br0 : q.row0;
      const int lim = p.x_row_shift ? (it.valid - 1) >> 5 : it.valid - 1;
      it.sbase = (const uint8_t*)mx_uniform_ptr((void*)(p.x_scale + srow * lds_s));
      it.soff = (uint32_t)(min(64 * wave_s + lane, lim) * lds_s);
    } else {
      it.sbase = (const uint8_t*)mx_uniform_ptr((void*)(p.w_scale + (int64_t)q.ct * kCol * lds_s));
      it.soff = (uint32_t)(min(64 * (wave_s - 4) + lane, it.wrows - 1) * lds_s);
    }
    return it;
  };

  const int count = fill_list(0);
  if (count == 0) return;  // uniform over the workgroup
  LinItem cur = make_item(0);

  // Stage g of an item (C_in bytes [64 g, 64 g + 64) of its X and W rows) goes to ring slot
  // (ss + g) & 3; an even stage is preceded by its scale chunk g / 2 (the E8M0 words of C_in bytes
  // [64 g, 64 g + 128)), which goes to scale slot (cs + g / 2) & 3. Step h of an item: wait until
  // stage h has landed, barrier, issue stage h + 3 into the slot of stage h - 1 (every wave read it
  // before the barrier), read stage h's operands and run its MFMAs: three stages are in flight while
  // one is used. With two chunks or more the stage stream runs on into the next item: its stages 0
  // and 1 are issued in steps nh - 3 and nh - 2, while its stage 2 waits until the epilogue has
  // finished with the two slots that stage the output. With one chunk each item starts from its own
  // prologue. A wait counts this wave's loads issued after the one it waits for (a stage is 4 direct
  // loads per wave, a scale chunk 1); loads land in issue order, and the epilogue's stores, issued
  // before some of them, can only delay a wait.
  const bool chain = nh >= 4;
  bool nxt_chain = chain && count > 1;  // the next item's first stages are issued in this item
  int ss = 0, cs = 0;
  auto issue = [&](const LinItem& it, int g, int sbase_slot, int cbase_slot) {
    if ((g & 1) == 0)
      mx_lds_dma4((MX_LDS void*)(lds_sc[(cbase_slot + (g >> 1)) & 3] + 256 * wave_s), it.sbase,
                  it.soff + 4u * (uint32_t)(g >> 1));
    const int slot = (sbase_slot + g) & 3;
    issue_stage_tile(lds[slot][0], (const uint8_t*)mx_uniform_ptr((void*)(it.xbase + g * kHalf)), it.valid, ldw,
                     wave_s, lane);
    issue_stage_tile(lds[slot][1], (const uint8_t*)mx_uniform_ptr((void*)(it.wbase + g * kHalf)), it.wrows, ldw,
                     wave_s, lane);
  };
  // this wave's loads for stage g (g >= nh: of the next item) issued before the item's epilogue
  auto loads_of = [&](int g) -> int {
    const bool issued = g < nh || (nxt_chain && g < nh + 2);
    return issued ? ((g & 1) ? 4 : 5) : 0;
  };

  // acc[i][j]: Y^T block of column block 4 cq + j and token block 2 tq + i (A = W rows, B = X rows)
  mx_v16f acc[2][4];
  // MFMAs of stage g: operands read from LDS, X rows of the wave's two token blocks, W rows of its
  // four column blocks; the scale codes of the stage's two 32-element K blocks are bytes 2 HF and
  // 2 HF + 1 of the chunk's scale words (selected per lane half, then by op_sel).
  auto stage_step = [&](auto HF_, int g, const uint32_t (&xsc)[2], const uint32_t (&wsc)[4]) {
    constexpr int hf = decltype(HF_)::value;
    const int slot = (ss + g) & 3;
    mx_v8i xb[2], wa[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) xb[i] = stage_operand(lds[slot][0], 64 * tq + 32 * i + r, hh);
#pragma unroll
    for (int j = 0; j < 4; ++j) wa[j] = stage_operand(lds[slot][1], 128 * cq + 32 * j + r, hh);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa[j], xb[i], acc[i][j], 0, 0, 2 * hf,
                                                                    (int)wsc[j], 2 * hf, (int)xsc[i]);
    __builtin_amdgcn_sched_barrier(0);  // the stage's MFMAs are issued before the next wait
  };

  auto prologue = [&]() {  // the item's stages 0 .. 2 (those it has)
#pragma unroll
    for (int g = 0; g < 3; ++g)
      if (g < nh) issue(cur, g, ss, cs);
  };
  prologue();

  for (int n = 0;; ++n) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mx_v16f{};

    auto issue_ahead = [&](int g) {  // stage g of the item, or of the next one, or nothing
      if (g < nh)
        issue(cur, g, ss, cs);
      else if (nxt_chain && g < nh + 2)
        issue(make_item(n + 1), g - nh, ss + nh, cs + nchunks);
    };
    for (int c = 0; c < nchunks; ++c) {
      const int h0 = 2 * c, h1 = 2 * c + 1;
      uint32_t xsc[2], wsc[4];
      // step h0
      wait_vm_var(loads_of(h0 + 1) + loads_of(h0 + 2));
      stage_barrier();
      issue_ahead(h0 + 3);
      {
        const uint32_t* sx = reinterpret_cast<const uint32_t*>(lds_sc[(cs + c) & 3]);
#pragma unroll
        for (int i = 0; i < 2; ++i) xsc[i] = sx[p.x_row_shift ? 2 * tq + i : 64 * tq + 32 * i + r] >> (8 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) wsc[j] = sx[256 + 128 * cq + 32 * j + r] >> (8 * hh);
      }
      stage_step(IntC<0>{}, h0, xsc, wsc);
      // step h1
      wait_vm_var(loads_of(h1 + 1) + loads_of(h1 + 2));
      stage_barrier();
      issue_ahead(h1 + 3);
      stage_step(IntC<1>{}, h1, xsc, wsc);
    }
    stage_barrier();  // every wave has read the last stage

    // ---- epilogue: one 32 x 32 output block per accumulator ----
    // The payload goes through LDS, in the two slots of the item's last two stages (every wave
    // finished reading them before the last step's barrier; the next item's first stages are in the
    // other two): a lane's accumulator holds 4-byte pieces of 32 different token rows, which as
    // direct stores would be partial-line writes; staged as a 256-token x 256-byte tile (16-byte
    // pieces XOR-swizzled by row) it leaves as whole 256-byte row segments, 16 bytes per lane.
    {
      uint8_t* stage = &lds[(ss + nh - 2) & 3][0][0];
      const LinPlace pl = place(n);  // the list still holds item n (a refill keeps the current item)
      const int valid = pl.valid, wrows = cur.wrows, ct = pl.ct;
      const int ncs = p.C_out >> 5;
      if (p.out_bf16) {
        // bf16 output: each lane writes its token's four runs of 4 consecutive columns per block
        // (8-byte stores; the two lane halves complete 16-byte runs)
        if (128 * cq < wrows) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int trow_l = 64 * tq + 32 * i + r;
            if (trow_l < valid) {
              uint16_t* orow = p.out_bf16 + (pl.row0 + trow_l) * (int64_t)p.C_out + ct * kCol + 128 * cq;
#pragma unroll
              for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const mx_v16f& y = acc[i][j];
                  uint2* dst = reinterpret_cast<uint2*>(orow + 32 * j + 8 * q + 4 * hh);
                  float v[4] = {y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]};
                  if (p.accumulate) {
                    const uint2 old = *dst;
                    v[0] += bf16_to_f32(old.x & 0xffffu);
                    v[1] += bf16_to_f32(old.x >> 16);
                    v[2] += bf16_to_f32(old.y & 0xffffu);
                    v[3] += bf16_to_f32(old.y >> 16);
                  }
                  *dst = make_uint2(f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16),
                                    f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16));
                }
            }
          }
        }
      } else if (128 * cq < wrows) {  // wave-uniform: the wave's column half exists
        // Rows past the sequence end hold finite values (their X rows re-read the last valid row):
        // they are converted and staged like the others but take no part in the block maximum and
        // are never stored, so the block loop has no lane-dependent branches.
        // |y| maximum of each lane's 16 values per block, by v_maximum3_f32 on absolute values: a NaN
        // propagates (a NaN block then gives a pattern above 0x7f800000, hence code 255), and as
        // non-negative floats the maxima order like their bit patterns.
        uint32_t v[8], amax[8];  // amax: wave-uniform, block (i, j) at 4 i + j
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const mx_v16f& y = acc[i][j];
            float m = abs_maximum3(fabsf(y[0]), y[1], y[2]);
#pragma unroll
            for (int e = 3; e < 15; e += 2) m = abs_maximum3(m, y[e], y[e + 1]);
            m = __builtin_elementwise_maximum(m, fabsf(y[15]));
            v[4 * i + j] = 64 * tq + 32 * i + r < valid ? __float_as_uint(m) : 0u;
          }
        wave_max8(v, amax);
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
                for (int q = 0; q < 4; ++q)
                  words[q] = pack4_div(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3], sc);
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
          const int64_t br = pl.br0 + 2 * tq + bi;
          const int cb = (ct * kCol + 128 * cq) / 32 + bj;
          p.scale[br * ncs + cb] = (uint8_t)mine;
          if (p.scale_t) p.scale_t[(int64_t)cb * nb_total + br] = (uint8_t)mine;
        }
      }
      __syncthreads();
      if (!p.out_bf16) {
        const int kq = tid & 15;  // 16-byte piece of the row
        const bool kq_live = 16 * kq < wrows;
        uint8_t* dtile = p.data + pl.row0 * (int64_t)p.C_out + ct * kCol + 16 * kq;
#pragma unroll
        for (int pass = 0; pass < kTok / 32; ++pass) {
          const int row = pass * 32 + (tid >> 4);
          if (row < valid && kq_live)
            *reinterpret_cast<uint4*>(dtile + row * (int64_t)p.C_out) =
                *reinterpret_cast<const uint4*>(stage + row * kCol + ((kq ^ (row & 15)) << 4));
        }
      }
    }
    if (n + 1 == count) break;
    stage_barrier();  // every wave has read its staged rows
    if (n + 2 < count && n + 2 >= n0 + kListCap) {
      n0 = n + 1;  // the list keeps the new current item (its epilogue) and the one after it
      fill_list(n0);
    }
    cur = make_item(n + 1);
    nxt_chain = chain && n + 2 < count;
    if (chain) {
      ss = (ss + nh) & 3;
      cs = (cs + nchunks) & 3;
      issue(cur, 2, ss, cs);
    } else {
      prologue();
    }
  }
  wait_vm_n<0>();  // no direct LDS load outlives the workgroup
}

}  // namespace

namespace mxfa {

hipError_t launch_linear_quantize(const MxOperand& x, const MxOperand& w, int64_t T, int C_in, int C_out,
                                  const int32_t* cu, int nseq, int max_seqlen, uint8_t* data,
                                  uint8_t* scale, uint8_t* scale_t, uint16_t* out_bf16, int accumulate,
                                  hipStream_t stream) {
  LinearParams p;
  p.x = x.data;
  p.x_scale = x.scale;
  p.x_row_shift = x.mode == 2 ? 5 : 0;
  p.w = w.data;
  p.w_scale = w.scale;
  p.cu = cu;
  p.nseq = nseq;
  p.n_coltiles = (C_out + kCol - 1) / kCol;
  p.C_in = C_in;
  p.C_out = C_out;
  p.data = data;
  p.scale = scale;
  p.scale_t = scale_t;
  p.out_bf16 = out_bf16;
  p.accumulate = accumulate;
  // an upper bound on the items (every sequence at max_seqlen)
  const int64_t items = (int64_t)nseq * ((max_seqlen + kTok - 1) / kTok) * p.n_coltiles;
  if (T == 0 || items == 0) return hipSuccess;
  // One workgroup per compute unit (the LDS ring admits one per CU), a multiple of 8 so that each
  // XCD gets the same number; fewer when there are fewer items.
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t full = cus >= 8 ? cus / 8 * 8 : 8;
  const int64_t grid = std::min<int64_t>(full, (items + 7) / 8 * 8);
  hipLaunchKernelGGL(linear_quantize_kernel, dim3((unsigned)grid), dim3(64 * kLinWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mxfa

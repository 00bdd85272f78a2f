// Tall-tile 4-bit linears for gfx950: the matrix-core-bound shapes, where a
// weight block meets hundreds or thousands of rows (the dense linears of the
// vision tower: q, k, v, o and the MLP's fused gate|up with its GeGLU).
//
// What is computed is the same as in qswitch.hip (diffusion-gemma model.ts
// page, the quantized linears; vision.ts page, VisionLinear.forward and
// DiffVisionMLP.forward for the GeGLU):
// y = x . dequant(W)^T with W = scale * q + bias per 64-wide group.  As in the
// weight-stationary kernel, the dequantized weight is rounded to bf16 once and
// every product and sum is done by the bf16 matrix cores with fp32
// accumulation.
//
// Shape of the work.  A workgroup owns a tile of BM = 16 MT rows x NB
// 128-row weight blocks.  Its waves split each block's 128 columns in two
// halves of 64 (four 16-column subtiles each) and, optionally (one block), the
// contraction in KS parts.  Each wave runs all BM rows against its 64
// columns, so the four subtiles it dequantizes per group (in registers,
// bf16(s q + b)) feed 8 MT matrix-core products: the vector work per product
// falls as 1 / MT.  The activations of a group (BM rows x 64 k, bf16) are
// the operand the waves share: loaded once per workgroup straight into LDS
// in matrix-core operand order, read from there by every wave.
//
// Pipeline per group g (one workgroup barrier each): the products of g
// (operands from LDS buffer g % 3, weights dequantized in the previous step)
// interleave with the dequantization of g + 1 and the loads of g + 2's
// activations straight into LDS buffer (g + 2) % 3; then the weight codes of
// g + 1 + PB are issued into the ring slot just dequantized.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kTallXcds = 8;
constexpr int kTallPB = 3;  // weight-code ring: groups in flight ahead of the dequantization

template <class F, int... I>
__device__ __forceinline__ void tall_steps(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// steps 0, 1, ... while i < n (short-circuit: a skipped step skips the rest)
template <class F, int... I>
__device__ __forceinline__ void tall_tail(F& f, const int& i, int n, std::integer_sequence<int, I...>) {
  (void)((i < n ? (f(std::integral_constant<int, I>{}), true) : false) && ...);
}

__device__ __forceinline__ void tall_wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One group's weight codes and (scale, bias) words for a wave's four
// subtiles: column half c holds subtiles 2c, 2c + 1 (codes in kilobyte c of
// the unit) and 2c + 4, 2c + 5 (kilobyte 2 + c).
struct TallSlot {
  u32x4_t c0, c1;  // code words: subtile t holds words 2 (t % 2), +1 of c0 (t < 2) or c1
  u32x2_t s0, s1;  // (scale, bias) of this lane's column: subtiles 2c, 2c + 1 and 2c + 4, 2c + 5
};

template <int MT>
constexpr int tall_tile_bytes() { return MT * 2048; }  // one group's operands: [m][h][lane] 16 bytes

}  // namespace

constexpr int kTallBufs = 3;  // LDS operand buffers per contraction part: loads run two groups ahead

template <int MT, int KS>
constexpr size_t tall_lds_bytes() { return (size_t)KS * kTallBufs * tall_tile_bytes<MT>(); }

// Waves per SIMD: one at MT = 8 (its 128 fp32 sums per lane sit in the
// accumulation registers, beside two groups of dequantized operands and the
// staging registers), two at MT <= 4.
template <int MT>
constexpr int tall_waves_per_simd() { return MT >= 8 ? 1 : 2; }

template <int MODE, int MT, int KS, int NB>
__global__ __launch_bounds__(128 * KS * NB)
__attribute__((amdgpu_waves_per_eu(tall_waves_per_simd<MT>(), tall_waves_per_simd<MT>()))) void qmm_tall_kernel(const SwitchArgs p) {
  static_assert(MODE == MODE_DENSE || MODE == MODE_DENSE_GEGLU || MODE == MODE_GATE_UP,
                "the dense linear (plain or with the GeGLU) or the gate_up switch linear");
  constexpr bool kRows = MODE == MODE_DENSE || MODE == MODE_DENSE_GEGLU;  // plain rows 0..M-1; else sorted expert rows
  static_assert(kRows || KS == 1, "the switch modes keep the contraction whole");
  static_assert(MT == 2 || MT == 4 || MT == 8, "2, 4 or 8 row tiles");
  static_assert(KS == 1 || KS == 2, "one or two contraction parts (KS = 2: G even, so that both parts' waves pass the same barriers)");
  static_assert(NB == 1 || (NB == 2 && KS == 1), "one weight block per workgroup, or two with the contraction whole");
  constexpr int BM = 16 * MT;
  constexpr int kTile = tall_tile_bytes<MT>();
  constexpr int PB = kTallPB;
  extern __shared__ __attribute__((aligned(16))) uint8_t tall_lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // column half c; with two contraction parts the part kp, with two blocks
  // the block bsel of the workgroup's pair
  const int c = wave & 1, kp = (KS == 2) ? wave >> 1 : 0, bsel = (NB == 2) ? wave >> 1 : 0;
  const int ln = lane & 15, lq = lane >> 4;
  const int K = p.K, G = K / kGroup, A = p.rows_total, nblk = p.nblk;
  const int grid = (int)gridDim.x, bid = (int)blockIdx.x;
  // A persistent grid: workgroup b takes positions pos0, pos0 + grid, ...
  // Workgroup b runs on die b % 8 and pos0 numbers the workgroups die by die,
  // so consecutive positions (the blocks of one row chunk, which read the same
  // activations) share a die's L2 in every round.
  const int pos0 = (grid % kTallXcds == 0) ? (bid % kTallXcds) * (grid / kTallXcds) + bid / kTallXcds : bid;
  // Items: (row chunk of BM rows, NB weight blocks); in the switch mode the
  // chunks of each expert's sorted rows, numbered expert by expert.
  const int nbp = (nblk + NB - 1) / NB;
  __shared__ ExpertChunks s_items;  // the switch mode's chunk tables, built once
  int n_items;
  if constexpr (kRows) {
    n_items = (A + BM - 1) / BM * nbp;
  } else {
    expert_chunk_tables<128 * KS * NB, BM>(s_items, p.offsets, p.E, A);
    n_items = s_items.cpre[p.E] * nbp;
  }

  for (int pos = pos0; pos < n_items; pos += grid) {
  // ---- this item: this wave's block blk (past the last block with an odd
  // count: the last block's weights, results never stored); in the switch
  // mode the chunk of expert e, tau0 its first activation tile
  int e = 0, r0 = 0, rows = 0, bp = 0, tau0 = 0;
  if constexpr (kRows) {
    const int ch = pos / nbp;
    bp = pos - ch * nbp;
    r0 = __builtin_amdgcn_readfirstlane(ch * BM);
    rows = __builtin_amdgcn_readfirstlane(min(BM, A - r0));
  } else {
    expert_chunk_at<BM>(s_items, p.E, nbp, pos, e, r0, rows, bp, tau0);
  }
  const int blk = __builtin_amdgcn_readfirstlane(bp * NB + bsel);
  const int wblk = min(blk, nblk - 1);
  const int mt = (rows + 15) >> 4;  // row tiles holding rows (the others are skipped)
  const int g0 = kp * G / KS, g1 = (kp + 1) * G / KS, ng = g1 - g0;

  // ---- operand addresses
  const uint8_t* const ubase = (const uint8_t*)p.w + ((size_t)e * nblk + wblk) * (size_t)G * kTiledUnit;
  const uint32_t cofs0 = (uint32_t)c * 1024 + lane * 16, cofs1 = (uint32_t)(2 + c) * 1024 + lane * 16;
  const uint32_t sofs0 = 4096 + ln * 16 + 8 * c, sofs1 = sofs0 + 256;
  const uint8_t* const abytes = (const uint8_t*)p.a;
  // the 2 NB waves of a contraction part share its activations: wave wl
  // loads row tiles m = wl + 2 NB s, lane (ln, lq) the 32 bytes of row
  // 16 m + ln that operand lanes (ln, lq) of both products hold
  constexpr int NW = 2 * NB;
  constexpr int NS = MT / NW;
  static_assert(NS >= 1, "every wave loads a row tile");
  const int wl = (KS == 2) ? c : wave;
  uint32_t aoff[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int rl = min(16 * (wl + NW * s) + ln, rows - 1);  // rows past the chunk read its last row
    int src = r0 + rl;
    if constexpr (MODE == MODE_GATE_UP) {  // the token of the sorted row's assignment
      const int a = p.assign[src];
      src = (a >= 0 && a < A) ? token_of(a, p.ktop_inv) : 0;
    }
    aoff[s] = (uint32_t)src * (uint32_t)(K * 2) + lq * 32;
  }
  uint8_t* const abuf = tall_lds + kp * kTallBufs * kTile;

  // (the group's offset goes into the uniform base, each lane adds a 32-bit
  // offset: the loads take the scalar-base form, no 64-bit vector adds)
  auto issue_b = [&](TallSlot& sl, int g) __attribute__((always_inline)) {
    const uint8_t* const u = ubase + (size_t)__builtin_amdgcn_readfirstlane(g) * kTiledUnit;
    uint32_t o0 = cofs0, o1 = cofs1, o2 = sofs0, o3 = sofs1;
    asm volatile("" : "+v"(o0), "+v"(o1), "+v"(o2), "+v"(o3));  // no instruction: keeps the offsets 32-bit
    sl.c0 = __builtin_nontemporal_load((const u32x4_t*)(u + o0));
    sl.c1 = __builtin_nontemporal_load((const u32x4_t*)(u + o1));
    sl.s0 = *(const u32x2_t*)(u + o2);
    sl.s1 = *(const u32x2_t*)(u + o3);
  };
  // The activations go straight from memory into LDS (one 16-byte piece per
  // lane and instruction, lane-ordered: the operand layout), two groups ahead
  // of the products, into the buffer every wave finished reading before the
  // last barrier.  Every row tile is loaded, also past the chunk's rows (they
  // read its last row), so that the step stays branch-free.
  auto dma_a = [&](int buf, int g) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int m = wl + NW * s;
      const uint8_t* const ag = abytes + (size_t)__builtin_amdgcn_readfirstlane(g) * 128u;
      uint32_t o[2] = {aoff[s], aoff[s] + 16u};
      asm volatile("" : "+v"(o[0]), "+v"(o[1]));  // no instruction: keeps the offsets 32-bit
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_global_load_lds((const void*)(ag + o[h]), (void*)(abuf + buf * kTile + (2 * m + h) * 1024), 16, 0, 0);
    }
  };
  // Waits until this wave's loads into the buffer published by the next
  // barrier have landed: the VMEM instructions issued after them are the
  // previous step's weight loads (4), this step's activation loads (2 NS)
  // and weight loads (4).
  constexpr int kAfter = 4 + 2 * NS + 4;
  static_assert(kAfter < 64, "vmcnt holds 6 bits");
  auto publish = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt((kAfter & 0xF) | (0x7 << 4) | (0xF << 8) | ((kAfter >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // subtile t's operands of one group, bf16(s q + b)
  const DequantConsts dk = dequant_consts();
  auto dequant_sub = [&](const TallSlot& sl, int t, u32x4_t (&bq)[4][2]) __attribute__((always_inline)) {
    const u32x4_t& cw = (t < 2) ? sl.c0 : sl.c1;
    const uint32_t sb = (t < 2) ? sl.s0[t] : sl.s1[t - 2];
    const float sc = __uint_as_float(sb << 16), bc = __uint_as_float(sb & 0xffff0000u);
    dequant_pair_bf16(cw[2 * (t & 1)], cw[2 * (t & 1) + 1], sc, bc, dk, bq[t][0], bq[t][1]);
  };

  f32x4_t acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[m][t] = zero4();
  // The products of one group (weights bq, activations from LDS buffer buf)
  // fused with the dequantization of the next group's slot into bn.  The step
  // is cut into regions of two row tiles by scheduling barriers; region r
  // issues the operand reads of region r + 1, then interleaves its 16
  // products with a quarter (MT = 8) of the next group's dequantization, one
  // product and then a few vector instructions at a time, so the vector unit
  // and LDS work while the matrix core does and no read is waited on right
  // after it is issued.
  constexpr int R = MT / 2;              // regions
  constexpr int SPR = 4 / R;             // subtiles dequantized per region
  constexpr int VPM = (47 * SPR + 15) / 16;  // vector instructions after each product
  // `mid` (the 2 NS activation loads into LDS) runs at the start of region
  // RM, after that region's reads.
  constexpr int RM = R > 1 ? 1 : 0;
  auto products = [&](const u32x4_t (&bq)[4][2], int buf, const TallSlot& next, u32x4_t (&bn)[4][2], auto&& mid)
      __attribute__((always_inline)) {
    const uint8_t* const src = abuf + buf * kTile;
    auto rd = [&](int m, int h) __attribute__((always_inline)) {
      return *(const u32x4_t*)(src + ((2 * m + h) * 64 + lane) * 16);
    };
    u32x4_t a[2][2][2];  // [region parity][tile of the region][half]
#pragma unroll
    for (int u = 0; u < 2; ++u) a[0][u][0] = rd(u, 0), a[0][u][1] = rd(u, 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      __builtin_amdgcn_sched_barrier(0);
      if (r + 1 < R) {
#pragma unroll
        for (int u = 0; u < 2; ++u) a[(r + 1) & 1][u][0] = rd(2 * r + 2 + u, 0), a[(r + 1) & 1][u][1] = rd(2 * r + 2 + u, 1);
      }
      if (r == RM) mid();
#pragma unroll
      for (int s = 0; s < SPR; ++s) dequant_sub(next, r * SPR + s, bn);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int m = 2 * r + u;  // all MT tiles: past the rows the results are never stored
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = mfma16x16x32(a[r & 1][u][0], bq[t][0], acc[m][t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = mfma16x16x32(a[r & 1][u][1], bq[t][1], acc[m][t]);
      }
      if (r + 1 < R) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // next region's reads first
      if (r == RM) __builtin_amdgcn_sched_group_barrier(0x020, 2 * NS, 0);  // the activation loads
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one product
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // then vector instructions
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next group's operands are complete here: keeps the dequantization in
    // this step (the compiler would sink it to the step that reads them)
#pragma unroll
    for (int t = 0; t < 4; ++t) asm volatile("" ::"v"(bn[t][0]), "v"(bn[t][1]));
  };

  // ---- prologue: PB groups of codes in flight, groups g0 and g0 + 1's
  // activations on their way into LDS buffers 0 and 1, g0 dequantized; then
  // the same VMEM order as a step's (weights of one group after the second
  // buffer's loads) and the wait for buffer 0
  TallSlot ring[PB];
#pragma unroll
  for (int d = 0; d < PB; ++d) {
    issue_b(ring[d], g0 + min(d, ng - 1));
    asm volatile("" ::: "memory");  // keeps the slots' loads in ring order
  }
  dma_a(0, g0);
  asm volatile("" ::: "memory");
  dma_a(1, g0 + min(1, ng - 1));
  asm volatile("" ::: "memory");
  u32x4_t bq[4][2], bn[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) dequant_sub(ring[0], t, bq);
  issue_b(ring[0], g0 + min(PB, ng - 1));
  {
    constexpr int kFirst = 2 * NS + 4;  // after buffer 0's loads: buffer 1's and one group of weights
    __builtin_amdgcn_s_waitcnt((kFirst & 0xF) | (0x7 << 4) | (0xF << 8) | ((kFirst >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  int i = 0;  // the group (g0 + i) whose products are next
  // Step s of a block of 2 PB steps (a multiple of the 3 LDS buffers): ring
  // slot (s + 1) % PB holds the next group's codes, LDS buffer s % 3 this
  // group's activations, and the dequantized operands ping-pong between bq
  // and bn with the parity of s (no copies).  Every buffer index is a
  // constant, so the compiler waits for an activation load only where its
  // own buffer is read.
  auto step = [&](auto s_tag) __attribute__((always_inline)) {
    constexpr int s = decltype(s_tag)::value;
    constexpr int dn = (s + 1) % PB;  // ring slot of group i + 1
    // One basic block per step (no branch inside, so that the dequantization
    // stays interleaved with the products): past the end every piece works on
    // the last group again, whose results are never used.
    auto mid = [&]() __attribute__((always_inline)) { dma_a((s + 2) % kTallBufs, g0 + min(i + 2, ng - 1)); };
    if constexpr (s % 2 == 0) products(bq, s % kTallBufs, ring[dn], bn, mid);
    else products(bn, s % kTallBufs, ring[dn], bq, mid);
    issue_b(ring[dn], g0 + min(i + 1 + PB, ng - 1));  // the slot just dequantized
    publish();
    ++i;
  };
  // Whole blocks of 2 PB steps in a loop with no exit inside (an exit from
  // the middle of a block would merge into the loop head, where the compiler
  // would then wait for every load in flight), then the remaining steps, each
  // taken only if the one before was.
  for (int b = ng / (2 * PB); b > 0; --b) tall_steps(step, std::make_integer_sequence<int, 2 * PB>{});
  tall_tail(step, i, ng, std::make_integer_sequence<int, 2 * PB - 1>{});
  // the loads issued past the end (weights into registers, activations into
  // LDS) complete before the LDS is reused below, in every wave
#pragma unroll
  for (int d = 0; d < PB; ++d) asm volatile("" ::"v"(ring[d].c0), "v"(ring[d].c1), "v"(ring[d].s0), "v"(ring[d].s1));
  __builtin_amdgcn_s_waitcnt((0 & 0xF) | (0x7 << 4) | (0xF << 8));
  __syncthreads();

  // ---- contraction parts: part 1 parks its sums in the LDS (every wave has
  // passed the last barrier, so the operand buffers are free), part 0 adds
  if constexpr (KS == 2) {
    f32x4_t* const red = (f32x4_t*)tall_lds + c * (MT * 4 * 64);
    if (kp == 1) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= mt) continue;
#pragma unroll
        for (int t = 0; t < 4; ++t) red[(m * 4 + t) * 64 + lane] = acc[m][t];
      }
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= mt) continue;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4_t o = red[(m * 4 + t) * 64 + lane];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[m][t][q] += o[q];
        }
      }
    }
  }
  // part 1's waves have no outputs (they pass the barrier below)
  if (kp == 0) {

  if constexpr (MODE == MODE_GATE_UP) {
    // ---- gate_up epilogue: gate subtile 2c + t and up subtile 2c + t + 4
    // (t = 0, 1) give columns 16 (2c + t) .. + 15 of block blk's 64 mid
    // columns; mid's activation tiles hold column 16 q + 8 h + i of tile row r
    // at byte h * 1024 + (16 q + r) * 16 + 2 i of the (tile, group) block, so
    // this wave's quarters q = 2c, 2c + 1 are bytes [512 c, 512 c + 512) of
    // each 1 KB half: staged per row tile in 1 KB of the LDS as [h][512], one
    // 16-byte store per lane
    uint8_t* const stg1 = tall_lds + (size_t)wave * 1024;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= mt) continue;
      const int tau = tau0 + m;
      if (tau < 0 || tau >= p.max_tiles || blk >= nblk) continue;
      tall_wave_fence();  // the previous tile's staging reads are done
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(uint16_t*)(stg1 + (ln >> 3) * 512 + (16 * t + 4 * lq + q) * 16 + (ln & 7) * 2) =
              f32_to_bf16_bits(gelu_tanh(acc[m][t][q]) * acc[m][t + 2][q]);
      tall_wave_fence();
      uint8_t* const dst = (uint8_t*)p.out + ((size_t)tau * (p.Nout / 64) + blk) * kActBlock;
      *(u32x4_t*)(dst + (lane >> 5) * 1024 + 512 * c + (lane & 31) * 16) = *(const u32x4_t*)(stg1 + lane * 16);
    }
  } else if constexpr (MODE == MODE_DENSE_GEGLU) {
    // ---- GeGLU epilogue (the weight tiled with split = Nout: block blk holds
    // gate rows 64 blk .. + 63 as subtiles 0-3 and the matching up rows as
    // 4-7): gate subtile 2c + t and up subtile 2c + t + 4 (t = 0, 1) give
    // output columns 64 blk + 32 c + 16 t .. + 15.  Staged per wave and row
    // tile as bf16 [16 rows][32 columns] (1 KB), written with 16-byte stores
    // (lane: row lane / 4, 8-column piece lane % 4).
    uint16_t* const stg = (uint16_t*)(tall_lds + (KS == 2 ? (size_t)c * MT * 4 * 64 * 16 : (size_t)wave * 1024));
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= mt) continue;
      if (m > 0) tall_wave_fence();  // the previous tile's staging reads are done
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          stg[(4 * lq + q) * 32 + 16 * t + ln] = f32_to_bf16_bits(gelu_tanh(acc[m][t][q]) * acc[m][t + 2][q]);
      tall_wave_fence();
      const int r = lane >> 2, lr = 16 * m + r;
      const int col = blk * 64 + 32 * c + 8 * (lane & 3);  // the last block may be partly past the width
      if (lr < rows && col < p.Nout && blk < nblk)
        *(u32x4_t*)((uint16_t*)p.out + (size_t)(r0 + lr) * p.Nout + col) = *(const u32x4_t*)(stg + r * 32 + 8 * (lane & 3));
    }
  } else {
  // ---- epilogue: acc[m][t][q] is row 16 m + 4 lq + q, column 16 j + ln of
  // the block with j = 2c + (t & 1) + 4 (t >> 1).  Staged per wave and row
  // tile as bf16 [16 rows][64 columns, t-major] in 2 KB of the LDS, written
  // with 16-byte stores (lane: row lane / 4, two 8-column pieces).
  // (with two contraction parts each wave stages in its own parked sums, which
  // it has read: its LDS operations run in order)
  uint16_t* const stg_out = (uint16_t*)(tall_lds + (KS == 2 ? (size_t)c * MT * 4 * 64 * 16 : (size_t)wave * 2048));
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= mt) continue;
    if (m > 0) tall_wave_fence();  // the previous tile's staging reads are done
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) stg_out[(4 * lq + q) * 64 + 16 * t + ln] = f32_to_bf16_bits(acc[m][t][q]);
    tall_wave_fence();
    const int r = lane >> 2, lr = 16 * m + r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int piece = 2 * (lane & 3) + h;  // 8-column piece of the 64 staged columns
      const int t = piece >> 1;
      const int col = blk * 128 + 16 * (2 * c + (t & 1) + 4 * (t >> 1)) + 8 * (piece & 1);
      if (lr < rows && col < p.Nout && blk < nblk)
        *(u32x4_t*)((uint16_t*)p.out + (size_t)(r0 + lr) * p.Nout + col) = *(const u32x4_t*)(stg_out + r * 64 + 8 * piece);
    }
  }
  }  // the epilogues
  }  // outputs of contraction part 0
  __syncthreads();  // every wave is done with the LDS before the next item's loads land there
  }  // items
}

// ------------------------------------------------------------------ launchers
namespace {

constexpr int kTallMaxDevices = 64;
// Weight blocks per workgroup of the 128-row configuration: the four waves of
// a two-block workgroup share one activation tile, so each loads half as many
// activation bytes per group as in a one-block workgroup (each kilobyte a wave
// loads per step costs it tens of cycles; 16384 x 2816 -> 2816: 357 -> 316 us).
constexpr int kTallPair = 2;

// A persistent grid: at most one workgroup per free slot (workgroups per CU at
// the configuration's waves per SIMD), each walking its items.
template <int MODE, int MT, int KS, int NB>
hipError_t launch_tall_cfg(const SwitchArgs& a, long long tiles, int num_cu, hipStream_t stream) {
  static std::atomic<int> attr_done[kTallMaxDevices];
  constexpr int lds = (int)tall_lds_bytes<MT, KS>();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kTallMaxDevices) dev = 0;
  if (!attr_done[dev].load(std::memory_order_acquire)) {
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&qmm_tall_kernel<MODE, MT, KS, NB>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    attr_done[dev].store(1, std::memory_order_release);
  }
  constexpr int kPerCu = tall_waves_per_simd<MT>() * 4 / (2 * KS * NB);
  static_assert(kPerCu >= 1, "a workgroup fits a CU");
  const long long slots = (long long)std::max(num_cu, 1) * kPerCu;
  const long long grid =
      std::min((std::max<long long>(tiles, 1) + kTallXcds - 1) / kTallXcds * kTallXcds, std::max<long long>(slots, 1));
  hipLaunchKernelGGL((qmm_tall_kernel<MODE, MT, KS, NB>), dim3((unsigned)grid), dim3(128 * KS * NB), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool tall_preferred(int mode, long long rows, int experts) {
  if (mode == MODE_DENSE || mode == MODE_DENSE_GEGLU) return experts == 1 && rows >= 512;
  if (mode == MODE_GATE_UP) return experts <= kChunkMaxExperts && rows >= 96LL * experts;
  return false;
}

template <int MODE>
hipError_t launch_tall(SwitchArgs a, int num_cu, hipStream_t stream) {
  a.ntiles = a.nblk;
  a.ktop_inv = ktop_inverse(a.ktop);
  const long long A = a.rows_total;
  if (A <= 0) return hipSuccess;
  if constexpr (MODE == MODE_GATE_UP) {
    // every row in its expert's chunks, at most one partial chunk per expert
    if (a.E > kChunkMaxExperts) return hipErrorInvalidValue;
    const long long items = ((A + 127) / 128 + std::min<long long>(a.E, A)) * ((a.nblk + kTallPair - 1) / kTallPair);
    return launch_tall_cfg<MODE, 8, 1, kTallPair>(a, items, num_cu, stream);
  } else {
  const int G = a.K / kGroup;
  // 128-row tiles where they give at least one wave per SIMD; else 64-row
  // tiles with the contraction split in two equal parts (both parts' waves
  // then pass the same number of workgroup barriers)
  const long long t8 = (A + 127) / 128 * a.nblk;
  if (2 * t8 >= 4LL * num_cu || G < 4 || G % 2 != 0)
    return launch_tall_cfg<MODE, 8, 1, kTallPair>(a, (A + 127) / 128 * ((a.nblk + kTallPair - 1) / kTallPair), num_cu,
                                                  stream);
  return launch_tall_cfg<MODE, 4, 2, 1>(a, (A + 63) / 64 * a.nblk, num_cu, stream);
  }
}

template hipError_t launch_tall<MODE_DENSE>(SwitchArgs, int, hipStream_t);
template hipError_t launch_tall<MODE_DENSE_GEGLU>(SwitchArgs, int, hipStream_t);
template hipError_t launch_tall<MODE_GATE_UP>(SwitchArgs, int, hipStream_t);

}  // namespace qmoe

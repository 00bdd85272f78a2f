// The weight-stationary 4-bit linear for gfx950, for weight blocks that meet
// many rows: the tied LM head with its softcap.
//
// What is computed is the same as in qswitch.hip (diffusion-gemma model.ts
// page, logitsFromHidden):
// y = x . dequant(W)^T with W = scale * q + bias per 64-wide group.  Here the
// dequantized weight is rounded to bf16 once, as a quantized matmul that
// dequantizes into the activations' type does, and every product and sum is
// done by the bf16 matrix cores with fp32 accumulation.
//
// Why a second kernel.  The chunked kernel streams each weight unit through
// one wave, which unpacks it and applies the group's affine in fp32 for at
// most 32 rows: at a few rows per expert that is the least work per weight
// byte, but with hundreds of rows per block the unpacking and the per-group
// epilogue are repeated for every 32-row chunk and the vector ALU, not the
// matrix cores, sets the pace.  Here a workgroup owns a tile of BM rows x one
// 128-row weight block over the whole contraction: per group its four waves
// dequantize the block's 4608-byte unit once, each wave a quarter, into LDS
// (bf16, already in matrix-core operand order), and every wave runs its
// 16 * MT rows against all 128 columns from there.
//
// Pipeline per group g (one workgroup barrier each): dequantize group g + 1
// (its codes were loaded kPD groups earlier) into the LDS buffer the previous
// group's products have finished reading; the products of group g from the
// other buffer; then the loads of group g + kPD into the register slot just
// consumed.  Activations are loaded straight into operand registers: the
// tiled weight's k order puts a lane's 16 k values of a group in 32
// contiguous bytes of an activation row.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kWsWaves = 4;
constexpr int kWsThreads = kWsWaves * 64;
constexpr int kBBuf = 8 * 2 * 64 * 16;      // one group's dequantized operands: 16 KB
constexpr int kWsLds = 2 * kBBuf;           // double buffer; the epilogue reuses it
constexpr int kWsXcds = 8;

template <class F, int... I>
__device__ __forceinline__ void ws_steps(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

__device__ __forceinline__ void ws_wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

template <int MODE, int MT, int kPD>
__global__ __launch_bounds__(kWsThreads, 2) void qmm_ws_kernel(const SwitchArgs p) {
  static_assert(MODE == MODE_DENSE_SOFTCAP, "the head");
  constexpr int BM = 16 * MT * kWsWaves;  // rows of the workgroup's tile
  static_assert(MT == 1 || MT == 2 || MT == 4, "1, 2 or 4 row tiles per wave (the epilogue stages at most 8 KB per wave)");
  extern __shared__ __attribute__((aligned(16))) uint8_t ws_lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lq = lane >> 4;
  const int K = p.K, G = K / kGroup, A = p.rows_total, nblk = p.nblk;
  const int grid = (int)gridDim.x, bid = (int)blockIdx.x;
  // workgroup b runs on die b % 8: consecutive positions (the blocks of one
  // row chunk, which read the same activations) share a die's L2
  const int pos = (grid % kWsXcds == 0) ? (bid % kWsXcds) * (grid / kWsXcds) + bid / kWsXcds : bid;

  // ---- this workgroup's item: (row chunk of BM rows, weight block)
  const int nch = (A + BM - 1) / BM;
  if (pos >= nch * nblk) return;
  const int ch = pos / nblk;
  const int blk = __builtin_amdgcn_readfirstlane(pos - ch * nblk);
  const int r0 = __builtin_amdgcn_readfirstlane(ch * BM);
  const int rows = __builtin_amdgcn_readfirstlane(min(BM, A - r0));

  // ---- operand addresses
  const uint8_t* const ubase = (const uint8_t*)p.w + (size_t)blk * (size_t)G * kTiledUnit;
  const uint32_t c_off = (uint32_t)wave * 1024 + lane * 16;           // this wave's quarter of the codes
  const uint32_t s_off = 4096 + ln * 16 + (uint32_t)(wave >> 1) * 256;  // (scale, bias) of its subtiles
  const uint8_t* const abytes = (const uint8_t*)p.a;
  uint32_t aoff[MT];
  const int wrow = 16 * MT * wave;  // first tile row of this wave
  const bool wave_rows = wrow < rows;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int rl = min(wrow + 16 * m + ln, rows - 1);  // rows past the chunk read its last row
    aoff[m] = (uint32_t)(r0 + rl) * (uint32_t)(K * 2) + lq * 32;
  }

  // ---- the ring of register slots: codes + scales of the wave's quarter of a
  // unit, and the activation operands of its row tiles
  u32x4_t rc[kPD], rs[kPD];
  u32x4_t ra[kPD][MT][2];
  auto issue = [&](u32x4_t& c, u32x4_t& s, u32x4_t (&a)[MT][2], int g) __attribute__((always_inline)) {
    const uint8_t* u = ubase + (size_t)g * kTiledUnit;
    c = __builtin_nontemporal_load((const u32x4_t*)(u + c_off));
    s = __builtin_nontemporal_load((const u32x4_t*)(u + s_off));
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint8_t* ab = abytes + (aoff[m] + (uint32_t)g * 128u);  // one 32-bit offset
      a[m][0] = *(const u32x4_t*)ab;
      a[m][1] = *(const u32x4_t*)(ab + 16);
    }
  };
  // dequantize the wave's two subtiles (2 wave, 2 wave + 1) of a unit into LDS
  // buffer `buf`: [subtile][half][lane] 16 bytes, the matrix cores' B order
  const DequantConsts dk = dequant_consts();
  auto dequant = [&](const u32x4_t& c, const u32x4_t& s, int buf) __attribute__((always_inline)) {
    uint8_t* const dst = ws_lds + buf * kBBuf;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = 2 * wave + t;
      const uint32_t sb = s[(2 * wave + t) & 3];
      const float sc = __uint_as_float(sb << 16), bc = __uint_as_float(sb & 0xffff0000u);
      u32x4_t d0, d1;
      dequant_pair_bf16(c[2 * t], c[2 * t + 1], sc, bc, dk, d0, d1);
      *(u32x4_t*)(dst + ((j * 2 + 0) * 64 + lane) * 16) = d0;
      *(u32x4_t*)(dst + ((j * 2 + 1) * 64 + lane) * 16) = d1;
    }
  };

  f32x4_t acc[MT][8];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = zero4();
  // The B operands of subtile j + 2 are read while subtile j's products run:
  // a read waited on right before its products leaves the LDS latency exposed
  // eight times per group.  The two halves of a subtile go to different
  // accumulators first (m, then k), so no product waits on the one before.
  auto products = [&](const u32x4_t (&a)[MT][2], int buf) __attribute__((always_inline)) {
    const uint8_t* const src = ws_lds + buf * kBBuf;
    auto rd = [&](int j, int h) __attribute__((always_inline)) {
      return *(const u32x4_t*)(src + ((j * 2 + h) * 64 + lane) * 16);
    };
    u32x4_t b[3][2];
    b[0][0] = rd(0, 0), b[0][1] = rd(0, 1);
    b[1][0] = rd(1, 0), b[1][1] = rd(1, 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 2 < 8) b[(j + 2) % 3][0] = rd(j + 2, 0), b[(j + 2) % 3][1] = rd(j + 2, 1);
      __builtin_amdgcn_sched_barrier(0);  // the scheduler would sink the reads to their first use
      const u32x4_t b0 = b[j % 3][0], b1 = b[j % 3][1];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m][j] = mfma16x16x32(a[m][0], b0, acc[m][j]);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m][j] = mfma16x16x32(a[m][1], b1, acc[m][j]);
    }
  };

#pragma unroll
  for (int d = 0; d < kPD; ++d) {
    issue(rc[d], rs[d], ra[d], min(d, G - 1));
    asm volatile("" ::: "memory");  // keeps the slots' loads in ring order
  }
  dequant(rc[0], rs[0], 0);
  __syncthreads();

  int g = 0;  // the group whose products are next
  auto step = [&](auto d_tag) __attribute__((always_inline)) {
    constexpr int d = decltype(d_tag)::value;
    constexpr int dn = (d + 1) % kPD;
    if (g >= G) return;  // uniform over the workgroup
    if (g + 1 < G) dequant(rc[dn], rs[dn], (g + 1) & 1);
    if (wave_rows) products(ra[d], g & 1);
    issue(rc[d], rs[d], ra[d], min(g + kPD, G - 1));  // past the end: the last group again (never used)
    asm volatile("" ::: "memory");
    __syncthreads();
    ++g;
  };
  do {
    ws_steps(step, std::make_integer_sequence<int, kPD>{});
  } while (g < G);
  // the loads issued past the end complete before the staging below
#pragma unroll
  for (int d = 0; d < kPD; ++d) {
    asm volatile("" ::"v"(rc[d]), "v"(rs[d]));
#pragma unroll
    for (int m = 0; m < MT; ++m) asm volatile("" ::"v"(ra[d][m][0]), "v"(ra[d][m][1]));
  }
  if (!wave_rows) return;  // no workgroup barrier follows

  // ---- epilogue: acc[m][j][i] is row wrow + 16 m + 4 lq + i, column
  // 16 j + ln of the block; staged per wave in its 8 KB of the LDS (the last
  // group's operands are no longer read: every wave passed the barrier)
  uint8_t* const wlds = ws_lds + (size_t)wave * (kWsLds / kWsWaves);
  {  // the head: logits rounded to bf16, widened, cap * tanh(z / cap)
    float* const stg = (float*)wlds;
    const int c = lane & 31;
    const int col = blk * 128 + 4 * c;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m > 0) ws_wave_fence();  // the previous tile's staging reads are done
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z = bf16_bits_to_f32(f32_to_bf16_bits(acc[m][j][i]));
          stg[(4 * lq + i) * 128 + 16 * j + ln] = p.cap * tanhf(z / p.cap);
        }
      ws_wave_fence();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = 2 * q + (lane >> 5), lr = wrow + 16 * m + r;
        if (lr < rows && col < p.Nout)
          *(u32x4_t*)((float*)p.out + (size_t)(r0 + lr) * p.Nout + col) = *(const u32x4_t*)(stg + r * 128 + 4 * c);
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
namespace {

constexpr int kWsMaxDevices = 64;

template <int MODE, int MT, int PD>
hipError_t launch_ws_cfg(const SwitchArgs& a, int grid, hipStream_t stream) {
  static std::atomic<int> attr_done[kWsMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kWsMaxDevices) dev = 0;
  if (!attr_done[dev].load(std::memory_order_acquire)) {
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&qmm_ws_kernel<MODE, MT, PD>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, kWsLds);
    if (attr != hipSuccess) return attr;
    attr_done[dev].store(1, std::memory_order_release);
  }
  hipLaunchKernelGGL((qmm_ws_kernel<MODE, MT, PD>), dim3((unsigned)grid), dim3(kWsThreads), kWsLds, stream, a);
  return hipGetLastError();
}

long long round8(long long n) { return (n + kWsXcds - 1) / kWsXcds * kWsXcds; }

}  // namespace

// Where the weight-stationary kernel is the faster one (measured on the
// 256-row head): the head from 128 rows.  Gate_up at prefill sizes went to
// the tall-tile kernel, which was faster there; the down pass, the dense
// linear and the dense GeGLU stayed off this kernel.
bool ws_preferred(int mode, long long rows, int experts) {
  (void)experts;
  return mode == MODE_DENSE_SOFTCAP && rows >= 128;
}

template <int MODE>
hipError_t launch_ws(SwitchArgs a, int num_cu, hipStream_t stream) {
  static_assert(MODE == MODE_DENSE_SOFTCAP, "the head");
  a.ntiles = a.nblk;
  const long long A = a.rows_total;
  if (A <= 0) return hipSuccess;
  // 64 rows per wave where that still gives two workgroups per compute unit
  const long long items4 = (A + 255) / 256 * a.nblk, items2 = (A + 127) / 128 * a.nblk;
  if (items2 > (1LL << 30)) return hipErrorInvalidValue;
  if (items4 >= 2LL * num_cu) return launch_ws_cfg<MODE, 4, 2>(a, (int)round8(items4), stream);
  return launch_ws_cfg<MODE, 2, 3>(a, (int)round8(items2), stream);
}

template hipError_t launch_ws<MODE_DENSE_SOFTCAP>(SwitchArgs, int, hipStream_t);

}  // namespace qmoe

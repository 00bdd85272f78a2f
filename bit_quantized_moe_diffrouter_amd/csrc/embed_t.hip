// The self-conditioning embedding (diffusion-gemma model.ts page,
// #embedCanvas): probabilities [L, V] times the 4-bit embedding table
// E [V, H] used without transposing, returned in bf16, times embed_scale:
//   out[l, h] = bf16( bf16( sum_v p[l, v] E[v, h] ) * scale )
//
// Here the contraction runs over the table's rows and each output column h
// sits in quantization group g = h / 64 of every row: E[v, h] = s[v, g] q[v, h]
// + b[v, g].  Per group g the sum splits as
//   sum_v (p s)[l, v] (128 + q[v, h]) - 128 sum_v (p s)[l, v] + sum_v (p b)[l, v]
// which is three bf16 MFMA products: A = bf16(p s) against the offset codes
// 128 + q (exact in bf16: 0x4300 | q), A against ones (the row sums X), and
// p against the biases b (exact bf16 operands; every column of that product
// holds the same sum Y).  Both uses of A see the same rounded values, so the
// 128 offsets cancel to fp32 accumulation order; the rounding of p s is the
// only one before the fp32 sums (the pages' quantized matmul rounds the
// dequantized table to bf16 instead).
//
// Table layout (qmoe_tile_weight_t): units of 1152 bytes, unit index
// g * (V / 32) + c for 64-column group g and 32-row chunk c.  Bytes [0, 1024):
// lane L = 16 kq + n holds at 16 L four words, word j with the codes of rows
// v = 32 c + 8 kq + t (t = 0..7) at column h = 64 g + 16 j + n, code t = 2p
// at bits 4p and t = 2p + 1 at bits 16 + 4p, so (word >> 4p) & 0x000F000F |
// 0x43004300 is the bf16 pair (128 + q_2p, 128 + q_2p+1) of the MFMA B operand
// (lane: column n, k = 8 kq .. 8 kq + 7).  Bytes [1024, 1152): the 32 rows'
// (scale, bias) bf16 pairs of group g, row 32 c + r at 1024 + 4 r.
//
// Work: a workgroup takes 64 rows, four column groups (one per wave) and a
// contiguous range of chunks: the waves read the same probabilities (64 rows
// x 32 entries per chunk) and each unpacks its own group's codes once for the
// four row tiles, two chunks in flight.  The fp32 sums for (64 rows, 64
// columns) go to the workspace; a second kernel adds the ranges in order,
// rounds, scales and rounds again.  (One group per workgroup with 256 rows,
// and rings of up to six chunks at one workgroup per CU, ran at the same
// speed: 1.12-1.16 ms for 256 x 262,144 x 2816.)
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {
constexpr int kUnitT = 1152;
constexpr int kTilesPerWave = 4;
constexpr int kRowsPerWg = 64;   // 4 row tiles of 16, shared by the workgroup's waves
constexpr int kRing = 2;         // chunks in flight per wave

struct ChunkRegs {
  u32x4_t w;       // codes: word j = column subtile j
  u32x4_t sb[2];   // (scale, bias) of rows 8 kq .. 8 kq + 7
  u32x4_t p[kTilesPerWave];  // probabilities: row tile t, k = 8 kq .. 8 kq + 7
};
}  // namespace

__global__ __launch_bounds__(256) void tile_weight_t_kernel(const uint32_t* __restrict__ w, const uint16_t* __restrict__ s,
                                                            const uint16_t* __restrict__ b, int V, int H,
                                                            uint8_t* __restrict__ dst) {
  // one thread per 16-byte piece: 64 code pieces and 8 scale pieces per unit
  const int G = H / 64, C = V / 32;
  const long long pieces = (long long)G * C * (kUnitT / 16);
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const long long u = i / (kUnitT / 16);
  const int piece = (int)(i - u * (kUnitT / 16));
  const int g = (int)(u / C), c = (int)(u - (long long)g * C);
  u32x4_t out;
  if (piece < 64) {
    const int L = piece, n = L & 15, kq = L >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 64 * g + 16 * j + n;
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int v = 32 * c + 8 * kq + t;
        const uint32_t code = (w[(size_t)v * (H / 8) + h / 8] >> (4 * (h & 7))) & 0xFu;
        word |= code << ((t & 1) ? 16 + 4 * (t >> 1) : 4 * (t >> 1));
      }
      out[j] = word;
    }
  } else {
    const int r0 = 4 * (piece - 64);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t si = (size_t)(32 * c + r0 + r) * G + g;
      out[r] = (uint32_t)s[si] | ((uint32_t)b[si] << 16);
    }
  }
  *(u32x4_t*)(dst + i * 16) = out;
}

__global__ __launch_bounds__(256, 2) void embed_t_kernel(const uint16_t* __restrict__ probs, int L, int V, int H,
                                                         const uint8_t* __restrict__ wt, int chunks_per_wg,
                                                         float* __restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int G = H / 64, C = V / 32;
  const int quads = (G + 3) / 4, quarters = (L + kRowsPerWg - 1) / kRowsPerWg;
  const int gq = blockIdx.x % quads, rq = (blockIdx.x / quads) % quarters, split = blockIdx.x / (quads * quarters);
  const int g = 4 * gq + wave;  // this wave's column group
  if (g >= G) return;           // no workgroup barrier in this kernel
  const int c0 = split * chunks_per_wg, c1 = min(c0 + chunks_per_wg, C);
  const uint8_t* const units = wt + (size_t)g * C * kUnitT;
  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float* const pout = part + (size_t)split * L * H;

  {
    const int b0 = rq * kRowsPerWg;
    // rows of the workgroup's four tiles, shared by its waves (clamped into
    // [0, L): rows past L repeat a valid row and are never stored)
    const uint16_t* prow[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t)
      prow[t] = probs + (size_t)min(b0 + 16 * t + n, L - 1) * V + 8 * kq;

    auto load = [&](int c, ChunkRegs& r) __attribute__((always_inline)) {
      const uint8_t* const u = units + (size_t)c * kUnitT;
      r.w = __builtin_nontemporal_load((const u32x4_t*)(u + 16 * lane));
      r.sb[0] = *(const u32x4_t*)(u + 1024 + 32 * kq);
      r.sb[1] = *(const u32x4_t*)(u + 1024 + 32 * kq + 16);
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t) r.p[t] = *(const u32x4_t*)(prow[t] + 32 * (size_t)c);
    };

    f32x4_t acc[kTilesPerWave][4], X[kTilesPerWave], Y[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      X[t] = zero4();
      Y[t] = zero4();
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[t][j] = zero4();
    }
    // a ring of kRing chunks in flight: chunk c's registers are slot c % kRing;
    // after a slot is consumed it is refilled with chunk c + kRing
    ChunkRegs ring[kRing];
#pragma unroll
    for (int d = 0; d < kRing; ++d)
      if (c0 + d < c1) load(c0 + d, ring[d]);
    auto compute = [&](const ChunkRegs& cur) __attribute__((always_inline)) {
      // B operands of the four column subtiles: offset codes 128 + q
      u32x4_t bq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) bq[j][pp] = ((cur.w[j] >> (4 * pp)) & 0x000F000Fu) | 0x43004300u;
      // scales of this lane's 8 rows; their biases as a bf16 B operand
      float sc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) sc[t] = bf16_lo_f32(cur.sb[t >> 2][t & 3]);
      u32x4_t bb;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
        bb[pp] = __builtin_amdgcn_perm(cur.sb[(2 * pp + 1) >> 2][(2 * pp + 1) & 3], cur.sb[(2 * pp) >> 2][(2 * pp) & 3],
                                       0x07060302u);
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t) {
        u32x4_t a;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          a[pp] = pack_bf16x2(bf16_lo_f32(cur.p[t][pp]) * sc[2 * pp], bf16_hi_f32(cur.p[t][pp]) * sc[2 * pp + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] = mfma16x16x32(a, bq[j], acc[t][j]);
        X[t] = mfma16x16x32(a, ones, X[t]);
        Y[t] = mfma16x16x32(cur.p[t], bb, Y[t]);
      }
    };
    for (int c = c0; c < c1; c += kRing) {
#pragma unroll
      for (int d = 0; d < kRing; ++d) {
        if (c + d >= c1) break;
        compute(ring[d]);
        if (c + d + kRing < c1) load(c + d + kRing, ring[d]);
      }
    }
    // sums of this chunk range: acc - 128 X + Y; lane (n, kq) holds rows
    // 4 kq + i of the tile and column n of each subtile
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = b0 + 16 * t + 4 * kq + i;
        if (row >= L) continue;
        float* const o = pout + (size_t)row * H + 64 * g + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[16 * j] = __builtin_fmaf(-128.f, X[t][i], acc[t][j][i]) + Y[t][i];
      }
  }
}

// out[l, h] = bf16( bf16( sum_s part[s][l][h] ) * scale ), ranges in order
__global__ __launch_bounds__(256) void embed_t_reduce_kernel(const float* __restrict__ part, int S, long long LH,
                                                             float scale, uint16_t* __restrict__ out) {
  const long long o = (long long)blockIdx.x * 256 + threadIdx.x;
  if (o >= LH) return;
  float acc = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] = (s0 + s < S) ? part[(size_t)(s0 + s) * LH + o] : 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s0 + s < S) acc += v[s];
  }
  out[o] = f32_to_bf16_bits(bf16_bits_to_f32(f32_to_bf16_bits(acc)) * scale);
}

// probs[l, v] = bf16( exp(z - max_l) / sum_v exp(z - max_l) ), fp32 inside
// (the precise softmax of the self-conditioning logits, cast to the
// embeddings' bf16).  One workgroup per row: a pass for the maximum and the
// sum (each thread's running pair rescaled as its maximum grows, then
// combined over the block in a fixed order), a pass for the outputs.
__global__ __launch_bounds__(256) void softmax_rows_bf16_kernel(const float* __restrict__ z, int V,
                                                                uint16_t* __restrict__ probs) {
  __shared__ float s_m[256], s_s[256];
  const int tid = threadIdx.x;
  const float* const row = z + (size_t)blockIdx.x * V;
  float m = -INFINITY, sum = 0.f;
  // eight 16-byte loads in flight per thread, then their values in order
  for (int v0 = 4 * tid; v0 < V; v0 += 8 * 1024) {
    f32x4_t xs[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = v0 + u * 1024;
      xs[u] = (v < V) ? *(const f32x4_t*)(row + v) : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = xs[u][i];
        if (x == -INFINITY) continue;
        if (x > m) {
          sum = sum * expf(m - x) + 1.f;
          m = x;
        } else {
          sum += expf(x - m);
        }
      }
  }
  s_m[tid] = m;
  s_s[tid] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      const float m1 = s_m[tid], m2 = s_m[tid + w];
      const float mm = fmaxf(m1, m2);
      const float a = (m1 == -INFINITY) ? 0.f : s_s[tid] * expf(m1 - mm);
      const float b = (m2 == -INFINITY) ? 0.f : s_s[tid + w] * expf(m2 - mm);
      s_m[tid] = mm;
      s_s[tid] = a + b;
    }
    __syncthreads();
  }
  const float mx = s_m[0], inv_den = s_s[0];
  uint16_t* const out = probs + (size_t)blockIdx.x * V;
  for (int v0 = 4 * tid; v0 < V; v0 += 8 * 1024) {
    f32x4_t xs[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = v0 + u * 1024;
      if (v < V) xs[u] = *(const f32x4_t*)(row + v);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = v0 + u * 1024;
      if (v >= V) continue;
      const f32x4_t x = xs[u];
      u32x2_t o;
      o[0] = pack_bf16x2(expf(x[0] - mx) / inv_den, expf(x[1] - mx) / inv_den);
      o[1] = pack_bf16x2(expf(x[2] - mx) / inv_den, expf(x[3] - mx) / inv_den);
      *(u32x2_t*)(out + v) = o;
    }
  }
}

hipError_t launch_softmax_rows_bf16(const float* z, int L, int V, uint16_t* probs, hipStream_t stream) {
  hipLaunchKernelGGL(softmax_rows_bf16_kernel, dim3((unsigned)L), dim3(256), 0, stream, z, V, probs);
  return hipGetLastError();
}

int embed_t_splits(int L, int V, int H) {
  const int C = V / 32;
  const int tiles = ((H / 64 + 3) / 4) * ((L + kRowsPerWg - 1) / kRowsPerWg);
  int S = (1024 + tiles - 1) / tiles;  // about 1024 workgroups
  if (S > C) S = C;
  if (S < 1) S = 1;
  return S;
}

hipError_t launch_tile_weight_t(const uint32_t* w, const uint16_t* s, const uint16_t* b, int V, int H, uint8_t* dst,
                                hipStream_t stream) {
  const long long pieces = (long long)(H / 64) * (V / 32) * (kUnitT / 16);
  hipLaunchKernelGGL(tile_weight_t_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, w, s, b, V, H,
                     dst);
  return hipGetLastError();
}

hipError_t launch_embed_t(const uint16_t* probs, int L, int V, int H, const void* wt, float scale, float* part,
                          uint16_t* out, hipStream_t stream) {
  const int G = H / 64, C = V / 32, S = embed_t_splits(L, V, H);
  const int per = (C + S - 1) / S;
  const long long wgs = (long long)((G + 3) / 4) * ((L + kRowsPerWg - 1) / kRowsPerWg) * S;
  hipLaunchKernelGGL(embed_t_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, probs, L, V, H,
                     (const uint8_t*)wt, per, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long LH = (long long)L * H;
  hipLaunchKernelGGL(embed_t_reduce_kernel, dim3((unsigned)((LH + 255) / 256)), dim3(256), 0, stream, part, S, LH,
                     scale, out);
  return hipGetLastError();
}

}  // namespace qmoe

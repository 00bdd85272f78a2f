// Unsorted switch linears for small batches (diffusion-gemma model.ts page,
// DiffExperts.forward: below 64 assignments the indices are not sorted and the
// gather matmuls read each assignment's expert directly; the model builds its
// decode layers with this arm when canvas length times top-k is under 64).
//
// What is computed is the same as on the sorted path: per assignment
// a = t k + j with expert e = indices[a],
//   gate_up:  mid[a] = gelu_tanh(x_t . gate_e) * (x_t . up_e)   (bf16 rows)
//   down:     d_a = bf16(mid[a] . down_e),  y_t = sum_j w_a d_a (fp32, j order)
//
// At a few assignments the work is a handful of matrix-vector products over
// tens of MB of weights: too few rows for matrix cores to matter and far too
// few (assignment, weight block) items to keep HBM busy if each item were one
// wave's sequential walk over the contraction.  Here every wave takes 1 to 4
// groups of one item (one 4608-byte tiled unit per group, all loads issued at
// once), so thousands of waves stream at the same time.  The four waves of a
// workgroup take consecutive parts of one item and add their partial sums in
// LDS in wave order, and the workgroup writes its 128 sums to the workspace.
// A second small kernel adds each item's parts in part order and applies the
// epilogue (GeGLU; or the bf16 rounding of the down rows and the weighted sum
// over k).  The hand-over between workgroups is the kernel boundary: a
// device-scope fence inside the first kernel would write back and invalidate
// the whole L2 of its die once per workgroup (measured: 110 us at one token
// instead of a few).  The sum order is fixed, so results are bitwise
// reproducible.
//
// Arithmetic per group: lane (n, q) holds codes 16q .. 16q+15 of rows
// 16 j + n (j = 0..7) of the block.  0x4300 | q is the bf16 pattern of 128 + q,
// so one v_and_or_b32 yields an exact bf16 pair of offset codes that matches a
// pair of consecutive bf16 activations; v_dot2_f32_bf16 adds their products
// (exact) to an fp32 sum P.  The group affine is applied in fp32 with the
// lane's activation sum X: sum_k x_k (s q_k + b) = s P + (b - 128 s) X.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {
constexpr int kUWaves = 4;       // waves per workgroup: consecutive parts of one item
constexpr int kUThreads = kUWaves * 64;
constexpr int kUMaxGpw = 4;      // groups per wave at most (all in flight together)
constexpr int kBlockRows = 128;  // rows of a tiled block: one partial sum each
constexpr int kUMaxParts = 16;   // workgroups per (assignment, block) at most

struct UnitRegs {
  u32x4_t w[4];  // codes: words of subtiles 2i, 2i+1 (16 codes each)
  u32x4_t s[2];  // (scale, bias) of subtiles 4h .. 4h+3
  u32x4_t x[2];  // activations k = 16q .. 16q+7, 16q+8 .. 16q+15
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// sum over the 8 codes of word w (code 2p at bits 4p, code 2p+1 at bits
// 16 + 4p) of (128 + code) * x, x as four bf16 pairs in natural order
__device__ __forceinline__ float word_dot(uint32_t w, const uint32_t (&xp)[4], float acc) {
#pragma unroll
  for (int p = 0; p < 4; ++p) acc = dot2_bf16(((w >> (4 * p)) & 0x000F000Fu) | 0x43004300u, xp[p], acc);
  return acc;
}
}  // namespace

template <int MODE>  // UNSORTED_GATE_UP or UNSORTED_DOWN
__global__ __launch_bounds__(kUThreads) void qswitch_unsorted_kernel(const UnsortedArgs p) {
  __shared__ float s_part[kUWaves][kBlockRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int item = blockIdx.x / p.S, s = blockIdx.x - item * p.S;  // item = (assignment a, block)
  const int a = item / p.nblk, blk = item - a * p.nblk;
  const int e = p.indices[a];
  const bool valid = e >= 0 && e < p.E;
  const int part = s * kUWaves + wave;
  const int g0 = min(part * p.gpw, p.G), g1 = min(g0 + p.gpw, p.G);
  // activation row: gate_up, token a / k of x; down, row a of mid
  const uint16_t* const xr = p.x + (size_t)(MODE == UNSORTED_GATE_UP ? a / p.k : a) * p.K;

  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  // groups [g0, g1) in batches of kUMaxGpw, each batch's loads issued together
  for (int gb = g0; valid && gb < g1; gb += kUMaxGpw) {
    const uint8_t* const u0 = (const uint8_t*)p.w + (((size_t)e * p.nblk + blk) * p.G + gb) * kTiledUnit;
    UnitRegs r[kUMaxGpw];
#pragma unroll
    for (int i = 0; i < kUMaxGpw; ++i) {
      if (gb + i >= g1) break;
      const uint8_t* const u = u0 + (size_t)i * kTiledUnit;
#pragma unroll
      for (int c = 0; c < 4; ++c) r[i].w[c] = __builtin_nontemporal_load((const u32x4_t*)(u + 1024 * c + 16 * lane));
#pragma unroll
      for (int h = 0; h < 2; ++h) r[i].s[h] = *(const u32x4_t*)(u + 4096 + 256 * h + 16 * n);
      const uint16_t* const xg = xr + (size_t)(gb + i) * kGroup + 16 * q;
      r[i].x[0] = *(const u32x4_t*)xg;
      r[i].x[1] = *(const u32x4_t*)(xg + 8);
    }
    const uint32_t ones = 0x3f803f80u;  // bf16 pair (1, 1)
#pragma unroll
    for (int i = 0; i < kUMaxGpw; ++i) {
      if (gb + i >= g1) break;
      const uint32_t xa[4] = {r[i].x[0][0], r[i].x[0][1], r[i].x[0][2], r[i].x[0][3]};
      const uint32_t xb[4] = {r[i].x[1][0], r[i].x[1][1], r[i].x[1][2], r[i].x[1][3]};
      float X = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) X = dot2_bf16(xa[m], ones, X);
#pragma unroll
      for (int m = 0; m < 4; ++m) X = dot2_bf16(xb[m], ones, X);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4_t& wv = r[i].w[j >> 1];
        float P = word_dot(wv[2 * (j & 1)], xa, 0.f);
        P = word_dot(wv[2 * (j & 1) + 1], xb, P);
        const uint32_t sb = r[i].s[j >> 2][j & 3];
        const float sc = bf16_lo_f32(sb), bi = bf16_hi_f32(sb);
        acc[j] = __builtin_fmaf(sc, P, __builtin_fmaf(bi - 128.f * sc, X, acc[j]));
      }
    }
  }
  // the four lanes of a row (q = 0..3), then the four waves in order
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] += __shfl_xor(acc[j], 16, 64);
    acc[j] += __shfl_xor(acc[j], 32, 64);
  }
  if (q == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_part[wave][16 * j + n] = acc[j];
  }
  __syncthreads();
  float* const part_out = p.part + ((size_t)item * p.S + s) * kBlockRows;
  if (tid < kBlockRows) {
    float v = s_part[0][tid];
#pragma unroll
    for (int w = 1; w < kUWaves; ++w) v += s_part[w][tid];
    part_out[tid] = v;
  }
}

// mid[a, 64 blk + c] = gelu_tanh(sum_s gate part) * (sum_s up part): gate row c
// of block blk is partial c, its up row partial 64 + c.  One thread per output.
__global__ __launch_bounds__(256) void unsorted_geglu_kernel(const UnsortedArgs p) {
  const long long o = (long long)blockIdx.x * 256 + threadIdx.x;
  if (o >= (long long)p.A * p.Nout) return;
  const int a = (int)(o / p.Nout), col = (int)(o - (long long)a * p.Nout);
  const int blk = col >> 6, c = col & 63;
  const float* const pp = p.part + ((size_t)a * p.nblk + blk) * p.S * kBlockRows + c;
  // a batch of parts' loads issued before its adds (the adds stay in part order)
  float g = 0.f, u = 0.f;
  for (int t0 = 0; t0 < p.S; t0 += kUMaxParts) {
    float gv[kUMaxParts], uv[kUMaxParts];
#pragma unroll
    for (int t = 0; t < kUMaxParts; ++t) {
      gv[t] = (t0 + t < p.S) ? pp[(t0 + t) * kBlockRows] : 0.f;
      uv[t] = (t0 + t < p.S) ? pp[(t0 + t) * kBlockRows + 64] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < kUMaxParts; ++t)
      if (t0 + t < p.S) g += gv[t], u += uv[t];
  }
  p.out[o] = f32_to_bf16_bits(gelu_tanh(g) * u);
}

// y[t, h] = sum_j w[t, j] * bf16(d_{t,j}[h]) in j order, d summed over its
// parts in order; dropped assignments are left out.  kp = k rounded up to a
// power of two threads per output: thread j forms d_j (all its parts' loads
// in flight together), then the first adds the k terms in j order from LDS.
__global__ __launch_bounds__(256) void unsorted_combine_kernel(const UnsortedArgs p, int kp) {
  __shared__ float s_v[256], s_w[256];
  __shared__ int s_ok[256];
  const int tid = threadIdx.x, j = tid & (kp - 1);
  const int T = p.A / p.k;
  const long long o = (long long)blockIdx.x * (256 / kp) + tid / kp;
  const bool live = o < (long long)T * p.Nout;
  const int t = live ? (int)(o / p.Nout) : 0, h = live ? (int)(o - (long long)t * p.Nout) : 0;
  const int blk = h / kBlockRows, r = h - blk * kBlockRows;
  float v = 0.f, wj = 0.f;
  int ok = 0;  // a dropped assignment contributes nothing
  if (live && j < p.k) {
    const int aj = t * p.k + j, ej = p.indices[aj];
    const float* const pp = p.part + ((size_t)aj * p.nblk + blk) * p.S * kBlockRows + r;
    float d = 0.f;
    for (int u0 = 0; u0 < p.S; u0 += kUMaxParts) {
      float dv[kUMaxParts];
#pragma unroll
      for (int u = 0; u < kUMaxParts; ++u) dv[u] = (u0 + u < p.S) ? pp[(u0 + u) * kBlockRows] : 0.f;
#pragma unroll
      for (int u = 0; u < kUMaxParts; ++u)
        if (u0 + u < p.S) d += dv[u];
    }
    v = bf16_bits_to_f32(f32_to_bf16_bits(d));  // the down row as the switch linear returns it
    ok = ej >= 0 && ej < p.E;
    if (ok) wj = p.weights[aj];
  }
  s_v[tid] = v;
  s_w[tid] = wj;
  s_ok[tid] = ok;
  __syncthreads();
  if (live && j == 0) {
    float y = 0.f;
    for (int i = 0; i < p.k; ++i)
      if (s_ok[tid + i]) y = __builtin_fmaf(s_w[tid + i], s_v[tid + i], y);
    p.out[o] = f32_to_bf16_bits(y);
  }
}

UnsortedPlan unsorted_plan(long long A, int nblk, int G) {
  UnsortedPlan pl;
  const long long units = A * nblk * G;
  pl.gpw = units <= 8192 ? 1 : (units <= 16384 ? 2 : kUMaxGpw);
  while ((G + pl.gpw * kUWaves - 1) / (pl.gpw * kUWaves) > kUMaxParts && pl.gpw < 64) ++pl.gpw;
  const int parts = (G + pl.gpw - 1) / pl.gpw;
  pl.S = (parts + kUWaves - 1) / kUWaves;
  pl.partials = A * nblk * pl.S * kBlockRows;
  return pl;
}

hipError_t launch_unsorted(int mode, UnsortedArgs a, hipStream_t stream) {
  const long long wgs = (long long)a.A * a.nblk * a.S;
  if (wgs <= 0) return hipSuccess;
  const long long outs = (mode == UNSORTED_GATE_UP) ? (long long)a.A * a.Nout : (long long)(a.A / a.k) * a.Nout;
  const unsigned rblocks = (unsigned)((outs + 255) / 256);
  if (mode == UNSORTED_GATE_UP) {
    hipLaunchKernelGGL(qswitch_unsorted_kernel<UNSORTED_GATE_UP>, dim3((unsigned)wgs), dim3(kUThreads), 0, stream, a);
    hipLaunchKernelGGL(unsorted_geglu_kernel, dim3(rblocks), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(qswitch_unsorted_kernel<UNSORTED_DOWN>, dim3((unsigned)wgs), dim3(kUThreads), 0, stream, a);
    int kp = 1;
    while (kp < a.k) kp *= 2;
    const unsigned cblocks = (unsigned)((outs + 256 / kp - 1) / (256 / kp));
    hipLaunchKernelGGL(unsorted_combine_kernel, dim3(cblocks), dim3(256), 0, stream, a, kp);
  }
  return hipGetLastError();
}

}  // namespace qmoe

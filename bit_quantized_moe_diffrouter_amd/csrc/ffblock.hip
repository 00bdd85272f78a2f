// The decoder's feed-forward block around the MoE (diffusion-gemma model.ts
// page, DiffDecoderLayer.forwardWith, after the attention residual):
//
//   h1  = postFfNorm1(mlp(preFfNorm(h)))          dense GeGLU branch
//   h2  = postFfNorm2(experts(preFfNorm2(h)))     the MoE, routed on the raw h
//   out = (h + postFfNorm(h1 + h2)) * layer_scalar
//
// Every norm is a plain RMSNorm, x / sqrt(mean(x^2) + eps) * w, with the stored
// weight used as is (the page's header note on the checkpoint).  Two row
// kernels cover the norms: ff_prenorm_kernel reads h once and writes both
// normalised copies (the dense branch's input and the experts' input);
// ff_combine_kernel takes the two branches' raw outputs and the residual and
// applies the three post-norms, the residual add and the scalar in one pass
// over each row.  One wave per row, fp32 arithmetic, sums in a fixed order
// (each lane's 8-column chunks in ascending order, then a butterfly over the
// 64 lanes), bf16 in and out.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {
constexpr int kRowsPerBlock = 4;  // one wave per row
constexpr int kRegChunks = 8;     // rows of up to 64 * 8 chunks of 8 (H <= 4096) stay in registers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum of squares of a bf16 row (n8 chunks of 8 values), this lane's share
// summed in chunk order, then over the wave.
__device__ __forceinline__ float row_sumsq(const uint16_t* row, int n8, int lane) {
  float ss = 0.f;
  for (int c = lane; c < n8; c += 64) {
    const u32x4_t v = *(const u32x4_t*)(row + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = bf16_lo_f32(v[q]), b = bf16_hi_f32(v[q]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
  return wave_sum(ss);
}

__device__ __forceinline__ float rms_factor(float sumsq, int H, float eps) {
  return 1.0f / sqrtf(sumsq / (float)H + eps);
}
}  // namespace

// NC > 0: each lane keeps its (at most NC) 8-column chunks of the row in
// registers, so the row is read once and every load is issued before the
// first sum; NC = 0: the row is re-read per pass (any H).
template <int NC>
__global__ __launch_bounds__(64 * kRowsPerBlock) void ff_prenorm_kernel(const uint16_t* __restrict__ h, int T, int H,
                                                                         const uint16_t* __restrict__ wa,
                                                                         const uint16_t* __restrict__ wb, float eps,
                                                                         uint16_t* __restrict__ xa,
                                                                         uint16_t* __restrict__ xb) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave; no barrier below
  const int n8 = H / 8;
  const uint16_t* row = h + (size_t)t * H;
  if constexpr (NC > 0) {
    // the row and both weight vectors are loaded before the first sum
    const u32x4_t z4 = {0u, 0u, 0u, 0u};
    u32x4_t v[NC], GA[NC], GB[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < n8;
      v[i] = ok ? *(const u32x4_t*)(row + 8 * c) : z4;
      GA[i] = ok ? *(const u32x4_t*)(wa + 8 * c) : z4;
      GB[i] = ok ? *(const u32x4_t*)(wb + 8 * c) : z4;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (lane + 64 * i >= n8) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = bf16_lo_f32(v[i][q]), b = bf16_hi_f32(v[i][q]);
        ss = __builtin_fmaf(a, a, ss);
        ss = __builtin_fmaf(b, b, ss);
      }
    }
    const float r = rms_factor(wave_sum(ss), H, eps);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c >= n8) break;
      const u32x4_t ga = GA[i], gb = GB[i];
      u32x4_t oa, ob;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf16_lo_f32(v[i][q]) * r, hi = bf16_hi_f32(v[i][q]) * r;
        oa[q] = pack_bf16x2(lo * bf16_lo_f32(ga[q]), hi * bf16_hi_f32(ga[q]));
        ob[q] = pack_bf16x2(lo * bf16_lo_f32(gb[q]), hi * bf16_hi_f32(gb[q]));
      }
      *(u32x4_t*)(xa + (size_t)t * H + 8 * c) = oa;
      *(u32x4_t*)(xb + (size_t)t * H + 8 * c) = ob;
    }
    return;
  }
  const float r = rms_factor(row_sumsq(row, n8, lane), H, eps);
  for (int c = lane; c < n8; c += 64) {
    const u32x4_t v = *(const u32x4_t*)(row + 8 * c);
    const u32x4_t ga = *(const u32x4_t*)(wa + 8 * c);
    const u32x4_t gb = *(const u32x4_t*)(wb + 8 * c);
    u32x4_t oa, ob;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16_lo_f32(v[q]) * r, hi = bf16_hi_f32(v[q]) * r;
      oa[q] = pack_bf16x2(lo * bf16_lo_f32(ga[q]), hi * bf16_hi_f32(ga[q]));
      ob[q] = pack_bf16x2(lo * bf16_lo_f32(gb[q]), hi * bf16_hi_f32(gb[q]));
    }
    *(u32x4_t*)(xa + (size_t)t * H + 8 * c) = oa;
    *(u32x4_t*)(xb + (size_t)t * H + 8 * c) = ob;
  }
}

// out = (res + N(N1(h1) + N2(h2))) * scalar; the sum s = N1(h1) + N2(h2) is
// formed twice (once for its norm, once for the output) from the same inputs
// in the same order, so both passes see the same fp32 values.
// NC as in ff_prenorm_kernel: h1 and h2 are read once into registers.
template <int NC>
__global__ __launch_bounds__(64 * kRowsPerBlock) void ff_combine_kernel(
    const uint16_t* __restrict__ res, const uint16_t* __restrict__ h1, const uint16_t* __restrict__ h2, int T, int H,
    const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w2, const uint16_t* __restrict__ w, float eps,
    float scalar, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave; no barrier below
  const int n8 = H / 8;
  const size_t o = (size_t)t * H;
  if constexpr (NC > 0) {
    // every load of the row is issued here, before the first sum
    const u32x4_t z4 = {0u, 0u, 0u, 0u};
    u32x4_t A[NC], B[NC], GA[NC], GB[NC], X[NC], G[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < n8;
      A[i] = ok ? *(const u32x4_t*)(h1 + o + 8 * c) : z4;
      B[i] = ok ? *(const u32x4_t*)(h2 + o + 8 * c) : z4;
      GA[i] = ok ? *(const u32x4_t*)(w1 + 8 * c) : z4;
      GB[i] = ok ? *(const u32x4_t*)(w2 + 8 * c) : z4;
      X[i] = ok ? *(const u32x4_t*)(res + o + 8 * c) : z4;
      G[i] = ok ? *(const u32x4_t*)(w + 8 * c) : z4;
    }
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (lane + 64 * i >= n8) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = bf16_lo_f32(A[i][q]), b = bf16_hi_f32(A[i][q]);
        s1 = __builtin_fmaf(a, a, s1);
        s1 = __builtin_fmaf(b, b, s1);
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (lane + 64 * i >= n8) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = bf16_lo_f32(B[i][q]), b = bf16_hi_f32(B[i][q]);
        s2 = __builtin_fmaf(a, a, s2);
        s2 = __builtin_fmaf(b, b, s2);
      }
    }
    const float r1 = rms_factor(wave_sum(s1), H, eps);
    const float r2 = rms_factor(wave_sum(s2), H, eps);
    // s = N1(h1) + N2(h2) per chunk, kept for the output pass
    float S[NC][8];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const u32x4_t ga = GA[i], gb = GB[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        S[i][2 * q] = bf16_lo_f32(A[i][q]) * r1 * bf16_lo_f32(ga[q]) + bf16_lo_f32(B[i][q]) * r2 * bf16_lo_f32(gb[q]);
        S[i][2 * q + 1] =
            bf16_hi_f32(A[i][q]) * r1 * bf16_hi_f32(ga[q]) + bf16_hi_f32(B[i][q]) * r2 * bf16_hi_f32(gb[q]);
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (lane + 64 * i >= n8) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(S[i][e], S[i][e], ss);
    }
    const float r = rms_factor(wave_sum(ss), H, eps);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c >= n8) break;
      const u32x4_t x = X[i], g = G[i];
      u32x4_t y;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        y[q] = pack_bf16x2((bf16_lo_f32(x[q]) + S[i][2 * q] * r * bf16_lo_f32(g[q])) * scalar,
                           (bf16_hi_f32(x[q]) + S[i][2 * q + 1] * r * bf16_hi_f32(g[q])) * scalar);
      *(u32x4_t*)(out + o + 8 * c) = y;
    }
    return;
  }
  const float r1 = rms_factor(row_sumsq(h1 + o, n8, lane), H, eps);
  const float r2 = rms_factor(row_sumsq(h2 + o, n8, lane), H, eps);
  // the 8 values of s in chunk c
  auto sum_chunk = [&](int c, float (&sv)[8]) __attribute__((always_inline)) {
    const u32x4_t a = *(const u32x4_t*)(h1 + o + 8 * c), b = *(const u32x4_t*)(h2 + o + 8 * c);
    const u32x4_t ga = *(const u32x4_t*)(w1 + 8 * c), gb = *(const u32x4_t*)(w2 + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sv[2 * q] = bf16_lo_f32(a[q]) * r1 * bf16_lo_f32(ga[q]) + bf16_lo_f32(b[q]) * r2 * bf16_lo_f32(gb[q]);
      sv[2 * q + 1] = bf16_hi_f32(a[q]) * r1 * bf16_hi_f32(ga[q]) + bf16_hi_f32(b[q]) * r2 * bf16_hi_f32(gb[q]);
    }
  };
  float ss = 0.f;
  for (int c = lane; c < n8; c += 64) {
    float sv[8];
    sum_chunk(c, sv);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(sv[i], sv[i], ss);
  }
  const float r = rms_factor(wave_sum(ss), H, eps);
  for (int c = lane; c < n8; c += 64) {
    float sv[8];
    sum_chunk(c, sv);
    const u32x4_t x = *(const u32x4_t*)(res + o + 8 * c), g = *(const u32x4_t*)(w + 8 * c);
    u32x4_t y;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      y[q] = pack_bf16x2((bf16_lo_f32(x[q]) + sv[2 * q] * r * bf16_lo_f32(g[q])) * scalar,
                         (bf16_hi_f32(x[q]) + sv[2 * q + 1] * r * bf16_hi_f32(g[q])) * scalar);
    *(u32x4_t*)(out + o + 8 * c) = y;
  }
}

hipError_t launch_ff_prenorm(const uint16_t* h, int T, int H, const uint16_t* wa, const uint16_t* wb, float eps,
                             uint16_t* xa, uint16_t* xb, hipStream_t stream) {
  const int blocks = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  if (H / 8 <= 64 * kRegChunks)
    hipLaunchKernelGGL(ff_prenorm_kernel<kRegChunks>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream, h, T, H, wa,
                       wb, eps, xa, xb);
  else
    hipLaunchKernelGGL(ff_prenorm_kernel<0>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream, h, T, H, wa, wb, eps,
                       xa, xb);
  return hipGetLastError();
}

hipError_t launch_ff_combine(const uint16_t* res, const uint16_t* h1, const uint16_t* h2, int T, int H,
                             const uint16_t* w1, const uint16_t* w2, const uint16_t* w, float eps, float scalar,
                             uint16_t* out, hipStream_t stream) {
  const int blocks = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  if (H / 8 <= 64 * kRegChunks)
    hipLaunchKernelGGL(ff_combine_kernel<kRegChunks>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream, res, h1, h2,
                       T, H, w1, w2, w, eps, scalar, out);
  else
    hipLaunchKernelGGL(ff_combine_kernel<0>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream, res, h1, h2, T, H,
                       w1, w2, w, eps, scalar, out);
  return hipGetLastError();
}

}  // namespace qmoe

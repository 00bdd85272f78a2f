// DiffRouter for gfx950 (diffusion-gemma model.ts page, DiffRouter.forward;
// the no-scale norm is vision.ts page, manualRms with a null weight):
//   r = x / sqrt(mean(x^2) + eps);  u = r * scale * H^-0.5
//   logits = u . dequant(W_r)^T (+ offset);  top-k (descending, ties to the
//   lower expert);  precise softmax over the k;  times per_expert_scale.
//
// The top-k decision is taken on fp32 logits.  Kernel 1 computes them with
// MFMA: u is split into three bf16 terms (u = hi + mid + lo to 24 bits), the
// router codes are unpacked to the exact bf16 values 16 + q, and the group
// affine is applied in fp32 (s P + (b - 16 s) U, U = sum of u over the
// group).  The norm is one positive factor per token, so kernel 1 works on
// x * scale * H^-0.5 and kernel 2 multiplies the summed logits by
// 1 / sqrt(mean(x^2) + eps).  A (token tile, k-range) grid fills the chip at
// 256 tokens; the partial logits go to a workspace and kernel 2 sums them in
// a fixed order, so the result is run-to-run reproducible.  Kernel 2 runs one
// wave per token: a radix select finds the k-th largest ordering key, the k
// best land in slots 0..k-1 in descending order, then the softmax in fp32.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {
constexpr int kRWaves = 8, kRThreads = kRWaves * 64;
constexpr int kTT = 16;              // tokens per workgroup
constexpr int kRKS = 4;              // groups per LDS stage
constexpr int kRRowB = kRKS * 128 + 16;
}  // namespace

// K parts of the logit kernel: enough (token tile, K part) workgroups to fill
// the chip at small T, and at least 4 at large T, where a single part per tile
// would walk all groups in latency-bound stages one after another; at most
// 16, the parts the top-k kernel sums with one round of loads (more parts at
// a few tokens cost the top-k kernel more than they save the logit kernel).
int route_ksplit(int T, int H) {
  const int G = H / kGroup;
  const int tiles = (T + kTT - 1) / kTT;
  int ks = 256 / (tiles > 0 ? tiles : 1);
  if (ks < 4) ks = 4;
  if (ks > 16) ks = 16;
  if (ks > G) ks = G;
  return ks;
}

template <int NPW>
__global__ __launch_bounds__(kRThreads) void route_logits_kernel(const RouteArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_u[3][kTT * kRRowB];
  __shared__ float s_U[kRKS][kTT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lq = lane >> 4;
  const int T = p.T, H = p.H, E = p.E, G = H / kGroup, KW = H / 8;
  const int t0 = blockIdx.x * kTT;
  const int ks = blockIdx.y;
  const int g_begin = (int)((long long)ks * G / p.ksplit);
  const int g_end = (int)((long long)(ks + 1) * G / p.ksplit);

  const int nte = (E + 15) / 16;
  int e0[NPW];
  bool act[NPW];
  const uint32_t* wp[NPW];
  const uint16_t* sp[NPW];
  const uint16_t* bp[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int nt = wave + kRWaves * j;
    e0[j] = 16 * nt;
    const int e = e0[j] + ln;
    act[j] = nt < nte;
    const bool rv = act[j] && e < E;
    const size_t row = rv ? (size_t)e : 0;
    wp[j] = p.w + row * KW + 2 * lq;
    sp[j] = p.s + row * G;
    bp[j] = p.b + row * G;
  }

  f32x4_t acc[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) acc[j] = zero4();

  // staging piece of this thread: token tt, group-in-stage gl, block blk
  const int s_tt = tid >> 5, s_gl = (tid >> 3) & 3, s_blk = tid & 7;
  float ssq = 0.f;  // this thread's share of sum(x^2) over the k-range (for the norm)

  for (int gs = g_begin; gs < g_end; gs += kRKS) {
    // weights of this stage (issued first so their latency hides under the staging)
    u32x2_t wr[kRKS][NPW];
    uint32_t sr[kRKS][NPW], br[kRKS][NPW];
#pragma unroll
    for (int gl = 0; gl < kRKS; ++gl)
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        const int g = gs + gl;
        const bool ok = act[j] && (e0[j] + ln < E) && g < g_end;
        wr[gl][j] = ok ? *(const u32x2_t*)(wp[j] + g * 8) : u32x2_t{0u, 0u};
        sr[gl][j] = ok ? (uint32_t)sp[j][g] : 0u;
        br[gl][j] = ok ? (uint32_t)bp[j][g] : 0u;
      }

    // u for 16 tokens x 4 groups, split into three bf16 terms
    {
      const int t = t0 + s_tt, g = gs + s_gl;
      float u[8];
      if (t < T && g < g_end) {
        const int h = g * kGroup + s_blk * 8;
        const u32x4_t xv = *(const u32x4_t*)(p.x + (size_t)t * H + h);
        const u32x4_t nv = *(const u32x4_t*)(p.norm_scale + h);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float xa = bf16_lo_f32(xv[q]), xb = bf16_hi_f32(xv[q]);
          ssq = __builtin_fmaf(xa, xa, ssq);
          ssq = __builtin_fmaf(xb, xb, ssq);
          u[2 * q] = (xa * bf16_lo_f32(nv[q])) * p.root;
          u[2 * q + 1] = (xb * bf16_hi_f32(nv[q])) * p.root;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) u[v] = 0.f;
      }
      u32x4_t hi, md, lo;
      float usum = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = u[2 * q], b = u[2 * q + 1];
        usum += a;
        usum += b;
        hi[q] = pack_bf16x2(a, b);
        const float ra = a - bf16_lo_f32(hi[q]), rb = b - bf16_hi_f32(hi[q]);
        md[q] = pack_bf16x2(ra, rb);
        lo[q] = pack_bf16x2(ra - bf16_lo_f32(md[q]), rb - bf16_hi_f32(md[q]));
      }
      const int off = s_tt * kRRowB + s_gl * 128 + s_blk * 16;
      *(u32x4_t*)(&lds_u[0][off]) = permute_pairs(hi);
      *(u32x4_t*)(&lds_u[1][off]) = permute_pairs(md);
      *(u32x4_t*)(&lds_u[2][off]) = permute_pairs(lo);
      usum += __shfl_xor(usum, 1, 64);
      usum += __shfl_xor(usum, 2, 64);
      usum += __shfl_xor(usum, 4, 64);
      if (s_blk == 0) s_U[s_gl][s_tt] = usum;
    }
    __syncthreads();

#pragma unroll
    for (int gl = 0; gl < kRKS; ++gl) {
      if (gs + gl >= g_end) break;
      u32x4_t a0[3], a1[3];
#pragma unroll
      for (int sp3 = 0; sp3 < 3; ++sp3) {
        const uint8_t* base = &lds_u[sp3][ln * kRRowB + gl * 128 + lq * 32];
        a0[sp3] = *(const u32x4_t*)base;
        a1[sp3] = *(const u32x4_t*)(base + 16);
      }
      float U[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) U[i] = s_U[gl][4 * lq + i];
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        if (!act[j]) continue;
        const u32x4_t b0 = unpack_offset16_codes(wr[gl][j].x);
        const u32x4_t b1 = unpack_offset16_codes(wr[gl][j].y);
        const float sc = bf16_bits_to_f32(sr[gl][j]);
        const float cc = bf16_bits_to_f32(br[gl][j]) - 16.0f * sc;
        f32x4_t P = zero4();
#pragma unroll
        for (int sp3 = 0; sp3 < 3; ++sp3) {
          P = mfma16x16x32(a0[sp3], b0, P);
          P = mfma16x16x32(a1[sp3], b1, P);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = __builtin_fmaf(cc, U[i], __builtin_fmaf(sc, P[i], acc[j][i]));
      }
    }
    __syncthreads();
  }

  // partial sum of squares of each token row over this k-range (32 threads per token)
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) ssq += __shfl_xor(ssq, o, 64);
  if ((tid & 31) == 0 && t0 + s_tt < T) p.part[(size_t)p.ksplit * T * E + (size_t)ks * T + t0 + s_tt] = ssq;

  // partial logits: lane holds expert e0 + ln, tokens t0 + 4 lq + i
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int e = e0[j] + ln;
    if (!act[j] || e >= E) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * lq + i;
      if (t < T) p.part[((size_t)ks * T + t) * E + e] = acc[j][i];
    }
  }
}

// Orders the wave's logits for selection: a larger key is a better expert.
// The high word is the logit mapped to an unsigned integer that sorts like
// the float (-0 folded into +0, so the two compare equal as floats do); the
// low word is 0xffff - e, so among equal logits the lower index wins.  Every
// real key is non-zero, which leaves 0 free to pad the table.
__device__ __forceinline__ unsigned long long select_key(float v, int e) {
  uint32_t u = v == 0.f ? 0u : __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(0xffff - e);
}

// Lanes of one wave exchange data through LDS: this orders the stores before
// the loads that follow (a wave's LDS operations complete in issue order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per token; NI = ceil(E / 64) logits per lane (expert lane + 64 i).
// Top-k by a radix select of the k-th largest key (ties to the lower
// expert), then the k selected keys rank each other; the logit of rank r
// lands in slot r, which is the descending order the softmax and the outputs
// take.
template <int NI>
__global__ __launch_bounds__(256) void route_topk_kernel(const RouteArgs p) {
  __shared__ __align__(16) unsigned long long s_key[4][64 * NI];
  __shared__ float s_sv[4][16];
  __shared__ int s_se[4][16];
  __shared__ float s_pes[4][16];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= p.T) return;  // whole wave leaves; only wave-level syncs below
  const int E = p.E, T = p.T;

  // per_expert_scale and the logit offset of this lane's experts, loaded with
  // the partials (not after the ranking: one round trip fewer)
  float pes_v[NI], bias_v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int e = lane + 64 * i;
    pes_v[i] = (e < E) ? bf16_bits_to_f32(p.pes[e]) : 0.f;
    bias_v[i] = (e < E && p.logit_bias) ? p.logit_bias[e] : 0.f;
  }
  // The logit kernel works on the un-normalised row: the norm is one positive
  // factor per token, 1 / sqrt(mean(x^2) + eps), applied here.  All partial
  // loads of a batch are issued before any is summed (fixed q order).
  float part[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) part[i] = 0.f;
  float ss = 0.f;
  const float* pb = p.part + (size_t)t * E + lane;
  const float* pss = p.part + (size_t)p.ksplit * T * E + t;
  const size_t pstride = (size_t)T * E;
  constexpr int kBatch = 16;  // partial loads in flight (the k-range split is at most 16 at 256 tokens)
  for (int q0 = 0; q0 < p.ksplit; q0 += kBatch) {
    float lv[kBatch][NI], sv[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const bool qok = q0 + q < p.ksplit;
      sv[q] = qok ? pss[(size_t)(q0 + q) * T] : 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) lv[q][i] = (qok && lane + 64 * i < E) ? pb[(q0 + q) * pstride + 64 * i] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      ss += sv[q];
#pragma unroll
      for (int i = 0; i < NI; ++i) part[i] += lv[q][i];
    }
  }
  const float rs = 1.0f / sqrtf(ss / (float)p.H + p.eps);

  float v[NI];
  unsigned long long key[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int e = lane + 64 * i;
    v[i] = -INFINITY;
    key[i] = 0;
    if (e < E) {
      float s = part[i] * rs;
      if (p.logit_bias) s += bias_v[i];
      if (p.logits_out) p.logits_out[(size_t)t * E + e] = s;
      v[i] = (s != s) ? -INFINITY : s;  // NaN never wins
      key[i] = select_key(v[i], e);
    }
  }

  // The k-th largest of the keys' high words (the logits in an order-keeping
  // integer form) by a radix select, one bit per step from the top, each
  // step counting with one ballot per key slot; then the keys above it and,
  // among those equal to it, the lowest experts are the selected ones.
  // Their order: each counts the selected 64-bit keys above its own.
  uint32_t hk[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) hk[i] = (uint32_t)(key[i] >> 32);  // 0 past E: below every real key
  auto count_ge = [&](uint32_t t) __attribute__((always_inline)) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) n += __popcll(__ballot(hk[i] >= t));
    return n;
  };
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    if (count_ge(cand) >= p.k) tau = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) n_gt += __popcll(__ballot(hk[i] > tau));
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int eq_before = 0, sel_before = 0;  // equal keys / selected keys of lower experts (slots i' < i, then lanes)
  bool sel[NI];
  int slot[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const unsigned long long eqm = __ballot(hk[i] == tau && key[i] != 0);
    const bool eq = hk[i] == tau && key[i] != 0;
    sel[i] = key[i] != 0 && (hk[i] > tau || (eq && n_gt + eq_before + __popcll(eqm & lt) < p.k));
    const unsigned long long sm = __ballot(sel[i]);
    slot[i] = sel_before + __popcll(sm & lt);
    eq_before += __popcll(eqm);
    sel_before += __popcll(sm);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i)
    if (sel[i]) s_key[wv][slot[i]] = key[i];  // the k selected keys, compacted
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (!sel[i]) continue;
    int rank = 0;
    for (int t = 0; t < p.k; ++t) rank += (int)(s_key[wv][t] > key[i]);
    s_sv[wv][rank] = v[i];
    s_se[wv][rank] = lane + 64 * i;
    s_pes[wv][rank] = pes_v[i];
  }
  wave_lds_sync();

  if (lane < p.k) {
    const float m = s_sv[wv][0];
    float sum = 0.f;
    for (int j = 0; j < p.k; ++j) sum += expf(s_sv[wv][j] - m);
    const int e = s_se[wv][lane];
    const float pj = expf(s_sv[wv][lane] - m) / sum;
    const float pes = s_pes[wv][lane];
    p.indices[(size_t)t * p.k + lane] = e;
    p.weights[(size_t)t * p.k + lane] = pj * pes;
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int tiles = (a.T + kTT - 1) / kTT;
  const dim3 grid1(tiles, a.ksplit);
  if (a.E <= 128)
    hipLaunchKernelGGL(route_logits_kernel<1>, grid1, dim3(kRThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(route_logits_kernel<2>, grid1, dim3(kRThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid2((a.T + 3) / 4);
  if (a.E <= 64)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid2, dim3(256), 0, stream, a);
  else if (a.E <= 128)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid2, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(route_topk_kernel<4>, grid2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qmoe

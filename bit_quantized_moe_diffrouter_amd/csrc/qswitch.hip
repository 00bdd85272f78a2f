// 4-bit switch linears (gate_up + GeGLU, down + weighted combine) and the
// dense 4-bit linear for gfx950.
//
// What is computed (diffusion-gemma model.ts page, DiffExperts.forward):
// every sorted row r of expert e multiplies its activation row by the
// dequantized weight of e; gate_up splits the 2I outputs at I and applies
// GeGLU (gelu_approx(gate) * up, vision.ts page, DiffVisionMLP); down scales
// each row by its routing weight for the per-token sum over k.
//
// How.  A workgroup (4 waves) owns a work item = (expert, chunk of up to BM
// sorted rows, tile of output columns).  The persistent grid walks the items
// derived on the device from expert_offsets, so no host synchronisation is
// needed for routing-dependent sizes.  Per 64-wide quantization group:
//  * each wave streams its own weight rows straight from HBM into registers
//    (8 bytes per lane, prefetched KS groups ahead) and turns every code into
//    the exact bf16 value 128 + q with two integer ops per pair;
//  * the activation chunk is staged once per workgroup in LDS, in the k order
//    the code unpacking produces;
//  * v_mfma_f32_16x16x32_bf16 forms P = sum_k x_k (128 + q_k) and, against a
//    ones operand, X = sum_k x_k; the group's affine is applied in fp32:
//        sum_k x_k (s q_k + b) = s P + (b - 128 s) X.
// All products are exact and the dequantized weight is never rounded, so the
// only roundings are fp32 accumulation (and the bf16 output).
#include "common.h"
#include "launch.h"

namespace qmoe {

enum : int { MODE_GATE_UP = 0, MODE_DOWN = 1, MODE_DENSE = 2 };

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

template <int MODE, int MT, int NS, int KS>
__global__ __launch_bounds__(kThreads) void qswitch_kernel(const SwitchArgs p) {
  constexpr int BM = 16 * MT;                 // rows per work item
  constexpr int ROWB = KS * 128 + 16;         // LDS bytes per staged row (padded)
  constexpr int CHUNKS = BM * KS * 8;         // 16-byte pieces per stage
  constexpr int CPT = CHUNKS / kThreads;      // pieces per thread
  static_assert(CHUNKS % kThreads == 0, "stage must split evenly over the workgroup");
  constexpr int NSH = (MODE == MODE_GATE_UP) ? NS / 2 : NS;  // output subtiles per wave
  static_assert(MODE != MODE_GATE_UP || NS % 2 == 0, "gate_up pairs gate and up subtiles");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * ROWB];
  __shared__ int s_cum[kThreads + 2];
  __shared__ int s_scan[kWaves];
  __shared__ int s_src[BM];
  __shared__ int s_dst[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lq = lane >> 4;
  const int K = p.K, G = K / kGroup, KW = K / 8;

  // ---- work decomposition: chunks of BM rows per expert bucket
  const int nb = (MODE == MODE_DOWN) ? p.E + 1 : p.E;  // down also zero-fills dropped rows
  int total_chunks;
  if constexpr (MODE == MODE_DENSE) {
    total_chunks = (p.rows_total + BM - 1) / BM;
  } else {
    auto bucket_chunks = [&](int e) {
      const int A = p.rows_total;
      int lo = min(max(p.offsets[e], 0), A);
      int hi = (e < p.E) ? min(max(p.offsets[e + 1], lo), A) : A;
      return (hi - lo + BM - 1) / BM;
    };
    const int c0 = (tid < nb) ? bucket_chunks(tid) : 0;
    const int c1 = (tid == kThreads - 1 && nb > kThreads) ? bucket_chunks(kThreads) : 0;
    int tot;
    const int incl = block_inclusive_scan<kThreads>(c0 + c1, s_scan, &tot);
    if (tid < nb) s_cum[tid + 1] = incl - c1;
    if (c1 > 0 || (tid == kThreads - 1 && nb > kThreads)) s_cum[kThreads + 1] = incl;
    if (tid == 0) s_cum[0] = 0;
    total_chunks = tot;
    __syncthreads();
  }
  const int total_items = total_chunks * p.ntiles;

  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    const int chunk = item / p.ntiles;
    const int ntile = item - chunk * p.ntiles;
    int e = 0, r0, rows;
    bool zero_only = false;
    if constexpr (MODE == MODE_DENSE) {
      r0 = chunk * BM;
      rows = min(BM, p.rows_total - r0);
    } else {
      int lo = 0, hi = nb;  // s_cum[lo] <= chunk < s_cum[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_cum[mid] <= chunk) lo = mid; else hi = mid;
      }
      e = lo;
      const int A = p.rows_total;
      const int seg_lo = min(max(p.offsets[e], 0), A);
      const int seg_hi = (e < p.E) ? min(max(p.offsets[e + 1], seg_lo), A) : A;
      r0 = seg_lo + (chunk - s_cum[e]) * BM;
      rows = min(BM, seg_hi - r0);
      zero_only = (MODE == MODE_DOWN) && (e == p.E);
    }

    __syncthreads();  // the previous item is done with s_src / s_dst / lds_a
    if (tid < BM) {
      const int r = r0 + tid;
      int src = -1, dst = -1;
      if (tid < rows) {
        if constexpr (MODE == MODE_DENSE) {
          src = r;
          dst = r;
        } else {
          const int a = p.assign[r];
          const bool ok = (a >= 0) && (a < p.rows_total);
          if constexpr (MODE == MODE_GATE_UP) {
            src = ok ? a / p.ktop : -1;
            dst = r;
          } else {
            src = r;
            dst = ok ? a : -1;
          }
        }
      }
      s_src[tid] = src;
      s_dst[tid] = dst;
    }
    __syncthreads();

    // ---- this wave's output subtiles and weight rows
    int wrow[NS], ocol[NSH];
    bool act[NS];
#pragma unroll
    for (int j = 0; j < NSH; ++j) {
      const int c = ntile * (kWaves * 16 * NSH) + wave * (16 * NSH) + 16 * j;
      ocol[j] = c;
      act[j] = c < p.Nout;
      wrow[j] = c;
      if constexpr (MODE == MODE_GATE_UP) {
        act[NSH + j] = act[j];
        wrow[NSH + j] = p.Nout + c;
      }
    }

    f32x4_t acc[MT][NS];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[m][j] = zero4();

    if (!zero_only) {
      const uint32_t* wp[NS];
      const uint16_t* sp[NS];
      const uint16_t* bp[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const size_t row = (size_t)e * p.Nw + (size_t)(act[j] ? wrow[j] + ln : 0);
        wp[j] = p.w + row * KW + 2 * lq;
        sp[j] = p.s + row * G;
        bp[j] = p.b + row * G;
      }

      // weight prefetch ring: slot = group % KS
      u32x2_t wr[KS][NS];
      uint32_t sr[KS][NS], br[KS][NS];
#pragma unroll
      for (int sl = 0; sl < KS; ++sl)
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if (act[j] && sl < G) {
            wr[sl][j] = *(const u32x2_t*)(wp[j] + sl * 8);
            sr[sl][j] = sp[j][sl];
            br[sl][j] = bp[j][sl];
          } else {
            wr[sl][j] = u32x2_t{0u, 0u};
            sr[sl][j] = 0u;
            br[sl][j] = 0u;
          }
        }

      // activation staging: piece c -> row c/(KS*8), group c/8 % KS, block c%8
      u32x4_t areg[CPT];
      auto load_stage = [&](int st) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          const int c = tid + kThreads * i;
          const int row = c / (KS * 8), rem = c % (KS * 8);
          const int g = st * KS + (rem >> 3), blk = rem & 7;
          const int src = s_src[row];
          if (src >= 0 && g < G)
            areg[i] = *(const u32x4_t*)(p.a + (size_t)src * K + g * kGroup + blk * 8);
          else
            areg[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
      };
      auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          const int c = tid + kThreads * i;
          const int row = c / (KS * 8), rem = c % (KS * 8);
          *(u32x4_t*)(&lds_a[buf][row * ROWB + (rem >> 3) * 128 + (rem & 7) * 16]) =
              permute_pairs(areg[i]);
        }
      };

      load_stage(0);
      store_stage(0);
      __syncthreads();

      const int NST = (G + KS - 1) / KS;
      for (int st = 0; st < NST; ++st) {
        const int buf = st & 1;
        if (st + 1 < NST) load_stage(st + 1);
#pragma unroll
        for (int gl = 0; gl < KS; ++gl) {
          const int g = st * KS + gl;
          if (g < G) {
            u32x4_t b0[NS], b1[NS];
            float sc[NS], cc[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j) {
              b0[j] = unpack_offset_codes(wr[gl][j].x);
              b1[j] = unpack_offset_codes(wr[gl][j].y);
              sc[j] = bf16_bits_to_f32(sr[gl][j]);
              cc[j] = bf16_bits_to_f32(br[gl][j]) - 128.0f * sc[j];
            }
            // refill this slot with group g + KS
            const int gn = g + KS;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
              if (act[j] && gn < G) {
                wr[gl][j] = *(const u32x2_t*)(wp[j] + gn * 8);
                sr[gl][j] = sp[j][gn];
                br[gl][j] = bp[j][gn];
              }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              const uint8_t* base = &lds_a[buf][(16 * m + ln) * ROWB + gl * 128 + lq * 32];
              const u32x4_t a0 = *(const u32x4_t*)base;
              const u32x4_t a1 = *(const u32x4_t*)(base + 16);
              f32x4_t X = mfma16x16x32(a0, ones, zero4());
              X = mfma16x16x32(a1, ones, X);
#pragma unroll
              for (int j = 0; j < NS; ++j) {
                if (act[j]) {
                  f32x4_t P = mfma16x16x32(a0, b0[j], zero4());
                  P = mfma16x16x32(a1, b1[j], P);
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    acc[m][j][i] = __builtin_fmaf(cc[j], X[i], __builtin_fmaf(sc[j], P[i], acc[m][j][i]));
                }
              }
            }
          }
        }
        if (st + 1 < NST) store_stage(buf ^ 1);
        __syncthreads();
      }
    }

    // ---- epilogue: lane holds column ocol[j] + ln, rows 16m + 4lq + i
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = 16 * m + 4 * lq + i;
        if (lr >= rows) continue;
        if constexpr (MODE == MODE_GATE_UP) {
          uint16_t* out = (uint16_t*)p.out;
          const size_t orow = (size_t)s_dst[lr] * p.Nout;
#pragma unroll
          for (int j = 0; j < NSH; ++j) {
            if (!act[j]) continue;
            const float gte = acc[m][j][i], up = acc[m][NSH + j][i];
            out[orow + ocol[j] + ln] = f32_to_bf16_bits(gelu_tanh(gte) * up);
          }
        } else if constexpr (MODE == MODE_DOWN) {
          const int a = s_dst[lr];
          if (a < 0) continue;
          float* out = (float*)p.out;
          const float wgt = zero_only ? 0.0f : p.route_w[a];
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            if (!act[j]) continue;
            out[(size_t)a * p.Nout + ocol[j] + ln] = zero_only ? 0.0f : wgt * acc[m][j][i];
          }
        } else {
          uint16_t* out = (uint16_t*)p.out;
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            if (!act[j]) continue;
            out[(size_t)(r0 + lr) * p.Nout + ocol[j] + ln] = f32_to_bf16_bits(acc[m][j][i]);
          }
        }
      }
    }
  }
}

// y[t, h] = bf16( sum_{j<k} D[t*k + j, h] ), summed in j order (fp32).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ D, int T, int k, int H,
                                                      uint16_t* __restrict__ y) {
  const int H4 = H / 4;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * H4) return;
  const int t = (int)(idx / H4), h = (int)(idx - (long long)t * H4) * 4;
  const float* base = D + (size_t)t * k * H + h;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float4 v = *(const float4*)(base + (size_t)j * H);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  u32x2_t o;
  o.x = pack_bf16x2(s.x, s.y);
  o.y = pack_bf16x2(s.z, s.w);
  *(u32x2_t*)(y + (size_t)t * H + h) = o;
}

// ------------------------------------------------------------------ launchers
namespace {
constexpr int kMT = 2, kKS = 4;
constexpr int kBM = 16 * kMT;
constexpr int kWgPerCu = 4;

template <int MODE, int NS>
hipError_t launch_switch(SwitchArgs a, int extra_buckets, int num_cu, hipStream_t stream) {
  constexpr int NSH = (MODE == MODE_GATE_UP) ? NS / 2 : NS;
  const int cols = kWaves * 16 * NSH;
  a.ntiles = (a.Nout + cols - 1) / cols;
  long long chunks;
  if (MODE == MODE_DENSE)
    chunks = (a.rows_total + kBM - 1) / kBM;
  else
    chunks = (a.rows_total + kBM - 1) / kBM + (long long)min(a.E, a.rows_total) + extra_buckets;
  long long items = chunks * a.ntiles;
  long long grid = min(items, (long long)num_cu * kWgPerCu);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((qswitch_kernel<MODE, kMT, NS, kKS>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gate_up_geglu(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_switch<MODE_GATE_UP, 2>(a, 0, num_cu, stream);
}
hipError_t launch_down(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_switch<MODE_DOWN, 2>(a, 1, num_cu, stream);
}
hipError_t launch_dense(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_switch<MODE_DENSE, 2>(a, 0, num_cu, stream);
}
hipError_t launch_combine(const float* D, int T, int k, int H, uint16_t* y, hipStream_t stream) {
  const long long n = (long long)T * (H / 4);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, D, T, k, H, y);
  return hipGetLastError();
}

}  // namespace qmoe

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
//  * each wave streams its own weight rows from HBM straight into a private
//    LDS ring with global_load_lds_dwordx4 (no VGPRs held while in flight;
//    the ring keeps D groups outstanding) and reads them one group ahead;
//  * every code becomes the exact bf16 value 128 + q with one v_and_or_b32
//    per pair (see unpack_offset_codes);
//  * the activation chunk and the group scales/biases are staged once per
//    workgroup in LDS, the activations in the k order the unpacking produces;
//  * v_mfma_f32_16x16x32_bf16 forms P = sum_k x_k (128 + q_k) and, against a
//    ones operand, X = sum_k x_k; the group's affine is applied in fp32:
//        sum_k x_k (s q_k + b) = s P + (b - 128 s) X.
// All products are exact and the dequantized weight is never rounded, so the
// only roundings are fp32 accumulation (and the bf16 output).
//
// The compiler does not order LDS reads after the LDS DMA that fills them,
// so the ring waits are explicit: every wave issues the same vector-memory
// operations in the same order, and the wait before reading group g+1 counts
// exactly the operations issued after that group's DMA (RING_WAIT below).
#include "common.h"
#include "launch.h"

#define QMOE_AS_GLOBAL __attribute__((address_space(1)))
#define QMOE_AS_LDS __attribute__((address_space(3)))

namespace qmoe {

enum : int { MODE_GATE_UP = 0, MODE_DOWN = 1, MODE_DENSE = 2 };

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

#ifndef QMOE_SWITCH_WAVES_PER_SIMD
#define QMOE_SWITCH_WAVES_PER_SIMD 2
#endif

// The switch kernels move every operand with LDS DMA (global_load_lds_*),
// issued from inline asm so the compiler neither reorders them nor adds its
// own (conservative) waits; the waits below are placed by hand from the fixed
// per-wave issue order (see the pipeline description in the kernel).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)((QMOE_AS_LDS const void*)p);
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 64 lanes x 16 bytes from per-lane global addresses to lds + 16 * lane.
__device__ __forceinline__ void dma_b128(const void* g, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform LDS base for M0
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(g) : "memory", "m0");
}
// 64 lanes x 4 bytes to lds + 4 * lane.
__device__ __forceinline__ void dma_b32(const void* g, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform LDS base for M0
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds), "v"(g) : "memory", "m0");
}
// 64 lanes x 2 bytes, each zero-extended into the 4-byte slot lds + 4 * lane.
__device__ __forceinline__ void dma_u16(const void* g, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform LDS base for M0
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, off"
               :: "s"(lds), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

template <int MODE, int MT, int NS, int KS, bool SBVEC>
__global__ __launch_bounds__(kThreads, QMOE_SWITCH_WAVES_PER_SIMD) void qswitch_kernel(const SwitchArgs p) {
  constexpr int BM = 16 * MT;                 // rows per work item
  constexpr int CHUNKS = BM * KS * 8;         // 16-byte activation pieces per stage
  static_assert(CHUNKS % kThreads == 0, "stage must split evenly over the workgroup");
  static_assert(BM % 8 == 0, "row-xor swizzle spans 8 rows");
  constexpr int NSH = (MODE == MODE_GATE_UP) ? NS / 2 : NS;  // output subtiles per wave
  static_assert(MODE != MODE_GATE_UP || NS % 2 == 0, "gate_up pairs gate and up subtiles");
  static_assert(NS == 2, "one 1 KB ring slot per group holds two 16-row subtiles");
  constexpr int SB_ROWS = kWaves * NS * 16;   // weight rows of the workgroup
#ifndef QMOE_SWITCH_STAGES_AHEAD
#define QMOE_SWITCH_STAGES_AHEAD 4
#endif
  // stages issued ahead of the one computed (the scalar scale path stages twice
  // the scale bytes, so it keeps one stage less to stay within 80 KB of LDS)
  constexpr int R = SBVEC ? QMOE_SWITCH_STAGES_AHEAD : QMOE_SWITCH_STAGES_AHEAD - 1;
  constexpr int D = R * KS;                    // weight ring depth (groups in flight per wave)
  static_assert(R >= 2, "at least two stages ahead");
  static_assert(2 * SB_ROWS == kThreads, "one thread per (row, scale|bias)");
  static_assert(!SBVEC || KS % 2 == 0, "vector scale loads read group pairs");
  // Pipeline (per wave, all DMA).  Stage s = KS groups; its activation pieces and
  // scales (shared by the workgroup) live in slot s % (R+1) of a ring, and each
  // wave's two 16-row weight subtiles of group g live in slot g % D of the
  // wave's private ring.  Issue order, which every wave follows exactly:
  //   prologue:   for s < R: act/scales(s), weights(s*KS .. s*KS+KS-1)
  //   stage st:   [wait act/scales(st)] barrier; act/scales(st+R);
  //               per group g: [wait weights(g+1)] read them; compute g; weights(g+D)
  // so the activations of a stage always precede its weights in the in-order
  // vmcnt counter and no wait drains the ring.  Ops issued after the one each
  // wait needs (checked against a simulation of this order):
  //   first ring read:       D - 1 + (R-1) LA
  //   act/scales(st):        KS + (R-1)(LA+KS)
  //   weights(g+1):          KS - 2 + (R-1)(LA+KS) + LA   (gl < KS-1)
  //                          2(KS-1) + (R-2)(LA+KS) + LA  (gl = KS-1)
  constexpr int APW = CHUNKS / kThreads;               // activation DMAs per wave per stage
  constexpr int SPW = SBVEC ? KS / 2 : KS;             // scale DMAs per wave per stage
  constexpr int LA = APW + SPW;
  constexpr int N_W0 = D - 1 + (R - 1) * LA;
  constexpr int N_ACT = KS + (R - 1) * (LA + KS);
  constexpr int N_RING = KS - 2 + (R - 1) * (LA + KS) + LA;
  constexpr int N_RING_LAST = 2 * (KS - 1) + (R - 2) * (LA + KS) + LA;
  static_assert(N_RING < 64 && N_W0 < 64 && N_ACT < 64, "wait counts must fit vmcnt");
  constexpr int A_BYTES = CHUNKS * 16;                 // activation bytes per stage
  constexpr int S_WORDS = SPW * kThreads;              // 4-byte scale slots per stage

  // activations of a stage: piece p = (gl * BM + row) * 8 + (blk ^ (row & 7)) at 16 p
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[R + 1][A_BYTES];
  // scales: slot [q][t], t = 2 * row + (0: scale, 1: bias); q = group pair (vector
  // path, two bf16 per slot) or group (scalar path, one zero-extended bf16)
  __shared__ __attribute__((aligned(16))) uint32_t lds_s[R + 1][S_WORDS];
  // per-wave weight ring: slot = group % D, 2 subtiles x 16 rows x 32 bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[kWaves][D][1024];
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
    if (tid == kThreads - 1 && nb > kThreads) s_cum[kThreads + 1] = incl;
    if (tid == 0) s_cum[0] = 0;
    total_chunks = tot;
    __syncthreads();
  }
  const int total_items = total_chunks * p.ntiles;

  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const OffsetCodeConsts kc = offset_code_consts();

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
      e = __builtin_amdgcn_readfirstlane(lo);
      const int A = p.rows_total;
      const int seg_lo = min(max(p.offsets[e], 0), A);
      const int seg_hi = (e < p.E) ? min(max(p.offsets[e + 1], seg_lo), A) : A;
      r0 = seg_lo + (chunk - s_cum[e]) * BM;
      rows = min(BM, seg_hi - r0);
      zero_only = (MODE == MODE_DOWN) && (e == p.E);
    }

    __syncthreads();  // the previous item is done with s_src / s_dst / lds_a / lds_sb
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

    // weight row (within the expert) of the workgroup's row slot t: wave t/(16 NS),
    // subtile t/16 % NS, row t % 16; rows of column tiles past the end map to a
    // valid row (computed on, never stored)
    auto wg_row = [&](int t) {
      const int tw = t / (16 * NS), tj = (t / 16) % NS, tn = t % 16;
      int c, row;
      if constexpr (MODE == MODE_GATE_UP) {
        c = ntile * (kWaves * 16 * NSH) + tw * (16 * NSH) + 16 * (tj % NSH);
        row = (tj < NSH) ? c : p.Nout + c;
      } else {
        c = ntile * (kWaves * 16 * NS) + tw * (16 * NS) + 16 * tj;
        row = c;
      }
      return (c < p.Nout ? row : 0) + tn;
    };
    // this wave's output subtiles
    int ocol[NSH];
    bool act[NSH];
#pragma unroll
    for (int j = 0; j < NSH; ++j) {
      ocol[j] = ntile * (kWaves * 16 * NSH) + wave * (16 * NSH) + 16 * j;
      act[j] = ocol[j] < p.Nout;
    }

    f32x4_t acc[MT][NS];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[m][j] = zero4();

    if (!zero_only) {
      // weight DMA: lane -> (subtile l/32, row l/2 % 16, half l % 2) of the 32-byte
      // group segment; past the last group it reloads the last one (not used)
      const uint32_t* wsrc =
          p.w + ((size_t)e * p.Nw + wg_row(wave * 32 + (lane >> 1))) * KW + (lane & 1) * 4;
      const uint8_t* ring = &lds_w[wave][0][0];
      const uint32_t ring_lds = lds_addr(ring);
      auto dma_weights = [&](int g) { dma_b128(wsrc + min(g, G - 1) * 8, ring_lds + (g % D) * 1024); };

      // scale DMA: thread t = 2 * row + which copies scale (which 0) or bias of row
      const uint16_t* ssrc = ((tid & 1) ? p.b : p.s) + ((size_t)e * p.Nw + wg_row(tid >> 1)) * G;
      // activation DMA: instruction i of this wave fills pieces (i * kWaves + wave) * 64 + lane
      const uint16_t* asrc[APW];
#pragma unroll
      for (int i = 0; i < APW; ++i) {
        const int pc = (i * kWaves + wave) * 64 + lane;
        const int row = (pc >> 3) % BM, gl = (pc >> 3) / BM, blk = (pc & 7) ^ (row & 7);
        const int src = s_src[row];
        asrc[i] = p.a + (size_t)(src >= 0 ? src : 0) * K + gl * kGroup + blk * 8;
      }
      const int NST = (G + KS - 1) / KS;
      auto dma_stage = [&](int st, int buf) {  // exactly LA DMAs into activation/scale slot buf
        const int stc = min(st, NST - 1);  // past the end: the last stage again (not used)
#pragma unroll
        for (int i = 0; i < APW; ++i) {
          // groups past G (last partial stage) reload group G-1; they are skipped in compute
          const int gl = ((i * kWaves + wave) * 64 + lane) / (8 * BM);
          const int g = min(stc * KS + gl, G - 1);
          dma_b128(asrc[i] + (g - gl) * kGroup, lds_addr(&lds_a[buf][(i * kWaves + wave) * 1024]));
        }
        const int g0 = stc * KS;
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
          const uint32_t dst = lds_addr(&lds_s[buf][q * kThreads + wave * 64]);
          if constexpr (SBVEC)
            dma_b32(ssrc + g0 + 2 * q, dst);
          else
            dma_u16(ssrc + min(g0 + q, G - 1), dst);
        }
      };

      // ---- prologue: R stages, each activations/scales then its weights
#pragma unroll
      for (int s0 = 0; s0 < R; ++s0) {
        dma_stage(s0, s0);
#pragma unroll
        for (int gl = 0; gl < KS; ++gl) dma_weights(s0 * KS + gl);
      }
      wait_vmcnt<N_W0>();
      u32x2_t wcur[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) wcur[j] = *(const u32x2_t*)(ring + j * 512 + ln * 32 + lq * 8);

      int buf = 0, issue_buf = R;  // activation slots of the stage computed / being issued
      for (int st = 0; st < NST; ++st) {
        wait_vmcnt<N_ACT>();
        __syncthreads();  // stage st landed for every wave; stage st-1's slot is free
        dma_stage(st + R, issue_buf);
#pragma unroll
        for (int gl = 0; gl < KS; ++gl) {
          const int g = st * KS + gl;
          if (gl < KS - 1) wait_vmcnt<N_RING>(); else wait_vmcnt<N_RING_LAST>();
          u32x2_t wnext[NS];
#pragma unroll
          for (int j = 0; j < NS; ++j)
            wnext[j] = *(const u32x2_t*)(ring + ((g + 1) % D) * 1024 + j * 512 + ln * 32 + lq * 8);

          if (g < G) {
            u32x4_t b0[NS], b1[NS];
            float sc[NS], cc[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j) {
              b0[j] = unpack_offset_codes(wcur[j].x, kc);
              b1[j] = unpack_offset_codes(wcur[j].y, kc);
              const int t2 = 2 * (wave * (16 * NS) + 16 * j + ln);
              const u32x2_t sb = *(const u32x2_t*)&lds_s[buf][(SBVEC ? gl / 2 : gl) * kThreads + t2];
              const int sh = (SBVEC && (gl & 1)) ? 0 : 16;
              sc[j] = __uint_as_float(sh ? (sb.x << 16) : (sb.x & 0xffff0000u));
              const float bias = __uint_as_float(sh ? (sb.y << 16) : (sb.y & 0xffff0000u));
              cc[j] = bias - 128.0f * sc[j];
            }
            // all MFMAs of the group first, then the fp32 affine
            u32x4_t a0[MT], a1[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              const int row = 16 * m + ln;
              const uint8_t* base = &lds_a[buf][(gl * BM + row) * 128];
              a0[m] = permute_pairs(*(const u32x4_t*)(base + (((2 * lq) ^ (row & 7)) * 16)));
              a1[m] = permute_pairs(*(const u32x4_t*)(base + (((2 * lq + 1) ^ (row & 7)) * 16)));
            }
            f32x4_t X[MT], P[MT][NS];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              X[m] = mfma16x16x32(a0[m], ones, zero4());
#pragma unroll
              for (int j = 0; j < NS; ++j) P[m][j] = mfma16x16x32(a0[m], b0[j], zero4());
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              X[m] = mfma16x16x32(a1[m], ones, X[m]);
#pragma unroll
              for (int j = 0; j < NS; ++j) P[m][j] = mfma16x16x32(a1[m], b1[j], P[m][j]);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int j = 0; j < NS; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  acc[m][j][i] = __builtin_fmaf(cc[j], X[m][i], __builtin_fmaf(sc[j], P[m][j][i], acc[m][j][i]));
          }
          // refill the slot of group g (read into wcur one group ago) with group g + D
          dma_weights(g + D);
#pragma unroll
          for (int j = 0; j < NS; ++j) wcur[j] = wnext[j];
        }
        buf = (buf == R) ? 0 : buf + 1;
        issue_buf = (issue_buf == R) ? 0 : issue_buf + 1;
      }
      wait_vmcnt<0>();  // drain the tail (reloads) before the buffers are reused
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
// Tile shape of the switch kernels (overridable at build time for tuning sweeps).
#ifndef QMOE_SWITCH_MT
#define QMOE_SWITCH_MT 2
#endif
#ifndef QMOE_SWITCH_KS
#define QMOE_SWITCH_KS 2
#endif
#ifndef QMOE_SWITCH_WG_PER_CU
#define QMOE_SWITCH_WG_PER_CU 2
#endif
constexpr int kMT = QMOE_SWITCH_MT, kKS = QMOE_SWITCH_KS;
constexpr int kBM = 16 * kMT;
constexpr int kWgPerCu = QMOE_SWITCH_WG_PER_CU;  // resident workgroups per CU (LDS-bound)

template <int MODE, int NS>
hipError_t launch_switch(SwitchArgs a, int extra_buckets, int num_cu, hipStream_t stream) {
  constexpr int NSH = (MODE == MODE_GATE_UP) ? NS / 2 : NS;
  const int cols = kWaves * 16 * NSH;
  a.ntiles = (a.Nout + cols - 1) / cols;
  const int G = a.K / 64;
  a.sb_vec = (kKS % 2 == 0) && (G % kKS == 0) && ((uintptr_t)a.s % 4 == 0) && ((uintptr_t)a.b % 4 == 0);
  long long chunks;
  if (MODE == MODE_DENSE)
    chunks = (a.rows_total + kBM - 1) / kBM;
  else
    chunks = (a.rows_total + kBM - 1) / kBM + (long long)min(a.E, a.rows_total) + extra_buckets;
  long long items = chunks * a.ntiles;
  long long grid = min(items, (long long)num_cu * kWgPerCu);
  if (grid < 1) grid = 1;
  if (a.sb_vec)
    hipLaunchKernelGGL((qswitch_kernel<MODE, kMT, NS, kKS, kKS % 2 == 0>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((qswitch_kernel<MODE, kMT, NS, kKS, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
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

// Device helpers shared by the gfx950 kernels of the 4-bit MoE layer.
//
// Packed-code convention (the reading used across the library): code c of a
// weight row lives in uint32 word c/8, bits 4*(c%8)..4*(c%8)+3.  A group is 64
// codes (8 words) sharing one bf16 scale and one bf16 bias; the weight value
// is scale*q + bias.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <utility>

namespace qmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16_lo_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 -> one dword of two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Two packed words (codes n0..n7 each) -> four dwords of bf16 pairs per word
// holding 128+q exactly: 0x4300 | q is the bf16 pattern of 128 + q for
// q < 128.  The pairs come out as (n0,n4) (n1,n5) (n2,n6) (n3,n7): the
// activation operand is stored in the same order (see permute_pairs), or the
// codes are pre-placed so that this order is the natural one.  gfx9 VOP3
// encodings take no literal, so the mask rides in a scalar register and the
// exponent pattern in a vector register, making each pair one v_and_or_b32;
// one 64-bit shift moves the nibbles of both words at once (the bits of the
// second word that enter the first word's top nibble fall outside the mask),
// so two words take 3 shifts + 8 v_and_or_b32.
struct OffsetCodeConsts {
  uint32_t mask;  // 0x000F000F, uniform (SGPR)
  uint32_t expo;  // 0x43004300, in a VGPR
  int zero;       // 0, uniform, opaque to the compiler (below)
};
// All of this is plain C: a vector instruction written as inline asm is
// invisible to the compiler's hazard checks, and it once reused the unread
// upper half of an in-flight MFMA result as the asm's output register (the
// MFMA then overwrote the unpacked codes).  The exponent pattern comes from
// an add to v_mbcnt_lo(0, 0) (zero, but not known to be uniform), so it lives
// in a VGPR; the shift amounts are 4p plus a uniform zero the compiler cannot
// fold, so each stays one 64-bit shift instead of an alignbit and a shift.
__device__ __forceinline__ OffsetCodeConsts offset_code_consts() {
  OffsetCodeConsts k;
  k.mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  const uint32_t lane_zero = __builtin_amdgcn_mbcnt_lo(0u, 0u);
  k.expo = 0x43004300u + lane_zero;
  k.zero = __builtin_amdgcn_readfirstlane((int)lane_zero);
  return k;
}
// (a & smask) | vor: selected as one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t smask, uint32_t vor) { return (a & smask) | vor; }
__device__ __forceinline__ void unpack_offset_code_pair(uint32_t w0, uint32_t w1, const OffsetCodeConsts& k,
                                                        u32x4_t& b0, u32x4_t& b1) {
  const uint64_t pr = ((uint64_t)w1 << 32) | w0;
  b0[0] = and_or(w0, k.mask, k.expo);
  b1[0] = and_or(w1, k.mask, k.expo);
#pragma unroll
  for (int p = 1; p < 4; ++p) {
    const uint64_t sh = pr >> (k.zero + 4 * p);
    b0[p] = and_or((uint32_t)sh, k.mask, k.expo);
    b1[p] = and_or((uint32_t)(sh >> 32), k.mask, k.expo);
  }
}

// One word as unpack_offset_code_pair unpacks it, but with the smallest offset
// a bf16 bit trick allows for unit steps: 0x4180 | (q << 3) is the bf16
// pattern of 16 + q.
// The smaller offset keeps the MFMA partial sums small, so the fp32 rounding
// left after the affine correction is about 8x smaller (one more op per word).
__device__ __forceinline__ u32x4_t unpack_offset16_codes(uint32_t w) {
  const uint32_t M = 0x00780078u, C = 0x41804180u;
  u32x4_t r;
  r.x = ((w << 3) & M) | C;
  r.y = ((w >> 1) & M) | C;
  r.z = ((w >> 5) & M) | C;
  r.w = ((w >> 9) & M) | C;
  return r;
}

// Eight consecutive bf16 (x0..x7 as pairs (x0,x1)(x2,x3)(x4,x5)(x6,x7)) ->
// the order (x0,x4)(x1,x5)(x2,x6)(x3,x7) that matches unpack_offset_code_pair.
__device__ __forceinline__ u32x4_t permute_pairs(u32x4_t v) {
  u32x4_t o;
  o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return o;
}

// Two operand-ordered code words (code 2p at bits 4p, code 2p + 1 at bits
// 16 + 4p) -> eight dwords of bf16 pairs bf16(s q + b), codes (2p, 2p + 1)
// of word i in dword p of d_i.  The nibbles are spread to bytes with one mask
// (low nibbles: codes 0, 4, 1, 5; after one 64-bit shift of both words by 4,
// high nibbles: codes 2, 6, 3, 7) and each byte goes through one
// byte-to-float conversion (v_cvt_f32_ubyte0..3), one FMA, and half a pack:
// 47 instructions per 16 codes.  The mask and the shift amount come in as
// values the compiler cannot fold (DequantConsts): with a known mask it
// re-derives each code as a 4-bit field extract of the word and converts
// from byte 0, one more instruction per code.
struct DequantConsts {
  uint32_t mask;  // 0x0F0F0F0F, uniform
  int four;       // 4, uniform
};
__device__ __forceinline__ DequantConsts dequant_consts() {
  const int zero = __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_mbcnt_lo(0u, 0u));
  return DequantConsts{0x0F0F0F0Fu + (uint32_t)zero, 4 + zero};
}
__device__ __forceinline__ void dequant_pair_bf16(uint32_t w0, uint32_t w1, float s, float b, const DequantConsts& k,
                                                  u32x4_t& d0, u32x4_t& d1) {
  const uint64_t sh = (((uint64_t)w1 << 32) | w0) >> k.four;
  const uint32_t lo0 = w0 & k.mask, lo1 = w1 & k.mask;
  const uint32_t hi0 = (uint32_t)sh & k.mask, hi1 = (uint32_t)(sh >> 32) & k.mask;
  auto f = [&](uint32_t v, int byte) __attribute__((always_inline)) {
    return __builtin_fmaf(s, (float)((v >> (8 * byte)) & 0xFFu), b);
  };
  d0[0] = pack_bf16x2(f(lo0, 0), f(lo0, 2));
  d0[1] = pack_bf16x2(f(hi0, 0), f(hi0, 2));
  d0[2] = pack_bf16x2(f(lo0, 1), f(lo0, 3));
  d0[3] = pack_bf16x2(f(hi0, 1), f(hi0, 3));
  d1[0] = pack_bf16x2(f(lo1, 0), f(lo1, 2));
  d1[1] = pack_bf16x2(f(hi1, 0), f(hi1, 2));
  d1[2] = pack_bf16x2(f(lo1, 1), f(lo1, 3));
  d1[3] = pack_bf16x2(f(hi1, 1), f(hi1, 3));
}

// D = A(16x32 bf16) * B(32x16 bf16) + C, fp32 accumulate.  Lane l holds row
// (l%16) of A and column (l%16) of B over the k-slice of lane group l/16; the
// result holds column l%16, rows 4*(l/16)+0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// tanh-form GELU, written as z * sigmoid(2a), a = sqrt(2/pi) (z + 0.044715 z^3)
// (0.5 (1 + tanh a) == 1 / (1 + exp(-2a))).  The reciprocal is the hardware's
// (about 1 ulp): the product is rounded to bf16, 2^16 times coarser, and a
// correctly rounded division costs six more instructions per element in the
// epilogues.  exp(-2a) = inf gives 1 / inf = 0, the limit, for very negative z.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float a = k0 * (z + 0.044715f * z * z * z);
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * a));
}

__device__ __forceinline__ int wave_lane() { return threadIdx.x & 63; }

// Inclusive scan of one int per thread over a workgroup of NT threads
// (NT a multiple of 64, at most 1024).  `scratch` holds NT/64 ints.  Ends with
// a barrier; every thread gets its inclusive prefix and the total.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int s = scratch[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return v + before;
}

// Items of a kernel that gives a workgroup a chunk of BM sorted rows of one
// expert and one or more weight blocks (the tall-tile kernel on the gate_up
// switch linear): expert e's rows [offsets[e], offsets[e+1]) (clamped to
// [0, A)) are cut into chunks of BM rows, numbered expert by expert, blocks
// minor.  Also gives the first 16-row activation tile of the chunk (the
// experts' tiles numbered the same way).  The tables are built by every
// thread of an NT-thread workgroup (workgroup barriers); E <= 2 NT and
// E <= 256.
constexpr int kChunkMaxExperts = 256;
struct alignas(16) ExpertChunks {
  alignas(16) int cpre[kChunkMaxExperts + 4];  // chunks before each expert (read as int4 by 64 lanes)
  int lo[kChunkMaxExperts + 1];
  int hi[kChunkMaxExperts + 1];
  int tpre[kChunkMaxExperts + 1];  // activation tiles before each expert
  int scan[16];
};
static_assert(offsetof(ExpertChunks, cpre) == 0, "the int4 reads need cpre 16-byte aligned");
// The tables (every thread of the workgroup; ends with a barrier) ...
template <int NT, int BM>
__device__ __forceinline__ void expert_chunk_tables(ExpertChunks& sh, const int32_t* offsets, int E, int A) {
  const int tid = threadIdx.x;
  for (int b = tid; b < E; b += NT) {
    const int o0 = offsets[b], o1 = offsets[b + 1];
    const int lo = min(max(o0, 0), A);
    sh.lo[b] = lo;
    sh.hi[b] = min(max(o1, lo), A);
  }
  __syncthreads();
  auto scan = [&](int v) __attribute__((always_inline)) {  // exclusive prefix over experts (two per thread)
    int all;
    const int incl = block_inclusive_scan<NT>(v, sh.scan, &all);
    return incl - v;
  };
  int c0 = 0, c1 = 0, t0 = 0, t1 = 0;
  const int b0 = 2 * tid, b1 = 2 * tid + 1;
  if (b0 < E) {
    const int n = sh.hi[b0] - sh.lo[b0];
    c0 = (n + BM - 1) / BM;
    t0 = (n + 15) / 16;
  }
  if (b1 < E) {
    const int n = sh.hi[b1] - sh.lo[b1];
    c1 = (n + BM - 1) / BM;
    t1 = (n + 15) / 16;
  }
  const int cx = scan(c0 + c1);
  const int tx = scan(t0 + t1);
  if (b0 <= E) sh.cpre[b0] = cx, sh.tpre[b0] = tx;
  if (b1 <= E) sh.cpre[b1] = cx + c0, sh.tpre[b1] = tx + t0;
  if (tid < 3 && E + 1 + tid < kChunkMaxExperts + 4) sh.cpre[E + 1 + tid] = 0x7fffffff;  // int4 reads past the end
  __syncthreads();
}
// ... and the item at position pos (one wave's work, no barrier): chunk
// pos / nblk of the experts' chunks (sh.cpre[E] of them), block pos % nblk.
// Returns false when pos is past the last item.
template <int BM>
__device__ __forceinline__ bool expert_chunk_at(const ExpertChunks& sh, int E, int nblk, int pos, int& e, int& r0,
                                                int& rows, int& blk, int& tau0) {
  const int lane = threadIdx.x & 63;
  const int nch = sh.cpre[E];
  if (pos >= nch * nblk) return false;
  const int ch = pos / nblk;
  blk = pos - ch * nblk;
  // the expert holding chunk ch: the number of experts whose first chunk is
  // at most ch, less one, counted by the wave (lane l holds cpre[4l..4l+3])
  const int4 c4 = ((const int4*)sh.cpre)[lane];
  const int eb = 4 * lane;
  const int n = __popcll(__ballot(eb < E && c4.x <= ch)) + __popcll(__ballot(eb + 1 < E && c4.y <= ch)) +
                __popcll(__ballot(eb + 2 < E && c4.z <= ch)) + __popcll(__ballot(eb + 3 < E && c4.w <= ch));
  e = __builtin_amdgcn_readfirstlane(n - 1);
  r0 = __builtin_amdgcn_readfirstlane(sh.lo[e] + (ch - sh.cpre[e]) * BM);
  rows = __builtin_amdgcn_readfirstlane(min(BM, sh.hi[e] - r0));
  tau0 = __builtin_amdgcn_readfirstlane(sh.tpre[e] + (r0 - sh.lo[e]) / 16);
  blk = __builtin_amdgcn_readfirstlane(blk);
  return true;
}
}  // namespace qmoe

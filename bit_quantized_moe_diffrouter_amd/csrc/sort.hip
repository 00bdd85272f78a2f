// Token-by-expert sort for gfx950 (diffusion-gemma model.ts page,
// DiffExperts.forward: argsort of the flat routing indices, read as a stable
// sort).  One workgroup of 1024 threads; wave w owns the contiguous range
// [w L, (w + 1) L) of assignment ids, walked in chunks of 64:
//   0. up to 32768 assignments: their buckets are staged in LDS (many loads
//      in flight); larger inputs read them in step 1, one chunk ahead;
//   1. per chunk, each lane finds the lanes that share its bucket with one
//      ballot per bit of the bucket id (bucket E collects indices outside
//      [0, E), which are dropped) and ranks itself among them with a
//      popcount; adding the wave's running count of that bucket gives its
//      rank within the wave's range.  Up to 32768 assignments keep the rank
//      in LDS for step 3; larger inputs recompute bucket and rank there;
//   2. per bucket, exclusive prefix of the 16 wave counts, then the exclusive
//      prefix over buckets -> expert_offsets;
//   3. sorted_assign[base[b] + wave prefix[w][b] + rank] = a (up to 32768
//      assignments through an inverse permutation in LDS, then coalesced).
// Ranges and chunks are visited in ascending order, so equal experts keep
// ascending assignment ids, and the number of workgroup barriers does not
// grow with the number of assignments.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {
constexpr int kSThreads = 1024, kSWaves = kSThreads / 64;
constexpr int kMaxBuckets = 257;  // E <= 256, plus the dropped bucket
constexpr int kCacheMax = 32768;  // assignments whose bucket and rank stay in LDS between steps 1 and 3
}  // namespace

__global__ __launch_bounds__(kSThreads) void sort_kernel(const int32_t* __restrict__ idx, int A, int E,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_assign) {
  __shared__ int wcnt[kSWaves][kMaxBuckets];  // step 1: running counts; after step 2: exclusive wave prefixes
  __shared__ int base[kMaxBuckets];
  __shared__ int scan_tmp[kSWaves];
  // A <= kCacheMax: bucket of each assignment, then its rank within its
  // wave's range (< 2048); larger A: running counts of step 3 instead
  __shared__ __attribute__((aligned(16))) uint16_t cache[2 * kCacheMax];
  uint16_t* const bcache = cache;
  uint16_t* const rcache = cache + kCacheMax;
  int(*const wrun)[kMaxBuckets] = reinterpret_cast<int(*)[kMaxBuckets]>(cache);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = E + 1;
  const bool cached = A <= kCacheMax;
  for (int i = tid; i < kSWaves * kMaxBuckets; i += kSThreads) {
    (&wcnt[0][0])[i] = 0;
    if (!cached) (&wrun[0][0])[i] = 0;
  }
  auto bucket_of = [&](int a) __attribute__((always_inline)) {
    const int e = idx[a];
    return (e >= 0 && e < E) ? e : E;
  };
  // 0. the buckets of all assignments into LDS, eight loads in flight per thread
  if (cached) {
    for (int a0 = tid; a0 < A; a0 += 8 * kSThreads) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (a0 + u * kSThreads < A) ? bucket_of(a0 + u * kSThreads) : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (a0 + u * kSThreads < A) bcache[a0 + u * kSThreads] = (uint16_t)v[u];
    }
  }
  __syncthreads();

  // this wave's range, a whole number of 64-assignment chunks
  const int per_wave = ((A + kSWaves - 1) / kSWaves + 63) & ~63;
  const int r0 = wave * per_wave, r1 = min(r0 + per_wave, A);
  const int nbits = 32 - __builtin_clz((unsigned)E);  // bits of the largest bucket id, E
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // rank of this lane's assignment among the chunk's lanes of the same
  // bucket, and their number; invalid lanes take part in no group
  auto chunk_rank = [&](bool valid, int bk, int& cnt) __attribute__((always_inline)) {
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      if (bit >= nbits) break;  // uniform
      const bool b = (bk >> bit) & 1;
      const unsigned long long m = __ballot(valid && b);
      peers &= b ? m : ~m;
    }
    cnt = __popcll(peers);
    return __popcll(peers & lt_mask);
  };
  // Walks the wave's chunks in order; f(a, valid, bk, rank) with the rank of
  // assignment a within the wave's range, counted in run[wave][*].  Buckets
  // come from LDS (step 0) or, past the cache, from memory one chunk ahead.
  auto walk = [&](int (*run)[kMaxBuckets], auto f) __attribute__((always_inline)) {
    int nxt = (!cached && r0 + lane < r1) ? bucket_of(r0 + lane) : 0;
    for (int c0 = r0; c0 < r1; c0 += 64) {
      const int a = c0 + lane;
      const bool valid = a < r1;
      int bk;
      if (cached) {
        bk = valid ? (int)bcache[a] : 0;
      } else {
        bk = valid ? nxt : 0;
        if (c0 + 64 < r1) nxt = (c0 + 64 + lane < r1) ? bucket_of(c0 + 64 + lane) : 0;
      }
      int cnt;
      const int r = chunk_rank(valid, bk, cnt);
      const int before = valid ? run[wave][bk] : 0;  // every lane reads before the leaders write
      if (valid && r == 0) run[wave][bk] = before + cnt;
      f(a, valid, bk, before + r);
    }
  };

  // 1. ranks within the ranges and the ranges' bucket counts
  walk(wcnt, [&](int a, bool valid, int bk, int rank) __attribute__((always_inline)) {
    if (cached && valid) rcache[a] = (uint16_t)rank;
  });
  __syncthreads();

  // 2. per bucket: exclusive prefix over the waves, then over the buckets
  int total = 0;
  if (tid < NB) {
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = total;
      total += c;
    }
  }
  int all;
  const int incl = block_inclusive_scan<kSThreads>(total, scan_tmp, &all);
  if (tid < NB) {
    base[tid] = incl - total;
    offsets[tid] = incl - total;  // offsets[E] = start of the dropped bucket = valid count
  }
  __syncthreads();

  // 3. scatter.  Cached: each position into rcache (16 bits suffice), the
  // inverse permutation through LDS in place of the buckets, then coalesced
  // stores (one CU's scattered 4-byte stores would be the slowest part).
  if (cached) {
    for (int a = r0 + lane; a < r1; a += 64) {
      const int bk = bcache[a];
      rcache[a] = (uint16_t)(base[bk] + wcnt[wave][bk] + rcache[a]);
    }
    __syncthreads();
    for (int a = tid; a < A; a += kSThreads) bcache[rcache[a]] = (uint16_t)a;
    __syncthreads();
    for (int i = tid; i < A; i += kSThreads) sorted_assign[i] = bcache[i];
  } else {
    walk(wrun, [&](int a, bool valid, int bk, int rank) __attribute__((always_inline)) {
      if (valid) sorted_assign[base[bk] + wcnt[wave][bk] + rank] = a;
    });
  }
}

hipError_t launch_sort(const int32_t* indices, int A, int E, int32_t* offsets, int32_t* sorted_assign,
                       hipStream_t stream) {
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kSThreads), 0, stream, indices, A, E, offsets, sorted_assign);
  return hipGetLastError();
}

}  // namespace qmoe

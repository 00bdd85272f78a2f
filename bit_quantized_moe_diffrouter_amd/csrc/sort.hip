// Token-by-expert sort for gfx950 (diffusion-gemma model.ts page,
// DiffExperts.forward: argsort of the flat routing indices, read as a stable
// sort).
//
// A range of assignment ids is sorted by one workgroup of 1024 threads; wave
// w owns the contiguous part [w L, (w + 1) L) of the range, walked in chunks
// of 64:
//   0. up to 32768 assignments: their buckets are staged in LDS (many loads
//      in flight); larger ranges read them in step 1, one chunk ahead;
//   1. per chunk, each lane finds the lanes that share its bucket with one
//      ballot per bit of the bucket id (bucket E collects indices outside
//      [0, E), which are dropped) and ranks itself among them with a
//      popcount; adding the wave's running count of that bucket gives its
//      rank within the wave's part.  Up to 32768 assignments keep the rank
//      in LDS for step 3; larger ranges recompute bucket and rank there;
//   2. per bucket, exclusive prefix of the 16 wave counts; the bucket's start
//      in the output (below);
//   3. sorted_assign[start[b] + wave prefix[w][b] + rank] = a.
// One range (the whole input, a single workgroup): start = exclusive prefix
// over the range's own bucket counts; up to 32768 assignments the positions
// are inverted through LDS so the stores are coalesced.
// Slices (8192 assignments and more, with the workspace): the input is cut
// into at most 256 slices of a multiple of 1024 assignments.  A first kernel
// writes each slice's bucket histogram; in the second, slice s's workgroup
// sums the histograms of all slices (bucket totals, exclusive prefix over
// buckets = the expert offsets) and of the slices before s, so its bucket b
// starts at offsets[b] + (b's count in slices < s).
// Parts, chunks and slices are visited in ascending order, so equal experts
// keep ascending assignment ids, and the number of workgroup barriers does
// not grow with the number of assignments.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {
constexpr int kSThreads = 1024, kSWaves = kSThreads / 64;
constexpr int kMaxBuckets = 257;  // E <= 256, plus the dropped bucket
constexpr int kCacheMax = 32768;  // assignments whose bucket and rank stay in LDS between steps 1 and 3
constexpr int kSliceMin = 8192;   // inputs from which the slice sort runs (given its workspace)
constexpr int kMaxSlices = 256;

struct SlicePlan {
  int slice, nslice;
};
SlicePlan slice_plan(int A) {
  const int per = (A + kMaxSlices * 1024 - 1) / (kMaxSlices * 1024);  // 1024-assignment units per slice
  const int slice = 1024 * (per < 1 ? 1 : per);
  return {slice, (A + slice - 1) / slice};
}
}  // namespace

size_t sort_workspace_bytes(int A, int E) {
  if (A < kSliceMin || E < 1) return 0;
  return (size_t)slice_plan(A).nslice * (size_t)(E + 1) * sizeof(int32_t);
}

// Slice histograms: cnt[s * (E + 1) + b] = assignments of slice s in bucket b.
__global__ __launch_bounds__(kSThreads) void sort_hist_kernel(const int32_t* __restrict__ idx, int A, int E, int S,
                                                              int32_t* __restrict__ cnt) {
  __shared__ int hist[kMaxBuckets];
  const int NB = E + 1, tid = threadIdx.x;
  const int lo = blockIdx.x * S, hi = min(lo + S, A);
  for (int i = tid; i < NB; i += kSThreads) hist[i] = 0;
  __syncthreads();
  for (int a = lo + tid; a < hi; a += kSThreads) {
    const int e = idx[a];
    atomicAdd(&hist[(e >= 0 && e < E) ? e : E], 1);
  }
  __syncthreads();
  for (int i = tid; i < NB; i += kSThreads) cnt[(size_t)blockIdx.x * NB + i] = hist[i];
}

// kSlices = false: one workgroup sorts [0, A).  kSlices = true: workgroup s
// sorts slice [s S, min((s + 1) S, A)) given the nslice histograms in cnt.
template <bool kSlices>
__global__ __launch_bounds__(kSThreads) void sort_kernel(const int32_t* __restrict__ idx, int A, int E, int S,
                                                         int nslice, const int32_t* __restrict__ cnt,
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
  const int lo = kSlices ? blockIdx.x * S : 0;
  const int hi = kSlices ? min(lo + S, A) : A;
  const int n = hi - lo;  // this workgroup's range [lo, hi)
  const bool cached = n <= kCacheMax;
  for (int i = tid; i < kSWaves * kMaxBuckets; i += kSThreads) {
    (&wcnt[0][0])[i] = 0;
    if (!cached) (&wrun[0][0])[i] = 0;
  }
  auto bucket_of = [&](int a) __attribute__((always_inline)) {
    const int e = idx[a];
    return (e >= 0 && e < E) ? e : E;
  };
  // 0. the buckets of the range into LDS (index a - lo), eight loads in flight per thread
  if (cached) {
    for (int a0 = tid; a0 < n; a0 += 8 * kSThreads) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (a0 + u * kSThreads < n) ? bucket_of(lo + a0 + u * kSThreads) : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (a0 + u * kSThreads < n) bcache[a0 + u * kSThreads] = (uint16_t)v[u];
    }
  }
  __syncthreads();

  // this wave's part of the range, a whole number of 64-assignment chunks
  const int per_wave = ((n + kSWaves - 1) / kSWaves + 63) & ~63;
  const int r0 = lo + wave * per_wave, r1 = min(r0 + per_wave, hi);
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
        bk = valid ? (int)bcache[a - lo] : 0;
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
    if (cached && valid) rcache[a - lo] = (uint16_t)rank;
  });
  __syncthreads();

  // 2. per bucket: exclusive prefix over the waves, then the bucket's start
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
  if constexpr (!kSlices) {
    const int incl = block_inclusive_scan<kSThreads>(total, scan_tmp, &all);
    if (tid < NB) {
      base[tid] = incl - total;
      offsets[tid] = incl - total;  // offsets[E] = start of the dropped bucket = valid count
    }
  } else {
    // bucket totals over all slices, and over the slices before this one
    int tot = 0, pre = 0;
    if (tid < NB) {
      const int me = blockIdx.x;
#pragma unroll 8
      for (int s = 0; s < nslice; ++s) {
        const int c = cnt[(size_t)s * NB + tid];
        tot += c;
        pre += (s < me) ? c : 0;
      }
    }
    const int incl = block_inclusive_scan<kSThreads>(tot, scan_tmp, &all);
    if (tid < NB) {
      base[tid] = incl - tot + pre;
      if (blockIdx.x == 0) offsets[tid] = incl - tot;
    }
  }
  __syncthreads();

  // 3. scatter.  One cached range: each position into rcache (16 bits
  // suffice), the inverse permutation through LDS in place of the buckets,
  // then coalesced stores (one CU's scattered 4-byte stores would be the
  // slowest part).  A cached slice stores each id at its position (the ids
  // of one bucket are consecutive there).  Positions are below A whenever
  // the indices are not changed during the call; the guard keeps a store
  // inside sorted_assign even if they are.
  if (cached && !kSlices) {
    for (int a = r0 + lane; a < r1; a += 64) {
      const int bk = bcache[a];
      rcache[a] = (uint16_t)(base[bk] + wcnt[wave][bk] + rcache[a]);
    }
    __syncthreads();
    for (int a = tid; a < A; a += kSThreads) bcache[rcache[a]] = (uint16_t)a;
    __syncthreads();
    for (int i = tid; i < A; i += kSThreads) sorted_assign[i] = bcache[i];
  } else if (cached) {
    for (int a = r0 + lane; a < r1; a += 64) {
      const int bk = bcache[a - lo];
      const int pos = base[bk] + wcnt[wave][bk] + rcache[a - lo];
      if ((unsigned)pos < (unsigned)A) sorted_assign[pos] = a;
    }
  } else {
    walk(wrun, [&](int a, bool valid, int bk, int rank) __attribute__((always_inline)) {
      const int pos = base[bk] + wcnt[wave][bk] + rank;
      if (valid && (unsigned)pos < (unsigned)A) sorted_assign[pos] = a;
    });
  }
}

hipError_t launch_sort(const int32_t* indices, int A, int E, int32_t* offsets, int32_t* sorted_assign, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  const size_t need = sort_workspace_bytes(A, E);
  if (need > 0 && ws != nullptr && ws_bytes >= need) {
    const SlicePlan p = slice_plan(A);
    int32_t* cnt = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(sort_hist_kernel, dim3(p.nslice), dim3(kSThreads), 0, stream, indices, A, E, p.slice, cnt);
    hipLaunchKernelGGL(sort_kernel<true>, dim3(p.nslice), dim3(kSThreads), 0, stream, indices, A, E, p.slice,
                       p.nslice, cnt, offsets, sorted_assign);
  } else {
    hipLaunchKernelGGL(sort_kernel<false>, dim3(1), dim3(kSThreads), 0, stream, indices, A, E, A, 1,
                       (const int32_t*)nullptr, offsets, sorted_assign);
  }
  return hipGetLastError();
}

}  // namespace qmoe

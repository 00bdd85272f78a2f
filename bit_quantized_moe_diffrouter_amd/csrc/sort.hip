// Token-by-expert sort for gfx950 (diffusion-gemma model.ts page,
// DiffExperts.forward: argsort of the flat routing indices, read as a stable
// sort).  One workgroup of 1024 threads:
//   1. LDS histogram of the T*k expert indices (bucket E collects indices
//      outside [0, E), which are dropped); up to 32768 bucket ids are kept in
//      LDS for step 3, larger inputs are read again;
//   2. exclusive prefix sum over the buckets -> expert_offsets;
//   3. stable scatter, 1024 assignments per round: each wave finds the lanes
//      that share its bucket with nine ballots (one per bit of the bucket id),
//      ranks itself among them with a popcount, and adds the counts of the
//      lower waves of the round; rounds are processed in order, so equal
//      experts keep ascending assignment ids.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {
constexpr int kSThreads = 1024, kSWaves = kSThreads / 64;
constexpr int kMaxBuckets = 257;  // E <= 256, plus the dropped bucket
constexpr int kCacheMax = 32768;  // assignments whose bucket ids stay in LDS between the passes
}  // namespace

__global__ __launch_bounds__(kSThreads) void sort_kernel(const int32_t* __restrict__ idx, int A, int E,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_assign) {
  __shared__ int cnt[kMaxBuckets];
  __shared__ int base[kMaxBuckets];
  __shared__ int wcnt[kSWaves][kMaxBuckets];
  __shared__ int scan_tmp[kSWaves];
  __shared__ uint16_t bcache[kCacheMax];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = E + 1;
  for (int i = tid; i < kSWaves * kMaxBuckets; i += kSThreads) (&wcnt[0][0])[i] = 0;
  if (tid < kMaxBuckets) cnt[tid] = 0;
  __syncthreads();

  auto bucket_of = [&](int a) {
    const int e = idx[a];
    return (e >= 0 && e < E) ? e : E;
  };
  const bool cached = A <= kCacheMax;

  // histogram; four loads in flight per thread before their atomics
  for (int a0 = tid; a0 < A; a0 += 4 * kSThreads) {
    int bk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int a = a0 + u * kSThreads;
      bk[u] = a < A ? bucket_of(a) : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (bk[u] < 0) continue;
      atomicAdd(&cnt[bk[u]], 1);
      if (cached) bcache[a0 + u * kSThreads] = (uint16_t)bk[u];
    }
  }
  __syncthreads();

  const int v = (tid < NB) ? cnt[tid] : 0;
  int total;
  const int incl = block_inclusive_scan<kSThreads>(v, scan_tmp, &total);
  if (tid < NB) {
    base[tid] = incl - v;
    offsets[tid] = incl - v;  // offsets[E] = start of the dropped bucket = valid count
  }
  __syncthreads();

  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < A; c0 += kSThreads) {
    const int a = c0 + tid;
    const bool valid = a < A;
    const int bk = !valid ? 0 : cached ? (int)bcache[a] : bucket_of(a);
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      const bool b = (bk >> bit) & 1;
      const unsigned long long m = __ballot(valid && b);
      peers &= b ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wave][bk] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = base[bk] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][bk];
      sorted_assign[pos] = a;
    }
    __syncthreads();
    if (tid < NB) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) {
        s += wcnt[w][tid];
        wcnt[w][tid] = 0;
      }
      base[tid] += s;
    }
    __syncthreads();
  }
}

hipError_t launch_sort(const int32_t* indices, int A, int E, int32_t* offsets, int32_t* sorted_assign,
                       hipStream_t stream) {
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kSThreads), 0, stream, indices, A, E, offsets, sorted_assign);
  return hipGetLastError();
}

}  // namespace qmoe

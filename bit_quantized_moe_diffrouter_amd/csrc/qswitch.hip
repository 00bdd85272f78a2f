// 4-bit switch linears (gate_up + GeGLU, down) and the dense 4-bit linear
// for gfx950, the weight tiling they read, and the weighted combine of the
// down rows.
//
// What is computed (diffusion-gemma model.ts page, DiffExperts.forward):
// every sorted row r of expert e multiplies its activation row by the
// dequantized weight of e; gate_up splits the 2I outputs at I and applies
// GeGLU (gelu_approx(gate) * up, vision.ts page, DiffVisionMLP); the down rows
// are summed per token with the routing weights.
//
// Weight tiling.  v_mfma_f32_16x16x32_bf16 wants lane l to hold operand row
// l % 16; read straight from row-major codes every lane of a load touches a
// different row and the vector L1 handles each lane as its own access.  The
// weights are therefore re-laid once (qmoe_tile_weight) into 4608-byte units,
// one per (expert, block of 128 weight rows, 64-wide group): 4096 bytes of
// codes in the exact per-lane operand order, then the 128 rows' (scale, bias)
// pairs in the order the lanes read them.  A wave streams one block: per group
// four 1 KB and two 256-byte fully coalesced loads.  Within a code word the
// nibbles are placed so that one v_and_or_b32 per pair yields two bf16 of
// 128 + q in natural k order (no activation shuffling).  Activations: gate_up
// and the dense linear read bf16 rows, 128 contiguous bytes per row and
// group (two loads of 8 rows per 16-row tile), and put them in operand order
// through LDS; the down pass reads mid as activation tiles (16 sorted rows x
// 64 columns already in operand order, written by the gate_up epilogue): two
// coalesced 1 KB loads per tile and group.
//
// Work items.  An item is (expert e, chunk of up to 32 sorted rows of e, one
// 128-row weight block).  A persistent grid derives the items on the device
// from expert_offsets (no host synchronisation).  A chunk of at most 16 rows
// is one 16-row MFMA tile, a larger one two; a wave computes every tile of its
// chunk from one unpacking of the weights (a one-tile chunk skips the second
// tile's arithmetic).  Each wave (or, for the long gate_up contraction, each
// pair of waves splitting it in two) walks its own items and writes their
// outputs itself, so after the prologue no workgroup barrier is needed; a wave
// streams its operands straight into registers through a ring of slots that
// runs on across its items.

// Arithmetic per group: P = sum_k x_k (128 + q_k) and, against a ones operand,
// X = sum_k x_k come from the MFMA; the group's affine is applied in fp32:
//     sum_k x_k (s q_k + b) = s P + (b - 128 s) X,
// s P with one FMA per output element, the bias terms of 4 groups at a time
// with one fp32 MFMA (a contraction over the groups).  The products are exact
// and the dequantized weight is never rounded; the only roundings are the
// fp32 accumulation and the output conversion.
#include <atomic>

#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 32;            // sorted rows per chunk (at most two 16-row tiles)
constexpr int kMaxBuckets = 257;   // experts (<= 256) + the dropped bucket of the down pass
constexpr int kNS = 8;             // 16-row subtiles per tiled block
constexpr int kXcds = 8;           // accelerator dies; workgroup b runs on die b % 8
constexpr int kMT = 2;             // row tiles held per slot and accumulator set
// LDS per wave: staging of two 16-row tiles, 64 bf16 columns wide (activation
// rows in; gate_up and dense GeGLU outputs) or 128 wide (down and dense outputs)
constexpr int wave_lds_bytes(int mode) {
  return (mode == MODE_DOWN || mode == MODE_DENSE || mode == MODE_DENSE_SOFTCAP) ? kMT * 16 * 128 * 2
                                                                                 : kMT * 16 * 64 * 2;
}
constexpr int kRedBytes = kMT * kNS * 64 * 16;  // one wave's fp32 accumulators (K-split hand-over)

struct Item {
  int e;     // expert whose weights are used (0 for the dropped bucket)
  int r0;    // first sorted row
  int rows;  // rows of the chunk, 1..32
  int blk;   // weight block (within the expert)
  int zero;  // down pass, dropped bucket: the rows are written as zeros
};

// One ring slot: operands of one quantization group for one wave and MT row tiles.
template <int MT>
struct Slot {
  u32x4_t w[4];      // codes: 16 bytes = the operand words of subtiles 2i, 2i+1
  u32x4_t s[2];      // (scale, bias) bf16 pairs of subtiles 4h .. 4h+3
  u32x4_t a[MT][2];  // activations of row tile m: k = 16lq .. 16lq+7, 16lq+8 .. 16lq+15
};

// Pins the ring order: the slot's registers pass through an empty asm, so the
// wait for its loads lands here and its consumers cannot be hoisted above the
// loads issued by earlier steps.
template <int MT>
__device__ __forceinline__ void fence_slot(Slot<MT>& sl) {
  asm volatile("" : "+v"(sl.w[0]), "+v"(sl.w[1]), "+v"(sl.w[2]), "+v"(sl.w[3])::"memory");
  asm volatile("" : "+v"(sl.s[0]), "+v"(sl.s[1])::"memory");
#pragma unroll
  for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(sl.a[m][0]), "+v"(sl.a[m][1])::"memory");
}

// Orders a wave's own LDS stores before its later loads.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Calls f(0), f(1), ... with compile-time indices.
template <class F, int... I>
__device__ __forceinline__ void run_steps(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

}  // namespace

// Work items and workers.  An item is (chunk of up to 32 sorted rows of one
// bucket, one 128-row weight block) over the whole contraction.  A worker is
// one wave (KS = 1) or KS = 2 or 4 waves of one workgroup that split the
// contraction into KS contiguous parts; every worker walks its own items, so
// after the prologue no wave waits for another except within its worker.  A
// wave streams its part of the block's units (contiguous in HBM) through a
// register ring that runs on across its items, computes every row tile of the
// chunk from one unpacking of the weights, and at the item's end the worker's
// first wave writes the outputs (KS > 1: the other waves hand it their
// partial sums through LDS, which it adds in contraction order).
template <int MODE, int KS, int D>
__global__ __launch_bounds__(kThreads, 2) void qmm_kernel(const SwitchArgs p) {
  static_assert(KS == 1 || KS == 2 || KS == 4, "a worker is 1, 2 or 4 waves");
  constexpr int kWaveLds = wave_lds_bytes(MODE);
  constexpr int MT = kMT;
  // plain rows 0..M-1, no buckets
  constexpr bool kRows = MODE == MODE_DENSE || MODE == MODE_DENSE_GEGLU || MODE == MODE_DENSE_SOFTCAP;
  // kWaveLds bytes per wave, then (KS > 1) kRedBytes per wave that is not the first of its worker
  extern __shared__ __attribute__((aligned(16))) uint8_t qmm_lds[];
  __shared__ int s_cum2[kMaxBuckets + 1];  // prefix per bucket of its two-tile chunks
  __shared__ int s_cum1[kMaxBuckets + 1];  // prefix per bucket of its one-tile chunk (0 or 1)
  __shared__ int s_lo[kMaxBuckets];       // clamped segment [lo, hi) of each bucket
  __shared__ int s_hi[kMaxBuckets];
  __shared__ int s_tcum[kMaxBuckets + 1];  // switch modes: first activation tile of each expert
  __shared__ int s_scan[kWaves];
  // down pass: assignment id of each chunk row, per wave and item (mod 4).  The
  // load cursor writes an item's entry when it enters the item; with a ring of
  // D <= min(2, G) slots it enters item c + 2 at the earliest during item c's
  // last step (when G <= D), never item c + 4 before item c is finished.
  __shared__ int s_dst[kWaves][4][kBM];
  // KS > 1, per wave that is not the first of its worker: items whose partial
  // sums it has handed over [0], and the first wave has taken [1]
  __shared__ int s_flag[kWaves][2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar branches below)
  const int ln = lane & 15, lq = lane >> 4;
  const int K = p.K, G = K / kGroup;
  const int A = p.rows_total;

  // ---- chunks.  A chunk is 32 sorted rows of one bucket (the last chunk of a
  // bucket may be shorter); chunks of more than 16 rows cost two tiles, the
  // others one.  Items are ranked two-tile chunks first, then one-tile ones,
  // blocks minor.
  const int nb = (MODE == MODE_DOWN) ? p.E + 1 : p.E;
  int total2, total1;
  if constexpr (kRows) {
    const int rem = A % kBM;
    total2 = A / kBM + (rem > 16 ? 1 : 0);
    total1 = (rem > 0 && rem <= 16) ? 1 : 0;
    if constexpr (KS > 1) {
      if (tid < 2 * kWaves) (&s_flag[0][0])[tid] = 0;
      __syncthreads();  // the only workgroup barrier of these modes
    }
  } else {
    // bucket b < E is expert b's segment; bucket E (down only) holds the dropped rows
    auto counts_of = [&](int b, int& one, int& tl) __attribute__((always_inline)) {
      const int o0 = p.offsets[b], o1 = p.offsets[min(b + 1, p.E)];  // both loads in flight together
      const int lo = min(max(o0, 0), A);
      const int hi = (b < p.E) ? min(max(o1, lo), A) : A;
      s_lo[b] = lo;
      s_hi[b] = hi;
      const int n = hi - lo, rem = n % kBM;
      one = (rem > 0 && rem <= 16) ? 1 : 0;
      tl = (b < p.E) ? (n + 15) / 16 : 0;  // the dropped bucket has no activation tiles
      return n / kBM + (rem > 16 ? 1 : 0);
    };
    // thread t counts bucket t; the last thread also bucket kThreads (E = 256, down)
    int o0 = 0, o1 = 0, t0 = 0, t1 = 0;
    const int c0 = (tid < nb) ? counts_of(tid, o0, t0) : 0;
    const int c1 = (tid == kThreads - 1 && nb > kThreads) ? counts_of(kThreads, o1, t1) : 0;
    int tot;
    int incl = block_inclusive_scan<kThreads>(c0 + c1, s_scan, &tot);
    if (tid < nb) s_cum2[tid + 1] = incl - c1;
    if (tid == kThreads - 1 && nb > kThreads) s_cum2[kThreads + 1] = incl;
    total2 = tot;
    incl = block_inclusive_scan<kThreads>(o0 + o1, s_scan, &tot);
    if (tid < nb) s_cum1[tid + 1] = incl - o1;
    if (tid == kThreads - 1 && nb > kThreads) s_cum1[kThreads + 1] = incl;
    total1 = tot;
    incl = block_inclusive_scan<kThreads>(t0 + t1, s_scan, &tot);
    if (tid < nb) s_tcum[tid] = incl - t1 - t0;
    if (tid == kThreads - 1 && nb > kThreads) s_tcum[kThreads] = incl - t1;
    if (tid == 0) {
      s_cum2[0] = 0;
      s_cum1[0] = 0;
    }
    if (tid < 2 * kWaves) (&s_flag[0][0])[tid] = 0;
    __syncthreads();  // the last workgroup barrier: from here on every worker runs on its own
  }
  total2 = __builtin_amdgcn_readfirstlane(total2);
  total1 = __builtin_amdgcn_readfirstlane(total1);

  // ---- worker slots.  The grid's workers form grid * 4 / KS slots; the worker
  // of slot s takes ranks s, 2S - 1 - s, 2S + s, ... (S slots: a boustrophedon over the
  // cost-sorted list).  Slot s sits at workgroup position s % grid; positions
  // are numbered XCD by XCD (workgroup b runs on die b % 8), so consecutive
  // ranks -- the blocks of one chunk, which read the same activations -- run on
  // one XCD and share its L2.  Within a workgroup the slot's role s / grid is
  // rotated by the position, so the costly first ranks spread over the SIMDs.
  const int total_items = __builtin_amdgcn_readfirstlane((total2 + total1) * p.nblk);
  const int grid = (int)gridDim.x, b = (int)blockIdx.x;
  const int pos = (grid % kXcds == 0) ? (b % kXcds) * (grid / kXcds) + b / kXcds : b;
  constexpr int kWorkers = kWaves / KS;     // workers per workgroup
  const int worker = wave / KS, kp = wave % KS;  // kp: this wave's part of the contraction
  const int gk0 = kp * G / KS, gk1 = (kp + 1) * G / KS;  // groups [gk0, gk1) of this wave
  const int nslots = grid * kWorkers;
  const int slot = ((worker + pos) & (kWorkers - 1)) * grid + pos;
  auto item_of = [&](int j) __attribute__((always_inline)) {  // rank of this wave's j-th item
    return j * nslots + ((j & 1) ? nslots - 1 - slot : slot);
  };
  auto has_item = [&](int j) __attribute__((always_inline)) { return item_of(j) < total_items; };
  if (!has_item(0)) return;  // no workgroup barrier follows; a pair leaves together

  // item rank -> (expert, rows, block); wave-uniform
  auto decode = [&](int item) __attribute__((always_inline)) {
    Item it;
    const int chunk = item / p.nblk;
    it.blk = item - chunk * p.nblk;
    if constexpr (kRows) {
      it.e = 0;
      it.zero = 0;
      it.r0 = chunk * kBM;  // the only possible one-tile chunk is the last one
      it.rows = min(kBM, A - it.r0);
    } else {
      const bool two = chunk < total2;
      const int c = two ? chunk : chunk - total2;
      const int* cum = two ? s_cum2 : s_cum1;
      int lo = 0, hi = nb;  // cum[lo] <= c < cum[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cum[mid] <= c) lo = mid; else hi = mid;
      }
      const int e = lo;
      // two-tile chunks are a bucket's first ones; its one-tile chunk is its last
      const int local = two ? c - s_cum2[e] : (s_cum2[e + 1] - s_cum2[e]);
      it.r0 = s_lo[e] + local * kBM;
      it.rows = min(kBM, s_hi[e] - it.r0);
      it.zero = (MODE == MODE_DOWN) && (e >= p.E);
      it.e = it.zero ? 0 : e;
    }
    it.e = __builtin_amdgcn_readfirstlane(it.e);
    it.r0 = __builtin_amdgcn_readfirstlane(it.r0);
    it.rows = __builtin_amdgcn_readfirstlane(it.rows);
    it.blk = __builtin_amdgcn_readfirstlane(it.blk);
    it.zero = __builtin_amdgcn_readfirstlane(it.zero);
    return it;
  };
  // activation tile of row tile m of an item (switch modes); a tile past the
  // buffers (inconsistent offsets) reads tile 0 and is never stored
  auto tile_of = [&](const Item& it, int m) __attribute__((always_inline)) {
    if constexpr (kRows) {
      return 0;
    } else {
      if (it.zero) return 0;
      const int tau = s_tcum[it.e] + (it.r0 - s_lo[it.e]) / 16 + m;
      return (tau >= 0 && tau < p.max_tiles) ? tau : -1;
    }
  };

  // ---- load cursor: the item and group whose operands are issued next
  const uint8_t* const wbytes = (const uint8_t*)p.w;
  const uint8_t* const abytes = (const uint8_t*)p.a;
  const uint32_t arow = K * 2;                     // gate_up, dense: bytes per activation row
  const uint32_t c_off = lane * 16;                // code bytes of this lane in a unit
  const uint32_t s_off = 4096 + ln * 16;           // scale bytes of this lane in a unit
  // chunk row of this lane's activation load (m, h): row 8 h + lane / 8 of tile
  // m; a one-tile chunk reads its tile twice
  auto row_of = [&](const Item& it, int m, int h) __attribute__((always_inline)) {
    const int mm = (it.rows > 16) ? m : 0;
    return min(16 * mm + 8 * h + (lane >> 3), it.rows - 1);
  };
  // Assignment ids an item needs, loaded when the load cursor enters the item
  // before it: gate_up, of this lane's four activation rows; down, of chunk
  // row lane % 32.
  auto load_ids = [&](const Item& it, int (&ids)[MT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (MODE == MODE_GATE_UP) ids[m][h] = p.assign[it.r0 + row_of(it, m, h)];
        else if constexpr (MODE == MODE_DOWN) ids[m][h] = (m == 0 && h == 0) ? p.assign[min(it.r0 + (lane & 31), A - 1)] : 0;
        else ids[m][h] = 0;
      }
  };
  Item linfo = decode(item_of(0));
  int lg = gk0;
  int n_j = 1;  // index (in this wave's sequence) of the item after the load cursor's
  bool n_valid = has_item(n_j);
  Item ninfo = n_valid ? decode(item_of(n_j)) : linfo;
  int ids_cur[MT][2], ids_next[MT][2];
  // unit (expert, block, group 0) of the load cursor's item
  const uint8_t* l_wbase = wbytes + ((size_t)linfo.e * p.nblk + linfo.blk) * (size_t)G * kTiledUnit;
  // per row tile m and half h: gate_up, dense: offset of the lane's 16 bytes
  // (row 8 h + lane / 8 of the tile, columns 8 (lane % 8) .. + 7 of a group)
  // in the activation rows; down: of the lane's operand words in the tile's
  // group-0 block (h = 1 unused)
  uint32_t l_aoff[MT][2];
  int l_loc = 0;  // items the load cursor has entered (s_dst entry)

  auto enter_item = [&](const Item& it) __attribute__((always_inline)) {
    l_wbase = wbytes + ((size_t)it.e * p.nblk + it.blk) * (size_t)G * kTiledUnit;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if constexpr (MODE == MODE_DOWN) {
        const int tau = max(tile_of(it, (it.rows > 16) ? m : 0), 0);
        l_aoff[m][0] = (uint32_t)tau * (uint32_t)(G * kActBlock) + lane * 16;
        l_aoff[m][1] = 0;
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int src;
          if constexpr (MODE == MODE_GATE_UP) {
            const int a = ids_cur[m][h];
            src = (a >= 0 && a < A) ? token_of(a, p.ktop_inv) : 0;
          } else {
            src = it.r0 + row_of(it, m, h);
          }
          l_aoff[m][h] = (uint32_t)src * arow + (lane & 7) * 16;
        }
      }
    }
    if constexpr (MODE == MODE_DOWN) {
      const int lr = lane & 31, raw = ids_cur[0][0];
      s_dst[wave][l_loc & 3][lr] = (lr < it.rows && raw >= 0 && raw < A) ? raw : -1;
    }
  };

  // Codes and scales of group g.  Each weight byte is read once; in the gate_up
  // pass the loads carry the non-temporal hint, which keeps the weight stream
  // from displacing in L2 the activation rows every block of a chunk re-reads
  // (3 us at 256 tokens; no gain in the down pass).
  auto issue_w = [&](Slot<MT>& sl, int g) __attribute__((always_inline)) {
    const uint8_t* u = l_wbase + (size_t)g * kTiledUnit;
    auto ld = [](const uint8_t* a) __attribute__((always_inline)) {
      if constexpr (MODE == MODE_GATE_UP || MODE == MODE_DENSE_GEGLU || MODE == MODE_DENSE_SOFTCAP)
        return __builtin_nontemporal_load((const u32x4_t*)a);
      else return *(const u32x4_t*)a;
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) sl.w[i] = ld(u + c_off + i * 1024);
#pragma unroll
    for (int h = 0; h < 2; ++h) sl.s[h] = ld(u + s_off + h * 256);
  };
  auto issue_a = [&](Slot<MT>& sl) __attribute__((always_inline)) {  // activations of group lg
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if constexpr (MODE == MODE_DOWN) {  // one coalesced kilobyte per operand register
        const uint8_t* ab = abytes + (l_aoff[m][0] + (uint32_t)lg * kActBlock);  // one 32-bit offset
        sl.a[m][0] = *(const u32x4_t*)(ab);
        sl.a[m][1] = *(const u32x4_t*)(ab + kActBlock / 2);
      } else {  // 8 rows x 128 bytes per load; compute puts them in operand order
#pragma unroll
        for (int h = 0; h < 2; ++h) sl.a[m][h] = *(const u32x4_t*)(abytes + (l_aoff[m][h] + (uint32_t)lg * 128u));
      }
    }
  };
  auto issue = [&](Slot<MT>& sl) __attribute__((always_inline)) {
    issue_w(sl, lg);
    issue_a(sl);
  };
  auto advance_load = [&]() __attribute__((always_inline)) {
    if (++lg < gk1) return;
    lg = gk0;
    if (!n_valid) return;  // past the last item: keep re-reading its groups (never used)
    linfo = ninfo;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h) ids_cur[m][h] = ids_next[m][h];
    ++l_loc;
    enter_item(linfo);
    ++n_j;
    n_valid = has_item(n_j);
    if (n_valid) {
      ninfo = decode(item_of(n_j));
      load_ids(ninfo, ids_next);
    }
  };

  load_ids(linfo, ids_cur);
  load_ids(ninfo, ids_next);
  enter_item(linfo);
  Slot<MT> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    issue(ring[d]);
    asm volatile("" ::: "memory");  // keeps the slots' loads in ring order
    advance_load();
  }

  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const OffsetCodeConsts kc = offset_code_consts();

  f32x4_t acc[MT][kNS];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < kNS; ++j) acc[m][j] = zero4();
  // The bias term of the affine, sum_g (b - 128 s)_g X_g, is a contraction
  // over the groups; blocks of 4 groups go through one fp32 MFMA
  // (v_mfma_f32_16x16x4_f32: lane (ln, lq) gives X of row ln and the
  // correction of column ln for the block's group lq).
  float xsel[MT];    // X of row ln, tile m, of the block's group lq (0 where not yet set)
  float ccsel[kNS];  // b - 128 s of column ln, subtile j, of the block's group lq
#pragma unroll
  for (int m = 0; m < MT; ++m) xsel[m] = 0.f;
#pragma unroll
  for (int j = 0; j < kNS; ++j) ccsel[j] = 0.f;

  int c_j = 0;  // index of the compute cursor's item in this wave's sequence
  Item cinfo = decode(item_of(0));
  int cg = gk0;
  uint8_t* const wlds = qmm_lds + (size_t)wave * kWaveLds;  // this wave's LDS

  // one group of the current item from slot `sl`, for the MT row tiles; the
  // weights are unpacked once for all of them.  kq: the group's place in its
  // block of 4.
  auto compute = [&](Slot<MT>& sl, int kq) __attribute__((always_inline)) {
    const bool t2 = cinfo.rows > 16;  // uniform: a second row tile to compute
    u32x4_t a[MT][2];  // operands: lane (ln, lq) holds row ln, columns 16 lq .. 16 lq + 15
    if constexpr (MODE == MODE_DOWN) {
#pragma unroll
      for (int m = 0; m < MT; ++m) a[m][0] = sl.a[m][0], a[m][1] = sl.a[m][1];
    } else {
      // through this wave's LDS: row r's 16-byte chunk c sits at slot c ^ swz(r),
      // so both the 8-lanes-per-row writes and the operand reads are conflict free
      auto swz = [](int r) __attribute__((always_inline)) { return ((r & 1) << 2) | ((r >> 1) & 3); };
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 8 * h + (lane >> 3);
          *(u32x4_t*)(wlds + m * 2048 + r * 128 + ((lane & 7) ^ swz(r)) * 16) = sl.a[m][h];
        }
      }
      wave_lds_fence();
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          a[m][h] = *(const u32x4_t*)(wlds + m * 2048 + ln * 128 + ((2 * lq + h) ^ swz(ln)) * 16);
      }
      wave_lds_fence();
    }
    const bool mine = lq == kq;  // this lane group holds the group's place in the block
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m > 0 && !t2) continue;
      // ones as the A operand: every row of the result holds the row sums, so
      // lane (ln, lq) gets X of activation row ln
      f32x4_t X = mfma16x16x32(ones, a[m][0], zero4());
      X = mfma16x16x32(ones, a[m][1], X);
      xsel[m] = mine ? X[0] : xsel[m];
    }
#pragma unroll
    for (int j = 0; j < kNS; ++j) {
      const uint32_t sb = sl.s[j >> 2][j & 3];
      const float sc = __uint_as_float(sb << 16);
      const float cc = __uint_as_float(sb & 0xffff0000u) - 128.0f * sc;
      ccsel[j] = mine ? cc : ccsel[j];
      u32x4_t b0, b1;
      unpack_offset_code_pair(sl.w[j >> 1][(j & 1) * 2], sl.w[j >> 1][(j & 1) * 2 + 1], kc, b0, b1);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
        f32x4_t P = mfma16x16x32(a[m][0], b0, zero4());
        P = mfma16x16x32(a[m][1], b1, P);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][j][i] = __builtin_fmaf(sc, P[i], acc[m][j][i]);
      }
    }
  };
  // adds the bias terms of the groups collected since the last call
  auto flush_bias = [&]() __attribute__((always_inline)) {
    const bool t2 = cinfo.rows > 16;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m > 0 && !t2) continue;
#pragma unroll
      for (int j = 0; j < kNS; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsel[m], ccsel[j], acc[m][j], 0, 0, 0);
      xsel[m] = 0.f;
    }
  };

  // Bounded wait on a hand-over flag: a protocol slip cannot hang the GPU (after
  // about 10^8 cycles the wave goes on, with wrong results, and raises the
  // device status word's kStatusSpin bit so that the caller can tell).
  auto pair_wait = [&](int* f, int v) __attribute__((always_inline)) {
    for (int it = 0; it < (1 << 21); ++it) {
      if (__hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= v) return;
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) __hip_atomic_fetch_or(p.status, kStatusSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  (void)pair_wait;

  // End of the compute cursor's item: the wave stages its outputs in its LDS
  // as bf16 and writes them with 16-byte stores.
  auto finish_item = [&]() __attribute__((always_inline)) {
    const bool t2 = cinfo.rows > 16;
    const int blk = cinfo.blk;
    if constexpr (KS > 1) {
      // Every other wave of the worker parks its partial sums for item c_j
      // once the first has taken its sums of item c_j - 1; the first adds them
      // after its own in contraction order (kp = 1, 2, ...) and writes the
      // outputs.
      f32x4_t* const red0 = (f32x4_t*)(qmm_lds + kWaves * kWaveLds) + worker * (KS - 1) * (MT * kNS * 64);
      if (kp != 0) {
        f32x4_t* const red = red0 + (kp - 1) * (MT * kNS * 64);
        pair_wait(&s_flag[wave][1], c_j);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m > 0 && !t2) continue;
#pragma unroll
          for (int j = 0; j < kNS; ++j) red[(m * kNS + j) * 64 + lane] = acc[m][j];
        }
        __hip_atomic_store(&s_flag[wave][0], c_j + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
#pragma unroll 1
        for (int q = 1; q < KS; ++q) {  // kept a loop: unrolled, the LDS reads of all parts would be hoisted
          const f32x4_t* const red = red0 + (q - 1) * (MT * kNS * 64);
          pair_wait(&s_flag[wave + q][0], c_j + 1);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m > 0 && !t2) continue;
#pragma unroll
            for (int j = 0; j < kNS; ++j) {
              const f32x4_t o = red[(m * kNS + j) * 64 + lane];
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[m][j][i] += o[i];
            }
          }
          __hip_atomic_store(&s_flag[wave + q][1], c_j + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
    if (kp != 0) {
      // not the first wave of its worker: no outputs
    } else if constexpr (MODE == MODE_GATE_UP) {
      // gate j and up j + 4 -> columns 16 j .. 16 j + 15 of group blk of the
      // activation tiles: column 16 q + 8 h + i of tile row r sits at byte
      // h * 1024 + (16 q + r) * 16 + 2 i of the tile's block
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *(uint16_t*)(wlds + m * 2048 + (ln >> 3) * 1024 + (16 * j + 4 * lq + i) * 16 + (ln & 7) * 2) =
                f32_to_bf16_bits(gelu_tanh(acc[m][j][i]) * acc[m][j + 4][i]);
      }
      wave_lds_fence();
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
        const int tau = tile_of(cinfo, m);
        if (tau < 0) continue;
        uint8_t* const dst = (uint8_t*)p.out + ((size_t)tau * (p.Nout / 64) + blk) * kActBlock + lane * 16;
#pragma unroll
        for (int h = 0; h < 2; ++h) *(u32x4_t*)(dst + h * 1024) = *(const u32x4_t*)(wlds + m * 2048 + h * 1024 + lane * 16);
      }
    } else if constexpr (MODE == MODE_DENSE_GEGLU) {
      // gate j and up j + 4 -> columns 64 blk + 16 j .. + 15 of the row-major
      // output: bf16 [16 rows][64 columns] per row tile, a store covers 8 rows
      uint16_t* const stg = (uint16_t*)wlds;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            stg[m * 1024 + (4 * lq + i) * 64 + 16 * j + ln] = f32_to_bf16_bits(gelu_tanh(acc[m][j][i]) * acc[m][j + 4][i]);
      }
      wave_lds_fence();
      const int c = lane & 7;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int r = 8 * q + (lane >> 3), lr = 16 * m + r;
          if (lr < cinfo.rows && blk * 64 + 8 * c < p.Nout)  // the last block may be partly past the width
            *(u32x4_t*)((uint16_t*)p.out + (size_t)(cinfo.r0 + lr) * p.Nout + blk * 64 + 8 * c) =
                *(const u32x4_t*)(stg + m * 1024 + r * 64 + 8 * c);
        }
      }
    } else if constexpr (MODE == MODE_DENSE_SOFTCAP) {
      // logits rounded to bf16 (the quantized matmul's output type), widened,
      // cap * tanh(z / cap); fp32 [16 rows][128 columns] per row tile staged
      // one tile at a time, a store covers 2 rows
      float* const stg = (float*)wlds;
      const int c = lane & 31;
      const int col = blk * 128 + 4 * c;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
        if (m > 0) wave_lds_fence();  // the previous tile's staging reads are done
#pragma unroll
        for (int j = 0; j < kNS; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float z = bf16_bits_to_f32(f32_to_bf16_bits(acc[m][j][i]));
            stg[(4 * lq + i) * 128 + 16 * j + ln] = p.cap * tanhf(z / p.cap);
          }
        wave_lds_fence();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = 2 * q + (lane >> 5), lr = 16 * m + r;
          if (lr < cinfo.rows && col < p.Nout)
            *(u32x4_t*)((float*)p.out + (size_t)(cinfo.r0 + lr) * p.Nout + col) = *(const u32x4_t*)(stg + r * 128 + 4 * c);
        }
      }
    } else {
      // bf16 [16 rows][128 columns] per row tile; a store covers 4 rows
      uint16_t* const stg = (uint16_t*)wlds;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
#pragma unroll
        for (int j = 0; j < kNS; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            stg[m * 2048 + (4 * lq + i) * 128 + 16 * j + ln] = cinfo.zero ? (uint16_t)0 : f32_to_bf16_bits(acc[m][j][i]);
      }
      wave_lds_fence();
      const int c = lane & 15;
      const int col = blk * 128 + 8 * c;  // a block past the last output column (N % 128 == 64) has none there
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m > 0 && !t2) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 4 * q + (lane >> 4), lr = 16 * m + r;
          int row;
          if constexpr (MODE == MODE_DOWN) row = s_dst[wave][c_j & 3][lr];
          else row = (lr < cinfo.rows) ? cinfo.r0 + lr : -1;
          if (row >= 0 && col < p.Nout)
            *(u32x4_t*)((uint16_t*)p.out + (size_t)row * p.Nout + col) = *(const u32x4_t*)(stg + m * 2048 + r * 128 + 8 * c);
        }
      }
    }
    wave_lds_fence();  // the staging reads are done before the LDS is written again
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < kNS; ++j) acc[m][j] = zero4();
  };

  // One ring step on slot d: compute the current group, refill the slot.  Every
  // step issues its loads, also after the last item (compute is skipped then):
  // the loop has a single exit at the end of a block of D steps and the wait
  // before each slot always counts the loads of the D - 1 slots issued after it.
  bool done = false;
  auto step = [&](auto d_tag) __attribute__((always_inline)) {
    constexpr int d = decltype(d_tag)::value;
    fence_slot(ring[d]);
    if (!done && !cinfo.zero) {
      const int kq = (cg - gk0) & 3;
      compute(ring[d], kq);
      if (kq == 3 || cg + 1 == gk1) flush_bias();
    }
    issue(ring[d]);
    asm volatile("" ::: "memory");  // keeps the slots' loads in ring order
    advance_load();
    if (done || ++cg < gk1) return;
    finish_item();
    if (!has_item(c_j + 1)) {
      done = true;
      return;
    }
    ++c_j;
    cinfo = decode(item_of(c_j));
    cg = gk0;
  };
  do {
    run_steps(step, std::make_integer_sequence<int, D>{});
  } while (!done);
  // the loads issued past the end are consumed here (they complete before the wave ends)
#pragma unroll
  for (int d = 0; d < D; ++d) fence_slot(ring[d]);
}

// ---------------------------------------------------------------- weight tiling
// Weight row of block b, subtile j, row n (split > 0: gate rows then up rows;
// past the gate half's end, -1: read as zero).
__device__ __forceinline__ int tiled_row(int b, int j, int n, int split) {
  if (split > 0) {
    const int c = 64 * b + 16 * (j & 3) + n;  // column of the pair
    if (c >= split) return -1;
    return (j < 4) ? c : split + c;
  }
  return 128 * b + 16 * j + n;
}

// Code word of 8 codes c0..c7 (code c at bits 4c) -> the operand order: code 2p
// at bits 4p, code 2p+1 at bits 16 + 4p (p = 0..3).
__device__ __forceinline__ uint32_t operand_word(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    r |= ((w >> (8 * pp)) & 0xFu) << (4 * pp);
    r |= ((w >> (8 * pp + 4)) & 0xFu) << (16 + 4 * pp);
  }
  return r;
}

// One thread per 16-byte piece of the tiled buffer.
__global__ __launch_bounds__(256) void tile_weight_kernel(const uint32_t* __restrict__ w, const uint16_t* __restrict__ s,
                                                          const uint16_t* __restrict__ bi, int E, int rows, int K,
                                                          int split, int nblk, uint8_t* __restrict__ dst) {
  const int G = K / 64, KW = K / 8;
  const long long pieces = (long long)E * nblk * G * (kTiledUnit / 16);
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  if (c >= pieces) return;
  const long long u = c / (kTiledUnit / 16);
  const int q = (int)(c - u * (kTiledUnit / 16));
  const int g = (int)(u % G);
  const int b = (int)((u / G) % nblk);
  const int e = (int)(u / ((long long)G * nblk));
  u32x4_t out = {0u, 0u, 0u, 0u};
  if (q < 256) {  // codes: instruction i, lane L -> subtiles 2i, 2i+1 of lane (L % 16, L / 16)
    const int i = q >> 6, L = q & 63, n = L & 15, kq = L >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = tiled_row(b, 2 * i + t, n, split);
      if (row >= 0 && row < rows) {
        const uint32_t* src = w + ((size_t)e * rows + row) * KW + g * 8 + 2 * kq;
        out[2 * t] = operand_word(src[0]);
        out[2 * t + 1] = operand_word(src[1]);
      }
    }
  } else {  // (scale, bias) of subtiles 4h .. 4h+3 for row n of each
    const int h = (q - 256) >> 4, n = (q - 256) & 15;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = tiled_row(b, 4 * h + jj, n, split);
      if (row >= 0 && row < rows) {
        const size_t si = ((size_t)e * rows + row) * G + g;
        out[jj] = (uint32_t)s[si] | ((uint32_t)bi[si] << 16);
      }
    }
  }
  *(u32x4_t*)(dst + c * 16) = out;
}

// ------------------------------------------------------------ activation tiles
long long act_tiles_max(long long A, int E) { return (A + 15) / 16 + std::min<long long>(E, A); }

// y[t, h] = bf16( sum_{j<k} w[t, j] * D[t*k + j, h] ), D in bf16 (the down
// rows as the switch linear returns them), products and sum in fp32, j order.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ D, const float* __restrict__ w,
                                                      int T, int k, int H, uint16_t* __restrict__ y) {
  const int H8 = H / 8;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * H8) return;
  const int t = (int)(idx / H8), h = (int)(idx - (long long)t * H8) * 8;
  const uint16_t* base = D + (size_t)t * k * H + h;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // the loads of up to 8 rows are issued before any is summed (few waves per
  // SIMD at a few hundred tokens, so one round trip per row would be exposed);
  // the terms are still added in j order
  for (int j0 = 0; j0 < k; j0 += 8) {
    u32x4_t v[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = j0 + u < k;
      v[u] = ok ? *(const u32x4_t*)(base + (size_t)(j0 + u) * H) : u32x4_t{0u, 0u, 0u, 0u};
      wj[u] = ok ? w[(size_t)t * k + j0 + u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u >= k) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s[2 * q] += wj[u] * bf16_lo_f32(v[u][q]);
        s[2 * q + 1] += wj[u] * bf16_hi_f32(v[u][q]);
      }
    }
  }
  u32x4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(s[2 * q], s[2 * q + 1]);
  *(u32x4_t*)(y + (size_t)t * H + h) = o;
}

// ------------------------------------------------------------------ launchers
namespace {

constexpr int kMaxDevices = 64;

}  // namespace

// One int per device (each device holds its own copy of the module's
// variables).
__device__ int g_qmoe_status;

int* device_status() {
  static int* addr[kMaxDevices];
  static std::atomic<int> ready[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (!ready[dev].load(std::memory_order_acquire)) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_qmoe_status)) != hipSuccess || ptr == nullptr) return nullptr;
    addr[dev] = static_cast<int*>(ptr);
    ready[dev].store(1, std::memory_order_release);
  }
  return addr[dev];
}

// Device scratch of the entry points that allocate nothing: one array per
// device (each device holds its own copy of the module's variables), kept
// until the process ends.  Host code never uses its name as an address: the
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* noalloc_scratch() {
  static void* addr[kMaxDevices];
  static std::atomic<int> ready[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (!ready[dev].load(std::memory_order_acquire)) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    addr[dev] = ptr;
    ready[dev].store(1, std::memory_order_release);
  }
  return addr[dev];
}

namespace {

// Items a launch can hold (every one of the A rows in its own bucket's
// chunks, at most one partial chunk per bucket).
template <int MODE>
long long max_items(const SwitchArgs& a, int extra_buckets) {
  long long chunks = (a.rows_total + kBM - 1) / kBM;
  if (MODE == MODE_GATE_UP || MODE == MODE_DOWN) chunks += (long long)std::min(a.E, a.rows_total) + extra_buckets;
  return chunks * a.nblk;
}

template <int MODE, int KS>
constexpr size_t lds_bytes() {
  return (size_t)kWaves * wave_lds_bytes(MODE) + (size_t)(kWaves / KS) * (KS - 1) * kRedBytes;
}

template <int MODE, int KS, int D>
hipError_t launch_cfg(SwitchArgs a, int extra_buckets, int num_cu, hipStream_t stream) {
  a.ntiles = a.nblk;
  a.ktop_inv = ktop_inverse(a.ktop);
  a.status = device_status();
  if (a.status == nullptr) return hipErrorInvalidSymbol;
  constexpr size_t lds = lds_bytes<MODE, KS>();
  const long long items = max_items<MODE>(a, extra_buckets);
  long long grid = std::min(items, (long long)num_cu * 2);
  if (grid < 1) grid = 1;
  // the dynamic-LDS limit is raised once per device (the attribute belongs to
  // the device's copy of the kernel)
  static std::atomic<int> attr_done[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  if (!attr_done[dev].load(std::memory_order_acquire)) {
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&qmm_kernel<MODE, KS, D>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    attr_done[dev].store(1, std::memory_order_release);
  }
  hipLaunchKernelGGL((qmm_kernel<MODE, KS, D>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

// Contraction split.  The gate_up pass with at least 8 groups splits it in two
// (its items then fill the chip at the canvas's 2048 rows).  A launch whose
// items give fewer than one wave per SIMD (small batches, the dense linears
// at a few hundred rows) splits it in two or four, as long as every wave keeps
// at least two groups: a wave's loads in flight are bounded by its ring, so
// fewer items need more waves per item to keep HBM busy.  Four-way splits of
// the down and dense passes hold 86 KB of LDS per workgroup (one per CU), and
// are taken only when the items fit one workgroup per CU.  Ring depth: two
// slots, one when a wave's part of the contraction is a single group (the
// down pass's row table relies on the load cursor never reaching item c + 4
// before item c is finished).
template <int MODE>
int choose_ks(const SwitchArgs& a, int extra_buckets, int num_cu) {
  const int G = a.K / 64;
  const long long items = max_items<MODE>(a, extra_buckets);
  const long long simds = 4LL * num_cu;
  constexpr size_t kStaticLds = 8192;  // the kernel's own __shared__ arrays, rounded up
  const bool four_fits = 2 * (lds_bytes<MODE, 4>() + kStaticLds) <= 160 * 1024 || items <= num_cu;
  int ks = (MODE == MODE_GATE_UP && G >= 8) ? 2 : 1;
  while (ks < 4 && items * ks < simds && G >= 4 * ks && (ks == 1 || four_fits)) ks *= 2;
  return ks;
}

template <int MODE>
hipError_t launch_mode(SwitchArgs a, int extra_buckets, int num_cu, hipStream_t stream) {
  const int G = a.K / 64;
  const int ks = choose_ks<MODE>(a, extra_buckets, num_cu);
  if (ks == 4) return launch_cfg<MODE, 4, 2>(a, extra_buckets, num_cu, stream);
  if (ks == 2) return launch_cfg<MODE, 2, 2>(a, extra_buckets, num_cu, stream);
  if (G >= 2) return launch_cfg<MODE, 1, 2>(a, extra_buckets, num_cu, stream);
  return launch_cfg<MODE, 1, 1>(a, extra_buckets, num_cu, stream);
}

}  // namespace

hipError_t launch_gate_up_geglu(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_mode<MODE_GATE_UP>(a, 0, num_cu, stream);
}
hipError_t launch_down(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_mode<MODE_DOWN>(a, 1, num_cu, stream);
}
hipError_t launch_dense(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_mode<MODE_DENSE>(a, 0, num_cu, stream);
}
hipError_t launch_dense_geglu(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_mode<MODE_DENSE_GEGLU>(a, 0, num_cu, stream);
}
hipError_t launch_dense_softcap(SwitchArgs a, int num_cu, hipStream_t stream) {
  return launch_mode<MODE_DENSE_SOFTCAP>(a, 0, num_cu, stream);
}
hipError_t launch_combine(const uint16_t* D, const float* w, int T, int k, int H, uint16_t* y, hipStream_t stream) {
  const long long n = (long long)T * (H / 8);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, D, w, T, k, H, y);
  return hipGetLastError();
}
int tiled_blocks(int rows, int split) { return split > 0 ? (split + 63) / 64 : (rows + 127) / 128; }
hipError_t launch_tile_weight(const uint32_t* w, const uint16_t* s, const uint16_t* b, int E, int rows, int K,
                              int split, uint8_t* dst, hipStream_t stream) {
  const int nblk = tiled_blocks(rows, split);
  const long long pieces = (long long)E * nblk * (K / 64) * (kTiledUnit / 16);
  const long long blocks = (pieces + 255) / 256;
  hipLaunchKernelGGL(tile_weight_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, s, b, E, rows, K, split,
                     nblk, dst);
  return hipGetLastError();
}

}  // namespace qmoe

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
// Work items.  An item is (expert e, chunk of up to 32 sorted rows of e, tile
// of NW weight blocks).  A persistent grid walks the items, derived on the
// device from expert_offsets (no host synchronisation).  A chunk of at most 16
// rows is one 16-row MFMA tile, a larger one two; a wave computes every tile
// of its chunk from one unpacking of the weights (a one-tile chunk skips the
// second tile's arithmetic).  The 4 waves of a workgroup split the contraction
// KW ways and the blocks NW ways (KW*NW = 4); each wave streams its operands
// straight into registers through a ring of slots that runs on across items.
// The K-split partial sums meet once per item in LDS, in a fixed order.
//
// Arithmetic per group: P = sum_k x_k (128 + q_k) and, against a ones operand,
// X = sum_k x_k come from the MFMA; the group's affine is applied in fp32:
//     sum_k x_k (s q_k + b) = s P + (b - 128 s) X,
// s P with one FMA per output element, the bias terms of 4 groups at a time
// with one fp32 MFMA (a contraction over the groups).  The products are exact
// and the dequantized weight is never rounded; the only roundings are the
// fp32 accumulation and the output conversion.
#include "common.h"
#include "launch.h"

namespace qmoe {

enum : int { MODE_GATE_UP = 0, MODE_DOWN = 1, MODE_DENSE = 2 };

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 32;            // sorted rows per chunk (at most two 16-row tiles)
constexpr int kMaxBuckets = 257;   // experts (<= 256) + the dropped bucket of the down pass
constexpr int kNS = 8;             // 16-row subtiles per tiled block
constexpr int kXcds = 8;           // accelerator dies; workgroup b runs on die b % 8
constexpr int kRingMax = 2;
constexpr int kMaxWgItems = 64;    // gate_up: items of one workgroup (token table in LDS)        // ring slots: two-tile slots fill the register file at 2 waves/SIMD

struct Item {
  int e;     // expert whose weights are used (0 for the dropped bucket)
  int r0;    // first sorted row
  int rows;  // rows of the chunk, 1..32
  int tile;  // block tile
  int zero;  // down pass, dropped bucket: the rows are written as zeros
};

// What one wave does for one item: the 4 waves split (K part, block), K
// 4 / NBI ways; each wave computes all row tiles of the chunk (one or two
// 16-row tiles) against a whole 128-row block (8 subtiles).
struct Role {
  int nk;   // K parts of the item
  int kp;   // this wave's K part
  int blk;  // weight block (within the expert)
  int gk0, gk1;  // groups [gk0, gk1) of the contraction
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

// Calls f(0), f(1), ... with compile-time indices.
template <class F, int... I>
__device__ __forceinline__ void run_steps(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

}  // namespace

template <int MODE, int NBI, int D>
__global__ __launch_bounds__(kThreads, 2) void qmm_kernel(const SwitchArgs p) {
  constexpr int BCOLS = (MODE == MODE_GATE_UP) ? 64 : 128;  // output columns per block

  extern __shared__ __attribute__((aligned(16))) uint8_t qmm_lds[];  // partial sums [wave][m][kNS][64] f32x4
  __shared__ int s_cum2[kMaxBuckets + 1];  // prefix per bucket of its two-tile chunks
  __shared__ int s_cum1[kMaxBuckets + 1];  // prefix per bucket of its one-tile chunk (0 or 1)
  __shared__ int s_lo[kMaxBuckets];       // clamped segment [lo, hi) of each bucket
  __shared__ int s_hi[kMaxBuckets];
  __shared__ int s_tcum[kMaxBuckets + 1];  // switch modes: first activation tile of each expert
  __shared__ int s_scan[kWaves];
  __shared__ int s_dst[2][kBM];           // down pass: assignment id of each chunk row
  __shared__ int s_tok[(MODE == MODE_GATE_UP) ? kMaxWgItems : 1][kBM];  // gate_up: token of each chunk row

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar branches below)
  const int ln = lane & 15, lq = lane >> 4;
  const int K = p.K, G = K / kGroup;
  const int A = p.rows_total;

  // ---- work items.  A chunk is 32 sorted rows of one bucket (the last chunk of
  // a bucket may be shorter); chunks of more than 16 rows cost two tiles, the
  // others one.  Items are ranked two-tile chunks first, then one-tile ones
  // (tile-minor), and workgroup b takes ranks b, 2 grid - 1 - b, 2 grid + b, ...
  // (a boustrophedon over the cost-sorted list), which evens out the work.
  const int nb = (MODE == MODE_DOWN) ? p.E + 1 : p.E;
  int total2, total1;
  if constexpr (MODE == MODE_DENSE) {
    const int rem = A % kBM;
    total2 = A / kBM + (rem > 16 ? 1 : 0);
    total1 = (rem > 0 && rem <= 16) ? 1 : 0;
  } else {
    // bucket b < E is expert b's segment; bucket E (down only) holds the dropped rows
    auto counts_of = [&](int b, int& one, int& tl) __attribute__((always_inline)) {
      const int lo = min(max(p.offsets[b], 0), A);
      const int hi = (b < p.E) ? min(max(p.offsets[b + 1], lo), A) : A;
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
    __syncthreads();
  }
  total2 = __builtin_amdgcn_readfirstlane(total2);
  total1 = __builtin_amdgcn_readfirstlane(total1);
  // Items are ranked two-tile chunks first (the costlier ones), then one-tile
  // chunks; the workgroup at position q takes ranks q, 2 grid - 1 - q,
  // 2 grid + q, ... (a boustrophedon over the cost-sorted list, which evens out
  // the work).  Workgroups are dealt to the 8 XCDs round-robin; positions are
  // numbered XCD by XCD, so consecutive ranks -- the column tiles of one chunk,
  // which read the same activation tiles -- run on one XCD and share its L2.
  const int total_items = __builtin_amdgcn_readfirstlane((total2 + total1) * p.ntiles);
  const int grid = (int)gridDim.x, b = (int)blockIdx.x;
  const int gb = (grid % kXcds == 0) ? (b % kXcds) * (grid / kXcds) + b / kXcds : b;
  auto item_of = [&](int j) __attribute__((always_inline)) {  // rank of this workgroup's j-th item
    return j * grid + ((j & 1) ? grid - 1 - gb : gb);
  };
  auto has_item = [&](int j) __attribute__((always_inline)) { return item_of(j) < total_items; };
  if (!has_item(0)) return;  // uniform: no barrier follows for this workgroup

  // item rank -> (expert, rows, tile); wave-uniform
  auto decode_raw = [&](int item) __attribute__((always_inline)) {
    Item it;
    const int chunk = item / p.ntiles;
    it.tile = item - chunk * p.ntiles;
    if constexpr (MODE == MODE_DENSE) {
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
    return it;
  };
  auto decode = [&](int item) __attribute__((always_inline)) {
    Item it = decode_raw(item);
    it.e = __builtin_amdgcn_readfirstlane(it.e);
    it.r0 = __builtin_amdgcn_readfirstlane(it.r0);
    it.rows = __builtin_amdgcn_readfirstlane(it.rows);
    it.tile = __builtin_amdgcn_readfirstlane(it.tile);
    it.zero = __builtin_amdgcn_readfirstlane(it.zero);
    return it;
  };
  // K parts per item: kWaves / NBI, fewer only for a contraction of fewer
  // groups.  The launcher takes NBI = 1 only when G >= 12, so nk is 1, 2 or 4
  // and the divisions by it below are shifts.
  auto role_of = [&](const Item& it) __attribute__((always_inline)) {
    Role r;
    r.nk = min(kWaves / NBI, G);
    if (wave < r.nk * NBI) {
      r.kp = wave % r.nk;
      r.blk = it.tile * NBI + wave / r.nk;
      r.gk0 = r.kp * G / r.nk;
      r.gk1 = (r.kp + 1) * G / r.nk;
    } else {  // spare wave (contraction shorter than the K split): streams, never stores
      r.kp = 0;
      r.blk = 0x7fffffff;
      r.gk0 = 0;
      r.gk1 = G;
    }
    return r;
  };
  // gate_up: the token of every row of this workgroup's items, once (the
  // launcher keeps a workgroup's items within kMaxWgItems)
  if constexpr (MODE == MODE_GATE_UP) {
    int nj = 0;
    while (nj < kMaxWgItems && has_item(nj)) ++nj;
    for (int t = tid; t < nj * kBM; t += kThreads) {
      const Item it = decode_raw(item_of(t / kBM));
      const int a = p.assign[it.r0 + min(t % kBM, it.rows - 1)];
      s_tok[t / kBM][t % kBM] = (a >= 0 && a < A) ? a / p.ktop : 0;
    }
    __syncthreads();
  }

  // activation tile of row tile m of an item (switch modes); a tile past the
  // buffers (inconsistent offsets) reads tile 0 and is never stored
  auto tile_of = [&](const Item& it, int m) __attribute__((always_inline)) {
    if constexpr (MODE == MODE_DENSE) {
      return 0;
    } else {
      if (it.zero) return 0;
      const int tau = s_tcum[it.e] + (it.r0 - s_lo[it.e]) / 16 + m;
      return (tau >= 0 && tau < p.max_tiles) ? tau : -1;
    }
  };
  // owner (K part) of subtile j among the waves of one block: gate_up keeps
  // gate j and up j + 4 together; the other modes give each K part a run of
  // kNS / nk contiguous subtiles
  auto owner_of = [&](int j, int nk) __attribute__((always_inline)) {
    return (MODE == MODE_GATE_UP) ? (j & 3) & (nk - 1) : (j * nk) >> 3;  // nk in {1, 2, 4}
  };

  // Slots and accumulators hold two row tiles; a one-tile chunk reads tile 0
  // twice and skips the second tile's arithmetic.
  auto body = [&](auto mt_tag) __attribute__((always_inline)) {
    constexpr int MT = decltype(mt_tag)::value;
    constexpr int DR = (D > kRingMax) ? kRingMax : D;  // ring depth
    // ---- load cursor (per wave): the item and group whose operands are issued next
    const uint8_t* const wbytes = (const uint8_t*)p.w;
    const uint8_t* const abytes = (const uint8_t*)p.a;
    const uint32_t arow = K * 2;                     // gate_up, dense: bytes per activation row
    const uint32_t c_off = lane * 16;                // code bytes of this lane in a unit
    const uint32_t s_off = 4096 + ln * 16;           // scale bytes of this lane in a unit
    Item linfo = decode(item_of(0));
    Role lrole = role_of(linfo);
    int lg = lrole.gk0;
    int n_j = 1;  // index (in this workgroup's sequence) of the item after the load cursor's
    bool n_valid = has_item(n_j);
    Item ninfo = n_valid ? decode(item_of(n_j)) : linfo;
    const uint8_t* l_wbase;  // unit (expert, block, group 0) of this wave
    // per row tile m and half h: gate_up, dense: offset of the lane's 16 bytes
    // (row 8 h + lane / 8 of the tile, columns 8 (lane % 8) .. + 7 of a group)
    // in the activation rows; down: of the lane's operand words in the tile's
    // group-0 block (h = 1 unused)
    uint32_t l_aoff[MT][2];
    int l_loc = 0;           // items the load cursor has entered (s_dst parity)
    // Down pass: assignment id of chunk row lane % 32 of the item after the load
    // cursor's, loaded at the end of every step (so the item switch uses a value
    // loaded at least a step before).
    int pf_raw = 0;

    auto set_weight_base = [&](const Item& it, const Role& r) __attribute__((always_inline)) {
      const int blk = min(r.blk, p.nblk - 1);  // past the last block: any valid one (never stored)
      l_wbase = wbytes + ((size_t)it.e * p.nblk + blk) * (size_t)G * kTiledUnit;
    };
    auto raw_assign = [&](const Item& it) __attribute__((always_inline)) {
      if constexpr (MODE == MODE_DOWN) {
        return p.assign[min(it.r0 + (lane & 31), A - 1)];
      } else {
        return 0;
      }
    };
    auto put_dst = [&](int loc, const Item& it, int raw) __attribute__((always_inline)) {  // down only
      const int lr = lane & 31;
      s_dst[loc & 1][lr] = (lr < it.rows && raw >= 0 && raw < A) ? raw : -1;
    };
    auto set_act_offset = [&](const Item& it, int j) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int mm = (it.rows > 16) ? m : 0;  // a one-tile chunk reads its tile twice
        if constexpr (MODE == MODE_DOWN) {
          const int tau = max(tile_of(it, mm), 0);
          l_aoff[m][0] = (uint32_t)tau * (uint32_t)(G * kActBlock) + lane * 16;
          l_aoff[m][1] = 0;
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rr = min(16 * mm + 8 * h + (lane >> 3), it.rows - 1);  // row of the chunk
            int src;
            if constexpr (MODE == MODE_GATE_UP) src = s_tok[min(j, kMaxWgItems - 1)][rr];
            else src = it.r0 + rr;
            l_aoff[m][h] = (uint32_t)src * arow + (lane & 7) * 16;
          }
        }
      }
    };
    {
      const int raw0 = raw_assign(linfo);
      pf_raw = raw_assign(ninfo);
      set_weight_base(linfo, lrole);
      set_act_offset(linfo, 0);
      if constexpr (MODE == MODE_DOWN) put_dst(0, linfo, raw0);
    }

    auto issue = [&](Slot<MT>& sl) __attribute__((always_inline)) {
      const uint8_t* u = l_wbase + (size_t)lg * kTiledUnit;
#pragma unroll
      for (int i = 0; i < 4; ++i) sl.w[i] = *(const u32x4_t*)(u + c_off + i * 1024);
#pragma unroll
      for (int h = 0; h < 2; ++h) sl.s[h] = *(const u32x4_t*)(u + s_off + h * 256);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if constexpr (MODE == MODE_DOWN) {  // one coalesced kilobyte per operand register
          const uint8_t* ab = abytes + l_aoff[m][0] + (uint32_t)lg * kActBlock;
          sl.a[m][0] = *(const u32x4_t*)(ab);
          sl.a[m][1] = *(const u32x4_t*)(ab + kActBlock / 2);
        } else {  // 8 rows x 128 bytes per load; compute puts them in operand order
#pragma unroll
          for (int h = 0; h < 2; ++h) sl.a[m][h] = *(const u32x4_t*)(abytes + l_aoff[m][h] + (uint32_t)lg * 128);
        }
      }
    };
    auto advance_load = [&]() __attribute__((always_inline)) {
      if (++lg < lrole.gk1) return;
      if (!n_valid) {  // past the last item: keep re-reading the last item's groups (never used)
        lg = lrole.gk0;
        return;
      }
      linfo = ninfo;
      lrole = role_of(linfo);
      lg = lrole.gk0;
      set_weight_base(linfo, lrole);
      set_act_offset(linfo, n_j);
      ++l_loc;
      if constexpr (MODE == MODE_DOWN) put_dst(l_loc, linfo, pf_raw);
      ++n_j;
      n_valid = has_item(n_j);
      if (n_valid) ninfo = decode(item_of(n_j));
    };

    Slot<MT> ring[DR];
#pragma unroll
    for (int d = 0; d < DR; ++d) {
      issue(ring[d]);
      asm volatile("" ::: "memory");  // keeps the slots' loads in ring order
      advance_load();
      if constexpr (MODE == MODE_DOWN) pf_raw = raw_assign(ninfo);
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

    int c_loc = 0;  // index of the compute cursor's item in this workgroup's sequence
    Item cinfo = decode(item_of(0));
    Role crole = role_of(cinfo);
    int cg = crole.gk0;

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
        // through this wave's own slice of the partial-sum buffer (free while
        // steps run): row r's 16-byte chunk c sits at slot c ^ swz(r), so both
        // the 8-lanes-per-row writes and the operand reads are conflict free
        uint8_t* const scr = qmm_lds + wave * (2 * kNS * 64 * 16);
        auto swz = [](int r) __attribute__((always_inline)) { return ((r & 1) << 2) | ((r >> 1) & 3); };
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m > 0 && !t2) continue;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = 8 * h + (lane >> 3);
            *(u32x4_t*)(scr + m * 2048 + r * 128 + ((lane & 7) ^ swz(r)) * 16) = sl.a[m][h];
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m > 0 && !t2) continue;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            a[m][h] = *(const u32x4_t*)(scr + m * 2048 + ln * 128 + ((2 * lq + h) ^ swz(ln)) * 16);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

    // End of the current item.  Each wave parks in LDS the partial sums of the
    // subtiles that other waves own; after a barrier every owner adds the K
    // parts of its subtiles in K order (its own part straight from registers),
    // stages the results in the part of its own LDS slice that nobody parked
    // into, and writes them with 16-byte stores.
    auto finish_item = [&]() __attribute__((always_inline)) {
      f32x4_t* red = (f32x4_t*)qmm_lds;
      const int nk = crole.nk, kp = crole.kp, blk = crole.blk;
      const bool t2 = cinfo.rows > 16;
      const bool member = wave < nk * NBI;  // not a spare wave
      auto slot_of = [&](int w, int m, int j) __attribute__((always_inline)) {
        return ((w * 2 + m) * kNS + j) * 64 + lane;
      };
      if (member) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int j = 0; j < kNS; ++j)
            if ((m == 0 || t2) && owner_of(j, nk) != kp) red[slot_of(wave, m, j)] = acc[m][j];
      }
      __syncthreads();
      const int wbase = wave - kp;  // wave of K part 0 with the same block
      // K parts of subtile j in K order; `mine` is this wave's part
      auto ksum = [&](int m, int j, f32x4_t mine) __attribute__((always_inline)) {
        f32x4_t v = (kp == 0) ? mine : red[slot_of(wbase, m, j)];
        for (int q = 1; q < nk; ++q) {
          const f32x4_t t = (q == kp) ? mine : red[slot_of(wbase + q, m, j)];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += t[i];
        }
        return v;
      };
      uint8_t* const own = qmm_lds + (size_t)wave * (2 * kNS * 1024);  // this wave's slice
      if (member && blk < p.nblk) {
        if constexpr (MODE == MODE_GATE_UP) {
          // gate j and up j + 4 -> 16 columns of mid, which the down pass reads as
          // group blk of activation tile tau: column 16 j + c of tile row r sits at
          // byte (c / 8) * 1024 + (r + 16 j) * 16 + (c % 8) * 2 of the block
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (owner_of(j, nk) != kp || cinfo.zero) continue;
            uint8_t* const stg = own + j * 1024;  // slot (0, j): owned, so never parked
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if (m > 0 && !t2) continue;
              const f32x4_t g = ksum(m, j, acc[m][j]), u = ksum(m, j + 4, acc[m][j + 4]);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                *(uint16_t*)(stg + m * 512 + (4 * lq + i) * 32 + ln * 2) = f32_to_bf16_bits(gelu_tanh(g[i]) * u[i]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int m = lane >> 5, r = lane & 15, h = (lane >> 4) & 1;
            const int tau = (m == 0 || t2) ? tile_of(cinfo, m) : -1;
            if (tau >= 0) {
              const u32x4_t v = *(const u32x4_t*)(stg + m * 512 + r * 32 + h * 16);
              *(u32x4_t*)((uint8_t*)p.out + ((size_t)tau * (p.Nout / 64) + blk) * kActBlock + h * (kActBlock / 2) +
                          (r + 16 * j) * 16) = v;
            }
          }
        } else if constexpr (MODE == MODE_DOWN) {
          // subtiles [j0, j0 + 8/nk) are this wave's: W = 128 / nk contiguous
          // columns, staged per row tile as bf16 [16 rows][W] in slots (m, j0 ..)
          const int lgnk = nk >> 1;  // log2 nk for nk in {1, 2}
          const int per = kNS >> lgnk, j0 = kp * per, W = 16 * per;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m > 0 && !t2) continue;
            uint16_t* const stg = (uint16_t*)(own + (m * kNS + j0) * 1024);
#pragma unroll
            for (int j = 0; j < kNS; ++j) {
              if (owner_of(j, nk) != kp) continue;
              const f32x4_t v = ksum(m, j, acc[m][j]);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                stg[(4 * lq + i) * W + 16 * (j - j0) + ln] = cinfo.zero ? (uint16_t)0 : f32_to_bf16_bits(v[i]);
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int lgcpr = 4 - lgnk, rpi = 64 >> lgcpr;  // 16-byte chunks per row (W / 8), rows per store
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m > 0 && !t2) continue;
            const uint16_t* const stg = (const uint16_t*)(own + (m * kNS + j0) * 1024);
            for (int r0 = 0; r0 < 16; r0 += rpi) {
              const int r = r0 + (lane >> lgcpr), c = lane & ((1 << lgcpr) - 1);
              const int a = s_dst[c_loc & 1][16 * m + r];
              // a block past the last output row (H % 128 == 64) has no columns there
              if (a >= 0 && blk * BCOLS + 16 * j0 + 8 * c < p.Nout)
                *(u32x4_t*)((uint16_t*)p.out + (size_t)a * p.Nout + blk * BCOLS + 16 * j0 + 8 * c) =
                    *(const u32x4_t*)(stg + r * W + 8 * c);
            }
          }
        } else {
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m > 0 && !t2) continue;
#pragma unroll
            for (int j = 0; j < kNS; ++j) {
              if (owner_of(j, nk) != kp) continue;
              const int col = blk * BCOLS + 16 * j + ln;
              const f32x4_t v = ksum(m, j, acc[m][j]);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int lr = 16 * m + 4 * lq + i;
                if (lr < cinfo.rows && col < p.Nout)
                  ((uint16_t*)p.out)[(size_t)(cinfo.r0 + lr) * p.Nout + col] = f32_to_bf16_bits(v[i]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < kNS; ++j) acc[m][j] = zero4();
      __syncthreads();  // partial-sum buffer free again
    };

    // One ring step on slot d: compute the current group, refill the slot.  Every
    // step issues its loads, also after the last item (compute is skipped then):
    // the loop has a single exit at the end of a block of D steps and the wait
    // before each slot always counts the loads of the D - 1 slots issued after it.
    bool done = false;
    auto step = [&](auto d_tag) __attribute__((always_inline)) {
      constexpr int d = decltype(d_tag)::value;
      fence_slot(ring[d]);
      if (!done && !cinfo.zero && crole.blk < p.nblk) {
        const int kq = (cg - crole.gk0) & 3;
        compute(ring[d], kq);
        if (kq == 3 || cg + 1 == crole.gk1) flush_bias();
      }
      issue(ring[d]);
      asm volatile("" ::: "memory");  // keeps the slots' loads in ring order
      advance_load();
      if constexpr (MODE == MODE_DOWN) pf_raw = raw_assign(ninfo);
      if (done || ++cg < crole.gk1) return;
      finish_item();
      if (!has_item(c_loc + 1)) {
        done = true;
        return;
      }
      ++c_loc;
      cinfo = decode(item_of(c_loc));
      crole = role_of(cinfo);
      cg = crole.gk0;
    };
    do {
      run_steps(step, std::make_integer_sequence<int, DR>{});
    } while (!done);
    // the loads issued past the end are consumed here (they complete before the wave ends)
#pragma unroll
    for (int d = 0; d < DR; ++d) fence_slot(ring[d]);
  };
  body(std::integral_constant<int, 2>{});
}

// ---------------------------------------------------------------- weight tiling
// Weight row of block b, subtile j, row n (split > 0: gate rows then up rows).
__device__ __forceinline__ int tiled_row(int b, int j, int n, int split) {
  if (split > 0) return (j < 4) ? 64 * b + 16 * j + n : split + 64 * b + 16 * (j - 4) + n;
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
      if (row < rows) {
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
      if (row < rows) {
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
  for (int j = 0; j < k; ++j) {
    const u32x4_t v = *(const u32x4_t*)(base + (size_t)j * H);
    const float wj = w[(size_t)t * k + j];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[2 * q] += wj * bf16_lo_f32(v[q]);
      s[2 * q + 1] += wj * bf16_hi_f32(v[q]);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(s[2 * q], s[2 * q + 1]);
  *(u32x4_t*)(y + (size_t)t * H + h) = o;
}

// ------------------------------------------------------------------ launchers
namespace {

template <int MODE, int NBI, int D>
hipError_t launch_cfg(SwitchArgs a, int extra_buckets, int num_cu, hipStream_t stream) {
  a.ntiles = (a.nblk + NBI - 1) / NBI;
  const size_t lds = (size_t)kWaves * 2 * kNS * 64 * 16;  // partial sums of every wave and row tile
  long long chunks;
  if (MODE == MODE_DENSE)
    chunks = (a.rows_total + kBM - 1) / kBM;
  else
    chunks = (a.rows_total + kBM - 1) / kBM + (long long)std::min(a.E, a.rows_total) + extra_buckets;
  const long long items = chunks * a.ntiles;
  long long grid = std::min(items, (long long)num_cu * 2);
  if (MODE == MODE_GATE_UP) grid = std::max(grid, (items + kMaxWgItems - 1) / kMaxWgItems);
  if (grid < 1) grid = 1;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&qmm_kernel<MODE, NBI, D>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((qmm_kernel<MODE, NBI, D>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

// Blocks per item and ring depth: one block per item when a single-tile chunk
// still leaves each of the 4 K parts at least 3 groups, else two; the ring is
// as deep as the fewest groups a wave owns allow (at most 4), so the load
// cursor is never more than one item ahead of the compute cursor.
template <int MODE>
hipError_t launch_mode(SwitchArgs a, int extra_buckets, int num_cu, hipStream_t stream) {
  const int G = a.K / 64;
  const int nbi = (G >= 12) ? 1 : 2;
  const int depth = std::min(4, std::max(1, G / (kWaves / nbi)));  // groups of the smallest K part
  if (nbi == 1) {
    if (depth >= 4) return launch_cfg<MODE, 1, 4>(a, extra_buckets, num_cu, stream);
    return launch_cfg<MODE, 1, 3>(a, extra_buckets, num_cu, stream);
  }
  if (depth >= 4) return launch_cfg<MODE, 2, 4>(a, extra_buckets, num_cu, stream);
  if (depth == 3) return launch_cfg<MODE, 2, 3>(a, extra_buckets, num_cu, stream);
  if (depth == 2) return launch_cfg<MODE, 2, 2>(a, extra_buckets, num_cu, stream);
  return launch_cfg<MODE, 2, 1>(a, extra_buckets, num_cu, stream);
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
hipError_t launch_combine(const uint16_t* D, const float* w, int T, int k, int H, uint16_t* y, hipStream_t stream) {
  const long long n = (long long)T * (H / 8);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, D, w, T, k, H, y);
  return hipGetLastError();
}
int tiled_blocks(int rows, int split) { return split > 0 ? split / 64 : (rows + 127) / 128; }
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

// Internal kernel-launch interface between the C ABI (abi.cpp) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

// ---------------------------------------------------------------- router
struct RouteArgs {
  const uint16_t* x;          // bf16 [T, H]
  const uint16_t* norm_scale; // bf16 [H]
  const uint32_t* w;          // router codes [E, H/8]
  const uint16_t* s;          // router scales [E, H/64]
  const uint16_t* b;          // router biases [E, H/64]
  const uint16_t* pes;        // bf16 [E]
  const float* logit_bias;    // fp32 [E] or null
  float* part;                // fp32 [ksplit, T, E] partial logits (workspace)
  int32_t* indices;           // [T, k]
  float* weights;             // [T, k]
  float* logits_out;          // [T, E] or null
  float eps;
  float root;                 // H^-0.5 rounded to fp32
  int T, H, E, k, ksplit;
};
int route_ksplit(int T, int H);
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- sort
// Workspace of the slice sort (0 below 8192 assignments); with less, the
// one-workgroup sort runs.
size_t sort_workspace_bytes(int A, int E);
hipError_t launch_sort(const int32_t* indices, int A, int E, int32_t* offsets, int32_t* sorted_assign, void* ws,
                       size_t ws_bytes, hipStream_t stream);

// ---------------------------------------------------------------- switch / dense linears
// Bytes of one tiled unit: (expert, block of 128 weight rows, 64-wide group) ->
// 4096 bytes of codes in operand order + 128 (scale, bias) pairs.
constexpr int kTiledUnit = 4608;
int tiled_blocks(int rows, int split);
hipError_t launch_tile_weight(const uint32_t* w, const uint16_t* s, const uint16_t* b, int E, int rows, int K,
                              int split, uint8_t* dst, hipStream_t stream);

// Activation tiles (mid, between the two switch linears): the rows of expert
// e's segment are cut into 16-row tiles, numbered expert by expert; per (tile,
// 64-wide group) one block of kActBlock bytes in MFMA operand order (layout in
// qmoe.h).
constexpr int kActBlock = 2048;
long long act_tiles_max(long long A, int E);

// gate_up + GeGLU and down over sorted expert rows; the dense linear; the
// dense linear with a fused gate|up weight and the GeGLU (the decoder's dense
// MLP branch, first half); the dense linear as the tied LM head, its bf16
// logits widened and softcapped to fp32
enum : int { MODE_GATE_UP = 0, MODE_DOWN = 1, MODE_DENSE = 2, MODE_DENSE_GEGLU = 3, MODE_DENSE_SOFTCAP = 4 };

struct SwitchArgs {
  const uint16_t* a;       // gate_up, dense: bf16 rows of length K; down: activation tiles
  const void* w;           // tiled weight [E, nblk, K/64] units of kTiledUnit bytes
  int nblk;                // tiled blocks per expert
  const int32_t* offsets;  // [E+1] sorted-row segments (switch modes)
  const int32_t* assign;   // [A] assignment id of each sorted row (switch modes)
  void* out;
  int K;           // contraction length (multiple of 64)
  int Nout;        // output columns
  int E;           // experts (1 for dense)
  int ktop;        // assignments per token
  uint32_t ktop_inv;  // floor(2^32 / ktop) + 1, or 0 when ktop is 1 (set by the launcher; see token_of)
  int rows_total;  // dense: M; switch: A = T*k
  int ntiles;      // column tiles per row chunk (set by the launcher)
  int max_tiles;   // switch: activation tiles the input and output buffers hold
  float cap;       // softcap of the LM-head mode
  int* status;     // device status word (set by the launcher)
};
// The token of assignment a (a / k, with 0 <= a < 2^24 and 1 <= k <= 16) as
// one multiply-high: a * (floor(2^32 / k) + 1) / 2^32 exceeds a / k by less
// than 2^24 / 2^32 = 2^-8, and the fraction of a / k is 0 or at least 1/16,
// so the floor is exact.  inv = 0 stands for k = 1.
inline uint32_t ktop_inverse(int k) { return k > 1 ? (uint32_t)((1ull << 32) / (unsigned)k + 1) : 0u; }
__device__ __forceinline__ int token_of(int a, uint32_t inv) {
  return inv ? (int)(((uint64_t)(uint32_t)a * inv) >> 32) : a;  // v_mul_hi_u32
}
// Device status word: bits a kernel raises when a bounded wait inside a
// workgroup gave up (its outputs are then wrong).
constexpr int kStatusSpin = 1;
// this device's status word (a device address), or null
int* device_status();
// Scratch held by the library for the entry points that allocate nothing:
// this device's array (a device address), or null
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
void* noalloc_scratch();
hipError_t launch_gate_up_geglu(SwitchArgs a, int num_cu, hipStream_t stream);
hipError_t launch_down(SwitchArgs a, int num_cu, hipStream_t stream);
hipError_t launch_dense(SwitchArgs a, int num_cu, hipStream_t stream);
// dense rows against a fused gate|up weight (tiled with split = Nout), GeGLU,
// row-major bf16 [rows_total, Nout] out
hipError_t launch_dense_geglu(SwitchArgs a, int num_cu, hipStream_t stream);
// dense rows against the tied head's weight; fp32 [rows_total, Nout] out,
// cap * tanh(bf16(logit) / cap)
hipError_t launch_dense_softcap(SwitchArgs a, int num_cu, hipStream_t stream);
hipError_t launch_combine(const uint16_t* D, const float* w, int T, int k, int H, uint16_t* y, hipStream_t stream);
// The weight-stationary kernel (many rows per weight block; the tied head):
// whether it is the faster one for `rows` rows, and its launcher (same
// arguments and outputs as launch_dense_softcap; the dequantized weight is
// rounded to bf16 once).
bool ws_preferred(int mode, long long rows, int experts);
template <int MODE>
hipError_t launch_ws(SwitchArgs a, int num_cu, hipStream_t stream);

// The tall-tile kernel (hundreds to thousands of rows per weight block; the
// dense linear, plain or with the GeGLU, and the gate_up switch linear):
// whether it is the faster one for `rows` rows (A = T*k for gate_up) over
// `experts` experts, and its launcher (same arguments and outputs as
// launch_dense, launch_dense_geglu and launch_gate_up_geglu; the dequantized
// weight is rounded to bf16 once).
bool tall_preferred(int mode, long long rows, int experts);
template <int MODE>
hipError_t launch_tall(SwitchArgs a, int num_cu, hipStream_t stream);

// ---------------------------------------------------------------- unsorted small-batch switch linears
enum : int { UNSORTED_GATE_UP = 0, UNSORTED_DOWN = 1 };
struct UnsortedArgs {
  const uint16_t* x;        // gate_up: bf16 [T, K] tokens; down: bf16 [A, K] mid rows
  const void* w;            // tiled weight [E, nblk, K/64] units
  const int32_t* indices;   // [A] expert of each assignment
  const float* weights;     // [A] routing weights (down)
  uint16_t* out;            // gate_up: bf16 [A, Nout] mid rows; down: bf16 [T, Nout] y
  float* part;              // workspace: [A * nblk * S][128] partial sums
  int A, k, K, G, nblk, E, Nout;
  int S;    // workgroups per (assignment, block)
  int gpw;  // groups per wave
};
struct UnsortedPlan {
  int gpw, S;
  long long partials;  // floats
};
UnsortedPlan unsorted_plan(long long A, int nblk, int G);
hipError_t launch_unsorted(int mode, UnsortedArgs a, hipStream_t stream);

// ---------------------------------------------------------------- self-conditioning embedding
// the untransposed table's tiling, 1152-byte units per (64-column group, 32-row chunk)
hipError_t launch_tile_weight_t(const uint32_t* w, const uint16_t* s, const uint16_t* b, int V, int H, uint8_t* dst,
                                hipStream_t stream);
int embed_t_splits(int L, int V, int H);  // row ranges summed by the second kernel (workspace: splits * L * H fp32)
hipError_t launch_embed_t(const uint16_t* probs, int L, int V, int H, const void* wt, float scale, float* part,
                          uint16_t* out, hipStream_t stream);
hipError_t launch_softmax_rows_bf16(const float* z, int L, int V, uint16_t* probs, hipStream_t stream);

// ---------------------------------------------------------------- feed-forward block norms
// xa = rms(h) * wa, xb = rms(h) * wb (bf16 [T, H] each, H % 8 == 0)
hipError_t launch_ff_prenorm(const uint16_t* h, int T, int H, const uint16_t* wa, const uint16_t* wb, float eps,
                             uint16_t* xa, uint16_t* xb, hipStream_t stream);
// out = (res + rms(rms(h1) w1 + rms(h2) w2) w) * scalar (bf16 [T, H], H % 8 == 0)
hipError_t launch_ff_combine(const uint16_t* res, const uint16_t* h1, const uint16_t* h2, int T, int H,
                             const uint16_t* w1, const uint16_t* w2, const uint16_t* w, float eps, float scalar,
                             uint16_t* out, hipStream_t stream);

}  // namespace qmoe

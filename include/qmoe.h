/*
 * qmoe.h -- C ABI of the 4-bit group-quantized mixture-of-experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the one of the DiffusionGemma decoder as the
 * "@mlx-bun/inference 0.0.0-stage -> 1.0.0" diff pages show it
 * (diffusion-gemma model.ts page: DiffRouter, DiffExperts and
 * DiffDecoderLayer.forwardWith; vision.ts page: VisionLinear, manualRms,
 * DiffVisionMLP).  One call per step of the layer:
 *
 *   moe_route             router: norm, scale, 4-bit projection, top-k,
 *                         precise softmax, per_expert_scale
 *   moe_sort              token-by-expert sort of the routing assignments
 *   qswitch_gate_up_geglu fused gate_up switch linear, split, GeGLU
 *   qswitch_down_combine  down switch linear + weighted sum over k per token
 *   qlinear               dense 4-bit linear
 *   qswitch_gate_up_geglu_unsorted, qswitch_down_combine_unsorted
 *                         the small-batch arm without the sort
 *   qlinear_softcap       the tied LM head with its fp32 tanh softcap
 *   softmax_rows_bf16, embed_matmul_t
 *                         the self-conditioning embedding (probabilities
 *                         times the untransposed 4-bit table)
 *   ff_prenorm, qlinear_geglu, ff_combine
 *                         the decoder's feed-forward block around the MoE
 *                         (pre-norms, dense GeGLU branch, post-norms and
 *                         residual)
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array pointers are DEVICE pointers (memory of the current HIP device),
 *   except the qmoe_qweight struct itself, which lives in host memory and is
 *   read during the call only.  Sizes are host integers.
 * - bf16 values are passed as their uint16_t bit patterns.  All arrays are
 *   dense and row-major.
 * - Quantized weights: 4-bit affine codes, group size 64, eight codes per
 *   uint32 word with code c of a row in bits 4*(c%8)..4*(c%8)+3 of word c/8
 *   (first code in the lowest bits); scales and biases are bf16, one per
 *   group; the weight value is scale*q + bias (model.ts page,
 *   dequantEmbedWeight).  The router takes this row-major layout as it is;
 *   the switch linears and qlinear take the tiled layout that
 *   qmoe_tile_weight produces from it once (same values, same bytes).
 * - Alignment: activation, weight-code, mid and output arrays must be 16-byte
 *   aligned; scales, biases and bf16 vectors 2-byte aligned; int32/fp32
 *   arrays 4-byte aligned.
 * - Ownership: the caller allocates and owns every buffer, including
 *   workspaces; the library allocates no device memory and keeps no pointer
 *   after a call returns.
 * - Ordering: every call enqueues its kernels on `stream` and returns
 *   without waiting.  Arguments are validated on the host before anything is
 *   enqueued: a call that returns an error has enqueued nothing.  Faults that
 *   happen inside a kernel surface at the caller's next synchronisation.
 * - T == 0 (or M == 0) is a no-op that returns QMOE_OK without reading any
 *   pointer.
 * - The calls are reentrant; the last error message is per thread.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define QMOE_OK 0
#define QMOE_ERR_INVALID (-1)     /* null pointer, bad size, misalignment        */
#define QMOE_ERR_UNSUPPORTED (-2) /* bits != 4, group != 64, E > 256, k > 16 ... */
#define QMOE_ERR_WORKSPACE (-3)   /* workspace missing or too small              */
#define QMOE_ERR_HIP (-4)         /* a HIP launch or query failed                */

/* Weight layouts (qmoe_qweight.layout). */
#define QMOE_LAYOUT_ROWS 0  /* row-major codes + separate scale/bias arrays   */
#define QMOE_LAYOUT_TILED 1 /* the tiled buffer written by qmoe_tile_weight   */
#define QMOE_LAYOUT_TILED_T 2 /* the buffer written by qmoe_tile_weight_t     */

/* A 4-bit group-quantized weight (one dense matrix, or `experts` stacked
 * matrices for a switch linear) of `rows` output rows and `in` inputs.
 *
 * layout QMOE_LAYOUT_ROWS:
 *   w       uint32 [experts, rows, in/8]
 *   scales  bf16   [experts, rows, in/64]
 *   biases  bf16   [experts, rows, in/64]
 *   split   ignored
 * layout QMOE_LAYOUT_TILED: `w` points to the qmoe_tile_weight buffer (codes,
 *   scales and biases together); `scales` and `biases` are ignored; `split`
 *   is the value the buffer was tiled with.
 * The struct is host memory; the arrays are device memory. */
typedef struct qmoe_qweight {
  const uint32_t* w;
  const uint16_t* scales;
  const uint16_t* biases;
  int32_t experts; /* 1 for a dense linear */
  int32_t rows;
  int32_t in;
  int32_t bits;   /* must be 4  */
  int32_t group;  /* must be 64 */
  int32_t layout; /* QMOE_LAYOUT_ROWS or QMOE_LAYOUT_TILED */
  int32_t split;  /* tiled only: 0, or the first row of the second half of a fused pair */
} qmoe_qweight;

/* Text of the last error raised on the calling thread ("" if none).  The
 * string is owned by the library and valid until the next call on this
 * thread. */
const char* qmoe_last_error(void);

/* The current device's status word: bits the kernels raise when a bounded
 * wait inside a workgroup gave up (1) or a workgroup met more sorted rows
 * than its LDS holds (2); the outputs of such a call are wrong.  0 means no
 * kernel has raised anything since the last reset.  Waits for the device
 * (hipDeviceSynchronize), then copies the word to *value and, if reset is
 * non-zero, clears it.  A debugging and testing aid; not needed for normal
 * use. */
int qmoe_device_status(int32_t* value, int32_t reset);

/* ------------------------------------------------------------------------
 * qmoe_tile_weight -- re-lays a row-major 4-bit weight into the tiled layout
 * the switch linears and qlinear read.  A pure permutation of the codes,
 * scales and biases (no arithmetic): the operation is the same QuantizedLinear
 * / QuantizedSwitchLinear weight (model.ts page, DiffExperts: gateUp, down;
 * vision.ts page, VisionLinear).  Done once when the weights are loaded.
 *
 * Tiled layout: units of 4608 bytes, unit index ((e * nblk + b) * (in/64) + g)
 * for expert e, row block b, group g; nblk = ceil(rows / 128) blocks for
 * split == 0, ceil(split / 64) for a fused pair.  Block b holds 8 subtiles of
 * 16 rows; row n of subtile j is weight row
 *   split == 0:  128 b + 16 j + n
 *   split  > 0:  with c = 64 b + 16 (j % 4) + n:  j < 4: c;  j >= 4: split + c
 * (so a fused gate|up weight keeps gate row c and up row split + c in one
 * block); rows past `rows`, and for a fused pair every c >= split, read as
 * zero.  Bytes [0, 4096) of a unit: for
 * i = 0..3 and lane L = 0..63 (n = L % 16, q = L / 16), 16 bytes at
 * 1024 i + 16 L = two code words of subtile 2i then two of subtile 2i+1 of
 * row n: word 2q and word 2q+1 of the group (codes 16q .. 16q+15), each with
 * its code 2p moved to bits 4p and code 2p+1 to bits 16+4p (p = 0..3).
 * Bytes [4096, 4608): for h = 0..1 and n = 0..15, 16 bytes at
 * 4096 + 256 h + 16 n = (scale, bias) bf16 pairs of subtiles 4h .. 4h+3, row n.
 *
 *   src        layout QMOE_LAYOUT_ROWS, in % 64 == 0
 *   split      0, or rows/2 for a fused pair (split % 16 == 0; the switch
 *              calls need split % 64 == 0 since their I is a multiple of 64)
 *   dst        device buffer of qmoe_tiled_weight_bytes(...) bytes, 16-byte
 *              aligned, owned by the caller (the tiled weight's `w`)
 * qmoe_tiled_weight_bytes returns 0 for sizes it does not accept.
 * ---------------------------------------------------------------------- */
size_t qmoe_tiled_weight_bytes(int32_t experts, int32_t rows, int32_t in, int32_t split);
int qmoe_tile_weight(const qmoe_qweight* src, int32_t split, void* dst, size_t dst_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_route -- the DiffRouter (model.ts page, DiffRouter.forward; the norm
 * is the no-scale RMS norm of vision.ts page, manualRms with a null weight):
 *
 *   r   = x / sqrt(mean_h(x^2) + eps)          per token
 *   u   = r * norm_scale[h] * H^-0.5
 *   l_e = u . dequant(proj)[e] (+ logit_bias[e])          fp32 logits
 *   indices[t, 0..k)  = the k largest l_e, descending, ties to lower e
 *   weights[t, j]     = softmax_j(l[indices]) * per_expert_scale[indices[t, j]]
 *
 * The router is evaluated in fp32 throughout (no intermediate bf16 rounding).
 *
 *   x_router          bf16 [T, H]   the residual stream rows the router sees
 *   norm_scale        bf16 [H]      per-dimension scale applied after the norm
 *   eps               norm epsilon (the build uses 1e-6)
 *   proj              experts = 1, rows = E, in = H, layout QMOE_LAYOUT_ROWS
 *   per_expert_scale  bf16 [E]
 *   logit_bias        fp32 [E] added to the logits before top-k, or NULL
 *   k                 1 <= k <= min(E, 16);  E <= 256;  H % 64 == 0
 *   indices (out)     int32 [T, k]
 *   weights (out)     fp32  [T, k]
 *   logits_out (out)  fp32  [T, E] logits incl. logit_bias, or NULL
 *   workspace         device scratch of at least moe_route_workspace(T, H, E)
 *                     bytes (partial logits and row sums of squares of the
 *                     k-range split; NULL allowed when that size is 0)
 * ---------------------------------------------------------------------- */
size_t moe_route_workspace(int32_t T, int32_t H, int32_t E);
int moe_route(const uint16_t* x_router, int32_t T, int32_t H, const uint16_t* norm_scale,
              float eps, const qmoe_qweight* proj, const uint16_t* per_expert_scale,
              const float* logit_bias, int32_t k, int32_t* indices, float* weights,
              float* logits_out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_sort -- token-by-expert sort (model.ts page, DiffExperts.forward:
 * argsort of the flat routing indices).  Assignment a = t*k + j goes to
 * expert indices[a].
 *
 *   indices            int32 [T*k], values in [0, E)
 *   expert_offsets(out) int32 [E+1]: offsets[e] = number of assignments with
 *                      an expert below e (offsets[E] = T*k)
 *   sorted_assign (out) int32 [T*k]: assignment ids grouped by expert,
 *                      ascending within an expert (stable)
 *
 * An index outside [0, E) is dropped: it is counted nowhere and offsets[E]
 * is then below T*k (the later calls process only offsets[E] rows); the
 * dropped ids fill sorted_assign[offsets[E] .. T*k) in ascending order.
 * E <= 256; T*k <= 2^24.
 *
 *   workspace          device, 4-byte aligned, moe_sort_workspace(T, k, E)
 *                      bytes (0 below 8192 assignments; about 1 KB per slice
 *                      of at least 1024 assignments, at most 256 slices).
 *                      With it, 8192 and more assignments are sorted by two
 *                      kernels over many workgroups (slice histograms, then
 *                      each slice placed at its offsets); with a null or
 *                      smaller workspace one workgroup sorts the whole input.
 *                      Both give the same output.  The call overwrites it.
 * ---------------------------------------------------------------------- */
size_t moe_sort_workspace(int32_t T, int32_t k, int32_t E);
int moe_sort(const int32_t* indices, int32_t T, int32_t k, int32_t E, int32_t* expert_offsets,
             int32_t* sorted_assign, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Activation tiles (the layout of mid)
 *
 * The sorted rows of expert e's segment [offsets[e], offsets[e+1]) are cut
 * into tiles of 16 rows (the last one of a segment may be partial); tiles are
 * numbered expert by expert, so tile tau of expert e's local tile j is
 *   tau = sum_{e' < e} ceil(n_e' / 16) + j,   n_e = offsets[e+1] - offsets[e].
 * Each (tile tau, 64-wide column group g) owns one 2048-byte block at
 *   (tau * (C / 64) + g) * 2048            (C = columns of the matrix)
 * holding the tile's 16 x 64 bf16 values in the operand order of
 * v_mfma_f32_16x16x32_bf16: the bf16 at byte h*1024 + L*16 + 2*i
 * (h in {0,1}, L in [0,64), i in [0,8)) is column 64 g + 16 (L/16) + 8 h + i
 * of tile row L % 16.  Rows past the end of a segment hold unspecified
 * values.  A buffer of C columns for T*k assignments and E experts takes
 *   qswitch_mid_bytes(T, k, C, E) = (ceil(T*k / 16) + min(E, T*k)) * (C/64) * 2048
 * bytes, which covers every possible split of the rows among the experts.
 * ---------------------------------------------------------------------- */
size_t qswitch_mid_bytes(int32_t T, int32_t k, int32_t C, int32_t E);

/* ------------------------------------------------------------------------
 * qswitch_gate_up_geglu -- fused gate_up QuantizedSwitchLinear over the
 * sorted rows, split at moe_intermediate, GeGLU (model.ts page,
 * DiffExperts.forward: gateUp.forward, split, geglu; the GeGLU is
 * gelu_approx(gate) * up as in vision.ts page, DiffVisionMLP):
 *
 *   for sorted row r in [0, offsets[E]):  a = sorted_assign[r], t = a / k,
 *   e = the expert whose segment holds r,
 *   g = x[t] . dequant(gate_up)[e]^T            (2I values, fp32 accumulate)
 *   mid[r, n] = gelu_tanh(g[n]) * g[I + n]      n < I, stored bf16
 *
 *   x_expert        bf16 [T, H]  the (normalised) rows the experts see
 *   gate_up         experts = E, rows = 2*I, in = H, layout QMOE_LAYOUT_TILED
 *                   tiled with split = I
 *   I               moe_intermediate, I % 64 == 0
 *   expert_offsets, sorted_assign   as produced by moe_sort
 *   mid (out)       activation tiles of I columns (layout above), at least
 *                   qswitch_mid_bytes(T, k, I, E) bytes (mid_bytes)
 * ---------------------------------------------------------------------- */
int qswitch_gate_up_geglu(const uint16_t* x_expert, int32_t T, int32_t H,
                          const qmoe_qweight* gate_up, int32_t I, int32_t k,
                          const int32_t* expert_offsets, const int32_t* sorted_assign,
                          void* mid, size_t mid_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * qswitch_down_combine -- down QuantizedSwitchLinear plus the weighted sum
 * back per token (model.ts page, DiffExperts.forward: down.forward, unsort,
 * (y * weights[..., None]).sum over k):
 *
 *   d_r  = mid[r] . dequant(down)[e]^T   (fp32 accumulate, rounded to bf16 as
 *          the pages' quantized matmul returns it)
 *   y[t] = sum_j weights[t, j] * d_{row of assignment t*k+j}   (fp32, j order)
 *   y is stored bf16 (round to nearest even).
 *
 *   mid             activation tiles of I columns as qswitch_gate_up_geglu
 *                   writes them, for the same expert_offsets
 *   down            experts = E, rows = H, in = I, layout QMOE_LAYOUT_TILED
 *                   tiled with split = 0
 *   weights         fp32 [T, k] routing weights (moe_route)
 *   y (out)         bf16 [T, H]; a token none of whose assignments is
 *                   present (dropped indices) gets the sum of the rest
 *   workspace       at least qswitch_down_combine_workspace(T, k, H, det)
 *                   bytes of device scratch
 *   deterministic   1: per-assignment bf16 rows d_r in the workspace, then a
 *                   fixed-order sum (bitwise
 *                   reproducible);  0: same path today (reserved for an
 *                   atomic scatter-sum)
 * ---------------------------------------------------------------------- */
size_t qswitch_down_combine_workspace(int32_t T, int32_t k, int32_t H, int32_t deterministic);
int qswitch_down_combine(const void* mid, int32_t T, int32_t k, int32_t I,
                         const qmoe_qweight* down, int32_t H, const int32_t* expert_offsets,
                         const int32_t* sorted_assign, const float* weights, uint16_t* y,
                         void* workspace, size_t ws_bytes, int32_t deterministic,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * qswitch_down_combine_noalloc -- qswitch_down_combine without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * qswitch_down_combine (bit for bit); the workspace is a 16 MiB array the
 * library holds on each device it runs on, until the process ends.
 *
 * Limit: qswitch_down_combine_workspace(T, k, H, det) <= 16 MiB, i.e.
 * T*k*H*2 <= 16777216 (the 256-token canvas at H 2816, top-8 takes 11.5 MB);
 * above it the call returns QMOE_ERR_UNSUPPORTED and does nothing.
 * Every call on one device shares that device's array: calls that overlap on
 * one device (other streams, other host threads) race and give wrong
 * results; serialize them.  Nothing in the array needs clearing between
 * calls (each call writes what it reads).
 * ---------------------------------------------------------------------- */
int qswitch_down_combine_noalloc(const void* mid, int32_t T, int32_t k, int32_t I,
                                 const qmoe_qweight* down, int32_t H,
                                 const int32_t* expert_offsets, const int32_t* sorted_assign,
                                 const float* weights, uint16_t* y, int32_t deterministic,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * Unsorted small-batch arm (model.ts page, DiffExperts.forward: below 64
 * assignments the flat indices are not sorted and the gather matmuls read
 * each assignment's expert directly; the model's decode layers use this arm
 * when canvas length times top-k is under 64).  Same results as the sorted
 * calls up to fp32 summation order:
 *
 *   qswitch_gate_up_geglu_unsorted:  mid_rows[a] = gelu_tanh(g) * u,
 *       (g, u) = x_expert[a / k] . dequant(gate_up[indices[a]])^T split at I
 *   qswitch_down_combine_unsorted:   d_a = bf16(mid_rows[a] . dequant(down[e_a])^T),
 *       y[t] = sum_j weights[t, j] * d_{t k + j}   (fp32, j order, bf16 out)
 *
 *   x_expert    bf16 [T, H]
 *   gate_up     experts = E, rows = 2I, in = H, tiled with split = I
 *   down        experts = E, rows = H, in = I, tiled with split = 0
 *   indices     int32 [T, k] (moe_route's output); an index outside [0, E)
 *               drops its assignment: its mid row is zero and y leaves it out
 *   mid_rows    bf16 [T*k, I], row a = assignment t*k + j (plain row-major;
 *               not the activation tiles of the sorted calls)
 *   weights     fp32 [T, k]
 *   y (out)     bf16 [T, H]
 *   workspace   qswitch_unsorted_workspace(T, k, H, I) bytes of device
 *               scratch (fp32 partial sums), 16-byte aligned, any contents;
 *               one buffer serves both calls.  Calls that share a workspace
 *               must not overlap in time.
 *
 * H % 64 == 0, I % 64 == 0, 1 <= k <= 16, E <= 256, T*k <= 4096 (larger
 * batches: the sorted calls; qswitch_unsorted_workspace returns 0 for sizes
 * it does not accept).  The result does not depend on how the work is split;
 * it is bitwise reproducible run to run.
 * ---------------------------------------------------------------------- */
size_t qswitch_unsorted_workspace(int32_t T, int32_t k, int32_t H, int32_t I);
int qswitch_gate_up_geglu_unsorted(const uint16_t* x_expert, int32_t T, int32_t H,
                                   const qmoe_qweight* gate_up, int32_t I, int32_t k,
                                   const int32_t* indices, uint16_t* mid_rows, void* workspace,
                                   size_t ws_bytes, hipStream_t stream);
int qswitch_down_combine_unsorted(const uint16_t* mid_rows, int32_t T, int32_t k, int32_t I,
                                  const qmoe_qweight* down, int32_t H, const int32_t* indices,
                                  const float* weights, uint16_t* y, void* workspace,
                                  size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * qlinear -- dense 4-bit QuantizedLinear (vision.ts page, VisionLinear.forward,
 * quantized arm; model.ts page, DiffRouter.proj):  y = x . dequant(W)^T,
 * fp32 accumulate, bf16 out.
 *
 *   x        bf16 [M, K]
 *   W        experts = 1, rows = N, in = K;  K % 64 == 0, N % 16 == 0;
 *            layout QMOE_LAYOUT_TILED, split = 0
 *   y (out)  bf16 [M, N]
 * ---------------------------------------------------------------------- */
int qlinear(const uint16_t* x, int32_t M, const qmoe_qweight* W, uint16_t* y,
            hipStream_t stream);

/* ------------------------------------------------------------------------
 * qlinear_softcap -- the tied LM head (model.ts page, logitsFromHidden): the
 * embedding's 4-bit weight used as a linear, its logits returned in bf16 as
 * the quantized matmul returns them, widened to fp32 and softcapped:
 *   y[m, v] = cap * tanh(bf16(x[m] . dequant(E)[v]) / cap)      (fp32 out)
 * cap is the model's final-logit softcapping (30 when the config leaves it
 * out, model.ts page, the decoder constructor).
 *
 *   x        bf16 [M, K]
 *   W        experts = 1, rows = N (vocabulary), in = K;  K % 64 == 0,
 *            N % 16 == 0; layout QMOE_LAYOUT_TILED, split = 0
 *   cap      finite, > 0
 *   y (out)  fp32 [M, N]
 * ---------------------------------------------------------------------- */
int qlinear_softcap(const uint16_t* x, int32_t M, const qmoe_qweight* W, float cap, float* y,
                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * The self-conditioning embedding (model.ts page, #embedCanvas): the
 * precise softmax of the self-conditioning logits cast to bf16, times the
 * embedding table's 4-bit weight used WITHOUT transposing, returned in bf16,
 * times embed_scale (sqrt(hidden) in the model):
 *
 *   softmax_rows_bf16:  probs[l, v] = bf16( exp(z - max) / sum exp(z - max) )
 *                       (fp32 inside)
 *   embed_matmul_t:     out[l, h] = bf16( bf16( sum_v probs[l, v] E[v, h] )
 *                                         * scale ),  E[v, h] = s q + b
 *
 * In the product each term is formed as bf16(p s) (128 + q) - 128 bf16(p s)
 * + bf16(p b) with fp32 sums (the pages' quantized matmul rounds the
 * dequantized table to bf16 instead; both round each term once).
 *
 * qmoe_tile_weight_t -- re-lays the table [V, H] (experts = 1, rows = V,
 * in = H, layout QMOE_LAYOUT_ROWS; V % 32 == 0, H % 64 == 0) for the product:
 * units of 1152 bytes, unit index g * (V/32) + c for 64-column group g and
 * 32-row chunk c.  Bytes [0, 1024): lane L = 16 kq + n (n = L % 16) holds at
 * 16 L four words; word j has the codes of rows 32 c + 8 kq + t (t = 0..7)
 * at column 64 g + 16 j + n, code t = 2p at bits 4p and t = 2p + 1 at bits
 * 16 + 4p.  Bytes [1024, 1152): the 32 rows' (scale, bias) bf16 pairs of
 * group g, row 32 c + r at 1024 + 4 r.  The result is described by a
 * qmoe_qweight with layout QMOE_LAYOUT_TILED_T, rows = V, in = H, w = dst.
 *
 *   z           fp32 [L, V], V % 4 == 0          (softmax_rows_bf16)
 *   probs       bf16 [L, V], V % 32 == 0         (embed_matmul_t input)
 *   W           layout QMOE_LAYOUT_TILED_T, experts = 1, rows = V, in = H
 *   out (out)   bf16 [L, H]
 *   workspace   embed_matmul_t_workspace(L, V, H) bytes (fp32 partial sums)
 * ---------------------------------------------------------------------- */
size_t qmoe_tiled_weight_t_bytes(int32_t V, int32_t H);
int qmoe_tile_weight_t(const qmoe_qweight* src, void* dst, size_t dst_bytes, hipStream_t stream);
int softmax_rows_bf16(const float* z, int32_t L, int32_t V, uint16_t* probs, hipStream_t stream);
size_t embed_matmul_t_workspace(int32_t L, int32_t V, int32_t H);
int embed_matmul_t(const uint16_t* probs, int32_t L, const qmoe_qweight* W, float scale, uint16_t* out,
                   void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The decoder's feed-forward block around the MoE (model.ts page,
 * DiffDecoderLayer.forwardWith, after the attention residual):
 *
 *   h1  = postFfNorm1(mlp(preFfNorm(h)))           dense GeGLU branch
 *   h2  = postFfNorm2(experts(preFfNorm2(h)))      the MoE layer above; the
 *                                                  router (moe_route) takes
 *                                                  the raw h
 *   out = (h + postFfNorm(h1 + h2)) * layer_scalar
 *
 * mlp(x) = down(gelu_approx(gate . x) * (up . x)) with three 4-bit linears.
 * Every norm is a plain RMSNorm, x / sqrt(mean(x^2) + eps) * w, the stored
 * weight used as is (model.ts page, header note on the checkpoint: no 1 + w
 * offset).  One block is
 *   ff_prenorm -> qlinear_geglu -> qlinear (down)      dense branch
 *   moe_route(h) -> moe_sort -> qswitch_gate_up_geglu -> qswitch_down_combine
 *   ff_combine
 * with bf16 tensors between the calls and fp32 arithmetic inside each.
 * ---------------------------------------------------------------------- */

/* ff_prenorm -- both pre-norms of the block from one read of h:
 *   x_dense = rms(h) * w_dense   (preFfNorm),  x_moe = rms(h) * w_moe
 *   (preFfNorm2),  rms(h) = 1 / sqrt(mean over H of h^2 + eps)
 *
 *   h                bf16 [T, H]; H % 8 == 0
 *   w_dense, w_moe   bf16 [H]
 *   x_dense, x_moe   bf16 [T, H] (out); must not overlap h
 * Every pointer here is 16-byte aligned.  eps >= 0 (an all-zero row with
 * eps = 0 gives NaN, as the formula does). */
int ff_prenorm(const uint16_t* h, int32_t T, int32_t H, const uint16_t* w_dense,
               const uint16_t* w_moe, float eps, uint16_t* x_dense, uint16_t* x_moe,
               hipStream_t stream);

/* qlinear_geglu -- the first half of the dense branch: gate and up
 * QuantizedLinears in one pass over the fused weight [gate; up] and the GeGLU
 * (model.ts page, DiffDecoderLayer's mlp; gelu_approx(gate) * up as in the
 * vision.ts page, DiffVisionMLP):
 *   y[m, i] = gelu_tanh(g) * u,  g = x[m] . dequant(gate)[i],
 *                                u = x[m] . dequant(up)[i]   (fp32 accumulate)
 *
 *   x        bf16 [M, K]
 *   W        experts = 1, rows = 2N, in = K (rows 0..N-1 gate, N..2N-1 up);
 *            K % 64 == 0, N % 16 == 0; layout QMOE_LAYOUT_TILED with split = N
 *   y (out)  bf16 [M, N]
 * The down projection is qlinear on y. */
int qlinear_geglu(const uint16_t* x, int32_t M, const qmoe_qweight* W, uint16_t* y,
                  hipStream_t stream);

/* ff_combine -- the post-norms, the residual add and the layer scalar:
 *   s   = rms(dense_out) * w_post1 + rms(moe_out) * w_post2
 *   out = (h + rms(s) * w_post) * layer_scalar
 *
 *   h                 bf16 [T, H] residual (the block's input); H % 8 == 0
 *   dense_out         bf16 [T, H] the dense branch before postFfNorm1
 *   moe_out           bf16 [T, H] the experts' output before postFfNorm2
 *   w_post1, w_post2, w_post   bf16 [H]
 *   out (out)         bf16 [T, H]; must not overlap the inputs
 * Every pointer here is 16-byte aligned; eps as in ff_prenorm. */
int ff_combine(const uint16_t* h, const uint16_t* dense_out, const uint16_t* moe_out, int32_t T,
               int32_t H, const uint16_t* w_post1, const uint16_t* w_post2,
               const uint16_t* w_post, float eps, float layer_scalar, uint16_t* out,
               hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */

// C ABI of the 4-bit MoE layer: host-side validation, workspace sizing and
// kernel launches.  Every argument is checked before anything is enqueued,
// so a call that returns an error has done nothing on the device.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/qmoe.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return QMOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p, align, name)                                                  \
  do {                                                                                \
    if ((p) == nullptr) return fail(QMOE_ERR_INVALID, "%s: null pointer", name);     \
    if (!aligned((p), (align)))                                                       \
      return fail(QMOE_ERR_INVALID, "%s: not %d-byte aligned", name, (int)(align));   \
  } while (0)

// Checks a quantized weight descriptor against the expected shape and layout
// (for the tiled layout also the fused-pair split it was tiled with).
int check_qweight(const qmoe_qweight* q, const char* what, int experts, int rows, int in, int layout = QMOE_LAYOUT_ROWS,
                  int split = 0) {
  REQUIRE(q != nullptr, QMOE_ERR_INVALID, "%s: null weight descriptor", what);
  REQUIRE(q->bits == 4, QMOE_ERR_UNSUPPORTED, "%s: bits=%d, only 4-bit weights are supported", what, q->bits);
  REQUIRE(q->group == 64, QMOE_ERR_UNSUPPORTED, "%s: group=%d, only group size 64 is supported", what, q->group);
  REQUIRE(q->experts == experts, QMOE_ERR_INVALID, "%s: experts=%d, expected %d", what, q->experts, experts);
  REQUIRE(q->rows == rows, QMOE_ERR_INVALID, "%s: rows=%d, expected %d", what, q->rows, rows);
  REQUIRE(q->in == in, QMOE_ERR_INVALID, "%s: in=%d, expected %d", what, q->in, in);
  REQUIRE(q->layout == layout, QMOE_ERR_INVALID, "%s: layout=%d, expected %d (%s)", what, q->layout, layout,
          layout == QMOE_LAYOUT_TILED ? "tile it with qmoe_tile_weight" : "row-major codes");
  if (layout == QMOE_LAYOUT_TILED) {
    REQUIRE(q->split == split, QMOE_ERR_INVALID, "%s: tiled with split=%d, expected %d", what, q->split, split);
    REQUIRE_PTR(q->w, 16, "tiled weight");
    return QMOE_OK;
  }
  if (layout == QMOE_LAYOUT_TILED_T) {
    REQUIRE_PTR(q->w, 16, "tiled table");
    return QMOE_OK;
  }
  REQUIRE_PTR(q->w, 16, "weight codes");
  REQUIRE_PTR(q->scales, 2, "weight scales");
  REQUIRE_PTR(q->biases, 2, "weight biases");
  return QMOE_OK;
}

// Number of compute units of the current device, cached per device.
int num_cu_current(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QMOE_ERR_HIP, "hipGetDevice failed");
  if (dev >= 0 && dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *out = v;
      return QMOE_OK;
    }
  }
  int n = 0;
  hipError_t err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess || n <= 0) return fail(QMOE_ERR_HIP, "querying the CU count failed: %s", hipGetErrorString(err));
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return QMOE_OK;
}

int launched(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(QMOE_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(err));
  return ok();
}

constexpr long long kMaxAssign = 1LL << 24;
constexpr long long kMaxUnsortedAssign = 4096;  // the unsorted path is sized for small batches

// Workspace of the unsorted pair: the partial sums of the larger of the two
// passes (fp32), written by the first kernel of a call and read by its second.
size_t unsorted_bytes(long long T, int k, int H, int I) {
  const long long A = T * k;
  const qmoe::UnsortedPlan gu = qmoe::unsorted_plan(A, qmoe::tiled_blocks(2 * I, I), H / 64);
  const qmoe::UnsortedPlan dn = qmoe::unsorted_plan(A, qmoe::tiled_blocks(H, 0), I / 64);
  return (size_t)std::max(gu.partials, dn.partials) * sizeof(float);
}

// the weight-stationary kernel where the weight blocks meet many rows
bool use_ws(int mode, long long rows, int experts) { return qmoe::ws_preferred(mode, rows, experts); }

int status_ptr(int** out) {
  int* s = qmoe::device_status();
  if (s == nullptr) return fail(QMOE_ERR_HIP, "the device status word is not available");
  *out = s;
  return QMOE_OK;
}

}  // namespace

extern "C" {

const char* qmoe_last_error(void) { return g_last_error.c_str(); }

int qmoe_device_status(int32_t* value, int32_t reset) {
  REQUIRE(value != nullptr, QMOE_ERR_INVALID, "qmoe_device_status: null value pointer");
  int* s = nullptr;
  if (int rc = status_ptr(&s)) return rc;
  hipError_t err = hipDeviceSynchronize();
  if (err == hipSuccess) err = hipMemcpy(value, s, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (err == hipSuccess && reset) {
    const int32_t zero = 0;
    err = hipMemcpy(s, &zero, sizeof(int32_t), hipMemcpyHostToDevice);
  }
  if (err != hipSuccess) return fail(QMOE_ERR_HIP, "qmoe_device_status: %s", hipGetErrorString(err));
  return ok();
}

size_t moe_route_workspace(int32_t T, int32_t H, int32_t E) {
  if (T <= 0 || H <= 0 || E <= 0 || H % 64 != 0) return 0;
  // per k-range: partial logits [T, E] and partial sums of squares [T]
  return (size_t)qmoe::route_ksplit(T, H) * (size_t)T * (size_t)(E + 1) * sizeof(float);
}

int moe_route(const uint16_t* x_router, int32_t T, int32_t H, const uint16_t* norm_scale, float eps,
              const qmoe_qweight* proj, const uint16_t* per_expert_scale, const float* logit_bias, int32_t k,
              int32_t* indices, float* weights, float* logits_out, void* workspace, size_t ws_bytes,
              hipStream_t stream) {
  REQUIRE(T >= 0, QMOE_ERR_INVALID, "moe_route: T=%d < 0", T);
  REQUIRE(H > 0 && H % 64 == 0, QMOE_ERR_INVALID, "moe_route: H=%d must be a positive multiple of 64", H);
  REQUIRE(proj != nullptr, QMOE_ERR_INVALID, "moe_route: null router weight descriptor");
  const int E = proj->rows;
  REQUIRE(E >= 1 && E <= 256, QMOE_ERR_UNSUPPORTED, "moe_route: E=%d outside [1, 256]", E);
  REQUIRE(k >= 1 && k <= E && k <= 16, QMOE_ERR_UNSUPPORTED, "moe_route: k=%d outside [1, min(E, 16)]", k);
  REQUIRE((long long)T * k <= kMaxAssign, QMOE_ERR_UNSUPPORTED, "moe_route: T*k above 2^24");
  REQUIRE(std::isfinite(eps) && eps >= 0.f, QMOE_ERR_INVALID, "moe_route: eps must be finite and >= 0");
  if (T == 0) return ok();
  if (int rc = check_qweight(proj, "moe_route proj", 1, E, H)) return rc;
  REQUIRE_PTR(x_router, 16, "moe_route x_router");
  REQUIRE_PTR(norm_scale, 16, "moe_route norm_scale");
  REQUIRE_PTR(per_expert_scale, 2, "moe_route per_expert_scale");
  if (logit_bias) REQUIRE_PTR(logit_bias, 4, "moe_route logit_bias");
  REQUIRE_PTR(indices, 4, "moe_route indices");
  REQUIRE_PTR(weights, 4, "moe_route weights");
  if (logits_out) REQUIRE_PTR(logits_out, 4, "moe_route logits_out");
  const size_t need = moe_route_workspace(T, H, E);
  REQUIRE(workspace != nullptr && ws_bytes >= need, QMOE_ERR_WORKSPACE,
          "moe_route: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  REQUIRE(aligned(workspace, 4), QMOE_ERR_INVALID, "moe_route: workspace not 4-byte aligned");

  qmoe::RouteArgs a{};
  a.x = x_router;
  a.norm_scale = norm_scale;
  a.w = proj->w;
  a.s = proj->scales;
  a.b = proj->biases;
  a.pes = per_expert_scale;
  a.logit_bias = logit_bias;
  a.part = static_cast<float*>(workspace);
  a.indices = indices;
  a.weights = weights;
  a.logits_out = logits_out;
  a.eps = eps;
  a.root = (float)std::pow((double)H, -0.5);
  a.T = T;
  a.H = H;
  a.E = E;
  a.k = k;
  a.ksplit = qmoe::route_ksplit(T, H);
  return launched(qmoe::launch_route(a, stream), "moe_route");
}

size_t moe_sort_workspace(int32_t T, int32_t k, int32_t E) {
  if (T <= 0 || k <= 0 || E < 1 || E > 256 || (long long)T * k > kMaxAssign) return 0;
  return qmoe::sort_workspace_bytes(T * k, E);
}

int moe_sort(const int32_t* indices, int32_t T, int32_t k, int32_t E, int32_t* expert_offsets,
             int32_t* sorted_assign, void* workspace, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(T >= 0, QMOE_ERR_INVALID, "moe_sort: T=%d < 0", T);
  REQUIRE(k >= 1, QMOE_ERR_INVALID, "moe_sort: k=%d < 1", k);
  REQUIRE(E >= 1 && E <= 256, QMOE_ERR_UNSUPPORTED, "moe_sort: E=%d outside [1, 256]", E);
  REQUIRE((long long)T * k <= kMaxAssign, QMOE_ERR_UNSUPPORTED, "moe_sort: T*k above 2^24");
  if (T == 0) return ok();
  REQUIRE_PTR(indices, 4, "moe_sort indices");
  REQUIRE_PTR(expert_offsets, 4, "moe_sort expert_offsets");
  REQUIRE_PTR(sorted_assign, 4, "moe_sort sorted_assign");
  if (workspace != nullptr) REQUIRE_PTR(workspace, 4, "moe_sort workspace");
  return launched(qmoe::launch_sort(indices, T * k, E, expert_offsets, sorted_assign, workspace, ws_bytes, stream),
                  "moe_sort");
}

size_t qswitch_mid_bytes(int32_t T, int32_t k, int32_t I, int32_t E) {
  if (T <= 0 || k <= 0 || I <= 0 || I % 64 != 0 || E <= 0) return 0;
  return (size_t)qmoe::act_tiles_max((long long)T * k, E) * (size_t)(I / 64) * qmoe::kActBlock;
}

int qswitch_gate_up_geglu(const uint16_t* x_expert, int32_t T, int32_t H, const qmoe_qweight* gate_up, int32_t I,
                          int32_t k, const int32_t* expert_offsets, const int32_t* sorted_assign, void* mid,
                          size_t mid_bytes, hipStream_t stream) {
  REQUIRE(T >= 0, QMOE_ERR_INVALID, "qswitch_gate_up_geglu: T=%d < 0", T);
  REQUIRE(H > 0 && H % 64 == 0, QMOE_ERR_INVALID, "qswitch_gate_up_geglu: H=%d must be a positive multiple of 64", H);
  REQUIRE(I > 0 && I % 64 == 0, QMOE_ERR_INVALID, "qswitch_gate_up_geglu: I=%d must be a positive multiple of 64", I);
  REQUIRE(k >= 1 && k <= 16, QMOE_ERR_UNSUPPORTED, "qswitch_gate_up_geglu: k=%d outside [1, 16]", k);
  REQUIRE((long long)T * k <= kMaxAssign, QMOE_ERR_UNSUPPORTED, "qswitch_gate_up_geglu: T*k above 2^24");
  REQUIRE(gate_up != nullptr, QMOE_ERR_INVALID, "qswitch_gate_up_geglu: null weight descriptor");
  const int E = gate_up->experts;
  REQUIRE(E >= 1 && E <= 256, QMOE_ERR_UNSUPPORTED, "qswitch_gate_up_geglu: E=%d outside [1, 256]", E);
  if (T == 0) return ok();
  if (int rc = check_qweight(gate_up, "qswitch_gate_up_geglu gate_up", E, 2 * I, H, QMOE_LAYOUT_TILED, I)) return rc;
  REQUIRE_PTR(x_expert, 16, "qswitch_gate_up_geglu x_expert");
  REQUIRE_PTR(expert_offsets, 4, "qswitch_gate_up_geglu expert_offsets");
  REQUIRE_PTR(sorted_assign, 4, "qswitch_gate_up_geglu sorted_assign");
  REQUIRE_PTR(mid, 16, "qswitch_gate_up_geglu mid");
  const size_t need_mid = qswitch_mid_bytes(T, k, I, E);
  REQUIRE((long long)T * H * 2 < (1LL << 32), QMOE_ERR_UNSUPPORTED,
          "qswitch_gate_up_geglu: activation bytes reach 2^32");
  REQUIRE(need_mid < (1ULL << 32), QMOE_ERR_UNSUPPORTED, "qswitch_gate_up_geglu: mid tiles reach 2^32 bytes");
  REQUIRE(mid_bytes >= need_mid, QMOE_ERR_INVALID, "qswitch_gate_up_geglu: mid of %zu bytes needed, %zu given",
          need_mid, mid_bytes);
  int ncu = 0;
  if (int rc = num_cu_current(&ncu)) return rc;
  qmoe::SwitchArgs a{};
  a.a = x_expert;
  a.max_tiles = (int)qmoe::act_tiles_max((long long)T * k, E);
  a.w = gate_up->w;
  a.nblk = qmoe::tiled_blocks(2 * I, I);
  a.offsets = expert_offsets;
  a.assign = sorted_assign;
  a.out = mid;
  a.K = H;
  a.Nout = I;
  a.E = E;
  a.ktop = k;
  a.rows_total = T * k;
  if (qmoe::tall_preferred(qmoe::MODE_GATE_UP, a.rows_total, E))
    return launched(qmoe::launch_tall<qmoe::MODE_GATE_UP>(a, ncu, stream), "qswitch_gate_up_geglu");
  return launched(qmoe::launch_gate_up_geglu(a, ncu, stream), "qswitch_gate_up_geglu");
}

size_t qswitch_down_combine_workspace(int32_t T, int32_t k, int32_t H, int32_t deterministic) {
  (void)deterministic;
  if (T <= 0 || k <= 0 || H <= 0) return 0;
  return (size_t)T * (size_t)k * (size_t)H * sizeof(uint16_t);  // the down rows, bf16
}

int qswitch_down_combine(const void* mid, int32_t T, int32_t k, int32_t I, const qmoe_qweight* down, int32_t H,
                         const int32_t* expert_offsets, const int32_t* sorted_assign, const float* weights,
                         uint16_t* y, void* workspace, size_t ws_bytes, int32_t deterministic, hipStream_t stream) {
  REQUIRE(T >= 0, QMOE_ERR_INVALID, "qswitch_down_combine: T=%d < 0", T);
  REQUIRE(H > 0 && H % 64 == 0, QMOE_ERR_INVALID, "qswitch_down_combine: H=%d must be a positive multiple of 64", H);
  REQUIRE(I > 0 && I % 64 == 0, QMOE_ERR_INVALID, "qswitch_down_combine: I=%d must be a positive multiple of 64", I);
  REQUIRE(k >= 1 && k <= 16, QMOE_ERR_UNSUPPORTED, "qswitch_down_combine: k=%d outside [1, 16]", k);
  REQUIRE((long long)T * k <= kMaxAssign, QMOE_ERR_UNSUPPORTED, "qswitch_down_combine: T*k above 2^24");
  REQUIRE(down != nullptr, QMOE_ERR_INVALID, "qswitch_down_combine: null weight descriptor");
  const int E = down->experts;
  REQUIRE(E >= 1 && E <= 256, QMOE_ERR_UNSUPPORTED, "qswitch_down_combine: E=%d outside [1, 256]", E);
  if (T == 0) return ok();
  if (int rc = check_qweight(down, "qswitch_down_combine down", E, H, I, QMOE_LAYOUT_TILED, 0)) return rc;
  REQUIRE_PTR(mid, 16, "qswitch_down_combine mid");
  REQUIRE_PTR(expert_offsets, 4, "qswitch_down_combine expert_offsets");
  REQUIRE_PTR(sorted_assign, 4, "qswitch_down_combine sorted_assign");
  REQUIRE_PTR(weights, 4, "qswitch_down_combine weights");
  REQUIRE_PTR(y, 16, "qswitch_down_combine y");
  REQUIRE(qswitch_mid_bytes(T, k, I, E) < (1ULL << 32), QMOE_ERR_UNSUPPORTED,
          "qswitch_down_combine: mid tiles reach 2^32 bytes");
  const size_t need = qswitch_down_combine_workspace(T, k, H, deterministic);
  REQUIRE(workspace != nullptr && ws_bytes >= need, QMOE_ERR_WORKSPACE,
          "qswitch_down_combine: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  REQUIRE(aligned(workspace, 16), QMOE_ERR_INVALID, "qswitch_down_combine: workspace not 16-byte aligned");
  int ncu = 0;
  if (int rc = num_cu_current(&ncu)) return rc;
  qmoe::SwitchArgs a{};
  a.a = static_cast<const uint16_t*>(mid);
  a.max_tiles = (int)qmoe::act_tiles_max((long long)T * k, E);
  a.w = down->w;
  a.nblk = qmoe::tiled_blocks(H, 0);
  a.offsets = expert_offsets;
  a.assign = sorted_assign;
  a.out = workspace;
  a.K = I;
  a.Nout = H;
  a.E = E;
  a.ktop = k;
  a.rows_total = T * k;
  hipError_t err = qmoe::launch_down(a, ncu, stream);
  if (err != hipSuccess) return launched(err, "qswitch_down_combine (down)");
  return launched(qmoe::launch_combine(static_cast<const uint16_t*>(workspace), weights, T, k, H, y, stream),
                  "qswitch_down_combine (combine)");
}

int qswitch_down_combine_noalloc(const void* mid, int32_t T, int32_t k, int32_t I, const qmoe_qweight* down,
                                 int32_t H, const int32_t* expert_offsets, const int32_t* sorted_assign,
                                 const float* weights, uint16_t* y, int32_t deterministic, hipStream_t stream) {
  if (T <= 0 || k <= 0 || H <= 0)  // nothing to do, or rejected by the validation below
    return qswitch_down_combine(mid, T, k, I, down, H, expert_offsets, sorted_assign, weights, y, nullptr, 0,
                                deterministic, stream);
  const size_t need = qswitch_down_combine_workspace(T, k, H, deterministic);
  REQUIRE(need <= qmoe::kNoAllocScratchBytes, QMOE_ERR_UNSUPPORTED,
          "qswitch_down_combine_noalloc: T*k*H = %lld needs %zu bytes of scratch, above the %zu the library "
          "holds (use qswitch_down_combine with a workspace)",
          (long long)T * k * H, need, qmoe::kNoAllocScratchBytes);
  void* s = qmoe::noalloc_scratch();
  REQUIRE(s != nullptr, QMOE_ERR_HIP, "qswitch_down_combine_noalloc: the library's scratch is not available");
  // every byte of scratch the down pass hands to the combine is written first
  // in this call (dropped rows as zeros), so nothing is cleared
  return qswitch_down_combine(mid, T, k, I, down, H, expert_offsets, sorted_assign, weights, y, s,
                              qmoe::kNoAllocScratchBytes, deterministic, stream);
}

size_t qmoe_tiled_weight_bytes(int32_t experts, int32_t rows, int32_t in, int32_t split) {
  if (experts <= 0 || rows <= 0 || in <= 0 || in % 64 != 0 || split < 0) return 0;
  if (split > 0 && (split % 16 != 0 || rows != 2 * split)) return 0;
  return (size_t)experts * (size_t)qmoe::tiled_blocks(rows, split) * (size_t)(in / 64) * (size_t)qmoe::kTiledUnit;
}

int qmoe_tile_weight(const qmoe_qweight* src, int32_t split, void* dst, size_t dst_bytes, hipStream_t stream) {
  REQUIRE(src != nullptr, QMOE_ERR_INVALID, "qmoe_tile_weight: null weight descriptor");
  REQUIRE(src->experts >= 1 && src->rows >= 1, QMOE_ERR_INVALID, "qmoe_tile_weight: experts=%d rows=%d",
          src->experts, src->rows);
  REQUIRE(src->in > 0 && src->in % 64 == 0, QMOE_ERR_INVALID, "qmoe_tile_weight: in=%d must be a positive multiple of 64",
          src->in);
  REQUIRE(split >= 0, QMOE_ERR_INVALID, "qmoe_tile_weight: split=%d < 0", split);
  REQUIRE(split == 0 || (split % 16 == 0 && src->rows == 2 * split), QMOE_ERR_INVALID,
          "qmoe_tile_weight: split=%d needs rows == 2*split and split %% 16 == 0 (rows=%d)", split, src->rows);
  if (int rc = check_qweight(src, "qmoe_tile_weight src", src->experts, src->rows, src->in)) return rc;
  REQUIRE((long long)src->experts * src->rows * (src->in / 8) < (1LL << 31), QMOE_ERR_UNSUPPORTED,
          "qmoe_tile_weight: more than 2^31 code words");
  const size_t need = qmoe_tiled_weight_bytes(src->experts, src->rows, src->in, split);
  REQUIRE_PTR(dst, 16, "qmoe_tile_weight dst");
  REQUIRE(dst_bytes >= need, QMOE_ERR_INVALID, "qmoe_tile_weight: %zu bytes needed, %zu given", need, dst_bytes);
  return launched(qmoe::launch_tile_weight(src->w, src->scales, src->biases, src->experts, src->rows, src->in, split,
                                           static_cast<uint8_t*>(dst), stream),
                  "qmoe_tile_weight");
}

int qlinear(const uint16_t* x, int32_t M, const qmoe_qweight* W, uint16_t* y, hipStream_t stream) {
  REQUIRE(M >= 0, QMOE_ERR_INVALID, "qlinear: M=%d < 0", M);
  REQUIRE(W != nullptr, QMOE_ERR_INVALID, "qlinear: null weight descriptor");
  const int N = W->rows, K = W->in;
  REQUIRE(K > 0 && K % 64 == 0, QMOE_ERR_INVALID, "qlinear: K=%d must be a positive multiple of 64", K);
  REQUIRE(N > 0 && N % 16 == 0, QMOE_ERR_INVALID, "qlinear: N=%d must be a positive multiple of 16", N);
  if (M == 0) return ok();
  if (int rc = check_qweight(W, "qlinear W", 1, N, K, QMOE_LAYOUT_TILED, 0)) return rc;
  REQUIRE_PTR(x, 16, "qlinear x");
  REQUIRE_PTR(y, 16, "qlinear y");
  REQUIRE((long long)M * K * 2 < (1LL << 32), QMOE_ERR_UNSUPPORTED, "qlinear: activation bytes reach 2^32");
  int ncu = 0;
  if (int rc = num_cu_current(&ncu)) return rc;
  qmoe::SwitchArgs a{};
  a.a = x;
  a.w = W->w;
  a.nblk = qmoe::tiled_blocks(N, 0);
  a.out = y;
  a.K = K;
  a.Nout = N;
  a.E = 1;
  a.ktop = 1;
  a.rows_total = M;
  if (qmoe::tall_preferred(qmoe::MODE_DENSE, M, 1))
    return launched(qmoe::launch_tall<qmoe::MODE_DENSE>(a, ncu, stream), "qlinear");
  return launched(qmoe::launch_dense(a, ncu, stream), "qlinear");
}

int qlinear_softcap(const uint16_t* x, int32_t M, const qmoe_qweight* W, float cap, float* y, hipStream_t stream) {
  REQUIRE(M >= 0, QMOE_ERR_INVALID, "qlinear_softcap: M=%d < 0", M);
  REQUIRE(W != nullptr, QMOE_ERR_INVALID, "qlinear_softcap: null weight descriptor");
  REQUIRE(std::isfinite(cap) && cap > 0.f, QMOE_ERR_INVALID, "qlinear_softcap: cap must be finite and > 0");
  const int N = W->rows, K = W->in;
  REQUIRE(K > 0 && K % 64 == 0, QMOE_ERR_INVALID, "qlinear_softcap: K=%d must be a positive multiple of 64", K);
  REQUIRE(N > 0 && N % 16 == 0, QMOE_ERR_INVALID, "qlinear_softcap: N=%d must be a positive multiple of 16", N);
  if (int rc = check_qweight(W, "qlinear_softcap W", 1, N, K, QMOE_LAYOUT_TILED, 0)) return rc;
  if (M == 0) return ok();
  REQUIRE_PTR(x, 16, "qlinear_softcap x");
  REQUIRE_PTR(y, 16, "qlinear_softcap y");
  REQUIRE((long long)M * K * 2 < (1LL << 32), QMOE_ERR_UNSUPPORTED, "qlinear_softcap: activation bytes reach 2^32");
  int ncu = 0;
  if (int rc = num_cu_current(&ncu)) return rc;
  qmoe::SwitchArgs a{};
  a.a = x;
  a.w = W->w;
  a.nblk = qmoe::tiled_blocks(N, 0);
  a.out = y;
  a.K = K;
  a.Nout = N;
  a.E = 1;
  a.ktop = 1;
  a.rows_total = M;
  a.cap = cap;
  if (use_ws(qmoe::MODE_DENSE_SOFTCAP, M, 1))
    return launched(qmoe::launch_ws<qmoe::MODE_DENSE_SOFTCAP>(a, ncu, stream), "qlinear_softcap");
  return launched(qmoe::launch_dense_softcap(a, ncu, stream), "qlinear_softcap");
}

int qlinear_geglu(const uint16_t* x, int32_t M, const qmoe_qweight* W, uint16_t* y, hipStream_t stream) {
  REQUIRE(M >= 0, QMOE_ERR_INVALID, "qlinear_geglu: M=%d < 0", M);
  REQUIRE(W != nullptr, QMOE_ERR_INVALID, "qlinear_geglu: null weight descriptor");
  const int K = W->in, N = W->split;
  REQUIRE(K > 0 && K % 64 == 0, QMOE_ERR_INVALID, "qlinear_geglu: K=%d must be a positive multiple of 64", K);
  REQUIRE(N > 0 && N % 16 == 0, QMOE_ERR_INVALID, "qlinear_geglu: split=%d must be a positive multiple of 16", N);
  if (int rc = check_qweight(W, "qlinear_geglu W", 1, 2 * N, K, QMOE_LAYOUT_TILED, N)) return rc;
  if (M == 0) return ok();
  REQUIRE_PTR(x, 16, "qlinear_geglu x");
  REQUIRE_PTR(y, 16, "qlinear_geglu y");
  REQUIRE((long long)M * K * 2 < (1LL << 32), QMOE_ERR_UNSUPPORTED, "qlinear_geglu: activation bytes reach 2^32");
  int ncu = 0;
  if (int rc = num_cu_current(&ncu)) return rc;
  qmoe::SwitchArgs a{};
  a.a = x;
  a.w = W->w;
  a.nblk = qmoe::tiled_blocks(2 * N, N);
  a.out = y;
  a.K = K;
  a.Nout = N;
  a.E = 1;
  a.ktop = 1;
  a.rows_total = M;
  if (qmoe::tall_preferred(qmoe::MODE_DENSE_GEGLU, M, 1))
    return launched(qmoe::launch_tall<qmoe::MODE_DENSE_GEGLU>(a, ncu, stream), "qlinear_geglu");
  return launched(qmoe::launch_dense_geglu(a, ncu, stream), "qlinear_geglu");
}

int ff_prenorm(const uint16_t* h, int32_t T, int32_t H, const uint16_t* w_dense, const uint16_t* w_moe, float eps,
               uint16_t* x_dense, uint16_t* x_moe, hipStream_t stream) {
  REQUIRE(T >= 0, QMOE_ERR_INVALID, "ff_prenorm: T=%d < 0", T);
  REQUIRE(H > 0 && H % 8 == 0, QMOE_ERR_INVALID, "ff_prenorm: H=%d must be a positive multiple of 8", H);
  REQUIRE(std::isfinite(eps) && eps >= 0.f, QMOE_ERR_INVALID, "ff_prenorm: eps must be finite and >= 0");
  if (T == 0) return ok();
  REQUIRE_PTR(h, 16, "ff_prenorm h");
  REQUIRE_PTR(w_dense, 16, "ff_prenorm w_dense");
  REQUIRE_PTR(w_moe, 16, "ff_prenorm w_moe");
  REQUIRE_PTR(x_dense, 16, "ff_prenorm x_dense");
  REQUIRE_PTR(x_moe, 16, "ff_prenorm x_moe");
  REQUIRE(T <= (1 << 30) / 4, QMOE_ERR_UNSUPPORTED, "ff_prenorm: T=%d too large", T);
  return launched(qmoe::launch_ff_prenorm(h, T, H, w_dense, w_moe, eps, x_dense, x_moe, stream), "ff_prenorm");
}

int ff_combine(const uint16_t* h, const uint16_t* dense_out, const uint16_t* moe_out, int32_t T, int32_t H,
               const uint16_t* w_post1, const uint16_t* w_post2, const uint16_t* w_post, float eps,
               float layer_scalar, uint16_t* out, hipStream_t stream) {
  REQUIRE(T >= 0, QMOE_ERR_INVALID, "ff_combine: T=%d < 0", T);
  REQUIRE(H > 0 && H % 8 == 0, QMOE_ERR_INVALID, "ff_combine: H=%d must be a positive multiple of 8", H);
  REQUIRE(std::isfinite(eps) && eps >= 0.f, QMOE_ERR_INVALID, "ff_combine: eps must be finite and >= 0");
  if (T == 0) return ok();
  REQUIRE_PTR(h, 16, "ff_combine h");
  REQUIRE_PTR(dense_out, 16, "ff_combine dense_out");
  REQUIRE_PTR(moe_out, 16, "ff_combine moe_out");
  REQUIRE_PTR(w_post1, 16, "ff_combine w_post1");
  REQUIRE_PTR(w_post2, 16, "ff_combine w_post2");
  REQUIRE_PTR(w_post, 16, "ff_combine w_post");
  REQUIRE_PTR(out, 16, "ff_combine out");
  REQUIRE(T <= (1 << 30) / 4, QMOE_ERR_UNSUPPORTED, "ff_combine: T=%d too large", T);
  return launched(qmoe::launch_ff_combine(h, dense_out, moe_out, T, H, w_post1, w_post2, w_post, eps, layer_scalar,
                                          out, stream),
                  "ff_combine");
}

}  // extern "C"

extern "C" {

size_t qswitch_unsorted_workspace(int32_t T, int32_t k, int32_t H, int32_t I) {
  if (T <= 0 || k <= 0 || H <= 0 || I <= 0 || H % 64 != 0 || I % 64 != 0) return 0;
  if ((long long)T * k > kMaxUnsortedAssign) return 0;
  return unsorted_bytes(T, k, H, I);
}

}  // extern "C"

namespace {
// Shared validation of the two unsorted calls; fills the common arguments.
int unsorted_common(const char* fn, int32_t T, int32_t k, int32_t H, int32_t I, const qmoe_qweight* W, int rows,
                    int in, int split, const int32_t* indices, void* workspace, size_t ws_bytes,
                    qmoe::UnsortedArgs* a) {
  REQUIRE(T >= 0, QMOE_ERR_INVALID, "%s: T=%d < 0", fn, T);
  REQUIRE(H > 0 && H % 64 == 0, QMOE_ERR_INVALID, "%s: H=%d must be a positive multiple of 64", fn, H);
  REQUIRE(I > 0 && I % 64 == 0, QMOE_ERR_INVALID, "%s: I=%d must be a positive multiple of 64", fn, I);
  REQUIRE(k >= 1 && k <= 16, QMOE_ERR_UNSUPPORTED, "%s: k=%d outside [1, 16]", fn, k);
  REQUIRE((long long)T * k <= kMaxUnsortedAssign, QMOE_ERR_UNSUPPORTED,
          "%s: T*k=%lld above %lld (use the sorted calls)", fn, (long long)T * k, kMaxUnsortedAssign);
  REQUIRE(W != nullptr, QMOE_ERR_INVALID, "%s: null weight descriptor", fn);
  const int E = W->experts;
  REQUIRE(E >= 1 && E <= 256, QMOE_ERR_UNSUPPORTED, "%s: E=%d outside [1, 256]", fn, E);
  if (T == 0) return QMOE_OK;
  char what[96];
  snprintf(what, sizeof(what), "%s weight", fn);
  if (int rc = check_qweight(W, what, E, rows, in, QMOE_LAYOUT_TILED, split)) return rc;
  REQUIRE_PTR(indices, 4, "indices");
  REQUIRE_PTR(workspace, 16, "workspace");
  const size_t need = unsorted_bytes(T, k, H, I);
  REQUIRE(ws_bytes >= need, QMOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  a->w = W->w;
  a->indices = indices;
  a->part = (float*)workspace;
  a->A = T * k;
  a->k = k;
  a->E = E;
  a->K = in;
  a->G = in / 64;
  a->nblk = qmoe::tiled_blocks(rows, split);
  const qmoe::UnsortedPlan pl = qmoe::unsorted_plan(a->A, a->nblk, a->G);
  a->S = pl.S;
  a->gpw = pl.gpw;
  return QMOE_OK;
}
}  // namespace

extern "C" {

int qswitch_gate_up_geglu_unsorted(const uint16_t* x_expert, int32_t T, int32_t H, const qmoe_qweight* gate_up,
                                   int32_t I, int32_t k, const int32_t* indices, uint16_t* mid_rows,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "qswitch_gate_up_geglu_unsorted";
  qmoe::UnsortedArgs a{};
  if (int rc = unsorted_common(fn, T, k, H, I, gate_up, 2 * I, H, I, indices, workspace, ws_bytes, &a)) return rc;
  if (T == 0) return ok();
  REQUIRE_PTR(x_expert, 16, "x_expert");
  REQUIRE_PTR(mid_rows, 16, "mid_rows");
  a.x = x_expert;
  a.out = mid_rows;
  a.Nout = I;
  return launched(qmoe::launch_unsorted(qmoe::UNSORTED_GATE_UP, a, stream), fn);
}

int qswitch_down_combine_unsorted(const uint16_t* mid_rows, int32_t T, int32_t k, int32_t I,
                                  const qmoe_qweight* down, int32_t H, const int32_t* indices,
                                  const float* weights, uint16_t* y, void* workspace, size_t ws_bytes,
                                  hipStream_t stream) {
  const char* fn = "qswitch_down_combine_unsorted";
  qmoe::UnsortedArgs a{};
  if (int rc = unsorted_common(fn, T, k, H, I, down, H, I, 0, indices, workspace, ws_bytes, &a)) return rc;
  if (T == 0) return ok();
  REQUIRE_PTR(mid_rows, 16, "mid_rows");
  REQUIRE_PTR(weights, 4, "weights");
  REQUIRE_PTR(y, 16, "y");
  a.x = mid_rows;
  a.weights = weights;
  a.out = y;
  a.Nout = H;
  return launched(qmoe::launch_unsorted(qmoe::UNSORTED_DOWN, a, stream), fn);
}

}  // extern "C"

extern "C" {

size_t qmoe_tiled_weight_t_bytes(int32_t V, int32_t H) {
  if (V <= 0 || H <= 0 || V % 32 != 0 || H % 64 != 0) return 0;
  return (size_t)(H / 64) * (size_t)(V / 32) * 1152;
}

int qmoe_tile_weight_t(const qmoe_qweight* src, void* dst, size_t dst_bytes, hipStream_t stream) {
  REQUIRE(src != nullptr, QMOE_ERR_INVALID, "qmoe_tile_weight_t: null weight descriptor");
  const int V = src->rows, H = src->in;
  REQUIRE(V > 0 && V % 32 == 0, QMOE_ERR_INVALID, "qmoe_tile_weight_t: rows=%d must be a positive multiple of 32", V);
  REQUIRE(H > 0 && H % 64 == 0, QMOE_ERR_INVALID, "qmoe_tile_weight_t: in=%d must be a positive multiple of 64", H);
  if (int rc = check_qweight(src, "qmoe_tile_weight_t src", 1, V, H, QMOE_LAYOUT_ROWS)) return rc;
  REQUIRE_PTR(dst, 16, "qmoe_tile_weight_t dst");
  const size_t need = qmoe_tiled_weight_t_bytes(V, H);
  REQUIRE(dst_bytes >= need, QMOE_ERR_INVALID, "qmoe_tile_weight_t: dst of %zu bytes needed, %zu given", need, dst_bytes);
  return launched(qmoe::launch_tile_weight_t(src->w, src->scales, src->biases, V, H, (uint8_t*)dst, stream),
                  "qmoe_tile_weight_t");
}

int softmax_rows_bf16(const float* z, int32_t L, int32_t V, uint16_t* probs, hipStream_t stream) {
  REQUIRE(L >= 0, QMOE_ERR_INVALID, "softmax_rows_bf16: L=%d < 0", L);
  REQUIRE(V > 0 && V % 4 == 0, QMOE_ERR_INVALID, "softmax_rows_bf16: V=%d must be a positive multiple of 4", V);
  if (L == 0) return ok();
  REQUIRE_PTR(z, 16, "softmax_rows_bf16 z");
  REQUIRE_PTR(probs, 16, "softmax_rows_bf16 probs");
  return launched(qmoe::launch_softmax_rows_bf16(z, L, V, probs, stream), "softmax_rows_bf16");
}

size_t embed_matmul_t_workspace(int32_t L, int32_t V, int32_t H) {
  if (L <= 0 || V <= 0 || H <= 0 || V % 32 != 0 || H % 64 != 0) return 0;
  return (size_t)qmoe::embed_t_splits(L, V, H) * (size_t)L * (size_t)H * sizeof(float);
}

int embed_matmul_t(const uint16_t* probs, int32_t L, const qmoe_qweight* W, float scale, uint16_t* out,
                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(L >= 0, QMOE_ERR_INVALID, "embed_matmul_t: L=%d < 0", L);
  REQUIRE(W != nullptr, QMOE_ERR_INVALID, "embed_matmul_t: null weight descriptor");
  REQUIRE(std::isfinite(scale), QMOE_ERR_INVALID, "embed_matmul_t: scale must be finite");
  const int V = W->rows, H = W->in;
  REQUIRE(V > 0 && V % 32 == 0, QMOE_ERR_INVALID, "embed_matmul_t: rows=%d must be a positive multiple of 32", V);
  REQUIRE(H > 0 && H % 64 == 0, QMOE_ERR_INVALID, "embed_matmul_t: in=%d must be a positive multiple of 64", H);
  if (int rc = check_qweight(W, "embed_matmul_t W", 1, V, H, QMOE_LAYOUT_TILED_T)) return rc;
  if (L == 0) return ok();
  REQUIRE_PTR(probs, 16, "embed_matmul_t probs");
  REQUIRE_PTR(out, 16, "embed_matmul_t out");
  REQUIRE_PTR(workspace, 16, "embed_matmul_t workspace");
  const size_t need = embed_matmul_t_workspace(L, V, H);
  REQUIRE(ws_bytes >= need, QMOE_ERR_WORKSPACE, "embed_matmul_t: workspace of %zu bytes needed, %zu given", need,
          ws_bytes);
  return launched(qmoe::launch_embed_t(probs, L, V, H, W->w, scale, (float*)workspace, out, stream),
                  "embed_matmul_t");
}

}  // extern "C"

// C ABI of the MoE layer forward and backward: argument validation, capacity arithmetic,
// workspace sizing and kernel launches. Every check runs on the host before
// anything is enqueued; see include/moe.h for the contract of each call.
#include "moe.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "gemm_frag.h"
#include "moe_internal.h"

namespace {

thread_local char g_err[512] = "no error";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == MOE_BF16 ? 2 : 4; }

int check_dtype(int32_t dtype) {
  if (dtype != MOE_F32 && dtype != MOE_BF16)
    return fail(MOE_ERR_DTYPE, "dtype %d is neither MOE_F32 (0) nor MOE_BF16 (1)", dtype);
  return MOE_OK;
}

// Row length rule for vector access: bf16 rows are a multiple of 8 elements,
// f32 rows a multiple of 4 (16 bytes either way).
int check_row(const char* name, int64_t len, int32_t dtype) {
  const int64_t q = dtype == MOE_BF16 ? 8 : 4;
  if (len % q != 0)
    return fail(MOE_ERR_ALIGN, "%s = %lld must be a multiple of %lld for this dtype", name,
                static_cast<long long>(len), static_cast<long long>(q));
  return MOE_OK;
}

int check_ptr16(const char* name, const void* p) {
  if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define MOE_TRY(x)            \
  do {                        \
    const int _rc = (x);      \
    if (_rc != MOE_OK) return _rc; \
  } while (0)

#define MOE_NONNULL(p) \
  do { if ((p) == nullptr) return fail(MOE_ERR_ARG, "%s must not be NULL", #p); } while (0)

int check_experts(int32_t E, int32_t k) {
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_SHAPE, "E = %d outside [1, %d]", E, MOE_MAX_E);
  if (k < 1 || k > E || k > MOE_MAX_K)
    return fail(MOE_ERR_SHAPE, "k = %d outside [1, min(E=%d, %d)]", k, E, MOE_MAX_K);
  return MOE_OK;
}

int check_ffn(const void* a, const int32_t* offsets, int32_t E, int64_t rows_max, int64_t d,
              int64_t d_ff, const void* w, int32_t dtype, const void* out) {
  MOE_TRY(check_dtype(dtype));
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_SHAPE, "E = %d outside [1, %d]", E, MOE_MAX_E);
  if (rows_max < 0 || d <= 0 || d_ff <= 0)
    return fail(MOE_ERR_ARG, "need rows_max >= 0, d > 0, d_ff > 0 (got %lld, %lld, %lld)",
                static_cast<long long>(rows_max), static_cast<long long>(d),
                static_cast<long long>(d_ff));
  if (d > (1 << 22) || d_ff > (1 << 22) || rows_max > 0x7fffffffLL)
    return fail(MOE_ERR_SHAPE, "d and d_ff must be <= 2^22 and rows_max < 2^31");
  if (dtype == MOE_BF16 && (d > (1 << 20) || d_ff > (1 << 20)))
    return fail(MOE_ERR_SHAPE, "bf16 layers need d and d_ff <= 2^20");
  MOE_TRY(check_row("d", d, dtype));
  MOE_TRY(check_row("d_ff", d_ff, dtype));
  if (rows_max == 0) return MOE_OK;
  MOE_NONNULL(a);
  MOE_NONNULL(offsets);
  MOE_NONNULL(w);
  MOE_NONNULL(out);
  MOE_TRY(check_ptr16("activation", a));
  MOE_TRY(check_ptr16("weight", w));
  MOE_TRY(check_ptr16("output", out));
  return MOE_OK;
}

int check_ffn_ws(int32_t dtype, const void* ws, size_t ws_bytes) {
  if (ws == nullptr || dtype != MOE_BF16) return MOE_OK;
  const size_t need = moe::ffn_workspace_bytes(dtype);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "expert-FFN workspace needs %zu bytes, got %zu", need, ws_bytes);
  return check_ptr16("workspace", ws);
}

}  // namespace

namespace moe {

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moe

extern "C" {

int64_t moe_capacity(int64_t n_tokens, int32_t n_experts, double capacity_factor) {
  if (n_tokens < 0 || n_experts < 1) return -2;
  if (!(capacity_factor > 0.0)) return -1;
  const double c = (static_cast<double>(n_tokens) / n_experts) * capacity_factor;
  return static_cast<int64_t>(std::nearbyint(c));   // default mode: round-half-even
}

int64_t moe_rows_max(int64_t T, int32_t k, int32_t E, int64_t capacity) {
  if (T < 0 || k < 1 || E < 1) return -1;
  const int64_t tk = T * k;
  if (capacity < 0) return tk;
  const int64_t ec = static_cast<int64_t>(E) * capacity;
  return tk < ec ? tk : ec;
}

int moe_router_topk_ex(const void* x, const void* w_gate, const float* bias, const float* noise,
                       int64_t T, int64_t d, int32_t E, int32_t k, int32_t dtype, uint32_t flags,
                       float temperature, int32_t* topk_idx, float* topk_w, float* probs,
                       float* lse, hipStream_t stream) {
  MOE_TRY(check_dtype(dtype));
  MOE_TRY(check_experts(E, k));
  if (T < 0 || d <= 0) return fail(MOE_ERR_ARG, "need T >= 0 and d > 0");
  if (T > (1LL << 31) / MOE_MAX_K) return fail(MOE_ERR_SHAPE, "T too large");
  if (flags & ~MOE_RENORM) return fail(MOE_ERR_ARG, "unknown flag bits 0x%x", flags);
  if (!(temperature > 0.0f) || !std::isfinite(temperature))
    return fail(MOE_ERR_ARG, "temperature must be finite and > 0");
  MOE_TRY(check_row("d", d, dtype));
  if (T == 0) return MOE_OK;
  MOE_NONNULL(x);
  MOE_NONNULL(w_gate);
  MOE_NONNULL(topk_idx);
  MOE_NONNULL(topk_w);
  MOE_TRY(check_ptr16("x", x));
  MOE_TRY(check_ptr16("w_gate", w_gate));
  moe::RouterArgs a;
  a.x = x;
  a.wg = w_gate;
  a.bias = bias;
  a.noise = noise;
  a.temperature = temperature;
  a.T = T;
  a.d = d;
  a.E = E;
  a.k = k;
  a.dtype = dtype;
  a.flags = flags;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.probs = probs;
  a.lse = lse;
  a.tile_cnt = nullptr;
  a.tile_colsum = nullptr;
  return hip_status(moe::launch_router(a, stream), "moe_router_topk launch");
}

int64_t moe_router_tiles(int64_t T, int32_t E) {
  if (T <= 0 || E < 1 || E > MOE_MAX_E) return 0;
  const int64_t tt = moe::router_tile_tokens(E);
  return (T + tt - 1) / tt;
}

int moe_router_topk_tiles(const void* x, const void* w_gate, const float* bias, int64_t T, int64_t d,
                          int32_t E, int32_t k, int32_t dtype, uint32_t flags, int32_t* topk_idx,
                          float* topk_w, float* probs, int32_t* tile_counts, double* tile_colsum,
                          hipStream_t stream) {
  MOE_TRY(check_dtype(dtype));
  if (dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "per-tile counts come from the bf16 router only");
  MOE_TRY(check_experts(E, k));
  if (T < 0 || d <= 0) return fail(MOE_ERR_ARG, "need T >= 0 and d > 0");
  if (T > (1LL << 31) / MOE_MAX_K) return fail(MOE_ERR_SHAPE, "T too large");
  if (flags & ~MOE_RENORM) return fail(MOE_ERR_ARG, "unknown flag bits 0x%x", flags);
  MOE_TRY(check_row("d", d, dtype));
  if (T == 0) return MOE_OK;
  MOE_NONNULL(x);
  MOE_NONNULL(w_gate);
  MOE_NONNULL(topk_idx);
  MOE_NONNULL(topk_w);
  MOE_NONNULL(tile_counts);
  MOE_TRY(check_ptr16("x", x));
  MOE_TRY(check_ptr16("w_gate", w_gate));
  if ((reinterpret_cast<uintptr_t>(tile_colsum) & 7u) != 0)
    return fail(MOE_ERR_ALIGN, "tile_colsum is not 8-byte aligned");
  moe::RouterArgs a;
  a.x = x;
  a.wg = w_gate;
  a.bias = bias;
  a.noise = nullptr;
  a.temperature = 1.0f;
  a.T = T;
  a.d = d;
  a.E = E;
  a.k = k;
  a.dtype = dtype;
  a.flags = flags;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.probs = probs;
  a.lse = nullptr;
  a.tile_cnt = tile_counts;
  a.tile_colsum = tile_colsum;
  return hip_status(moe::launch_router(a, stream), "moe_router_topk_tiles launch");
}

int moe_dispatch_plan_tiles(const int32_t* topk_idx, const int32_t* tile_counts, const double* tile_colsum,
                            int64_t T, int32_t k, int32_t E, int64_t capacity, float alpha, int32_t* counts,
                            int32_t* offsets, int32_t* dest, int32_t* src, float* loss, hipStream_t stream) {
  MOE_TRY(check_experts(E, k));
  if (T < 0) return fail(MOE_ERR_ARG, "need T >= 0");
  if (T * k >= (1LL << 31)) return fail(MOE_ERR_SHAPE, "T * k must stay below 2^31");
  MOE_NONNULL(counts);
  MOE_NONNULL(offsets);
  if ((tile_colsum == nullptr) != (loss == nullptr))
    return fail(MOE_ERR_ARG, "tile_colsum and loss go together (both or neither)");
  const int64_t rows = moe_router_tiles(T, E);
  if (rows * E > moe::dispatch_tiles_max())
    return fail(MOE_ERR_SHAPE, "%lld tiles x %d experts exceed %d (use moe_dispatch_plan)",
                static_cast<long long>(rows), E, moe::dispatch_tiles_max());
  if (T > 0) {
    MOE_NONNULL(topk_idx);
    MOE_NONNULL(tile_counts);
    MOE_NONNULL(dest);
    MOE_NONNULL(src);
    if ((reinterpret_cast<uintptr_t>(tile_counts) & 15u) != 0)
      return fail(MOE_ERR_ALIGN, "tile_counts is not 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(tile_colsum) & 7u) != 0)
      return fail(MOE_ERR_ALIGN, "tile_colsum is not 8-byte aligned");
  }
  return hip_status(moe::launch_dispatch_plan_tiles(topk_idx, tile_counts, tile_colsum, moe::router_tile_tokens(E),
                                                    T, k, E, capacity, alpha, counts, offsets, dest, src, loss,
                                                    stream),
                    "moe_dispatch_plan_tiles launch");
}

int moe_router_topk(const void* x, const void* w_gate, const float* bias, int64_t T, int64_t d,
                    int32_t E, int32_t k, int32_t dtype, uint32_t flags, int32_t* topk_idx,
                    float* topk_w, float* probs, hipStream_t stream) {
  return moe_router_topk_ex(x, w_gate, bias, nullptr, T, d, E, k, dtype, flags, 1.0f, topk_idx,
                            topk_w, probs, nullptr, stream);
}

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  (void)k;
  if (T <= 0 || E < 1) return 0;
  return moe::dispatch_ws_ints(T, E) * sizeof(int32_t);
}

namespace {

int check_plan(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t* counts,
               int32_t* offsets, int32_t* dest, int32_t* src, const void* workspace,
               size_t workspace_bytes, bool own_scratch = false) {
  MOE_TRY(check_experts(E, k));
  if (T < 0) return fail(MOE_ERR_ARG, "need T >= 0");
  if (T * k >= (1LL << 31)) return fail(MOE_ERR_SHAPE, "T * k must stay below 2^31");
  MOE_NONNULL(counts);
  MOE_NONNULL(offsets);
  if (T > 0) {
    MOE_NONNULL(topk_idx);
    MOE_NONNULL(dest);
    MOE_NONNULL(src);
    const size_t need = moe_dispatch_workspace_bytes(T, k, E);
    if (own_scratch) {
      if (need > moe::noalloc_scratch_bytes())
        return fail(MOE_ERR_WORKSPACE,
                    "this plan needs %zu bytes of scratch; the library's static scratch holds %zu "
                    "(use moe_dispatch_plan with a workspace)",
                    need, moe::noalloc_scratch_bytes());
      return MOE_OK;
    }
    if (workspace == nullptr || workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                  workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0)
      return fail(MOE_ERR_ALIGN, "workspace is not 4-byte aligned");
  }
  return MOE_OK;
}

int check_permute(const void* x, int64_t d, int32_t dtype, const int32_t* src,
                  const int32_t* offsets, int32_t E, int64_t rows_max, const void* x_perm) {
  MOE_TRY(check_dtype(dtype));
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_SHAPE, "E = %d outside [1, %d]", E, MOE_MAX_E);
  if (d <= 0 || rows_max < 0) return fail(MOE_ERR_ARG, "need d > 0 and rows_max >= 0");
  MOE_TRY(check_row("d", d, dtype));
  if (rows_max == 0) return MOE_OK;
  MOE_NONNULL(x);
  MOE_NONNULL(src);
  MOE_NONNULL(offsets);
  MOE_NONNULL(x_perm);
  MOE_TRY(check_ptr16("x", x));
  MOE_TRY(check_ptr16("x_perm", x_perm));
  return MOE_OK;
}

}  // namespace

int moe_dispatch_plan(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int64_t capacity,
                      int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_plan(topk_idx, T, k, E, counts, offsets, dest, src, workspace, workspace_bytes));
  return hip_status(moe::launch_dispatch_plan(topk_idx, T, k, E, capacity, counts, offsets, dest,
                                              src, static_cast<int32_t*>(workspace), stream),
                    "moe_dispatch_plan launch");
}

size_t moe_dispatch_plan_aux_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  (void)k;
  if (T <= 0 || E < 1) return 0;
  return moe::dispatch_aux_ws_bytes(T, E);
}

int moe_dispatch_plan_aux(const int32_t* topk_idx, const float* probs, int64_t T, int32_t k, int32_t E,
                          int64_t capacity, float alpha, int32_t* counts, int32_t* offsets, int32_t* dest,
                          int32_t* src, float* loss, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  MOE_TRY(check_experts(E, k));
  if (T < 0) return fail(MOE_ERR_ARG, "need T >= 0");
  if (T * k >= (1LL << 31)) return fail(MOE_ERR_SHAPE, "T * k must stay below 2^31");
  MOE_NONNULL(counts);
  MOE_NONNULL(offsets);
  MOE_NONNULL(loss);
  if (T > 0) {
    MOE_NONNULL(topk_idx);
    MOE_NONNULL(probs);
    MOE_NONNULL(dest);
    MOE_NONNULL(src);
    MOE_TRY(check_ptr16("probs", probs));
    const size_t need = moe_dispatch_plan_aux_workspace_bytes(T, k, E);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                  workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
      return fail(MOE_ERR_ALIGN, "workspace is not 8-byte aligned");
  }
  return hip_status(moe::launch_dispatch_plan_aux(topk_idx, T, k, E, capacity, probs, alpha, counts, offsets,
                                                  dest, src, loss, workspace, stream),
                    "moe_dispatch_plan_aux launch");
}

int moe_dispatch_plan_noalloc(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                              int64_t capacity, int32_t* counts, int32_t* offsets, int32_t* dest,
                              int32_t* src, hipStream_t stream) {
  MOE_TRY(check_plan(topk_idx, T, k, E, counts, offsets, dest, src, nullptr, 0, true));
  return hip_status(moe::launch_dispatch_plan_noalloc(topk_idx, T, k, E, capacity, counts, offsets,
                                                      dest, src, stream),
                    "moe_dispatch_plan_noalloc launch");
}

size_t moe_dispatch_plan_noalloc_scratch_bytes(void) { return moe::noalloc_scratch_bytes(); }

int moe_permute(const void* x, int64_t d, int32_t dtype, const int32_t* src,
                const int32_t* offsets, int32_t E, int64_t rows_max, void* x_perm,
                hipStream_t stream) {
  MOE_TRY(check_permute(x, d, dtype, src, offsets, E, rows_max, x_perm));
  return hip_status(moe::launch_permute(x, d, elem_bytes(dtype), src, offsets, E, rows_max,
                                        x_perm, stream),
                    "moe_permute launch");
}

int moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int64_t capacity,
                 const void* x, int64_t d, int32_t dtype, int32_t* counts, int32_t* offsets,
                 int32_t* dest, int32_t* src, void* x_perm, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_dtype(dtype));
  MOE_TRY(check_plan(topk_idx, T, k, E, counts, offsets, dest, src, workspace, workspace_bytes));
  if (d <= 0) return fail(MOE_ERR_ARG, "need d > 0");
  MOE_TRY(check_row("d", d, dtype));
  const int64_t rows_max = moe_rows_max(T, k, E, capacity);
  if (T > 0) MOE_TRY(check_permute(x, d, dtype, src, offsets, E, rows_max, x_perm));
  MOE_TRY(hip_status(moe::launch_dispatch_plan(topk_idx, T, k, E, capacity, counts, offsets, dest,
                                               src, static_cast<int32_t*>(workspace), stream),
                     "moe_dispatch launch"));
  if (T == 0) return MOE_OK;
  return hip_status(moe::launch_permute(x, d, elem_bytes(dtype), src, offsets, E, rows_max,
                                        x_perm, stream),
                    "moe_dispatch launch");
}

int moe_expert_up_gelu(const void* x_perm, const int32_t* offsets, int32_t E, int64_t rows_max,
                       int64_t d, int64_t d_ff, const void* w1, int32_t dtype, void* h,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(x_perm, offsets, E, rows_max, d, d_ff, w1, dtype, h));
  MOE_TRY(check_ffn_ws(dtype, workspace, workspace_bytes));
  return hip_status(moe::launch_up_gelu(x_perm, offsets, E, rows_max, d, d_ff, w1, dtype, h,
                                        nullptr, workspace, stream),
                    "moe_expert_up_gelu launch");
}

int moe_expert_up_gelu_gather(const void* x, int64_t T, const int32_t* src, const int32_t* offsets,
                              int32_t E, int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                              void* h, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(x, offsets, E, rows_max, d, d_ff, w1, MOE_BF16, h));
  MOE_TRY(check_ffn_ws(MOE_BF16, workspace, workspace_bytes));
  if (T < 0) return fail(MOE_ERR_ARG, "T = %lld must be >= 0", static_cast<long long>(T));
  if (T * d > 0x3fffffffLL)
    return fail(MOE_ERR_SHAPE, "moe_expert_up_gelu_gather needs T * d * 2 < 2^31 bytes of x");
  if (rows_max > 0) MOE_NONNULL(src);
  return hip_status(moe::launch_up_gelu_gather(x, T, src, offsets, E, rows_max, d, d_ff, w1, h, workspace,
                                               stream),
                    "moe_expert_up_gelu_gather launch");
}

int64_t moe_frag_rows(int64_t rows_max, int32_t E) {
  if (rows_max < 0 || E < 1 || E > MOE_MAX_E) return -1;
  return moe::frag_rows(rows_max, E);
}

int moe_permute_frag(const void* x, int64_t d, const int32_t* src, const int32_t* offsets,
                     int32_t E, int64_t rows_max, void* x_frag, hipStream_t stream) {
  MOE_TRY(check_permute(x, d, MOE_BF16, src, offsets, E, rows_max, x_frag));
  if (d % 16 != 0) return fail(MOE_ERR_ALIGN, "d = %lld must be a multiple of 16", static_cast<long long>(d));
  if (rows_max > 0x7fffffffLL - 32LL * MOE_MAX_E || d > (1 << 20))
    return fail(MOE_ERR_SHAPE, "moe_permute_frag needs rows_max < 2^31 - 8192 and d <= 2^20");
  return hip_status(moe::launch_permute_frag(x, d, src, offsets, E, rows_max, x_frag, stream),
                    "moe_permute_frag launch");
}

int moe_expert_up_gelu_frag(const void* x_frag, const int32_t* offsets, int32_t E, int64_t rows_max,
                            int64_t d, int64_t d_ff, const void* w1, void* h, int32_t h_order,
                            hipStream_t stream) {
  MOE_TRY(check_ffn(x_frag, offsets, E, rows_max, d, d_ff, w1, MOE_BF16, h));
  if (d % 256 != 0) return fail(MOE_ERR_ALIGN, "d = %lld must be a multiple of 256", static_cast<long long>(d));
  if (h_order != MOE_ORDER_ROWS && h_order != MOE_ORDER_FRAG)
    return fail(MOE_ERR_ARG, "h_order %d is neither MOE_ORDER_ROWS nor MOE_ORDER_FRAG", h_order);
  if (h_order == MOE_ORDER_FRAG && d_ff % 256 != 0)
    return fail(MOE_ERR_ALIGN, "h in fragment order needs d_ff = %lld a multiple of 256", static_cast<long long>(d_ff));
  if (rows_max > 0x7fffffffLL - 32LL * MOE_MAX_E)
    return fail(MOE_ERR_SHAPE, "moe_expert_up_gelu_frag needs rows_max < 2^31 - 8192");
  return hip_status(moe::launch_up_gelu_frag(x_frag, offsets, E, rows_max, d, d_ff, w1, h,
                                             h_order == MOE_ORDER_FRAG, stream),
                    "moe_expert_up_gelu_frag launch");
}

int moe_expert_down_frag(const void* h_frag, const int32_t* offsets, int32_t E, int64_t rows_max, int64_t d,
                         int64_t d_ff, const void* w2_f16, float* y_perm, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(h_frag, offsets, E, rows_max, d, d_ff, w2_f16, MOE_BF16, y_perm));
  MOE_TRY(check_ffn_ws(MOE_BF16, workspace, workspace_bytes));
  if (d_ff % 256 != 0)
    return fail(MOE_ERR_ALIGN, "d_ff = %lld must be a multiple of 256", static_cast<long long>(d_ff));
  if (rows_max > 0x7fffffffLL - 32LL * MOE_MAX_E)
    return fail(MOE_ERR_SHAPE, "moe_expert_down_frag needs rows_max < 2^31 - 8192");
  return hip_status(moe::launch_down_frag(h_frag, offsets, E, rows_max, d, d_ff, w2_f16, y_perm, workspace, stream),
                    "moe_expert_down_frag launch");
}

int moe_expert_down(const void* h, const int32_t* offsets, int32_t E, int64_t rows_max, int64_t d,
                    int64_t d_ff, const void* w2, int32_t dtype, float* y_perm, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(h, offsets, E, rows_max, d, d_ff, w2, dtype, y_perm));
  MOE_TRY(check_ffn_ws(dtype, workspace, workspace_bytes));
  return hip_status(moe::launch_down(h, offsets, E, rows_max, d, d_ff, w2, dtype, y_perm,
                                     workspace, stream),
                    "moe_expert_down launch");
}

int moe_weights_bf16_to_f16(const void* w, int64_t n, void* w_f16, uint64_t* report,
                            hipStream_t stream) {
  if (n < 0) return fail(MOE_ERR_ARG, "n = %lld < 0", static_cast<long long>(n));
  if ((reinterpret_cast<uintptr_t>(report) & 7u) != 0)
    return fail(MOE_ERR_ALIGN, "report is not 8-byte aligned");
  if (n > 0) {
    MOE_NONNULL(w);
    MOE_NONNULL(w_f16);
    MOE_TRY(check_ptr16("w", w));
    MOE_TRY(check_ptr16("w_f16", w_f16));
  }
  return hip_status(moe::launch_bf16_to_f16(w, n, w_f16, report, stream),
                    "moe_weights_bf16_to_f16 launch");
}

int moe_expert_down_f16w(const void* h, const int32_t* offsets, int32_t E, int64_t rows_max, int64_t d,
                         int64_t d_ff, const void* w2_f16, float* y_perm, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(h, offsets, E, rows_max, d, d_ff, w2_f16, MOE_BF16, y_perm));
  MOE_TRY(check_ffn_ws(MOE_BF16, workspace, workspace_bytes));
  return hip_status(moe::launch_down_f16w(h, offsets, E, rows_max, d, d_ff, w2_f16, y_perm, workspace, stream),
                    "moe_expert_down_f16w launch");
}

int moe_grouped_ffn(const void* x_perm, const int32_t* offsets, int32_t E, int64_t rows_max,
                    int64_t d, int64_t d_ff, const void* w1, const void* w2, int32_t dtype,
                    void* h, float* y_perm, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  MOE_TRY(check_ffn(x_perm, offsets, E, rows_max, d, d_ff, w1, dtype, h));
  MOE_TRY(check_ffn(h, offsets, E, rows_max, d, d_ff, w2, dtype, y_perm));
  MOE_TRY(check_ffn_ws(dtype, workspace, workspace_bytes));
  MOE_TRY(hip_status(moe::launch_up_gelu(x_perm, offsets, E, rows_max, d, d_ff, w1, dtype, h,
                                         nullptr, workspace, stream),
                     "moe_grouped_ffn up-projection launch"));
  return hip_status(moe::launch_down(h, offsets, E, rows_max, d, d_ff, w2, dtype, y_perm,
                                     workspace, stream),
                    "moe_grouped_ffn down-projection launch");
}

size_t moe_ffn_workspace_bytes(int32_t dtype) {
  return dtype == MOE_BF16 ? moe::ffn_workspace_bytes(dtype) : 0;
}

int moe_combine(const float* y_perm, const int32_t* dest, const float* topk_w, int64_t T,
                int32_t k, int64_t d, void* y, int32_t out_dtype, hipStream_t stream) {
  MOE_TRY(check_dtype(out_dtype));
  if (T < 0 || d <= 0 || k < 1 || k > MOE_MAX_K)
    return fail(MOE_ERR_ARG, "need T >= 0, d > 0, 1 <= k <= %d", MOE_MAX_K);
  if (d % 4 != 0) return fail(MOE_ERR_ALIGN, "d = %lld must be a multiple of 4", static_cast<long long>(d));
  if (T == 0) return MOE_OK;
  MOE_NONNULL(dest);
  MOE_NONNULL(topk_w);
  MOE_NONNULL(y);
  MOE_NONNULL(y_perm);
  MOE_TRY(check_ptr16("y_perm", y_perm));
  if (out_dtype == MOE_BF16) {
    if ((reinterpret_cast<uintptr_t>(y) & 7u) != 0) return fail(MOE_ERR_ALIGN, "y is not 8-byte aligned");
  } else {
    MOE_TRY(check_ptr16("y", y));
  }
  return hip_status(moe::launch_combine(y_perm, dest, topk_w, T, k, d, y, out_dtype, stream),
                    "moe_combine launch");
}

size_t moe_aux_loss_workspace_bytes(int64_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return moe::aux_ws_doubles(T, E) * sizeof(double);
}

int moe_aux_loss(const float* probs, const int32_t* counts, int64_t T, int32_t E, int32_t k,
                 float alpha, float* loss, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  MOE_TRY(check_experts(E, k));
  if (T < 0) return fail(MOE_ERR_ARG, "need T >= 0");
  MOE_NONNULL(loss);
  MOE_NONNULL(counts);
  if (T > 0) MOE_NONNULL(probs);
  const size_t need = moe_aux_loss_workspace_bytes(T, E);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
    return fail(MOE_ERR_ALIGN, "workspace is not 8-byte aligned");
  return hip_status(moe::launch_aux_loss(probs, counts, T, E, k, alpha, loss,
                                         static_cast<double*>(workspace), stream),
                    "moe_aux_loss launch");
}

size_t moe_z_loss_workspace_bytes(int64_t T) {
  if (T < 0) return 0;
  return moe::z_ws_doubles(T) * sizeof(double);
}

int moe_z_loss(const float* lse, int64_t T, float coeff, float* loss, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  if (T < 0) return fail(MOE_ERR_ARG, "need T >= 0");
  MOE_NONNULL(loss);
  if (T > 0) MOE_NONNULL(lse);
  const size_t need = moe_z_loss_workspace_bytes(T);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
    return fail(MOE_ERR_ALIGN, "workspace is not 8-byte aligned");
  return hip_status(moe::launch_z_loss(lse, T, coeff, loss, static_cast<double*>(workspace), stream),
                    "moe_z_loss launch");
}

// ------------------------------------------------------------------ backward

namespace {

// The bf16 backward GEMMs address a weight matrix of one expert, and the rows
// of one expert's activations, through 32-bit buffer ranges.
int check_bwd_limits(int64_t rows_max, int64_t d, int64_t d_ff, int32_t dtype) {
  if (dtype != MOE_BF16) return MOE_OK;
  const int64_t wide = d > d_ff ? d : d_ff;
  if (d * d_ff >= (1LL << 30) || rows_max * wide >= (1LL << 30))
    return fail(MOE_ERR_SHAPE, "backward needs d * d_ff < 2^30 and rows_max * max(d, d_ff) < 2^30");
  return MOE_OK;
}

}  // namespace

int moe_expert_up_gelu_z(const void* x_perm, const int32_t* offsets, int32_t E, int64_t rows_max,
                         int64_t d, int64_t d_ff, const void* w1, int32_t dtype, void* h, void* z,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(x_perm, offsets, E, rows_max, d, d_ff, w1, dtype, h));
  MOE_TRY(check_ffn_ws(dtype, workspace, workspace_bytes));
  if (rows_max > 0) {
    MOE_NONNULL(z);
    MOE_TRY(check_ptr16("z", z));
  }
  return hip_status(moe::launch_up_gelu(x_perm, offsets, E, rows_max, d, d_ff, w1, dtype, h, z,
                                        workspace, stream),
                    "moe_expert_up_gelu_z launch");
}

int moe_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                         const float* topk_w, int64_t T, int32_t k, int64_t d, int32_t dtype,
                         void* d_out_perm, float* d_topk_w, hipStream_t stream) {
  MOE_TRY(check_dtype(dtype));
  if (T < 0 || d <= 0 || k < 1 || k > MOE_MAX_K)
    return fail(MOE_ERR_ARG, "need T >= 0, d > 0, 1 <= k <= %d", MOE_MAX_K);
  MOE_TRY(check_row("d", d, dtype));
  if (T == 0) return MOE_OK;
  MOE_NONNULL(dy);
  MOE_NONNULL(y_perm);
  MOE_NONNULL(dest);
  MOE_NONNULL(topk_w);
  MOE_NONNULL(d_out_perm);
  MOE_NONNULL(d_topk_w);
  MOE_TRY(check_ptr16("dy", dy));
  MOE_TRY(check_ptr16("y_perm", y_perm));
  MOE_TRY(check_ptr16("d_out_perm", d_out_perm));
  return hip_status(moe::launch_combine_backward(dy, y_perm, dest, topk_w, T, k, d, dtype,
                                                 d_out_perm, d_topk_w, stream),
                    "moe_combine_backward launch");
}

int moe_expert_down_backward(const void* d_out_perm, const int32_t* offsets, int32_t E,
                             int64_t rows_max, int64_t d, int64_t d_ff, const void* w2,
                             const void* z, int32_t dtype, void* dz, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(d_out_perm, offsets, E, rows_max, d, d_ff, w2, dtype, dz));
  MOE_TRY(check_ffn_ws(dtype, workspace, workspace_bytes));
  MOE_TRY(check_bwd_limits(rows_max, d, d_ff, dtype));
  if (rows_max == 0) return MOE_OK;
  MOE_NONNULL(z);
  MOE_TRY(check_ptr16("z", z));
  return hip_status(moe::launch_down_backward(d_out_perm, offsets, E, rows_max, d, d_ff, w2, z,
                                              dtype, dz, workspace, stream),
                    "moe_expert_down_backward launch");
}

int moe_expert_up_backward(const void* dz, const int32_t* offsets, int32_t E, int64_t rows_max,
                           int64_t d, int64_t d_ff, const void* w1, int32_t dtype, float* dx_perm,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_ffn(dz, offsets, E, rows_max, d, d_ff, w1, dtype, dx_perm));
  MOE_TRY(check_ffn_ws(dtype, workspace, workspace_bytes));
  MOE_TRY(check_bwd_limits(rows_max, d, d_ff, dtype));
  return hip_status(moe::launch_up_backward(dz, offsets, E, rows_max, d, d_ff, w1, dtype, dx_perm,
                                            workspace, stream),
                    "moe_expert_up_backward launch");
}

int moe_expert_weight_grads(const void* x_perm, const void* h, const void* d_out_perm,
                            const void* dz, const int32_t* offsets, int32_t E, int64_t rows_max,
                            int64_t d, int64_t d_ff, int32_t dtype, float* dw1, float* dw2,
                            hipStream_t stream) {
  MOE_TRY(check_dtype(dtype));
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_SHAPE, "E = %d outside [1, %d]", E, MOE_MAX_E);
  if (rows_max < 0 || d <= 0 || d_ff <= 0)
    return fail(MOE_ERR_ARG, "need rows_max >= 0, d > 0, d_ff > 0");
  if (d > (1 << 22) || d_ff > (1 << 22) || rows_max > 0x7fffffffLL)
    return fail(MOE_ERR_SHAPE, "d and d_ff must be <= 2^22 and rows_max < 2^31");
  if (dtype == MOE_BF16 && (d > (1 << 20) || d_ff > (1 << 20)))
    return fail(MOE_ERR_SHAPE, "bf16 layers need d and d_ff <= 2^20");
  MOE_TRY(check_row("d", d, dtype));
  MOE_TRY(check_row("d_ff", d_ff, dtype));
  MOE_TRY(check_bwd_limits(rows_max, d, d_ff, dtype));
  MOE_NONNULL(offsets);
  if (dw1 != nullptr) {
    MOE_NONNULL(dz);
    MOE_NONNULL(x_perm);
    MOE_TRY(check_ptr16("dz", dz));
    MOE_TRY(check_ptr16("x_perm", x_perm));
    MOE_TRY(check_ptr16("dw1", dw1));
  }
  if (dw2 != nullptr) {
    MOE_NONNULL(d_out_perm);
    MOE_NONNULL(h);
    MOE_TRY(check_ptr16("d_out_perm", d_out_perm));
    MOE_TRY(check_ptr16("h", h));
    MOE_TRY(check_ptr16("dw2", dw2));
  }
  if (dw2 != nullptr)
    MOE_TRY(hip_status(moe::launch_expert_dw2(d_out_perm, h, offsets, E, d, d_ff, dtype, dw2, stream),
                       "moe_expert_weight_grads dW2 launch"));
  if (dw1 != nullptr)
    MOE_TRY(hip_status(moe::launch_expert_dw1(dz, x_perm, offsets, E, d, d_ff, dtype, dw1, stream),
                       "moe_expert_weight_grads dW1 launch"));
  return MOE_OK;
}

int moe_gate_backward(const float* d_topk_w, const int32_t* topk_idx, const float* topk_w,
                      const float* probs, const int32_t* counts, const float* lse, int64_t T,
                      int32_t E, int32_t k, uint32_t flags, float temperature, float alpha,
                      float aux_grad, float z_coeff, float* d_logits, hipStream_t stream) {
  MOE_TRY(check_experts(E, k));
  if (T < 0) return fail(MOE_ERR_ARG, "need T >= 0");
  if (!(temperature > 0.0f) || !std::isfinite(temperature))
    return fail(MOE_ERR_ARG, "temperature must be finite and > 0");
  if (!std::isfinite(alpha) || !std::isfinite(aux_grad) || !std::isfinite(z_coeff))
    return fail(MOE_ERR_ARG, "alpha, aux_grad and z_coeff must be finite");
  if (T == 0) return MOE_OK;
  MOE_NONNULL(d_topk_w);
  MOE_NONNULL(topk_idx);
  MOE_NONNULL(probs);
  MOE_NONNULL(counts);
  MOE_NONNULL(d_logits);
  if (flags & MOE_RENORM) MOE_NONNULL(topk_w);
  if (z_coeff != 0.0f) MOE_NONNULL(lse);
  return hip_status(moe::launch_gate_backward(d_topk_w, topk_idx, topk_w, probs, counts, lse, T,
                                              E, k, (flags & MOE_RENORM) != 0, temperature, alpha,
                                              aux_grad, z_coeff, d_logits, stream),
                    "moe_gate_backward launch");
}

size_t moe_gate_weight_grads_workspace_bytes(int64_t T, int64_t d, int32_t E) {
  if (T < 0 || d <= 0 || E < 1) return 0;
  return moe::gate_wgrad_ws_floats(T, d, E) * sizeof(float);
}

int moe_gate_weight_grads(const float* d_logits, const void* x, int64_t T, int64_t d, int32_t E,
                          int32_t dtype, float* d_w_gate, float* d_bias, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_dtype(dtype));
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_SHAPE, "E = %d outside [1, %d]", E, MOE_MAX_E);
  if (T < 0 || d <= 0) return fail(MOE_ERR_ARG, "need T >= 0 and d > 0");
  MOE_TRY(check_row("d", d, dtype));
  MOE_NONNULL(d_w_gate);
  MOE_TRY(check_ptr16("d_w_gate", d_w_gate));
  if (T > 0) {
    MOE_NONNULL(d_logits);
    MOE_NONNULL(x);
    MOE_TRY(check_ptr16("x", x));
  }
  const size_t need = moe_gate_weight_grads_workspace_bytes(T, d, E);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
  MOE_TRY(check_ptr16("workspace", workspace));
  return hip_status(moe::launch_gate_wgrad(d_logits, x, T, d, E, dtype, d_w_gate, d_bias,
                                           static_cast<float*>(workspace), stream),
                    "moe_gate_weight_grads launch");
}

int moe_dispatch_backward(const float* dx_perm, const int32_t* dest, const float* d_logits,
                          const void* w_gate, int64_t T, int32_t k, int64_t d, int32_t E,
                          int32_t dtype, float* dx, hipStream_t stream) {
  MOE_TRY(check_dtype(dtype));
  if (T < 0 || d <= 0 || k < 1 || k > MOE_MAX_K)
    return fail(MOE_ERR_ARG, "need T >= 0, d > 0, 1 <= k <= %d", MOE_MAX_K);
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_SHAPE, "E = %d outside [1, %d]", E, MOE_MAX_E);
  MOE_TRY(check_row("d", d, dtype));
  if ((d_logits == nullptr) != (w_gate == nullptr))
    return fail(MOE_ERR_ARG, "d_logits and w_gate are both given or both NULL");
  if (T == 0) return MOE_OK;
  MOE_NONNULL(dx_perm);
  MOE_NONNULL(dest);
  MOE_NONNULL(dx);
  MOE_TRY(check_ptr16("dx_perm", dx_perm));
  MOE_TRY(check_ptr16("dx", dx));
  if (w_gate != nullptr) MOE_TRY(check_ptr16("w_gate", w_gate));
  return hip_status(moe::launch_dispatch_backward(dx_perm, dest, d_logits, w_gate, T, k, d, E,
                                                  dtype, dx, stream),
                    "moe_dispatch_backward launch");
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"

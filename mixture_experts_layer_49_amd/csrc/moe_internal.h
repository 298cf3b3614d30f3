// Internal declarations shared by the kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;
constexpr int kDispatchTok = 256;   // tokens per dispatch workgroup

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Launchers (host). Arguments are validated by the C-ABI layer before these
// run; each enqueues on `s` and returns the launch status.
// Router arguments (validated by the C-ABI layer).
struct RouterArgs {
  const void* x;
  const void* wg;
  const float* bias;    // nullable [E]
  const float* noise;   // nullable [T, E], added to the logits
  float temperature;    // > 0; scores = (logits + noise) / temperature
  int64_t T, d;
  int E, k, dtype;
  uint32_t flags;
  int32_t* topk_idx;
  float* topk_w;
  float* probs;         // nullable [T, E]
  float* lse;           // nullable [T]: log sum_e exp(score)
  // nullable (bf16 only): per token tile of router_tile_tokens(E) tokens, how
  // many of its assignments name each expert, and (tile_colsum, nullable)
  // the tile's probabilities summed per expert in double, in token order
  int32_t* tile_cnt;    // [ntiles, E]
  double* tile_colsum;  // [ntiles, E]
};
// Tokens per router workgroup for E experts (bf16 kernel).
int router_tile_tokens(int E);
hipError_t launch_router(const RouterArgs& a, hipStream_t s);

hipError_t launch_dispatch_plan(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                                int32_t* ws, hipStream_t s);

// The dispatch plan from the router's per-tile counts (tile_tokens tokens per
// tile, dividing kDispatchTok; ntiles x E <= dispatch_tiles_max()): one
// launch, no workspace. With tile_colsum (and loss) also the aux loss.
int dispatch_tiles_max();
hipError_t launch_dispatch_plan_tiles(const int32_t* topk_idx, const int32_t* tile_cnt,
                                      const double* tile_colsum, int tile_tokens, int64_t T, int k,
                                      int E, int64_t cap, float alpha, int32_t* counts,
                                      int32_t* offsets, int32_t* dest, int32_t* src, float* loss,
                                      hipStream_t s);

hipError_t launch_permute(const void* x, int64_t d, int elem_bytes, const int32_t* src,
                          const int32_t* offsets, int E, int64_t rows_max, void* x_perm,
                          hipStream_t s);

// ws: the expert-FFN workspace (ffn_workspace_bytes(dtype) bytes) or null.
// z: nullable; receives the pre-activation in the hidden storage type.
hipError_t launch_up_gelu(const void* x_perm, const int32_t* offsets, int E, int64_t rows_max,
                          int64_t d, int64_t d_ff, const void* w1, int dtype, void* h, void* z,
                          void* ws, hipStream_t s);
// bf16: launch_up_gelu on x [T, d] read through src (row r = x[src[r]]).
hipError_t launch_up_gelu_gather(const void* x, int64_t T, const int32_t* src, const int32_t* offsets,
                                 int E, int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                                 void* h, void* ws, hipStream_t s);

hipError_t launch_down(const void* h, const int32_t* offsets, int E, int64_t rows_max,
                       int64_t d, int64_t d_ff, const void* w2, int dtype, float* y_perm,
                       void* ws, hipStream_t s);

// bf16 layers: the segmented MFMA GEMM. Row-segmented kinds (rows of A and C
// grouped by expert, K fixed):
//   kUp:   A [R, K] bf16,  B = W1 [E, N, K] bf16 -> C = fp16 gelu(A B^T)
//          (and, with Z, the fp16 pre-activation A B^T in Z [R, N])
//   kUpGather: kUp with A = x [a_rows, K] bf16 read through the row map gsrc:
//          row r of the product is x[gsrc[r]] (Z not supported)
//   kDown: A [R, K] fp16,  B = W2 [E, N, K] bf16 -> C = A B^T f32
//   kDownF16: as kDown with W2 stored as fp16 (no conversion in the kernel)
//   kDh:   A [R, K] bf16,  B = W2 [E, K, N] bf16 -> C = bf16((A B) * gelu'(Z)), Z [R, N] fp16
//   kDx:   A [R, K] bf16,  B = W1 [E, K, N] bf16 -> C = A B f32
// K-segmented kinds (the contraction runs over each expert's rows):
//   kDw2:  A [R, M] bf16,  B [R, N] fp16 -> C[e] = A_e^T B_e f32 [E, M, N]
//   kDw1:  A [R, M] bf16,  B [R, N] bf16 -> C[e] = A_e^T B_e f32 [E, M, N]
// With a workspace, output tiles of a short last round of a row-segmented
// kind are split along K.
enum class GemmKind { kUp, kUpGather, kDown, kDownF16, kDh, kDx, kDw2, kDw1 };
hipError_t launch_gemm_mfma(GemmKind kind, const void* A, const int32_t* offsets, int E,
                            int64_t rows_max, int M, int N, int K, const void* B, void* C,
                            void* Z, void* ws, hipStream_t s, const int32_t* gsrc = nullptr,
                            int64_t a_rows = 0);
inline hipError_t launch_ffn_mfma(bool up, const void* A, const int32_t* offsets, int E,
                                  int64_t rows_max, int N, int K, const void* B, void* C,
                                  void* ws, hipStream_t s) {
  return launch_gemm_mfma(up ? GemmKind::kUp : GemmKind::kDown, A, offsets, E, rows_max, 0, N, K,
                          B, C, nullptr, ws, s);
}

// Workspace bytes of the expert FFN on the current device (0 for f32 layers).
size_t ffn_workspace_bytes(int dtype);
size_t ffn_mfma_workspace_bytes();

// W2 in fp16 for the down-projection (grouped_ffn.hip): n bf16 values -> fp16, RNE.
hipError_t launch_bf16_to_f16(const void* src, int64_t n, void* dst, uint64_t* report, hipStream_t s);
hipError_t launch_down_f16w(const void* h, const int32_t* offsets, int E, int64_t rows_max, int64_t d,
                            int64_t d_ff, const void* w2_f16, float* y_perm, void* ws, hipStream_t s);

hipError_t launch_combine(const float* y_perm, const int32_t* dest, const float* topk_w,
                          int64_t T, int k, int64_t d, void* y, int out_dtype, hipStream_t s);

// Router z-loss: loss = coeff * mean_t lse[t]^2; ws as for the aux loss.
hipError_t launch_z_loss(const float* lse, int64_t T, float coeff, float* loss, double* ws,
                         hipStream_t s);
size_t z_ws_doubles(int64_t T);

hipError_t launch_aux_loss(const float* probs, const int32_t* counts, int64_t T, int E, int k,
                           float alpha, float* loss, double* ws, hipStream_t s);

size_t dispatch_ws_ints(int64_t T, int E);
// The plan and the aux loss in one pass (dispatch.hip): the workspace holds
// the plan's ints, then one double per (256-token chunk, expert).
size_t dispatch_aux_ws_bytes(int64_t T, int E);
hipError_t launch_dispatch_plan_aux(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                    const float* probs, float alpha, int32_t* counts, int32_t* offsets,
                                    int32_t* dest, int32_t* src, float* loss, void* ws, hipStream_t s);
// The aux loss from per-chunk column sums of the probabilities (combine_aux.hip).
hipError_t launch_aux_final_chunks(const double* colsum, int nchunks, const int32_t* counts, int64_t T, int E,
                                   int k, float alpha, float* loss, hipStream_t s);
// The plan on the library's own per-GPU scratch (dispatch.hip).
size_t noalloc_scratch_bytes();
hipError_t launch_dispatch_plan_noalloc(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                        int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                                        hipStream_t s);
size_t aux_ws_doubles(int64_t T, int E);

// Backward (backward.hip). Gradient storage of a layer: bf16 for dtype 1, f32
// for dtype 0; dx_perm, dW1, dW2, dWg and db are f32.
hipError_t launch_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                                   const float* topk_w, int64_t T, int k, int64_t d, int dtype,
                                   void* d_out, float* dw, hipStream_t s);
hipError_t launch_gate_backward(const float* dw, const int32_t* topk_idx, const float* topk_w,
                                const float* probs, const int32_t* counts, const float* lse,
                                int64_t T, int E, int k, bool renorm, float temperature,
                                float alpha, float aux_grad, float z_coeff, float* dl,
                                hipStream_t s);
size_t gate_wgrad_ws_floats(int64_t T, int64_t d, int E);
hipError_t launch_gate_wgrad(const float* dl, const void* x, int64_t T, int64_t d, int E,
                             int dtype, float* dwg, float* db, float* ws, hipStream_t s);
hipError_t launch_dispatch_backward(const float* dx_perm, const int32_t* dest, const float* dl,
                                    const void* wg, int64_t T, int k, int64_t d, int E, int dtype,
                                    float* dx, hipStream_t s);
hipError_t launch_down_backward(const void* d_out, const int32_t* offsets, int E, int64_t rows_max,
                                int64_t d, int64_t d_ff, const void* w2, const void* z, int dtype,
                                void* dz, void* ws, hipStream_t s);
hipError_t launch_up_backward(const void* dz, const int32_t* offsets, int E, int64_t rows_max,
                              int64_t d, int64_t d_ff, const void* w1, int dtype, float* dx_perm,
                              void* ws, hipStream_t s);
hipError_t launch_expert_dw2(const void* d_out, const void* h, const int32_t* offsets, int E,
                             int64_t d, int64_t d_ff, int dtype, float* dw2, hipStream_t s);
hipError_t launch_expert_dw1(const void* dz, const void* x_perm, const int32_t* offsets, int E,
                             int64_t d, int64_t d_ff, int dtype, float* dw1, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe

// Internal declarations shared by the kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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
  float* zsq;           // nullable [T]: (log sum_e exp(score))^2
};
hipError_t launch_router(const RouterArgs& a, hipStream_t s);

hipError_t launch_dispatch_plan(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                                int32_t* ws, hipStream_t s);

hipError_t launch_permute(const void* x, int64_t d, int elem_bytes, const int32_t* src,
                          const int32_t* offsets, int E, int64_t rows_max, void* x_perm,
                          hipStream_t s);

// ws: the expert-FFN workspace (ffn_workspace_bytes(dtype) bytes) or null.
hipError_t launch_up_gelu(const void* x_perm, const int32_t* offsets, int E, int64_t rows_max,
                          int64_t d, int64_t d_ff, const void* w1, int dtype, void* h, void* ws,
                          hipStream_t s);

hipError_t launch_down(const void* h, const int32_t* offsets, int E, int64_t rows_max,
                       int64_t d, int64_t d_ff, const void* w2, int dtype, float* y_perm,
                       void* ws, hipStream_t s);

// bf16 layers: the segmented MFMA GEMM (up: GELU -> fp16 h; down: f32 out).
// With a workspace, output tiles of a short last round are split along K.
hipError_t launch_ffn_mfma(bool up, const void* A, const int32_t* offsets, int E, int64_t rows_max,
                           int N, int K, const void* B, void* C, void* ws, hipStream_t s);

// Workspace bytes of the expert FFN on the current device (0 for f32 layers).
size_t ffn_workspace_bytes(int dtype);
size_t ffn_mfma_workspace_bytes();

hipError_t launch_combine(const float* y_perm, const int32_t* dest, const float* topk_w,
                          int64_t T, int k, int64_t d, void* y, int out_dtype, hipStream_t s);

// Router z-loss: loss = coeff * mean_t zsq[t]; ws as for the aux loss.
hipError_t launch_z_loss(const float* zsq, int64_t T, float coeff, float* loss, double* ws,
                         hipStream_t s);
size_t z_ws_doubles(int64_t T);

hipError_t launch_aux_loss(const float* probs, const int32_t* counts, int64_t T, int E, int k,
                           float alpha, float* loss, double* ws, hipStream_t s);

size_t dispatch_ws_ints(int64_t T, int E);
size_t aux_ws_doubles(int64_t T, int E);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe

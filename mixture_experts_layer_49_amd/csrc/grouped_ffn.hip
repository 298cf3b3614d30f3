// Grouped expert FFN (ETP page "ETP专家并行加速MoE模型": each expert is an
// up-projection w1 and a down-projection w2, e.g. 4096 -> 16384 -> 4096;
// EP tutorial "专家并行：混合专家模型的分布式训练方案", section 2.1 step 4: every
// expert computes on the tokens routed to it).
//
// Both projections are one segmented "NT" GEMM, C[m, n] = sum_k A[m, k] B[n, k]
// with A and B K-contiguous, over the expert-major row segments that
// offsets[] describes:
//   up:   A = x_perm [R, d],  B = W1[e] [d_ff, d], C = gelu_tanh(.) -> h
//   down: A = h [R, d_ff],    B = W2[e] [d, d_ff], C -> y_perm (f32)
//
// bf16 layers run on the MFMA kernel in gemm_mfma.hip. The hidden activation h
// of a bf16 layer is kept as IEEE fp16, not bf16: same size, three more
// significand bits, which cuts the rounding error it adds to the layer output
// about eight-fold; the down-projection then multiplies fp16 by fp16, W2's
// bf16 values being rounded to fp16 (nearest even) on their way into LDS.
// That rounding is exact for 2^-17 <= |w| <= 65280 and for 0: smaller values
// may lose low bits (fp16 subnormals), larger finite ones become +-inf. h itself
// saturates the same way: |gelu(z)| >= 65520 is stored as +-inf, and the
// output rows that use it are then inf or NaN.
//
// f32 layers run on the plain 64x64 LDS-tiled FMA kernel below, over the same
// device-side tile list.
#include "ffn_common.h"

namespace moe {
namespace {

using namespace ffn;

constexpr int FM = 64, FN = 64, FK = 16;

template <bool UP>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float* __restrict__ A,
                                                        const int32_t* __restrict__ offsets,
                                                        int E, int N, int K,
                                                        const float* __restrict__ B,
                                                        float* __restrict__ C,
                                                        float* __restrict__ Z) {
  __shared__ float As[FK][FM + 4];
  __shared__ float Bs[FK][FN + 4];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_tmp[kMaxE];
  build_tile_prefix(offsets, E, FM, s_pref, s_tmp);
  const int tiles_n = (N + FN - 1) / FN;
  const int64_t total = static_cast<int64_t>(s_pref[E]) * tiles_n;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  for (int64_t id = blockIdx.x; id < total; id += gridDim.x) {
    const Tile tl = find_tile(s_pref, E, tiles_n, id);
    const int seg1 = offsets[tl.e + 1];
    const int m0 = offsets[tl.e] + tl.mi * FM, n0 = tl.nt * FN;
    const float* Be = B + static_cast<int64_t>(tl.e) * N * K;
    const int lr = tid >> 2, lk = (tid & 3) * 4;   // loader: row, 4 k-values
    const float* ap = A + static_cast<int64_t>(min(m0 + lr, seg1 - 1)) * K;
    const float* bp = Be + static_cast<int64_t>(min(n0 + lr, N - 1)) * K;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += FK) {
      const bool ok = k0 + lk < K;
      const float4 av = ok ? *reinterpret_cast<const float4*>(ap + k0 + lk) : float4{0, 0, 0, 0};
      const float4 bv = ok ? *reinterpret_cast<const float4*>(bp + k0 + lk) : float4{0, 0, 0, 0};
      __syncthreads();
      As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
      Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < FK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + ty * 4 + i;
      if (row >= seg1) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col >= N) continue;
        C[static_cast<int64_t>(row) * N + col] = UP ? gelu_tanh(acc[i][j]) : acc[i][j];
        if (UP && Z != nullptr) Z[static_cast<int64_t>(row) * N + col] = acc[i][j];
      }
    }
    __syncthreads();
  }
}

template <bool UP>
hipError_t launch_gemm(const void* A, const int32_t* offsets, int E, int64_t rows_max, int N,
                       int K, const void* B, int dtype, void* C, void* Z, void* ws, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  if (dtype == 1)
    return launch_gemm_mfma(UP ? GemmKind::kUp : GemmKind::kDown, A, offsets, E, rows_max, 0, N,
                            K, B, C, Z, ws, s);
  const int64_t tiles_n = (N + FN - 1) / FN;
  int64_t g = (rows_max / FM + E) * tiles_n;
  if (g > 65535) g = 65535;
  hipLaunchKernelGGL(grouped_gemm_f32<UP>, dim3(static_cast<unsigned>(g)), dim3(256), 0, s,
                     static_cast<const float*>(A), offsets, E, N, K, static_cast<const float*>(B),
                     static_cast<float*>(C), static_cast<float*>(Z));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_up_gelu(const void* x_perm, const int32_t* offsets, int E, int64_t rows_max,
                          int64_t d, int64_t d_ff, const void* w1, int dtype, void* h, void* z,
                          void* ws, hipStream_t s) {
  return launch_gemm<true>(x_perm, offsets, E, rows_max, static_cast<int>(d_ff),
                           static_cast<int>(d), w1, dtype, h, z, ws, s);
}

hipError_t launch_up_gelu_gather(const void* x, int64_t T, const int32_t* src, const int32_t* offsets,
                                 int E, int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                                 void* h, void* ws, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  return launch_gemm_mfma(GemmKind::kUpGather, x, offsets, E, rows_max, 0, static_cast<int>(d_ff),
                          static_cast<int>(d), w1, h, nullptr, ws, s, src, T);
}

hipError_t launch_down(const void* h, const int32_t* offsets, int E, int64_t rows_max, int64_t d,
                       int64_t d_ff, const void* w2, int dtype, float* y_perm, void* ws,
                       hipStream_t s) {
  return launch_gemm<false>(h, offsets, E, rows_max, static_cast<int>(d), static_cast<int>(d_ff),
                            w2, dtype, y_perm, nullptr, ws, s);
}

namespace {

// What rounding a bf16 value to fp16 did: bit 0 set when the fp16 value
// differs from a finite nonzero input and is finite (low bits lost), bit 1
// when a finite input became +-inf. Infinities and NaNs pass through
// unflagged.
__device__ __forceinline__ int f16_rounding_flags(float f, _Float16 h) {
  const float back = static_cast<float>(h);
  if (!__builtin_isfinite(f)) return 0;
  if (__builtin_isinf(back)) return 2;
  return back != f ? 1 : 0;
}

// Eight bf16 values per thread and step, grid-stride; the tail (n % 8) by the
// first threads one value each. With REPORT, each wave adds its counts of
// flagged values to report[0] (inexact) and report[1] (overflow) with one
// vector atomic add per counter: integer sums, so the totals do not depend on
// the order of the adds.
template <bool REPORT>
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint4* __restrict__ src, int64_t n8,
                                                          uint4* __restrict__ dst, const uint16_t* __restrict__ src_tail,
                                                          int tail, uint16_t* __restrict__ dst_tail,
                                                          unsigned long long* __restrict__ report) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t n_inexact = 0, n_over = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 v = src[i];
    const uint4 o = bf16x8_to_f16x8(v);
    dst[i] = o;
    if constexpr (REPORT) {
      const uint32_t in[4] = {v.x, v.y, v.z, v.w}, out[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f16x2 h = __builtin_bit_cast(f16x2, out[w]);
        const int f0 = f16_rounding_flags(__uint_as_float(in[w] << 16), h[0]);
        const int f1 = f16_rounding_flags(__uint_as_float(in[w] & 0xffff0000u), h[1]);
        n_inexact += (f0 & 1) + (f1 & 1);
        n_over += (f0 >> 1) + (f1 >> 1);
      }
    }
  }
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < tail) {
    const float f = bf16_to_f32(src_tail[t]);
    const _Float16 h = static_cast<_Float16>(f);
    dst_tail[t] = __builtin_bit_cast(uint16_t, h);
    if constexpr (REPORT) {
      const int fl = f16_rounding_flags(f, h);
      n_inexact += fl & 1;
      n_over += fl >> 1;
    }
  }
  if constexpr (REPORT) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      n_inexact += __shfl_xor(n_inexact, o, kWave);
      n_over += __shfl_xor(n_over, o, kWave);
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
      if (n_inexact) atomicAdd(&report[0], static_cast<unsigned long long>(n_inexact));
      if (n_over) atomicAdd(&report[1], static_cast<unsigned long long>(n_over));
    }
  }
}

__global__ void clear_report_kernel(unsigned long long* __restrict__ report) {
  if (threadIdx.x < 2) report[threadIdx.x] = 0ull;
}

}  // namespace

hipError_t launch_bf16_to_f16(const void* src, int64_t n, void* dst, uint64_t* report, hipStream_t s) {
  if (report != nullptr) {
    hipLaunchKernelGGL(clear_report_kernel, dim3(1), dim3(kWave), 0, s,
                       reinterpret_cast<unsigned long long*>(report));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n <= 0) return hipSuccess;
  const int64_t n8 = n / 8;
  int64_t g = (n8 + 255) / 256;
  g = g < 1 ? 1 : (g > 8192 ? 8192 : g);
  auto* kern = report != nullptr ? bf16_to_f16_kernel<true> : bf16_to_f16_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(g)), dim3(256), 0, s,
                     static_cast<const uint4*>(src), n8, static_cast<uint4*>(dst),
                     static_cast<const uint16_t*>(src) + n8 * 8, static_cast<int>(n - n8 * 8),
                     static_cast<uint16_t*>(dst) + n8 * 8, reinterpret_cast<unsigned long long*>(report));
  return hipGetLastError();
}

hipError_t launch_down_f16w(const void* h, const int32_t* offsets, int E, int64_t rows_max, int64_t d,
                            int64_t d_ff, const void* w2_f16, float* y_perm, void* ws, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  return launch_gemm_mfma(GemmKind::kDownF16, h, offsets, E, rows_max, 0, static_cast<int>(d),
                          static_cast<int>(d_ff), w2_f16, y_perm, nullptr, ws, s);
}

size_t ffn_workspace_bytes(int dtype) { return dtype == 1 ? ffn_mfma_workspace_bytes() : 0; }

}  // namespace moe

// Weighted combine and auxiliary load-balance loss.
//
// Combine (EP tutorial "专家并行：混合专家模型的分布式训练方案", section 2.1
// step 5: expert outputs return to their tokens' original positions; section
// 2.2: a dropped assignment takes no part): written in gather form -- each
// output row reads its <= k grouped rows, weights them and sums in slot order
// -- so it needs no atomics and no zero-fill pass and is deterministic.
//
// Aux loss (same tutorial, section 5.1): L = alpha * E * sum_i f_i * P_i with
// f_i = counts_i / (T k) and P_i the mean gate probability of expert i. The
// column sums of probs run in double, in a fixed two-level order.
#include "moe_internal.h"

namespace moe {
namespace {

// tpw token rows per workgroup (grid-stride over groups of tpw), 256 / tpw
// threads per row, float4 lanes over d: rows of fewer than 1024 float4 share
// a workgroup, so that each thread still has U columns of loads in flight.
// Each thread takes U float4 columns per step and issues all their loads
// (U x KM rows) before it sums, so several round trips to memory overlap. KM
// >= k bounds the slots held in registers (2 for top-1/top-2, else kMaxK).
template <bool BF16_OUT, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ topk_w, int64_t T,
                                                      int k, int64_t d, void* __restrict__ y, int tpw) {
  constexpr int U = KM <= 2 ? 4 : 1;
  const int64_t dv = d / 4;
  const int tpt = static_cast<int>(blockDim.x) / tpw;   // threads per token row
  const int ts = static_cast<int>(threadIdx.x) / tpt, tl = static_cast<int>(threadIdx.x) % tpt;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * tpw + ts; t < T; t += static_cast<int64_t>(gridDim.x) * tpw) {
    int32_t rows[KM];
    float w[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      rows[j] = j < k ? dest[t * k + j] : -1;
      w[j] = j < k ? topk_w[t * k + j] : 0.f;
    }
    for (int64_t v0 = tl; v0 < dv; v0 += U * static_cast<int64_t>(tpt)) {
      float4 o[U][KM];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + static_cast<int64_t>(u) * tpt;
#pragma unroll
        for (int j = 0; j < KM; ++j)
          o[u][j] = (v < dv && rows[j] >= 0)
                        ? reinterpret_cast<const float4*>(y_perm + static_cast<int64_t>(rows[j]) * d)[v]
                        : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + static_cast<int64_t>(u) * tpt;
        if (v >= dv) break;
        // Slot order; a dropped slot is skipped (not added as zero).
        float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (rows[j] >= 0) {
            acc.x = fmaf(w[j], o[u][j].x, acc.x);
            acc.y = fmaf(w[j], o[u][j].y, acc.y);
            acc.z = fmaf(w[j], o[u][j].z, acc.z);
            acc.w = fmaf(w[j], o[u][j].w, acc.w);
          }
        }
        if (BF16_OUT) {
          ushort4 bb;
          bb.x = f32_to_bf16(acc.x); bb.y = f32_to_bf16(acc.y);
          bb.z = f32_to_bf16(acc.z); bb.w = f32_to_bf16(acc.w);
          reinterpret_cast<ushort4*>(static_cast<uint16_t*>(y) + t * d)[v] = bb;
        } else {
          reinterpret_cast<float4*>(static_cast<float*>(y) + t * d)[v] = acc;
        }
      }
    }
  }
}

constexpr int kAuxBlocks = 256;    // partial-sum workgroups
constexpr int kAuxThreads = 256;

// Partial column sums: workgroup b takes tokens [b*chunk, (b+1)*chunk); thread
// (e = tid % E, g = tid / E) sums tokens t = g, g + G, ... of the chunk; the
// G per-thread sums are then added in g order. Fixed order -> deterministic.
// SQUARE: sums of squares (the z-loss).
template <bool SQUARE>
__global__ __launch_bounds__(kAuxThreads) void aux_partial_kernel(const float* __restrict__ probs,
                                                                  int64_t T, int E, int64_t chunk,
                                                                  double* __restrict__ part) {
  __shared__ double s[kAuxThreads];
  const int tid = threadIdx.x;
  const int G = kAuxThreads / E;   // E <= 256 -> G >= 1
  const int e = tid % E, g = tid / E;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t t1 = min(t0 + chunk, T);
  double acc = 0.0;
  if (g < G) {
    // Eight rows' loads in flight at a time (rows past the chunk re-read its
    // last row and are not added); the sum still runs in row order.
    constexpr int U = 8;
    for (int64_t tb = t0 + g; tb < t1; tb += static_cast<int64_t>(U) * G) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = probs[min(tb + static_cast<int64_t>(u) * G, t1 - 1) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (tb + static_cast<int64_t>(u) * G < t1) {
          const double x = static_cast<double>(v[u]);
          acc += SQUARE ? x * x : x;
        }
      }
    }
  }
  s[tid] = acc;
  __syncthreads();
  if (tid < E) {
    double tot = 0.0;
    for (int gg = 0; gg < G; ++gg) tot += s[gg * E + tid];
    part[static_cast<int64_t>(blockIdx.x) * E + tid] = tot;
  }
}

__global__ __launch_bounds__(kMaxE) void aux_final_kernel(const double* __restrict__ part,
                                                          int nblocks,
                                                          const int32_t* __restrict__ counts,
                                                          int64_t T, int E, int k, float alpha,
                                                          float* __restrict__ loss) {
  __shared__ double s[kMaxE];
  __shared__ double g_part[kMaxE];
  const int tid = threadIdx.x;
  // Thread (e = tid % E, g = tid / E) adds partials b = g, g + G, ...; the G
  // group sums of each expert are then added in g order.
  const int G = kMaxE / E;
  const int e_t = tid % E, g_t = tid / E;
  double acc = 0.0;
  if (g_t < G) {
    // Eight partials in flight at a time, added in block order.
    constexpr int U = 8;
    for (int b0 = g_t; b0 < nblocks; b0 += U * G) {
      double v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = part[static_cast<int64_t>(min(b0 + u * G, nblocks - 1)) * E + e_t];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b0 + u * G < nblocks) acc += v[u];
    }
  }
  g_part[tid] = acc;
  __syncthreads();
  const int e = tid;
  double term = 0.0;
  if (e < E && T > 0) {
    double col = 0.0;
    for (int g = 0; g < G; ++g) col += g_part[g * E + e];
    const double P = col / static_cast<double>(T);
    const double f = static_cast<double>(counts[e]) / (static_cast<double>(T) * k);
    term = f * P;
  }
  __syncthreads();
  s[e] = term;
  __syncthreads();
  for (int o = kMaxE / 2; o > 0; o >>= 1) {
    if (e < o) s[e] += s[e + o];
    __syncthreads();
  }
  if (e == 0) loss[0] = static_cast<float>(static_cast<double>(alpha) * E * s[0]);
}

// Router z-loss: the per-block partial sums of lse^2 come from
// aux_partial_kernel<true> with E = 1; this adds them in block order.
__global__ __launch_bounds__(kMaxE) void z_final_kernel(const double* __restrict__ part,
                                                        int nblocks, int64_t T, float coeff,
                                                        float* __restrict__ loss) {
  __shared__ double s[kMaxE];
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int b = tid; b < nblocks; b += kMaxE) acc += part[b];   // b = tid, tid + 256, ...
  s[tid] = acc;
  __syncthreads();
  for (int o = kMaxE / 2; o > 0; o >>= 1) {
    if (tid < o) s[tid] += s[tid + o];
    __syncthreads();
  }
  if (tid == 0) loss[0] = T > 0 ? static_cast<float>(static_cast<double>(coeff) * s[0] / static_cast<double>(T)) : 0.f;
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* dest, const float* topk_w, int64_t T,
                          int k, int64_t d, void* y, int out_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // token rows per workgroup: enough that a row of d / 4 float4 gives each of
  // its threads four columns (1 at d >= 4096, 4 at d = 1024), at most 32
  int tpw = 1;
  while (tpw < 32 && static_cast<int64_t>(256 / (2 * tpw)) * 4 >= d / 4) tpw *= 2;
  const int64_t groups = (T + tpw - 1) / tpw;
  const int64_t grid = groups < 65536 ? groups : 65536;
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  if (k <= 2) {
    if (out_dtype == 1) hipLaunchKernelGGL((combine_kernel<true, 2>), g, b, 0, s, y_perm, dest, topk_w, T, k, d, y, tpw);
    else hipLaunchKernelGGL((combine_kernel<false, 2>), g, b, 0, s, y_perm, dest, topk_w, T, k, d, y, tpw);
  } else {
    if (out_dtype == 1)
      hipLaunchKernelGGL((combine_kernel<true, kMaxK>), g, b, 0, s, y_perm, dest, topk_w, T, k, d, y, tpw);
    else hipLaunchKernelGGL((combine_kernel<false, kMaxK>), g, b, 0, s, y_perm, dest, topk_w, T, k, d, y, tpw);
  }
  return hipGetLastError();
}

size_t aux_ws_doubles(int64_t T, int E) {
  (void)T;
  return static_cast<size_t>(kAuxBlocks) * E;
}

hipError_t launch_aux_final_chunks(const double* colsum, int nchunks, const int32_t* counts, int64_t T, int E,
                                   int k, float alpha, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(kMaxE), 0, s, colsum, nchunks, counts, T, E, k, alpha, loss);
  return hipGetLastError();
}

hipError_t launch_aux_loss(const float* probs, const int32_t* counts, int64_t T, int E, int k,
                           float alpha, float* loss, double* ws, hipStream_t s) {
  int nblocks = 0;
  if (T > 0) {
    const int64_t chunk = (T + kAuxBlocks - 1) / kAuxBlocks;
    nblocks = static_cast<int>((T + chunk - 1) / chunk);
    hipLaunchKernelGGL(aux_partial_kernel<false>, dim3(nblocks), dim3(kAuxThreads), 0, s, probs, T, E,
                       chunk, ws);
  }
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(kMaxE), 0, s, ws, nblocks, counts, T, E, k,
                     alpha, loss);
  return hipGetLastError();
}

size_t z_ws_doubles(int64_t T) {
  (void)T;
  return static_cast<size_t>(kAuxBlocks);
}

hipError_t launch_z_loss(const float* lse, int64_t T, float coeff, float* loss, double* ws,
                         hipStream_t s) {
  int nblocks = 0;
  if (T > 0) {
    const int64_t chunk = (T + kAuxBlocks - 1) / kAuxBlocks;
    nblocks = static_cast<int>((T + chunk - 1) / chunk);
    hipLaunchKernelGGL(aux_partial_kernel<true>, dim3(nblocks), dim3(kAuxThreads), 0, s, lse, T, 1,
                       chunk, ws);
  }
  hipLaunchKernelGGL(z_final_kernel, dim3(1), dim3(kMaxE), 0, s, ws, nblocks, T, coeff, loss);
  return hipGetLastError();
}

}  // namespace moe

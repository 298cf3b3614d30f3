// Capacity-limited dispatch plan and permute (EP tutorial "专家并行：混合专家
// 模型的分布式训练方案", section 2.1 step 2: build the dispatch plan from the
// target expert indices; section 2.2: capacity = round(T/E x cf), extra tokens
// dropped; section 5.3: pack and sort tokens so each expert's data is
// contiguous).
//
// Integer work, bit-exact and deterministic (no atomics on outputs):
//   1. hist   one workgroup per 256-token chunk. Each wave builds, per expert,
//             a 64-bit mask of its lanes (tokens) that chose the expert
//             (LDS atomicOr -- order-free); the chunk count per expert is the
//             sum of popcounts.
//   2. scan   per expert, an exclusive scan of the chunk counts over chunks
//             (token order), the total count, kept = min(count, C) and the
//             exclusive scan over experts -> offsets. While all chunk counts
//             fit in 64 KiB of LDS (chunks x experts <= 16384: every workload
//             here), each place workgroup does this itself from the counts it
//             loads whole, and workgroup 0 writes counts and offsets -- no
//             launch of its own; beyond that, one scan workgroup.
//   3. place  same masks again; an assignment's position inside its expert is
//             chunk base + earlier waves' popcounts + popcount of lower lanes.
//             Kept iff position < C. dest and src follow.
//   4. gather x_perm[r] = x[src[r]] with 16-byte vector copies.
// The aux loss (EP tutorial 5.1, L = alpha E sum_i f_i P_i) can ride along
// (moe_dispatch_plan_aux): the histogram workgroups also add up their chunk's
// softmax columns in double, in token order, and place workgroup 0 adds those
// chunk sums in chunk order and forms L from them and the counts.
// moe_dispatch_plan_tiles skips step 1: the bf16 router already counted each
// of its token tiles' choices per expert (and summed the tile's softmax
// columns), so one place launch scans those rows instead.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = kDispatchTok;   // one token per thread
constexpr int kWaves = kThreads / kWave;

// Expert of slot j of token t, or -1 when out of range or already named by an
// earlier slot of the same token.
__device__ __forceinline__ int slot_expert(const int32_t* __restrict__ idx, int64_t t, int k,
                                           int j, int E) {
  const int e = idx[t * k + j];
  if (e < 0 || e >= E) return -1;
  for (int jj = 0; jj < j; ++jj)
    if (idx[t * k + jj] == e) return -1;
  return e;
}

__device__ void build_masks(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                            unsigned long long (*mask)[kMaxE]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kWaves * kMaxE; i += kThreads) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = slot_expert(idx, t, k, j, E);
      if (e >= 0) atomicOr(&mask[wave][e], 1ull << lane);
    }
  }
  __syncthreads();
}

// With probs (the aux loss): colsum[chunk, e] = sum over the chunk's tokens
// of probs[t, e] in double, in a fixed order. When 4 divides E and E divides
// 1024, thread (q = tid % (E/4), r = tid / (E/4)) reads experts 4q .. 4q+3 of
// tokens r, r + R, ... (R = 1024 / E) as float4 loads, eight in flight, and
// the R partial sums of each expert are then added in r order; otherwise
// thread (e = tid % E, g = tid / E) adds tokens g, g + G, ... one value at a
// time and the G sums are added in g order.
template <bool AUX>
__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx,
                                                        int64_t T, int k, int E,
                                                        int32_t* __restrict__ chunk_cnt,
                                                        const float* __restrict__ probs,
                                                        double* __restrict__ colsum) {
  __shared__ unsigned long long mask[kWaves][kMaxE];
  if constexpr (AUX) {
    // the loads of this chunk's probabilities are issued first, so that they
    // are in flight while the masks are built
    __shared__ double s_sum[4 * kThreads];
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kThreads;
    const int64_t t1 = min(t0 + kThreads, T);
    constexpr int U = 8;
    const bool vec = (E % 4) == 0 && (1024 % E) == 0;
    int rows;   // partial sums per expert in s_sum, added in row order
    if (vec) {
      const int EQ = E / 4, q = tid % EQ, r = tid / EQ;
      rows = kThreads / EQ;
      double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
      for (int64_t tb = t0 + r; tb < t1; tb += static_cast<int64_t>(U) * rows) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          v[u] = *reinterpret_cast<const float4*>(probs + min(tb + static_cast<int64_t>(u) * rows, t1 - 1) * E + 4 * q);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (tb + static_cast<int64_t>(u) * rows < t1) {
            a0 += static_cast<double>(v[u].x);
            a1 += static_cast<double>(v[u].y);
            a2 += static_cast<double>(v[u].z);
            a3 += static_cast<double>(v[u].w);
          }
        }
      }
      s_sum[r * E + 4 * q] = a0;
      s_sum[r * E + 4 * q + 1] = a1;
      s_sum[r * E + 4 * q + 2] = a2;
      s_sum[r * E + 4 * q + 3] = a3;
    } else {
      const int G = kThreads / E;   // E <= 256 -> G >= 1
      const int e = tid % E, g = tid / E;
      rows = G;
      double acc = 0.0;
      if (g < G) {
        for (int64_t tb = t0 + g; tb < t1; tb += static_cast<int64_t>(U) * G) {
          float v[U];
#pragma unroll
          for (int u = 0; u < U; ++u) v[u] = probs[min(tb + static_cast<int64_t>(u) * G, t1 - 1) * E + e];
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (tb + static_cast<int64_t>(u) * G < t1) acc += static_cast<double>(v[u]);
        }
        s_sum[g * E + e] = acc;
      }
    }
    build_masks(idx, T, k, E, mask);   // its barriers also order s_sum
    if (tid < E) {
      double tot = 0.0;
      for (int rr = 0; rr < rows; ++rr) tot += s_sum[rr * E + tid];
      colsum[static_cast<int64_t>(blockIdx.x) * E + tid] = tot;
    }
  } else {
    build_masks(idx, T, k, E, mask);
  }
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c += __popcll(mask[w][e]);
    chunk_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = c;
  }
}

__global__ __launch_bounds__(kMaxE) void scan_kernel(const int32_t* __restrict__ chunk_cnt,
                                                     int32_t* __restrict__ chunk_base,
                                                     int nchunks, int E, int64_t cap,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int32_t buf[2][kMaxE];
  const int e = threadIdx.x;
  int32_t kept = 0;
  if (e < E) {
    // Eight chunks' counts in flight at a time, scanned in chunk order.
    constexpr int U = 8;
    int32_t run = 0;
    for (int b0 = 0; b0 < nchunks; b0 += U) {
      int32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        c[u] = b0 + u < nchunks ? chunk_cnt[static_cast<int64_t>(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + u < nchunks) chunk_base[static_cast<int64_t>(b0 + u) * E + e] = run;
        run += c[u];
      }
    }
    counts[e] = run;
    kept = (cap < 0 || run < cap) ? run : static_cast<int32_t>(cap);
  }
  // Inclusive Hillis-Steele scan of kept over experts, then shift to exclusive.
  int cur = 0;
  buf[0][e] = kept;
  __syncthreads();
  for (int o = 1; o < kMaxE; o <<= 1) {
    int v = buf[cur][e];
    if (e >= o) v += buf[cur][e - o];
    buf[cur ^ 1][e] = v;
    cur ^= 1;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = buf[cur][e];
  if (e == 0) offsets[0] = 0;
}

__global__ __launch_bounds__(kThreads) void place_kernel(const int32_t* __restrict__ idx,
                                                         int64_t T, int k, int E, int64_t cap,
                                                         const int32_t* __restrict__ chunk_base,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ dest,
                                                         int32_t* __restrict__ src) {
  __shared__ unsigned long long mask[kWaves][kMaxE];
  build_masks(idx, T, k, E, mask);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int e = slot_expert(idx, t, k, j, E);
    int32_t out = -1;
    if (e >= 0) {
      int64_t pos = chunk_base[static_cast<int64_t>(blockIdx.x) * E + e];
      for (int w = 0; w < wave; ++w) pos += __popcll(mask[w][e]);
      pos += __popcll(mask[wave][e] & below);
      if (cap < 0 || pos < cap) {
        out = offsets[e] + static_cast<int32_t>(pos);
        src[out] = static_cast<int32_t>(t);
      }
    }
    dest[t * k + j] = out;
  }
}

// place with the scan folded in (count rows x experts <= kScanLds): every
// workgroup loads all count rows into LDS, scans them for its own chunk's
// bases and for the offsets; workgroup 0 writes counts and offsets. With AUX
// the launch has one more workgroup (index nchunks, no tokens of its own)
// that forms the aux loss from the rows' column sums and the totals, so that
// its column-sum loads do not hold up a place workgroup. A count row covers
// kThreads / tpc tokens: the histogram's chunks (tpc = 1) or the router's
// token tiles (tpc = kThreads / tile tokens), so chunk c starts at row c tpc.
constexpr int kScanLds = 16384;
template <bool AUX>
__global__ __launch_bounds__(kThreads) void place_scan_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, int64_t cap, int nchunks, int tpc,
    const int32_t* __restrict__ chunk_cnt, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ dest, int32_t* __restrict__ src, const double* __restrict__ colsum,
    float alpha, float* __restrict__ loss) {
  __shared__ unsigned long long mask[kWaves][kMaxE];
  __shared__ int32_t s_cnt[kScanLds];
  __shared__ int32_t s_base[kMaxE];
  __shared__ int32_t s_buf[2][kMaxE];
  __shared__ int32_t s_part[2][kThreads];
  __shared__ double s_red[kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = nchunks * E;
  const int place_wgs = static_cast<int>((T + kThreads - 1) / kThreads);
  const bool aux_wg = AUX && static_cast<int>(blockIdx.x) == place_wgs;
  // The aux workgroup adds up the column sums first, so those loads overlap
  // the count loads: thread (ee = tid % E, g = tid / E) adds the rows g,
  // g + G, ... of expert ee in order, sixteen in flight, thirty-two when it
  // has more than sixteen rows (64 experts x 256 token tiles: two rounds
  // instead of four); the G group sums are added in g order below.
  double part = 0.0;
  if constexpr (AUX) {
    const int G = kThreads / E;
    const int ee = tid % E, g = tid / E;
    auto add_rows = [&](auto u_c) {
      constexpr int U = decltype(u_c)::value;
      for (int c0 = g; c0 < nchunks; c0 += U * G) {
        double v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = colsum[static_cast<int64_t>(min(c0 + u * G, nchunks - 1)) * E + ee];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (c0 + u * G < nchunks) part += v[u];
      }
    };
    if (aux_wg && g < G) {
      if (nchunks > 16 * G) add_rows(std::integral_constant<int, 32>{});
      else add_rows(std::integral_constant<int, 16>{});
    }
  }
  // all chunk counts, 16 bytes per load where the count is a multiple of 4,
  // sixteen loads in flight per thread before they go to LDS
  if ((n & 3) == 0) {
    const int4* c4 = reinterpret_cast<const int4*>(chunk_cnt);
    const int n4 = n / 4;
    constexpr int UL = 16;
    for (int i0 = tid; i0 < n4; i0 += kThreads * UL) {
      int4 v[UL];
#pragma unroll
      for (int u = 0; u < UL; ++u) v[u] = c4[min(i0 + u * kThreads, n4 - 1)];
#pragma unroll
      for (int u = 0; u < UL; ++u)
        if (i0 + u * kThreads < n4) reinterpret_cast<int4*>(s_cnt)[i0 + u * kThreads] = v[u];
    }
  } else {
    for (int i = tid; i < n; i += kThreads) s_cnt[i] = chunk_cnt[i];
  }
  build_masks(idx, T, k, E, mask);   // its barriers also publish s_cnt
  // Per expert, the rows before this chunk's first (its base) and all rows
  // (the total): thread (ee = tid % E, g = tid / E) adds rows g, g + G, ...,
  // and the G partial sums meet in LDS (integer sums: any order is exact).
  const int c0 = blockIdx.x * tpc;
  {
    const int G = kThreads / E, ee = tid % E, g = tid / E;
    int32_t pre = 0, tot = 0;
    if (g < G) {
      for (int cc = g; cc < nchunks; cc += G) {
        const int32_t v = s_cnt[cc * E + ee];
        tot += v;
        pre += cc < c0 ? v : 0;
      }
    }
    s_part[0][tid] = pre;
    s_part[1][tid] = tot;
  }
  __syncthreads();
  int32_t kept = 0, total = 0;
  if (tid < E) {
    const int G = kThreads / E;
    int32_t base = 0;
    for (int g = 0; g < G; ++g) {
      base += s_part[0][g * E + tid];
      total += s_part[1][g * E + tid];
    }
    s_base[tid] = base;
    kept = (cap < 0 || total < cap) ? total : static_cast<int32_t>(cap);
  }
  // inclusive scan of kept over experts (Hillis-Steele), then exclusive
  const int e = tid;
  int cur = 0;
  if (e < kMaxE) s_buf[0][e] = kept;
  __syncthreads();
  for (int o = 1; o < kMaxE; o <<= 1) {
    int v = 0;
    if (e < kMaxE) {
      v = s_buf[cur][e];
      if (e >= o) v += s_buf[cur][e - o];
      s_buf[cur ^ 1][e] = v;
    }
    cur ^= 1;
    __syncthreads();
  }
  // offsets[e] = s_buf[cur][e - 1] (0 for e = 0)
  if (blockIdx.x == 0) {
    if (e < E) {
      counts[e] = total;
      offsets[e + 1] = s_buf[cur][e];
    }
    if (e == 0) offsets[0] = 0;
  }
  if (aux_wg) {
    if constexpr (AUX) {
      double term = 0.0;
      const int G = kThreads / E;
      s_red[tid] = part;
      __syncthreads();
      if (e < E && T > 0) {
        double col = 0.0;
        for (int gg = 0; gg < G; ++gg) col += s_red[gg * E + e];
        const double P = col / static_cast<double>(T);
        const double f = static_cast<double>(total) / (static_cast<double>(T) * k);
        term = f * P;
      }
      __syncthreads();
      s_red[e] = term;
      __syncthreads();
      for (int o = kMaxE / 2; o > 0; o >>= 1) {
        if (e < o) s_red[e] += s_red[e + o];
        __syncthreads();
      }
      if (e == 0) loss[0] = static_cast<float>(static_cast<double>(alpha) * E * s_red[0]);
    }
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int ej = slot_expert(idx, t, k, j, E);
    int32_t out = -1;
    if (ej >= 0) {
      int64_t pos = s_base[ej];
      for (int w = 0; w < wave; ++w) pos += __popcll(mask[w][ej]);
      pos += __popcll(mask[wave][ej] & below);
      if (cap < 0 || pos < cap) {
        out = (ej == 0 ? 0 : s_buf[cur][ej - 1]) + static_cast<int32_t>(pos);
        src[out] = static_cast<int32_t>(t);
      }
    }
    dest[t * k + j] = out;
  }
}

// One workgroup per grouped row (grid-stride); 16-byte lanes.
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x,
                                                     const int32_t* __restrict__ src,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int64_t row_vecs, uint4* __restrict__ x_perm) {
  const int64_t R = offsets[E];
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const int64_t s = src[r];
    const uint4* in = x + s * row_vecs;
    uint4* out = x_perm + r * row_vecs;
    for (int64_t v = threadIdx.x; v < row_vecs; v += blockDim.x) out[v] = in[v];
  }
}

__global__ void zero_kernel(int32_t* __restrict__ a, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a[i] = 0;
}

}  // namespace

size_t dispatch_ws_ints(int64_t T, int E) {
  const int64_t nchunks = (T + kThreads - 1) / kThreads;
  return static_cast<size_t>(2 * nchunks * E);
}

namespace {

__global__ void zero_float_kernel(float* __restrict__ a) {
  if (threadIdx.x == 0) a[0] = 0.f;
}

hipError_t plan_impl(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap, int32_t* counts,
                     int32_t* offsets, int32_t* dest, int32_t* src, int32_t* ws, const float* probs,
                     double* colsum, float alpha, float* loss, hipStream_t s) {
  if (T == 0) {
    // Nothing routed: zero counts and offsets so later calls see empty
    // segments (a fill kernel, not a memset node, so the call can be captured).
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(kMaxE), 0, s, counts, E);
    hipLaunchKernelGGL(zero_kernel, dim3(2), dim3(kMaxE), 0, s, offsets, E + 1);
    if (loss != nullptr) hipLaunchKernelGGL(zero_float_kernel, dim3(1), dim3(kWave), 0, s, loss);
    return hipGetLastError();
  }
  const int nchunks = static_cast<int>((T + kThreads - 1) / kThreads);
  int32_t* chunk_cnt = ws;
  const bool aux = probs != nullptr;
  if (aux)
    hipLaunchKernelGGL(hist_kernel<true>, dim3(nchunks), dim3(kThreads), 0, s, topk_idx, T, k, E, chunk_cnt,
                       probs, colsum);
  else
    hipLaunchKernelGGL(hist_kernel<false>, dim3(nchunks), dim3(kThreads), 0, s, topk_idx, T, k, E, chunk_cnt,
                       nullptr, nullptr);
  if (static_cast<int64_t>(nchunks) * E <= kScanLds) {
    if (aux)
      hipLaunchKernelGGL(place_scan_kernel<true>, dim3(nchunks + 1), dim3(kThreads), 0, s, topk_idx, T, k, E, cap,
                         nchunks, 1, chunk_cnt, counts, offsets, dest, src, colsum, alpha, loss);
    else
      hipLaunchKernelGGL(place_scan_kernel<false>, dim3(nchunks), dim3(kThreads), 0, s, topk_idx, T, k, E, cap,
                         nchunks, 1, chunk_cnt, counts, offsets, dest, src, nullptr, 0.f, nullptr);
    return hipGetLastError();
  }
  int32_t* chunk_base = ws + static_cast<int64_t>(nchunks) * E;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kMaxE), 0, s, chunk_cnt, chunk_base, nchunks, E,
                     cap, counts, offsets);
  hipLaunchKernelGGL(place_kernel, dim3(nchunks), dim3(kThreads), 0, s, topk_idx, T, k, E, cap,
                     chunk_base, offsets, dest, src);
  if (aux) {
    // the chunk column sums are there already; the aux loss from them
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_aux_final_chunks(colsum, nchunks, counts, T, E, k, alpha, loss, s);
  }
  return hipGetLastError();
}

}  // namespace

size_t dispatch_aux_ws_bytes(int64_t T, int E) {
  const int64_t nchunks = (T + kThreads - 1) / kThreads;
  return dispatch_ws_ints(T, E) * sizeof(int32_t) + static_cast<size_t>(nchunks * E) * sizeof(double);
}

int dispatch_tiles_max() { return kScanLds; }

hipError_t launch_dispatch_plan_tiles(const int32_t* topk_idx, const int32_t* tile_cnt,
                                      const double* tile_colsum, int tile_tokens, int64_t T, int k,
                                      int E, int64_t cap, float alpha, int32_t* counts,
                                      int32_t* offsets, int32_t* dest, int32_t* src, float* loss,
                                      hipStream_t s) {
  if (T == 0) return plan_impl(topk_idx, T, k, E, cap, counts, offsets, dest, src, nullptr, nullptr, nullptr,
                               alpha, loss, s);
  if (tile_tokens < 1 || kThreads % tile_tokens != 0) return hipErrorInvalidValue;
  const int nchunks = static_cast<int>((T + kThreads - 1) / kThreads);
  const int nrows = static_cast<int>((T + tile_tokens - 1) / tile_tokens);
  const int tpc = kThreads / tile_tokens;
  if (tile_colsum != nullptr)
    hipLaunchKernelGGL(place_scan_kernel<true>, dim3(nchunks + 1), dim3(kThreads), 0, s, topk_idx, T, k, E, cap,
                       nrows, tpc, tile_cnt, counts, offsets, dest, src, tile_colsum, alpha, loss);
  else
    hipLaunchKernelGGL(place_scan_kernel<false>, dim3(nchunks), dim3(kThreads), 0, s, topk_idx, T, k, E, cap,
                       nrows, tpc, tile_cnt, counts, offsets, dest, src, nullptr, 0.f, nullptr);
  return hipGetLastError();
}

hipError_t launch_dispatch_plan(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                                int32_t* ws, hipStream_t s) {
  return plan_impl(topk_idx, T, k, E, cap, counts, offsets, dest, src, ws, nullptr, nullptr, 0.f, nullptr, s);
}

hipError_t launch_dispatch_plan_aux(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                    const float* probs, float alpha, int32_t* counts, int32_t* offsets,
                                    int32_t* dest, int32_t* src, float* loss, void* ws, hipStream_t s) {
  // workspace: the plan's ints, then the chunk column sums (8-byte aligned:
  // the plan's part is an even number of ints)
  int32_t* wsi = static_cast<int32_t*>(ws);
  double* colsum = reinterpret_cast<double*>(wsi + dispatch_ws_ints(T, E));
  return plan_impl(topk_idx, T, k, E, cap, counts, offsets, dest, src, wsi, probs, colsum, alpha, loss, s);
}

// Scratch of moe_dispatch_plan_noalloc: the per-chunk counts and bases that
// moe_dispatch_plan keeps in its caller's workspace, here in device memory the
// library holds itself (1 MiB on every GPU it runs on, until the process
// ends). Host code never passes `scratch` itself to a kernel: on the host that
// name stands for a host-side shadow, not a device address. The device
// address of each GPU's copy is looked up once per device (below) and used
// from then on.
constexpr size_t kNoAllocInts = size_t{1} << 18;
static __device__ __align__(256) int32_t scratch[kNoAllocInts];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the GPU that `s` launches on, looked up
// with that device current on the first call for it.
hipError_t noalloc_scratch(hipStream_t s, int32_t** out) {
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocInts * sizeof(int32_t); }

hipError_t launch_dispatch_plan_noalloc(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                        int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                                        hipStream_t s) {
  if (dispatch_ws_ints(T, E) > kNoAllocInts) return hipErrorInvalidValue;   // the C ABI checks first
  int32_t* ws = nullptr;
  if (T > 0) {
    const hipError_t e = noalloc_scratch(s, &ws);
    if (e != hipSuccess) return e;
  }
  // every scratch word the plan reads is written earlier in the same call
  // (chunk counts by the histogram, bases by the scan): nothing to clear
  return launch_dispatch_plan(topk_idx, T, k, E, cap, counts, offsets, dest, src, ws, s);
}

hipError_t launch_permute(const void* x, int64_t d, int elem_bytes, const int32_t* src,
                          const int32_t* offsets, int E, int64_t rows_max, void* x_perm,
                          hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  const int64_t row_vecs = d * elem_bytes / 16;
  const int64_t grid = rows_max < 16384 ? rows_max : 16384;
  hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     static_cast<const uint4*>(x), src, offsets, E, row_vecs,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe

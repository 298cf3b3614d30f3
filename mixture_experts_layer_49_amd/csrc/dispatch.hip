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
//   2. scan   one workgroup: per expert, an exclusive scan of the chunk counts
//             over chunks (token order), the total count, kept = min(count, C)
//             and the exclusive scan over experts -> offsets.
//   3. place  same masks again; an assignment's position inside its expert is
//             chunk base + earlier waves' popcounts + popcount of lower lanes.
//             Kept iff position < C. dest and src follow.
//   4. gather x_perm[r] = x[src[r]] with 16-byte vector copies.
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

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx,
                                                        int64_t T, int k, int E,
                                                        int32_t* __restrict__ chunk_cnt) {
  __shared__ unsigned long long mask[kWaves][kMaxE];
  build_masks(idx, T, k, E, mask);
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

hipError_t launch_dispatch_plan(const int32_t* topk_idx, int64_t T, int k, int E, int64_t cap,
                                int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                                int32_t* ws, hipStream_t s) {
  if (T == 0) {
    // Nothing routed: zero counts and offsets so later calls see empty
    // segments (a fill kernel, not a memset node, so the call can be captured).
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(kMaxE), 0, s, counts, E);
    hipLaunchKernelGGL(zero_kernel, dim3(2), dim3(kMaxE), 0, s, offsets, E + 1);
    return hipGetLastError();
  }
  const int nchunks = static_cast<int>((T + kThreads - 1) / kThreads);
  int32_t* chunk_cnt = ws;
  int32_t* chunk_base = ws + static_cast<int64_t>(nchunks) * E;
  hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(kThreads), 0, s, topk_idx, T, k, E,
                     chunk_cnt);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kMaxE), 0, s, chunk_cnt, chunk_base, nchunks, E,
                     cap, counts, offsets);
  hipLaunchKernelGGL(place_kernel, dim3(nchunks), dim3(kThreads), 0, s, topk_idx, T, k, E, cap,
                     chunk_base, offsets, dest, src);
  return hipGetLastError();
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

// Measurement kernels for the benchmark only (libmoe_bench.so, separate from
// the layer's library): a plain streaming read, the reference that the
// HBM-bound kernels' cold-cache rates are compared with.
//
// probe_clock: one wave reads the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) at its start and again after about
// `ticks` real-time ticks; (clock delta / real delta) * 100 MHz is the
// graphics clock over that interval. Launched right after a kernel, it sees
// the clock that kernel ran at (the power manager moves it on a millisecond
// scale).
//
// probe_stream_read: every byte of [p, p + bytes) is read once with 16-byte
// vector loads, U of them in flight per thread, grid-stride over 16-byte
// chunks; each thread folds what it read into one word (xor) and each
// workgroup writes one word of `sink` (gridDim.x words), so no load is
// optimised away. bytes must be a multiple of 16 and p 16-byte aligned.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int U = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  uint32_t acc = 0;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t s[kThreads];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int t = 0; t < kThreads; ++t) a ^= s[t];
    sink[blockIdx.x] = a;
  }
}

__global__ __launch_bounds__(64) void clock_kernel(unsigned long long* __restrict__ out, int ticks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long r1 = r0;
  // bounded spin: ends after `ticks` real-time ticks or 2^22 rounds
  for (int i = 0; i < (1 << 22) && r1 - r0 < static_cast<unsigned long long>(ticks); ++i) {
    __builtin_amdgcn_s_sleep(2);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// out: device, two uint64 words (shader-clock ticks, 100 MHz ticks).
int probe_clock(unsigned long long* out, int ticks, hipStream_t stream) {
  if (out == nullptr || ticks < 1) return -1;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, stream, out, ticks);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Returns 0 on success, -1 on bad arguments, -5 when the launch failed.
// sink: device, at least `grid` uint32 words.
int probe_stream_read(const void* p, int64_t bytes, uint32_t* sink, int grid, hipStream_t stream) {
  if (bytes <= 0 || (bytes & 15) != 0 || grid < 1 || p == nullptr || sink == nullptr ||
      (reinterpret_cast<uintptr_t>(p) & 15u) != 0)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(p), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"

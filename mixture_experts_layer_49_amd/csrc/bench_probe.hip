// Measurement kernels for the benchmark only (libmoe_bench.so, separate from
// the layer's library): a plain streaming read, the reference that the
// HBM-bound kernels' cold-cache rates are compared with; a clock probe; and
// an MFMA-only loop, the reference for the matrix-core-bound kernels.
//
// probe_clock: one wave reads the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) at its start and again after about
// `ticks` real-time ticks; (clock delta / real delta) * 100 MHz is the
// graphics clock over that interval. Launched right after a kernel, it sees
// the clock that kernel ran at (the power manager moves it on a millisecond
// scale).
//
// probe_mfma_loop: the matrix-core ceiling under the power cap. One
// workgroup of four waves per CU; each wave runs `iters` rounds of 16
// independent v_mfma_f32_32x32x16_bf16 on operands held in registers (no
// memory traffic), 16 accumulators of 32 x 32, and writes their sum to `out`
// (grid x 256 floats) so nothing is optimised away. Workgroup 0 also records
// the shader-clock and 100 MHz ticks over its loop in clk[0..1]. Flops per
// launch: grid x 4 x iters x 16 x 32768.
// probe_mfma_loop16: the same with v_mfma_f32_16x16x32_bf16, 64 independent
// accumulators of 16 x 16 (the form the fragment-ordered expert GEMM uses;
// per flop it moves half the accumulator data, and the power cap lets it run
// at a higher clock). Flops per launch: grid x 4 x iters x 64 x 16384.
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t lcg_operand(unsigned s) {
  bf16x8_t v;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s = s * 1664525u + 1013904223u;
    v[i] = static_cast<__bf16>(static_cast<float>((s >> 9) & 0xffffu) * (1.0f / 65536.0f) - 0.5f);
  }
  return v;
}

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters,
                                                        unsigned long long* __restrict__ clk) {
  const unsigned seed = blockIdx.x * 1000u + threadIdx.x * 7u;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = lcg_operand(seed + i);
    b[i] = lcg_operand(seed + 100u + i);
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x16_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], b[(i >> 2) & 3], acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

__global__ __launch_bounds__(256) void mfma_loop16_kernel(float* __restrict__ out, int iters,
                                                          unsigned long long* __restrict__ clk) {
  const unsigned seed = blockIdx.x * 1000u + threadIdx.x * 7u;
  u32x4_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(u32x4_t, lcg_operand(seed + i));
    b[i] = __builtin_bit_cast(u32x4_t, lcg_operand(seed + 100u + i));
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x4_t acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = f32x4_t{};
  for (int it = 0; it < iters; ++it) {
    // wait states between the accumulator writes that set them to zero
    // (placed ahead of the loop) and the first MFMAs reading them
    asm volatile("s_nop 2" ::: "memory");
#pragma unroll
    for (int i = 0; i < 64; ++i)   // accumulate in place (inline assembly: see the expert GEMM)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(a[i & 3]), "v"(b[(i >> 2) & 3]));
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // results complete before they are read
  __builtin_amdgcn_sched_barrier(0);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[i][r];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// out: device, grid x 256 floats; clk: device, two uint64 words. Returns 0,
// -1 on bad arguments, -5 when the launch failed.
int probe_mfma_loop(float* out, int iters, unsigned long long* clk, int grid, hipStream_t stream) {
  if (out == nullptr || clk == nullptr || iters < 1 || grid < 1) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, out, iters, clk);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int probe_mfma_loop16(float* out, int iters, unsigned long long* clk, int grid, hipStream_t stream) {
  if (out == nullptr || clk == nullptr || iters < 1 || grid < 1) return -1;
  hipLaunchKernelGGL(mfma_loop16_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, out, iters, clk);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

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

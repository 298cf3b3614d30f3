// Pieces shared by the grouped expert-FFN kernels: the device-side tile list
// over the expert segments, GELU-tanh and the bf16 -> fp16 conversion.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace ffn {

// s_pref[e] = number of BM-row tiles of experts < e (e = 0..E), from the
// segment bounds offsets[] (device memory); every thread of the block calls.
__device__ inline void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int BM,
                                         int* s_pref, int* s_tmp) {
  const int tid = threadIdx.x;
  for (int e = tid; e < kMaxE; e += blockDim.x) {
    int mt = 0;
    if (e < E) {
      const int rows = offsets[e + 1] - offsets[e];
      mt = (rows + BM - 1) / BM;
    }
    s_tmp[e] = mt;
  }
  __syncthreads();
  // Inclusive scan over kMaxE entries (Hillis-Steele, ping-pong s_tmp/s_pref).
  int* in = s_tmp;
  int* out = s_pref + 1;
  for (int o = 1; o < kMaxE; o <<= 1) {
    for (int e = tid; e < kMaxE; e += blockDim.x) out[e] = in[e] + (e >= o ? in[e - o] : 0);
    __syncthreads();
    int* t = in;
    in = out;
    out = t;
  }
  // 8 steps (even): the result is back in s_tmp.
  for (int e = tid; e < kMaxE; e += blockDim.x) s_pref[e + 1] = in[e];
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
}

struct Tile {
  int e, mi, nt;
};

// Tiles are numbered expert by expert; inside an expert, n-panel by n-panel,
// and inside an n-panel, m-tile by m-tile.
__device__ __forceinline__ Tile find_tile(const int* s_pref, int E, int tiles_n, int64_t id) {
  int lo = 0, hi = E;   // largest e with s_pref[e] * tiles_n <= id
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(s_pref[mid]) * tiles_n <= id) lo = mid;
    else hi = mid;
  }
  const int mt = s_pref[lo + 1] - s_pref[lo];
  const int64_t local = id - static_cast<int64_t>(s_pref[lo]) * tiles_n;
  Tile t;
  t.e = lo;
  t.nt = static_cast<int>(local / mt);
  t.mi = static_cast<int>(local % mt);
  return t;
}

constexpr int kPiecesPerWg = 2;   // split pieces one workgroup may run (workspace slots per workgroup)

// How an XCD's share of a row-segmented tile list runs: tiles r_beg ..
// r_beg + n_x - 1, `full` whole rounds over its P workgroups, then the rem
// tiles left, each split into S k-ranges when the workspace allows it. The
// rem * S pieces go round-robin over the P workgroups, at most kPiecesPerWg
// each, and S is the count that ends the last round soonest: the round
// takes ceil(rem S / P) / S of a tile (ties: fewer pieces). Pieces keep >= 32
// stages when they only fill a last round (measured on 64-stage tiles:
// 2-way splits gain 4-7%); when the whole launch is a partial round, pieces of
// 16 stages still pay.
struct RowPlan {
  int64_t r_beg, n_x, full;
  int rem, S;
};
__device__ __forceinline__ RowPlan row_plan(int64_t total, int xcd, int P, int nk2, int max_split) {
  RowPlan p;
  p.r_beg = total * xcd / 8;
  p.n_x = total * (xcd + 1) / 8 - p.r_beg;
  p.full = p.n_x / P;
  p.rem = static_cast<int>(p.n_x - p.full * P);
  p.S = 1;
  if (p.rem > 0 && max_split > 1) {
    const int smax = min(max_split, nk2 / (p.full == 0 ? 16 : 32));
    int best_num = 1, best_den = 1;   // last round = best_num / best_den tiles
    for (int s = 2; s <= smax; ++s) {
      if (p.rem * s > kPiecesPerWg * P) break;
      const int num = (p.rem * s + P - 1) / P;
      if (num * best_den < best_num * s) {
        best_num = num;
        best_den = s;
      }
    }
    p.S = best_den;
  }
  return p;
}

// gelu_tanh(z) = z/2 (1 + tanh(u)) = z * sigmoid(2u), u = sqrt(2/pi)(z + 0.044715 z^3)
__device__ __forceinline__ float gelu_tanh(float z) {
  const float u = 0.7978845608028654f * fmaf(0.044715f * z, z * z, z);
  return z / (1.0f + __expf(-2.0f * u));
}

// d/dz gelu_tanh(z) = s (1 + 2 z (1 - s) u'), s = sigmoid(2u) = (1 + tanh u) / 2,
// u' = sqrt(2/pi)(1 + 3 * 0.044715 z^2).
__device__ __forceinline__ float gelu_tanh_grad(float z) {
  const float c = 0.7978845608028654f;
  const float u = c * fmaf(0.044715f * z, z * z, z);
  const float s = 1.0f / (1.0f + __expf(-2.0f * u));
  const float du = c * fmaf(3.0f * 0.044715f * z, z, 1.0f);
  return s * fmaf(2.0f * z * (1.0f - s), du, 1.0f);
}

// The same function with hardware exp2 and reciprocal (about 1e-6 relative
// error), for results that are rounded to 16-bit floats anyway.
__device__ __forceinline__ float gelu_tanh_fast(float z) {
  // z sigmoid(2u) = z / (1 + 2^(z (a + b z^2))), a = -2 sqrt(2/pi) log2(e),
  // b = 0.044715 a: seven VALU operations with the constants folded.
  constexpr float a = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float b = 0.044715f * a;
  const float q = z * fmaf(b, z * z, a);
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(q));
}

// gelu_tanh_grad with hardware exp2 and reciprocal.
__device__ __forceinline__ float gelu_tanh_grad_fast(float z) {
  const float c = 0.7978845608028654f;
  const float u = c * fmaf(0.044715f * z, z * z, z);
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * u));
  const float du = c * fmaf(3.0f * 0.044715f * z, z, 1.0f);
  return s * fmaf(2.0f * z * (1.0f - s), du, 1.0f);
}

// Two bf16 values (one 32-bit word) -> two IEEE fp16 values, round to nearest
// even. Exact for every bf16 value inside the fp16 normal range.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  const f16x2 h = {static_cast<_Float16>(__uint_as_float(v << 16)),
                   static_cast<_Float16>(__uint_as_float(v & 0xffff0000u))};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  return uint4{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z),
               bf16x2_to_f16x2(v.w)};
}

// Two fp16 values -> two bf16 values, round to nearest even.
__device__ __forceinline__ uint32_t f16x2_to_bf16x2(uint32_t v) {
  const f16x2 h = __builtin_bit_cast(f16x2, v);
  const bf16x2 b = {static_cast<__bf16>(static_cast<float>(h[0])),
                    static_cast<__bf16>(static_cast<float>(h[1]))};
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint4 f16x8_to_bf16x8(uint4 v) {
  return uint4{f16x2_to_bf16x2(v.x), f16x2_to_bf16x2(v.y), f16x2_to_bf16x2(v.z),
               f16x2_to_bf16x2(v.w)};
}

}  // namespace ffn
}  // namespace moe

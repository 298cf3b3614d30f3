// Backward of the MoE layer (EP tutorial "专家并行：混合专家模型的分布式训练方案",
// section 5.1: the load-balance loss is there for its gradient on the gate;
// the reverse path takes combine, expert FFN, dispatch and the gate in turn).
// This file holds the memory-bound steps and the f32 expert GEMMs:
//   * combine backward: d_out[r] = w[t,j] dy[t] and dw[t,j] = dy[t] . o[r]
//     for every kept slot (r = dest[t,j]);
//   * gate backward: gradient of the gate's linear output from dw, the aux
//     loss and the router z-loss, through the optional renormalisation, the
//     softmax and the temperature;
//   * gate weight gradients dWg = dl^T x and db = sum_t dl, in a fixed order;
//   * dispatch backward: dx[t] = sum_j dx_perm[dest[t,j]] + sum_e dl[t,e] Wg[e];
//   * f32 layers: the four expert GEMMs of the backward on a plain LDS-tiled
//     FMA kernel (bf16 layers run them on gemm_mfma.hip).
// Every reduction runs in a fixed order: results are the same run to run.
#include <type_traits>

#include "ffn_common.h"

namespace moe {
namespace {

using namespace ffn;

constexpr int kThreads = 256;

// Sum over the 256 threads of a workgroup in a fixed order (xor butterfly in
// each wave, then the four wave sums in wave order). Every thread gets it.
__device__ __forceinline__ float block_sum(float v, float* s_red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[wave] = v;
  __syncthreads();
  return ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b) {
  return fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
}

__device__ __forceinline__ float4 scale4(float s, const float4& a) {
  return float4{s * a.x, s * a.y, s * a.z, s * a.w};
}

// Four floats -> the gradient storage of a bf16 layer (bf16, RNE) or f32.
template <bool BF16>
__device__ __forceinline__ void store4(void* base, int64_t i4, const float4& v) {
  if constexpr (BF16) {
    ushort4 b;
    b.x = f32_to_bf16(v.x); b.y = f32_to_bf16(v.y); b.z = f32_to_bf16(v.z); b.w = f32_to_bf16(v.w);
    reinterpret_cast<ushort4*>(base)[i4] = b;
  } else {
    reinterpret_cast<float4*>(base)[i4] = v;
  }
}

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* base, int64_t i4) {
  if constexpr (BF16) {
    const ushort4 b = reinterpret_cast<const ushort4*>(base)[i4];
    return float4{bf16_to_f32(b.x), bf16_to_f32(b.y), bf16_to_f32(b.z), bf16_to_f32(b.w)};
  } else {
    return reinterpret_cast<const float4*>(base)[i4];
  }
}

// ------------------------------------------------------------ combine backward
// One workgroup per token (grid-stride); each thread takes U float4 columns
// per pass with all loads issued before the arithmetic.
template <bool BF16, int KM>
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(
    const float* __restrict__ dy, const float* __restrict__ y_perm,
    const int32_t* __restrict__ dest, const float* __restrict__ topk_w, int64_t T, int k,
    int64_t d, void* __restrict__ d_out, float* __restrict__ dw) {
  constexpr int U = 4;
  __shared__ float s_red[4];
  const int tid = threadIdx.x;
  const int64_t d4 = d >> 2;
  const float4* dy4 = reinterpret_cast<const float4*>(dy);
  const float4* yp4 = reinterpret_cast<const float4*>(y_perm);
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    int64_t r[KM];
    float wt[KM], part[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      r[j] = j < k ? dest[t * k + j] : -1;
      wt[j] = j < k ? topk_w[t * k + j] : 0.f;
      part[j] = 0.f;
    }
    for (int64_t v0 = tid; v0 < d4; v0 += U * kThreads) {
      float4 g[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * kThreads;
        g[u] = v < d4 ? dy4[t * d4 + v] : float4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (r[j] < 0) continue;
        float4 o[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + u * kThreads;
          o[u] = v < d4 ? yp4[r[j] * d4 + v] : float4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + u * kThreads;
          if (v < d4) {
            part[j] += dot4(g[u], o[u]);
            store4<BF16>(d_out, r[j] * d4 + v, scale4(wt[j], g[u]));
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= k) break;
      const float s = block_sum(part[j], s_red);
      if (tid == 0) dw[t * k + j] = r[j] >= 0 ? s : 0.f;
    }
  }
}

// --------------------------------------------------------------- gate backward
// One wave per token; lane q owns experts e = q + 64 i.
constexpr int kGateNT = kMaxE / 64;

__global__ __launch_bounds__(kThreads) void gate_backward_kernel(
    const float* __restrict__ dw, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ probs,
    const int32_t* __restrict__ counts, const float* __restrict__ lse, int64_t T, int E, int k,
    int renorm, float inv_temp, float aux_c, float z_c, float* __restrict__ dl) {
  const int wave = threadIdx.x >> 6, q = threadIdx.x & 63;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave; t < T;
       t += static_cast<int64_t>(gridDim.x) * 4) {
    // Gradient of each chosen expert's probability from its slot weight.
    float g[kMaxK];
    int ex[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      ex[j] = j < k ? topk_idx[t * k + j] : -1;
      g[j] = j < k ? dw[t * k + j] : 0.f;
    }
    if (renorm) {
      float S = 0.f, c = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k && ex[j] >= 0) {
          S += probs[t * E + ex[j]];
          c += g[j] * topk_w[t * k + j];
        }
      }
      const float inv_s = 1.0f / S;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) g[j] = (g[j] - c) * inv_s;
    }
    float p[kGateNT], dp[kGateNT];
    float pdp = 0.f;
#pragma unroll
    for (int i = 0; i < kGateNT; ++i) {
      const int e = q + 64 * i;
      p[i] = 0.f;
      dp[i] = 0.f;
      if (e < E) {
        p[i] = probs[t * E + e];
        float v = aux_c * static_cast<float>(counts[e]);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
          if (j < k && ex[j] == e) v += g[j];
        dp[i] = v;
        pdp = fmaf(p[i], v, pdp);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pdp += __shfl_xor(pdp, o);
    const float zl = z_c != 0.f ? z_c * lse[t] : 0.f;
#pragma unroll
    for (int i = 0; i < kGateNT; ++i) {
      const int e = q + 64 * i;
      if (e < E) dl[t * E + e] = (p[i] * (dp[i] - pdp) + zl * p[i]) * inv_temp;
    }
  }
}

// -------------------------------------------------------- gate weight gradient
// Partial sums over token chunks: workgroup (cb, ch) takes columns
// 256 cb .. +255 and tokens [ch * chunk, (ch + 1) * chunk). Thread (cg, tl):
// columns 4 cg .. +3, tokens tl, tl + 4, ... in 256-token sub-chunks; experts
// 16 at a time. The four token lanes meet in LDS in lane order. Column block 0
// also sums the chunk's dl columns (the bias gradient), in a fixed order.
constexpr int kWgSub = 256;
constexpr int kWgTU = 8;                       // tokens per lane per pass
constexpr int kWgRows = kWgSub + 4 * kWgTU;    // staged dl rows: a pass may run 4 TU - 4 past n
constexpr int kWgE = 16;                       // experts per pass over x

template <bool BF16>
__global__ __launch_bounds__(kThreads) void gate_wgrad_partial_kernel(
    const float* __restrict__ dl, const void* __restrict__ x, int64_t T, int64_t d, int E,
    int64_t chunk, float* __restrict__ part, float* __restrict__ part_b) {
  __shared__ float s_dl[kWgRows][kWgE];   // rows >= n hold zeros
  __shared__ float4 s_red[4][8][64];
  __shared__ float s_bias[kThreads];
  const int tid = threadIdx.x, cg = tid & 63, tl = tid >> 6;
  const int64_t ch = blockIdx.y;
  const int64_t t0 = ch * chunk, t1 = min(t0 + chunk, T);
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 256 + 4 * cg;
  const bool col_ok = c0 < d;
  for (int e0 = 0; e0 < E; e0 += kWgE) {
    float4 acc[kWgE];
    float bsum = 0.f;
#pragma unroll
    for (int e = 0; e < kWgE; ++e) acc[e] = float4{0, 0, 0, 0};
    for (int64_t s0 = t0; s0 < t1; s0 += kWgSub) {
      const int n = static_cast<int>(min<int64_t>(kWgSub, t1 - s0));
      __syncthreads();
      // Thread tid stages expert e0 + (tid % kWgE) of tokens tid / kWgE,
      // + 256 / kWgE, ... and keeps their sum for the bias gradient.
      for (int i = tid; i < kWgRows * kWgE; i += kThreads) {
        const int tt = i / kWgE, e = i % kWgE;
        const float v = (tt < n && e0 + e < E) ? dl[(s0 + tt) * E + e0 + e] : 0.f;
        s_dl[tt][e] = v;
        bsum += v;
      }
      __syncthreads();
      if (col_ok) {
        // Eight of this lane's tokens per pass, their loads issued together.
        constexpr int TU = kWgTU;
        for (int tb = tl; tb < n; tb += 4 * TU) {
          // Raw loads first (clamped to a real token so all eight stay
          // unconditional), converted only once all are in flight.
          using Raw = typename std::conditional<BF16, uint2, float4>::type;
          Raw raw[TU];
#pragma unroll
          for (int u = 0; u < TU; ++u) {
            const int tt = min(tb + 4 * u, n - 1);
            raw[u] = reinterpret_cast<const Raw*>(x)[((s0 + tt) * d + c0) >> 2];
          }
          __builtin_amdgcn_sched_barrier(0);
          float4 xv[TU];
#pragma unroll
          for (int u = 0; u < TU; ++u) {
            if constexpr (BF16)
              xv[u] = float4{__uint_as_float(raw[u].x << 16), __uint_as_float(raw[u].x & 0xffff0000u),
                             __uint_as_float(raw[u].y << 16), __uint_as_float(raw[u].y & 0xffff0000u)};
            else
              xv[u] = raw[u];
          }
          // a token past the chunk has dl = 0 staged (tt < n + 4 TU <= kWgRows),
          // so its clamped stand-in adds exactly zero; no branch splits the loads
#pragma unroll
          for (int u = 0; u < TU; ++u) {
            const int tt = tb + 4 * u;
#pragma unroll
            for (int e = 0; e < kWgE; ++e) {
              const float a = s_dl[tt][e];
              acc[e].x = fmaf(a, xv[u].x, acc[e].x);
              acc[e].y = fmaf(a, xv[u].y, acc[e].y);
              acc[e].z = fmaf(a, xv[u].z, acc[e].z);
              acc[e].w = fmaf(a, xv[u].w, acc[e].w);
            }
          }
        }
      }
    }
    // the four token lanes meet in LDS, eight experts at a time
#pragma unroll
    for (int h = 0; h < kWgE / 8; ++h) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[tl][e][cg] = acc[8 * h + e];
      __syncthreads();
      if (tl == 0 && col_ok) {
        for (int e = 0; e < 8 && e0 + 8 * h + e < E; ++e) {
          const float4 a = s_red[0][e][cg], b = s_red[1][e][cg], c = s_red[2][e][cg], f = s_red[3][e][cg];
          const float4 s = float4{((a.x + b.x) + c.x) + f.x, ((a.y + b.y) + c.y) + f.y,
                                  ((a.z + b.z) + c.z) + f.z, ((a.w + b.w) + c.w) + f.w};
          *reinterpret_cast<float4*>(part + (ch * E + e0 + 8 * h + e) * d + c0) = s;
        }
      }
    }
    // Bias (column block 0): the threads of each expert add up in tid order.
    if (blockIdx.x == 0) {
      s_bias[tid] = bsum;
      __syncthreads();
      if (tid < kWgE && e0 + tid < E) {
        float b = 0.f;
        for (int q = 0; q < kThreads / kWgE; ++q) b += s_bias[tid + kWgE * q];
        part_b[ch * E + e0 + tid] = b;
      }
      __syncthreads();
    }
  }
}

// Wide gates (E > 16): the same partial sums on the f32 matrix cores
// (v_mfma_f32_32x32x2_f32, twice the rate of plain f32 FMAs, products exact as
// with FMAs). Workgroup (cb, ch, eb) takes columns 256 cb .. +255, experts
// 64 eb .. +63 and the tokens of chunk ch; wave w holds the 64 x 64 block of
// experts x columns 256 cb + 64 w .. +63 in four 32 x 32 accumulator tiles.
// Sixteen tokens at a time are staged in LDS (dl as f32, x as stored), the
// next sixteen loaded into registers meanwhile; an MFMA takes two tokens:
// lane l gives dl[t0 + l / 32][e0 + l % 32] and x[t0 + l / 32][c0 + l % 32].
// Column block 0 also sums the chunk's dl columns (the bias gradient) in
// token order.
constexpr int kWgMt = 16;   // tokens per staged block
template <bool BF16>
__global__ __launch_bounds__(kThreads) void gate_wgrad_mfma_kernel(
    const float* __restrict__ dl, const void* __restrict__ x, int64_t T, int64_t d, int E,
    int64_t chunk, float* __restrict__ part, float* __restrict__ part_b) {
  using XT = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int XV = 16 / sizeof(XT);            // x elements per 16-byte load
  constexpr int XL = kWgMt * 256 / XV / kThreads;   // 16-byte x loads per thread per block
  __shared__ float s_dl[2][kWgMt][64];
  __shared__ XT s_x[2][kWgMt][256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t ch = blockIdx.y;
  const int64_t t0 = ch * chunk, t1 = min(t0 + chunk, T);
  const int64_t cb = static_cast<int64_t>(blockIdx.x) * 256;
  const int e0 = blockIdx.z * 64;
  // Registers for the next block: dl token tid / 16, experts 4 (tid % 16) .. +3;
  // x token (tid XL + h) / (256 / XV), columns XV ((tid XL + h) % (256 / XV)) .. .
  float rd[4];
  uint4 rx[XL];
  auto load_block = [&](int64_t tb) {
    const int tt = tid >> 4, eq = 4 * (tid & 15);
    const int64_t t = tb + tt;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + eq + u;
      rd[u] = (t < t1 && e < E) ? dl[t * E + e] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < XL; ++h) {
      const int f = tid * XL + h;
      const int xt = f / (256 / XV), xc = (f % (256 / XV)) * XV;
      const int64_t tx = tb + xt, c = cb + xc;
      rx[h] = (tx < t1 && c < d) ? *reinterpret_cast<const uint4*>(static_cast<const XT*>(x) + tx * d + c)
                                 : uint4{0, 0, 0, 0};
    }
  };
  auto store_block = [&](int buf) {
    const int tt = tid >> 4, eq = 4 * (tid & 15);
#pragma unroll
    for (int u = 0; u < 4; ++u) s_dl[buf][tt][eq + u] = rd[u];
#pragma unroll
    for (int h = 0; h < XL; ++h) {
      const int f = tid * XL + h;
      const int xt = f / (256 / XV), xc = (f % (256 / XV)) * XV;
      *reinterpret_cast<uint4*>(&s_x[buf][xt][xc]) = rx[h];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
  float bsum = 0.f;   // bias: thread tid < 64 sums expert e0 + tid
  const int l32 = lane & 31, hl = lane >> 5;
  int buf = 0;
  if (t0 < t1) {
    load_block(t0);
    store_block(0);
  }
  for (int64_t tb = t0; tb < t1; tb += kWgMt) {
    __syncthreads();   // block tb is in buffer buf; buffer buf ^ 1 is free
    const bool more = tb + kWgMt < t1;
    if (more) load_block(tb + kWgMt);
    if (blockIdx.x == 0 && tid < 64) {
#pragma unroll
      for (int tt = 0; tt < kWgMt; ++tt) bsum += s_dl[buf][tt][tid];
    }
#pragma unroll
    for (int p = 0; p < kWgMt / 2; ++p) {
      const int tt = 2 * p + hl;
      float a[2], b[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) a[mb] = s_dl[buf][tt][32 * mb + l32];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const XT v = s_x[buf][tt][64 * wave + 32 * nb + l32];
        if constexpr (BF16) b[nb] = __uint_as_float(static_cast<uint32_t>(v) << 16);
        else b[nb] = v;
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) store_block(buf ^ 1);
    buf ^= 1;
  }
  // D layout of a 32 x 32 tile: lane l holds column l % 32, rows
  // 8 (r / 4) + 4 (l / 32) + r % 4 in register r.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t c = cb + 64 * wave + 32 * nb + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = e0 + 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (e < E && c < d) part[(ch * E + e) * d + c] = acc[mb][nb][r];
      }
    }
  if (blockIdx.x == 0 && tid < 64 && e0 + tid < E) part_b[ch * E + e0 + tid] = bsum;
}

__global__ __launch_bounds__(kThreads) void gate_wgrad_final_kernel(
    const float* __restrict__ part, const float* __restrict__ part_b, int nch, int64_t d, int E,
    float* __restrict__ dwg, float* __restrict__ db) {
  const int64_t n = static_cast<int64_t>(E) * d;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    // Eight chunks' partials in flight at a time, added in chunk order.
    constexpr int U = 8;
    float s = 0.f;
    for (int c0 = 0; c0 < nch; c0 += U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = part[static_cast<int64_t>(min(c0 + u, nch - 1)) * n + i];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u < nch) s += v[u];
    }
    dwg[i] = s;
  }
  if (blockIdx.x == 0 && db != nullptr) {
    for (int e = threadIdx.x; e < E; e += kThreads) {
      float s = 0.f;
      for (int c = 0; c < nch; ++c) s += part_b[c * E + e];
      db[e] = s;
    }
  }
}

// ----------------------------------------------------------- dispatch backward
template <bool WG_BF16>
__global__ __launch_bounds__(kThreads) void dispatch_backward_kernel(
    const float* __restrict__ dx_perm, const int32_t* __restrict__ dest, const float* __restrict__ dl,
    const void* __restrict__ wg, int64_t T, int k, int64_t d, int E, float* __restrict__ dx) {
  constexpr int U = 4;
  __shared__ float s_dl[kMaxE];
  const int tid = threadIdx.x;
  const int64_t d4 = d >> 2;
  const float4* xp4 = reinterpret_cast<const float4*>(dx_perm);
  const bool gate = dl != nullptr;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    __syncthreads();
    if (gate)
      for (int e = tid; e < E; e += kThreads) s_dl[e] = dl[t * E + e];
    __syncthreads();
    int64_t r[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) r[j] = j < k ? dest[t * k + j] : -1;
    for (int64_t v0 = tid; v0 < d4; v0 += U * kThreads) {
      float4 acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = float4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        if (r[j] < 0) continue;
        float4 o[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + u * kThreads;
          o[u] = v < d4 ? xp4[r[j] * d4 + v] : float4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          acc[u].x += o[u].x; acc[u].y += o[u].y; acc[u].z += o[u].z; acc[u].w += o[u].w;
        }
      }
      if (gate) {
        for (int e = 0; e < E; ++e) {
          const float a = s_dl[e];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * kThreads;
            if (v < d4) {
              const float4 w = load4<WG_BF16>(wg, e * d4 + v);
              acc[u].x = fmaf(a, w.x, acc[u].x);
              acc[u].y = fmaf(a, w.y, acc[u].y);
              acc[u].z = fmaf(a, w.z, acc[u].z);
              acc[u].w = fmaf(a, w.w, acc[u].w);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * kThreads;
        if (v < d4) reinterpret_cast<float4*>(dx)[t * d4 + v] = acc[u];
      }
    }
  }
}

// A thread owns one 4-column group of dx for kDispTok tokens: it sums the
// tokens' kept rows of dx_perm, then adds the gate term 16 experts at a time
// with those experts' gate-weight columns in registers (loaded once for all
// kDispTok tokens). Rows and weights come through range-checked buffer loads,
// so a dropped slot or an expert past E reads zeros without a branch.
constexpr int kDispTok = 16;
constexpr int kDispEChunk = 16;

template <bool WG_BF16, int KM>
__global__ __launch_bounds__(kThreads) void dispatch_backward_tok_kernel(
    const float* __restrict__ dx_perm, const int32_t* __restrict__ dest, const float* __restrict__ dl,
    const void* __restrict__ wg, int64_t T, int k, int64_t d, int E, float* __restrict__ dx) {
  constexpr int TU = KM <= 2 ? 4 : 1;   // tokens whose rows are loaded together
  __shared__ float s_dl[kDispTok][kMaxE];
  __shared__ int s_dest[kDispTok][kMaxK];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kDispTok;
  const bool gate = dl != nullptr;
  const int e_pad = (E + kDispEChunk - 1) / kDispEChunk * kDispEChunk;
  for (int i = tid; i < kDispTok * kMaxK; i += kThreads) {
    const int tt = i / kMaxK, j = i % kMaxK;
    s_dest[tt][j] = (t0 + tt < T && j < k) ? dest[(t0 + tt) * k + j] : -1;
  }
  if (gate)
    for (int i = tid; i < kDispTok * e_pad; i += kThreads) {
      const int tt = i / e_pad, e = i % e_pad;
      s_dl[tt][e] = (t0 + tt < T && e < E) ? dl[(t0 + tt) * E + e] : 0.f;
    }
  __syncthreads();
  const int64_t d4 = d >> 2;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
  if (v >= d4) return;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(dx_perm), 0, 0x7fffffff, 0x00020000);
  float4 acc[kDispTok];
#pragma unroll
  for (int tt0 = 0; tt0 < kDispTok; tt0 += TU) {
    float4 o[TU][KM];
#pragma unroll
    for (int u = 0; u < TU; ++u)
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const int r = s_dest[tt0 + u][j];
        const uint32_t off = r >= 0 ? static_cast<uint32_t>((static_cast<int64_t>(r) * d4 + v) * 16) : 0x80000000u;
        o[u][j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      }
    __builtin_amdgcn_sched_barrier(0);   // the group's loads before its sums
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      float4 a = float4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < KM; ++j)   // slot order; a dropped slot is skipped
        if (s_dest[tt0 + u][j] >= 0) {
          a.x += o[u][j].x; a.y += o[u][j].y; a.z += o[u][j].z; a.w += o[u][j].w;
        }
      acc[tt0 + u] = a;
    }
  }
  if (gate) {
    const int eb = WG_BF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(wg), 0, static_cast<int>(static_cast<int64_t>(E) * d * eb), 0x00020000);
#pragma unroll 1
    for (int e0 = 0; e0 < E; e0 += kDispEChunk) {
      float4 w[kDispEChunk];
#pragma unroll
      for (int e = 0; e < kDispEChunk; ++e) {
        const uint32_t off = static_cast<uint32_t>((static_cast<int64_t>(e0 + e) * d + 4 * v) * eb);
        if constexpr (WG_BF16) {
          const uint2 b = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(wr, off, 0, 0));
          w[e] = float4{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                        __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u)};
        } else {
          w[e] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0));
        }
      }
      // experts past E carry zero weights and zero s_dl: their terms add 0
#pragma unroll
      for (int tt = 0; tt < kDispTok; ++tt)
#pragma unroll
        for (int e = 0; e < kDispEChunk; ++e) {
          const float a = s_dl[tt][e0 + e];
          acc[tt].x = fmaf(a, w[e].x, acc[tt].x);
          acc[tt].y = fmaf(a, w[e].y, acc[tt].y);
          acc[tt].z = fmaf(a, w[e].z, acc[tt].z);
          acc[tt].w = fmaf(a, w[e].w, acc[tt].w);
        }
    }
  }
#pragma unroll
  for (int tt = 0; tt < kDispTok; ++tt)
    if (t0 + tt < T) reinterpret_cast<float4*>(dx)[(t0 + tt) * d4 + v] = acc[tt];
}

// ------------------------------------------------------------ f32 expert GEMMs
// 64 x 64 tiles, 16-deep k steps through LDS, 4 x 4 outputs per thread.
// A and B are each K-contiguous (row pitch K) or k-major (stored [K][M or N]).
// Row-segmented (SEG_K false): rows of A and C are the expert segments of
// offsets[], K fixed, B_e = B + e * K * N. K-segmented: C_e = A_e^T B_e over
// the rows of expert e, C [E, M, N]. EPI: 0 = store, 1 = times gelu'(Z).
constexpr int FM = 64, FN = 64, FK = 16;

template <bool A_KM, bool B_KM, bool SEG_K, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ offsets, int E, int M, int N, int K,
    const float* __restrict__ B, float* __restrict__ C, const float* __restrict__ Z) {
  __shared__ float As[FK][FM + 4];
  __shared__ float Bs[FK][FN + 4];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_tmp[kMaxE];
  const int tiles_n = (N + FN - 1) / FN;
  int64_t total;
  if constexpr (SEG_K) {
    total = static_cast<int64_t>(E) * ((M + FM - 1) / FM) * tiles_n;
  } else {
    build_tile_prefix(offsets, E, FM, s_pref, s_tmp);
    total = static_cast<int64_t>(s_pref[E]) * tiles_n;
  }
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int64_t id = blockIdx.x; id < total; id += gridDim.x) {
    int e, m0, n0, mend, k0r, kn;
    if constexpr (SEG_K) {
      const int tm = (M + FM - 1) / FM;
      e = static_cast<int>(id / (static_cast<int64_t>(tm) * tiles_n));
      const int local = static_cast<int>(id - static_cast<int64_t>(e) * tm * tiles_n);
      m0 = (local / tiles_n) * FM;
      n0 = (local % tiles_n) * FN;
      mend = M;
      k0r = offsets[e];
      kn = offsets[e + 1] - k0r;
    } else {
      const Tile tl = find_tile(s_pref, E, tiles_n, id);
      e = tl.e;
      mend = offsets[e + 1];
      m0 = offsets[e] + tl.mi * FM;
      n0 = tl.nt * FN;
      k0r = 0;
      kn = K;
    }
    float acc[4][4] = {};
    for (int k0 = 0; k0 < kn; k0 += FK) {
      float4 av, bv;
      // K-contiguous loader: row tid / 4, k-values 4 (tid % 4) .. +3.
      // k-major loader: k-row tid / 16, columns 4 (tid % 16) .. +3.
      if constexpr (A_KM) {
        const int kr = tid >> 4, mq = (tid & 15) * 4;
        const bool ok = k0 + kr < kn && m0 + mq < M;
        av = ok ? *reinterpret_cast<const float4*>(A + static_cast<int64_t>(k0r + k0 + kr) * M + m0 + mq)
                : float4{0, 0, 0, 0};
      } else {
        const int lr = tid >> 2, lk = (tid & 3) * 4;
        const bool ok = k0 + lk < kn;
        const float* ap = A + static_cast<int64_t>(min(m0 + lr, mend - 1)) * K;
        av = ok ? *reinterpret_cast<const float4*>(ap + k0 + lk) : float4{0, 0, 0, 0};
      }
      if constexpr (B_KM) {
        const int kr = tid >> 4, nq = (tid & 15) * 4;
        const bool ok = k0 + kr < kn && n0 + nq < N;
        const float* bb = SEG_K ? B + static_cast<int64_t>(k0r + k0 + kr) * N
                                : B + (static_cast<int64_t>(e) * K + k0 + kr) * N;
        bv = ok ? *reinterpret_cast<const float4*>(bb + n0 + nq) : float4{0, 0, 0, 0};
      } else {
        const int lr = tid >> 2, lk = (tid & 3) * 4;
        const bool ok = k0 + lk < kn;
        const float* bp = B + (static_cast<int64_t>(e) * N + min(n0 + lr, N - 1)) * K;
        bv = ok ? *reinterpret_cast<const float4*>(bp + k0 + lk) : float4{0, 0, 0, 0};
      }
      __syncthreads();
      if constexpr (A_KM) {
        const int kr = tid >> 4, mq = (tid & 15) * 4;
        As[kr][mq + 0] = av.x; As[kr][mq + 1] = av.y; As[kr][mq + 2] = av.z; As[kr][mq + 3] = av.w;
      } else {
        const int lr = tid >> 2, lk = (tid & 3) * 4;
        As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
      }
      if constexpr (B_KM) {
        const int kr = tid >> 4, nq = (tid & 15) * 4;
        Bs[kr][nq + 0] = bv.x; Bs[kr][nq + 1] = bv.y; Bs[kr][nq + 2] = bv.z; Bs[kr][nq + 3] = bv.w;
      } else {
        const int lr = tid >> 2, lk = (tid & 3) * 4;
        Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
      }
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
      if (row >= mend) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col >= N) continue;
        const int64_t at = (SEG_K ? static_cast<int64_t>(e) * M + row : static_cast<int64_t>(row)) * N + col;
        C[at] = EPI == 1 ? acc[i][j] * gelu_tanh_grad(Z[at]) : acc[i][j];
      }
    }
    __syncthreads();
  }
}

template <bool A_KM, bool B_KM, bool SEG_K, int EPI>
hipError_t launch_f32(const void* A, const int32_t* offsets, int E, int64_t rows_max, int M, int N,
                      int K, const void* B, void* C, const void* Z, hipStream_t s) {
  int64_t g;
  if (SEG_K) g = static_cast<int64_t>(E) * ((M + FM - 1) / FM) * ((N + FN - 1) / FN);
  else g = (rows_max / FM + E) * ((N + FN - 1) / FN);
  if (g == 0) return hipSuccess;
  if (g > 65535) g = 65535;
  hipLaunchKernelGGL((gemm_f32_kernel<A_KM, B_KM, SEG_K, EPI>), dim3(static_cast<unsigned>(g)),
                     dim3(256), 0, s, static_cast<const float*>(A), offsets, E, M, N, K,
                     static_cast<const float*>(B), static_cast<float*>(C),
                     static_cast<const float*>(Z));
  return hipGetLastError();
}

constexpr int kWgMaxChunks = 64;

}  // namespace

hipError_t launch_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                                   const float* topk_w, int64_t T, int k, int64_t d, int dtype,
                                   void* d_out, float* dw, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(T < 65536 ? T : 65536)), b(kThreads);
  if (k <= 2) {
    if (dtype == 1) hipLaunchKernelGGL((combine_backward_kernel<true, 2>), g, b, 0, s, dy, y_perm, dest, topk_w, T, k, d, d_out, dw);
    else hipLaunchKernelGGL((combine_backward_kernel<false, 2>), g, b, 0, s, dy, y_perm, dest, topk_w, T, k, d, d_out, dw);
  } else {
    if (dtype == 1) hipLaunchKernelGGL((combine_backward_kernel<true, kMaxK>), g, b, 0, s, dy, y_perm, dest, topk_w, T, k, d, d_out, dw);
    else hipLaunchKernelGGL((combine_backward_kernel<false, kMaxK>), g, b, 0, s, dy, y_perm, dest, topk_w, T, k, d, d_out, dw);
  }
  return hipGetLastError();
}

hipError_t launch_gate_backward(const float* dw, const int32_t* topk_idx, const float* topk_w,
                                const float* probs, const int32_t* counts, const float* lse,
                                int64_t T, int E, int k, bool renorm, float temperature,
                                float alpha, float aux_grad, float z_coeff, float* dl,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  const double Td = static_cast<double>(T);
  const float aux_c = static_cast<float>(static_cast<double>(aux_grad) * alpha * E / (Td * Td * k));
  const float z_c = static_cast<float>(2.0 * z_coeff / Td);
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(gate_backward_kernel, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                     dim3(kThreads), 0, s, dw, topk_idx, topk_w, probs, counts, lse, T, E, k,
                     renorm ? 1 : 0, 1.0f / temperature, aux_c, z_c, dl);
  return hipGetLastError();
}

static int wgrad_chunks(int64_t T) {
  const int64_t c = (T + 127) / 128;   // 128-token chunks, at most kWgMaxChunks
  return static_cast<int>(c < 1 ? 1 : (c > kWgMaxChunks ? kWgMaxChunks : c));
}

size_t gate_wgrad_ws_floats(int64_t T, int64_t d, int E) {
  return static_cast<size_t>(wgrad_chunks(T)) * E * (d + 1);
}

hipError_t launch_gate_wgrad(const float* dl, const void* x, int64_t T, int64_t d, int E,
                             int dtype, float* dwg, float* db, float* ws, hipStream_t s) {
  const int nch = wgrad_chunks(T);
  const int64_t chunk = T > 0 ? (T + nch - 1) / nch : 0;
  float* part = ws;
  float* part_b = ws + static_cast<size_t>(nch) * E * d;
  if (T > 0 && E > kWgE) {
    const dim3 g(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>(nch), static_cast<unsigned>((E + 63) / 64));
    if (dtype == 1) hipLaunchKernelGGL(gate_wgrad_mfma_kernel<true>, g, dim3(kThreads), 0, s, dl, x, T, d, E, chunk, part, part_b);
    else hipLaunchKernelGGL(gate_wgrad_mfma_kernel<false>, g, dim3(kThreads), 0, s, dl, x, T, d, E, chunk, part, part_b);
  } else if (T > 0) {
    const dim3 g(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>(nch));
    if (dtype == 1) hipLaunchKernelGGL(gate_wgrad_partial_kernel<true>, g, dim3(kThreads), 0, s, dl, x, T, d, E, chunk, part, part_b);
    else hipLaunchKernelGGL(gate_wgrad_partial_kernel<false>, g, dim3(kThreads), 0, s, dl, x, T, d, E, chunk, part, part_b);
  }
  const int real = T > 0 ? static_cast<int>((T + chunk - 1) / chunk) : 0;   // chunks with tokens
  const int64_t n = static_cast<int64_t>(E) * d;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(gate_wgrad_final_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                     dim3(kThreads), 0, s, part, part_b, real, d, E, dwg, db);
  return hipGetLastError();
}

hipError_t launch_dispatch_backward(const float* dx_perm, const int32_t* dest, const float* dl,
                                    const void* wg, int64_t T, int k, int64_t d, int E, int dtype,
                                    float* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if ((T + kDispTok - 1) / kDispTok <= 65535 &&
      static_cast<int64_t>(T) * k * d * 4 < 0x7fffffffLL &&   // grouped rows <= T k
      static_cast<int64_t>(E) * d * 4 < 0x7fffffffLL) {
    const dim3 g(static_cast<unsigned>(((d >> 2) + kThreads - 1) / kThreads),
                 static_cast<unsigned>((T + kDispTok - 1) / kDispTok));
    if (k <= 2) {
      if (dtype == 1) hipLaunchKernelGGL((dispatch_backward_tok_kernel<true, 2>), g, dim3(kThreads), 0, s, dx_perm, dest, dl, wg, T, k, d, E, dx);
      else hipLaunchKernelGGL((dispatch_backward_tok_kernel<false, 2>), g, dim3(kThreads), 0, s, dx_perm, dest, dl, wg, T, k, d, E, dx);
    } else {
      if (dtype == 1) hipLaunchKernelGGL((dispatch_backward_tok_kernel<true, kMaxK>), g, dim3(kThreads), 0, s, dx_perm, dest, dl, wg, T, k, d, E, dx);
      else hipLaunchKernelGGL((dispatch_backward_tok_kernel<false, kMaxK>), g, dim3(kThreads), 0, s, dx_perm, dest, dl, wg, T, k, d, E, dx);
    }
    return hipGetLastError();
  }
  const dim3 g(static_cast<unsigned>(T < 65536 ? T : 65536)), b(kThreads);
  if (dtype == 1) hipLaunchKernelGGL(dispatch_backward_kernel<true>, g, b, 0, s, dx_perm, dest, dl, wg, T, k, d, E, dx);
  else hipLaunchKernelGGL(dispatch_backward_kernel<false>, g, b, 0, s, dx_perm, dest, dl, wg, T, k, d, E, dx);
  return hipGetLastError();
}

// Expert backward GEMMs. dtype 1: the MFMA kernels; dtype 0: the f32 kernel.
hipError_t launch_down_backward(const void* d_out, const int32_t* offsets, int E, int64_t rows_max,
                                int64_t d, int64_t d_ff, const void* w2, const void* z, int dtype,
                                void* dz, void* ws, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  if (dtype == 1)
    return launch_gemm_mfma(GemmKind::kDh, d_out, offsets, E, rows_max, 0, static_cast<int>(d_ff),
                            static_cast<int>(d), w2, dz, const_cast<void*>(z), ws, s);
  return launch_f32<false, true, false, 1>(d_out, offsets, E, rows_max, 0, static_cast<int>(d_ff),
                                           static_cast<int>(d), w2, dz, z, s);
}

hipError_t launch_up_backward(const void* dz, const int32_t* offsets, int E, int64_t rows_max,
                              int64_t d, int64_t d_ff, const void* w1, int dtype, float* dx_perm,
                              void* ws, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  if (dtype == 1)
    return launch_gemm_mfma(GemmKind::kDx, dz, offsets, E, rows_max, 0, static_cast<int>(d),
                            static_cast<int>(d_ff), w1, dx_perm, nullptr, ws, s);
  return launch_f32<false, true, false, 0>(dz, offsets, E, rows_max, 0, static_cast<int>(d),
                                           static_cast<int>(d_ff), w1, dx_perm, nullptr, s);
}

hipError_t launch_expert_dw2(const void* d_out, const void* h, const int32_t* offsets, int E,
                             int64_t d, int64_t d_ff, int dtype, float* dw2, hipStream_t s) {
  if (dtype == 1)
    return launch_gemm_mfma(GemmKind::kDw2, d_out, offsets, E, 0, static_cast<int>(d),
                            static_cast<int>(d_ff), 0, h, dw2, nullptr, nullptr, s);
  return launch_f32<true, true, true, 0>(d_out, offsets, E, 0, static_cast<int>(d),
                                         static_cast<int>(d_ff), 0, h, dw2, nullptr, s);
}

hipError_t launch_expert_dw1(const void* dz, const void* x_perm, const int32_t* offsets, int E,
                             int64_t d, int64_t d_ff, int dtype, float* dw1, hipStream_t s) {
  if (dtype == 1)
    return launch_gemm_mfma(GemmKind::kDw1, dz, offsets, E, 0, static_cast<int>(d_ff),
                            static_cast<int>(d), 0, x_perm, dw1, nullptr, nullptr, s);
  return launch_f32<true, true, true, 0>(dz, offsets, E, 0, static_cast<int>(d_ff),
                                         static_cast<int>(d), 0, x_perm, dw1, nullptr, s);
}

}  // namespace moe

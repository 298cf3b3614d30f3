// Gate linear + softmax + top-k, fused (EP tutorial "专家并行：混合专家模型的
// 分布式训练方案", section 1.1 and 2.1 step 1; deployment guide
// "细粒度专家并行部署实践与优化指南", section 5 step 3: the gate outputs each
// token's expert-assignment probabilities).
//
// One workgroup = 4 waves = 16 TT tokens. The logits l = x . Wg^T (+ b) are a
// [16 TT x d] x [d x E] contraction: bf16 inputs go through
// v_mfma_f32_16x16x32_bf16 with each wave taking every 4th 128-wide slice of d
// for all TT 16-token tiles, so each gate-weight fragment it loads serves
// 16 TT tokens (wide gates: the gate weight is most of the bytes a 16-token
// workgroup would read); the four partial tiles meet in LDS and are summed in
// a fixed order. Softmax and top-k then run with 16 lanes per token, each lane
// owning experts e = lane%16 + 16*i, so a token's E logits never leave
// registers.
// Balancing knobs (SP/EP page, EP section: routing temperature and a random
// perturbation; ETP page: routing z-loss): softmax and top-k see the scores
// s = (l + noise) / temperature, and the per-token log sum_e exp s that the
// z-loss squares (and its gradient needs) falls out of the softmax's max and
// sum.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTok = 16;      // tokens per workgroup
constexpr int kThreads = 256;
constexpr int kChunk = 128;   // d-elements one wave consumes per step

// Softmax + top-k for one token held by a 16-lane group; lane q owns experts
// e = q + 16*i (i < NT). Invalid experts (e >= E) carry -inf and are skipped.
template <int NT>
__device__ void softmax_topk(float (&lg)[NT], int E, int k, uint32_t flags, int64_t t,
                            int q, int32_t* topk_idx, float* topk_w, float* probs,
                            float* lse) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT; ++i) m = fmaxf(m, lg[i]);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  float ex[NT];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int e = q + 16 * i;
    ex[i] = (e < E) ? expf(lg[i] - m) : 0.f;
    s += ex[i];
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
  const float inv_s = 1.0f / s;
  if (lse != nullptr && q == 0) lse[t] = m + logf(s);
  if (probs) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = q + 16 * i;
      if (e < E) probs[t * E + e] = ex[i] * inv_s;
    }
  }
  // k rounds of a (logit desc, index asc) arg-max over the unchosen experts.
  uint32_t chosen = 0;
  float wsel[kMaxK];
  int esel[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= k) break;
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = q + 16 * i;
      if (e < E && !((chosen >> i) & 1u)) {
        if (lg[i] > bv || (lg[i] == bv && e < be)) { bv = lg[i]; be = e; }
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if (be != 0x7fffffff) {
      if ((be & 15) == q) chosen |= 1u << (be >> 4);
      esel[j] = be;
      wsel[j] = expf(bv - m) * inv_s;   // same arithmetic as probs[t, be]
    } else {                            // only NaN logits were left
      esel[j] = -1;
      wsel[j] = 0.f;
    }
  }
  if (q == 0) {
    float norm = 1.f;
    if (flags & 1u) {
      float tot = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) tot += wsel[j];
      norm = 1.0f / tot;
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        topk_idx[t * k + j] = esel[j];
        topk_w[t * k + j] = (flags & 1u) ? wsel[j] * norm : wsel[j];
      }
    }
  }
}

// bf16: MFMA logits, LDS reduction over the four d-slices, then softmax/top-k.
template <int NT, int TT>
__global__ __launch_bounds__(kThreads) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const float* __restrict__ bias, const float* __restrict__ noise, float temperature,
    int64_t T, int64_t d, int E, int k, uint32_t flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ probs, float* __restrict__ lse) {
  __shared__ float red[4][kTok * TT][NT * 16];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok * TT;
  const uint16_t* xrow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)   // tail rows re-read the last token
    xrow[tt] = x + min(t0 + tt * kTok + r, T - 1) * d;

  f32x4 acc[TT][NT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[tt][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* wrow[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) wrow[n] = wg + static_cast<int64_t>(min(n * 16 + r, E - 1)) * d;

  // U slices per step, all their loads issued before the MFMAs that use
  // them (one slice per step would leave each wave with one round trip to
  // memory in flight); fewer for wide gates and several token tiles, whose
  // fragments need more registers. Within a 128-wide slice, MFMA s takes
  // columns 32 s .. 32 s + 31 and lane group g the eight from 32 s + 8 g, so
  // the four groups of a row read 64 contiguous bytes.
  constexpr int U = (NT * (TT + 1)) <= 4 ? 4 : ((NT * (TT + 1)) <= 8 ? 2 : 1);
  for (int64_t c00 = static_cast<int64_t>(wave) * kChunk; c00 < d; c00 += 4 * U * kChunk) {
    bf16x8 a[U][TT][4], b[U][NT][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c0 = c00 + static_cast<int64_t>(u) * 4 * kChunk;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t col = c0 + s * 32 + g * 8;
        const bool in = col < d;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          a[u][tt][s] = in ? *reinterpret_cast<const bf16x8*>(xrow[tt] + col) : bf16x8{};
#pragma unroll
        for (int n = 0; n < NT; ++n)
          b[u][n][s] = in ? *reinterpret_cast<const bf16x8*>(wrow[n] + col) : bf16x8{};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[tt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][tt][s], b[u][n][s], acc[tt][n], 0, 0, 0);
  }
  // D layout of a 16x16 tile: lane holds rows 4*(lane/16)+i, column lane%16.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][tt * kTok + g * 4 + i][n * 16 + r] = acc[tt][n][i];
  __syncthreads();

  const int q = tid & 15;
#pragma unroll 1
  for (int tt = 0; tt < TT; ++tt) {
    const int tok = tt * kTok + (tid >> 4);
    const int64_t t = t0 + tok;
    float lg[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = q + 16 * i;
      float v = red[0][tok][e] + red[1][tok][e] + red[2][tok][e] + red[3][tok][e];
      if (bias != nullptr && e < E) v += bias[e];
      if (noise != nullptr && e < E && t < T) v += noise[t * E + e];
      lg[i] = (e < E) ? v / temperature : -INFINITY;
    }
    if (t < T) softmax_topk<NT>(lg, E, k, flags, t, q, topk_idx, topk_w, probs, lse);
  }
}

// f32: plain FMA dot products, one (token, expert) pair per lane and step.
template <int NT>
__global__ __launch_bounds__(kThreads) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    const float* __restrict__ noise, float temperature, int64_t T, int64_t d, int E, int k,
    uint32_t flags, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ probs, float* __restrict__ lse) {
  const int tid = threadIdx.x;
  const int tok = tid >> 4, q = tid & 15;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTok + tok;
  const float* xr = x + min(t, T - 1) * d;
  float lg[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int e = q + 16 * i;
    if (e < E) {
      const float* wr = wg + static_cast<int64_t>(e) * d;
      float v = 0.f;
      for (int64_t c = 0; c < d; ++c) v = fmaf(xr[c], wr[c], v);
      if (bias != nullptr) v += bias[e];
      if (noise != nullptr && t < T) v += noise[t * E + e];
      lg[i] = v / temperature;
    } else {
      lg[i] = -INFINITY;
    }
  }
  if (t < T) softmax_topk<NT>(lg, E, k, flags, t, q, topk_idx, topk_w, probs, lse);
}

// Token tiles per bf16 workgroup: gates of 17..64 experts share each
// gate-weight fragment over 4 tiles (LDS reduction buffer <= 64 KiB, two
// waves per SIMD); narrow gates keep one (x is most of their bytes already),
// and wider ones too (their fragments fill the registers).
template <int NT>
constexpr int router_tiles() { return NT == 2 || NT == 4 ? 4 : 1; }

template <int NT>
hipError_t launch_nt(const RouterArgs& a, hipStream_t s) {
  constexpr int TT = router_tiles<NT>();
  const dim3 grid(static_cast<unsigned>((a.T + kTok * TT - 1) / (kTok * TT))), block(kThreads);
  const dim3 grid_f32(static_cast<unsigned>((a.T + kTok - 1) / kTok));
  if (a.dtype == 1)
    hipLaunchKernelGGL((router_bf16_kernel<NT, TT>), grid, block, 0, s,
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.wg), a.bias,
                       a.noise, a.temperature, a.T, a.d, a.E, a.k, a.flags, a.topk_idx, a.topk_w,
                       a.probs, a.lse);
  else
    hipLaunchKernelGGL(router_f32_kernel<NT>, grid_f32, block, 0, s, static_cast<const float*>(a.x),
                       static_cast<const float*>(a.wg), a.bias, a.noise, a.temperature, a.T, a.d,
                       a.E, a.k, a.flags, a.topk_idx, a.topk_w, a.probs, a.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nt = (a.E + 15) / 16;
  if (nt <= 1) return launch_nt<1>(a, s);
  if (nt <= 2) return launch_nt<2>(a, s);
  if (nt <= 4) return launch_nt<4>(a, s);
  if (nt <= 8) return launch_nt<8>(a, s);
  return launch_nt<16>(a, s);
}

}  // namespace moe

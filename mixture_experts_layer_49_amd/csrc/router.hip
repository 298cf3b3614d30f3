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
// registers; the 16 lanes are one DPP row, and their max, sum and arg-max
// reductions are DPP moves within it.
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

// A token's 16-lane group is one DPP row: its reductions combine lane pairs
// by DPP moves (no LDS round trip) -- xor 1 and xor 2 by quad permutations,
// then the mirror within each half-row and within the row. Each step pairs
// lanes holding the same partial set, so with a commutative combine every
// lane of the row ends with the same value.
template <int CTRL>
__device__ __forceinline__ int row_dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float row_dpp(float v) {
  return __builtin_bit_cast(float, row_dpp<CTRL>(__builtin_bit_cast(int, v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, row_dpp<kDppXor1>(v));
  v = fmaxf(v, row_dpp<kDppXor2>(v));
  v = fmaxf(v, row_dpp<kDppHalfMirror>(v));
  return fmaxf(v, row_dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += row_dpp<kDppXor1>(v);
  v += row_dpp<kDppXor2>(v);
  v += row_dpp<kDppHalfMirror>(v);
  return v + row_dpp<kDppMirror>(v);
}
// (value desc, index asc) arg-max step against the partner lane's pair
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& be) {
  const float ov = row_dpp<CTRL>(bv);
  const int oe = row_dpp<CTRL>(be);
  const bool take = (ov > bv) | ((ov == bv) & (oe < be));   // no short-circuit: selects, not branches
  bv = take ? ov : bv;
  be = take ? oe : be;
}

// Softmax + top-k for one token held by a 16-lane group; lane q owns experts
// e = q + 16*i (i < NT). Invalid experts (e >= E) carry -inf and are skipped.
// With s_cnt (LDS, E ints) the token's valid choices are counted into it;
// with s_p (LDS, E floats) its probabilities are also left there.
template <int NT>
__device__ void softmax_topk(float (&lg)[NT], int E, int k, uint32_t flags, int64_t t,
                            int q, int32_t* topk_idx, float* topk_w, float* probs,
                            float* lse, int* s_cnt = nullptr, float* s_p = nullptr) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT; ++i) m = fmaxf(m, lg[i]);
  m = row_max(m);
  float ex[NT];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int e = q + 16 * i;
    ex[i] = (e < E) ? expf(lg[i] - m) : 0.f;
    s += ex[i];
  }
  s = row_sum(s);
  const float inv_s = 1.0f / s;
  if (lse != nullptr && q == 0) lse[t] = m + logf(s);
  if (probs) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = q + 16 * i;
      if (e < E) probs[t * E + e] = ex[i] * inv_s;
    }
  }
  if (s_p) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int e = q + 16 * i;
      if (e < E) s_p[e] = ex[i] * inv_s;
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
      const bool take = (e < E) & (((chosen >> i) & 1u) == 0u) & ((lg[i] > bv) | ((lg[i] == bv) & (e < be)));
      bv = take ? lg[i] : bv;
      be = take ? e : be;
    }
    argmax_step<kDppXor1>(bv, be);
    argmax_step<kDppXor2>(bv, be);
    argmax_step<kDppHalfMirror>(bv, be);
    argmax_step<kDppMirror>(bv, be);
    // be stays 0x7fffffff when only NaN logits were left
    const bool found = be != 0x7fffffff;
    chosen |= (found & ((be & 15) == q)) ? 1u << ((be >> 4) & 31) : 0u;
    esel[j] = found ? be : -1;
    wsel[j] = found ? expf(bv - m) * inv_s : 0.f;   // same arithmetic as probs[t, be]
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
        if (s_cnt != nullptr && esel[j] >= 0) atomicAdd(&s_cnt[esel[j]], 1);   // integer: order-free
      }
    }
  }
}

// bf16: MFMA logits, LDS reduction over the four d-slices, then softmax/top-k.
// WLU > 0 (one 16-expert tile, one token tile, d = 512 WLU): the gate weight
// is staged once per workgroup in LDS by LDS-DMA (rows kWlPad bytes apart
// beyond d, so the 16 rows of a fragment read fall on distinct banks) and
// each wave issues all of its x loads at once, no gate-weight loads among
// them; the MFMAs run in the same order as the other form's, so the logits
// are bit-identical to it.
constexpr int kWlPad = 16;
constexpr int kWlMaxBytes = 64 * 1024;   // gate weight staged in LDS at most
// WS (64 experts or fewer in four expert tiles, four token tiles, d a
// multiple of 512): the gate weight goes through LDS one 512-column slice at
// a time, by LDS-DMA into two slots of 64 rows kWsRow bytes apart (1 KiB of
// the slice + 16 bytes, so the 16 rows of a fragment read fall on distinct
// banks), issued one slice ahead together with that slice's x loads; the
// reduction buffer then reuses the slots.
constexpr int kWsRow = 4 * 128 * 2 + 16;
template <int NT, int TT, int WLU, bool WS = false>
__global__ __launch_bounds__(kThreads) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const float* __restrict__ bias, const float* __restrict__ noise, float temperature,
    int64_t T, int64_t d, int E, int k, uint32_t flags, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ probs, float* __restrict__ lse,
    int32_t* __restrict__ tile_cnt, double* __restrict__ tile_colsum) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  // the two weight slots are separate LDS variables, so the compiler can see
  // that reading one never aliases the DMA still filling the other
  __shared__ __attribute__((aligned(16))) unsigned char s_w0[WS ? 64 * kWsRow : 16];
  __shared__ __attribute__((aligned(16))) unsigned char s_w1[WS ? 64 * kWsRow : 16];
  __shared__ float red_s[WS ? 1 : 4][kTok * TT][NT * 16];
  float (*const red)[kTok * TT][NT * 16] =
      WS ? reinterpret_cast<float (*)[kTok * TT][NT * 16]>(s_w0) : red_s;
  __shared__ int s_cnt[kMaxE];
  const int tid = threadIdx.x;
  if (tile_cnt != nullptr)
    for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;   // published by the barrier below
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

  constexpr bool WL = WLU > 0;
  if constexpr (WL) {
    static_assert(NT == 1 && TT == 1, "one expert tile, one token tile");
    unsigned char* const s_wg = s_dyn;
    const int64_t rs = d * 2 + kWlPad;   // bytes per staged row
    // the gate weight goes to LDS by LDS-DMA (no registers): wave-wide load
    // j carries bytes 1024 j .. +1023 of the weight, inside one row (2 d is a
    // multiple of 1024); then every x load of this wave is issued
    {
      const int64_t wbytes = static_cast<int64_t>(E) * d * 2;
      const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(wg), 0, static_cast<int>(wbytes), 0x00020000);
      const int njobs = static_cast<int>(wbytes / 1024);
      for (int j = wave; j < njobs; j += 4) {
        const int64_t off = static_cast<int64_t>(j) * 1024;
        unsigned char* dst = s_wg + (off / (d * 2)) * rs + off % (d * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)dst, 16,
                                                 static_cast<uint32_t>(lane) * 16u, static_cast<uint32_t>(off), 0, 0);
      }
    }
    // d = 512 WLU: every one of the 4 WLU loads is in range, so the wait
    // below counts exactly the x loads younger than the weight's DMA
    bf16x8 a[WLU][4];
#pragma unroll
    for (int u = 0; u < WLU; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int col = wave * kChunk + u * 4 * kChunk + s * 32 + g * 8;
        a[u][s] = *reinterpret_cast<const bf16x8*>(xrow[0] + col);
      }
    // the weight's DMA is older than the x loads: wait for it alone, then
    // every wave's share is in LDS after the barrier
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((WLU * 4) & 15) | (((WLU * 4) >> 4) << 14));
    __syncthreads();
    const unsigned char* const brow = s_wg + static_cast<int64_t>(min(r, E - 1)) * rs;
#pragma unroll
    for (int u = 0; u < WLU; ++u) {
      const int c0 = wave * kChunk + u * 4 * kChunk;
      bf16x8 b[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s] = *reinterpret_cast<const bf16x8*>(brow + (c0 + s * 32 + g * 8) * 2);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][s], b[s], acc[0][0], 0, 0, 0);
    }
  }
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
  // 33..64 experts (four expert tiles, four token tiles): one slice per step
  // with room for two sets of x fragments, the x loads of the next slice
  // issued right after this slice's gate-weight loads, so they are in flight
  // while this slice's MFMAs run (the weight loads, from L2, are waited for;
  // the next slice's x loads are not). Workgroup b starts at slice b mod the
  // slice count and wraps around, so that at any moment the workgroups read
  // different column windows of their rows rather than one window of every
  // row (the per-token sums then run over the slices in that rotated order).
  // Measured at 64 experts, d = 2048: 49 -> 40 us from cold caches, 31 ->
  // 26 us warm, with the row reductions below; with d a multiple of 512 the
  // WS form below takes the gate-weight loads off the waves' path as well
  // (26.7 -> 24.0 us warm, the same logits bit for bit).
  constexpr bool PIPE = !WL && !WS && U == 1 && NT == 4;
  if constexpr (WS) {
    static_assert(NT == 4 && TT == 4 && !WL, "four expert tiles, four token tiles");
    // d % 512 == 0 (checked at launch): every x load and every weight-row
    // piece below is in range, so each wave issues exactly 16 weight DMA
    // loads and 16 x loads per slice and the waits count them
    const int nsl = static_cast<int>(d / (4 * kChunk));
    const int rot = static_cast<int>(blockIdx.x % nsl);
    auto cof = [&](int i) -> int64_t { return static_cast<int64_t>((i + rot) % nsl) * 4 * kChunk; };
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(wg), 0, static_cast<int>(static_cast<int64_t>(E) * d * 2), 0x00020000);
    // staged row j holds gate row min(j, E - 1): 64 rows, 16 per wave (the
    // wave index made uniform, so offsets and LDS addresses sit in SGPRs)
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto stage_w = [&](int i, unsigned char* base) __attribute__((always_inline)) {
      const int64_t c0 = cof(i);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int row = jj * 4 + wv;
        const uint32_t soff = static_cast<uint32_t>((static_cast<int64_t>(min(row, E - 1)) * d + c0) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(base + row * kWsRow),
                                                 16, static_cast<uint32_t>(lane) * 16u, soff, 0, 0);
      }
    };
    bf16x8 a[2][TT][4];
    auto load_a = [&](bf16x8 (&av)[TT][4], int64_t c0) __attribute__((always_inline)) {
#pragma unroll
      for (int sx = 0; sx < 4; ++sx)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          av[tt][sx] = *reinterpret_cast<const bf16x8*>(xrow[tt] + c0 + wave * kChunk + sx * 32 + g * 8);
    };
    auto mma = [&](const bf16x8 (&av)[TT][4], const unsigned char* slot) __attribute__((always_inline)) {
      const unsigned char* const base = slot + (wave * kChunk + g * 8) * 2;
      bf16x8 b[NT][4];
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int sx = 0; sx < 4; ++sx)
          b[n][sx] = *reinterpret_cast<const bf16x8*>(base + min(n * 16 + r, E - 1) * kWsRow + sx * 64);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int sx = 0; sx < 4; ++sx)
            acc[tt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][sx], b[n][sx], acc[tt][n], 0, 0, 0);
    };
    // one slice: issue the next slice's weight DMA and x loads (32 per
    // wave), wait for everything older, then every wave's share of this
    // slice's weight is in LDS after the barrier; the second barrier keeps
    // the slot from being refilled while a wave still reads it
    // (the loop below has no branch inside its body, so the compiler's own
    // waits before the MFMAs count the loads in flight exactly)
    auto step = [&](int i, bf16x8 (&cur)[TT][4], bf16x8 (&nxt)[TT][4], unsigned char* slot,
                    unsigned char* other, auto has_next) __attribute__((always_inline)) {
      if constexpr (decltype(has_next)::value) {
        stage_w(i + 1, other);
        load_a(nxt, cof(i + 1));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (32 & 15) | ((32 >> 4) << 14));
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      // plain barriers (a release fence would also wait for the next
      // slice's loads): the wait above covers this slice's DMA
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      mma(cur, slot);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    stage_w(0, s_w0);
    load_a(a[0], cof(0));
    const std::true_type more;
    const std::false_type last;
    int i = 0;
    for (; i + 2 < nsl; i += 2) {
      step(i, a[0], a[1], s_w0, s_w1, more);
      step(i + 1, a[1], a[0], s_w1, s_w0, more);
    }
    if (i + 1 < nsl) {
      step(i, a[0], a[1], s_w0, s_w1, more);
      step(i + 1, a[1], a[0], s_w1, s_w0, last);
    } else {
      step(i, a[0], a[1], s_w0, s_w1, last);
    }
  }
  if constexpr (PIPE) {
    const int64_t cw = static_cast<int64_t>(wave) * kChunk;
    const int nsl = cw < d ? static_cast<int>((d - cw + 4 * kChunk - 1) / (4 * kChunk)) : 0;
    bf16x8 a[2][TT][4], b[NT][4];
    auto load_a = [&](bf16x8 (&av)[TT][4], int64_t c0) __attribute__((always_inline)) {
#pragma unroll
      for (int sx = 0; sx < 4; ++sx) {
        const int64_t col = c0 + sx * 32 + g * 8;
        const bool in = col < d;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          av[tt][sx] = in ? *reinterpret_cast<const bf16x8*>(xrow[tt] + col) : bf16x8{};
      }
    };
    auto load_b = [&](int64_t c0) __attribute__((always_inline)) {
#pragma unroll
      for (int sx = 0; sx < 4; ++sx) {
        const int64_t col = c0 + sx * 32 + g * 8;
        const bool in = col < d;
#pragma unroll
        for (int n = 0; n < NT; ++n)
          b[n][sx] = in ? *reinterpret_cast<const bf16x8*>(wrow[n] + col) : bf16x8{};
      }
    };
    auto mma = [&](const bf16x8 (&av)[TT][4]) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int sx = 0; sx < 4; ++sx)
            acc[tt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][sx], b[n][sx], acc[tt][n], 0, 0, 0);
    };
    const int rot = nsl > 0 ? static_cast<int>(blockIdx.x % nsl) : 0;
    auto cof = [&](int i) -> int64_t { return cw + static_cast<int64_t>((i + rot) % nsl) * 4 * kChunk; };
    if (nsl > 0) load_a(a[0], cof(0));
    for (int i = 0; i < nsl; i += 2) {
      load_b(cof(i));
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < nsl) load_a(a[1], cof(i + 1));
      __builtin_amdgcn_sched_barrier(0);
      mma(a[0]);
      if (i + 1 >= nsl) break;
      load_b(cof(i + 1));
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 < nsl) load_a(a[0], cof(i + 2));
      __builtin_amdgcn_sched_barrier(0);
      mma(a[1]);
    }
  }
  for (int64_t c00 = static_cast<int64_t>(wave) * kChunk; !WL && !WS && !PIPE && c00 < d; c00 += 4 * U * kChunk) {
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
    // The token's row of red[0] is read above by the same lanes that may now
    // leave its probabilities there (tile_colsum).
    if (t < T)
      softmax_topk<NT>(lg, E, k, flags, t, q, topk_idx, topk_w, probs, lse,
                       tile_cnt != nullptr ? s_cnt : nullptr, tile_colsum != nullptr ? &red[0][tok][0] : nullptr);
  }
  if (tile_cnt != nullptr) {
    __syncthreads();
    const int64_t ntok = min<int64_t>(kTok * TT, T - t0);
    for (int e = tid; e < E; e += kThreads) {
      tile_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = s_cnt[e];
      if (tile_colsum != nullptr) {
        double acc = 0.0;
        for (int64_t tok = 0; tok < ntok; ++tok) acc += static_cast<double>(red[0][tok][e]);
        tile_colsum[static_cast<int64_t>(blockIdx.x) * E + e] = acc;
      }
    }
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
  // the staged-weight form for one expert tile with the weight within 64 KiB
  // where it measured faster: d = 4096 (8 experts: router 21.8 -> 20.2 us with
  // cold caches); at d = 1024 (16 experts) it measured slower (9.6 -> 10.1 us),
  // the weight being as many bytes per workgroup as its tokens' rows
  const int wlu = (NT == 1 && TT == 1 && static_cast<int64_t>(a.E) * a.d * 2 <= kWlMaxBytes && a.d == 4096)
                      ? 8 : 0;
  const size_t lds = static_cast<size_t>(a.E) * static_cast<size_t>(a.d * 2 + kWlPad);
  auto launch_wl = [&](auto u_c) {
    constexpr int WU = decltype(u_c)::value;
    hipLaunchKernelGGL((router_bf16_kernel<NT, TT, WU>), grid, block, lds, s,
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.wg), a.bias,
                       a.noise, a.temperature, a.T, a.d, a.E, a.k, a.flags, a.topk_idx, a.topk_w,
                       a.probs, a.lse, a.tile_cnt, a.tile_colsum);
  };
  if (a.dtype == 1 && wlu > 0) {
    if constexpr (NT == 1 && TT == 1) {
      launch_wl(std::integral_constant<int, 8>{});
    }
  } else if (NT == 4 && TT == 4 && a.dtype == 1 && a.d % 512 == 0) {
    if constexpr (NT == 4 && TT == 4)
      hipLaunchKernelGGL((router_bf16_kernel<NT, TT, 0, true>), grid, block, 0, s,
                         static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.wg), a.bias,
                         a.noise, a.temperature, a.T, a.d, a.E, a.k, a.flags, a.topk_idx, a.topk_w,
                         a.probs, a.lse, a.tile_cnt, a.tile_colsum);
  } else if (a.dtype == 1)
    hipLaunchKernelGGL((router_bf16_kernel<NT, TT, 0>), grid, block, 0, s,
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.wg), a.bias,
                       a.noise, a.temperature, a.T, a.d, a.E, a.k, a.flags, a.topk_idx, a.topk_w,
                       a.probs, a.lse, a.tile_cnt, a.tile_colsum);
  else
    hipLaunchKernelGGL(router_f32_kernel<NT>, grid_f32, block, 0, s, static_cast<const float*>(a.x),
                       static_cast<const float*>(a.wg), a.bias, a.noise, a.temperature, a.T, a.d,
                       a.E, a.k, a.flags, a.topk_idx, a.topk_w, a.probs, a.lse);
  return hipGetLastError();
}

}  // namespace

int router_tile_tokens(int E) {
  const int nt = (E + 15) / 16;
  const int tt = nt <= 1 ? router_tiles<1>() : nt <= 2 ? router_tiles<2>() : nt <= 4 ? router_tiles<4>()
               : nt <= 8 ? router_tiles<8>() : router_tiles<16>();
  return kTok * tt;
}

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

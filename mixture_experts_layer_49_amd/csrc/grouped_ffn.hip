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
// bf16 path (gfx950 MFMA): 256x256x64 workgroup tiles, 4 waves in a 2x2 grid,
// each wave owning a 128x128 sub-tile = 4x4 32x32x16 MFMA tiles, accumulators
// in AGPRs. The hidden activation h is kept as IEEE fp16, not bf16: same
// size, three more significand bits, which cuts the rounding error it adds to
// the layer output about eight-fold. So the up-projection is bf16 x bf16
// (v_mfma_f32_32x32x16_bf16) with a GELU -> fp16 epilogue, and the
// down-projection is fp16 h x fp16 W2 (v_mfma_f32_32x32x16_f16), W2's bf16
// values being converted exactly to fp16 on their way into LDS.
//
// Staging: global -> LDS with buffer_load_dwordx4 ... lds (no VGPR round trip)
// wherever the bytes go to LDS unchanged; W2 of the down-projection goes
// through VGPRs for its conversion. Two 64 KiB LDS stages: stage k+1 streams
// in while the MFMAs consume stage k, and each wave prefetches the next
// k-slice's fragments into a second register set. The 16-byte chunk c of tile
// row r lives at chunk c ^ (r & 7) of that row, so the MFMA fragment reads
// (eight rows, same c) hit eight different bank groups.
//
// Persistent: one workgroup per CU walks the tile list, which it derives on
// the device from offsets[] (no host read-back). Tiles are ordered expert,
// n-panel, m-tile, and each round of gridDim tiles is laid out so that the 32
// workgroups of an XCD take consecutive tiles and share W panels in their L2.
//
// f32 path: a plain 64x64 LDS-tiled FMA kernel over the same tile list.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// ----------------------------------------------------------- tile list --
// s_pref[e] = number of m-tiles of experts < e (e = 0..E).
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int BM,
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

// gelu_tanh(z) = z/2 (1 + tanh(u)) = z * sigmoid(2u), u = sqrt(2/pi)(z + 0.044715 z^3)
__device__ __forceinline__ float gelu_tanh(float z) {
  const float u = 0.7978845608028654f * fmaf(0.044715f * z, z * z, z);
  return z / (1.0f + __expf(-2.0f * u));
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

// ------------------------------------------------------------ bf16 MFMA --
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int WM = 2, WN = 2;                     // waves per dimension
constexpr int MI = BM / WM / 32;                  // 32x32 tiles per wave along M
constexpr int NI = BN / WN / 32;                  // ... along N
constexpr int kRowsPerInstr = kWave / 8;          // one wave-wide 16-B load = 8 rows
constexpr int kLoadsA = BM / kRowsPerInstr / kWaves;   // per wave per stage
constexpr int kLoadsB = BN / kRowsPerInstr / kWaves;
constexpr int kStageChunks = (BM + BN) * BK / 8;  // uint4 per LDS stage
constexpr int kRegB = BN * BK / 8 / kThreads;     // register-staged W2 chunks per thread

// UP:   A = x_perm (bf16), B = W1 (bf16), C = fp16 gelu_tanh(acc)
// DOWN: A = h (fp16),      B = W2 (bf16 -> fp16 through VGPRs), C = f32 acc
template <bool UP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mfma(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E, int N, int K,
    const uint16_t* __restrict__ B, void* __restrict__ Cout) {
  __shared__ uint4 lds[2][kStageChunks];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_tmp[kMaxE];

  build_tile_prefix(offsets, E, BM, s_pref, s_tmp);
  const int tiles_n = (N + BN - 1) / BN;
  const int64_t total = static_cast<int64_t>(s_pref[E]) * tiles_n;

  const int tid = threadIdx.x;
  // The wave index is uniform across the wave; say so, so that the LDS-DMA
  // destination (M0) is computed in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hl = lane >> 5;
  const int nk = (K + BK - 1) / BK;
  const bool k_tail = (K % BK) != 0;

  const int G = gridDim.x;                        // multiple of 8
  const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // Loader: wave-wide load j of wave w fills LDS chunks [64 (4j + w), +64) =
  // rows 8 (4j + w) .. +8. Lane l lands in chunk slot l of that block: row
  // offset l/8, physical chunk l%8, hence logical chunk (l%8) ^ (l/8) (the
  // block starts on a multiple of 8 rows, so row & 7 = l/8).
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2u;
  const int ld_r = lane >> 3, ld_c = (lane & 7) ^ (lane >> 3);
  const uint32_t ld_voff = ld_r * row_bytes + ld_c * 16u;
  // Register-staged W2 loader (down only): 16-byte chunk q = tid + 256 i is
  // row q/8 = tid/8 + 32 i, logical chunk tid%8, stored at st0 + 256 i.
  const int rs_row = tid >> 3, rs_c = tid & 7;
  const int rs_st0 = rs_row * 8 + (rs_c ^ (rs_row & 7));
  const uint32_t rs_voff = rs_row * row_bytes + rs_c * 16u;

  // Fragment reads: row l32 of each 32-row sub-tile, chunk (2 kk + hl) ^ (l32 & 7).
  const int a_base = (wm * (BM / WM) + l32) * 8;
  const int b_base = BM * 8 + (wn * (BN / WN) + l32) * 8;
  const int sw = l32 & 7;

  for (int64_t base = 0;; base += G) {
    const int64_t id = base + slot;
    if (id >= total) break;
    const Tile tl = find_tile(s_pref, E, tiles_n, id);
    const int seg1 = offsets[tl.e + 1];
    const int m0 = offsets[tl.e] + tl.mi * BM;
    const int n0 = tl.nt * BN;
    // Buffer resources cover exactly the tile's valid rows: loads of rows past
    // the segment end (A) or past N (B) return zeros.
    const int a_rows = min(seg1 - m0, BM), b_rows = min(N - n0, BN);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A + static_cast<int64_t>(m0) * K), 0,
        static_cast<int>(a_rows * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(B + (static_cast<int64_t>(tl.e) * N + n0) * K), 0,
        static_cast<int>(b_rows * row_bytes), 0x00020000);

    uint4 rb[UP ? 1 : kRegB];
    // Issue every load of stage kt into LDS buffer `buf`; nothing waits here.
    auto issue = [&](int kt, int buf) {
      const uint32_t k_bytes = static_cast<uint32_t>(kt) * BK * 2u;
#pragma unroll
      for (int j = 0; j < kLoadsA; ++j) {
        const int blk = j * kWaves + wave;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_ptr_t)(&lds[buf][blk * kWave]), 16, ld_voff,
            blk * kRowsPerInstr * row_bytes + k_bytes, 0, 0);
      }
      if (UP) {
#pragma unroll
        for (int j = 0; j < kLoadsB; ++j) {
          const int blk = j * kWaves + wave;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              b_rsrc, (lds_ptr_t)(&lds[buf][BM * 8 + blk * kWave]), 16, ld_voff,
              blk * kRowsPerInstr * row_bytes + k_bytes, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kRegB; ++i)
          rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                b_rsrc, rs_voff, i * 32u * row_bytes + k_bytes, 0));
      }
    };
    // Down only: convert the staged W2 chunks and write them to LDS.
    auto store_b = [&](int buf) {
      if (!UP) {
#pragma unroll
        for (int i = 0; i < kRegB; ++i)
          lds[buf][BM * 8 + rs_st0 + 256 * i] = bf16x8_to_f16x8(rb[i]);
      }
    };
    // After a stage has landed: zero the chunks past K (only the last stage,
    // only when K is not a multiple of 64).
    auto zero_tail = [&](int kt, int buf) {
      const int k0 = kt * BK;
      for (int p = tid; p < kStageChunks; p += kThreads) {
        const int c = (p & 7) ^ ((p >> 3) & 7);
        if (k0 + c * 8 >= K) lds[buf][p] = uint4{0, 0, 0, 0};
      }
    };

    uint4 fa[2][MI], fb[2][NI];
    auto read_frags = [&](int buf, int kk, int sl) {
      const int c = (kk * 2 + hl) ^ sw;
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[sl][i] = lds[buf][a_base + i * 32 * 8 + c];
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[sl][j] = lds[buf][b_base + j * 32 * 8 + c];
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    __syncthreads();   // previous tile's readers are done with both buffers
    issue(0, 0);
    store_b(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (k_tail && nk == 1) {
      zero_tail(0, 0);
      __syncthreads();
    }
    read_frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) issue(kt + 1, cur ^ 1);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int sl = kk & 1;
        if (kk + 1 < BK / 16) read_frags(cur, kk + 1, sl ^ 1);   // prefetch next k-slice
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            if (UP)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, fa[sl][i]), __builtin_bit_cast(bf16x8, fb[sl][j]),
                  acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8, fa[sl][i]), __builtin_bit_cast(f16x8, fb[sl][j]),
                  acc[i][j], 0, 0, 0);
          }
      }
      if (more) {
        store_b(cur ^ 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      if (more) {
        if (k_tail && kt + 2 == nk) {
          zero_tail(kt + 1, cur ^ 1);
          __syncthreads();
        }
        read_frags(cur ^ 1, 0, 0);
      }
    }

    // Epilogue. 32x32 D layout: lane holds column lane%32 and, for register r,
    // row 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = n0 + wn * (BN / WN) + j * 32 + l32;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * (BM / WM) + i * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (row < seg1) {
            const int64_t o = static_cast<int64_t>(row) * N + col;
            if (UP)
              static_cast<_Float16*>(Cout)[o] = static_cast<_Float16>(gelu_tanh(acc[i][j][r]));
            else
              static_cast<float*>(Cout)[o] = acc[i][j][r];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- f32 --
constexpr int FM = 64, FN = 64, FK = 16;

template <bool UP>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float* __restrict__ A,
                                                        const int32_t* __restrict__ offsets,
                                                        int E, int N, int K,
                                                        const float* __restrict__ B,
                                                        float* __restrict__ C) {
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
        if (col < N) C[static_cast<int64_t>(row) * N + col] = UP ? gelu_tanh(acc[i][j]) : acc[i][j];
      }
    }
    __syncthreads();
  }
}

template <bool UP>
hipError_t launch_gemm(const void* A, const int32_t* offsets, int E, int64_t rows_max, int N,
                       int K, const void* B, int dtype, void* C, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  if (dtype == 1) {
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t upper = (rows_max / BM + E) * tiles_n;   // >= sum_e ceil(kept_e / BM) * tiles_n
    int64_t g = device_cu_count();
    if (upper < g) g = upper;
    g = (g + 7) / 8 * 8;
    hipLaunchKernelGGL(grouped_gemm_mfma<UP>, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0,
                       s, static_cast<const uint16_t*>(A), offsets, E, N, K,
                       static_cast<const uint16_t*>(B), C);
  } else {
    const int64_t tiles_n = (N + FN - 1) / FN;
    int64_t g = (rows_max / FM + E) * tiles_n;
    if (g > 65535) g = 65535;
    hipLaunchKernelGGL(grouped_gemm_f32<UP>, dim3(static_cast<unsigned>(g)), dim3(256), 0, s,
                       static_cast<const float*>(A), offsets, E, N, K,
                       static_cast<const float*>(B), static_cast<float*>(C));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_up_gelu(const void* x_perm, const int32_t* offsets, int E, int64_t rows_max,
                          int64_t d, int64_t d_ff, const void* w1, int dtype, void* h,
                          hipStream_t s) {
  return launch_gemm<true>(x_perm, offsets, E, rows_max, static_cast<int>(d_ff),
                           static_cast<int>(d), w1, dtype, h, s);
}

hipError_t launch_down(const void* h, const int32_t* offsets, int E, int64_t rows_max, int64_t d,
                       int64_t d_ff, const void* w2, int dtype, float* y_perm, hipStream_t s) {
  return launch_gemm<false>(h, offsets, E, rows_max, static_cast<int>(d), static_cast<int>(d_ff),
                            w2, dtype, y_perm, s);
}

}  // namespace moe

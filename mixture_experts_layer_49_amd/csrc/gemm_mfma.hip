// Segmented bf16/fp16 MFMA GEMM for the grouped expert FFN on gfx950.
//
// C[m, n] = sum_k A[m, k] B[n, k] over the expert-major row segments given by
// offsets[] (A and B K-contiguous):
//   up:   A = x_perm [R, d] bf16, B = W1[e] [d_ff, d] bf16 -> h = fp16(gelu_tanh(C))
//   down: A = h [R, d_ff] fp16,   B = W2[e] [d, d_ff] bf16 (-> fp16) -> y_perm = C (f32)
// (ETP page "ETP专家并行加速MoE模型": up-projection w1, down-projection w2;
// EP tutorial "专家并行：混合专家模型的分布式训练方案", 2.1 step 4.)
//
// Shape of the work: 256x256 output tiles, 4 waves in a 2x2 grid, each wave
// 128x128 = 4x4 v_mfma_f32_32x32x16_{bf16,f16} tiles with its 256
// accumulators in AGPRs. K advances 32 at a time through a ring of four
// 32 KiB LDS stages:
//   * stages are fetched three ahead with buffer_load_dwordx4 ... lds: the
//     data goes HBM/L2 -> LDS without touching VGPRs. In the down-projection
//     W2 lands in LDS as bf16 and each wave converts its B fragments to fp16
//     (exactly) in registers, interleaved with the MFMAs of the previous
//     k-slice;
//   * the four stages are four separate LDS variables, addressed with
//     compile-time slot numbers (the stage loop is unrolled by four), so the
//     compiler can see that reading one stage never aliases the DMA still
//     filling another and does not wait on it; barriers are plain s_barrier
//     (no release fence, which would wait for every load in flight);
//   * one barrier per stage, placed between its two 16-deep k-slices: by then
//     the next stage has landed, so the first fragments of the next stage are
//     read while the second k-slice's MFMAs run, and the stage three ahead can
//     reuse the slot the previous stage freed;
//   * LDS layout: a tile row is 4 chunks of 16 B; logical chunk c of row r sits
//     at chunk c ^ ((r >> 2) & 3). A fragment read touches 16 consecutive rows
//     at one logical chunk per LDS cycle, which this spreads over all 64 banks.
// Epilogue: accumulators go through two free LDS stages so that the outputs
// leave in whole rows, 16 B per lane; meanwhile the next tile's first two
// stages are already streaming into the other two.
// Persistent: one workgroup per CU walks the tile list that it derives on the
// device from offsets[] (no host read-back). The list (expert, n-panel,
// m-tile order) is cut into eight contiguous ranges, one per XCD, so an XCD
// owns one or a few experts: their weights and rows come from HBM about once
// and are reused from that XCD's L2, and within the XCD the workgroups take
// consecutive tiles, i.e. the m-tiles of the same weight panel.
#include "ffn_common.h"

namespace moe {
namespace {

using namespace ffn;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 256, BN = 256, BK = 32, NS = 4;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int WM = 2, WN = 2;
constexpr int MI = BM / WM / 32, NI = BN / WN / 32;
constexpr int kCpr = BK / 8;                            // 16-B chunks per tile row
constexpr int kRowsPerLoad = kWave / kCpr;              // rows per wave-wide 16-B load
constexpr int kLoadsA = BM / kRowsPerLoad / kWaves;     // LDS-DMA loads per wave per stage
constexpr int kLoadsB = BN / kRowsPerLoad / kWaves;
constexpr int kStage = (BM + BN) * kCpr;                // uint4 per stage
static_assert(NS == 4 && BK == 32 && kLoadsA + kLoadsB == 8, "the pipeline below assumes these");

// s_waitcnt vmcnt(n) (n < 16), other counters untouched, through the builtin
// so that the compiler's own wait bookkeeping sees it (gfx9 encoding: vmcnt
// in bits 3:0, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
#define MOE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))
// Workgroup barrier without __syncthreads()'s release fence: that fence would
// wait for every LDS-DMA load in flight, i.e. also for the stages fetched
// ahead. Each wave instead waits for exactly the stage it needs (MOE_WAIT_VM)
// and for its own LDS accesses (lgkmcnt) before the barrier.
#define MOE_BARRIER()                                       \
  do {                                                      \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      \
    __builtin_amdgcn_s_barrier();                           \
    asm volatile("" ::: "memory");                          \
  } while (0)

struct Ctx {
  __amdgpu_buffer_rsrc_t a, b;
  int m0, n0, seg1;
};

template <bool UP>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E, int N, int K,
    const uint16_t* __restrict__ B, void* __restrict__ Cout) {
  __shared__ uint4 st0[kStage];
  __shared__ uint4 st1[kStage];
  __shared__ uint4 st2[kStage];
  __shared__ uint4 st3[kStage];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_off[kMaxE + 1];   // offsets[], kept on chip for the tile lookups
  __shared__ int s_tmp[kMaxE];
  uint4* const L[NS] = {st0, st1, st2, st3};   // always indexed by a constant

  for (int e = threadIdx.x; e <= E; e += kThreads) s_off[e] = offsets[e];
  build_tile_prefix(offsets, E, BM, s_pref, s_tmp);   // ends with a barrier
  const int tiles_n = (N + BN - 1) / BN;
  const int64_t total = static_cast<int64_t>(s_pref[E]) * tiles_n;
  // The tile list is cut into 8 equal contiguous ranges, one per XCD
  // (workgroup b runs on XCD b % 8); the XCD's workgroups walk their range
  // with stride G/8. A range covers one or a few experts, so each XCD streams
  // its experts' weights and rows from HBM about once and reuses them in its
  // own L2.
  const int G = gridDim.x;   // a multiple of 8
  const int xcd = blockIdx.x & 7, per_xcd = G >> 3;
  const int64_t r_end = total * (xcd + 1) / 8;
  int64_t id = total * xcd / 8 + (blockIdx.x >> 3);
  if (id >= r_end) return;

  const int tid = threadIdx.x;
  // Uniform across the wave: lets the LDS-DMA destination (M0) live in SGPRs.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hl = lane >> 5;
  const int nk = (K + BK - 1) / BK;
  const int tail_kt = (K % BK) ? nk - 1 : -1;   // the stage that needs zero fill
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2u;

  // LDS-DMA: wave-wide load j of wave w fills 16 rows starting at 16 (4j + w);
  // lane l lands in row + l/4, physical chunk l%4, so it fetches logical chunk
  // (l%4) ^ ((row >> 2) & 3) = (l%4) ^ ((l >> 4) & 3).
  const uint32_t ld_voff = (lane >> 2) * row_bytes + (((lane & 3) ^ ((lane >> 4) & 3)) * 16u);
  // Fragments: rows wm*128 + 32 i + l32 (A) and wn*128 + 32 j + l32 (B).
  const int fr_a = (wm * (BM / WM) + l32) * kCpr;
  const int fr_b = BM * kCpr + (wn * (BN / WN) + l32) * kCpr;
  const int fr_sw = (l32 >> 2) & 3;

  auto make_ctx = [&](int64_t tile_id, Ctx& c) {
    const Tile tl = find_tile(s_pref, E, tiles_n, tile_id);
    c.seg1 = s_off[tl.e + 1];
    c.m0 = s_off[tl.e] + tl.mi * BM;
    c.n0 = tl.nt * BN;
    // The resources cover exactly the tile's valid rows: rows past the
    // segment end (A) or past N (B) read as zeros.
    const int a_rows = min(c.seg1 - c.m0, BM), b_rows = min(N - c.n0, BN);
    c.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A + static_cast<int64_t>(c.m0) * K),
                                            0, static_cast<int>(a_rows * row_bytes), 0x00020000);
    c.b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(B + (static_cast<int64_t>(tl.e) * N + c.n0) * K), 0,
        static_cast<int>(b_rows * row_bytes), 0x00020000);
  };

  // Start every load of stage kt into slot S = kt % 4 (a constant at each call).
  auto issue = [&](const Ctx& c, int kt, int S) {
    uint4* const dst = L[S];
    const uint32_t kb = static_cast<uint32_t>(kt) * BK * 2u;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
      const int blk = j * kWaves + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.a, (lds_ptr_t)(dst + blk * kWave), 16, ld_voff,
                                               blk * kRowsPerLoad * row_bytes + kb, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
      const int blk = j * kWaves + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.b, (lds_ptr_t)(dst + BM * kCpr + blk * kWave), 16,
                                               ld_voff, blk * kRowsPerLoad * row_bytes + kb, 0, 0);
    }
  };
  // Zero the chunks of stage kt (slot S) that lie past K (only when K % 32 != 0).
  auto zero_tail = [&](int kt, int S) {
    for (int p = tid; p < kStage; p += kThreads) {
      const int c = (p & 3) ^ ((p >> 4) & 3);
      if (kt * BK + c * 8 >= K) L[S][p] = uint4{0, 0, 0, 0};
    }
  };

  uint4 fa[2][MI], fb[2][NI];
  auto read_frags = [&](int S, int kk, int fs) {
    const int c = (kk * 2 + hl) ^ fr_sw;
    int ab = fr_a + c, bb = fr_b + c;
    // Opaque to the optimiser: the two bases are recomputed here (two adds)
    // instead of 32 per-slot addresses being hoisted out of the loop and
    // spilled; the i / j steps stay immediate offsets.
    asm volatile("" : "+v"(ab), "+v"(bb));
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[fs][i] = L[S][ab + i * 32 * kCpr];
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[fs][j] = L[S][bb + j * 32 * kCpr];
  };
  // Down: W2 fragments arrive as bf16; fp16 is exact for them.
  auto conv_fb = [&](int fs) {
    if (!UP) {
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[fs][j] = bf16x8_to_f16x8(fb[fs][j]);
    }
  };

  f32x16 acc[MI][NI];
  // 16 MFMAs on fragment set fs; in the down-projection, set cs (read just
  // before) is converted in between them: four MFMAs first (the LDS reads
  // land meanwhile), then one MFMA per four VALU conversion ops.
  auto mfma_block = [&](int fs, int cs) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if (UP)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, fa[fs][i]), __builtin_bit_cast(bf16x8, fb[fs][j]),
              acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, fa[fs][i]), __builtin_bit_cast(f16x8, fb[fs][j]),
              acc[i][j], 0, 0, 0);
      }
    if (!UP) {
      conv_fb(cs);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#pragma unroll
      for (int q = 0; q < 12; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
  };

  // One stage (kt, slot S = kt % 4): k-slice 0; then, when a next stage
  // exists, wait for it, publish it with the barrier, refill the slot freed
  // by stage kt-1 with stage kt+3 and prefetch the next stage's first
  // fragments; then k-slice 1.
  // Steady state (kt + 3 < nk, no tail): the same without a branch, so the
  // compiler's wait bookkeeping stays exact.
  Ctx cur;
  auto steady = [&](int kt, int S) {
    const int S1 = (S + 1) & (NS - 1), S3 = (S + 3) & (NS - 1);
    read_frags(S, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(0, 1);
    __builtin_amdgcn_sched_barrier(0);
    MOE_WAIT_VM(8);   // stage kt+1 has landed; only stage kt+2 may be in flight
    MOE_BARRIER();
    issue(cur, kt + 3, S3);
    read_frags(S1, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(1, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto stage = [&](int kt, int S) {
    const int S1 = (S + 1) & (NS - 1), S3 = (S + 3) & (NS - 1);
    read_frags(S, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(0, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      if (kt + 2 < nk) MOE_WAIT_VM(8);   // only stage kt+2 may still be in flight
      else MOE_WAIT_VM(0);
      MOE_BARRIER();
      if (kt + 1 == tail_kt) {
        zero_tail(kt + 1, S1);
        MOE_BARRIER();
      }
      if (kt + 3 < nk) issue(cur, kt + 3, S3);
      read_frags(S1, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(1, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Epilogue through LDS slots 2 and 3 (one per 128-column half, wn), in four
  // passes of 64 rows. A pass first copies the raw f32 accumulators of its
  // rows into LDS (no arithmetic, so the 256 accumulators need no extra
  // registers), then a compact loop turns 64 x 256 values into output: GELU
  // and fp16 packing for the up-projection, plain f32 for the down one, as
  // whole-row 16-byte stores. Staged element (row, col) sits at column
  // col ^ (32 * ((row >> 2) & 1)), so the two half-waves of a write (rows r
  // and r + 4) land on different banks.
  auto epilogue = [&](const Ctx& c) {
    float* const h0 = reinterpret_cast<float*>(st2);
    float* const h1 = reinterpret_cast<float*>(st3);
#pragma unroll
    for (int p = 0; p < BM / 64; ++p) {
      if (wm == p / 2) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * (p & 1) + ii;
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = ii * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
              const int col = (j * 32 + l32) ^ (hl * 32);
              if (wn == 0) h0[row * 128 + col] = acc[i][j][r];
              else h1[row * 128 + col] = acc[i][j][r];
            }
        }
      }
      MOE_BARRIER();
      constexpr int VPC = UP ? 8 : 4;   // output values per 16-byte store
#pragma unroll 1
      for (int q = tid; q < 64 * BN / VPC; q += kThreads) {
        const int row = q / (BN / VPC);
        const int col = (q % (BN / VPC)) * VPC;   // 0..255, multiple of VPC
        const int grow = c.m0 + p * 64 + row;
        const int gcol = c.n0 + col;
        if (grow >= c.seg1 || gcol >= N) continue;
        const float* src = (col < 128 ? h0 : h1) + row * 128 + ((col & 127) ^ (((row >> 2) & 1) * 32));
        uint4 out;
        if (UP) {
          const float4 a = *reinterpret_cast<const float4*>(src);
          const float4 b = *reinterpret_cast<const float4*>(src + 4);
          const f16x2 p0 = {static_cast<_Float16>(gelu_tanh_fast(a.x)), static_cast<_Float16>(gelu_tanh_fast(a.y))};
          const f16x2 p1 = {static_cast<_Float16>(gelu_tanh_fast(a.z)), static_cast<_Float16>(gelu_tanh_fast(a.w))};
          const f16x2 p2 = {static_cast<_Float16>(gelu_tanh_fast(b.x)), static_cast<_Float16>(gelu_tanh_fast(b.y))};
          const f16x2 p3 = {static_cast<_Float16>(gelu_tanh_fast(b.z)), static_cast<_Float16>(gelu_tanh_fast(b.w))};
          out = uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                      __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
        } else {
          out = *reinterpret_cast<const uint4*>(src);
        }
        char* dst = static_cast<char*>(Cout) + (static_cast<int64_t>(grow) * N + gcol) * (UP ? 2 : 4);
        *reinterpret_cast<uint4*>(dst) = out;
      }
      MOE_BARRIER();
    }
  };

  make_ctx(id, cur);
  issue(cur, 0, 0);
  if (nk > 1) issue(cur, 1, 1);
  if (nk > 2) issue(cur, 2, 2);

  for (;;) {
    // Stage 0 of this tile (and, conservatively, everything else in flight,
    // including the previous tile's output stores).
    MOE_WAIT_VM(0);
    MOE_BARRIER();
    if (tail_kt == 0) {
      zero_tail(0, 0);
      MOE_BARRIER();
    }
    read_frags(0, 0, 0);
    conv_fb(0);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    int kt = 0;
    if (nk % NS == 0 && tail_kt < 0) {
      // K a multiple of 128: every stage runs the steady body. The last three
      // stages prefetch stages past the end of K, which is harmless: those
      // bytes are either inside the tile's buffer range (other rows, never
      // used) or past it (the buffer load returns zeros), and the slots they
      // fill hold no live stage.
      for (; kt < nk; kt += NS) {
        steady(kt, 0);
        steady(kt + 1, 1);
        steady(kt + 2, 2);
        steady(kt + 3, 3);
      }
    }
    for (; kt + 6 < nk; kt += NS) {   // four steady stages: (kt + 3) + 3 < nk
      steady(kt, 0);
      steady(kt + 1, 1);
      steady(kt + 2, 2);
      steady(kt + 3, 3);
    }
    // The last (at most six) stages, slot numbers continuing from 0.
    if (kt < nk) stage(kt, 0);
    if (kt + 1 < nk) stage(kt + 1, 1);
    if (kt + 2 < nk) stage(kt + 2, 2);
    if (kt + 3 < nk) stage(kt + 3, 3);
    if (kt + 4 < nk) stage(kt + 4, 0);
    if (kt + 5 < nk) stage(kt + 5, 1);

    // The next tile's first two stages stream into slots 0 and 1 while this
    // tile's outputs go out through slots 2 and 3.
    const Ctx done = cur;
    const int64_t nid = id + per_xcd;
    const bool has_next = nid < r_end;
    MOE_WAIT_VM(0);  // every load of this tile has landed (no DMA into slots 2, 3)
    MOE_BARRIER();   // every wave has finished reading LDS
    if (has_next) {
      make_ctx(nid, cur);
      issue(cur, 0, 0);
      if (nk > 1) issue(cur, 1, 1);
    }
    epilogue(done);
    if (!has_next) break;
    if (nk > 2) issue(cur, 2, 2);
    id = nid;
  }
}

}  // namespace

hipError_t launch_ffn_mfma(bool up, const void* A, const int32_t* offsets, int E, int64_t rows_max,
                           int N, int K, const void* B, void* C, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t upper = (rows_max / BM + E) * tiles_n;   // >= sum_e ceil(kept_e / BM) * tiles_n
  int64_t g = device_cu_count();
  if (upper < g) g = upper;
  g = (g + 7) / 8 * 8;
  if (up)
    hipLaunchKernelGGL(gemm_mfma_kernel<true>, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0,
                       s, static_cast<const uint16_t*>(A), offsets, E, N, K,
                       static_cast<const uint16_t*>(B), C);
  else
    hipLaunchKernelGGL(gemm_mfma_kernel<false>, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0,
                       s, static_cast<const uint16_t*>(A), offsets, E, N, K,
                       static_cast<const uint16_t*>(B), C);
  return hipGetLastError();
}

}  // namespace moe

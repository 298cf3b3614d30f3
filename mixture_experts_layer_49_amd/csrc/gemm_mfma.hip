// Segmented bf16/fp16 MFMA GEMM for the grouped expert FFN on gfx950, forward
// and backward.
//
// Row-segmented kinds: C[m, n] = sum_k A[m, k] B_e(n, k) over the expert-major
// row segments given by offsets[] (A K-contiguous):
//   up:   A = x_perm [R, d] bf16, B = W1[e] [d_ff, d] bf16 -> h = fp16(gelu_tanh(C)),
//         optionally also the pre-activation z = fp16(C) for the backward
//   down: A = h [R, d_ff] fp16,   B = W2[e] [d, d_ff] bf16 (-> fp16) -> y_perm = C (f32)
//   dh:   A = do [R, d] bf16,     B = W2[e] read as [d][d_ff] (k-major) -> dz = bf16(C gelu'(z))
//   dx:   A = dz [R, d_ff] bf16,  B = W1[e] read as [d_ff][d] (k-major) -> dx_perm = C (f32)
// K-segmented kinds (weight gradients): C_e[m, n] = sum over the rows r of
// expert e of A[r, m] B[r, n], both operands k-major:
//   dW2:  A = do [R, d] bf16, B = h [R, d_ff] fp16 (-> bf16) -> dW2 [E, d, d_ff] f32
//   dW1:  A = dz [R, d_ff] bf16, B = x_perm [R, d] bf16      -> dW1 [E, d_ff, d] f32
// (ETP page "ETP专家并行加速MoE模型": up-projection w1, down-projection w2;
// EP tutorial "专家并行：混合专家模型的分布式训练方案", 2.1 step 4; the
// backward is the same chain taken in reverse.)
//
// Shape of the work: 256x256 output tiles, 4 waves in a 2x2 grid, each wave
// 128x128 = 4x4 v_mfma_f32_32x32x16_{bf16,f16} tiles with its 256
// accumulators in AGPRs. K advances 64 at a time through two 64 KiB LDS
// stages:
//   * stages are fetched with buffer_load_dwordx4 ... lds: the data goes
//     HBM/L2 -> LDS without touching VGPRs, and every row of a stage is whole
//     128-byte lines (half-line rows would double the L2 -> CU traffic). A
//     16-bit operand of the other float format is converted in registers,
//     interleaved with the MFMAs of the previous k-slice;
//   * the two stages are two separate LDS variables, addressed with
//     compile-time slot numbers (the stage loop is unrolled by two), so the
//     compiler can see that reading one stage never aliases the DMA still
//     filling the other and does not wait on it; barriers are plain s_barrier
//     (no release fence, which would wait for every load in flight);
//   * one barrier per stage, after three of its four 16-deep k-slices: by
//     then the next stage has landed and every wave holds the last slice's
//     fragments, so the stage two ahead is issued into the freed slot and the
//     next stage's first fragments are read while the fourth slice's MFMAs run;
//   * the k-slices are laid out instruction by instruction: after each MFMA
//     comes at most one LDS read of the next slice's fragments (in the order
//     its MFMAs need them), one memory load and, for converting kinds, one
//     fragment's conversion, each fenced so the compiler keeps the order;
//   * K-contiguous operand in LDS: a tile row is 8 chunks of 16 B; logical
//     chunk c of row r sits at chunk c ^ ((r >> 1) & 7). A fragment read
//     touches 16 consecutive rows at one logical chunk per LDS cycle, which
//     this spreads over all 64 banks;
//   * k-major operand (stored [K][M or N]) in LDS: 64 k-rows of 256 values;
//     each wave-wide DMA load fills 1 KiB = two k-rows, in which the 16-B
//     chunk (row bit rb, column half h, 32-column block ib, chunk j) sits at
//     slot 16 ib + 4 ((2 h + rb) ^ 2 p) + j, p = bit 1 of the row. Fragments
//     come out with ds_read_b64_tr_b16, which hands each lane four k-values
//     of one column: one read covers four k-rows, which this layout puts on
//     distinct banks, and the 32-column blocks sit 256 B apart, so every read
//     of a slice is one lane address plus a constant.
// Epilogue: accumulators go through the freed LDS stage so that the outputs
// leave in whole rows, 16 B per lane, while the next tile's first stage
// streams into the other one.
// Persistent: one workgroup per CU walks the tile list that it derives on the
// device from offsets[] (no host read-back). The list is cut into eight
// contiguous ranges, one per XCD, so an XCD owns one or a few experts: their
// weights and rows come from HBM about once and are reused from that XCD's
// L2, and within the XCD the workgroups take consecutive tiles. Row-segmented
// lists run expert, n-panel, m-tile and are cut into equal tile counts; when
// the last round of an XCD has fewer tiles than workgroups, those tiles are
// split along K over the idle workgroups (needs the workspace): each piece
// stores its float32 partial sum, and a second kernel adds the pieces up in
// split order and applies the epilogue. K-segmented lists run expert, group of eight m-tiles, n-tile,
// m-tile (a round of an XCD's 32 workgroups then shares eight A and four B
// blocks; measured best against groups of 4 and 16) and are cut into equal
// shares of k-steps, since an expert's tiles cost its row count.
#include "ffn_common.h"

namespace moe {
namespace {

using namespace ffn;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int BM = 256, BN = 256, BK = 64, NS = 2;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int WM = 2, WN = 2;
constexpr int MI = BM / WM / 32, NI = BN / WN / 32;
constexpr int kCpr = BK / 8;                            // 16-B chunks per tile row (8)
constexpr int kRowsPerLoad = kWave / kCpr;              // rows per wave-wide 16-B load (8)
constexpr int kLoadsA = BM / kRowsPerLoad / kWaves;     // LDS-DMA loads per wave per stage (8)
constexpr int kLoadsB = BN / kRowsPerLoad / kWaves;
constexpr int kStage = (BM + BN) * kCpr;                // uint4 per stage (64 KiB)
constexpr uint32_t kBRegion = BM * kCpr * 16;           // byte offset of the B half of a stage
static_assert(NS == 2 && BK == 64 && kWaves % 2 == 0, "the pipeline below assumes these");
static_assert(BM == 256 && BN == 256, "the k-major LDS layout assumes 256-wide tiles");
constexpr size_t kPartBytes = static_cast<size_t>(BM) * BN * sizeof(float);   // one split partial
constexpr int kMaxSplit = 8;
constexpr int kEpiCost = 4;   // epilogue of a tile, in k-steps (K-segmented load balance)
constexpr int kSegGroup = 8;  // m-tiles per group of the K-segmented tile order
constexpr int kEpiPitch = 136;   // floats per row of a wave's epilogue staging buffer (see epilogue_wave)

// s_waitcnt with vmcnt = n (0..62; bits 3:0 and 15:14), expcnt and lgkmcnt not waited on.
#define MOE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
#define MOE_BARRIER()                                       \
  do {                                                      \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      \
    __builtin_amdgcn_s_barrier();                           \
    asm volatile("" ::: "memory");                          \
  } while (0)

enum Cvt { kCvtNone, kCvtBf16ToF16, kCvtF16ToBf16 };
enum Epi { kEpiGelu, kEpiF32, kEpiDGelu };

// One kind of product: operand layouts (k-major = stored [K][M or N]), the
// tile list (row- or K-segmented), the MFMA input type, the conversion of B
// and the epilogue.
// GATHER: A's rows are read through a row map (A row r = token gsrc[r]).
template <bool A_KM, bool B_KM, bool SEG_K, bool F16, int CVT_B, int EPI, bool SAVE_Z, bool GATHER = false>
struct GemmOp {
  static constexpr bool kAKM = A_KM, kBKM = B_KM, kSegK = SEG_K, kF16 = F16, kSaveZ = SAVE_Z;
  static constexpr bool kGather = GATHER;
  static constexpr int kCvt = CVT_B, kEpi = EPI;
};
using OpUp = GemmOp<false, false, false, false, kCvtNone, kEpiGelu, false>;
using OpUpG = GemmOp<false, false, false, false, kCvtNone, kEpiGelu, false, true>;
using OpUpZ = GemmOp<false, false, false, false, kCvtNone, kEpiGelu, true>;
using OpDown = GemmOp<false, false, false, true, kCvtBf16ToF16, kEpiF32, false>;
using OpDownF16 = GemmOp<false, false, false, true, kCvtNone, kEpiF32, false>;
using OpDh = GemmOp<false, true, false, false, kCvtNone, kEpiDGelu, false>;
using OpDx = GemmOp<false, true, false, false, kCvtNone, kEpiF32, false>;
using OpDw2 = GemmOp<true, true, true, false, kCvtF16ToBf16, kEpiF32, false>;
using OpDw1 = GemmOp<true, true, true, false, kCvtNone, kEpiF32, false>;

typedef unsigned int u32x4v __attribute__((__vector_size__(16)));

// 16-byte buffer store; a lane whose offset is past the buffer's range stores nothing.
__device__ __forceinline__ void store16(const uint4& v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const u32x4v x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, 0, 0);
}

struct Ctx {
  __amdgpu_buffer_rsrc_t a, b;
  int m0, n0, seg1, e;
  uint32_t ga[kLoadsA];   // gathered A: this lane's row byte offsets, one per A load of a stage
};

// Four consecutive k-values of one column from the k-major LDS tile (see the
// layout above); `p` is this lane's address.
__device__ __forceinline__ uint2 ds_read_tr(const char* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Byte offset, within a k-major operand's half of a stage, of the 8 bytes
// this lane gives to ds_read_b64_tr_b16 for k-slice 0, first k-quad, column
// block 0 of column half `hx`. Lane l = 16 g + s reads k-row
// 8 (g >> 1) + (s >> 2) at columns 128 hx + 16 (g & 1) + 4 (s & 3) .. +3, so
// that after the transpose lane l holds column l % 32 at k-rows
// 8 (l / 32) .. +3, the MFMA operand layout. Slice kk, quad h2 and block ib
// add 8192 kk + 2048 h2 + 256 ib.
__device__ __forceinline__ uint32_t kmajor_lane_offset(int lane, int hx) {
  const int g = lane >> 4, s = lane & 15;
  const int blk = 4 * (g >> 1) + (s >> 3);
  const int rb = (s >> 2) & 1, p = (s >> 3) & 1;
  const int slot = 4 * ((2 * hx + rb) ^ (2 * p)) + 2 * (g & 1) + ((s & 3) >> 1);
  return static_cast<uint32_t>(blk * 1024 + slot * 16 + (s & 1) * 8);
}

// Per-lane global byte offset of a wave-wide LDS-DMA load of a k-major
// operand: lane L lands at slot L of the 1 KiB block, i.e. k-row rb of the
// block's two, logical chunk 16 h + 4 ib + j (see the layout above); p is bit
// 1 of the block's first k-row, the parity of the block index.
__device__ __forceinline__ uint32_t kmajor_dma_offset(int lane, int p, uint32_t row_bytes) {
  const int ib = lane >> 4, f = (lane >> 2) & 3, j = lane & 3;
  const int g2 = f ^ (2 * p);
  const int h = g2 >> 1, rb = g2 & 1;
  return static_cast<uint32_t>(rb) * row_bytes + static_cast<uint32_t>(16 * h + 4 * ib + j) * 16u;
}

// K-segmented lists: k-steps of expert e, rounded up to the even count the
// stage pairs need (two all-zero stages for an expert with no rows).
__device__ __forceinline__ int seg_k_steps(const int* s_off, int e) {
  const int nk = (s_off[e + 1] - s_off[e] + BK - 1) / BK;
  return max(2, (nk + 1) & ~1);
}

// VPC consecutive outputs at element offset `at` (and of Z), given as floats
// (b holds values 4..7 when VPC is 8): GELU -> fp16 (and the fp16
// pre-activation); f32; or the GELU backward: bf16(value * gelu'(z)) with z
// read from Z.
template <class Op>
__device__ __forceinline__ void emit_values(void* Cout, uint16_t* Z, int64_t at, const float4& a,
                                            const float4& b) {
  if constexpr (Op::kEpi == kEpiGelu) {
    const f16x2 p0 = {static_cast<_Float16>(gelu_tanh_fast(a.x)), static_cast<_Float16>(gelu_tanh_fast(a.y))};
    const f16x2 p1 = {static_cast<_Float16>(gelu_tanh_fast(a.z)), static_cast<_Float16>(gelu_tanh_fast(a.w))};
    const f16x2 p2 = {static_cast<_Float16>(gelu_tanh_fast(b.x)), static_cast<_Float16>(gelu_tanh_fast(b.y))};
    const f16x2 p3 = {static_cast<_Float16>(gelu_tanh_fast(b.z)), static_cast<_Float16>(gelu_tanh_fast(b.w))};
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(Cout) + at) =
        uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
              __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    if constexpr (Op::kSaveZ) {
      const f16x2 z0 = {static_cast<_Float16>(a.x), static_cast<_Float16>(a.y)};
      const f16x2 z1 = {static_cast<_Float16>(a.z), static_cast<_Float16>(a.w)};
      const f16x2 z2 = {static_cast<_Float16>(b.x), static_cast<_Float16>(b.y)};
      const f16x2 z3 = {static_cast<_Float16>(b.z), static_cast<_Float16>(b.w)};
      *reinterpret_cast<uint4*>(Z + at) =
          uint4{__builtin_bit_cast(uint32_t, z0), __builtin_bit_cast(uint32_t, z1),
                __builtin_bit_cast(uint32_t, z2), __builtin_bit_cast(uint32_t, z3)};
    }
  } else if constexpr (Op::kEpi == kEpiDGelu) {
    const uint4 zr = *reinterpret_cast<const uint4*>(Z + at);
    const f16x2 z0 = __builtin_bit_cast(f16x2, zr.x), z1 = __builtin_bit_cast(f16x2, zr.y);
    const f16x2 z2 = __builtin_bit_cast(f16x2, zr.z), z3 = __builtin_bit_cast(f16x2, zr.w);
    const bf16x2 q0 = {static_cast<__bf16>(a.x * gelu_tanh_grad_fast(static_cast<float>(z0[0]))),
                       static_cast<__bf16>(a.y * gelu_tanh_grad_fast(static_cast<float>(z0[1])))};
    const bf16x2 q1 = {static_cast<__bf16>(a.z * gelu_tanh_grad_fast(static_cast<float>(z1[0]))),
                       static_cast<__bf16>(a.w * gelu_tanh_grad_fast(static_cast<float>(z1[1])))};
    const bf16x2 q2 = {static_cast<__bf16>(b.x * gelu_tanh_grad_fast(static_cast<float>(z2[0]))),
                       static_cast<__bf16>(b.y * gelu_tanh_grad_fast(static_cast<float>(z2[1])))};
    const bf16x2 q3 = {static_cast<__bf16>(b.z * gelu_tanh_grad_fast(static_cast<float>(z3[0]))),
                       static_cast<__bf16>(b.w * gelu_tanh_grad_fast(static_cast<float>(z3[1])))};
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(Cout) + at) =
        uint4{__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
              __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3)};
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(Cout) + at) = a;
  }
}

template <class Op>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E, int M, int N,
    int K, const uint16_t* __restrict__ B, void* __restrict__ Cout, uint16_t* __restrict__ Z,
    float* __restrict__ part, int max_split, const int32_t* __restrict__ gsrc, int a_bytes) {
  constexpr bool AKM = Op::kAKM, BKM = Op::kBKM, SEGK = Op::kSegK, F16 = Op::kF16;
  constexpr bool GATHER = Op::kGather;
  static_assert(!GATHER || (!AKM && !SEGK), "the row map applies to a K-contiguous, row-segmented A");
  constexpr int CVT = Op::kCvt, EPI = Op::kEpi;
  // Both operands K-contiguous: chunks past K hold the next row's values and
  // are zeroed; a k-major operand reads zeros past K (the buffer ends there),
  // which cancels whatever finite values the other operand holds.
  constexpr bool ZERO_TAIL = !AKM && !BKM;
  // Output: VPC consecutive values per 16-byte store.
  constexpr int VPC = EPI == kEpiF32 ? 4 : 8;
  constexpr int OUT_BYTES = EPI == kEpiF32 ? 4 : 2;
  constexpr int ITEMS = 8 * (BN / WN) / VPC / kWave;              // 16-B items per lane per chunk
  constexpr int NST = MI * 4 * ITEMS * (Op::kSaveZ ? 2 : 1);      // stores per lane per tile
  static_assert(ITEMS * VPC * kWave == 8 * (BN / WN), "a chunk is 8 rows of the quadrant");
  constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
  // A steady stage's loads leave in three parts: kSpread0 between the MFMAs
  // after the stage barrier, kSpreadPer in each of the next two k-slices, so
  // the TA queue does not fill and hold up the MFMA issue behind it. Measured
  // per kind: 8/4/4 for the plain and k-major-B kinds, 12/2/2 for the
  // converting down-projection (its slices carry the conversion VALU work);
  // the K-segmented kinds (short tiles of both-k-major operands) issue the
  // whole stage at the barrier.
  constexpr int kSpread0 = SEGK ? kLoadsPerStage : (CVT != kCvtNone ? 12 : kLoadsPerStage / 2);
  constexpr int kSpreadPer = (kLoadsPerStage - kSpread0) / 2;
  static_assert(kSpread0 + 2 * kSpreadPer == kLoadsPerStage, "the parts cover the stage");
  // After a per-wave epilogue the memory operations in flight are, oldest
  // first: the next unit's stage klo, its stage klo+1, then the NST stores.
  constexpr int kWaitFirstStage = kLoadsPerStage + NST < 62 ? kLoadsPerStage + NST : 62;
  constexpr int kWaitAfterStores = NST < 62 ? NST : 62;
  __shared__ uint4 st0[kStage];
  __shared__ uint4 st1[kStage];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_tmp[kMaxE];
  __shared__ long long s_cost[SEGK ? kMaxE + 1 : 1];
  __shared__ float s_epi[kWaves][8 * kEpiPitch];   // per-wave epilogue staging
  // Stage slot S (0 or 1, a compile-time value at every use).
  auto L = [&](int S) -> uint4* { return S ? st1 : st0; };
  const int tid = threadIdx.x;

  for (int e = tid; e <= E; e += kThreads) s_off[e] = offsets[e];
  if constexpr (!SEGK) build_tile_prefix(offsets, E, BM, s_pref, s_tmp);
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = SEGK ? (M + BM - 1) / BM : 0;
  const int tpe = tiles_m * tiles_n;   // K-segmented: tiles per expert
  const int nk = SEGK ? 0 : (K + BK - 1) / BK;
  const int nk2 = (nk + 1) & ~1;     // stages run in pairs; a padding stage is all zeros
  const int kz = ZERO_TAIL ? K / BK : 0x7fffffff;   // first stage with columns past K
  const int P = gridDim.x >> 3;   // the grid is a multiple of 8
  const int xcd = blockIdx.x & 7, w = blockIdx.x >> 3;
  // Row-segmented: the tile list is cut into 8 equal contiguous ranges, one
  // per XCD (workgroup b runs on XCD b % 8); the XCD's P workgroups take the
  // range's tiles round-robin. When the last round has fewer tiles than
  // workgroups (rem < P), each of those tiles is split into S k-ranges so the
  // round keeps every workgroup busy; the split partial sums meet in `part`.
  // K-segmented: the 8 ranges hold equal shares of k-steps.
  int64_t r_beg, n_x;
  if constexpr (SEGK) {
    __syncthreads();
    if (tid == 0) {
      long long c = 0;
      for (int e = 0; e < E; ++e) {
        s_cost[e] = c;
        c += static_cast<long long>(tpe) * (seg_k_steps(s_off, e) + kEpiCost);
      }
      s_cost[E] = c;
    }
    __syncthreads();
    const long long tot = s_cost[E];
    // First tile whose cumulative cost reaches c.
    auto tile_at = [&](long long c) -> int64_t {
      if (c >= tot) return static_cast<int64_t>(E) * tpe;
      int lo = 0, hi = E;   // largest e with s_cost[e] <= c
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_cost[mid] <= c) lo = mid;
        else hi = mid;
      }
      const long long per = seg_k_steps(s_off, lo) + kEpiCost;
      return static_cast<int64_t>(lo) * tpe + (c - s_cost[lo] + per - 1) / per;
    };
    r_beg = tile_at(tot * xcd / 8);
    n_x = tile_at(tot * (xcd + 1) / 8) - r_beg;
  } else {
    const int64_t total =
        static_cast<int64_t>(__builtin_amdgcn_readfirstlane(s_pref[E])) * tiles_n;
    r_beg = total * xcd / 8;
    n_x = total * (xcd + 1) / 8 - r_beg;
  }
  const int64_t full = n_x / P;
  const int rem = static_cast<int>(n_x - full * P);
  const int S = SEGK ? 1 : row_plan(static_cast<int64_t>(s_pref[E]) * tiles_n, xcd, P, nk2, max_split).S;
  const int64_t n_units = full + (S == 1 ? (w < rem ? 1 : 0)
                                          : (w < rem * S ? 1 : 0) + (w + P < rem * S ? 1 : 0));
  if (n_units == 0) return;
  // Unit q of this workgroup: a whole tile of round q, or (q >= full) piece
  // u = (q - full) P + w of the last round: split u / rem of tile u % rem.
  struct Unit {
    int64_t tile;
    int klo, khi, tail;   // tail: the piece index u, or -1 for a whole tile
  };
  auto unit = [&](int64_t q) {
    Unit u;
    if (q < full || S == 1) {
      u.tile = r_beg + w + q * P;
      u.klo = 0;
      if constexpr (SEGK)
        u.khi = seg_k_steps(s_off, __builtin_amdgcn_readfirstlane(static_cast<int>(u.tile / tpe)));
      else
        u.khi = nk2;
      u.tail = -1;
    } else {
      const int pc = static_cast<int>(q - full) * P + w;
      const int tr = pc % rem, si = pc / rem, np = nk2 / 2;
      u.tile = r_beg + full * P + tr;
      u.klo = 2 * (si * np / S);
      u.khi = 2 * ((si + 1) * np / S);
      u.tail = pc;
    }
    return u;
  };

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hl = lane >> 5;
  // Row pitch of each operand in global memory.
  const uint32_t a_rb = static_cast<uint32_t>(AKM ? M : K) * 2u;
  const uint32_t b_rb = static_cast<uint32_t>(BKM ? N : K) * 2u;

  // LDS-DMA, K-contiguous operand: wave-wide load j of wave w fills the 8 rows
  // from 8 (4j + w); lane l lands in row + l/8 at physical chunk l%8 and
  // fetches logical chunk (l%8) ^ ((row >> 1) & 7) = (l%8) ^ (4 (w & 1) + l/16).
  // k-major operand: load j of wave w fills k-rows 2 (4j + w) and the next.
  auto dma_voff = [&](bool kmaj, uint32_t rb) -> uint32_t {
    if (kmaj) return kmajor_dma_offset(lane, wave & 1, rb);
    return (lane >> 3) * rb + (((lane & 7) ^ (((wave & 1) << 2) | (lane >> 4))) * 16u);
  };
  const uint32_t ld_voff_a = dma_voff(AKM, a_rb);
  const uint32_t ld_voff_b = dma_voff(BKM, b_rb);
  const int fr_a = (wm * (BM / WM) + l32) * kCpr;
  const int fr_b = BM * kCpr + (wn * (BN / WN) + l32) * kCpr;
  const int fr_x = hl ^ ((l32 >> 1) & 7);   // chunk (2 kk + hl) sits at (2 kk) ^ fr_x
  const uint32_t tr_a = kmajor_lane_offset(lane, wm);
  const uint32_t tr_b = kBRegion + kmajor_lane_offset(lane, wn);

  auto make_ctx = [&](int64_t tile_id, Ctx& c) {
    // Every lane computes the same tile; readfirstlane makes that visible to
    // the compiler, so the buffer resources live in SGPRs (a resource in VGPRs
    // would turn each LDS-DMA load into a waterfall loop).
    if constexpr (SEGK) {
      const int te = __builtin_amdgcn_readfirstlane(static_cast<int>(tile_id / tpe));
      const int local = static_cast<int>(tile_id - static_cast<int64_t>(te) * tpe);
      const int r0 = __builtin_amdgcn_readfirstlane(s_off[te]);
      const int rows = __builtin_amdgcn_readfirstlane(s_off[te + 1]) - r0;
      c.e = te;
      c.seg1 = M;
      // Grouped order: kSegGroup m-tiles at a time, each group sweeping the
      // n-tiles with its m-tiles inner, so a round of an XCD's workgroups
      // shares a few A and B blocks and the group's A blocks stay in L2.
      const int gm = min(kSegGroup, tiles_m - (local / (kSegGroup * tiles_n)) * kSegGroup);
      const int gbase = (local / (kSegGroup * tiles_n)) * kSegGroup;
      const int in_g = local - gbase * tiles_n;
      c.m0 = __builtin_amdgcn_readfirstlane((gbase + in_g % gm) * BM);
      c.n0 = __builtin_amdgcn_readfirstlane((in_g / gm) * BN);
      const int64_t na = max<int64_t>(0, static_cast<int64_t>(rows) * M - c.m0);
      const int64_t nb = max<int64_t>(0, static_cast<int64_t>(rows) * N - c.n0);
      c.a = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(A + static_cast<int64_t>(r0) * M + c.m0), 0, static_cast<int>(na * 2), 0x00020000);
      c.b = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(B + static_cast<int64_t>(r0) * N + c.n0), 0, static_cast<int>(nb * 2), 0x00020000);
    } else {
      const Tile tl = find_tile(s_pref, E, tiles_n, tile_id);
      const int te = __builtin_amdgcn_readfirstlane(tl.e);
      c.e = te;
      c.seg1 = __builtin_amdgcn_readfirstlane(s_off[te + 1]);
      c.m0 = __builtin_amdgcn_readfirstlane(s_off[te] + tl.mi * BM);
      c.n0 = __builtin_amdgcn_readfirstlane(tl.nt * BN);
      if constexpr (GATHER) {
        // A is the token matrix itself (a_bytes long): the tile's row i is
        // token gsrc[m0 + i]. Each lane keeps the byte offset of its row in
        // each of the stage's A loads; rows past the segment get an offset
        // past the buffer, so their loads return zeros.
        c.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, a_bytes, 0x00020000);
        const uint32_t chunk = static_cast<uint32_t>((lane & 7) ^ (((wave & 1) << 2) | (lane >> 4))) * 16u;
#pragma unroll
        for (int jj = 0; jj < kLoadsA; ++jj) {
          const int r = c.m0 + (jj * kWaves + wave) * kRowsPerLoad + (lane >> 3);
          c.ga[jj] = r < c.seg1 ? static_cast<uint32_t>(gsrc[r]) * a_rb + chunk : 0x80000000u;
        }
      } else {
        const int a_rows = min(c.seg1 - c.m0, BM);
        c.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A + static_cast<int64_t>(c.m0) * K),
                                                0, static_cast<int>(a_rows * a_rb), 0x00020000);
      }
      if constexpr (BKM) {
        // B_e is [K][N]: the tile's columns start at n0 of every k-row; the
        // buffer ends after k-row K - 1.
        const int64_t nb = static_cast<int64_t>(K) * N - c.n0;
        c.b = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(B + static_cast<int64_t>(te) * K * N + c.n0), 0, static_cast<int>(nb * 2), 0x00020000);
      } else {
        const int b_rows = min(N - c.n0, BN);
        c.b = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(B + (static_cast<int64_t>(te) * N + c.n0) * K), 0,
            static_cast<int>(b_rows * b_rb), 0x00020000);
      }
    }
  };

  // Loads j0 .. j1-1 of stage kt into slot S: the A loads are 0 .. kLoadsA-1,
  // the B loads follow.
  auto issue_range = [&](const Ctx& c, int kt, int S, int j0, int j1) __attribute__((always_inline)) {
    uint4* const dst = L(S);
#pragma unroll
    for (int jj = j0; jj < j1; ++jj) {
      if (jj < kLoadsA) {
        const int blk = jj * kWaves + wave;
        if constexpr (GATHER) {
          // the k offset goes into the lane offset, which the range check covers
          __builtin_amdgcn_raw_ptr_buffer_load_lds(c.a, (lds_ptr_t)(dst + blk * kWave), 16,
                                                   c.ga[jj] + static_cast<uint32_t>(kt) * BK * 2u, 0, 0, 0);
        } else {
          const uint32_t so = AKM ? (static_cast<uint32_t>(2 * blk + kt * BK) * a_rb)
                                  : (blk * kRowsPerLoad * a_rb + static_cast<uint32_t>(kt) * BK * 2u);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(c.a, (lds_ptr_t)(dst + blk * kWave), 16, ld_voff_a, so, 0, 0);
        }
      } else {
        const int blk = (jj - kLoadsA) * kWaves + wave;
        const uint32_t so = BKM ? (static_cast<uint32_t>(2 * blk + kt * BK) * b_rb)
                                : (blk * kRowsPerLoad * b_rb + static_cast<uint32_t>(kt) * BK * 2u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.b, (lds_ptr_t)(dst + BM * kCpr + blk * kWave), 16,
                                                 ld_voff_b, so, 0, 0);
      }
    }
  };
  auto issue = [&](const Ctx& c, int kt, int S) __attribute__((always_inline)) {
    issue_range(c, kt, S, 0, kLoadsPerStage);
  };
  // Zero the chunks of stage kt (slot S) that lie past K.
  auto zero_tail = [&](int kt, int S) __attribute__((always_inline)) {
    for (int p = tid; p < kStage; p += kThreads) {
      const int c = (p & 7) ^ ((p >> 4) & 7);
      if (kt * BK + c * 8 >= K) L(S)[p] = uint4{0, 0, 0, 0};
    }
  };

  Ctx cur;
  // A steady boundary left loads kSpread0 .. of the stage after the current one
  // for the next k-slices to issue.
  bool pend = false;
  uint4 fa[2][MI], fb[2][NI];
  auto read_frags = [&](int S, int kk, int fs) __attribute__((always_inline)) {
    // The lane terms are made opaque here so that the bases are recomputed
    // (a few adds) rather than eight of them held across the loop.
    int x = fr_x;
    asm volatile("" : "+v"(x));
    const int c = x ^ (kk * 2);
    const int ab = fr_a + c, bb = fr_b + c;
    const char* const base = reinterpret_cast<const char*>(L(S));
    if constexpr (AKM) {
      uint32_t t = tr_a;
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const char* p = base + t + kk * 8192 + i * 256;
        const uint2 lo = ds_read_tr(p), hi = ds_read_tr(p + 2048);
        fa[fs][i] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[fs][i] = L(S)[ab + i * 32 * kCpr];
    }
    if constexpr (BKM) {
      uint32_t t = tr_b;
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const char* p = base + t + kk * 8192 + j * 256;
        const uint2 lo = ds_read_tr(p), hi = ds_read_tr(p + 2048);
        fb[fs][j] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[fs][j] = L(S)[bb + j * 32 * kCpr];
    }
  };
  auto conv_fb = [&](int fs) __attribute__((always_inline)) {
    if constexpr (CVT == kCvtBf16ToF16) {
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[fs][j] = bf16x8_to_f16x8(fb[fs][j]);
    } else if constexpr (CVT == kCvtF16ToBf16) {
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[fs][j] = f16x8_to_bf16x8(fb[fs][j]);
    }
  };

  // Reads of one slice in the order the next slice's MFMAs need them (tile
  // (m / 4, m % 4) for MFMA m): A0, B0 .. B3, A1 .. A3, a k-major fragment
  // as two reads (its lower and upper four k-values).
  constexpr int kPA = AKM ? 2 : 1, kPB = BKM ? 2 : 1;
  constexpr int kNR = MI * kPA + NI * kPB;   // reads per slice
  auto read_one = [&](int S, int kk, int fs, int r) __attribute__((always_inline)) {
    const char* const base = reinterpret_cast<const char*>(L(S));
    const int c = fr_x ^ (kk * 2);
    bool isa;
    int idx, part;
    if (r < kPA) {
      isa = true, idx = 0, part = r;
    } else if (r < kPA + NI * kPB) {
      isa = false, idx = (r - kPA) / kPB, part = (r - kPA) % kPB;
    } else {
      isa = true, idx = 1 + (r - kPA - NI * kPB) / kPA, part = (r - kPA - NI * kPB) % kPA;
    }
    if (isa) {
      if constexpr (AKM) {
        const uint2 v = ds_read_tr(base + tr_a + kk * 8192 + idx * 256 + part * 2048);
        if (part == 0) fa[fs][idx].x = v.x, fa[fs][idx].y = v.y;
        else fa[fs][idx].z = v.x, fa[fs][idx].w = v.y;
      } else {
        fa[fs][idx] = L(S)[fr_a + c + idx * 32 * kCpr];
      }
    } else {
      if constexpr (BKM) {
        const uint2 v = ds_read_tr(base + tr_b + kk * 8192 + idx * 256 + part * 2048);
        if (part == 0) fb[fs][idx].x = v.x, fb[fs][idx].y = v.y;
        else fb[fs][idx].z = v.x, fb[fs][idx].w = v.y;
      } else {
        fb[fs][idx] = L(S)[fr_b + c + idx * 32 * kCpr];
      }
    }
  };
  // position of read r in a slice, and of B fragment j's conversion
  auto read_pos = [](int r) { return (r * 16) / kNR; };
  auto conv_pos = [&](int j) {
    const int last = read_pos(kPA + j * kPB + kPB - 1);   // B fragment j's last read
    return last + 6 < 16 ? last + 6 : 15;
  };

  f32x16 acc[MI][NI];
  // 16 MFMAs of set fs laid out one by one: after MFMA m (tile (m / 4, m % 4))
  // come, where the plan puts them, one read of the next slice (slot rS,
  // k-slice rkk >= 0, into set fs ^ 1), one load (ND of them, loads l0 .. of
  // stage lkt into slot lS, spread evenly) and, for converting kinds, the
  // conversion of one B fragment of set fs ^ 1 once its read has landed; each
  // piece is fenced so the compiler keeps the order.
  auto xblock = [&](int fs, int rS, int rkk, auto nd_c, int lkt, int lS, int l0) __attribute__((always_inline)) {
    constexpr int ND = decltype(nd_c)::value;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int i = m >> 2, j = m & 3;
      if constexpr (!F16)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[fs][i]),
                                                            __builtin_bit_cast(bf16x8, fb[fs][j]), acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fa[fs][i]),
                                                           __builtin_bit_cast(f16x8, fb[fs][j]), acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (rkk >= 0) {
#pragma unroll
        for (int r = 0; r < kNR; ++r)
          if (read_pos(r) == m) {
            read_one(rS, rkk, fs ^ 1, r);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      if constexpr (ND > 0) {
#pragma unroll
        for (int v = 0; v < ND; ++v)
          if ((v * 16) / ND + (ND < 16 ? 1 : 0) == m) {
            issue_range(cur, lkt, lS, l0 + v, l0 + v + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      if constexpr (CVT != kCvtNone) {
        if (rkk >= 0) {
#pragma unroll
          for (int jc = 0; jc < NI; ++jc)
            if (conv_pos(jc) == m) {
              if constexpr (CVT == kCvtBf16ToF16) fb[fs ^ 1][jc] = bf16x8_to_f16x8(fb[fs ^ 1][jc]);
              else fb[fs ^ 1][jc] = f16x8_to_bf16x8(fb[fs ^ 1][jc]);
              __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
    }
  };
  using NoLoads = std::integral_constant<int, 0>;
  using SliceLoads = std::integral_constant<int, kSpreadPer>;
  // The first three k-slices of stage kt (slot S); set 0 holds slice 0 on entry,
  // set 1 holds slice 3 on exit. PEND (compile time): the loads kSpread0 ..
  // of stage kt+1 (slot S^1) go out during slices 0 and 1.
  auto slices012 = [&](int S, int kt, auto pend_c) __attribute__((always_inline)) {
    constexpr bool PEND = decltype(pend_c)::value;
    using L01 = std::conditional_t<PEND, SliceLoads, NoLoads>;
    __builtin_amdgcn_sched_barrier(0);
    xblock(0, S, 1, L01{}, kt + 1, S ^ 1, kSpread0);
    xblock(1, S, 2, L01{}, kt + 1, S ^ 1, kSpread0 + kSpreadPer);
    xblock(0, S, 3, NoLoads{}, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Loads of stage kt+1 (slot S^1) a steady boundary left, issued at once
  // where no steady stage follows.
  auto flush_pending = [&](int kt, int S) __attribute__((always_inline)) {
    if (pend) issue_range(cur, kt + 1, S ^ 1, kSpread0, kLoadsPerStage);
    pend = false;
  };
  // The fourth slice with the next stage's first fragments read from slot
  // rS (rS < 0: none, the last slice of a unit).
  auto slice3 = [&](int rS) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    xblock(1, rS < 0 ? 0 : rS, rS < 0 ? -1 : 0, NoLoads{}, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // After the stage barrier: the fourth slice's 16 MFMAs (fragment set 1) with
  // the first kSpread0 loads of stage kt+2 and the reads of the next stage's
  // first fragments (set 0) issued between them, so the matrix unit is not
  // idle while the wave issues the loads; converting kinds convert set 0 in
  // the second half, once its reads have landed. The rest of stage kt+2
  // follows during the next stage's first two slices.
  auto boundary = [&](int kt, int S) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    xblock(1, S ^ 1, 0, std::integral_constant<int, kSpread0>{}, kt + 2, S, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Steady stage: stage kt+1 needs no zero fill and stage kt+2 belongs to this tile.
  auto steady = [&](int kt, int S) __attribute__((always_inline)) {
    slices012(S, kt, std::true_type{});
    MOE_WAIT_VM(0);   // stage kt+1 has landed (the only one in flight)
    MOE_BARRIER();    // ... for every wave, and every wave is done with slot S
    boundary(kt, S);
  };
  // The first stage of a unit that follows a per-wave epilogue: stage kt+1 was
  // issued before that epilogue's NST stores, so waiting until at most NST
  // memory operations are in flight is enough (the stores drain meanwhile).
  auto steady_relaxed = [&](int kt, int S) __attribute__((always_inline)) {
    slices012(S, kt, std::false_type{});
    MOE_WAIT_VM(kWaitAfterStores);
    MOE_BARRIER();
    boundary(kt, S);
  };
  // Any stage before the last two: zero-fills stage kt+1 where it passes K.
  auto stage = [&](int kt, int S) __attribute__((always_inline)) {
    flush_pending(kt, S);
    slices012(S, kt, std::false_type{});
    MOE_WAIT_VM(0);
    MOE_BARRIER();
    if (kt + 1 >= kz) {
      zero_tail(kt + 1, S ^ 1);
      MOE_BARRIER();
    }
    issue(cur, kt + 2, S);
    slice3(S ^ 1);
  };

  auto emit = [&](int c_e, int grow, int gcol, const float4& a, const float4& b) {
    const int64_t at = (SEGK ? static_cast<int64_t>(c_e) * M + grow : static_cast<int64_t>(grow)) * N + gcol;
    emit_values<Op>(Cout, Z, at, a, b);
  };
  // Epilogue through LDS slot 1 in four passes of 64 rows: a pass first copies
  // the raw f32 accumulators of its rows into LDS (no arithmetic, so the 256
  // accumulators need no extra registers), then a compact loop reads them back
  // as whole rows: either the tile's output (emit), or, for a split tile, this
  // split's partial sum into its slot of `part` (row-major 256 x 256 f32).
  // Staged element (row, col) of a 128-column half sits at column
  // col ^ (32 * ((row >> 2) & 1)), so the two half-waves of a write (rows r
  // and r + 4) land on different banks.
  // split_fixup_kernel later adds a split tile's S partials up in split
  // order (the sum does not depend on which piece finished last) and emits it.
  auto epilogue = [&](int c_m0, int c_n0, int c_seg1, int c_e, int tail) {
    float* const h0 = reinterpret_cast<float*>(st1);
    float* const h1 = reinterpret_cast<float*>(st1 + kStage / 2);
    float* const hw = wn == 0 ? h0 : h1;   // this wave's 128-column half
    float* const mine = part + static_cast<int64_t>(xcd * kPiecesPerWg * P + tail) * (BM * BN);
#pragma unroll
    for (int p = 0; p < BM / 64; ++p) {
      if (wm == p / 2) {
        // For this lane's column block j the staged position is one of two
        // bases plus a constant.
        int be = l32 + hl * (4 * 128 + 32), bo = l32 + hl * (4 * 128 - 32);
        asm volatile("" : "+v"(be), "+v"(bo));
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * (p & 1) + ii;
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              hw[((j & 1) ? bo : be) + (ii * 32 + (r >> 2) * 8 + (r & 3)) * 128 + j * 32] = acc[i][j][r];
        }
      }
      MOE_BARRIER();
      if (tail < 0) {
#pragma unroll 1
        for (int q = tid; q < 64 * BN / VPC; q += kThreads) {
          const int row = q / (BN / VPC);
          const int col = (q % (BN / VPC)) * VPC;   // 0..255, multiple of VPC
          const int grow = c_m0 + p * 64 + row;
          const int gcol = c_n0 + col;
          if (grow >= c_seg1 || gcol >= N) continue;
          const float* src = (col < 128 ? h0 : h1) + row * 128 + ((col & 127) ^ (((row >> 2) & 1) * 32));
          const float4 a = *reinterpret_cast<const float4*>(src);
          const float4 b = VPC == 8 ? *reinterpret_cast<const float4*>(src + 4) : a;
          emit(c_e, grow, gcol, a, b);
        }
      } else {
#pragma unroll 4
        for (int q = tid; q < 64 * BN / 4; q += kThreads) {
          const int row = q / (BN / 4);
          const int col = (q % (BN / 4)) * 4;
          if (c_m0 + p * 64 + row >= c_seg1) continue;   // rows past the segment: never read back
          const float* src = (col < 128 ? h0 : h1) + row * 128 + ((col & 127) ^ (((row >> 2) & 1) * 32));
          *reinterpret_cast<float4*>(mine + (p * 64 + row) * BN + col) = *reinterpret_cast<const float4*>(src);
        }
      }
      MOE_BARRIER();
    }
  };

  // Per-wave epilogue of a whole (unsplit) tile: each wave stages its
  // 128 x 128 quadrant through its own LDS buffer, eight rows at a time (no
  // workgroup barrier), and writes whole output rows with 16-byte buffer
  // stores. Lanes outside the output get an offset past the buffer's range and
  // are dropped by the hardware, so every wave issues exactly NST stores, which
  // the next unit's first waits count on. Staged element (row, col) of a chunk
  // sits at row * kEpiPitch + col: the half-waves of a write (rows r and r + 4)
  // are 32 banks apart.
  auto epilogue_wave = [&](int c_m0, int c_n0, int c_seg1, int c_e) {
    float* const buf = s_epi[wave];
    // An opaque copy of the lane index: the per-item offsets below are then
    // recomputed in each epilogue instead of being hoisted out of the unit
    // loop (dozens of them, which would spill).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int el32 = ln & 31, ehl = ln >> 5;
    const int rows_ok = min(c_seg1 - c_m0, BM), cols_ok = min(N - c_n0, BN);
    const int64_t base = (SEGK ? static_cast<int64_t>(c_e) * M + c_m0 : static_cast<int64_t>(c_m0)) * N + c_n0;
    const int nrec = rows_ok * N * OUT_BYTES;
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(Cout) + base * OUT_BYTES, 0, nrec, 0x00020000);
    __amdgpu_buffer_rsrc_t zr = out;
    if constexpr (Op::kSaveZ || EPI == kEpiDGelu)
      zr = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(Z) + base * 2, 0, rows_ok * N * 2, 0x00020000);
    // Chunk k = 4 i + c: rows 32 i + 8 c .. +7 of this wave's quadrant. Item q
    // of a lane: staged row `row`, column `col` of the chunk.
    auto item_row = [&](int q) { const int f = ln + kWave * q; return VPC == 4 ? (f >> 5) : (f >> 4); };
    auto item_col = [&](int q) { const int f = ln + kWave * q; return VPC == 4 ? ((f & 31) << 2) : ((f & 15) << 3); };
    auto item_voff = [&](int k, int q) -> uint32_t {
      const int trow = wm * (BM / WM) + 8 * k + item_row(q), tcol = wn * (BN / WN) + item_col(q);
      return (trow < rows_ok && tcol < cols_ok) ? static_cast<uint32_t>((trow * N + tcol) * OUT_BYTES)
                                                : 0x80000000u;
    };
    // GELU backward: z of chunk k is loaded two chunks ahead, so each load is
    // issued before the stores it would otherwise wait behind.
    constexpr int ZD = EPI == kEpiDGelu ? 2 : 0;
    constexpr int ZN = EPI == kEpiDGelu ? MI * 4 : 1;
    uint4 zv[ZN][ITEMS];
    auto load_z = [&](int k) {
      if constexpr (EPI == kEpiDGelu) {
#pragma unroll
        for (int q = 0; q < ITEMS; ++q)
          zv[k][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(zr, item_voff(k, q), 0, 0));
      }
    };
#pragma unroll
    for (int k = 0; k < ZD; ++k) load_z(k);
#pragma unroll
    for (int k = 0; k < MI * 4; ++k) {
      const int i = k >> 2, c = k & 3;
      if (k + ZD < MI * 4) load_z(k + ZD);
      if constexpr (EPI == kEpiDGelu) __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead
      // register 4 c + rr of block (i, j) holds row 4 hl + rr of the chunk, column 32 j + l32
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          buf[(4 * ehl + rr) * kEpiPitch + 32 * j + el32] = acc[i][j][4 * c + rr];
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        const int row = item_row(q), col = item_col(q);
        const float4 a = *reinterpret_cast<const float4*>(buf + row * kEpiPitch + col);
        const float4 b = VPC == 8 ? *reinterpret_cast<const float4*>(buf + row * kEpiPitch + col + 4) : a;
        const uint32_t voff = item_voff(k, q);
        if constexpr (EPI == kEpiGelu) {
          const f16x2 p0 = {static_cast<_Float16>(gelu_tanh_fast(a.x)), static_cast<_Float16>(gelu_tanh_fast(a.y))};
          const f16x2 p1 = {static_cast<_Float16>(gelu_tanh_fast(a.z)), static_cast<_Float16>(gelu_tanh_fast(a.w))};
          const f16x2 p2 = {static_cast<_Float16>(gelu_tanh_fast(b.x)), static_cast<_Float16>(gelu_tanh_fast(b.y))};
          const f16x2 p3 = {static_cast<_Float16>(gelu_tanh_fast(b.z)), static_cast<_Float16>(gelu_tanh_fast(b.w))};
          store16(uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                        __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)},
                  out, voff);
          if constexpr (Op::kSaveZ) {
            const f16x2 z0 = {static_cast<_Float16>(a.x), static_cast<_Float16>(a.y)};
            const f16x2 z1 = {static_cast<_Float16>(a.z), static_cast<_Float16>(a.w)};
            const f16x2 z2 = {static_cast<_Float16>(b.x), static_cast<_Float16>(b.y)};
            const f16x2 z3 = {static_cast<_Float16>(b.z), static_cast<_Float16>(b.w)};
            store16(uint4{__builtin_bit_cast(uint32_t, z0), __builtin_bit_cast(uint32_t, z1),
                          __builtin_bit_cast(uint32_t, z2), __builtin_bit_cast(uint32_t, z3)},
                    zr, voff);
          }
        } else if constexpr (EPI == kEpiDGelu) {
          const uint4 zq = zv[k][q];
          const f16x2 z0 = __builtin_bit_cast(f16x2, zq.x), z1 = __builtin_bit_cast(f16x2, zq.y);
          const f16x2 z2 = __builtin_bit_cast(f16x2, zq.z), z3 = __builtin_bit_cast(f16x2, zq.w);
          const bf16x2 q0 = {static_cast<__bf16>(a.x * gelu_tanh_grad_fast(static_cast<float>(z0[0]))),
                             static_cast<__bf16>(a.y * gelu_tanh_grad_fast(static_cast<float>(z0[1])))};
          const bf16x2 q1 = {static_cast<__bf16>(a.z * gelu_tanh_grad_fast(static_cast<float>(z1[0]))),
                             static_cast<__bf16>(a.w * gelu_tanh_grad_fast(static_cast<float>(z1[1])))};
          const bf16x2 q2 = {static_cast<__bf16>(b.x * gelu_tanh_grad_fast(static_cast<float>(z2[0]))),
                             static_cast<__bf16>(b.y * gelu_tanh_grad_fast(static_cast<float>(z2[1])))};
          const bf16x2 q3 = {static_cast<__bf16>(b.z * gelu_tanh_grad_fast(static_cast<float>(z3[0]))),
                             static_cast<__bf16>(b.w * gelu_tanh_grad_fast(static_cast<float>(z3[1])))};
          store16(uint4{__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
                        __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3)},
                  out, voff);
        } else {
          store16(__builtin_bit_cast(uint4, a), out, voff);
        }
      }
    }
  };

  Unit u = unit(0);
  make_ctx(u.tile, cur);
  issue(cur, u.klo, 0);
  issue(cur, u.klo + 1, 1);

  bool after_wave_epi = false;   // the previous unit ended with epilogue_wave
  for (int64_t q = 0;; ++q) {
    // Stage klo of this unit has landed (after a per-wave epilogue, stage klo+1
    // and the stores may still be in flight).
    if (after_wave_epi) MOE_WAIT_VM(kWaitFirstStage);
    else MOE_WAIT_VM(0);
    MOE_BARRIER();
    if (u.klo >= kz) {
      zero_tail(u.klo, 0);
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

    const int khi = u.khi;
    int kt = u.klo;
    if (kt + 3 < khi && kt + 2 < kz) {
      steady_relaxed(kt, 0);
      steady(kt + 1, 1);
      kt += 2;
    }
    for (; kt + 3 < khi && kt + 2 < kz; kt += 2) {
      steady(kt, 0);
      steady(kt + 1, 1);
    }
    pend = kt > u.klo;   // a steady boundary came last
    for (; kt + 2 < khi; kt += 2) {
      stage(kt, 0);
      stage(kt + 1, 1);
    }
    // The last two stages (slots 0 and 1); slot 0, once free, takes the next
    // unit's first stage, slot 1 then stages this unit's outputs.
    const int m0 = cur.m0, n0 = cur.n0, seg1 = cur.seg1, te = cur.e, tail = u.tail;
    const bool has_next = q + 1 < n_units;
    flush_pending(kt, 0);
    slices012(0, kt, std::false_type{});
    MOE_WAIT_VM(0);
    MOE_BARRIER();
    if (kt + 1 >= kz) {
      zero_tail(kt + 1, 1);
      MOE_BARRIER();
    }
    if (has_next) {
      u = unit(q + 1);
      make_ctx(u.tile, cur);
      issue(cur, u.klo, 0);
    }
    slice3(1);
    slices012(1, kt + 1, std::false_type{});
    slice3(-1);

    MOE_BARRIER();   // every wave is done reading slot 1
    // A whole tile leaves through the per-wave epilogue, after the next unit's
    // second stage has been issued into slot 1; a split tile's partial sum
    // stages through slot 1 first.
    const bool wave_epi = tail < 0;
    if (wave_epi) {
      if (has_next) issue(cur, u.klo + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");   // the stores stay after those loads
      epilogue_wave(m0, n0, seg1, te);
    } else {
      epilogue(m0, n0, seg1, te, tail);
      if (has_next) issue(cur, u.klo + 1, 1);
    }
    if (!has_next) break;
    after_wave_epi = wave_epi;
  }
}

// Split tiles of a row-segmented launch (two fix-up workgroups per GEMM
// workgroup): the split tiles of XCD x's last round (rem of them) are shared
// out over the launch's workgroups b with b % 8 == x, in bands of `rows` rows
// (a power of two from 4 to 256, the smallest with which the XCD's
// gridDim / 8 workgroups cover all rem tiles):
// workgroup b takes band j % (256 / rows) of split tile j / (256 / rows),
// j = b / 8, adds its S partials in split order and emits the outputs. The
// tile list and the splits are derived from offsets[] exactly as the GEMM
// derived them (P workgroups per XCD). The kernel boundary orders the partial
// stores before these loads, so the pieces need no fence or ticket.
template <class Op>
__global__ __launch_bounds__(kThreads) void split_fixup_kernel(
    const int32_t* __restrict__ offsets, int E, int N, int K, int P, int max_split,
    const float* __restrict__ part, void* __restrict__ Cout, uint16_t* __restrict__ Z) {
  constexpr int VPC = Op::kEpi == kEpiF32 ? 4 : 8;
  constexpr int NV = VPC / 4;
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_tmp[kMaxE];
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int tiles_n = (N + BN - 1) / BN;
  const int nk2 = (((K + BK - 1) / BK) + 1) & ~1;
  // The tile count first, each wave on its own (no barrier): in launches that
  // split nothing, or where this workgroup has no band, it ends here, before
  // the tile prefix.
  int tot = 0;
  for (int e = threadIdx.x & 63; e < E; e += 64) tot += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
  const RowPlan pl = row_plan(static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tot)) * tiles_n, xcd, P, nk2,
                             max_split);
  if (pl.S == 1) return;
  const int per_xcd = static_cast<int>(gridDim.x >> 3);
  int rows = 4;
  while (rows < BM && rows * per_xcd < pl.rem * BM) rows <<= 1;
  const int bands = BM / rows, tr = j / bands, band = j % bands;
  if (tr >= pl.rem) return;
  build_tile_prefix(offsets, E, BM, s_pref, s_tmp);
  const Tile tl = find_tile(s_pref, E, tiles_n, pl.r_beg + pl.full * P + tr);
  const int e0 = offsets[tl.e], seg1 = offsets[tl.e + 1];
  const int m0 = e0 + tl.mi * BM, n0 = tl.nt * BN;
  const int r0 = band * rows;
  // a band wholly past the segment has nothing to add (its rows were not stored)
  if (m0 + r0 >= seg1) return;
  // piece si of the tile is u = si * rem + tr, at slot u of the XCD's kPiecesPerWg P
  const float* const first = part + static_cast<int64_t>(xcd * kPiecesPerWg * P + tr) * (BM * BN);
  const int64_t step = static_cast<int64_t>(pl.rem) * (BM * BN);
  const int S = pl.S;
  // Four items per thread per pass (two of the 8-value kinds), the values of
  // all S pieces loaded before any is added (the piece count is uniform, so
  // the guards are branches).
  constexpr int QU = NV == 1 ? 4 : 2;
  const int items = rows * (BN / VPC);
#pragma unroll 1
  for (int q0 = threadIdx.x; q0 < items; q0 += kThreads * QU) {
    float4 v[kMaxSplit][QU][NV];
#pragma unroll
    for (int si = 0; si < kMaxSplit; ++si) {
      if (si < S) {
#pragma unroll
        for (int u = 0; u < QU; ++u) {
          const int q = min(q0 + u * kThreads, items - 1);
          const int row = r0 + q / (BN / VPC), col = (q % (BN / VPC)) * VPC;
          const float* src = first + si * step + row * BN + col;
          const bool live = m0 + row < seg1;   // rows past the segment were not stored
#pragma unroll
          for (int h = 0; h < NV; ++h)
            v[si][u][h] = live ? *reinterpret_cast<const float4*>(src + 4 * h) : float4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int q = q0 + u * kThreads;
      const int row = r0 + q / (BN / VPC), col = (q % (BN / VPC)) * VPC;
      float4 a = v[0][u][0], b = v[0][u][NV - 1];
#pragma unroll
      for (int si = 1; si < kMaxSplit; ++si) {
        if (si < S) {
          const float4 a2 = v[si][u][0];
          a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
          if constexpr (NV == 2) {
            const float4 b2 = v[si][u][1];
            b.x += b2.x; b.y += b2.y; b.z += b2.z; b.w += b2.w;
          }
        }
      }
      const int grow = m0 + row, gcol = n0 + col;
      if (q < items && grow < seg1 && gcol < N)
        emit_values<Op>(Cout, Z, static_cast<int64_t>(grow) * N + gcol, a, b);
    }
  }
}

// One workgroup per CU, a multiple of 8 (one group per XCD).
int ffn_mfma_grid() { return (device_cu_count() + 7) / 8 * 8; }

template <class Op>
void launch_op(dim3 g, hipStream_t s, const void* A, const int32_t* offsets, int E, int M, int N,
               int K, const void* B, void* C, void* Z, float* part, int max_split,
               const int32_t* gsrc = nullptr, int a_bytes = 0) {
  hipLaunchKernelGGL(gemm_mfma_kernel<Op>, g, dim3(kThreads), 0, s, static_cast<const uint16_t*>(A),
                     offsets, E, M, N, K, static_cast<const uint16_t*>(B), C,
                     static_cast<uint16_t*>(Z), part, max_split, gsrc, a_bytes);
  // A tile can split only into pieces of >= 16 stages: with fewer than 32
  // stages per tile nothing is split and there is nothing to add up.
  const int nk2 = (((K + BK - 1) / BK) + 1) & ~1;
  if constexpr (!Op::kSegK) {
    if (max_split > 1 && nk2 >= 32)
      hipLaunchKernelGGL(split_fixup_kernel<Op>, dim3(2 * g.x), dim3(kThreads), 0, s, offsets, E, N, K,
                         static_cast<int>(g.x / 8), max_split, part, C, static_cast<uint16_t*>(Z));
  }
}

}  // namespace

hipError_t launch_split_fixup_down(const int32_t* offsets, int E, int N, int K, int grid, int max_split,
                                   const float* part, float* y, hipStream_t s) {
  hipLaunchKernelGGL(split_fixup_kernel<OpDownF16>, dim3(2 * grid), dim3(kThreads), 0, s, offsets, E, N, K, grid / 8,
                     max_split, part, y, nullptr);
  return hipGetLastError();
}

size_t ffn_mfma_workspace_bytes() {
  return static_cast<size_t>(ffn_mfma_grid()) * kPiecesPerWg * kPartBytes;
}

hipError_t launch_gemm_mfma(GemmKind kind, const void* A, const int32_t* offsets, int E,
                            int64_t rows_max, int M, int N, int K, const void* B, void* C,
                            void* Z, void* ws, hipStream_t s, const int32_t* gsrc, int64_t a_rows) {
  const bool seg_k = kind == GemmKind::kDw2 || kind == GemmKind::kDw1;
  const int grid_max = ffn_mfma_grid();
  int64_t g = grid_max;
  float* part = nullptr;
  int max_split = 1;
  if (seg_k) {
    // Every expert's M x N block is written, zeros for an expert with no rows.
    const int64_t tiles = static_cast<int64_t>(E) * ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (tiles == 0) return hipSuccess;
    if (tiles < g) g = (tiles + 7) / 8 * 8;
  } else {
    if (rows_max == 0) return hipSuccess;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t upper = (rows_max / BM + E) * tiles_n;   // >= sum_e ceil(kept_e / BM) * tiles_n
    // Split tiles need the workspace: kPiecesPerWg partial tiles per workgroup.
    if (ws != nullptr) {
      part = static_cast<float*>(ws);
      max_split = kMaxSplit;
    }
    // Without splitting, workgroups beyond the tile count would find no work;
    // with it, a short list still spreads over every XCD's workgroups.
    if (max_split == 1 && upper < g) g = (upper + 7) / 8 * 8;
  }
  const dim3 grid(static_cast<unsigned>(g));
  switch (kind) {
    case GemmKind::kUp:
      if (Z != nullptr) launch_op<OpUpZ>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, max_split);
      else launch_op<OpUp>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, max_split);
      break;
    case GemmKind::kUpGather:
      launch_op<OpUpG>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, max_split, gsrc,
                       static_cast<int>(a_rows * K * 2));
      break;
    case GemmKind::kDown: launch_op<OpDown>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, max_split); break;
    case GemmKind::kDownF16:
      launch_op<OpDownF16>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, max_split);
      break;
    case GemmKind::kDh: launch_op<OpDh>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, max_split); break;
    case GemmKind::kDx: launch_op<OpDx>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, max_split); break;
    case GemmKind::kDw2: launch_op<OpDw2>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, 1); break;
    case GemmKind::kDw1: launch_op<OpDw1>(grid, s, A, offsets, E, M, N, K, B, C, Z, part, 1); break;
  }
  return hipGetLastError();
}

}  // namespace moe

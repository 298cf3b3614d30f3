// The grouped expert FFN of bf16 layers with the activations in
// MFMA-fragment order (ETP page "ETP专家并行加速MoE模型": each expert's
// up-projection w1 and down-projection w2; EP tutorial
// "专家并行：混合专家模型的分布式训练方案", section 2.1 steps 3-4: the permuted
// tokens of each expert go through its FFN).
//
// Fragment order. The rows of each expert segment are padded to a multiple of
// 32 (padded segment e starts at row pad[e] = sum over e' < e of
// round_up(kept_e', 32)); element (padded row r, k) of an activation with K
// columns sits at
//   ((r / 32) (K / 16) + k / 16) 512 + ((r % 32) + 32 ((k / 8) % 2)) 8 + k % 8,
// so each 32-row x 16-k block is 1 KiB in the lane order of the MFMA A operand
// (lane l: row l % 32, k = 8 (l / 32) .. +7). Padding rows hold zeros. x_frag
// (K = d) feeds the up-projection, h_frag (K = d_ff) the down-projection.
//
// permute_frag_kernel writes x_frag from x and src[] (the gather of the
// permute, EP tutorial section 5.3: tokens of one expert made contiguous),
// staging 32-row x 256-column blocks in LDS so that both the row reads and
// the fragment writes are whole 16-byte-per-lane wave accesses.
//
// frag_gemm_kernel<KIND>: C = A B[e]^T over the segments, A fragment-ordered,
// B = W1 or W2 [E, N, K] K-contiguous. 256 x 256 tiles, four waves as 4 x 1
// (wave w: rows 64 w .. +63, all 256 columns, 4 x 16 accumulator tiles of
// 16 x 16, v_mfma_f32_16x16x32 on bf16 or fp16: per flop it moves half the
// accumulator data of the 32 x 32 x 16 form, and under the chip's power cap
// an MFMA-only loop of it holds a clock about 14% higher at the same issue
// rate). Each wave loads its A fragments (16 rows x 32 k: four 256-byte runs
// of the 32-row x 16-k blocks) straight into registers, four stages of
// register buffers issued three stages ahead; only B goes through LDS, in a
// ring of four 32 KiB slots filled by LDS-DMA three stages ahead. One barrier
// per 64-deep stage. The k-loop is laid out instruction by instruction: each
// MFMA is followed by at most one LDS fragment read and one memory load, so
// neither kind arrives in bursts that hold up the next MFMA. Tiles continue
// across a workgroup's units: the last three stages of a tile prefetch the
// next tile's first three, so those loads are in flight during the per-wave
// epilogue. The kinds (below) differ in the MFMA input type and the epilogue.
// The products are those of the row-major GEMM (32 x 32 x 16 MFMAs), added
// in float32; on every shape tested the results were equal to its own bit
// for bit, without a workspace.
#include "ffn_common.h"
#include "gemm_frag.h"

namespace moe {
namespace {

using namespace ffn;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef unsigned int u32x4v __attribute__((__vector_size__(16)));

constexpr int FBM = 256, FBN = 256, FBK = 64;
constexpr int kFT = 256;                       // threads
constexpr int kFW = kFT / kWave;               // waves (4)
constexpr int FMI = 4, FNI = 16;               // 16 x 16 accumulator tiles per wave (64 x 256)
constexpr int kFABuf = 4;                      // A register buffers (stages)
constexpr int kFCpr = FBK / 8;                 // 16-byte chunks per W1 row of a stage (8)
constexpr int kFSlotU4 = FBN * kFCpr;          // uint4 per LDS slot (32 KiB)
constexpr int kFBLoads = FBN / 8 / kFW;        // LDS-DMA loads per wave per stage (8)
constexpr int kFAFrag = FMI * 2;               // A fragments per wave per stage (8): 4 row blocks x 2 k-slices
constexpr int kFBRing = 4;                     // B fragments held in registers, read three ahead
constexpr int kFMf = FMI * FNI * 2;            // MFMAs per wave per stage (128)
constexpr int kFEpiP = 68;                     // floats per row of the row-major epilogue's staging (16 rows)
constexpr int kFFragP = 20;                    // the same for the fragment epilogue (32 rows)
constexpr int kFEpiFloats = 16 * kFEpiP;       // per-wave staging buffer
static_assert(32 * kFFragP <= kFEpiFloats, "one per-wave buffer serves both epilogues");
constexpr int kFragMaxSplit = 8;               // as the row-major GEMM (its fix-up kernel sums up to 8)

#define FR_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
#define FR_BARRIER()                                        \
  do {                                                      \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      \
    __builtin_amdgcn_s_barrier();                           \
    asm volatile("" ::: "memory");                          \
  } while (0)

// s_pad[e] = padded start row of segment e (e = 0..E), from offsets[]; every
// thread of the block calls. s_tmp: kMaxE ints of scratch.
__device__ void build_pad_offsets(const int32_t* __restrict__ offsets, int E, int* s_pad, int* s_tmp) {
  const int tid = threadIdx.x;
  for (int e = tid; e < kMaxE; e += blockDim.x)
    s_tmp[e] = e < E ? (offsets[e + 1] - offsets[e] + 31) / 32 * 32 : 0;
  __syncthreads();
  int* in = s_tmp;
  int* out = s_pad + 1;
  for (int o = 1; o < kMaxE; o <<= 1) {   // inclusive Hillis-Steele scan
    for (int e = tid; e < kMaxE; e += blockDim.x) out[e] = in[e] + (e >= o ? in[e - o] : 0);
    __syncthreads();
    int* t = in;
    in = out;
    out = t;
  }
  for (int e = tid; e < kMaxE; e += blockDim.x) s_pad[e + 1] = in[e];   // 8 steps: result in s_tmp
  if (tid == 0) s_pad[0] = 0;
  __syncthreads();
}

// The segment holding padded row t (a multiple of 32), found by each wave on
// its own (no barrier): lane j takes experts 4 j .. 4 j + 3 (E <= 256), sums
// their padded lengths, and a wave-wide inclusive scan gives every lane its
// range of padded rows. Returns false when t is past the last segment.
struct SegPos {
  int e, p0, seg0, kept;   // expert, t's row within the segment, its first row, its rows
};
__device__ __forceinline__ bool find_padded_segment(const int32_t* __restrict__ offsets, int E, int t, SegPos& sp) {
  const int lane = threadIdx.x & (kWave - 1);
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) o[i] = offsets[min(4 * lane + i, E)];
  int rk[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rk[i] = (o[i + 1] - o[i] + 31) & ~31;   // 0 past expert E-1: both ends are offsets[E]
    sum += rk[i];
  }
  int incl = sum;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const int v = __shfl_up(incl, dd, kWave);
    if (lane >= dd) incl += v;
  }
  const int excl = incl - sum;
  const unsigned long long hit = __ballot(excl <= t && t < incl);
  if (hit == 0) return false;
  const int L = __builtin_ctzll(hit);
  // in lane L: step over its experts that end at or before t
  int e = 4 * lane, base = excl;
  bool past = true;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    past = past && t >= base + rk[i];
    if (past) {
      base += rk[i];
      e = 4 * lane + i + 1;
    }
  }
  const int ie = e - 4 * lane;
  const int seg0 = ie == 0 ? o[0] : ie == 1 ? o[1] : ie == 2 ? o[2] : o[3];
  const int seg1 = ie == 0 ? o[1] : ie == 1 ? o[2] : ie == 2 ? o[3] : o[4];
  sp.e = __shfl(e, L, kWave);
  sp.p0 = t - __shfl(base, L, kWave);
  sp.seg0 = __shfl(seg0, L, kWave);
  sp.kept = __shfl(seg1 - seg0, L, kWave);
  return true;
}

constexpr int kPermCB = 4;   // 256-column blocks per permute workgroup

// Workgroup (b, g): padded block b (32 rows), columns 256 kPermCB g .. +256 kPermCB - 1.
// Thread t reads 16-byte chunk t % 32 of rows t / 32 + 8 u (u = 0..3) of each
// column block, all 4 kPermCB loads in flight; then, block by block, the
// 32 x 256 piece goes through LDS and leaves as 16 fragments of 1 KiB: unit l
// of fragment fs (16 columns = chunks 2 fs, 2 fs + 1) is row l % 32, chunk
// 2 fs + l / 32, and thread t writes units t % 64 of fragments t / 64 + 4 u.
__global__ __launch_bounds__(256) void permute_frag_kernel(
    const uint4* __restrict__ x, int64_t d, const int32_t* __restrict__ src,
    const int32_t* __restrict__ offsets, int E, uint4* __restrict__ x_frag) {
  __shared__ uint4 s_blk[2][32][32 + 1];   // two column blocks; +1: no bank aliasing
  const int b = blockIdx.x;
  SegPos sp;
  if (!find_padded_segment(offsets, E, b * 32, sp)) return;   // uniform over the workgroup
  const int64_t d16 = d >> 3;   // 16-byte chunks per row
  const int tid = threadIdx.x, cc = tid % 32;
  int64_t row[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = sp.p0 + tid / 32 + 8 * u;
    row[u] = p < sp.kept ? static_cast<int64_t>(src[sp.seg0 + p]) : -1;
  }
  uint4 v[kPermCB][4];
#pragma unroll
  for (int c = 0; c < kPermCB; ++c) {
    const int64_t ch = (static_cast<int64_t>(blockIdx.y) * kPermCB + c) * 32 + cc;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[c][u] = (row[u] >= 0 && ch < d16) ? x[row[u] * d16 + ch] : uint4{0, 0, 0, 0};
  }
#pragma unroll
  for (int c = 0; c < kPermCB; ++c) {
    const int64_t c0 = (static_cast<int64_t>(blockIdx.y) * kPermCB + c) * 32;   // first chunk of the block
    if (c0 >= d16) break;   // uniform
    auto& blk = s_blk[c & 1];
#pragma unroll
    for (int u = 0; u < 4; ++u) blk[tid / 32 + 8 * u][cc] = v[c][u];
    __syncthreads();   // also: every thread is done reading this buffer two blocks ago
    const int64_t frag0 = static_cast<int64_t>(b) * (d >> 4) + (c0 >> 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int fs = tid / 64 + 4 * u, l = tid % 64;
      if (c0 + 2 * fs < d16) x_frag[(frag0 + fs) * 64 + l] = blk[l % 32][2 * fs + l / 32];
    }
  }
}

// What one instance computes from a fragment-ordered A:
//   kFragUpRows: C = A W1[e]^T, bf16; h = fp16(gelu_tanh(C)) row-major [rows, N]
//   kFragUpFrag: the same h written in fragment order (padded rows; the K of
//                the down-projection is N)
//   kFragDown:   C = A W2[e]^T, fp16 A (h) and fp16 W2; y_perm f32 row-major
//                [rows, N]; with a workspace, the tiles of a short last round
//                split along K like the row-major GEMM's (same plan), their
//                f32 partial sums added by its fix-up kernel
enum FragKind { kFragUpRows, kFragUpFrag, kFragDown };

struct FCtx {
  __amdgpu_buffer_rsrc_t a, b;
  int m0, n0, seg1, pad_blk, blocks;
  int klo, khi, tail;   // the unit's stages [klo, khi); tail: split piece index, or -1
};

__device__ __forceinline__ void fr_store16(const uint4& v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff = 0) {
  const u32x4v x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, 0);
}

// One 16 x 16 x 32 MFMA accumulating in place (the accumulator tied to the
// destination in the same accumulation registers). Written as inline assembly
// because the compiler, given sixty-four 4-register accumulators, chose
// separate destination registers and moved accumulators through VGPRs in the
// loop. The compiler does not know these are MFMAs, so the kernel adds the
// wait states the hardware needs where other instructions meet them: after
// the accumulators are set to zero (before the k-loop) and before the
// epilogue reads the results.
template <bool F16>
__device__ __forceinline__ void mfma16_acc(f32x4& acc, const uint4& a, const uint4& b) {
  const u32x4v av = __builtin_bit_cast(u32x4v, a), bv = __builtin_bit_cast(u32x4v, b);
  if constexpr (F16)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(av), "v"(bv));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(av), "v"(bv));
}

// f(integral_constant<int, I>) for I = B .. E-1, in order, at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int KIND>
__global__ __launch_bounds__(kFT, 1) void frag_gemm_kernel(
    const uint16_t* __restrict__ Afrag, const int32_t* __restrict__ offsets, int E, int N, int K,
    const uint16_t* __restrict__ B, void* __restrict__ Cout, float* __restrict__ part, int max_split) {
  constexpr bool DOWN = KIND == kFragDown, HFRAG = KIND == kFragUpFrag;
  // One LDS variable per slot: with a single array the compiler cannot tell
  // the slot being read from the ones the DMA is filling and waits for all.
  __shared__ uint4 sb0[kFSlotU4];
  __shared__ uint4 sb1[kFSlotU4];
  __shared__ uint4 sb2[kFSlotU4];
  __shared__ uint4 sb3[kFSlotU4];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_pad[kMaxE + 1];
  __shared__ int s_tmp[kMaxE];
  __shared__ float s_epi[kFW][kFEpiFloats];   // per-wave epilogue staging
  auto SL = [&](int S) -> uint4* { return S == 0 ? sb0 : (S == 1 ? sb1 : (S == 2 ? sb2 : sb3)); };
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kFT) s_off[e] = offsets[e];
  build_tile_prefix(offsets, E, FBM, s_pref, s_tmp);
  build_pad_offsets(offsets, E, s_pad, s_tmp);
  const int tiles_n = (N + FBN - 1) / FBN;
  const int nk = K / FBK;   // the host checks K % 256 == 0: nk is a multiple of 4
  // Tile list as in the row-segmented GEMM: eight contiguous ranges, one per
  // XCD (workgroup b runs on XCD b % 8), taken round-robin by its P workgroups.
  // With splitting (DOWN with a workspace) the XCD's last round is cut into
  // pieces exactly as row_plan says, so the fix-up kernel finds them.
  const int P = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, w = blockIdx.x >> 3;
  const int64_t total = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(s_pref[E])) * tiles_n;
  const RowPlan pl = row_plan(total, xcd, P, nk, DOWN ? max_split : 1);
  const int S = pl.S, rem = pl.rem, nq = nk / 4;
  const int64_t full = pl.full;
  const int64_t n_units = full + (S == 1 ? (w < rem ? 1 : 0)
                                          : (w < rem * S ? 1 : 0) + (w + P < rem * S ? 1 : 0));
  if (n_units == 0) return;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint32_t b_rb = static_cast<uint32_t>(K) * 2u;
  const uint32_t a_blk = static_cast<uint32_t>(K) * 64u;   // bytes per 32-row block of x_frag
  // LDS-DMA of W1: wave-wide load j fills rows 8 (4 j + wave) + lane / 8 of
  // the slot at physical chunk lane % 8, fetching logical chunk
  // (lane % 8) ^ ((row >> 1) & 7); fragment reads undo the XOR.
  const uint32_t ld_voff_b = (lane >> 3) * b_rb + (((lane & 7) ^ (((wave & 1) << 2) | (lane >> 4))) * 16u);
  // A fragment of 16 rows x 32 k (lane l: row l % 16, k = 8 (l / 16) .. +7)
  // out of the 32-row x 16-k blocks of x_frag: the lane's 16 bytes sit at
  // unit (row % 32) + 32 ((k / 8) % 2) of 16-k block k / 16. Per lane:
  const uint32_t a_voff = (static_cast<uint32_t>((lane & 15) + 32 * ((lane >> 4) & 1)) * 16u) +
                          static_cast<uint32_t>(lane >> 5) * 1024u;
  // B fragment (16 W1 rows x 32 k: lane l row l % 16, logical chunk 4 s + l / 16)
  // in a slot: uint4 (b_base ^ 4 s) + 128 j for column block j, k-slice s.
  const int b_base = (lane & 15) * kFCpr + ((lane >> 4) ^ ((lane & 15) >> 1));

  // Unit q: a whole tile of round q, or (q >= full) piece pc = (q - full) P + w
  // of the last round: k-range pc / rem (in quads of stages) of tile pc % rem.
  auto make_ctx = [&](int64_t q, FCtx& c) {
    int64_t tile;
    int klo = 0, khi = nk, tail = -1;
    if (q < full || S == 1) {
      tile = pl.r_beg + w + q * P;
    } else {
      const int pc = static_cast<int>(q - full) * P + w;
      const int tr = pc % rem, si = pc / rem;
      tile = pl.r_beg + full * P + tr;
      klo = 4 * (si * nq / S);
      khi = 4 * ((si + 1) * nq / S);
      tail = pc;
    }
    c.klo = __builtin_amdgcn_readfirstlane(klo);
    c.khi = __builtin_amdgcn_readfirstlane(khi);
    c.tail = __builtin_amdgcn_readfirstlane(tail);
    const Tile tl = find_tile(s_pref, E, tiles_n, tile);
    const int te = __builtin_amdgcn_readfirstlane(tl.e);
    c.seg1 = __builtin_amdgcn_readfirstlane(s_off[te + 1]);
    c.m0 = __builtin_amdgcn_readfirstlane(s_off[te] + tl.mi * FBM);
    c.n0 = __builtin_amdgcn_readfirstlane(tl.nt * FBN);
    const int pad_blk = __builtin_amdgcn_readfirstlane(s_pad[te] / 32 + tl.mi * (FBM / 32));
    const int blocks = (min(c.seg1 - c.m0, FBM) + 31) / 32;
    c.pad_blk = pad_blk;
    c.blocks = blocks;
    c.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Afrag) + static_cast<int64_t>(pad_blk) * (a_blk / 2),
                                            0, static_cast<int>(blocks * a_blk), 0x00020000);
    const int b_rows = min(N - c.n0, FBN);
    c.b = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(B + (static_cast<int64_t>(te) * N + c.n0) * K),
                                            0, static_cast<int>(b_rows * b_rb), 0x00020000);
  };

  uint4 fa[kFABuf][kFAFrag];   // [stage buffer][4 s + i]: k-slice s, 16-row block i
  uint4 fb[kFBRing];           // B fragments, fragment f of a stage in fb[f % 4]
  f32x4 acc[FMI][FNI];

  // A fragment v = 4 s + i of stage kt into buffer AB: rows 16 i .. +15 of the
  // wave's 64 (32-row block 2 wave + i / 2, its half i % 2), k = 64 kt + 32 s ..
  auto issue_a = [&](const FCtx& c, int kt, auto ab_c, int v) __attribute__((always_inline)) {
    constexpr int AB = decltype(ab_c)::value;
    const int s = v >> 2, i = v & 3;
    const uint32_t so = static_cast<uint32_t>(2 * wave + (i >> 1)) * a_blk +
                        static_cast<uint32_t>(4 * kt + 2 * s) * 1024u + static_cast<uint32_t>(i & 1) * 256u;
    fa[AB][v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(c.a, a_voff, so, 0));
  };
  // W1 load j of stage kt into slot S.
  auto issue_b = [&](const FCtx& c, int kt, int S, int j) __attribute__((always_inline)) {
    const int blk = j * kFW + wave;
    const uint32_t so = blk * 8 * b_rb + static_cast<uint32_t>(kt) * FBK * 2u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.b, (lds_ptr_t)(SL(S) + blk * kWave), 16, ld_voff_b, so, 0, 0);
  };
  // B fragment f (k-slice f / 16, column block f % 16) of slot S into the ring.
  auto rd = [&](int S, int f) __attribute__((always_inline)) {
    fb[f & (kFBRing - 1)] = SL(S)[(b_base ^ ((f >> 4) << 2)) + (f & 15) * 16 * kFCpr];
  };
  // MFMA m of a stage: fragment f = m / 4 (k-slice f / 16, column block
  // f % 16) times A block i = m % 4; each B fragment feeds four MFMAs in a row.
  auto mf = [&](auto ab_c, auto m_c) __attribute__((always_inline)) {
    constexpr int AB = decltype(ab_c)::value, m = decltype(m_c)::value;
    constexpr int f = m >> 2, i = m & 3, s = f >> 4, j = f & 15;
    mfma16_acc<DOWN>(acc[i][j], fa[AB][4 * s + i], fb[f & (kFBRing - 1)]);
  };

  FCtx cur, nxt;
  make_ctx(0, cur);
  if (n_units > 1) make_ctx(1, nxt);
  else nxt = cur;   // past the last unit the prefetches re-read this one (never used)
  // Prologue: the first three stages of the first unit (klo is a multiple of
  // four, so stage kt always uses slot and A buffer kt % 4).
#pragma unroll
  for (int v = 0; v < kFAFrag; ++v) issue_a(cur, cur.klo, std::integral_constant<int, 0>{}, v);
#pragma unroll
  for (int j = 0; j < kFBLoads; ++j) issue_b(cur, cur.klo, 0, j);
#pragma unroll
  for (int v = 0; v < kFAFrag; ++v) issue_a(cur, cur.klo + 1, std::integral_constant<int, 1>{}, v);
#pragma unroll
  for (int j = 0; j < kFBLoads; ++j) issue_b(cur, cur.klo + 1, 1, j);
#pragma unroll
  for (int v = 0; v < kFAFrag; ++v) issue_a(cur, cur.klo + 2, std::integral_constant<int, 2>{}, v);
#pragma unroll
  for (int j = 0; j < kFBLoads; ++j) issue_b(cur, cur.klo + 2, 2, j);

  // Stage kt (slot and A buffer SB = kt % 4, compile time) of unit q: 128
  // MFMAs in a fixed order, each B fragment feeding four in a row (one per A
  // block). After MFMA m (m % 4 == 0) comes the read of B fragment m / 4 + 3
  // into the ring (12 MFMAs before its use; the last three of the stage are
  // the next stage's first fragments, from its slot S1), and after MFMAs 1,
  // 9, .., 89 and 116, 120, 124, 127 one memory load each of stage kt+3 of
  // unit q or, past the end, of unit q+1 (after the last unit: an in-bounds
  // stage into buffers nobody reads, so every stage issues the same 16 loads):
  // the 8 A fragments and W1 loads 0-3 before the barrier, W1 loads 4-7 after
  // it. Every piece is fenced so the compiler keeps this order. After MFMA
  // 116 each wave waits for stage kt+1, whose loads are older than the 16 of
  // stage kt+2 and the 12 of stage kt+3 issued so far and, in the first two
  // stages after a per-wave epilogue, that epilogue's NST stores; the barrier
  // then tells every wave that stage kt+1 is in LDS and that no wave reads
  // slot SB any more (its last fragment was read after MFMA 112), so the next
  // stage's fragments may be read and W1 loads may fill the slot of stage
  // kt-1 (free since the previous stage's barrier).
  int64_t q = 0;
  bool after_epi = false;
  auto stage = [&](auto sb_c, int kt) __attribute__((always_inline)) {
    constexpr int SB = decltype(sb_c)::value;
    constexpr int SN = (SB + 3) % 4;     // slot and buffer of stage kt+3 (those of kt-1)
    constexpr int S1 = (SB + 1) % 4;     // of stage kt+1
    const int kp = kt + 3;
    const bool pre_cur = kp < cur.khi;
    const FCtx pc = pre_cur ? cur : nxt;
    const int pk = pre_cur ? kp : nxt.klo + (kp - cur.khi);
    using AB = std::integral_constant<int, SB>;
    using SNc = std::integral_constant<int, SN>;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, kFMf>([&](auto m_c) __attribute__((always_inline)) {
      constexpr int m = decltype(m_c)::value;
      mf(AB{}, m_c);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m == 4 * (33 - kFBRing)) {   // before the first read of the next stage's slot
        if (after_epi && kt - cur.klo < 2) FR_WAIT_VM(60);
        else FR_WAIT_VM(28);
        FR_BARRIER();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr ((m & 3) == 0) {
        constexpr int f = (m >> 2) + kFBRing - 1;
        if constexpr (f < 32) rd(SB, f);
        else rd(S1, f - 32);
        __builtin_amdgcn_sched_barrier(0);
      }
      constexpr int v = (m < 96 && (m & 7) == 1) ? (m >> 3)                        // 0 .. 11
                        : (m == 116 || m == 120 || m == 124) ? 12 + (m - 116) / 4  // 12 .. 14
                        : m == 127 ? 15 : -1;
      if constexpr (v >= 0) {
        if constexpr (v < kFAFrag) issue_a(pc, pk, SNc{}, v);
        else issue_b(pc, pk, SN, v - kFAFrag);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };

  // Per-wave epilogues. Accumulator tile (i, j) holds rows 16 i + 4 (lane / 16)
  // + r (register r) and column 16 j + lane % 16 of the wave's 64 x 256 block.
  // Row-major outputs go through the wave's LDS buffer in chunks of 16 rows x
  // 64 columns (tiles (i, 4 g .. 4 g + 3)) and leave in whole 16-byte stores;
  // lanes outside the output get an offset past the buffer's range and are
  // dropped, so every lane issues exactly NST stores (fp16 h) or 2 NST (f32).
  constexpr int NST = 32;   // stores per lane per tile of the fp16 epilogues
  // The waits above count 32 stores after an epilogue; the f32 one issues 64
  // (the waits then also cover the oldest 32 of those stores: more waiting,
  // never less).
  auto stage_chunk = [&](float* buf, int i, int g) __attribute__((always_inline)) {
    const int el16 = lane & 15, eq = lane >> 4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) buf[(4 * eq + r) * kFEpiP + 16 * jj + el16] = acc[i][4 * g + jj][r];
  };
  // h row-major (kFragUpRows): GELU, fp16, eight values per 16-byte store.
  auto epilogue_rows_h = [&](const FCtx& c) {
    float* const buf = s_epi[wave];
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int rows_ok = min(c.seg1 - c.m0, FBM), cols_ok = min(N - c.n0, FBN);
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint16_t*>(Cout) + (static_cast<int64_t>(c.m0) * N + c.n0), 0, rows_ok * N * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < FMI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        stage_chunk(buf, i, g);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int f = ln + kWave * it;
          const int row = f >> 3, col = (f & 7) << 3;
          const float4 a = *reinterpret_cast<const float4*>(buf + row * kFEpiP + col);
          const float4 b = *reinterpret_cast<const float4*>(buf + row * kFEpiP + col + 4);
          const int trow = 64 * wave + 16 * i + row, tcol = 64 * g + col;
          const uint32_t voff = (trow < rows_ok && tcol < cols_ok)
                                    ? static_cast<uint32_t>((trow * N + tcol) * 2) : 0x80000000u;
          const f16x2 p0 = {static_cast<_Float16>(gelu_tanh_fast(a.x)), static_cast<_Float16>(gelu_tanh_fast(a.y))};
          const f16x2 p1 = {static_cast<_Float16>(gelu_tanh_fast(a.z)), static_cast<_Float16>(gelu_tanh_fast(a.w))};
          const f16x2 p2 = {static_cast<_Float16>(gelu_tanh_fast(b.x)), static_cast<_Float16>(gelu_tanh_fast(b.y))};
          const f16x2 p3 = {static_cast<_Float16>(gelu_tanh_fast(b.z)), static_cast<_Float16>(gelu_tanh_fast(b.w))};
          fr_store16(uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                           __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)},
                     out, voff);
        }
      }
  };

  // h in fragment order: each 32-row x 16-column block of h (accumulator
  // tiles (2 p, q) and (2 p + 1, q)) goes through the wave's LDS buffer (rows
  // 20 floats apart: the four row groups of a write land on distinct banks),
  // then lane l reads row l % 32, columns 8 (l / 32) .. +7 -- unit l of the
  // block -- applies GELU and fp16 and writes it with one 16-byte store (1 KiB
  // per wave store). Blocks past the padded segment are past the buffer's
  // range and dropped; rows inside the last block but past the segment hold
  // GELU(0) = 0 (their A rows are zero). 32 stores per lane per tile, as NST.
  auto epilogue_frag = [&](const FCtx& c) {
    float* const buf = s_epi[wave];
    const uint32_t h_blk = static_cast<uint32_t>(N) * 64u;   // bytes per 32-row block of h
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint16_t*>(Cout) + static_cast<int64_t>(c.pad_blk) * (h_blk / 2), 0,
        static_cast<int>(c.blocks * h_blk), 0x00020000);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int el16 = ln & 15, eq = ln >> 4;
    const uint32_t lo = static_cast<uint32_t>(ln) * 16u;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int qb = 0; qb < FNI; ++qb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          buf[(4 * eq + r) * kFFragP + el16] = acc[2 * p][qb][r];
          buf[(16 + 4 * eq + r) * kFFragP + el16] = acc[2 * p + 1][qb][r];
        }
        const float4 a = *reinterpret_cast<const float4*>(buf + (ln & 31) * kFFragP + 8 * (ln >> 5));
        const float4 b = *reinterpret_cast<const float4*>(buf + (ln & 31) * kFFragP + 8 * (ln >> 5) + 4);
        const f16x2 p0 = {static_cast<_Float16>(gelu_tanh_fast(a.x)), static_cast<_Float16>(gelu_tanh_fast(a.y))};
        const f16x2 p1 = {static_cast<_Float16>(gelu_tanh_fast(a.z)), static_cast<_Float16>(gelu_tanh_fast(a.w))};
        const f16x2 p2 = {static_cast<_Float16>(gelu_tanh_fast(b.x)), static_cast<_Float16>(gelu_tanh_fast(b.y))};
        const f16x2 p3 = {static_cast<_Float16>(gelu_tanh_fast(b.z)), static_cast<_Float16>(gelu_tanh_fast(b.w))};
        const uint32_t so = static_cast<uint32_t>(2 * wave + p) * h_blk +
                            static_cast<uint32_t>((c.n0 >> 4) + qb) * 1024u;
        fr_store16(uint4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                         __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)},
                   out, lo, so);
      }
  };

  // f32 output (down-projection): four values per 16-byte store; a split
  // piece writes its 256 x 256 partial sum (the rows inside the segment),
  // row-major, to its workspace slot xcd * 2 P + piece.
  auto epilogue_down = [&](const FCtx& c) {
    float* const buf = s_epi[wave];
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const bool piece = c.tail >= 0;
    const int pitch = piece ? FBN : N;
    // a piece stores only the rows inside the segment (the fix-up reads no others)
    const int rows_ok = min(c.seg1 - c.m0, FBM), cols_ok = piece ? FBN : min(N - c.n0, FBN);
    float* const base = piece ? part + static_cast<int64_t>(xcd * kPiecesPerWg * P + c.tail) * (FBM * FBN)
                              : static_cast<float*>(Cout) + static_cast<int64_t>(c.m0) * N + c.n0;
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(base, 0, rows_ok * pitch * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < FMI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        stage_chunk(buf, i, g);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int f = ln + kWave * it;
          const int row = f >> 4, col = (f & 15) << 2;
          const float4 a = *reinterpret_cast<const float4*>(buf + row * kFEpiP + col);
          const int trow = 64 * wave + 16 * i + row, tcol = 64 * g + col;
          const bool ok = trow < rows_ok && tcol < cols_ok;
          const uint32_t voff = ok ? static_cast<uint32_t>((trow * pitch + tcol) * 4) : 0x80000000u;
          fr_store16(uint4{__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w)},
                     out, voff);
        }
      }
  };

  for (;;) {
    // Stage 0 of this unit has landed (older than stages 1-2's loads and, after
    // an epilogue, its stores).
    if (after_epi) FR_WAIT_VM(62);
    else FR_WAIT_VM(32);
    FR_BARRIER();
#pragma unroll
    for (int f = 0; f < kFBRing - 1; ++f) rd(0, f);
#pragma unroll
    for (int i = 0; i < FMI; ++i)
#pragma unroll
      for (int j = 0; j < FNI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = cur.klo; kt < cur.khi; kt += 4) {
      // The accumulator writes that set them to zero come before the loop
      // (the compiler places them ahead of its header): wait states before
      // the first MFMAs read them.
      asm volatile("s_nop 2" ::: "memory");
      stage(std::integral_constant<int, 0>{}, kt);
      stage(std::integral_constant<int, 1>{}, kt + 1);
      stage(std::integral_constant<int, 2>{}, kt + 2);
      stage(std::integral_constant<int, 3>{}, kt + 3);
    }
    const FCtx done = cur;
    ++q;
    const bool has_next = q < n_units;
    __builtin_amdgcn_sched_barrier(0);
    // the last MFMAs' results are complete before the epilogue reads them
    // (more wait states than the longest 16 x 16 x 32 MFMA needs)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // also: the stores stay after the prefetches
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KIND == kFragUpRows) epilogue_rows_h(done);
    else if constexpr (HFRAG) epilogue_frag(done);
    else epilogue_down(done);
    if (!has_next) {
      FR_WAIT_VM(0);   // the last prefetches (some into LDS) end before the workgroup
      break;
    }
    cur = nxt;
    if (q + 1 < n_units) make_ctx(q + 1, nxt);
    else nxt = cur;
    after_epi = true;
  }
}

}  // namespace

// One workgroup per CU (a multiple of 8); without splitting, no more than the
// tile count needs.
dim3 frag_grid(int64_t rows_max, int E, int64_t n, bool split) {
  int64_t g = (device_cu_count() + 7) / 8 * 8;
  const int64_t upper = (rows_max / FBM + E) * ((n + FBN - 1) / FBN);   // >= the tile count
  if (!split && upper < g) g = (upper + 7) / 8 * 8;
  return dim3(static_cast<unsigned>(g));
}

int64_t frag_rows(int64_t rows_max, int E) { return (rows_max + 31 * static_cast<int64_t>(E) + 31) / 32 * 32; }

hipError_t launch_permute_frag(const void* x, int64_t d, const int32_t* src, const int32_t* offsets,
                               int E, int64_t rows_max, void* x_frag, hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(frag_rows(rows_max, E) / 32),
               static_cast<unsigned>((d + 256 * kPermCB - 1) / (256 * kPermCB)));
  hipLaunchKernelGGL(permute_frag_kernel, g, dim3(256), 0, s, static_cast<const uint4*>(x), d, src, offsets, E,
                     static_cast<uint4*>(x_frag));
  return hipGetLastError();
}

hipError_t launch_up_gelu_frag(const void* x_frag, const int32_t* offsets, int E, int64_t rows_max, int64_t d,
                               int64_t d_ff, const void* w1, void* h, bool h_frag_order, hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  const dim3 g = frag_grid(rows_max, E, d_ff, false);
  if (h_frag_order)
    hipLaunchKernelGGL(frag_gemm_kernel<kFragUpFrag>, g, dim3(kFT), 0, s, static_cast<const uint16_t*>(x_frag), offsets,
                       E, static_cast<int>(d_ff), static_cast<int>(d), static_cast<const uint16_t*>(w1), h, nullptr, 1);
  else
    hipLaunchKernelGGL(frag_gemm_kernel<kFragUpRows>, g, dim3(kFT), 0, s, static_cast<const uint16_t*>(x_frag), offsets,
                       E, static_cast<int>(d_ff), static_cast<int>(d), static_cast<const uint16_t*>(w1), h, nullptr, 1);
  return hipGetLastError();
}

hipError_t launch_down_frag(const void* h_frag, const int32_t* offsets, int E, int64_t rows_max, int64_t d,
                            int64_t d_ff, const void* w2_f16, float* y_perm, void* ws, hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  const bool split = ws != nullptr;
  const dim3 g = frag_grid(rows_max, E, d, split);
  const int max_split = split ? kFragMaxSplit : 1;
  hipLaunchKernelGGL(frag_gemm_kernel<kFragDown>, g, dim3(kFT), 0, s, static_cast<const uint16_t*>(h_frag), offsets, E,
                     static_cast<int>(d), static_cast<int>(d_ff), static_cast<const uint16_t*>(w2_f16), y_perm,
                     static_cast<float*>(ws), max_split);
  // pieces are at least 16 stages: with fewer than 32 stages nothing splits
  if (split && d_ff / FBK >= 32) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_fixup_down(offsets, E, static_cast<int>(d), static_cast<int>(d_ff), static_cast<int>(g.x),
                                   max_split, static_cast<const float*>(ws), y_perm, s);
  }
  return hipGetLastError();
}

}  // namespace moe

/*
 * moe.h -- C ABI of the single-GPU Mixture-of-Experts layer, forward and
 *          backward (gfx950 / CDNA4, HIP).
 *
 * The layer replaces a Transformer FFN with a gate, a set of expert FFNs and
 * sparse top-K activation (EP tutorial "专家并行：混合专家模型的分布式训练方案",
 * section 1.1). One forward is five calls, in the order the pages give:
 *
 *   moe_router_topk  gate linear -> softmax -> top-k          (tutorial 1.1, 2.1 step 1;
 *                    deployment guide "细粒度专家并行部署实践与优化指南", section 5 step 3)
 *   moe_dispatch     capacity-limited dispatch plan + permute  (tutorial 2.1 step 2, 2.2, 5.3)
 *   moe_grouped_ffn  per-expert up-proj, GELU-tanh, down-proj  (ETP page "ETP专家并行加速MoE模型",
 *                    the w1 / w2 up- and down-projection example; tutorial 2.1 step 4)
 *   moe_combine      weighted return to token order            (tutorial 2.1 step 5)
 *   moe_aux_loss     L_aux = alpha * E * sum_i f_i * P_i       (tutorial 5.1)
 *
 * For bf16 layers without a backward, moe_dispatch_plan + moe_permute_frag +
 * moe_expert_up_gelu_frag + moe_expert_down compute the same dispatch and FFN
 * with the activations in matrix-core fragment order (faster up-projection).
 *
 * The backward (see the section near the end) runs the same path in reverse:
 * moe_combine_backward, moe_expert_down_backward, moe_expert_up_backward,
 * moe_expert_weight_grads, moe_gate_backward, moe_gate_weight_grads,
 * moe_dispatch_backward.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers, row-major, densely packed, owned
 *    by the caller. The library never allocates, frees or synchronises; every
 *    call validates its arguments on the host, enqueues its kernels on
 *    `stream` and returns. Results are ready once the caller synchronises.
 *  - dtype codes: MOE_F32 (IEEE binary32) or MOE_BF16 (bfloat16, RNE).
 *    bf16 tensors need 16-byte aligned base pointers and a row length that is
 *    a multiple of 8 elements; f32 tensors need 16-byte alignment and a row
 *    length that is a multiple of 4.
 *  - Return value: MOE_OK, or a negative moe_status. On an argument error
 *    nothing is enqueued; moe_last_error() gives a text for the calling thread.
 *    A launch failure returns MOE_ERR_HIP. A fault inside a kernel surfaces at
 *    the caller's next synchronisation, as with any stream API.
 *  - T == 0 is a valid no-op for every call (aux loss writes 0).
 *  - Values are not checked: NaN/Inf inputs give unspecified routing.
 *  - The library keeps no state apart from the thread-local error text and a
 *    per-device cache of the compute-unit count; calls are re-entrant.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum { MOE_ORDER_ROWS = 0, MOE_ORDER_FRAG = 1 };   /* layout of h (moe_expert_up_gelu_frag) */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,       /* null pointer, negative or inconsistent size   */
  MOE_ERR_DTYPE = -2,     /* unsupported dtype code                         */
  MOE_ERR_SHAPE = -3,     /* size outside what the kernels support          */
  MOE_ERR_WORKSPACE = -4, /* workspace missing or smaller than required     */
  MOE_ERR_HIP = -5,       /* a HIP runtime call or kernel launch failed     */
  MOE_ERR_ALIGN = -6      /* pointer or row length breaks the 16-B rule     */
} moe_status;

#define MOE_MAX_E 256   /* experts per layer                      */
#define MOE_MAX_K 8     /* experts per token                      */
#define MOE_RENORM 0x1u /* router flag: rescale the k weights to sum to 1 */

/* Expert capacity (EP tutorial section 2.2): round((n_tokens / n_experts) x
 * capacity_factor), computed in double, round-half-even. A factor <= 0 means
 * "no dropping" and returns -1 (ms-swift page, section 4.1, drop switch off).
 * n_tokens < 0 or n_experts < 1 returns -2. Host-only, no GPU needed. */
int64_t moe_capacity(int64_t n_tokens, int32_t n_experts, double capacity_factor);

/* Rows of the grouped (expert-major) buffers x_perm / h / y_perm:
 * min(T*k, E*capacity), or T*k when capacity < 0. Host-only. */
int64_t moe_rows_max(int64_t T, int32_t k, int32_t E, int64_t capacity);

/* Gate, softmax and top-k (EP tutorial 1.1: a linear gate scores each token
 * against every expert and picks the Top-K; deployment guide section 5
 * step 3: the gate outputs per-token assignment probabilities).
 *   x        [T, d]  dtype        token representations
 *   w_gate   [E, d]  dtype        gate weight (row e scores expert e)
 *   bias     [E]     f32 or NULL  added to the logits
 *   topk_idx [T, k]  int32 out    chosen experts, best first; ties between
 *                                 equal float32 logits go to the lower index
 *   topk_w   [T, k]  f32   out    softmax probability of each chosen expert
 *                                 (rescaled to sum 1 iff flags & MOE_RENORM)
 *   probs    [T, E]  f32   out    full softmax, or NULL when not wanted
 * Logits and softmax are float32 (bf16 products accumulate in float32).
 * Limits: 1 <= E <= MOE_MAX_E, 1 <= k <= min(E, MOE_MAX_K). */
int moe_router_topk(const void* x, const void* w_gate, const float* bias,
                    int64_t T, int64_t d, int32_t E, int32_t k, int32_t dtype,
                    uint32_t flags, int32_t* topk_idx, float* topk_w, float* probs,
                    hipStream_t stream);

/* The router with the pages' balancing knobs for hot experts (SP/EP page,
 * EP section: adjust the routing temperature, add a random perturbation;
 * ETP page: a routing z-loss spreads the gate's choices). Same as
 * moe_router_topk, with softmax and top-k taken over the scores
 *   s[t, e] = (l[t, e] + noise[t, e]) / temperature
 *   noise       [T, E] f32 in, nullable (0): a perturbation the caller draws
 *   temperature  finite, > 0 (1: the plain router)
 *   lse         [T] f32 out, nullable: log sum_e exp s[t, e], whose square
 *               is the per-token term of the router z-loss (see moe_z_loss)
 *               and which the z-loss gradient needs (moe_gate_backward)
 * moe_router_topk == moe_router_topk_ex(noise NULL, temperature 1, lse NULL). */
int moe_router_topk_ex(const void* x, const void* w_gate, const float* bias,
                       const float* noise, int64_t T, int64_t d, int32_t E, int32_t k,
                       int32_t dtype, uint32_t flags, float temperature,
                       int32_t* topk_idx, float* topk_w, float* probs, float* lse,
                       hipStream_t stream);

/* Bytes of device workspace moe_dispatch needs (0 when T == 0). */
size_t moe_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t E);

/* Dispatch plan with capacity dropping, then the permute (EP tutorial 2.1
 * step 2: map each token to its target expert; 2.2: assignments beyond an
 * expert's capacity are dropped; 5.3: tokens packed so each expert's rows are
 * contiguous). Assignments are ranked inside their expert in token order
 * (token t, then slot j); the first `capacity` of them are kept
 * (capacity < 0: all kept).
 *   topk_idx [T, k] int32 in   expert of each slot; ids outside [0, E) and a
 *                              repeat of an expert already named earlier in the
 *                              same token are ignored (not counted, dest -1)
 *   x        [T, d] dtype in   token rows to permute
 *   counts   [E]    int32 out  assignments per expert before dropping
 *   offsets  [E+1]  int32 out  exclusive scan of kept rows per expert;
 *                              offsets[E] = R, the total kept rows
 *   dest     [T, k] int32 out  grouped row of each slot, or -1 if dropped
 *   src      [rows_max] int32 out   token of each grouped row (first R valid)
 *   x_perm   [rows_max, d] dtype out x_perm[r] = x[src[r]] for r < R
 *   workspace / workspace_bytes: device scratch of at least
 *             moe_dispatch_workspace_bytes(T, k, E) bytes, 4-byte aligned.
 * rows_max = moe_rows_max(T, k, E, capacity). Deterministic: no atomics on
 * any output. Requires T * k < 2^31. */
int moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                 int64_t capacity, const void* x, int64_t d, int32_t dtype,
                 int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src,
                 void* x_perm, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* The two halves of moe_dispatch, callable on their own (same arguments and
 * layouts as above; moe_dispatch == plan then permute on the same stream).
 * moe_dispatch_plan: the integer plan only -- counts, offsets, dest, src
 *   (EP tutorial 2.1 step 2, 2.2); bit-exact and deterministic.
 * moe_permute: x_perm[r] = x[src[r]] for r < offsets[E] (EP tutorial 5.3);
 *   offsets and src as written by moe_dispatch_plan, rows_max the row count of
 *   the x_perm buffer (moe_rows_max); rows past offsets[E] are not touched. */
int moe_dispatch_plan(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                      int64_t capacity, int32_t* counts, int32_t* offsets,
                      int32_t* dest, int32_t* src, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);
int moe_permute(const void* x, int64_t d, int32_t dtype, const int32_t* src,
                const int32_t* offsets, int32_t E, int64_t rows_max, void* x_perm,
                hipStream_t stream);

/* moe_dispatch_plan and moe_aux_loss in one pass (the same outputs; the loss
 * adds the same terms in another order, so it agrees to double rounding, not
 * bit for bit): the plan's histogram also sums each 256-token chunk's
 * softmax columns, and the plan's last step forms
 * L = alpha * E * sum_i (counts_i / (T k)) * (sum_t probs[t, i] / T)
 * (EP tutorial 5.1) -- two launches instead of five.
 *   probs [T, E] f32 device, 16-byte aligned (the router's softmax), alpha the loss weight,
 *   loss: device scalar (0 when T == 0).
 * moe_dispatch_plan_aux_workspace_bytes: workspace size (8-byte aligned). */
size_t moe_dispatch_plan_aux_workspace_bytes(int64_t T, int32_t k, int32_t E);
int moe_dispatch_plan_aux(const int32_t* topk_idx, const float* probs, int64_t T, int32_t k,
                          int32_t E, int64_t capacity, float alpha, int32_t* counts,
                          int32_t* offsets, int32_t* dest, int32_t* src, float* loss,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_dispatch_plan without a workspace, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation. Same arguments (minus the workspace) and
 * the same outputs, bit for bit, as moe_dispatch_plan. The per-chunk counts
 * live in a scratch array the library holds on each GPU it runs on
 * (moe_dispatch_plan_noalloc_scratch_bytes(), 1 MiB, kept until the process
 * ends); the call itself allocates nothing. A plan that needs more than that
 * (moe_dispatch_workspace_bytes(T, k, E) above it: for example more than
 * 131072 tokens with 256 experts) is rejected with MOE_ERR_WORKSPACE before
 * anything is enqueued. Every call on one GPU shares that GPU's scratch:
 * calls that may overlap in time on one GPU (other streams, other threads)
 * race and must be ordered by the caller. Nothing in the scratch needs
 * clearing between calls. */
int moe_dispatch_plan_noalloc(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                              int64_t capacity, int32_t* counts, int32_t* offsets,
                              int32_t* dest, int32_t* src, hipStream_t stream);
size_t moe_dispatch_plan_noalloc_scratch_bytes(void);

/* The router and the dispatch plan handing over per-tile counts, so the plan
 * needs no histogram pass of its own (EP tutorial 2.1 steps 1-2: the gate
 * picks each token's experts, then the dispatch plan is built from those
 * choices; 2.2: drop beyond capacity; 5.1: the aux loss).
 *   moe_router_tiles(T, E): how many token tiles the bf16 router works in
 *     (16 tokens each, 64 for 17..64 experts); 0 for T <= 0 or E outside
 *     1..MOE_MAX_E.
 *   moe_router_topk_tiles: moe_router_topk for bf16 (other dtypes:
 *     MOE_ERR_DTYPE), and per tile i and expert e
 *       tile_counts [tiles, E] int32 out: how many of the tile's tokens chose e
 *         (16-byte aligned, required)
 *       tile_colsum [tiles, E] double out, nullable: the tile's softmax
 *         probabilities of e added in double in token order (8-byte aligned)
 *   moe_dispatch_plan_tiles: moe_dispatch_plan from those counts in one
 *     launch and without a workspace; with tile_colsum (and a device scalar
 *     `loss`, both or neither) also the aux loss as moe_aux_loss defines it,
 *     its column sums added tile by tile in tile order. topk_idx must be the
 *     router's output the counts came from. Needs tiles x E <= 16384
 *     (MOE_ERR_SHAPE otherwise: use moe_dispatch_plan). counts, offsets,
 *     dest and src are bit-identical to moe_dispatch_plan's. */
int64_t moe_router_tiles(int64_t T, int32_t E);
int moe_router_topk_tiles(const void* x, const void* w_gate, const float* bias, int64_t T,
                          int64_t d, int32_t E, int32_t k, int32_t dtype, uint32_t flags,
                          int32_t* topk_idx, float* topk_w, float* probs, int32_t* tile_counts,
                          double* tile_colsum, hipStream_t stream);
int moe_dispatch_plan_tiles(const int32_t* topk_idx, const int32_t* tile_counts,
                            const double* tile_colsum, int64_t T, int32_t k, int32_t E,
                            int64_t capacity, float alpha, int32_t* counts, int32_t* offsets,
                            int32_t* dest, int32_t* src, float* loss, hipStream_t stream);

/* Grouped expert FFN over the expert-major segments given by `offsets`
 * (ETP page: up-projection w1 then down-projection w2, e.g.
 * 4096 -> 16384 -> 4096; EP tutorial 2.1 step 4: each expert computes on its
 * own tokens). For every expert e and row r in [offsets[e], offsets[e+1]):
 *   h[r]      = gelu_tanh(W1[e] . x_perm[r])
 *   y_perm[r] = W2[e] . h[r]                     (float32)
 * with gelu_tanh(z) = z / 2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3))).
 *   x_perm [rows_max, d]      dtype    w1 [E, d_ff, d] dtype (K contiguous)
 *   h      [rows_max, d_ff]   hidden   w2 [E, d, d_ff] dtype (K contiguous)
 *   y_perm [rows_max, d]      f32
 *   offsets [E+1] int32, device: read by the kernels, never by the host.
 * Hidden-activation storage: f32 when dtype is MOE_F32; IEEE fp16 (RNE) when
 * dtype is MOE_BF16 -- the same two bytes as bf16 with three more significand
 * bits; the down-projection then runs fp16 x fp16 with W2's bf16 values
 * rounded to fp16 (nearest even; where that is exact: moe_weights_bf16_to_f16).
 * |h| or |W2| of 65520 or more become +-inf there, and nothing checks for it.
 * Products accumulate in float32. Rows >= offsets[E] are not touched.
 * Limits: d, d_ff <= 2^22.
 * workspace / workspace_bytes: device scratch of at least
 *   moe_ffn_workspace_bytes(dtype) bytes (16-byte aligned), or NULL. With it,
 *   output tiles of a short last round of work are split along K over idle
 *   compute units and their float32 partial sums added up in a fixed order
 *   (results stay deterministic); with NULL, no tile is split. Calls that
 *   share one workspace must not overlap in time (same stream, or ordered).
 * Errors: MOE_ERR_WORKSPACE when a non-NULL workspace is smaller than needed. */
int moe_grouped_ffn(const void* x_perm, const int32_t* offsets, int32_t E,
                    int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                    const void* w2, int32_t dtype, void* h, float* y_perm,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two halves of moe_grouped_ffn, callable on their own (same arguments,
 * same layouts, `dtype` is the layer's dtype in both): the up-projection with
 * its GELU-tanh epilogue, and the down-projection. moe_grouped_ffn == up then
 * down on the same stream. */
int moe_expert_up_gelu(const void* x_perm, const int32_t* offsets, int32_t E,
                       int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                       int32_t dtype, void* h, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);
int moe_expert_down(const void* h, const int32_t* offsets, int32_t E,
                    int64_t rows_max, int64_t d, int64_t d_ff, const void* w2,
                    int32_t dtype, float* y_perm, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* The permute folded into the up-projection, for bf16 layers without a
 * backward (EP tutorial 5.3's packed rows are never stored): h[r] =
 * fp16(gelu_tanh(W1[e] . x[src[r]])) for every expert e and row r in
 * [offsets[e], offsets[e+1]) -- the h of moe_permute followed by
 * moe_expert_up_gelu, bit for bit, with the same workspace argument.
 *   x [T, d] bf16 token rows (device, 16-byte aligned, T * d * 2 < 2^31),
 *   src [rows_max] int32 and offsets [E+1] as moe_dispatch_plan writes them
 *   (device, read only by the kernel; an src entry outside [0, T) reads zeros
 *   or another row of x, never memory outside x), the other arguments as for
 *   moe_expert_up_gelu with dtype MOE_BF16.
 * Errors: those of moe_expert_up_gelu; MOE_ERR_ARG for T < 0 or a NULL src
 *   when rows_max > 0; MOE_ERR_SHAPE when x holds 2^31 bytes or more. */
int moe_expert_up_gelu_gather(const void* x, int64_t T, const int32_t* src, const int32_t* offsets,
                              int32_t E, int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                              void* h, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* W2 stored in fp16, for bf16 layers (an inference-time weight format; the
 * down-projection of moe_expert_down converts every bf16 W2 value to fp16 in
 * registers before the fp16 x fp16 products, this does it once up front).
 * moe_weights_bf16_to_f16: w_f16[i] = fp16(w[i]) for i < n, round to nearest
 *   even, the same rounding the kernels apply. It is exact for 0 and for
 *   2^-17 <= |w| <= 65280; below 2^-17 only multiples of fp16's subnormal
 *   step 2^-24 are kept exactly (the rest lose low bits, and nonzero values
 *   under 2^-25 round to 0), finite values of magnitude 65536 and above
 *   become +-inf, infinities and NaNs stay what they are.
 *   16-byte aligned device pointers. `report` (nullable, device, 8-byte
 *   aligned, two counters): when given, report[0] = how many finite nonzero
 *   values lost bits, report[1] = how many finite values became +-inf; the
 *   call sets both (no clearing needed), and they are exact counts whatever
 *   order the GPU adds in. With n = 0 and a report it writes two zeros.
 * moe_expert_down_f16w: moe_expert_down (dtype MOE_BF16) with w2_f16 [E, d,
 *   d_ff] fp16 = moe_weights_bf16_to_f16(W2); y_perm bit-identical to
 *   moe_expert_down on the bf16 W2 with the same workspace argument.
 * The hidden activation h of bf16 layers is fp16 too (moe_grouped_ffn): a
 * |gelu(z)| of 65520 or more is stored as +-inf, and the output rows that
 * use it become inf or NaN; nothing checks for it. */
int moe_weights_bf16_to_f16(const void* w, int64_t n, void* w_f16, uint64_t* report,
                            hipStream_t stream);
int moe_expert_down_f16w(const void* h, const int32_t* offsets, int32_t E, int64_t rows_max,
                         int64_t d, int64_t d_ff, const void* w2_f16, float* y_perm,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of expert-FFN workspace for the current device: two 256 x 256
 * float32 partial tiles per compute unit (128 MiB on a 256-CU MI355X) for
 * MOE_BF16; 0 for MOE_F32 (whose kernels never split). */
size_t moe_ffn_workspace_bytes(int32_t dtype);

/* The expert FFN of bf16 layers on fragment-ordered activations (inference:
 * moe_permute_frag, then moe_expert_up_gelu_frag with MOE_ORDER_FRAG, then
 * moe_expert_down_frag). The products are those of the row-major calls,
 * added in float32 in the matrix cores' 16 x 16 x 32 steps instead of
 * 32 x 32 x 16 ones: h and y_perm equal the row-major calls' (without a
 * workspace) up to float32 summation order; on every shape tested they were
 * equal bit for bit. The fragment-ordered copy of x_perm holds
 * the permuted rows of EP tutorial 5.3 laid out for the matrix cores: each
 * expert segment is padded with zero rows to a multiple of 32 (padded segment
 * e starts at pad[e] = sum over e' < e of roundup(offsets[e'+1] - offsets[e'],
 * 32)), and element (padded row r, column c) sits at element
 *   ((r / 32) * (d / 16) + c / 16) * 512 + ((r % 32) + 32 * ((c / 8) % 2)) * 8 + c % 8,
 * so every 32-row x 16-column block is one contiguous 1 KiB piece.
 *
 * moe_frag_rows: padded row count to allocate for x_frag ([moe_frag_rows, d]
 *   bf16), an upper bound on pad[E] for any offsets with offsets[E] <= rows_max;
 *   -1 for rows_max < 0 or E outside [1, MOE_MAX_E].
 * moe_permute_frag: x_frag from x [T, d] bf16 and the plan's src/offsets
 *   (as written by moe_dispatch_plan); writes rows [0, pad[E]) of x_frag,
 *   zeros in the padding rows. d a multiple of 16.
 * moe_expert_up_gelu_frag: h[r] = fp16(gelu_tanh(W1[e] . x_perm[r])) for every
 *   expert e and unpadded row r in [offsets[e], offsets[e+1]) (ETP page w1;
 *   EP tutorial 2.1 step 4). h_order MOE_ORDER_ROWS: h [rows_max, d_ff]
 *   row-major as for moe_expert_up_gelu, rows >= offsets[E] not touched;
 *   MOE_ORDER_FRAG: h [moe_frag_rows(rows_max, E), d_ff] in the fragment order
 *   above (K = d_ff), rows [0, pad[E]) written, padding rows zero, d_ff a
 *   multiple of 256. d a multiple of 256, d_ff of 8, d and d_ff <= 2^20. No
 *   output tile is split along K.
 * moe_expert_down_frag: y_perm[r] = W2[e] . h[r] (float32, row-major
 *   [rows_max, d], rows >= offsets[E] not touched; ETP page w2) from h in
 *   fragment order and w2_f16 = moe_weights_bf16_to_f16(W2) [E, d, d_ff];
 *   d_ff a multiple of 256. Without a workspace, equal to
 *   moe_expert_down_f16w without one as above; with moe_ffn_workspace_bytes of
 *   workspace, the tiles of a short last round are split along K (pieces of
 *   whole 256-deep quads, so the sums may round differently from the
 *   row-major kernel's splits; fixed order, deterministic).
 * Pointers 16-byte aligned device memory; offsets (and src) read only by the
 * kernels, and must be as moe_dispatch_plan writes them. These calls take
 * bf16 data only (no dtype argument).
 * Errors: MOE_ERR_ALIGN for d, d_ff or a pointer that breaks the rules above;
 *   MOE_ERR_SHAPE for E or sizes out of range; MOE_ERR_ARG for a NULL pointer
 *   when rows_max > 0. */
int64_t moe_frag_rows(int64_t rows_max, int32_t E);
int moe_permute_frag(const void* x, int64_t d, const int32_t* src, const int32_t* offsets,
                     int32_t E, int64_t rows_max, void* x_frag, hipStream_t stream);
int moe_expert_up_gelu_frag(const void* x_frag, const int32_t* offsets, int32_t E,
                            int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                            void* h, int32_t h_order, hipStream_t stream);
int moe_expert_down_frag(const void* h_frag, const int32_t* offsets, int32_t E, int64_t rows_max,
                         int64_t d, int64_t d_ff, const void* w2_f16, float* y_perm,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Weighted combine back to token order (EP tutorial 2.1 step 5; 2.2: a
 * dropped slot takes no part):
 *   y[t] = sum over j with dest[t,j] >= 0 of topk_w[t,j] * y_perm[dest[t,j]],
 * summed in slot order; a token with no kept slot gets zeros.
 *   y_perm [rows, d] f32, dest [T, k] int32, topk_w [T, k] f32,
 *   y [T, d] in out_dtype (MOE_F32 or MOE_BF16). Deterministic, no atomics. */
int moe_combine(const float* y_perm, const int32_t* dest, const float* topk_w,
                int64_t T, int32_t k, int64_t d, void* y, int32_t out_dtype,
                hipStream_t stream);

/* Bytes of device workspace moe_aux_loss needs. */
size_t moe_aux_loss_workspace_bytes(int64_t T, int32_t E);

/* Auxiliary load-balance loss (EP tutorial 5.1):
 *   L = alpha * E * sum_i f_i * P_i,  f_i = counts[i] / (T * k),
 *   P_i = (1/T) * sum_t probs[t, i].
 * counts are the pre-drop assignment counts moe_dispatch writes.
 *   probs [T, E] f32, counts [E] int32, loss: one f32 written on the device.
 * Sums run in double in a fixed order: bit-identical from run to run. */
int moe_aux_loss(const float* probs, const int32_t* counts, int64_t T, int32_t E,
                 int32_t k, float alpha, float* loss, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Router z-loss (ETP page names it; no formula there -- read as the usual
 * one): *loss = coeff * (1/T) * sum_t lse[t]^2, lse from moe_router_topk_ex.
 * Summed in double in a fixed order (deterministic); T == 0 gives 0.
 * workspace: moe_z_loss_workspace_bytes(T) bytes, 8-byte aligned. */
size_t moe_z_loss_workspace_bytes(int64_t T);
int moe_z_loss(const float* lse, int64_t T, float coeff, float* loss, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------- backward --
 * The layer's backward on one GPU. The pages train the layer end to end and
 * keep the aux loss for its gradient on the gate (EP tutorial 5.1); the
 * reverse path runs combine, the expert FFN, dispatch and the gate in turn.
 * Readings: the routing choice (top-k indices, capacity drops) and the counts
 * in f_i are constants of the backward; a caller-drawn noise is an input.
 * Gradient storage of a layer: bf16 (RNE) when dtype is MOE_BF16, f32 when
 * MOE_F32; dx_perm, dx and every weight gradient are f32. The bf16 GEMMs
 * accumulate in f32 on the MFMA units.
 * Limits on top of the forward's for MOE_BF16: d * d_ff < 2^30 and
 * rows_max * max(d, d_ff) < 2^30. */

/* moe_expert_up_gelu that also stores the pre-activation
 *   z[r] = W1[e] . x_perm[r]       z [rows_max, d_ff] in the hidden storage
 * (fp16 for MOE_BF16, f32 for MOE_F32), which moe_expert_down_backward needs. */
int moe_expert_up_gelu_z(const void* x_perm, const int32_t* offsets, int32_t E,
                         int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                         int32_t dtype, void* h, void* z, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Transpose of moe_combine. For every slot (t, j) with r = dest[t,j] >= 0:
 *   d_out_perm[r] = topk_w[t,j] * dy[t]       (gradient storage, [rows, d])
 *   d_topk_w[t,j] = dy[t] . y_perm[r]          (f32 [T, k]; 0 when dropped)
 * dy [T, d] f32, y_perm [rows, d] f32 (the expert outputs of the forward).
 * Rows of d_out_perm that no slot names are not written. Dot products are
 * summed in a fixed order (deterministic). */
int moe_combine_backward(const float* dy, const float* y_perm, const int32_t* dest,
                         const float* topk_w, int64_t T, int32_t k, int64_t d,
                         int32_t dtype, void* d_out_perm, float* d_topk_w,
                         hipStream_t stream);

/* Backward of the down-projection and the GELU, per expert segment:
 *   dz[r] = (W2[e]^T d_out_perm[r]) * gelu_tanh'(z[r])    [rows_max, d_ff]
 * d_out_perm [rows_max, d] and dz in gradient storage, z from
 * moe_expert_up_gelu_z, w2 [E, d, d_ff] as in the forward. workspace as for
 * moe_grouped_ffn (optional split tiles, deterministic). */
int moe_expert_down_backward(const void* d_out_perm, const int32_t* offsets, int32_t E,
                             int64_t rows_max, int64_t d, int64_t d_ff, const void* w2,
                             const void* z, int32_t dtype, void* dz, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Backward of the up-projection to the grouped rows:
 *   dx_perm[r] = W1[e]^T dz[r]         f32 [rows_max, d]
 * w1 [E, d_ff, d] as in the forward; workspace as for moe_grouped_ffn. */
int moe_expert_up_backward(const void* dz, const int32_t* offsets, int32_t E,
                           int64_t rows_max, int64_t d, int64_t d_ff, const void* w1,
                           int32_t dtype, float* dx_perm, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Expert weight gradients, summed over each expert's kept rows:
 *   dw1[e] = sum_r dz[r]^T x_perm[r]          f32 [E, d_ff, d]   (NULL: skip)
 *   dw2[e] = sum_r d_out_perm[r]^T h[r]       f32 [E, d, d_ff]   (NULL: skip)
 * Every expert's block is written (zeros for an expert with no rows). For
 * MOE_BF16, h (fp16) is rounded to bf16 on its way into the product. */
int moe_expert_weight_grads(const void* x_perm, const void* h, const void* d_out_perm,
                            const void* dz, const int32_t* offsets, int32_t E,
                            int64_t rows_max, int64_t d, int64_t d_ff, int32_t dtype,
                            float* dw1, float* dw2, hipStream_t stream);

/* Gradient of the gate's linear output l = x Wg^T + b, [T, E] f32, for
 *   L = <dy, y> + aux_grad * L_aux + z_coeff * (1/T) sum_t lse[t]^2.
 * With s = (l + noise) / temperature and p = softmax(s) (moe_router_topk_ex):
 *   g[t,j] = d_topk_w[t,j], or, with flags & MOE_RENORM (w = p / S, S the
 *            sum of the chosen p), (d_topk_w[t,j] - sum_i d_topk_w[t,i] w[t,i]) / S;
 *   dp[t,e] = sum over slots j choosing e of g[t,j]
 *             + aux_grad * alpha * E * counts[e] / (T k) / T   (EP tutorial 5.1);
 *   ds = p (dp - sum_e p dp) + z_coeff * 2 lse[t] p / T;  d_logits = ds / temperature.
 * topk_w may be NULL without MOE_RENORM; lse may be NULL when z_coeff == 0. */
int moe_gate_backward(const float* d_topk_w, const int32_t* topk_idx, const float* topk_w,
                      const float* probs, const int32_t* counts, const float* lse,
                      int64_t T, int32_t E, int32_t k, uint32_t flags, float temperature,
                      float alpha, float aux_grad, float z_coeff, float* d_logits,
                      hipStream_t stream);

/* Gate weight gradients: d_w_gate = d_logits^T x  (f32 [E, d]) and
 * d_bias = column sums of d_logits (f32 [E], nullable). x [T, d] in dtype.
 * Partial sums over token chunks are added in chunk order (deterministic).
 * workspace: moe_gate_weight_grads_workspace_bytes(T, d, E) bytes, 16-byte
 * aligned. */
size_t moe_gate_weight_grads_workspace_bytes(int64_t T, int64_t d, int32_t E);
int moe_gate_weight_grads(const float* d_logits, const void* x, int64_t T, int64_t d,
                          int32_t E, int32_t dtype, float* d_w_gate, float* d_bias,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Transpose of dispatch plus the gate's input gradient:
 *   dx[t] = sum over kept slots j (in slot order) of dx_perm[dest[t,j]]
 *           + sum_e d_logits[t,e] * w_gate[e]          f32 [T, d]
 * d_logits and w_gate ([E, d] in dtype) are both given or both NULL (a layer
 * with caller-given routing). */
int moe_dispatch_backward(const float* dx_perm, const int32_t* dest, const float* d_logits,
                          const void* w_gate, int64_t T, int32_t k, int64_t d, int32_t E,
                          int32_t dtype, float* dx, hipStream_t stream);

/* Text describing the last non-OK status returned on the calling thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

// Launchers of the fragment-ordered permute and up-projection (gemm_frag.hip);
// arguments are validated by the C-ABI layer before these run.
#pragma once

#include "moe_internal.h"

namespace moe {

// Rows to allocate for the fragment-ordered copy: every segment padded to 32.
int64_t frag_rows(int64_t rows_max, int E);
hipError_t launch_permute_frag(const void* x, int64_t d, const int32_t* src, const int32_t* offsets,
                               int E, int64_t rows_max, void* x_frag, hipStream_t s);
// h row-major, or (h_frag_order) in fragment order with padded rows.
hipError_t launch_up_gelu_frag(const void* x_frag, const int32_t* offsets, int E, int64_t rows_max,
                               int64_t d, int64_t d_ff, const void* w1, void* h, bool h_frag_order,
                               hipStream_t s);
// Down-projection from h in fragment order on fp16 W2 (ws: the expert-FFN
// workspace or null).
hipError_t launch_down_frag(const void* h_frag, const int32_t* offsets, int E, int64_t rows_max, int64_t d,
                            int64_t d_ff, const void* w2_f16, float* y_perm, void* ws, hipStream_t s);
// The row-major GEMM's fix-up kernel for f32 down-projection outputs (gemm_mfma.hip):
// adds the split pieces' partial sums of a launch of `grid` workgroups.
hipError_t launch_split_fixup_down(const int32_t* offsets, int E, int N, int K, int grid, int max_split,
                                   const float* part, float* y, hipStream_t s);

}  // namespace moe

// Launchers of the fragment-ordered permute and up-projection (gemm_frag.hip);
// arguments are validated by the C-ABI layer before these run.
#pragma once

#include "moe_internal.h"

namespace moe {

// Rows to allocate for the fragment-ordered copy: every segment padded to 32.
int64_t frag_rows(int64_t rows_max, int E);
hipError_t launch_permute_frag(const void* x, int64_t d, const int32_t* src, const int32_t* offsets,
                               int E, int64_t rows_max, void* x_frag, hipStream_t s);
hipError_t launch_up_gelu_frag(const void* x_frag, const int32_t* offsets, int E, int64_t rows_max,
                               int64_t d, int64_t d_ff, const void* w1, void* h, hipStream_t s);

}  // namespace moe

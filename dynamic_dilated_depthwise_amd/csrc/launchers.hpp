// launchers.hpp -- internal host launchers behind the C ABI (not exported).
// Arguments are validated by the ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

namespace ddpm {

// `vec`: pixels per thread for the materialised filter (W % vec == 0 and the
// pointers aligned to vec elements), chosen by the ABI layer.
hipError_t launch_filter_fwd(const void *x, const void *taps, void *out, int N, int C, int H, int W, int K,
                             bool bf16, int vec, hipStream_t stream);

// `aligned4`: W % 4 == 0 and every tensor pointer 16-byte aligned.
hipError_t launch_fused_fwd(const void *x, const void *y, const void *wg, const void *bg, void *out, int N,
                            int C, int H, int W, int K, bool bf16, bool aligned4, hipStream_t stream);

// bfloat16 forward for K = 3, C = 64 as persistent workgroups streaming their tiles
// into LDS; fused_fwd_pers_applies tells whether a shape can take it.
bool fused_fwd_pers_applies(int N, int C, int H, int W, int K, bool bf16, bool al);
hipError_t launch_fused_fwd_pers(const void *x, const void *y, const void *wg, const void *bg, void *out, int N,
                                 int H, int W, hipStream_t stream);

// gx, gy or (dw_part, db_part) may be null: that part is skipped.
hipError_t launch_fused_bwd(const void *x, const void *y, const void *wg, const void *bg, const void *gout,
                            void *gx, void *gy, float *dw_part, float *db_part, int S, int N, int C, int H,
                            int W, int K, bool bf16, bool aligned4, hipStream_t stream);

// dX of the fused backward (one kernel); bwd_dx_blocks is its grid size.
int64_t bwd_dx_blocks(int N, int C, int H, int W);
hipError_t launch_bwd_dx(const void *y, const void *wg, const void *bg, const void *gout, void *gx, int N, int C,
                         int H, int W, int K, bool bf16, bool al, hipStream_t stream);

// dX for C = 64 staged by source row (both dtypes); bwd_dx_rows_applies tells
// whether a shape can take it.
bool bwd_dx_rows_applies(int C, int H, int W, bool al, bool bf16);
hipError_t launch_bwd_dx_rows(const void *y, const void *wg, const void *bg, const void *gout, void *gx, int N,
                              int H, int W, int K, bool bf16, hipStream_t stream);

// dY for C = 64 staged by source row (both dtypes); bwd_dy_rows_applies tells
// whether a shape can take it, bwd_dy_rows_blocks gives its grid size.
bool bwd_dy_rows_applies(int C, int H, int W, bool al, bool bf16);
int64_t bwd_dy_rows_blocks(int N, int H, int W, bool bf16);
hipError_t launch_bwd_dy_rows(const void *x, const void *wg, const void *gout, void *gy, int N, int H, int W, int K,
                              bool bf16, hipStream_t stream);

// dW / db partials for C = 64 staged by row segment (both dtypes); the grid and
// token ranges are those of the general kernel.
bool bwd_dw_rows_applies(int C, int H, int W, bool al, bool bf16);
hipError_t launch_bwd_dw_rows(const void *x, const void *y, const void *gout, float *dw_part, float *db_part, int S,
                              int N, int H, int W, int K, bool bf16, hipStream_t stream);

// gx or gtaps may be null: that output is skipped (not both).
hipError_t launch_filter_bwd(const void *x, const void *taps, const void *gout, void *gx, void *gtaps, int N, int C,
                             int H, int W, int K, bool bf16, int vec, bool aligned, hipStream_t stream);

hipError_t launch_reduce_partials(const float *dw_part, const float *db_part, int S, void *gw, void *gb,
                                  int64_t R, int C, bool bf16, hipStream_t stream);

}  // namespace ddpm

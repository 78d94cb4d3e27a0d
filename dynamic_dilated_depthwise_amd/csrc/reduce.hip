// reduce.hip -- the second, short kernel of the split weight-gradient reduction
// (page "lartpang/DynamicConvolutionOperator", section "CUDA Flash 式融合训练":
// large sizes split the tokens into at most 16 float32 partials and a second short
// kernel reduces them).
//
// grad[m] = sum_{s=0}^{S-1} partial[s][m] in ascending s, in float32, written in
// the parameter dtype.  A pure stream, one launch for the weight and the bias; four
// elements per thread when the length and the pointers allow 16-byte accesses.
#include "common.hpp"
#include "launchers.hpp"

namespace ddpm {

constexpr int kMaxPartials = 16;

// One element (or four, VEC4) of one gradient: all S partials are loaded first (they
// are independent), then added in ascending s.
template <typename T, bool VEC4>
__device__ __forceinline__ void reduce_item(const float *__restrict__ part, int S, int64_t M, int64_t i,
                                            T *__restrict__ dst) {
    if constexpr (VEC4) {
        f32x4 v[kMaxPartials];
#pragma unroll
        for (int s = 0; s < kMaxPartials; ++s)
            if (s < S) v[s] = *(const f32x4 *)(part + (int64_t)s * M + 4 * i);
        f32x4 acc = v[0];
#pragma unroll
        for (int s = 1; s < kMaxPartials; ++s)
            if (s < S) acc += v[s];
        store4_row(dst + 4 * i, 0, 4, acc, true);
    } else {
        float v[kMaxPartials];
#pragma unroll
        for (int s = 0; s < kMaxPartials; ++s)
            if (s < S) v[s] = part[(int64_t)s * M + i];
        float acc = v[0];
#pragma unroll
        for (int s = 1; s < kMaxPartials; ++s)
            if (s < S) acc += v[s];
        dst[i] = Elem<T>::from_f32(acc);
    }
}

// Both gradients in one launch: items [0, nw) are the weight's (four elements each
// when vw), items [nw, nw + nb) the bias's (four each when vb).
template <typename T>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ pw,
                                                              const float *__restrict__ pb, int S, int64_t Mw,
                                                              int64_t Mb, T *__restrict__ gw, T *__restrict__ gb,
                                                              int vw, int vb) {
    const int64_t nw = vw ? Mw / 4 : Mw;
    const int64_t nb = vb ? Mb / 4 : Mb;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nw + nb; i += stride) {
        if (i < nw) {
            if (vw) reduce_item<T, true>(pw, S, Mw, i, gw);
            else reduce_item<T, false>(pw, S, Mw, i, gw);
        } else {
            const int64_t k = i - nw;
            if (vb) reduce_item<T, true>(pb, S, Mb, k, gb);
            else reduce_item<T, false>(pb, S, Mb, k, gb);
        }
    }
}

hipError_t launch_reduce_partials(const float *dw_part, const float *db_part, int S, void *gw, void *gb, int64_t R,
                                  int C, bool bf16, hipStream_t stream) {
    if (S < 1 || S > kMaxPartials) return hipErrorInvalidValue;
    const int64_t Mw = R * C;
    const bool vw = (Mw % 4) == 0 && ((uintptr_t)dw_part % 16) == 0 && ((uintptr_t)gw % (bf16 ? 8 : 16)) == 0;
    const bool vb = (R % 4) == 0 && ((uintptr_t)db_part % 16) == 0 && ((uintptr_t)gb % (bf16 ? 8 : 16)) == 0;
    const int64_t items = (vw ? Mw / 4 : Mw) + (vb ? R / 4 : R);
    int64_t blocks = (items + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    if (bf16)
        hipLaunchKernelGGL((reduce_partials_kernel<bf16_t>), dim3((unsigned)blocks), dim3(256), 0, stream, dw_part,
                           db_part, S, Mw, R, (bf16_t *)gw, (bf16_t *)gb, vw ? 1 : 0, vb ? 1 : 0);
    else
        hipLaunchKernelGGL((reduce_partials_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, stream, dw_part,
                           db_part, S, Mw, R, (float *)gw, (float *)gb, vw ? 1 : 0, vb ? 1 : 0);
    return hipGetLastError();
}

}  // namespace ddpm

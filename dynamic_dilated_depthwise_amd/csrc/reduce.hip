// reduce.hip -- the second, short kernel of the split weight-gradient reduction
// (page "lartpang/DynamicConvolutionOperator", section "CUDA Flash 式融合训练":
// large sizes split the tokens into at most 16 float32 partials and a second short
// kernel reduces them).
//
// grad[m] = sum_{s=0}^{S-1} partial[s][m] in ascending s, in float32, written in
// the parameter dtype.  A pure stream; four elements per thread when the length
// and the pointers allow 16-byte accesses.
#include "common.hpp"
#include "launchers.hpp"

namespace ddpm {

template <typename T, bool VEC4>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ part, int S, int64_t M,
                                                              T *__restrict__ dst) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VEC4) {
        const int64_t M4 = M / 4;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M4; i += stride) {
            f32x4 acc = *(const f32x4 *)(part + 4 * i);
            for (int s = 1; s < S; ++s) acc += *(const f32x4 *)(part + (int64_t)s * M + 4 * i);
            store4_row(dst + 4 * i, 0, 4, acc, true);
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M; i += stride) {
            float acc = part[i];
            for (int s = 1; s < S; ++s) acc += part[(int64_t)s * M + i];
            dst[i] = Elem<T>::from_f32(acc);
        }
    }
}

template <typename T>
static hipError_t launch_one(const float *part, int S, int64_t M, void *dst, bool vec4, hipStream_t stream) {
    const int64_t work = vec4 ? M / 4 : M;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    if (vec4)
        hipLaunchKernelGGL((reduce_partials_kernel<T, true>), dim3((unsigned)blocks), dim3(256), 0, stream, part, S, M,
                           (T *)dst);
    else
        hipLaunchKernelGGL((reduce_partials_kernel<T, false>), dim3((unsigned)blocks), dim3(256), 0, stream, part, S,
                           M, (T *)dst);
    return hipGetLastError();
}

hipError_t launch_reduce_partials(const float *dw_part, const float *db_part, int S, void *gw, void *gb, int64_t R,
                                  int C, bool bf16, hipStream_t stream) {
    const int64_t Mw = R * C;
    const bool v4 = (Mw % 4) == 0 && ((uintptr_t)dw_part % 16) == 0 && ((uintptr_t)gw % (bf16 ? 8 : 16)) == 0;
    hipError_t e = bf16 ? launch_one<bf16_t>(dw_part, S, Mw, gw, v4, stream)
                        : launch_one<float>(dw_part, S, Mw, gw, v4, stream);
    if (e != hipSuccess) return e;
    const bool vb = (R % 4) == 0 && ((uintptr_t)db_part % 16) == 0 && ((uintptr_t)gb % (bf16 ? 8 : 16)) == 0;
    return bf16 ? launch_one<bf16_t>(db_part, S, R, gb, vb, stream) : launch_one<float>(db_part, S, R, gb, vb, stream);
}

}  // namespace ddpm

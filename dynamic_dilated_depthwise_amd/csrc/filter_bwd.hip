// filter_bwd.hip -- backward of the materialised dynamic dilated filter (gfx950).
//
// Operation (page "lartpang/DynamicConvolutionOperator", section "CUDA 动态过滤":
// the backward fuses dX and dK, the gradient of the dynamic kernels, without
// building a patch matrix).  With G = dL/d out split as [G_x, G_0, G_1, G_2]:
//   dK[n, o(b,c,t), p] = G_b[n, c, p] * x[n, c, p + d_bt]              (zero outside)
//   dX[n, c, q]        = G_x[n, c, q] + sum_{b,t} taps[n, o, q - d_bt] * G_b[n, c, q - d_bt]
// dX is a gather: every output pixel reads the taps that were applied at its
// source pixels, so each output element is written once, with no atomics.
//
// Like the forward filter this is an HBM stream (3K^2 tap planes read for dX, 3K^2
// dK planes written).  One workgroup = one (n, c) plane x a TH x TW tile in
// XCD-contiguous order; x and / or the three G_b planes of the tile plus a
// 5*(K-1)/2 halo are staged once in LDS (zero outside the image), so the dilated
// neighbourhoods come from LDS; each thread owns VEC consecutive pixels of a row.
// The dK planes are streamed out with non-temporal vector stores.
#include "common.hpp"
#include "launchers.hpp"

namespace ddpm {

// VEC shifted pixels w..w+VEC-1 of one tap row, widened to float, zero outside.
template <typename T, int VEC>
__device__ __forceinline__ void load_run(const T *__restrict__ row, int w, int W, bool row_ok, bool aligned,
                                         float (&v)[VEC]) {
    if constexpr (VEC == 4) {
        const f32x4 t = load4_row(row, w, W, row_ok, aligned && ((w & 3) == 0));
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = t[k];
    } else if constexpr (VEC == 8) {
        load8_bf16_row(row, w, W, row_ok, v);
    } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int ww = w + k;
            v[k] = (row_ok && ww >= 0 && ww < W) ? Elem<T>::to_f32(row[ww]) : 0.f;
        }
    }
}

template <typename T, int K, int VEC, bool WANT_DX, bool WANT_DK>
__global__ __launch_bounds__(256) void filter_bwd_kernel(const T *__restrict__ x, const T *__restrict__ taps,
                                                         const T *__restrict__ gout, T *__restrict__ gx,
                                                         T *__restrict__ gtaps, int C, int H, int W, int TH, int TW,
                                                         int nbands, int ncolt, int aligned) {
    constexpr int r = (K - 1) / 2;
    constexpr int HALO = 5 * r;
    constexpr int PADC = (HALO + 3) & ~3;
    constexpr int KK = K * K;
    typedef typename VecOf<T, VEC>::type V;
    extern __shared__ float lds[];

    const int LW = TW + 2 * PADC;
    const int LH = TH + 2 * HALO;
    const int LP = LH * LW;  // one staged plane
    const int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int colt = L % ncolt;
    const int band = (L / ncolt) % nbands;
    const int nc = L / (ncolt * nbands);
    const int n = nc / C;
    const int c = nc - n * C;
    const int h0 = band * TH;
    const int w0 = colt * TW;
    const int64_t HW = (int64_t)H * W;
    const T *__restrict__ gn = gout + (int64_t)n * 4 * C * HW;

    // Staged planes: [0] x (for dK), [1 + b] G_b (for dX).
    float *xs = lds;
    float *gs = lds + (WANT_DK ? LP : 0);
    for (int i = threadIdx.x; i < LP; i += blockDim.x) {
        const int lr = i / LW;
        const int lc = i - lr * LW;
        const int hh = h0 - HALO + lr;
        const int ww = w0 - PADC + lc;
        const bool in = hh >= 0 && hh < H && ww >= 0 && ww < W;
        const int64_t pix = (int64_t)hh * W + ww;
        if constexpr (WANT_DK) xs[i] = in ? Elem<T>::to_f32(x[(int64_t)nc * HW + pix]) : 0.f;
        if constexpr (WANT_DX) {
#pragma unroll
            for (int b = 0; b < 3; ++b)
                gs[b * LP + i] = in ? Elem<T>::to_f32(gn[(int64_t)((1 + b) * C + c) * HW + pix]) : 0.f;
        }
    }
    __syncthreads();

    const int64_t R = 3LL * C * KK;
    const T *__restrict__ tp = taps + (int64_t)n * R * HW;
    T *__restrict__ dkp = gtaps + (int64_t)n * R * HW;
    const int gpr = TW / VEC;
    for (int gi = threadIdx.x; gi < TH * gpr; gi += blockDim.x) {
        const int lr = gi / gpr;
        const int lc = (gi - lr * gpr) * VEC;
        const int h = h0 + lr;
        const int w = w0 + lc;
        if (h >= H || w >= W) continue;  // W % VEC == 0: a vector is wholly in or out
        const int64_t pix = (int64_t)h * W + w;
        const int ctr = (lr + HALO) * LW + lc + PADC;  // staged index of this run's first pixel

        if constexpr (WANT_DK) {
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                const int D = dilation(b);
                float gv[VEC];
                if constexpr (WANT_DX) {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) gv[k] = gs[b * LP + ctr + k];
                } else {
                    const T *gb = gn + (int64_t)((1 + b) * C + c) * HW + pix;
#pragma unroll
                    for (int k = 0; k < VEC; ++k) gv[k] = Elem<T>::to_f32(gb[k]);
                }
#pragma unroll
                for (int t = 0; t < KK; ++t) {
                    const int ki = t / K, kj = t % K;
                    const float *xn = xs + ctr + (ki - r) * D * LW + (kj - r) * D;
                    V dv;
#pragma unroll
                    for (int k = 0; k < VEC; ++k) set_lane<V, T, VEC>(dv, k, Elem<T>::from_f32(gv[k] * xn[k]));
                    const int64_t plane = (int64_t)(b * C + c) * KK + t;
                    __builtin_nontemporal_store(dv, (V *)(dkp + plane * HW + pix));
                }
            }
        }
        if constexpr (WANT_DX) {
            float acc[VEC];
            const T *gxs = gn + (int64_t)c * HW + pix;
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[k] = Elem<T>::to_f32(gxs[k]);
            // One dilation (K <= 3, VEC <= 4) or one kernel row at a time: the shifted tap
            // runs of a chunk are issued together without holding all 3K^2 in registers.
            constexpr int CH = (K <= 3 && VEC <= 4) ? KK : K;
#pragma unroll 1
            for (int bt = 0; bt < 3 * KK; bt += CH) {
                const int b = bt / KK;
                const int D = dilation(b);
#pragma unroll
                for (int j = 0; j < CH; ++j) {
                    const int t = bt - b * KK + j;
                    const int ki = t / K, kj = t % K;
                    const int dr = (ki - r) * D, dc = (kj - r) * D;
                    const int hs = h - dr;
                    const bool hok = hs >= 0 && hs < H;
                    const int64_t plane = (int64_t)(b * C + c) * KK + t;
                    float tv[VEC];
                    load_run<T, VEC>(tp + plane * HW + (int64_t)(hok ? hs : 0) * W, w - dc, W, hok, aligned != 0,
                                     tv);
                    const float *gsn = gs + b * LP + ctr - dr * LW - dc;
#pragma unroll
                    for (int k = 0; k < VEC; ++k) acc[k] += tv[k] * gsn[k];
                }
            }
            V ov;
#pragma unroll
            for (int k = 0; k < VEC; ++k) set_lane<V, T, VEC>(ov, k, Elem<T>::from_f32(acc[k]));
            *(V *)(gx + (int64_t)nc * HW + pix) = ov;
        }
    }
}

template <typename T, int K, int VEC, bool DX, bool DK>
static hipError_t launch_filter_bwd_t(const void *x, const void *taps, const void *gout, void *gx, void *gtaps, int N,
                                      int C, int H, int W, bool al, hipStream_t stream) {
    // dK alone stages one plane: wide rows as in the forward filter.  dX stages three
    // G_b planes: narrower, taller tiles keep the halo share and the LDS per block down.
    const int max_tpr = DX ? 32 : 64;
    int tw = VEC;
    while (tw < W && tw < max_tpr * VEC) tw *= 2;
    const int TW = tw;
    const int TH = 256 / (TW / VEC) > 0 ? 256 / (TW / VEC) : 1;
    constexpr int HALO = 5 * ((K - 1) / 2);
    constexpr int PADC = (HALO + 3) & ~3;
    const size_t planes = (DK ? 1 : 0) + (DX ? 3 : 0);
    const size_t lds = sizeof(float) * planes * (size_t)(TH + 2 * HALO) * (TW + 2 * PADC);
    auto kern = filter_bwd_kernel<T, K, VEC, DX, DK>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int nbands = (H + TH - 1) / TH;
    const int ncolt = (W + TW - 1) / TW;
    const int64_t nblk = (int64_t)N * C * nbands * ncolt;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), lds, stream, (const T *)x, (const T *)taps,
                       (const T *)gout, (T *)gx, (T *)gtaps, C, H, W, TH, TW, nbands, ncolt, al ? 1 : 0);
    return hipGetLastError();
}

template <typename T, int K, int VEC>
static hipError_t launch_filter_bwd_v(const void *x, const void *taps, const void *gout, void *gx, void *gtaps, int N,
                                      int C, int H, int W, bool al, hipStream_t stream) {
    if (gx != nullptr && gtaps != nullptr)
        return launch_filter_bwd_t<T, K, VEC, true, true>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    if (gx != nullptr)
        return launch_filter_bwd_t<T, K, VEC, true, false>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    return launch_filter_bwd_t<T, K, VEC, false, true>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
}

template <typename T, int K>
static hipError_t launch_filter_bwd_k(const void *x, const void *taps, const void *gout, void *gx, void *gtaps, int N,
                                      int C, int H, int W, int vec, bool al, hipStream_t stream) {
    if constexpr (Elem<T>::is_bf16) {
        if (vec == 8) return launch_filter_bwd_v<T, K, 8>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    } else {
        if (vec == 4) return launch_filter_bwd_v<T, K, 4>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    }
    if (vec == 2) return launch_filter_bwd_v<T, K, 2>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    return launch_filter_bwd_v<T, K, 1>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
}

hipError_t launch_filter_bwd(const void *x, const void *taps, const void *gout, void *gx, void *gtaps, int N, int C,
                             int H, int W, int K, bool bf16, int vec, bool al, hipStream_t stream) {
    if (bf16) {
        switch (K) {
            case 1: return launch_filter_bwd_k<bf16_t, 1>(x, taps, gout, gx, gtaps, N, C, H, W, vec, al, stream);
            case 3: return launch_filter_bwd_k<bf16_t, 3>(x, taps, gout, gx, gtaps, N, C, H, W, vec, al, stream);
            default: return launch_filter_bwd_k<bf16_t, 5>(x, taps, gout, gx, gtaps, N, C, H, W, vec, al, stream);
        }
    }
    switch (K) {
        case 1: return launch_filter_bwd_k<float, 1>(x, taps, gout, gx, gtaps, N, C, H, W, vec, al, stream);
        case 3: return launch_filter_bwd_k<float, 3>(x, taps, gout, gx, gtaps, N, C, H, W, vec, al, stream);
        default: return launch_filter_bwd_k<float, 5>(x, taps, gout, gx, gtaps, N, C, H, W, vec, al, stream);
    }
}

}  // namespace ddpm

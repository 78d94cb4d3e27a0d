// filter_fwd.hip -- dynamic dilated filter with materialised taps (gfx950).
//
// Operation (page "lartpang/DynamicConvolutionOperator", section "CUDA 动态过滤"):
// with the taps already generated, one pass serves the three dilations (1, 3, 5)
// from one spatial tile, accumulates in float32 and writes [x, d1, d3, d5].
//
// The pass is a pure stream: per pixel and channel it reads 3*K*K taps and one x
// value and writes four outputs, so it is bound by HBM bandwidth.  Design:
//   * one workgroup = one (n, c) plane x a TH x TW pixel tile;
//   * the x tile plus a 5*(K-1)/2 halo is staged once in LDS (as float), so every
//     dilation's neighbourhood is read from LDS, never re-fetched from HBM;
//   * each thread owns VEC consecutive pixels of a row (4 float32 or 4-8 bfloat16)
//     and streams the taps with non-temporal vector loads (they are touched
//     exactly once), and writes the four output planes with non-temporal vector
//     stores;
//   * for runs of 4 or more the staged x row of each row offset is read once as
//     aligned 16-byte LDS words, and every tap of that offset picks its values out
//     of those registers (fewer, conflict-free LDS reads than one read per tap);
//   * the x block of the output is copied from the staged tile bit-exactly.
#include "common.hpp"
#include "launchers.hpp"

namespace ddpm {

template <typename T, int K, int VEC>
__global__ __launch_bounds__(256) void filter_fwd_kernel(const T *__restrict__ x, const T *__restrict__ taps,
                                                         T *__restrict__ out, int C, int H, int W, int TH, int TW,
                                                         int nbands, int ncolt, int vec_stage) {
    constexpr int r = (K - 1) / 2;
    constexpr int HALO = 5 * r;
    constexpr int PADC = (HALO + 3) & ~3;  // column pad, rounded up so staged rows stay 16-byte aligned
    constexpr int KK = K * K;
    typedef typename VecOf<T, VEC>::type V;
    extern __shared__ float xs[];

    const int LW = TW + 2 * PADC;
    const int LH = TH + 2 * HALO;
    const int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int colt = L % ncolt;
    const int band = (L / ncolt) % nbands;
    const int nc = L / (ncolt * nbands);
    const int n = nc / C;
    const int c = nc - n * C;
    const int h0 = band * TH;
    const int w0 = colt * TW;
    const int64_t HW = (int64_t)H * W;

    // Stage rows h0-HALO .. h0+TH+HALO-1, columns w0-PADC .. w0+TW+PADC-1 of x
    // (vec_stage: W % 4 == 0 and x 16-byte (float) / 8-byte (bf16) aligned).
    stage_rows<T>(x + (int64_t)nc * HW, h0, w0, H, W, HALO, PADC, LW, 0, LH, xs, vec_stage != 0);
    __syncthreads();

    const int64_t R = 3LL * C * KK;
    const T *__restrict__ tp = taps + (int64_t)n * R * HW;
    T *__restrict__ op = out + (int64_t)n * 4 * C * HW;
    const int gpr = TW / VEC;
    for (int gi = threadIdx.x; gi < TH * gpr; gi += blockDim.x) {
        const int lr = gi / gpr;
        const int lc = (gi - lr * gpr) * VEC;
        const int h = h0 + lr;
        const int w = w0 + lc;
        if (h >= H || w >= W) continue;  // W % VEC == 0: a vector is wholly in or out
        const int64_t pix = (int64_t)h * W + w;
        const float *xc = xs + (lr + HALO) * LW + (lc + PADC);

        float acc[3][VEC];
#pragma unroll
        for (int b = 0; b < 3; ++b)
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[b][k] = 0.f;
        if constexpr (VEC >= 4) {
            // The taps of one row offset dr = (ki - r) * D read one staged row: it is
            // loaded once as aligned 16-byte runs covering columns lc - PADC ..
            // lc + VEC - 1 + PADC, and each tap takes its VEC values from the window at
            // a compile-time position.
            constexpr int NWIN = VEC / 4 + PADC / 2;  // 16-byte runs in the window
            V tv[3][KK];
#pragma unroll
            for (int b = 0; b < 3; ++b)
#pragma unroll
                for (int t = 0; t < KK; ++t)
                    tv[b][t] = __builtin_nontemporal_load(
                        (const V *)(tp + ((int64_t)(b * C + c) * KK + t) * HW + pix));
            const float *xw = xs + (lr + HALO) * LW + lc;  // window column 0 = pixel lc - PADC
#pragma unroll
            for (int dr = -HALO; dr <= HALO; ++dr) {
                bool used = false;
#pragma unroll
                for (int b = 0; b < 3; ++b)
#pragma unroll
                    for (int ki = 0; ki < K; ++ki) used = used || (ki - r) * dilation(b) == dr;
                if (!used) continue;
                float win[4 * NWIN];
#pragma unroll
                for (int q = 0; q < NWIN; ++q) {
                    const f32x4 v = *(const f32x4 *)(xw + dr * LW + 4 * q);
#pragma unroll
                    for (int e = 0; e < 4; ++e) win[4 * q + e] = v[e];
                }
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int D = dilation(b);
#pragma unroll
                    for (int t = 0; t < KK; ++t) {
                        const int ki = t / K, kj = t % K;
                        if ((ki - r) * D != dr) continue;
#pragma unroll
                        for (int k = 0; k < VEC; ++k)
                            acc[b][k] += Elem<T>::to_f32(lane_of<V, T, VEC>(tv[b][t], k)) *
                                         win[PADC + (kj - r) * D + k];
                    }
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                const int D = dilation(b);
#pragma unroll
                for (int t = 0; t < KK; ++t) {
                    const int ki = t / K, kj = t % K;
                    const int64_t plane = (int64_t)(b * C + c) * KK + t;
                    const V tv = __builtin_nontemporal_load((const V *)(tp + plane * HW + pix));
                    const float *xn = xc + (ki - r) * D * LW + (kj - r) * D;
#pragma unroll
                    for (int k = 0; k < VEC; ++k)
                        acc[b][k] += Elem<T>::to_f32(lane_of<V, T, VEC>(tv, k)) * xn[k];
                }
            }
        }
        V xv;
#pragma unroll
        for (int k = 0; k < VEC; ++k) set_lane<V, T, VEC>(xv, k, exact_narrow<T>(xc[k]));
        __builtin_nontemporal_store(xv, (V *)(op + (int64_t)c * HW + pix));
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            V ov;
#pragma unroll
            for (int k = 0; k < VEC; ++k) set_lane<V, T, VEC>(ov, k, Elem<T>::from_f32(acc[b][k]));
            __builtin_nontemporal_store(ov, (V *)(op + (int64_t)((1 + b) * C + c) * HW + pix));
        }
    }
}

// Tile choice: TW is the row segment one workgroup covers (a power of two, at most
// 64 vectors), TH the rows that give each of the 256 threads one vector.  Small
// tiles in XCD-contiguous order measured best on MI355X (fp32 256x256x64: 4-row
// tiles 90 us vs 8-row 98 us vs 16-row 108 us).
static void filter_tile(int W, int VEC, int &TH, int &TW) {
    int tw = VEC;
    while (tw < W && tw < 64 * VEC) tw *= 2;
    TW = tw;
    const int gpr = TW / VEC;
    TH = 256 / gpr > 0 ? 256 / gpr : 1;
}

template <typename T, int K, int VEC>
static hipError_t launch_filter_t(const void *x, const void *taps, void *out, int N, int C, int H, int W,
                                  hipStream_t stream) {
    int TH, TW;
    filter_tile(W, VEC, TH, TW);
    constexpr int HALO = 5 * ((K - 1) / 2);
    constexpr int PADC = (HALO + 3) & ~3;
    const size_t lds = sizeof(float) * (size_t)(TH + 2 * HALO) * (TW + 2 * PADC);
    auto kern = filter_fwd_kernel<T, K, VEC>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int nbands = (H + TH - 1) / TH;
    const int ncolt = (W + TW - 1) / TW;
    const int64_t nblk = (int64_t)N * C * nbands * ncolt;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const uintptr_t xal = Elem<T>::is_bf16 ? 8 : 16;
    const int vec_stage = (W % 4 == 0) && ((uintptr_t)x % xal == 0);
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), lds, stream, (const T *)x, (const T *)taps, (T *)out, C,
                       H, W, TH, TW, nbands, ncolt, vec_stage);
    return hipGetLastError();
}

template <typename T, int K>
static hipError_t launch_filter_k(const void *x, const void *taps, void *out, int N, int C, int H, int W,
                                  hipStream_t stream, int vec) {
    switch (vec) {
        case 8:
            if constexpr (Elem<T>::is_bf16) return launch_filter_t<T, K, 8>(x, taps, out, N, C, H, W, stream);
            return hipErrorInvalidValue;
        case 4: return launch_filter_t<T, K, 4>(x, taps, out, N, C, H, W, stream);
        case 2: return launch_filter_t<T, K, 2>(x, taps, out, N, C, H, W, stream);
        default: return launch_filter_t<T, K, 1>(x, taps, out, N, C, H, W, stream);
    }
}

hipError_t launch_filter_fwd(const void *x, const void *taps, void *out, int N, int C, int H, int W, int K,
                             bool bf16, int vec, hipStream_t stream) {
    if (bf16) {
        switch (K) {
            case 1: return launch_filter_k<bf16_t, 1>(x, taps, out, N, C, H, W, stream, vec);
            case 3: return launch_filter_k<bf16_t, 3>(x, taps, out, N, C, H, W, stream, vec);
            default: return launch_filter_k<bf16_t, 5>(x, taps, out, N, C, H, W, stream, vec);
        }
    }
    switch (K) {
        case 1: return launch_filter_k<float, 1>(x, taps, out, N, C, H, W, stream, vec);
        case 3: return launch_filter_k<float, 3>(x, taps, out, N, C, H, W, stream, vec);
        default: return launch_filter_k<float, 5>(x, taps, out, N, C, H, W, stream, vec);
    }
}

}  // namespace ddpm

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
// XCD-contiguous order, and each thread owns VEC consecutive pixels of a row.  The
// dilated neighbourhoods come from LDS (float, zero outside the image): x with the
// full 5*(K-1)/2 halo for dK, and for dX one G_b plane per dilation, staged with
// only that dilation's D*(K-1)/2 halo, so two planes of LDS serve all three.  The
// dK planes are streamed out with non-temporal vector stores.
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

// The value v holds in the lane `off` places away in this wave (lane l reads lane
// l + off), through whole-wave DPP shifts: wave_shr:1 moves lane l-1 into lane l,
// wave_shl:1 lane l+1.  Lanes past either end of the wave read 0.  `off` is a
// compile-time constant wherever this is inlined, so the loops fold away.
__device__ __forceinline__ float lane_from(float v, int off) {
    for (; off < 0; ++off) v = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true));
    for (; off > 0; --off) v = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true));
    return v;
}

constexpr int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// LS (lane shift): one tile spans the whole image row, so the VEC-pixel runs of a row
// sit in consecutive lanes of one wave.  Every operand is then read at the lane's own
// aligned position of the shifted row and the column offset is taken from
// neighbouring lanes; otherwise shifted runs are read from LDS at the offset column
// and tap runs are loaded at the shifted column with bounds checks.
template <typename T, int K, int VEC, bool WANT_DX, bool WANT_DK, bool LS>
__global__ __launch_bounds__(256) void filter_bwd_kernel(const T *__restrict__ x, const T *__restrict__ taps,
                                                         const T *__restrict__ gout, T *__restrict__ gx,
                                                         T *__restrict__ gtaps, int C, int H, int W, int TH, int TW,
                                                         int nbands, int ncolt, int aligned, int vec_stage) {
    constexpr int r = (K - 1) / 2;
    constexpr int HALO = 5 * r;
    constexpr int PADC = LS ? 0 : (HALO + 3) & ~3;  // lane shifts never read beyond the tile's columns
    constexpr int KK = K * K;
    typedef typename VecOf<T, VEC>::type V;
    // Lane shifts read LDS only at the lane's own aligned runs: the input's own bits
    // are staged (half the LDS for bfloat16); the checked path reads shifted floats.
    typedef typename std::conditional<LS, T, float>::type LT;
    extern __shared__ __align__(16) unsigned char lds_bytes[];

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
    const bool vst = vec_stage != 0;

    // LDS: x with the full halo (dK), then one G_b plane at a time (dX).
    LT *xs = (LT *)lds_bytes;
    LT *gs = xs + (WANT_DK ? LP : 0);
    if constexpr (WANT_DK) stage_rows<T>(x + (int64_t)nc * HW, h0, w0, H, W, HALO, PADC, LW, 0, LH, xs, vst);

    // TH * TW / VEC == 256: each thread owns one run of VEC pixels of one row.
    const int gpr = TW / VEC;
    const int lr = threadIdx.x / gpr;
    const int lc = (threadIdx.x - lr * gpr) * VEC;
    const int h = h0 + lr;
    const int w = w0 + lc;
    const bool active = h < H && w < W;  // W % VEC == 0: a run is wholly in or out
    const int64_t pix = (int64_t)h * W + w;
    const int ctr = (lr + HALO) * LW + lc + PADC;  // staged index of the run's first pixel
    const int64_t R = 3LL * C * KK;
    const T *__restrict__ tp = taps + (int64_t)n * R * HW;
    T *__restrict__ dkp = gtaps + (int64_t)n * R * HW;

    float acc[VEC];
    if constexpr (WANT_DX) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[k] = active ? Elem<T>::to_f32(gn[(int64_t)c * HW + pix + k]) : 0.f;
    }

#pragma unroll
    for (int b = 0; b < 3; ++b) {
        const int D = dilation(b);
        const T *__restrict__ gbp = gn + (int64_t)((1 + b) * C + c) * HW;
        if constexpr (WANT_DX) {
            // G_b is read only D*r rows and columns beyond the tile.
            if (b > 0) __syncthreads();  // every thread is done with G_{b-1}
            stage_rows<T>(gbp, h0, w0, H, W, HALO, PADC, LW, HALO - D * r, HALO + TH + D * r, gs, vst);
        }
        if (b == 0 || WANT_DX) __syncthreads();

        if constexpr (LS) {
            // Per kernel row: one aligned row of x (dK) and of G_b (dX) from LDS serves
            // all K taps; the column offset is taken from neighbouring lanes.  Every
            // lane of the wave takes part; lanes past the image hold zeros or are
            // masked.  A value moved in from lane l + m counts only if that lane's run
            // starts inside this image row.
            constexpr int LM = (HALO + VEC - 1) / VEC + 1;
            bool src_ok[2 * LM + 1];
#pragma unroll
            for (int m = -LM; m <= LM; ++m) src_ok[m + LM] = (unsigned)(w + m * VEC) < (unsigned)W;
            // Runs start at multiples of VEC elements of LDS (LW = TW, lc and the plane
            // size are multiples of VEC), so they are read as aligned vectors.
            auto lds_run = [](const LT *p, float(&v)[VEC]) {
                const V u = *(const V *)p;
#pragma unroll
                for (int k = 0; k < VEC; ++k) v[k] = Elem<T>::to_f32(lane_of<V, T, VEC>(u, k));
            };
            float gv[VEC];  // G_b at the lane's own pixels (dK)
            if constexpr (WANT_DK) {
                if constexpr (WANT_DX) {
                    lds_run(gs + ctr, gv);
                } else {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) gv[k] = active ? Elem<T>::to_f32(gbp[pix + k]) : 0.f;
                }
            }
#pragma unroll 1
            for (int ki = 0; ki < K; ++ki) {
                const int dr = (ki - r) * D;
                if constexpr (WANT_DK) {
                    // dK[p] = G_b[p] * x[p + (dr, dc)]
                    float xr[VEC];
                    lds_run(xs + ctr + dr * LW, xr);
#pragma unroll
                    for (int kj = 0; kj < K; ++kj) {
                        const int dc = (kj - r) * D;
                        V dv;
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const int src = e + dc;
                            const int m = floor_div(src, VEC);
                            float xv = lane_from(xr[src - m * VEC], m);
                            if (m != 0) xv = src_ok[m + LM] ? xv : 0.f;
                            set_lane<V, T, VEC>(dv, e, Elem<T>::from_f32(gv[e] * xv));
                        }
                        const int64_t plane = (int64_t)(b * C + c) * KK + ki * K + kj;
                        if (active) __builtin_nontemporal_store(dv, (V *)(dkp + plane * HW + pix));
                    }
                }
                if constexpr (WANT_DX) {
                    // dX[q] += taps[q - (dr, dc)] * G_b[q - (dr, dc)]: the product is formed
                    // at the source pixel (the lane's own aligned run of row h - dr) and
                    // then moved by dc columns.
                    const int hs = h - dr;
                    const bool hok = active && hs >= 0 && hs < H;
                    const int64_t row =
                        (int64_t)((b * C + c) * KK + ki * K) * HW + (int64_t)(hok ? hs : 0) * W + w;
                    float gr[VEC];
                    lds_run(gs + ctr - dr * LW, gr);
#pragma unroll
                    for (int kj = 0; kj < K; ++kj) {
                        const int dc = (kj - r) * D;
                        V rv = {};
                        if (hok) rv = __builtin_nontemporal_load((const V *)(tp + row + (int64_t)kj * HW));
                        float pr[VEC];
#pragma unroll
                        for (int e = 0; e < VEC; ++e) pr[e] = Elem<T>::to_f32(lane_of<V, T, VEC>(rv, e)) * gr[e];
#pragma unroll
                        for (int j = 0; j < VEC; ++j) {
                            const int src = j - dc;  // column of the source pixel, relative to w
                            const int m = floor_div(src, VEC);
                            float v = lane_from(pr[src - m * VEC], m);
                            if (m != 0) v = src_ok[m + LM] ? v : 0.f;
                            acc[j] += v;
                        }
                    }
                }
            }
        } else {
            if (WANT_DK && active) {
                float gv[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) gv[k] = WANT_DX ? gs[ctr + k] : Elem<T>::to_f32(gbp[pix + k]);
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
            if constexpr (WANT_DX) {
                if (!active) continue;
                // The source runs of one kernel row (K = 5, or 8-wide runs) or of the whole
                // dilation are issued together, without holding all 3K^2 in registers.
                constexpr int CH = (K <= 3 && VEC <= 4) ? KK : K;
#pragma unroll 1
                for (int t0 = 0; t0 < KK; t0 += CH) {
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        const int t = t0 + j;
                        const int ki = t / K, kj = t % K;
                        const int dr = (ki - r) * D, dc = (kj - r) * D;
                        const int hs = h - dr;
                        const bool hok = hs >= 0 && hs < H;
                        const int64_t plane = (int64_t)(b * C + c) * KK + t;
                        float tv[VEC];
                        load_run<T, VEC>(tp + plane * HW + (int64_t)(hok ? hs : 0) * W, w - dc, W, hok, aligned != 0,
                                         tv);
                        const float *gsn = gs + ctr - dr * LW - dc;
#pragma unroll
                        for (int k = 0; k < VEC; ++k) acc[k] += tv[k] * gsn[k];
                    }
                }
            }
        }
    }
    if constexpr (WANT_DX) {
        if (active) {
            V ov;
#pragma unroll
            for (int k = 0; k < VEC; ++k) set_lane<V, T, VEC>(ov, k, Elem<T>::from_f32(acc[k]));
            *(V *)(gx + (int64_t)nc * HW + pix) = ov;
        }
    }
}

template <typename T, int K, int VEC, bool DX, bool DK, bool LS>
static hipError_t launch_filter_bwd_t(const void *x, const void *taps, const void *gout, void *gx, void *gtaps, int N,
                                      int C, int H, int W, bool al, hipStream_t stream) {
    // dK alone and the lane-shift dX: wide rows (a tile spans the row when it fits in
    // 64 runs).  The checked dX re-stages G_b per dilation: narrower, taller tiles
    // keep the halo share down.
    const int max_tpr = (DX && !LS) ? 32 : 64;
    int tw = VEC;
    while (tw < W && tw < max_tpr * VEC) tw *= 2;
    const int TW = tw;
    if (LS && TW < W) return hipErrorInvalidValue;
    const int TH = 256 / (TW / VEC) > 0 ? 256 / (TW / VEC) : 1;
    constexpr int HALO = 5 * ((K - 1) / 2);
    constexpr int PADC = LS ? 0 : (HALO + 3) & ~3;
    const size_t planes = (DK ? 1 : 0) + (DX ? 1 : 0);
    const size_t lds = (LS ? sizeof(T) : sizeof(float)) * planes * (size_t)(TH + 2 * HALO) * (TW + 2 * PADC);
    auto kern = filter_bwd_kernel<T, K, VEC, DX, DK, LS>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int nbands = (H + TH - 1) / TH;
    const int ncolt = (W + TW - 1) / TW;
    const int64_t nblk = (int64_t)N * C * nbands * ncolt;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const uintptr_t pal = Elem<T>::is_bf16 ? 8 : 16;
    const int vec_stage = (W % 4 == 0) && ((uintptr_t)x % pal == 0) && ((uintptr_t)gout % pal == 0);
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), lds, stream, (const T *)x, (const T *)taps,
                       (const T *)gout, (T *)gx, (T *)gtaps, C, H, W, TH, TW, nbands, ncolt, al ? 1 : 0, vec_stage);
    return hipGetLastError();
}

template <typename T, int K, int VEC>
static hipError_t launch_filter_bwd_v(const void *x, const void *taps, const void *gout, void *gx, void *gtaps, int N,
                                      int C, int H, int W, bool al, hipStream_t stream) {
    // Lane shifts need the row in one tile (and, for dX, vector-aligned tap runs).
    if (gx == nullptr) {
        if (W <= 64 * VEC)
            return launch_filter_bwd_t<T, K, VEC, false, true, true>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
        return launch_filter_bwd_t<T, K, VEC, false, true, false>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    }
    const bool ls = W <= 64 * VEC && (uintptr_t)taps % (VEC * sizeof(T)) == 0;
    if (gtaps != nullptr) {
        if (ls) return launch_filter_bwd_t<T, K, VEC, true, true, true>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
        return launch_filter_bwd_t<T, K, VEC, true, true, false>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    }
    if (ls) return launch_filter_bwd_t<T, K, VEC, true, false, true>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
    return launch_filter_bwd_t<T, K, VEC, true, false, false>(x, taps, gout, gx, gtaps, N, C, H, W, al, stream);
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

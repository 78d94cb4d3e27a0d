/*
 * ddpm_oracle.c -- plain fp64 CPU oracle for the Dynamic Dilated Pyramid Module (DDPM).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check of the
 * package entry file and the cpu_baseline leg of the benchmark may load this
 * library.  It shares no code, header, table or helper with the HIP library; it
 * knows nothing of tiles, MFMA, LDS, partial splits or reduced precision.
 *
 * Source of truth: the page "lartpang/DynamicConvolutionOperator -- Better and
 * Faster Implementation Dynamic Dilated Pyramid Module from HDFNet (ECCV 2020)".
 *   - Intro ("Dynamic Convolution Operator"): the unfold implementation is the
 *     mathematical reference of the method.
 *   - "问题与目标" (problem and goal): the reference builds three Unfold(x) patch
 *     tensors and a generator output of N*3*C*K^2*H*W dynamic kernels; the
 *     optimised versions keep the ordinary dynamic depthwise convolution maths.
 *   - "CUDA 动态过滤" (dynamic filter): one pass over dilations (1, 3, 5), output
 *     written as [x, d1, d3, d5]; backward produces dX and dK.
 *   - "CUDA 融合生成器推理" (fused generator inference): a 1x1 generator
 *     dot(weight, y) produces the taps that are consumed with shifted x.
 *   - "CUDA Flash 式融合训练" (flash-style fused training): dX gathers each
 *     dilation's contribution with recomputed taps; dK = shifted(x) * grad is
 *     contracted with the generator weight for dY and reduced over space for
 *     dWeight / dbias.
 *
 * Readings taken where the page leaves a step open (each one is listed in the
 * design notes of the repository):
 *   - generator channel order o(b,c,t) = (b*C + c)*K*K + t, dilation-major, then
 *     channel, then tap, which is the order N*3*C*K^2*H*W the page lists;
 *   - tap t = ki*K + kj (row-major), applied as a cross-correlation without
 *     flipping, exactly as an unfold patch is laid out;
 *   - branch b uses dilation D_b in {1,3,5}, zero padding D_b*(K-1)/2, stride 1,
 *     so every branch has the input's spatial size;
 *   - out-of-image neighbours contribute nothing (zero padding), which the
 *     loops below express as a bounds test, not as a padded copy.
 *
 * Every sum is accumulated in double in the plain loop order written here, so
 * results are independent of the number of OpenMP threads.
 *
 * Layouts (all contiguous, row-major):
 *   x, y      [N][C][H][W]
 *   Wg        [R][C]      with R = 3*C*K*K
 *   bg        [R]
 *   taps      [N][R][H][W]
 *   out, G    [N][4C][H][W]   channel blocks: x, d1, d3, d5
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

static const int DILATION[3] = {1, 3, 5};

/* Generator channel of branch b, depthwise channel c, tap t. */
static int64_t gen_row(int b, int64_t c, int t, int64_t C, int K)
{
    return ((int64_t)b * C + c) * (int64_t)(K * K) + t;
}

/* 1x1 generator at one pixel: T[o] = bg[o] + sum_c' Wg[o][c'] * y[c'][pixel]. */
static void generator_at_pixel(const double *y, const double *Wg, const double *bg,
                               int64_t n, int64_t h, int64_t w,
                               int64_t C, int64_t H, int64_t W, int K,
                               double *yv /* [C] scratch */, double *T /* [R] */)
{
    const int64_t R = 3 * C * K * K;
    for (int64_t ci = 0; ci < C; ++ci)
        yv[ci] = y[((n * C + ci) * H + h) * W + w];
    for (int64_t o = 0; o < R; ++o) {
        double acc = bg[o];
        const double *wrow = Wg + o * C;
        for (int64_t ci = 0; ci < C; ++ci)
            acc += wrow[ci] * yv[ci];
        T[o] = acc;
    }
}

/*
 * Materialise the generator output taps[N][R][H][W] (the page's second big
 * intermediate, N*3*C*K^2*H*W elements).
 */
void ddpm_oracle_generator(const double *y, const double *Wg, const double *bg, double *taps,
                           int64_t N, int64_t C, int64_t H, int64_t W, int K)
{
    const int64_t R = 3 * C * K * K;
    const int64_t HW = H * W;
#pragma omp parallel
    {
        double *yv = (double *)malloc(sizeof(double) * (size_t)C);
        double *T = (double *)malloc(sizeof(double) * (size_t)R);
#pragma omp for schedule(static)
        for (int64_t np = 0; np < N * HW; ++np) {
            const int64_t n = np / HW, h = (np % HW) / W, w = np % W;
            generator_at_pixel(y, Wg, bg, n, h, w, C, H, W, K, yv, T);
            for (int64_t o = 0; o < R; ++o)
                taps[(n * R + o) * HW + h * W + w] = T[o];
        }
        free(yv);
        free(T);
    }
}

/*
 * One output pixel of the three branches given its taps T[o] (o over all R rows
 * of this pixel, stride tstride between consecutive rows).
 *   O_b[n,c,h,w] = sum_t T[o(b,c,t)] * x[n, c, h+(ki-r)*D_b, w+(kj-r)*D_b]
 * with out-of-image x taken as zero.
 */
static double branch_at_pixel(const double *x, const double *T, int64_t tstride,
                              int b, int64_t n, int64_t c, int64_t h, int64_t w,
                              int64_t C, int64_t H, int64_t W, int K)
{
    const int r = (K - 1) / 2;
    const int D = DILATION[b];
    double acc = 0.0;
    for (int ki = 0; ki < K; ++ki) {
        for (int kj = 0; kj < K; ++kj) {
            const int64_t hh = h + (int64_t)(ki - r) * D;
            const int64_t ww = w + (int64_t)(kj - r) * D;
            if (hh < 0 || hh >= H || ww < 0 || ww >= W)
                continue;
            const int t = ki * K + kj;
            acc += T[gen_row(b, c, t, C, K) * tstride] * x[((n * C + c) * H + hh) * W + ww];
        }
    }
    return acc;
}

/*
 * Dynamic dilated filter with materialised taps ("CUDA 动态过滤"):
 *   out[:, 0:C] = x,   out[:, C(1+b):C(2+b)] = O_b,  b = 0,1,2 for D = 1,3,5.
 */
void ddpm_oracle_filter_fwd(const double *x, const double *taps, double *out,
                            int64_t N, int64_t C, int64_t H, int64_t W, int K)
{
    const int64_t R = 3 * C * K * K;
    const int64_t HW = H * W;
#pragma omp parallel for schedule(static)
    for (int64_t np = 0; np < N * HW; ++np) {
        const int64_t n = np / HW, h = (np % HW) / W, w = np % W;
        const double *T = taps + n * R * HW + h * W + w; /* row o at T[o*HW] */
        for (int64_t c = 0; c < C; ++c) {
            out[((n * 4 * C + c) * H + h) * W + w] = x[((n * C + c) * H + h) * W + w];
            for (int b = 0; b < 3; ++b)
                out[((n * 4 * C + (1 + b) * C + c) * H + h) * W + w] =
                    branch_at_pixel(x, T, HW, b, n, c, h, w, C, H, W, K);
        }
    }
}

/*
 * Generator fused with the filter ("CUDA 融合生成器推理"): the taps of a pixel are
 * produced from y at that same pixel and consumed at once.  The result is the
 * same as ddpm_oracle_generator followed by ddpm_oracle_filter_fwd.
 */
void ddpm_oracle_fused_fwd(const double *x, const double *y, const double *Wg, const double *bg,
                           double *out, int64_t N, int64_t C, int64_t H, int64_t W, int K)
{
    const int64_t R = 3 * C * K * K;
    const int64_t HW = H * W;
#pragma omp parallel
    {
        double *yv = (double *)malloc(sizeof(double) * (size_t)C);
        double *T = (double *)malloc(sizeof(double) * (size_t)R);
#pragma omp for schedule(static)
        for (int64_t np = 0; np < N * HW; ++np) {
            const int64_t n = np / HW, h = (np % HW) / W, w = np % W;
            generator_at_pixel(y, Wg, bg, n, h, w, C, H, W, K, yv, T);
            for (int64_t c = 0; c < C; ++c) {
                out[((n * 4 * C + c) * H + h) * W + w] = x[((n * C + c) * H + h) * W + w];
                for (int b = 0; b < 3; ++b)
                    out[((n * 4 * C + (1 + b) * C + c) * H + h) * W + w] =
                        branch_at_pixel(x, T, 1, b, n, c, h, w, C, H, W, K);
            }
        }
        free(yv);
        free(T);
    }
}

/*
 * Backward of the fused forward ("CUDA Flash 式融合训练"), written as the plain
 * adjoint of the loops above.  G = dL/d out is [N][4C][H][W]; G_x = G[:,0:C] and
 * G_b = G[:, C(1+b):C(2+b)].
 *
 *   dK[n,o,p]  = G_b[n,c,p] * x[n,c,p+delta_{b,t}]            (zero outside)
 *   dX[n,c,q]  = G_x[n,c,q] + sum_{b,t,p : p+delta=q} T[n,o,p] * G_b[n,c,p]
 *   dY[n,c',p] = sum_o Wg[o,c'] * dK[n,o,p]
 *   dWg[o,c']  = sum_{n,p} dK[n,o,p] * y[n,c',p]
 *   dbg[o]     = sum_{n,p} dK[n,o,p]
 *
 * dX is formed here by scattering each source pixel's contribution to the
 * neighbour it read in the forward pass; the GPU library gathers instead, so the
 * two sides do not share a formulation.
 */
void ddpm_oracle_fused_bwd(const double *x, const double *y, const double *Wg, const double *bg,
                           const double *G, double *dx, double *dy, double *dWg, double *dbg,
                           int64_t N, int64_t C, int64_t H, int64_t W, int K)
{
    const int64_t R = 3 * C * K * K;
    const int64_t HW = H * W;
    const int r = (K - 1) / 2;
    const int KK = K * K;

    /* dX: one owner per (n, c) plane, so the scatter needs no synchronisation. */
#pragma omp parallel
    {
        double *yv = (double *)malloc(sizeof(double) * (size_t)C);
        double *Tc = (double *)malloc(sizeof(double) * (size_t)(3 * KK));
#pragma omp for schedule(static)
        for (int64_t nc = 0; nc < N * C; ++nc) {
            const int64_t n = nc / C, c = nc % C;
            double *dxp = dx + (n * C + c) * HW;
            const double *Gx = G + (n * 4 * C + c) * HW;
            for (int64_t q = 0; q < HW; ++q)
                dxp[q] = Gx[q];
            for (int64_t h = 0; h < H; ++h) {
                for (int64_t w = 0; w < W; ++w) {
                    /* the 3*K*K taps of channel c at source pixel (h, w) */
                    for (int64_t ci = 0; ci < C; ++ci)
                        yv[ci] = y[((n * C + ci) * H + h) * W + w];
                    for (int b = 0; b < 3; ++b) {
                        for (int t = 0; t < KK; ++t) {
                            const int64_t o = gen_row(b, c, t, C, K);
                            double acc = bg[o];
                            for (int64_t ci = 0; ci < C; ++ci)
                                acc += Wg[o * C + ci] * yv[ci];
                            Tc[b * KK + t] = acc;
                        }
                    }
                    for (int b = 0; b < 3; ++b) {
                        const double gb = G[((n * 4 * C + (1 + b) * C + c) * H + h) * W + w];
                        const int D = DILATION[b];
                        for (int ki = 0; ki < K; ++ki) {
                            for (int kj = 0; kj < K; ++kj) {
                                const int64_t hh = h + (int64_t)(ki - r) * D;
                                const int64_t ww = w + (int64_t)(kj - r) * D;
                                if (hh < 0 || hh >= H || ww < 0 || ww >= W)
                                    continue;
                                dxp[hh * W + ww] += Tc[b * KK + ki * K + kj] * gb;
                            }
                        }
                    }
                }
            }
        }
        free(yv);
        free(Tc);
    }

    /* dY: one owner per pixel. */
#pragma omp parallel
    {
        double *dK = (double *)malloc(sizeof(double) * (size_t)R);
#pragma omp for schedule(static)
        for (int64_t np = 0; np < N * HW; ++np) {
            const int64_t n = np / HW, h = (np % HW) / W, w = np % W;
            for (int b = 0; b < 3; ++b) {
                const int D = DILATION[b];
                for (int64_t c = 0; c < C; ++c) {
                    const double gb = G[((n * 4 * C + (1 + b) * C + c) * H + h) * W + w];
                    for (int ki = 0; ki < K; ++ki) {
                        for (int kj = 0; kj < K; ++kj) {
                            const int64_t hh = h + (int64_t)(ki - r) * D;
                            const int64_t ww = w + (int64_t)(kj - r) * D;
                            double xv = 0.0;
                            if (hh >= 0 && hh < H && ww >= 0 && ww < W)
                                xv = x[((n * C + c) * H + hh) * W + ww];
                            dK[gen_row(b, c, ki * K + kj, C, K)] = gb * xv;
                        }
                    }
                }
            }
            for (int64_t ci = 0; ci < C; ++ci) {
                double acc = 0.0;
                for (int64_t o = 0; o < R; ++o)
                    acc += Wg[o * C + ci] * dK[o];
                dy[((n * C + ci) * H + h) * W + w] = acc;
            }
        }
        free(dK);
    }

    /* dWg, dbg: one owner per generator row o; sum over (n, p) in ascending order. */
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < R; ++o) {
        const int b = (int)(o / (C * KK));
        const int64_t c = (o / KK) % C;
        const int t = (int)(o % KK);
        const int ki = t / K, kj = t % K;
        const int D = DILATION[b];
        double sb = 0.0;
        double *wrow = dWg + o * C;
        for (int64_t ci = 0; ci < C; ++ci)
            wrow[ci] = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t h = 0; h < H; ++h) {
                for (int64_t w = 0; w < W; ++w) {
                    const int64_t hh = h + (int64_t)(ki - r) * D;
                    const int64_t ww = w + (int64_t)(kj - r) * D;
                    if (hh < 0 || hh >= H || ww < 0 || ww >= W)
                        continue; /* dK is exactly zero here */
                    const double dk = G[((n * 4 * C + (1 + b) * C + c) * H + h) * W + w] *
                                      x[((n * C + c) * H + hh) * W + ww];
                    sb += dk;
                    for (int64_t ci = 0; ci < C; ++ci)
                        wrow[ci] += dk * y[((n * C + ci) * H + h) * W + w];
                }
            }
        }
        dbg[o] = sb;
    }
}

/*
 * Backward of the materialised filter ("CUDA 动态过滤": the backward produces dX and
 * dK, the gradient of the dynamic kernels).  With G = dL/d out:
 *   dtaps[n,o,p] = G_b[n,c,p] * x[n,c,p+delta_{b,t}]            (zero outside)
 *   dx[n,c,q]    = G_x[n,c,q] + sum_{b,t,p : p+delta=q} taps[n,o,p] * G_b[n,c,p]
 * dx is formed by scattering each source pixel's contribution, as in the fused
 * backward above.
 */
void ddpm_oracle_filter_bwd(const double *x, const double *taps, const double *G, double *dx, double *dtaps,
                            int64_t N, int64_t C, int64_t H, int64_t W, int K)
{
    const int64_t R = 3 * C * K * K;
    const int64_t HW = H * W;
    const int r = (K - 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t nc = 0; nc < N * C; ++nc) {
        const int64_t n = nc / C, c = nc % C;
        double *dxp = dx + (n * C + c) * HW;
        const double *Gx = G + (n * 4 * C + c) * HW;
        for (int64_t q = 0; q < HW; ++q)
            dxp[q] = Gx[q];
        for (int b = 0; b < 3; ++b) {
            const int D = DILATION[b];
            const double *Gb = G + (n * 4 * C + (1 + b) * C + c) * HW;
            for (int ki = 0; ki < K; ++ki) {
                for (int kj = 0; kj < K; ++kj) {
                    const int64_t o = gen_row(b, c, ki * K + kj, C, K);
                    const double *tp = taps + (n * R + o) * HW;
                    double *dtp = dtaps + (n * R + o) * HW;
                    for (int64_t h = 0; h < H; ++h) {
                        for (int64_t w = 0; w < W; ++w) {
                            const int64_t hh = h + (int64_t)(ki - r) * D;
                            const int64_t ww = w + (int64_t)(kj - r) * D;
                            const int inside = hh >= 0 && hh < H && ww >= 0 && ww < W;
                            dtp[h * W + w] = inside ? Gb[h * W + w] * x[((n * C + c) * H + hh) * W + ww] : 0.0;
                            if (inside)
                                dxp[hh * W + ww] += tp[h * W + w] * Gb[h * W + w];
                        }
                    }
                }
            }
        }
    }
}

/*
 * Sum of per-split fp32 partials, in ascending split order, in double.
 * partial[s][m] for s < S, m < M  ->  sum[m].
 */
void ddpm_oracle_sum_partials(const double *partial, double *sum, int64_t S, int64_t M)
{
    for (int64_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int64_t s = 0; s < S; ++s)
            acc += partial[s * M + m];
        sum[m] = acc;
    }
}

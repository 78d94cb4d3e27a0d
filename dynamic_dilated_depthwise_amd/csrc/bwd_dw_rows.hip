// bwd_dw_rows.hip -- weight / bias gradient partials of the fused training backward
// for C = 64 (gfx950), staged by row segment.
//
// Operation (page "lartpang/DynamicConvolutionOperator", section
// "CUDA Flash 式融合训练": dWeight / dbias form dK on chip and reduce it over space
// into at most 16 float32 partials over contiguous token ranges):
//     dK[o(b,c,t), p] = G_b[c, p] * x[c, p + d_bt]      (x zero outside the image),
//     dW_s[o, c']     = sum_{p in range s} dK[o, p] * y[c', p],
//     db_s[o]         = sum_{p in range s} dK[o, p].
//
// Work decomposition: workgroup = one (branch b, kernel row ki) x 16 depthwise
// channels c0 .. c0+15 x all 64 input channels c' x one token range s (the same
// grid and ranges as the general kernel).  The range is walked in row segments of
// SEG tokens (64 float32, 128 bfloat16; a segment ends early at a row end or at the
// range end).  Per segment, y (64 channel rows), G_b (16 rows) and the x row
// h + (ki - r) * D_b with a column halo (16 rows) are copied into LDS with
// coalesced 16-byte loads; the buffers are double-buffered, so one barrier per
// segment separates the copy of segment i+1 from the products of segment i, and the
// global loads of segment i+2 are in flight meanwhile.  The four waves take one
// quarter of the segment's tokens each and sum their partial products in wave order
// through LDS at the end.
//   MFMA rows    = channel c0 + i of tap (ki, kj) (one 16-row tile per tap kj);
//   MFMA columns = c' = 16 nb + j (four blocks);
//   contraction  = tokens: float32 4 per k-step (lane group g holds 4 consecutive
//                  tokens, one per k-step), bfloat16 32 per k-step (8 per group).
// bfloat16: dK is rounded to bfloat16 as the MFMA operand; db sums the unrounded
// products, obtained from one more MFMA per tap that multiplies the raw G_b and
// shifted-x operands (exact bf16 products, float32 sums) and keeps the diagonal.
#include <type_traits>

#include "common.hpp"
#include "launchers.hpp"

namespace ddpm {
namespace {

constexpr int kChW = 64;   // channels this kernel serves
constexpr int kWvW = 4;    // waves per workgroup

template <typename T, int K> struct DwPlan {
    static constexpr bool BF = Elem<T>::is_bf16;
    static constexpr int ES = sizeof(T);             // bytes per element
    static constexpr int VE = 16 / ES;               // elements per 16-byte slot
    static constexpr int TPW = BF ? 32 : 16;         // tokens per wave per segment
    static constexpr int SEG = kWvW * TPW;           // tokens per segment (256 bytes of a row)
    static constexpr int r = (K - 1) / 2;
    static constexpr int KK = K * K;
    static constexpr int HALO = 5 * r;
    static constexpr int LP = (HALO + VE - 1) / VE * VE;  // staged x columns left of the segment
    static constexpr int XW = SEG + 2 * LP;          // staged x columns
    // Row strides (elements): 16 bytes past a multiple of 32 bytes, so the 16 rows
    // that one MFMA operand read touches start in 16 distinct 16-byte bank groups.
    static constexpr int YR = SEG + VE;
    static constexpr int XR = XW + VE;
    static constexpr int YSL = kChW * SEG / VE;      // 16-byte slots per segment: y
    static constexpr int GSL = 16 * SEG / VE;        //   G_b (256)
    static constexpr int XSR = XW / VE;              //   x slots per row
    static constexpr int XSL = 16 * XSR;             //   x
    static constexpr int YIT = YSL / 256;
    static constexpr int XIT = (XSL + 255) / 256;
    static constexpr int YB = kChW * YR * ES;        // bytes per buffer part
    static constexpr int GB = 16 * YR * ES;
    static constexpr int XB = 16 * XR * ES;
    static constexpr int DB = 64 * 16;               // x slots past the staged width land here
    static constexpr int BUF = YB + GB + XB + DB;
    static constexpr int RED = (kWvW * 16 * 64 + kWvW * 64) * 4;  // one tap's cross-wave sums
    static constexpr int LDS = 2 * BUF > RED ? 2 * BUF : RED;
    static_assert(GSL == 256, "one G_b slot per thread");
    static_assert(YSL % 256 == 0, "whole y slots per thread");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_a2 __attribute__((ext_vector_type(8), aligned(2)));

// WHOLE: the batch's y, x and gradient tensors each fit one buffer resource (the
// host checks the byte sizes): the resources are built once and an image is a scalar
// offset, so a segment's loads cost no descriptor or 64-bit pointer arithmetic.
template <typename T, int K, bool WHOLE>
__global__ __launch_bounds__(256, 2) void bwd_dw_rows_kernel(const T *__restrict__ x, const T *__restrict__ y,
                                                             const T *__restrict__ gout, float *__restrict__ dw_part,
                                                             float *__restrict__ db_part, int N, int H, int W, int S) {
    using P = DwPlan<T, K>;
    constexpr bool BF = P::BF;
    constexpr int r = P::r;
    constexpr int KK = P::KK;
    constexpr int C = kChW;
    constexpr int SEG = P::SEG;
    constexpr int VE = P::VE;
    extern __shared__ __align__(16) unsigned char lds_w[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    // Logical order: (b, ki) fastest, then the channel block, then the split, laid
    // out XCD-contiguously so that the workgroups of one split (which read the same
    // y, x and G rows) share an L2.
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int combo = L % (3 * K);
    L /= 3 * K;
    const int c0 = (L & 3) * 16;
    const int s = L >> 2;
    const int b = combo / K;
    const int ki = combo - b * K;
    const int D = 1 + 2 * b;
    const int dr = (ki - r) * D;
    const int HW = H * W;
    const int64_t ntok = (int64_t)N * HW;
    // Split s covers [t0, t1): the even cut ntok*s/S rounded down to a multiple of
    // 64 (float32) or 128 (bfloat16) tokens; the last split ends at ntok.
    constexpr int64_t ROUND = BF ? 128 : 64;
    const int64_t t0 = ntok * s / S / ROUND * ROUND;
    const int64_t t1 = s + 1 == S ? ntok : ntok * (s + 1) / S / ROUND * ROUND;

    // ---- the segment loader: cursor (tl; image ln, row lh, column lw).  Buffer
    // loads: a slot outside the segment or the image gets an offset past the
    // buffer's end, which reads as zero; the per-thread parts of the offsets are
    // fixed, the row position is a scalar offset.  (WHOLE: fewer than 2^31 tokens,
    // so the cursor is 32-bit.)
    using TokT = typename std::conditional<WHOLE, int, int64_t>::type;
    TokT tl = (TokT)t0;
    const TokT tend = (TokT)t1;
    int ln = 0, lh = 0, lw = 0;
    if (tl < tend) {
        ln = (int)(tl / HW);
        const int rem = (int)(tl - (int64_t)ln * HW);
        lh = rem / W;
        lw = rem - lh * W;
    }
    constexpr unsigned OOB = 0x7ffffff0u;
    constexpr int W3 = 0x00020000;  // buffer descriptor word 3 (gfx9: raw 32-bit data)
    unsigned yoff[P::YIT], xrow[P::XIT];
    int xcol[P::XIT];
#pragma unroll
    for (int k = 0; k < P::YIT; ++k) {
        const int q = tid + 256 * k;
        yoff[k] = (unsigned)(((q >> 4) * HW + (q & 15) * VE) * P::ES);
    }
    const unsigned goff = (unsigned)(((tid >> 4) * HW + (tid & 15) * VE) * P::ES);
    const int ycol = (tid & 15) * VE;  // the y / G slot's column within the segment
#pragma unroll
    for (int k = 0; k < P::XIT; ++k) {
        const int q = tid + 256 * k;
        const int row = q / P::XSR;
        xrow[k] = (unsigned)(row * HW);
        xcol[k] = q < P::XSL ? (q - row * P::XSR) * VE - P::LP : -(1 << 30);  // past the width: never valid
    }
    // one segment's 16-byte slots in registers; two sets in turn keep the loads of a
    // segment in flight for two segments' products
    struct Regs {
        u32x4 y[P::YIT], g, x[P::XIT];
    };
    // image bases of the cursor, advanced with it: pointers, or (WHOLE) byte offsets
    // into resources over the whole tensors
    const T *yb = y + (int64_t)ln * C * HW;
    const T *gb = gout + ((int64_t)ln * 4 * C + (1 + b) * C + c0) * HW;
    const T *xb = x + ((int64_t)ln * C + c0) * HW;
    int iy = 0, ig = 0, ix = 0;
    if constexpr (WHOLE) {
        iy = ln * C * HW * P::ES;
        ig = ((ln * 4 + 1 + b) * C + c0) * HW * P::ES;
        ix = (ln * C + c0) * HW * P::ES;
    }
    const __amdgpu_buffer_rsrc_t wy = __builtin_amdgcn_make_buffer_rsrc((void *)y, 0, WHOLE ? N * C * HW * P::ES : 0, W3);
    const __amdgpu_buffer_rsrc_t wg =
        __builtin_amdgcn_make_buffer_rsrc((void *)gout, 0, WHOLE ? N * 4 * C * HW * P::ES : 0, W3);
    const __amdgpu_buffer_rsrc_t wx = __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, WHOLE ? N * C * HW * P::ES : 0, W3);
    auto load_seg = [&](Regs &o) {  // the segment at the cursor -> o; advances the cursor
        const TokT left = tend - tl;  // may be <= 0 past the range: every slot reads zero
        const int lc = left < 0 ? 0 : (left > SEG ? SEG : (int)left);
        const int wl = W - lw;
        const int len = lc < wl ? lc : wl;
        const __amdgpu_buffer_rsrc_t ry =
            WHOLE ? wy : __builtin_amdgcn_make_buffer_rsrc((void *)yb, 0, C * HW * P::ES, W3);
        const __amdgpu_buffer_rsrc_t rg =
            WHOLE ? wg : __builtin_amdgcn_make_buffer_rsrc((void *)gb, 0, 16 * HW * P::ES, W3);
        const __amdgpu_buffer_rsrc_t rx =
            WHOLE ? wx : __builtin_amdgcn_make_buffer_rsrc((void *)xb, 0, 16 * HW * P::ES, W3);
        const int by = iy, bgo = ig, bx = ix;  // the image's scalar offsets (zero unless WHOLE)
        const int soff = (lh * W + lw) * P::ES;
        const bool yok = ycol < len;
#pragma unroll
        for (int k = 0; k < P::YIT; ++k)
            o.y[k] = __builtin_bit_cast(u32x4,
                                        __builtin_amdgcn_raw_buffer_load_b128(ry, yok ? yoff[k] : OOB, by + soff, 0));
        o.g = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, yok ? goff : OOB, bgo + soff, 0));
        // x row lh + dr, columns lw - LP .. (W % VE == 0: a slot is wholly in or out)
        const int hs = lh + dr;
        const bool rok = hs >= 0 && hs < H && len > 0;
        const int xs_off = rok ? hs * W * P::ES : 0;
#pragma unroll
        for (int k = 0; k < P::XIT; ++k) {
            const int col = lw + xcol[k];
            const bool ok = rok && col >= 0 && col < W;
            o.x[k] = __builtin_bit_cast(
                u32x4,
                __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (xrow[k] + (unsigned)col) * P::ES : OOB, bx + xs_off, 0));
        }
        // advance (selects, no branches)
        tl += len;
        lw += len;
        const bool wrap = lw == W;
        lw = wrap ? 0 : lw;
        lh += wrap ? 1 : 0;
        const bool wrap2 = lh == H;
        lh = wrap2 ? 0 : lh;
        ln += wrap2 ? 1 : 0;
        if constexpr (WHOLE) {
            iy += wrap2 ? C * HW * P::ES : 0;
            ig += wrap2 ? 4 * C * HW * P::ES : 0;
            ix += wrap2 ? C * HW * P::ES : 0;
        } else {
            yb += wrap2 ? (int64_t)C * HW : 0;
            gb += wrap2 ? (int64_t)4 * C * HW : 0;
            xb += wrap2 ? (int64_t)C * HW : 0;
        }
    };
    // staged-slot destinations (elements from the buffer start); x slots past the
    // staged width go to the dummy area, one slot per lane
    int ydst[P::YIT], xdst[P::XIT];
#pragma unroll
    for (int k = 0; k < P::YIT; ++k) {
        const int q = tid + 256 * k;
        ydst[k] = (q >> 4) * P::YR + (q & 15) * VE;
    }
    const int gdst = P::YB / P::ES + (tid >> 4) * P::YR + (tid & 15) * VE;
#pragma unroll
    for (int k = 0; k < P::XIT; ++k) {
        const int q = tid + 256 * k;
        const int row = q / P::XSR;
        xdst[k] = q < P::XSL ? (P::YB + P::GB) / P::ES + row * P::XR + (q - row * P::XSR) * VE
                             : (P::YB + P::GB + P::XB) / P::ES + lane * VE;
    }
    auto store_seg = [&](const Regs &o, int buf) {
        T *base = (T *)(lds_w + buf * P::BUF);
#pragma unroll
        for (int k = 0; k < P::YIT; ++k) *(u32x4 *)(base + ydst[k]) = o.y[k];
        *(u32x4 *)(base + gdst) = o.g;
#pragma unroll
        for (int k = 0; k < P::XIT; ++k) *(u32x4 *)(base + xdst[k]) = o.x[k];
    };

    // ---- accumulators: dW tile per tap kj and nb; db per tap
    f32x4 acc[K][4];
    f32x4 dbm[K];     // bfloat16: G x x^T tile per tap (its diagonal is db)
    float dbacc[K];   // float32: per-lane sum of the lane's dK
#pragma unroll
    for (int kj = 0; kj < K; ++kj) {
        dbm[kj] = f32x4{0.f, 0.f, 0.f, 0.f};
        dbacc[kj] = 0.f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[kj][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // lane's operands within a buffer: y row 16nb + j, G and x row j (A role: channel
    // c0 + j), tokens TPW*wave + (4 | 8) g ..
    constexpr int LT = BF ? 8 : 4;  // tokens per lane
    const int ytok = P::TPW * wave + LT * g;
    // The products of one segment run in NGRP groups of MFMAs (float32: one k-step
    // per group; bfloat16: one tap per group).  The copy of the next segment into the
    // other buffer follows the first group and the loads of the segment three ahead
    // the second, so each wave interleaves its own staging with its MFMAs and every
    // load has two segments' products to land.
    constexpr int NGRP = BF ? K : 4;
    // step: products of the segment in buffer `buf`; copies `rs` (the next segment,
    // if `have_store`) into the other buffer, then loads the segment at the cursor
    // into `rs`.  Returns whether that segment exists.
    auto step = [&](int buf, Regs &rs, bool have_store) {
        const unsigned char *base = lds_w + buf * P::BUF;
        const T *ys = (const T *)base + j * P::YR + ytok;
        const T *gs = (const T *)(base + P::YB) + j * P::YR + ytok;
        const T *xs = (const T *)(base + P::YB + P::GB) + j * P::XR + P::LP + ytok;
        // the copy and the loads run whether or not those segments exist (past the
        // range every slot reads zero and the copy is never read), so the step is
        // one straight block the scheduler can interleave
        (void)have_store;
        const bool loaded = tl < tend;
        auto between = [&](int grp) {
            if (grp == 0) store_seg(rs, buf ^ 1);
            if (grp == (NGRP > 1 ? 1 : 0)) load_seg(rs);
        };
        if constexpr (!BF) {
            const f32x4 gv = *(const f32x4 *)gs;
            f32x4 yv[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) yv[nb] = *(const f32x4 *)(ys + 16 * nb * P::YR);
            float a[K][4];
#pragma unroll
            for (int kj = 0; kj < K; ++kj) {
                const f32x4 xv = *(const f32x4_a4 *)(xs + (kj - r) * D);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    a[kj][kk] = gv[kk] * xv[kk];
                    dbacc[kj] += a[kj][kk];
                }
            }
#pragma unroll
            for (int kk = 0; kk < NGRP; ++kk) {
#pragma unroll
                for (int kj = 0; kj < K; ++kj)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) acc[kj][nb] = mfma_16x16x4_f32(a[kj][kk], yv[nb][kk], acc[kj][nb]);
                between(kk);
            }
        } else {
            const u32x4 graw = *(const u32x4 *)gs;
            float gf[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                gf[2 * m] = __uint_as_float(graw[m] << 16);
                gf[2 * m + 1] = __uint_as_float(graw[m] & 0xffff0000u);
            }
            bf16x8 yv[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) yv[nb] = __builtin_bit_cast(bf16x8, *(const u16x8 *)(ys + 16 * nb * P::YR));
#pragma unroll
            for (int kj = 0; kj < NGRP; ++kj) {
                const u16x8 xr = *(const u16x8_a2 *)(xs + (kj - r) * D);
                const u32x4 xw = __builtin_bit_cast(u32x4, xr);
                u16x8 u;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    u[2 * m] = f32_to_bf16_bits(gf[2 * m] * __uint_as_float(xw[m] << 16));
                    u[2 * m + 1] = f32_to_bf16_bits(gf[2 * m + 1] * __uint_as_float(xw[m] & 0xffff0000u));
                }
                const bf16x8 av = __builtin_bit_cast(bf16x8, u);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[kj][nb] = mfma_16x16x32_bf16(av, yv[nb], acc[kj][nb]);
                dbm[kj] = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, graw), __builtin_bit_cast(bf16x8, xr), dbm[kj]);
                between(kj);
            }
        }
        return loaded;
    };

    // ---- the segment pipeline.  At the top of a step computing segment i from
    // buffer i & 1: segment i+1 is in the register set of parity i+1 (h1), segment
    // i+2 is in flight into the set of parity i (h2).
    Regs r0, r1;
    bool h0 = tl < tend;
    load_seg(r0);
    bool h1 = tl < tend;
    load_seg(r1);
    store_seg(r0, 0);
    __syncthreads();
    bool h2 = tl < tend;
    load_seg(r0);
    while (h0) {
        bool h3 = step(0, r1, h1);
        __syncthreads();
        h0 = h1;
        h1 = h2;
        h2 = h3;
        if (!h0) break;
        h3 = step(1, r0, h1);
        __syncthreads();
        h0 = h1;
        h1 = h2;
        h2 = h3;
    }

    // ---- fixed-order sums over the four waves, one tap at a time
    float *red = (float *)lds_w;                  // [wave][nb*4 + v][lane]
    float *redb = red + kWvW * 16 * 64;           // [wave][64]
    float *dwp = dw_part + (int64_t)s * (3 * C * KK) * C;
    float *dbp = db_part + (int64_t)s * (3 * C * KK);
#pragma unroll
    for (int kj = 0; kj < K; ++kj) {
        const int t = ki * K + kj;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(wave * 16 + nb * 4 + v) * 64 + lane] = acc[kj][nb][v];
        if constexpr (BF) {
            // lane (g, j) holds G x x^T[4g + v][j]; the diagonal sits at v = j - 4g
            float dv = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (j == 4 * g + v) dv = dbm[kj][v];
            redb[wave * 64 + lane] = dv;
        } else {
            redb[wave * 64 + lane] = dbacc[kj];
        }
        __syncthreads();
        {
            const int nb = wave;
            const int cp = 16 * nb + j;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int c = c0 + 4 * g + v;
                float sum = red[(0 * 16 + nb * 4 + v) * 64 + lane];
#pragma unroll
                for (int wv = 1; wv < kWvW; ++wv) sum += red[(wv * 16 + nb * 4 + v) * 64 + lane];  // fixed order
                dwp[((int64_t)(b * C + c) * KK + t) * C + cp] = sum;
            }
        }
        if (wave == 0 && g == 0) {
            float sb = 0.f;
            if constexpr (BF) {
#pragma unroll
                for (int wv = 0; wv < kWvW; ++wv) sb += redb[wv * 64 + (j >> 2) * 16 + j];
            } else {
#pragma unroll
                for (int wv = 0; wv < kWvW; ++wv)
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) sb += redb[wv * 64 + gg * 16 + j];
            }
            dbp[(int64_t)(b * C + c0 + j) * KK + t] = sb;
        }
        __syncthreads();
    }
}

template <typename T, int K>
static hipError_t launch_dw_rows_t(const void *x, const void *y, const void *gout, float *dwp, float *dbp, int S,
                                   int N, int H, int W, hipStream_t stream) {
    constexpr int lds = DwPlan<T, K>::LDS;
    // bfloat16 with the whole gradient tensor (the largest of the three) within a
    // buffer resource's range, below the offset that reads zero (bf16 256x256, K = 3:
    // 66.7 -> 62.2 us; float32 measured 2 % slower that way at K = 3 and keeps the
    // per-image resources)
    const bool whole =
        Elem<T>::is_bf16 && (int64_t)N * 4 * kChW * H * W * (int64_t)sizeof(T) < (int64_t)0x7ffffff0;
    auto kern = bwd_dw_rows_kernel<T, K, false>;
    if constexpr (Elem<T>::is_bf16) {
        if (whole) kern = bwd_dw_rows_kernel<T, K, true>;
    }
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    const int64_t nblk = (int64_t)3 * K * 4 * S;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), lds, stream, (const T *)x, (const T *)y, (const T *)gout,
                       dwp, dbp, N, H, W, S);
    return hipGetLastError();
}

}  // namespace

// Applicability: C = 64, 16-byte aligned tensors (checked by the caller), W a
// multiple of 4 (float32) or 8 (bfloat16), and an image's 64 channel planes within
// 2^31 bytes (the buffer offsets).
bool bwd_dw_rows_applies(int C, int H, int W, bool al, bool bf16) {
    return C == kChW && al && (W % (bf16 ? 8 : 4)) == 0 && (int64_t)kChW * H * W * (bf16 ? 2 : 4) < (int64_t(1) << 31);
}

hipError_t launch_bwd_dw_rows(const void *x, const void *y, const void *gout, float *dw_part, float *db_part, int S,
                              int N, int H, int W, int K, bool bf16, hipStream_t stream) {
    if (bf16) {
        switch (K) {
            case 1: return launch_dw_rows_t<bf16_t, 1>(x, y, gout, dw_part, db_part, S, N, H, W, stream);
            case 3: return launch_dw_rows_t<bf16_t, 3>(x, y, gout, dw_part, db_part, S, N, H, W, stream);
            default: return launch_dw_rows_t<bf16_t, 5>(x, y, gout, dw_part, db_part, S, N, H, W, stream);
        }
    }
    switch (K) {
        case 1: return launch_dw_rows_t<float, 1>(x, y, gout, dw_part, db_part, S, N, H, W, stream);
        case 3: return launch_dw_rows_t<float, 3>(x, y, gout, dw_part, db_part, S, N, H, W, stream);
        default: return launch_dw_rows_t<float, 5>(x, y, gout, dw_part, db_part, S, N, H, W, stream);
    }
}

}  // namespace ddpm

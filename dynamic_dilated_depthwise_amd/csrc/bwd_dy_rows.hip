// bwd_dy_rows.hip -- dY of the fused training backward in float32 for C = 64 (gfx950),
// staged by source row.
//
// Operation (page "lartpang/DynamicConvolutionOperator", section
// "CUDA Flash 式融合训练": dY forms dK = shifted(x) * grad on chip and contracts it
// with the generator weight at once):
//     dK[o(b,c,t), p] = G_b[c, p] * x[c, p + d_bt]      (x zero outside the image),
//     dY[c', p]       = sum_o W[o, c'] * dK[o, p].
//
// Work decomposition: workgroup = one 64-pixel row segment (row h, columns w0..) x
// all 64 output channels c'; the four waves split the contraction by input channel
// (wave v takes c = 16v .. 16v+15, four k-steps of 4) and every wave walks the same
// (branch, kernel row) stages, so one staging serves them all: per stage the x row
// h + dr (dr = (ki - r) * D_b, with a column halo) and, when the branch changes,
// the G_b row h are copied into LDS as channel rows, once, between two barriers;
// their global loads are issued a whole stage ahead.  Each tap is 64 MFMAs
// (v_mfma_f32_16x16x4_f32) per wave:
//   rows    = 16 output channels of block mb: row i is channel 4i + mb, so a lane's
//             four weights of one generator row are one 16-byte load;
//   columns = 16 lanes x 4 adjacent pixels 4j + pb (one product per pb);
//   k       = lane group g: input channel 16v + 4s + g in k-step s.
// The B operand dK is formed in registers from the staged G and x.  The four waves'
// partial sums are added in wave order through LDS at the end; a stage whose x row
// lies outside the image contributes nothing and is skipped.
#include "common.hpp"
#include "launchers.hpp"

namespace ddpm {
namespace {

constexpr int kSegY = 64;  // pixels per workgroup (one row segment)
constexpr int kChY = 64;   // channels this kernel serves

template <int K> struct DyPlan {
    static constexpr int r = (K - 1) / 2;
    static constexpr int KK = K * K;
    static constexpr int NT = 3 * KK;
    static constexpr int NST = 3 * K;                 // (branch, kernel row) stages, branch-major
    static constexpr int HALO = 5 * r;
    static constexpr int LP = (HALO + 3) & ~3;        // staged x columns left of the segment
    static constexpr int SW = kSegY + 2 * LP;         // staged x columns
    static constexpr int XROW = SW + 4;               // floats per staged x channel row
    static constexpr int GROW = kSegY + 4;            // floats per staged G channel row
    static constexpr int XBUF = kChY * XROW;
    static constexpr int GBUF = kChY * GROW;
    static constexpr int RED = 4 * 64 * 32;           // floats: the partials of two output blocks of four waves
    static constexpr int LDS = (XBUF + GBUF) > RED ? (XBUF + GBUF) : RED;
};

template <int K>
__global__ __launch_bounds__(256, 2) void bwd_dy_f32_kernel(const float *__restrict__ x,
                                                            const float *__restrict__ wg,
                                                            const float *__restrict__ gout,
                                                            float *__restrict__ gy, int H, int W) {
    using P = DyPlan<K>;
    constexpr int r = P::r;
    constexpr int KK = P::KK;
    constexpr int NT = P::NT;
    constexpr int NST = P::NST;
    constexpr int C = kChY;
    __shared__ __align__(16) float lds[P::LDS];
    float *xs = lds;             // staged x row   [c][XROW]
    float *gsb = lds + P::XBUF;  // staged G_b row [c][GROW]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    const int nseg = (W + kSegY - 1) / kSegY;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int w0 = (L % nseg) * kSegY;
    L /= nseg;
    const int h = L % H;
    const int n = L / H;
    const int HW = H * W;
    const float *__restrict__ xn = x + (int64_t)n * C * HW;
    const float *__restrict__ gn = gout + (int64_t)n * 4 * C * HW;

    // ---- staging: runs of 4 pixels of one channel row, copied as they are; runs
    // outside the image (W % 4 == 0: wholly in or out) load the row's first run and
    // are zeroed
    constexpr int NXR = kChY * (P::SW / 4);           // x runs
    constexpr int XIT = (NXR + 255) / 256;
    constexpr int NGR = kChY * (kSegY / 4);           // G runs
    constexpr int GIT = NGR / 256;
    f32x4 xreg[XIT], greg[GIT];
    unsigned xoff[XIT], goff[GIT];
    int xdst[XIT], gdst[GIT];
    bool xok[XIT], xex[XIT], gok[GIT];
#pragma unroll
    for (int k = 0; k < XIT; ++k) {
        const int q = tid + 256 * k;
        const int ch = q / (P::SW / 4);
        const int px4 = q - ch * (P::SW / 4);
        const int col = w0 - P::LP + 4 * px4;
        xex[k] = q < NXR;
        xok[k] = xex[k] && col >= 0 && col < W;
        xoff[k] = (unsigned)((xex[k] ? ch : 0) * HW + (xok[k] ? col : 0));
        xdst[k] = ch * P::XROW + 4 * px4;
    }
#pragma unroll
    for (int k = 0; k < GIT; ++k) {
        const int q = tid + 256 * k;
        const int ch = q >> 4;
        const int px4 = q & 15;
        const int col = w0 + 4 * px4;
        gok[k] = col < W;
        goff[k] = (unsigned)(ch * HW + (gok[k] ? col : 0));
        gdst[k] = ch * P::GROW + 4 * px4;
    }
    auto x_row = [&](int st) { return h + ((st % K) - r) * (1 + 2 * (st / K)); };
    auto load_stage = [&](int st) {
        const int hs = x_row(st);
        if (hs >= 0 && hs < H) {  // wave-uniform: otherwise the stage is skipped
            const float *xb = xn + hs * W;
#pragma unroll
            for (int k = 0; k < XIT; ++k) {
                const f32x4 v = *(const f32x4 *)(xb + xoff[k]);
                xreg[k] = xok[k] ? v : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (st % K == 0) {  // a new branch: its G row
            const float *gb = gn + (1 + st / K) * C * HW + h * W;
#pragma unroll
            for (int k = 0; k < GIT; ++k) {
                const f32x4 v = *(const f32x4 *)(gb + goff[k]);
                greg[k] = gok[k] ? v : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto store_stage = [&](int st) {
        const int hs = x_row(st);
        if (hs >= 0 && hs < H) {
#pragma unroll
            for (int k = 0; k < XIT; ++k)
                if (xex[k]) *(f32x4 *)(xs + xdst[k]) = xreg[k];
        }
        if (st % K == 0) {
#pragma unroll
            for (int k = 0; k < GIT; ++k) *(f32x4 *)(gsb + gdst[k]) = greg[k];
        }
    };

    // ---- weights of tap (b, t), one tap ahead: for k-step s, the generator row of
    // input channel c = 16v + 4s + g, output channels 4j .. 4j+3
    const float *__restrict__ wl = wg + (16 * wave + g) * KK * C + 4 * j;
    struct WOps { f32x4 w[4]; };
    auto fetch = [&](int bt, WOps &o) {  // bt = b*KK + t
        const int b = bt / KK;
        const int t = bt - b * KK;
        const float *wt = wl + (b * C * KK + t) * C;
#pragma unroll
        for (int s = 0; s < 4; ++s) o.w[s] = *(const f32x4 *)(wt + 4 * s * KK * C);
    };

    f32x4 acc[4][4];  // [mb][pb]
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[mb][pb] = f32x4{0.f, 0.f, 0.f, 0.f};

    WOps ring[2];  // operands of tap bt in ring[bt & 1]
    load_stage(0);
    fetch(0, ring[0]);
    // lane's x / G runs: channel 16v + 4s + g, pixels 4j .. 4j+3 (x shifted by dc)
    const int x_lane = (16 * wave + g) * P::XROW + 4 * j;
    const int g_lane = (16 * wave + g) * P::GROW + 4 * j;
#pragma clang loop unroll(full)
    for (int st = 0; st < NST; ++st) {
        const int b = st / K;
        const int ki = st % K;
        const int D = 1 + 2 * b;
        const int hs = h + (ki - r) * D;
        const bool rok = hs >= 0 && hs < H;
        if (st > 0) __syncthreads();  // every wave is done reading the previous stage
        store_stage(st);
        __syncthreads();
        if (st + 1 < NST) load_stage(st + 1);
#pragma clang loop unroll(full)
        for (int kj = 0; kj < K; ++kj) {
            const int bt = b * KK + ki * K + kj;
            const WOps &cur = ring[bt & 1];
            if (bt + 1 < NT) fetch(bt + 1, ring[(bt + 1) & 1]);
            if (rok) {
                const int dc = (kj - r) * D;
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 gv = *(const f32x4 *)(gsb + g_lane + 4 * s * P::GROW);
                    const f32x4 xv = *(const f32x4_a4 *)(xs + x_lane + 4 * s * P::XROW + P::LP + dc);
                    f32x4 dk;
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) dk[pb] = gv[pb] * xv[pb];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int pb = 0; pb < 4; ++pb)
                            acc[mb][pb] = mfma_16x16x4_f32(cur.w[s][mb], dk[pb], acc[mb][pb]);
                }
                __builtin_amdgcn_s_setprio(0);
            }
        }
    }

    // ---- the four waves' partial sums, added in wave order: two output blocks at a
    // time through LDS; wave (mb & 1) ... sums block mb
    float *red = lds;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();  // the staged rows (or the previous half) are no longer read
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
                *(f32x4 *)(red + ((wave * 64 + lane) * 2 + q) * 16 + 4 * pb) = acc[2 * half + q][pb];
        __syncthreads();
        if (wave < 2) {
            const int mb = 2 * half + wave;
            f32x4 sum[4];
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) sum[pb] = *(const f32x4 *)(red + ((0 * 64 + lane) * 2 + wave) * 16 + 4 * pb);
#pragma unroll
            for (int wv = 1; wv < 4; ++wv)
#pragma unroll
                for (int pb = 0; pb < 4; ++pb)
                    sum[pb] += *(const f32x4 *)(red + ((wv * 64 + lane) * 2 + wave) * 16 + 4 * pb);
            // row 4g + v of block mb is output channel 4(4g + v) + mb; columns are
            // pixels 4j + pb
            float *yo = gy + (int64_t)n * C * HW + h * W + w0 + 4 * j;
            if (w0 + 4 * j < W) {  // W % 4 == 0: runs are whole
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int cp = 4 * (4 * g + v) + mb;
                    *(f32x4 *)(yo + cp * HW) = f32x4{sum[0][v], sum[1][v], sum[2][v], sum[3][v]};
                }
            }
        }
    }
}

}  // namespace

// Applicability: float32, C = 64, W % 4 == 0, 16-byte aligned tensors (checked by
// the caller) and plane offsets within 32 bits.
bool bwd_dy_rows_applies(int C, int H, int W, bool al) {
    return C == kChY && al && (W % 4) == 0 && (int64_t)4 * kChY * H * W < (int64_t(1) << 31);
}

hipError_t launch_bwd_dy_rows(const void *x, const void *wg, const void *gout, void *gy, int N, int H, int W, int K,
                              hipStream_t stream) {
    const int64_t nblk = (int64_t)N * H * ((W + kSegY - 1) / kSegY);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nblk), block(256);
    const float *X = (const float *)x, *Wg = (const float *)wg, *G = (const float *)gout;
    float *GY = (float *)gy;
    switch (K) {
        case 1: hipLaunchKernelGGL(bwd_dy_f32_kernel<1>, grid, block, 0, stream, X, Wg, G, GY, H, W); break;
        case 3: hipLaunchKernelGGL(bwd_dy_f32_kernel<3>, grid, block, 0, stream, X, Wg, G, GY, H, W); break;
        default: hipLaunchKernelGGL(bwd_dy_f32_kernel<5>, grid, block, 0, stream, X, Wg, G, GY, H, W); break;
    }
    return hipGetLastError();
}

}  // namespace ddpm

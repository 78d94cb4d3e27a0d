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
// the G_b row h are copied into LDS as channel rows, once; x is double-buffered by
// stage and G_b by branch, so the copy of the next stage follows the current
// stage's products with one barrier per stage, and its global loads are issued two
// stages ahead.  Each tap is 64 MFMAs
// (v_mfma_f32_16x16x4_f32) per wave:
//   rows    = 16 output channels of block mb: row i is channel 4i + mb, so a lane's
//             four weights of one generator row are one 16-byte load;
//   columns = 16 lanes x 4 adjacent pixels 4j + pb (one product per pb);
//   k       = lane group g: input channel 16v + 4s + g in k-step s.
// The B operand dK is formed in registers from the staged G and x.  The four waves'
// partial sums are added in wave order through LDS at the end; a stage whose x row
// lies outside the image contributes nothing and is skipped.
//
// bfloat16 (bwd_dy_bf16_kernel): one MFMA k-step covers 32 input channels, so the
// waves split pixels instead and each forms dK only for its own pixels, once:
// workgroup = one 256-pixel row segment, wave v = pixels 32v .. 32v+31 x all 64
// output channels (for small grids: one 128-pixel segment x 32 output channels, the
// segment's two halves in neighbouring workgroups) (v_mfma_f32_16x16x32_bf16):
//   rows    = 16 pixels 16pb + i of the wave (two blocks pb);
//   columns = 16 output channels 16nb + j (four blocks nb, two when split);
//   k       = 32 input channels 32ks + 8g + e (two k-steps ks).
// x and G_b are staged as [channel/8][pixel][8] so that a lane's eight channels of
// one pixel are one 16-byte LDS read at any column shift; each wave keeps its
// pixels' G_b in float32 registers for a whole branch.  The K taps' weight rows of
// a stage are staged as they are stored ([c][c'] per tap) and read transposed into
// the B layout with ds_read_b64_tr_b16.  dK = rne(G * x) (exact product, one
// rounding) is the A operand; the sums stay in float32 and are rounded once.
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
    // two x buffers (stage parity) and two G_b buffers (branch parity): the copy of
    // the next stage goes to the buffers the current stage does not read
    static constexpr int LDS = 2 * (XBUF + GBUF) > RED ? 2 * (XBUF + GBUF) : RED;
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
    // staged x rows [2][c][XROW] by stage parity, G_b rows [2][c][GROW] by branch parity
    float *xs0 = lds;
    float *gs0 = lds + 2 * P::XBUF;

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
        float *xs = xs0 + (st & 1) * P::XBUF;
        float *gsb = gs0 + ((st / K) & 1) * P::GBUF;
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
    // lane's x / G runs: channel 16v + 4s + g, pixels 4j .. 4j+3 (x shifted by dc)
    const int x_lane = (16 * wave + g) * P::XROW + 4 * j;
    const int g_lane = (16 * wave + g) * P::GROW + 4 * j;
    // stage 0 is copied before the loop; the copy of stage st+1 follows stage st's
    // products, into the other buffers, and one barrier per stage separates them
    load_stage(0);
    fetch(0, ring[0]);
    store_stage(0);
    __syncthreads();
    if (NST > 1) load_stage(1);
#pragma clang loop unroll(full)
    for (int st = 0; st < NST; ++st) {
        const int b = st / K;
        const int ki = st % K;
        const int D = 1 + 2 * b;
        const int hs = h + (ki - r) * D;
        const bool rok = hs >= 0 && hs < H;
        const float *xs = xs0 + (st & 1) * P::XBUF;
        const float *gsb = gs0 + (b & 1) * P::GBUF;
#pragma clang loop unroll(full)
        for (int kj = 0; kj < K; ++kj) {
            const int bt = b * KK + ki * K + kj;
            const WOps &cur = ring[bt & 1];
            if (bt + 1 < NT) fetch(bt + 1, ring[(bt + 1) & 1]);
            if (rok) {
                const int dc = (kj - r) * D;
                // the x run starts dc columns off an aligned word (a constant once the
                // loops are unrolled); an unaligned start reads two aligned 16-byte words
                const int xo = P::LP + dc;
                const int xm = xo & 3;
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 gv = *(const f32x4 *)(gsb + g_lane + 4 * s * P::GROW);
                    const float *xa = xs + x_lane + 4 * s * P::XROW + (xo - xm);
                    const f32x4 x0 = *(const f32x4 *)xa;
                    f32x4 xv = x0;
                    if (xm != 0) {
                        const f32x4 x1 = *(const f32x4 *)(xa + 4);
                        if (xm == 1) xv = f32x4{x0[1], x0[2], x0[3], x1[0]};
                        else if (xm == 2) xv = f32x4{x0[2], x0[3], x1[0], x1[1]};
                        else xv = f32x4{x0[3], x1[0], x1[1], x1[2]};
                    }
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
        if (st + 1 < NST) store_stage(st + 1);
        __syncthreads();
        if (st + 2 < NST) load_stage(st + 2);
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


// ============================================================================ bfloat16
constexpr int kPxB = 32;    // pixels per wave (two MFMA row blocks)

// SEG pixels per workgroup (SEG / 32 waves), NCP of the 64 output channels per
// workgroup (64, or 32 with the two halves in neighbouring workgroups, for grids
// that are otherwise too small: each half forms the segment's dK itself).
template <int K, int SEG, int NCP> struct DyPlanB {
    static constexpr int WAVES = SEG / kPxB;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int NB = NCP / 16;          // output-channel blocks per wave
    static constexpr int r = (K - 1) / 2;
    static constexpr int KK = K * K;
    static constexpr int NST = 3 * K;            // (branch, kernel row) stages, branch-major
    static constexpr int HALO = 5 * r;
    static constexpr int LP = (HALO + 7) & ~7;   // staged x pixels left of the segment (8-pixel runs)
    static constexpr int XS = SEG + 2 * LP;      // staged x pixels
    // 16-byte slots per channel-group plane: one more than a multiple of 16, so the
    // staging writes of 16 consecutive lanes (8 planes x 2 runs) hit distinct banks
    static constexpr int XP = (XS + 15) / 16 * 16 + 1;
    static constexpr int GP = SEG + 1;
    static constexpr int WR = NCP + 16;          // bf16 elements per staged weight row (NCP + pad)
    static constexpr int WSR = NCP / 8;          // 16-byte weight slots per row
    static constexpr int NXI = XS;               // x items (8 channels x 8 pixels): 8 planes x XS/8
    static constexpr int XIT = (NXI + THREADS - 1) / THREADS;
    static constexpr int NGI = SEG;              // G items, taken by the last SEG threads
    static constexpr int WIT = K * 64 * WSR / THREADS;  // 16-byte weight slots per thread per stage
    static_assert(K * 64 * WSR % THREADS == 0, "whole weight slots per thread");
    static constexpr int XOFF = 0;               // byte offsets of the LDS regions
    static constexpr int GOFF = XOFF + 8 * XP * 16;
    static constexpr int WOFF = GOFF + 8 * GP * 16;
    static constexpr int LDS = WOFF + K * 64 * WR * 2;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Eight channel runs of eight pixels (u[e] = channel e, pixels 0..7 as bf16 pairs)
// to eight pixel runs of eight channels (o[k] = pixel k, channels 0..7): each output
// pair is one v_perm_b32, whose selector bytes 0-3 address the second operand's
// bytes and 4-7 the first's (low halves: 0x05040100, high halves: 0x07060302).
__device__ __forceinline__ void transpose8x8_bf16(const u32x4 (&u)[8], u32x4 (&o)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            o[k][m] = __builtin_amdgcn_perm(u[2 * m + 1][k >> 1], u[2 * m][k >> 1],
                                            (k & 1) ? 0x07060302u : 0x05040100u);
}

template <int K, int SEG, int NCP>
__global__ __launch_bounds__((DyPlanB<K, SEG, NCP>::THREADS), 1) void bwd_dy_bf16_kernel(const bf16_t *__restrict__ x,
                                                             const bf16_t *__restrict__ wg,
                                                             const bf16_t *__restrict__ gout,
                                                             bf16_t *__restrict__ gy, int H, int W) {
    using P = DyPlanB<K, SEG, NCP>;
    constexpr int r = P::r;
    constexpr int KK = P::KK;
    constexpr int NST = P::NST;
    constexpr int C = kChY;
    constexpr int kThreadsB = P::THREADS;
    constexpr int NB = P::NB;
    extern __shared__ __align__(16) unsigned char lds_b[];
    bf16_t *xs = (bf16_t *)(lds_b + P::XOFF);  // [8][XP][8]
    bf16_t *gs = (bf16_t *)(lds_b + P::GOFF);  // [8][GP][8]
    bf16_t *ws = (bf16_t *)(lds_b + P::WOFF);  // [K][64][WR]: columns cp0 .. cp0 + NCP - 1

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int i = lane & 15;
    constexpr int NSPL = 64 / NCP;
    const int nseg = (W + SEG - 1) / SEG;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int cp0 = (L % NSPL) * NCP;  // the workgroup's output channels (halves of a segment are neighbours)
    L /= NSPL;
    const int w0 = (L % nseg) * SEG;
    L /= nseg;
    const int h = L % H;
    const int n = L / H;
    const int HW = H * W;
    const bf16_t *__restrict__ xn = x + (int64_t)n * C * HW;
    const bf16_t *__restrict__ gn = gout + (int64_t)n * 4 * C * HW;

    // ---- staging: item q = 8 channels (plane q & 7) x 8 pixels (run q >> 3), loaded
    // as eight 16-byte channel runs and written as eight 16-byte pixel slots; runs
    // outside the image (W % 8 == 0: wholly in or out) are zero
    u32x4 xreg[P::XIT][8], greg[8], wreg[P::WIT];
    const int qg = tid - (kThreadsB - P::NGI);  // G item of this thread (the last SEG threads)
    auto x_row = [&](int st) { return h + ((st % K) - r) * (1 + 2 * (st / K)); };
    auto load_stage = [&](int st) {
        const int hs = x_row(st);
        if (hs >= 0 && hs < H) {  // workgroup-uniform: otherwise the stage is skipped
#pragma unroll
            for (int k = 0; k < P::XIT; ++k) {
                const int q = tid + kThreadsB * k;
                const int col = w0 - P::LP + 8 * (q >> 3);
                const bool ok = q < P::NXI && col >= 0 && col < W;
                const unsigned off = (unsigned)(8 * (q & 7) * HW + hs * W + (ok ? col : 0));
#pragma unroll
                for (int e = 0; e < 8; ++e) xreg[k][e] = *(const u32x4 *)(xn + (off + (unsigned)(e * HW)));
            }
            const int b = st / K, ki = st % K;
            const bf16_t *wb = wg + (int64_t)(b * C * KK + ki * K) * C;
#pragma unroll
            for (int k = 0; k < P::WIT; ++k) {
                const int q = tid + kThreadsB * k;  // slot: tap, row c, 8 columns
                const int tap = q / (64 * P::WSR);
                const int rem = q - tap * 64 * P::WSR;
                const int c = rem / P::WSR;
                wreg[k] = *(const u32x4 *)(wb + (c * KK + tap) * C + cp0 + 8 * (rem - c * P::WSR));
            }
        }
        if (st % K == 0 && qg >= 0) {  // a new branch: its G row
            const int col = w0 + 8 * (qg >> 3);
            const unsigned off = (unsigned)(((1 + st / K) * C + 8 * (qg & 7)) * HW + h * W + (col < W ? col : 0));
#pragma unroll
            for (int e = 0; e < 8; ++e) greg[e] = *(const u32x4 *)(gn + (off + (unsigned)(e * HW)));
        }
    };
    auto store_stage = [&](int st) {
        const int hs = x_row(st);
        if (hs >= 0 && hs < H) {
#pragma unroll
            for (int k = 0; k < P::XIT; ++k) {
                const int q = tid + kThreadsB * k;
                const int col = w0 - P::LP + 8 * (q >> 3);
                if (q < P::NXI) {
                    bf16_t *d = xs + ((q & 7) * P::XP + 8 * (q >> 3)) * 8;
                    if (col >= 0 && col < W) {
                        u32x4 o[8];
                        transpose8x8_bf16(xreg[k], o);
#pragma unroll
                        for (int p = 0; p < 8; ++p) *(u32x4 *)(d + 8 * p) = o[p];
                    } else {  // a run outside the image reads as zero
#pragma unroll
                        for (int p = 0; p < 8; ++p) *(u32x4 *)(d + 8 * p) = u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < P::WIT; ++k) {
                const int q = tid + kThreadsB * k;
                const int tap = q / (64 * P::WSR);
                const int rem = q - tap * 64 * P::WSR;
                const int c = rem / P::WSR;
                *(u32x4 *)(ws + (tap * 64 + c) * P::WR + 8 * (rem - c * P::WSR)) = wreg[k];
            }
        }
        if (st % K == 0 && qg >= 0) {
            bf16_t *d = gs + ((qg & 7) * P::GP + 8 * (qg >> 3)) * 8;
            if (w0 + 8 * (qg >> 3) < W) {
                u32x4 o[8];
                transpose8x8_bf16(greg, o);
#pragma unroll
                for (int p = 0; p < 8; ++p) *(u32x4 *)(d + 8 * p) = o[p];
            } else {
#pragma unroll
                for (int p = 0; p < 8; ++p) *(u32x4 *)(d + 8 * p) = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    constexpr int NPB = kPxB / 16;
    // lane's slots: channel plane 4ks + g, pixel kPxB*wave + 16pb + i (x: + LP + dc)
    const bf16_t *x_lane = xs + (g * P::XP + kPxB * wave + i + P::LP) * 8;
    const bf16_t *g_lane = gs + (g * P::GP + kPxB * wave + i) * 8;
    // weight rows 32ks + 8g + 4hh + (i >> 2), columns 16nb + 4(i & 3)
    const bf16_t *w_lane = ws + (8 * g + (i >> 2)) * P::WR + 4 * (i & 3);

    f32x4 acc[NPB][NB];  // [pb][nb]
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[pb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float gf[NPB][2][8];  // G_b of the lane's pixels: [pb][ks][e]

    load_stage(0);
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
        if (ki == 0) {
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const u32x4 v = *(const u32x4 *)(g_lane + (4 * ks * P::GP + 16 * pb) * 8);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        gf[pb][ks][2 * m] = __uint_as_float(v[m] << 16);
                        gf[pb][ks][2 * m + 1] = __uint_as_float(v[m] & 0xffff0000u);
                    }
                }
        }
        if (rok) {
#pragma clang loop unroll(full)
            for (int kj = 0; kj < K; ++kj) {
                const int dc = (kj - r) * D;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    bf16x8 a[NPB];
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb) {
                        const u32x4 v = *(const u32x4 *)(x_lane + (4 * ks * P::XP + 16 * pb + dc) * 8);
                        u16x8 u;
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            u[2 * m] = f32_to_bf16_bits(gf[pb][ks][2 * m] * __uint_as_float(v[m] << 16));
                            u[2 * m + 1] = f32_to_bf16_bits(gf[pb][ks][2 * m + 1] * __uint_as_float(v[m] & 0xffff0000u));
                        }
                        a[pb] = __builtin_bit_cast(bf16x8, u);
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const bf16_t *wp = w_lane + (kj * 64 + 32 * ks) * P::WR + 16 * nb;
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(wp));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(wp + 4 * P::WR));
                        const bf16x8 bq = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                        for (int pb = 0; pb < NPB; ++pb) acc[pb][nb] = mfma_16x16x32_bf16(a[pb], bq, acc[pb][nb]);
                    }
                }
            }
        }
    }

    // ---- rows 4g + v of block pb are pixels 16pb + 4g + v; columns are output
    // channels 16nb + i
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
        const int col = w0 + kPxB * wave + 16 * pb + 4 * g;
        if (col < W) {  // W % 8 == 0: runs of four are whole
            bf16_t *yo = gy + (int64_t)n * C * HW + h * W + col;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                u16x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = f32_to_bf16_bits(acc[pb][nb][v]);
                *(u16x4 *)(yo + (cp0 + 16 * nb + i) * HW) = o;
            }
        }
    }
}

}  // namespace

// Applicability: C = 64, 16-byte aligned tensors (checked by the caller), W % 4 == 0
// (float32) or W % 8 == 0 (bfloat16), and plane offsets within 32 bits.
bool bwd_dy_rows_applies(int C, int H, int W, bool al, bool bf16) {
    return C == kChY && al && (W % (bf16 ? 8 : 4)) == 0 && (int64_t)4 * kChY * H * W < (int64_t(1) << 31);
}

// bfloat16: 256-pixel segments x all 64 output channels when rows are wider than 128
// pixels and that grid gives every CU a segment; else 128-pixel segments x 32 output
// channels (the two halves of a segment in neighbouring workgroups) when that grid
// does; else 64-pixel segments x 16 output channels (two waves, the four quarters in
// neighbouring workgroups, each forming its segment's dK itself), which brings grids
// too small for the halves to the row-staged kernel (64 x 64 at K = 3: 49 -> 28 us
// against the general kernel) but loses to the halves where both apply (128 x 128:
// 35 -> 42 us).
enum DyVariant { kDyWide, kDyHalf, kDyQuarter };
static DyVariant dy_bf16_variant(int N, int H, int W) {
    if (W > 128 && (int64_t)N * H * ((W + 255) / 256) >= 256) return kDyWide;
    if ((int64_t)N * H * ((W + 127) / 128) * 2 >= 256) return kDyHalf;
    return kDyQuarter;
}

int64_t bwd_dy_rows_blocks(int N, int H, int W, bool bf16) {
    if (!bf16) return (int64_t)N * H * ((W + kSegY - 1) / kSegY);
    switch (dy_bf16_variant(N, H, W)) {
        case kDyWide: return (int64_t)N * H * ((W + 255) / 256);
        case kDyHalf: return (int64_t)N * H * ((W + 127) / 128) * 2;
        default: return (int64_t)N * H * ((W + 63) / 64) * 4;
    }
}

template <int K, int SEG, int NCP>
static hipError_t launch_dy_bf16(dim3 grid, const void *x, const void *wg, const void *gout, void *gy, int H, int W,
                                 hipStream_t stream) {
    using P = DyPlanB<K, SEG, NCP>;
    constexpr int lds = P::LDS;
    auto kern = bwd_dy_bf16_kernel<K, SEG, NCP>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(P::THREADS), lds, stream, (const bf16_t *)x, (const bf16_t *)wg,
                       (const bf16_t *)gout, (bf16_t *)gy, H, W);
    return hipGetLastError();
}

template <int K>
static hipError_t launch_dy_bf16_k(dim3 grid, DyVariant var, const void *x, const void *wg, const void *gout,
                                   void *gy, int H, int W, hipStream_t stream) {
    if (var == kDyWide) return launch_dy_bf16<K, 256, 64>(grid, x, wg, gout, gy, H, W, stream);
    if (var == kDyHalf) return launch_dy_bf16<K, 128, 32>(grid, x, wg, gout, gy, H, W, stream);
    return launch_dy_bf16<K, 64, 16>(grid, x, wg, gout, gy, H, W, stream);
}

hipError_t launch_bwd_dy_rows(const void *x, const void *wg, const void *gout, void *gy, int N, int H, int W, int K,
                              bool bf16, hipStream_t stream) {
    const int64_t nblk = bwd_dy_rows_blocks(N, H, W, bf16);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nblk), block(256);
    if (bf16) {
        const DyVariant var = dy_bf16_variant(N, H, W);
        switch (K) {
            case 1: return launch_dy_bf16_k<1>(grid, var, x, wg, gout, gy, H, W, stream);
            case 3: return launch_dy_bf16_k<3>(grid, var, x, wg, gout, gy, H, W, stream);
            default: return launch_dy_bf16_k<5>(grid, var, x, wg, gout, gy, H, W, stream);
        }
    }
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

// bwd_dx_rows.hip -- dX of the fused training backward for C = 64 (gfx950), in
// bfloat16 and float32: tap recompute + gather, staged by source row.
//
// Operation (page "lartpang/DynamicConvolutionOperator", section
// "CUDA Flash 式融合训练": the backward recomputes the dynamic taps and gathers
// each dilation's contribution):
//     dX[c, q] = G_x[c, q] + sum_{b,t} rne(T[o(b,c,t), q - d_bt]) * G_b[c, q - d_bt],
//     T[o, p]  = bias[o] + sum_c' W[o, c'] y[c', p]      (float32 sum, one rounding).
//
// Work decomposition: workgroup = one 64-pixel row segment (row h, columns w0..)
// x the 64 output channels, four waves, wave v owning channels 16v..16v+15.
// The generator block of tap (b, t) is an MFMA product with
//   rows    = 16 pixels (four blocks cover the segment),
//   columns = the wave's 16 output channels,
//   k       = the 64 input channels c' (two k-steps of 32),
// A = y at the source pixels q - d_bt, B = weight rows (16 contiguous bytes per
// lane).  Lane (g, i) receives the taps of channel 16v + i at four consecutive
// pixels 16pb + 4g .. +3 of each block pb, so G_b at the same source pixels is one
// 8-byte run per block and the products stay lane-local.
//
// Taps that read the same source row h - dr share one staging of y: the row's
// segment with a column halo, all 64 channels, in LDS as eight planes of 8
// channels ([c/8][pixel][c%8], 16 bytes per pixel), so any column shift is an
// immediate offset and the 16 lanes of a fragment read 256 contiguous bytes.
// bfloat16 stages are the 3K (branch, kernel row) pairs, y and G_b together,
// double-buffered with one barrier each and loaded two stages ahead with buffer
// loads (fixed per-thread offsets, the row as a scalar offset, zero outside the
// image); G_b is read back as aligned dwords, since 2-byte-aligned 8-byte LDS
// reads cost the kernel a sixth of its time.  A stage whose source row lies
// outside the image contributes nothing and is skipped.  Every tap is unrolled at
// compile time, so no index arithmetic runs per tap.  The sum over taps runs in
// stage order in float32 (bfloat16: pairs of taps through the two-term dot
// instruction), then G_x is added.
#include "common.hpp"
#include "launchers.hpp"

namespace ddpm {
namespace {

constexpr int kSegX = 64;  // pixels per workgroup (one row segment)
constexpr int kChX = 64;   // channels (input and output) this kernel serves

// Stages are the (branch b, kernel row ki) pairs: the K taps of a stage read one
// source row, h - dr with dr = (ki - r) * D_b, and one G block, G_b.
template <int K> struct DxPlan {
    static constexpr int r = (K - 1) / 2;
    static constexpr int KK = K * K;
    static constexpr int NT = 3 * KK;
    static constexpr int NST = 3 * K;                  // stages
    static constexpr int HALO = 5 * r;                 // largest column shift
    static constexpr int LP = (HALO + 3) & ~3;         // staged columns left of the segment
    static constexpr int SW = kSegX + 2 * LP;          // staged columns
    static constexpr int PLANE = SW * 16;              // bytes of one 8-channel plane of y
    static constexpr int YBUF = 8 * PLANE;             // bytes of one staged y row (64 channels)
    static constexpr int GROW = SW + 4;                // elements per staged G channel row
    static constexpr int GBUF = kChX * GROW * 2;       // bytes of one staged G row
};

// LDS image of one stage: y as eight planes of 8 channels ([c/8][pixel][c%8]) and
// G_b as channel rows ([c][pixel], padded by 4 columns against bank conflicts).
template <int K> struct DxStageBuf {
    unsigned char y[DxPlan<K>::YBUF];
    unsigned char g[DxPlan<K>::GBUF];
};

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Widen a run of four bf16 values (two dwords) to float.
__device__ __forceinline__ void widen4(const u16x4 u, float (&f)[4]) {
    const u32x2_t d = __builtin_bit_cast(u32x2_t, u);
    f[0] = __uint_as_float(d[0] << 16);
    f[1] = __uint_as_float(d[0] & 0xffff0000u);
    f[2] = __uint_as_float(d[1] << 16);
    f[3] = __uint_as_float(d[1] & 0xffff0000u);
}

// Two floats rounded to bfloat16 (nearest even) in one dword: lo, hi.
__device__ __forceinline__ bf16x2_t rne_pair(float lo, float hi) { return bf16x2_t{(__bf16)lo, (__bf16)hi}; }

// Buffer resource over `bytes` bytes at p (gfx9 word 3: raw 32-bit data).  A load
// whose offset lies past the end reads zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
constexpr unsigned kOob = 0x7ffffff0u;  // a buffer offset that always reads zero

template <int K>
__global__ __launch_bounds__(256, 2) void bwd_dx_bf16_kernel(const bf16_t *__restrict__ y,
                                                             const bf16_t *__restrict__ wg,
                                                             const bf16_t *__restrict__ bg,
                                                             const bf16_t *__restrict__ gout,
                                                             bf16_t *__restrict__ gx, int H, int W) {
    using P = DxPlan<K>;
    constexpr int r = P::r;
    constexpr int KK = P::KK;
    constexpr int NT = P::NT;
    constexpr int NST = P::NST;
    constexpr int C = kChX;
    __shared__ __align__(16) DxStageBuf<K> sb[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int i = lane & 15;
    const int nseg = (W + kSegX - 1) / kSegX;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int w0 = (L % nseg) * kSegX;
    L /= nseg;
    const int h = L % H;
    const int n = L / H;
    const int HW = H * W;
    const bf16_t *__restrict__ yn = y + (int64_t)n * C * HW;
    const bf16_t *__restrict__ gn = gout + (int64_t)n * 4 * C * HW;
    const int c = 16 * wave + i;  // the output channel of this lane's MFMA column

    // ---- staging through buffer loads: every per-thread offset is fixed, the
    // stage's row is a scalar offset, and a run outside the image reads zero (no
    // branches, no 64-bit address arithmetic).  y: thread tid covers blocks of 4
    // channels x 4 pixels (transposed into the planes); G_b: runs of 4 pixels of one
    // channel row (copied as they are).
    const __amdgpu_buffer_rsrc_t ry = buf_rsrc(yn, C * HW * 2);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gn, 4 * C * HW * 2);
    constexpr int NB4 = P::SW / 4;            // 4-pixel runs per staged row
    constexpr int NBLK = 16 * NB4;            // y blocks
    constexpr int YIT = (NBLK + 255) / 256;   // y blocks per thread
    constexpr int NRUN = kChX * NB4;          // G runs
    constexpr int GIT = (NRUN + 255) / 256;   // G runs per thread
    u32x2_t yreg[YIT][4];
    u32x2_t greg[GIT];
    unsigned yvo[YIT][4], gvo[GIT];  // byte offsets within the stage's row, or kOob
    int ydst[YIT], gdst[GIT];
    bool yex[YIT], gex[GIT];
#pragma unroll
    for (int k = 0; k < YIT; ++k) {
        const int q = tid + 256 * k;
        const int c4 = q / NB4;
        const int px4 = q - c4 * NB4;
        const int col = w0 - P::LP + 4 * px4;
        yex[k] = q < NBLK;
        const bool ok = yex[k] && col >= 0 && col < W;  // W % 4 == 0: a run is wholly in or out
#pragma unroll
        for (int e = 0; e < 4; ++e) yvo[k][e] = ok ? (unsigned)((4 * c4 + e) * HW + col) * 2u : kOob;
        ydst[k] = (c4 >> 1) * P::PLANE + 4 * px4 * 16 + (c4 & 1) * 8;
    }
#pragma unroll
    for (int k = 0; k < GIT; ++k) {
        const int q = tid + 256 * k;
        const int ch = q / NB4;
        const int px4 = q - ch * NB4;
        const int col = w0 - P::LP + 4 * px4;
        gex[k] = q < NRUN;
        const bool ok = gex[k] && col >= 0 && col < W;
        gvo[k] = ok ? (unsigned)(ch * HW + col) * 2u : kOob;
        gdst[k] = (ch * P::GROW + 4 * px4) * 2;
    }
    // global loads of stage st (branch b = st / K, kernel row ki = st % K) into registers
    auto load_stage = [&](int st) {
        const int b = st / K;
        const int ki = st - b * K;
        const int hs = h - (ki - r) * (1 + 2 * b);
        if (hs < 0 || hs >= H) return;  // wave-uniform: the stage is skipped
        const int yso = hs * W * 2;
        const int gso = ((1 + b) * C * HW + hs * W) * 2;
#pragma unroll
        for (int k = 0; k < YIT; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) yreg[k][e] = __builtin_amdgcn_raw_buffer_load_b64(ry, yvo[k][e], yso, 0);
#pragma unroll
        for (int k = 0; k < GIT; ++k) greg[k] = __builtin_amdgcn_raw_buffer_load_b64(rg, gvo[k], gso, 0);
    };
    auto store_stage = [&](int st, int buf) {
        const int b = st / K;
        const int ki = st - b * K;
        const int hs = h - (ki - r) * (1 + 2 * b);
        if (hs < 0 || hs >= H) return;
#pragma unroll
        for (int k = 0; k < YIT; ++k) {
            if (!yex[k]) continue;
            unsigned char *d = sb[buf].y + ydst[k];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                u16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(u16x4, yreg[k][e])[p];
                *(u16x4 *)(d + 16 * p) = o;
            }
        }
#pragma unroll
        for (int k = 0; k < GIT; ++k)
            if (gex[k]) *(u32x2_t *)(sb[buf].g + gdst[k]) = greg[k];
    };

    // ---- weight fragments of tap (b, t): row o = (b*C + c)*KK + t, columns 32 sub +
    // 8g .. +7, and the row's bias, by buffer loads whose tap part is a constant
    // offset.  A ring of four: the taps of the current pair and of the next.
    // One resource per branch: a tap's part of the offset, t*C*2 (+64) bytes, fits the
    // instructions' 12-bit immediate offset, so no scalar constant is set per load.
    const __amdgpu_buffer_rsrc_t rw0 = buf_rsrc(wg, C * KK * C * 2);
    const __amdgpu_buffer_rsrc_t rw1 = buf_rsrc(wg + C * KK * C, C * KK * C * 2);
    const __amdgpu_buffer_rsrc_t rw2 = buf_rsrc(wg + 2 * C * KK * C, C * KK * C * 2);
    const __amdgpu_buffer_rsrc_t rb0 = buf_rsrc(bg, C * KK * 2);
    const __amdgpu_buffer_rsrc_t rb1 = buf_rsrc(bg + C * KK, C * KK * 2);
    const __amdgpu_buffer_rsrc_t rb2 = buf_rsrc(bg + 2 * C * KK, C * KK * 2);
    const unsigned wvo = (unsigned)(c * KK * C + 8 * g) * 2u;
    const unsigned bvo = (unsigned)(c * KK) * 2u;
    struct WOps { bf16x8 b0, b1; uint16_t bias; };
    WOps wring[4];
    auto fetch_w = [&](int bt, WOps &o) {  // bt = b*KK + t (a constant once unrolled)
        const int b = bt / KK;
        const int t = bt - b * KK;
        const __amdgpu_buffer_rsrc_t rw = b == 0 ? rw0 : (b == 1 ? rw1 : rw2);
        const __amdgpu_buffer_rsrc_t rb = b == 0 ? rb0 : (b == 1 ? rb1 : rb2);
        o.b0 = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rw, wvo + t * C * 2, 0, 0));
        o.b1 = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rw, wvo + t * C * 2 + 64, 0, 0));
        o.bias = __builtin_amdgcn_raw_buffer_load_b16(rb, bvo + t * 2, 0, 0);
    };
    // A fragment (y): plane 4*sub + g, pixel 16pb + i + (LP - dc)
    const int a_lane = g * P::PLANE + i * 16;
    // G_b run: channel c, pixels 16pb + 4g + (LP - dc) .. +3 of the staged row
    const int g_lane = (c * P::GROW + 4 * g) * 2;

    float dacc[4][4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) dacc[pb][v] = 0.f;

    load_stage(0);
    store_stage(0, 0);
    fetch_w(0, wring[0]);
    if (NT > 1) fetch_w(1, wring[1]);
    if (NST > 1) load_stage(1);
    __syncthreads();

    // The K taps of a stage run as pairs (kj, kj + 1) and, for odd K, a last single
    // tap.  A pair's two rounded taps meet G_b at their two source pixels in one
    // two-term bf16 dot product with float32 accumulation (v_dot2_f32_bf16), which
    // sums the pair's two exact products into the running sum.  An item (a pair or
    // single, one pixel block) is applied after the next item's MFMAs of the same
    // stage, so its MFMA results are not waited for right away; a stage's last item
    // is applied at the stage's end.  pacc / pg: the pending item, pend: whether
    // there is one.
    constexpr int NPAIR = K / 2;
    constexpr int NGRP = (K + 1) / 2;
    f32x4 pacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // G_b runs are read from LDS as aligned dwords: the run of a tap whose column
    // shift is odd starts in the high half of its first dword and spans three.  A
    // group's first tap (and a single tap) has shift parity r & 1, its second the
    // other, whatever the branch, so the position of each value is a constant.
    constexpr int PAR0 = r & 1;
    uint32_t pg[2][3] = {{0u, 0u, 0u}, {0u, 0u, 0u}};
    bool pend = false;
    auto retire = [&](bool pair, int ppb) {
        if (pair) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bf16x2_t q = rne_pair(pacc[0][v], pacc[1][v]);
                // lo half: value v of the first tap's run, hi half: of the second's
                const int p0 = PAR0 + v, p1 = 1 - PAR0 + v;
                const uint32_t sel = (p0 & 1 ? 0x0302u : 0x0100u) | (p1 & 1 ? 0x07060000u : 0x05040000u);
                const uint32_t gw = __builtin_amdgcn_perm(pg[1][p1 >> 1], pg[0][p0 >> 1], sel);
                dacc[ppb][v] = __builtin_amdgcn_fdot2_f32_bf16(q, __builtin_bit_cast(bf16x2_t, gw), dacc[ppb][v], false);
            }
        } else {
            // a single tap: the same dot instruction with a zero second term (the
            // rounded tap and its G_b value in the low halves, exact zeros above)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bf16x2_t q = rne_pair(pacc[0][v], 0.f);
                const int p0 = PAR0 + v;
                const uint32_t gw = p0 & 1 ? pg[0][p0 >> 1] >> 16 : pg[0][p0 >> 1] & 0xffffu;
                dacc[ppb][v] = __builtin_amdgcn_fdot2_f32_bf16(q, __builtin_bit_cast(bf16x2_t, gw), dacc[ppb][v], false);
            }
        }
    };

    // LDS operands of one item (group gi, pixel block pb): per tap, the two A
    // fragments and the G_b run.
    struct Ops {
        bf16x8 a0[2], a1[2];
        uint32_t g[2][3];
    };
    int fetched = NT > 1 ? 2 : 1;  // taps whose weights are requested (compile-time after unrolling)
    // request the weights up to two taps past group gi of stage st (ring slot = tap
    // % 4; the slot's previous tap belongs to an earlier group)
    auto fetch_upto = [&](int st, int gi) {
        const int bt0 = st * K + 2 * gi;
        const int nt = gi < NPAIR ? 2 : 1;
        for (; fetched < NT && fetched < bt0 + nt + 2; ++fetched) fetch_w(fetched, wring[fetched & 3]);
    };
#pragma clang loop unroll(full)
    for (int st = 0; st < NST; ++st) {
        const int b = st / K;
        const int ki = st - b * K;
        const int D = 1 + 2 * b;
        const int hs = h - (ki - r) * D;
        const bool rok = hs >= 0 && hs < H;  // wave-uniform: taps reading outside the image add nothing
        const unsigned char *ybuf = sb[st & 1].y + a_lane;
        const unsigned char *gbuf = sb[st & 1].g + g_lane;
        auto load_ops = [&](int gi, int pb, Ops &o) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u >= (gi < NPAIR ? 2 : 1)) continue;
                const int dc = (2 * gi + u - r) * D;
                const unsigned char *ab = ybuf + (P::LP - dc) * 16 + pb * 256;
                o.a0[u] = __builtin_bit_cast(bf16x8, *(const u16x8 *)ab);
                o.a1[u] = __builtin_bit_cast(bf16x8, *(const u16x8 *)(ab + 4 * P::PLANE));
                const int par = u == 0 ? PAR0 : 1 - PAR0;  // == (LP - dc) & 1
                const uint32_t *gw = (const uint32_t *)(gbuf + (P::LP - dc - par) * 2 + pb * 32);
#pragma unroll
                for (int m = 0; m < 3; ++m) o.g[u][m] = m < 2 + par ? gw[m] : 0u;
            }
        };
        if (rok) {
            constexpr int NIT = 4 * NGRP;  // items of the stage: (group, pixel block)
            f32x4 bias4[2];
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int gi = it / 4;
                const int pb = it % 4;
                const bool pair = gi < NPAIR;
                const int nt = pair ? 2 : 1;
                const int bt0 = st * K + 2 * gi;  // first tap of the group; taps run in (b, t) order
                if (pb == 0) {
                    fetch_upto(st, gi);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const float bias = bf16_bits_to_f32(wring[(bt0 + u) & 3].bias);
                        if (u < nt) bias4[u] = f32x4{bias, bias, bias, bias};
                    }
                }
                Ops o;
                load_ops(gi, pb, o);
                f32x4 acc[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (u >= nt) continue;
                    const WOps &cur = wring[(bt0 + u) & 3];
                    acc[u] = mfma_16x16x32_bf16(o.a0[u], cur.b0, bias4[u]);
                    acc[u] = mfma_16x16x32_bf16(o.a1[u], cur.b1, acc[u]);
                }
                // the pending item: the previous one of this stage
                if (pend) {
                    if (pb > 0) retire(pair, pb - 1);
                    else retire(gi - 1 < NPAIR, 3);
                }
                pacc[0] = acc[0];
#pragma unroll
                for (int m = 0; m < 3; ++m) pg[0][m] = o.g[0][m];
                if (pair) {
                    pacc[1] = acc[1];
#pragma unroll
                    for (int m = 0; m < 3; ++m) pg[1][m] = o.g[1][m];
                }
                pend = true;
                __builtin_amdgcn_sched_barrier(0);
            }
            // The stage's last item is applied before the stage ends, so that no
            // pending value is live across the branch that skips a stage (the two
            // paths would otherwise merge it through register copies).
            retire(NGRP - 1 < NPAIR, 3);
            pend = false;
        } else {
#pragma unroll
            for (int gi = 0; gi < NGRP; ++gi) fetch_upto(st, gi);
        }
        if (st + 1 < NST) {
            store_stage(st + 1, (st + 1) & 1);
            __syncthreads();
            if (st + 2 < NST) load_stage(st + 2);
        }
    }


    // dX = G_x + the gathered sum, rounded once
    const bf16_t *gxr = gn + c * HW + h * W + w0 + 4 * g;
    bf16_t *dst = gx + (int64_t)n * C * HW + c * HW + h * W + w0 + 4 * g;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
        if (w0 + 16 * pb + 4 * g >= W) continue;  // W % 4 == 0: runs are whole
        float gf[4];
        widen4(*(const u16x4 *)(gxr + 16 * pb), gf);
        u16x4 o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = f32_to_bf16_bits(dacc[pb][v] + gf[v]);
        *(u16x4 *)(dst + 16 * pb) = o;
    }
}

// ---------------------------------------------------------------------------- float32
// The same decomposition in float32 with v_mfma_f32_16x16x4_f32: MFMA rows = 16
// pixels (blocks pb = 0..3 cover the segment), columns = the wave's 16 output
// channels, and k-step s (0..15) takes input channel 16g + s from lane group g, so
// a lane's A values for one pixel block are 16 contiguous channels of one pixel
// (four 16-byte LDS reads) and its B values 16 contiguous weights of one row (four
// 16-byte loads).  A tap is 64 MFMAs per wave.  Per (branch, kernel row) stage, y
// is staged as [pixel][64 channels + 4 pad] (272-byte pixel rows: the 16 pixels of
// a fragment start in distinct 4-dword bank groups) in one of two LDS images: the
// next stage's row is loaded at the start of a stage and written into the other
// image after the stage's first tap, so one barrier per stage suffices.  G_b is
// staged as channel rows of GROW floats (the 16 channels of a read start in
// distinct 4-dword bank groups); each wave reads only its own 16 channel rows, so
// it stages them itself, at the end of a stage, with no barrier.  G_b runs start at
// a column shift that is a compile-time constant per tap; shifts that are not a
// multiple of four are read as two aligned 16-byte words.  The weight rows come
// from global memory one tap ahead.
template <int K> struct DxPlanF {
    static constexpr int r = (K - 1) / 2;
    static constexpr int KK = K * K;
    static constexpr int NT = 3 * KK;
    static constexpr int NST = 3 * K;
    static constexpr int HALO = 5 * r;
    static constexpr int LP = (HALO + 3) & ~3;
    static constexpr int SW = kSegX + 2 * LP;
    static constexpr int PROW = kChX + 4;         // floats per staged y pixel
    static constexpr int YBUF = SW * PROW;        // floats of one staged y row
    static constexpr int GROW = ((SW + 12) / 16) * 16 + 4;  // floats per staged G channel row (== 4 mod 16)
    static constexpr int GBUF = kChX * GROW;      // floats of the staged G rows (16 per wave)
    static constexpr int BYTES = 4 * (2 * YBUF + GBUF);
    // Stage order: the 3(K-1) (branch, kernel row) pairs with a row shift first
    // (branch-major), then the three unshifted kernel rows (ki = r) of branches
    // 0, 1, 2, which read the same y row and stage it once.
    static constexpr int NSHIFT = 3 * (K - 1);
    static constexpr int KM = K > 1 ? K - 1 : 1;  // shifted kernel rows per branch (K = 1: none)
    static constexpr int stage_b(int s) { return s < NSHIFT ? s / KM : s - NSHIFT; }
    static constexpr int stage_ki(int s) { return s < NSHIFT ? (s % KM < r ? s % KM : s % KM + 1) : r; }
    static constexpr bool new_y(int s) { return s <= NSHIFT; }  // stage s stages its own y row
    static constexpr int y_image(int s) { return (s < NSHIFT ? s : NSHIFT) & 1; }
};

// Barrier for the staged y rows: this wave's LDS operations complete, then every
// wave of the workgroup arrives.  Outstanding global loads (the next stage's rows,
// the next tap's weights) stay in flight; their registers are waited for where used.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int K>
__global__ __launch_bounds__(256, 2) void bwd_dx_f32_kernel(const float *__restrict__ y,
                                                            const float *__restrict__ wg,
                                                            const float *__restrict__ bg,
                                                            const float *__restrict__ gout,
                                                            float *__restrict__ gx, int H, int W) {
    using P = DxPlanF<K>;
    constexpr int r = P::r;
    constexpr int KK = P::KK;
    constexpr int NT = P::NT;
    constexpr int NST = P::NST;
    constexpr int C = kChX;
    extern __shared__ __align__(16) float dsm[];
    float *const ys = dsm;                  // two y images of YBUF floats
    float *const gs = dsm + 2 * P::YBUF;    // G_b channel rows

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int i = lane & 15;
    const int nseg = (W + kSegX - 1) / kSegX;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int w0 = (L % nseg) * kSegX;
    L /= nseg;
    const int h = L % H;
    const int n = L / H;
    const int HW = H * W;
    const float *__restrict__ yn = y + (int64_t)n * C * HW;
    const float *__restrict__ gn = gout + (int64_t)n * 4 * C * HW;
    const int c = 16 * wave + i;  // the output channel of this lane's MFMA column

    // ---- staging.  y: thread tid covers blocks of 4 channels x 4 pixels, transposed
    // in registers into four pixel entries of 4 channels; G_b: runs of 4 pixels of
    // one of the wave's channel rows, copied as they are.  Runs outside the image
    // (W % 4 == 0: wholly in or out) load the row's first run and are zeroed.
    constexpr int NB4 = P::SW / 4;
    constexpr int YIT = (NB4 + 15) / 16;   // y blocks per thread (16 runs of 4 pixels per iteration)
    constexpr int NRUN = 16 * NB4;         // G_b runs of one wave
    constexpr int GIT = (NRUN + 63) / 64;
    f32x4 yreg[YIT][4];
    f32x4 greg[GIT];
    unsigned yoff[YIT], goff[GIT];
    int ydst[YIT], gdst[GIT];
    bool yok[YIT], yex[YIT], gok[GIT], gex[GIT];
    // y block of thread tid, iteration k: channel quad c4 = (tid / 4) % 16, 4-pixel
    // run px4 = 4 * (tid / 64 + 4k) + tid % 4.  Four lanes read 64 contiguous bytes
    // of one channel row, and the 16 lanes of a quarter wave write pixel entries
    // whose 16-byte pieces fall in distinct bank groups (pixel rows are 68 floats).
#pragma unroll
    for (int k = 0; k < YIT; ++k) {
        const int c4 = (tid >> 2) & 15;
        const int px4 = 4 * ((tid >> 6) + 4 * k) + (tid & 3);
        const int col = w0 - P::LP + 4 * px4;
        yex[k] = px4 < NB4;
        yok[k] = yex[k] && col >= 0 && col < W;
        yoff[k] = (unsigned)(4 * c4 * HW + (yok[k] ? col : 0));
        ydst[k] = 4 * px4 * P::PROW + 4 * c4;
    }
#pragma unroll
    for (int k = 0; k < GIT; ++k) {
        const int q = lane + 64 * k;
        const int ch = q / NB4;
        const int px4 = q - ch * NB4;
        const int col = w0 - P::LP + 4 * px4;
        gex[k] = q < NRUN;
        gok[k] = gex[k] && col >= 0 && col < W;
        goff[k] = (unsigned)((16 * wave + (gex[k] ? ch : 0)) * HW + (gok[k] ? col : 0));
        gdst[k] = (16 * wave + ch) * P::GROW + 4 * px4;
    }
    auto stage_row = [&](int st) {  // the stage's source row (may lie outside the image)
        return h - (P::stage_ki(st) - r) * (1 + 2 * P::stage_b(st));
    };
    // Loads of stage st, unconditional: a row outside the image loads the nearest
    // image row instead, whose staged copy no tap reads (its taps are skipped), so
    // no branch holds the loaded registers and nothing waits for them before they
    // are stored.  y goes first, so that waiting for it leaves the G_b loads in flight.
    auto load_stage = [&](int st) {
        const int hr = stage_row(st);
        const int hs = hr < 0 ? 0 : (hr >= H ? H - 1 : hr);
        if (P::new_y(st)) {
            const float *ybase = yn + hs * W;
#pragma unroll
            for (int k = 0; k < YIT; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) yreg[k][e] = *(const f32x4 *)(ybase + (yoff[k] + (unsigned)(e * HW)));
        }
        const float *gbase = gn + (1 + P::stage_b(st)) * C * HW + hs * W;
#pragma unroll
        for (int k = 0; k < GIT; ++k) greg[k] = *(const f32x4 *)(gbase + goff[k]);
    };
    // Runs outside the image (columns) are written as zeros.
    auto store_y = [&](int st) {
        if (!P::new_y(st)) return;
        float *img = ys + P::y_image(st) * P::YBUF;
#pragma unroll
        for (int k = 0; k < YIT; ++k) {
            if (!yex[k]) continue;
            float *d = img + ydst[k];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f32x4 v = {yreg[k][0][p], yreg[k][1][p], yreg[k][2][p], yreg[k][3][p]};
                *(f32x4 *)(d + p * P::PROW) = yok[k] ? v : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto store_g = [&]() {
#pragma unroll
        for (int k = 0; k < GIT; ++k)
            if (gex[k]) *(f32x4 *)(gs + gdst[k]) = gok[k] ? greg[k] : f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // ---- weight rows from global memory, one tap ahead: tap (b, t) for channel c,
    // columns 16g .. 16g+15, and its bias
    const float *__restrict__ wl = wg + c * KK * C + 16 * g;
    const float *__restrict__ bgl = bg + c * KK;
    struct WOps {
        f32x4 w[4];
        float bias;
    };
    auto fetch = [&](int bt, WOps &o) {  // bt = b*KK + t
        const int b = bt / KK;
        const int t = bt - b * KK;
        const float *wt = wl + (b * C * KK + t) * C;
#pragma unroll
        for (int q = 0; q < 4; ++q) o.w[q] = *(const f32x4 *)(wt + 4 * q);
        o.bias = bgl[b * C * KK + t];
    };

    float dacc[4][4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int v = 0; v < 4; ++v) dacc[pb][v] = 0.f;

    // Tap ti of the stage order (stage ti / K, kernel column ti % K) as b*KK + t.
    auto tap_bt = [&](int ti) {
        const int sn = ti / K;
        return P::stage_b(sn) * KK + P::stage_ki(sn) * K + ti % K;
    };
    // Operands of tap ti in ring[ti % 3], fetched two taps ahead: a stage's loads
    // are issued at its start, after the weights of its first two taps, so those
    // two taps never wait for them (load counters retire in order).
    WOps ring[3];
    load_stage(0);
    store_y(0);
    store_g();
    fetch(tap_bt(0), ring[0]);
    if (NT > 1) fetch(tap_bt(1), ring[1]);
    // A fragment: pixel 16pb + i + (LP - dc), channels 16g .. 16g + 15
    const int a_lane = i * P::PROW + 16 * g;
    // G_b run: channel c, pixels 16pb + 4g + (LP - dc) .. +3
    const int g_lane = c * P::GROW + 4 * g;
#pragma clang loop unroll(full)
    for (int st = 0; st < NST; ++st) {
        const int b = P::stage_b(st);
        const int ki = P::stage_ki(st);
        const int D = 1 + 2 * b;
        const int hs = h - (ki - r) * D;
        const bool rok = hs >= 0 && hs < H;  // wave-uniform: taps reading outside the image add nothing
        lds_barrier();  // y of this stage written; every wave done reading the image it replaces
        if (st + 1 < NST) load_stage(st + 1);
        const float *yimg = ys + P::y_image(st) * P::YBUF;
#pragma clang loop unroll(full)
        for (int kj = 0; kj < K; ++kj) {
            const int ti = st * K + kj;  // position in the tap order
            const WOps &cur = ring[ti % 3];
            if (ti + 2 < NT) fetch(tap_bt(ti + 2), ring[(ti + 2) % 3]);
            if (rok) {
                const int dc = (kj - r) * D;
                const float *ab = yimg + a_lane + (P::LP - dc) * P::PROW;
                const int go = P::LP - dc;     // a constant once the loops are unrolled
                const int gm = go & 3;         // misalignment of the G_b run in floats
                const float *gb = gs + g_lane + (go - gm);
                // the A reads of block pb + 1 are issued before block pb's MFMAs
                f32x4 a[2][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) a[0][q] = *(const f32x4 *)(ab + 4 * q);
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    if (pb + 1 < 4) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            a[(pb + 1) & 1][q] = *(const f32x4 *)(ab + (pb + 1) * 16 * P::PROW + 4 * q);
                    }
                    const f32x4 g0 = *(const f32x4 *)(gb + 16 * pb);
                    f32x4 gv = g0;
                    if (gm != 0) {
                        const f32x4 g1 = *(const f32x4 *)(gb + 16 * pb + 4);
                        if (gm == 1) gv = f32x4{g0[1], g0[2], g0[3], g1[0]};
                        else if (gm == 2) gv = f32x4{g0[2], g0[3], g1[0], g1[1]};
                        else gv = f32x4{g0[3], g1[0], g1[1], g1[2]};
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    f32x4 acc = {cur.bias, cur.bias, cur.bias, cur.bias};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc = mfma_16x16x4_f32(a[pb & 1][q][e], cur.w[q][e], acc);
#pragma unroll
                    for (int v = 0; v < 4; ++v) dacc[pb][v] += acc[v] * gv[v];
                }
            }
            // the next stage's y row goes into the other image once its loads have had two
            // taps' time (K = 1: one)
            if (kj == (K > 1 ? 1 : 0) && st + 1 < NST) store_y(st + 1);
        }
        if (st + 1 < NST) {
            // this wave's G_b rows: its reads of this stage are issued (LDS executes a
            // wave's operations in order); keep the compiler from moving them across
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            store_g();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    }

    // dX = G_x + the gathered sum
    const float *gxr = gn + c * HW + h * W + w0 + 4 * g;
    float *dst = gx + (int64_t)n * C * HW + c * HW + h * W + w0 + 4 * g;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
        if (w0 + 16 * pb + 4 * g >= W) continue;  // W % 4 == 0: runs are whole
        const f32x4 gxv = *(const f32x4 *)(gxr + 16 * pb);
        f32x4 o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = dacc[pb][v] + gxv[v];
        *(f32x4 *)(dst + 16 * pb) = o;
    }
}

}  // namespace

// Applicability: C = 64, W % 4 == 0, 16-byte aligned tensors (checked by the
// caller) and the 4C gradient planes of an image within 32-bit offsets (float32:
// element offsets; bfloat16: the buffer loads' byte offsets).
bool bwd_dx_rows_applies(int C, int H, int W, bool al, bool bf16) {
    return C == kChX && al && (W % 4) == 0 && (int64_t)4 * kChX * H * W * (bf16 ? 2 : 1) < (int64_t(1) << 31);
}

namespace {
template <int K>
hipError_t launch_dx_f32(dim3 grid, hipStream_t stream, const float *y, const float *wg, const float *bg,
                         const float *gout, float *gx, int H, int W) {
    constexpr int bytes = DxPlanF<K>::BYTES;
    if (bytes > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void *)bwd_dx_f32_kernel<K>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bwd_dx_f32_kernel<K>, grid, dim3(256), bytes, stream, y, wg, bg, gout, gx, H, W);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_bwd_dx_rows(const void *y, const void *wg, const void *bg, const void *gout, void *gx, int N,
                              int H, int W, int K, bool bf16, hipStream_t stream) {
    const int64_t nblk = (int64_t)N * H * ((W + kSegX - 1) / kSegX);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nblk), block(256);
    if (!bf16) {
        const float *Y = (const float *)y, *Wg = (const float *)wg, *Bg = (const float *)bg, *G = (const float *)gout;
        float *GX = (float *)gx;
        switch (K) {
            case 1: return launch_dx_f32<1>(grid, stream, Y, Wg, Bg, G, GX, H, W);
            case 3: return launch_dx_f32<3>(grid, stream, Y, Wg, Bg, G, GX, H, W);
            default: return launch_dx_f32<5>(grid, stream, Y, Wg, Bg, G, GX, H, W);
        }
    }
    const bf16_t *Y = (const bf16_t *)y, *Wg = (const bf16_t *)wg, *Bg = (const bf16_t *)bg,
                 *G = (const bf16_t *)gout;
    bf16_t *GX = (bf16_t *)gx;
    switch (K) {
        case 1: hipLaunchKernelGGL(bwd_dx_bf16_kernel<1>, grid, block, 0, stream, Y, Wg, Bg, G, GX, H, W); break;
        case 3: hipLaunchKernelGGL(bwd_dx_bf16_kernel<3>, grid, block, 0, stream, Y, Wg, Bg, G, GX, H, W); break;
        default: hipLaunchKernelGGL(bwd_dx_bf16_kernel<5>, grid, block, 0, stream, Y, Wg, Bg, G, GX, H, W); break;
    }
    return hipGetLastError();
}

}  // namespace ddpm

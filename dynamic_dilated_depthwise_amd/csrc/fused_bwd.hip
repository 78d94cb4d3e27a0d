// fused_bwd.hip -- training backward of the fused DDPM with tap recompute (gfx950).
//
// Operation (page "lartpang/DynamicConvolutionOperator", section
// "CUDA Flash 式融合训练"): no tap tensor is saved; the backward
//   * dX: recomputes the dynamic taps and gathers each dilation's contribution,
//       dX[c,q] = G_x[c,q] + sum_{b,t} T[o, q-d_bt] * G_b[c, q-d_bt];
//   * dY: forms dK = shifted(x) * grad on chip and contracts it with the
//       generator weight at once, dY[c',p] = sum_o W[o,c'] * dK[o,p];
//   * dWeight / dbias: forms dK on chip and reduces it over space into at most 16
//       float32 partials over contiguous token ranges (the second short kernel,
//       reduce.hip, sums them).
// Every output element is stored once; nothing is accumulated through atomics, so
// results are bit-identical from run to run.
#include "gen_mma.hpp"
#include "launchers.hpp"

namespace ddpm {

constexpr int kCUs = 256;  // compute units of the chip (MI355X)
constexpr int kCols = 64;  // 16 lanes x 4 pixels

// ============================================================================ dY
// dY = W^T dK as an MFMA product: rows = output channels c' (16 per block, MB
// blocks), columns = one 64-pixel row segment (4 pixels per lane), contraction
// over the generator rows o = (b, c, t).  The B operand dK[o, p] = G_b[c, p] *
// x[c, p + d_bt] is formed in registers from G and the shifted x and never stored.
//   float32: one k-step = 4 generator rows (b, 4cq + g, t), lane group g;
//   bfloat16: one k-step = 32 generator rows (b, 32cq + 8g + e, t); dK is rounded
//   to bfloat16 as the MFMA operand.
// The contraction items (channel chunk cq, branch b, tap t) are split into NW
// contiguous ranges, one per wave, and the NW partial products are summed in a
// fixed order through LDS, so one workgroup per row segment still fills the chip.
// NW = 4 normally; NW = 8 when the grid is small (at most two workgroups per CU),
// which doubles the waves each SIMD has to hide latency with.
template <typename T, int K, int MB, int NW>
__global__ __launch_bounds__(64 * NW, NW == 16 ? 4 : (NW == 4 ? 2 : 1)) void bwd_dy_kernel(const T *__restrict__ x,
                                                                         const T *__restrict__ wg,
                                                                         const T *__restrict__ gout,
                                                                         T *__restrict__ gy, int C, int H, int W,
                                                                         int al) {
    constexpr int r = (K - 1) / 2;
    constexpr int KK = K * K;
    constexpr bool BF = Elem<T>::is_bf16;
    constexpr int CK = BF ? 32 : 4;  // generator channels per k-step
    __shared__ f32x4 red[NW - 1][4][64];  // one 16-channel block of the cross-wave sum at a time

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int g = lane >> 4;
    const int j = lane & 15;
    const int nMG = (C + 63) >> 6;
    const int ncolt = (W + kCols - 1) / kCols;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int cm0 = (L % nMG) * 64;
    L /= nMG;
    const int w = (L % ncolt) * kCols + 4 * j;
    L /= ncolt;
    const int h = L % H;
    const int n = L / H;
    const int64_t HW = (int64_t)H * W;
    const bool aligned4 = al != 0;
    const T *__restrict__ xn = x + (int64_t)n * C * HW;
    const T *__restrict__ gn = gout + (int64_t)n * 4 * C * HW;
    const int64_t rowoff = (int64_t)h * W;

    f32x4 acc[MB][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[m][pb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int w0 = w - 4 * j;  // row segment's first column (wave-uniform)
    // Wave-uniform: every generator channel chunk, output channel and column exists.
    const bool full = (C % CK == 0) && (cm0 + 16 * MB <= C) && (w0 + kCols <= W);
    const int ncq = (C + CK - 1) / CK;
    const int nitems = ncq * 3 * KK;  // (cq, b, t), t fastest
    const int i0 = (int)((int64_t)nitems * wave / NW);
    const int i1 = (int)((int64_t)nitems * (wave + 1) / NW);

    if constexpr (!BF) {
        // The wave's items are walked by (channel chunk, branch) pair, then tap: G_b at
        // the output row is loaded once per pair and the pair's indices and base
        // pointers are formed once.  Items keep their order, so the sums do too.
        const int p0 = i0 / KK;
        const int p1 = (i1 + KK - 1) / KK;
#pragma unroll 1
        for (int p = p0; p < p1; ++p) {
            const int b = p % 3;
            const int c = CK * (p / 3) + g;
            const bool c_ok = c < C;
            const int cs = c_ok ? c : 0;
            const int D = dilation(b);
            const int tlo = i0 - p * KK;  // the pair's taps in [tlo, thi) belong to this wave
            const int thi = i1 - p * KK;
            const f32x4 gb = full ? load4_unchecked(gn + (int64_t)((1 + b) * C + c) * HW + rowoff, w, aligned4, true,
                                                    false)
                                  : load4_row(gn + (int64_t)((1 + b) * C + cs) * HW + rowoff, w, W, c_ok, aligned4);
            const T *__restrict__ xc = xn + (int64_t)cs * HW;
            const T *__restrict__ wb = wg + (int64_t)(b * C + cs) * KK * C;
            const int ta = max(tlo, 0), tb = min(thi, KK);
#pragma unroll 1
            for (int t = ta; t < tb; ++t) {
                const int ki = t / K;
                const int kj = t - ki * K;
                const int hh = h + (ki - r) * D;
                const int dc = (kj - r) * D;
                f32x4 xs;
                float a[MB];
                if (full && hh >= 0 && hh < H && w0 + dc - (dc & 1) >= 0 && w0 + kCols - 1 + dc < W) {  // wave-uniform
                    xs = load4_unchecked(xc + (int64_t)hh * W, w + dc, aligned4 && ((dc & 3) == 0), true, false);
#pragma unroll
                    for (int m = 0; m < MB; ++m) a[m] = wb[t * C + cm0 + j + 16 * m];
                } else {
                    const bool rok = c_ok && hh >= 0 && hh < H;
                    xs = load4_row(xc + (int64_t)(rok ? hh : 0) * W, w + dc, W, rok, aligned4 && ((dc & 3) == 0));
#pragma unroll
                    for (int m = 0; m < MB; ++m) {
                        const int cp = cm0 + 16 * m + j;
                        a[m] = (c_ok && cp < C) ? wb[t * C + cp] : 0.f;
                    }
                }
                // raised issue priority while this wave's MFMAs go out, so that waves doing
                // their address arithmetic do not hold the matrix pipe idle
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) acc[m][pb] = mfma_16x16x4_f32(a[m], gb[pb] * xs[pb], acc[m][pb]);
                __builtin_amdgcn_s_setprio(0);
            }
        }
    } else {
        // as for float32: by (channel chunk, branch) pair, then tap
        const int p0 = i0 / KK;
        const int p1 = (i1 + KK - 1) / KK;
#pragma unroll 1
        for (int p = p0; p < p1; ++p) {
            const int b = p % 3;
            const int cq = p / 3;
            const int D = dilation(b);
            f32x4 gb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = CK * cq + 8 * g + e;
                if (full)
                    gb[e] = load4_unchecked(gn + (int64_t)((1 + b) * C + c) * HW + rowoff, w, aligned4, aligned4,
                                            false);
                else
                    gb[e] = load4_row(gn + (int64_t)((1 + b) * C + (c < C ? c : 0)) * HW + rowoff, w, W, c < C,
                                      aligned4);
            }
            const int ta = max(i0 - p * KK, 0), tb = min(i1 - p * KK, KK);
#pragma unroll 1
            for (int t = ta; t < tb; ++t) {
                const int ki = t / K;
                const int kj = t - ki * K;
                const int hh = h + (ki - r) * D;
                const int dc = (kj - r) * D;
                const bool hok = hh >= 0 && hh < H;
                uint16_t bv[4][8];
                uint16_t av[MB][8];
                if (full && hok && w0 + dc - (dc & 1) >= 0 && w0 + kCols - 1 + dc < W) {  // wave-uniform
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int c = CK * cq + 8 * g + e;
                        const f32x4 xs = load4_unchecked(xn + (int64_t)c * HW + (int64_t)hh * W, w + dc,
                                                         aligned4 && ((dc & 3) == 0), aligned4, (dc & 1) != 0);
#pragma unroll
                        for (int pb = 0; pb < 4; ++pb) bv[pb][e] = f32_to_bf16_bits(gb[e][pb] * xs[pb]);
                        const T *wrow = wg + ((int64_t)(b * C + c) * KK + t) * C + cm0 + j;
#pragma unroll
                        for (int m = 0; m < MB; ++m) av[m][e] = wrow[16 * m];
                    }
                } else
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = CK * cq + 8 * g + e;
                    const bool c_ok = c < C;
                    const f32x4 xs = load4_row(xn + (int64_t)(c_ok ? c : 0) * HW + (int64_t)(hok ? hh : 0) * W,
                                               w + dc, W, c_ok && hok, aligned4 && ((dc & 3) == 0));
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) bv[pb][e] = f32_to_bf16_bits(gb[e][pb] * xs[pb]);
                    const T *wrow = wg + ((int64_t)(b * C + (c_ok ? c : 0)) * KK + t) * C;
#pragma unroll
                    for (int m = 0; m < MB; ++m) {
                        const int cp = cm0 + 16 * m + j;
                        av[m][e] = (c_ok && cp < C) ? wrow[cp] : (uint16_t)0;
                    }
                }
                bf16x8 bq[4];
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) bq[pb] = pack_bf16x8(bv[pb]);
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const bf16x8 aq = pack_bf16x8(av[m]);
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) acc[m][pb] = mfma_16x16x32_bf16(aq, bq[pb], acc[m][pb]);
                }
            }
        }
    }

    // Fixed-order sum of the waves' partial products, ((w0 + w1) + w2) + ..., one
    // 16-channel block at a time through LDS.
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        if (wave > 0) {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) red[wave - 1][pb][lane] = acc[m][pb];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int k = 0; k < NW - 1; ++k)
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) acc[m][pb] += red[k][pb][lane];
        }
        __syncthreads();
    }
    if (wave != 0) return;

    T *__restrict__ yo = gy + (int64_t)n * C * HW;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int cp = cm0 + 16 * m + 4 * g + v;
            if (cp >= C) continue;
            store4_row(yo + (int64_t)cp * HW + rowoff, w, W,
                       f32x4{acc[m][0][v], acc[m][1][v], acc[m][2][v], acc[m][3][v]}, aligned4);
        }
    }
}

// ============================================================================ dW / db
// One workgroup = CG generator (branch, tap) pairs x 16 depthwise channels x up to
// 64 input channels c' of the weight gradient x one token split s.  With CG = K the
// pairs are the K taps of one kernel row of one branch: they share G_b, which is
// then loaded once per chunk.  The kDwWaves waves
// split the token range (bfloat16: contiguous quarters; float32: interleaved
// chunks) and are summed in a fixed order
// through LDS at the end, so each partial element is stored exactly once.
//   MFMA rows    = channel c0 + i of one (b, t) pair (i = lane%16 as A supplier);
//   MFMA columns = c' = cn0 + 16*nb + j (j = lane%16 as B supplier);
//   contraction  = tokens: float32 4 per k-step (lane group g), four k-steps per
//                  16-token chunk; bfloat16 32 per k-step (8 per lane group).
constexpr int kDwWaves = 4;  // waves per dW workgroup; they split the token range

template <typename T, int K, int CG, int NB>
__global__ __launch_bounds__(64 * kDwWaves) void bwd_dw_kernel(const T *__restrict__ x, const T *__restrict__ y,
                                                     const T *__restrict__ gout, float *__restrict__ dw_part,
                                                     float *__restrict__ db_part, int N, int C, int H, int W, int S) {
    constexpr int r = (K - 1) / 2;
    constexpr int KK = K * K;
    constexpr int NCOMBO = 3 * KK;
    constexpr bool BF = Elem<T>::is_bf16;
    constexpr int RL = Run<T>::RL;  // tokens per lane per chunk
    constexpr int KC = 4 * RL;      // tokens per wave per chunk
    __shared__ float red[kDwWaves][NB * 4][64];
    __shared__ float redb[kDwWaves][4][16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int g = lane >> 4;
    const int j = lane & 15;
    // Logical order: (b, t) group fastest, then channel block x c' group, then split,
    // laid out XCD-contiguously so the workgroups of one token split (which read the
    // same y, x and G rows) share an L2.
    const int nCG = (NCOMBO + CG - 1) / CG;
    const int nCB = (C + 15) >> 4;
    const int nNG = (C + 63) >> 6;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int combo0 = (L % nCG) * CG;
    L /= nCG;
    const int cb = L % nCB;
    L /= nCB;
    const int c0 = cb * 16;
    const int cn0 = (L % nNG) * 64;
    const int s = L / nNG;
    const int64_t HW = (int64_t)H * W;
    const int64_t CHW = (int64_t)C * HW;
    const int64_t ntok = (int64_t)N * HW;
    // Split s covers [t0, t1): the even cut ntok*s/S rounded down to a whole round
    // of the four waves' chunks, so that every chunk starts on a chunk boundary
    // (the last split ends at ntok).
    constexpr int64_t ROUND = (int64_t)kDwWaves * 4 * Run<T>::RL;
    const int64_t t0 = ntok * s / S / ROUND * ROUND;
    const int64_t t1 = s + 1 == S ? ntok : ntok * (s + 1) / S / ROUND * ROUND;
    const int64_t R = 3LL * C * KK;

    // Per combo: branch, row/column shift; invalid combos get b = -1.
    int cb_b[CG], cb_dr[CG], cb_dc[CG];
#pragma unroll
    for (int cc = 0; cc < CG; ++cc) {
        const int combo = combo0 + cc;
        if (combo < NCOMBO) {
            const int b = combo / KK;
            const int t = combo - b * KK;
            const int ki = t / K;
            const int kj = t - ki * K;
            cb_b[cc] = b;
            cb_dr[cc] = (ki - r) * dilation(b);
            cb_dc[cc] = (kj - r) * dilation(b);
        } else {
            cb_b[cc] = -1;
            cb_dr[cc] = 0;
            cb_dc[cc] = 0;
        }
    }
    const int cA = c0 + j;         // A role: depthwise channel
    const bool cA_ok = cA < C;
    constexpr bool ROWGROUP = CG == K;  // one kernel row of one branch: G_b shared

    f32x4 acc[CG][NB];
    float dbacc[CG];
#pragma unroll
    for (int cc = 0; cc < CG; ++cc) {
        dbacc[cc] = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[cc][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The wave walks chunks of KC tokens of [wl, wh), keeping the chunk's (image,
    // row, column) position incrementally.  bfloat16: each wave takes a contiguous
    // quarter of the split, so that consecutive chunks of one wave read the two
    // halves of the same cache lines (measured faster); float32: the waves take
    // interleaved chunks (wave, wave + 4, ...) of the whole split (measured faster).
    // A chunk that lies in one image row loads each operand as one run of RL pixels
    // per lane; a chunk that crosses a row end or the range end takes the per-token
    // path.
    constexpr bool CONTIG = BF;
    constexpr int STEP = CONTIG ? KC : kDwWaves * KC;  // tokens from one chunk of the wave to its next
    const int64_t span = t1 - t0;
    const int64_t wl = CONTIG ? t0 + span * wave / kDwWaves / KC * KC : t0 + (int64_t)wave * KC;
    const int64_t wh = (!CONTIG || wave + 1 == kDwWaves) ? t1 : t0 + span * (wave + 1) / kDwWaves / KC * KC;
    int64_t p0 = wl;
    int pn = 0, ph = 0, pw = 0;
    if (p0 < wh) {
        pn = (int)(p0 / HW);
        const int64_t rem = p0 - (int64_t)pn * HW;
        ph = (int)(rem / W);
        pw = (int)(rem - (int64_t)ph * W);
    }
    const bool al = ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0) && ((uintptr_t)gout % 16 == 0) &&
                    (W % 4 == 0);
    const bool chfull = c0 + 16 <= C;            // all 16 depthwise channels exist (wave-uniform)
    const bool cpfull = cn0 + 16 * NB <= C;      // all NB blocks of c' exist (wave-uniform)
    // Raw operands of one chunk: G_b and shifted x per (b, t) pair (their product is
    // the A operand dK), y per c' block (the B operand).
    struct Raw {
        Run<T> gv[CG];
        Run<T> xv[CG];
        Run<T> yv[NB];
    };
    // For loading, a (b, t) slot past the last pair reads the b = 0, zero-shift
    // plane (always valid); its product is zeroed by cb_valid at consumption.
    int cb_bl[CG];
    float cb_valid[CG];
#pragma unroll
    for (int cc = 0; cc < CG; ++cc) {
        cb_bl[cc] = cb_b[cc] >= 0 ? cb_b[cc] : 0;
        cb_valid[cc] = cb_b[cc] >= 0 ? 1.f : 0.f;
    }
    auto load_chunk = [&](int64_t q0, int qn, int qh, int qw, Raw &o) {
        const bool in_row = (q0 + KC <= wh) && (qw + KC <= W);
        // Wave-uniform: the whole chunk is one row segment, every channel exists and
        // every shifted run lies inside its row -> one straight-line block of loads.
        bool fast = in_row && chfull && cpfull;
#pragma unroll
        for (int cc = 0; cc < CG; ++cc) {
            const int hs = qh + cb_dr[cc];
            const int dc = cb_dc[cc];
            fast = fast && hs >= 0 && hs < H && qw + dc - ((qw + dc) & 1) >= 0 && qw + KC - 1 + dc < W;
        }
        if (fast) {
            const int w = qw + RL * g;
            const T *xn = x + (int64_t)qn * CHW;
            const T *gn = gout + (int64_t)qn * 4 * CHW;
            const T *yn = y + (int64_t)qn * CHW;
            const int64_t rowoff = (int64_t)qh * W;
            const bool wal = al && (qw % RL == 0) && (!BF || (W % 8 == 0));  // unshifted runs vector-aligned
            const bool odd = (qw & 1) != 0;
#pragma unroll
            for (int cc = 0; cc < CG; ++cc) {
                const int dc = cb_dc[cc];
                if (!ROWGROUP || cc == 0)
                    o.gv[cc] = Run<T>::fast(gn + (int64_t)((1 + cb_bl[cc]) * C + cA) * HW + rowoff, w, wal, al, odd);
                o.xv[cc] = Run<T>::fast(xn + (int64_t)cA * HW + (int64_t)(qh + cb_dr[cc]) * W, w + dc,
                                        wal && (dc % RL == 0), al, ((qw + dc) & 1) != 0);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                o.yv[nb] = Run<T>::fast(yn + (int64_t)(cn0 + 16 * nb + j) * HW + rowoff, w, wal, al, odd);
            return;
        }
#pragma unroll
        for (int cc = 0; cc < CG; ++cc) o.gv[cc] = o.xv[cc] = Run<T>::zero();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o.yv[nb] = Run<T>::zero();
        if (in_row) {
            const int w = qw + RL * g;
            const T *xn = x + (int64_t)qn * CHW;
            const T *gn = gout + (int64_t)qn * 4 * CHW;
            const T *yn = y + (int64_t)qn * CHW;
            const int64_t rowoff = (int64_t)qh * W;
#pragma unroll
            for (int cc = 0; cc < CG; ++cc) {
                const int b = cb_b[cc];
                if (b >= 0 && cA_ok) {
                    if (!ROWGROUP || cc == 0)
                        o.gv[cc] = Run<T>::checked(gn + (int64_t)((1 + b) * C + cA) * HW + rowoff, w, W, true, al);
                    const int hs = qh + cb_dr[cc];
                    const bool hok = hs >= 0 && hs < H;
                    o.xv[cc] = Run<T>::checked(xn + (int64_t)cA * HW + (int64_t)(hok ? hs : 0) * W, w + cb_dc[cc], W,
                                               hok, al);
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int cp = cn0 + 16 * nb + j;
                if (cp < C) o.yv[nb] = Run<T>::checked(yn + (int64_t)cp * HW + rowoff, w, W, true, al);
            }
        } else {
            const int64_t pf = q0 + (int64_t)g * RL;  // this lane's first token
            int nn = qn, hh = qh, ww = qw + RL * g;
            while (ww >= W) {
                ww -= W;
                if (++hh == H) {
                    hh = 0;
                    ++nn;
                }
            }
#pragma unroll
            for (int k = 0; k < RL; ++k) {
                if (pf + k < wh) {
                    const T *xn = x + (int64_t)nn * CHW;
                    const T *gn = gout + (int64_t)nn * 4 * CHW;
                    const T *yn = y + (int64_t)nn * CHW;
                    const int64_t pix = (int64_t)hh * W + ww;
#pragma unroll
                    for (int cc = 0; cc < CG; ++cc) {
                        const int b = cb_b[cc];
                        if (b >= 0 && cA_ok) {
                            const int hs = hh + cb_dr[cc];
                            const int ws = ww + cb_dc[cc];
                            const bool in = hs >= 0 && hs < H && ws >= 0 && ws < W;
                            if (ROWGROUP ? cc == 0 : in)  // shared G_b: the token's own pixel
                                o.gv[cc].set_raw(k, gn[(int64_t)((1 + b) * C + cA) * HW + pix]);
                            if (in) o.xv[cc].set_raw(k, xn[(int64_t)cA * HW + (int64_t)hs * W + ws]);
                        }
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const int cp = cn0 + 16 * nb + j;
                        if (cp < C) o.yv[nb].set_raw(k, yn[(int64_t)cp * HW + pix]);
                    }
                }
                if (++ww == W) {
                    ww = 0;
                    if (++hh == H) {
                        hh = 0;
                        ++nn;
                    }
                }
            }
        }
    };
    auto advance = [&](int64_t &q0, int &qn, int &qh, int &qw) {
        q0 += STEP;
        qw += STEP;
        while (qw >= W) {
            qw -= W;
            if (++qh == H) {
                qh = 0;
                ++qn;
            }
        }
    };
    auto consume = [&](const Raw &o) {
        float a[CG][RL];
#pragma unroll
        for (int cc = 0; cc < CG; ++cc)
#pragma unroll
            for (int k = 0; k < RL; ++k) {
                // (when CG divides the pair count every slot is a real pair: no mask)
                a[cc][k] = o.gv[ROWGROUP ? 0 : cc].at(k) * o.xv[cc].at(k);
                if constexpr (NCOMBO % CG != 0) a[cc][k] *= cb_valid[cc];
                dbacc[cc] += a[cc][k];
            }
        if constexpr (!BF) {
#pragma unroll
            for (int k = 0; k < RL; ++k)
#pragma unroll
                for (int cc = 0; cc < CG; ++cc)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[cc][nb] = mfma_16x16x4_f32(a[cc][k], o.yv[nb].at(k), acc[cc][nb]);
        } else {
            bf16x8 bq[NB];  // y is already the bf16 operand
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) bq[nb] = __builtin_bit_cast(bf16x8, o.yv[nb].v);
#pragma unroll
            for (int cc = 0; cc < CG; ++cc) {
                uint16_t u[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) u[k] = f32_to_bf16_bits(a[cc][k]);
                const bf16x8 aq = pack_bf16x8(u);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[cc][nb] = mfma_16x16x32_bf16(aq, bq[nb], acc[cc][nb]);
            }
        }
    };

    // The next chunk's loads are issued before this chunk's products and MFMAs.
    {
        Raw nxt;
        if (p0 < wh) load_chunk(p0, pn, ph, pw, nxt);
        while (p0 < wh) {
            const Raw cur = nxt;
            advance(p0, pn, ph, pw);
            if (p0 < wh) load_chunk(p0, pn, ph, pw, nxt);
            consume(cur);
        }
    }

    // Fixed-order reduction over the four waves, one (b, t) pair at a time.
    float *dwp = dw_part + (int64_t)s * R * C;
    float *dbp = db_part + (int64_t)s * R;
#pragma unroll
    for (int cc = 0; cc < CG; ++cc) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][nb * 4 + v][lane] = acc[cc][nb][v];
        redb[wave][g][j] = dbacc[cc];
        __syncthreads();
        const int combo = combo0 + cc;
        if (combo < NCOMBO) {
            const int b = combo / KK;
            const int t = combo - b * KK;
            if (wave < NB) {
                const int nb = wave;
                const int cp = cn0 + 16 * nb + j;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int c = c0 + 4 * g + v;
                    float sum = red[0][nb * 4 + v][lane];
#pragma unroll
                    for (int wv = 1; wv < kDwWaves; ++wv) sum += red[wv][nb * 4 + v][lane];  // fixed order
                    if (c < C && cp < C) dwp[((int64_t)(b * C + c) * KK + t) * C + cp] = sum;
                }
            }
            if (wave == 0 && g == 0 && cn0 == 0 && cA_ok) {
                float sb = 0.f;
#pragma unroll
                for (int wv = 0; wv < kDwWaves; ++wv)
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) sb += redb[wv][gg][j];
                dbp[(int64_t)(b * C + cA) * KK + t] = sb;
            }
        }
        __syncthreads();
    }
}

// ============================================================================ launch
template <typename T, int K>
static hipError_t launch_bwd_k(const void *x, const void *y, const void *wg, const void *bg, const void *gout,
                               void *gx, void *gy, float *dwp, float *dbp, int S, int N, int C, int H, int W, bool al,
                               hipStream_t stream) {
    const int iA = al ? 1 : 0;
    // (b, t) pairs per dW workgroup: the K taps of one kernel row (they share G_b and
    // each y run; measured faster than 2 or 4 consecutive pairs at 256x256, C=64).
    constexpr int CG = K;
    constexpr int NCOMBO = 3 * K * K;
    // Every grid is checked before the first launch, so a refused call writes nothing.
    const int64_t nblk_dx = bwd_dx_blocks(N, C, H, W);
    const int64_t nblk_dy = (int64_t)((W + kCols - 1) / kCols) * H * N * ((C + 63) / 64);
    const int64_t nblk_dw = (int64_t)((NCOMBO + CG - 1) / CG) * ((C + 15) / 16) * ((C + 63) / 64) * S;
    if ((gx != nullptr && nblk_dx > 0x7fffffffLL) || (gy != nullptr && nblk_dy > 0x7fffffffLL) ||
        (dwp != nullptr && nblk_dw > 0x7fffffffLL))
        return hipErrorInvalidConfiguration;
    // dX (bwd_dx.hip)
    if (gx != nullptr) {
        hipError_t e = launch_bwd_dx(y, wg, bg, gout, gx, N, C, H, W, K, Elem<T>::is_bf16, al, stream);
        if (e != hipSuccess) return e;
    }
    // dY staged by source row (bwd_dy_rows.hip) for C = 64 when its grid gives at
    // least one row segment (64 pixels float32, 256 bfloat16) per CU
    constexpr bool BF = Elem<T>::is_bf16;
    if (gy != nullptr && bwd_dy_rows_applies(C, H, W, al, BF) && bwd_dy_rows_blocks(N, H, W, BF) >= kCUs) {
        hipError_t e = launch_bwd_dy_rows(x, wg, gout, gy, N, H, W, K, BF, stream);
        if (e != hipSuccess) return e;
    } else if (gy != nullptr) {
        const dim3 grid((unsigned)nblk_dy);
        const int mb = (C >= 64) ? 4 : (C + 15) / 16;
        // eight waves per workgroup when the grid gives at most two workgroups per CU;
        // sixteen (float32) when at most one
        const bool wide = nblk_dy <= 2 * kCUs;
        const bool wider = !Elem<T>::is_bf16 && nblk_dy <= kCUs;
        auto args = [&](auto kern, int nw) {
            hipLaunchKernelGGL(kern, grid, dim3(64 * nw), 0, stream, (const T *)x, (const T *)wg, (const T *)gout,
                               (T *)gy, C, H, W, iA);
        };
        if (wider) {
            if constexpr (!Elem<T>::is_bf16) {  // (bfloat16 would spill at 128 registers)
                if (mb == 1) args(bwd_dy_kernel<T, K, 1, 16>, 16);
                else if (mb == 2) args(bwd_dy_kernel<T, K, 2, 16>, 16);
                else args(bwd_dy_kernel<T, K, 4, 16>, 16);
            }
        } else if (wide) {
            if (mb == 1) args(bwd_dy_kernel<T, K, 1, 8>, 8);
            else if (mb == 2) args(bwd_dy_kernel<T, K, 2, 8>, 8);
            else args(bwd_dy_kernel<T, K, 4, 8>, 8);
        } else {
            if (mb == 1) args(bwd_dy_kernel<T, K, 1, 4>, 4);
            else if (mb == 2) args(bwd_dy_kernel<T, K, 2, 4>, 4);
            else args(bwd_dy_kernel<T, K, 4, 4>, 4);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // dW / db partials (C = 64: staged by row segment, bwd_dw_rows.hip)
    if (dwp != nullptr && bwd_dw_rows_applies(C, H, W, al, BF)) {
        hipError_t e = launch_bwd_dw_rows(x, y, gout, dwp, dbp, S, N, H, W, K, BF, stream);
        if (e != hipSuccess) return e;
    } else if (dwp != nullptr) {
        const dim3 grid((unsigned)nblk_dw);
        const int nb = (C >= 64) ? 4 : (C + 15) / 16;
        auto args = [&](auto kern) {
            hipLaunchKernelGGL(kern, grid, dim3(64 * kDwWaves), 0, stream, (const T *)x, (const T *)y, (const T *)gout, dwp, dbp,
                               N, C, H, W, S);
        };
        if (nb == 1) args(bwd_dw_kernel<T, K, CG, 1>);
        else if (nb == 2) args(bwd_dw_kernel<T, K, CG, 2>);
        else args(bwd_dw_kernel<T, K, CG, 4>);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_fused_bwd(const void *x, const void *y, const void *wg, const void *bg, const void *gout, void *gx,
                            void *gy, float *dw_part, float *db_part, int S, int N, int C, int H, int W, int K,
                            bool bf16, bool al, hipStream_t stream) {
    if (bf16) {
        switch (K) {
            case 1: return launch_bwd_k<bf16_t, 1>(x, y, wg, bg, gout, gx, gy, dw_part, db_part, S, N, C, H, W, al, stream);
            case 3: return launch_bwd_k<bf16_t, 3>(x, y, wg, bg, gout, gx, gy, dw_part, db_part, S, N, C, H, W, al, stream);
            default: return launch_bwd_k<bf16_t, 5>(x, y, wg, bg, gout, gx, gy, dw_part, db_part, S, N, C, H, W, al, stream);
        }
    }
    switch (K) {
        case 1: return launch_bwd_k<float, 1>(x, y, wg, bg, gout, gx, gy, dw_part, db_part, S, N, C, H, W, al, stream);
        case 3: return launch_bwd_k<float, 3>(x, y, wg, bg, gout, gx, gy, dw_part, db_part, S, N, C, H, W, al, stream);
        default: return launch_bwd_k<float, 5>(x, y, wg, bg, gout, gx, gy, dw_part, db_part, S, N, C, H, W, al, stream);
    }
}

}  // namespace ddpm

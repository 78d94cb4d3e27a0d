// fused_fwd.hip -- 1x1 generator fused with the dynamic dilated filter (gfx950).
//
// Operation (page "lartpang/DynamicConvolutionOperator", section
// "CUDA 融合生成器推理"): per channel tile x spatial tile, weight x y-tile gives the
// dynamic taps, which are consumed at once with the shifted x; the taps live only
// in registers and never reach global memory.  Output [x, d1, d3, d5].
//
// Work decomposition
//   workgroup = 4 waves = image n, 16 depthwise channels c0.., 4 rows x 64 columns;
//   wave      = one row of the tile (64 pixels, four per lane);
//   per (branch b, tap t) the wave runs the generator block for its 16 channels
//   (see gen_mma.hpp), adds the bias, rounds the taps to the dtype, and
//   multiplies them with x at the dilated offset, read from an LDS copy of the
//   x tile with its 5*(K-1)/2 halo.  The three branch sums stay in registers.
//   bfloat16 takes the taps of a branch in pairs and adds each pair's two products
//   with one v_dot2_f32_bf16.
// bfloat16 grids with one workgroup per CU instead run workgroups of three such
// four-wave groups, one per dilation branch, sharing the staged x tile.
// y is read once per wave into registers (the MFMA B operand is the same for
// all 3*K*K generator blocks) when C <= 64; larger C streams it per block.
// bfloat16 at K = 3 and C = 64 (W % 8 == 0, 16-byte aligned tensors) goes to the
// persistent kernel of fused_fwd_pers.hip instead: same arithmetic, tiles streamed
// into LDS behind the compute.
// The staged x planes of channels 4g..4g+3 (lane group g) are shifted by g floats
// so that the four groups' reads fall on different LDS banks.
#include <algorithm>
#include <type_traits>

#include "gen_mma.hpp"
#include "launchers.hpp"

namespace ddpm {

constexpr int kTileRows = 4;   // one row per wave
constexpr int kTileCols = 64;  // 16 lanes x 4 pixels
constexpr int kCUs = 256;        // compute units of the chip (MI355X)

template <int K> struct XTile {
    static constexpr int r = (K - 1) / 2;
    static constexpr int HALO = 5 * r;                 // rows and columns of halo
    static constexpr int PADC = (HALO + 3) & ~3;       // left column pad, a multiple of 4
    static constexpr int LH = kTileRows + 2 * HALO;
    static constexpr int LW = kTileCols + 2 * PADC;    // a multiple of 4
    static constexpr int PLANE = LH * LW;
    static constexpr int NV = 16 * PLANE / 4;          // 4-column runs of the 16-channel tile
    static constexpr int BIAS = 3 * K * K * 16;  // bias of the 16 channels for every (b, t)
    static constexpr int BOFF = 16 * PLANE + 4;  // where the bias slice starts (floats)
    static constexpr size_t bytes = sizeof(float) * (BOFF + BIAS);
    // Plane of channel ch.  A wave reads channel 4g+v in lane group g at columns 4j+..,
    // and 4*PLANE is a multiple of the 64 banks, so the four groups would hit the same
    // 16 banks; shifting group g's planes by g floats spreads them over all 64.
    static __device__ __forceinline__ int plane(int ch) { return ch * PLANE + (ch >> 2); }
};

// Stage x[n, c0..c0+15, h0-HALO .., w0-PADC ..] into LDS as float, zero outside the
// image and for channels >= C.  `vec`: W % 4 == 0 and 16-byte aligned x, so every
// 4-column run (w0 and PADC are multiples of 4) lies wholly inside or outside the
// image and is one vector load.  The trip counts are compile-time constants, so the
// loads of a batch are all issued before the first LDS store waits for them.
template <typename T, int K>
__device__ __forceinline__ void stage_x_tile(float *xs, const T *__restrict__ xn, int c0, int C, int H, int W,
                                             int64_t HW, int h0, int w0, bool vec) {
    using X = XTile<K>;
    constexpr int NT = 256;
    constexpr int VPR = X::LW / 4;
    if (vec) {
        constexpr int IT = (X::NV + NT - 1) / NT;
        constexpr int BATCH = 9;
#pragma unroll
        for (int k0 = 0; k0 < IT; k0 += BATCH) {
            f32x4 v[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                if (k0 + k >= IT) continue;
                const int i = (k0 + k) * NT + (int)threadIdx.x;
                const int row = i / VPR;  // channel * LH + lr
                const int cv = i - row * VPR;
                const int ch = row / X::LH;
                const int lr = row - ch * X::LH;
                const int c = c0 + ch;
                const int hh = h0 - X::HALO + lr;
                const int ww = w0 - X::PADC + 4 * cv;
                const bool ok = i < X::NV && c < C && hh >= 0 && hh < H && ww >= 0 && ww < W;
                // branch-free: a run outside the image reads the image's first run and is zeroed
                const T *src = xn + (ok ? (int64_t)c * HW + (int64_t)hh * W + ww : 0);
                f32x4 t;
                if constexpr (Elem<T>::is_bf16) {
                    const u16x4 u = *(const u16x4 *)src;
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[e] = bf16_bits_to_f32(u[e]);
                } else {
                    t = *(const f32x4 *)src;
                }
                v[k] = ok ? t : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const int i = (k0 + k) * NT + (int)threadIdx.x;
                if (k0 + k < IT && i < X::NV) {
                    // shifted planes: 4-byte aligned, two ds_write2_b32
                    float *d = xs + 4 * i + (i / (X::NV / 4));
#pragma unroll
                    for (int e = 0; e < 4; ++e) d[e] = v[k][e];
                }
            }
        }
    } else {
        constexpr int NE = 16 * X::PLANE;
        constexpr int IT = (NE + NT - 1) / NT;
        constexpr int BATCH = 16;
#pragma unroll
        for (int k0 = 0; k0 < IT; k0 += BATCH) {
            float v[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                if (k0 + k >= IT) continue;
                const int i = (k0 + k) * NT + (int)threadIdx.x;
                const int row = i / X::LW;
                const int lc = i - row * X::LW;
                const int ch = row / X::LH;
                const int lr = row - ch * X::LH;
                const int c = c0 + ch;
                const int hh = h0 - X::HALO + lr;
                const int ww = w0 - X::PADC + lc;
                const bool ok = i < NE && c < C && hh >= 0 && hh < H && ww >= 0 && ww < W;
                const float e = Elem<T>::to_f32(xn[ok ? (int64_t)c * HW + (int64_t)hh * W + ww : 0]);
                v[k] = ok ? e : 0.f;
            }
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const int i = (k0 + k) * NT + (int)threadIdx.x;
                if (k0 + k < IT && i < NE) xs[i + i / (NE / 4)] = v[k];
            }
        }
    }
}

// Store four values that were widened exactly from T (float, or bf16 bits << 16)
// back as their original bits: the x block of the output is a bit-exact copy.
template <typename T>
__device__ __forceinline__ void store4_bits(T *__restrict__ row, int w, int W, f32x4 v, bool aligned4) {
    if (w + 3 < W && aligned4) {
        if constexpr (Elem<T>::is_bf16) {
            u16x4 u;
#pragma unroll
            for (int k = 0; k < 4; ++k) u[k] = exact_narrow<T>(v[k]);
            *(u16x4 *)(row + w) = u;
        } else {
            *(f32x4 *)(row + w) = v;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (w + k < W) row[w + k] = exact_narrow<T>(v[k]);
    }
}

template <typename T, int K, int KQ, bool SPLIT, bool GRP3>
__global__ __launch_bounds__(GRP3 ? 768 : 256, GRP3 ? 3 : 2) void fused_fwd_kernel(const T *__restrict__ x, const T *__restrict__ y,
                                                           const T *__restrict__ wg, const T *__restrict__ bg,
                                                           T *__restrict__ out, int C, int H, int W, int al) {
    using G = Gen<T>;
    using X = XTile<K>;
    constexpr int r = X::r;
    constexpr int KK = K * K;
    extern __shared__ float xs[];

    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int wave = GRP3 ? (wave_all & 3) : wave_all;  // the tile row this wave computes
    const int g = lane >> 4;
    const int j = lane & 15;
    const int nCB = (C + 15) >> 4;
    // logical tile order: (branch when SPLIT,) channel block, column tile, row band,
    // image.  SPLIT: each workgroup computes one dilation branch of its tile (the
    // three write separate output blocks), for grids too small to fill the chip.
    const int ncolt = (W + kTileCols - 1) / kTileCols;
    const int nbands = (H + kTileRows - 1) / kTileRows;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    // the branch this workgroup (SPLIT) or wave group (GRP3) computes, -1: all
    const int bsel = SPLIT ? L % 3 : (GRP3 ? (wave_all >> 2) : -1);
    if (SPLIT) L /= 3;
    const int c0 = (L % nCB) * 16;
    L /= nCB;
    const int w0 = (L % ncolt) * kTileCols;
    L /= ncolt;
    const int h0 = (L % nbands) * kTileRows;
    const int n = L / nbands;
    const int64_t HW = (int64_t)H * W;
    const bool aligned4 = al != 0;
    const bool cvec = Elem<T>::is_bf16 ? (al != 0 && (C & 7) == 0) : (al != 0 && (C & 3) == 0);

    const T *__restrict__ xn = x + (int64_t)n * C * HW;
    const T *__restrict__ yn = y + (int64_t)n * C * HW;
    // bias slice: bl[(b*KK + t)*16 + ch] = bias[(b*C + c0 + ch)*KK + t]
    float *bl = xs + X::BOFF;
    if (!GRP3 || wave_all < 4) {  // the first 256 threads stage the shared tile
        stage_x_tile<T, K>(xs, xn, c0, C, H, W, HW, h0, w0, aligned4);
#pragma unroll
        for (int k = 0; k < (X::BIAS + 255) / 256; ++k) {
            const int i = k * 256 + (int)threadIdx.x;
            if (i >= X::BIAS) break;
            const int combo = i >> 4;
            const int c = c0 + (i & 15);
            const int b = combo / KK;
            const int t = combo - b * KK;
            bl[i] = c < C ? Elem<T>::to_f32(bg[(int64_t)(b * C + c) * KK + t]) : 0.f;
        }
    }

    const int h = h0 + wave;
    const bool row_ok = h < H;
    const int w = w0 + 4 * j;
    const int64_t rowoff = (int64_t)h * W;
    const int nq = (C + G::CH - 1) / G::CH;

    typename G::BFrag bres[KQ > 0 ? KQ : 1];
    if constexpr (KQ > 0) {
#pragma unroll
        for (int q = 0; q < KQ; ++q) bres[q] = G::load_B(yn, q, g, C, HW, rowoff, w, W, row_ok, aligned4);
    }
    __syncthreads();

    // Outputs are stored as soon as they are final, so that the stores overlap the
    // remaining taps: the x block now, from the staged tile (its interior holds the
    // row's 64 pixels of the 16 channels), and each branch after its last tap.
    T *__restrict__ on = out + (int64_t)n * 4 * C * HW;
    auto store_branch = [&](int b, const float (&ob)[4][4]) {
        if (!row_ok) return;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = c0 + 4 * g + v;
            if (c < C)
                store4_row(on + (int64_t)((1 + b) * C + c) * HW + rowoff, w, W,
                           f32x4{ob[v][0], ob[v][1], ob[v][2], ob[v][3]}, aligned4);
        }
    };
    if (row_ok && (!(SPLIT || GRP3) || bsel == 0)) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = c0 + 4 * g + v;
            const float *xp = xs + X::plane(4 * g + v) + (wave + X::HALO) * X::LW + X::PADC + 4 * j;
            const f32x4 xv = {xp[0], xp[1], xp[2], xp[3]};
            if (c < C) store4_bits(on + (int64_t)c * HW + rowoff, w, W, xv, aligned4);
        }
    }

    const int cA = c0 + j;  // channel of the generator row this lane supplies
    // Wave-uniform: all 16 channels exist, every weight chunk is whole and vector-aligned.
    // (KQ chunks must cover exactly C channels: the fp32 KQ=4 instance also serves C = 48.)
    const bool full = (c0 + 16 <= C) && cvec && (KQ * G::CH == C);
    float oacc[3][4][4];    // [branch][v][pb]
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) oacc[b][v][pb] = 0.f;

    const int aoff = cA * KK * C + 4 * (Elem<T>::is_bf16 ? 2 : 1) * g;  // lane's offset inside a (b, t) slice
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        if ((SPLIT || GRP3) && b != bsel) continue;  // wave-uniform
        const int D = dilation(b);
        // Generator-row operand of tap t of this branch.
        auto fetch = [&](int t, typename G::AFrag (&af)[KQ > 0 ? KQ : 1]) {
            if (full) {  // wave-uniform: every row and column exists
                // uniform slice base + 32-bit lane offset
                const T *wbt = wg + ((int64_t)b * C * KK + t) * C;
#pragma unroll
                for (int q = 0; q < (KQ > 0 ? KQ : 1); ++q) af[q] = G::load_A_off(wbt, aoff + G::CH * q);
                return;
            }
            const T *arow = cA < C ? wg + ((int64_t)(b * C + cA) * KK + t) * C : nullptr;
#pragma unroll
            for (int q = 0; q < (KQ > 0 ? KQ : 1); ++q) af[q] = G::load_A(arow, q, g, C, cvec);
        };
        if constexpr (Elem<T>::is_bf16 && KQ > 0) {
            // bfloat16: taps in pairs (t, t+1).  The pair's two rounded taps of one
            // channel and pixel share a packed dword (v_cvt_pk_bf16_f32), their x
            // values another (the high halves of the staged floats, which are the
            // bf16 inputs exactly; v_perm_b32), and v_dot2_f32_bf16 adds both exact
            // products to the float32 sum.  An odd last tap pairs with zeros.  The
            // weights of the next pair are fetched into the fragments of this one once
            // its MFMAs are issued; the biases and x values are read before the MFMAs.
            // FULL (wave-uniform) is tested once, outside the loop.
            auto run_pairs = [&](auto fullc) {
                constexpr bool FULL = decltype(fullc)::value;
                auto fetch2 = [&](int t, typename G::AFrag (&af)[KQ]) {
                    if constexpr (FULL) {
                        // a buffer load: the lane's part of the offset is fixed, the
                        // tap's part a scalar (no 64-bit address arithmetic per tap)
                        const __amdgpu_buffer_rsrc_t rw =
                            __builtin_amdgcn_make_buffer_rsrc((void *)wg, 0, 3 * C * KK * C * 2, 0x00020000);
                        const int so = (b * C * KK + t) * C * 2;
#pragma unroll
                        for (int q = 0; q < KQ; ++q)
                            af[q].v = __builtin_bit_cast(
                                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rw, (unsigned)(aoff + G::CH * q) * 2u, so, 0));
                    } else {
                        const T *arow = cA < C ? wg + ((int64_t)(b * C + cA) * KK + t) * C : nullptr;
#pragma unroll
                        for (int q = 0; q < KQ; ++q) af[q] = G::load_A(arow, q, g, C, cvec);
                    }
                };
                auto read_x = [&](int t, float (&xv)[4][4]) {
                    const int ki = t / K;
                    const int kj = t - ki * K;
                    const float *xl = xs + (wave + X::HALO + (ki - r) * D) * X::LW + 4 * j + X::PADC + (kj - r) * D;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
#pragma unroll
                        for (int pb = 0; pb < 4; ++pb) xv[v][pb] = xl[X::plane(4 * g + v) + pb];
                };
                typename G::AFrag wa0[KQ], wa1[KQ];
                fetch2(0, wa0);
                if (KK > 1) fetch2(1, wa1);
                int t = 0;
#pragma unroll 1
                for (; t + 1 < KK; t += 2) {
                    const f32x4 bias0 = *(const f32x4 *)(bl + (b * KK + t) * 16 + 4 * g);
                    const f32x4 bias1 = *(const f32x4 *)(bl + (b * KK + t + 1) * 16 + 4 * g);
                    float x0[4][4], x1[4][4];
                    read_x(t, x0);
                    read_x(t + 1, x1);
                    f32x4 acc0[4], acc1[4];
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) {
                        acc0[pb] = bias0;
                        acc1[pb] = bias1;
                    }
#pragma unroll
                    for (int q = 0; q < KQ; ++q) G::mma(acc0, wa0[q], bres[q]);
#pragma unroll
                    for (int q = 0; q < KQ; ++q) G::mma(acc1, wa1[q], bres[q]);
                    if (t + 2 < KK) fetch2(t + 2, wa0);
                    if (t + 3 < KK) fetch2(t + 3, wa1);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
#pragma unroll
                        for (int pb = 0; pb < 4; ++pb) {
                            const bf16x2_t qp = bf16x2_t{(__bf16)acc0[pb][v], (__bf16)acc1[pb][v]};
                            const uint32_t xp = __builtin_amdgcn_perm(__float_as_uint(x1[v][pb]),
                                                                      __float_as_uint(x0[v][pb]), 0x07060302u);
                            oacc[b][v][pb] = __builtin_amdgcn_fdot2_f32_bf16(qp, __builtin_bit_cast(bf16x2_t, xp),
                                                                             oacc[b][v][pb], false);
                        }
                }
                if (t < KK) {  // the odd last tap, its weights in wa0
                    const f32x4 bias0 = *(const f32x4 *)(bl + (b * KK + t) * 16 + 4 * g);
                    float x0[4][4];
                    read_x(t, x0);
                    f32x4 acc0[4];
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) acc0[pb] = bias0;
#pragma unroll
                    for (int q = 0; q < KQ; ++q) G::mma(acc0, wa0[q], bres[q]);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
#pragma unroll
                        for (int pb = 0; pb < 4; ++pb) {
                            const bf16x2_t qp = bf16x2_t{(__bf16)acc0[pb][v], (__bf16)0.f};
                            const uint32_t xp = __float_as_uint(x0[v][pb]) >> 16;
                            oacc[b][v][pb] = __builtin_amdgcn_fdot2_f32_bf16(qp, __builtin_bit_cast(bf16x2_t, xp),
                                                                             oacc[b][v][pb], false);
                        }
                }
            };
            if (full)
                run_pairs(std::true_type{});
            else
                run_pairs(std::false_type{});
            store_branch(b, oacc[b]);
            continue;
        }
        typename G::AFrag anext[KQ > 0 ? KQ : 1];
        if constexpr (KQ > 0) fetch(0, anext);
#pragma unroll 1
        for (int t = 0; t < KK; ++t) {
            const f32x4 bias = *(const f32x4 *)(bl + (b * KK + t) * 16 + 4 * g);
            f32x4 acc[4];
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) acc[pb] = bias;
            if constexpr (KQ > 0) {
                // operands of tap t were fetched one tap ahead; fetch tap t+1 now
                typename G::AFrag acur[KQ];
#pragma unroll
                for (int q = 0; q < KQ; ++q) acur[q] = anext[q];
                if (t + 1 < KK) fetch(t + 1, anext);
#pragma unroll
                for (int q = 0; q < KQ; ++q) G::mma(acc, acur[q], bres[q]);
            } else {
                const T *arow = cA < C ? wg + ((int64_t)(b * C + cA) * KK + t) * C : nullptr;
                for (int q = 0; q < nq; ++q)
                    G::mma(acc, G::load_A(arow, q, g, C, cvec),
                           G::load_B(yn, q, g, C, HW, rowoff, w, W, row_ok, aligned4));
            }
            const int ki = t / K;
            const int kj = t - ki * K;
            const float *xl = xs + (wave + X::HALO + (ki - r) * D) * X::LW + 4 * j + X::PADC + (kj - r) * D;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float *xr = xl + X::plane(4 * g + v);
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) oacc[b][v][pb] += Elem<T>::quant(acc[pb][v]) * xr[pb];
            }
        }
        store_branch(b, oacc[b]);
    }
}

template <typename T, int K, int KQ>
static hipError_t launch_fused_t(const void *x, const void *y, const void *wg, const void *bg, void *out, int N,
                                 int C, int H, int W, bool al, hipStream_t stream) {
    auto kern = fused_fwd_kernel<T, K, KQ, false, false>;
    auto kern_split = fused_fwd_kernel<T, K, KQ, true, false>;
    // bfloat16 only: a workgroup of three four-wave groups, one per branch (float32's
    // longer MFMAs keep the pipe busy with fewer waves; measured no gain there)
    auto kern_grp3 = fused_fwd_kernel<T, K, KQ, false, Elem<T>::is_bf16>;
    const size_t lds = XTile<K>::bytes;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)kern_split, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess && Elem<T>::is_bf16)
            e = hipFuncSetAttribute((const void *)kern_grp3, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t nblk = (int64_t)((W + kTileCols - 1) / kTileCols) * ((H + kTileRows - 1) / kTileRows) * N *
                         ((C + 15) / 16);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // When one workgroup per (tile, branch) still fits the chip in one round (256 CUs,
    // each holding as many of these workgroups as its 160 KB of LDS allows, at most
    // two), split the branches: each workgroup then does a third of the serial taps.
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(2, (int64_t)(160 * 1024) / (int64_t)lds));
    if (nblk * 3 <= kCUs * per_cu)
        hipLaunchKernelGGL(kern_split, dim3((unsigned)(nblk * 3)), dim3(256), lds, stream, (const T *)x, (const T *)y,
                           (const T *)wg, (const T *)bg, (T *)out, C, H, W, al ? 1 : 0);
    // bfloat16 with one workgroup per CU (the K = 5 tile's LDS, or a grid of at most one
    // per CU): three branch groups share the workgroup's x tile, tripling the waves
    else if (Elem<T>::is_bf16 && (per_cu == 1 || nblk <= kCUs))
        hipLaunchKernelGGL(kern_grp3, dim3((unsigned)nblk), dim3(768), lds, stream, (const T *)x, (const T *)y,
                           (const T *)wg, (const T *)bg, (T *)out, C, H, W, al ? 1 : 0);
    else
        hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), lds, stream, (const T *)x, (const T *)y,
                           (const T *)wg, (const T *)bg, (T *)out, C, H, W, al ? 1 : 0);
    return hipGetLastError();
}

template <typename T, int K>
static hipError_t launch_fused_k(const void *x, const void *y, const void *wg, const void *bg, void *out, int N,
                                 int C, int H, int W, bool al, hipStream_t stream) {
    const int nq = (C + Gen<T>::CH - 1) / Gen<T>::CH;
    if constexpr (Elem<T>::is_bf16) {
        if (nq == 1) return launch_fused_t<T, K, 1>(x, y, wg, bg, out, N, C, H, W, al, stream);
        if (nq == 2) return launch_fused_t<T, K, 2>(x, y, wg, bg, out, N, C, H, W, al, stream);
    } else {
        if (nq == 1) return launch_fused_t<T, K, 1>(x, y, wg, bg, out, N, C, H, W, al, stream);
        if (nq == 2) return launch_fused_t<T, K, 2>(x, y, wg, bg, out, N, C, H, W, al, stream);
        if (nq <= 4) return launch_fused_t<T, K, 4>(x, y, wg, bg, out, N, C, H, W, al, stream);
    }
    return launch_fused_t<T, K, 0>(x, y, wg, bg, out, N, C, H, W, al, stream);
}

hipError_t launch_fused_fwd(const void *x, const void *y, const void *wg, const void *bg, void *out, int N, int C,
                            int H, int W, int K, bool bf16, bool al, hipStream_t stream) {
    if (fused_fwd_pers_applies(N, C, H, W, K, bf16, al))
        return launch_fused_fwd_pers(x, y, wg, bg, out, N, H, W, stream);
    if (bf16) {
        switch (K) {
            case 1: return launch_fused_k<bf16_t, 1>(x, y, wg, bg, out, N, C, H, W, al, stream);
            case 3: return launch_fused_k<bf16_t, 3>(x, y, wg, bg, out, N, C, H, W, al, stream);
            default: return launch_fused_k<bf16_t, 5>(x, y, wg, bg, out, N, C, H, W, al, stream);
        }
    }
    switch (K) {
        case 1: return launch_fused_k<float, 1>(x, y, wg, bg, out, N, C, H, W, al, stream);
        case 3: return launch_fused_k<float, 3>(x, y, wg, bg, out, N, C, H, W, al, stream);
        default: return launch_fused_k<float, 5>(x, y, wg, bg, out, N, C, H, W, al, stream);
    }
}

}  // namespace ddpm

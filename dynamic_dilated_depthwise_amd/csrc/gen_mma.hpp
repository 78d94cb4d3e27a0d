// gen_mma.hpp -- the 1x1 generator contraction on MFMA, per wave.
//
// Tile shape used by the fused forward and by the dX recompute:
//   MFMA rows    = 16 depthwise channels c0 + i sharing one (branch, tap) pair,
//                  so row i of the generator block is o = (b*C + c0 + i)*K*K + t;
//   MFMA columns = 16 lanes j, each owning four neighbouring pixels
//                  w + 4j + pb (pb = 0..3), one 16x16 product per pb;
//   contraction  = the C input channels of y, in chunks of CH channels.
// Lane (g = lane/16, j = lane%16) receives the taps of channels c0 + 4g + v
// (v = 0..3) at its four pixels, i.e. D[4g+v][j] of each of the four products.
//
// float32: v_mfma_f32_16x16x4_f32, chunk CH = 16 channels = four k-steps; in
//   k-step s lane group g carries channel 16q + 4g + s, so one 16-byte load of a
//   weight row feeds four k-steps and one 16-byte load of a y row feeds four
//   pixels.
// bfloat16: v_mfma_f32_16x16x32_bf16, chunk CH = 32 channels = one k-step; lane
//   group g carries channels 32q + 8g + e (e = 0..7), one 16-byte load of a
//   weight row; y is gathered as 4-pixel runs of 8 channels and transposed in
//   registers.
#pragma once

#include "common.hpp"

namespace ddpm {

template <typename T> struct Gen;

template <> struct Gen<float> {
    static constexpr int CH = 16;
    struct BFrag { f32x4 v[4]; };  // v[s][pb]
    struct AFrag { f32x4 v; };     // v[s]

    // y rows of chunk q for this lane group at pixels w..w+3 of row `rowoff`.
    __device__ __forceinline__ static BFrag load_B(const float *__restrict__ yn, int q, int g, int C, int64_t HW,
                                                   int64_t rowoff, int w, int W, bool row_ok, bool al) {
        BFrag b;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = 16 * q + 4 * g + s;
            b.v[s] = load4_row(yn + (int64_t)(c < C ? c : 0) * HW + rowoff, w, W, row_ok && c < C, al);
        }
        return b;
    }
    // As load_B with every lane's run known to be in range (wave-uniform test by the
    // caller): no per-lane bounds checks.  `w_al`: w % 4 == 0 with aligned rows.
    __device__ __forceinline__ static BFrag load_B_fast(const float *__restrict__ yn, int q, int g, int64_t HW,
                                                        int64_t rowoff, int w, bool w_al, bool, bool) {
        BFrag b;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.v[s] = load4_unchecked(yn + (int64_t)(16 * q + 4 * g + s) * HW + rowoff, w, w_al, true, false);
        return b;
    }
    // Fragment at a wave-uniform base plus a 32-bit lane offset (16-byte aligned).
    __device__ __forceinline__ static AFrag load_A_off(const float *__restrict__ base, int off) {
        AFrag a;
        a.v = *(const f32x4 *)(base + off);
        return a;
    }
    // load_B_fast addressed as a wave-uniform row base of the chunk's first channel
    // plus a 32-bit lane offset (lane group g's plane and column); planes HW apart.
    __device__ __forceinline__ static BFrag load_B_off(const float *__restrict__ base, int off, int HW, bool w_al,
                                                       bool, bool) {
        BFrag b;
#pragma unroll
        for (int s = 0; s < 4; ++s) b.v[s] = load4_unchecked(base + (int64_t)s * HW, off, w_al, true, false);
        return b;
    }
    // As load_A for an existing row with C % 4 == 0 and a 16-byte aligned weight.
    __device__ __forceinline__ static AFrag load_A_fast(const float *__restrict__ arow, int q, int g) {
        AFrag a;
        a.v = *(const f32x4 *)(arow + 16 * q + 4 * g);
        return a;
    }
    // Weight row `arow` (nullptr when the row does not exist), columns 16q+4g..+3.
    __device__ __forceinline__ static AFrag load_A(const float *__restrict__ arow, int q, int g, int C, bool c4) {
        AFrag a;
        a.v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (arow == nullptr) return a;
        const int c = 16 * q + 4 * g;
        if (c4 && c + 3 < C) {
            a.v = *(const f32x4 *)(arow + c);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (c + s < C) a.v[s] = arow[c + s];
        }
        return a;
    }
    __device__ __forceinline__ static void mma(f32x4 (&acc)[4], const AFrag &a, const BFrag &b) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) acc[pb] = mfma_16x16x4_f32(a.v[s], b.v[s][pb], acc[pb]);
    }
};

template <> struct Gen<bf16_t> {
    static constexpr int CH = 32;
    struct BFrag { bf16x8 v[4]; };  // v[pb]
    struct AFrag { bf16x8 v; };

    __device__ __forceinline__ static void load4_raw(const bf16_t *__restrict__ row, int w, int W, bool ok,
                                                     bool al, uint16_t (&o)[4]) {
        o[0] = o[1] = o[2] = o[3] = 0;
        if (!ok) return;
        if (w >= 0 && w + 3 < W && al) {
            const u16x4 u = *(const u16x4 *)(row + w);
            o[0] = u[0]; o[1] = u[1]; o[2] = u[2]; o[3] = u[3];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int ww = w + k;
                if (ww >= 0 && ww < W) o[k] = row[ww];
            }
        }
    }
    __device__ __forceinline__ static BFrag load_B(const bf16_t *__restrict__ yn, int q, int g, int C, int64_t HW,
                                                   int64_t rowoff, int w, int W, bool row_ok, bool al) {
        uint16_t v[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 32 * q + 8 * g + e;
            load4_raw(yn + (int64_t)(c < C ? c : 0) * HW + rowoff, w, W, row_ok && c < C, al, v[e]);
        }
        BFrag b;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            uint16_t col[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) col[e] = v[e][pb];
            b.v[pb] = pack_bf16x8(col);
        }
        return b;
    }
    // Four raw bf16 values at row[w..w+3] with no bounds checks (see load4_unchecked).
    __device__ __forceinline__ static void load4_raw_fast(const bf16_t *__restrict__ row, int w, bool w_al,
                                                          bool row_even, bool odd, uint16_t (&o)[4]) {
        if (w_al) {
            const u16x4 u = *(const u16x4 *)(row + w);
            o[0] = u[0]; o[1] = u[1]; o[2] = u[2]; o[3] = u[3];
        } else if (row_even && !odd) {
            const u32x2_a4 d = *(const u32x2_a4 *)(row + w);
            o[0] = (uint16_t)d[0]; o[1] = (uint16_t)(d[0] >> 16);
            o[2] = (uint16_t)d[1]; o[3] = (uint16_t)(d[1] >> 16);
        } else if (row_even) {
            const u32x2_a4 d = *(const u32x2_a4 *)(row + w - 1);
            o[0] = (uint16_t)(d[0] >> 16); o[1] = (uint16_t)d[1];
            o[2] = (uint16_t)(d[1] >> 16); o[3] = row[w + 3];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = row[w + k];
        }
    }
    __device__ __forceinline__ static BFrag load_B_fast(const bf16_t *__restrict__ yn, int q, int g, int64_t HW,
                                                        int64_t rowoff, int w, bool w_al, bool row_even, bool odd) {
        uint16_t v[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            load4_raw_fast(yn + (int64_t)(32 * q + 8 * g + e) * HW + rowoff, w, w_al, row_even, odd, v[e]);
        BFrag b;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            uint16_t col[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) col[e] = v[e][pb];
            b.v[pb] = pack_bf16x8(col);
        }
        return b;
    }
    __device__ __forceinline__ static BFrag load_B_off(const bf16_t *__restrict__ base, int off, int HW, bool w_al,
                                                       bool row_even, bool odd) {
        uint16_t v[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e) load4_raw_fast(base + (int64_t)e * HW, off, w_al, row_even, odd, v[e]);
        BFrag b;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            uint16_t col[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) col[e] = v[e][pb];
            b.v[pb] = pack_bf16x8(col);
        }
        return b;
    }
    __device__ __forceinline__ static AFrag load_A_off(const bf16_t *__restrict__ base, int off) {
        AFrag a;
        a.v = __builtin_bit_cast(bf16x8, *(const u16x8 *)(base + off));
        return a;
    }
    // As load_A for an existing row with C % 8 == 0 and a 16-byte aligned weight.
    __device__ __forceinline__ static AFrag load_A_fast(const bf16_t *__restrict__ arow, int q, int g) {
        AFrag a;
        a.v = __builtin_bit_cast(bf16x8, *(const u16x8 *)(arow + 32 * q + 8 * g));
        return a;
    }
    __device__ __forceinline__ static AFrag load_A(const bf16_t *__restrict__ arow, int q, int g, int C, bool c8) {
        const int c = 32 * q + 8 * g;
        uint16_t u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        AFrag a;
        if (arow != nullptr) {
            if (c8 && c + 7 < C) {
                a.v = __builtin_bit_cast(bf16x8, *(const u16x8 *)(arow + c));
                return a;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (c + e < C) u[e] = arow[c + e];
        }
        a.v = pack_bf16x8(u);
        return a;
    }
    __device__ __forceinline__ static void mma(f32x4 (&acc)[4], const AFrag &a, const BFrag &b) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[pb] = mfma_16x16x32_bf16(a.v, b.v[pb], acc[pb]);
    }
};

}  // namespace ddpm

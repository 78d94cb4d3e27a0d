// common.hpp -- device helpers shared by the DDPM kernels (gfx950 / CDNA4, wave64).
//
// Storage types: float for float32 tensors, uint16_t for bfloat16 tensors (raw
// bits).  Arithmetic is always float32; bf16 values widen exactly and narrow with
// the hardware round-to-nearest-even conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ddpm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

typedef uint16_t bf16_t;

constexpr int kWave = 64;

// Branch b uses dilation 1 + 2b, i.e. (1, 3, 5).
__host__ __device__ constexpr int dilation(int b) { return 1 + 2 * b; }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
    return __uint_as_float((uint32_t)u << 16);
}
// Round-to-nearest-even narrowing (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float round_to_bf16(float f) {
    return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr bool is_bf16 = false;
    __device__ __forceinline__ static float to_f32(float v) { return v; }
    __device__ __forceinline__ static float from_f32(float v) { return v; }
    // Value as it is used inside the method after the dtype's own rounding.
    __device__ __forceinline__ static float quant(float v) { return v; }
};
template <> struct Elem<bf16_t> {
    static constexpr bool is_bf16 = true;
    __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_bits_to_f32(v); }
    __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16_bits(v); }
    __device__ __forceinline__ static float quant(float v) { return round_to_bf16(v); }
};

// Workgroup order across the chip.  Consecutive workgroup IDs are dispatched
// round-robin over the 8 XCDs, each with its own L2; remapping so that every XCD
// receives a contiguous run of logical tiles keeps tiles that share data (halo
// rows, the channel blocks of one pixel tile) in the same L2.  Bijective for any
// count.
__device__ __forceinline__ int xcd_contiguous(int id, int count) {
    constexpr int kXcd = 8;
    const int q = count / kXcd, rem = count % kXcd;
    const int xcd = id % kXcd, idx = id / kXcd;
    return xcd * q + (xcd < rem ? xcd : rem) + idx;
}

// ---------------------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16] and B[l/16][l%16];
// lane l receives D[4*(l/16) + v][l%16] in component v.
__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8*(l/16) + e] and
// B[8*(l/16) + e][l%16] for e = 0..7; D as for the f32 variant.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const uint16_t (&v)[8]) {
    u16x8 u;
    u[0] = v[0]; u[1] = v[1]; u[2] = v[2]; u[3] = v[3];
    u[4] = v[4]; u[5] = v[5]; u[6] = v[6]; u[7] = v[7];
    return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------------------- loads
// Four consecutive pixels w..w+3 of one image row `row` (a pointer to element 0 of
// the row), widened to float; pixels outside [0, W) and rows that are not valid
// read as zero.  `aligned4` promises that w is a multiple of 4 and the row start
// is 16-byte aligned for float (8-byte for bf16) so a single vector load is legal.
template <typename T>
__device__ __forceinline__ f32x4 load4_row(const T *__restrict__ row, int w, int W, bool row_ok,
                                           bool aligned4) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (!row_ok) return v;
    if (w >= 0 && w + 3 < W) {
        if constexpr (Elem<T>::is_bf16) {
            if (aligned4) {
                u16x4 u = *(const u16x4 *)(row + w);
                v[0] = bf16_bits_to_f32(u[0]); v[1] = bf16_bits_to_f32(u[1]);
                v[2] = bf16_bits_to_f32(u[2]); v[3] = bf16_bits_to_f32(u[3]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = bf16_bits_to_f32(row[w + k]);
            }
        } else {
            if (aligned4) {
                v = *(const f32x4 *)(row + w);
            } else {
                f32x4_a4 t = *(const f32x4_a4 *)(row + w);
                v = t;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int ww = w + k;
            if (ww >= 0 && ww < W) v[k] = Elem<T>::to_f32(row[ww]);
        }
    }
    return v;
}

typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// Four consecutive pixels w..w+3 of a row with no bounds checks, for the case the
// caller has shown (with wave-uniform tests) that every lane's run is in range:
// w + 3 < W, and w >= 0 (w >= 1 when a bf16 run starts at an odd column).
// `aligned4`: w % 4 == 0 and the row start is 16-byte (float) / 8-byte (bf16)
// aligned; `row_even`: the row start is 4-byte aligned (bf16 only); `odd`: w is
// odd (bf16 only; a wave-uniform property of the shift).
template <typename T>
__device__ __forceinline__ f32x4 load4_unchecked(const T *__restrict__ row, int w, bool aligned4, bool row_even,
                                                 bool odd) {
    f32x4 v;
    if constexpr (Elem<T>::is_bf16) {
        if (aligned4) {
            const u16x4 u = *(const u16x4 *)(row + w);
            v[0] = bf16_bits_to_f32(u[0]); v[1] = bf16_bits_to_f32(u[1]);
            v[2] = bf16_bits_to_f32(u[2]); v[3] = bf16_bits_to_f32(u[3]);
        } else if (row_even && !odd) {
            const u32x2_a4 d = *(const u32x2_a4 *)(row + w);
            v[0] = __uint_as_float(d[0] << 16); v[1] = __uint_as_float(d[0] & 0xffff0000u);
            v[2] = __uint_as_float(d[1] << 16); v[3] = __uint_as_float(d[1] & 0xffff0000u);
        } else if (row_even) {
            const u32x2_a4 d = *(const u32x2_a4 *)(row + w - 1);
            v[0] = __uint_as_float(d[0] & 0xffff0000u); v[1] = __uint_as_float(d[1] << 16);
            v[2] = __uint_as_float(d[1] & 0xffff0000u); v[3] = bf16_bits_to_f32(row[w + 3]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = bf16_bits_to_f32(row[w + k]);
        }
    } else {
        if (aligned4) {
            v = *(const f32x4 *)(row + w);
        } else {
            const f32x4_a4 t = *(const f32x4_a4 *)(row + w);
            v = t;
        }
    }
    return v;
}

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint16_t u16x8_a16 __attribute__((ext_vector_type(8), aligned(16)));

// Eight consecutive bf16 pixels w..w+7 of one row, widened to float; zero outside
// [0, W) or when !row_ok.  Uses one 16-byte load when the address allows it, else
// dword loads (realigned in registers), else element loads at the row ends.
__device__ __forceinline__ void load8_bf16_row(const bf16_t *__restrict__ row, int w, int W, bool row_ok,
                                               float (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
    if (!row_ok) return;
    const uintptr_t a = (uintptr_t)(row + w);
    if (w >= 0 && w + 7 < W && ((a & 3) == 0 || w >= 1)) {
        if ((a & 15) == 0) {
            const u16x8 u = *(const u16x8_a16 *)(row + w);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = bf16_bits_to_f32(u[k]);
        } else if ((a & 3) == 0) {
            const u32x4_a4 d = *(const u32x4_a4 *)(row + w);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = __uint_as_float(d[k] << 16);
                v[2 * k + 1] = __uint_as_float(d[k] & 0xffff0000u);
            }
        } else {
            // row + w - 1 is 4-byte aligned and w - 1 >= 0 lies in this row.
            const u32x4_a4 d = *(const u32x4_a4 *)(row + w - 1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = __uint_as_float(d[k] & 0xffff0000u);
                if (k < 3) v[2 * k + 1] = __uint_as_float(d[k + 1] << 16);
            }
            v[7] = bf16_bits_to_f32(row[w + 7]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int ww = w + k;
            if (ww >= 0 && ww < W) v[k] = bf16_bits_to_f32(row[ww]);
        }
    }
}

// A run of consecutive pixels of one row kept as loaded: four float32 values, or
// eight raw bfloat16 values (which feed a bf16 MFMA operand without conversion).
template <typename T> struct Run;
template <> struct Run<float> {
    static constexpr int RL = 4;
    f32x4 v;
    __device__ __forceinline__ float at(int k) const { return v[k]; }
    __device__ __forceinline__ void set_raw(int k, float e) { v[k] = e; }
    __device__ __forceinline__ static Run zero() { return Run{f32x4{0.f, 0.f, 0.f, 0.f}}; }
    // No bounds checks (caller: w >= 0, w + 3 < W).  `wal`: w % 4 == 0 with
    // 16-byte aligned rows.
    __device__ __forceinline__ static Run fast(const float *__restrict__ row, int w, bool wal, bool, bool) {
        return Run{load4_unchecked(row, w, wal, true, false)};
    }
    // Zero outside [0, W) or when !ok.  `al`: rows 16-byte aligned.
    __device__ __forceinline__ static Run checked(const float *__restrict__ row, int w, int W, bool ok, bool al) {
        return Run{load4_row(row, w, W, ok, al && ((w & 3) == 0))};
    }
};
template <> struct Run<bf16_t> {
    static constexpr int RL = 8;
    u16x8 v;
    __device__ __forceinline__ float at(int k) const { return bf16_bits_to_f32(v[k]); }
    __device__ __forceinline__ void set_raw(int k, bf16_t e) { v[k] = e; }
    __device__ __forceinline__ static Run zero() { return Run{u16x8{0, 0, 0, 0, 0, 0, 0, 0}}; }
    // No bounds checks (caller: w + 7 < W, and w >= 1 when w is odd).  `wal`: w % 8 == 0
    // with 16-byte aligned rows; `row_even`: 4-byte aligned rows; `odd`: w is odd.
    __device__ __forceinline__ static Run fast(const bf16_t *__restrict__ row, int w, bool wal, bool row_even,
                                               bool odd) {
        Run r;
        if (wal) {
            r.v = *(const u16x8_a16 *)(row + w);
        } else if (row_even && !odd) {
            r.v = __builtin_bit_cast(u16x8, *(const u32x4_a4 *)(row + w));
        } else if (row_even) {
            // dwords cover w-1 .. w+6; the last pixel comes on its own
            const u32x4_a4 d = *(const u32x4_a4 *)(row + w - 1);
            const uint32_t e = row[w + 7];
            u32x4_a4 o;
            o[0] = __builtin_amdgcn_alignbit(d[1], d[0], 16);
            o[1] = __builtin_amdgcn_alignbit(d[2], d[1], 16);
            o[2] = __builtin_amdgcn_alignbit(d[3], d[2], 16);
            o[3] = __builtin_amdgcn_alignbit(e, d[3], 16);
            r.v = __builtin_bit_cast(u16x8, o);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) r.v[k] = row[w + k];
        }
        return r;
    }
    // Zero outside [0, W) or when !ok; vector loads whenever the run is in range
    // (chosen by the run's address).
    __device__ __forceinline__ static Run checked(const bf16_t *__restrict__ row, int w, int W, bool ok, bool) {
        if (!ok) return zero();
        if (w >= 0 && w + 7 < W) {
            const uintptr_t a = (uintptr_t)(row + w);
            if ((a & 15) == 0) return fast(row, w, true, true, false);
            if ((a & 3) == 0) return fast(row, w, false, true, false);
            if (w >= 1) return fast(row, w, false, true, true);  // row + w - 1 is 4-byte aligned
        }
        Run r = zero();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int ww = w + k;
            if (ww >= 0 && ww < W) r.v[k] = row[ww];
        }
        return r;
    }
};

// VEC consecutive elements of a row as one vector register value (VEC = 1: scalar).
template <typename T, int VEC> struct VecOf;
template <> struct VecOf<float, 4> { typedef float type __attribute__((ext_vector_type(4))); };
template <> struct VecOf<float, 2> { typedef float type __attribute__((ext_vector_type(2))); };
template <> struct VecOf<float, 1> { typedef float type; };
template <> struct VecOf<bf16_t, 8> { typedef uint16_t type __attribute__((ext_vector_type(8))); };
template <> struct VecOf<bf16_t, 4> { typedef uint16_t type __attribute__((ext_vector_type(4))); };
template <> struct VecOf<bf16_t, 2> { typedef uint16_t type __attribute__((ext_vector_type(2))); };
template <> struct VecOf<bf16_t, 1> { typedef uint16_t type; };

template <typename V, typename T, int VEC>
__device__ __forceinline__ T lane_of(const V &v, int k) {
    if constexpr (VEC == 1) return v; else return v[k];
}
template <typename V, typename T, int VEC>
__device__ __forceinline__ void set_lane(V &v, int k, T val) {
    if constexpr (VEC == 1) v = val; else v[k] = val;
}

// Exact narrowing of a value that was widened from T (used for the x copy).
template <typename T> __device__ __forceinline__ T exact_narrow(float v);
template <> __device__ __forceinline__ float exact_narrow<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t exact_narrow<bf16_t>(float v) {
    return (bf16_t)(__float_as_uint(v) >> 16);
}

// Stage LDS rows [lr0, lr1) of a tile of one image plane: LDS row lr, column lc
// holds pixel (h0 - HALO + lr, w0 - PADC + lc), zero outside the image, as float
// (D = float) or as the input's own bits (D = T).  Rows are LW elements.  vec: four
// pixels per load, which needs W % 4 == 0, LW and w0 - PADC multiples of 4, and a
// plane base aligned to four elements.
template <typename D, typename T> __device__ __forceinline__ D lds_elem(float v) {
    if constexpr (sizeof(D) == sizeof(float)) return v;
    else return exact_narrow<T>(v);
}
template <typename T, typename D = float>
__device__ __forceinline__ void stage_rows(const T *__restrict__ p, int h0, int w0, int H, int W, int HALO, int PADC,
                                           int LW, int lr0, int lr1, D *__restrict__ dst, bool vec) {
    if (vec) {
        const int vpr = LW >> 2;
        const int nv = (lr1 - lr0) * vpr;
        for (int i = threadIdx.x; i < nv; i += blockDim.x) {
            const int q = i / vpr;
            const int cv = i - q * vpr;
            const int lr = lr0 + q;
            const int hh = h0 - HALO + lr;
            const bool ok = hh >= 0 && hh < H;
            const f32x4 v = load4_row(p + (int64_t)(ok ? hh : 0) * W, w0 - PADC + 4 * cv, W, ok, true);
            if constexpr (sizeof(D) == sizeof(float)) {
                *(f32x4 *)(dst + lr * LW + 4 * cv) = v;
            } else {
                u16x4 u;
#pragma unroll
                for (int k = 0; k < 4; ++k) u[k] = exact_narrow<T>(v[k]);
                *(u16x4 *)(dst + lr * LW + 4 * cv) = u;
            }
        }
    } else {
        const int n = (lr1 - lr0) * LW;
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int q = i / LW;
            const int lc = i - q * LW;
            const int lr = lr0 + q;
            const int hh = h0 - HALO + lr;
            const int ww = w0 - PADC + lc;
            float v = 0.f;
            if (hh >= 0 && hh < H && ww >= 0 && ww < W) v = Elem<T>::to_f32(p[(int64_t)hh * W + ww]);
            dst[lr * LW + lc] = lds_elem<D, T>(v);
        }
    }
}

// Raw (bit-exact) copy helpers for the x block of the output.
template <typename T>
__device__ __forceinline__ void copy4_row(const T *__restrict__ src, T *__restrict__ dst, int w, int W,
                                          bool aligned4) {
    if (w + 3 < W && aligned4) {
        if constexpr (Elem<T>::is_bf16) {
            *(u16x4 *)(dst + w) = *(const u16x4 *)(src + w);
        } else {
            *(f32x4 *)(dst + w) = *(const f32x4 *)(src + w);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (w + k < W) dst[w + k] = src[w + k];
    }
}

template <typename T>
__device__ __forceinline__ void store4_row(T *__restrict__ row, int w, int W, f32x4 v, bool aligned4) {
    if (w + 3 < W && aligned4) {
        if constexpr (Elem<T>::is_bf16) {
            u16x4 u;
            u[0] = f32_to_bf16_bits(v[0]); u[1] = f32_to_bf16_bits(v[1]);
            u[2] = f32_to_bf16_bits(v[2]); u[3] = f32_to_bf16_bits(v[3]);
            *(u16x4 *)(row + w) = u;
        } else {
            *(f32x4 *)(row + w) = v;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (w + k < W) row[w + k] = Elem<T>::from_f32(v[k]);
    }
}

}  // namespace ddpm

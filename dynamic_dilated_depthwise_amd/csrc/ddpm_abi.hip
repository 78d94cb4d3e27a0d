// ddpm_abi.hip -- the exported C ABI (include/ddpm.h): argument validation and
// dispatch to the gfx950 kernels.  Validation completes before anything is
// enqueued, so a rejected call has no effect.
#include <stdint.h>

#include "../../include/ddpm.h"
#include "launchers.hpp"

namespace {

bool bad_ptr(const void *p, int dtype) {
    if (p == nullptr) return true;
    const uintptr_t a = (uintptr_t)p;
    return dtype == DDPM_BF16 ? (a % 2) != 0 : (a % 4) != 0;
}

bool aligned16(const void *p) { return ((uintptr_t)p % 16) == 0; }

// Common shape checks.  Returns DDPM_OK or an error code.
int check_shape(int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype) {
    if (dtype != DDPM_F32 && dtype != DDPM_BF16) return DDPM_ERR_INVALID_ARG;
    if (N < 1 || C < 1 || H < 1 || W < 1) return DDPM_ERR_INVALID_ARG;
    if (C > DDPM_MAX_C) return DDPM_ERR_INVALID_ARG;
    if (H * W >= (int64_t(1) << 31)) return DDPM_ERR_INVALID_ARG;
    if (K != 1 && K != 3 && K != 5) return DDPM_ERR_UNSUPPORTED;
    // The largest tensor anywhere is the tap tensor, N * 3*C*K*K * H * W elements.
    const double elems = (double)N * 3.0 * (double)C * K * K * (double)H * (double)W;
    if (elems > 4.0e18) return DDPM_ERR_INVALID_ARG;
    if ((double)N * H * W >= 2147483648.0) return DDPM_ERR_INVALID_ARG;
    return DDPM_OK;
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// The launchers refuse, before enqueueing anything, grids beyond the hardware's
// workgroup-count limit with hipErrorInvalidConfiguration: that is a shape this
// library does not support, not a runtime failure.
int status_of(hipError_t e) {
    if (e == hipSuccess) return DDPM_OK;
    return e == hipErrorInvalidConfiguration ? DDPM_ERR_UNSUPPORTED : DDPM_ERR_HIP;
}

}  // namespace

extern "C" {

const char *ddpm_status_string(int status) {
    switch (status) {
        case DDPM_OK: return "DDPM_OK";
        case DDPM_ERR_INVALID_ARG: return "DDPM_ERR_INVALID_ARG";
        case DDPM_ERR_UNSUPPORTED: return "DDPM_ERR_UNSUPPORTED";
        case DDPM_ERR_HIP: return "DDPM_ERR_HIP";
        default: return "DDPM_ERR_UNKNOWN";
    }
}

int ddpm_filter_fwd(const void *x, const void *taps, void *out, int64_t N, int64_t C, int64_t H, int64_t W, int K,
                    int dtype, hipStream_t stream) {
    int st = check_shape(N, C, H, W, K, dtype);
    if (st != DDPM_OK) return st;
    if (bad_ptr(x, dtype) || bad_ptr(taps, dtype) || bad_ptr(out, dtype)) return DDPM_ERR_INVALID_ARG;
    const int64_t es = dtype == DDPM_BF16 ? 2 : 4;
    const int64_t HW = H * W;
    const int64_t R = 3 * C * K * K;
    if (overlaps(out, N * 4 * C * HW * es, x, N * C * HW * es) || overlaps(out, N * 4 * C * HW * es, taps, N * R * HW * es))
        return DDPM_ERR_INVALID_ARG;
    const bool bf16 = dtype == DDPM_BF16;
    // Runs of 4 pixels in both dtypes: for bfloat16 the 64-lane, 4-row tiles this gives
    // stream faster than 8-pixel runs (measured 48 vs 56 us at 1x64x256x256).
    int vec = 1;
    for (int v = 4; v > 1; v /= 2) {
        const uintptr_t al = (uintptr_t)v * es;
        if (W % v == 0 && (uintptr_t)x % al == 0 && (uintptr_t)taps % al == 0 && (uintptr_t)out % al == 0) {
            vec = v;
            break;
        }
    }
    (void)hipGetLastError();
    return status_of(ddpm::launch_filter_fwd(x, taps, out, (int)N, (int)C, (int)H, (int)W, K, bf16, vec, stream));
}

int ddpm_filter_bwd(const void *x, const void *taps, const void *grad_out, void *grad_x, void *grad_taps, int64_t N,
                    int64_t C, int64_t H, int64_t W, int K, int dtype, hipStream_t stream) {
    int st = check_shape(N, C, H, W, K, dtype);
    if (st != DDPM_OK) return st;
    if (bad_ptr(x, dtype) || bad_ptr(taps, dtype) || bad_ptr(grad_out, dtype)) return DDPM_ERR_INVALID_ARG;
    if (grad_x == nullptr && grad_taps == nullptr) return DDPM_ERR_INVALID_ARG;
    if ((grad_x != nullptr && bad_ptr(grad_x, dtype)) || (grad_taps != nullptr && bad_ptr(grad_taps, dtype)))
        return DDPM_ERR_INVALID_ARG;
    const int64_t es = dtype == DDPM_BF16 ? 2 : 4;
    const int64_t HW = H * W;
    const int64_t R = 3 * C * K * K;
    const int64_t xb = N * C * HW * es, tb = N * R * HW * es, gb = N * 4 * C * HW * es;
    const void *ins[3] = {x, taps, grad_out};
    const int64_t inb[3] = {xb, tb, gb};
    void *outs[2] = {grad_x, grad_taps};
    const int64_t outb[2] = {xb, tb};
    for (int o = 0; o < 2; ++o) {
        if (outs[o] == nullptr) continue;
        for (int i = 0; i < 3; ++i)
            if (overlaps(outs[o], outb[o], ins[i], inb[i])) return DDPM_ERR_INVALID_ARG;
    }
    if (grad_x != nullptr && grad_taps != nullptr && overlaps(grad_x, xb, grad_taps, tb)) return DDPM_ERR_INVALID_ARG;
    const bool bf16 = dtype == DDPM_BF16;
    int vec = 1;
    for (int v = bf16 ? 8 : 4; v > 1; v /= 2) {
        const uintptr_t a = (uintptr_t)v * es;
        if (W % v == 0 && (grad_x == nullptr || (uintptr_t)grad_x % a == 0) &&
            (grad_taps == nullptr || (uintptr_t)grad_taps % a == 0)) {
            vec = v;
            break;
        }
    }
    const bool al = (W % 4) == 0 && aligned16(taps);
    (void)hipGetLastError();
    return status_of(ddpm::launch_filter_bwd(x, taps, grad_out, grad_x, grad_taps, (int)N, (int)C, (int)H, (int)W, K,
                                             bf16, vec, al, stream));
}

int ddpm_fused_fwd(const void *x, const void *y, const void *weight, const void *bias, void *out, int64_t N,
                   int64_t C, int64_t H, int64_t W, int K, int dtype, hipStream_t stream) {
    int st = check_shape(N, C, H, W, K, dtype);
    if (st != DDPM_OK) return st;
    if (bad_ptr(x, dtype) || bad_ptr(y, dtype) || bad_ptr(weight, dtype) || bad_ptr(bias, dtype) ||
        bad_ptr(out, dtype))
        return DDPM_ERR_INVALID_ARG;
    const int64_t es = dtype == DDPM_BF16 ? 2 : 4;
    const int64_t HW = H * W;
    const int64_t R = 3 * C * K * K;
    const int64_t ob = N * 4 * C * HW * es;
    if (overlaps(out, ob, x, N * C * HW * es) || overlaps(out, ob, y, N * C * HW * es) ||
        overlaps(out, ob, weight, R * C * es) || overlaps(out, ob, bias, R * es))
        return DDPM_ERR_INVALID_ARG;
    const bool al = (W % 4) == 0 && aligned16(x) && aligned16(y) && aligned16(weight) && aligned16(out);
    (void)hipGetLastError();
    return status_of(ddpm::launch_fused_fwd(x, y, weight, bias, out, (int)N, (int)C, (int)H, (int)W, K,
                                            dtype == DDPM_BF16, al, stream));
}

int ddpm_fused_bwd(const void *x, const void *y, const void *weight, const void *bias, const void *grad_out,
                   void *grad_x, void *grad_y, float *dweight_partials, float *dbias_partials, int num_partials,
                   int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype, hipStream_t stream) {
    int st = check_shape(N, C, H, W, K, dtype);
    if (st != DDPM_OK) return st;
    if (bad_ptr(x, dtype) || bad_ptr(y, dtype) || bad_ptr(weight, dtype) || bad_ptr(bias, dtype) ||
        bad_ptr(grad_out, dtype))
        return DDPM_ERR_INVALID_ARG;
    const bool want_dx = grad_x != nullptr;
    const bool want_dy = grad_y != nullptr;
    if ((dweight_partials == nullptr) != (dbias_partials == nullptr)) return DDPM_ERR_INVALID_ARG;
    const bool want_dw = dweight_partials != nullptr;
    if (!want_dx && !want_dy && !want_dw) return DDPM_ERR_INVALID_ARG;
    if ((want_dx && bad_ptr(grad_x, dtype)) || (want_dy && bad_ptr(grad_y, dtype)) ||
        (want_dw && (bad_ptr(dweight_partials, DDPM_F32) || bad_ptr(dbias_partials, DDPM_F32))))
        return DDPM_ERR_INVALID_ARG;
    if (want_dw && (num_partials < 1 || num_partials > DDPM_MAX_PARTIALS)) return DDPM_ERR_INVALID_ARG;
    const int64_t es = dtype == DDPM_BF16 ? 2 : 4;
    const int64_t HW = H * W;
    const int64_t R = 3 * C * K * K;
    const int64_t xb = N * C * HW * es, gb = N * 4 * C * HW * es;
    const int64_t S = want_dw ? num_partials : 0;
    const int64_t pwb = S * R * C * 4, pbb = S * R * 4;
    const void *ins[5] = {x, y, weight, bias, grad_out};
    const int64_t inb[5] = {xb, xb, R * C * es, R * es, gb};
    void *outs[4] = {grad_x, grad_y, dweight_partials, dbias_partials};
    const int64_t outb[4] = {xb, xb, pwb, pbb};
    for (int o = 0; o < 4; ++o) {
        if (outs[o] == nullptr) continue;
        for (int i = 0; i < 5; ++i)
            if (overlaps(outs[o], outb[o], ins[i], inb[i])) return DDPM_ERR_INVALID_ARG;
        for (int p = o + 1; p < 4; ++p)
            if (outs[p] != nullptr && overlaps(outs[o], outb[o], outs[p], outb[p])) return DDPM_ERR_INVALID_ARG;
    }
    const bool al = (W % 4) == 0 && aligned16(x) && aligned16(y) && aligned16(weight) && aligned16(grad_out) &&
                    (!want_dx || aligned16(grad_x)) && (!want_dy || aligned16(grad_y));
    (void)hipGetLastError();
    return status_of(ddpm::launch_fused_bwd(x, y, weight, bias, grad_out, grad_x, grad_y, dweight_partials,
                                            dbias_partials, want_dw ? num_partials : 1, (int)N, (int)C, (int)H,
                                            (int)W, K, dtype == DDPM_BF16, al, stream));
}

int ddpm_reduce_partials(const float *dweight_partials, const float *dbias_partials, int num_partials,
                         void *grad_weight, void *grad_bias, int64_t C, int K, int dtype, hipStream_t stream) {
    if (dtype != DDPM_F32 && dtype != DDPM_BF16) return DDPM_ERR_INVALID_ARG;
    if (C < 1 || C > DDPM_MAX_C) return DDPM_ERR_INVALID_ARG;
    if (K != 1 && K != 3 && K != 5) return DDPM_ERR_UNSUPPORTED;
    if (num_partials < 1 || num_partials > DDPM_MAX_PARTIALS) return DDPM_ERR_INVALID_ARG;
    if (bad_ptr(dweight_partials, DDPM_F32) || bad_ptr(dbias_partials, DDPM_F32) || bad_ptr(grad_weight, dtype) ||
        bad_ptr(grad_bias, dtype))
        return DDPM_ERR_INVALID_ARG;
    const int64_t es = dtype == DDPM_BF16 ? 2 : 4;
    const int64_t R = 3 * C * K * K;
    const int64_t pwb = (int64_t)num_partials * R * C * 4, pbb = (int64_t)num_partials * R * 4;
    if (overlaps(grad_weight, R * C * es, dweight_partials, pwb) || overlaps(grad_weight, R * C * es, dbias_partials, pbb) ||
        overlaps(grad_bias, R * es, dweight_partials, pwb) || overlaps(grad_bias, R * es, dbias_partials, pbb) ||
        overlaps(grad_weight, R * C * es, grad_bias, R * es))
        return DDPM_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return status_of(ddpm::launch_reduce_partials(dweight_partials, dbias_partials, num_partials, grad_weight,
                                                  grad_bias, R, (int)C, dtype == DDPM_BF16, stream));
}

}  // extern "C"

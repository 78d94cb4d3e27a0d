// ddpm_abi.hip -- the exported C ABI (include/ddpm.h): argument validation and
// dispatch to the gfx950 kernels.  Validation completes before anything is
// enqueued, so a rejected call has no effect.
#include <stdint.h>

#include <mutex>

#include "../../include/ddpm.h"
#include "launchers.hpp"

// Device memory of ddpm_fused_bwd_noalloc: the float32 weight/bias partials live
// here instead of in a caller workspace.  Every GPU the library runs on holds its
// own copy (loaded with the code object) until the process ends.  In host code the
// name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, once per device (scratch_of_current_device).
static __device__ __align__(256) float scratch[DDPM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first call
// made with that device current and kept.  DDPM_OK or DDPM_ERR_HIP.
int scratch_of_current_device(float **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DDPM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DDPM_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float *>(g_scratch_ptr[dev]);
    return DDPM_OK;
}

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
        case DDPM_ERR_SCRATCH_LIMIT: return "DDPM_ERR_SCRATCH_LIMIT";
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
    // Runs of 4 pixels (16-byte float32 / 8-byte bfloat16 tap loads).  bfloat16 rows
    // of 256 pixels or more take runs of 8 (16-byte loads): measured 5.24 vs 5.07 TB/s
    // at 1x64x256x256, while at 128x128 the taller tiles they imply halve the
    // workgroup count and lose (3.77 vs 4.01 TB/s).
    int vec = 1;
    for (int v = bf16 && W >= 256 ? 8 : 4; v > 1; v /= 2) {
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

}  // extern "C"

namespace {

// Validation shared by ddpm_fused_bwd and ddpm_fused_bwd_noalloc: the inputs, the
// requested outputs (want_dw: the partials, of pwb / pbb bytes, are written) and
// their overlaps.  `al` receives the kernels' 16-byte alignment flag.
int check_fused_bwd(const void *x, const void *y, const void *weight, const void *bias, const void *grad_out,
                    void *grad_x, void *grad_y, void *out3, void *out4, int64_t b3, int64_t b4, bool want_dw,
                    int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype, bool *al) {
    int st = check_shape(N, C, H, W, K, dtype);
    if (st != DDPM_OK) return st;
    if (bad_ptr(x, dtype) || bad_ptr(y, dtype) || bad_ptr(weight, dtype) || bad_ptr(bias, dtype) ||
        bad_ptr(grad_out, dtype))
        return DDPM_ERR_INVALID_ARG;
    const bool want_dx = grad_x != nullptr;
    const bool want_dy = grad_y != nullptr;
    if (!want_dx && !want_dy && !want_dw) return DDPM_ERR_INVALID_ARG;
    if ((want_dx && bad_ptr(grad_x, dtype)) || (want_dy && bad_ptr(grad_y, dtype))) return DDPM_ERR_INVALID_ARG;
    const int64_t es = dtype == DDPM_BF16 ? 2 : 4;
    const int64_t HW = H * W;
    const int64_t R = 3 * C * K * K;
    const int64_t xb = N * C * HW * es, gb = N * 4 * C * HW * es;
    const void *ins[5] = {x, y, weight, bias, grad_out};
    const int64_t inb[5] = {xb, xb, R * C * es, R * es, gb};
    void *outs[4] = {grad_x, grad_y, want_dw ? out3 : nullptr, want_dw ? out4 : nullptr};
    const int64_t outb[4] = {xb, xb, b3, b4};
    for (int o = 0; o < 4; ++o) {
        if (outs[o] == nullptr) continue;
        for (int i = 0; i < 5; ++i)
            if (overlaps(outs[o], outb[o], ins[i], inb[i])) return DDPM_ERR_INVALID_ARG;
        for (int p = o + 1; p < 4; ++p)
            if (outs[p] != nullptr && overlaps(outs[o], outb[o], outs[p], outb[p])) return DDPM_ERR_INVALID_ARG;
    }
    *al = (W % 4) == 0 && aligned16(x) && aligned16(y) && aligned16(weight) && aligned16(grad_out) &&
          (!want_dx || aligned16(grad_x)) && (!want_dy || aligned16(grad_y));
    return DDPM_OK;
}

}  // namespace

extern "C" {

int ddpm_fused_bwd(const void *x, const void *y, const void *weight, const void *bias, const void *grad_out,
                   void *grad_x, void *grad_y, float *dweight_partials, float *dbias_partials, int num_partials,
                   int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype, hipStream_t stream) {
    if ((dweight_partials == nullptr) != (dbias_partials == nullptr)) return DDPM_ERR_INVALID_ARG;
    const bool want_dw = dweight_partials != nullptr;
    if (want_dw && (bad_ptr(dweight_partials, DDPM_F32) || bad_ptr(dbias_partials, DDPM_F32)))
        return DDPM_ERR_INVALID_ARG;
    if (want_dw && (num_partials < 1 || num_partials > DDPM_MAX_PARTIALS)) return DDPM_ERR_INVALID_ARG;
    const int64_t R = 3 * C * K * K;
    const int64_t S = want_dw ? num_partials : 0;
    bool al = false;
    const int st = check_fused_bwd(x, y, weight, bias, grad_out, grad_x, grad_y, dweight_partials, dbias_partials,
                                   S * R * C * 4, S * R * 4, want_dw, N, C, H, W, K, dtype, &al);
    if (st != DDPM_OK) return st;
    (void)hipGetLastError();
    return status_of(ddpm::launch_fused_bwd(x, y, weight, bias, grad_out, grad_x, grad_y, dweight_partials,
                                            dbias_partials, want_dw ? num_partials : 1, (int)N, (int)C, (int)H,
                                            (int)W, K, dtype == DDPM_BF16, al, stream));
}

int ddpm_fused_bwd_noalloc(const void *x, const void *y, const void *weight, const void *bias, const void *grad_out,
                           void *grad_x, void *grad_y, void *grad_weight, void *grad_bias, int num_partials,
                           int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype, hipStream_t stream) {
    if ((grad_weight == nullptr) != (grad_bias == nullptr)) return DDPM_ERR_INVALID_ARG;
    const bool want_dw = grad_weight != nullptr;
    if (want_dw && (bad_ptr(grad_weight, dtype) || bad_ptr(grad_bias, dtype))) return DDPM_ERR_INVALID_ARG;
    if (want_dw && (num_partials < 1 || num_partials > DDPM_MAX_PARTIALS)) return DDPM_ERR_INVALID_ARG;
    const int64_t es = dtype == DDPM_BF16 ? 2 : 4;
    const int64_t R = 3 * C * K * K;
    bool al = false;
    int st = check_fused_bwd(x, y, weight, bias, grad_out, grad_x, grad_y, grad_weight, grad_bias, R * C * es,
                             R * es, want_dw, N, C, H, W, K, dtype, &al);
    if (st != DDPM_OK) return st;
    // Partials of the weight at float 0, of the bias at the next 256-byte boundary.
    const int64_t S = want_dw ? num_partials : 0;
    const int64_t bias_off = (S * R * C + 63) / 64 * 64;
    if (want_dw && (bias_off + S * R) * (int64_t)sizeof(float) > (int64_t)DDPM_NOALLOC_SCRATCH_BYTES)
        return DDPM_ERR_SCRATCH_LIMIT;
    if (stream != nullptr && stream != hipStreamPerThread) {
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) return DDPM_ERR_HIP;
        if (cur != sdev) return DDPM_ERR_INVALID_ARG;
    }
    float *pw = nullptr, *pb = nullptr;
    if (want_dw) {
        float *base = nullptr;
        st = scratch_of_current_device(&base);
        if (st != DDPM_OK) return st;
        pw = base;
        pb = base + bias_off;
    }
    (void)hipGetLastError();
    st = status_of(ddpm::launch_fused_bwd(x, y, weight, bias, grad_out, grad_x, grad_y, pw, pb,
                                          want_dw ? num_partials : 1, (int)N, (int)C, (int)H, (int)W, K,
                                          dtype == DDPM_BF16, al, stream));
    if (st != DDPM_OK || !want_dw) return st;
    return status_of(ddpm::launch_reduce_partials(pw, pb, num_partials, grad_weight, grad_bias, R, (int)C,
                                                  dtype == DDPM_BF16, stream));
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

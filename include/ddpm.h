/*
 * ddpm.h -- C ABI of the MI355X (gfx950) library for the Dynamic Dilated Pyramid
 * Module (DDPM) of HDFNet (ECCV 2020).
 *
 * The operation (page "lartpang/DynamicConvolutionOperator", sections
 * "问题与目标" / problem and goal, "CUDA 动态过滤" / dynamic filter,
 * "CUDA 融合生成器推理" / fused generator inference and "CUDA Flash 式融合训练" /
 * flash-style fused training):
 *
 *   A 1x1 generator over guidance features y produces, at every pixel, K*K
 *   depthwise taps per channel for each of the dilations D = (1, 3, 5):
 *       T[n, o, p] = bias[o] + sum_c' weight[o, c'] * y[n, c', p]
 *   with generator channel o = (b*C + c)*K*K + t, branch b for dilation D_b,
 *   tap t = ki*K + kj.  Branch b of channel c at pixel p = (h, w) is
 *       O_b[n, c, h, w] = sum_t T[n, o, h, w] * x[n, c, h + (ki-r)*D_b, w + (kj-r)*D_b]
 *   with r = (K-1)/2 and x read as zero outside the image (zero padding
 *   D_b*r, stride 1).  The output is the concatenation [x, O_0, O_1, O_2]
 *   along channels, shape [N, 4C, H, W].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer is a DEVICE pointer to contiguous row-major memory
 *   owned by the caller: x, y, grad_x, grad_y are [N, C, H, W]; weight is
 *   [3*C*K*K, C]; bias is [3*C*K*K]; taps is [N, 3*C*K*K, H, W]; out and
 *   grad_out are [N, 4*C, H, W].  Tensors are in `dtype` unless stated; the
 *   weight-gradient partials are always float32.  The library never allocates,
 *   frees or synchronises; apart from the fixed device buffer of
 *   ddpm_fused_bwd_noalloc it keeps no state between calls.  Outputs must not
 *   overlap inputs or each other.  Every output element is written exactly once
 *   (nothing is accumulated into), so outputs need no zeroing.
 * Streams.  Work is enqueued on `stream` (0 = the null stream) and the call
 *   returns without waiting; faults inside kernels surface at the caller's next
 *   synchronisation.
 * Precision (page section "CUDA Flash 式融合训练", precision policy).  All sums
 *   are accumulated in float32.  float32 calls use full float32 matrix
 *   arithmetic (no reduced-precision operands).  bfloat16 calls round each
 *   generated tap to bfloat16 (round-to-nearest-even) before it is used, round
 *   each formed dK value to bfloat16 where it feeds a matrix product, and round
 *   every bfloat16 output once at the end.  The x block of `out` is a bit-exact
 *   copy of x.
 * Errors.  Every function validates all arguments before it enqueues anything;
 *   a call that fails validation writes nothing.
 *     DDPM_ERR_INVALID_ARG  a null pointer, a pointer not aligned to its element,
 *                           N, C, H or W < 1, H*W or N*H*W >= 2^31,
 *                           C > DDPM_MAX_C, an unknown dtype, an output that
 *                           overlaps another tensor of the call, or
 *                           num_partials outside [1, DDPM_MAX_PARTIALS];
 *     DDPM_ERR_UNSUPPORTED  K not in {1, 3, 5} (the dilation set is fixed), or a
 *                           shape whose grid exceeds 2^31 - 1 workgroups;
 *     DDPM_ERR_HIP          a HIP launch or attribute call failed;
 *     DDPM_ERR_SCRATCH_LIMIT (ddpm_fused_bwd_noalloc only) the partials do not
 *                           fit the library's fixed device buffer.
 *   No C++ exception crosses this interface.  Calls are re-entrant and
 *   thread-safe.
 */
#ifndef DDPM_H_
#define DDPM_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DDPM_F32 = 0, DDPM_BF16 = 1 } ddpm_dtype;

typedef enum {
    DDPM_OK = 0,
    DDPM_ERR_INVALID_ARG = -1,
    DDPM_ERR_UNSUPPORTED = -2,
    DDPM_ERR_HIP = -3,
    DDPM_ERR_SCRATCH_LIMIT = -4
} ddpm_status;

/* Largest depthwise channel count accepted. */
#define DDPM_MAX_C 1024
/* Largest number of float32 weight-gradient partials (page section
 * "CUDA Flash 式融合训练": tokens are split into at most 16 fp32 partials). */
#define DDPM_MAX_PARTIALS 16

/*
 * ddpm_filter_fwd -- dynamic dilated filter with materialised taps
 * (page section "CUDA 动态过滤": one pass serves dilations 1, 3 and 5 from one
 * spatial tile, float32 accumulation, output written directly as [x, d1, d3, d5]).
 *
 *   x    [N, C, H, W]            in   dtype
 *   taps [N, 3*C*K*K, H, W]      in   dtype, generator channel order as above
 *   out  [N, 4*C, H, W]          out  dtype
 *
 * Returns DDPM_OK or an error code from the list above.
 */
int ddpm_filter_fwd(const void *x, const void *taps, void *out,
                    int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype,
                    hipStream_t stream);

/*
 * ddpm_filter_bwd -- backward of the materialised filter (page section
 * "CUDA 动态过滤": the backward fuses dX and dK, the gradient of the dynamic
 * kernels, with no patch matrix).  With G = grad_out = [G_x, G_0, G_1, G_2]:
 *   grad_taps[n, o(b,c,t), p] = G_b[n, c, p] * x[n, c, p + d_bt]   (zero outside)
 *   grad_x[n, c, q] = G_x[n, c, q] + sum_{b,t} taps[n, o, q - d_bt] * G_b[n, c, q - d_bt]
 *
 *   x         [N, C, H, W]            in   dtype
 *   taps      [N, 3*C*K*K, H, W]      in   dtype
 *   grad_out  [N, 4*C, H, W]          in   dtype
 *   grad_x    [N, C, H, W]            out  dtype, or NULL (not computed)
 *   grad_taps [N, 3*C*K*K, H, W]      out  dtype, or NULL (not computed)
 * At least one output must be requested (else DDPM_ERR_INVALID_ARG).  bfloat16
 * outputs are rounded once from float32 products and sums.
 */
int ddpm_filter_bwd(const void *x, const void *taps, const void *grad_out, void *grad_x, void *grad_taps,
                    int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype, hipStream_t stream);

/*
 * ddpm_fused_fwd -- generator fused with the filter (page section
 * "CUDA 融合生成器推理": weight x y-tile -> taps -> consumed with shifted x; the
 * taps never reach global memory).
 *
 *   x, y    [N, C, H, W]         in   dtype
 *   weight  [3*C*K*K, C]         in   dtype
 *   bias    [3*C*K*K]            in   dtype
 *   out     [N, 4*C, H, W]       out  dtype
 */
int ddpm_fused_fwd(const void *x, const void *y, const void *weight, const void *bias,
                   void *out, int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype,
                   hipStream_t stream);

/*
 * ddpm_fused_bwd -- training backward with tap recompute (page section
 * "CUDA Flash 式融合训练"): dX recomputes the taps and gathers each dilation's
 * contribution; dY forms dK = shifted(x) * grad on chip and contracts it with
 * the generator weight; dWeight / dbias form dK on chip and reduce it over
 * space into float32 partials, one per contiguous token range.
 *
 *   x, y, weight, bias     in   as for ddpm_fused_fwd
 *   grad_out [N, 4*C, H, W]           in   dtype (dL/d out)
 *   grad_x   [N, C, H, W]             out  dtype (includes the x-block passthrough)
 *   grad_y   [N, C, H, W]             out  dtype
 *   dweight_partials [num_partials, 3*C*K*K, C]   out  float32
 *   dbias_partials   [num_partials, 3*C*K*K]      out  float32
 *   num_partials in [1, DDPM_MAX_PARTIALS]: the T = N*H*W tokens, in (n, h, w)
 *   order, are cut into num_partials contiguous ranges; range s starts at
 *   floor(T*s/num_partials) rounded down to a multiple of 64 tokens (float32) or
 *   128 tokens (bfloat16), the last ends at T (a range may be empty; its partial
 *   is zero); partial s holds the sum over range s.  Reduce them with
 *   ddpm_reduce_partials.  Which count is fastest depends on the grid; the
 *   Python binding's num_partials_for picks one.
 *   Optional outputs: grad_x may be NULL (dX is not computed), grad_y may be
 *   NULL (dY is not computed), and dweight_partials / dbias_partials may both be
 *   NULL (dWeight / dbias are not computed; then num_partials is ignored).  At
 *   least one of the three must be requested, and the two partial pointers must
 *   be both NULL or both non-NULL; otherwise DDPM_ERR_INVALID_ARG.  Each part
 *   runs as its own kernel, so requesting a subset does only that work.
 */
int ddpm_fused_bwd(const void *x, const void *y, const void *weight, const void *bias,
                   const void *grad_out, void *grad_x, void *grad_y,
                   float *dweight_partials, float *dbias_partials, int num_partials,
                   int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype,
                   hipStream_t stream);

/*
 * ddpm_reduce_partials -- the short second kernel of the split reduction
 * (page section "CUDA Flash 式融合训练"): sums the partials in ascending split
 * order in float32 and writes the gradients in `dtype`.
 *
 *   dweight_partials [num_partials, 3*C*K*K, C]  in   float32
 *   dbias_partials   [num_partials, 3*C*K*K]     in   float32
 *   grad_weight      [3*C*K*K, C]                out  dtype
 *   grad_bias        [3*C*K*K]                   out  dtype
 */
int ddpm_reduce_partials(const float *dweight_partials, const float *dbias_partials,
                         int num_partials, void *grad_weight, void *grad_bias,
                         int64_t C, int K, int dtype, hipStream_t stream);

/* Size of the device buffer inside the library that ddpm_fused_bwd_noalloc keeps its
 * partials in (one per GPU, held until the process ends). */
#define DDPM_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

/*
 * ddpm_fused_bwd_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * ddpm_fused_bwd followed by ddpm_reduce_partials, with the float32 partials kept
 * in a fixed buffer inside the library instead of a caller workspace.  The call
 * allocates and frees nothing and calls no allocating routine.
 *
 *   x, y, weight, bias, grad_out, grad_x, grad_y   as for ddpm_fused_bwd
 *   grad_weight [3*C*K*K, C]   out  dtype
 *   grad_bias   [3*C*K*K]      out  dtype
 *   num_partials in [1, DDPM_MAX_PARTIALS]: the token split, as for ddpm_fused_bwd.
 * The results equal those of ddpm_fused_bwd + ddpm_reduce_partials with the same
 * num_partials.  grad_x or grad_y may be NULL (skipped); grad_weight and grad_bias
 * are both NULL (skipped, num_partials ignored) or both non-NULL.
 * Limit: the partials take num_partials * (3*C*K*K*C + 3*C*K*K) floats (plus at
 * most 63 floats of alignment) of the DDPM_NOALLOC_SCRATCH_BYTES buffer; a larger
 * request returns DDPM_ERR_SCRATCH_LIMIT before anything is enqueued (C = 64 fits
 * up to K = 5 with 16 partials; use fewer partials or ddpm_fused_bwd beyond it).
 * `stream` must belong to the current device (else DDPM_ERR_INVALID_ARG).
 * Sharing: every call on one GPU uses that GPU's one buffer, so calls that may run
 * at the same time on one GPU (different streams, or host threads) race and give
 * wrong gradients; order them on one stream.  Each call writes every partial it
 * later reads, so nothing needs clearing between calls.
 */
int ddpm_fused_bwd_noalloc(const void *x, const void *y, const void *weight, const void *bias,
                           const void *grad_out, void *grad_x, void *grad_y,
                           void *grad_weight, void *grad_bias, int num_partials,
                           int64_t N, int64_t C, int64_t H, int64_t W, int K, int dtype,
                           hipStream_t stream);

/* Static, human-readable name of a ddpm_status value. */
const char *ddpm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DDPM_H_ */

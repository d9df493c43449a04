/*
 * nrm.h -- fused row-wise normalisation on AMD Instinct MI355X (gfx950): C ABI.
 *
 * Four operations over the last axis of a row-major array, each one HIP kernel launch:
 *   nrm_rms_norm      RMSNorm                      x / sqrt(mean(x^2) + eps) * w
 *   nrm_add_rms_norm  residual add + RMSNorm       h = x + r;  out = RMSNorm(h);  returns both
 *   nrm_layer_norm    LayerNorm                    (x - mean) / sqrt(var + eps) * w + b
 *   nrm_norm_rope     RMSNorm + rotary embedding   per [b, h, l] row, position offset + l
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array pointer is DEVICE memory on the current HIP device, owned by the
 *           caller, C-contiguous with the normalised axis innermost. The library allocates
 *           nothing and keeps no state beyond a thread-local error string.
 * Dtypes.   dtype is the storage type of the activations and of every output (x, r, out, h,
 *           cache). The weights w and b are stored either in dtype or in NRM_F32 (w_dtype);
 *           NRM_F32 activations take NRM_F32 weights. Arithmetic is fp32 with fp32
 *           accumulation for RMS statistics; results are rounded once, to nearest even.
 * Optional. w == NULL means the scalar 1 and b == NULL the scalar 0.
 * Scalars.  eps, base and scale are float (the pages hold them as f32 bit patterns).
 * Streams.  Work is enqueued on `stream` (NULL = the default stream) and is asynchronous:
 *           NRM_OK means "enqueued"; a device fault surfaces at the caller's next
 *           synchronisation with the stream.
 * Errors.   On any error the call returns a non-zero nrm_status, records a message for
 *           nrm_last_error(), and launches nothing and writes nothing. Argument errors
 *           are found on the host, before any HIP call. An empty call (zero rows, or
 *           B * H * L == 0) with valid dtypes and sizes is a successful no-op whatever the
 *           pointers (an empty torch tensor may have a NULL data pointer).
 * Aliasing. An output may be exactly the same array as an input where stated (in-place
 *           use); any other overlap between an output and another array is NRM_ERR_ALIAS.
 * Threads.  Calls are thread-safe.
 */
#ifndef NRM_H
#define NRM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { NRM_F32 = 0, NRM_BF16 = 1 } nrm_dtype;

typedef enum {
  NRM_OK = 0,
  NRM_ERR_NULL = 1,   /* a required pointer is NULL                                     */
  NRM_ERR_SHAPE = 2,  /* a size or position is out of range                             */
  NRM_ERR_DTYPE = 3,  /* an unsupported dtype or dtype combination                      */
  NRM_ERR_ALIAS = 4,  /* an output overlaps another array other than as allowed         */
  NRM_ERR_DEVICE = 5  /* the HIP runtime refused the launch                             */
} nrm_status;

/*
 * RMSNorm over the last axis.
 * Source: nuvec-core 0.5.0, enum fast::FastOp (docs.rs), variant RmsNorm -- x divided by the
 * root of (mean of x squared plus eps), times w; w is 1-D or the scalar 1; eps is an f32.
 * Layer defaults (nuvec-nn 0.4.0 layers.rs, RmsNorm::new): w all ones, eps 1e-5.
 *
 *   x      [rows, hidden] dtype, input
 *   w      [hidden] w_dtype, or NULL (= 1)
 *   out    [rows, hidden] dtype, output; may be exactly x (in place)
 *   rows   >= 0 (0: no-op);  hidden: 1 .. 2^31 - 1
 * Errors: NULL x/out -> NRM_ERR_NULL; bad sizes -> NRM_ERR_SHAPE; dtype not in
 * {NRM_F32, NRM_BF16} or w_dtype not in {dtype, NRM_F32} -> NRM_ERR_DTYPE; out partly
 * overlapping x, or overlapping w -> NRM_ERR_ALIAS; launch refused -> NRM_ERR_DEVICE.
 */
nrm_status nrm_rms_norm(const void* x, const void* w, void* out, int64_t rows, int64_t hidden,
                        float eps, nrm_dtype dtype, nrm_dtype w_dtype, hipStream_t stream);

/*
 * Residual add fused with RMSNorm; returns the normalised value and the new residual.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant AddRmsNorm -- h is x + r and the result is
 * RmsNorm of h; MinivLLM API reference "Layers", section LayerNorm, forward(x, residual):
 * the sum is normalised and also handed back as the residual of the next sub-layer.
 * h is x + r rounded to dtype, written in the same pass, and it is this rounded h that is
 * normalised (so out == nrm_rms_norm(h) and h is bit-exact: one fp32 add, one rounding).
 *
 *   x, r   [rows, hidden] dtype, inputs (may be the same array)
 *   w      [hidden] w_dtype, or NULL (= 1)
 *   out    [rows, hidden] dtype, output RMSNorm(h); may be exactly x or exactly r
 *   h_out  [rows, hidden] dtype, output x + r; may be exactly x or exactly r (in-place
 *          residual update); must not overlap out
 * Errors: as nrm_rms_norm; NULL r/h_out -> NRM_ERR_NULL; out overlapping h_out, or any
 * partial overlap with x or r -> NRM_ERR_ALIAS.
 */
nrm_status nrm_add_rms_norm(const void* x, const void* r, const void* w, void* out, void* h_out,
                            int64_t rows, int64_t hidden, float eps, nrm_dtype dtype,
                            nrm_dtype w_dtype, hipStream_t stream);

/*
 * LayerNorm over the last axis.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant LayerNorm -- (x - mean) / root(var + eps) *
 * w + b; w and b are 1-D or the scalars 1 and 0. nuvec-nn 0.4.0 layers.rs, LayerNorm:
 * affine by default; without_bias drops b (pass b = NULL); affine(false) drops both.
 * var is the biased (divide by hidden) variance about the mean. The row statistics and the
 * per-element (x - mean) * rstd * w + b are evaluated in fp64, so that results near zero
 * (where w * normalised x nearly cancels b) still round to within one unit of the last place.
 *
 *   x      [rows, hidden] dtype;  w, b [hidden] w_dtype or NULL;  out [rows, hidden] dtype,
 *          may be exactly x
 * Errors: as nrm_rms_norm (b may not overlap out either).
 */
nrm_status nrm_layer_norm(const void* x, const void* w, const void* b, void* out, int64_t rows,
                          int64_t hidden, float eps, nrm_dtype dtype, nrm_dtype w_dtype,
                          hipStream_t stream);

/*
 * NormRope: RMS-normalise each [b, h, l] row of x (all D features, times w), then rotate its
 * first dims features as a rotary position embedding at position offset + l.
 * Source: nuvec-core 0.5.0 fast::FastOp, variants NormRope (eps optional: none means no
 * normalisation; result returned as a new [B, H, L, D] array or written into a cache at the
 * rows' positions) and Rope (dims even; traditional rotates neighbouring pairs (2i, 2i+1),
 * otherwise the halves (i, i + dims/2); base and scale are f32, scale multiplies the
 * position; forward = 0 is the inverse rotation). nuvec-nn 0.4.0 layers.rs, Rope: defaults
 * half pairs, base 10000, scale 1; frequencies are computed, never loaded.
 * Formula (textbook RoPE, RoFormer section 3.2): theta_i = base^(-2i/dims), angle
 * a = scale * (offset + l) * theta_i, (u, v) -> (u cos a - v sin a, u sin a + v cos a);
 * the inverse uses -a. Angles and sin/cos are computed in the kernel in fp64; features at
 * index >= dims are normalised but not rotated.
 *
 *   x          [B, H, L, D] dtype, input
 *   w          [D] w_dtype, or NULL (= 1); ignored when normalize == 0
 *   out_or_cache
 *              cache == 0: [B, H, L, D] dtype output, may be exactly x;
 *              cache != 0: [B, H, cache_len, D] dtype; rows offset .. offset + L - 1 of each
 *              (b, h) are written, every other element is left untouched; must not overlap x
 *   normalize  0: rotation only (eps and w unused);  eps: added to the mean square
 *   dims       even, 0 <= dims <= D (0: normalisation only)
 *   traditional, base, scale, offset (>= 0), forward (0 = inverse) as above
 *   cache_len  used only with cache != 0; needs offset + L <= cache_len
 * Errors: NULL x/out_or_cache -> NRM_ERR_NULL; negative B/H/L/offset, D < 1, odd dims,
 * dims > D, offset + L > cache_len -> NRM_ERR_SHAPE; dtypes -> NRM_ERR_DTYPE; overlaps ->
 * NRM_ERR_ALIAS; launch refused -> NRM_ERR_DEVICE.
 */
nrm_status nrm_norm_rope(const void* x, const void* w, void* out_or_cache, int64_t B, int64_t H,
                         int64_t L, int64_t D, int normalize, float eps, int64_t dims,
                         int traditional, float base, float scale, int64_t offset, int forward,
                         int cache, int64_t cache_len, nrm_dtype dtype, nrm_dtype w_dtype,
                         hipStream_t stream);

/* The message of the last failed nrm_* call on this thread ("" if none): "<function>: <what>
 * <reason>, got <value>". Valid until the next nrm_* call on the same thread. */
const char* nrm_last_error(void);

/* Name of a status code ("NRM_OK", "NRM_ERR_SHAPE", ...). */
const char* nrm_status_name(nrm_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int nrm_version(void);

/*
 * Measurement helper, not one of the operations above: a plain copy of `bytes` bytes with
 * 16-byte loads and stores (src and dst device memory, 16-byte aligned, not overlapping).
 * Used as the achievable-bandwidth ceiling and to calibrate the hardware byte counters.
 * Errors: NULL -> NRM_ERR_NULL; bytes < 0 or not a multiple of 16 -> NRM_ERR_SHAPE;
 * misaligned or overlapping -> NRM_ERR_ALIAS.
 */
nrm_status nrm_bench_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NRM_H */

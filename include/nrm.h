/*
 * nrm.h -- fused row-wise normalisation on AMD Instinct MI355X (gfx950): C ABI.
 *
 Operations over the last axis of a row-major array:
 *   nrm_rms_norm        RMSNorm                     x / sqrt(mean(x^2) + eps) * w
 *   nrm_add_rms_norm    residual add + RMSNorm      h = x + r;  out = RMSNorm(h);  returns both
 *   nrm_layer_norm      LayerNorm                   (x - mean) / sqrt(var + eps) * w + b
 *   nrm_norm_rope       RMSNorm + rotary embedding  per [b, h, l] row, position offset + l
 *   nrm_rope            rotary embedding            per [n, l] row, position offset + l
 *   nrm_rope_positions  rotary embedding of query and key rows at per-token positions
 *   nrm_softmax         softmax                     exp(x - max) / sum, fp32 accumulation
 *   nrm_causal_softmax  softmax of causally masked scores (blocked attention mask)
 *   nrm_logsumexp       log(sum(exp(x)))            the last axis becomes size 1
 *   nrm_cross_entropy   logsumexp(logits) - logits[target], fp32 per row
 *   nrm_cross_entropy_vjp  its gradient for the logits
 *   nrm_rms_norm_vjp    RMSNorm backward            dx, dw from the output cotangent g
 *   nrm_layer_norm_vjp  LayerNorm backward          dx, dw, db from the output cotangent g
 * The forward operations are one HIP kernel launch each; the backward ones add a second,
 * small launch that sums the per-block parameter-gradient partials.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array pointer is DEVICE memory on the current HIP device, owned by the
 *           caller, C-contiguous with the normalised axis innermost. The library allocates
 *           nothing and keeps no state beyond a thread-local error string; the backward
 *           operations take their scratch space as a caller-provided workspace.
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
 *           pointers (an empty torch tensor may have a NULL data pointer), except that the
 *           backward operations set a requested dw / db to zero.
 * Aliasing. An output may be exactly the same array as an input where stated (in-place
 *           use); any other overlap between an output and another array is NRM_ERR_ALIAS.
 * Threads.  Calls are thread-safe.
 */
#ifndef NRM_H
#define NRM_H

#include <stddef.h>
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
 * position; forward = 0 is the inverse rotation; an optional freqs vector replaces base).
 * nuvec-nn 0.4.0 layers.rs, Rope: defaults half pairs, base 10000, scale 1.
 * Formula (textbook RoPE, RoFormer section 3.2): theta_i = base^(-2i/dims), or
 * theta_i = 1 / freqs[i] with freqs (freqs[i] divides the position, the convention of the
 * fast rope the pages name; the defaults correspond to freqs[i] = base^(2i/dims)), angle
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
 *   freqs      [dims / 2] fp32 device array, or NULL (use base); must not overlap the output
 *   cache_len  used only with cache != 0; needs offset + L <= cache_len
 * Errors: NULL x/out_or_cache -> NRM_ERR_NULL; negative B/H/L/offset, D < 1, odd dims,
 * dims > D, offset + L > cache_len -> NRM_ERR_SHAPE; dtypes -> NRM_ERR_DTYPE; overlaps ->
 * NRM_ERR_ALIAS; launch refused -> NRM_ERR_DEVICE.
 */
nrm_status nrm_norm_rope(const void* x, const void* w, void* out_or_cache, int64_t B, int64_t H,
                         int64_t L, int64_t D, int normalize, float eps, int64_t dims,
                         int traditional, float base, float scale, int64_t offset, int forward,
                         const float* freqs, int cache, int64_t cache_len, nrm_dtype dtype,
                         nrm_dtype w_dtype, hipStream_t stream);

/*
 * Rope: rotary position embedding of the first dims features of each row of x [N, L, D]
 * (N = the product of the leading axes), row l at position offset + l.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant Rope, inputs (x, offset[, freqs]), fields
 * dims, traditional, base, scale, forward; nuvec-nn 0.4.0 layers.rs, Rope (x as
 * [..., sequence, features], positions offset, offset + 1, ...; optionally scaled
 * frequencies, see nrm_rope_freqs_*). The rotation is NormRope's without the
 * normalisation; mscale multiplies the rotated features (the attention factor of YaRN and
 * LongRoPE scaling; 1 for plain RoPE). Features at index >= dims are copied.
 *
 *   x          [N, L, D] dtype, input;  out [N, L, D] dtype, may be exactly x
 *   freqs      [dims / 2] fp32 device array, or NULL (use base)
 * Errors: as nrm_norm_rope.
 */
nrm_status nrm_rope(const void* x, void* out, int64_t N, int64_t L, int64_t D, int64_t dims,
                    int traditional, float base, float scale, int64_t offset, int forward,
                    const float* freqs, float mscale, nrm_dtype dtype, hipStream_t stream);

/*
 * Rope on query and key rows at per-token positions, both tensors in one launch.
 * Source: MinivLLM API reference, "Layers", RotaryEmbedding: forward(positions, query, key)
 * rotates query [total_tokens, num_heads, head_dim] and key [total_tokens, num_kv_heads,
 * head_dim] for the 1-D integer positions of the tokens (batched [B, seq, heads, head_dim]
 * inputs are the same rows with T = B * seq and positions repeated per sequence), optionally
 * with Llama 3 frequency scaling (pass its freqs from nrm_rope_freqs_llama3). Every head of
 * token t turns at position positions[t]; otherwise as nrm_rope.
 *
 *   q          [T, Hq, D] dtype;  q_out [T, Hq, D], may be exactly q
 *   k          [T, Hk, D] dtype, or NULL when Hk == 0;  k_out likewise, may be exactly k
 *   positions  [T] int32 (pos_int64 == 0) or int64 (pos_int64 != 0) device array
 *   freqs      [dims / 2] fp32 device array, or NULL (use base)
 * Errors: as nrm_rope; NULL positions with T > 0 -> NRM_ERR_NULL.
 */
nrm_status nrm_rope_positions(const void* q, const void* k, void* q_out, void* k_out,
                              const void* positions, int pos_int64, int64_t T, int64_t Hq,
                              int64_t Hk, int64_t D, int64_t dims, int traditional, float base,
                              float scale, int forward, const float* freqs, float mscale,
                              nrm_dtype dtype, hipStream_t stream);

/*
 * Frequency scalings for long contexts: fill freqs_out (HOST memory, dims / 2 floats) with
 * the per-pair divisors to pass as `freqs`, and *mscale_out (when not NULL) with the factor
 * on the rotated features. All arithmetic is fp64, each divisor rounded once to fp32.
 * Source: nuvec-nn 0.4.0 layers.rs, Rope (Rope::scaled: mlx-lm's Llama3RoPE, YarnRoPE,
 * SuScaledRoPE, ProportionalRoPE; frequencies computed from the settings); the MinivLLM API
 * reference, RotaryEmbedding (Llama 3 settings and defaults). The formulas are those of the
 * published methods (the pages print none); ProportionalRoPE is not provided.
 * With f_i = base^(2i/dims):
 *   llama3  Meta's Llama 3.1 scaling: wavelength 2 pi f_i below original_max /
 *           high_freq_factor keeps f_i; above original_max / low_freq_factor gives
 *           factor * f_i; between, with s = (original_max / wavelength - low_freq_factor) /
 *           (high_freq_factor - low_freq_factor), f_i / ((1 - s) / factor + s). mscale 1.
 *   yarn    YaRN (Peng et al. 2023): a linear ramp over pair indices from
 *           floor(d(beta_fast)) to ceil(d(beta_slow)) (clamped to [0, dims - 1]),
 *           d(r) = dims ln(original_max / (2 pi r)) / (2 ln base), blends 1/f_i (below the
 *           ramp) into 1/(factor f_i) (above it); mscale = g(factor, mscale) /
 *           g(factor, mscale_all_dim), g(s, m) = 0.1 m ln s + 1 (1 for s <= 1).
 *   su      LongRoPE (Phi-3 "su" scaling): long_factor[i] * f_i (long_factor in HOST
 *           memory); mscale = sqrt(1 + ln(max_position / original_max) / ln(original_max)).
 * Errors: NULL outputs (or long_factor) -> NRM_ERR_NULL; dims < 2 or odd, base <= 1,
 * factor <= 0, a non-positive length or a low_freq_factor >= high_freq_factor ->
 * NRM_ERR_SHAPE. Host-only: no HIP call.
 */
nrm_status nrm_rope_freqs_llama3(int64_t dims, float base, float factor, float low_freq_factor,
                                 float high_freq_factor, int64_t original_max,
                                 float* freqs_out, float* mscale_out);
nrm_status nrm_rope_freqs_yarn(int64_t dims, float base, float factor, int64_t original_max,
                               float beta_fast, float beta_slow, float mscale,
                               float mscale_all_dim, float* freqs_out, float* mscale_out);
nrm_status nrm_rope_freqs_su(int64_t dims, float base, const float* long_factor,
                             int64_t max_position, int64_t original_max, float* freqs_out,
                             float* mscale_out);

/* The message of the last failed nrm_* call on this thread ("" if none): "<function>: <what>
 * <reason>, got <value>". Valid until the next nrm_* call on the same thread. */
const char* nrm_last_error(void);

/*
 * Workspace bytes that nrm_rms_norm_vjp (layer_norm = 0) or nrm_layer_norm_vjp
 * (layer_norm != 0) needs for `rows` rows of `hidden` features when a parameter gradient
 * (dw or db) is requested: P * hidden * 8 for RMSNorm and twice that for LayerNorm, where
 * P = ceil(rows / ceil(rows / 256)) <= 256 is the number of fp64 partial rows (one per
 * block of consecutive rows). 0 for rows <= 0 or hidden < 1. Depends on the shape only,
 * not on the device.
 */
size_t nrm_norm_vjp_workspace_bytes(int64_t rows, int64_t hidden, int layer_norm);

/*
 * RMSNorm backward: the gradients of RMSNorm (out = x / sqrt(mean(x^2) + eps) * w) for x and
 * for w, given the output cotangent g.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant RmsNormVjp, inputs (x, w, g), the gradients
 * of RmsNorm for x and w; eps an f32. Per row, with r = 1 / sqrt(sum(x^2) / D + eps):
 *   dx = r * g * w - x * r^3 * sum(g * w * x) / D,      dw = sum over rows of g * x * r.
 * Row sums accumulate in fp64, as do r, the per-element dx and the dw column sums (dx is a
 * difference that can cancel), so each result is within one unit of the last place of the
 * exact value. dw is the same bits on every run (fixed summation order).
 *
 *   x, g       [rows, hidden] dtype, inputs
 *   w          [hidden] w_dtype, or NULL (= 1)
 *   dx         [rows, hidden] dtype output; may be exactly x or exactly g
 *   dw         [hidden] w_dtype output, or NULL (not computed). With w == NULL it is the
 *              gradient for a weight of ones. For rows == 0 it is set to zero.
 *   workspace  device scratch of at least nrm_norm_vjp_workspace_bytes(rows, hidden, 0)
 *              bytes, 16-byte aligned, overlapping no other argument; contents on return
 *              are unspecified. Unused (may be NULL) when dw == NULL. Calls that share a
 *              workspace must be ordered (the same stream).
 * Errors: NULL x/g/dx (rows > 0), or NULL workspace with dw -> NRM_ERR_NULL; bad sizes or
 * workspace_bytes too small -> NRM_ERR_SHAPE; dtypes -> NRM_ERR_DTYPE; dx partly overlapping
 * x or g, any other overlap, or a misaligned workspace -> NRM_ERR_ALIAS; launch refused ->
 * NRM_ERR_DEVICE.
 */
nrm_status nrm_rms_norm_vjp(const void* x, const void* w, const void* g, void* dx, void* dw,
                            int64_t rows, int64_t hidden, float eps, nrm_dtype dtype,
                            nrm_dtype w_dtype, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * LayerNorm backward: the gradients of LayerNorm (out = (x - mean) / sqrt(var + eps) * w + b)
 * for x, w and b, given the output cotangent g.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant LayerNormVjp, inputs (x, w, b, g), the
 * gradients of LayerNorm for x, w and b; eps an f32. b does not enter any gradient, so it is
 * not an argument. Per row, with xh = (x - mean) * r, r = 1 / sqrt(var + eps) (biased
 * variance) and d = g * w:
 *   dx = r * (d - mean(d) - xh * mean(d * xh)),   dw = sum over rows of g * xh,
 *   db = sum over rows of g.
 * Row statistics, dx and the column sums are evaluated in fp64; each result is within one
 * unit of the last place of the exact value, and the same bits on every run.
 *
 *   x, g, w, dx as nrm_rms_norm_vjp
 *   dw, db     [hidden] w_dtype outputs, each may be NULL (not computed); zero for rows == 0
 *   workspace  at least nrm_norm_vjp_workspace_bytes(rows, hidden, 1) bytes when dw or db is
 *              requested, as for nrm_rms_norm_vjp
 * Errors: as nrm_rms_norm_vjp.
 */
nrm_status nrm_layer_norm_vjp(const void* x, const void* w, const void* g, void* dx, void* dw,
                              void* db, int64_t rows, int64_t hidden, float eps,
                              nrm_dtype dtype, nrm_dtype w_dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * nrm_layer_norm_vjp without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid it). The
 * fp64 partial column sums of dw and db go to a scratch array that the library holds in
 * device memory (32 MiB per GPU it runs on, kept until the process ends), not to a caller's
 * workspace; the call allocates nothing. Arguments, layout, results and errors are those of
 * nrm_layer_norm_vjp (the same kernels, the same bits), except:
 *   - rows x hidden may need at most 32 MiB of partial sums, i.e. hidden <= 8192 at any row
 *     count (with dw or db requested); beyond that -> NRM_ERR_SHAPE, nothing launched;
 *   - every call on one GPU shares that GPU's scratch: calls that may overlap on one GPU
 *     (different streams, different host threads) race and must be ordered by the caller;
 *     calls on one stream are ordered already. The scratch holds the last call's partial
 *     sums; each call writes every partial sum it reads, so nothing needs clearing.
 *   - the scratch's device address is looked up (hipGetSymbolAddress) on the first call on
 *     each device; failure there -> NRM_ERR_DEVICE.
 */
nrm_status nrm_layer_norm_vjp_noalloc(const void* x, const void* w, const void* g, void* dx,
                                      void* dw, void* db, int64_t rows, int64_t hidden,
                                      float eps, nrm_dtype dtype, nrm_dtype w_dtype,
                                      hipStream_t stream);

/*
 * Softmax over the last axis of x [rows, n]: out = exp(x - max) / sum(exp(x - max)).
 * Source: nuvec-core 0.5.0 fast::FastOp, variant Softmax ((x): softmax over the last axis,
 * accumulated in float32). Arithmetic fp32; the result is rounded once to dtype; every
 * element is within one unit in the last place (bf16) or 1e-5 relative + 1e-6 absolute
 * (fp32) of the exact value. NaN or +inf in a row makes the row NaN.
 *
 *   x, out     [rows, n] dtype; out may be exactly x
 * Errors: NULL x/out (rows > 0) -> NRM_ERR_NULL; rows < 0, n outside [1, 2^31) ->
 * NRM_ERR_SHAPE; dtype -> NRM_ERR_DTYPE; out partly overlapping x -> NRM_ERR_ALIAS.
 */
nrm_status nrm_softmax(const void* x, void* out, int64_t rows, int64_t n, nrm_dtype dtype,
                       hipStream_t stream);

/*
 * Softmax of causally masked scores x [N, R, L] (R a multiple of rows_per_block): row r of
 * the R axis keeps the columns c <= r % rows_per_block + L - rows_per_block; the other scores
 * are replaced by the dtype's lowest finite value (so they come out 0, unless a row keeps no
 * column at all: then every score is that value and the row is uniform).
 * Source: nuvec-core 0.5.0 fast::FastOp, variant CausalSoftmax (field rows: rows per block;
 * MLX's blocked attention mask). Otherwise as nrm_softmax.
 * Errors: as nrm_softmax; rows_per_block < 1 or R not a multiple of it -> NRM_ERR_SHAPE.
 */
nrm_status nrm_causal_softmax(const void* x, void* out, int64_t N, int64_t R, int64_t L,
                              int64_t rows_per_block, nrm_dtype dtype, hipStream_t stream);

/*
 * LogSumExp over the last axis: out[row] = log(sum_j exp(x[row, j])), computed as
 * max + log(sum exp(x - max)) in fp32 and rounded once to dtype.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant LogSumExp ((x): the last axis becomes
 * size 1).
 *   x [rows, n] dtype;  out [rows] dtype (the [rows, 1] result), must not overlap x
 * Errors: as nrm_softmax (out may not overlap x at all).
 */
nrm_status nrm_logsumexp(const void* x, void* out, int64_t rows, int64_t n, nrm_dtype dtype,
                         hipStream_t stream);

/*
 * Cross-entropy per row: loss[row] = logsumexp(logits[row]) - logits[row, targets[row]],
 * fp32. Computed as log1p(R / e_t) with e_t = exp(x_t - max) and R the sum of the other
 * columns' exp(x - max), so small losses keep their relative precision. A target outside
 * [0, V) gives NaN.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant CrossEntropy ((logits, targets):
 * logsumexp(logits) - logits[target] per row, in float32).
 *   logits     [rows, V] dtype
 *   targets    [rows] int32 (targets_int64 == 0) or int64 device array
 *   loss       [rows] fp32 output; must not overlap logits or targets
 * Errors: as nrm_softmax; NULL targets/loss -> NRM_ERR_NULL.
 */
nrm_status nrm_cross_entropy(const void* logits, const void* targets, int targets_int64,
                             float* loss, int64_t rows, int64_t V, nrm_dtype dtype,
                             hipStream_t stream);

/*
 * Gradient of nrm_cross_entropy for the logits: dlogits[row, j] = g[row] * (softmax(
 * logits[row])_j - [j == target]); the target's entry is formed as -g R / (R + e_t) (no
 * cancellation). Rounded once to dtype; a target outside [0, V) gives a NaN row.
 * Source: nuvec-core 0.5.0 fast::FastOp, variant CrossEntropyVjp ((logits, targets, loss,
 * g): the gradient of CrossEntropy for the logits).
 *   logits, targets as nrm_cross_entropy
 *   loss       [rows] fp32 forward output: accepted, not read (the kernel rebuilds the row's
 *              normaliser from the logits it reads anyway); may be NULL
 *   g          [rows] fp32 cotangent of the loss
 *   dlogits    [rows, V] dtype output; may be exactly logits
 * Errors: as nrm_cross_entropy; NULL g/dlogits -> NRM_ERR_NULL.
 */
nrm_status nrm_cross_entropy_vjp(const void* logits, const void* targets, int targets_int64,
                                 const float* loss, const float* g, void* dlogits,
                                 int64_t rows, int64_t V, nrm_dtype dtype, hipStream_t stream);

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

/*
 * Measurement helper, not one of the operations above: dst1 = src1 and dst2 = src2, `bytes`
 * bytes each, with one 16-byte load of each source and one 16-byte store of each destination
 * per thread, 512-thread blocks at two per compute unit (the fastest shape measured for this
 * pattern): the residual add-RMSNorm's byte pattern (two arrays in, two out) without
 * arithmetic, reported as that pattern's achievable-bandwidth ceiling. All four arrays are
 * device memory, 16-byte aligned; no destination may overlap a source or the other
 * destination (the two sources may overlap). Errors: NULL -> NRM_ERR_NULL; bytes < 0 or not
 * a multiple of 16 -> NRM_ERR_SHAPE; misaligned or overlapping -> NRM_ERR_ALIAS.
 */
nrm_status nrm_bench_copy2(const void* src1, const void* src2, void* dst1, void* dst2,
                           int64_t bytes, hipStream_t stream);

/*
 * Measurement helper, not one of the operations above: the copy of nrm_bench_copy2 (dst1 =
 * src1, dst2 = src2, `bytes` bytes each) in the shape of the row kernels' work unit. Each
 * 512-thread block copies one unit of `unit_bytes` of each source (unit_bytes / 8192 16-byte
 * chunks per thread, at chunks t, t + 512, ...), and a barrier after its loads keeps every
 * store of the block waiting until its whole unit has arrived, as a row's outputs wait for
 * the row's statistic. With unit_bytes = 16384 this is the residual add-RMSNorm's memory
 * traffic on [rows, 8192] bf16 rows (x and r read, out and h written) in its kernel's shape,
 * without the arithmetic: the ceiling of that access pattern, reported beside the pattern's
 * best copy (nrm_bench_copy2), whose blocks store each chunk as soon as it arrives.
 * unit_bytes is 8192, 16384 or 32768; bytes a multiple of it. Arrays and errors as
 * nrm_bench_copy2, and unit_bytes outside that set -> NRM_ERR_SHAPE.
 */
nrm_status nrm_bench_copy2_row(const void* src1, const void* src2, void* dst1, void* dst2,
                               int64_t bytes, int64_t unit_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NRM_H */

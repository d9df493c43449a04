// Frequency scalings of RoPE for long contexts, computed on the host: the per-pair divisors
// of the position passed to the rope kernels as `freqs`, and the factor on the rotated
// features. No HIP call.
//
// Sources: nuvec-nn 0.4.0 layers.rs docs, Rope (Rope::scaled: mlx-lm's Llama3RoPE,
// YarnRoPE, SuScaledRoPE; the frequencies are computed from the settings, never loaded);
// the MinivLLM API reference, "Layers", RotaryEmbedding (Llama 3 NTK-by-parts settings:
// factor, low_freq_factor, high_freq_factor, original_max_position_embeddings). The pages
// print no formula; each function follows the published method it names. All arithmetic is
// fp64 on the fp32 parameters; each divisor is rounded once to fp32.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "nrm.h"

namespace nrm {
void set_last_error(const char* msg);  // the thread-local message of nrm_last_error()
}

namespace {

constexpr double kTwoPi = 6.283185307179586;

nrm_status bad(nrm_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  nrm::set_last_error(buf);
  return code;
}

// Unscaled divisor of pair i: base^(2i/dims).
double period(double base, int64_t i, int64_t dims) {
  return std::pow(base, (double)(2 * i) / (double)dims);
}

nrm_status check_common(const char* fn, int64_t dims, float base, const float* out) {
  if (!out) return bad(NRM_ERR_NULL, "%s: freqs_out must not be NULL, got NULL", fn);
  if (dims < 2 || dims % 2 || dims > (int64_t)1 << 30)
    return bad(NRM_ERR_SHAPE, "%s: dims must be even and in [2, 2^30], got %lld", fn,
               (long long)dims);
  if (!(base > 1.f))
    return bad(NRM_ERR_SHAPE, "%s: base must be > 1, got %g", fn, (double)base);
  return NRM_OK;
}

}  // namespace

extern "C" {

// Meta's Llama 3.1 frequency scaling (NTK-by-parts).
nrm_status nrm_rope_freqs_llama3(int64_t dims, float base, float factor, float low_freq_factor,
                                 float high_freq_factor, int64_t original_max,
                                 float* freqs_out, float* mscale_out) {
  static const char* fn = "nrm_rope_freqs_llama3";
  nrm::set_last_error("");
  nrm_status st = check_common(fn, dims, base, freqs_out);
  if (st) return st;
  if (!(factor > 0.f))
    return bad(NRM_ERR_SHAPE, "%s: factor must be > 0, got %g", fn, (double)factor);
  if (!(low_freq_factor > 0.f) || !(high_freq_factor > low_freq_factor))
    return bad(NRM_ERR_SHAPE,
               "%s: need 0 < low_freq_factor < high_freq_factor, got %g and %g", fn,
               (double)low_freq_factor, (double)high_freq_factor);
  if (original_max < 1)
    return bad(NRM_ERR_SHAPE, "%s: original_max must be >= 1, got %lld", fn,
               (long long)original_max);
  const double orig = (double)original_max, lo = (double)low_freq_factor;
  const double hi = (double)high_freq_factor, fac = (double)factor;
  const double low_wavelen = orig / lo;    // longer wavelengths: fully scaled
  const double high_wavelen = orig / hi;   // shorter wavelengths: unchanged
  for (int64_t i = 0; i < dims / 2; ++i) {
    const double f = period((double)base, i, dims);
    const double wl = kTwoPi * f;
    double g = f;                                   // short wavelengths keep f
    if (wl > low_wavelen) {
      g = f * fac;                                  // long wavelengths: scaled by factor
    } else if (wl > high_wavelen && wl < low_wavelen) {
      const double s = (orig / wl - lo) / (hi - lo);  // 1 at the short edge, 0 at the long
      g = f / ((1.0 - s) / fac + s);
    }
    freqs_out[i] = (float)g;
  }
  if (mscale_out) *mscale_out = 1.f;
  return NRM_OK;
}

// YaRN: NTK-by-parts with a linear ramp over pair indices, and the attention factor.
nrm_status nrm_rope_freqs_yarn(int64_t dims, float base, float factor, int64_t original_max,
                               float beta_fast, float beta_slow, float mscale,
                               float mscale_all_dim, float* freqs_out, float* mscale_out) {
  static const char* fn = "nrm_rope_freqs_yarn";
  nrm::set_last_error("");
  nrm_status st = check_common(fn, dims, base, freqs_out);
  if (st) return st;
  if (!(factor > 0.f))
    return bad(NRM_ERR_SHAPE, "%s: factor must be > 0, got %g", fn, (double)factor);
  if (original_max < 1)
    return bad(NRM_ERR_SHAPE, "%s: original_max must be >= 1, got %lld", fn,
               (long long)original_max);
  if (!(beta_fast > 0.f) || !(beta_slow > 0.f))
    return bad(NRM_ERR_SHAPE, "%s: beta_fast and beta_slow must be > 0, got %g and %g", fn,
               (double)beta_fast, (double)beta_slow);
  const double b = (double)base, orig = (double)original_max, fac = (double)factor;
  // Pair index whose wavelength fits `turns` rotations in the original context.
  auto corr_dim = [&](double turns) {
    return (double)dims * std::log(orig / (turns * kTwoPi)) / (2.0 * std::log(b));
  };
  double low = std::floor(corr_dim((double)beta_fast));
  double high = std::ceil(corr_dim((double)beta_slow));
  if (low < 0.0) low = 0.0;
  if (high > (double)(dims - 1)) high = (double)(dims - 1);
  if (low == high) high += 0.001;
  for (int64_t i = 0; i < dims / 2; ++i) {
    const double f = period(b, i, dims);
    double ramp = ((double)i - low) / (high - low);
    ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
    const double keep = 1.0 - ramp;  // weight of the unscaled inverse frequency
    const double inv = keep / f + (1.0 - keep) / (fac * f);
    freqs_out[i] = (float)(1.0 / inv);
  }
  if (mscale_out) {
    auto g = [&](double m) { return fac <= 1.0 ? 1.0 : 0.1 * m * std::log(fac) + 1.0; };
    *mscale_out = (float)(g((double)mscale) / g((double)mscale_all_dim));
  }
  return NRM_OK;
}

// LongRoPE / Phi-3 "su" scaling.
nrm_status nrm_rope_freqs_su(int64_t dims, float base, const float* long_factor,
                             int64_t max_position, int64_t original_max, float* freqs_out,
                             float* mscale_out) {
  static const char* fn = "nrm_rope_freqs_su";
  nrm::set_last_error("");
  nrm_status st = check_common(fn, dims, base, freqs_out);
  if (st) return st;
  if (!long_factor) return bad(NRM_ERR_NULL, "%s: long_factor must not be NULL, got NULL", fn);
  if (original_max < 2 || max_position < 1)
    return bad(NRM_ERR_SHAPE,
               "%s: need original_max >= 2 and max_position >= 1, got %lld and %lld", fn,
               (long long)original_max, (long long)max_position);
  for (int64_t i = 0; i < dims / 2; ++i)
    freqs_out[i] = (float)((double)long_factor[i] * period((double)base, i, dims));
  if (mscale_out) {
    const double orig = (double)original_max;
    *mscale_out = (float)std::sqrt(1.0 + std::log((double)max_position / orig) / std::log(orig));
  }
  return NRM_OK;
}

}  // extern "C"

// C ABI of the row-wise normalisation library: argument validation, error reporting and
// dispatch to the kernel launchers. Every argument check runs on the host before any HIP
// call, so a failed call launches nothing and writes nothing.
//
// Error convention (after nuvec-nn's layers: an invalid argument gives a failure that names
// the operation and states what was wrong, as Dropout does for a probability outside
// [0, 1)): a non-zero nrm_status plus a thread-local message
// "<function>: <argument> <reason>, got <value>".
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "launch.hpp"
#include "nrm.h"
#include "rope.hpp"
#include "softmax.hpp"
#include "vjp.hpp"

namespace {

thread_local std::string g_err;

nrm_status fail(nrm_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int64_t esize(nrm_dtype d) { return d == NRM_BF16 ? 2 : 4; }

struct Span {  // [lo, lo + bytes)
  uintptr_t lo;
  uintptr_t bytes;
};
Span span(const void* p, int64_t bytes) { return Span{(uintptr_t)p, (uintptr_t)bytes}; }
bool overlap(Span a, Span b) {
  return a.bytes > 0 && b.bytes > 0 && a.lo < b.lo + b.bytes && b.lo < a.lo + a.bytes;
}
bool same(Span a, Span b) { return a.lo == b.lo && a.bytes == b.bytes; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

nrm_status check_dtypes(const char* fn, nrm_dtype dtype, nrm_dtype w_dtype) {
  if (dtype != NRM_F32 && dtype != NRM_BF16)
    return fail(NRM_ERR_DTYPE, "%s: dtype must be NRM_F32 (0) or NRM_BF16 (1), got %d", fn,
                (int)dtype);
  if (w_dtype != dtype && w_dtype != NRM_F32)
    return fail(NRM_ERR_DTYPE,
                "%s: w_dtype must equal dtype (%d) or be NRM_F32 (0), got %d", fn, (int)dtype,
                (int)w_dtype);
  return NRM_OK;
}

nrm_status check_rows(const char* fn, int64_t rows, int64_t hidden, nrm_dtype dtype) {
  if (rows < 0) return fail(NRM_ERR_SHAPE, "%s: rows must be >= 0, got %lld", fn, (long long)rows);
  if (hidden < 1 || hidden > INT32_MAX)
    return fail(NRM_ERR_SHAPE, "%s: hidden must be in [1, 2147483647], got %lld", fn,
                (long long)hidden);
  if (rows > 0 && rows > INT64_MAX / hidden / esize(dtype))
    return fail(NRM_ERR_SHAPE, "%s: rows * hidden overflows the address range, got %lld x %lld",
                fn, (long long)rows, (long long)hidden);
  return NRM_OK;
}

// An output must either be exactly `in` (when allowed) or not overlap it at all.
nrm_status check_out_vs(const char* fn, const char* out_name, Span out, const char* in_name,
                        Span in, bool exact_ok) {
  if (!overlap(out, in)) return NRM_OK;
  if (exact_ok && same(out, in)) return NRM_OK;
  return fail(NRM_ERR_ALIAS, "%s: %s must %s %s, got a %s overlap", fn, out_name,
              exact_ok ? "be exactly or not overlap" : "not overlap", in_name,
              same(out, in) ? "full" : "partial");
}

// Rope arguments with no second tensor, no positions array, no freqs and mscale 1.
nrm::RopeArgs rope_defaults() {
  nrm::RopeArgs a;
  a.x = a.w = a.x2 = nullptr;
  a.out = a.out2 = nullptr;
  a.BH = a.BH1 = a.L = 0;
  a.x_sbh = a.x_sl = a.o_sbh = a.o_sl = a.o_row0 = 0;
  a.x2_sbh = a.x2_sl = a.o2_sbh = a.o2_sl = 0;
  a.D = a.dims = 0;
  a.normalize = 0; a.eps = 0.f; a.traditional = 0; a.base = 10000.f; a.scale = 1.f;
  a.offset = 0; a.forward = 1; a.freqs = nullptr; a.positions = nullptr; a.pos_i64 = 0;
  a.mscale = 1.f; a.w_f32 = 0; a.iters = 1;
  return a;
}

// Checks shared by the rope entry points: D, dims (even, <= D).
nrm_status check_rope_dims(const char* fn, int64_t D, int64_t dims) {
  if (D < 1 || D > INT32_MAX)
    return fail(NRM_ERR_SHAPE, "%s: D must be in [1, 2147483647], got %lld", fn, (long long)D);
  if (dims < 0 || dims > D)
    return fail(NRM_ERR_SHAPE, "%s: dims must be in [0, D = %lld], got %lld", fn, (long long)D,
                (long long)dims);
  if (dims % 2) return fail(NRM_ERR_SHAPE, "%s: dims must be even, got %lld", fn, (long long)dims);
  return NRM_OK;
}

nrm_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(NRM_ERR_DEVICE, "%s: kernel launch failed: %s, got HIP error %d", fn,
                hipGetErrorString(e), (int)e);
  return NRM_OK;
}

nrm::RowArgs row_args(const void* x, const void* r, const void* w, const void* b, void* out,
                      void* h, int64_t rows, int64_t hidden, float eps, nrm_dtype w_dtype) {
  nrm::RowArgs a;
  a.x = x; a.r = r; a.w = w; a.b = b; a.out = out; a.h = h;
  a.rows = rows; a.hidden = hidden; a.eps = eps;
  a.w_f32 = w_dtype == NRM_F32;
  a.inv_n = hidden > 0 ? 1.0 / (double)hidden : 0.0;
  return a;
}

template <int OP>
hipError_t dispatch_row(const nrm::RowArgs& a, nrm_dtype dtype, bool al, hipStream_t s) {
  return dtype == NRM_BF16 ? nrm::launch_row<true, OP>(a, al, s)
                           : nrm::launch_row<false, OP>(a, al, s);
}

}  // namespace

namespace nrm {
void set_last_error(const char* msg) { g_err = msg; }
}  // namespace nrm

extern "C" {

nrm_status nrm_rms_norm(const void* x, const void* w, void* out, int64_t rows, int64_t hidden,
                        float eps, nrm_dtype dtype, nrm_dtype w_dtype, hipStream_t stream) {
  static const char* fn = "nrm_rms_norm";
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, w_dtype);
  if (st) return st;
  if ((st = check_rows(fn, rows, hidden, dtype))) return st;
  if (rows == 0) return NRM_OK;  // empty: nothing to read or write, any pointers accepted
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!out) return fail(NRM_ERR_NULL, "%s: out must not be NULL, got NULL", fn);
  const int64_t nb = rows * hidden * esize(dtype);
  const Span sx = span(x, nb), so = span(out, nb), sw = span(w, w ? hidden * esize(w_dtype) : 0);
  if ((st = check_out_vs(fn, "out", so, "x", sx, true))) return st;
  if ((st = check_out_vs(fn, "out", so, "w", sw, false))) return st;
  const bool al = aligned16(x) && aligned16(out) && (!w || aligned16(w));
  const nrm::RowArgs a = row_args(x, nullptr, w, nullptr, out, nullptr, rows, hidden, eps, w_dtype);
  return launched(fn, dispatch_row<nrm::OP_RMS>(a, dtype, al, stream));
}

nrm_status nrm_add_rms_norm(const void* x, const void* r, const void* w, void* out, void* h_out,
                            int64_t rows, int64_t hidden, float eps, nrm_dtype dtype,
                            nrm_dtype w_dtype, hipStream_t stream) {
  static const char* fn = "nrm_add_rms_norm";
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, w_dtype);
  if (st) return st;
  if ((st = check_rows(fn, rows, hidden, dtype))) return st;
  if (rows == 0) return NRM_OK;  // empty: nothing to read or write, any pointers accepted
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!r) return fail(NRM_ERR_NULL, "%s: r must not be NULL, got NULL", fn);
  if (!out) return fail(NRM_ERR_NULL, "%s: out must not be NULL, got NULL", fn);
  if (!h_out) return fail(NRM_ERR_NULL, "%s: h_out must not be NULL, got NULL", fn);
  const int64_t nb = rows * hidden * esize(dtype);
  const Span sx = span(x, nb), sr = span(r, nb), so = span(out, nb), sh = span(h_out, nb);
  const Span sw = span(w, w ? hidden * esize(w_dtype) : 0);
  if ((st = check_out_vs(fn, "out", so, "h_out", sh, false))) return st;
  if ((st = check_out_vs(fn, "out", so, "x", sx, true))) return st;
  if ((st = check_out_vs(fn, "out", so, "r", sr, true))) return st;
  if ((st = check_out_vs(fn, "h_out", sh, "x", sx, true))) return st;
  if ((st = check_out_vs(fn, "h_out", sh, "r", sr, true))) return st;
  if ((st = check_out_vs(fn, "out", so, "w", sw, false))) return st;
  if ((st = check_out_vs(fn, "h_out", sh, "w", sw, false))) return st;
  const bool al = aligned16(x) && aligned16(r) && aligned16(out) && aligned16(h_out) &&
                  (!w || aligned16(w));
  const nrm::RowArgs a = row_args(x, r, w, nullptr, out, h_out, rows, hidden, eps, w_dtype);
  return launched(fn, dispatch_row<nrm::OP_ADD_RMS>(a, dtype, al, stream));
}

nrm_status nrm_layer_norm(const void* x, const void* w, const void* b, void* out, int64_t rows,
                          int64_t hidden, float eps, nrm_dtype dtype, nrm_dtype w_dtype,
                          hipStream_t stream) {
  static const char* fn = "nrm_layer_norm";
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, w_dtype);
  if (st) return st;
  if ((st = check_rows(fn, rows, hidden, dtype))) return st;
  if (rows == 0) return NRM_OK;  // empty: nothing to read or write, any pointers accepted
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!out) return fail(NRM_ERR_NULL, "%s: out must not be NULL, got NULL", fn);
  const int64_t nb = rows * hidden * esize(dtype);
  const int64_t pb = hidden * esize(w_dtype);
  const Span sx = span(x, nb), so = span(out, nb);
  const Span sw = span(w, w ? pb : 0), sb = span(b, b ? pb : 0);
  if ((st = check_out_vs(fn, "out", so, "x", sx, true))) return st;
  if ((st = check_out_vs(fn, "out", so, "w", sw, false))) return st;
  if ((st = check_out_vs(fn, "out", so, "b", sb, false))) return st;
  const bool al = aligned16(x) && aligned16(out) && (!w || aligned16(w)) && (!b || aligned16(b));
  const nrm::RowArgs a = row_args(x, nullptr, w, b, out, nullptr, rows, hidden, eps, w_dtype);
  return launched(fn, dispatch_row<nrm::OP_LN>(a, dtype, al, stream));
}

nrm_status nrm_norm_rope(const void* x, const void* w, void* out_or_cache, int64_t B, int64_t H,
                         int64_t L, int64_t D, int normalize, float eps, int64_t dims,
                         int traditional, float base, float scale, int64_t offset, int forward,
                         const float* freqs, int cache, int64_t cache_len, nrm_dtype dtype,
                         nrm_dtype w_dtype, hipStream_t stream) {
  static const char* fn = "nrm_norm_rope";
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, w_dtype);
  if (st) return st;
  if (B < 0) return fail(NRM_ERR_SHAPE, "%s: B must be >= 0, got %lld", fn, (long long)B);
  if (H < 0) return fail(NRM_ERR_SHAPE, "%s: H must be >= 0, got %lld", fn, (long long)H);
  if (L < 0) return fail(NRM_ERR_SHAPE, "%s: L must be >= 0, got %lld", fn, (long long)L);
  if ((st = check_rope_dims(fn, D, dims))) return st;
  if (offset < 0)
    return fail(NRM_ERR_SHAPE, "%s: offset must be >= 0, got %lld", fn, (long long)offset);
  if (cache) {
    if (cache_len < 0 || L > cache_len || offset > cache_len - L)
      return fail(NRM_ERR_SHAPE, "%s: offset + L must be <= cache_len (%lld), got %lld + %lld", fn,
                  (long long)cache_len, (long long)offset, (long long)L);
  }
  // Sizes in bytes, guarding against overflow of B * H * rows * D * element size.
  const int64_t es = esize(dtype);
  const int64_t out_rows = cache ? cache_len : L;
  const int64_t lim = INT64_MAX / es / D;
  if ((B && H > lim / B) || (B && H && L > lim / (B * H)) || (B && H && out_rows > lim / (B * H)))
    return fail(NRM_ERR_SHAPE, "%s: B * H * L * D overflows the address range, got %lld x %lld", fn,
                (long long)B, (long long)H);
  const int64_t BH = B * H;
  if (BH * L == 0) return NRM_OK;  // empty: nothing to read or write
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!out_or_cache) return fail(NRM_ERR_NULL, "%s: out_or_cache must not be NULL, got NULL", fn);
  const Span sx = span(x, BH * L * D * es), so = span(out_or_cache, BH * out_rows * D * es);
  const Span sw = span(w, w ? D * esize(w_dtype) : 0);
  const Span sf = span(freqs, freqs ? dims / 2 * 4 : 0);
  if ((st = check_out_vs(fn, cache ? "cache" : "out", so, "x", sx, !cache))) return st;
  if ((st = check_out_vs(fn, cache ? "cache" : "out", so, "w", sw, false))) return st;
  if ((st = check_out_vs(fn, cache ? "cache" : "out", so, "freqs", sf, false))) return st;

  nrm::RopeArgs a = rope_defaults();
  a.x = x; a.w = w; a.out = out_or_cache;
  a.BH = a.BH1 = BH; a.L = L; a.D = (int)D; a.dims = (int)dims;
  a.x_sbh = L; a.x_sl = 1;
  a.o_sbh = out_rows; a.o_sl = 1; a.o_row0 = cache ? offset : 0;
  a.normalize = normalize != 0; a.eps = eps; a.traditional = traditional != 0;
  a.base = base; a.scale = scale; a.offset = offset; a.forward = forward != 0;
  a.freqs = freqs;
  a.w_f32 = w_dtype == NRM_F32;
  const bool al = aligned16(x) && aligned16(out_or_cache) && (!w || aligned16(w));
  return launched(fn, dtype == NRM_BF16 ? nrm::launch_norm_rope<true>(a, al, stream)
                                        : nrm::launch_norm_rope<false>(a, al, stream));
}

size_t nrm_norm_vjp_workspace_bytes(int64_t rows, int64_t hidden, int layer_norm) {
  if (rows <= 0 || hidden < 1 || hidden > INT32_MAX) return 0;
  return (size_t)nrm::vjp_partials(rows) * (size_t)hidden * sizeof(double) *
         (layer_norm ? 2 : 1);
}

}  // extern "C"

namespace {

// Shared by the two backward entry points; db is always NULL for RMSNorm.
nrm_status norm_vjp(const char* fn, bool ln, const void* x, const void* w, const void* g,
                    void* dx, void* dw, void* db, int64_t rows, int64_t hidden, float eps,
                    nrm_dtype dtype, nrm_dtype w_dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, w_dtype);
  if (st) return st;
  if ((st = check_rows(fn, rows, hidden, dtype))) return st;
  const int64_t pb = hidden * esize(w_dtype);
  const Span sw = span(w, w ? pb : 0), sdw = span(dw, dw ? pb : 0), sdb = span(db, db ? pb : 0);
  if ((st = check_out_vs(fn, "dw", sdw, "w", sw, false))) return st;
  if ((st = check_out_vs(fn, "db", sdb, "w", sw, false))) return st;
  if ((st = check_out_vs(fn, "db", sdb, "dw", sdw, false))) return st;
  nrm::VjpArgs a;
  a.x = x; a.w = w; a.g = g; a.dx = dx;
  a.part_w = a.part_b = nullptr;
  a.rows = rows; a.hidden = hidden; a.rpb = 1; a.eps = eps; a.inv_n = 1.0 / (double)hidden;
  a.w_f32 = w_dtype == NRM_F32; a.team = 64;
  auto go = [&](bool al) {
    if (ln)
      return dtype == NRM_BF16 ? nrm::launch_vjp<true, nrm::VJP_LN>(a, dw, db, al, stream)
                               : nrm::launch_vjp<false, nrm::VJP_LN>(a, dw, db, al, stream);
    return dtype == NRM_BF16 ? nrm::launch_vjp<true, nrm::VJP_RMS>(a, dw, db, al, stream)
                             : nrm::launch_vjp<false, nrm::VJP_RMS>(a, dw, db, al, stream);
  };
  if (rows == 0) return launched(fn, go(false));  // only zeroes dw / db
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!g) return fail(NRM_ERR_NULL, "%s: g must not be NULL, got NULL", fn);
  if (!dx) return fail(NRM_ERR_NULL, "%s: dx must not be NULL, got NULL", fn);
  const int64_t nb = rows * hidden * esize(dtype);
  const Span sx = span(x, nb), sg = span(g, nb), sdx = span(dx, nb);
  if ((st = check_out_vs(fn, "dx", sdx, "x", sx, true))) return st;
  if ((st = check_out_vs(fn, "dx", sdx, "g", sg, true))) return st;
  if ((st = check_out_vs(fn, "dx", sdx, "w", sw, false))) return st;
  if ((st = check_out_vs(fn, "dw", sdw, "x", sx, false))) return st;
  if ((st = check_out_vs(fn, "dw", sdw, "g", sg, false))) return st;
  if ((st = check_out_vs(fn, "dw", sdw, "dx", sdx, false))) return st;
  if ((st = check_out_vs(fn, "db", sdb, "x", sx, false))) return st;
  if ((st = check_out_vs(fn, "db", sdb, "g", sg, false))) return st;
  if ((st = check_out_vs(fn, "db", sdb, "dx", sdx, false))) return st;
  if (dw || db) {
    const size_t need = nrm_norm_vjp_workspace_bytes(rows, hidden, ln ? 1 : 0);
    if (!workspace) return fail(NRM_ERR_NULL, "%s: workspace must not be NULL, got NULL", fn);
    if (workspace_bytes < need)
      return fail(NRM_ERR_SHAPE, "%s: workspace_bytes must be >= %zu, got %zu", fn, need,
                  workspace_bytes);
    if (!aligned16(workspace))
      return fail(NRM_ERR_ALIAS, "%s: workspace must be 16-byte aligned, got %p", fn, workspace);
    const Span sws = span(workspace, (int64_t)need);
    const char* names[] = {"x", "g", "w", "dx", "dw", "db"};
    const Span spans[] = {sx, sg, sw, sdx, sdw, sdb};
    for (int i = 0; i < 6; ++i)
      if ((st = check_out_vs(fn, "workspace", sws, names[i], spans[i], false))) return st;
    a.part_w = (double*)workspace;
    if (ln) a.part_b = a.part_w + nrm::vjp_partials(rows) * hidden;
  }
  const bool al = aligned16(x) && aligned16(g) && aligned16(dx) && (!w || aligned16(w));
  return launched(fn, go(al));
}

}  // namespace

extern "C" {

nrm_status nrm_rms_norm_vjp(const void* x, const void* w, const void* g, void* dx, void* dw,
                            int64_t rows, int64_t hidden, float eps, nrm_dtype dtype,
                            nrm_dtype w_dtype, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return norm_vjp("nrm_rms_norm_vjp", false, x, w, g, dx, dw, nullptr, rows, hidden, eps, dtype,
                  w_dtype, workspace, workspace_bytes, stream);
}

nrm_status nrm_layer_norm_vjp(const void* x, const void* w, const void* g, void* dx, void* dw,
                              void* db, int64_t rows, int64_t hidden, float eps,
                              nrm_dtype dtype, nrm_dtype w_dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return norm_vjp("nrm_layer_norm_vjp", true, x, w, g, dx, dw, db, rows, hidden, eps, dtype,
                  w_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of nrm_layer_norm_vjp_noalloc: the fp64 partial column sums of dw and db, in a
// file-scope device array (each GPU the library runs on holds its own copy until the process
// ends) instead of a caller workspace. 32 MiB covers LayerNorm rows of up to 8192 values at any
// row count (at most 256 partial rows of dw and of db). In host code the array's name is only
// a stand-in: its device address, which differs per GPU, comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)32 << 20;
__device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device of `stream` (the current device for the null stream),
// looked up on the first call on each device, with that device current.
nrm_status scratch_on(const char* fn, hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess)
    return fail(NRM_ERR_DEVICE, "%s: no current device: %s, got HIP error %d", fn,
                hipGetErrorString(e), (int)e);
  int dev = cur;
  if (stream != nullptr && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess)
    return fail(NRM_ERR_DEVICE, "%s: stream's device unknown: %s, got HIP error %d", fn,
                hipGetErrorString(e), (int)e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(NRM_ERR_DEVICE, "%s: device index must be below %d, got %d", fn, kMaxDevices, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(NRM_ERR_DEVICE, "%s: cannot select device %d: %s, got HIP error %d", fn, dev,
                  hipGetErrorString(e), (int)e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return fail(NRM_ERR_DEVICE, "%s: scratch address on device %d: %s, got HIP error %d", fn,
                  dev, hipGetErrorString(e), (int)e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NRM_OK;
}

}  // namespace

extern "C" {

nrm_status nrm_layer_norm_vjp_noalloc(const void* x, const void* w, const void* g, void* dx,
                                      void* dw, void* db, int64_t rows, int64_t hidden,
                                      float eps, nrm_dtype dtype, nrm_dtype w_dtype,
                                      hipStream_t stream) {
  static const char* fn = "nrm_layer_norm_vjp_noalloc";
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, w_dtype);
  if (st) return st;
  if ((st = check_rows(fn, rows, hidden, dtype))) return st;
  void* ws = nullptr;
  if ((dw || db) && rows > 0) {
    const size_t need = nrm_norm_vjp_workspace_bytes(rows, hidden, 1);
    if (need > kScratchBytes)
      return fail(NRM_ERR_SHAPE,
                  "%s: rows x hidden must need at most %zu scratch bytes (hidden <= 8192 at any "
                  "row count), got %lld x %lld needing %zu", fn, kScratchBytes,
                  (long long)rows, (long long)hidden, need);
    if ((st = scratch_on(fn, stream, &ws))) return st;
  }
  return norm_vjp(fn, true, x, w, g, dx, dw, db, rows, hidden, eps, dtype, w_dtype, ws,
                  ws ? kScratchBytes : 0, stream);
}

nrm_status nrm_rope(const void* x, void* out, int64_t N, int64_t L, int64_t D, int64_t dims,
                    int traditional, float base, float scale, int64_t offset, int forward,
                    const float* freqs, float mscale, nrm_dtype dtype, hipStream_t stream) {
  static const char* fn = "nrm_rope";
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, dtype);
  if (st) return st;
  if (N < 0) return fail(NRM_ERR_SHAPE, "%s: N must be >= 0, got %lld", fn, (long long)N);
  if (L < 0) return fail(NRM_ERR_SHAPE, "%s: L must be >= 0, got %lld", fn, (long long)L);
  if ((st = check_rope_dims(fn, D, dims))) return st;
  if (offset < 0)
    return fail(NRM_ERR_SHAPE, "%s: offset must be >= 0, got %lld", fn, (long long)offset);
  const int64_t es = esize(dtype);
  if (N && L > INT64_MAX / es / D / N)
    return fail(NRM_ERR_SHAPE, "%s: N * L * D overflows the address range, got %lld x %lld", fn,
                (long long)N, (long long)L);
  if (N * L == 0) return NRM_OK;
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!out) return fail(NRM_ERR_NULL, "%s: out must not be NULL, got NULL", fn);
  const Span sx = span(x, N * L * D * es), so = span(out, N * L * D * es);
  const Span sf = span(freqs, freqs ? dims / 2 * 4 : 0);
  if ((st = check_out_vs(fn, "out", so, "x", sx, true))) return st;
  if ((st = check_out_vs(fn, "out", so, "freqs", sf, false))) return st;
  nrm::RopeArgs a = rope_defaults();
  a.x = x; a.out = out;
  a.BH = a.BH1 = N; a.L = L; a.D = (int)D; a.dims = (int)dims;
  a.x_sbh = L; a.x_sl = 1; a.o_sbh = L; a.o_sl = 1;
  a.traditional = traditional != 0; a.base = base; a.scale = scale; a.offset = offset;
  a.forward = forward != 0; a.freqs = freqs; a.mscale = mscale;
  const bool al = aligned16(x) && aligned16(out);
  return launched(fn, dtype == NRM_BF16 ? nrm::launch_norm_rope<true>(a, al, stream)
                                        : nrm::launch_norm_rope<false>(a, al, stream));
}

nrm_status nrm_rope_positions(const void* q, const void* k, void* q_out, void* k_out,
                              const void* positions, int pos_int64, int64_t T, int64_t Hq,
                              int64_t Hk, int64_t D, int64_t dims, int traditional, float base,
                              float scale, int forward, const float* freqs, float mscale,
                              nrm_dtype dtype, hipStream_t stream) {
  static const char* fn = "nrm_rope_positions";
  g_err.clear();
  nrm_status st = check_dtypes(fn, dtype, dtype);
  if (st) return st;
  if (T < 0) return fail(NRM_ERR_SHAPE, "%s: T must be >= 0, got %lld", fn, (long long)T);
  if (Hq < 0) return fail(NRM_ERR_SHAPE, "%s: Hq must be >= 0, got %lld", fn, (long long)Hq);
  if (Hk < 0) return fail(NRM_ERR_SHAPE, "%s: Hk must be >= 0, got %lld", fn, (long long)Hk);
  if ((st = check_rope_dims(fn, D, dims))) return st;
  const int64_t es = esize(dtype);
  const int64_t lim = INT64_MAX / es / D;
  if ((T && Hq > lim / T) || (T && Hk > lim / T) || (Hq > INT64_MAX - Hk))
    return fail(NRM_ERR_SHAPE, "%s: T * H * D overflows the address range, got %lld x %lld", fn,
                (long long)T, (long long)(Hq > Hk ? Hq : Hk));
  if (T == 0 || Hq + Hk == 0) return NRM_OK;
  if (!positions) return fail(NRM_ERR_NULL, "%s: positions must not be NULL, got NULL", fn);
  if (Hq && !q) return fail(NRM_ERR_NULL, "%s: q must not be NULL, got NULL", fn);
  if (Hq && !q_out) return fail(NRM_ERR_NULL, "%s: q_out must not be NULL, got NULL", fn);
  if (Hk && !k) return fail(NRM_ERR_NULL, "%s: k must not be NULL, got NULL", fn);
  if (Hk && !k_out) return fail(NRM_ERR_NULL, "%s: k_out must not be NULL, got NULL", fn);
  const Span sq = span(q, T * Hq * D * es), sqo = span(q_out, T * Hq * D * es);
  const Span sk = span(k, T * Hk * D * es), sko = span(k_out, T * Hk * D * es);
  const Span sp = span(positions, T * (pos_int64 ? 8 : 4));
  const Span sf = span(freqs, freqs ? dims / 2 * 4 : 0);
  if ((st = check_out_vs(fn, "q_out", sqo, "q", sq, true))) return st;
  if ((st = check_out_vs(fn, "q_out", sqo, "k", sk, false))) return st;
  if ((st = check_out_vs(fn, "q_out", sqo, "k_out", sko, false))) return st;
  if ((st = check_out_vs(fn, "k_out", sko, "k", sk, true))) return st;
  if ((st = check_out_vs(fn, "k_out", sko, "q", sq, false))) return st;
  const char* in_names[] = {"positions", "freqs"};
  const Span in_spans[] = {sp, sf};
  for (int i = 0; i < 2; ++i) {
    if ((st = check_out_vs(fn, "q_out", sqo, in_names[i], in_spans[i], false))) return st;
    if ((st = check_out_vs(fn, "k_out", sko, in_names[i], in_spans[i], false))) return st;
  }
  nrm::RopeArgs a = rope_defaults();
  // Tensor A is the query (Hq rows per token), tensor B the key (Hk rows per token).
  a.x = q; a.out = q_out; a.x2 = k; a.out2 = k_out;
  a.BH = Hq + Hk; a.BH1 = Hq; a.L = T; a.D = (int)D; a.dims = (int)dims;
  a.x_sbh = 1; a.x_sl = Hq; a.o_sbh = 1; a.o_sl = Hq;
  a.x2_sbh = 1; a.x2_sl = Hk; a.o2_sbh = 1; a.o2_sl = Hk;
  a.traditional = traditional != 0; a.base = base; a.scale = scale;
  a.forward = forward != 0; a.freqs = freqs; a.mscale = mscale;
  a.positions = positions; a.pos_i64 = pos_int64 != 0;
  const bool al = (!Hq || (aligned16(q) && aligned16(q_out))) &&
                  (!Hk || (aligned16(k) && aligned16(k_out)));
  return launched(fn, dtype == NRM_BF16 ? nrm::launch_norm_rope<true>(a, al, stream)
                                        : nrm::launch_norm_rope<false>(a, al, stream));
}

}  // extern "C"

namespace {

nrm::SmArgs sm_args(const void* x, void* out, int64_t rows, int64_t n) {
  nrm::SmArgs a;
  a.x = x; a.out = out; a.targets = nullptr; a.tgt_i64 = 0; a.g = nullptr; a.loss = nullptr;
  a.rows = rows; a.n = n; a.causal_R = 1; a.causal_rows = 1; a.team = 64;
  return a;
}

template <int OP>
hipError_t dispatch_sm(const nrm::SmArgs& a, nrm_dtype dtype, bool al, hipStream_t s) {
  return dtype == NRM_BF16 ? nrm::launch_softmax<true, OP>(a, al, s)
                           : nrm::launch_softmax<false, OP>(a, al, s);
}

// Shared checks of the softmax family: dtype, rows >= 0, 1 <= n < 2^31, no overflow.
nrm_status check_sm(const char* fn, int64_t rows, int64_t n, nrm_dtype dtype) {
  nrm_status st = check_dtypes(fn, dtype, dtype);
  if (st) return st;
  return check_rows(fn, rows, n, dtype);
}

}  // namespace

extern "C" {

nrm_status nrm_softmax(const void* x, void* out, int64_t rows, int64_t n, nrm_dtype dtype,
                       hipStream_t stream) {
  static const char* fn = "nrm_softmax";
  g_err.clear();
  nrm_status st = check_sm(fn, rows, n, dtype);
  if (st) return st;
  if (rows == 0) return NRM_OK;
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!out) return fail(NRM_ERR_NULL, "%s: out must not be NULL, got NULL", fn);
  const int64_t nb = rows * n * esize(dtype);
  if ((st = check_out_vs(fn, "out", span(out, nb), "x", span(x, nb), true))) return st;
  return launched(fn, dispatch_sm<nrm::SM_SOFTMAX>(sm_args(x, out, rows, n), dtype,
                                                   aligned16(x) && aligned16(out), stream));
}

nrm_status nrm_causal_softmax(const void* x, void* out, int64_t N, int64_t R, int64_t L,
                              int64_t rows_per_block, nrm_dtype dtype, hipStream_t stream) {
  static const char* fn = "nrm_causal_softmax";
  g_err.clear();
  if (N < 0) return fail(NRM_ERR_SHAPE, "%s: N must be >= 0, got %lld", fn, (long long)N);
  if (R < 0) return fail(NRM_ERR_SHAPE, "%s: R must be >= 0, got %lld", fn, (long long)R);
  if (rows_per_block < 1)
    return fail(NRM_ERR_SHAPE, "%s: rows_per_block must be >= 1, got %lld", fn,
                (long long)rows_per_block);
  if (R % rows_per_block)
    return fail(NRM_ERR_SHAPE, "%s: R must be a multiple of rows_per_block (%lld), got %lld", fn,
                (long long)rows_per_block, (long long)R);
  if (N && R > INT64_MAX / N)
    return fail(NRM_ERR_SHAPE, "%s: N * R overflows, got %lld x %lld", fn, (long long)N,
                (long long)R);
  nrm_status st = check_sm(fn, N * R, L, dtype);
  if (st) return st;
  if (N * R == 0) return NRM_OK;
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!out) return fail(NRM_ERR_NULL, "%s: out must not be NULL, got NULL", fn);
  const int64_t nb = N * R * L * esize(dtype);
  if ((st = check_out_vs(fn, "out", span(out, nb), "x", span(x, nb), true))) return st;
  nrm::SmArgs a = sm_args(x, out, N * R, L);
  a.causal_R = R;
  a.causal_rows = rows_per_block;
  return launched(fn, dispatch_sm<nrm::SM_CAUSAL>(a, dtype, aligned16(x) && aligned16(out),
                                                  stream));
}

nrm_status nrm_logsumexp(const void* x, void* out, int64_t rows, int64_t n, nrm_dtype dtype,
                         hipStream_t stream) {
  static const char* fn = "nrm_logsumexp";
  g_err.clear();
  nrm_status st = check_sm(fn, rows, n, dtype);
  if (st) return st;
  if (rows == 0) return NRM_OK;
  if (!x) return fail(NRM_ERR_NULL, "%s: x must not be NULL, got NULL", fn);
  if (!out) return fail(NRM_ERR_NULL, "%s: out must not be NULL, got NULL", fn);
  const int64_t es = esize(dtype);
  if ((st = check_out_vs(fn, "out", span(out, rows * es), "x", span(x, rows * n * es), false)))
    return st;
  return launched(fn, dispatch_sm<nrm::SM_LSE>(sm_args(x, out, rows, n), dtype, aligned16(x),
                                               stream));
}

nrm_status nrm_cross_entropy(const void* logits, const void* targets, int targets_int64,
                             float* loss, int64_t rows, int64_t V, nrm_dtype dtype,
                             hipStream_t stream) {
  static const char* fn = "nrm_cross_entropy";
  g_err.clear();
  nrm_status st = check_sm(fn, rows, V, dtype);
  if (st) return st;
  if (rows == 0) return NRM_OK;
  if (!logits) return fail(NRM_ERR_NULL, "%s: logits must not be NULL, got NULL", fn);
  if (!targets) return fail(NRM_ERR_NULL, "%s: targets must not be NULL, got NULL", fn);
  if (!loss) return fail(NRM_ERR_NULL, "%s: loss must not be NULL, got NULL", fn);
  const Span sx = span(logits, rows * V * esize(dtype));
  const Span st_ = span(targets, rows * (targets_int64 ? 8 : 4)), sl = span(loss, rows * 4);
  if ((st = check_out_vs(fn, "loss", sl, "logits", sx, false))) return st;
  if ((st = check_out_vs(fn, "loss", sl, "targets", st_, false))) return st;
  nrm::SmArgs a = sm_args(logits, nullptr, rows, V);
  a.targets = targets; a.tgt_i64 = targets_int64 != 0; a.loss = loss;
  return launched(fn, dispatch_sm<nrm::SM_CE>(a, dtype, aligned16(logits), stream));
}

nrm_status nrm_cross_entropy_vjp(const void* logits, const void* targets, int targets_int64,
                                 const float* loss, const float* g, void* dlogits,
                                 int64_t rows, int64_t V, nrm_dtype dtype, hipStream_t stream) {
  static const char* fn = "nrm_cross_entropy_vjp";
  g_err.clear();
  (void)loss;  // not needed: see nrm.h
  nrm_status st = check_sm(fn, rows, V, dtype);
  if (st) return st;
  if (rows == 0) return NRM_OK;
  if (!logits) return fail(NRM_ERR_NULL, "%s: logits must not be NULL, got NULL", fn);
  if (!targets) return fail(NRM_ERR_NULL, "%s: targets must not be NULL, got NULL", fn);
  if (!g) return fail(NRM_ERR_NULL, "%s: g must not be NULL, got NULL", fn);
  if (!dlogits) return fail(NRM_ERR_NULL, "%s: dlogits must not be NULL, got NULL", fn);
  const int64_t nb = rows * V * esize(dtype);
  const Span sx = span(logits, nb), sd = span(dlogits, nb);
  const Span st_ = span(targets, rows * (targets_int64 ? 8 : 4)), sg = span(g, rows * 4);
  if ((st = check_out_vs(fn, "dlogits", sd, "logits", sx, true))) return st;
  if ((st = check_out_vs(fn, "dlogits", sd, "targets", st_, false))) return st;
  if ((st = check_out_vs(fn, "dlogits", sd, "g", sg, false))) return st;
  nrm::SmArgs a = sm_args(logits, dlogits, rows, V);
  a.targets = targets; a.tgt_i64 = targets_int64 != 0; a.g = g;
  return launched(fn, dispatch_sm<nrm::SM_CE_VJP>(a, dtype,
                                                  aligned16(logits) && aligned16(dlogits),
                                                  stream));
}

const char* nrm_last_error(void) { return g_err.c_str(); }

const char* nrm_status_name(nrm_status status) {
  switch (status) {
    case NRM_OK: return "NRM_OK";
    case NRM_ERR_NULL: return "NRM_ERR_NULL";
    case NRM_ERR_SHAPE: return "NRM_ERR_SHAPE";
    case NRM_ERR_DTYPE: return "NRM_ERR_DTYPE";
    case NRM_ERR_ALIAS: return "NRM_ERR_ALIAS";
    case NRM_ERR_DEVICE: return "NRM_ERR_DEVICE";
  }
  return "NRM_ERR_UNKNOWN";
}

int nrm_version(void) { return 100; }

nrm_status nrm_bench_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  static const char* fn = "nrm_bench_copy";
  g_err.clear();
  if (bytes < 0 || bytes % 16)
    return fail(NRM_ERR_SHAPE, "%s: bytes must be a non-negative multiple of 16, got %lld", fn,
                (long long)bytes);
  if (bytes == 0) return NRM_OK;
  if (!src) return fail(NRM_ERR_NULL, "%s: src must not be NULL, got NULL", fn);
  if (!dst) return fail(NRM_ERR_NULL, "%s: dst must not be NULL, got NULL", fn);
  if (!aligned16(src) || !aligned16(dst))
    return fail(NRM_ERR_ALIAS, "%s: src and dst must be 16-byte aligned, got %p and %p", fn, src,
                dst);
  if (overlap(span(src, bytes), span(dst, bytes)))
    return fail(NRM_ERR_ALIAS, "%s: dst must not overlap src, got an overlap", fn);
  return launched(fn, nrm::launch_copy16(src, dst, bytes / 16, stream));
}

nrm_status nrm_bench_copy2(const void* src1, const void* src2, void* dst1, void* dst2,
                           int64_t bytes, hipStream_t stream) {
  static const char* fn = "nrm_bench_copy2";
  g_err.clear();
  if (bytes < 0 || bytes % 16)
    return fail(NRM_ERR_SHAPE, "%s: bytes must be a non-negative multiple of 16, got %lld", fn,
                (long long)bytes);
  if (bytes == 0) return NRM_OK;
  if (!src1 || !src2 || !dst1 || !dst2)
    return fail(NRM_ERR_NULL, "%s: src1, src2, dst1 and dst2 must not be NULL, got %p %p %p %p",
                fn, src1, src2, dst1, dst2);
  if (!aligned16(src1) || !aligned16(src2) || !aligned16(dst1) || !aligned16(dst2))
    return fail(NRM_ERR_ALIAS, "%s: every array must be 16-byte aligned, got %p %p %p %p", fn,
                src1, src2, dst1, dst2);
  const auto s1 = span(src1, bytes), s2 = span(src2, bytes), o1 = span(dst1, bytes),
             o2 = span(dst2, bytes);
  if (overlap(o1, s1) || overlap(o1, s2) || overlap(o2, s1) || overlap(o2, s2) || overlap(o1, o2))
    return fail(NRM_ERR_ALIAS, "%s: a destination overlaps a source or the other destination",
                fn);
  return launched(fn, nrm::launch_copy16x2(src1, src2, dst1, dst2, bytes / 16, stream));
}

nrm_status nrm_bench_copy2_row(const void* src1, const void* src2, void* dst1, void* dst2,
                               int64_t bytes, int64_t unit_bytes, hipStream_t stream) {
  static const char* fn = "nrm_bench_copy2_row";
  g_err.clear();
  if (unit_bytes != 8192 && unit_bytes != 16384 && unit_bytes != 32768)
    return fail(NRM_ERR_SHAPE, "%s: unit_bytes must be 8192, 16384 or 32768, got %lld", fn,
                (long long)unit_bytes);
  if (bytes < 0 || bytes % unit_bytes)
    return fail(NRM_ERR_SHAPE, "%s: bytes must be a non-negative multiple of unit_bytes (%lld), "
                "got %lld", fn, (long long)unit_bytes, (long long)bytes);
  if (bytes == 0) return NRM_OK;
  if (!src1 || !src2 || !dst1 || !dst2)
    return fail(NRM_ERR_NULL, "%s: src1, src2, dst1 and dst2 must not be NULL, got %p %p %p %p",
                fn, src1, src2, dst1, dst2);
  if (!aligned16(src1) || !aligned16(src2) || !aligned16(dst1) || !aligned16(dst2))
    return fail(NRM_ERR_ALIAS, "%s: every array must be 16-byte aligned, got %p %p %p %p", fn,
                src1, src2, dst1, dst2);
  const auto s1 = span(src1, bytes), s2 = span(src2, bytes), o1 = span(dst1, bytes),
             o2 = span(dst2, bytes);
  if (overlap(o1, s1) || overlap(o1, s2) || overlap(o2, s1) || overlap(o2, s2) || overlap(o1, o2))
    return fail(NRM_ERR_ALIAS, "%s: a destination overlaps a source or the other destination",
                fn);
  return launched(fn, nrm::launch_copy16x2_row(src1, src2, dst1, dst2, bytes / 16,
                                               (int)(unit_bytes / 8192), stream));
}

}  // extern "C"

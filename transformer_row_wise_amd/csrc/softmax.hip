// Softmax family over the last axis: Softmax, CausalSoftmax, LogSumExp, CrossEntropy and its
// gradient for the logits.
//
// Sources: nuvec-core 0.5.0 fast::FastOp, variants Softmax ((x): softmax over the last axis,
// accumulated in float32), CausalSoftmax ((x), field rows: row r of the second-to-last axis
// keeps the columns c <= r % rows + L - rows, the others become the dtype's lowest finite
// value and so 0), LogSumExp ((x): log(sum(exp(x))), the last axis becomes size 1),
// CrossEntropy ((logits, targets): logsumexp(logits) - logits[target] per row, float32) and
// CrossEntropyVjp ((logits, targets, loss, g): its gradient for the logits).
//
// Arithmetic: fp32 throughout (the pages' float32 accumulation). Per row, m = max and
// S = sum exp(x - m) over the row. The exponentials are formed scaled by 2^64, as
// 2^(fma(t, log2 e, 64)) on the hardware exp2 (three instructions, no range test): the
// hardware's results stop at the normal range, and the scale keeps every exponential that
// fp32 or bf16 can hold away from that floor. The scale cancels in every ratio (outputs,
// the loss's log1p and its gradient) and is taken off exactly, by a power-of-two product of
// a sum of at least 2^64, before a logarithm. Rounding t log2 e + 64 to fp32 costs at most
// ~1.3e-6 relative per exponential. A probability below the normal range comes out of one
// product with the row's reciprocal sum, rounded once. Cross-entropy keeps the
// target's term apart: with e_t = exp(x_t - m) and R = the sum over the other columns,
//   loss = log1p(R / e_t)                      (= logsumexp - x_t, no cancellation)
//   d loss / d x_t = -R / (R + e_t),   d loss / d x_j = exp(x_j - m) / (R + e_t)
// so a confident row (loss near 0) still gets its small loss and gradient to full relative
// precision; the gradient is then scaled by g. The loss input of the gradient is not needed
// (the row is read anyway) and is not read. A target outside [0, V) gives NaN.
//
// sm_rows: a team of T threads per row, each thread keeping NV 16-byte chunks of the row in
// registers: the row is read from HBM once, then max, sum and output passes run over
// registers. T is 16 or 32 lanes (SUB: the team's reductions are DPP exchanges inside a
// wave, no barrier) or a multiple of 64 (reductions through LDS, one barrier each); NV is at
// least 4 where the row allows, so that every thread keeps 64 bytes in flight. Rows of up
// to 2048 chunks (16384 bf16 or 8192 fp32 values) take it.
// sm_stream: 256 threads per row (1024 for rows of 16384 values or more that have a row
// output or number fewer than 512) looping over the row, U = 4 chunks (16-byte or single
// elements) per step loaded together, an online (max, sum) per thread (the sum rescaled when
// the maximum grows), then, for the operations with a row output, a second pass over the
// row (which the first pass left in the caches where it fits). Any width; the vocabulary-
// sized rows of the loss (128256 columns) take it at 8 blocks per compute unit.
#include "softmax.hpp"

namespace nrm {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// 2^64 exp(t) for t <= 0 (or NaN), fp32.
__device__ __forceinline__ float sm_exp64(float t) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(t, kLog2e, 64.0f));
}

// exp(t) for t <= 0, fp32, for the factors that rescale a sum to a larger maximum: a factor
// below the normal range flushes to 0, which only drops terms at least 2^62 times smaller
// than the sum they join (whose maximum contributes 2^64).
__device__ __forceinline__ float sm_factor(float t) {
  return __builtin_amdgcn_exp2f(t * kLog2e);
}

__device__ __forceinline__ float lowest_of(bool bf16) {
  return bf16 ? -3.3895313892515355e38f : -3.4028234663852886e38f;
}

// The dtype's lowest finite value in every element of a 16-byte chunk.
template <bool BF16>
__device__ __forceinline__ u32x4 lowest_chunk() {
  const unsigned b = BF16 ? 0xff7fff7fu : 0xff7fffffu;
  return u32x4{b, b, b, b};
}

// Chunk v, whose first element is column `first`, with each column past `cut` replaced by
// the dtype's lowest finite value (the causal mask, applied once to the packed scores).
template <bool BF16>
__device__ __forceinline__ u32x4 mask_past(u32x4 v, int first, int cut) {
  const int keep = cut - first + 1;  // leading elements kept
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (BF16) {
      // Element 2d in the low half of dword d, 2d + 1 in the high half.
      const unsigned lo = 2 * d < keep ? (v[d] & 0xffffu) : 0xff7fu;
      const unsigned hi = 2 * d + 1 < keep ? (v[d] & 0xffff0000u) : 0xff7f0000u;
      v[d] = lo | hi;
    } else {
      v[d] = d < keep ? v[d] : 0xff7fffffu;
    }
  }
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) { return dpp<CTRL>(v); }

// Max or sum over a wave, returned wave-uniform (DPP in each row of 16, then the four row
// results read with readlane and combined in a fixed order).
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = op(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = op(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = op(v, dpp_f<DPP_ROW_MIRROR>(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return op(op(r0, r1), op(r2, r3));
}

// Max or sum over a team of nwt waves starting at wave0; red holds one slot per wave of the
// block. Every team of the block calls this the same number of times (one barrier each).
template <bool MAX>
__device__ __forceinline__ float team_reduce(float v, float* red, int wave0, int nwt) {
  v = wave_reduce<MAX>(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[wave0];
  for (int q = 1; q < nwt; ++q) t = MAX ? fmaxf(t, red[wave0 + q]) : t + red[wave0 + q];
  return t;
}

// Max or sum over aligned groups of G lanes (G = 16 or 32) of a wave; every lane of a
// group gets the same bits (each exchange pairs lanes symmetrically).
template <bool MAX, int G>
__device__ __forceinline__ float group_reduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = op(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = op(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = op(v, dpp_f<DPP_ROW_MIRROR>(v));
  if constexpr (G == 32) v = op(v, __shfl_xor(v, 16, 64));
  return v;
}

// Per-row context shared by both kernels.
struct SmRow {
  int64_t row;
  int64_t cut;     // CAUSAL: last kept column (may be negative); others: n - 1
  int64_t target;  // CE: target column, or -1 when out of range
  bool bad;        // CE: target out of range
  float g;         // CE_VJP: cotangent
};

template <int OP>
__device__ __forceinline__ SmRow sm_row(const SmArgs& a, int64_t row) {
  SmRow r;
  r.row = row;
  r.cut = a.n - 1;
  if constexpr (OP == SM_CAUSAL) {
    const int64_t rr = (row % a.causal_R) % a.causal_rows;
    r.cut = rr + a.n - a.causal_rows;
  }
  r.target = -1;
  r.bad = false;
  r.g = 1.f;
  if constexpr (OP == SM_CE || OP == SM_CE_VJP) {
    const int64_t t = a.tgt_i64 ? ((const int64_t*)a.targets)[row]
                                : (int64_t)((const int32_t*)a.targets)[row];
    r.bad = t < 0 || t >= a.n;
    r.target = r.bad ? -1 : t;
  }
  if constexpr (OP == SM_CE_VJP) r.g = a.g[row];
  return r;
}

// log(sum exp(x)) from the row's maximum m and s = 2^64 sum exp(x - m); an infinite maximum
// is the result itself (+inf: some score is +inf; -inf: every score is -inf, the sum is 0).
__device__ __forceinline__ float lse_of(float m, float s) {
  if (__builtin_isinf(m)) return m;
  return m + __builtin_amdgcn_logf(s * 0x1p-64f) * 0.6931471805599453f;
}

// The loss from the row's maximum m, the target's logit x_t, e_t = 2^64 exp(x_t - m) and the
// sum R of the other columns' exponentials (scaled alike).
__device__ __forceinline__ float ce_loss(float m, float x_t, float e_t, float rest) {
  if (m - x_t < 60.f) return log1pf(rest / e_t);
  return (m - x_t) + logf((rest + e_t) * 0x1p-64f);
}

}  // namespace

template <bool BF16, int OP, int NV, bool EXACT, int SUB>
__global__ void __launch_bounds__(1024)
sm_rows(SmArgs a) {
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr bool CE = OP == SM_CE || OP == SM_CE_VJP;
  __shared__ float red_m[16], red_s[16], xt_s[64];
  const int T = SUB ? SUB : a.team;
  const int team = threadIdx.x / T;
  const int tid = threadIdx.x - team * T;
  const int nwt = SUB ? 1 : T >> 6, wave0 = SUB ? 0 : team * nwt;
  const int nvec = (int)(a.n / V);
  const int64_t row_raw = (int64_t)blockIdx.x * (blockDim.x / T) + team;
  const bool live = row_raw < a.rows;
  const int64_t row = live ? row_raw : a.rows - 1;
  const SmRow r = sm_row<OP>(a, row);
  const float lowest = lowest_of(BF16);
  auto reduce_max = [&](float v) {
    if constexpr (SUB) return group_reduce<true, SUB>(v);
    else return team_reduce<true>(v, red_m, wave0, nwt);
  };
  auto reduce_sum = [&](float v) {
    if constexpr (SUB) return group_reduce<false, SUB>(v);
    else return team_reduce<false>(v, red_s, wave0, nwt);
  };

  // Chunk k of this thread is chunk tid + k * T of the row; past the row's end (only when
  // not EXACT) its loads are clamped to the last chunk and its results dropped. Indices are
  // recomputed where used rather than kept in registers.
  auto chunk = [&](int k) { return tid + k * T; };
  auto ok = [&](int k) { return EXACT || chunk(k) < nvec; };
  const int cut = (int)r.cut;
  // CausalSoftmax with eight chunks per thread masks the packed scores once, as they are
  // loaded: a compare per element in each pass took the kernel into scratch (~1700 spilled
  // registers; [2048, 12000] bf16 1119 -> 22 us). With fewer chunks the per-element compare
  // measured faster ([256, 512, 512] bf16 42 against 47 us).
  constexpr bool MASK_LOAD = OP == SM_CAUSAL && NV >= 8;
  // The target's chunk and its element within the chunk (team-uniform): per chunk one
  // vector compare says whether this thread owns it, per element a scalar compare.
  const int tgt_chunk = r.target < 0 ? -1 : (int)(r.target / V);
  const int tgt_e = r.target < 0 ? -1 : (int)(r.target % V);
  auto is_tgt = [&](int k, int e) { return e == tgt_e && chunk(k) == tgt_chunk; };
  const char* xr = (const char*)a.x + row * a.n * ESZ;
  u32x4 xv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if constexpr (MASK_LOAD) {
      // A chunk wholly past the row's causal cut is never read; masked scores become the
      // lowest value here, once, so that the passes below read plain scores.
      xv[k] = lowest_chunk<BF16>();
      if (chunk(k) * V <= cut)
        xv[k] = mask_past<BF16>(
            ld16_nt(xr + (int64_t)(EXACT ? chunk(k) : min(chunk(k), nvec - 1)) * 16),
            chunk(k) * V, cut);
    } else if constexpr (OP == SM_CAUSAL) {
      // A chunk wholly past the row's causal cut is never read: its scores are replaced.
      xv[k] = u32x4{0, 0, 0, 0};
      if (chunk(k) * V <= cut)
        xv[k] = ld16_nt(xr + (int64_t)(EXACT ? chunk(k) : min(chunk(k), nvec - 1)) * 16);
    } else {
      xv[k] = ld16_nt(xr + (int64_t)(EXACT ? chunk(k) : min(chunk(k), nvec - 1)) * 16);
    }
  }

  // Score of element e of chunk k as the operation sees it (masked, or -inf when absent).
  auto score = [&](int k, int e, float f) {
    if (!ok(k)) return -__builtin_inff();
    if constexpr (OP == SM_CAUSAL && !MASK_LOAD) return chunk(k) * V + e <= cut ? f : lowest;
    return f;
  };

  // CausalSoftmax with up to four chunks per thread: a chunk slot that lies wholly past the
  // causal cut in every lane of the wave (all its scores are the lowest value, or absent past
  // the row's end) is handled as a whole, behind a wave-uniform branch. It adds that value to
  // the maximum; once every lane's maximum exceeds it, its exponentials are exactly +0 (the
  // difference is at least 2^104), so the sum pass adds nothing for it. Rows of a causal
  // block keep half their columns on average, so a wave skips ~3/8 of the per-element work:
  // bf16 [32, 2048, 2048] 72.5 -> 70.7 us, [64, 1024, 1024] 37.1 -> 36.2 us, fp32
  // [256, 512, 512] 73.6 -> 72.9 us. Teams of 16 lanes (four rows per wave) measured slower
  // with the branches (bf16 [256, 512, 512] 44.5 -> 47.4 us) and keep the straight passes.
  constexpr bool SKIP = OP == SM_CAUSAL && !MASK_LOAD && SUB != 16;
  auto wave_none = [&](bool c) { return __builtin_amdgcn_ballot_w64(c) == 0; };
  auto past_cut = [&](int k) { return chunk(k) * V > cut; };

  float m = -__builtin_inff();
  float xt = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if constexpr (SKIP) {
      if (wave_none(!past_cut(k))) {
        m = fmaxf(m, ok(k) ? lowest : -__builtin_inff());
        continue;
      }
    }
    float f[V];
    unpack<BF16>(xv[k], f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      m = fmaxf(m, score(k, e, f[e]));
      if constexpr (CE) {
        if (is_tgt(k, e)) xt = f[e];
      }
    }
  }
  if constexpr (CE) {
    // The one thread that holds the target's logit publishes it (team slot in LDS); a
    // barrier (block teams) or the group's own lanes (sub-wave teams) order the read.
    if constexpr (SUB) {
      // The owner is lane tgt_chunk % SUB of this team's lanes of the wave.
      const int base = (threadIdx.x & 63) - tid;
      xt = __shfl(xt, base + (tgt_chunk < 0 ? 0 : tgt_chunk % SUB), 64);
    } else {
      if (tgt_chunk >= 0 && tgt_chunk % T == tid) xt_s[team] = xt;
    }
  }
  m = reduce_max(m);
  if constexpr (CE && !SUB) xt = r.bad ? 0.f : xt_s[team];
  // A row whose scores are all -inf keeps m = -inf; exp(x - m) is then NaN, as
  // exp(-inf + inf) is in the definition.

  // Each pass widens the raw chunks again: the opaque redefinition keeps the compiler from
  // holding a previous pass's widened values (two floats per bf16 pair) across the barrier.
  // Operations with a row output keep the exponentials of up to four chunks (32 registers)
  // for the output pass instead of forming them twice.
  constexpr bool OUT = OP == SM_SOFTMAX || OP == SM_CAUSAL || OP == SM_CE_VJP;
  constexpr bool KEEP = OUT && NV <= 4;
  float ek[KEEP ? NV : 1][V];
#pragma unroll
  for (int k = 0; k < NV; ++k) __asm__ volatile("" : "+v"(xv[k]));
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if constexpr (SKIP) {
      if (wave_none(!past_cut(k) || !(m > lowest))) {
        if constexpr (KEEP) {
#pragma unroll
          for (int e = 0; e < V; ++e) ek[k][e] = 0.f;
        }
        continue;
      }
    }
    float f[V];
    unpack<BF16>(xv[k], f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float ex = sm_exp64(score(k, e, f[e]) - m);
      if (!ok(k)) ex = 0.f;
      if constexpr (CE) {
        if (is_tgt(k, e)) ex = 0.f;  // R excludes the target
      }
      if constexpr (KEEP) ek[k][e] = ex;
      s += ex;
    }
  }
  s = reduce_sum(s);

  if constexpr (OP == SM_LSE) {
    if (live && tid == 0) {
      float o[1] = {lse_of(m, s)};
      store_act<BF16, 1>(a.out, row, o);
    }
    return;
  }
  if constexpr (OP == SM_CE) {
    if (live && tid == 0) {
      const float e_t = sm_exp64(xt - m);
      a.loss[row] = r.bad ? __builtin_nanf("") : ce_loss(m, xt, e_t, s);
    }
    return;
  }
  // Softmax, CausalSoftmax, CrossEntropyVjp: the output row.
  float inv, gt = 0.f;
  if constexpr (OP == SM_CE_VJP) {
    const float e_t = sm_exp64(xt - m);
    const float tot = s + e_t;
    inv = r.g / tot;
    gt = -r.g * (s / tot);  // d loss / d x_t, times g
    if (r.bad) inv = gt = __builtin_nanf("");
  } else {
    inv = 1.f / s;
  }
  if (!live) return;
  char* orow = (char*)a.out + row * a.n * ESZ;
  if constexpr (!KEEP) {
#pragma unroll
    for (int k = 0; k < NV; ++k) __asm__ volatile("" : "+v"(xv[k]));
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float f[V];
    if constexpr (!KEEP) unpack<BF16>(xv[k], f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float p = (KEEP ? ek[k][e] : sm_exp64(score(k, e, f[e]) - m)) * inv;
      if constexpr (OP == SM_CE_VJP) {
        if (is_tgt(k, e)) p = gt;
      }
      f[e] = p;
    }
    if (ok(k)) st16_nt(orow + (int64_t)chunk(k) * 16, pack<BF16>(f));
  }
}

template <bool BF16, int OP, int V, int TPB>
__global__ void __launch_bounds__(TPB)
sm_stream(SmArgs a) {
  constexpr bool CE = OP == SM_CE || OP == SM_CE_VJP;
  constexpr int U = 4;  // chunks loaded together per step
  constexpr bool OUT = OP == SM_SOFTMAX || OP == SM_CAUSAL || OP == SM_CE_VJP;
  constexpr int NW = TPB / 64;
  __shared__ float red_m[NW], red_s[NW], xt_s[1];
  const int64_t row = blockIdx.x;
  const SmRow r = sm_row<OP>(a, row);
  const float lowest = lowest_of(BF16);
  const int64_t nch = a.n / V;
  const int64_t e0 = row * a.n;
  const int64_t tgt_chunk = r.target < 0 ? -1 : r.target / V;
  const int tgt_e = r.target < 0 ? -1 : (int)(r.target % V);
  auto score = [&](int64_t c, float f) {
    if constexpr (OP == SM_CAUSAL) return c <= r.cut ? f : lowest;
    return f;
  };
  // Pass 1: online maximum and rescaled sum per thread (while a thread's maximum is still
  // -inf every score it has seen is -inf, and contributes 0). Each step loads U chunks
  // (clamped to the row, unconditional) before using any.
  // Rows with an output pass park HU of the U chunks of their first step per thread in LDS,
  // so that the second pass reads them from LDS: the oldest data of pass 1 is the likeliest
  // to have left the caches by then (cross-entropy gradient [4096, 128256] 428 -> 419 us;
  // parking the last step instead measured slower, 453 us).
  // The second step's U chunks stay in registers for the second pass (16 VGPRs, within the
  // 64 that keep two 1024-thread blocks per CU; the gradient 394 -> 380 us).
  constexpr bool HOLD = OUT && V == Fmt<BF16>::VEC;
  constexpr int HU = 3;
  extern __shared__ u32x4 held[];  // HOLD: HU * TPB chunks
  u32x4 kept[HOLD ? U : 1];
  const int64_t stepc = (int64_t)TPB * U;
  const int64_t nsteps = (nch + stepc - 1) / stepc;
  float m = -__builtin_inff(), s = 0.f;
  for (int64_t si = 0; si < nsteps; ++si) {
    const int64_t j0 = threadIdx.x + si * stepc;
    if (j0 >= nch) break;
    float f[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = min(j0 + (int64_t)u * TPB, nch - 1);
      if constexpr (V == Fmt<BF16>::VEC) {
        const void* p = (const char*)a.x + (e0 + j * V) * Fmt<BF16>::ESZ;
        // Rows with an output pass are read with cached loads, so that the second read
        // of this block's row finds it in the caches.
        const u32x4 raw = OUT ? ld16(p) : ld16_nt(p);
        if constexpr (HOLD) {
          if (u < HU && si == 0) held[u * TPB + threadIdx.x] = raw;
          if (si == 1) kept[u] = raw;
        }
        unpack<BF16>(raw, f[u]);
      } else {
        load_act<BF16, V>(a.x, e0 + j * V, f[u]);
      }
    }
    float cm = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + (int64_t)u * TPB < nch) {
#pragma unroll
        for (int e = 0; e < V; ++e) cm = fmaxf(cm, score((j0 + u * TPB) * V + e, f[u][e]));
      }
    }
    if (cm > m) {
      s = s * sm_factor(m - cm);
      m = cm;
    }
    const float mm = m == -__builtin_inff() ? 0.f : m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + (int64_t)u * TPB;
      if (j < nch) {
        // CE: one compare per chunk says whether it holds the target (tgt_chunk), then a
        // scalar compare per element.
        const bool own = CE && j == tgt_chunk;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          float ex = sm_exp64(score(j * V + e, f[u][e]) - mm);
          if (own && e == tgt_e) {
            xt_s[0] = f[u][e];  // published by the barrier of the maximum's reduction
            ex = 0.f;
          }
          s += ex;
        }
      }
    }
  }
  const float M = team_reduce<true>(m, red_m, 0, NW);
  float xt = 0.f;
  if constexpr (CE) xt = r.bad ? 0.f : xt_s[0];
  // Rescale each thread's sum to the row maximum, then add in a fixed order.
  const float S = team_reduce<false>(m == -__builtin_inff() ? 0.f : s * sm_factor(m - M), red_s, 0, NW);

  if constexpr (OP == SM_LSE) {
    if (threadIdx.x == 0) {
      float o[1] = {lse_of(M, S)};
      store_act<BF16, 1>(a.out, row, o);
    }
    return;
  }
  if constexpr (OP == SM_CE) {
    if (threadIdx.x == 0)
      a.loss[row] = r.bad ? __builtin_nanf("") : ce_loss(M, xt, sm_exp64(xt - M), S);
    return;
  }
  float inv, gt = 0.f;
  if constexpr (OP == SM_CE_VJP) {
    const float e_t = sm_exp64(xt - M);
    const float tot = S + e_t;
    inv = r.g / tot;
    gt = -r.g * (S / tot);
    if (r.bad) inv = gt = __builtin_nanf("");
  } else {
    inv = 1.f / S;
  }
  // Pass 2: each thread re-reads exactly the chunks it read in pass 1 (so in-place use is
  // safe: no thread writes a chunk another thread still has to read), the parked ones from
  // LDS (each thread its own slots: no barrier).
  for (int64_t si = 0; si < nsteps; ++si) {
    const int64_t j0 = threadIdx.x + si * stepc;
    if (j0 >= nch) break;
    float f[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = min(j0 + (int64_t)u * TPB, nch - 1);
      if constexpr (V == Fmt<BF16>::VEC) {
        if (HOLD && u < HU && si == 0)
          unpack<BF16>(held[u * TPB + threadIdx.x], f[u]);
        else if (HOLD && si == 1)
          unpack<BF16>(kept[u], f[u]);
        else
          unpack<BF16>(ld16_nt((const char*)a.x + (e0 + j * V) * Fmt<BF16>::ESZ), f[u]);
      } else {
        load_act<BF16, V>(a.x, e0 + j * V, f[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + (int64_t)u * TPB;
      if (j < nch) {
        const bool own = OP == SM_CE_VJP && j == tgt_chunk;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          float p = sm_exp64(score(j * V + e, f[u][e]) - M) * inv;
          if (own && e == tgt_e) p = gt;
          f[u][e] = p;
        }
        if constexpr (V == Fmt<BF16>::VEC) {
          st16_nt((char*)a.out + (e0 + j * V) * Fmt<BF16>::ESZ, pack<BF16>(f[u]));
        } else {
          store_act<BF16, V>(a.out, e0 + j * V, f[u]);
        }
      }
    }
  }
}

// sm_mis: rows whose width or start is not a whole number of 16-byte chunks (an odd
// vocabulary such as 50257 columns), for every operation but CausalSoftmax. Each row splits
// into a head of hd < VEC elements up to its first 16-byte boundary, a body of whole chunks
// and a tail of fewer than VEC elements; thread t < hd + tail holds one head or tail element
// as a scalar, and the body streams as in sm_stream (U chunks per step, an online maximum and
// rescaled sum per thread, then for row outputs a second, cached pass). The output row has
// the input row's phase (the host checks that the two bases agree modulo 16), so its body
// chunks are 16-byte aligned too.
template <bool BF16, int OP, int TPB>
__global__ void __launch_bounds__(TPB)
sm_mis(SmArgs a) {
  constexpr bool CE = OP == SM_CE || OP == SM_CE_VJP;
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int U = 4;
  constexpr bool OUT = OP == SM_SOFTMAX || OP == SM_CE_VJP;
  constexpr int NW = TPB / 64;
  __shared__ float red_m[NW], red_s[NW], xt_s[1];
  const int64_t row = blockIdx.x;
  const SmRow r = sm_row<OP>(a, row);
  const int64_t n = a.n;
  const int64_t e0 = row * n;
  const char* xrow = (const char*)a.x + e0 * ESZ;
  const int hd = (int)min((int64_t)((16 - ((uintptr_t)xrow & 15)) & 15) / ESZ, n);
  const int64_t nch = (n - hd) / V;
  const int tl = (int)(n - hd - nch * V);
  const char* xbody = xrow + (int64_t)hd * ESZ;  // 16-byte aligned
  // This thread's scalar element (column sc), if any.
  const bool has_s = (int)threadIdx.x < hd + tl;
  const int64_t sc = (int)threadIdx.x < hd ? (int64_t)threadIdx.x
                                            : hd + nch * V + ((int64_t)threadIdx.x - hd);
  float sv = -__builtin_inff();
  if (has_s) {
    float t[1];
    load_act<BF16, 1>(a.x, e0 + sc, t);
    sv = t[0];
  }
  const int64_t tb = r.target < 0 ? -1 : r.target - hd;  // CE: target's index in the body
  const int64_t tgt_chunk = tb < 0 || tb >= nch * V ? -1 : tb / V;
  const int tgt_e = tgt_chunk < 0 ? -1 : (int)(tb % V);
  const bool s_tgt = CE && has_s && sc == r.target;

  // Pass 1: the scalar element first, then the body, online (max, rescaled sum) per thread.
  float m = -__builtin_inff(), s = 0.f;
  if (has_s) {
    m = fmaxf(m, sv);
    const float mm = m == -__builtin_inff() ? 0.f : m;
    float ex = sm_exp64(sv - mm);
    if (s_tgt) {
      xt_s[0] = sv;  // published by the barrier of the maximum's reduction
      ex = 0.f;
    }
    s = ex;
  }
  const int64_t stepc = (int64_t)TPB * U;
  const int64_t nsteps = (nch + stepc - 1) / stepc;
  for (int64_t si = 0; si < nsteps; ++si) {
    const int64_t j0 = threadIdx.x + si * stepc;
    if (j0 >= nch) break;
    float f[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = min(j0 + (int64_t)u * TPB, nch - 1);
      const u32x4 raw = OUT ? ld16(xbody + j * 16) : ld16_nt(xbody + j * 16);
      unpack<BF16>(raw, f[u]);
    }
    float cm = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + (int64_t)u * TPB < nch) {
#pragma unroll
        for (int e = 0; e < V; ++e) cm = fmaxf(cm, f[u][e]);
      }
    }
    if (cm > m) {
      s = s * sm_factor(m - cm);
      m = cm;
    }
    const float mm = m == -__builtin_inff() ? 0.f : m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + (int64_t)u * TPB;
      if (j < nch) {
        const bool own = CE && j == tgt_chunk;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          float ex = sm_exp64(f[u][e] - mm);
          if (own && e == tgt_e) {
            xt_s[0] = f[u][e];
            ex = 0.f;
          }
          s += ex;
        }
      }
    }
  }
  const float M = team_reduce<true>(m, red_m, 0, NW);
  float xt = 0.f;
  if constexpr (CE) xt = r.bad ? 0.f : xt_s[0];
  const float S = team_reduce<false>(m == -__builtin_inff() ? 0.f : s * sm_factor(m - M), red_s, 0, NW);

  if constexpr (OP == SM_LSE) {
    if (threadIdx.x == 0) {
      float o[1] = {lse_of(M, S)};
      store_act<BF16, 1>(a.out, row, o);
    }
    return;
  }
  if constexpr (OP == SM_CE) {
    if (threadIdx.x == 0)
      a.loss[row] = r.bad ? __builtin_nanf("") : ce_loss(M, xt, sm_exp64(xt - M), S);
    return;
  }
  float inv, gt = 0.f;
  if constexpr (OP == SM_CE_VJP) {
    const float e_t = sm_exp64(xt - M);
    const float tot = S + e_t;
    inv = r.g / tot;
    gt = -r.g * (S / tot);
    if (r.bad) inv = gt = __builtin_nanf("");
  } else {
    inv = 1.f / S;
  }
  // Pass 2: each thread writes exactly what it read (in-place use is safe).
  char* obody = (char*)a.out + (e0 + hd) * ESZ;
  if (has_s) {
    float o[1] = {s_tgt ? gt : sm_exp64(sv - M) * inv};
    store_act<BF16, 1>(a.out, e0 + sc, o);
  }
  for (int64_t si = 0; si < nsteps; ++si) {
    const int64_t j0 = threadIdx.x + si * stepc;
    if (j0 >= nch) break;
    float f[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = min(j0 + (int64_t)u * TPB, nch - 1);
      unpack<BF16>(ld16_nt(xbody + j * 16), f[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + (int64_t)u * TPB;
      if (j < nch) {
        const bool own = OP == SM_CE_VJP && j == tgt_chunk;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          float p = sm_exp64(f[u][e] - M) * inv;
          if (own && e == tgt_e) p = gt;
          f[u][e] = p;
        }
        st16_nt(obody + j * 16, pack<BF16>(f[u]));
      }
    }
  }
}

namespace {

constexpr int64_t kSmMaxGrid = 0x7fffffff;

template <bool BF16, int OP, int NV, bool EXACT, int SUB>
hipError_t go_sm_rows(const SmArgs& a0, int team, hipStream_t stream) {
  SmArgs a = a0;
  a.team = team;
  // Several teams per 256-thread block when the team divides 256 (16 .. 128 threads), else
  // one team per block (192 threads, or 256 and more): a block holds whole teams only.
  const int threads = team < 256 && 256 % team == 0 ? 256 : team;
  const int G = threads / team;
  const int64_t blocks = (a.rows + G - 1) / G;
  if (blocks > kSmMaxGrid) return hipErrorInvalidConfiguration;
  sm_rows<BF16, OP, NV, EXACT, SUB><<<(unsigned)blocks, threads, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int NV>
hipError_t sm_team(const SmArgs& a, int team, bool exact, hipStream_t stream) {
  if (team == 16)
    return exact ? go_sm_rows<BF16, OP, NV, true, 16>(a, 16, stream)
                 : go_sm_rows<BF16, OP, NV, false, 16>(a, 16, stream);
  if (team == 32)
    return exact ? go_sm_rows<BF16, OP, NV, true, 32>(a, 32, stream)
                 : go_sm_rows<BF16, OP, NV, false, 32>(a, 32, stream);
  return exact ? go_sm_rows<BF16, OP, NV, true, 0>(a, team, stream)
               : go_sm_rows<BF16, OP, NV, false, 0>(a, team, stream);
}

// Operations with a row output read the row twice. With 1024-thread blocks (two per
// compute unit) about 512 rows are in flight, so the second read of a 256 KB vocabulary row
// still finds it in the 256 MB Infinity Cache; eight 256-thread blocks per CU keep the same
// bytes in flight but four times the rows, which evicts each row before its second read.
// The reductions (LogSumExp, CrossEntropy) take 1024 threads too when there are fewer than
// 512 rows: with one block per row and most compute units idle, each block's own bytes in
// flight set the pace (LogSumExp [64, 128256] bf16 18.1 -> 9.6 us, [256, 128256] 20.2 ->
// 12.8 us).
template <bool BF16, int OP, int V>
hipError_t go_sm_stream(const SmArgs& a, hipStream_t stream) {
  constexpr bool OUT = OP == SM_SOFTMAX || OP == SM_CAUSAL || OP == SM_CE_VJP;
  if (a.rows > kSmMaxGrid) return hipErrorInvalidConfiguration;
  const size_t lds1 = OUT && V == Fmt<BF16>::VEC ? 3 * 1024 * 16 : 0;
  const size_t lds2 = OUT && V == Fmt<BF16>::VEC ? 3 * 256 * 16 : 0;
  if (a.n >= 16384 && (OUT || a.rows < 512))
    sm_stream<BF16, OP, V, 1024><<<(unsigned)a.rows, 1024, lds1, stream>>>(a);
  else
    sm_stream<BF16, OP, V, 256><<<(unsigned)a.rows, 256, lds2, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

// Register kernel for rows of up to 2048 chunks: NV = ceil(chunks / 256) (at most 8), raised
// towards 4 as far as the team keeps 16 lanes; T = ceil(chunks / NV), rounded up to 16, 32
// or a multiple of 64. Longer rows: the streaming kernel. Rows that are not whole chunks:
// sm_mis (CausalSoftmax, or an output of another phase: the streaming kernel one element at a
// time).
template <bool BF16, int OP>
hipError_t launch_softmax(const SmArgs& a, bool aligned16, hipStream_t stream) {
  constexpr int V = Fmt<BF16>::VEC;
  const int path = forced_path();
  const bool vec = aligned16 && a.n % V == 0 && path != PATH_SCALAR;
  if (!vec) {
    // Rows not made of whole 16-byte chunks: head, chunk body and tail per row (sm_mis),
    // when an output row shares its input row's phase; otherwise one element at a time.
    if constexpr (OP != SM_CAUSAL) {
      constexpr bool OUT = OP == SM_SOFTMAX || OP == SM_CE_VJP;
      const bool same_phase = !OUT || (((uintptr_t)a.x ^ (uintptr_t)a.out) & 15u) == 0;
      if (path != PATH_SCALAR && same_phase && ((uintptr_t)a.x & (Fmt<BF16>::ESZ - 1)) == 0) {
        if (a.rows > kSmMaxGrid) return hipErrorInvalidConfiguration;
        if (OUT && a.n >= 16384)
          sm_mis<BF16, OP, 1024><<<(unsigned)a.rows, 1024, 0, stream>>>(a);
        else
          sm_mis<BF16, OP, 256><<<(unsigned)a.rows, 256, 0, stream>>>(a);
        return hipGetLastError();
      }
    }
    return go_sm_stream<BF16, OP, 1>(a, stream);
  }
  const int64_t n = a.n / V;
  if (path != PATH_CHUNKED && n <= 2048) {
    int nv = (int)std::min<int64_t>(8, (n + 255) / 256);
    if (nv < 4) nv = (int)std::max<int64_t>(nv, std::min<int64_t>(4, n / 16));
    if (nv < 1) nv = 1;
    nv = nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : 8;
    const int64_t per = (n + nv - 1) / nv;
    const int team = per <= 16 ? 16 : per <= 32 ? 32 : (int)((per + 63) / 64 * 64);
    const bool exact = (int64_t)team * nv == n;
    switch (nv) {
      case 1: return sm_team<BF16, OP, 1>(a, team, exact, stream);
      case 2: return sm_team<BF16, OP, 2>(a, team, exact, stream);
      case 4: return sm_team<BF16, OP, 4>(a, team, exact, stream);
      default: return sm_team<BF16, OP, 8>(a, team, exact, stream);
    }
  }
  return go_sm_stream<BF16, OP, V>(a, stream);
}

#define NRM_SM_INST(OP)                                                                     \
  template hipError_t launch_softmax<true, OP>(const SmArgs&, bool, hipStream_t);          \
  template hipError_t launch_softmax<false, OP>(const SmArgs&, bool, hipStream_t);
NRM_SM_INST(SM_SOFTMAX)
NRM_SM_INST(SM_CAUSAL)
NRM_SM_INST(SM_LSE)
NRM_SM_INST(SM_CE)
NRM_SM_INST(SM_CE_VJP)
#undef NRM_SM_INST

}  // namespace nrm

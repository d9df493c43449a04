// Row kernels for RMSNorm, residual add-RMSNorm and LayerNorm over the last axis.
//
// Operations (nuvec-core 0.5.0 fast::FastOp, variants RmsNorm, AddRmsNorm and LayerNorm):
//   RMS      out = x * rstd * w,             rstd = 1 / sqrt(sum(x^2) / D + eps)
//   ADD_RMS  h = RN(x + r); out = h * rstd * w, rstd from sum(h^2) of the rounded h
//   LN       out = (x - mu) * rstd * w + b,  mu = sum(x) / D, rstd = 1 / sqrt(sum((x-mu)^2)/D + eps)
//
// Shapes of the same arithmetic:
//   row_block               one block of up to 1024 threads per row, NV 16-byte chunks per
//                           thread in registers (the default for rows of 129 to 8192 chunks,
//                           and for the RMS forms' bf16 rows beside fp32 w up to 6144);
//   row_team                the same with a team of 4 .. 64 lanes per row and 256 / team
//                           rows per block (rows of up to 128 chunks);
//   row_ln_pair,            LayerNorm (with w or b) and RMSNorm (with fp32 w) as row_block
//   row_rms_pair            with two rows per block (the parameters loaded once per pair);
//   row_regs<..., WPR = 1>  one wave64 per row, the whole row in registers (hidden <= 64*NV*VEC);
//                           a block holds four independent waves (four rows);
//   row_regs<..., WPR = 8>  one 512-thread block per row, row in registers, cross-wave sums
//                           through LDS (hidden <= 512*NV*VEC);
//   row_elems               one block per row, K single elements per thread in registers:
//                           rows whose width or base addresses are not 16-byte multiples,
//                           up to 12288 elements (add-RMSNorm: bf16 rows up to 2048);
//   row_chunked             one 256-thread block per row looping over the row: any width, and
//                           V = 1 for the other rows of that kind. The row is re-read (L2)
//                           for the second pass.
// Every element of x (and r) is read from HBM once and every output element written once;
// w and b are small and come from L2.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace nrm {

enum RowOp : int { OP_RMS = 0, OP_ADD_RMS = 1, OP_LN = 2 };

struct RowArgs {
  const void* x;
  const void* r;   // ADD_RMS only
  const void* w;   // may be null (= 1)
  const void* b;   // LN only, may be null (= 0)
  void* out;
  void* h;         // ADD_RMS only
  int64_t rows;
  int64_t hidden;  // elements per row, < 2^31
  float eps;
  int w_f32;       // w and b stored as fp32 (else bf16, only with bf16 activations)
  double inv_n;    // 1 / hidden, rounded to fp64
};

// Cross-lane sum over the threads of one row: the wave itself (WPR == 1) or the block,
// through `red` (one slot per wave) in LDS.
template <int WPR, typename T>
__device__ __forceinline__ T row_sum(T v, T* red) {
  v = wave_sum(v);
  if constexpr (WPR > 1) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    T t = red[0];
#pragma unroll
    for (int i = 1; i < WPR; ++i) t += red[i];
    v = t;
  }
  return v;
}

// out = (x - mu) * rstd * w + b in fp64 for one chunk of V elements, with w / b optional.
template <bool BF16, int V, bool HAS_W, bool HAS_B>
__device__ __forceinline__ void ln_chunk_out(const float (&f)[V], const RowArgs& a, int64_t i,
                                             double mu, double rstd, float (&y)[V]) {
  float wv[V], bv[V];
  if constexpr (HAS_W) load_param<BF16, V>(a.w, a.w_f32, i, wv);
  if constexpr (HAS_B) load_param<BF16, V>(a.b, a.w_f32, i, bv);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    double t = ((double)f[e] - mu) * rstd;
    if constexpr (HAS_W && HAS_B) t = __builtin_fma(t, (double)wv[e], (double)bv[e]);
    else if constexpr (HAS_W) t = t * (double)wv[e];
    else if constexpr (HAS_B) t = t + (double)bv[e];
    y[e] = f64_to_f32(t);
  }
}

template <bool BF16, int OP, int NV, int WPR>
__global__ void __launch_bounds__(WPR == 1 ? 256 : 64 * WPR)
row_regs(RowArgs a) {
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int TPR = 64 * WPR;  // threads per row
  __shared__ float red_f[WPR > 1 ? WPR : 1];
  __shared__ double red_d[2][WPR > 1 ? WPR : 1];

  const int64_t row = WPR == 1 ? (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6) : (int64_t)blockIdx.x;
  const int tid = WPR == 1 ? (threadIdx.x & 63) : threadIdx.x;
  if (row >= a.rows) return;  // uniform over the wave (WPR == 1) or the block (WPR > 1)

  const int nvec = (int)(a.hidden / V);
  const int64_t base = row * a.hidden * ESZ;  // byte offset of the row
  const char* xr = (const char*)a.x + base;

  // All loads of the row are issued before any store, so an output that is exactly an
  // input (in-place use) is read before it is written.
  u32x4 xv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = tid + k * TPR;
    if (j < nvec) xv[k] = ld16(xr + (int64_t)j * 16);
  }

  if constexpr (OP == OP_RMS || OP == OP_ADD_RMS) {
    float acc = 0.f;
    if constexpr (OP == OP_ADD_RMS) {
      const char* rr = (const char*)a.r + base;
      u32x4 rv[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int j = tid + k * TPR;
        if (j < nvec) rv[k] = ld16(rr + (int64_t)j * 16);
      }
      char* hr = (char*)a.h + base;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int j = tid + k * TPR;
        if (j < nvec) {
          float fx[V], fr[V];
          unpack<BF16>(xv[k], fx);
          unpack<BF16>(rv[k], fr);
#pragma unroll
          for (int e = 0; e < V; ++e) fx[e] = fx[e] + fr[e];
          xv[k] = pack<BF16>(fx);  // h rounded to the storage type, kept for the output pass
          st16(hr + (int64_t)j * 16, xv[k]);
          unpack<BF16>(xv[k], fx);
#pragma unroll
          for (int e = 0; e < V; ++e) acc = __builtin_fmaf(fx[e], fx[e], acc);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int j = tid + k * TPR;
        if (j < nvec) {
          float fx[V];
          unpack<BF16>(xv[k], fx);
#pragma unroll
          for (int e = 0; e < V; ++e) acc = __builtin_fmaf(fx[e], fx[e], acc);
        }
      }
    }
    const float ss = row_sum<WPR>(acc, red_f);
    const float rstd = (float)rstd_f64((double)ss, a.hidden, a.eps);

    char* orow = (char*)a.out + base;
    const bool has_w = a.w != nullptr;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int j = tid + k * TPR;
      if (j < nvec) {
        float f[V], wv[V];
        unpack<BF16>(xv[k], f);
        if (has_w) {
          load_param<BF16, V>(a.w, a.w_f32, (int64_t)j * V, wv);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) wv[e] = 1.f;
        }
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = (f[e] * rstd) * wv[e];
        st16(orow + (int64_t)j * 16, pack<BF16>(f));
      }
    }
  } else {  // OP_LN: fp64 statistics and output arithmetic
    double s1 = 0.0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int j = tid + k * TPR;
      if (j < nvec) {
        float f[V];
        unpack<BF16>(xv[k], f);
#pragma unroll
        for (int e = 0; e < V; ++e) s1 += (double)f[e];
      }
    }
    const double mu = row_sum<WPR>(s1, red_d[0]) / (double)a.hidden;
    double s2 = 0.0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int j = tid + k * TPR;
      if (j < nvec) {
        float f[V];
        unpack<BF16>(xv[k], f);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const double d = (double)f[e] - mu;
          s2 = __builtin_fma(d, d, s2);
        }
      }
    }
    const double rstd = rstd_f64(row_sum<WPR>(s2, red_d[1]), a.hidden, a.eps);

    char* orow = (char*)a.out + base;
    const bool hw = a.w != nullptr, hb = a.b != nullptr;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int j = tid + k * TPR;
      if (j < nvec) {
        float f[V], y[V];
        unpack<BF16>(xv[k], f);
        const int64_t i = (int64_t)j * V;
        if (hw && hb) ln_chunk_out<BF16, V, true, true>(f, a, i, mu, rstd, y);
        else if (hw) ln_chunk_out<BF16, V, true, false>(f, a, i, mu, rstd, y);
        else if (hb) ln_chunk_out<BF16, V, false, true>(f, a, i, mu, rstd, y);
        else ln_chunk_out<BF16, V, false, false>(f, a, i, mu, rstd, y);
        st16(orow + (int64_t)j * 16, pack<BF16>(y));
      }
    }
  }
}

// Sum over the T threads of a block that owns one row (nw = T / 64 waves, at most 16):
// DPP inside each wave, then the wave sums through `red` in a fixed order. One barrier.
template <typename T>
__device__ __forceinline__ T block_row_sum(T v, T* red, int nw) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  T t = red[0];
  for (int i = 1; i < nw; ++i) t += red[i];
  return t;
}

// How the scale and shift vectors are stored, fixed at compile time so that no branch sits
// around their loads: absent (1 and 0), in the activations' dtype, or fp32 (with bf16
// activations).
enum ParamKind : int { PK_NONE = 0, PK_SAME = 1, PK_F32 = 2 };

template <bool BF16, int PK, int V>
__device__ __forceinline__ void load_pk(const void* p, int64_t i, float (&f)[V]) {
  if constexpr (PK == PK_NONE) {
#pragma unroll
    for (int e = 0; e < V; ++e) f[e] = 1.f;
  } else {
    load_param<BF16, V>(p, PK == PK_F32, i, f);
  }
}

// One row per block of T = blockDim.x threads (a multiple of 64, at most 1024): thread t
// keeps chunks t, t + T, ... (NV of them) of the row in registers between the statistic and
// the output. This is the shape that streams fastest on MI355X: at [16384, 8192] bf16 the
// add-RMSNorm runs at ~79% of 8 TB/s, against ~64% for one wave per row and ~73% for a
// persistent grid that prefetches the next row (16 waves per row keep more independent
// requests in flight, and a finished block is replaced at once). x, r, h and out are
// streamed with non-temporal accesses. EXACT means T * NV chunks cover the row exactly:
// no tail guards. Otherwise a chunk index past the row end is clamped to the last chunk
// for loads (so every load is unconditional and the compiler's waits stay exact) and the
// stores of such chunks are skipped.
// SUB > 0 (4 .. 64, narrow rows): a team of SUB lanes per row instead, 256 / SUB rows per
// block, the row's sums by lane exchanges inside the team (no LDS, no barrier); a team past
// the last row loads that row and stores nothing.
template <bool BF16, int OP, int NV, int PK, bool EXACT, int SUB>
__device__ __forceinline__ void row_block_body(RowArgs a) {
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  __shared__ float red_f[16];
  __shared__ double red4[16 * 4];
  const int T = SUB ? SUB : blockDim.x;
  const int nw = T >> 6;
  const int tid = SUB ? (int)(threadIdx.x & (SUB - 1)) : (int)threadIdx.x;
  const int nvec = (int)(a.hidden / V);
  bool live = true;
  int64_t row = blockIdx.x;
  if constexpr (SUB > 0) {
    row = (int64_t)blockIdx.x * (blockDim.x / SUB) + threadIdx.x / SUB;
    live = row < a.rows;
    if (!live) row = a.rows - 1;
  }
  const int64_t base = row * a.hidden * ESZ;

  int jj[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = tid + k * T;
    ok[k] = EXACT || j < nvec;
    jj[k] = EXACT ? j : min(j, nvec - 1);
  }
  // LayerNorm with bf16 w and b keeps them packed (8 registers per chunk instead of 16) and
  // widens them where the output uses them.
  constexpr bool LN_PACKED = OP == OP_LN && BF16 && PK == PK_SAME;
  // From 4 chunks per thread on, w is loaded after the row's sums, chunk by chunk where the
  // output uses it: x, r and a widened w of 8 chunks would not fit the 128 registers of a
  // 1024-thread block (add-RMSNorm bf16 [512, 65536] 55 -> 49 us), and at 4 the 768- and
  // 1024-thread rows then hold two blocks per CU instead of one (LayerNorm fp32 [2730, 12288]
  // affine 61 -> 50 us, RMSNorm bf16 [1024, 32768] 27.7 -> 25.7 us). The RMS forms at 6
  // chunks load all of w right after the sum instead: chunk by chunk measured 2-7% slower
  // there (add-RMSNorm fp32 [682, 24576]).
  constexpr bool W_LATE = PK != PK_NONE && NV >= 4;
  float wv[NV][V];
  u32x4 wpk[NV];
  if constexpr (!W_LATE) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if constexpr (LN_PACKED) wpk[k] = ld16((const uint16_t*)a.w + (int64_t)jj[k] * V);
      else load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wv[k]);
    }
  }
  u32x4 xv[NV], rv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    xv[k] = ld16_nt((const char*)a.x + base + (int64_t)jj[k] * 16);
    if constexpr (OP == OP_ADD_RMS) rv[k] = ld16_nt((const char*)a.r + base + (int64_t)jj[k] * 16);
  }

  if constexpr (OP == OP_RMS || OP == OP_ADD_RMS) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float f[V];
      unpack<BF16>(xv[k], f);
      if constexpr (OP == OP_ADD_RMS) {
        float fr[V];
        unpack<BF16>(rv[k], fr);
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = f[e] + fr[e];
        xv[k] = pack<BF16>(f);  // h, rounded to the storage type (stored with out, below)
        unpack<BF16>(xv[k], f);
      }
      if (ok[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) acc = __builtin_fmaf(f[e], f[e], acc);
      }
    }
    float ss;
    if constexpr (SUB > 0) ss = group_sum<SUB>(acc);
    else ss = block_row_sum(acc, red_f, nw);
    const float rstd = (float)rstd_f64((double)ss, a.hidden, a.eps);
    if constexpr (W_LATE && NV == 6) {
#pragma unroll
      for (int k = 0; k < NV; ++k) load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wv[k]);
    }
    // h is stored here, beside out, rather than right after the add: a block's loads and its
    // stores then form two phases, which streams faster on MI355X (add-RMSNorm [16384, 8192]
    // bf16 172.2-172.8 -> 170.5-171.4 us, [65536, 5120] fp32 921 -> 897 us).
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if constexpr (W_LATE && NV != 6) load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wv[k]);
      float f[V];
      unpack<BF16>(xv[k], f);
      if constexpr (OP == OP_ADD_RMS) {
        if (live && ok[k]) st16_nt((char*)a.h + base + (int64_t)jj[k] * 16, xv[k]);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) f[e] = (f[e] * rstd) * wv[k][e];
      if (live && ok[k]) st16_nt((char*)a.out + base + (int64_t)jj[k] * 16, pack<BF16>(f));
    }
  } else {  // OP_LN, fp64 statistics and output arithmetic
    // One pass: the sum and the sum of squares of x - p in fp64 about the row's first
    // element p (the row pivots of common.hpp), reduced together with one barrier; var =
    // sum((x-p)^2)/n - (mean - p)^2 loses at most log2(n) bits however large |mean| / sigma
    // is. A constant row gets x - p = 0 everywhere, so mean = p, var = 0 and x - mean = 0
    // exactly: its output is exactly b. Below 4 chunks per thread b (like w) is loaded
    // before the row's statistics.
    const bool has_b = a.b != nullptr;
    float bv[NV][V];
    u32x4 bpk[NV];
    // Rows past 4 chunks, and rows of 4 with w, load b chunk by chunk in the output loop, one
    // copy of which is compiled for rows with b and one for rows without, so that no test of
    // b sits between a chunk's loads and its arithmetic.
    constexpr bool B_LATE = W_LATE || NV > 4;
    // Chunk k's w (when loaded late) and b (when hb).
    auto load_wb = [&](int k, bool hb) {
      if constexpr (W_LATE) {
        if constexpr (LN_PACKED) wpk[k] = ld16((const uint16_t*)a.w + (int64_t)jj[k] * V);
        else load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wv[k]);
      }
      if constexpr (LN_PACKED) {
        bpk[k] = hb ? ld16((const uint16_t*)a.b + (int64_t)jj[k] * V) : u32x4{0u, 0u, 0u, 0u};
      } else if (hb) {
        // b has w's dtype; without w its kind is only known at run time.
        if constexpr (PK == PK_NONE) load_param<BF16, V>(a.b, a.w_f32, (int64_t)jj[k] * V, bv[k]);
        else load_pk<BF16, PK, V>(a.b, (int64_t)jj[k] * V, bv[k]);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) bv[k][e] = 0.f;
      }
    };
    if constexpr (!B_LATE) {
#pragma unroll
      for (int k = 0; k < NV; ++k) load_wb(k, has_b);
    }
    // A team's first lane holds the row's chunk 0; a block reads the row's first element
    // through the scalar cache.
    double piv;
    if constexpr (SUB > 0) piv = (double)first_elem<BF16>(group_first<SUB>(xv[0][0]));
    else piv = (double)sload_elem<BF16>((const char*)a.x + base, 0);
    double ds[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float f[V];
      unpack<BF16>(xv[k], f);
      if (ok[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const double xs = (double)f[e] - piv;
          ds[e & 1] += xs;
          ds[2 + (e & 1)] = __builtin_fma(xs, xs, ds[2 + (e & 1)]);
        }
      }
    }
    ds[0] += ds[1];
    ds[1] = ds[2] + ds[3];
    ds[2] = ds[3] = 0.0;
    if constexpr (SUB > 0) {
      ds[0] = group_sum<SUB>(ds[0]);
      ds[1] = group_sum<SUB>(ds[1]);
    } else {
      team_sum4(ds, red4, 0, nw);
    }
    // mean - p = sum / n through the reciprocal and one residual step, which lands on the
    // correctly rounded quotient.
    const double n = (double)a.hidden, inv_n = a.inv_n;
    double q = ds[0] * inv_n;
    q = __builtin_fma(__builtin_fma(-q, n, ds[0]), inv_n, q);
    const double mu = piv + q;
    // Clamp rounding below zero, but keep a NaN (an infinite row gives inf - inf).
    const double v0 = ds[1] * inv_n - q * q;
    const double var = v0 < 0.0 ? 0.0 : v0;
    const double rstd = rsqrt_row(var + (double)a.eps);
    auto out_row = [&](auto hb) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if constexpr (B_LATE) load_wb(k, decltype(hb)::value);
        u32x4 xr = xv[k];
        __asm__ volatile("" : "+v"(xr));  // widen again rather than hold fp64 copies
        float f[V], wf[V], bf[V];
        unpack<BF16>(xr, f);
        if constexpr (LN_PACKED) {
          u32x4 wr = wpk[k], br = bpk[k];
          __asm__ volatile("" : "+v"(wr), "+v"(br));  // widen here, not at the load
          unpack<true>(wr, wf);
          unpack<true>(br, bf);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) wf[e] = wv[k][e], bf[e] = bv[k][e];
        }
#pragma unroll
        for (int e = 0; e < V; ++e)
          f[e] = f64_to_f32(__builtin_fma(((double)f[e] - mu) * rstd, (double)wf[e], (double)bf[e]));
        if (live && ok[k]) st16_nt((char*)a.out + base + (int64_t)jj[k] * 16, pack<BF16>(f));
      }
    };
    if constexpr (B_LATE) {
      if (has_b) out_row(std::true_type{});
      else out_row(std::false_type{});
    } else {
      out_row(std::true_type{});
    }
  }
}

template <bool BF16, int OP, int NV, int PK, bool EXACT>
__global__ void __launch_bounds__(1024)
row_block(RowArgs a) {
  row_block_body<BF16, OP, NV, PK, EXACT, 0>(a);
}

// Narrow rows: teams of SUB lanes (4 .. 64) with two chunks per lane, 256 / SUB rows per
// 256-thread block.
template <bool BF16, int OP, int PK, bool EXACT, int SUB>
__global__ void __launch_bounds__(256)
row_team(RowArgs a) {
  row_block_body<BF16, OP, 2, PK, EXACT, SUB>(a);
}

// LayerNorm, two rows per block: thread t keeps chunks t, t + T, ... (NV of them) of both
// rows in registers, loads w and b once for the pair, and the four row sums (sum x and
// sum x^2 of each row) take one team_sum4, so a row costs half a barrier and half the
// parameter loads of row_block. The statistics and output arithmetic are row_block's. The
// second row of the last block may be past the end: it then repeats the first row's loads
// and stores nothing.
template <bool BF16, int NV, int PK, bool EXACT>
__global__ void __launch_bounds__(1024)
row_ln_pair(RowArgs a) {
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr bool LN_PACKED = BF16 && PK == PK_SAME;
  __shared__ double red4[16 * 4];
  const int T = blockDim.x, nw = T >> 6, tid = threadIdx.x;
  const int nvec = (int)(a.hidden / V);
  const int64_t r0 = 2 * (int64_t)blockIdx.x;
  const bool live1 = r0 + 1 < a.rows;
  const int64_t base[2] = {r0 * a.hidden * ESZ, (live1 ? r0 + 1 : r0) * a.hidden * ESZ};
  int jj[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = tid + k * T;
    ok[k] = EXACT || j < nvec;
    jj[k] = EXACT ? j : min(j, nvec - 1);
  }
  const bool has_b = a.b != nullptr;
  float wv[NV][V], bv[NV][V];
  u32x4 wpk[NV], bpk[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if constexpr (LN_PACKED) {
      wpk[k] = ld16((const uint16_t*)a.w + (int64_t)jj[k] * V);
      bpk[k] = has_b ? ld16((const uint16_t*)a.b + (int64_t)jj[k] * V) : u32x4{0u, 0u, 0u, 0u};
    } else {
      load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wv[k]);
      if (has_b) {
        if constexpr (PK == PK_NONE) load_param<BF16, V>(a.b, a.w_f32, (int64_t)jj[k] * V, bv[k]);
        else load_pk<BF16, PK, V>(a.b, (int64_t)jj[k] * V, bv[k]);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) bv[k][e] = 0.f;
      }
    }
  }
  u32x4 xv[2][NV];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int k = 0; k < NV; ++k) xv[r][k] = ld16_nt((const char*)a.x + base[r] + (int64_t)jj[k] * 16);
  }
  // Each row's sums about its first element (the row pivots of common.hpp); the two rows'
  // four sums take one reduction.
  double piv[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) piv[r] = (double)sload_elem<BF16>((const char*)a.x + base[r], 0);
  double ds[4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    double p[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float f[V];
      unpack<BF16>(xv[r][k], f);
      if (ok[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const double xs = (double)f[e] - piv[r];
          p[e & 1] += xs;
          p[2 + (e & 1)] = __builtin_fma(xs, xs, p[2 + (e & 1)]);
        }
      }
    }
    ds[2 * r] = p[0] + p[1];
    ds[2 * r + 1] = p[2] + p[3];
  }
  team_sum4(ds, red4, 0, nw);
  const double n = (double)a.hidden, inv_n = a.inv_n;
  double mu[2], rstd[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    double q = ds[2 * r] * inv_n;
    q = __builtin_fma(__builtin_fma(-q, n, ds[2 * r]), inv_n, q);
    mu[r] = piv[r] + q;
    const double v0 = ds[2 * r + 1] * inv_n - q * q;
    const double var = v0 < 0.0 ? 0.0 : v0;
    rstd[r] = rsqrt_row(var + (double)a.eps);
  }
  // Chunk by chunk, both rows: a chunk's w and b are widened to fp64 once for the pair.
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float wf[V], bf[V];
    if constexpr (LN_PACKED) {
      u32x4 wr = wpk[k], br = bpk[k];
      __asm__ volatile("" : "+v"(wr), "+v"(br));  // widen here, not at the load
      unpack<true>(wr, wf);
      unpack<true>(br, bf);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) wf[e] = wv[k][e], bf[e] = bv[k][e];
    }
    double wd[V], bd[V];
#pragma unroll
    for (int e = 0; e < V; ++e) wd[e] = (double)wf[e], bd[e] = (double)bf[e];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r == 1 && !live1) break;
      u32x4 xr = xv[r][k];
      __asm__ volatile("" : "+v"(xr));  // widen again rather than hold fp64 copies
      float f[V];
      unpack<BF16>(xr, f);
#pragma unroll
      for (int e = 0; e < V; ++e)
        f[e] = f64_to_f32(__builtin_fma(((double)f[e] - mu[r]) * rstd[r], wd[e], bd[e]));
      if (ok[k]) st16_nt((char*)a.out + base[r] + (int64_t)jj[k] * 16, pack<BF16>(f));
    }
  }
}

// RMSNorm with an fp32 scale, two rows per block, as row_ln_pair: each thread holds its NV chunks
// of both rows and loads w once for the pair; the two rows' fp32 sums of squares are reduced
// together (one barrier), in row_block's order. The arithmetic is row_block's.
template <bool BF16, int NV, int PK, bool EXACT>
__global__ void __launch_bounds__(1024)
row_rms_pair(RowArgs a) {
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  __shared__ float red[16 * 2];
  const int T = blockDim.x, nw = T >> 6, tid = threadIdx.x;
  const int nvec = (int)(a.hidden / V);
  const int64_t r0 = 2 * (int64_t)blockIdx.x;
  const bool live1 = r0 + 1 < a.rows;
  const int64_t base[2] = {r0 * a.hidden * ESZ, (live1 ? r0 + 1 : r0) * a.hidden * ESZ};
  int jj[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = tid + k * T;
    ok[k] = EXACT || j < nvec;
    jj[k] = EXACT ? j : min(j, nvec - 1);
  }
  float wv[NV][V];
#pragma unroll
  for (int k = 0; k < NV; ++k) load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wv[k]);
  u32x4 xv[2][NV];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int k = 0; k < NV; ++k) xv[r][k] = ld16_nt((const char*)a.x + base[r] + (int64_t)jj[k] * 16);
  }
  float acc[2] = {0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float f[V];
      unpack<BF16>(xv[r][k], f);
      if (ok[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) acc[r] = __builtin_fmaf(f[e], f[e], acc[r]);
      }
    }
    acc[r] = wave_sum(acc[r]);
  }
  if ((tid & 63) == 0) {
    red[(tid >> 6) * 2] = acc[0];
    red[(tid >> 6) * 2 + 1] = acc[1];
  }
  __syncthreads();
  float ss[2] = {red[0], red[1]};
  for (int i = 1; i < nw; ++i) {
    ss[0] += red[2 * i];
    ss[1] += red[2 * i + 1];
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (r == 1 && !live1) break;
    const float rstd = (float)rstd_f64((double)ss[r], a.hidden, a.eps);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float f[V];
      unpack<BF16>(xv[r][k], f);
#pragma unroll
      for (int e = 0; e < V; ++e) f[e] = (f[e] * rstd) * wv[k][e];
      if (ok[k]) st16_nt((char*)a.out + base[r] + (int64_t)jj[k] * 16, pack<BF16>(f));
    }
  }
}

// One block of 256 threads per row, looping over the row in chunks of V elements
// (V = VEC for 16-byte aligned rows, 1 otherwise). Grid-strided over rows.
template <bool BF16, int OP, int V>
__global__ void __launch_bounds__(256)
row_chunked(RowArgs a) {
  constexpr int WPR = 4;
  __shared__ float red_f[WPR];
  __shared__ double red_d[2][WPR];
  const int64_t nch = a.hidden / V;
  const bool has_w = a.w != nullptr, has_b = a.b != nullptr;

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t e0 = row * a.hidden;  // element offset of the row
    if constexpr (OP == OP_RMS || OP == OP_ADD_RMS) {
      float acc = 0.f;
      for (int64_t j = threadIdx.x; j < nch; j += 256) {
        float f[V];
        load_act<BF16, V>(a.x, e0 + j * V, f);
        if constexpr (OP == OP_ADD_RMS) {
          float fr[V];
          load_act<BF16, V>(a.r, e0 + j * V, fr);
#pragma unroll
          for (int e = 0; e < V; ++e) f[e] = f[e] + fr[e];
          round_to_storage<BF16, V>(f);
          store_act<BF16, V>(a.h, e0 + j * V, f);
        }
#pragma unroll
        for (int e = 0; e < V; ++e) acc = __builtin_fmaf(f[e], f[e], acc);
      }
      const float rstd = (float)rstd_f64((double)row_sum<WPR>(acc, red_f), a.hidden, a.eps);
      // Each thread re-reads exactly the chunks it wrote or read in the first pass.
      const void* src = OP == OP_ADD_RMS ? (const void*)a.h : a.x;
      for (int64_t j = threadIdx.x; j < nch; j += 256) {
        float f[V], wv[V];
        load_act<BF16, V>(src, e0 + j * V, f);
        if (has_w) {
          load_param<BF16, V>(a.w, a.w_f32, j * V, wv);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) wv[e] = 1.f;
        }
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = (f[e] * rstd) * wv[e];
        store_act<BF16, V>(a.out, e0 + j * V, f);
      }
    } else {
      double s1 = 0.0;
      for (int64_t j = threadIdx.x; j < nch; j += 256) {
        float f[V];
        load_act<BF16, V>(a.x, e0 + j * V, f);
#pragma unroll
        for (int e = 0; e < V; ++e) s1 += (double)f[e];
      }
      const double mu = row_sum<WPR>(s1, red_d[0]) / (double)a.hidden;
      double s2 = 0.0;
      for (int64_t j = threadIdx.x; j < nch; j += 256) {
        float f[V];
        load_act<BF16, V>(a.x, e0 + j * V, f);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const double d = (double)f[e] - mu;
          s2 = __builtin_fma(d, d, s2);
        }
      }
      const double rstd = rstd_f64(row_sum<WPR>(s2, red_d[1]), a.hidden, a.eps);
      for (int64_t j = threadIdx.x; j < nch; j += 256) {
        float f[V], y[V];
        load_act<BF16, V>(a.x, e0 + j * V, f);
        if (has_w && has_b) ln_chunk_out<BF16, V, true, true>(f, a, j * V, mu, rstd, y);
        else if (has_w) ln_chunk_out<BF16, V, true, false>(f, a, j * V, mu, rstd, y);
        else if (has_b) ln_chunk_out<BF16, V, false, true>(f, a, j * V, mu, rstd, y);
        else ln_chunk_out<BF16, V, false, false>(f, a, j * V, mu, rstd, y);
        store_act<BF16, V>(a.out, e0 + j * V, y);
      }
    }
    __syncthreads();  // the LDS slots are reused by the next row of this block
  }
}

// One element of x / r / h / out at element index i, non-temporal (touched once).
template <bool BF16>
__device__ __forceinline__ float ld1_nt(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(__builtin_nontemporal_load((const uint16_t*)p + i));
  else return __builtin_nontemporal_load((const float*)p + i);
}
template <bool BF16>
__device__ __forceinline__ void st1_nt(void* p, int64_t i, float v) {
  if constexpr (BF16) __builtin_nontemporal_store(f32_to_bf16(v), (uint16_t*)p + i);
  else __builtin_nontemporal_store(v, (float*)p + i);
}

// Rows that are not whole 16-byte chunks (an odd width, or a base off a 16-byte boundary),
// up to 12288 elements: one row per block of T threads, thread t holding the K elements at
// columns t + T e in registers (a wave's accesses are consecutive elements), so the row is
// read once; the arithmetic is row_chunked's. The launch keeps T (K - 1) <= hidden, so only
// a thread's last element can fall past the row's end; such an element loads as 0 (adding
// nothing to the sums; LayerNorm's second sum skips it) and is not stored. HB: LayerNorm
// with a shift vector.
template <bool BF16, int OP, int K, int PK, bool HB>
__global__ void __launch_bounds__(1024)
row_elems(RowArgs a) {
  __shared__ float red_f[16];
  __shared__ double red_d[2][16];
  const int T = blockDim.x, nw = T >> 6;
  const int64_t H = a.hidden;
  const int64_t e0 = (int64_t)blockIdx.x * H + threadIdx.x;
  bool ok[K];
  float f[K];
#pragma unroll
  for (int e = 0; e < K; ++e) {
    ok[e] = e < K - 1 || threadIdx.x + (int64_t)T * e < H;
    f[e] = ok[e] ? ld1_nt<BF16>(a.x, e0 + (int64_t)T * e) : 0.f;
  }
  if constexpr (OP == OP_ADD_RMS) {
    // Every r load is issued before the first h store: h may be x or r itself, so the
    // compiler cannot move a load above an earlier store, and loads interleaved with the
    // stores would wait for memory one element at a time ([16384, 2047] bf16 75.5 -> 63.7 us).
    float fr[K];
#pragma unroll
    for (int e = 0; e < K; ++e) fr[e] = ok[e] ? ld1_nt<BF16>(a.r, e0 + (int64_t)T * e) : 0.f;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      float t[1] = {f[e] + fr[e]};
      round_to_storage<BF16, 1>(t);
      f[e] = t[0];
      if (ok[e]) st1_nt<BF16>(a.h, e0 + (int64_t)T * e, f[e]);
    }
  }
  // Scale (and shift) at this thread's columns; a column past the end reads the last one.
  float wv[K], bv[K];
#pragma unroll
  for (int e = 0; e < K; ++e) {
    const int64_t c = min((int64_t)threadIdx.x + (int64_t)T * e, H - 1);
    float t[1];
    load_pk<BF16, PK, 1>(a.w, c, t);
    wv[e] = t[0];
    if constexpr (HB) {
      if constexpr (PK == PK_NONE) load_param<BF16, 1>(a.b, a.w_f32, c, t);  // b without w
      else load_pk<BF16, PK, 1>(a.b, c, t);
      bv[e] = t[0];
    }
  }
  float y[K];
  if constexpr (OP == OP_RMS || OP == OP_ADD_RMS) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < K; ++e) acc = __builtin_fmaf(f[e], f[e], acc);
    const float rstd = (float)rstd_f64((double)block_row_sum(acc, red_f, nw), a.hidden, a.eps);
#pragma unroll
    for (int e = 0; e < K; ++e) y[e] = (f[e] * rstd) * wv[e];
  } else {
    double s1 = 0.0;
#pragma unroll
    for (int e = 0; e < K; ++e) s1 += (double)f[e];
    const double mu = block_row_sum(s1, red_d[0], nw) / (double)a.hidden;
    double s2 = 0.0;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const double d = ok[e] ? (double)f[e] - mu : 0.0;
      s2 = __builtin_fma(d, d, s2);
    }
    const double rstd = rstd_f64(block_row_sum(s2, red_d[1], nw), a.hidden, a.eps);
#pragma unroll
    for (int e = 0; e < K; ++e) {
      double t = ((double)f[e] - mu) * rstd;
      if constexpr (PK != PK_NONE && HB) t = __builtin_fma(t, (double)wv[e], (double)bv[e]);
      else if constexpr (PK != PK_NONE) t = t * (double)wv[e];
      else if constexpr (HB) t = t + (double)bv[e];
      y[e] = f64_to_f32(t);
    }
  }
#pragma unroll
  for (int e = 0; e < K; ++e) {
    if (ok[e]) st1_nt<BF16>(a.out, e0 + (int64_t)T * e, y[e]);
  }
}

// Host-side launch of one row operation; picks the kernel shape from the row width and
// alignment. Returns the HIP error of the launch.
template <bool BF16, int OP>
hipError_t launch_row(const RowArgs& a, bool aligned16, hipStream_t stream);

}  // namespace nrm

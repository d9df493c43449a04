// Backward (vector-Jacobian products) of RMSNorm and LayerNorm over the last axis.
//
// Operations (nuvec-core 0.5.0 fast::FastOp, variants RmsNormVjp and LayerNormVjp): given the
// cotangent g of the output, the gradients for x and for the scale w (and the shift b).
// Per row of D features, with r the row's reciprocal standard deviation:
//   RMS  r = 1/sqrt(sum(x^2)/D + eps), c = r^3 * sum(g w x) / D
//        dx = r (g w) - x c,                 dw += g x r
//   LN   mu = sum(x)/D, var = sum((x - mu)^2)/D, r = 1/sqrt(var + eps), xh = (x - mu) r,
//        d = g w, m1 = sum(d)/D, m2 = sum(d xh)/D = r sum((d - m1)(x - mu)) / D
//        dx = r (d - m1 - xh m2),            dw += g xh,   db += g
// All row statistics come from one pass, accumulated in fp64, so a row needs a single
// cross-thread reduction. LN's four sums are taken about pivots from the row (x and d of an
// element of the row: the row pivots of common.hpp), so neither the variance nor m2
// cancels catastrophically when a mean is large against the spread. The statistics and the per-element
// outputs are fp64 because dx is a difference of two terms that can cancel, and the bar is
// one unit in the last place of the result: an fp32 statistic would miss it on a few
// elements per million.
//
// dw and db sum over rows. A block owns a fixed set of rows (vjp_rows and vjp_team: rows
// strided across the blocks; vjp_generic and vjp_elems: a contiguous run) and accumulates its column sums
// in fp64 (registers, or LDS for vjp_rows' dw at 16 elements per thread; each thread always
// holds the same columns); at the end the block writes one fp64 partial row to the caller's
// workspace, and vjp_colsum adds the partial rows in a fixed order. Results are therefore
// identical run to run.
#pragma once

#include "row_kernels.hpp"

namespace nrm {

enum VjpOp : int { VJP_RMS = 0, VJP_LN = 1 };

// Partial rows of the column sums: one per block, at most this many. Fixed (not derived
// from the device) so that the workspace size and the summation order depend only on the
// problem shape.
constexpr int64_t VJP_MAX_PARTIALS = 256;

struct VjpArgs {
  const void* x;
  const void* w;      // may be null (= 1)
  const void* g;
  void* dx;
  double* part_w;     // [blocks][hidden] partial sums for dw, or null (dw not wanted)
  double* part_b;     // [blocks][hidden] partial sums for db (LN), or null
  int64_t rows;
  int64_t hidden;     // < 2^31
  int64_t rpb;        // rows per block, at most
  double inv_n;       // 1 / hidden
  float eps;
  int w_f32;          // w stored as fp32 (else bf16, only with bf16 activations)
  int team;           // threads per row (fast kernel): a multiple of 64
};

// Row scalars of one row, from its sums (two for RMS, four for LN).
struct VjpRow {
  double r;    // reciprocal standard deviation
  double c;    // RMS: r^3 sum(g w x) / D
  double mu;   // LN
  double m1;   // LN: mean(d)
  double m2;   // LN: mean(d xh)
};

__device__ __forceinline__ VjpRow vjp_rms_scalars(double ss, double dot, double inv_n, float eps) {
  VjpRow s;
  s.r = rsqrt_row(ss * inv_n + (double)eps);
  s.c = s.r * s.r * s.r * (dot * inv_n);
  s.mu = s.m1 = s.m2 = 0.0;
  return s;
}

// LN from its sums about the pivots px (of x) and pd (of d = g w): sx = sum(x - px),
// sxx = sum((x - px)^2), sd = sum(d - pd), sdx = sum((d - pd)(x - px)). With qx = mean(x) -
// px and qd = mean(d) - pd: var = sxx/D - qx^2 and sum((d - m1)(x - mu))/D = sdx/D - qx qd.
__device__ __forceinline__ VjpRow vjp_ln_scalars(double sx, double sxx, double sd, double sdx,
                                                 double px, double pd, double inv_n, float eps) {
  VjpRow s;
  const double qx = sx * inv_n, qd = sd * inv_n;
  s.mu = px + qx;
  const double v0 = sxx * inv_n - qx * qx;
  const double var = v0 < 0.0 ? 0.0 : v0;  // clamps rounding, keeps a NaN (inf - inf)
  s.r = rsqrt_row(var + (double)eps);
  s.c = 0.0;
  s.m1 = pd + qd;
  s.m2 = s.r * __builtin_fma(-qx, qd, sdx * inv_n);
  return s;
}

// Statistic sums of V elements, all accumulated in fp64: RMS (sum x^2, sum g w x), LN (sum
// x - px, sum (x - px)^2, sum d - pd, sum (d - pd)(x - px)) with d = g w about the pivots
// px, pd. XF: x, g and w are bf16 values (8 significant bits), so x^2, g w and g w x are
// exact in fp32 and only need widening; otherwise the products are formed in fp64 (exact up
// to one rounding of g w x). on(e): element e belongs to the row. RMS takes masked elements
// as zeros, which add nothing; LN's shifted terms of a masked element are set to zero.
template <int OP, int V, bool XF, typename ON>
__device__ __forceinline__ void vjp_accumulate(const float (&f)[V], const float (&gv)[V],
                                               const float (&wv)[V], double (&ds)[4],
                                               double px, double pd, ON on) {
#pragma unroll
  for (int e = 0; e < V; ++e) {
    if constexpr (OP == VJP_RMS) {
      if constexpr (XF) {
        // x^2 and (g w) x are exact products either way; the fused form spares the fp32
        // multiplies and rounds only the sums, as before.
        const double xd = (double)f[e];
        ds[0] = __builtin_fma(xd, xd, ds[0]);
        ds[1] = __builtin_fma((double)(gv[e] * wv[e]), xd, ds[1]);
      } else {
        const double xd = (double)f[e];
        ds[0] = __builtin_fma(xd, xd, ds[0]);
        ds[1] = __builtin_fma((double)gv[e] * (double)wv[e], xd, ds[1]);
      }
    } else {
      const double d = XF ? (double)(gv[e] * wv[e]) : (double)gv[e] * (double)wv[e];
      const bool in = on(e);
      const double xs = in ? (double)f[e] - px : 0.0;
      const double dd = in ? d - pd : 0.0;
      ds[0] += xs;
      ds[1] = __builtin_fma(xs, xs, ds[1]);
      ds[2] += dd;
      ds[3] = __builtin_fma(dd, xs, ds[3]);
    }
  }
}

// Every element of the row counts (chunks wholly inside the row).
struct AllOn {
  __device__ __forceinline__ bool operator()(int) const { return true; }
};
// Every element of a chunk counts or none does.
struct ChunkOn {
  bool on;
  __device__ __forceinline__ bool operator()(int) const { return on; }
};

// LN's pivots of a row: px = x and pd = d = g w (formed as vjp_accumulate forms d) of one
// element of the row (x0, g0, w0), the same in every thread of the row.
template <bool XF>
__device__ __forceinline__ void vjp_pivots(float x0, float g0, float w0, double& px, double& pd) {
  px = (double)x0;
  pd = XF ? (double)(g0 * w0) : (double)g0 * (double)w0;
}

// w at column 0 (1 when absent), read once per kernel through the scalar cache.
template <bool BF16>
__device__ __forceinline__ float vjp_w0(const VjpArgs& a) {
  if (a.w == nullptr) return 1.f;
  return (!BF16 || a.w_f32) ? sload_elem<false>(a.w, 0) : sload_elem<true>(a.w, 0);
}

// A thread's V column accumulators in LDS, element e at p[e * stride] (element-major, so
// that the lanes of a wave touch consecutive doubles).
struct LdsCols {
  double* p;
  int stride;
  __device__ __forceinline__ double& operator[](int e) const { return p[e * stride]; }
};

// dx of V elements, and the dw / db column accumulators (registers, or LdsCols), in fp64.
template <int OP, int V, bool DW, bool DB, bool XF, typename AW, typename AB>
__device__ __forceinline__ void vjp_outputs(const float (&f)[V], const float (&gv)[V],
                                            const float (&wv)[V], const VjpRow& s,
                                            float (&dxv)[V], AW accw, AB accb) {
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const double xd = (double)f[e];
    const double gd = (double)gv[e];
    const double d = XF ? (double)(gv[e] * wv[e]) : gd * (double)wv[e];
    // Four elements at a time: converting all eight to fp64 together costs more registers
    // than the loads kept in flight can spare.
    if (e == 4) __builtin_amdgcn_sched_barrier(0);
    if constexpr (OP == VJP_RMS) {
      dxv[e] = f64_to_f32(__builtin_fma(s.r, d, -(xd * s.c)));
      if constexpr (DW) {
        const double gx = XF ? (double)(gv[e] * f[e]) : gd * xd;
        accw[e] = __builtin_fma(gx, s.r, accw[e]);
      }
    } else {
      // d - m1 as one fma: g w is exact in fp64 (bf16 or fp32 values), so this is the
      // exact difference rounded once, as (d - m1) from the exact d would be; it is exactly
      // 0 where d equals its row mean (a one-element row).
      const double xh = (xd - s.mu) * s.r;
      const double dm = __builtin_fma(gd, (double)wv[e], -s.m1);
      dxv[e] = f64_to_f32(__builtin_fma(-xh, s.m2, dm) * s.r);
      if constexpr (DW) accw[e] = __builtin_fma(gd, xh, accw[e]);
      if constexpr (DB) accb[e] += gd;
    }
  }
}

// team_sum4 (common.hpp) in three parts, with the same arithmetic in the same order, so
// that a caller can put work between the barrier and the use of the sums: post (each wave's
// four totals to red), then after the caller's barrier read (this lane's team slot), then
// finish (the team totals, read from lanes 0 .. 3 into every lane).
__device__ __forceinline__ void team_sum4_post(const double (&s)[4], double* red) {
  const int lane = threadIdx.x & 63;
  const bool b = lane & 1, c = lane & 2;
  double k0 = b ? s[1] : s[0], u0 = b ? s[0] : s[1];
  double k1 = b ? s[3] : s[2], u1 = b ? s[2] : s[3];
  k0 += dpp<DPP_QUAD_XOR1>(u0);
  k1 += dpp<DPP_QUAD_XOR1>(u1);
  double k = c ? k1 : k0;
  const double u = c ? k0 : k1;
  k += dpp<DPP_QUAD_XOR2>(u);
  k = lanes_sum_mod4(k);
  if (lane < 4) red[(threadIdx.x >> 6) * 4 + lane] = k;
}

__device__ __forceinline__ double team_sum4_read(const double* red, int wave0, int nwt) {
  const int lane = threadIdx.x & 63;
  const int w = lane >> 2;
  return w < nwt ? red[(wave0 + w) * 4 + (lane & 3)] : 0.0;
}

__device__ __forceinline__ void team_sum4_finish(double t, double (&s)[4]) {
  t = lanes_sum_mod4(t);
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = readlane_f64(t, i);
}

// The same for two sums (RMS): lanes pair up (lane l keeps sum l & 1 of the pair), the rest
// of the wave reduction keeps a lane's parity, and each wave posts two totals; after the
// barrier lanes 0 .. 2 nwt - 1 hold the team's posted values (nwt <= 16) and the parity
// classes of the lower 32 lanes are summed. Lanes 0 and 1 end with the two team totals.
__device__ __forceinline__ void team_sum2_post(double s0, double s1, double* red) {
  const int lane = threadIdx.x & 63;
  const bool b = lane & 1;
  double k = b ? s1 : s0;
  const double u = b ? s0 : s1;
  k += dpp<DPP_QUAD_XOR1>(u);
  k += dpp<DPP_QUAD_XOR2>(k);
  k = lanes_sum_mod4(k);
  if (lane < 2) red[(threadIdx.x >> 6) * 2 + lane] = k;
}

__device__ __forceinline__ double team_sum2_read(const double* red, int wave0, int nwt) {
  const int lane = threadIdx.x & 63;
  const int w = lane >> 1;
  return w < nwt ? red[(wave0 + w) * 2 + (lane & 1)] : 0.0;
}

__device__ __forceinline__ void team_sum2_finish(double t, double (&s)[2]) {
  t += dpp<DPP_QUAD_XOR2>(t);
  t += dpp<DPP_ROW_ROR4>(t);
  t += dpp<DPP_ROW_ROR8>(t);
  t = swap_sum<16>(t);
  s[0] = readlane_f64(t, 0);
  s[1] = readlane_f64(t, 1);
}

// A value every lane holds, moved to scalar registers (the compiler cannot tell that the
// lanes agree).
__device__ __forceinline__ double uniform_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ VjpRow vjp_row_uniform(VjpRow s) {
  s.r = uniform_f64(s.r);
  s.c = uniform_f64(s.c);
  s.mu = uniform_f64(s.mu);
  s.m1 = uniform_f64(s.m1);
  s.m2 = uniform_f64(s.m2);
  return s;
}

// Fast kernel: a block of G teams of T = a.team threads (G * T = blockDim.x); a team owns
// one row at a time, thread t of a team keeping chunks t, t + T, ... (NV of them) of the
// row in registers. With P blocks, step it of team i of block b takes row (it G + i) P + b:
// the blocks walk the rows strided, so that at any moment the grid streams a contiguous
// window of the arrays (blocks that each walked a contiguous run of rows read addresses a
// run apart, which measured slower). Every team runs the same number of iterations (a team
// past the end reloads the last row and discards it), so the block barriers line up. EXACT: T * NV
// chunks cover the row; otherwise chunk indexes past the end are clamped for loads and their results
// dropped. PG: parameter gradients wanted (dw for RMS; dw and db for LN).
template <bool BF16, int OP, int NV, int PK, bool EXACT, bool PG>
__global__ void __launch_bounds__(1024)
vjp_rows(VjpArgs a) {
  constexpr bool DW = PG, DB = PG && OP == VJP_LN;
  constexpr bool XF = BF16 && PK != PK_F32;
  constexpr int V = Fmt<BF16>::VEC;
  // LW: 16 elements per thread (rows of up to 16384 with one 1024-thread team, G = 1): the
  // dw accumulators live in LDS, NV * V * T doubles (128 KB at T = 1024), since in
  // registers beside LN's db they would spill.
  constexpr bool LW = DW && NV * V >= 16;
  __shared__ double red[2][16 * 4];          // [iteration parity][wave * sums + sum]
  extern __shared__ double comb[];           // (G - 1) * T * V doubles (team combine), or
                                             // LW: the dw accumulators
  const int T = a.team;
  const int G = blockDim.x / T;
  // T is a multiple of 64, so a wave belongs to one team: the team index, its rows and their
  // addresses are scalars.
  const int team = __builtin_amdgcn_readfirstlane(threadIdx.x / T);
  const int tid = threadIdx.x - team * T;
  const int nwt = T >> 6;                    // waves per team
  const int wave0 = team * nwt;
  const int nvec = (int)(a.hidden / V);
  const int iters = (int)((a.rpb + G - 1) / G);

  int jj[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = tid + k * T;
    ok[k] = EXACT || j < nvec;
    jj[k] = EXACT ? j : min(j, nvec - 1);
  }
  // bf16 w of LayerNorm rows at 16 elements per thread stays packed (8 registers rather than
  // 16) and is widened at each use.
  constexpr bool PACK_W = BF16 && PK == PK_SAME && OP == VJP_LN && NV * V >= 16;
  float wv[NV][V];
  u32x4 wpk[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if constexpr (PACK_W) wpk[k] = ld16((const uint16_t*)a.w + (int64_t)jj[k] * V);
    else load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wv[k]);
  }
  double accw[NV][V], accb[NV][V];
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < V; ++e) accw[k][e] = accb[k][e] = 0.0;
  // LW: element e of chunk k of this thread's columns at comb[(k V + e) T + tid]; each
  // thread reads and writes only its own slots, so no barrier orders them.
  auto lw_cols = [&](int k) { return LdsCols{comb + (k * V) * T + tid, T}; };
  if constexpr (LW) {
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int e = 0; e < V; ++e) lw_cols(k)[e] = 0.0;
  }
  // fp32 parameters beside bf16 data take fp64 products with g, and the compiler would hold
  // their fp64 conversions (16 registers) across the loop, which spilled it to scratch.
  // With 16 elements per thread w is read again (an L2 hit) at each use; at ragged widths
  // with fewer, an opaque copy at each use makes it convert them again (8 instructions a
  // row; at whole-wave widths holding them measured faster). LayerNorm's outputs convert w
  // as well, and it takes the opaque copy for bf16 rows at up to 8 elements per thread (spills
  // 47 registers -> 7; [16384, 4096] 110 -> 104 us) and fp32 rows at 16 ([8192, 16384]
  // 690 -> 546 us); bf16 rows at 16 and fp32 rows at up to 8 measured slower with it.
  constexpr bool OPAQUE_W = (PK == PK_F32 && !EXACT) ||
                            (OP == VJP_LN && PK != PK_NONE && (BF16 == (NV * V < 16)));
  auto wuse = [&](int k, float (&wl)[V]) {
    if constexpr (PK == PK_F32 && NV * V >= 16) {
      load_pk<BF16, PK, V>(a.w, (int64_t)jj[k] * V, wl);
      return;
    }
    if constexpr (PACK_W) {
      u32x4 wr = wpk[k];
      __asm__ volatile("" : "+v"(wr));
      unpack<true>(wr, wl);
      return;
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      wl[e] = wv[k][e];
      if constexpr (OPAQUE_W) __asm__ volatile("" : "+v"(wl[e]));
    }
  };

  auto row_of = [&](int it) {
    return ((int64_t)it * G + team) * (int64_t)gridDim.x + blockIdx.x;
  };
  // LN: w at column 0, for the rows' d pivots.
  const float w0 = OP == VJP_LN ? vjp_w0<BF16>(a) : 1.f;
  // A row's chunks, and (LN) its pivots x and g at column 0 through the scalar cache (scalar
  // registers: nothing held in vector registers while the row is in flight).
  struct Piv { float x, g; };
  auto load_row = [&](int it, u32x4 (&xv)[NV], u32x4 (&gv)[NV], Piv& pv) {
    const int64_t row = min(row_of(it), a.rows - 1);
    const char* xr = (const char*)a.x + row * a.hidden * Fmt<BF16>::ESZ;
    const char* gr = (const char*)a.g + row * a.hidden * Fmt<BF16>::ESZ;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      xv[k] = ld16_nt(xr + (int64_t)jj[k] * 16);
      gv[k] = ld16_nt(gr + (int64_t)jj[k] * 16);
    }
    if constexpr (OP == VJP_LN) {
      pv.x = sload_elem<BF16>(xr, 0);
      pv.g = sload_elem<BF16>(gr, 0);
    }
  };

  // Statistics of a row: its sums (LN: about the row's pivots, which are returned), reduced
  // within each wave and posted to red[it & 1].
  struct RowPiv { double x, d; };
  auto stats = [&](int it, const u32x4 (&xv)[NV], const u32x4 (&gv)[NV], const Piv& pv) {
    double ds[4] = {0.0, 0.0, 0.0, 0.0};
    double px = 0.0, pd = 0.0;
    if constexpr (OP == VJP_LN) vjp_pivots<XF>(pv.x, pv.g, w0, px, pd);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if constexpr (EXACT) {
        if (ok[k]) {
          float f[V], gf[V], wl[V];
          unpack<BF16>(xv[k], f);
          unpack<BF16>(gv[k], gf);
          if constexpr (PACK_W) wuse(k, wl);
          vjp_accumulate<OP, V, XF>(f, gf, PACK_W ? wl : wv[k], ds, px, pd, AllOn{});
        }
      } else {
        // A chunk past the row's end (a clamped duplicate) enters as zeros, which add
        // exactly nothing to any sum: a select rather than a branch, which kept the ring's
        // registers live around it and spilled them to scratch.
        const u32x4 z = u32x4{0, 0, 0, 0};
        float f[V], gf[V], wl[V];
        unpack<BF16>(ok[k] ? xv[k] : z, f);
        unpack<BF16>(ok[k] ? gv[k] : z, gf);
        wuse(k, wl);
        vjp_accumulate<OP, V, XF>(f, gf, wl, ds, px, pd, ChunkOn{ok[k]});
      }
    }
    if constexpr (OP == VJP_RMS) team_sum2_post(ds[0], ds[1], red[it & 1]);
    else team_sum4_post(ds, red[it & 1]);
    return RowPiv{px, pd};
  };
  // After that barrier: this lane's slot of the posted sums (with the row's pivots).
  struct Posted { double t, px, pd; };
  auto sums_read = [&](int it, const RowPiv& rp) {
    Posted p{0.0, rp.x, rp.d};
    if constexpr (OP == VJP_RMS) p.t = team_sum2_read(red[it & 1], wave0, nwt);
    else p.t = team_sum4_read(red[it & 1], wave0, nwt);
    return p;
  };
  // Then the row's scalars, the same in every lane.
  auto scalars = [&](const Posted& p) {
    VjpRow s;
    if constexpr (OP == VJP_RMS) {
      double ds[2];
      team_sum2_finish(p.t, ds);
      s = vjp_rms_scalars(ds[0], ds[1], a.inv_n, a.eps);
    } else {
      double ds[4];
      team_sum4_finish(p.t, ds);
      s = vjp_ln_scalars(ds[0], ds[1], ds[2], ds[3], p.px, p.pd, a.inv_n, a.eps);
    }
    return vjp_row_uniform(s);
  };
  // dx of a row, and its dw / db terms.
  auto outputs = [&](int it, const u32x4 (&xv)[NV], const u32x4 (&gv)[NV], const VjpRow& s) {
    const int64_t row = row_of(it);
    if (row >= a.rows) return;
    char* dr = (char*)a.dx + row * a.hidden * Fmt<BF16>::ESZ;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      // Re-derive the elements from the raw chunks: the opaque copy stops the compiler from
      // keeping the statistic pass's fp64 conversions alive across the barrier, which
      // costs more registers than converting again.
      u32x4 xr = xv[k], gr = gv[k];
      __asm__ volatile("" : "+v"(xr), "+v"(gr));
      float f[V], gf[V], dxv[V], wl[V];
      unpack<BF16>(xr, f);
      unpack<BF16>(gr, gf);
      wuse(k, wl);
      if constexpr (LW) vjp_outputs<OP, V, DW, DB, XF>(f, gf, wl, s, dxv, lw_cols(k), accb[k]);
      else vjp_outputs<OP, V, DW, DB, XF>(f, gf, wl, s, dxv, accw[k], accb[k]);
      if (ok[k]) st16_nt(dr + (int64_t)jj[k] * 16, pack<BF16>(dxv));
    }
  };

  if constexpr (NV > 1) {
    // Two chunks per thread and the column accumulators leave no registers for the ring
    // below: one buffer pair, the next row copied in after each row, and each row's
    // statistics, barrier and outputs in turn.
    // LayerNorm at 16 elements per thread loads each row at the top of its own step instead
    // (NOPF): the next row's buffers beside the current one's and the db column sums spilled
    // ~60 registers.
    constexpr bool NOPF = OP == VJP_LN && NV * V >= 16;
    u32x4 xa[NV], ga[NV];
    Piv pa{0.f, 0.f};
    if constexpr (!NOPF) load_row(0, xa, ga, pa);
    for (int it = 0; it < iters; ++it) {
      u32x4 xb[NV], gb[NV];
      Piv pb{0.f, 0.f};
      if constexpr (NOPF) load_row(it, xa, ga, pa);
      else if (it + 1 < iters) load_row(it + 1, xb, gb, pb);
      const RowPiv rp = stats(it, xa, ga, pa);
      __syncthreads();
      const VjpRow s = scalars(sums_read(it, rp));
      outputs(it, xa, ga, s);
      if (!NOPF && it + 1 < iters) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          xa[k] = xb[k];
          ga[k] = gb[k];
        }
        pa = pb;
      }
    }
  } else {
    // Software pipeline over a ring of R row buffers. Step it loads row it + R - 1 into the
    // buffer row it - 1 has released, posts the statistics of row it + 1, passes the
    // barrier, issues the LDS reads of those sums, writes the outputs of row it (whose
    // scalars the previous step finished) while the reads are in flight, and only then
    // finishes the scalars of row it + 1. The barrier's latency thus overlaps a row's
    // output arithmetic instead of stalling every wave of the block. The loop is unrolled
    // by R so that each buffer keeps its registers: copying a buffer that is still being
    // loaded would wait for the load.
    // LayerNorm keeps three rows in flight where a fourth buffer spilled: bf16 rows
    // ([65536, 1024] 115 -> 107 us at three), fp32 parameters beside bf16 data, ragged widths.
    // fp32 rows at whole widths keep four ([16384, 4096] 144 us, 149 at three).
    constexpr int R = OP == VJP_LN && (BF16 || PK == PK_F32 || !EXACT) ? 3 : 4;
    u32x4 xs[R][NV], gs[R][NV];
    Piv ps[R];
#pragma unroll
    for (int q = 0; q < R - 1; ++q) load_row(q, xs[q], gs[q], ps[q]);
    RowPiv rp = stats(0, xs[0], gs[0], ps[0]);
    __syncthreads();
    VjpRow s = scalars(sums_read(0, rp));
    auto step = [&](int it, int q, bool load, bool next) {
      if (load) load_row(it + R - 1, xs[(q + R - 1) % R], gs[(q + R - 1) % R], ps[(q + R - 1) % R]);
      Posted t{0.0, 0.0, 0.0};
      if (next) {
        const RowPiv np = stats(it + 1, xs[(q + 1) % R], gs[(q + 1) % R], ps[(q + 1) % R]);
        __syncthreads();
        t = sums_read(it + 1, np);
      }
      outputs(it, xs[q], gs[q], s);
      if (next) s = scalars(t);
    };
    int it0 = 0;
    for (; it0 + 2 * R - 1 <= iters; it0 += R) {
#pragma unroll
      for (int q = 0; q < R; ++q) step(it0 + q, q, true, true);
    }
    // The last rows (fewer than 2R - 1): loads and statistics only for rows that exist.
#pragma unroll
    for (int q = 0; q < 2 * R - 2; ++q) {
      const int it = it0 + q;
      if (it >= iters) break;
      step(it, q % R, it + R - 1 < iters, it + 1 < iters);
    }
  }

  if constexpr (DW || DB) {
    // Team 0 adds teams 1 .. G-1 (in that order) through LDS, one chunk slot at a time,
    // then writes the block's partial row.
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if ((pass == 0 && !DW) || (pass == 1 && !DB)) continue;
      double (&acc)[NV][V] = pass == 0 ? accw : accb;
      double* part = (pass == 0 ? a.part_w : a.part_b) + (int64_t)blockIdx.x * a.hidden;
      if (LW && pass == 0) {  // one team per block: its LDS columns are the partial row
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          if (ok[k]) {
            double* p = part + (int64_t)jj[k] * V;
#pragma unroll
            for (int e = 0; e < V; ++e) p[e] = lw_cols(k)[e];
          }
        }
        continue;
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if (G > 1) {
          __syncthreads();
          if (team > 0) {
            double* slot = comb + ((int64_t)(team - 1) * T + tid) * V;
#pragma unroll
            for (int e = 0; e < V; ++e) slot[e] = acc[k][e];
          }
          __syncthreads();
          if (team == 0) {
            for (int q = 1; q < G; ++q) {
              const double* slot = comb + ((int64_t)(q - 1) * T + tid) * V;
#pragma unroll
              for (int e = 0; e < V; ++e) acc[k][e] += slot[e];
            }
          }
        }
        if (team == 0 && ok[k]) {
          double* p = part + (int64_t)jj[k] * V;
#pragma unroll
          for (int e = 0; e < V; ++e) p[e] = acc[k][e];
        }
      }
    }
  }
}

// Narrow rows (at most 32 chunks): a team of SUB = 8, 16 or 32 lanes per row, one chunk per
// lane, 1024 / SUB teams per 1024-thread block (the grid is one block per partial row, at
// most 256, so the block has to fill the compute unit). With P blocks, step it of team i of
// block b takes row (it (1024 / SUB) + i) P + b, as in vjp_rows. A row's sums are lane
// exchanges inside the team (no LDS, no barrier); the next row's chunks are loaded while the
// current one is computed (two buffers, the loop unrolled by two so that no buffer is
// copied). A team past the last row computes on a clamped row and neither stores nor
// accumulates it. At the end the teams' column sums meet in LDS and are added in team order
// into the block's partial row.
template <bool BF16, int OP, int PK, bool EXACT, int SUB, bool PG>
__global__ void __launch_bounds__(1024)
vjp_team(VjpArgs a) {
  constexpr bool DW = PG, DB = PG && OP == VJP_LN;
  constexpr bool XF = BF16 && PK != PK_F32;
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int TB = 1024 / SUB;             // teams per block
  __shared__ double comb[1024 * V];          // [thread][element], the column sums' meeting
  const int team = threadIdx.x / SUB;
  const int tid = threadIdx.x & (SUB - 1);
  const int nvec = (int)(a.hidden / V);
  const int iters = (int)((a.rpb + TB - 1) / TB);
  const bool ok = EXACT || tid < nvec;
  const int jj = EXACT ? tid : min(tid, nvec - 1);
  float wv[V];
  load_pk<BF16, PK, V>(a.w, (int64_t)jj * V, wv);
  double accw[V], accb[V];
#pragma unroll
  for (int e = 0; e < V; ++e) accw[e] = accb[e] = 0.0;

  auto row_of = [&](int it) {
    return ((int64_t)it * TB + team) * (int64_t)gridDim.x + blockIdx.x;
  };
  auto load = [&](int it, u32x4& xv, u32x4& gv) {
    const int64_t row = min(row_of(it), a.rows - 1);
    xv = ld16_nt((const char*)a.x + (row * a.hidden + (int64_t)jj * V) * Fmt<BF16>::ESZ);
    gv = ld16_nt((const char*)a.g + (row * a.hidden + (int64_t)jj * V) * Fmt<BF16>::ESZ);
  };
  auto process = [&](int it, const u32x4& xv, const u32x4& gv) {
    const int64_t row = row_of(it);
    const u32x4 z = u32x4{0, 0, 0, 0};
    // LN: the row's pivots, x, g and w at column 0, which the team's first lane holds.
    double px = 0.0, pd = 0.0;
    if constexpr (OP == VJP_LN) {
      auto first = [](float v) {
        return __builtin_bit_cast(float, group_first<SUB>(__builtin_bit_cast(uint32_t, v)));
      };
      vjp_pivots<XF>(first(first_elem<BF16>(xv[0])), first(first_elem<BF16>(gv[0])), first(wv[0]),
                     px, pd);
    }
    float f[V], gf[V];
    unpack<BF16>(ok ? xv : z, f);  // a lane past the row's end adds nothing to the sums
    unpack<BF16>(ok ? gv : z, gf);
    double ds[4] = {0.0, 0.0, 0.0, 0.0};
    vjp_accumulate<OP, V, XF>(f, gf, wv, ds, px, pd, ChunkOn{ok});
    VjpRow s;
    if constexpr (OP == VJP_RMS) {
      s = vjp_rms_scalars(group_sum<SUB>(ds[0]), group_sum<SUB>(ds[1]), a.inv_n, a.eps);
    } else {
      s = vjp_ln_scalars(group_sum<SUB>(ds[0]), group_sum<SUB>(ds[1]), group_sum<SUB>(ds[2]),
                         group_sum<SUB>(ds[3]), px, pd, a.inv_n, a.eps);
    }
    if (row >= a.rows) return;
    u32x4 xr = xv, gr = gv;
    __asm__ volatile("" : "+v"(xr), "+v"(gr));  // widen again rather than hold the fp64 copies
    float dxv[V];
    unpack<BF16>(xr, f);
    unpack<BF16>(gr, gf);
    vjp_outputs<OP, V, DW, DB, XF>(f, gf, wv, s, dxv, accw, accb);
    if (ok) st16_nt((char*)a.dx + (row * a.hidden + (int64_t)jj * V) * Fmt<BF16>::ESZ,
                    pack<BF16>(dxv));
  };

  u32x4 xa, ga, xb, gb;
  if (iters > 0) load(0, xa, ga);
  for (int it = 0; it < iters; it += 2) {
    if (it + 1 < iters) load(it + 1, xb, gb);
    process(it, xa, ga);
    if (it + 1 >= iters) break;
    if (it + 2 < iters) load(it + 2, xa, ga);
    process(it + 1, xb, gb);
  }

  if constexpr (DW || DB) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if ((pass == 0 && !DW) || (pass == 1 && !DB)) continue;
      const double* acc = pass == 0 ? accw : accb;
      if (pass == 1) __syncthreads();  // the dw pass has read its slots
#pragma unroll
      for (int e = 0; e < V; ++e) comb[threadIdx.x * V + e] = acc[e];
      __syncthreads();
      if (team == 0 && ok) {
        double t[V];
#pragma unroll
        for (int e = 0; e < V; ++e) t[e] = comb[tid * V + e];
        for (int q = 1; q < TB; ++q) {
#pragma unroll
          for (int e = 0; e < V; ++e) t[e] += comb[(q * SUB + tid) * V + e];
        }
        double* p = (pass == 0 ? a.part_w : a.part_b) + (int64_t)blockIdx.x * a.hidden +
                    (int64_t)jj * V;
#pragma unroll
        for (int e = 0; e < V; ++e) p[e] = t[e];
      }
    }
  }
}

// Generic kernel: any row width, V elements per access (VEC for 16-byte aligned rows, else
// 1). One 256-thread block per run of rows; each row is read twice (the second pass mostly
// from L2), and the block's partial row in the workspace is updated in place by the thread
// that owns each column (the same thread for every row, so no other thread touches it).
template <bool BF16, int OP, int V, bool PG>
__global__ void __launch_bounds__(256)
vjp_generic(VjpArgs a) {
  constexpr bool DW = PG, DB = PG && OP == VJP_LN;
  __shared__ double red[4 * 4];
  const int64_t nch = a.hidden / V;
  const bool has_w = a.w != nullptr;
  const bool xf = BF16 && !a.w_f32;  // exact fp32 products (see vjp_accumulate)
  const int64_t row0 = (int64_t)blockIdx.x * a.rpb;
  const int64_t row_end = min(a.rows, row0 + a.rpb);
  double* pw = DW ? a.part_w + (int64_t)blockIdx.x * a.hidden : nullptr;
  double* pb = DB ? a.part_b + (int64_t)blockIdx.x * a.hidden : nullptr;

  const float w0 = OP == VJP_LN ? vjp_w0<BF16>(a) : 1.f;
  for (int64_t row = row0; row < row_end; ++row) {
    const int64_t e0 = row * a.hidden;
    double ds[4] = {0.0, 0.0, 0.0, 0.0};
    // LN: the row's pivots (x and d = g w at column 0).
    double px = 0.0, pd = 0.0;
    if constexpr (OP == VJP_LN) {
      const float x0 = sload_elem<BF16>(a.x, e0), g0 = sload_elem<BF16>(a.g, e0);
      if (xf) vjp_pivots<BF16>(x0, g0, w0, px, pd);
      else vjp_pivots<false>(x0, g0, w0, px, pd);
    }
    for (int64_t j = threadIdx.x; j < nch; j += 256) {
      float f[V], gf[V], wv[V];
      load_act<BF16, V>(a.x, e0 + j * V, f);
      load_act<BF16, V>(a.g, e0 + j * V, gf);
      if (has_w) {
        load_param<BF16, V>(a.w, a.w_f32, j * V, wv);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) wv[e] = 1.f;
      }
      if (xf) vjp_accumulate<OP, V, BF16>(f, gf, wv, ds, px, pd, AllOn{});
      else vjp_accumulate<OP, V, false>(f, gf, wv, ds, px, pd, AllOn{});
    }
    team_sum4(ds, red, 0, 4);
    __syncthreads();  // red is rewritten by the next row
    VjpRow s;
    if constexpr (OP == VJP_RMS) s = vjp_rms_scalars(ds[0], ds[1], a.inv_n, a.eps);
    else s = vjp_ln_scalars(ds[0], ds[1], ds[2], ds[3], px, pd, a.inv_n, a.eps);
    const bool first = row == row0;
    for (int64_t j = threadIdx.x; j < nch; j += 256) {
      float f[V], gf[V], wv[V], dxv[V];
      load_act<BF16, V>(a.x, e0 + j * V, f);
      load_act<BF16, V>(a.g, e0 + j * V, gf);
      if (has_w) {
        load_param<BF16, V>(a.w, a.w_f32, j * V, wv);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) wv[e] = 1.f;
      }
      double aw[V], ab[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        aw[e] = (DW && !first) ? pw[j * V + e] : 0.0;
        ab[e] = (DB && !first) ? pb[j * V + e] : 0.0;
      }
      if (xf) vjp_outputs<OP, V, DW, DB, BF16>(f, gf, wv, s, dxv, aw, ab);
      else vjp_outputs<OP, V, DW, DB, false>(f, gf, wv, s, dxv, aw, ab);
      store_act<BF16, V>(a.dx, e0 + j * V, dxv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if constexpr (DW) pw[j * V + e] = aw[e];
        if constexpr (DB) pb[j * V + e] = ab[e];
      }
    }
  }
}

// Rows of up to 8192 elements, in single elements (for widths that are not whole 16-byte
// chunks, or rows that do not start on a 16-byte boundary). One block of T threads per run
// of rows; thread t holds the K elements at columns t + T e of a row (so a wave's loads are
// consecutive elements), and its dw / db column sums in registers for the whole run. Each
// row is read once, and the loads of the next rows (one to three, as the registers allow)
// are in flight during the current row's reduction. XF: bf16 x, g and w (exact fp32
// products, see vjp_accumulate). At 8 elements per thread the dw and db sums live in LDS
// (LW, K * T doubles each, element-major): in registers, LN's 32 accumulator registers push
// the kernel into scratch.
template <bool BF16, int OP, int K, bool PG, bool XF>
__global__ void __launch_bounds__(1024)
vjp_elems(VjpArgs a) {
  constexpr bool DW = PG, DB = PG && OP == VJP_LN;
  constexpr bool LW = DW && K >= 8, LB = DB && K >= 8;
  __shared__ double red[2][16 * 4];
  extern __shared__ double colw[];
  const int T = blockDim.x;
  const int tid = threadIdx.x;
  const int64_t H = a.hidden;
  const int64_t row0 = (int64_t)blockIdx.x * a.rpb;
  const int64_t row_end = min(a.rows, row0 + a.rpb);
  bool ok[K];
  float wv[K];
  double aw[K], ab[K];
#pragma unroll
  for (int e = 0; e < K; ++e) {
    const int64_t c = tid + (int64_t)T * e;
    ok[e] = e < K - 1 || c < H;  // the launch keeps T (K - 1) <= H
    float t[1] = {1.f};
    if (ok[e] && a.w != nullptr) load_param<BF16, 1>(a.w, a.w_f32, c, t);
    wv[e] = ok[e] ? t[0] : 0.f;
    aw[e] = ab[e] = 0.0;
  }
  // This thread's columns, touched by no other thread: no barrier needed.
  const LdsCols lw{colw + tid, T}, lb{colw + K * T + tid, T};
#pragma unroll
  for (int e = 0; e < K; ++e) {
    if constexpr (LW) lw[e] = 0.0;
    if constexpr (LB) lb[e] = 0.0;
  }
  // Ring of R register sets: the loads for row i + R - 1 are issued before row i's sums.
  // LN: with each row's pivots, x and g at column 0, read through the scalar cache.
  constexpr int R = K <= 2 ? 4 : K <= 4 ? 3 : 2;
  float xs[R][K], gs[R][K], pxs[R], pgs[R];
  const float w0 = OP == VJP_LN ? vjp_w0<BF16>(a) : 1.f;
  auto load = [&](int64_t row, float (&xv)[K], float (&gv)[K], float& px0, float& pg0) {
    if constexpr (OP == VJP_LN) {
      px0 = sload_elem<BF16>(a.x, row * H);
      pg0 = sload_elem<BF16>(a.g, row * H);
    }
    const int64_t e0 = row * H + tid;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      float t[1] = {0.f}, u[1] = {0.f};
      if (ok[e]) {
        load_act<BF16, 1>(a.x, e0 + (int64_t)T * e, t);
        load_act<BF16, 1>(a.g, e0 + (int64_t)T * e, u);
      }
      xv[e] = t[0];
      gv[e] = u[0];
    }
  };
  auto on = [&](int e) { return ok[e]; };
  auto step = [&](int64_t row, const float (&xv)[K], const float (&gv)[K], float px0, float pg0,
                  double* rb) {
    double ds[4] = {0.0, 0.0, 0.0, 0.0};
    double px = 0.0, pd = 0.0;
    if constexpr (OP == VJP_LN) vjp_pivots<XF>(px0, pg0, w0, px, pd);
    vjp_accumulate<OP, K, XF>(xv, gv, wv, ds, px, pd, on);
    team_sum4(ds, rb, 0, T >> 6);
    VjpRow s;
    if constexpr (OP == VJP_RMS) s = vjp_rms_scalars(ds[0], ds[1], a.inv_n, a.eps);
    else s = vjp_ln_scalars(ds[0], ds[1], ds[2], ds[3], px, pd, a.inv_n, a.eps);
    float dxv[K];
    if constexpr (LB) vjp_outputs<OP, K, DW, DB, XF>(xv, gv, wv, s, dxv, lw, lb);
    else if constexpr (LW) vjp_outputs<OP, K, DW, DB, XF>(xv, gv, wv, s, dxv, lw, ab);
    else vjp_outputs<OP, K, DW, DB, XF>(xv, gv, wv, s, dxv, aw, ab);
    const int64_t e0 = row * H + tid;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const float t[1] = {dxv[e]};
      if (ok[e]) store_act<BF16, 1>(a.dx, e0 + (int64_t)T * e, t);
    }
  };
  // R rows per trip, so that the register sets are picked at compile time; consecutive rows
  // alternate reduction slots (a slot is rewritten only after the next row's barrier, which
  // every thread reaches after reading it). Loads past the last row repeat the last row, so
  // every load is unconditional.
  if (row0 < row_end) {
#pragma unroll
    for (int i = 0; i < R - 1; ++i) load(min(row0 + i, row_end - 1), xs[i], gs[i], pxs[i], pgs[i]);
  }
  for (int64_t row = row0; row < row_end; row += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (row + i >= row_end) break;
      load(min(row + i + R - 1, row_end - 1), xs[(i + R - 1) % R], gs[(i + R - 1) % R],
           pxs[(i + R - 1) % R], pgs[(i + R - 1) % R]);
      step(row + i, xs[i], gs[i], pxs[i], pgs[i], red[R % 2 == 0 ? i & 1 : (row + i - row0) & 1]);
    }
  }
  if constexpr (PG) {
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const int64_t c = tid + (int64_t)T * e;
      if (!ok[e]) continue;
      if constexpr (DW) a.part_w[(int64_t)blockIdx.x * H + c] = LW ? lw[e] : aw[e];
      if constexpr (DB) a.part_b[(int64_t)blockIdx.x * H + c] = LB ? lb[e] : ab[e];
    }
  }
}

// Column sums of the partial rows: out[c] = sum over p < nparts of part[p][c], added in a
// fixed order (16 interleaved slices, then the slices in order), rounded once to the
// parameter dtype. gridDim.y is the number of outputs (1 or 2); blockIdx.y picks the pair
// (part0, out0) or (part1, out1). The host passes only outputs that were asked for.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256)
vjp_colsum(const double* part0, void* out0, const double* part1, void* out1, int64_t nparts,
           int64_t hidden) {
  __shared__ double red[16][17];
  const double* part = blockIdx.y == 0 ? part0 : part1;
  void* out = blockIdx.y == 0 ? out0 : out1;
  const int c = threadIdx.x & 15;
  const int s = threadIdx.x >> 4;
  const int64_t col = (int64_t)blockIdx.x * 16 + c;
  // nparts <= 256: at most 16 rows per thread, all loaded before any is added (one memory
  // latency instead of sixteen), then added in order.
  static_assert(VJP_MAX_PARTIALS <= 16 * 16, "vjp_colsum covers at most 256 partial rows");
  double v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t p = s + 16 * i;
    v[i] = (col < hidden && p < nparts) ? part[p * hidden + col] : 0.0;
  }
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += v[i];
  red[s][c] = acc;
  __syncthreads();
  if (s == 0 && col < hidden) {
    double t = red[0][c];
#pragma unroll
    for (int q = 1; q < 16; ++q) t += red[q][c];
    if constexpr (OUT_BF16) ((uint16_t*)out)[col] = f32_to_bf16(f64_to_f32(t));
    else ((float*)out)[col] = (float)t;
  }
}

// Host-side launch: picks the kernel and writes dx, and dw / db (either may be null) through
// the workspace. With rows == 0 it only zeroes dw / db.
template <bool BF16, int OP>
hipError_t launch_vjp(const VjpArgs& a, void* dw, void* db, bool aligned16, hipStream_t stream);

// Number of partial rows (and blocks) for `rows` rows: ceil(rows / ceil(rows / 256)).
inline int64_t vjp_partials(int64_t rows) {
  if (rows <= 0) return 0;
  const int64_t p = rows < VJP_MAX_PARTIALS ? rows : VJP_MAX_PARTIALS;
  const int64_t rpb = (rows + p - 1) / p;
  return (rows + rpb - 1) / rpb;
}

}  // namespace nrm

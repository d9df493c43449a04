// Rotary position embeddings over rows of D features, three layouts sharing one kernel:
//   NormRope  RMS-normalise each [b, h, l] row of a [B, H, L, D] array (all D features, times
//             w), then rotate its first `dims` features at position offset + l; write a new
//             [B, H, L, D] array or rows offset + l of a [B, H, cache_len, D] cache;
//   Rope      the rotation alone on [N, L, D] rows, position offset + l;
//   positions query [T, Hq, D] and key [T, Hk, D] rows rotated in one launch, every head of
//             token t at position positions[t].
//
// Sources: nuvec-core 0.5.0 fast::FastOp, variants NormRope and Rope (optional freqs that
// replace base); the MinivLLM API reference, "Layers", RotaryEmbedding.forward(positions,
// query, key). The rotation is the textbook RoPE (RoFormer, section 3.2): pair i turns by
// a = scale * position * theta_i with theta_i = base^(-2i/dims), or 1 / freqs[i] when a
// freqs vector is given (it holds the divisor of the position for each pair, as in the fast
// rope the pages name); half mode pairs (i, i + dims/2), traditional mode (2i, 2i+1); the
// inverse rotation (forward = 0) turns by -a. mscale multiplies the rotated features (the
// attention factor of the scaled variants; 1 otherwise).
//
// Precision: the angle, theta and sin/cos are fp64 (an fp32 angle at positions in the
// thousands is off by ~1e-4 rad). The rotation of a pair (x_i, x_j) with scales (w_i, w_j)
// runs in fp64, every product exact or rounded once in fp64 (relative ~1e-16), so cancellation
// between its two terms costs nothing at fp32 or bf16 output precision; the row statistic
// (fp32 sum of squares, fp64 rstd) only scales the result. Features at index >= dims get
// x * rstd * w in fp32.
//
// rope_fast: one block per (position l, chunk of rows at that position). The block first
// computes, for every pair at its position, the rotation's coefficients with the scales
// folded in (w_i cos, w_j sin, w_i sin, w_j cos) into LDS, once; then each group of G lanes
// takes rows: in half mode a lane loads the 16-byte chunk at feature j*VEC and its partner
// chunk at dims/2 + j*VEC, so each rotated pair sits in one lane and no lane exchange is
// needed; in traditional mode a chunk holds VEC/2 neighbouring pairs. The row's sum of squares
// is a DPP reduction over the G lanes. Rows with the same l share the LDS table. A lane group
// issues the loads of R rows before computing any of them (memory-level parallelism: a
// 128-wide bf16 row is only 256 bytes); the table is built while the first rows are in
// flight, and every row's stores follow the whole step's arithmetic (storing each row as
// soon as it is done measured 10% slower on NormRope [8, 32, 512, 128]).
// rope_multi: rows of few heads at many positions (fewer than 256 rows per position, at least
// 4096 positions, every feature rotated): a block takes several consecutive positions.
// rope_generic: any D / dims / alignment, one wave per row, element at a time.
#include <algorithm>

#include "rope.hpp"

namespace nrm {

namespace {

// Position of index l: positions[l] when a positions array is given, else offset + l.
__device__ __forceinline__ int64_t rope_position(const RopeArgs& a, int64_t l) {
  if (a.positions == nullptr) return a.offset + l;
  return a.pos_i64 ? ((const int64_t*)a.positions)[l] : (int64_t)((const int32_t*)a.positions)[l];
}

// Frequency of pair t: 1 / freqs[t], or base^(-2t/dims) as 2^(-2t/dims * log2(base)) with
// log2(base) from the host. The exponent's rounding (|exponent| <= log2(base)) leaves theta a
// relative error of a few 1e-15: an angle error of ~1e-10 radians at position 1e5. The
// general fp64 pow would hold ~35 more registers beside the rows in flight.
__device__ __forceinline__ double rope_theta(const RopeArgs& a, int t) {
  if (a.freqs != nullptr) return 1.0 / (double)a.freqs[t];
  return exp2((double)(-2 * t) / (double)a.dims * a.log2_base);
}

// Element offset of row (bh, l) in the input, and in the output.
__device__ __forceinline__ const char* rope_in_row(const RopeArgs& a, int64_t bh, int64_t l,
                                                   int esz) {
  if (bh < a.BH1) return (const char*)a.x + (bh * a.x_sbh + l * a.x_sl) * a.D * esz;
  return (const char*)a.x2 + ((bh - a.BH1) * a.x2_sbh + l * a.x2_sl) * a.D * esz;
}
__device__ __forceinline__ char* rope_out_row(const RopeArgs& a, int64_t bh, int64_t l, int esz) {
  if (bh < a.BH1) return (char*)a.out + (bh * a.o_sbh + (a.o_row0 + l) * a.o_sl) * a.D * esz;
  return (char*)a.out2 + ((bh - a.BH1) * a.o2_sbh + l * a.o2_sl) * a.D * esz;
}

// A global-memory address held as an integer, as a pointer that the compiler still knows to
// be global (so that accesses through it are global, not flat, instructions).
__device__ __forceinline__ const char* global_ptr(int64_t v) {
  return (const char*)(const __attribute__((address_space(1))) char*)v;
}

}  // namespace

// sin and cos of a rotation angle in fp64, with few registers (the general library sincos
// carries a large-argument reduction whose registers, live next to a block's in-flight rows,
// cost the kernel half its occupancy). Method: Cody-Waite reduction by pi/2 with pi/2 split
// into three doubles and each step one fused multiply-add, so r = a - k*pi/2 is accurate
// to ~1e-16 absolute for |k| < 2^40; then the Taylor series of sin and cos on
// [-pi/4, pi/4] (terms to r^19 and r^18: truncation below 1e-20) and the quadrant k mod 4.
// The angle itself carries a relative rounding of ~1e-16 from scale * position * theta.
__device__ __forceinline__ void rope_sincos(double a, double* sn, double* cs) {
  constexpr double kTwoOverPi = 0.6366197723675814;
  constexpr double kPio2Hi = 1.5707963267948966;        // pi/2 = hi + mid + lo (to ~1e-49)
  constexpr double kPio2Mid = 6.123233995736766e-17;
  constexpr double kPio2Lo = -1.4973849048591698e-33;
  const double k = __builtin_rint(a * kTwoOverPi);
  double r = __builtin_fma(-k, kPio2Hi, a);
  r = __builtin_fma(-k, kPio2Mid, r);
  r = __builtin_fma(-k, kPio2Lo, r);
  const double r2 = r * r;
  // sin r = r (1 - r^2/3! + r^4/5! - ...),  cos r = 1 - r^2/2! + r^4/4! - ...
  double ps = -1.0 / 121645100408832000.0;               // -1/19!
  ps = __builtin_fma(ps, r2, 1.0 / 355687428096000.0);   //  1/17!
  ps = __builtin_fma(ps, r2, -1.0 / 1307674368000.0);    // -1/15!
  ps = __builtin_fma(ps, r2, 1.0 / 6227020800.0);        //  1/13!
  ps = __builtin_fma(ps, r2, -1.0 / 39916800.0);         // -1/11!
  ps = __builtin_fma(ps, r2, 1.0 / 362880.0);            //  1/9!
  ps = __builtin_fma(ps, r2, -1.0 / 5040.0);             // -1/7!
  ps = __builtin_fma(ps, r2, 1.0 / 120.0);               //  1/5!
  ps = __builtin_fma(ps, r2, -1.0 / 6.0);                // -1/3!
  const double sr = __builtin_fma(ps * r2, r, r);
  double pc = -1.0 / 6402373705728000.0;                 // -1/18!
  pc = __builtin_fma(pc, r2, 1.0 / 20922789888000.0);    //  1/16!
  pc = __builtin_fma(pc, r2, -1.0 / 87178291200.0);      // -1/14!
  pc = __builtin_fma(pc, r2, 1.0 / 479001600.0);         //  1/12!
  pc = __builtin_fma(pc, r2, -1.0 / 3628800.0);          // -1/10!
  pc = __builtin_fma(pc, r2, 1.0 / 40320.0);             //  1/8!
  pc = __builtin_fma(pc, r2, -1.0 / 720.0);              // -1/6!
  pc = __builtin_fma(pc, r2, 1.0 / 24.0);                //  1/4!
  pc = __builtin_fma(pc, r2, -0.5);                      // -1/2!
  const double cr = __builtin_fma(pc, r2, 1.0);
  const int q = (int)((int64_t)k & 3);
  const double s0 = (q & 1) ? cr : sr;
  const double c0 = (q & 1) ? sr : cr;
  *sn = (q & 2) ? -s0 : s0;
  *cs = ((q + 1) & 2) ? -c0 : c0;
}

// Lane layouts of the rotated features. HALF: a lane holds chunk j of the first half and
// chunk j of the second half (pairs (i, i + dims/2) across the two). TRAD2: a lane holds the
// same two chunks, each a run of whole neighbouring pairs (2i, 2i+1), so interleaved rows
// keep two chunks (32 bytes of bf16) per lane in flight like half-split ones. TRAD1: one
// chunk per lane (interleaved rows whose half is not a whole number of chunks).
enum RopeMode : int { M_HALF = 0, M_TRAD1 = 1, M_TRAD2 = 2 };

// (cos, sin) table slot of pair p: one padding slot after every eight, so that the lanes of
// a group (eight pairs apart in half mode) read different LDS banks.
__device__ __forceinline__ int cs_slot(int p) { return p + (p >> 3); }

template <bool BF16, int MODE, int G, int QC, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QC == 0 ? 4 : 1)))
rope_fast(RopeArgs a) {
  constexpr bool HALF = MODE == M_HALF;
  constexpr bool TWO = MODE != M_TRAD1;       // two chunks per lane
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int RPW = 64 / G;                 // row slots per wave
  constexpr int RPB = 4 * RPW;                // row slots per block
  constexpr int PAIRS = TWO ? V : V / 2;      // rotated pairs per lane
  constexpr int MAXP = G * PAIRS;             // pairs one group can hold
  constexpr int QN = QC > 0 ? QC : 1;
  // Per pair p with features (i, j) (i < j) and scales (w_i, w_j): the rotation's products
  // with the scales folded in, ab = (w_i cos, w_j sin) and cd = (w_i sin, w_j cos), sin signed
  // for the direction, by cs_slot(p).
  __shared__ double2 tab_ab[MAXP + MAXP / 8], tab_cd[MAXP + MAXP / 8];

  const int64_t l = blockIdx.x;
  const int64_t pos = rope_position(a, l);
  const int half = a.dims / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / G, lj = lane % G;
  const int npc = TWO ? half / V : a.dims / V;  // lanes' rotated chunks (or chunk pairs)
  const int nqc = (a.D - a.dims) / V;            // pass-through chunks
  const bool has_pc = lj < npc;
  const bool norm = a.normalize != 0;
  const bool has_w = norm && a.w != nullptr;
  const double inv_d = 1.0 / (double)a.D;

  // Chunk offsets (in elements) within a row. A lane without a rotated chunk (lj >= npc)
  // or without a pass-through chunk still loads a valid chunk of the row (clamped), so that
  // a row's loads take no per-lane condition; it never stores it.
  const int off_u = min(lj, max(npc - 1, 0)) * V;
  const int off_v = TWO ? half + off_u : 0;
  int off_q[QN];
  bool has_q[QN];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    has_q[q] = QC > 0 && lj + G * q < nqc;
    off_q[q] = a.dims + min(lj + G * q, max(nqc - 1, 0)) * V;
  }

  // Row addresses at this position: row bh of tensor A at inA + bh sA, of tensor B at
  // inB + bh sB (the offset of B's first row folded into inB), outputs likewise. A lane's rows
  // in a step are RPB apart, so their addresses advance by uniform steps from the first one:
  // one set of 64-bit multiplies (quarter rate) per step instead of one per row.
  const int64_t rowb = (int64_t)a.D * ESZ;
  const int64_t inA = (int64_t)a.x + l * a.x_sl * rowb, sA = a.x_sbh * rowb;
  const int64_t inB = (int64_t)a.x2 + (l * a.x2_sl - a.BH1 * a.x2_sbh) * rowb, sB = a.x2_sbh * rowb;
  const int64_t outA = (int64_t)a.out + (a.o_row0 + l) * a.o_sl * rowb, oA = a.o_sbh * rowb;
  const int64_t outB = (int64_t)a.out2 + (l * a.o2_sl - a.BH1 * a.o2_sbh) * rowb, oB = a.o2_sbh * rowb;

  // Each step handles R rows per lane group: all their loads are issued first. The loads
  // of the first step are issued before the rotation table of this position is built, so
  // that the table's latency overlaps them.
  const int64_t bh_blk = (int64_t)blockIdx.y * a.iters * RPB * R;
  u32x4 xu[R], xv[R], xq[R][QN];
  int64_t bh0 = 0;
  // Rows past BH (uniform over a lane group) load the last row instead, so that every load
  // is unconditional and the compiler's waits for them stay exact; they store nothing.
  const int64_t last = a.BH - 1;
  const int64_t p_last = last < a.BH1 ? inA + last * sA : inB + last * sB;
  auto load_step = [&](int it) {
    bh0 = bh_blk + (int64_t)it * R * RPB + wave * RPW + g;
    int64_t pa = inA + bh0 * sA, pb = inB + bh0 * sB;
#pragma unroll
    for (int r = 0; r < R; ++r, pa += RPB * sA, pb += RPB * sB) {
      const int64_t bh = bh0 + r * RPB;
      const char* xrow = global_ptr(bh >= a.BH ? p_last : bh < a.BH1 ? pa : pb);
      xu[r] = ld16_nt(xrow + off_u * ESZ);
      xv[r] = TWO ? ld16_nt(xrow + off_v * ESZ) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < QN; ++q)
        xq[r][q] = QC > 0 ? ld16_nt(xrow + (int64_t)off_q[q] * ESZ) : u32x4{0, 0, 0, 0};
    }
  };
  // The scales and freqs entry of this thread's first table pair are loaded (the scales as
  // raw 32-bit words, widened only when used) before the rows: loads return in issue order,
  // so the table waits for them alone, not for the rows issued behind them. Only the waves
  // that hold table pairs load them (a lane past the table reads entry 0), and only what
  // the launch has (w, freqs).
  const bool w32 = !BF16 || a.w_f32;
  auto scale_word = [&](int i) {  // the word holding w[i]
    return *(const uint32_t*)((const char*)a.w + (w32 ? 4 * (int64_t)i : (2 * (int64_t)i & ~3)));
  };
  auto scale_of = [&](uint32_t word, int i) {
    if (!has_w) return 1.f;
    if (w32) return __builtin_bit_cast(float, word);
    return (i & 1) ? bf16hi(word) : bf16lo(word);
  };
  const int t0 = threadIdx.x;
  const bool tab_wave = __builtin_amdgcn_readfirstlane(wave) * 64 < half;
  const int tc = t0 < half ? t0 : 0;
  uint32_t wi0 = 0u, wj0 = 0u;
  float fr0 = 0.f;
  if (tab_wave && has_w) {
    wi0 = scale_word(HALF ? tc : 2 * tc);
    wj0 = scale_word(HALF ? tc + half : 2 * tc + 1);
  }
  if (tab_wave && a.freqs != nullptr) fr0 = a.freqs[tc];
  load_step(0);
  // Pair t's coefficients from its scale words and freqs entry. The first pair of each thread
  // takes the words loaded above, outside any loop, so that its waits cover those loads only.
  auto build = [&](int t, uint32_t wiw, uint32_t wjw, float fr) {
    const double theta = a.freqs != nullptr ? 1.0 / (double)fr : rope_theta(a, t);
    const double ang = ((double)a.scale * (double)pos) * theta;
    double sn, cs;
    rope_sincos(ang, &sn, &cs);
    if (!a.forward) sn = -sn;
    const double wi = scale_of(wiw, HALF ? t : 2 * t), wj = scale_of(wjw, HALF ? t + half : 2 * t + 1);
    tab_ab[cs_slot(t)] = double2{wi * cs, wj * sn};
    tab_cd[cs_slot(t)] = double2{wi * sn, wj * cs};
  };
  // A table that loads nothing (rotation only, base frequencies) is built after the rows have
  // arrived: measured faster for that case (Rope [8, 32, 512, 128] bf16 14.7 -> 13.2 us),
  // while with scales building it under the rows' loads is (NormRope 15.1 -> 14.3 us).
  if (!has_w && a.freqs == nullptr) __builtin_amdgcn_s_waitcnt(0);
  if (t0 < half) build(t0, wi0, wj0, fr0);
  for (int t = t0 + 256; t < half; t += 256) {
    const uint32_t wiw = has_w ? scale_word(HALF ? t : 2 * t) : 0u;
    const uint32_t wjw = has_w ? scale_word(HALF ? t + half : 2 * t + 1) : 0u;
    build(t, wiw, wjw, a.freqs != nullptr ? a.freqs[t] : 0.f);
  }
  float wq[QN][V];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
#pragma unroll
    for (int e = 0; e < V; ++e) wq[q][e] = 1.f;
    if (has_w && has_q[q]) load_param<BF16, V>(a.w, a.w_f32, off_q[q], wq[q]);
  }
  __syncthreads();

  // Pair p of this lane's e-th rotated pair.
  auto pair_of = [&](int e) {
    return HALF ? lj * V + e
                : (e < V / 2 ? lj * (V / 2) + e : half / 2 + lj * (V / 2) + (e - V / 2));
  };
  // Element e of a packed chunk as fp32.
  auto elem = [](const u32x4& v, int e) {
    if constexpr (BF16) return (e & 1) ? bf16hi(v[e >> 1]) : bf16lo(v[e >> 1]);
    else return __builtin_bit_cast(float, (uint32_t)v[e]);
  };

  for (int it = 0; it < a.iters; ++it) {
    if (it > 0) load_step(it);
    // The rows' scales: rstd * mscale for the rotated features (rstd = 1 without the
    // normalisation), from each row's fp32 sum of squares over all D features.
    double rs[R];
    float rstd_f[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      double rstd = 1.0;
      if (norm) {
        float ss = 0.f;
        if (has_pc) {
          float f[V];
          unpack<BF16>(xu[r], f);
#pragma unroll
          for (int e = 0; e < V; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
          if (TWO) {
            unpack<BF16>(xv[r], f);
#pragma unroll
            for (int e = 0; e < V; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
          }
        }
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          if (has_q[q]) {
            float fq[V];
            unpack<BF16>(xq[r][q], fq);
#pragma unroll
            for (int e = 0; e < V; ++e) ss = __builtin_fmaf(fq[e], fq[e], ss);
          }
        }
        rstd = rstd_f64_newton((double)group_sum<G>(ss), inv_d, a.eps);
      }
      rs[r] = rstd * (double)a.mscale;
      rstd_f[r] = (float)rstd;
    }
    // Rotation, pair by pair (two pairs at a time, whose results pack into one 32-bit
    // word): each pair's folded products are read from LDS once and applied to the step's R
    // rows, and the results replace the inputs in their registers. A pair (u, v) of scaled
    // features becomes ((u ab.x - v ab.y) rs, (u cd.x + v cd.y) rs).
    if (has_pc) {
      if constexpr (HALF) {
#pragma unroll
        for (int e = 0; e < V; e += 2) {
          const double2 ab0 = tab_ab[cs_slot(pair_of(e))], cd0 = tab_cd[cs_slot(pair_of(e))];
          const double2 ab1 = tab_ab[cs_slot(pair_of(e + 1))], cd1 = tab_cd[cs_slot(pair_of(e + 1))];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const double u0 = elem(xu[r], e), v0 = elem(xv[r], e);
            const double u1 = elem(xu[r], e + 1), v1 = elem(xv[r], e + 1);
            float ou[2], ov[2];
            ou[0] = f64_to_f32((u0 * ab0.x - v0 * ab0.y) * rs[r]);
            ov[0] = f64_to_f32((u0 * cd0.x + v0 * cd0.y) * rs[r]);
            ou[1] = f64_to_f32((u1 * ab1.x - v1 * ab1.y) * rs[r]);
            ov[1] = f64_to_f32((u1 * cd1.x + v1 * cd1.y) * rs[r]);
            if constexpr (BF16) {
              xu[r][e >> 1] = pack_bf16x2(ou[0], ou[1]);
              xv[r][e >> 1] = pack_bf16x2(ov[0], ov[1]);
            } else {
              xu[r][e] = __builtin_bit_cast(unsigned, ou[0]);
              xu[r][e + 1] = __builtin_bit_cast(unsigned, ou[1]);
              xv[r][e] = __builtin_bit_cast(unsigned, ov[0]);
              xv[r][e + 1] = __builtin_bit_cast(unsigned, ov[1]);
            }
          }
        }
      } else {
        // Neighbouring pairs (2e, 2e + 1) of chunk u (pairs 0 .. V/2 - 1 of the lane) and of
        // chunk v (pairs V/2 .. V - 1).
#pragma unroll
        for (int c2 = 0; c2 < (TWO ? 2 : 1); ++c2) {
#pragma unroll
          for (int e = 0; e < V / 2; ++e) {
            const int slot = cs_slot(pair_of(c2 * (V / 2) + e));
            const double2 ab = tab_ab[slot], cd = tab_cd[slot];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              u32x4& xc = c2 ? xv[r] : xu[r];
              const double u = elem(xc, 2 * e), v = elem(xc, 2 * e + 1);
              const float o0 = f64_to_f32((u * ab.x - v * ab.y) * rs[r]);
              const float o1 = f64_to_f32((u * cd.x + v * cd.y) * rs[r]);
              if constexpr (BF16) {
                xc[e] = pack_bf16x2(o0, o1);
              } else {
                xc[2 * e] = __builtin_bit_cast(unsigned, o0);
                xc[2 * e + 1] = __builtin_bit_cast(unsigned, o1);
              }
            }
          }
        }
      }
    }
    int64_t pa = outA + bh0 * oA, pb = outB + bh0 * oB;
#pragma unroll
    for (int r = 0; r < R; ++r, pa += RPB * oA, pb += RPB * oB) {
      const int64_t bh = bh0 + r * RPB;
      const bool live = bh < a.BH;
      char* orow = (char*)global_ptr(bh < a.BH1 ? pa : pb);
      if (live && has_pc) {
        st16_nt(orow + off_u * ESZ, xu[r]);
        if constexpr (TWO) st16_nt(orow + off_v * ESZ, xv[r]);
      }
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        if (live && has_q[q]) {
          float fq[V];
          unpack<BF16>(xq[r][q], fq);
#pragma unroll
          for (int e = 0; e < V; ++e) fq[e] = norm ? (fq[e] * rstd_f[r]) * wq[q][e] : fq[e];
          st16_nt(orow + (int64_t)off_q[q] * ESZ, pack<BF16>(fq));
        }
      }
    }
  }
}

// Rotation-only rows over many positions, few rows per position (the query/key form: one
// token's heads): a block of 256 threads takes PB consecutive positions, builds their
// (cos, sin) tables in one pass of its threads (LDS), and walks its PB * BH row slots
// (position-major) in steps of 256 / G rows, one row per lane group, through a ring of two
// steps' loads (the next step in flight while one is rotated; 123 VGPRs, four waves per SIMD:
// a ring of three at 131 VGPRs and eight positions per block both measured slower). Each row
// reads its position's (cos, sin) from LDS. One position per block measured slower still:
// every block paid the table's latency (and the frequency load) for only BH rows, and its
// rows took two steps whose second waited for the first. The arithmetic is rope_fast's, term
// for term: without normalisation the features enter unscaled and the rotation is scaled by
// mscale; with it (NORM, every feature rotated) the row's sum of squares is a lane exchange
// inside the group, x w is rotated and the result scaled by rstd mscale.
template <bool BF16, int MODE, int G, bool MS, bool NORM>
__global__ void __launch_bounds__(256)
rope_multi(RopeArgs a) {
  constexpr bool HALF = MODE == M_HALF;
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int SPS = 256 / G;  // row slots per step
  constexpr int NR = 2;         // ring of steps
  extern __shared__ double2 cs_t[];  // [PB][half] (cos, sin)
  const int PB = a.pb;
  const int half = a.dims / 2;
  const int lane = threadIdx.x & 63;
  const int g = threadIdx.x / G;  // lane group of the block
  const int lj = lane % G;
  const int64_t l0 = (int64_t)blockIdx.x * PB;
  const int npos = (int)min((int64_t)PB, a.L - l0);
  const int nslots = npos * (int)a.BH;
  const int nsteps = (nslots + SPS - 1) / SPS;
  const int off_u = lj * V;
  const int off_v = half + off_u;
  const double ms = (double)a.mscale;  // MS: mscale != 1 (else the product is skipped: exact)
  float wu[V], wv[V];
#pragma unroll
  for (int e = 0; e < V; ++e) wu[e] = wv[e] = 1.f;
  if (NORM && a.w != nullptr) {
    load_param<BF16, V>(a.w, a.w_f32, off_u, wu);
    load_param<BF16, V>(a.w, a.w_f32, off_v, wv);
  }

  u32x4 xu[NR], xv[NR];
  auto slot_of = [&](int k) { return k * SPS + g; };
  auto load = [&](int k, u32x4& u, u32x4& v) {
    const int sl = min(slot_of(k), nslots - 1);
    const int p = sl / (int)a.BH, bh = sl - p * (int)a.BH;
    const char* xrow = rope_in_row(a, bh, l0 + p, ESZ);
    u = ld16_nt(xrow + off_u * ESZ);
    v = ld16_nt(xrow + off_v * ESZ);
  };
#pragma unroll
  for (int q = 0; q < NR - 1; ++q) load(q, xu[q], xv[q]);
  for (int t = threadIdx.x; t < npos * half; t += 256) {
    const int p = t / half, i = t - p * half;
    const double theta = rope_theta(a, i);
    const double ang = ((double)a.scale * (double)rope_position(a, l0 + p)) * theta;
    double sn, cs;
    rope_sincos(ang, &sn, &cs);
    cs_t[t] = double2{cs, a.forward ? sn : -sn};
  }
  __syncthreads();

  auto rotate = [&](int k, const u32x4& ru, const u32x4& rv) {
    const int sl = slot_of(k);
    if (sl >= nslots) return;
    const int p = sl / (int)a.BH, bh = sl - p * (int)a.BH;
    const double2* tab = cs_t + p * half;
    float fu[V], fv[V];
    unpack<BF16>(ru, fu);
    unpack<BF16>(rv, fv);
    // The rotation's scale: mscale, times the row's rstd with NORM (then x w is rotated).
    double rs = ms;
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) ss = __builtin_fmaf(fu[e], fu[e], ss);
#pragma unroll
      for (int e = 0; e < V; ++e) ss = __builtin_fmaf(fv[e], fv[e], ss);
      rs = rstd_f64((double)group_sum<G>(ss), a.D, a.eps) * ms;
    }
    constexpr bool SCALE = MS || NORM;
    if constexpr (HALF) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const double2 t = tab[lj * V + e];
        const double u = NORM ? (double)fu[e] * (double)wu[e] : (double)fu[e];
        const double v = NORM ? (double)fv[e] * (double)wv[e] : (double)fv[e];
        fu[e] = f64_to_f32(SCALE ? (u * t.x - v * t.y) * rs : u * t.x - v * t.y);
        fv[e] = f64_to_f32(SCALE ? (u * t.y + v * t.x) * rs : u * t.y + v * t.x);
      }
    } else {
#pragma unroll
      for (int e = 0; e < V / 2; ++e) {
        const double2 t1 = tab[lj * (V / 2) + e];
        const double2 t2 = tab[half / 2 + lj * (V / 2) + e];
        const double u = NORM ? (double)fu[2 * e] * (double)wu[2 * e] : (double)fu[2 * e];
        const double v =
            NORM ? (double)fu[2 * e + 1] * (double)wu[2 * e + 1] : (double)fu[2 * e + 1];
        fu[2 * e] = f64_to_f32(SCALE ? (u * t1.x - v * t1.y) * rs : u * t1.x - v * t1.y);
        fu[2 * e + 1] = f64_to_f32(SCALE ? (u * t1.y + v * t1.x) * rs : u * t1.y + v * t1.x);
        const double u2 = NORM ? (double)fv[2 * e] * (double)wv[2 * e] : (double)fv[2 * e];
        const double v2 =
            NORM ? (double)fv[2 * e + 1] * (double)wv[2 * e + 1] : (double)fv[2 * e + 1];
        fv[2 * e] = f64_to_f32(SCALE ? (u2 * t2.x - v2 * t2.y) * rs : u2 * t2.x - v2 * t2.y);
        fv[2 * e + 1] = f64_to_f32(SCALE ? (u2 * t2.y + v2 * t2.x) * rs : u2 * t2.y + v2 * t2.x);
      }
    }
    char* orow = rope_out_row(a, bh, l0 + p, ESZ);
    st16_nt(orow + off_u * ESZ, pack<BF16>(fu));
    st16_nt(orow + off_v * ESZ, pack<BF16>(fv));
  };
  // Unrolled by NR so that every ring buffer keeps its registers (as in the backward).
  int k0 = 0;
  for (; k0 + 2 * NR - 1 <= nsteps; k0 += NR) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      load(k0 + q + NR - 1, xu[(q + NR - 1) % NR], xv[(q + NR - 1) % NR]);
      rotate(k0 + q, xu[q], xv[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 2 * NR - 2; ++q) {
    const int k = k0 + q;
    if (k >= nsteps) break;
    if (k + NR - 1 < nsteps) load(k + NR - 1, xu[(q + NR - 1) % NR], xv[(q + NR - 1) % NR]);
    rotate(k, xu[q % NR], xv[q % NR]);
  }
}

template <bool BF16>
__global__ void __launch_bounds__(256)
rope_generic(RopeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t nrows = a.BH * a.L;
  const int half = a.dims / 2;
  const bool norm = a.normalize != 0;
  const bool has_w = norm && a.w != nullptr;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < nrows;
       row += (int64_t)gridDim.x * 4) {
    const int64_t bh = row / a.L, l = row % a.L;
    const char* xr = rope_in_row(a, bh, l, Fmt<BF16>::ESZ);
    char* orow = rope_out_row(a, bh, l, Fmt<BF16>::ESZ);
    float ss = 0.f;
    for (int e = lane; e < a.D; e += 64) {
      float f[1];
      load_act<BF16, 1>(xr, e, f);
      ss = __builtin_fmaf(f[0], f[0], ss);
    }
    // The wave sum also orders every read of the row before the first write below.
    const double rstd = norm ? rstd_f64((double)wave_sum(ss), a.D, a.eps) : 1.0;
    const double rs = rstd * (double)a.mscale;
    const double pos = (double)rope_position(a, l);
    for (int p = lane; p < half; p += 64) {
      const int iu = a.traditional ? 2 * p : p;
      const int iv = a.traditional ? 2 * p + 1 : p + half;
      float fu[1], fv[1], wu[1] = {1.f}, wv[1] = {1.f};
      load_act<BF16, 1>(xr, iu, fu);
      load_act<BF16, 1>(xr, iv, fv);
      if (has_w) {
        load_param<BF16, 1>(a.w, a.w_f32, iu, wu);
        load_param<BF16, 1>(a.w, a.w_f32, iv, wv);
      }
      const double theta = rope_theta(a, p);
      double s, c;
      rope_sincos(((double)a.scale * pos) * theta, &s, &c);
      if (!a.forward) s = -s;
      const double u = (double)fu[0] * (double)wu[0];
      const double v = (double)fv[0] * (double)wv[0];
      float ou[1] = {f64_to_f32((u * c - v * s) * rs)};
      float ov[1] = {f64_to_f32((u * s + v * c) * rs)};
      store_act<BF16, 1>(orow, iu, ou);
      store_act<BF16, 1>(orow, iv, ov);
    }
    const float rstd_f = (float)rstd;
    for (int e = a.dims + lane; e < a.D; e += 64) {
      float f[1], wv[1] = {1.f};
      load_act<BF16, 1>(xr, e, f);
      if (has_w) load_param<BF16, 1>(a.w, a.w_f32, e, wv);
      f[0] = norm ? (f[0] * rstd_f) * wv[0] : f[0];
      store_act<BF16, 1>(orow, e, f);
    }
  }
}

namespace {

template <bool BF16, int MODE, int G, int QC, int R>
hipError_t go_fast(const RopeArgs& a0, hipStream_t stream) {
  RopeArgs a = a0;
  constexpr int RPB = 4 * (64 / G);
  const int64_t steps = (a.BH + (int64_t)RPB * R - 1) / ((int64_t)RPB * R);
  // Enough blocks for about one full round on the chip (~1024 blocks of 256 threads, four
  // per compute unit at <= 128 VGPRs), while each block's sin/cos table is shared by as many
  // rows as possible.
  int64_t chunks = (1024 + a.L - 1) / a.L;
  if (chunks > steps) chunks = steps;
  if (chunks > 65535) chunks = 65535;
  if (chunks < 1) chunks = 1;
  a.iters = (int)((steps + chunks - 1) / chunks);
  chunks = (steps + a.iters - 1) / a.iters;
  dim3 grid((unsigned)a.L, (unsigned)chunks);
  rope_fast<BF16, MODE, G, QC, R><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

// R = 4 rows per lane group per step when there are enough b*h rows, else 1.
template <bool BF16, int MODE, int G, int QC>
hipError_t pick_r(const RopeArgs& a, hipStream_t stream) {
  constexpr int RPB = 4 * (64 / G);
  if (a.BH >= 2 * RPB * 4) return go_fast<BF16, MODE, G, QC, 4>(a, stream);
  return go_fast<BF16, MODE, G, QC, 1>(a, stream);
}

template <bool BF16, int MODE, int G>
hipError_t pick_qc(const RopeArgs& a, int qc, hipStream_t stream) {
  if (qc == 0) return pick_r<BF16, MODE, G, 0>(a, stream);
  if (qc == 1) return pick_r<BF16, MODE, G, 1>(a, stream);
  return pick_r<BF16, MODE, G, 2>(a, stream);
}

template <bool BF16, int MODE>
hipError_t pick_g(const RopeArgs& a, int g, int qc, hipStream_t stream) {
  switch (g) {
    case 4: return pick_qc<BF16, MODE, 4>(a, qc, stream);
    case 8: return pick_qc<BF16, MODE, 8>(a, qc, stream);
    case 16: return pick_qc<BF16, MODE, 16>(a, qc, stream);
    case 32: return pick_qc<BF16, MODE, 32>(a, qc, stream);
    default: return pick_qc<BF16, MODE, 64>(a, qc, stream);
  }
}

// rope_multi: normalised rows always scale the rotation (by rstd mscale); rotation-only rows
// skip a unit mscale's product (exact either way).
template <bool BF16, int MODE, int G>
hipError_t go_multi(const RopeArgs& a, int64_t blocks, hipStream_t stream) {
  const size_t lds = (size_t)a.pb * (a.dims / 2) * sizeof(double2);
  const unsigned nb = (unsigned)blocks;
  if (a.normalize) rope_multi<BF16, MODE, G, false, true><<<nb, 256, lds, stream>>>(a);
  else if (a.mscale != 1.f) rope_multi<BF16, MODE, G, true, false><<<nb, 256, lds, stream>>>(a);
  else rope_multi<BF16, MODE, G, false, false><<<nb, 256, lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

// The fast kernel applies when every chunk is a whole 16-byte vector: D, the rotated
// chunks and the pass-through chunks are VEC-multiples and the arrays are 16-byte aligned.
template <bool BF16>
hipError_t launch_norm_rope(const RopeArgs& a0, bool aligned16, hipStream_t stream) {
  RopeArgs a = a0;
  a.log2_base = std::log2((double)a0.base);
  constexpr int V = Fmt<BF16>::VEC;
  const int half = a.dims / 2;
  const bool chunks_ok = aligned16 && a.D % V == 0 && a.dims % V == 0 &&
                         (a.traditional || half % V == 0) && a.L <= 0x7fffffff;
  if (chunks_ok && !force_generic_path()) {
    // Interleaved rows whose half is a whole number of chunks use the two-chunk layout.
    const int mode = !a.traditional ? M_HALF : (half % V == 0 ? M_TRAD2 : M_TRAD1);
    const int npc = mode == M_TRAD1 ? a.dims / V : half / V;
    const int nqc = (a.D - a.dims) / V;
    // Every feature rotated, few rows per position and many positions: several positions
    // per block (rope_multi). With the normalisation, for 64-feature rows, or for rows of
    // fewer than 32 heads: its variant holds 139 registers (three waves per SIMD), which at
    // 128 features and 32 heads measured no faster than one position per block (NormRope
    // [1, 32, 4096, 128] bf16: 20.2 us either way; [4, 8, 8192, 64]: 31.1 -> 20.9 us), while
    // with fewer heads one position per block leaves most of its lane groups idle ([1, 8,
    // 32768, 128] 73.7 -> 43.2 us at four positions per block).
    if (nqc == 0 && mode != M_TRAD1 && a.BH < 256 && a.L >= 4096 &&
        (npc == 4 || ((npc == 8 || npc == 16) && (!a.normalize || a.BH < 32)))) {
      // Positions per block: 8 for 64-feature rows (at 32 rows per position a block then
      // holds 256 rows, and its table is one entry per thread), else 4. NormRope rows of
      // fewer than 32 heads take enough for 256 rows, at most 32 and at most L / 1024 (a full
      // round of blocks on the chip): [1, 8, 32768, 128] 43.2 -> 39.5 us at 32, [2, 8, 16384,
      // 128] 41.9 -> 39.8 us at 16. Rotation-only rows measured slower that way ([1, 16, 32768,
      // 128] 50.9 -> 69.3 us at 16).
      const int64_t pb_min = npc == 4 ? 8 : 4;
      int64_t pb = pb_min;
      if (a.normalize && a.BH < 32)
        pb = std::max(pb_min, std::min({(int64_t)32, 256 / a.BH, a.L / 1024}));
      const int64_t blocks = (a.L + pb - 1) / pb;
      if (blocks <= 0x7fffffff) {
        a.pb = (int)pb;
        const bool half_mode = mode == M_HALF;
        if (npc == 4)
          return half_mode ? go_multi<BF16, M_HALF, 4>(a, blocks, stream)
                           : go_multi<BF16, M_TRAD2, 4>(a, blocks, stream);
        if (npc == 8)
          return half_mode ? go_multi<BF16, M_HALF, 8>(a, blocks, stream)
                           : go_multi<BF16, M_TRAD2, 8>(a, blocks, stream);
        return half_mode ? go_multi<BF16, M_HALF, 16>(a, blocks, stream)
                         : go_multi<BF16, M_TRAD2, 16>(a, blocks, stream);
      }
    }
    for (int g = 4; g <= 64; g *= 2) {
      if (npc <= g && nqc <= 2 * g) {
        const int qc = (nqc + g - 1) / g;
        if (mode == M_HALF) return pick_g<BF16, M_HALF>(a, g, qc, stream);
        if (mode == M_TRAD2) return pick_g<BF16, M_TRAD2>(a, g, qc, stream);
        return pick_g<BF16, M_TRAD1>(a, g, qc, stream);
      }
    }
  }
  const int64_t nrows = a.BH * a.L;
  int64_t blocks = (nrows + 3) / 4;
  if (blocks > 1048576) blocks = 1048576;
  rope_generic<BF16><<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template hipError_t launch_norm_rope<true>(const RopeArgs&, bool, hipStream_t);
template hipError_t launch_norm_rope<false>(const RopeArgs&, bool, hipStream_t);

}  // namespace nrm

// Device helpers shared by the row-wise normalisation kernels (gfx950 / CDNA4, wave64).
//
// * bf16 values travel packed, two per 32-bit register (element 2k in the low half, 2k+1 in
//   the high half, the little-endian memory order). Widening is a shift (exact); narrowing
//   is v_cvt_pk_bf16_f32, round-to-nearest-even on two floats at once.
// * Global memory is touched in 16-byte chunks (global_load_dwordx4 / global_store_dwordx4):
//   8 bf16 or 4 fp32 elements per lane per instruction.
// * Cross-lane sums use DPP within a 16-lane row (quad_perm, row_half_mirror, row_mirror)
//   and v_readlane across the four rows of a wave. At every step a lane adds its partner's
//   partial sum to its own, and fp addition is commutative, so every lane of a group ends
//   with the same bits, and the order is fixed: results are identical run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nrm {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Elements per 16-byte chunk.
template <bool BF16> struct Fmt;
template <> struct Fmt<true> { static constexpr int VEC = 8; static constexpr int ESZ = 2; };
template <> struct Fmt<false> { static constexpr int VEC = 4; static constexpr int ESZ = 4; };

// ------------------------------------------------------------------ bf16 <-> fp32

__device__ __forceinline__ float bf16lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) {
  return __builtin_bit_cast(float, u & 0xffff0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ------------------------------------------------------------------ 16-byte chunks

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

// Streaming (non-temporal, `nt`) 16-byte access for data touched exactly once: on MI355X
// this lifts a 50/50 read/write stream from ~6.0 to ~6.4 TB/s.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, (u32x4*)p);
}

// Unpack a 16-byte chunk into VEC floats.
template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4& v, float (&f)[Fmt<BF16>::VEC]) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = bf16lo(v[k]);
      f[2 * k + 1] = bf16hi(v[k]);
    }
  } else {
    // Each element goes through a scalar first: __builtin_bit_cast applied directly to an
    // ext_vector element reads element 0 whatever the index (seen with this hipcc).
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned u = v[k];
      f[k] = __builtin_bit_cast(float, u);
    }
  }
}

// Pack VEC floats (rounded to the storage type) into a 16-byte chunk.
template <bool BF16>
__device__ __forceinline__ u32x4 pack(const float (&f)[Fmt<BF16>::VEC]) {
  u32x4 v;
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = pack_bf16x2(f[2 * k], f[2 * k + 1]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(unsigned, f[k]);
  }
  return v;
}

// V weights starting at element i: fp32 storage, or bf16 storage (only with bf16
// activations). V is VEC (16-byte aligned chunk of activations) or 1 (scalar path).
template <bool BF16, int V>
__device__ __forceinline__ void load_param(const void* p, bool p_f32, int64_t i, float (&f)[V]) {
  if (!BF16 || p_f32) {
    const float* q = (const float*)p + i;
    if constexpr (V % 4 == 0) {
#pragma unroll
      for (int k = 0; k < V / 4; ++k) {
        f32x4 t = *(const f32x4*)(q + 4 * k);
        f[4 * k] = t[0]; f[4 * k + 1] = t[1]; f[4 * k + 2] = t[2]; f[4 * k + 3] = t[3];
      }
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) f[k] = q[k];
    }
  } else {
    const uint16_t* q = (const uint16_t*)p + i;
    if constexpr (V == 8) {
      float t[8];
      unpack<true>(ld16(q), t);
#pragma unroll
      for (int k = 0; k < 8; ++k) f[k] = t[k];
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) f[k] = bf16_to_f32(q[k]);
    }
  }
}

// V activations at element i (16-byte chunk when V == VEC, else element by element).
template <bool BF16, int V>
__device__ __forceinline__ void load_act(const void* p, int64_t i, float (&f)[V]) {
  if constexpr (V == Fmt<BF16>::VEC) {
    unpack<BF16>(ld16((const char*)p + i * Fmt<BF16>::ESZ), f);
  } else if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < V; ++k) f[k] = bf16_to_f32(((const uint16_t*)p)[i + k]);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) f[k] = ((const float*)p)[i + k];
  }
}

template <bool BF16, int V>
__device__ __forceinline__ void store_act(void* p, int64_t i, const float (&f)[V]) {
  if constexpr (V == Fmt<BF16>::VEC) {
    st16((char*)p + i * Fmt<BF16>::ESZ, pack<BF16>(f));
  } else if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < V; ++k) ((uint16_t*)p)[i + k] = f32_to_bf16(f[k]);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) ((float*)p)[i + k] = f[k];
  }
}

// fp64 -> fp32, round to nearest even, kept opaque to the optimiser (an empty asm with the
// value in a VGPR; no memory access). Without it the compiler fuses a following fp32 ->
// bf16 conversion into one exactly rounded fp64 -> bf16 conversion done by a round-to-odd
// sequence of about eight instructions per element. Going through fp32 differs from direct
// rounding only when the fp32 value lands exactly on a bf16 midpoint, and then by one unit
// in the last place, which the one-ulp bar allows.
__device__ __forceinline__ float f64_to_f32(double d) {
  float f = (float)d;
  __asm__ volatile("" : "+v"(f));
  return f;
}

// Round V floats to the storage type and back (the value that a store would keep).
template <bool BF16, int V>
__device__ __forceinline__ void round_to_storage(float (&f)[V]) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < V; ++k) f[k] = bf16_to_f32(f32_to_bf16(f[k]));
  }
}

// ------------------------------------------------------------------ DPP reductions

// DPP control words (gfx9 encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum over aligned groups of G lanes (G = 1, 2, 4, 8, 16, 32 or 64); every lane of a
// group receives the group's sum.
template <int G, typename T>
__device__ __forceinline__ T group_sum(T v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "G");
  if constexpr (G >= 2) v += dpp<DPP_QUAD_XOR1>(v);
  if constexpr (G >= 4) v += dpp<DPP_QUAD_XOR2>(v);
  if constexpr (G >= 8) v += dpp<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (G >= 16) v += dpp<DPP_ROW_MIRROR>(v);
  if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Sum over the whole wave, returned wave-uniform: DPP inside each 16-lane row, then the
// four row sums read with v_readlane and added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_sum(double v) {
  v = group_sum<16>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;

// v of lane l plus v of lane l ^ 16 (ROWS = 16) or l ^ 32 (ROWS = 32), through the gfx950
// lane swaps (VALU, no LDS round trip). A swap of a register with itself hands every lane
// the pair's lower-lane value and its upper-lane value; both lanes of a pair add them in that
// order, so they agree bit for bit.
template <int ROWS>
__device__ __forceinline__ double swap_sum(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  uint32_t l0, l1, h0, h1;
  if constexpr (ROWS == 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = a[0], l1 = a[1], h0 = b[0], h1 = b[1];
  } else {
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = a[0], l1 = a[1], h0 = b[0], h1 = b[1];
  }
  return __builtin_bit_cast(double, ((uint64_t)h0 << 32) | l0) +
         __builtin_bit_cast(double, ((uint64_t)h1 << 32) | l1);
}

// Sum over the 64 lanes of a wave, every lane ending with a total (the lanes need not agree
// bit for bit; callers read a fixed lane): rotations by 4 and 8 inside each 16-lane row keep
// a lane's index mod 4, and so do the xor-16 / xor-32 exchanges across rows.
__device__ __forceinline__ double lanes_sum_mod4(double v) {
  v += dpp<DPP_ROW_ROR4>(v);
  v += dpp<DPP_ROW_ROR8>(v);
  v = swap_sum<16>(v);
  v = swap_sum<32>(v);
  return v;
}

// Four fp64 row sums over a team of nwt waves, with one barrier. Within a quad of lanes the
// four sums are transposed (lane l keeps sum l & 3 of the quad), so the rest of the wave
// reduction handles one value per lane instead of four; each wave's four totals go to LDS
// (red: 4 slots per wave of the block), and after the barrier lane l of every wave adds up
// sum l & 3 of team wave l >> 2. The order of every addition is fixed: results are the same
// on every run, and the same in every thread of the team (they are read from lanes 0..3).
__device__ __forceinline__ void team_sum4(double (&s)[4], double* red, int wave0, int nwt) {
  const int lane = threadIdx.x & 63;
  const bool b = lane & 1, c = lane & 2;
  double k0 = b ? s[1] : s[0], u0 = b ? s[0] : s[1];
  double k1 = b ? s[3] : s[2], u1 = b ? s[2] : s[3];
  k0 += dpp<DPP_QUAD_XOR1>(u0);  // sum b of the lane pair
  k1 += dpp<DPP_QUAD_XOR1>(u1);  // sum 2 + b
  double k = c ? k1 : k0;
  const double u = c ? k0 : k1;
  k += dpp<DPP_QUAD_XOR2>(u);    // sum lane & 3 of the quad
  k = lanes_sum_mod4(k);         // ... of the wave
  if (lane < 4) red[(threadIdx.x >> 6) * 4 + lane] = k;
  __syncthreads();
  const int w = lane >> 2;
  double t = w < nwt ? red[(wave0 + w) * 4 + (lane & 3)] : 0.0;
  t = lanes_sum_mod4(t);         // sum lane & 3 of the team
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = readlane_f64(t, i);
}

// ------------------------------------------------------------------ row pivots
//
// LayerNorm's statistics are sums about a pivot taken from the row, not raw moments. The
// variance from sum(x^2)/n - mean^2 cancels catastrophically when |mean| is far above the
// standard deviation sigma (an fp32 row such as 1e4 + N(0, 0.01) loses every bit of fp64).
// About a pivot p that is one of the row's values, |p - mean| <= sigma sqrt(n - 1)
// (Samuelson's inequality), so sum((x - p)^2) / n <= n sigma^2 and the variance
// sum((x - p)^2) / n - (mean - p)^2 loses at most log2(n) bits. x - p is exact in fp64
// for bf16 and fp32 values whose exponents are within 29 of each other, and off by one
// rounding otherwise. Every thread of a row uses the same pivot (the row's first element),
// so the sums combine as they are.

// A 32-bit word at a wave-uniform, 4-byte aligned address, through the scalar data cache
// (into scalar registers, no vector registers held while it is in flight). Only for data
// the kernel has not written before this read.
__device__ __forceinline__ uint32_t sload_u32(const void* p) {
  return *(const __attribute__((address_space(4))) uint32_t*)p;
}

// Element i of a bf16 or fp32 array, at a wave-uniform address, by a scalar load of the
// aligned word that holds it (a bf16 element is either half of its word).
template <bool BF16>
__device__ __forceinline__ float sload_elem(const void* p, int64_t i) {
  if constexpr (BF16) {
    const uintptr_t a = (uintptr_t)((const uint16_t*)p + i);
    const uint32_t w = sload_u32((const void*)(a & ~(uintptr_t)3));
    return __builtin_bit_cast(float, (a & 2) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __builtin_bit_cast(float, sload_u32((const float*)p + i));
  }
}

// The first lane's 32-bit value of each aligned group of G lanes (G = 1 .. 64) in every lane
// of the group: the pivot of a team of G lanes that owns one row.
template <int G>
__device__ __forceinline__ uint32_t group_first(uint32_t v) {
  if constexpr (G == 64) return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
  else return (uint32_t)__shfl((int)v, (int)(threadIdx.x & 63 & ~(G - 1)), 64);
}

// Decode one element from the first 32 bits of a chunk (element 0: the low half of a bf16
// pair, or the fp32 value).
template <bool BF16>
__device__ __forceinline__ float first_elem(uint32_t raw) {
  if constexpr (BF16) return bf16lo(raw);
  else return __builtin_bit_cast(float, raw);
}

// 1 / sqrt(v) in fp64 for a row scalar: the hardware's fp64 estimate (good to about single
// precision), refined by two Newton steps y += y (1 - v y^2) / 2, each of which about squares
// the relative error, so the result is within a few fp64 units in the last place (far below
// what fp32 and bf16 outputs resolve).
// Zero, subnormal, huge, infinite, negative and NaN arguments take the exact expression.
__device__ __forceinline__ double rsqrt_row(double v) {
  if (v >= 0x1p-1000 && v <= 0x1p+1000) {
    const double vh = 0.5 * v;
    double y = __builtin_amdgcn_rsq(v);
#pragma unroll
    for (int i = 0; i < 2; ++i) y = __builtin_fma(y, __builtin_fma(-(vh * y), y, 0.5), y);
    return y;
  }
  return 1.0 / __builtin_sqrt(v);
}

// rstd = 1 / sqrt(sum / n + eps), formed in fp64 from an fp32 or fp64 sum (one row scalar).
__device__ __forceinline__ double rstd_f64(double sum, int64_t n, float eps) {
  return 1.0 / __builtin_sqrt(sum / (double)n + (double)eps);
}

// The same statistic from inv_n = 1/n, for short rows where its instruction count shows: the
// fp32 hardware reciprocal square root (relative error ~1e-7) refined by two Newton steps
// y <- y + y (1 - t y^2) / 2, each of which squares the relative error, so the result is
// within a few fp64 ulp; about a third of the instructions of the divisions and square root.
// Arguments outside the fp32 normal range (0, inf and NaN among them) take the exact form.
__device__ __forceinline__ double rstd_f64_newton(double sum, double inv_n, float eps) {
  const double t = __builtin_fma(sum, inv_n, (double)eps);
  if (!(t > 1e-36 && t < 1e36)) return 1.0 / __builtin_sqrt(t);
  double y = (double)__builtin_amdgcn_rsqf((float)t);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const double r = __builtin_fma(-t * y, y, 1.0);
    y = __builtin_fma(0.5 * y, r, y);
  }
  return y;
}

}  // namespace nrm

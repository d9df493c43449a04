// Kernel-shape choice and launch of the RMSNorm / LayerNorm backward kernels.
//
// For rows of n = hidden / VEC 16-byte chunks (VEC = 8 bf16, 4 fp32), when hidden and the
// base addresses are 16-byte granular and hidden <= 16384:
//   vjp_rows, a team of T = ceil(n / NV) threads (rounded up to a wave) per row, NV the
//   smallest chunk count per thread that keeps T <= 1024 among NV * VEC = 8 elements or
//   fewer (column sums in registers; hidden <= 8192) and NV * VEC = 16 (one team per block,
//   the dw column sums in LDS); G = min(1024 / T, 8) teams per block. The grid is
//   vjp_partials(rows) blocks of at most rpb rows each, taken strided (with parameter
//   gradients, one partial row per block).
// Rows of at most 32 chunks take vjp_team instead: teams of 8, 16 or 32 lanes, one chunk per
// lane, 1024 / team rows in flight per block.
// Rows that are not whole 16-byte chunks (or not 16-byte aligned), up to 8192 elements
// (6144 with fp32 data or weights): vjp_elems, single elements, 1 to 8 per thread (4 for most
// rows up to 2048), one block per run of rows.
// Otherwise vjp_generic (256 threads, 16-byte chunks or single elements, any width).
// The partial rows are then added by vjp_colsum.
#pragma once

#include <algorithm>

#include "launch.hpp"
#include "vjp.hpp"

namespace nrm {

namespace {

constexpr int64_t kVjpMaxGrid = 0x7fffffff;

__global__ void vjp_zero_kernel(unsigned char* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t zero_bytes(void* p, int64_t n, hipStream_t stream) {
  if (p == nullptr || n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  vjp_zero_kernel<<<(unsigned)blocks, 256, 0, stream>>>((unsigned char*)p, n);
  return hipGetLastError();
}

template <bool BF16, int OP, int NV, int PK, bool EXACT, bool PG>
hipError_t go_vjp_rows(const VjpArgs& a, int64_t blocks, int threads, hipStream_t stream) {
  constexpr int V = Fmt<BF16>::VEC;
  const int G = threads / a.team;
  const size_t lds = PG && NV * V >= 16 ? (size_t)NV * V * a.team * sizeof(double)
                     : PG && G > 1    ? (size_t)(G - 1) * a.team * V * sizeof(double)
                                      : 0;
  vjp_rows<BF16, OP, NV, PK, EXACT, PG><<<(unsigned)blocks, threads, lds, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int NV, bool PG>
hipError_t vjp_rows_pk(const VjpArgs& a, int64_t blocks, int threads, bool exact,
                       hipStream_t stream) {
  // Rows of 16 elements per thread, LayerNorm on bf16 and RMSNorm on fp32, always take the
  // ragged-width form (at whole widths its selects are always true). The whole-width form
  // of bf16 LayerNorm with fp32 parameters spilled inside its loop (~40 scratch accesses a
  // row; [8192, 16384] 591 -> 230 us), and the others measured faster too (bf16 LayerNorm
  // 219 -> 190 us, fp32 RMSNorm 353 -> 322 us); bf16 RMSNorm and fp32 LayerNorm measured
  // faster in the whole-width form.
  if constexpr (NV * Fmt<BF16>::VEC >= 16 && (OP == VJP_LN) == BF16) {
    (void)exact;
    if (a.w == nullptr)
      return go_vjp_rows<BF16, OP, NV, PK_NONE, false, PG>(a, blocks, threads, stream);
    if constexpr (BF16) {
      if (a.w_f32)
        return go_vjp_rows<BF16, OP, NV, PK_F32, false, PG>(a, blocks, threads, stream);
    }
    return go_vjp_rows<BF16, OP, NV, PK_SAME, false, PG>(a, blocks, threads, stream);
  } else {
    if (a.w == nullptr)
      return exact ? go_vjp_rows<BF16, OP, NV, PK_NONE, true, PG>(a, blocks, threads, stream)
                   : go_vjp_rows<BF16, OP, NV, PK_NONE, false, PG>(a, blocks, threads, stream);
    if constexpr (BF16) {
      if (a.w_f32)
        return exact ? go_vjp_rows<BF16, OP, NV, PK_F32, true, PG>(a, blocks, threads, stream)
                     : go_vjp_rows<BF16, OP, NV, PK_F32, false, PG>(a, blocks, threads, stream);
    }
    return exact ? go_vjp_rows<BF16, OP, NV, PK_SAME, true, PG>(a, blocks, threads, stream)
                 : go_vjp_rows<BF16, OP, NV, PK_SAME, false, PG>(a, blocks, threads, stream);
  }
}

template <bool BF16, int OP, int NV>
hipError_t vjp_rows_pg(const VjpArgs& a, bool pg, int64_t blocks, int threads, bool exact,
                       hipStream_t stream) {
  return pg ? vjp_rows_pk<BF16, OP, NV, true>(a, blocks, threads, exact, stream)
            : vjp_rows_pk<BF16, OP, NV, false>(a, blocks, threads, exact, stream);
}

template <bool BF16, int OP, int PK, bool EXACT, int SUB>
hipError_t go_vjp_team(const VjpArgs& a, bool pg, int64_t blocks, hipStream_t stream) {
  if (pg) vjp_team<BF16, OP, PK, EXACT, SUB, true><<<(unsigned)blocks, 1024, 0, stream>>>(a);
  else vjp_team<BF16, OP, PK, EXACT, SUB, false><<<(unsigned)blocks, 1024, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int SUB>
hipError_t vjp_team_pk(const VjpArgs& a, bool pg, bool exact, int64_t blocks,
                       hipStream_t stream) {
  if (a.w == nullptr)
    return exact ? go_vjp_team<BF16, OP, PK_NONE, true, SUB>(a, pg, blocks, stream)
                 : go_vjp_team<BF16, OP, PK_NONE, false, SUB>(a, pg, blocks, stream);
  if constexpr (BF16) {
    if (a.w_f32)
      return exact ? go_vjp_team<BF16, OP, PK_F32, true, SUB>(a, pg, blocks, stream)
                   : go_vjp_team<BF16, OP, PK_F32, false, SUB>(a, pg, blocks, stream);
  }
  return exact ? go_vjp_team<BF16, OP, PK_SAME, true, SUB>(a, pg, blocks, stream)
               : go_vjp_team<BF16, OP, PK_SAME, false, SUB>(a, pg, blocks, stream);
}

// Rows of at most 32 chunks (256 bf16 or 128 fp32 values): vjp_team with one chunk per lane
// and the smallest team of 8, 16 or 32 lanes that covers the row. vjp_rows' teams are whole
// waves, which at these widths leave most lanes idle (a 128-wide bf16 row is 16 chunks).
template <bool BF16, int OP>
hipError_t try_vjp_team(VjpArgs a, bool pg, int64_t n, hipStream_t stream, bool* done) {
  *done = false;
  if (n > 32) return hipSuccess;
  const int sub = n <= 8 ? 8 : n <= 16 ? 16 : 32;
  const bool exact = n == sub;
  const int64_t blocks = vjp_partials(a.rows);
  a.rpb = (a.rows + blocks - 1) / blocks;
  *done = true;
  switch (sub) {
    case 8: return vjp_team_pk<BF16, OP, 8>(a, pg, exact, blocks, stream);
    case 16: return vjp_team_pk<BF16, OP, 16>(a, pg, exact, blocks, stream);
    default: return vjp_team_pk<BF16, OP, 32>(a, pg, exact, blocks, stream);
  }
}

// Fast path; *done = false when the row does not fit it.
template <bool BF16, int OP>
hipError_t try_vjp_rows(VjpArgs a, bool pg, int64_t n, hipStream_t stream, bool* done) {
  constexpr int V = Fmt<BF16>::VEC;
  // Up to 8 elements per thread with the fp64 column accumulators in registers; rows of up
  // to 16384 elements take 16 per thread (one 1024-thread team per row) with the dw
  // accumulators in LDS (128 KB): in registers, 16 of them beside LN's db (64 registers)
  // push the kernel past 128 registers, into scratch.
  constexpr int MAX_NV = 8 / V;   // 1 for bf16, 2 for fp32
  constexpr int WIDE_NV = 16 / V;  // 2 for bf16, 4 for fp32
  *done = false;
  int nv = 1;
  while (nv <= MAX_NV && (n + nv - 1) / nv > 1024) nv *= 2;
  if (nv > MAX_NV) {
    if ((n + WIDE_NV - 1) / WIDE_NV > 1024) return hipSuccess;
    nv = WIDE_NV;
  }
  const int team = (int)((((n + nv - 1) / nv) + 63) / 64 * 64);
  const bool exact = (int64_t)team * nv == n;
  const int gmax = std::max(1, std::min(8, 1024 / team));
  // The same persistent grid with or without parameter gradients: at [16384, 8192] bf16 it
  // streams dx-only work faster (RMSNorm ~155 us) than one short-lived block per row
  // (~211 us), since a block keeps loading its next row while it reduces the current one.
  const int64_t blocks = vjp_partials(a.rows);
  a.rpb = (a.rows + blocks - 1) / blocks;
  const int G = (int)std::min<int64_t>(gmax, a.rpb);
  a.team = team;
  *done = true;
  const int threads = G * team;
  switch (nv) {
    case 1: return vjp_rows_pg<BF16, OP, 1>(a, pg, blocks, threads, exact, stream);
    case 2: return vjp_rows_pg<BF16, OP, 2>(a, pg, blocks, threads, exact, stream);
    case 4:
      if constexpr (!BF16) return vjp_rows_pg<BF16, OP, 4>(a, pg, blocks, threads, exact, stream);
      break;
    default: break;
  }
  *done = false;
  return hipSuccess;
}

template <bool BF16, int OP, int K, bool PG, bool XF>
void go_elems(const VjpArgs& a, int64_t blocks, unsigned threads, size_t lds,
              hipStream_t stream) {
  vjp_elems<BF16, OP, K, PG, XF><<<(unsigned)blocks, threads, lds, stream>>>(a);
}

template <bool BF16, int OP, int K>
hipError_t go_vjp_elems(VjpArgs a, bool pg, hipStream_t stream) {
  const int64_t blocks = vjp_partials(a.rows);
  a.rpb = (a.rows + blocks - 1) / blocks;
  const int64_t per = (a.hidden + K - 1) / K;
  const unsigned threads = (unsigned)((per + 63) / 64 * 64);
  // Only a thread's last element can fall past the row's end (vjp_elems relies on it).
  if ((int64_t)threads * (K - 1) > a.hidden || threads > 1024) return hipErrorInvalidConfiguration;
  // vjp_elems' LDS column sums: dw, and db for LN.
  const size_t lds = pg && K >= 8 ? (size_t)(OP == VJP_LN ? 2 : 1) * K * threads * 8 : 0;
  if constexpr (BF16) {
    if (!a.w_f32) {
      if (pg) go_elems<BF16, OP, K, true, true>(a, blocks, threads, lds, stream);
      else go_elems<BF16, OP, K, false, true>(a, blocks, threads, 0, stream);
      return hipGetLastError();
    }
  }
  if constexpr (K < 8) {  // try_vjp_elems takes 8 only with bf16 weights
    if (pg) go_elems<BF16, OP, K, true, false>(a, blocks, threads, lds, stream);
    else go_elems<BF16, OP, K, false, false>(a, blocks, threads, 0, stream);
  }
  return hipGetLastError();
}

// Rows of single elements: vjp_elems with K elements per thread. Rows of up to 2048 take 4
// where the thread count allows it (only a thread's last element past the row's end), else
// 2, else 1: at one element per thread the row's reduction costs more than its elements
// (1001-wide fp32 rows 77 -> 53 us, bf16 163 -> 137 us). Wider rows take the fewest of 6 or
// 8 that fit a 1024-thread block; 8 only with bf16 x, g and w: with fp64 products (fp32
// data or weights) that variant runs out of registers. *done = false for wider rows.
template <bool BF16, int OP>
hipError_t try_vjp_elems(const VjpArgs& a, bool pg, hipStream_t stream, bool* done) {
  const int64_t n = a.hidden;
  *done = n <= (BF16 && !a.w_f32 ? 8 : 6) * 1024;
  if (!*done) return hipSuccess;
  auto fits = [n](int64_t k) {
    const int64_t t = ((n + k - 1) / k + 63) / 64 * 64;
    return t * (k - 1) <= n && t <= 1024;
  };
  if (n <= 2048 && fits(4)) return go_vjp_elems<BF16, OP, 4>(a, pg, stream);
  if (n <= 2048 && fits(2)) return go_vjp_elems<BF16, OP, 2>(a, pg, stream);
  if (n <= 1024) return go_vjp_elems<BF16, OP, 1>(a, pg, stream);
  if (n <= 4096) return go_vjp_elems<BF16, OP, 4>(a, pg, stream);
  if (n <= 6144) return go_vjp_elems<BF16, OP, 6>(a, pg, stream);
  return go_vjp_elems<BF16, OP, 8>(a, pg, stream);
}

template <bool BF16, int OP, int V>
hipError_t go_vjp_generic(VjpArgs a, bool pg, hipStream_t stream) {
  int64_t blocks;
  if (pg) {
    blocks = vjp_partials(a.rows);
    a.rpb = (a.rows + blocks - 1) / blocks;
  } else {
    a.rpb = 1;
    blocks = a.rows;
  }
  if (blocks > kVjpMaxGrid) return hipErrorInvalidConfiguration;
  if (pg) vjp_generic<BF16, OP, V, true><<<(unsigned)blocks, 256, 0, stream>>>(a);
  else vjp_generic<BF16, OP, V, false><<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

template <bool BF16, int OP>
hipError_t launch_vjp(const VjpArgs& a, void* dw, void* db, bool aligned16, hipStream_t stream) {
  constexpr int V = Fmt<BF16>::VEC;
  const int pbytes = (!BF16 || a.w_f32) ? 4 : 2;  // parameter element size
  if (a.rows == 0) {
    hipError_t e = zero_bytes(dw, a.hidden * pbytes, stream);
    if (e == hipSuccess) e = zero_bytes(db, a.hidden * pbytes, stream);
    return e;
  }
  const bool pg = dw != nullptr || db != nullptr;
  const int path = forced_path();
  const bool vec = aligned16 && a.hidden % V == 0 && path != PATH_SCALAR;
  hipError_t err = hipSuccess;
  bool done = false;
  if (vec && path == PATH_AUTO) err = try_vjp_team<BF16, OP>(a, pg, a.hidden / V, stream, &done);
  if (vec && !done && path != PATH_CHUNKED)
    err = try_vjp_rows<BF16, OP>(a, pg, a.hidden / V, stream, &done);
  if (!vec && path == PATH_AUTO) err = try_vjp_elems<BF16, OP>(a, pg, stream, &done);
  if (!done) err = vec ? go_vjp_generic<BF16, OP, V>(a, pg, stream)
                       : go_vjp_generic<BF16, OP, 1>(a, pg, stream);
  if (err != hipSuccess || !pg) return err;
  // Only the requested outputs are passed: (part_w, dw) and/or (part_b, db).
  const double* parts[2];
  void* outs[2];
  int n = 0;
  if (dw != nullptr) { parts[n] = a.part_w; outs[n] = dw; ++n; }
  if (OP == VJP_LN && db != nullptr) { parts[n] = a.part_b; outs[n] = db; ++n; }
  if (n == 1) { parts[1] = parts[0]; outs[1] = outs[0]; }
  const int64_t nparts = vjp_partials(a.rows);
  const dim3 grid((unsigned)((a.hidden + 15) / 16), (unsigned)n);
  if (BF16 && !a.w_f32)
    vjp_colsum<true><<<grid, 256, 0, stream>>>(parts[0], outs[0], parts[1], outs[1], nparts,
                                               a.hidden);
  else
    vjp_colsum<false><<<grid, 256, 0, stream>>>(parts[0], outs[0], parts[1], outs[1], nparts,
                                                a.hidden);
  return hipGetLastError();
}

}  // namespace nrm

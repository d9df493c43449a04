// Kernel-shape choice and launch of the row kernels (RMSNorm, add-RMSNorm, LayerNorm).
//
// For a row of n = hidden / VEC 16-byte chunks (VEC = 8 bf16 or 4 fp32), automatic choice:
//   n <= 128                         row_team: teams of SUB = 4 .. 64 lanes (two chunks each,
//                                    the smallest power of two that covers the row), 256 / SUB
//                                    rows per block;
//   n <= 8192 (the RMS forms' bf16   row_block: one block of T threads per row, NV chunks per
//   rows beside fp32 w: 6144)        thread, NV = max(2, ceil(n / 1024)), 5 and 7 taken as
//                                    6 and 8 (LayerNorm: clamp(ceil(n / 256), 2, 4) up to
//                                    4096 chunks; with fp32 w beside bf16 x 2 up to 2048,
//                                    then at least 4), w (and b) loaded after the row's sums
//                                    from 4 chunks on; T = ceil(n / NV) rounded up to a wave
//                                    (hidden 8192 bf16: 512 threads with 2 chunks each,
//                                    LayerNorm 256 threads with 4); LayerNorm with w or b,
//                                    and RMSNorm with fp32 w, over 4096 rows or more at up
//                                    to 4 chunks (LayerNorm beside bf16 x: 2):
//                                    row_ln_pair / row_rms_pair, the same per thread for two
//                                    rows per block;
//   hidden or a base address not 16-byte granular, hidden <= 12288: row_elems, one block per
//   row, K single elements per thread in registers;
//   otherwise the looping kernel (16-byte chunks, or single elements).
// Measured on MI355X for add-RMSNorm bf16 [16384, 8192]: row_block streams at ~6.25 TB/s,
// one wave per row (the whole row in one wave's registers) at ~5.2 TB/s, the 512-thread
// register kernel without streaming hints at ~5.9 TB/s. Those two stay available through
// NRM_FORCE_PATH=wave / block.
#pragma once

#include <algorithm>

#include "launch.hpp"

namespace nrm {

namespace {

constexpr int64_t kMaxGrid = 0x7fffffff;

template <bool BF16, int OP, int NV>
hipError_t go_wave(const RowArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + 3) / 4;
  row_regs<BF16, OP, NV, 1><<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int NV>
hipError_t go_block(const RowArgs& a, hipStream_t stream) {
  row_regs<BF16, OP, NV, 8><<<(unsigned)a.rows, 512, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int V>
hipError_t go_chunked(const RowArgs& a, hipStream_t stream) {
  const int64_t blocks = a.rows < 1048576 ? a.rows : 1048576;
  row_chunked<BF16, OP, V><<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int K, int PK>
void go_elems_hb(const RowArgs& a, unsigned threads, hipStream_t stream) {
  if (OP == OP_LN && a.b != nullptr)
    row_elems<BF16, OP, K, PK, OP == OP_LN><<<(unsigned)a.rows, threads, 0, stream>>>(a);
  else
    row_elems<BF16, OP, K, PK, false><<<(unsigned)a.rows, threads, 0, stream>>>(a);
}

template <bool BF16, int OP, int K>
hipError_t go_rowelems(const RowArgs& a, hipStream_t stream) {
  const int64_t t = ((a.hidden + K - 1) / K + 63) / 64 * 64;
  // Only a thread's last element can fall past the row's end (row_elems relies on it).
  if (t * (K - 1) > a.hidden || t > 1024 || a.rows > kMaxGrid) return hipErrorInvalidConfiguration;
  const unsigned threads = (unsigned)t;
  if (a.w == nullptr) go_elems_hb<BF16, OP, K, PK_NONE>(a, threads, stream);
  else if (BF16 && a.w_f32) go_elems_hb<BF16, OP, K, BF16 ? PK_F32 : PK_SAME>(a, threads, stream);
  else go_elems_hb<BF16, OP, K, PK_SAME>(a, threads, stream);
  return hipGetLastError();
}

// row_elems with k elements per thread, k in [K, KMAX], picked at run time.
template <bool BF16, int OP, int K, int KMAX>
hipError_t go_rowelems_k(const RowArgs& a, int k, hipStream_t stream) {
  if (k == K) return go_rowelems<BF16, OP, K>(a, stream);
  if constexpr (K < KMAX) return go_rowelems_k<BF16, OP, K + 1, KMAX>(a, k, stream);
  return hipErrorInvalidConfiguration;
}

// Rows of single elements (a width or base that is not 16-byte granular), in blocks of at most
// 256 threads where possible, so that several rows are in flight per compute unit: rows of 1025
// to 4096 take K = ceil(n / 256) elements per thread (5 to 16) in blocks of 256 (then only a
// thread's last element can be past the row's end); narrower rows the fewest K of 1, 2 or 4 whose
// block has at most 256 threads with the same property. add-RMSNorm takes these shapes for bf16
// rows up to 2048 only. Otherwise RMSNorm and LayerNorm rows up to 4096 take K = 4, 2 or 1
// (blocks of up to 1024 threads), rows of 4097 to 8192 K = ceil(n / 512) (9 to 16) in blocks of
// 512 (bf16 [5000, 6500] RMSNorm 36.6 -> 31.7 us, LayerNorm 61.0 -> 43.2 us against K = 8 in
// blocks of up to 1024), rows of 8193 to 12288 K = ceil(n / 768) (11 to 16) in blocks of up to
// 768 (bf16 [3000, 10001] LayerNorm 61.2 -> 40.7 us against K = 12 in blocks of up to 1024);
// add-RMSNorm rows the looping kernel (*done = false). On MI355X (us, against K = 4 or 8 in
// blocks of up to 1024 threads, and add-RMSNorm on the looping kernel): RMSNorm bf16 [16384,
// 1300] 35.7 -> 24.9, [12288, 2500] 46.4 -> 29.1, [8192, 4095] 43.0 -> 33.0, LayerNorm bf16 53.5
// -> 38.9, 69.2 -> 37.5 and 72.5 -> 36.2, fp32 [4096, 4095] 38.3 -> 28.9; add-RMSNorm bf16
// [16384, 1300] 56.3 -> 44.2, [33520, 1001] 82.5 -> 64.6, [16384, 2047] 75.8 -> 63.7. add-RMSNorm
// here measured no faster at 16 per thread (bf16 [8192, 4095] 72.1 against 72.8) nor in fp32
// ([8192, 2047] 51.1 against 56.0), nor at [8184, 4100] bf16 with 576 threads per row (44% of
// peak on the looping kernel, 40% here).
template <bool BF16, int OP>
hipError_t try_rowelems(const RowArgs& a, hipStream_t stream, bool* done) {
  const int64_t n = a.hidden;
  *done = true;
  constexpr bool ADD = OP == OP_ADD_RMS;
  if (n > 1024 && n <= (ADD ? 2048 : 4096) && (!ADD || BF16))
    return go_rowelems_k<BF16, OP, 5, ADD ? 8 : 16>(a, (int)((n + 255) / 256), stream);
  auto threads = [n](int64_t k) { return ((n + k - 1) / k + 63) / 64 * 64; };
  auto small = [&](int64_t k) {
    if (ADD && !BF16) return false;
    return threads(k) <= 256 && threads(k) * (k - 1) <= n;
  };
  if (small(1)) return go_rowelems<BF16, OP, 1>(a, stream);
  if (small(2)) return go_rowelems<BF16, OP, 2>(a, stream);
  if (small(4)) return go_rowelems<BF16, OP, 4>(a, stream);
  *done = !ADD && n <= 12288;
  if (!*done) return hipSuccess;
  auto fits = [&](int64_t k) { return threads(k) * (k - 1) <= n && threads(k) <= 1024; };
  if (n > 8192) return go_rowelems_k<BF16, OP, 11, 16>(a, (int)((n + 767) / 768), stream);
  if (n > 4096) return go_rowelems_k<BF16, OP, 9, 16>(a, (int)((n + 511) / 512), stream);
  if (fits(4)) return go_rowelems<BF16, OP, 4>(a, stream);
  if (fits(2)) return go_rowelems<BF16, OP, 2>(a, stream);
  return go_rowelems<BF16, OP, 1>(a, stream);
}

template <bool BF16, int OP, int NV, int PK, bool EXACT>
hipError_t go_rowblock(const RowArgs& a, int threads, hipStream_t stream) {
  row_block<BF16, OP, NV, PK, EXACT><<<(unsigned)a.rows, threads, 0, stream>>>(a);
  return hipGetLastError();
}

// Narrow rows: teams of SUB lanes, two chunks each, 256 / SUB rows per 256-thread block.
template <bool BF16, int OP, int PK, bool EXACT, int SUB>
hipError_t go_rowsub(const RowArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + 256 / SUB - 1) / (256 / SUB);
  if (blocks > kMaxGrid) return hipErrorInvalidConfiguration;
  row_team<BF16, OP, PK, EXACT, SUB><<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int OP, int SUB>
hipError_t rowsub_pk(const RowArgs& a, bool exact, hipStream_t stream) {
  if (a.w == nullptr)
    return exact ? go_rowsub<BF16, OP, PK_NONE, true, SUB>(a, stream)
                 : go_rowsub<BF16, OP, PK_NONE, false, SUB>(a, stream);
  if constexpr (BF16) {
    if (a.w_f32)
      return exact ? go_rowsub<BF16, OP, PK_F32, true, SUB>(a, stream)
                   : go_rowsub<BF16, OP, PK_F32, false, SUB>(a, stream);
  }
  return exact ? go_rowsub<BF16, OP, PK_SAME, true, SUB>(a, stream)
               : go_rowsub<BF16, OP, PK_SAME, false, SUB>(a, stream);
}

// Rows of at most 128 chunks (1024 bf16 or 512 fp32 values): two chunks per lane and the
// smallest team of 4 .. 64 lanes that covers the row. A block of one row's team would be
// mostly idle lanes (a 128-wide bf16 row is 16 chunks, so 8 of a wave's 64 lanes).
template <bool BF16, int OP>
hipError_t try_rowsub(const RowArgs& a, int64_t n, hipStream_t stream, bool* done) {
  *done = false;
  if (n > 128) return hipSuccess;
  const int64_t half = (n + 1) / 2;
  const int sub = half <= 4 ? 4 : half <= 8 ? 8 : half <= 16 ? 16 : half <= 32 ? 32 : 64;
  const bool exact = 2 * (int64_t)sub == n;
  *done = true;
  switch (sub) {
    case 4: return rowsub_pk<BF16, OP, 4>(a, exact, stream);
    case 8: return rowsub_pk<BF16, OP, 8>(a, exact, stream);
    case 16: return rowsub_pk<BF16, OP, 16>(a, exact, stream);
    case 32: return rowsub_pk<BF16, OP, 32>(a, exact, stream);
    default: return rowsub_pk<BF16, OP, 64>(a, exact, stream);
  }
}

template <bool BF16, int OP, int NV>
hipError_t rowblock_pk(const RowArgs& a, int threads, bool exact, hipStream_t stream) {
  if (a.w == nullptr)
    return exact ? go_rowblock<BF16, OP, NV, PK_NONE, true>(a, threads, stream)
                 : go_rowblock<BF16, OP, NV, PK_NONE, false>(a, threads, stream);
  // (LayerNorm with fp32 parameters beside bf16 data takes two chunks or at least four, and
  // the RMS forms' bf16 rows with fp32 w stop at six: try_rowblock does not come here with
  // the others, and those kernels are not instantiated.)
  if constexpr (BF16 && (OP == OP_LN ? NV == 3 : NV == 8)) {
    if (a.w_f32) return hipErrorInvalidValue;
  } else if constexpr (BF16) {
    if (a.w_f32)
      return exact ? go_rowblock<BF16, OP, NV, PK_F32, true>(a, threads, stream)
                   : go_rowblock<BF16, OP, NV, PK_F32, false>(a, threads, stream);
  }
  return exact ? go_rowblock<BF16, OP, NV, PK_SAME, true>(a, threads, stream)
               : go_rowblock<BF16, OP, NV, PK_SAME, false>(a, threads, stream);
}

// One block per row: NV = max(2, ceil(n / 1024)) chunks per thread (at most 8), T = ceil(n /
// NV) rounded up to a wave. Two 16-byte chunks per thread measured best for the RMS forms:
// at hidden 8192 bf16, 512 threads with two chunks each beat 1024 threads with one
// (add-RMSNorm 172 vs 182 us, RMSNorm 86 vs 95 us); four per thread gain nothing. LayerNorm
// is bound by its fp64 arithmetic rather than by bytes in flight, and its per-row work (the
// reduction, the row scalars) is better spread over more elements per thread: NV =
// clamp(ceil(n / 256), 2, 4) (affine [16384, 8192] bf16 106 -> 102 us), except with fp32
// parameters beside bf16 data, whose widened w and b leave room for only two chunks.
template <bool BF16, int NV, int PK, bool EXACT>
hipError_t go_lnpair(const RowArgs& a, int threads, hipStream_t stream) {
  row_ln_pair<BF16, NV, PK, EXACT><<<(unsigned)((a.rows + 1) / 2), threads, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool BF16, int NV>
hipError_t lnpair_pk(const RowArgs& a, int threads, bool exact, hipStream_t stream) {
  if (a.w == nullptr)
    return exact ? go_lnpair<BF16, NV, PK_NONE, true>(a, threads, stream)
                 : go_lnpair<BF16, NV, PK_NONE, false>(a, threads, stream);
  if constexpr (BF16 && NV <= 2) {
    if (a.w_f32)
      return exact ? go_lnpair<BF16, NV, PK_F32, true>(a, threads, stream)
                   : go_lnpair<BF16, NV, PK_F32, false>(a, threads, stream);
  } else if constexpr (BF16) {
    if (a.w_f32) return hipErrorInvalidValue;  // not instantiated; try_rowblock never asks
  }
  return exact ? go_lnpair<BF16, NV, PK_SAME, true>(a, threads, stream)
               : go_lnpair<BF16, NV, PK_SAME, false>(a, threads, stream);
}

template <bool BF16, int NV, int PK, bool EXACT>
hipError_t go_rmspair(const RowArgs& a, int threads, hipStream_t stream) {
  row_rms_pair<BF16, NV, PK, EXACT><<<(unsigned)((a.rows + 1) / 2), threads, 0, stream>>>(a);
  return hipGetLastError();
}

// fp32 weights only (fp32 data, or fp32 w beside bf16 data).
template <bool BF16, int NV>
hipError_t rmspair_pk(const RowArgs& a, int threads, bool exact, hipStream_t stream) {
  constexpr int PK = BF16 ? PK_F32 : PK_SAME;
  return exact ? go_rmspair<BF16, NV, PK, true>(a, threads, stream)
               : go_rmspair<BF16, NV, PK, false>(a, threads, stream);
}

template <bool BF16, int OP>
hipError_t try_rowblock(const RowArgs& a, int64_t n, hipStream_t stream, bool* done) {
  *done = false;
  const bool ln_wide = OP == OP_LN && !(BF16 && a.w_f32);
  int64_t nv = ln_wide ? std::min<int64_t>(4, std::max<int64_t>(2, (n + 255) / 256))
                       : std::max<int64_t>(2, (n + 1023) / 1024);
  // LayerNorm past 4096 chunks: as many per thread as 1024 threads need. With fp32
  // parameters beside bf16 data, rows past 2048 chunks take at least four, the count from
  // which w and b are loaded chunk by chunk after the row's sums.
  if (ln_wide && n > 4096) nv = (n + 1023) / 1024;
  if (OP == OP_LN && !ln_wide && nv > 2) nv = std::max<int64_t>(4, nv);
  // Past 4096 chunks (16384 fp32 / 32768 bf16 values): 6 or 8 chunks per thread (the only
  // counts instantiated above 4), up to 8192 chunks, w (and b) loaded after the row's sums.
  // The RMS forms' bf16 rows with fp32 w stop at 6: eight widened fp32 w chunks spill at 8.
  if (nv > 4) nv = nv <= 6 ? 6 : 8;
  if (OP != OP_LN && nv == 8 && BF16 && a.w != nullptr && a.w_f32) return hipSuccess;
  if (nv > 8 || n > nv * 1024 || a.rows > kMaxGrid) return hipSuccess;
  const int threads = (int)((((n + nv - 1) / nv) + 63) / 64 * 64);
  const bool exact = (int64_t)threads * nv == n;
  *done = true;
  // LayerNorm with a scale or shift over 4096 rows or more: two rows per block (w and b
  // loaded once per pair). bf16 [16384, 8192] 99 -> 92 us, fp32 207 -> 173 us, bf16 beside
  // fp32 w and b [16384, 4096] 62 -> 52 us. Without parameters the pair's extra registers cost
  // more than it saves (84 -> 88 us), so that case keeps one row per block.
  // RMSNorm with fp32 weights over 4096 rows or more: two rows per block as well (w is as
  // large as an fp32 row, twice a bf16 one): fp32 [16384, 8192] 177 -> 168 us, bf16 beside
  // fp32 w [16384, 4096] 49 -> 44 us. With bf16 w it measured no faster.
  if constexpr (OP == OP_RMS) {
    if (a.rows >= 4096 && a.w != nullptr && (!BF16 || a.w_f32)) {
      switch (nv) {
        case 2: return rmspair_pk<BF16, 2>(a, threads, exact, stream);
        case 3: return rmspair_pk<BF16, 3>(a, threads, exact, stream);
        case 4: return rmspair_pk<BF16, 4>(a, threads, exact, stream);
        default: break;
      }
    }
  }
  if constexpr (OP == OP_LN) {
    // (fp32 parameters beside bf16 data pair only at two chunks: lnpair_pk reads them as fp32
    // there alone.)
    if (a.rows >= 4096 && (a.w != nullptr || a.b != nullptr) && (ln_wide || nv == 2)) {
      switch (nv) {
        case 2: return lnpair_pk<BF16, 2>(a, threads, exact, stream);
        case 3: return lnpair_pk<BF16, 3>(a, threads, exact, stream);
        case 4: return lnpair_pk<BF16, 4>(a, threads, exact, stream);
        default: break;
      }
    }
  }
  switch (nv) {
    case 1: return rowblock_pk<BF16, OP, 1>(a, threads, exact, stream);
    case 2: return rowblock_pk<BF16, OP, 2>(a, threads, exact, stream);
    case 3: return rowblock_pk<BF16, OP, 3>(a, threads, exact, stream);
    case 4: return rowblock_pk<BF16, OP, 4>(a, threads, exact, stream);
    case 6: return rowblock_pk<BF16, OP, 6>(a, threads, exact, stream);
    case 8: return rowblock_pk<BF16, OP, 8>(a, threads, exact, stream);
    default: break;
  }
  *done = false;
  return hipSuccess;
}

// One wave per row: chunks per lane needed -> instantiated NV (0: does not fit).
template <bool BF16, int OP>
hipError_t try_wave(const RowArgs& a, int per_lane, hipStream_t stream, bool* done) {
  *done = true;
  if constexpr (BF16) {  // hidden <= 8192
    switch (per_lane) {
      case 1: return go_wave<BF16, OP, 1>(a, stream);
      case 2: return go_wave<BF16, OP, 2>(a, stream);
      case 3: case 4: return go_wave<BF16, OP, 4>(a, stream);
      case 5: case 6: return go_wave<BF16, OP, 6>(a, stream);
      case 7: case 8: return go_wave<BF16, OP, 8>(a, stream);
      case 9: case 10: return go_wave<BF16, OP, 10>(a, stream);
      case 11: case 12: return go_wave<BF16, OP, 12>(a, stream);
      case 13: case 14: case 15: case 16: return go_wave<BF16, OP, 16>(a, stream);
      default: break;
    }
  } else {  // hidden <= 8192
    switch (per_lane) {
      case 1: return go_wave<BF16, OP, 1>(a, stream);
      case 2: return go_wave<BF16, OP, 2>(a, stream);
      case 3: case 4: return go_wave<BF16, OP, 4>(a, stream);
      case 5: case 6: case 7: case 8: return go_wave<BF16, OP, 8>(a, stream);
      case 9: case 10: case 11: case 12: return go_wave<BF16, OP, 12>(a, stream);
      case 13: case 14: case 15: case 16: return go_wave<BF16, OP, 16>(a, stream);
      case 17: case 18: case 19: case 20: return go_wave<BF16, OP, 20>(a, stream);
      case 21: case 22: case 23: case 24: return go_wave<BF16, OP, 24>(a, stream);
      default:
        if (per_lane <= 32) return go_wave<BF16, OP, 32>(a, stream);
        break;
    }
  }
  *done = false;
  return hipSuccess;
}

template <bool BF16, int OP>
hipError_t try_block(const RowArgs& a, int per_thread, hipStream_t stream, bool* done) {
  *done = true;
  switch (per_thread) {
    case 1: return go_block<BF16, OP, 1>(a, stream);
    case 2: return go_block<BF16, OP, 2>(a, stream);
    case 3: case 4: return go_block<BF16, OP, 4>(a, stream);
    case 5: case 6: case 7: case 8: return go_block<BF16, OP, 8>(a, stream);
    default:
      if (per_thread <= 16) return go_block<BF16, OP, 16>(a, stream);
      break;
  }
  *done = false;
  return hipSuccess;
}

template <bool BF16, int OP>
hipError_t launch_row_once(const RowArgs& a, bool aligned16, hipStream_t stream) {
  constexpr int V = Fmt<BF16>::VEC;
  const int path = forced_path();
  const bool vec = aligned16 && a.hidden % V == 0 && path != PATH_SCALAR;
  if (!vec) {
    if (path == PATH_AUTO) {
      bool done = false;
      const hipError_t e = try_rowelems<BF16, OP>(a, stream, &done);
      if (done) return e;
    }
    return go_chunked<BF16, OP, 1>(a, stream);
  }
  const int64_t n = a.hidden / V;
  bool done = false;
  hipError_t err = hipSuccess;
  if (path == PATH_WAVE && (a.rows + 3) / 4 <= kMaxGrid) {
    err = try_wave<BF16, OP>(a, (int)((n + 63) / 64), stream, &done);
    if (done) return err;
  }
  if (path == PATH_BLOCK && a.rows <= kMaxGrid) {
    err = try_block<BF16, OP>(a, (int)((n + 511) / 512), stream, &done);
    if (done) return err;
  }
  if (path == PATH_AUTO) {
    err = try_rowsub<BF16, OP>(a, n, stream, &done);
    if (done) return err;
  }
  if (path == PATH_AUTO || path == PATH_ROWBLOCK || path == PATH_WAVE || path == PATH_BLOCK) {
    err = try_rowblock<BF16, OP>(a, n, stream, &done);
    if (done) return err;
  }
  return go_chunked<BF16, OP, V>(a, stream);
}

// Bytes one launch streams at most (every array's rows: x and out, and r and h for
// add-RMSNorm). On MI355X one launch over much more than 1 GiB streams slower than the same
// rows launched in consecutive pieces of about 1 GiB, though each piece ends with a drain:
// add-RMSNorm bf16 [65536, 5120] 445.6 -> 434.7 us, fp32 [65536, 5120] 890.3 -> 862.4 us, bf16
// [65536, 8192] 745.6 -> 701.2 us; at 1 GiB itself (bf16 [16384, 8192]) one launch is fastest.
constexpr int64_t kLaunchBytes = int64_t(1) << 30;

}  // namespace

// Rows of whole 16-byte chunks on the automatic path are launched in pieces of at most
// kLaunchBytes (an even number of rows, so that the two-row kernels see whole pairs); each
// piece is the same call on the rows it covers, at offset pointers (a row's outputs depend on
// that row and the parameters only).
template <bool BF16, int OP>
hipError_t launch_row(const RowArgs& a, bool aligned16, hipStream_t stream) {
  constexpr int V = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  const int64_t row_bytes = a.hidden * ESZ * (OP == OP_ADD_RMS ? 4 : 2);
  const bool whole = aligned16 && a.hidden % V == 0 && forced_path() == PATH_AUTO;
  if (!whole || row_bytes <= 0 || a.rows <= kLaunchBytes / row_bytes)
    return launch_row_once<BF16, OP>(a, aligned16, stream);
  const int64_t per = std::max<int64_t>(2, (kLaunchBytes / row_bytes) & ~int64_t(1));
  for (int64_t r0 = 0; r0 < a.rows; r0 += per) {
    RowArgs p = a;
    const int64_t off = r0 * a.hidden * ESZ;
    p.x = (const char*)a.x + off;
    if (a.r) p.r = (const char*)a.r + off;
    p.out = (char*)a.out + off;
    if (a.h) p.h = (char*)a.h + off;
    p.rows = std::min(per, a.rows - r0);
    const hipError_t e = launch_row_once<BF16, OP>(p, aligned16, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nrm

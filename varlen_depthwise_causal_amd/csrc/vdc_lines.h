// Which of a lane's row stores cover a whole 128-byte cache line together
// with the other lanes of the same wave, for rows that are not a multiple of
// 128 bytes.  Kept apart, in 64-bit host/device arithmetic, so that a CPU
// program can check it against every byte of a simulated grid.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define VDC_LINES_HD __host__ __device__
#else
#define VDC_LINES_HD
#endif

namespace vdc {

// The lanes of a wave that share a band write one contiguous piece of each
// row: lane `lane` (0..63) holds channel vector `vec` (0..nvec-1) of its
// band, `lane_bytes` bytes, and vec counts up by one per lane within the
// band.  Bit p of the result is set when the lane's bytes of the store at
// byte address at0 + p row_bytes lie in a 128-byte line that the lane's
// piece covers entirely: no other wave, and no other row, writes into that
// line.  With lane_bytes and row_bytes multiples of 16, the line offset of
// a row start repeats every 8 rows, so bits 0..7 describe every row whose
// distance from at0's row is congruent to p modulo 8.
VDC_LINES_HD inline uint32_t whole_line_bits(int64_t at0, int64_t row_bytes, uint32_t lane,
                                             uint32_t vec, int64_t nvec, int lane_bytes) {
  const int64_t first = lane >= vec ? (int64_t)(lane - vec) : 0;
  const int64_t last_in_band = (int64_t)lane + (nvec - 1 - (int64_t)vec);
  const int64_t last = last_in_band < 63 ? last_in_band : 63;
  uint32_t bits = 0;
  for (int p = 0; p < 8; ++p) {
    const int64_t at = at0 + (int64_t)p * row_bytes;
    const int64_t piece_lo = at - (int64_t)lane_bytes * ((int64_t)lane - first);
    const int64_t piece_hi = at + (int64_t)lane_bytes * (last - (int64_t)lane + 1);
    const int64_t line = at & ~(int64_t)127;
    if (line >= piece_lo && line + 128 <= piece_hi) bits |= 1u << p;
  }
  return bits;
}

}  // namespace vdc

// CPU check of the forward's store-policy split on rows that are not a
// multiple of 128 bytes (varlen_depthwise_causal_amd/csrc/vdc_lines.h).
// A grid of bands of T rows, lanes laid out as band * nvec + vec, is
// simulated for many row lengths, band lengths, base alignments and waves;
// for every lane and row phase the function's answer must equal the brute
// force one: every 8-byte slot of the lane's 128-byte line is written, for
// the same row, by a lane of the same wave and band.  Base addresses are
// 8-byte aligned or more.  The answer must not change when a multiple of 8
// rows is added.  Prints "lines_check: ok" and exits 0, or names the
// failing case.
#include <stdint.h>
#include <stdio.h>

#include "vdc_lines.h"

namespace {

// Lane owning byte `addr` for row t of some band, or -1 (outside the grid
// or another row).  Rows of band b are rows b*T .. b*T+T-1 of the tensor.
int64_t owner(int64_t base, int64_t addr, int64_t row_bytes, int64_t T, int64_t t, int64_t nvec,
              int64_t bands) {
  const int64_t rel = addr - base;
  if (rel < 0) return -1;
  const int64_t row = rel / row_bytes;
  const int64_t band = row / T;
  if (row % T != t || band >= bands) return -1;
  return band * nvec + (rel % row_bytes) / 8;
}

}  // namespace

int main() {
  const int64_t Cs[] = {8, 16, 24, 40, 56, 64, 120, 264, 520, 1000, 1544, 2048, 4104, 6400};
  const int64_t Ts[] = {16, 32, 48, 128};
  const int64_t bases[] = {0, 8, 16, 24, 48, 256, 4096 + 80, 4096 + 8};
  long checked = 0, whole = 0;
  for (int64_t C : Cs)
    for (int64_t T : Ts)
      for (int64_t base : bases) {
        const int64_t nvec = C / 4, row_bytes = 2 * C, bands = 40;
        const int64_t lanes = bands * nvec;
        for (int64_t w0 = 0; w0 + 64 <= lanes; w0 += 64 * 3) {
          for (uint32_t l = 0; l < 64; ++l) {
            const int64_t g = w0 + l;
            const int64_t band = g / nvec, vec = g % nvec;
            // Address of the lane's bytes in row 0 of its band, and the
            // function's answer for rows 0..7 (and 8..15 from at0 + 8 rows).
            const int64_t at0 = base + band * T * row_bytes + vec * 8;
            const uint32_t bits =
                vdc::whole_line_bits(at0, row_bytes, l, (uint32_t)vec, nvec, 8);
            const uint32_t bits8 =
                vdc::whole_line_bits(at0 + 8 * row_bytes, row_bytes, l, (uint32_t)vec, nvec, 8);
            if (bits != bits8) {
              printf("not periodic: C=%lld T=%lld base=%lld lane=%lld\n", (long long)C,
                     (long long)T, (long long)base, (long long)g);
              return 1;
            }
            for (int64_t t = 0; t < 8 && t < T; ++t) {
              const int64_t at = at0 + t * row_bytes;
              const int64_t line = at & ~(int64_t)127;
              bool all = true;
              for (int64_t q = 0; q < 16 && all; ++q) {
                const int64_t o = owner(base, line + 8 * q, row_bytes, T, t, nvec, bands);
                all = o >= w0 && o < w0 + 64 && o / nvec == band;
              }
              const bool got = (bits >> t) & 1u;
              ++checked;
              whole += got;
              if (got != all) {
                printf("mismatch: C=%lld T=%lld base=%lld lane=%lld row=%lld got=%d want=%d\n",
                       (long long)C, (long long)T, (long long)base, (long long)g, (long long)t,
                       (int)got, (int)all);
                return 1;
              }
            }
          }
        }
      }
  printf("lines_check: ok (%ld lane-rows, %ld in whole lines)\n", checked, whole);
  return 0;
}

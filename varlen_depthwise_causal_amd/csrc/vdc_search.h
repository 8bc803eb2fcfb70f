// Bracket arithmetic of the 64-ary lower-bound search over cu_seqlens that
// the kernels run with one wave (64 lanes probing at once).  Kept apart, in
// 64-bit arithmetic, so that a CPU program can run the same steps with an
// emulated ballot: the bracket reaches 2^31 - 1 entries, where 32-bit sums
// of the probe offsets would wrap.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define VDC_HD __host__ __device__
#else
#define VDC_HD
#endif

namespace vdc {

// Spacing of the 64 probes in the bracket [lo, hi) (lo < hi): probe q sits
// at lo + q * step, so the probes span the bracket.
VDC_HD inline int64_t search_step(int64_t lo, int64_t hi) { return (hi - lo + 63) >> 6; }

// Entry probed by lane q, or -1 when it lies at or past hi (no probe).
VDC_HD inline int64_t search_probe(int64_t lo, int64_t hi, int64_t step, int q) {
  const int64_t idx = lo + (int64_t)q * step;
  return idx < hi ? idx : -1;
}

// Narrows [lo, hi) given c, the number of leading probes (lanes 0 .. c-1)
// whose entry is below the value sought: the answer lies after probe c-1
// and at or before probe c.  The bracket shrinks at least 64-fold per round
// and stays inside the previous one.
VDC_HD inline void search_narrow(int64_t& lo, int64_t& hi, int64_t step, int c) {
  const int64_t nlo = c == 0 ? lo : lo + (int64_t)(c - 1) * step + 1;
  const int64_t nhi = lo + (int64_t)c * step;
  hi = nhi < hi ? nhi : hi;
  lo = nlo;
}

}  // namespace vdc

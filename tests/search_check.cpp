// CPU check of the kernels' 64-ary lower-bound search over cu_seqlens
// (varlen_depthwise_causal_amd/csrc/vdc_search.h): the same bracket steps,
// with the wave's ballot emulated by a loop over 64 lanes.  cu is a
// function of the index, so brackets of up to 2^31 - 1 entries need no
// memory.  Checks, for sorted and for arbitrary (malformed) contents:
// every probe lies in [0, n), the search ends within 6 rounds, and for
// sorted contents it returns the first index whose entry is >= v.
// Prints "search_check: ok" and exits 0, or names the failing case.
#include <stdint.h>
#include <stdio.h>

#include <functional>

#include "vdc_search.h"

namespace {

int64_t emulated_search(const std::function<int32_t(int64_t)>& cu, int64_t n, int32_t v,
                        int& rounds, bool& in_range) {
  int64_t lo = 0, hi = n;
  rounds = 0;
  in_range = true;
  while (lo < hi) {
    const int64_t step = vdc::search_step(lo, hi);
    uint64_t ball = 0;
    for (int q = 0; q < 64; ++q) {
      const int64_t idx = vdc::search_probe(lo, hi, step, q);
      if (idx >= 0 && (idx >= n || idx < 0)) in_range = false;
      if (idx >= n) in_range = false;
      const bool less = idx >= 0 && idx < n && cu(idx) < v;
      if (less) ball |= uint64_t(1) << q;
    }
    const int c = ~ball == 0 ? 64 : __builtin_ctzll(~ball);
    vdc::search_narrow(lo, hi, step, c);
    if (++rounds > 6) return -1;
  }
  return lo;
}

// First index with cu[i] >= v for nondecreasing cu, by bisection.
int64_t reference(const std::function<int32_t(int64_t)>& cu, int64_t n, int32_t v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (cu(mid) < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

uint64_t mix(uint64_t x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdull;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ull;
  return x ^ (x >> 33);
}

int failures = 0;

void check(const char* what, const std::function<int32_t(int64_t)>& cu, int64_t n, int32_t v,
           bool sorted) {
  int rounds = 0;
  bool in_range = true;
  const int64_t got = emulated_search(cu, n, v, rounds, in_range);
  bool ok = got >= 0 && got <= n && in_range;
  if (ok && sorted) ok = got == reference(cu, n, v);
  if (!ok) {
    ++failures;
    printf("FAIL %s: n=%lld v=%d got=%lld rounds=%d in_range=%d\n", what, (long long)n, v,
           (long long)got, rounds, (int)in_range);
  }
}

}  // namespace

int main() {
  const int64_t kMaxN = (int64_t(1) << 31) - 1;  // entries: num_docs + 1 <= 2^31 - 1
  const int64_t sizes[] = {1, 2, 3, 63, 64, 65, 4095, 4096, 4097, 20001, 1 << 20,
                           (int64_t(1) << 30) + 7, kMaxN - 64, kMaxN - 1, kMaxN};
  for (int64_t n : sizes) {
    // cu[i] = i: every document of length 1 (S = n - 1).
    auto ident = [](int64_t i) { return (int32_t)i; };
    const int32_t top = (int32_t)(n - 1);
    const int32_t vs[] = {0, 1, top / 3, top / 2, top - 1, top, top == INT32_MAX ? top : top + 1};
    for (int32_t v : vs) check("identity", ident, n, v, true);
    // mostly empty documents: cu[i] = floor(i / 1000)
    auto sparse = [](int64_t i) { return (int32_t)(i / 1000); };
    for (int32_t v : {0, 1, (int32_t)((n - 1) / 2000), (int32_t)((n - 1) / 1000)})
      check("empty documents", sparse, n, v, true);
    // arbitrary contents (a caller's broken cu_seqlens): only safety holds
    for (uint64_t seed = 0; seed < 4; ++seed) {
      auto junk = [seed](int64_t i) { return (int32_t)(mix((uint64_t)i ^ (seed << 40)) >> 33); };
      for (int32_t v : {0, 12345, 1 << 30, INT32_MAX}) check("malformed", junk, n, v, false);
    }
  }
  if (failures) {
    printf("search_check: %d failures\n", failures);
    return 1;
  }
  printf("search_check: ok\n");
  return 0;
}

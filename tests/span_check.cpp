// Host-only check of packed_side (exact_block_wise_amd/csrc/span.hpp): for
// any prefix-sum values the clamped span stays inside the tensors and inside
// the launch bound, and for arrays that keep the documented rules it is the
// identity.  Built with g++ and the address / undefined-behaviour
// sanitizers by tests/test_span_cpu.py; prints "ok <cases>" on success.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "span.hpp"

using exattn::packed_side;

static int fails = 0;
static long cases = 0;

static void check_bounds(int lo, int hi, int max_len, int64_t total) {
  int r, n;
  packed_side(lo, hi, max_len, total, r, n);
  ++cases;
  const int64_t t = total > 0 ? total : 0;
  const int64_t cap = max_len > 0 ? max_len : 0;
  const bool ok = r >= 0 && n >= 0 && (int64_t)r + n <= t && n <= cap && (int64_t)r <= t;
  if (!ok && fails++ < 10)
    printf("out of bounds: lo=%d hi=%d max=%d total=%lld -> row0=%d n=%d\n", lo, hi, max_len,
           (long long)total, r, n);
}

static void check_identity(int lo, int hi, int max_len, int64_t total) {
  int r, n;
  packed_side(lo, hi, max_len, total, r, n);
  ++cases;
  if ((r != lo || n != hi - lo) && fails++ < 10)
    printf("well-formed span changed: lo=%d hi=%d max=%d total=%lld -> row0=%d n=%d\n", lo, hi,
           max_len, (long long)total, r, n);
}

// splitmix64: a fixed, seeded stream of test values
static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint64_t next64() {
  uint64_t z = (state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

int main() {
  const int edge[] = {INT_MIN, INT_MIN + 1, -1000000, -33, -1, 0, 1, 7, 31, 32, 33,
                      196, 1568, 4096, 1 << 20, INT_MAX - 1, INT_MAX};
  const int64_t totals[] = {0, 1, 32, 196, 6272, 1 << 20, (int64_t)INT_MAX, (int64_t)1 << 35};
  for (int lo : edge)
    for (int hi : edge)
      for (int mx : edge)
        for (int64_t t : totals) check_bounds(lo, hi, mx, t);
  for (int i = 0; i < 2000000; ++i) {
    const uint64_t x = next64(), y = next64();
    const int lo = (int)(x & 0xffffffffu), hi = (int)(x >> 32);
    const int mx = (int)(y & 0xffffffffu) >> (y >> 59);
    const int64_t t = (int64_t)((y >> 32) & 0x7fffffffu) >> ((y >> 27) & 31);
    check_bounds(lo, hi, mx, t);
    check_bounds(lo & 0xfff, hi & 0xfff, mx & 0x3ff, t & 0x1fff);
  }
  // well-formed spans: 0 <= lo <= hi <= total and hi - lo <= max_len
  for (int i = 0; i < 200000; ++i) {
    const uint64_t x = next64();
    const int64_t total = (int64_t)(x & 0xffffff);
    const int lo = total ? (int)((x >> 24) % (uint64_t)(total + 1)) : 0;
    const int len = (int)((x >> 48) % (uint64_t)(total - lo + 1));
    const int extra = (int)(next64() & 0xff);
    check_identity(lo, lo + len, len + extra, total);
    check_identity(lo, lo + len, len > 0 ? len : 1, total);
  }
  // a pair out of order is an empty sequence
  for (int lo = 0; lo < 64; ++lo)
    for (int hi = 0; hi < lo; ++hi) {
      int r, n;
      packed_side(lo, hi, 1 << 20, 100, r, n);
      ++cases;
      if (n != 0 && fails++ < 10) printf("decreasing pair %d > %d gave n=%d\n", lo, hi, n);
    }
  if (fails) {
    printf("FAILED %d of %ld\n", fails, cases);
    return 1;
  }
  printf("ok %ld\n", cases);
  return 0;
}

// Row spans of packed variable-length sequences, shared by the kernels
// (through seq_span in kernels.hpp) and by a host-only unit test, so it
// includes no HIP header.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define EXATTN_HD __host__ __device__
#else
#define EXATTN_HD
#endif

namespace exattn {

// The rows of one (sequence, head) problem: dense [B,H,N,d] tensors, or
// packed variable-length sequences.
struct SeqSpan {
  int q_row0, kv_row0;  // first query / key token of the sequence (0: dense)
  int nq, nkv;          // its query and key/value lengths
  int64_t stat0;        // index of its first query row in LSE and D
};

// One side of packed sequence s from its prefix-sum entries lo = cu[s] and
// hi = cu[s + 1]: the first token row0 and the length n.  The caller's
// arrays are device data that the host never sees, so they are clamped
// here rather than trusted: the rows always lie in [0, total) and n never
// exceeds max_len (the launch bound), whatever lo and hi hold.  For arrays
// that keep the documented rules (0 <= lo <= hi <= total, hi - lo <=
// max_len) this is the identity; a pair out of order is an empty sequence.
EXATTN_HD inline void packed_side(int lo, int hi, int max_len, int64_t total, int& row0,
                                  int& n) {
  const int64_t t = total > 0 ? total : 0;
  int64_t r = lo > 0 ? lo : 0;
  if (r > t) r = t;
  int64_t e = hi < t ? hi : t;
  if (e < r) e = r;
  int64_t len = e - r;
  const int64_t cap = max_len > 0 ? max_len : 0;
  if (len > cap) len = cap;
  row0 = (int)r;
  n = (int)len;
}

}  // namespace exattn

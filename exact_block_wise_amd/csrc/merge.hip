// Exact merge of partial attention results over disjoint key/value sets.
//
// exp(LSE) of a union of key sets is the sum of the parts' exp(LSE), so
//   M = max_c LSE_c, LSE = M + ln sum_c exp(LSE_c - M),
//   O = sum_c exp(LSE_c - LSE) O_c
// reproduces the unsplit result exactly (LV-XAttn abstract and lay summary:
// the distributed cross-attention is exact and leaves the output unchanged).
// The kernel is bandwidth-bound: one thread per 4 output values, 16-byte
// loads of each partial, the row's n_parts LSE values re-read from L1/L2.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace exattn {

template <bool OUT_F32>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  const int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int d4 = a.d / 4;
  const int64_t rows = (int64_t)a.B * a.H * a.Nq;
  if (e4 >= rows * d4) return;
  const int c4 = (int)(e4 % d4) * 4;
  const int64_t row = e4 / d4;
  float mx = -INFINITY;
  for (int p = 0; p < a.n_parts; ++p) mx = fmaxf(mx, a.lse_parts[(int64_t)p * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float tot = 0.f;
    for (int p = 0; p < a.n_parts; ++p) tot += expf(a.lse_parts[(int64_t)p * rows + row] - mx);
    lse = mx + logf(tot);
    for (int p = 0; p < a.n_parts; ++p) {
      const float wgt = expf(a.lse_parts[(int64_t)p * rows + row] - lse);
      const f32x4 v =
          *reinterpret_cast<const f32x4*>(a.o_parts + ((int64_t)p * rows + row) * a.d + c4);
      acc += wgt * v;
    }
  }
  const int i = (int)(row % a.Nq);
  const int64_t bh = row / a.Nq;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int64_t off = b * a.os.sb + h * a.os.sh + (int64_t)i * a.os.sn + c4;
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>((float*)a.o + off) = acc;
  } else {
    bf16x4 o4 = {(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
    *reinterpret_cast<bf16x4*>((bf16*)a.o + off) = o4;
  }
  if (c4 == 0) a.lse[row] = lse;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const long long n4 = (long long)a.B * a.H * a.Nq * (a.d / 4);
  const long long grid = (n4 + 255) / 256;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.out_f32)
    hipLaunchKernelGGL(lse_merge_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(lse_merge_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace exattn

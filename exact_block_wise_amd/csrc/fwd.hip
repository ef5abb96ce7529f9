// Forward kernels: block-wise exact softmax attention with an online softmax.
//
// The Nq x Nkv weights are never stored: each workgroup keeps, per query
// row, the running maximum m, the running sum l and an fp32 output
// accumulator in registers, and folds in one key/value tile at a time
// ("Training a Large Video Model on a Single Machine in a Day", sections 1
// and 3: block results combined into the final output, O(N) memory).
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace exattn {

// --------------------------------------------------------------------------
// bf16 inputs, bf16 matrix cores (32x32x16), fp32 accumulation.
//
// Workgroup: 4 waves, 128 query rows (32 per wave).  Key/value tiles of 64
// rows are staged in LDS: K row-major, V transposed.  Each wave computes the
// transposed score tile S^T = K Q^T so that every lane owns one query row
// (column n = lane % 32 of the accumulator): the softmax statistics are then
// per-lane scalars, and the exponentiated tile is already laid out as the B
// operand of O^T += V^T P^T.
// --------------------------------------------------------------------------
namespace fwdk {
constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NT = 256;
}  // namespace fwdk

template <int D, bool OUT_F32>
__global__ __launch_bounds__(fwdk::NT) void fwd_bf16_kernel(FwdArgs a) {
  using namespace fwdk;
  constexpr int DP = (D + 31) / 32 * 32;  // output rows in 32-row blocks
  constexpr int NDB = DP / 32;
  constexpr int KC = D / 16;              // contraction chunks of QK^T
  constexpr int KS = D + 8;               // K tile row stride (elements)
  constexpr int VS = BN + 4;              // V^T tile row stride (elements)
  __shared__ __attribute__((aligned(16))) bf16 Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[DP * VS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ln = lane & 31, g = lane >> 5;

  const int nqb = (a.Nq + BM - 1) / BM;
  int idx = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = idx % nqb;
  idx /= nqb;
  const int h = idx % a.H;
  idx /= a.H;
  const int b = idx % a.B;
  const int c = idx / a.B;

  const int kv_lo = c * a.chunk_len;
  const int kv_hi = min(a.Nkv, kv_lo + a.chunk_len);
  const int n_kv = max(0, kv_hi - kv_lo);

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh + (int64_t)kv_lo * a.ks.sn;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh + (int64_t)kv_lo * a.vs.sn;

  const int q0 = qb * BM + w * 32;
  const bool wave_active = q0 < a.Nq;
  const int qrow = q0 + ln;
  const bool qvalid = qrow < a.Nq;

  // Padding rows of V^T (D <= d < DP) feed only discarded output rows; clear
  // them once so they hold finite values.
  if constexpr (DP != D) {
    for (int i = tid; i < (DP - D) * VS; i += NT) Vt[D * VS + i] = (bf16)0.f;
  }

  bf16x8 qreg[KC];
  const bf16x8 zero8 = {};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qreg[kc] = qvalid ? load_bf16x8(qp + (int64_t)qrow * a.qs.sn + 16 * kc + 8 * g) : zero8;

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;  // running max of the log2-scaled scores
  float l = 0.f;        // this lane's share of the running sum
  const float sl2 = a.scale * kLog2e;

  for (int j0 = 0; j0 < n_kv; j0 += BN) {
    __syncthreads();
    // K tile, row-major: consecutive threads read consecutive 16-byte pieces
    // of a row.
    for (int e = tid; e < BN * (D / 8); e += NT) {
      const int r = e / (D / 8), cc = e % (D / 8);
      bf16x8 val = zero8;
      if (j0 + r < n_kv) val = load_bf16x8(kp + (int64_t)(j0 + r) * a.ks.sn + 8 * cc);
      *reinterpret_cast<bf16x8*>(&Ks[r * KS + 8 * cc]) = val;
    }
    // V tile, transposed: consecutive threads take consecutive rows so the
    // 2-byte LDS writes of one instruction fall in distinct banks.
    for (int e = tid; e < BN * (D / 8); e += NT) {
      const int r = e % BN, cc = e / BN;
      bf16x8 val = zero8;
      if (j0 + r < n_kv) val = load_bf16x8(vp + (int64_t)(j0 + r) * a.vs.sn + 8 * cc);
#pragma unroll
      for (int i = 0; i < 8; ++i) Vt[(8 * cc + i) * VS + r] = val[i];
    }
    __syncthreads();
    if (!wave_active) continue;

    // S^T (two 32-row key blocks) = K Q^T
    f32x16 s[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      s[cb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8 ka = load_bf16x8(&Ks[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
        s[cb] = mfma32(ka, qreg[kc], s[cb]);
      }
    }
    // scale to log2 units, mask the ragged tail, row maximum
    float mx = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kv = j0 + 32 * cb + 8 * (e >> 2) + 4 * g + (e & 3);
        const float x = kv < n_kv ? s[cb][e] * sl2 : -INFINITY;
        s[cb][e] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(s[cb][e] - m_new);
        s[cb][e] = p;
        rs += p;
      }
    }
    l = l * alpha + rs;
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;

    // O^T += V^T P^T over four 16-key chunks.  Chunk t = 2*cb + hh holds,
    // for group g, keys 16t + 4g + (0..3) and 16t + 8 + 4g + (0..3): the
    // accumulator entries 8hh .. 8hh+7 of key block cb.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 pb = acc_half_to_bf16(s[t >> 1], t & 1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16* vr = &Vt[(32 * db + ln) * VS + 16 * t + 4 * g];
        const bf16x8 va = cat4(*reinterpret_cast<const bf16x4*>(vr),
                               *reinterpret_cast<const bf16x4*>(vr + 8));
        oacc[db] = mfma32(va, pb, oacc[db]);
      }
    }
  }

  if (!wave_active) return;
  l += xor32(l);
  if (!qvalid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (int64_t)c * a.o_chunk_stride + b * a.os.sb + h * a.os.sh +
                       (int64_t)qrow * a.os.sn;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * g;
      if (d0 < D) {
        if constexpr (OUT_F32) {
          f32x4 v4 = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv,
                      oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv};
          *reinterpret_cast<f32x4*>((float*)a.o + orow + d0) = v4;
        } else {
          bf16x4 v4 = {(bf16)(oacc[db][4 * i] * inv), (bf16)(oacc[db][4 * i + 1] * inv),
                       (bf16)(oacc[db][4 * i + 2] * inv), (bf16)(oacc[db][4 * i + 3] * inv)};
          *reinterpret_cast<bf16x4*>((bf16*)a.o + orow + d0) = v4;
        }
      }
    }
  }
  if (g == 0) {
    const int64_t li = (int64_t)c * a.lse_chunk_stride + ((int64_t)b * a.H + h) * a.Nq + qrow;
    a.lse[li] = l > 0.f ? m * kLn2 + logf(l) : -INFINITY;
  }
}

// --------------------------------------------------------------------------
// fp32 inputs: genuine fp32 products and sums on the vector ALUs, exact
// library exp/log.  One lane per query row; key/value tiles of 32 rows in
// LDS are read by broadcast.  Meant for small problems that need fp32
// accuracy; it is not tuned.
// --------------------------------------------------------------------------
namespace fwdf {
constexpr int BM = 64;
constexpr int BN = 32;
}  // namespace fwdf

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgs a) {
  using namespace fwdf;
  __shared__ float Ks[BN][D];
  __shared__ float Vs[BN][D];
  const int tid = threadIdx.x;
  const int nqb = (a.Nq + BM - 1) / BM;
  int idx = blockIdx.x;
  const int qb = idx % nqb;
  idx /= nqb;
  const int h = idx % a.H;
  idx /= a.H;
  const int b = idx % a.B;
  const int c = idx / a.B;
  const int kv_lo = c * a.chunk_len;
  const int n_kv = max(0, min(a.Nkv, kv_lo + a.chunk_len) - kv_lo);

  const float* qp = (const float*)a.q + b * a.qs.sb + h * a.qs.sh;
  const float* kp = (const float*)a.k + b * a.ks.sb + h * a.ks.sh + (int64_t)kv_lo * a.ks.sn;
  const float* vp = (const float*)a.v + b * a.vs.sb + h * a.vs.sh + (int64_t)kv_lo * a.vs.sn;
  const int qrow = qb * BM + tid;
  const bool qvalid = qrow < a.Nq;

  float qv[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qv[i] = qvalid ? qp[(int64_t)qrow * a.qs.sn + i] : 0.f;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 < n_kv; j0 += BN) {
    __syncthreads();
    for (int e = tid; e < BN * D; e += 64) {
      const int r = e / D, cc = e % D;
      const bool ok = j0 + r < n_kv;
      Ks[r][cc] = ok ? kp[(int64_t)(j0 + r) * a.ks.sn + cc] : 0.f;
      Vs[r][cc] = ok ? vp[(int64_t)(j0 + r) * a.vs.sn + cc] : 0.f;
    }
    __syncthreads();
    const int nj = min(BN, n_kv - j0);
    float sc[BN];
    float mx = -INFINITY;
    for (int j = 0; j < BN; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = fmaf(qv[i], Ks[j][i], dot);
      sc[j] = j < nj ? dot * a.scale : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= alpha;
    for (int j = 0; j < BN; ++j) {
      const float p = expf(sc[j] - m_new);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(p, Vs[j][i], acc[i]);
    }
    m = m_new;
  }
  if (!qvalid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (int64_t)c * a.o_chunk_stride + b * a.os.sb + h * a.os.sh +
                       (int64_t)qrow * a.os.sn;
  for (int i = 0; i < D; ++i) ((float*)a.o)[orow + i] = acc[i] * inv;
  const int64_t li = (int64_t)c * a.lse_chunk_stride + ((int64_t)b * a.H + h) * a.Nq + qrow;
  a.lse[li] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D>
static hipError_t fwd_bf16_d(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + fwdk::BM - 1) / fwdk::BM;
  const long long grid = (long long)nqb * a.H * a.B * a.n_chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.out_f32)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, true>), dim3((unsigned)grid), dim3(fwdk::NT), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, false>), dim3((unsigned)grid), dim3(fwdk::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return fwd_bf16_d<64>(a, s);
    case 80: return fwd_bf16_d<80>(a, s);
    case 128: return fwd_bf16_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t fwd_f32_d(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + fwdf::BM - 1) / fwdf::BM;
  const long long grid = (long long)nqb * a.H * a.B * a.n_chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return fwd_f32_d<64>(a, s);
    case 80: return fwd_f32_d<80>(a, s);
    case 128: return fwd_f32_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace exattn

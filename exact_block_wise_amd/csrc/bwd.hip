// Backward kernels: gradients from the saved log-sum-exp, weights recomputed
// block by block (never stored), following the closed-form derivative of
// O = softmax(scale Q K^T) V:
//   P = exp(scale Q K^T - LSE), dV = P^T dO, dP = dO V^T,
//   D_i = dO_i . O_i, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
// Recomputing P from one statistic per row is the memory-for-compute trade
// of "Training a Large Video Model on a Single Machine in a Day", section
// 4.1, and the activation recomputation of the LV-XAttn abstract.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace exattn {

// --------------------------------------------------------------------------
// Preprocess: D_i = sum_c dO_ic O_ic in fp32, one 16-lane group per row;
// optionally clears the row of the fp32 dQ accumulator.
// --------------------------------------------------------------------------
template <typename T, typename TO>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, int d) {
  const int gi = threadIdx.x >> 4, li = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + gi;  // over B*H*Nq
  const int64_t nrows = (int64_t)a.B * a.H * a.Nq;
  if (row >= nrows) return;  // whole 16-lane groups leave together
  const int i = (int)(row % a.Nq);
  const int64_t bh = row / a.Nq;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const T* dop = (const T*)a.dout + b * a.dos.sb + h * a.dos.sh + (int64_t)i * a.dos.sn;
  const TO* op = (const TO*)a.o + b * a.os.sb + h * a.os.sh + (int64_t)i * a.os.sn;
  float acc = 0.f;
  for (int c = li; c < d; c += 16) acc = fmaf(io<T>::ld(dop + c), io<TO>::ld(op + c), acc);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (li == 0) a.dsum[row] = acc;
  if (a.zero_dq_acc) {
    float* dqr = a.dq_acc + b * a.dqa.sb + h * a.dqa.sh + (int64_t)i * a.dqa.sn;
    for (int c = li; c < d; c += 16) dqr[c] = 0.f;
  }
}

// --------------------------------------------------------------------------
// bf16 main kernel, key/value-outer.
//
// Workgroup: 4 waves own 128 key rows (32 each); K and V of those rows stay
// in registers as matrix-core operands for the whole query loop, and the
// fp32 dK, dV accumulators stay in registers too.  The query loop walks
// 64-row tiles of Q, dO (staged in LDS both row-major and transposed), LSE
// and D.  Per tile and wave:
//   S = Q K^T, dP = dO V^T       (lane owns one key column, 16 query rows)
//   P, dS elementwise            (fp32)
//   dV += P^T dO, dK += dS^T Q   (accumulator entries reused as operands)
// then dS goes to LDS and the 4 waves compute this tile's dQ = dS K over all
// 128 keys, added to the fp32 accumulator with atomics.
// --------------------------------------------------------------------------
namespace bwdk {
constexpr int BN = 128;
constexpr int BM = 64;
constexpr int NT = 256;
}  // namespace bwdk

template <int D>
struct BwdLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int RS = D + 8;               // row-major tiles
  static constexpr int TS = bwdk::BM + 4;        // transposed Q / dO tiles
  static constexpr int KTS = bwdk::BN + 8;       // transposed K
  static constexpr int SS = bwdk::BN + 8;        // dS [q][key]
  static constexpr int q_off = 0;
  static constexpr int do_off = q_off + bwdk::BM * RS;
  static constexpr int qt_off = do_off + bwdk::BM * RS;
  static constexpr int dot_off = qt_off + DP * TS;
  static constexpr int kt_off = dot_off + DP * TS;
  static constexpr int ds_off = kt_off + DP * KTS;
  static constexpr int n_bf16 = ds_off + bwdk::BM * SS;
  static constexpr int bytes = n_bf16 * 2 + 2 * bwdk::BM * 4;
};

template <int D>
__global__ __launch_bounds__(bwdk::NT) void bwd_bf16_kernel(BwdArgs a) {
  using namespace bwdk;
  using L = BwdLds<D>;
  constexpr int DP = L::DP;
  constexpr int NDB = DP / 32;
  constexpr int KC = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* const lds = reinterpret_cast<bf16*>(smem);
  bf16* const Qs = lds + L::q_off;
  bf16* const dOs = lds + L::do_off;
  bf16* const Qt = lds + L::qt_off;
  bf16* const dOt = lds + L::dot_off;
  bf16* const Kt = lds + L::kt_off;
  bf16* const dSs = lds + L::ds_off;
  float* const lse2s = reinterpret_cast<float*>(lds + L::n_bf16);
  float* const Ds = lse2s + BM;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ln = lane & 31, g = lane >> 5;

  const int nkb = (a.Nkv + BN - 1) / BN;
  int idx = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = idx % nkb;
  idx /= nkb;
  const int h = idx % a.H;
  const int b = idx / a.H;

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh;
  const bf16* dop = (const bf16*)a.dout + b * a.dos.sb + h * a.dos.sh;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh;
  const float* lsep = a.lse + ((int64_t)b * a.H + h) * a.Nq;
  const float* dsp = a.dsum + ((int64_t)b * a.H + h) * a.Nq;
  float* dqp = a.dq_acc + b * a.dqa.sb + h * a.dqa.sh;

  const int k0 = kb * BN;             // first key row of the workgroup
  const int kw = k0 + 32 * w;         // first key row of this wave
  const bool wave_active = kw < a.Nkv;
  const int krow = kw + ln;
  const bool kvalid = krow < a.Nkv;
  const bf16x8 zero8 = {};

  // this wave's K and V rows as B operands (lane: key krow, d 16kc+8g..+7)
  bf16x8 kreg[KC], vreg[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    kreg[kc] = kvalid ? load_bf16x8(kp + (int64_t)krow * a.ks.sn + 16 * kc + 8 * g) : zero8;
    vreg[kc] = kvalid ? load_bf16x8(vp + (int64_t)krow * a.vs.sn + 16 * kc + 8 * g) : zero8;
  }
  // K^T of the workgroup's 128 keys for the dQ product; padding rows zero
  for (int e = tid; e < BN * (D / 8); e += NT) {
    const int r = e % BN, cc = e / BN;
    bf16x8 val = zero8;
    if (k0 + r < a.Nkv) val = load_bf16x8(kp + (int64_t)(k0 + r) * a.ks.sn + 8 * cc);
#pragma unroll
    for (int i = 0; i < 8; ++i) Kt[(8 * cc + i) * L::KTS + r] = val[i];
  }
  if constexpr (DP != D) {
    for (int i = tid; i < (DP - D) * L::KTS; i += NT) Kt[D * L::KTS + i] = (bf16)0.f;
    for (int i = tid; i < (DP - D) * L::TS; i += NT) {
      Qt[D * L::TS + i] = (bf16)0.f;
      dOt[D * L::TS + i] = (bf16)0.f;
    }
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const float sl2 = a.scale * kLog2e;

  for (int q0 = 0; q0 < a.Nq; q0 += BM) {
    __syncthreads();
    // Q and dO tiles: row-major (consecutive threads along a row) ...
    for (int e = tid; e < BM * (D / 8); e += NT) {
      const int r = e / (D / 8), cc = e % (D / 8);
      bf16x8 qv = zero8, dv8 = zero8;
      if (q0 + r < a.Nq) {
        qv = load_bf16x8(qp + (int64_t)(q0 + r) * a.qs.sn + 8 * cc);
        dv8 = load_bf16x8(dop + (int64_t)(q0 + r) * a.dos.sn + 8 * cc);
      }
      *reinterpret_cast<bf16x8*>(&Qs[r * L::RS + 8 * cc]) = qv;
      *reinterpret_cast<bf16x8*>(&dOs[r * L::RS + 8 * cc]) = dv8;
    }
    // ... and transposed (consecutive threads along a column)
    for (int e = tid; e < BM * (D / 8); e += NT) {
      const int r = e % BM, cc = e / BM;
      bf16x8 qv = zero8, dv8 = zero8;
      if (q0 + r < a.Nq) {
        qv = load_bf16x8(qp + (int64_t)(q0 + r) * a.qs.sn + 8 * cc);
        dv8 = load_bf16x8(dop + (int64_t)(q0 + r) * a.dos.sn + 8 * cc);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Qt[(8 * cc + i) * L::TS + r] = qv[i];
        dOt[(8 * cc + i) * L::TS + r] = dv8[i];
      }
    }
    if (tid < BM) {
      const bool ok = q0 + tid < a.Nq;
      // rows past Nq get P = exp2(-inf) = 0
      lse2s[tid] = ok ? lsep[q0 + tid] * kLog2e : INFINITY;
      Ds[tid] = ok ? dsp[q0 + tid] : 0.f;
    }
    __syncthreads();

    if (wave_active) {
#pragma unroll
      for (int nb = 0; nb < BM / 32; ++nb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const bf16x8 qa = load_bf16x8(&Qs[(32 * nb + ln) * L::RS + 16 * kc + 8 * g]);
          const bf16x8 da = load_bf16x8(&dOs[(32 * nb + ln) * L::RS + 16 * kc + 8 * g]);
          s = mfma32(qa, kreg[kc], s);
          dp = mfma32(da, vreg[kc], dp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qi = 32 * nb + 8 * i + 4 * g;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[qi]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[qi]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = kvalid ? fast_exp2(s[4 * i + r] * sl2 - l4[r]) : 0.f;
            s[4 * i + r] = p;
            dp[4 * i + r] = p * (dp[4 * i + r] - d4[r]);
          }
        }
        // dV += P^T dO, dK += dS^T Q over two 16-query chunks
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int t = 2 * nb + hh;
          const bf16x8 pa = acc_half_to_bf16(s, hh);
          const bf16x8 sa = acc_half_to_bf16(dp, hh);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16* dr = &dOt[(32 * db + ln) * L::TS + 16 * t + 4 * g];
            const bf16* qr = &Qt[(32 * db + ln) * L::TS + 16 * t + 4 * g];
            const bf16x8 db8 = cat4(*reinterpret_cast<const bf16x4*>(dr),
                                    *reinterpret_cast<const bf16x4*>(dr + 8));
            const bf16x8 qb8 = cat4(*reinterpret_cast<const bf16x4*>(qr),
                                    *reinterpret_cast<const bf16x4*>(qr + 8));
            dv[db] = mfma32(pa, db8, dv[db]);
            dk[db] = mfma32(sa, qb8, dk[db]);
          }
        }
        // dS to LDS as [query][key] for the dQ product
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qi = 32 * nb + 8 * (e >> 2) + 4 * g + (e & 3);
          dSs[qi * L::SS + 32 * w + ln] = (bf16)dp[e];
        }
      }
    } else {
      // keys past Nkv: this wave's share of dS is zero
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int qi = 8 * (e >> 2) + 4 * g + (e & 3);
        dSs[qi * L::SS + 32 * w + ln] = (bf16)0.f;
      }
    }
    __syncthreads();

    // dQ tile (BM x D) = dS (BM x 128) K (128 x D), split over the waves in
    // 32x32 blocks; atomically added to the fp32 accumulator.
    for (int blk = w; blk < (BM / 32) * NDB; blk += 4) {
      const int qbk = blk / NDB, db = blk % NDB;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int t = 0; t < BN / 16; ++t) {
        const bf16x8 sa = load_bf16x8(&dSs[(32 * qbk + ln) * L::SS + 16 * t + 8 * g]);
        const bf16x8 kb8 = load_bf16x8(&Kt[(32 * db + ln) * L::KTS + 16 * t + 8 * g]);
        acc = mfma32(sa, kb8, acc);
      }
      const int dcol = 32 * db + ln;
      if (dcol < D) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qi = q0 + 32 * qbk + 8 * (e >> 2) + 4 * g + (e & 3);
          if (qi < a.Nq)
            __hip_atomic_fetch_add(dqp + (int64_t)qi * a.dqa.sn + dcol, acc[e] * a.scale,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  if (!wave_active) return;
  // dK (scaled) and dV: lane owns column d = 32db + ln, key rows 8i+4g+r
  bf16* dkp = (bf16*)a.dk + b * a.dks.sb + h * a.dks.sh;
  bf16* dvp = (bf16*)a.dv + b * a.dvs.sb + h * a.dvs.sh;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dcol = 32 * db + ln;
    if (dcol >= D) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = kw + 8 * (e >> 2) + 4 * g + (e & 3);
      if (kr < a.Nkv) {
        dkp[(int64_t)kr * a.dks.sn + dcol] = (bf16)(dk[db][e] * a.scale);
        dvp[(int64_t)kr * a.dvs.sn + dcol] = (bf16)dv[db][e];
      }
    }
  }
}

// dQ accumulator (fp32) -> dQ (bf16), one thread per 4 elements
__global__ __launch_bounds__(256) void dq_finalize_kernel(BwdArgs a, int d) {
  const int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int dq4 = d / 4;
  const int64_t n4 = (int64_t)a.B * a.H * a.Nq * dq4;
  if (e4 >= n4) return;
  const int c = (int)(e4 % dq4) * 4;
  const int64_t row = e4 / dq4;
  const int i = (int)(row % a.Nq);
  const int64_t bh = row / a.Nq;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const f32x4 v = *reinterpret_cast<const f32x4*>(a.dq_acc + b * a.dqa.sb + h * a.dqa.sh +
                                                  (int64_t)i * a.dqa.sn + c);
  bf16x4 o4 = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>((bf16*)a.dq + b * a.dqs.sb + h * a.dqs.sh + (int64_t)i * a.dqs.sn +
                             c) = o4;
}

// --------------------------------------------------------------------------
// fp32 inputs: genuine fp32 arithmetic, exact library exp.  Not tuned.
//  - dK, dV: one lane per key row (its K, V rows in padded LDS, its dK, dV
//    accumulators in registers), query tiles of 16 rows read by broadcast.
//  - dQ: one lane per query row (its Q, dO rows in padded LDS, dQ in
//    registers), key tiles of 16 rows read by broadcast.
// --------------------------------------------------------------------------
namespace bwdf {
constexpr int RB = 32;  // rows owned per workgroup (one per lane)
constexpr int TB = 16;  // streamed tile rows
}  // namespace bwdf

template <int D>
__global__ __launch_bounds__(bwdf::RB) void bwd_f32_dkdv_kernel(BwdArgs a) {
  using namespace bwdf;
  __shared__ float Kown[RB][D + 1], Vown[RB][D + 1];
  __shared__ float Qt[TB][D], dOt[TB][D];
  __shared__ float lse_t[TB], D_t[TB];
  const int tid = threadIdx.x;
  const int nkb = (a.Nkv + RB - 1) / RB;
  const int kb = blockIdx.x % nkb;
  const int bh = blockIdx.x / nkb;
  const int h = bh % a.H, b = bh / a.H;
  const float* qp = (const float*)a.q + b * a.qs.sb + h * a.qs.sh;
  const float* dop = (const float*)a.dout + b * a.dos.sb + h * a.dos.sh;
  const float* kp = (const float*)a.k + b * a.ks.sb + h * a.ks.sh;
  const float* vp = (const float*)a.v + b * a.vs.sb + h * a.vs.sh;
  const float* lsep = a.lse + ((int64_t)b * a.H + h) * a.Nq;
  const float* dsp = a.dsum + ((int64_t)b * a.H + h) * a.Nq;
  const int k0 = kb * RB;
  for (int e = tid; e < RB * D; e += RB) {
    const int r = e / D, cc = e % D;
    const bool ok = k0 + r < a.Nkv;
    Kown[r][cc] = ok ? kp[(int64_t)(k0 + r) * a.ks.sn + cc] : 0.f;
    Vown[r][cc] = ok ? vp[(int64_t)(k0 + r) * a.vs.sn + cc] : 0.f;
  }
  float dk[D], dv[D];
#pragma unroll
  for (int i = 0; i < D; ++i) dk[i] = dv[i] = 0.f;
  for (int q0 = 0; q0 < a.Nq; q0 += TB) {
    __syncthreads();
    for (int e = tid; e < TB * D; e += RB) {
      const int r = e / D, cc = e % D;
      const bool ok = q0 + r < a.Nq;
      Qt[r][cc] = ok ? qp[(int64_t)(q0 + r) * a.qs.sn + cc] : 0.f;
      dOt[r][cc] = ok ? dop[(int64_t)(q0 + r) * a.dos.sn + cc] : 0.f;
    }
    if (tid < TB) {
      const bool ok = q0 + tid < a.Nq;
      lse_t[tid] = ok ? lsep[q0 + tid] : INFINITY;
      D_t[tid] = ok ? dsp[q0 + tid] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < TB; ++j) {
      float s = 0.f, dpv = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s = fmaf(Qt[j][i], Kown[tid][i], s);
        dpv = fmaf(dOt[j][i], Vown[tid][i], dpv);
      }
      const float p = expf(s * a.scale - lse_t[j]);
      const float ds = p * (dpv - D_t[j]);
#pragma unroll
      for (int i = 0; i < D; ++i) {
        dv[i] = fmaf(p, dOt[j][i], dv[i]);
        dk[i] = fmaf(ds, Qt[j][i], dk[i]);
      }
    }
  }
  const int kr = k0 + tid;
  if (kr >= a.Nkv) return;
  float* dkp = (float*)a.dk + b * a.dks.sb + h * a.dks.sh + (int64_t)kr * a.dks.sn;
  float* dvp = (float*)a.dv + b * a.dvs.sb + h * a.dvs.sh + (int64_t)kr * a.dvs.sn;
  for (int i = 0; i < D; ++i) {
    dkp[i] = dk[i] * a.scale;
    dvp[i] = dv[i];
  }
}

template <int D>
__global__ __launch_bounds__(bwdf::RB) void bwd_f32_dq_kernel(BwdArgs a, int accumulate) {
  using namespace bwdf;
  __shared__ float Qown[RB][D + 1], dOown[RB][D + 1];
  __shared__ float Kt[TB][D], Vt[TB][D];
  const int tid = threadIdx.x;
  const int nqb = (a.Nq + RB - 1) / RB;
  const int qb = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;
  const int h = bh % a.H, b = bh / a.H;
  const float* qp = (const float*)a.q + b * a.qs.sb + h * a.qs.sh;
  const float* dop = (const float*)a.dout + b * a.dos.sb + h * a.dos.sh;
  const float* kp = (const float*)a.k + b * a.ks.sb + h * a.ks.sh;
  const float* vp = (const float*)a.v + b * a.vs.sb + h * a.vs.sh;
  const int q0 = qb * RB;
  for (int e = tid; e < RB * D; e += RB) {
    const int r = e / D, cc = e % D;
    const bool ok = q0 + r < a.Nq;
    Qown[r][cc] = ok ? qp[(int64_t)(q0 + r) * a.qs.sn + cc] : 0.f;
    dOown[r][cc] = ok ? dop[(int64_t)(q0 + r) * a.dos.sn + cc] : 0.f;
  }
  const int qi = q0 + tid;
  const bool qvalid = qi < a.Nq;
  const float lse_i = qvalid ? a.lse[((int64_t)b * a.H + h) * a.Nq + qi] : INFINITY;
  const float D_i = qvalid ? a.dsum[((int64_t)b * a.H + h) * a.Nq + qi] : 0.f;
  float dq[D];
#pragma unroll
  for (int i = 0; i < D; ++i) dq[i] = 0.f;
  for (int j0 = 0; j0 < a.Nkv; j0 += TB) {
    __syncthreads();
    for (int e = tid; e < TB * D; e += RB) {
      const int r = e / D, cc = e % D;
      const bool ok = j0 + r < a.Nkv;
      Kt[r][cc] = ok ? kp[(int64_t)(j0 + r) * a.ks.sn + cc] : 0.f;
      Vt[r][cc] = ok ? vp[(int64_t)(j0 + r) * a.vs.sn + cc] : 0.f;
    }
    __syncthreads();
    const int nj = min(TB, a.Nkv - j0);
    for (int j = 0; j < nj; ++j) {
      float s = 0.f, dpv = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s = fmaf(Qown[tid][i], Kt[j][i], s);
        dpv = fmaf(dOown[tid][i], Vt[j][i], dpv);
      }
      const float p = expf(s * a.scale - lse_i);
      const float ds = p * (dpv - D_i);
#pragma unroll
      for (int i = 0; i < D; ++i) dq[i] = fmaf(ds, Kt[j][i], dq[i]);
    }
  }
  if (!qvalid) return;
  float* dqp = (float*)a.dq + b * a.dqs.sb + h * a.dqs.sh + (int64_t)qi * a.dqs.sn;
  for (int i = 0; i < D; ++i) {
    const float v = dq[i] * a.scale;
    dqp[i] = accumulate ? dqp[i] + v : v;
  }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
static hipError_t launch_pre(const BwdArgs& a, int d, int is_bf16, hipStream_t s) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  const long long grid = (rows + 15) / 16;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (is_bf16) {
    if (a.o_f32)
      hipLaunchKernelGGL((bwd_pre_kernel<bf16, float>), dim3((unsigned)grid), dim3(256), 0, s, a, d);
    else
      hipLaunchKernelGGL((bwd_pre_kernel<bf16, bf16>), dim3((unsigned)grid), dim3(256), 0, s, a, d);
  } else {
    hipLaunchKernelGGL((bwd_pre_kernel<float, float>), dim3((unsigned)grid), dim3(256), 0, s, a, d);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t bwd_bf16_d(const BwdArgs& a, int finalize_dq, hipStream_t s) {
  hipError_t e = launch_pre(a, D, 1, s);
  if (e != hipSuccess) return e;
  const int nkb = (a.Nkv + bwdk::BN - 1) / bwdk::BN;
  const long long grid = (long long)nkb * a.H * a.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int lds = BwdLds<D>::bytes;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwd_bf16_kernel<D>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((bwd_bf16_kernel<D>), dim3((unsigned)grid), dim3(bwdk::NT), lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || !finalize_dq) return e;
  const long long n4 = (long long)a.B * a.H * a.Nq * (D / 4);
  hipLaunchKernelGGL(dq_finalize_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a, D);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, int finalize_dq, hipStream_t s) {
  switch (d) {
    case 64: return bwd_bf16_d<64>(a, finalize_dq, s);
    case 80: return bwd_bf16_d<80>(a, finalize_dq, s);
    case 128: return bwd_bf16_d<128>(a, finalize_dq, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t bwd_f32_d(const BwdArgs& a, int accumulate, hipStream_t s) {
  hipError_t e = launch_pre(a, D, 0, s);
  if (e != hipSuccess) return e;
  const long long gk = (long long)((a.Nkv + bwdf::RB - 1) / bwdf::RB) * a.H * a.B;
  const long long gq = (long long)((a.Nq + bwdf::RB - 1) / bwdf::RB) * a.H * a.B;
  if (gk > 0x7fffffffLL || gq > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D>), dim3((unsigned)gk), dim3(bwdf::RB), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_f32_dq_kernel<D>), dim3((unsigned)gq), dim3(bwdf::RB), 0, s, a, accumulate);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const BwdArgs& a, int d, int accumulate, hipStream_t s) {
  switch (d) {
    case 64: return bwd_f32_d<64>(a, accumulate, s);
    case 80: return bwd_f32_d<80>(a, accumulate, s);
    case 128: return bwd_f32_d<128>(a, accumulate, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace exattn

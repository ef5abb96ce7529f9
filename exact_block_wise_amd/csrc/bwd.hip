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

#include <algorithm>
#include <type_traits>

#include <math.h>


// pin the dK/dV accumulators of one-wave-per-SIMD instances in AGPRs
#ifndef EXATTN_PIN_ACC
#define EXATTN_PIN_ACC 1
#endif

namespace exattn {

// --------------------------------------------------------------------------
// Preprocess: D_i = sum_c dO_ic O_ic in fp32, one 16-lane group per row.
// (D_i also equals sum_j P_ij dP_ij, the row term of the softmax Jacobian.)
// --------------------------------------------------------------------------
// fp32 dO (and O): one 16-lane group per row.
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
}

// bf16 dO: D in exactly the order the dQ kernel forms it when it computes D
// itself (two half-rows d = 16kc + 8g + j, each an fma chain in (kc, j)
// order, then their sum), so that both routes give the same bits.  Two
// threads per row.
template <typename TO>
__global__ __launch_bounds__(256) void bwd_pre_bf16_kernel(BwdArgs a, int d) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t >> 1;  // over B*H*Nq
  const int g = (int)(t & 1);
  const int64_t nrows = (int64_t)a.B * a.H * a.Nq;
  if (row >= nrows) return;  // both threads of a row leave together
  const int i = (int)(row % a.Nq);
  const int64_t bh = row / a.Nq;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const bf16* dop = (const bf16*)a.dout + b * a.dos.sb + h * a.dos.sh + (int64_t)i * a.dos.sn;
  const TO* op = (const TO*)a.o + b * a.os.sb + h * a.os.sh + (int64_t)i * a.os.sn;
  float acc = 0.f;
  for (int kc = 0; kc < d / 16; ++kc) {
    const int c = 16 * kc + 8 * g;
    const bf16x8 dv8 = load_bf16x8(dop + c);
    float o8[8];
    if constexpr (sizeof(TO) == 4) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(op + c);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(op + c + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o8[j] = lo[j];
        o8[4 + j] = hi[j];
      }
    } else {
      const bf16x8 v = load_bf16x8(reinterpret_cast<const bf16*>(op) + c);
#pragma unroll
      for (int j = 0; j < 8; ++j) o8[j] = (float)v[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf((float)dv8[j], o8[j], acc);
  }
  const float total = acc + __shfl_xor(acc, 1);
  if (g == 0) a.dsum[row] = total;
}

// --------------------------------------------------------------------------
// bf16 dK / dV kernel, key/value-outer.
//
// Workgroup: 4 waves, each owning KW key rows (KW = 32 or 64).  K and V of a
// wave's rows stay in registers as matrix-core operands for the whole query
// loop, and so do the fp32 dK, dV accumulators.  The query loop walks 64-row
// tiles of Q and dO, staged row-major in LDS and double-buffered (the next
// tile's global loads are in flight while the current one is used).  Per
// tile and 32-row query block:
//   S = Q K^T, dP = dO V^T       (lane owns one key column, 16 query rows)
//   P = exp(S - LSE), dS = P (dP - D)           (fp32, registers)
//   dV += P^T dO, dK += dS^T Q   (accumulators reused as A operands; dO and
//                                 Q columns read with LDS transpose reads)
// Query rows past Nq arrive as zeros with LSE = +inf (P = 0); key rows past
// Nkv are zero and their gradients are never stored.
// --------------------------------------------------------------------------
// query rows per staged tile of the dK/dV kernel
#ifndef EXATTN_DKDV_BM
#define EXATTN_DKDV_BM 64
#endif
namespace bwdk {
constexpr int BM = EXATTN_DKDV_BM;
constexpr int NT = 256;
}  // namespace bwdk

template <int D>
struct DkdvLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int RS = tile_stride(DP);                  // row stride of Q, dO tiles
  static constexpr int tile = bwdk::BM * RS;
  static constexpr int n_bf16 = 4 * tile;                    // Q, dO x double buffer
  static constexpr int bytes = n_bf16 * 2 + 2 * 2 * bwdk::BM * 4;  // + (LSE, D) x 2
};

// One 32-query block against a wave's NCB x 32 keys: S = Q K^T and
// E = D - dP (queries as A operands, the wave's K rows and NEGATED V rows as
// B operands, the matrix-core chain of E starting from D instead of zero),
// P = exp2(S log2e scale - LSE2), -dS = P E, then dV += P^T dO and
// (-dK) += (-dS)^T Q with the accumulator halves as A operands and the dO / Q
// columns from LDS transpose reads.  Folding D into the accumulator and the
// sign into V leaves one multiply per score for dS.  Qs / dOs: row-major bf16
// query rows (row stride rs), lse2s / Ds: their LSE in log2 units and D.
template <int D, int NCB, bool PIN, bool FIRST = false>
__device__ __forceinline__ void dkdv_qblock(const bf16* Qs, const bf16* dOs, int rs,
                                            const float* lse2s, const float* Ds, int nb,
                                            float sl2, const bf16x8 (&kreg)[NCB][D / 16],
                                            const bf16x8 (&vneg)[NCB][D / 16],
                                            f32x16 (&dk)[NCB][(D + 31) / 32],
                                            f32x16 (&dv)[NCB][(D + 31) / 32], int lane) {
  constexpr int KC = D / 16, NDB = (D + 31) / 32;
  const int ln = lane & 31, g = lane >> 5;
  // D of the accumulator rows: entry 4i + r is query 32nb + 8i + 4g + r
  f32x16 dinit;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[32 * nb + 8 * i + 4 * g]);
#pragma unroll
    for (int r = 0; r < 4; ++r) dinit[4 * i + r] = d4[r];
  }
  f32x16 s[NCB], e[NCB];
  // The Q / dO row operands of all KC d-chunks are read at once, except at
  // d = 128 with one key block per wave (the one-wave-per-SIMD kernels), where
  // 16 of them would crowd the vector registers: there they come in two
  // fenced halves over d.
  constexpr int PARTS = (NCB == 1 && KC == 8) ? 2 : 1;
  constexpr int KP = KC / PARTS;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    s[cb] = f32x16{};
    e[cb] = dinit;
  }
  prio_mfma();
#pragma unroll
  for (int part = 0; part < PARTS; ++part) {
    bf16x8 qa[KP], da[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int kc = part * KP + j;
      qa[j] = load_bf16x8(&Qs[(32 * nb + ln) * rs + 16 * kc + 8 * g]);
      da[j] = load_bf16x8(&dOs[(32 * nb + ln) * rs + 16 * kc + 8 * g]);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const int kc = part * KP + j;
        s[cb] = mfma32(qa[j], kreg[cb][kc], s[cb]);
        e[cb] = mfma32(da[j], vneg[cb][kc], e[cb]);
      }
    if constexpr (PARTS > 1) __builtin_amdgcn_sched_barrier(0);
  }
  prio_valu();
  // d = 128, one key block per wave: the transposed dO / Q operands of both
  // query halves are read here, ahead of the exponentials, so that the
  // VALU work covers their latency (elsewhere they are read just before
  // each product, and other waves cover it).  The LSE rows come first:
  // LDS reads complete in order, and the exponentials wait only for them.
  constexpr bool EARLY = PARTS > 1;
  f32x4 l4s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) l4s[i] = *reinterpret_cast<const f32x4*>(&lse2s[32 * nb + 8 * i + 4 * g]);
  bf16x8 dob_e[EARLY ? 2 : 1][EARLY ? NDB : 1], qbv_e[EARLY ? 2 : 1][EARLY ? NDB : 1];
  if constexpr (EARLY) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int t = 2 * nb + hh;
        dob_e[hh][db] = tr_operand(dOs + 32 * db, rs, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
        qbv_e[hh][db] = tr_operand(Qs + 32 * db, rs, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 l4 = l4s[i];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(s[cb][4 * i + r], sl2, -l4[r]));
        s[cb][4 * i + r] = p;
        e[cb][4 * i + r] *= p;
      }
  }
  // dV^T += dO^T P, (-dK)^T += Q^T (-dS) over two 16-query chunks t = 2 nb +
  // hh: slot group g holds queries 16t + 4g + (0..3) and 16t + 8 + 4g +
  // (0..3).  The dO / Q columns (LDS transpose reads) are the A operands and
  // the accumulator halves of P and -dS the B operands, so the gradients come
  // out transposed: a lane owns one key and runs of 4 consecutive d, which
  // leave in 8-byte stores.
  prio_mfma();
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int t = 2 * nb + hh;
    bf16x8 pa[NCB], sa[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      pa[cb] = acc_half_to_bf16(s[cb], hh);
      sa[cb] = acc_half_to_bf16(e[cb], hh);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x8 dob, qbv;
      if constexpr (EARLY) {
        dob = dob_e[hh][db];
        qbv = qbv_e[hh][db];
      } else {
        dob = tr_operand(dOs + 32 * db, rs, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
        qbv = tr_operand(Qs + 32 * db, rs, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        // FIRST: the block's first products start the accumulators from zero
        if constexpr (PIN && FIRST) {
          if (hh == 0) {
            mfma32_agpr_zero(dob, pa[cb], dv[cb][db]);
            mfma32_agpr_zero(qbv, sa[cb], dk[cb][db]);
          } else {
            mfma32_agpr(dob, pa[cb], dv[cb][db]);
            mfma32_agpr(qbv, sa[cb], dk[cb][db]);
          }
        } else if constexpr (PIN) {
          mfma32_agpr(dob, pa[cb], dv[cb][db]);
          mfma32_agpr(qbv, sa[cb], dk[cb][db]);
        } else if constexpr (FIRST) {
          dv[cb][db] = mfma32(dob, pa[cb], hh == 0 ? f32x16{} : dv[cb][db]);
          dk[cb][db] = mfma32(qbv, sa[cb], hh == 0 ? f32x16{} : dk[cb][db]);
        } else {
          dv[cb][db] = mfma32(dob, pa[cb], dv[cb][db]);
          dk[cb][db] = mfma32(qbv, sa[cb], dk[cb][db]);
        }
      }
    }
  }
  prio_valu();
}

// V rows as the negated B operands dkdv_qblock takes (sign bits flipped)
template <int NCB, int KC>
__device__ __forceinline__ void negate_rows(bf16x8 (&v)[NCB][KC]) {
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 u = __builtin_bit_cast(u32x4, v[cb][kc]);
      u ^= 0x80008000u;
      v[cb][kc] = __builtin_bit_cast(bf16x8, u);
    }
}

// dK and dV of a wave's keys kw .. kw + 32 NCB - 1 from the transposed
// accumulators (dk holds -dK / scale, see dkdv_qblock).  A lane owns key
// kw + 32cb + ln and, per 32-column block db, the runs d = 32db + 8i + 4g +
// (0..3) (accumulator entries 4i .. 4i+3); the runs go through this wave's
// LDS staging rows (`stage`, 32 NCB rows of stride DP + 8) and leave as
// whole rows (store_staged_rows).
template <int D, int NCB, bool NT = (EXATTN_NT_OUT != 0)>
__device__ __forceinline__ void dkdv_store(const BwdArgs& a, int b, int h, const SeqSpan& sp,
                                           int kw, const f32x16 (&dk)[NCB][(D + 31) / 32],
                                           const f32x16 (&dv)[NCB][(D + 31) / 32], bf16* stage,
                                           int lane) {
  constexpr int NDB = (D + 31) / 32, SRS = NDB * 32 + 8;
  const int ln = lane & 31, g = lane >> 5;
#pragma unroll
  for (int t = 0; t < 2; ++t) {  // dK, then dV
    const f32x16 (&acc)[NCB][NDB] = t == 0 ? dk : dv;
    const float sc = t == 0 ? -a.scale : 1.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * db + 8 * i + 4 * g;
          if (d0 >= D) continue;
          const f32x16& x = acc[cb][db];
          const bf16x4 r4 = {(bf16)(x[4 * i] * sc), (bf16)(x[4 * i + 1] * sc),
                             (bf16)(x[4 * i + 2] * sc), (bf16)(x[4 * i + 3] * sc)};
          *reinterpret_cast<bf16x4*>(&stage[(32 * cb + ln) * SRS + d0]) = r4;
        }
    bf16* out = t == 0 ? (bf16*)a.dk + b * a.dks.sb + h * a.dks.sh +
                             (int64_t)(sp.kv_row0 + kw) * a.dks.sn
                       : (bf16*)a.dv + b * a.dvs.sb + h * a.dvs.sh +
                             (int64_t)(sp.kv_row0 + kw) * a.dvs.sn;
    const int64_t sn = t == 0 ? a.dks.sn : a.dvs.sn;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      store_staged_rows<bf16, D, SRS, NT>(stage + 32 * cb * SRS, out + (int64_t)32 * cb * sn, sn,
                                      sp.nkv - kw - 32 * cb, lane);
  }
}

template <int D, int KW>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a) {
  using namespace bwdk;
  using L = DkdvLds<D>;
  constexpr int DP = L::DP, NDB = DP / 32, KC = D / 16, RS = L::RS;
  constexpr int NCB = KW / 32;                 // 32-row key blocks per wave
  // pin dK/dV in AGPRs only in the one-wave-per-SIMD instances, where the
  // registers fit without spilling (see mfma32_agpr)
  constexpr bool kPinAcc = EXATTN_PIN_ACC && (KW == 64 || D > 80);
  constexpr int BN = 4 * KW;                   // key rows per workgroup
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* const lds = reinterpret_cast<bf16*>(smem);
  float* const stats = reinterpret_cast<float*>(lds + L::n_bf16);  // [2][LSE2 | D][BM]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31, g = lane >> 5;

  const int nkb = (a.Nkv + BN - 1) / BN;
  int idx = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = idx % nkb;
  idx /= nkb;
  const int h = idx % a.H;
  const int b = idx / a.H;
  const SeqSpan sp = seq_span(a, b, h);
  if (kb * BN >= sp.nkv) return;  // a packed sequence shorter than the longest

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh + (int64_t)sp.q_row0 * a.qs.sn;
  const bf16* dop =
      (const bf16*)a.dout + b * a.dos.sb + h * a.dos.sh + (int64_t)sp.q_row0 * a.dos.sn;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh + (int64_t)sp.kv_row0 * a.ks.sn;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh + (int64_t)sp.kv_row0 * a.vs.sn;
  const float* lsep = a.lse + sp.stat0;
  const float* dsp = a.dsum + sp.stat0;

  const int kw = kb * BN + KW * w;             // first key row of this wave
  const bool wave_active = kw < sp.nkv;

  // this wave's K and V rows as B operands (lane: key kw + 32cb + ln,
  // d = 16kc + 8g .. +7; rows past Nkv read as zeros)
  bf16x8 kreg[NCB][KC], vreg[NCB][KC];
  {
    const auto rk = rows_rsrc(kp + (int64_t)kw * a.ks.sn, sp.nkv - kw, 2 * a.ks.sn, 2 * D);
    const auto rv = rows_rsrc(vp + (int64_t)kw * a.vs.sn, sp.nkv - kw, 2 * a.vs.sn, 2 * D);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int col = 2 * (16 * kc + 8 * g);
        kreg[cb][kc] = buffer_load_bf16x8(rk, (uint32_t)((32 * cb + ln) * 2 * a.ks.sn + col));
        vreg[cb][kc] = buffer_load_bf16x8(rv, (uint32_t)((32 * cb + ln) * 2 * a.vs.sn + col));
      }
  }

  // Query tiles are staged with direct-to-LDS loads (no registers, no LDS
  // stores in the loop; see LdsTileDma), and so is D.  The LSE goes through
  // registers of the first BM / 64 waves, which convert it to log2 units once
  // per staged row (instead of once per score) when the tile lands.  Query
  // rows past Nq read as zero (Q = dO = 0, LSE = D = 0): their P is finite
  // and their dS and dO rows are zero, so they add nothing.
  constexpr int NSI = BM / 64;                 // 64-float pieces of LSE (and of D)
  static_assert(NSI >= 1 && 2 * NSI <= 4, "one statistics piece per wave");
  LdsTileDma<D, RS, BM> tq, td;
  tq.init(w, lane, a.qs.sn);
  td.init(w, lane, a.dos.sn);
  float lse_next = 0.f;
  auto load_tile = [&](int q0, int buf) {
    const int rows = sp.nq - q0;
    const auto rq = rows_rsrc(qp + (int64_t)q0 * a.qs.sn, rows, 2 * a.qs.sn, 2 * D);
    const auto rd = rows_rsrc(dop + (int64_t)q0 * a.dos.sn, rows, 2 * a.dos.sn, 2 * D);
    const uint32_t qbase = lds_address(lds + buf * 2 * L::tile);
    const uint32_t dbase = qbase + 2 * L::tile;
    tq.issue(rq, qbase, w);
    td.issue(rd, dbase, w);
    if (w < NSI) {
      lse_next = buffer_load_f32(rows_rsrc(lsep + q0, rows, 4, 4), 4 * (64 * w + lane));
    } else if (w < 2 * NSI) {
      const int part = w - NSI;
      buffer_load_lds4(rows_rsrc(dsp + q0, rows, 4, 4),
                       lds_address(stats + buf * 2 * BM + BM + 64 * part), 256 * part + 4 * lane);
    }
  };
  // after the tile's loads have landed (wait_vmem), before the barrier
  auto finish_tile = [&](int buf) {
    if (w < NSI) stats[buf * 2 * BM + 64 * w + lane] = lse_next * kLog2e;
  };

  f32x16 dk[NCB][NDB], dv[NCB][NDB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      dk[cb][i] = f32x16{};
      dv[cb][i] = f32x16{};
    }
  const float sl2 = a.scale * kLog2e;
  const int nqt = max(1, (sp.nq + BM - 1) / BM);  // (no query rows: one empty tile)

  // one query tile; NEXT: tile it + 1 exists and is staged into the other
  // buffer while this one is computed (waited for before the barrier)
  auto tile = [&](auto next_tag, int it) {
    constexpr bool NEXT = decltype(next_tag)::value;
    const int buf = it & 1;
    if (NEXT) load_tile((it + 1) * BM, buf ^ 1);
    if (wave_active) {
      const bf16* Qs = lds + buf * 2 * L::tile;
      const bf16* dOs = Qs + L::tile;
      const float* lse2s = stats + buf * 2 * BM;
      const float* Ds = lse2s + BM;
      // one 32-row query block at a time keeps the live registers of a block
      // (its S, E and operands) from being doubled by interleaving; blocks
      // wholly past Nq (in the last tile) are skipped
      const int nbs = min(BM / 32, (sp.nq - it * BM + 31) / 32);
#pragma unroll 1
      for (int nb = 0; nb < nbs; ++nb)
        dkdv_qblock<D, NCB, kPinAcc>(Qs, dOs, RS, lse2s, Ds, nb, sl2, kreg, vreg, dk, dv, lane);
    }
    wait_vmem();
    if (NEXT) finish_tile(buf ^ 1);
    __syncthreads();
  };
  load_tile(0, 0);
  wait_vmem();
  finish_tile(0);
  negate_rows(vreg);  // landed with the wait above
  __syncthreads();
  int it = 0;
  for (; it + 1 < nqt; ++it) tile(std::true_type{}, it);
  tile(std::false_type{}, it);

  if (!wave_active) return;
  if constexpr (kPinAcc) agpr_results_ready();
  // the query tiles are free after the last tile's barrier: they stage the
  // output rows (32 NCB rows of stride RS per wave)
  static_assert(4 * 32 * NCB <= 4 * BM, "staging fits the query tiles");
  dkdv_store<D, NCB>(a, b, h, sp, kw, dk, dv, lds + w * 32 * NCB * RS, lane);
}

// --------------------------------------------------------------------------
// bf16 dK / dV for a short query block against a long key range
// (Nq <= 128, e.g. a query block attending to a long video or image-token
// cache, as in the cross-attention setting of "LV-XAttn", section 3).
//
// The whole query side (Q, dO, LSE, D: at most 128 rows) is loaded into LDS
// once per workgroup and stays there.  The workgroup then walks its share of
// the head's 128-key blocks; each wave owns 32 keys of a block, holds their
// K / V rows in registers, and loads the rows of its next block while it
// computes the current one (so the key stream overlaps the matrix work):
// into registers at d = 64 and 80, into its own LDS rows by direct-to-LDS
// loads at d = 128, where the registers are needed for the accumulators.
// No barrier is needed inside the key loop: the query side is read-only and
// each wave's keys and LDS rows are its own.  dK and dV leave as each block
// completes.
// --------------------------------------------------------------------------
namespace resk {
constexpr int QR = 128;  // resident query rows
constexpr int NT = 256;
constexpr int KB = 128;  // keys per workgroup step (4 waves x 32)
}  // namespace resk

template <int D>
struct ResLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int RS = tile_stride(DP);                  // row stride of Q, dO
  static constexpr int stage = 32 * RS;                       // output rows per wave
  // d = 128: the next key block's K and V rows reach LDS by direct-to-LDS
  // loads instead of registers, which the accumulators need.  Each wave
  // owns a region holding its 32 K and 32 V rows (row stride KS, whole 1 KB
  // load instructions); its output staging reuses the region once the rows
  // have been read into registers.
  static constexpr bool kv_lds = D == 128;
  static constexpr int KS = DP + 16;
  static constexpr int region = kv_lds && 64 * KS > stage ? 64 * KS : stage;
  static constexpr int bytes = 2 * resk::QR * RS * 2 + 2 * resk::QR * 4 + 4 * region * 2;
};

#ifndef EXATTN_DKDV_RESIDENT
#define EXATTN_DKDV_RESIDENT 1
#endif

template <int D>
__global__ __launch_bounds__(resk::NT) void dkdv_resident_kernel(BwdArgs a, int groups) {
  using namespace resk;
  using L = ResLds<D>;
  constexpr int KC = D / 16, NDB = (D + 31) / 32, RS = L::RS;
  constexpr bool kPin = EXATTN_PIN_ACC && D > 80;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* const Qs = reinterpret_cast<bf16*>(smem);
  bf16* const dOs = Qs + QR * RS;
  float* const lse2s = reinterpret_cast<float*>(dOs + QR * RS);
  float* const Ds = lse2s + QR;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31, g = lane >> 5;
  bf16* const stage = reinterpret_cast<bf16*>(Ds + QR) + w * L::region;  // this wave's region

  int idx = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = idx % groups;
  idx /= groups;
  const int h = idx % a.H;
  const int b = idx / a.H;

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh;
  const bf16* dop = (const bf16*)a.dout + b * a.dos.sb + h * a.dos.sh;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh;
  const float* lsep = a.lse + ((int64_t)b * a.H + h) * a.Nq;
  const float* dsp = a.dsum + ((int64_t)b * a.H + h) * a.Nq;

  // the query side; rows past Nq are zero with LSE = +inf (P = 0)
  {
    constexpr int PT = QR * (D / 8) / NT;  // 16-byte pieces per thread and tensor
    const auto rq = rows_rsrc(qp, a.Nq, 2 * a.qs.sn, 2 * D);
    const auto rd = rows_rsrc(dop, a.Nq, 2 * a.dos.sn, 2 * D);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int e = tid + u * NT;
      const int r = e / (D / 8), cc = e % (D / 8);
      const bf16x8 vq = buffer_load_bf16x8(rq, (uint32_t)(r * 2 * a.qs.sn + 16 * cc));
      const bf16x8 vd = buffer_load_bf16x8(rd, (uint32_t)(r * 2 * a.dos.sn + 16 * cc));
      *reinterpret_cast<bf16x8*>(&Qs[r * RS + 8 * cc]) = vq;
      *reinterpret_cast<bf16x8*>(&dOs[r * RS + 8 * cc]) = vd;
    }
    const int r = tid & (QR - 1);
    const float l = buffer_load_f32(rows_rsrc(lsep, a.Nq, 4, 4), 4 * r);
    const float dd = buffer_load_f32(rows_rsrc(dsp, a.Nq, 4, 4), 4 * r);
    if (tid < QR)
      lse2s[r] = r < a.Nq ? l * kLog2e : INFINITY;
    else
      Ds[r] = dd;
  }
  __syncthreads();

  const int nkb = (a.Nkv + KB - 1) / KB;
  const int nqb = (a.Nq + 31) / 32;
  const float sl2 = a.scale * kLog2e;
  int kb = grp;
  if (kb >= nkb) return;  // the whole workgroup; no barrier follows

  // this wave's 32 keys of block kb_ as B operands (rows past Nkv: zero)
  auto load_kv = [&](int kb_, bf16x8 (&kr)[1][KC], bf16x8 (&vr)[1][KC]) {
    const int kw = kb_ * KB + 32 * w;
    const auto rk = rows_rsrc(kp + (int64_t)kw * a.ks.sn, a.Nkv - kw, 2 * a.ks.sn, 2 * D);
    const auto rv = rows_rsrc(vp + (int64_t)kw * a.vs.sn, a.Nkv - kw, 2 * a.vs.sn, 2 * D);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int col = 2 * (16 * kc + 8 * g);
      kr[0][kc] = buffer_load_bf16x8(rk, (uint32_t)(ln * 2 * a.ks.sn + col));
      vr[0][kc] = buffer_load_bf16x8(rv, (uint32_t)(ln * 2 * a.vs.sn + col));
    }
  };
  bf16x8 kreg[1][KC], vreg[1][KC], knext[1][KC], vnext[1][KC];
  f32x16 dk[1][NDB], dv[1][NDB];
  // K and V rows through LDS (L::kv_lds): piece p = 64 j + lane of load
  // instruction j is row p / KCPR, 16-byte column p % KCPR of the wave's
  // rows; lanes on a row's padding re-load its first piece
  constexpr int KCPR = L::KS / 8, KNI = 32 * KCPR / 64;
  static_assert(!L::kv_lds || (32 * KCPR) % 64 == 0, "whole instructions");
  bf16* const kbuf = stage;
  bf16* const vbuf = stage + 32 * L::KS;
  auto load_kv_lds = [&](int kb_) {
    const int kw = kb_ * KB + 32 * w;
    const auto rk = rows_rsrc(kp + (int64_t)kw * a.ks.sn, a.Nkv - kw, 2 * a.ks.sn, 2 * D);
    const auto rv = rows_rsrc(vp + (int64_t)kw * a.vs.sn, a.Nkv - kw, 2 * a.vs.sn, 2 * D);
    const uint32_t kl = lds_address(kbuf), vl = lds_address(vbuf);
#pragma unroll
    for (int j = 0; j < KNI; ++j) {
      const int pc = 64 * j + lane, r = pc / KCPR, ch = pc % KCPR;
      const uint32_t col = 16 * (ch < D / 8 ? ch : 0);
      buffer_load_lds16(rk, kl + 1024 * j, (uint32_t)(r * 2 * a.ks.sn) + col);
      buffer_load_lds16(rv, vl + 1024 * j, (uint32_t)(r * 2 * a.vs.sn) + col);
    }
  };
  auto read_kv_lds = [&] {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kreg[0][kc] = load_bf16x8(&kbuf[ln * L::KS + 16 * kc + 8 * g]);
      vreg[0][kc] = load_bf16x8(&vbuf[ln * L::KS + 16 * kc + 8 * g]);
    }
  };
  auto block = [&](int kb_, bool next) {
    negate_rows(vreg);
    // the first query block's products start dK and dV from zero (no
    // clearing of the accumulators per key block)
    dkdv_qblock<D, 1, kPin, true>(Qs, dOs, RS, lse2s, Ds, 0, sl2, kreg, vreg, dk, dv, lane);
#pragma unroll 1
    for (int nb = 1; nb < nqb; ++nb)
      dkdv_qblock<D, 1, kPin>(Qs, dOs, RS, lse2s, Ds, nb, sl2, kreg, vreg, dk, dv, lane);
    if constexpr (kPin) agpr_results_ready();
    // The next block's rows were requested a whole block ago: wait for them
    // here, before this block's stores.  Loads and stores share one counter
    // and the compiler treats a mix of both as unordered, so a wait for the
    // rows placed after the stores drains the stores as well, every block.
    wait_vmem();
    if constexpr (L::kv_lds) {
      if (next) {
        // the next rows into registers before the staging reuses their LDS
        read_kv_lds();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      }
    }
    dkdv_store<D, 1>(a, b, h, seq_span(a, b, h), kb_ * KB + 32 * w, dk, dv, stage, lane);
  };
  load_kv(kb, kreg, vreg);
  // Take the first rows here.  A load still pending on entry would make the
  // compiler wait at the top of every iteration for whatever was issued
  // before that iteration's prefetch (the previous block's stores, too).
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) asm volatile("" ::"v"(kreg[0][kc]), "v"(vreg[0][kc]));
  for (; kb + groups < nkb; kb += groups) {
    if constexpr (L::kv_lds) {
      // the staging reads of the previous block are done before the rows
      // land over them
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      load_kv_lds(kb + groups);
      block(kb, true);
    } else {
      load_kv(kb + groups, knext, vnext);
      block(kb, true);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        kreg[0][kc] = knext[0][kc];
        vreg[0][kc] = vnext[0][kc];
      }
    }
  }
  block(kb, false);
}

// --------------------------------------------------------------------------
// bf16 dQ kernel, query-outer.
//
// Same shape as the forward: 4 waves, each owning QW query rows; key/value
// tiles of 64 rows stream through LDS (row-major, double-buffered).  Per tile
// each wave recomputes the transposed tiles S^T = K Q^T and dP^T = V dO^T, so
// every lane owns one query row (its LSE and D are per-lane scalars), forms
// dS = P (dP - D), and accumulates dQ in registers from the accumulator
// halves of dS and the K columns (LDS transpose reads) as (dQ)^T = K^T dS^T,
// so a lane ends up holding its query row's runs of d (d = 80: dQ = dS K,
// see below).  Each dQ row belongs to one workgroup, so no atomics are
// needed and the result is bitwise reproducible.  Key rows past Nkv are zero
// in LDS and add nothing (their K rows multiply dS).
// --------------------------------------------------------------------------
namespace dqk {
constexpr int BN = 64;
constexpr int NT = 256;
}  // namespace dqk

template <int D>
struct DqLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int KS = tile_stride(DP);
  static constexpr int tile = dqk::BN * KS;
  static constexpr int bytes = 4 * tile * 2;   // K, V x double buffer
};

template <int D, int QW>
__device__ __forceinline__ void dq_body(const BwdArgs& a, int accumulate) {
  using namespace dqk;
  using L = DqLds<D>;
  constexpr int DP = L::DP, NDB = DP / 32, KC = D / 16, KS = L::KS;
  constexpr int NQB = QW / 32;
  constexpr int BM = 4 * QW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* const lds = reinterpret_cast<bf16*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31, g = lane >> 5;

  const int nqb = (a.Nq + BM - 1) / BM;
  int idx = xcd_remap(blockIdx.x, gridDim.x);
  const int qblk = idx % nqb;
  idx /= nqb;
  const int split = idx % a.dq_splits;   // key range [split * len, ...)
  idx /= a.dq_splits;
  const int h = idx % a.H;
  const int b = idx / a.H;
  const SeqSpan sp = seq_span(a, b, h);
  if (qblk * BM >= sp.nq) return;  // a packed sequence shorter than the longest
  const int kv_lo = split * a.dq_split_len;

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh + (int64_t)sp.q_row0 * a.qs.sn;
  const bf16* dop =
      (const bf16*)a.dout + b * a.dos.sb + h * a.dos.sh + (int64_t)sp.q_row0 * a.dos.sn;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh +
                   (int64_t)(sp.kv_row0 + kv_lo) * a.ks.sn;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh +
                   (int64_t)(sp.kv_row0 + kv_lo) * a.vs.sn;
  const float* lsep = a.lse + sp.stat0;
  const float* dsp = a.dsum + sp.stat0;

  const int q0 = qblk * BM + w * QW;
  const bool wave_active = q0 < sp.nq;

  const int n_kv = min(sp.nkv - kv_lo, a.dq_split_len);
  const int ntiles = (n_kv + BN - 1) / BN;
  // direct-to-LDS staging of the key/value tiles (see LdsTileDma); rows
  // past the end of the key range read as zeros
  LdsTileDma<D, KS, BN> tk, tv;
  tk.init(w, lane, a.ks.sn);
  tv.init(w, lane, a.vs.sn);
  auto load_tile = [&](int j0, int buf) {
    const auto rk = rows_rsrc(kp + (int64_t)j0 * a.ks.sn, n_kv - j0, 2 * a.ks.sn, 2 * D);
    const auto rv = rows_rsrc(vp + (int64_t)j0 * a.vs.sn, n_kv - j0, 2 * a.vs.sn, 2 * D);
    const uint32_t kbase = lds_address(lds + buf * 2 * L::tile);
    tk.issue(rk, kbase, w);
    tv.issue(rv, kbase + 2 * L::tile, w);
  };

  // this wave's Q and dO rows as B operands, with their LSE (log2 units) and
  // D; rows past Nq read as zeros with LSE = +inf
  bf16x8 qreg[NQB][KC], doreg[NQB][KC];
  float lse2[NQB], dsum[NQB];
  {
    const int rows = sp.nq - q0;
    const auto rq = rows_rsrc(qp + (int64_t)q0 * a.qs.sn, rows, 2 * a.qs.sn, 2 * D);
    const auto rd = rows_rsrc(dop + (int64_t)q0 * a.dos.sn, rows, 2 * a.dos.sn, 2 * D);
    const auto rl = rows_rsrc(lsep + q0, rows, 4, 4);
    const auto rs = rows_rsrc(dsp + q0, rows, 4, 4);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int r = 32 * qb + ln;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        doreg[qb][kc] = buffer_load_bf16x8(rd, (uint32_t)(r * 2 * a.dos.sn + 2 * (16 * kc + 8 * g)));
    }
    auto load_q = [&] {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int r = 32 * qb + ln;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          qreg[qb][kc] = buffer_load_bf16x8(rq, (uint32_t)(r * 2 * a.qs.sn + 2 * (16 * kc + 8 * g)));
        const float l = buffer_load_f32(rl, 4 * r);
        lse2[qb] = r < rows ? l * kLog2e : INFINITY;
      }
    };
    // the Q rows and LSE go out with the dO rows (one round trip for all);
    // at d = 128 only after D, where holding them early costs more than the
    // round trip (measured, like the early first tile below)
    constexpr bool kQFirst = D != 128;
    if constexpr (kQFirst) load_q();
    // the first key/value tile goes out with the rows (one round trip;
    // not at d = 128, as above)
    if (kQFirst && n_kv > 0) load_tile(0, 0);
    if (a.dq_computes_d) {
      // D_i = dO_i . O_i from the stored bf16 O (the backward preprocess,
      // done here on the rows this wave holds);
      // lanes l and l + 32 hold the two halves of each row's d.  Key range 0
      // writes D for the dK/dV pass.  (An fp32 O goes through the preprocess
      // kernel instead: one straight path here lets the O loads go out
      // together.)
      const bf16* opb = (const bf16*)a.o + b * a.os.sb + h * a.os.sh + (int64_t)sp.q_row0 * a.os.sn;
      const auto ro = rows_rsrc(opb + (int64_t)q0 * a.os.sn, rows, 2 * a.os.sn, 2 * D);
      float part[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int r = 32 * qb + ln;
        part[qb] = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const bf16x8 v = buffer_load_bf16x8(ro, (uint32_t)(r * 2 * a.os.sn + 2 * (16 * kc + 8 * g)));
#pragma unroll
          for (int j = 0; j < 8; ++j) part[qb] = fmaf((float)doreg[qb][kc][j], (float)v[j], part[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int r = 32 * qb + ln;
        dsum[qb] = sum_halves(part[qb]);
        if (split == 0 && g == 0 && r < rows) a.dsum[sp.stat0 + q0 + r] = dsum[qb];
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) dsum[qb] = buffer_load_f32(rs, 4 * (32 * qb + ln));
    }
    if constexpr (!kQFirst) load_q();
  }
  // E^T = D - dP^T: the matrix-core chain of dP^T = V dO^T runs on the
  // negated dO rows and starts from D (every entry of a lane's accumulator
  // belongs to its query), so dS needs one multiply per score: -dS = P E.
  // At d = 80 the 16 registers of D do not fit three waves per SIMD; there
  // D is added per score instead.
  constexpr bool kFoldD = D != 80;
  constexpr bool kRowOut = D != 80;  // orientation of the dQ accumulators (below)
  f32x16 dinit[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) dinit[qb][e] = kFoldD ? dsum[qb] : 0.f;
  }
  negate_rows(doreg);

  f32x16 dq[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[qb][db] = f32x16{};
  const float sl2 = a.scale * kLog2e;


  // One key/value tile; NEXT: tile it + 1 exists and is staged into the
  // other buffer while this one is computed (waited for before the barrier).
  // NCB = 1: a last tile of at most 32 keys, whose second 32-key block would
  // add nothing (its K rows are zero), is left out.
  auto tile = [&](auto next_tag, auto ncb_tag, int it) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int NCB = decltype(ncb_tag)::value;
    const int buf = it & 1;
    if (NEXT) load_tile((it + 1) * BN, buf ^ 1);
    if (wave_active) {
      const bf16* Kt = lds + buf * 2 * L::tile;
      const bf16* Vt = Kt + L::tile;
      f32x16 st[NCB][NQB], dpt[NCB][NQB];
      // the tile's K and V operands (A operands of S^T and dP^T)
      bf16x8 ka[NCB][KC], va[NCB][KC];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          ka[cb][kc] = load_bf16x8(&Kt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
          va[cb][kc] = load_bf16x8(&Vt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
        }
      prio_mfma();
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          st[cb][qb] = f32x16{};
          dpt[cb][qb] = dinit[qb];
        }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            st[cb][qb] = mfma32(ka[cb][kc], qreg[qb][kc], st[cb][qb]);
            dpt[cb][qb] = mfma32(va[cb][kc], doreg[qb][kc], dpt[cb][qb]);
          }
        }
      }
      prio_valu();
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(fmaf(st[cb][qb][e], sl2, -lse2[qb]));
            st[cb][qb][e] = p * (kFoldD ? dpt[cb][qb][e] : dpt[cb][qb][e] + dsum[qb]);
          }
      // (-dQ)^T += K^T (-dS)^T over four 16-key chunks (slot group g: keys
      // 16t + 4g + (0..3) and 16t + 8 + 4g + (0..3) = accumulator entries
      // 8hh..8hh+7): the K columns (transpose reads) are the A operand, so a
      // lane's accumulator holds its query row's runs of 4 consecutive d.
      // At d = 80 that orientation costs spills at three waves per SIMD;
      // there the product is -dQ += (-dS) K and a lane holds one d column.
      prio_mfma();
#pragma unroll
      for (int t = 0; t < 2 * NCB; ++t) {
        bf16x8 sa[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) sa[qb] = acc_half_to_bf16(st[t >> 1][qb], t & 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 kb8 = tr_operand(Kt + 32 * db, KS, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            dq[qb][db] = kRowOut ? mfma32(kb8, sa[qb], dq[qb][db]) : mfma32(sa[qb], kb8, dq[qb][db]);
        }
      }
      prio_valu();
    }
    wait_vmem();
    __syncthreads();
  };
  // (a packed sequence without keys: dQ = 0)
  if (n_kv > 0) {
    if (D == 128) load_tile(0, 0);
    wait_vmem();  // the first tile (at d != 128 requested with the rows)
    __syncthreads();
    using Full = std::integral_constant<int, 2>;
    using Half = std::integral_constant<int, 1>;
    int it = 0;
    for (; it + 1 < ntiles; ++it) tile(std::true_type{}, Full{}, it);
    if (n_kv - it * BN > 32)
      tile(std::false_type{}, Full{}, it);
    else
      tile(std::false_type{}, Half{}, it);
  }

  if (!wave_active) return;
  const float sc = -a.scale;
  if constexpr (!kRowOut) {
    // lane owns column d = 32db + ln, query rows 8i + 4g + r of each block.
    // The three destinations are chosen outside the unrolled loops, and the
    // accumulating one reads every value it adds to before its first store
    // (one round trip instead of one per value).
    auto each = [&](auto&& f) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int dcol = 32 * db + ln;
          if (dcol >= D) continue;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int qr = q0 + 32 * qb + 8 * (e >> 2) + 4 * g + (e & 3);
            if (qr < sp.nq) f(qb, db, e, qr, dcol);
          }
        }
    };
    if (a.dq_splits > 1) {  // this key range's share, summed by dq_reduce_kernel
      each([&](int qb, int db, int e, int qr, int dcol) {
        a.dq_part[((((int64_t)split * a.B + b) * a.H + h) * a.Nq + qr) * D + dcol] =
            dq[qb][db][e] * sc;
      });
    } else if (accumulate) {
      float* const base = (float*)a.dq + b * a.dqs.sb + h * a.dqs.sh + (int64_t)sp.q_row0 * a.dqs.sn;
      float old[NQB][NDB][16];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) old[qb][db][e] = 0.f;
      each([&](int qb, int db, int e, int qr, int dcol) {
        old[qb][db][e] = base[(int64_t)qr * a.dqs.sn + dcol];
      });
      // every sum before the first store (a wait for a read issued before a
      // pending store would wait for that store too); the empty asm keeps
      // the compiler from sinking the sums next to their stores
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            old[qb][db][e] += dq[qb][db][e] * sc;
            asm volatile("" : "+v"(old[qb][db][e]));
          }
      each([&](int qb, int db, int e, int qr, int dcol) {
        base[(int64_t)qr * a.dqs.sn + dcol] = old[qb][db][e];
      });
    } else {
      bf16* const base = (bf16*)a.dq + b * a.dqs.sb + h * a.dqs.sh + (int64_t)sp.q_row0 * a.dqs.sn;
      each([&](int qb, int db, int e, int qr, int dcol) {
        base[(int64_t)qr * a.dqs.sn + dcol] = (bf16)(dq[qb][db][e] * sc);
      });
    }
    return;
  }
  // lane owns query row q0 + 32qb + ln and, per 32-column block db, the runs
  // d = 32db + 8i + 4g + (0..3) (accumulator entries 4i .. 4i+3)
  if (a.dq_splits > 1 || accumulate) {
    // fp32: 16-byte pieces straight from the runs (a key range's share for
    // dq_reduce_kernel, or added to an fp32 dQ)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qr = q0 + 32 * qb + ln;
      if (qr >= sp.nq) continue;
      float* const row =
          a.dq_splits > 1
              ? a.dq_part + (((int64_t)split * a.B + b) * a.H + h) * a.Nq * D + (int64_t)qr * D
              : (float*)a.dq + b * a.dqs.sb + h * a.dqs.sh + (int64_t)(sp.q_row0 + qr) * a.dqs.sn;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * db + 8 * i + 4 * g;
          if (d0 >= D) continue;
          const f32x16& x = dq[qb][db];
          const f32x4 v4 = {x[4 * i] * sc, x[4 * i + 1] * sc, x[4 * i + 2] * sc, x[4 * i + 3] * sc};
          f32x4* const p = reinterpret_cast<f32x4*>(row + d0);
          if (a.dq_splits > 1)
            *p = v4;
          else
            *p = *p + v4;
        }
    }
    return;
  }
  // bf16: the runs go through this wave's rows of the (now free) key/value
  // tiles and leave as whole rows; the last tile's barrier has retired every
  // read of the tiles
  constexpr int SRS = DP + 8;
  static_assert(4 * 32 * SRS <= 4 * L::tile, "staging fits the tiles");
  bf16* const stage = lds + w * 32 * SRS;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * g;
        if (d0 >= D) continue;
        const f32x16& x = dq[qb][db];
        const bf16x4 v4 = {(bf16)(x[4 * i] * sc), (bf16)(x[4 * i + 1] * sc),
                           (bf16)(x[4 * i + 2] * sc), (bf16)(x[4 * i + 3] * sc)};
        *reinterpret_cast<bf16x4*>(&stage[ln * SRS + d0]) = v4;
      }
    const int r0 = q0 + 32 * qb;
    bf16* const out = (bf16*)a.dq + b * a.dqs.sb + h * a.dqs.sh + (int64_t)(sp.q_row0 + r0) * a.dqs.sn;
    store_staged_rows<bf16, D, SRS>(stage, out, a.dqs.sn, sp.nq - r0, lane);
  }
}

// --------------------------------------------------------------------------
// dQ over split key ranges: dQ = sum over ranges of the partials, in range
// order (so the result does not depend on scheduling), then written in dQ's
// dtype or added to an fp32 dQ.  One thread per 4 consecutive d.
// --------------------------------------------------------------------------
template <typename TO>
__global__ __launch_bounds__(256) void dq_reduce_kernel(BwdArgs a, int d, int accumulate) {
  const int64_t rows = (int64_t)a.B * a.H * a.Nq;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int dv4 = d / 4;
  if (i >= rows * dv4) return;
  const int64_t row = i / dv4;
  const int c = 4 * (int)(i % dv4);
  f32x4 acc = *reinterpret_cast<const f32x4*>(a.dq_part + row * d + c);
  for (int sp = 1; sp < a.dq_splits; ++sp)
    acc += *reinterpret_cast<const f32x4*>(a.dq_part + (sp * rows + row) * d + c);
  const int q = (int)(row % a.Nq);
  const int64_t bh = row / a.Nq;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int64_t o = b * a.dqs.sb + h * a.dqs.sh + (int64_t)q * a.dqs.sn + c;
  if constexpr (sizeof(TO) == 4) {
    f32x4* p = reinterpret_cast<f32x4*>((float*)a.dq + o);
    *p = accumulate ? *p + acc : acc;
  } else {
    const bf16x4 v = {(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
    *reinterpret_cast<bf16x4*>((bf16*)a.dq + o) = v;
  }
}

// Query blocks per dQ workgroup are 128 rows; below this many workgroups the
// key range is split (each range at least 8 key tiles of 64).
constexpr long long kDqTargetWorkgroups = 1024;

int dq_key_splits(int B, int H, int Nq, int Nkv) {
  const long long base = (long long)((Nq + 127) / 128) * H * B;
  const int ntiles = (Nkv + dqk::BN - 1) / dqk::BN;
  if (base >= kDqTargetWorkgroups) return 1;
  int s = (int)((kDqTargetWorkgroups + base - 1) / base);
  s = min(s, ntiles / 8);
  if (s < 2) return 1;
  const int per = (ntiles + s - 1) / s;  // tiles per range; every range non-empty
  return (ntiles + per - 1) / per;
}

// Occupancy: kernels whose registers fit request two waves per SIMD.
#ifndef EXATTN_DKDV_WAVES
#define EXATTN_DKDV_WAVES 2
#endif
template <int D, int KW>
__global__ __launch_bounds__(bwdk::NT)
__attribute__((amdgpu_waves_per_eu(KW == 32 && D <= 80 ? EXATTN_DKDV_WAVES : 1)))
void dkdv_bf16_kernel(BwdArgs a) {
  dkdv_body<D, KW>(a);
}
// Occupancy of the dQ kernel: three waves per SIMD fit d = 64 and d = 80
// without spills, two fit d = 128.
#ifndef EXATTN_DQ_WAVES
#define EXATTN_DQ_WAVES 3
#endif
template <int D, int QW>
__global__ __launch_bounds__(dqk::NT)
__attribute__((amdgpu_waves_per_eu(D <= 80 ? EXATTN_DQ_WAVES : 2)))
void dq_bf16_kernel(BwdArgs a, int accumulate) {
  dq_body<D, QW>(a, accumulate);
}

// --------------------------------------------------------------------------
// fp32 inputs: genuine fp32 arithmetic, exact library exp.  As in the fp32
// forward, a workgroup owns 64 rows (one per lane, the same rows in each of
// its W waves) and splits the streamed rows over the waves; the waves'
// partial gradients are summed through LDS at the end.
//  - dK, dV: owned key rows (K, V in padded LDS, dK, dV in registers),
//    streamed query tiles read by broadcast.
//  - dQ: owned query rows (Q, dO in padded LDS, dQ in registers), streamed
//    key tiles read by broadcast.
// --------------------------------------------------------------------------
namespace bwdf {
constexpr int RB = 64;      // owned rows per workgroup, one per lane
constexpr int TB = 2;       // streamed rows per wave per staged tile
// waves splitting the streamed rows: eight where two waves per SIMD keep
// their accumulators in registers, else four (one per SIMD: the dK + dV
// accumulators, 2d registers, need the larger register file)
template <int D, bool DKDV = false>
constexpr int waves() { return D <= 80 && !DKDV ? 8 : 4; }
}  // namespace bwdf

// x[lane] of every wave summed into wave 0's x (buf: [RB][D + 1] floats)
template <int W, int D>
__device__ __forceinline__ void sum_over_waves(float (&x)[D], float (*buf)[D + 1], int w,
                                               int lane) {
  for (int r = 1; r < W; ++r) {
    __syncthreads();
    if (w == r) {
#pragma unroll
      for (int i = 0; i < D; ++i) buf[lane][i] = x[i];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int i = 0; i < D; ++i) x[i] += buf[lane][i];
    }
  }
}

template <int D>
__global__ __launch_bounds__((64 * bwdf::waves<D, true>())) void bwd_f32_dkdv_kernel(BwdArgs a) {
  using namespace bwdf;
  constexpr int W = waves<D, true>(), BS = W * TB;  // BS: streamed rows per staged tile
  __shared__ float Kown[RB][D + 1], Vown[RB][D + 1];
  __shared__ float Qt[BS][D], dOt[BS][D];
  __shared__ float lse_t[BS], D_t[BS];
  __shared__ float Ab[RB][D + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  for (int e = tid; e < RB * D; e += 64 * W) {
    const int r = e / D, cc = e % D;
    const bool ok = k0 + r < a.Nkv;
    Kown[r][cc] = ok ? kp[(int64_t)(k0 + r) * a.ks.sn + cc] : 0.f;
    Vown[r][cc] = ok ? vp[(int64_t)(k0 + r) * a.vs.sn + cc] : 0.f;
  }
  // One pass over the query rows accumulates the gradients in GRADS (1: dV,
  // 2: dK, 3: both).  At d = 128 the two accumulators (256 registers) do not
  // fit the vector registers a VALU instruction can address, so dV and dK
  // take a pass each (the scores computed twice) instead of spilling.
  const int kr = k0 + lane;
  auto pass = [&](auto grads_tag) {
    constexpr int GR = decltype(grads_tag)::value;
    constexpr bool DV = GR & 1, DK = GR & 2;
    float acc_v[DV ? D : 1], acc_k[DK ? D : 1];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if constexpr (DV) acc_v[i] = 0.f;
      if constexpr (DK) acc_k[i] = 0.f;
    }
    for (int q0 = 0; q0 < a.Nq; q0 += BS) {
      __syncthreads();
      for (int e = tid; e < BS * D; e += 64 * W) {
        const int r = e / D, cc = e % D;
        const bool ok = q0 + r < a.Nq;
        Qt[r][cc] = ok ? qp[(int64_t)(q0 + r) * a.qs.sn + cc] : 0.f;
        dOt[r][cc] = ok ? dop[(int64_t)(q0 + r) * a.dos.sn + cc] : 0.f;
      }
      if (tid < BS) {
        const bool ok = q0 + tid < a.Nq;
        lse_t[tid] = ok ? lsep[q0 + tid] : INFINITY;
        D_t[tid] = ok ? dsp[q0 + tid] : 0.f;
      }
      __syncthreads();
#pragma unroll 1
      for (int t = 0; t < TB; ++t) {
        const int j = w * TB + t;  // rows past Nq: Q = dO = 0, LSE = +inf, so P = 0
        // the lane's own K / V row; at d = 128 it is re-read from LDS per
        // query row rather than held in registers (that would not fit)
        const float* krow = Kown[lane];
        const float* vrow = Vown[lane];
        if constexpr (D > 80) asm volatile("" : "+v"(krow), "+v"(vrow));
        float s4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < D; ++i) {
          s4[i & 3] = fmaf(Qt[j][i], krow[i], s4[i & 3]);
          if constexpr (DK) p4[i & 3] = fmaf(dOt[j][i], vrow[i], p4[i & 3]);
        }
        const float sv = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        const float p = expf(sv * a.scale - lse_t[j]);
        float ds = 0.f;
        if constexpr (DK) {
          const float dpv = (p4[0] + p4[1]) + (p4[2] + p4[3]);
          ds = p * (dpv - D_t[j]);
        }
#pragma unroll
        for (int i = 0; i < D; ++i) {
          if constexpr (DV) acc_v[i] = fmaf(p, dOt[j][i], acc_v[i]);
          if constexpr (DK) acc_k[i] = fmaf(ds, Qt[j][i], acc_k[i]);
        }
      }
    }
    if constexpr (DK) sum_over_waves<W, D>(acc_k, Ab, w, lane);
    if constexpr (DV) sum_over_waves<W, D>(acc_v, Ab, w, lane);
    if (w == 0 && kr < a.Nkv) {
      if constexpr (DK) {
        float* dkp = (float*)a.dk + b * a.dks.sb + h * a.dks.sh + (int64_t)kr * a.dks.sn;
        for (int i = 0; i < D; ++i) dkp[i] = acc_k[i] * a.scale;
      }
      if constexpr (DV) {
        float* dvp = (float*)a.dv + b * a.dvs.sb + h * a.dvs.sh + (int64_t)kr * a.dvs.sn;
        for (int i = 0; i < D; ++i) dvp[i] = acc_v[i];
      }
    }
  };
  if constexpr (D > 80) {
    pass(std::integral_constant<int, 1>{});
    pass(std::integral_constant<int, 2>{});
  } else {
    pass(std::integral_constant<int, 3>{});
  }
}

template <int D>
__global__ __launch_bounds__(64 * bwdf::waves<D>()) void bwd_f32_dq_kernel(BwdArgs a,
                                                                       int accumulate) {
  using namespace bwdf;
  constexpr int W = waves<D>(), BS = W * TB;
  __shared__ float Qown[RB][D + 1], dOown[RB][D + 1];
  __shared__ float Kt[BS][D], Vt[BS][D];
  __shared__ float Ab[RB][D + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (a.Nq + RB - 1) / RB;
  const int qb = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;
  const int h = bh % a.H, b = bh / a.H;
  const float* qp = (const float*)a.q + b * a.qs.sb + h * a.qs.sh;
  const float* dop = (const float*)a.dout + b * a.dos.sb + h * a.dos.sh;
  const float* kp = (const float*)a.k + b * a.ks.sb + h * a.ks.sh;
  const float* vp = (const float*)a.v + b * a.vs.sb + h * a.vs.sh;
  const int q0 = qb * RB;
  for (int e = tid; e < RB * D; e += 64 * W) {
    const int r = e / D, cc = e % D;
    const bool ok = q0 + r < a.Nq;
    Qown[r][cc] = ok ? qp[(int64_t)(q0 + r) * a.qs.sn + cc] : 0.f;
    dOown[r][cc] = ok ? dop[(int64_t)(q0 + r) * a.dos.sn + cc] : 0.f;
  }
  const int qi = q0 + lane;
  const bool qvalid = qi < a.Nq;
  const float lse_i = qvalid ? a.lse[((int64_t)b * a.H + h) * a.Nq + qi] : INFINITY;
  const float D_i = qvalid ? a.dsum[((int64_t)b * a.H + h) * a.Nq + qi] : 0.f;
  float dq[D];
#pragma unroll
  for (int i = 0; i < D; ++i) dq[i] = 0.f;
  for (int j0 = 0; j0 < a.Nkv; j0 += BS) {
    __syncthreads();
    for (int e = tid; e < BS * D; e += 64 * W) {
      const int r = e / D, cc = e % D;
      const bool ok = j0 + r < a.Nkv;
      Kt[r][cc] = ok ? kp[(int64_t)(j0 + r) * a.ks.sn + cc] : 0.f;
      Vt[r][cc] = ok ? vp[(int64_t)(j0 + r) * a.vs.sn + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int t = 0; t < TB; ++t) {
      const int j = w * TB + t;
      if (j0 + j >= a.Nkv) continue;  // (uniform) keys past the end
      float s4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s4[i & 3] = fmaf(Qown[lane][i], Kt[j][i], s4[i & 3]);
        p4[i & 3] = fmaf(dOown[lane][i], Vt[j][i], p4[i & 3]);
      }
      const float sv = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      const float dpv = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      const float p = expf(sv * a.scale - lse_i);
      const float ds = p * (dpv - D_i);
#pragma unroll
      for (int i = 0; i < D; ++i) dq[i] = fmaf(ds, Kt[j][i], dq[i]);
    }
  }
  sum_over_waves<W, D>(dq, Ab, w, lane);
  if (w != 0 || !qvalid) return;
  float* dqp = (float*)a.dq + b * a.dqs.sb + h * a.dqs.sh + (int64_t)qi * a.dqs.sn;
  for (int i = 0; i < D; ++i) {
    const float v = dq[i] * a.scale;
    dqp[i] = accumulate ? dqp[i] + v : v;
  }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
hipError_t launch_bwd_pre(const BwdArgs& a, int d, int in_bf16, hipStream_t s) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  const long long grid = (rows + 15) / 16;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (in_bf16) {
    const long long g2 = (2 * rows + 255) / 256;
    if (g2 > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.o_f32)
      hipLaunchKernelGGL((bwd_pre_bf16_kernel<float>), dim3((unsigned)g2), dim3(256), 0, s, a, d);
    else
      hipLaunchKernelGGL((bwd_pre_bf16_kernel<bf16>), dim3((unsigned)g2), dim3(256), 0, s, a, d);
  } else {
    hipLaunchKernelGGL((bwd_pre_kernel<float, float>), dim3((unsigned)grid), dim3(256), 0, s, a, d);
  }
  return hipGetLastError();
}

template <typename K>
static hipError_t allow_lds(K kernel, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D, int KW>
static hipError_t launch_dkdv(const BwdArgs& a, hipStream_t s) {
  const long long grid = (long long)((a.Nkv + 4 * KW - 1) / (4 * KW)) * a.H * a.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int lds = DkdvLds<D>::bytes;
  static const hipError_t attr = allow_lds(&dkdv_bf16_kernel<D, KW>, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((dkdv_bf16_kernel<D, KW>), dim3((unsigned)grid), dim3(bwdk::NT), lds, s, a);
  return hipGetLastError();
}

template <int D, int QW>
static hipError_t launch_dq(const BwdArgs& a_in, int accumulate, hipStream_t s) {
  BwdArgs a = a_in;
  const int ntiles = (a.Nkv + dqk::BN - 1) / dqk::BN;
  a.dq_splits = a.dq_part ? dq_key_splits(a.B, a.H, a.Nq, a.Nkv) : 1;
  a.dq_split_len = ((ntiles + a.dq_splits - 1) / a.dq_splits) * dqk::BN;
  const long long grid =
      (long long)((a.Nq + 4 * QW - 1) / (4 * QW)) * a.H * a.B * a.dq_splits;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int lds = DqLds<D>::bytes;
  static const hipError_t attr = allow_lds(&dq_bf16_kernel<D, QW>, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((dq_bf16_kernel<D, QW>), dim3((unsigned)grid), dim3(dqk::NT), lds, s, a,
                     accumulate);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.dq_splits == 1) return e;
  const long long n4 = (long long)a.B * a.H * a.Nq * (D / 4);
  const unsigned rg = (unsigned)((n4 + 255) / 256);
  if (accumulate)
    hipLaunchKernelGGL((dq_reduce_kernel<float>), dim3(rg), dim3(256), 0, s, a, D, 1);
  else
    hipLaunchKernelGGL((dq_reduce_kernel<bf16>), dim3(rg), dim3(256), 0, s, a, D, 0);
  return hipGetLastError();
}

static int compute_units() {
  static const int n = [] {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
      return 256;
    return cu;
  }();
  return n;
}

// resident query side: at most 128 query rows and at least 4 key blocks
static bool use_resident_dkdv(const BwdArgs& a) {
  return EXATTN_DKDV_RESIDENT && !a.cu_q && a.Nq <= resk::QR &&
         (a.Nkv + resk::KB - 1) / resk::KB >= 4;
}

template <int D>
static hipError_t launch_dkdv_resident(const BwdArgs& a, hipStream_t s) {
  const long long nkb = (a.Nkv + resk::KB - 1) / resk::KB;
  const long long heads = (long long)a.B * a.H;
  // about one workgroup per compute unit, each walking a share of its head
  const long long groups = std::min(nkb, std::max(1LL, (compute_units() + heads - 1) / heads));
  const long long grid = heads * groups;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int lds = ResLds<D>::bytes;
  static const hipError_t attr = allow_lds(&dkdv_resident_kernel<D>, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((dkdv_resident_kernel<D>), dim3((unsigned)grid), dim3(resk::NT), lds, s, a,
                     (int)groups);
  return hipGetLastError();
}

template <int D, int KW, int QW>
static hipError_t bwd_bf16_d(const BwdArgs& a, int do_dkdv, int do_dq, int accumulate,
                             hipStream_t s) {
  // dQ first: when it computes D (no preprocess), dK/dV reads that D
  if (do_dq) {
    const hipError_t e = launch_dq<D, QW>(a, accumulate, s);
    if (e != hipSuccess) return e;
  }
  if (do_dkdv)
    return use_resident_dkdv(a) ? launch_dkdv_resident<D>(a, s) : launch_dkdv<D, KW>(a, s);
  return hipSuccess;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, int do_dkdv, int do_dq, int accumulate,
                           hipStream_t s) {
  if (EXATTN_SHORT && short_slot(a.Nq, a.Nkv))
    return launch_bwd_short(a, d, do_dkdv, do_dq, accumulate, s);
  switch (d) {
    case 64: return bwd_bf16_d<64, 32, 32>(a, do_dkdv, do_dq, accumulate, s);
    case 80: return bwd_bf16_d<80, 32, 32>(a, do_dkdv, do_dq, accumulate, s);
    case 128: return bwd_bf16_d<128, 32, 32>(a, do_dkdv, do_dq, accumulate, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t bwd_f32_d(const BwdArgs& a, int do_dkdv, int do_dq, int accumulate,
                            hipStream_t s) {
  const long long gk = (long long)((a.Nkv + bwdf::RB - 1) / bwdf::RB) * a.H * a.B;
  const long long gq = (long long)((a.Nq + bwdf::RB - 1) / bwdf::RB) * a.H * a.B;
  if (gk > 0x7fffffffLL || gq > 0x7fffffffLL) return hipErrorInvalidValue;
  if (do_dkdv) {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D>), dim3((unsigned)gk),
                       dim3(64 * bwdf::waves<D, true>()), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (do_dq) {
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D>), dim3((unsigned)gq), dim3(64 * bwdf::waves<D>()),
                       0, s, a, accumulate);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd_f32(const BwdArgs& a, int d, int do_dkdv, int do_dq, int accumulate,
                          hipStream_t s) {
  switch (d) {
    case 64: return bwd_f32_d<64>(a, do_dkdv, do_dq, accumulate, s);
    case 80: return bwd_f32_d<80>(a, do_dkdv, do_dq, accumulate, s);
    case 128: return bwd_f32_d<128>(a, do_dkdv, do_dq, accumulate, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace exattn

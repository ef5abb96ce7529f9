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

#include <type_traits>

// occupancy request (waves per SIMD) of the bf16 forward for d = 64; d = 80
// and 128 ask for two (three would spill).  At d = 64 the allocation stays
// at 113 registers, which allows four waves per SIMD, and the 36.9 KB of
// double-buffered K/V tiles per workgroup also allow four workgroups per
// compute unit: asking for five cannot be met (the compiler then falls back
// to its default register budget).
#ifndef EXATTN_FWD_WAVES
#define EXATTN_FWD_WAVES 2
#endif

namespace exattn {

// --------------------------------------------------------------------------
// bf16 inputs, bf16 matrix cores (32x32x16), fp32 accumulation.
//
// Workgroup: 4 waves, each owning QW = 32 query rows.  Key/value tiles of 64
// rows are staged in LDS row-major and double-buffered with direct-to-LDS
// loads: the next tile's loads are issued before the current tile is
// computed and waited for after it, so one barrier per tile suffices and the
// load latency hides behind the matrix work.
//
// Each wave computes the transposed score tile S^T = K Q^T: every lane then
// owns one query row (accumulator column lane % 32), the softmax statistics
// are per-lane scalars, and the exponentiated tile is already in the B-operand
// layout of O^T += V^T P^T.  The V^T operand is read straight from the
// row-major V tile with LDS transpose reads.
//
// The running maximum is refreshed lazily: the reference value m used in
// exp2(s - m) is raised only when a row's maximum exceeds it by more than
// 2^8 in the exponent, which bounds the weights by 256; any reference value
// gives the same O and LSE, so this changes rounding only.
// --------------------------------------------------------------------------
namespace fwdk {
constexpr int BN = 64;
constexpr int NT = 256;
constexpr float kLazy = 8.0f;  // log2 of the largest weight allowed before rescaling
// the largest partial sum of a lane's 32 weights that skips the row maxima:
// 2^kLazy, so a tile is taken as it is only where the maxima would not have
// raised the reference either.  (A looser bound, 2^(kLazy + 5), was faster
// on the spatial shape but keeps stale references on peaky rows: their
// dominant weight then carries bf16 rounding instead of being exactly 1
// after a raise, and the O error of a peaky d = 128 case grew from 0.014 to
// 0.022, past the 2e-2 tolerance once the output's own rounding adds in.)
constexpr float kSumBound = 256.0f;
}  // namespace fwdk

template <int D>
struct FwdLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int KS = tile_stride(DP);       // row stride of the K and V tiles
  static constexpr int tile = fwdk::BN * KS;        // elements per tile
  static constexpr int bytes = 4 * tile * 2;        // K, V x double buffer
};

template <int D, int QW, bool OUT_F32>
__global__ __launch_bounds__(fwdk::NT)
__attribute__((amdgpu_waves_per_eu(D == 64 ? EXATTN_FWD_WAVES : 2)))
void fwd_bf16_kernel(FwdArgs a) {
  using namespace fwdk;
  using L = FwdLds<D>;
  constexpr int DP = L::DP, NDB = DP / 32, KC = D / 16, KS = L::KS;
  constexpr int NQB = QW / 32;          // 32-row query blocks per wave
  constexpr int BM = 4 * QW;            // query rows per workgroup
  __shared__ __attribute__((aligned(16))) bf16 lds[4 * L::tile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31, g = lane >> 5;

  const int nqb = (a.Nq + BM - 1) / BM;
  int idx = xcd_remap(blockIdx.x, gridDim.x);
  const int qblk = idx % nqb;
  idx /= nqb;
  const int h = idx % a.H;
  idx /= a.H;
  const int b = idx % a.B;
  const int c = idx / a.B;
  const SeqSpan sp = seq_span(a, b, h);
  if (qblk * BM >= sp.nq) return;  // a packed sequence shorter than the longest

  const int kv_lo = c * a.chunk_len;
  const int n_kv = max(0, min(sp.nkv, kv_lo + a.chunk_len) - kv_lo);
  const int ntiles = (n_kv + BN - 1) / BN;

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh + (int64_t)sp.q_row0 * a.qs.sn;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh +
                   (int64_t)(sp.kv_row0 + kv_lo) * a.ks.sn;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh +
                   (int64_t)(sp.kv_row0 + kv_lo) * a.vs.sn;

  const int q0 = qblk * BM + w * QW;
  const bool wave_active = q0 < sp.nq;

  // this wave's query rows as B operands: lane -> row q0 + 32 qb + ln,
  // d = 16 kc + 8 g .. +7 (rows past Nq read as zeros)
  bf16x8 qreg[NQB][KC];
  {
    const auto rq = rows_rsrc(qp + (int64_t)q0 * a.qs.sn, sp.nq - q0, 2 * a.qs.sn, 2 * D);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        qreg[qb][kc] = buffer_load_bf16x8(
            rq, (uint32_t)((32 * qb + ln) * 2 * a.qs.sn + 2 * (16 * kc + 8 * g)));
  }

  // direct-to-LDS staging of key/value tiles (see LdsTileDma); rows past
  // the end read as zeros
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

  f32x16 oacc[NDB][NQB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) oacc[db][qb] = f32x16{};
  float mref[NQB], lsum[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    mref[qb] = -INFINITY;
    lsum[qb] = 0.f;
  }
  const float sl2 = a.scale * kLog2e;
  const float lazy = kLazy / sl2;  // threshold in raw score units

  // One key/value tile.  In the steady state (TAIL false) the caller
  // guarantees that tile it + 1 exists to be staged and that tile it is
  // full: the body then has no condition and no masking.  The last tile
  // (TAIL true) masks keys past the end.
  auto tile = [&](auto tail_tag, int it) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int buf = it & 1;
    const int j0 = it * BN;
    if (!TAIL) load_tile(j0 + BN, buf ^ 1);
    if (wave_active) {
      const bf16* Kt = lds + buf * 2 * L::tile;
      const bf16* Vt = Kt + L::tile;
      // S^T = K Q^T for two 32-key blocks x NQB query blocks; keys past the
      // end weigh nothing
      // (a last tile of at most 32 keys skips the second key block's
      // products; its scores stay zero and are masked below, and the value
      // products of 16-key chunks past the end are skipped too)
      const int rem = n_kv - j0;
      const bool second = !TAIL || rem > 32;
      const int nchunks = TAIL ? (rem + 15) / 16 : 4;
      f32x16 s[2][NQB];
      // (the memory fence keeps the compiler from reusing the first pass's
      // scores in the second one, which would hold them in 32 more registers)
      auto scores = [&] {
        asm volatile("" ::: "memory");
        prio_mfma();
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[cb][qb] = f32x16{};
          if (cb == 1 && !second) break;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            const bf16x8 ka = load_bf16x8(&Kt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) s[cb][qb] = mfma32(ka, qreg[qb][kc], s[cb][qb]);
          }
        }
        prio_valu();
        if constexpr (TAIL) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const bool dead = j0 + 32 * cb + 8 * (e >> 2) + 4 * g + (e & 3) >= n_kv;
#pragma unroll
              for (int qb = 0; qb < NQB; ++qb)
                if (dead) s[cb][qb][e] = -INFINITY;
            }
        }
      };
      // P = exp2(sl2 (s - mref)) in place, and this lane's sum of its 32
      // weights per query block.  The sum is taken over the fp32 weights: a
      // peaky row's few dominant weights would carry their bf16 rounding
      // into the LSE.
      float psum[NQB];
      auto weigh = [&] {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float moff = mref[qb] * sl2;
          float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float p = fast_exp2(fmaf(s[cb][qb][e], sl2, -moff));
              s[cb][qb][e] = p;
              part[e & 3] += p;
            }
          psum[qb] = (part[0] + part[1]) + (part[2] + part[3]);
        }
      };
      scores();
      // After the first tile the weights are formed against the current
      // reference first.  A partial sum of at most 2^kLazy (a NaN or
      // infinite one fails the test) bounds each of its 32 weights by that
      // much, and then the tile needs no row maximum.  Otherwise, and on
      // the first tile, the scores are formed again, the row maxima taken,
      // and the reference raised (rescaling what O and l hold so far) where
      // a row's maximum exceeds it by more than 2^kLazy.
      bool slow = it == 0;
      if (!slow) {
        weigh();
        bool big = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) big |= !(psum[qb] <= kSumBound);
        slow = __builtin_amdgcn_ballot_w64(big) != 0;
        if (slow) scores();
      }
      if (slow) {
        float mx[NQB];
        bool raise = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float m = s[0][qb][0];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, s[cb][qb][e]);
          mx[qb] = max_halves(m);
          raise |= mx[qb] > mref[qb] + lazy;
        }
        if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float mnew = fmaxf(mref[qb], mx[qb]);
            const float alpha = fast_exp2((mref[qb] - mnew) * sl2);
            mref[qb] = mnew;
            lsum[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
          }
        }
        weigh();
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) lsum[qb] += psum[qb];
      // O^T += V^T P^T over four 16-key chunks.  Chunk t = 2 cb + hh holds,
      // for slot group g, keys 16t + 4g + (0..3) and 16t + 8 + 4g + (0..3):
      // accumulator entries 8hh .. 8hh+7 of block cb.
      bf16x8 pb[4][NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int t = 0; t < 4; ++t) pb[t][qb] = acc_half_to_bf16(s[t >> 1][qb], t & 1);
      prio_mfma();
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t >= nchunks) break;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 va = tr_operand(Vt + 32 * db, KS, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) oacc[db][qb] = mfma32(va, pb[t][qb], oacc[db][qb]);
        }
      }
      prio_valu();
    }
    wait_vmem();
    __syncthreads();
  };
  // (an empty key range skips the loop)
  if (ntiles > 0) {
    load_tile(0, 0);
    wait_vmem();
    __syncthreads();
    int it = 0;
    for (; it + 1 < ntiles; ++it) tile(std::false_type{}, it);
    tile(std::true_type{}, it);
  }

  if (!wave_active) return;
  // O leaves through this wave's rows of the (now free) key/value tiles:
  // a lane owns one query row and runs of 4 d of it, which go to LDS first
  // and then out as whole rows (store_staged_rows); the last tile's barrier
  // has retired every read of the tiles
  using OT = std::conditional_t<OUT_F32, float, bf16>;
  constexpr int SRS = OUT_F32 ? D + 4 : DP + 8;  // staging row stride (16-byte rows)
  static_assert(4 * 32 * SRS * sizeof(OT) <= sizeof(lds), "staging fits the tiles");
  OT* const stage = reinterpret_cast<OT*>(lds) + w * 32 * SRS;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float l = sum_halves(lsum[qb]);
    const int qrow = q0 + 32 * qb + ln;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * g;
        if (d0 < D) {
          const f32x16& o = oacc[db][qb];
          if constexpr (OUT_F32) {
            const f32x4 v4 = {o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv,
                              o[4 * i + 3] * inv};
            *reinterpret_cast<f32x4*>(&stage[ln * SRS + d0]) = v4;
          } else {
            const bf16x4 v4 = {(bf16)(o[4 * i] * inv), (bf16)(o[4 * i + 1] * inv),
                               (bf16)(o[4 * i + 2] * inv), (bf16)(o[4 * i + 3] * inv)};
            *reinterpret_cast<bf16x4*>(&stage[ln * SRS + d0]) = v4;
          }
        }
      }
    }
    const int r0 = q0 + 32 * qb;
    OT* const out = reinterpret_cast<OT*>(a.o) + (int64_t)c * a.o_chunk_stride + b * a.os.sb +
                    h * a.os.sh + (int64_t)(sp.q_row0 + r0) * a.os.sn;
    store_staged_rows<OT, D, SRS>(stage, out, a.os.sn, sp.nq - r0, lane);
    if (g == 0 && qrow < sp.nq) {
      const int64_t li = (int64_t)c * a.lse_chunk_stride + sp.stat0 + qrow;
      a.lse[li] = l > 0.f ? (mref[qb] * sl2 + log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

// --------------------------------------------------------------------------
// fp32 inputs: genuine fp32 products and sums on the vector ALUs, exact
// library exp/log.  Meant for small problems that need fp32 accuracy, where
// a workgroup per 64 query rows alone would leave the chip almost empty, so
// each workgroup splits its key range over W waves: every lane owns one
// query row in every wave, the waves take disjoint keys of each staged tile
// and run their own online softmax, and the W partial (m, l, O) are merged
// exactly at the end (the LSE merge of the LV-XAttn abstract, over waves).
// --------------------------------------------------------------------------
namespace fwdf {
constexpr int BM = 64;      // query rows per workgroup, one per lane
constexpr int TB = 4;       // keys per wave per staged tile
// waves splitting the keys: eight (two per SIMD) up to d = 80, four at 128
template <int D>
constexpr int waves() { return D <= 80 ? 8 : 4; }
}  // namespace fwdf

template <int D>
__global__ __launch_bounds__(64 * fwdf::waves<D>()) void fwd_f32_kernel(FwdArgs a) {
  using namespace fwdf;
  constexpr int W = waves<D>(), BN = W * TB;  // BN: keys per staged tile
  __shared__ float Ks[BN][D];
  __shared__ float Vs[BN][D];
  __shared__ float Ms[BM], Ls[BM];
  __shared__ float Ab[BM][D + 1];  // a partial O being merged (padded rows)
  // the query rows stay in registers up to d = 80; at d = 128 they and the
  // accumulator would not both fit, so the rows are read from LDS
  constexpr bool QREG = D <= 80;
  __shared__ float Qs[QREG ? 1 : BM][D + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int qrow = qb * BM + lane;
  const bool qvalid = qrow < a.Nq;

  float qv[QREG ? D : 1], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    if constexpr (QREG) qv[i] = qvalid ? qp[(int64_t)qrow * a.qs.sn + i] : 0.f;
    acc[i] = 0.f;
  }
  if constexpr (!QREG) {
    for (int e = tid; e < BM * D; e += 64 * W) {
      const int r = e / D, cc = e % D;
      Qs[r][cc] = qb * BM + r < a.Nq ? qp[(int64_t)(qb * BM + r) * a.qs.sn + cc] : 0.f;
    }
  }
  auto qval = [&](int i) -> float {
    if constexpr (QREG) return qv[i];
    else return Qs[lane][i];
  };
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 < n_kv; j0 += BN) {
    __syncthreads();
    for (int e = tid; e < BN * D; e += 64 * W) {
      const int r = e / D, cc = e % D;
      const bool ok = j0 + r < n_kv;
      Ks[r][cc] = ok ? kp[(int64_t)(j0 + r) * a.ks.sn + cc] : 0.f;
      Vs[r][cc] = ok ? vp[(int64_t)(j0 + r) * a.vs.sn + cc] : 0.f;
    }
    __syncthreads();
    if (j0 + w * TB >= n_kv) continue;  // this wave's keys of the tile are all past the end
    float sc[TB];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int j = w * TB + t;
      float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < D; ++i) d4[i & 3] = fmaf(qval(i), Ks[j][i], d4[i & 3]);
      sc[t] = j0 + j < n_kv ? ((d4[0] + d4[1]) + (d4[2] + d4[3])) * a.scale : -INFINITY;
      mx = fmaxf(mx, sc[t]);
    }
    const float m_new = fmaxf(m, mx);  // finite: key w * TB of the tile exists
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= alpha;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const float p = expf(sc[t] - m_new);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(p, Vs[w * TB + t][i], acc[i]);
    }
    m = m_new;
  }
  // merge the waves' partials into wave 0, one wave at a time
  for (int r = 1; r < W; ++r) {
    __syncthreads();
    if (w == r) {
      Ms[lane] = m;
      Ls[lane] = l;
#pragma unroll
      for (int i = 0; i < D; ++i) Ab[lane][i] = acc[i];
    }
    __syncthreads();
    if (w == 0) {
      const float mo = Ms[lane];
      const float mn = fmaxf(m, mo);
      if (mn != -INFINITY) {  // both empty: nothing to merge
        const float a0 = expf(m - mn), a1 = expf(mo - mn);
        l = l * a0 + Ls[lane] * a1;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] = acc[i] * a0 + Ab[lane][i] * a1;
        m = mn;
      }
    }
  }
  if (w != 0 || !qvalid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (int64_t)c * a.o_chunk_stride + b * a.os.sb + h * a.os.sh +
                       (int64_t)qrow * a.os.sn;
  for (int i = 0; i < D; ++i) ((float*)a.o)[orow + i] = acc[i] * inv;
  const int64_t li = (int64_t)c * a.lse_chunk_stride + ((int64_t)b * a.H + h) * a.Nq + qrow;
  a.lse[li] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D, int QW>
static hipError_t fwd_bf16_d(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + 4 * QW - 1) / (4 * QW);
  const long long grid = (long long)nqb * a.H * a.B * a.n_chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.out_f32)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QW, true>), dim3((unsigned)grid), dim3(fwdk::NT), 0,
                       s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QW, false>), dim3((unsigned)grid), dim3(fwdk::NT), 0,
                       s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t s) {
  if (EXATTN_SHORT && a.n_chunks == 1 && short_slot(a.Nq, a.Nkv)) return launch_fwd_short(a, d, s);
  switch (d) {
    case 64: return fwd_bf16_d<64, 32>(a, s);
    case 80: return fwd_bf16_d<80, 32>(a, s);
    case 128: return fwd_bf16_d<128, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t fwd_f32_d(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + fwdf::BM - 1) / fwdf::BM;
  const long long grid = (long long)nqb * a.H * a.B * a.n_chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)grid), dim3(64 * fwdf::waves<D>()), 0, s,
                     a);
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

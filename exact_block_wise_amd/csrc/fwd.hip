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

// query rows per wave of the bf16 forward for d = 64 and d = 80
#ifndef EXATTN_FWD_QW64
#define EXATTN_FWD_QW64 32
#endif
#ifndef EXATTN_FWD_QW80
#define EXATTN_FWD_QW80 32
#endif
// occupancy request (waves per SIMD) of the bf16 forward for d = 64 (its
// registers then still fit three);
// d = 80 and 128 ask for two (three would spill)
#ifndef EXATTN_FWD_WAVES
#define EXATTN_FWD_WAVES 2
#endif

namespace exattn {

// --------------------------------------------------------------------------
// bf16 inputs, bf16 matrix cores (32x32x16), fp32 accumulation.
//
// Workgroup: 4 waves, each owning QW query rows (QW = 32 or 64).  Key/value
// tiles of 64 rows are staged in LDS row-major and double-buffered: the next
// tile's global loads are issued into registers before the current tile is
// computed and written to the other buffer after it, so one barrier per tile
// suffices and the load latency hides behind the matrix work.
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
constexpr float kSumCap = 256.0f;  // 2^kLazy
}  // namespace fwdk

template <int D>
struct FwdLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int KS = DP + 8;                // row stride of the K and V tiles
  static constexpr int tile = fwdk::BN * KS;        // elements per tile
  static constexpr int bytes = 4 * tile * 2;        // K, V x double buffer
};

// Weigh each tile against the running reference first and take the exact
// row maximum only when the weights come out too large (see the tile body).
#ifndef EXATTN_FWD_SUMCHECK
#define EXATTN_FWD_SUMCHECK 0
#endif

// Issue a tile's K operand reads in bulk ahead of its score products.
#ifndef EXATTN_FWD_KSTAGE
#define EXATTN_FWD_KSTAGE 0
#endif
// Stage key/value tiles with direct-to-LDS loads (one tile ahead, two LDS
// buffers) instead of through registers.
#ifndef EXATTN_FWD_DMA
#define EXATTN_FWD_DMA 1
#endif
// Prefetch depth in tiles when staging through registers: two where the
// second register set fits.
template <int D>
constexpr int fwd_prefetch() { return D <= 80 ? 2 : 1; }

template <int D, int QW, bool OUT_F32>
__global__ __launch_bounds__(fwdk::NT)
__attribute__((amdgpu_waves_per_eu(D == 64 ? EXATTN_FWD_WAVES : 2)))
void fwd_bf16_kernel(FwdArgs a) {
  using namespace fwdk;
  using L = FwdLds<D>;
  constexpr int DP = L::DP, NDB = DP / 32, KC = D / 16, KS = L::KS;
  constexpr int NQB = QW / 32;          // 32-row query blocks per wave
  constexpr int BM = 4 * QW;            // query rows per workgroup
  constexpr int CH = BN * (D / 8);      // 16-byte pieces per tile
  constexpr int PT = (CH + NT - 1) / NT;
  constexpr int PF = fwd_prefetch<D>();
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

  const int kv_lo = c * a.chunk_len;
  const int n_kv = max(0, min(a.Nkv, kv_lo + a.chunk_len) - kv_lo);
  const int ntiles = (n_kv + BN - 1) / BN;

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh + (int64_t)kv_lo * a.ks.sn;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh + (int64_t)kv_lo * a.vs.sn;

  const int q0 = qblk * BM + w * QW;
  const bool wave_active = q0 < a.Nq;

  // this wave's query rows as B operands: lane -> row q0 + 32 qb + ln,
  // d = 16 kc + 8 g .. +7 (rows past Nq read as zeros)
  bf16x8 qreg[NQB][KC];
  {
    const auto rq = rows_rsrc(qp + (int64_t)q0 * a.qs.sn, a.Nq - q0, 2 * a.qs.sn, 2 * D);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        qreg[qb][kc] = buffer_load_bf16x8(
            rq, (uint32_t)((32 * qb + ln) * 2 * a.qs.sn + 2 * (16 * kc + 8 * g)));
  }

  // Tile loader with two register sets.  With PF = 2, tile t goes global ->
  // set t % 2 (issued two tiles ahead) -> LDS buffer t % 2 (stored one tile
  // ahead), so each load has two tiles of work to land; with PF = 1 the load
  // is issued one tile ahead.  Piece e -> row e / (D/8), 16-byte column piece
  // e % (D/8).  The loads are unconditional buffer loads (rows past the end
  // come back as zeros), so no branch separates a load from its use and the
  // waits before the LDS stores cover only the tile being stored.
  uint32_t koff[PT], voff[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = tid + u * NT;
    const int r = e / (D / 8), cc = e % (D / 8);
    koff[u] = (uint32_t)(r * 2 * a.ks.sn + 16 * cc);
    voff[u] = (uint32_t)(r * 2 * a.vs.sn + 16 * cc);
  }
  bf16x8 pk[2][PT], pv[2][PT];
  auto load_tile = [&](auto set_tag, int j0) {
    constexpr int S = decltype(set_tag)::value;
    const auto rk = rows_rsrc(kp + (int64_t)j0 * a.ks.sn, n_kv - j0, 2 * a.ks.sn, 2 * D);
    const auto rv = rows_rsrc(vp + (int64_t)j0 * a.vs.sn, n_kv - j0, 2 * a.vs.sn, 2 * D);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      pk[S][u] = buffer_load_bf16x8(rk, koff[u]);
      pv[S][u] = buffer_load_bf16x8(rv, voff[u]);
    }
  };
  auto store_tile = [&](auto set_tag, int buf) {
    constexpr int S = decltype(set_tag)::value;
    bf16* Kt = lds + buf * 2 * L::tile;
    bf16* Vt = Kt + L::tile;
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int e = tid + u * NT;
      if (CH % NT == 0 || e < CH) {
        const int r = e / (D / 8), cc = e % (D / 8);
        *reinterpret_cast<bf16x8*>(&Kt[r * KS + 8 * cc]) = pk[S][u];
        *reinterpret_cast<bf16x8*>(&Vt[r * KS + 8 * cc]) = pv[S][u];
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // direct-to-LDS staging (see LdsTileDma): one tile ahead, no registers
  LdsTileDma<D, KS, BN> tk, tv;
  if constexpr (EXATTN_FWD_DMA) {
    tk.init(w, lane, a.ks.sn);
    tv.init(w, lane, a.vs.sn);
  }
  auto load_tile_dma = [&](int j0, int buf) {
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
  // guarantees that tile it + PF exists to be loaded and tile it + 1 to be
  // stored, and that tile it is full: the body then has no condition, no
  // masking and no branch between loads and their waits.  The last tiles
  // (TAIL true) test both at run time and mask keys past the end.
  // With PF = 2 the register set SET = it % 2 receives tile it + 2 and LDS
  // buffer SET is read; with PF = 1 a single register set is used and the
  // buffer alternates at run time.
  auto tile = [&](auto tail_tag, auto set_tag, int it) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    constexpr int SET = decltype(set_tag)::value;
    using LoadSet = std::integral_constant<int, PF == 2 ? SET : 0>;
    using StoreSet = std::integral_constant<int, PF == 2 ? 1 - SET : 0>;
    // two-set register staging: buffer SET; otherwise (one set, or direct
    // staging) the buffer alternates with the tile
    const int buf = (PF == 2 && !EXATTN_FWD_DMA) ? SET : (it & 1);
    const int j0 = it * BN;
    if constexpr (EXATTN_FWD_DMA) {
      if (!TAIL || it + 1 < ntiles) load_tile_dma(j0 + BN, buf ^ 1);
    } else {
      if (!TAIL || it + PF < ntiles) load_tile(LoadSet{}, j0 + PF * BN);
    }
    if (wave_active) {
      const bf16* Kt = lds + buf * 2 * L::tile;
      const bf16* Vt = Kt + L::tile;
      f32x16 s[2][NQB];
      // S^T = K Q^T for two 32-key blocks x NQB query blocks; keys past the
      // end weigh nothing
      auto scores = [&]() {
        prio_mfma();
        if constexpr (EXATTN_FWD_KSTAGE) {
          // all K operand reads of the tile first, then the products
          bf16x8 ka[2][KC];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
              ka[cb][kc] = load_bf16x8(&Kt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) s[cb][qb] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
#pragma unroll
              for (int qb = 0; qb < NQB; ++qb) s[cb][qb] = mfma32(ka[cb][kc], qreg[qb][kc], s[cb][qb]);
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) s[cb][qb] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
              const bf16x8 ka = load_bf16x8(&Kt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
#pragma unroll
              for (int qb = 0; qb < NQB; ++qb) s[cb][qb] = mfma32(ka, qreg[qb][kc], s[cb][qb]);
            }
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
      auto weights = [&](float* psum) {
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
      // raise the reference to the rows' maxima over this tile (when higher),
      // rescaling what O and l hold so far
      auto raise_reference = [&](const float* mx) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float mnew = fmaxf(mref[qb], mx[qb]);
          const float alpha = fast_exp2((mref[qb] - mnew) * sl2);
          mref[qb] = mnew;
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
        }
      };
      auto row_max = [&](float* mx) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float m = s[0][qb][0];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, s[cb][qb][e]);
          mx[qb] = max_halves(m);
        }
      };
      float psum[NQB], mx[NQB];
      scores();
      if constexpr (EXATTN_FWD_SUMCHECK) {
        // Optimistic: weigh against the current reference and check the
        // lane sums afterwards.  A sum within 2^kLazy bounds every weight by
        // 2^kLazy; a larger sum (or inf / NaN: the reference is -inf before
        // the first tile) sends the wave through the exact path once: the
        // scores are recomputed, the reference is raised to their maximum
        // and the weights are taken again.  This drops the per-tile row
        // maximum from the common path.
        weights(psum);
        bool low = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) low |= !(psum[qb] <= kSumCap);
        if (__builtin_amdgcn_ballot_w64(low)) {
          // re-read K from LDS rather than keep the fast path's operands live
          asm volatile("" ::: "memory");
          scores();
          row_max(mx);
          raise_reference(mx);
          weights(psum);
        }
      } else {
        // row maxima; raise the reference only when it is exceeded by > 2^8
        row_max(mx);
        bool raise = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) raise |= mx[qb] > mref[qb] + lazy;
        if (__builtin_amdgcn_ballot_w64(raise)) raise_reference(mx);
        weights(psum);
      }
      // O^T += V^T P^T over four 16-key chunks.  Chunk t = 2 cb + hh holds,
      // for slot group g, keys 16t + 4g + (0..3) and 16t + 8 + 4g + (0..3):
      // accumulator entries 8hh .. 8hh+7 of block cb.
      bf16x8 pb[4][NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        lsum[qb] += psum[qb];
#pragma unroll
        for (int t = 0; t < 4; ++t) pb[t][qb] = acc_half_to_bf16(s[t >> 1][qb], t & 1);
      }
      prio_mfma();
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 va = tr_operand(Vt + 32 * db, KS, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) oacc[db][qb] = mfma32(va, pb[t][qb], oacc[db][qb]);
        }
      }
      prio_valu();
    }
    if constexpr (EXATTN_FWD_DMA) {
      wait_vmem();
    } else {
      if (!TAIL || it + 1 < ntiles) store_tile(StoreSet{}, buf ^ 1);
    }
    __syncthreads();
  };
  // (an empty key range skips the loop; the wait bookkeeping of the loop
  // then only ever sees the prologue's loads completed)
  if (ntiles > 0) {
    if constexpr (EXATTN_FWD_DMA) {
      load_tile_dma(0, 0);
      wait_vmem();
    } else {
      load_tile(S0{}, 0);
      store_tile(S0{}, 0);
      if (PF == 2 && ntiles > 1) load_tile(S1{}, BN);
    }
    __syncthreads();
    int it = 0;
    if constexpr (PF == 2 && !EXATTN_FWD_DMA) {
      // steady state: tiles it and it + 1 both have a tile to prefetch
      for (; it + 3 < ntiles; it += 2) {
        tile(std::false_type{}, S0{}, it);
        tile(std::false_type{}, S1{}, it + 1);
      }
      // the last two or three tiles; `it` is even here
      for (; it < ntiles; it += 2) {
        tile(std::true_type{}, S0{}, it);
        if (it + 1 < ntiles) tile(std::true_type{}, S1{}, it + 1);
      }
    } else {
      for (; it + 1 < ntiles; ++it) tile(std::false_type{}, S0{}, it);
      tile(std::true_type{}, S0{}, it);
    }
  }

  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float l = sum_halves(lsum[qb]);
    const int qrow = q0 + 32 * qb + ln;
    if (qrow >= a.Nq) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t orow = (int64_t)c * a.o_chunk_stride + b * a.os.sb + h * a.os.sh +
                         (int64_t)qrow * a.os.sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * g;
        if (d0 < D) {
          const f32x16& o = oacc[db][qb];
          if constexpr (OUT_F32) {
            f32x4 v4 = {o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv,
                        o[4 * i + 3] * inv};
            *reinterpret_cast<f32x4*>((float*)a.o + orow + d0) = v4;
          } else {
            bf16x4 v4 = {(bf16)(o[4 * i] * inv), (bf16)(o[4 * i + 1] * inv),
                         (bf16)(o[4 * i + 2] * inv), (bf16)(o[4 * i + 3] * inv)};
            *reinterpret_cast<bf16x4*>((bf16*)a.o + orow + d0) = v4;
          }
        }
      }
    }
    if (g == 0) {
      const int64_t li = (int64_t)c * a.lse_chunk_stride + ((int64_t)b * a.H + h) * a.Nq + qrow;
      a.lse[li] = l > 0.f ? (mref[qb] * sl2 + log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

// --------------------------------------------------------------------------
// bf16 forward, software-pipelined (d = 64, 80).
//
// Same workgroup shape as fwd_bf16_kernel (4 waves x 32 query rows), but
// each wave overlaps the matrix and vector work of consecutive tiles:
//   step a:  S_{j+1} = K_{j+1} Q^T         ||  P_j = exp2(S_j - m), sums, cvt
//   step b:  O^T += V_j^T P_j^T            ||  max of S_{j+1}, rescale test
//   step c:  (rare) rescale O and l after PV_j, raise the reference for j+1
// Steps a and b are single branch-free regions in which scheduling hints
// alternate matrix instructions with vector instructions.  K is needed one
// tile ahead of V, so LDS holds three K slots and two V slots; the pair
// (K_{j+2}, V_{j+1}) is loaded during iteration j and stored at its end.
// --------------------------------------------------------------------------
#ifndef EXATTN_FWD_SP
#define EXATTN_FWD_SP 0
#endif
#ifndef EXATTN_SP_HINTS
#define EXATTN_SP_HINTS 1
#endif

namespace spk {
constexpr int BN = 64;
constexpr int NT = 256;
constexpr int QW = 32;
constexpr int BM = 4 * QW;
}  // namespace spk

template <int D>
struct SpLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int KS = DP + 8;
  static constexpr int tile = spk::BN * KS;
  static constexpr int bytes = 5 * tile * 2;  // K x 3 slots, V x 2 slots
};

template <int D, bool OUT_F32>
__global__ __launch_bounds__(spk::NT) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_sp_kernel(FwdArgs a) {
  using namespace spk;
  using L = SpLds<D>;
  constexpr int DP = L::DP, NDB = DP / 32, KC = D / 16, KS = L::KS;
  constexpr int CH = BN * (D / 8);
  constexpr int PT = (CH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16 lds[5 * L::tile];
  bf16* const Kslot = lds;                  // [3][tile]
  bf16* const Vslot = lds + 3 * L::tile;    // [2][tile]

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

  const int kv_lo = c * a.chunk_len;
  const int n_kv = max(0, min(a.Nkv, kv_lo + a.chunk_len) - kv_lo);
  const int ntiles = (n_kv + BN - 1) / BN;
  const bool ragged = (n_kv % BN) != 0;

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh + (int64_t)kv_lo * a.ks.sn;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh + (int64_t)kv_lo * a.vs.sn;

  const int q0 = qblk * BM + w * QW;
  const bool wave_active = q0 < a.Nq;
  const int qrow = q0 + ln;
  bf16x8 qreg[KC];
  {
    const auto rq = rows_rsrc(qp + (int64_t)q0 * a.qs.sn, a.Nq - q0, 2 * a.qs.sn, 2 * D);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qreg[kc] = buffer_load_bf16x8(rq, (uint32_t)(ln * 2 * a.qs.sn + 2 * (16 * kc + 8 * g)));
  }

  // unconditional buffer loads of a tile's rows (rows past the end are zero)
  bf16x8 pk[PT], pv[PT];
  auto load_rows = [&](const bf16* base, int64_t sn, int j0, bf16x8* dst) {
    const auto r = rows_rsrc(base + (int64_t)j0 * sn, n_kv - j0, 2 * sn, 2 * D);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int e = tid + u * NT;
      dst[u] = buffer_load_bf16x8(r, (uint32_t)((e / (D / 8)) * 2 * sn + 16 * (e % (D / 8))));
    }
  };
  auto store_rows = [&](bf16* slot, const bf16x8* src) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int e = tid + u * NT;
      if (CH % NT == 0 || e < CH) {
        const int r = e / (D / 8), cc = e % (D / 8);
        *reinterpret_cast<bf16x8*>(&slot[r * KS + 8 * cc]) = src[u];
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  f32x16 scur[2], snxt[2];
  float mref = -INFINITY, lsum = 0.f;
  const float sl2 = a.scale * kLog2e;
  const float lazy = fwdk::kLazy / sl2;

  auto scores = [&](int j, f32x16* sdst) {
    const bf16* Kt = Kslot + (j % 3) * L::tile;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      sdst[cb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8 ka = load_bf16x8(&Kt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
        sdst[cb] = mfma32(ka, qreg[kc], sdst[cb]);
      }
    }
  };
  auto mask = [&](int j, f32x16* sv) {
    const int j0 = j * BN;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (j0 + 32 * cb + 8 * (e >> 2) + 4 * g + (e & 3) >= n_kv) sv[cb][e] = -INFINITY;
  };
  auto rowmax = [&](const f32x16* sv) {
    float m = sv[0][0];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, sv[cb][e]);
    return max_halves(m);
  };
  // (rare) raise the reference to mx; O and l hold tiles up to the current one
  auto raise_ref = [&](float mx) {
    const float mnew = fmaxf(mref, mx);
    const float alpha = fast_exp2((mref - mnew) * sl2);
    mref = mnew;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
  };

  // iteration j; NEXT: tile j + 1 exists, MASKN: it is the ragged last tile;
  // TAIL: K_{j+2} / V_{j+1} may not exist (tested at run time), otherwise
  // both are loaded and stored unconditionally
  auto iteration = [&](auto next_tag, auto maskn_tag, auto tail_tag, int j) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool MASKN = decltype(maskn_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;
    if (!TAIL || j + 2 < ntiles) load_rows(kp, a.ks.sn, (j + 2) * BN, pk);
    if (!TAIL || j + 1 < ntiles) load_rows(vp, a.vs.sn, (j + 1) * BN, pv);
    if (wave_active) {
      // step a: S_{j+1} || softmax of S_j.  The K operands are read first,
      // so that the products need no LDS wait once they start.
      bf16x8 ka[2][KC];
      if constexpr (NEXT) {
        const bf16* Kt = Kslot + ((j + 1) % 3) * L::tile;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            ka[cb][kc] = load_bf16x8(&Kt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NEXT) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          snxt[cb] = f32x16{};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) snxt[cb] = mfma32(ka[cb][kc], qreg[kc], snxt[cb]);
        }
      }
      const float moff = mref * sl2;
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(fmaf(scur[cb][e], sl2, -moff));
          scur[cb][e] = p;
          part[e & 3] += p;
        }
      lsum += (part[0] + part[1]) + (part[2] + part[3]);
      bf16x8 pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) pb[t] = acc_half_to_bf16(scur[t >> 1], t & 1);
      if constexpr (EXATTN_SP_HINTS && NEXT) {
#pragma unroll
        for (int k = 0; k < 2 * KC; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // a product
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // vector work
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // step b: PV_j || maximum of S_{j+1}
      const bf16* Vt = Vslot + (j & 1) * L::tile;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 va = tr_operand(Vt + 32 * db, KS, 16 * t + 4 * g, 16 * t + 8 + 4 * g, lane);
          oacc[db] = mfma32(va, pb[t], oacc[db]);
        }
      float mx = 0.f;
      if constexpr (NEXT) {
        if constexpr (MASKN) mask(j + 1, snxt);
        mx = rowmax(snxt);
      }
      if constexpr (EXATTN_SP_HINTS) {
#pragma unroll
        for (int k = 0; k < 4 * NDB; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // step c: rare rescale, after PV_j is in O
      if constexpr (NEXT) {
        if (__builtin_amdgcn_ballot_w64(mx > mref + lazy)) raise_ref(mx);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) scur[cb] = snxt[cb];
      }
    }
    if (!TAIL || j + 2 < ntiles) store_rows(Kslot + ((j + 2) % 3) * L::tile, pk);
    if (!TAIL || j + 1 < ntiles) store_rows(Vslot + ((j + 1) & 1) * L::tile, pv);
    __syncthreads();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (ntiles > 0) {
    // prologue: K_0, K_1, V_0 in LDS; S_0 and its reference maximum
    load_rows(kp, a.ks.sn, 0, pk);
    store_rows(Kslot, pk);
    load_rows(vp, a.vs.sn, 0, pv);
    store_rows(Vslot, pv);
    if (ntiles > 1) {
      load_rows(kp, a.ks.sn, BN, pk);
      store_rows(Kslot + L::tile, pk);
    }
    __syncthreads();
    if (wave_active) {
      scores(0, scur);
      if (ntiles == 1 && ragged) mask(0, scur);
      raise_ref(rowmax(scur));
    }
    int j = 0;
    for (; j + 2 < ntiles; ++j) iteration(T_{}, F_{}, F_{}, j);
    if (j + 1 < ntiles) {
      if (ragged)
        iteration(T_{}, T_{}, T_{}, j);
      else
        iteration(T_{}, F_{}, T_{}, j);
      ++j;
    }
    iteration(F_{}, F_{}, T_{}, j);
  }

  if (!wave_active) return;
  const float l = sum_halves(lsum);
  if (qrow >= a.Nq) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (int64_t)c * a.o_chunk_stride + b * a.os.sb + h * a.os.sh +
                       (int64_t)qrow * a.os.sn;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * g;
      if (d0 < D) {
        const f32x16& o = oacc[db];
        if constexpr (OUT_F32) {
          f32x4 v4 = {o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv, o[4 * i + 3] * inv};
          *reinterpret_cast<f32x4*>((float*)a.o + orow + d0) = v4;
        } else {
          bf16x4 v4 = {(bf16)(o[4 * i] * inv), (bf16)(o[4 * i + 1] * inv),
                       (bf16)(o[4 * i + 2] * inv), (bf16)(o[4 * i + 3] * inv)};
          *reinterpret_cast<bf16x4*>((bf16*)a.o + orow + d0) = v4;
        }
      }
    }
  }
  if (g == 0) {
    const int64_t li = (int64_t)c * a.lse_chunk_stride + ((int64_t)b * a.H + h) * a.Nq + qrow;
    a.lse[li] = l > 0.f ? (mref * sl2 + log2f(l)) * kLn2 : -INFINITY;
  }
}

// --------------------------------------------------------------------------
// bf16 forward, ping-pong variant for long query sequences (d = 64, 80).
//
// Workgroup: 8 waves in two groups of four; wave w and wave w + 4 share a
// SIMD (group = w / 4 by default).  Each wave owns 32 query rows (256 per
// workgroup).  Per tile, a wave runs a matrix phase M(j) -- S_j = K_j Q^T
// and O^T += V_{j-1}^T P_{j-1}^T -- and a vector phase V(j) -- maximum, lazy
// rescale, P_j = exp2(S_j - m), row sums.  Group 1 runs one phase behind
// group 0, and a barrier separates phases, so on every SIMD one wave's
// matrix instructions overlap the other wave's vector instructions.
//
// LDS holds two K slots and two V slots.  Around phase step 2t all waves
// store K_{t+1} (slot (t+1) % 2) and V_t (slot t % 2) from registers loaded
// one tile earlier: K_j is read in steps 2j, 2j+1 and V_j in 2j+2, 2j+3, so a
// slot is rewritten only after both groups are done with it.
// --------------------------------------------------------------------------
#ifndef EXATTN_PP_GROUP_BY_HALF
#define EXATTN_PP_GROUP_BY_HALF 1
#endif

namespace ppk {
constexpr int BN = 64;
constexpr int NT = 512;
constexpr int QW = 32;
constexpr int BM = 8 * QW;
}  // namespace ppk

template <int D>
struct PpLds {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int KS = DP + 8;
  static constexpr int tile = ppk::BN * KS;
  static constexpr int bytes = 4 * tile * 2;  // K x 2 slots, V x 2 slots
};

template <int D, bool OUT_F32>
__global__ __launch_bounds__(ppk::NT) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_pp_kernel(FwdArgs a) {
  using namespace ppk;
  using L = PpLds<D>;
  constexpr int DP = L::DP, NDB = DP / 32, KC = D / 16, KS = L::KS;
  constexpr int CH = BN * (D / 8);
  constexpr int PT = (CH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16 lds[4 * L::tile];
  bf16* const Kslot = lds;                  // [2][tile]
  bf16* const Vslot = lds + 2 * L::tile;    // [2][tile]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31, g = lane >> 5;
  const int grp = EXATTN_PP_GROUP_BY_HALF ? (w >> 2) : (w & 1);

  const int nqb = (a.Nq + BM - 1) / BM;
  int idx = xcd_remap(blockIdx.x, gridDim.x);
  const int qblk = idx % nqb;
  idx /= nqb;
  const int h = idx % a.H;
  const int b = idx / a.H;
  const int n_kv = a.Nkv;
  const int ntiles = (n_kv + BN - 1) / BN;

  const bf16* qp = (const bf16*)a.q + b * a.qs.sb + h * a.qs.sh;
  const bf16* kp = (const bf16*)a.k + b * a.ks.sb + h * a.ks.sh;
  const bf16* vp = (const bf16*)a.v + b * a.vs.sb + h * a.vs.sh;

  const int q0 = qblk * BM + w * QW;
  const bool wave_active = q0 < a.Nq;
  const int qrow = q0 + ln;

  bf16x8 qreg[KC];
  {
    const auto rq = rows_rsrc(qp + (int64_t)q0 * a.qs.sn, a.Nq - q0, 2 * a.qs.sn, 2 * D);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qreg[kc] = buffer_load_bf16x8(rq, (uint32_t)(ln * 2 * a.qs.sn + 2 * (16 * kc + 8 * g)));
  }

  // prefetch registers for one (K_{t+1}, V_t) pair; unconditional buffer
  // loads (rows past the end are zero)
  bf16x8 pk[PT], pv[PT];
  auto load_rows = [&](const bf16* base, int64_t sn, int j0, bf16x8* dst) {
    const auto r = rows_rsrc(base + (int64_t)j0 * sn, n_kv - j0, 2 * sn, 2 * D);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int e = tid + u * NT;
      dst[u] = buffer_load_bf16x8(r, (uint32_t)((e / (D / 8)) * 2 * sn + 16 * (e % (D / 8))));
    }
  };
  auto store_rows = [&](bf16* slot, const bf16x8* src) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int e = tid + u * NT;
      if (CH % NT == 0 || e < CH) {
        const int r = e / (D / 8), cc = e % (D / 8);
        *reinterpret_cast<bf16x8*>(&slot[r * KS + 8 * cc]) = src[u];
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  f32x16 s[2];
  bf16x8 pb[4];
  float mref = -INFINITY, lsum = 0.f;
  const float sl2 = a.scale * kLog2e;
  const float lazy = fwdk::kLazy / sl2;

  // matrix phase M(t): S_t (when t < ntiles) and PV of tile t - 1 (t >= 1)
  auto mphase = [&](int t) __attribute__((always_inline)) {
    if (t < ntiles) {
      const bf16* Kt = Kslot + (t & 1) * L::tile;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        s[cb] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const bf16x8 ka = load_bf16x8(&Kt[(32 * cb + ln) * KS + 16 * kc + 8 * g]);
          s[cb] = mfma32(ka, qreg[kc], s[cb]);
        }
      }
    }
    if (t >= 1) {
      const bf16* Vt = Vslot + ((t - 1) & 1) * L::tile;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 va = tr_operand(Vt + 32 * db, KS, 16 * u + 4 * g, 16 * u + 8 + 4 * g, lane);
          oacc[db] = mfma32(va, pb[u], oacc[db]);
        }
    }
  };
  // vector phase V(t): P_t from S_t (keys past the end masked)
  auto vphase = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * BN;
    if (j0 + BN > n_kv) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (j0 + 32 * cb + 8 * (e >> 2) + 4 * g + (e & 3) >= n_kv) s[cb][e] = -INFINITY;
    }
    float m = s[0][0];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, s[cb][e]);
    const float mx = max_halves(m);
    if (__builtin_amdgcn_ballot_w64(mx > mref + lazy)) {
      const float mnew = fmaxf(mref, mx);
      const float alpha = fast_exp2((mref - mnew) * sl2);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    const float moff = mref * sl2;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(fmaf(s[cb][e], sl2, -moff));
        s[cb][e] = p;
        part[e & 3] += p;
      }
    lsum += (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
    for (int u = 0; u < 4; ++u) pb[u] = acc_half_to_bf16(s[u >> 1], u & 1);
  };

  // Step pair t: the even step stores the pair (K_{t+1}, V_t) loaded one pair
  // earlier and loads (K_{t+2}, V_{t+1}); group 0 runs M(t) then V(t),
  // group 1 runs V(t - 1) then M(t), so on every SIMD one wave multiplies
  // while the other exponentiates.  In the steady state (TAIL false) all
  // four tiles exist and every phase runs; the last pairs test at run time.
  const bool g0 = grp == 0;
  auto pair = [&](auto tail_tag, int t) __attribute__((always_inline)) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    if (!TAIL || t + 1 < ntiles) store_rows(Kslot + ((t + 1) & 1) * L::tile, pk);
    if (!TAIL || t < ntiles) store_rows(Vslot + (t & 1) * L::tile, pv);
    if (!TAIL || t + 2 < ntiles) load_rows(kp, a.ks.sn, (t + 2) * BN, pk);
    if (!TAIL || t + 1 < ntiles) load_rows(vp, a.vs.sn, (t + 1) * BN, pv);
    if (wave_active) {
      if (g0) {
        if (!TAIL || t <= ntiles) mphase(t);
      } else {
        if (!TAIL || (t >= 1 && t - 1 < ntiles)) vphase(t - 1);
      }
    }
    __syncthreads();
    if (wave_active) {
      if (g0) {
        if (!TAIL || t < ntiles) vphase(t);
      } else {
        if (!TAIL || t <= ntiles) mphase(t);
      }
    }
    __syncthreads();
  };

  // prologue: K_0 into its slot, the pair (K_1, V_0) into registers
  load_rows(kp, a.ks.sn, 0, pk);
  store_rows(Kslot, pk);
  load_rows(kp, a.ks.sn, BN, pk);
  load_rows(vp, a.vs.sn, 0, pv);
  __syncthreads();
  // pair 0 has no V(-1) / PV(-1); pairs 1 .. ntiles - 3 are the steady
  // state; the rest (through pair ntiles, which only finishes PV) are tails
  pair(std::true_type{}, 0);
  int t = 1;
  for (; t + 2 < ntiles; ++t) pair(std::false_type{}, t);
  for (; t <= ntiles; ++t) pair(std::true_type{}, t);

  if (!wave_active) return;
  const float l = sum_halves(lsum);
  if (qrow >= a.Nq) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = b * a.os.sb + h * a.os.sh + (int64_t)qrow * a.os.sn;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * g;
      if (d0 < D) {
        const f32x16& o = oacc[db];
        if constexpr (OUT_F32) {
          f32x4 v4 = {o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv, o[4 * i + 3] * inv};
          *reinterpret_cast<f32x4*>((float*)a.o + orow + d0) = v4;
        } else {
          bf16x4 v4 = {(bf16)(o[4 * i] * inv), (bf16)(o[4 * i + 1] * inv),
                       (bf16)(o[4 * i + 2] * inv), (bf16)(o[4 * i + 3] * inv)};
          *reinterpret_cast<bf16x4*>((bf16*)a.o + orow + d0) = v4;
        }
      }
    }
  }
  if (g == 0) {
    const int64_t li = ((int64_t)b * a.H + h) * a.Nq + qrow;
    a.lse[li] = l > 0.f ? (mref * sl2 + log2f(l)) * kLn2 : -INFINITY;
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

#ifndef EXATTN_FWD_PP
#define EXATTN_FWD_PP 0
#endif

template <int D>
static hipError_t fwd_pp_d(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + ppk::BM - 1) / ppk::BM;
  const long long grid = (long long)nqb * a.H * a.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.out_f32)
    hipLaunchKernelGGL((fwd_pp_kernel<D, true>), dim3((unsigned)grid), dim3(ppk::NT), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_pp_kernel<D, false>), dim3((unsigned)grid), dim3(ppk::NT), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t fwd_sp_d(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + spk::BM - 1) / spk::BM;
  const long long grid = (long long)nqb * a.H * a.B * a.n_chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.out_f32)
    hipLaunchKernelGGL((fwd_sp_kernel<D, true>), dim3((unsigned)grid), dim3(spk::NT), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_sp_kernel<D, false>), dim3((unsigned)grid), dim3(spk::NT), 0, s, a);
  return hipGetLastError();
}

template <int D, int QW>
static hipError_t fwd_bf16_d(const FwdArgs& a, hipStream_t s) {
  if constexpr (D <= 80) {
    if (EXATTN_FWD_SP) return fwd_sp_d<D>(a, s);
    // long query sequences, one key/value range: the ping-pong kernel
    if (EXATTN_FWD_PP && a.n_chunks == 1 && a.Nq >= ppk::BM) return fwd_pp_d<D>(a, s);
  }
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
    case 64: return fwd_bf16_d<64, EXATTN_FWD_QW64>(a, s);
    case 80: return fwd_bf16_d<80, EXATTN_FWD_QW80>(a, s);
    case 128: return fwd_bf16_d<128, 32>(a, s);
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

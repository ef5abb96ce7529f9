// Short sequences (bf16): Nq, Nkv <= 32.
//
// Divided space-time attention runs attention separately over the t frames
// of every spatial position (temporal) and over the h*w positions of every
// frame (spatial): huge batches of short sequences ("Video Transformer" of
// "Training a Large Video Model on a Single Machine in a Day" contrasts it
// with joint space-time attention; the NeMo video-model page's Table 2 lists
// the temporal (b*h*w, t, d) and spatial (b*t, h*w, d) layers).  A tile
// built for long sequences would leave almost all of its rows empty at
// t = 8, so here one wave owns a 32-row tile that holds 32 / S sequences of
// S slots each (S = 8, 16 or 32, the smallest that holds Nq and Nkv).  The
// products run on the whole 32 x 32 tile and scores across sequences are
// masked off, i.e. each sequence's exact softmax over its own keys.
//
// These shapes are bound by HBM traffic (a few flops per byte), so the
// kernels aim at one pass over the tensors: operand rows are loaded straight
// from global memory into registers (one row per lane), and only the tiles
// that must be read transposed (V in the forward; K, Q, dO in the backward)
// go through LDS.  One wave per workgroup; no barrier.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace exattn {

namespace shortk {
constexpr int ROWS = 32;  // rows of a wave's tile (query side and key side)
}  // namespace shortk

// Row r of a tile belongs to problem x = seq0 + r / S (a flat b*H + h
// index) at slot r % S.  A lane holds one row; Row describes it.
template <int S>
struct ShortRow {
  bool ok;     // the problem exists
  int b, h, pos;
  SeqSpan sp;  // its rows (dense, or a packed variable-length sequence)
  template <typename Args>
  __device__ __forceinline__ ShortRow(const Args& a, int seq0, int r) {
    const int x = seq0 + r / S;
    ok = x < a.B * a.H;
    b = ok ? x / a.H : 0;
    h = ok ? x % a.H : 0;
    pos = r % S;
    sp = seq_span(a, b, h);
  }
  __device__ __forceinline__ bool q_ok() const { return ok && pos < sp.nq; }
  __device__ __forceinline__ bool kv_ok() const { return ok && pos < sp.nkv; }
  __device__ __forceinline__ int64_t q_off(const Strides& st) const {
    return (int64_t)b * st.sb + (int64_t)h * st.sh + (int64_t)(sp.q_row0 + pos) * st.sn;
  }
  __device__ __forceinline__ int64_t kv_off(const Strides& st) const {
    return (int64_t)b * st.sb + (int64_t)h * st.sh + (int64_t)(sp.kv_row0 + pos) * st.sn;
  }
  __device__ __forceinline__ int64_t stat() const { return sp.stat0 + pos; }
};

// One row per lane as matrix-core operands: lane (l % 32, g = l / 32) holds
// d = 16 kc + 8 g .. +7 of its row for each kc (zeros when !ok).  The zeros
// are written first and the loads go out under one condition: a select of
// each loaded piece would use it at once and make every call wait for its
// own loads.
template <int KC>
__device__ __forceinline__ void load_row_operands(bf16x8 (&dst)[KC], const bf16* row, bool ok,
                                                  int g) {
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) dst[kc] = bf16x8{};
  if (ok) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) dst[kc] = load_bf16x8(row + 16 * kc + 8 * g);
  }
}

// The same pieces into a row-major LDS tile (row stride RS), for transpose
// reads; with d = 80 the columns 80..95 stay unwritten and only feed output
// rows d >= 80, which are never stored.
template <int KC, int RS>
__device__ __forceinline__ void stage_rows(bf16* tile, const bf16x8 (&src)[KC], int ln, int g) {
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    *reinterpret_cast<bf16x8*>(&tile[ln * RS + 16 * kc + 8 * g]) = src[kc];
}

// LDS writes of this wave are complete before its transpose reads
__device__ __forceinline__ void lds_written() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D>
struct ShortDims {
  static constexpr int KC = D / 16, NDB = (D + 31) / 32, DP = NDB * 32, RS = DP + 8;
  static constexpr int tile = shortk::ROWS * RS;  // bf16 elements
};

// --------------------------------------------------------------------------
// Forward.  S^T = K Q^T (lane: one query column, accumulator entry 4i + r:
// key row 8i + 4g + r), masked to the query's own sequence and its first
// Nkv slots; then the row maximum and sum over the lane and its partner
// lane l ^ 32, P^T in bf16, and O^T = V^T P^T with V^T read from LDS.
// --------------------------------------------------------------------------
template <int D, int S, bool OUT_F32>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D <= 80 ? 6 : 3)))
void fwd_short_kernel(FwdArgs a) {
  using Dm = ShortDims<D>;
  constexpr int KC = Dm::KC, NDB = Dm::NDB, RS = Dm::RS;
  constexpr int P = shortk::ROWS / S;
  __shared__ __attribute__((aligned(16))) bf16 vt[Dm::tile];
  __shared__ int64_t roff[shortk::ROWS];  // output row offsets (staged stores)
  const int lane = threadIdx.x, ln = lane & 31, g = lane >> 5;
  const ShortRow<S> row(a, (int)blockIdx.x * P, ln);  // this lane's query and key row

  const bool rq = row.q_ok(), rk = row.kv_ok();
  bf16x8 qb[KC], ka[KC], vr[KC];
  load_row_operands(qb, (const bf16*)a.q + row.q_off(a.qs), rq, g);
  load_row_operands(ka, (const bf16*)a.k + row.kv_off(a.ks), rk, g);
  load_row_operands(vr, (const bf16*)a.v + row.kv_off(a.vs), rk, g);
  stage_rows<KC, RS>(vt, vr, ln, g);

  f32x16 s = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) s = mfma32(ka[kc], qb[kc], s);

  // keys of this query's sequence among the lane's entries
  const int c = ln;
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int kr = 8 * (e >> 2) + 4 * g + (e & 3);
    const bool ok = kr / S == c / S && kr % S < row.sp.nkv;
    s[e] = ok ? s[e] : -INFINITY;
    m = fmaxf(m, s[e]);
  }
  m = max_halves(m);
  const float sl2 = a.scale * kLog2e;
  const float moff = m == -INFINITY ? 0.f : m * sl2;  // a query without keys: O = 0
  float l = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    s[e] = fast_exp2(fmaf(s[e], sl2, -moff));
    l += s[e];
  }
  l = sum_halves(l);

  lds_written();
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const bf16x8 pb = acc_half_to_bf16(s, h2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16x8 va = tr_operand(vt + 32 * db, RS, 16 * h2 + 4 * g, 16 * h2 + 8 + 4 * g, lane);
      o[db] = mfma32(va, pb, o[db]);
    }
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;  // l >= 1 when the query has keys
  if constexpr (OUT_F32) {
    if (!rq) return;
    const int64_t orow = row.q_off(a.os);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * g;
        if (d0 >= D) continue;
        const f32x4 v4 = {o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                          o[db][4 * i + 3] * inv};
        *reinterpret_cast<f32x4*>((float*)a.o + orow + d0) = v4;
      }
  } else {
    // a lane holds runs of 4 d of its query row: through the V tile (its
    // transpose reads are done) and out as whole rows
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * g;
        if (d0 >= D) continue;
        const bf16x4 v4 = {(bf16)(o[db][4 * i] * inv), (bf16)(o[db][4 * i + 1] * inv),
                           (bf16)(o[db][4 * i + 2] * inv), (bf16)(o[db][4 * i + 3] * inv)};
        *reinterpret_cast<bf16x4*>(&vt[ln * RS + d0]) = v4;
      }
    if (g == 0) roff[ln] = rq ? row.q_off(a.os) : -1;
    store_staged_rows_at<bf16, D, RS>(vt, (bf16*)a.o, roff, lane);
    if (!rq) return;
  }
  if (g == 0) a.lse[row.stat()] = l > 0.f ? m * a.scale + logf(l) : -INFINITY;
}

// --------------------------------------------------------------------------
// Backward.  Part 1 (dQ): S^T = K Q^T and dP^T = V dO^T with a lane per query
// column, P^T = exp(scale S^T - LSE), dS^T = P^T (dP^T - D), and
// dQ^T = K^T dS^T with K^T read from LDS.  Part 2 (dK, dV): S = Q K^T and
// dP = dO V^T with a lane per key column (the same operand registers with
// the roles of A and B swapped; LSE and D of the accumulator rows from LDS),
// then dV^T = dO^T P and dK^T = Q^T dS with dO^T, Q^T read from LDS.  LDS
// holds two tiles: K, then Q in the same slot once part 1 is done, and dO.
// D = dO . O is formed here from the stored O (and written to the
// workspace) unless it is given.
// --------------------------------------------------------------------------
template <int D>
struct ShortBwdLds {
  static constexpr int tile = ShortDims<D>::tile;
  static constexpr int bytes = 2 * tile * 2 + 2 * shortk::ROWS * 4;  // K then Q, dO; LSE2, D
};

template <int D, int S>
// occupancy: four waves per SIMD at d = 64 (125 registers, no spills; 5%
// faster than three on the temporal layer), three at d = 80, two at 128
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : D <= 80 ? 3 : 2)))
void bwd_short_kernel(BwdArgs a, int do_dq, int do_dkdv, int accumulate) {
  using Dm = ShortDims<D>;
  constexpr int KC = Dm::KC, NDB = Dm::NDB, RS = Dm::RS, TL = Dm::tile;
  constexpr int P = shortk::ROWS / S;
  __shared__ __attribute__((aligned(16))) unsigned char smem[ShortBwdLds<D>::bytes];
  bf16* const KQs = reinterpret_cast<bf16*>(smem);  // K in part 1, then Q
  bf16* const dOs = KQs + TL;
  float* const lse2s = reinterpret_cast<float*>(dOs + TL);
  float* const Dss = lse2s + shortk::ROWS;
  __shared__ int64_t roff[shortk::ROWS];  // output row offsets (staged stores)

  const int lane = threadIdx.x, ln = lane & 31, g = lane >> 5;
  const ShortRow<S> row(a, (int)blockIdx.x * P, ln);  // this lane's query and key row
  const bool rq = row.q_ok(), rk = row.kv_ok();

  bf16x8 qb[KC], ka[KC], va[KC], dob[KC];
  load_row_operands(qb, (const bf16*)a.q + row.q_off(a.qs), rq, g);
  load_row_operands(ka, (const bf16*)a.k + row.kv_off(a.ks), rk, g);
  load_row_operands(va, (const bf16*)a.v + row.kv_off(a.vs), rk, g);
  load_row_operands(dob, (const bf16*)a.dout + row.q_off(a.dos), rq, g);

  // this lane's query row: LSE in log2 units and D.  A missing row, or one
  // whose sequence has no keys (LSE = -inf), gets +inf: P = 0.
  const int64_t srow = row.stat();
  const float lse_r = rq ? a.lse[srow] : INFINITY;
  const float lse2 = lse_r == -INFINITY ? INFINITY : lse_r * kLog2e;
  float dsum = 0.f;
  if (a.dq_computes_d) {
    // D from the stored bf16 O (an fp32 O goes through the preprocess
    // kernel): all of the row's pieces are requested under one condition, so
    // they arrive together
    bf16x8 ov[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) ov[kc] = bf16x8{};
    if (rq) {
      const bf16* orow = (const bf16*)a.o + row.q_off(a.os);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) ov[kc] = load_bf16x8(orow + 16 * kc + 8 * g);
    }
    float part = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf((float)dob[kc][j], (float)ov[kc][j], part);
    dsum = sum_halves(part);
    if (g == 0 && rq) a.dsum[srow] = dsum;
  } else if (rq) {
    dsum = a.dsum[srow];
  }

  if (do_dq) stage_rows<KC, RS>(KQs, ka, ln, g);
  stage_rows<KC, RS>(dOs, dob, ln, g);
  if (g == 0) {
    lse2s[ln] = lse2;
    Dss[ln] = dsum;
  }
  lds_written();
  const float sl2 = a.scale * kLog2e;

  if (do_dq) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      s = mfma32(ka[kc], qb[kc], s);
      dp = mfma32(va[kc], dob[kc], dp);
    }
    const int c = ln;  // query column; entries: key rows 8i + 4g + r
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = 8 * (e >> 2) + 4 * g + (e & 3);
      const bool ok = kr / S == c / S && kr % S < row.sp.nkv;
      const float p = ok ? fast_exp2(fmaf(s[e], sl2, -lse2)) : 0.f;
      s[e] = p * (dp[e] - dsum);
    }
    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const bf16x8 sb = acc_half_to_bf16(s, h2);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 kt = tr_operand(KQs + 32 * db, RS, 16 * h2 + 4 * g, 16 * h2 + 8 + 4 * g, lane);
        dq[db] = mfma32(kt, sb, dq[db]);
      }
    }
    if (accumulate) {
      if (rq) {
        const int64_t qrow = row.q_off(a.dqs);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * g;
            if (d0 >= D) continue;
            f32x4 v4 = {dq[db][4 * i], dq[db][4 * i + 1], dq[db][4 * i + 2], dq[db][4 * i + 3]};
            v4 *= a.scale;
            f32x4* p = reinterpret_cast<f32x4*>((float*)a.dq + qrow + d0);
            *p = *p + v4;
          }
      }
    } else {
      // runs of 4 d of the lane's query row, through the K tile (its
      // transpose reads are done; Q replaces it afterwards) and out as rows
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 32 * db + 8 * i + 4 * g;
          if (d0 >= D) continue;
          const bf16x4 b4 = {(bf16)(dq[db][4 * i] * a.scale), (bf16)(dq[db][4 * i + 1] * a.scale),
                             (bf16)(dq[db][4 * i + 2] * a.scale),
                             (bf16)(dq[db][4 * i + 3] * a.scale)};
          *reinterpret_cast<bf16x4*>(&KQs[ln * RS + d0]) = b4;
        }
      if (g == 0) roff[ln] = rq ? row.q_off(a.dqs) : -1;
      store_staged_rows_at<bf16, D, RS>(KQs, (bf16*)a.dq, roff, lane);
    }
  }

  if (do_dkdv) {
    // Q replaces K in LDS (the wave's LDS operations run in order, so part
    // 1's reads of K come first)
    stage_rows<KC, RS>(KQs, qb, ln, g);
    lds_written();
    // S = Q K^T, dP = dO V^T: lane owns key column c, entries are query rows
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      s = mfma32(qb[kc], ka[kc], s);
      dp = mfma32(dob[kc], va[kc], dp);
    }
    const int c = ln;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[8 * i + 4 * g]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Dss[8 * i + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qr = 8 * i + 4 * g + r;
        const bool ok = qr / S == c / S;  // missing query rows have LSE = +inf
        const float p = ok ? fast_exp2(fmaf(s[4 * i + r], sl2, -l4[r])) : 0.f;
        s[4 * i + r] = p;
        dp[4 * i + r] = p * (dp[4 * i + r] - d4[r]);
      }
    }
    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dk[db] = f32x16{};
      dv[db] = f32x16{};
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const bf16x8 pb = acc_half_to_bf16(s, h2);
      const bf16x8 sb = acc_half_to_bf16(dp, h2);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 dot = tr_operand(dOs + 32 * db, RS, 16 * h2 + 4 * g, 16 * h2 + 8 + 4 * g, lane);
        const bf16x8 qt = tr_operand(KQs + 32 * db, RS, 16 * h2 + 4 * g, 16 * h2 + 8 + 4 * g, lane);
        dv[db] = mfma32(dot, pb, dv[db]);
        dk[db] = mfma32(qt, sb, dk[db]);
      }
    }
    // runs of 4 d of the lane's key row, through the Q and dO tiles (their
    // transpose reads are done) and out as whole rows
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * g;
        if (d0 >= D) continue;
        const bf16x4 k4 = {(bf16)(dk[db][4 * i] * a.scale), (bf16)(dk[db][4 * i + 1] * a.scale),
                           (bf16)(dk[db][4 * i + 2] * a.scale),
                           (bf16)(dk[db][4 * i + 3] * a.scale)};
        const bf16x4 v4 = {(bf16)dv[db][4 * i], (bf16)dv[db][4 * i + 1],
                           (bf16)dv[db][4 * i + 2], (bf16)dv[db][4 * i + 3]};
        *reinterpret_cast<bf16x4*>(&KQs[ln * RS + d0]) = k4;
        *reinterpret_cast<bf16x4*>(&dOs[ln * RS + d0]) = v4;
      }
    if (g == 0) roff[ln] = rk ? row.kv_off(a.dks) : -1;
    store_staged_rows_at<bf16, D, RS>(KQs, (bf16*)a.dk, roff, lane);
    if (g == 0) roff[ln] = rk ? row.kv_off(a.dvs) : -1;
    store_staged_rows_at<bf16, D, RS>(dOs, (bf16*)a.dv, roff, lane);
  }
}

// slot size for a short problem (0: not short)
int short_slot(int Nq, int Nkv) {
  const int n = Nq > Nkv ? Nq : Nkv;
  return n <= 8 ? 8 : n <= 16 ? 16 : n <= 32 ? 32 : 0;
}

template <int D, int S>
static hipError_t fwd_short_s(const FwdArgs& a, hipStream_t s) {
  const long long bh = (long long)a.B * a.H;
  const long long grid = (bh + shortk::ROWS / S - 1) / (shortk::ROWS / S);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.out_f32)
    hipLaunchKernelGGL((fwd_short_kernel<D, S, true>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_short_kernel<D, S, false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t fwd_short_d(const FwdArgs& a, hipStream_t s) {
  switch (short_slot(a.Nq, a.Nkv)) {
    case 8: return fwd_short_s<D, 8>(a, s);
    case 16: return fwd_short_s<D, 16>(a, s);
    case 32: return fwd_short_s<D, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_short(const FwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return fwd_short_d<64>(a, s);
    case 80: return fwd_short_d<80>(a, s);
    case 128: return fwd_short_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int S>
static hipError_t bwd_short_s(const BwdArgs& a, int do_dkdv, int do_dq, int accumulate,
                              hipStream_t s) {
  const long long bh = (long long)a.B * a.H;
  const long long grid = (bh + shortk::ROWS / S - 1) / (shortk::ROWS / S);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_short_kernel<D, S>), dim3((unsigned)grid), dim3(64), 0, s, a, do_dq,
                     do_dkdv, accumulate);
  return hipGetLastError();
}

template <int D>
static hipError_t bwd_short_d(const BwdArgs& a, int do_dkdv, int do_dq, int accumulate,
                              hipStream_t s) {
  switch (short_slot(a.Nq, a.Nkv)) {
    case 8: return bwd_short_s<D, 8>(a, do_dkdv, do_dq, accumulate, s);
    case 16: return bwd_short_s<D, 16>(a, do_dkdv, do_dq, accumulate, s);
    case 32: return bwd_short_s<D, 32>(a, do_dkdv, do_dq, accumulate, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_short(const BwdArgs& a, int d, int do_dkdv, int do_dq, int accumulate,
                            hipStream_t s) {
  switch (d) {
    case 64: return bwd_short_d<64>(a, do_dkdv, do_dq, accumulate, s);
    case 80: return bwd_short_d<80>(a, do_dkdv, do_dq, accumulate, s);
    case 128: return bwd_short_d<128>(a, do_dkdv, do_dq, accumulate, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace exattn

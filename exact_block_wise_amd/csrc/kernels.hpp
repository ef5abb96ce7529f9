// Kernel argument blocks and launcher declarations (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "span.hpp"

namespace exattn {

struct Strides {
  int64_t sb, sh, sn;
};

// Forward over key rows [c*chunk_len, min((c+1)*chunk_len, Nkv)) for chunk
// c in [0, n_chunks).  A plain forward is n_chunks = 1, chunk_len = Nkv.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Strides qs, ks, vs, os;
  int64_t o_chunk_stride;    // elements between chunks' outputs
  int64_t lse_chunk_stride;  // elements between chunks' LSE rows
  int B, H, Nq, Nkv;
  int n_chunks, chunk_len;
  float scale;
  int out_f32;               // 1: o is fp32, 0: o is the input dtype
  // Packed variable-length sequences (null: dense).  Sequence b owns query
  // tokens [cu_q[b], cu_q[b+1]) and key/value tokens [cu_kv[b], cu_kv[b+1]);
  // B is then the number of sequences, Nq / Nkv bound their lengths, sb is
  // 0 (tokens are rows of stride sn) and LSE is [H, total_q].
  const int* cu_q;
  const int* cu_kv;
  int64_t total_q, total_kv;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;      // dQ: input dtype, or fp32 when accumulating
  void* dk;
  void* dv;
  float* dsum;   // [B,H,Nq] contiguous: D_i = dO_i . O_i
  float* dq_part;  // [dq_splits,B,H,Nq,d] fp32 partials (dq_splits > 1)
  Strides qs, ks, vs, os, dos, dqs, dks, dvs;
  int B, H, Nq, Nkv;
  float scale;
  int o_f32;     // o dtype is fp32
  int dq_splits;     // key ranges the dQ pass is split into (1: none)
  int dq_split_len;  // keys per range, a multiple of the key tile
  int dq_computes_d; // the bf16 dQ kernel forms D from a bf16 o and dout and writes dsum
  // packed variable-length sequences, as in FwdArgs (LSE and D [H, total_q])
  const int* cu_q;
  const int* cu_kv;
  int64_t total_q, total_kv;
};

// The rows of problem (b, h).  Packed prefix sums are clamped (packed_side)
// so that no value of cu_q / cu_kv can address rows outside the tensors.
template <typename Args>
__device__ __forceinline__ SeqSpan seq_span(const Args& a, int b, int h) {
  SeqSpan s;
  if (a.cu_q) {
    packed_side(a.cu_q[b], a.cu_q[b + 1], a.Nq, a.total_q, s.q_row0, s.nq);
    packed_side(a.cu_kv[b], a.cu_kv[b + 1], a.Nkv, a.total_kv, s.kv_row0, s.nkv);
    s.stat0 = (int64_t)h * a.total_q + s.q_row0;
  } else {
    s.q_row0 = 0;
    s.kv_row0 = 0;
    s.nq = a.Nq;
    s.nkv = a.Nkv;
    s.stat0 = ((int64_t)b * a.H + h) * a.Nq;
  }
  return s;
}

struct MergeArgs {
  const float* o_parts;
  const float* lse_parts;
  void* o;
  float* lse;
  Strides os;
  int n_parts, B, H, Nq, d;
  int out_f32;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_bwd_pre(const BwdArgs& a, int d, int in_bf16, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, int d, int do_dkdv, int do_dq, int accumulate,
                           hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int d, int do_dkdv, int do_dq, int accumulate,
                          hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

// Short sequences (bf16, Nq and Nkv <= 32): several sequences per product
// tile (EXATTN_SHORT=0 sends them through the general kernels instead).
// short_slot is the rows per sequence in a tile (8, 16 or 32), or 0 when the
// problem is not short.
#ifndef EXATTN_SHORT
#define EXATTN_SHORT 1
#endif
int short_slot(int Nq, int Nkv);
hipError_t launch_fwd_short(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_bwd_short(const BwdArgs& a, int d, int do_dkdv, int do_dq, int accumulate,
                            hipStream_t s);

// Number of key ranges the bf16 dQ pass splits Nkv into (1 = unsplit): a
// split is used only when the query blocks alone would leave most compute
// units idle (a short query block against a long key range).
int dq_key_splits(int B, int H, int Nq, int Nkv);

}  // namespace exattn

// C-ABI entry points: host-side validation, then kernel dispatch on the
// caller's stream.  Nothing here allocates, copies, synchronises or keeps
// mutable state; an argument error returns before any work is enqueued.
#include "exattn.h"

#include <math.h>
#include <string.h>

#include <mutex>

#include "kernels.hpp"

using namespace exattn;

namespace {

constexpr size_t kWsAlign = 256;
constexpr int64_t kMaxRowStrideBytes = int64_t(1) << 24;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool supported_d(int d) { return d == 64 || d == 80 || d == 128; }

int elem_bytes(int dtype) { return dtype == ATTN_BF16 ? 2 : 4; }

bool valid_dtype(int dtype) { return dtype == ATTN_F32 || dtype == ATTN_BF16; }

attn_status check_problem(const attn_problem* p) {
  if (!p) return ATTN_E_INVALID;
  if (p->B < 1 || p->H < 1 || p->Nq < 1 || p->Nkv < 1 || p->d < 1) return ATTN_E_INVALID;
  if (!isfinite(p->scale)) return ATTN_E_INVALID;
  // the bf16 kernels take the running maximum over raw scores and mask keys
  // with -inf before scaling, which holds for a positive scale only
  if (!(p->scale > 0.f)) return ATTN_E_UNSUPPORTED;
  if (!supported_d(p->d)) return ATTN_E_UNSUPPORTED;
  // kernels index (batch, head) pairs with 32-bit integers
  if ((int64_t)p->B * p->H > INT32_MAX) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

// pointer, dtype, non-negative strides; then 16-byte vector access rules
attn_status check_tensor(const attn_tensor& t) {
  if (!t.ptr || !valid_dtype(t.dtype)) return ATTN_E_INVALID;
  if (t.sb < 0 || t.sh < 0 || t.sn < 0) return ATTN_E_INVALID;
  const int64_t vec = 16 / elem_bytes(t.dtype);
  if (reinterpret_cast<uintptr_t>(t.ptr) % 16 != 0) return ATTN_E_UNSUPPORTED;
  if (t.sb % vec || t.sh % vec || t.sn % vec) return ATTN_E_UNSUPPORTED;
  // a tile of up to 128 rows must stay within 32-bit buffer offsets
  if (t.sn * elem_bytes(t.dtype) > kMaxRowStrideBytes) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

attn_status first_error(std::initializer_list<attn_status> sts) {
  for (attn_status s : sts)
    if (s != ATTN_OK) return s;
  return ATTN_OK;
}

Strides strides_of(const attn_tensor& t) { return Strides{t.sb, t.sh, t.sn}; }

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_HIP; }

size_t dsum_bytes(const attn_problem* p) {
  return round_up((size_t)p->B * p->H * p->Nq * sizeof(float), kWsAlign);
}

// fp32 dQ partials of a split key range (see dq_key_splits), after D
size_t dq_part_bytes(const attn_problem* p, uint32_t flags) {
  if (flags & ATTN_BWD_NO_DQ) return 0;
  const int splits = dq_key_splits(p->B, p->H, p->Nq, p->Nkv);
  if (splits <= 1) return 0;
  return round_up((size_t)splits * p->B * p->H * p->Nq * p->d * sizeof(float), kWsAlign);
}

// o / dout dtypes the preprocess serves: dout BF16 with o BF16 or F32;
// dout F32 with o F32
bool pre_dtypes_ok(int o_dtype, int do_dtype) {
  return do_dtype == ATTN_BF16 ? (o_dtype == ATTN_BF16 || o_dtype == ATTN_F32)
                               : o_dtype == ATTN_F32;
}

attn_status check_varlen(const attn_varlen* p) {
  if (!p) return ATTN_E_INVALID;
  if (p->n_seq < 1 || p->H < 1 || p->d < 1 || p->max_q < 1 || p->max_kv < 1) return ATTN_E_INVALID;
  if (p->total_q < 0 || p->total_kv < 0 || !p->cu_q || !p->cu_kv) return ATTN_E_INVALID;
  if (!isfinite(p->scale)) return ATTN_E_INVALID;
  if (!(p->scale > 0.f)) return ATTN_E_UNSUPPORTED;  // as for attn_problem
  if (!supported_d(p->d)) return ATTN_E_UNSUPPORTED;
  if ((int64_t)p->n_seq * p->H > INT32_MAX) return ATTN_E_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(p->cu_q) % 4 || reinterpret_cast<uintptr_t>(p->cu_kv) % 4)
    return ATTN_E_UNSUPPORTED;
  // the statistics index h * total_q + t and the grid must fit their types
  if ((int64_t)p->H * p->total_q > (int64_t(1) << 40)) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

// packed tensors: token and head strides only
Strides packed_strides(const attn_tensor& t) { return Strides{0, t.sh, t.sn}; }

size_t varlen_dsum_bytes(const attn_varlen* p) {
  return round_up((size_t)p->H * p->total_q * sizeof(float), kWsAlign);
}

// attn_bwd's validation and, when `launch` is set, its launches.  With
// launch false it returns after the host-side checks (nothing enqueued).
attn_status bwd_dense(const attn_problem* p, const attn_tensor& q, const attn_tensor& k,
                      const attn_tensor& v, const attn_tensor& o, const attn_tensor& dout,
                      const float* lse, const attn_tensor& dq, const attn_tensor& dk,
                      const attn_tensor& dv, void* workspace, size_t workspace_bytes,
                      uint32_t flags, void* stream, bool launch) {
  constexpr uint32_t kAll = ATTN_BWD_DQ_ACCUMULATE | ATTN_BWD_D_PRECOMPUTED | ATTN_BWD_NO_DQ |
                            ATTN_BWD_NO_DKDV;
  if (flags & ~kAll) return ATTN_E_INVALID;
  const bool acc = flags & ATTN_BWD_DQ_ACCUMULATE;
  const bool pre_done = flags & ATTN_BWD_D_PRECOMPUTED;
  const bool do_dq = !(flags & ATTN_BWD_NO_DQ);
  const bool do_dkdv = !(flags & ATTN_BWD_NO_DKDV);
  if (!do_dq && !do_dkdv) return ATTN_E_INVALID;
  attn_status st = first_error({check_problem(p), check_tensor(q), check_tensor(k),
                                check_tensor(v), check_tensor(dout),
                                pre_done ? ATTN_OK : check_tensor(o),
                                do_dq ? check_tensor(dq) : ATTN_OK,
                                do_dkdv ? check_tensor(dk) : ATTN_OK,
                                do_dkdv ? check_tensor(dv) : ATTN_OK});
  if (st != ATTN_OK) return st;
  const int dt = q.dtype;
  if (k.dtype != dt || v.dtype != dt || dout.dtype != dt) return ATTN_E_INVALID;
  if (!pre_done && !pre_dtypes_ok(o.dtype, dt)) return ATTN_E_INVALID;
  if (do_dkdv && (dk.dtype != dt || dv.dtype != dt)) return ATTN_E_INVALID;
  if (do_dq && (acc ? dq.dtype != ATTN_F32 : dq.dtype != dt)) return ATTN_E_INVALID;
  if (!lse) return ATTN_E_INVALID;
  if (reinterpret_cast<uintptr_t>(lse) % 4) return ATTN_E_UNSUPPORTED;
  const size_t part_bytes = dq_part_bytes(p, flags);
  if (!workspace || workspace_bytes < dsum_bytes(p) + part_bytes) return ATTN_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kWsAlign) return ATTN_E_WORKSPACE;
  if (!launch) return ATTN_OK;

  BwdArgs a{};
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.o = o.ptr; a.dout = dout.ptr; a.lse = lse;
  a.dq = dq.ptr; a.dk = dk.ptr; a.dv = dv.ptr;
  a.qs = strides_of(q); a.ks = strides_of(k); a.vs = strides_of(v); a.os = strides_of(o);
  a.dos = strides_of(dout); a.dqs = strides_of(dq); a.dks = strides_of(dk);
  a.dvs = strides_of(dv);
  a.dsum = static_cast<float*>(workspace);
  a.dq_part = part_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                    dsum_bytes(p))
                         : nullptr;
  a.dq_splits = 1;
  a.dq_split_len = p->Nkv;
  a.B = p->B; a.H = p->H; a.Nq = p->Nq; a.Nkv = p->Nkv;
  a.scale = p->scale;
  a.o_f32 = o.dtype == ATTN_F32;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!pre_done) {
    if (do_dq && dt == ATTN_BF16 && !a.o_f32) {
      a.dq_computes_d = 1;  // the bf16 dQ kernel forms D from a bf16 O and runs first
    } else {
      const hipError_t e = launch_bwd_pre(a, p->d, dt == ATTN_BF16, s);
      if (e != hipSuccess) return ATTN_E_HIP;
    }
  }
  if (dt == ATTN_F32) return from_hip(launch_bwd_f32(a, p->d, do_dkdv, do_dq, acc, s));
  return from_hip(launch_bwd_bf16(a, p->d, do_dkdv, do_dq, acc, s));
}

// --------------------------------------------------------------------------
// Scratch of attn_bwd_noalloc: a file-scope device array, one copy per GPU,
// allocated with the library's code object (so a call allocates nothing).
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress, looked
// up once per device with that device current, and only that address is
// ever passed to kernels.
// --------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The scratch address on the device that runs `stream` (the current device
// for the null stream).
attn_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return ATTN_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_E_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    hipError_t r = hipGetDevice(&cur);
    if (r == hipSuccess && cur != dev) r = hipSetDevice(dev);
    void* ptr = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (r == hipSuccess) r = back;
    }
    g_scratch_err[dev] = r;
    g_scratch_ptr[dev] = r == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return ATTN_E_HIP;
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_string(attn_status st) {
  // a C caller may pass any int; reading it as the enum type would be
  // undefined in C++ for values outside the enumerators' range
  int v;
  memcpy(&v, &st, sizeof v);
  switch (v) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_E_INVALID: return "ATTN_E_INVALID: invalid argument";
    case ATTN_E_UNSUPPORTED: return "ATTN_E_UNSUPPORTED: head dim, stride or alignment not served";
    case ATTN_E_WORKSPACE: return "ATTN_E_WORKSPACE: workspace missing or too small";
    case ATTN_E_HIP: return "ATTN_E_HIP: HIP runtime error";
  }
  return "unknown attn_status";
}

attn_status attn_fwd(const attn_problem* p, attn_tensor q, attn_tensor k, attn_tensor v,
                     attn_tensor o, float* lse, void* stream) {
  attn_status st = first_error({check_problem(p), check_tensor(q), check_tensor(k),
                                check_tensor(v), check_tensor(o)});
  if (st != ATTN_OK) return st;
  if (k.dtype != q.dtype || v.dtype != q.dtype) return ATTN_E_INVALID;
  if (o.dtype != q.dtype && o.dtype != ATTN_F32) return ATTN_E_INVALID;
  if (!lse) return ATTN_E_INVALID;
  if (reinterpret_cast<uintptr_t>(lse) % 4) return ATTN_E_UNSUPPORTED;
  FwdArgs a{};
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.o = o.ptr; a.lse = lse;
  a.qs = strides_of(q); a.ks = strides_of(k); a.vs = strides_of(v); a.os = strides_of(o);
  a.B = p->B; a.H = p->H; a.Nq = p->Nq; a.Nkv = p->Nkv;
  a.n_chunks = 1; a.chunk_len = p->Nkv;
  a.scale = p->scale;
  a.out_f32 = o.dtype == ATTN_F32;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(q.dtype == ATTN_BF16 ? launch_fwd_bf16(a, p->d, s) : launch_fwd_f32(a, p->d, s));
}

attn_status attn_fwd_chunked(const attn_problem* p, int32_t n_chunks, attn_tensor q,
                             attn_tensor k, attn_tensor v, float* o_parts, float* lse_parts,
                             void* stream) {
  attn_status st = first_error({check_problem(p), check_tensor(q), check_tensor(k),
                                check_tensor(v)});
  if (st != ATTN_OK) return st;
  if (n_chunks < 1) return ATTN_E_INVALID;
  if (k.dtype != q.dtype || v.dtype != q.dtype) return ATTN_E_INVALID;
  if (!o_parts || !lse_parts) return ATTN_E_INVALID;
  if (reinterpret_cast<uintptr_t>(o_parts) % 16 || reinterpret_cast<uintptr_t>(lse_parts) % 4)
    return ATTN_E_UNSUPPORTED;
  FwdArgs a{};
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.o = o_parts; a.lse = lse_parts;
  a.qs = strides_of(q); a.ks = strides_of(k); a.vs = strides_of(v);
  const int64_t d = p->d;
  a.os = Strides{(int64_t)p->H * p->Nq * d, (int64_t)p->Nq * d, d};
  a.o_chunk_stride = (int64_t)p->B * p->H * p->Nq * d;
  a.lse_chunk_stride = (int64_t)p->B * p->H * p->Nq;
  a.B = p->B; a.H = p->H; a.Nq = p->Nq; a.Nkv = p->Nkv;
  a.n_chunks = n_chunks;
  a.chunk_len = (int)(((int64_t)p->Nkv + n_chunks - 1) / n_chunks);
  a.scale = p->scale;
  a.out_f32 = 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(q.dtype == ATTN_BF16 ? launch_fwd_bf16(a, p->d, s) : launch_fwd_f32(a, p->d, s));
}

attn_status attn_lse_merge(int32_t n_parts, int32_t B, int32_t H, int32_t Nq, int32_t d,
                           const float* o_parts, const float* lse_parts, attn_tensor o,
                           float* lse, void* stream) {
  if (n_parts < 1 || B < 1 || H < 1 || Nq < 1 || d < 1) return ATTN_E_INVALID;
  if (!o_parts || !lse_parts || !lse) return ATTN_E_INVALID;
  attn_status st = check_tensor(o);
  if (st != ATTN_OK) return st;
  if (d % 4) return ATTN_E_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(o_parts) % 16 || reinterpret_cast<uintptr_t>(lse_parts) % 4 ||
      reinterpret_cast<uintptr_t>(lse) % 4)
    return ATTN_E_UNSUPPORTED;
  MergeArgs a{};
  a.o_parts = o_parts; a.lse_parts = lse_parts; a.o = o.ptr; a.lse = lse;
  a.os = strides_of(o);
  a.n_parts = n_parts; a.B = B; a.H = H; a.Nq = Nq; a.d = d;
  a.out_f32 = o.dtype == ATTN_F32;
  return from_hip(launch_merge(a, reinterpret_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(const attn_problem* p, uint32_t flags) {
  if (check_problem(p) != ATTN_OK) return 0;
  return dsum_bytes(p) + dq_part_bytes(p, flags);
}

attn_status attn_bwd_preprocess(const attn_problem* p, attn_tensor o, attn_tensor dout,
                                float* dsum, void* stream) {
  attn_status st = first_error({check_problem(p), check_tensor(o), check_tensor(dout)});
  if (st != ATTN_OK) return st;
  if (!pre_dtypes_ok(o.dtype, dout.dtype)) return ATTN_E_INVALID;
  if (!dsum) return ATTN_E_INVALID;
  if (reinterpret_cast<uintptr_t>(dsum) % 4) return ATTN_E_UNSUPPORTED;
  BwdArgs a{};
  a.o = o.ptr; a.dout = dout.ptr; a.dsum = dsum;
  a.os = strides_of(o); a.dos = strides_of(dout);
  a.B = p->B; a.H = p->H; a.Nq = p->Nq; a.Nkv = p->Nkv;
  a.o_f32 = o.dtype == ATTN_F32;
  return from_hip(launch_bwd_pre(a, p->d, dout.dtype == ATTN_BF16,
                                 reinterpret_cast<hipStream_t>(stream)));
}

attn_status attn_bwd(const attn_problem* p, attn_tensor q, attn_tensor k, attn_tensor v,
                     attn_tensor o, attn_tensor dout, const float* lse, attn_tensor dq,
                     attn_tensor dk, attn_tensor dv, void* workspace, size_t workspace_bytes,
                     uint32_t flags, void* stream) {
  return bwd_dense(p, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, flags,
                   stream, true);
}

attn_status attn_bwd_noalloc(const attn_problem* p, attn_tensor q, attn_tensor k,
                             attn_tensor v, attn_tensor o, attn_tensor dout, const float* lse,
                             attn_tensor dq, attn_tensor dk, attn_tensor dv, uint32_t flags,
                             void* stream) {
  // every host-side check first, with a stand-in for the scratch address
  // (aligned, never dereferenced): a problem whose workspace exceeds the
  // scratch is ATTN_E_WORKSPACE, and nothing touches the GPU before this
  const attn_status st = bwd_dense(p, q, k, v, o, dout, lse, dq, dk, dv,
                                   reinterpret_cast<void*>(kWsAlign), ATTN_NOALLOC_SCRATCH_BYTES,
                                   flags, stream, false);
  if (st != ATTN_OK) return st;
  void* ws = nullptr;
  const attn_status sst = scratch_for(reinterpret_cast<hipStream_t>(stream), &ws);
  if (sst != ATTN_OK) return sst;
  return bwd_dense(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ATTN_NOALLOC_SCRATCH_BYTES, flags,
                   stream, true);
}

attn_status attn_fwd_varlen(const attn_varlen* p, attn_tensor q, attn_tensor k, attn_tensor v,
                            attn_tensor o, float* lse, void* stream) {
  attn_status st = first_error({check_varlen(p), check_tensor(q), check_tensor(k),
                                check_tensor(v), check_tensor(o)});
  if (st != ATTN_OK) return st;
  if (k.dtype != q.dtype || v.dtype != q.dtype) return ATTN_E_INVALID;
  if (o.dtype != q.dtype && o.dtype != ATTN_F32) return ATTN_E_INVALID;
  if (q.dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (!lse) return ATTN_E_INVALID;
  if (reinterpret_cast<uintptr_t>(lse) % 4) return ATTN_E_UNSUPPORTED;
  FwdArgs a{};
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.o = o.ptr; a.lse = lse;
  a.qs = packed_strides(q); a.ks = packed_strides(k); a.vs = packed_strides(v);
  a.os = packed_strides(o);
  a.B = p->n_seq; a.H = p->H; a.Nq = p->max_q; a.Nkv = p->max_kv;
  a.n_chunks = 1; a.chunk_len = p->max_kv;
  a.scale = p->scale;
  a.out_f32 = o.dtype == ATTN_F32;
  a.cu_q = p->cu_q; a.cu_kv = p->cu_kv; a.total_q = p->total_q; a.total_kv = p->total_kv;
  return from_hip(launch_fwd_bf16(a, p->d, reinterpret_cast<hipStream_t>(stream)));
}

size_t attn_bwd_varlen_workspace_bytes(const attn_varlen* p) {
  if (check_varlen(p) != ATTN_OK) return 0;
  return varlen_dsum_bytes(p);
}

attn_status attn_bwd_varlen(const attn_varlen* p, attn_tensor q, attn_tensor k, attn_tensor v,
                            attn_tensor o, attn_tensor dout, const float* lse, attn_tensor dq,
                            attn_tensor dk, attn_tensor dv, void* workspace,
                            size_t workspace_bytes, uint32_t flags, void* stream) {
  constexpr uint32_t kAll = ATTN_BWD_DQ_ACCUMULATE | ATTN_BWD_D_PRECOMPUTED | ATTN_BWD_NO_DQ |
                            ATTN_BWD_NO_DKDV;
  if (flags & ~kAll) return ATTN_E_INVALID;
  const bool acc = flags & ATTN_BWD_DQ_ACCUMULATE;
  const bool pre_done = flags & ATTN_BWD_D_PRECOMPUTED;
  const bool do_dq = !(flags & ATTN_BWD_NO_DQ);
  const bool do_dkdv = !(flags & ATTN_BWD_NO_DKDV);
  if (!do_dq && !do_dkdv) return ATTN_E_INVALID;
  attn_status st = first_error({check_varlen(p), check_tensor(q), check_tensor(k),
                                check_tensor(v), check_tensor(dout),
                                pre_done ? ATTN_OK : check_tensor(o),
                                do_dq ? check_tensor(dq) : ATTN_OK,
                                do_dkdv ? check_tensor(dk) : ATTN_OK,
                                do_dkdv ? check_tensor(dv) : ATTN_OK});
  if (st != ATTN_OK) return st;
  const int dt = q.dtype;
  if (k.dtype != dt || v.dtype != dt || dout.dtype != dt) return ATTN_E_INVALID;
  if (dt != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (!pre_done && !pre_dtypes_ok(o.dtype, dt)) return ATTN_E_INVALID;
  if (do_dkdv && (dk.dtype != dt || dv.dtype != dt)) return ATTN_E_INVALID;
  if (do_dq && (acc ? dq.dtype != ATTN_F32 : dq.dtype != dt)) return ATTN_E_INVALID;
  if (!lse) return ATTN_E_INVALID;
  if (reinterpret_cast<uintptr_t>(lse) % 4) return ATTN_E_UNSUPPORTED;
  if (!workspace || workspace_bytes < varlen_dsum_bytes(p)) return ATTN_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kWsAlign) return ATTN_E_WORKSPACE;

  BwdArgs a{};
  a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.o = o.ptr; a.dout = dout.ptr; a.lse = lse;
  a.dq = dq.ptr; a.dk = dk.ptr; a.dv = dv.ptr;
  a.qs = packed_strides(q); a.ks = packed_strides(k); a.vs = packed_strides(v);
  a.os = packed_strides(o); a.dos = packed_strides(dout); a.dqs = packed_strides(dq);
  a.dks = packed_strides(dk); a.dvs = packed_strides(dv);
  a.dsum = static_cast<float*>(workspace);
  a.dq_part = nullptr;
  a.dq_splits = 1;
  a.dq_split_len = p->max_kv;
  a.B = p->n_seq; a.H = p->H; a.Nq = p->max_q; a.Nkv = p->max_kv;
  a.scale = p->scale;
  a.o_f32 = o.dtype == ATTN_F32;
  a.cu_q = p->cu_q; a.cu_kv = p->cu_kv; a.total_q = p->total_q; a.total_kv = p->total_kv;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!pre_done) {
    if (do_dq && !a.o_f32) {
      a.dq_computes_d = 1;  // the dQ kernel (or the packed-tile kernel) forms D from a bf16 O
    } else {
      // D over all packed query tokens: the dense preprocess of one
      // [1, H, total_q, d] problem writes the same [H, total_q] order
      BwdArgs pa = a;
      pa.cu_q = pa.cu_kv = nullptr;
      pa.B = 1;
      pa.Nq = (int)p->total_q;
      pa.os.sb = pa.dos.sb = 0;
      if (p->total_q > 0x7fffffffLL) return ATTN_E_UNSUPPORTED;
      if (p->total_q > 0) {
        const hipError_t e = launch_bwd_pre(pa, p->d, 1, s);
        if (e != hipSuccess) return ATTN_E_HIP;
      }
    }
  }
  return from_hip(launch_bwd_bf16(a, p->d, do_dkdv, do_dq, acc, s));
}

}  // extern "C"

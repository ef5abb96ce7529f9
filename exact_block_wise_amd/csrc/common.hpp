// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 matrix-core product, fp32 accumulate.
// Operand lane layout (wave64, l = lane):
//   A (32 x 16): lane l holds row m = l % 32 and 8 contraction slots of
//                group g = l / 32;
//   B (16 x 32): lane l holds column n = l % 32 and the 8 slots of group g;
//   C (32 x 32): lane l holds column n = l % 32, rows 8*i + 4*g + r at
//                accumulator index 4*i + r (i, r in 0..3).
// The hardware pairs slot j of group g in A with slot j of group g in B, so
// any assignment of contraction indices to (g, j) works as long as A and B
// use the same one.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with the accumulator pinned in AGPRs.  For accumulators
// that only matrix instructions touch inside a loop (dK, dV), this keeps the
// register allocator from parking them in AGPRs and copying them to VGPRs and
// back around every product.  Chains of these on one accumulator need no
// wait states (same shape, destination = srcC).  The compiler's hazard
// tracking does not look inside inline assembly, so the leading s_nop covers
// an accumulator the allocator may have just rewritten (v_accvgpr_write)
// before the product reads it; kernels using this must still not spill.
// Before VALU code reads the accumulator, call agpr_results_ready().
__device__ __forceinline__ void mfma32_agpr(bf16x8 a, bf16x8 b, f32x16& c) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+a"(c) : "v"(a), "v"(b));
}
// The same product with a zero accumulator operand (the first product of an
// accumulator): nothing has to clear the AGPRs beforehand.
__device__ __forceinline__ void mfma32_agpr_zero(bf16x8 a, bf16x8 b, f32x16& c) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
               : "=a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void agpr_results_ready() {
  // covers the longest result latency of a 32x32 product (16 passes)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Wave priority around matrix-instruction blocks: a wave about to issue
// products is favoured, so co-resident waves in their vector phase fill the
// gaps instead of all waves reaching the matrix unit at once.
#ifndef EXATTN_SETPRIO
#define EXATTN_SETPRIO 0
#endif
__device__ __forceinline__ void prio_mfma() {
  if constexpr (EXATTN_SETPRIO) __builtin_amdgcn_s_setprio(1);
}
__device__ __forceinline__ void prio_valu() {
  if constexpr (EXATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// value of the other half-wave (lane ^ 32), through the LDS crossbar
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: every lane sees
// both halves' values, no LDS traffic)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// LDS transpose read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// i receives element (i % 4) of the 8-byte pieces read by lanes
// 4e + i / 4, e = 0..3.  So if lane j of the group reads row r(j / 4),
// columns c0 + 4 (j % 4) .. +3 of a row-major tile, lane i receives column
// c0 + i of rows r(0..3): a column of the tile, as a matrix-core operand.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4_t*)(const_cast<bf16*>(p)));
}

// Operand of a 32x32x16 product whose lane l must hold column (l % 32) of a
// row-major LDS tile at 8 rows: rows rows_lo + (0..3) and rows_hi + (0..3),
// where rows_lo / rows_hi already include this lane's slot group.  `tile`
// points at element (0, c0) of the 32 columns; `ld` is the row stride.
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int ld, int rows_lo, int rows_hi,
                                             int lane) {
  const int i = lane & 15;
  const int col = 16 * ((lane >> 4) & 1) + 4 * (i & 3);
  const bf16x4 lo = lds_read_tr(tile + (rows_lo + (i >> 2)) * ld + col);
  const bf16x4 hi = lds_read_tr(tile + (rows_hi + (i >> 2)) * ld + col);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of the 8 bf16 values of an operand, accumulated in fp32 (v_dot2 with 1)
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3,
                                       float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

// Accumulator entries 8h .. 8h+7 of a 32x32 tile as one bf16x8 operand.
__device__ __forceinline__ bf16x8 acc_half_to_bf16(const f32x16& s, int h) {
  return cvt8(s[8 * h + 0], s[8 * h + 1], s[8 * h + 2], s[8 * h + 3],
              s[8 * h + 4], s[8 * h + 5], s[8 * h + 6], s[8 * h + 7]);
}

// Row stride, in elements, of a bf16 LDS tile with DP columns that is read
// both as rows (16-byte pieces, 16 lanes per pass) and as columns
// (ds_read_b64_tr_b16: per half-wave four rows of 64 bytes).  With 64
// four-byte banks, a stride of S banks puts the four rows of a column read at
// banks 0, S, 2S, 3S (mod 64), each 16 banks wide, and the 16 rows of a row
// read at 0, S, .., 15S, each 4 wide.  DP + 8 serves d = 64 and 80 (column
// reads at most two-way conflicted, row reads free); at DP = 128 it gives
// S = 4 (mod 64) and four-way conflicted column reads, and DP + 24 (S = 12)
// keeps row reads free with column reads overlapping on 4 banks only.
#ifndef EXATTN_STRIDE128
#define EXATTN_STRIDE128 152
#endif
constexpr int tile_stride(int dp) { return dp == 128 ? EXATTN_STRIDE128 : dp + 8; }

// Buffer resource over rows [0, rows) of a row-major tensor that starts at
// `base`, rows `stride_bytes` apart and `row_bytes` long.  Raw buffer loads
// check each access against the record count and return zeros past it, so
// tile loaders need no branch for rows beyond the end: row r >= rows starts
// at r * stride_bytes >= (rows - 1) * stride_bytes + row_bytes.  Offsets are
// 32-bit, so callers rebase the resource at each tile and keep a tile within
// 2 GiB (the library bounds row strides).
constexpr int kBufferDword3 = 0x00020000;  // 32-bit data format (gfx9 encoding)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows,
                                                            int64_t stride_bytes, int row_bytes) {
  int64_t n = rows > 0 ? (int64_t)(rows - 1) * stride_bytes + row_bytes : 0;
  n = n < 0xffffffffll ? n : 0xffffffffll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)n,
                                           kBufferDword3);
}
__device__ __forceinline__ bf16x8 buffer_load_bf16x8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Direct-to-LDS buffer loads: lane L's 16 (or 4) bytes from byte offset
// `off` of the buffer land at LDS byte address lds + 16 L (4 L), without
// passing through registers; `lds` must be wave-uniform.  They are written
// as inline assembly so that the compiler's wait bookkeeping, which cannot
// tell that a later LDS read of another buffer does not overlap them,
// inserts no wait: callers must wait_vmem() before the barrier that
// publishes the data, and must keep no compiler-issued vector-memory load
// outstanding across them that a wait computed for it would under-count.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t lds,
                                                  uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(off), "s"(r) : "memory");
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, uint32_t lds,
                                                 uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(off), "s"(r) : "memory");
}
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt unconstrained
}

// Direct-to-LDS staging of a ROWS x D bf16 tile (rows `sn` elements apart
// in HBM) into a row-padded LDS tile of row stride RS elements: the tile's
// ROWS * RS / 8 sixteen-byte chunks are written by wave instructions of 64
// chunks each, instruction i by wave i % 4 of the workgroup; lane L of
// instruction i carries chunk 64 i + L, i.e. row (64 i + L) / (RS / 8),
// chunk (64 i + L) % (RS / 8).  Lanes on padding chunks re-load chunk 0 of
// their row, so no lane is masked off.
template <int D, int RS, int ROWS>
struct LdsTileDma {
  static constexpr int CPR = RS / 8;
  static constexpr int NI = ROWS * CPR / 64;
  static constexpr int NIW = (NI + 3) / 4;
  static_assert(RS % 8 == 0 && RS >= D && ROWS * CPR % 64 == 0,
                "tile must be whole wave instructions");
  uint32_t off[NIW];
  __device__ __forceinline__ void init(int w, int lane, int64_t sn) {
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int pc = 64 * (w + 4 * j) + lane;
      const int r = pc / CPR, ch = pc % CPR;
      off[j] = (uint32_t)(r * 2 * sn + 16 * (ch < D / 8 ? ch : 0));
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, uint32_t lds, int w) const {
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int i = w + 4 * j;
      if (NI % 4 == 0 || i < NI) buffer_load_lds16(r, lds + 1024 * i, off[j]);
    }
  }
};

// Output rows staged in LDS, written out whole.  Kernels whose accumulator
// layout gives a lane one output row and runs of a few columns would make
// every wave store instruction touch 32 rows with 8-16 bytes each (one L2
// request per piece); they write the runs to a wave-private LDS tile first
// and this copies rows [0, rows) of that tile (row stride SRS elements of T,
// D columns) to `out` (rows `sn` elements apart) in 16-byte pieces, so each
// instruction covers contiguous row memory.  A wave's LDS operations
// complete in order, so the tile needs no barrier when only its wave uses it.
// The rows go out with streaming (non-temporal) stores: every output row is
// written once, and keeping it out of the caches spares the reads of the
// kernels that follow (measured: ViT-B step -1%, spatial layer -6%, and the
// cross-attention forward that follows its dK/dV -9%).
#ifndef EXATTN_NT_OUT
#define EXATTN_NT_OUT 1
#endif
template <typename T, int D, int SRS, bool NT = (EXATTN_NT_OUT != 0)>
__device__ __forceinline__ void store_staged_rows(const T* stage, T* out, int64_t sn, int rows,
                                                  int lane) {
  constexpr int PER = 16 / (int)sizeof(T), PPR = D / PER, NP = 32 * PPR / 64;
  static_assert(D % PER == 0 && 32 * PPR % 64 == 0, "whole 16-byte pieces, whole instructions");
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e = 64 * j + lane, r = e / PPR, pc = e % PPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[r * SRS + PER * pc]);
    u32x4* const dst = reinterpret_cast<u32x4*>(out + (int64_t)r * sn + PER * pc);
    if (r < rows) {
      if constexpr (NT)
        __builtin_nontemporal_store(v, dst);
      else
        *dst = v;
    }
  }
}

// The same for tiles whose rows are not evenly spaced in memory (rows of
// different sequences and heads): row r of the staging tile goes to
// out + offs[r] (elements), or nowhere when offs[r] < 0.  `offs` is LDS the
// wave filled before the call.
template <typename T, int D, int SRS, bool NT = (EXATTN_NT_OUT != 0)>
__device__ __forceinline__ void store_staged_rows_at(const T* stage, T* out,
                                                     const int64_t* offs, int lane) {
  constexpr int PER = 16 / (int)sizeof(T), PPR = D / PER, NP = 32 * PPR / 64;
  static_assert(D % PER == 0 && 32 * PPR % 64 == 0, "whole 16-byte pieces, whole instructions");
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e = 64 * j + lane, r = e / PPR, pc = e % PPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[r * SRS + PER * pc]);
    const int64_t off = offs[r];
    u32x4* const dst = reinterpret_cast<u32x4*>(out + off + PER * pc);
    if (off >= 0) {
      if constexpr (NT)
        __builtin_nontemporal_store(v, dst);
      else
        *dst = v;
    }
  }
}

// The hardware dispatches workgroup i of a launch to XCD i % 8.  Renumber
// so that each XCD runs a contiguous range of logical workgroups: logical
// neighbours (tiles of one head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = i & 7, k = i >> 3;
  return x * q + (x < r ? x : r) + k;
}

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct io<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p) { return (float)*p; }
  static __device__ __forceinline__ void st(bf16* p, float v) { *p = (bf16)v; }
};

}  // namespace exattn

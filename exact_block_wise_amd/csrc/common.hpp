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

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// value of the other half-wave (lane ^ 32)
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

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

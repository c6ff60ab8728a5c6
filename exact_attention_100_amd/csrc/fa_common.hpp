// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the CDNA4 bf16 / fp32 matrix-core (MFMA) operations, fast
// exp2 / log2, bf16 packing and the workgroup -> tile schedule.
//
// MFMA register layouts used throughout (64-lane wavefront, 32x32 output):
//   A operand (32 x K):  lane l holds row (l % 32); its K values are the slots
//                        of lane group g = l / 32.
//   B operand (K x 32):  lane l holds column (l % 32), slots of group g.
//   C / D (32 x 32 f32): lane l holds column (l % 32); register r holds row
//                        8 * (r / 4) + 4 * g + (r % 4).
// Which K index a (group, slot) pair stands for is our choice, as long as the
// A and B operands of one instruction make the same choice; every kernel
// documents the choice it makes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16)
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, f32) += A(32x2, f32) * B(2x32, f32); lane group g holds K index g.
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round two floats to bf16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Eight floats -> bf16x8 operand (element i = f[i]).
__device__ __forceinline__ bf16x8 pack_bf16x8(float f0, float f1, float f2, float f3, float f4,
                                              float f5, float f6, float f7) {
  u32x4 u;
  u[0] = pack_bf16x2(f0, f1);
  u[1] = pack_bf16x2(f2, f3);
  u[2] = pack_bf16x2(f4, f5);
  u[3] = pack_bf16x2(f6, f7);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 concat_bf16x4(bf16x4 lo, bf16x4 hi) {
  u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  u32x4 u;
  u[0] = a[0];
  u[1] = a[1];
  u[2] = b[0];
  u[3] = b[1];
  return __builtin_bit_cast(bf16x8, u);
}

// Value held by lane (l ^ 32): the lane holding the same MFMA column in the
// other lane group.
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

// Build the low/high bf16 halves of four packed bf16 pairs into two 4-element
// rows: in[j] = (x_j, y_j) -> xs = (x_0..x_3), ys = (y_0..y_3).
__device__ __forceinline__ void split_pairs4(uint32_t in0, uint32_t in1, uint32_t in2, uint32_t in3,
                                             u32x2& xs, u32x2& ys) {
  xs[0] = (in0 & 0xFFFFu) | (in1 << 16);
  xs[1] = (in2 & 0xFFFFu) | (in3 << 16);
  ys[0] = (in0 >> 16) | (in1 & 0xFFFF0000u);
  ys[1] = (in2 >> 16) | (in3 & 0xFFFF0000u);
}

// Workgroup -> (instance, tile) schedule. Consecutive workgroup ids are handed
// to the 8 XCDs in turn; when the instance count allows it, all tiles of one
// (batch, head) instance go to the same XCD so its K/V (or Q/dO) re-reads hit
// that XCD's L2. Tiles are issued in `rank` order; the caller turns the rank
// into a tile index (e.g. heaviest tile first).
__device__ __forceinline__ void schedule_tile(int bid, int n_inst, int n_tiles, int& inst, int& rank) {
  if ((n_inst & 7) == 0) {
    const int xcd = bid & 7, idx = bid >> 3, per = n_inst >> 3;
    rank = idx / per;
    inst = xcd * per + (idx - rank * per);
  } else {
    rank = bid / n_inst;
    inst = bid - rank * n_inst;
  }
  (void)n_tiles;
}

}  // namespace fa

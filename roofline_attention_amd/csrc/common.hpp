// Device-side building blocks shared by the gfx950 attention kernels: vector types, bf16
// conversion, the MFMA wrappers and wave-level exchanges.
//
// MFMA register layouts used throughout (CDNA3/CDNA4 matrix-core conventions, wave64):
//   v_mfma_f32_32x32x16_bf16, D(32x32) += A(32x16) * B(16x32):
//     A: lane l holds row  (l % 32) and 8 consecutive k values of k-group (l / 32);
//     B: lane l holds col  (l % 32) and the same 8 k values of k-group (l / 32);
//     D: lane l holds col  (l % 32) and rows 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
// Only the row/col placement of A, B and D is relied on. Which physical k an element slot
// carries does not matter as long as A and B use the same slot for the same logical k, which
// every kernel here guarantees by construction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// float -> bf16, round to nearest even (gfx950 lowers this to v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ float shfl_xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

// max(a, b, c) in one v_maximum3_f32 (NaN-propagating maximum; no quieting of the inputs).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// acc + a + b for two bf16 values, in one v_dot2c_f32_bf16 against (1, 1).
__device__ __forceinline__ float bf16_pair_sum(bf16 a, bf16 b, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t x = {a, b};
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(x, ones, acc, false);
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));  // xor 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));  // xor 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true)); // half mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true)); // mirror
  return x;
}

// Maps a linear workgroup id so that consecutive logical work items run on the same XCD.
// Workgroups are handed to the 8 XCDs round-robin, so hardware slot L lands on XCD L % 8;
// giving XCD x the logical range [x*per, (x+1)*per) keeps work that shares K/V in one L2.
__device__ __forceinline__ int xcd_remap(int L, int total) {
  constexpr int kXcd = 8;
  if (total % kXcd != 0) return L;
  const int per = total / kXcd;
  return (L % kXcd) * per + L / kXcd;
}

// Items that share data come in groups of `ipg` consecutive indices (e.g. the query heads and
// tiles of one KV head of one sequence). Workgroup slot L runs on XCD L % 8; this mapping gives XCD
// x the groups x, x + 8, x + 16, ..., so every XCD receives the same share of every sequence
// whatever the sequences' lengths, while a group stays on one XCD's L2. (A contiguous split of
// the item range, as xcd_remap makes, hands whole sequences to single XCDs.)
__device__ __forceinline__ int xcd_group_remap(int L, int total, int ipg) {
  constexpr int kXcd = 8;
  if (ipg <= 0 || total % ipg != 0 || (total / ipg) % kXcd != 0) return L;
  const int x = L % kXcd;
  const int j = L / kXcd;
  return ((j / ipg) * kXcd + x) * ipg + j % ipg;
}

}  // namespace ra

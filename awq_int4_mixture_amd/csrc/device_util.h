// Device helpers shared by the stage and router kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq_moe {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Cross-lane sums in the VALU (DPP row operations and lane shuffles), no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;

// Sum four per-lane values over the 16 lanes that share lane bits 0..1 (one
// column quad of a wave): two DPP row rotations sum within each 16-lane row
// in the VALU; then a reduce-scatter across rows: the xor-16 exchange trades
// two of the four values, the xor-32 exchange one, so lane l ends with the
// full sum of value 2*b4 + b5 (b4, b5 = lane bits 4, 5). The lanes with
// (lane & 12) == 0 carry the four results of their quad.
__device__ __forceinline__ float sum4_lane_bits_2to5(float p0, float p1, float p2, float p3) {
  p0 += dpp<kRowRor4>(p0);
  p1 += dpp<kRowRor4>(p1);
  p2 += dpp<kRowRor4>(p2);
  p3 += dpp<kRowRor4>(p3);
  p0 += dpp<kRowRor8>(p0);
  p1 += dpp<kRowRor8>(p1);
  p2 += dpp<kRowRor8>(p2);
  p3 += dpp<kRowRor8>(p3);
  const int lane = threadIdx.x & 63;
  const bool b4 = (lane & 16) != 0, b5 = (lane & 32) != 0;
  float k0 = b4 ? p2 : p0, k1 = b4 ? p3 : p1;
  k0 += __shfl_xor(b4 ? p0 : p2, 16);
  k1 += __shfl_xor(b4 ? p1 : p3, 16);
  float k = b5 ? k1 : k0;
  k += __shfl_xor(b5 ? k0 : k1, 32);
  return k;
}

// Sum over aligned groups of 8 lanes (lane bits 0..2); every lane gets the sum.
__device__ __forceinline__ float sum_lane_bits_0to2(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowHalfMirror>(v);
  return v;
}

// Sum over the wave with the lane pairs of an xor butterfly over offsets
// 32, 16, 8, 4, 2, 1 (every lane gets the sum). After the offsets above 2^k
// the value is the same on lanes that differ only above bit k, so any source
// lane with bit k flipped and bits below k equal gives the same sum: the
// row rotations and quad permutes stand in for offsets 8, 4, 2, 1.
__device__ __forceinline__ float wave_sum_xor_order(float v) {
  v += __shfl_xor(v, 32);
  v += __shfl_xor(v, 16);
  v += dpp<kRowRor8>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kQuadSwap1>(v);
  return v;
}

}  // namespace awq_moe

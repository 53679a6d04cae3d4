// Device helpers of the q8_1 quantization shared by the quantize prepass and the GEMM for few
// tokens that quantizes its own activations (one copy of the arithmetic, so both produce the
// same bytes): the per-value rounding and the reductions over the lanes that own a block.
#pragma once
#include "mmq_internal.h"

namespace mmq {

__device__ __forceinline__ int quant1(float x, float id) {
  const float p = x * id;
  if (p != p) return 0;  // 0 * inf, only when 1/d overflowed for a block of tiny values
  return (int)fminf(fmaxf(roundf(p), -127.0f), 127.0f);
}

// Reductions over the 8 lanes of a group with DPP moves: swap neighbours, swap pairs, then
// mirror within the 8 lanes, after which every lane holds the group's result.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7 - i within 8 lanes
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, __int_as_float(dpp<kSwap1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp<kSwap2>(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp<kHalfMirror>(__float_as_int(v))));
}
__device__ __forceinline__ int group_sum(int v) {
  v += dpp<kSwap1>(v);
  v += dpp<kSwap2>(v);
  return v + dpp<kHalfMirror>(v);
}

}  // namespace mmq

// q8_1 quantize prepass: f32 activations -> int8 blocks of 32 with an f16 scale and the
// integer block sum, the format of the r15 page ("f32-accumulate mma probe + rank-1 term2
// rescale", section 2.1), computed "for free" by the prepass as on that page (section 2.1).
// It also writes the GEMM's planes, so that the GEMM stages them with direct-to-LDS loads
// and never converts: da as f32 in block-major order, and the folded row factor da*sa of
// term2 (r16 page, "Narrow kernel gets the rank-1 fold", section 2.1) as three bf16 pieces
// that sum to it exactly, grouped per super-block of 8 blocks for the GEMM's bf16 matrix
// instruction. HBM-bound: 4 bytes read and about 1.44 bytes written per element.
//
// Mapping: 8 lanes own one 32-element block (one float4 each), so a wavefront covers 8
// consecutive blocks = 1 KiB of contiguous input; the max and the sum are reduced with
// xor-shuffles inside the 8-lane group.
#include "mmq_internal.h"

namespace mmq {
namespace {

__device__ __forceinline__ int quant1(float x, float id) {
  const float p = x * id;
  if (p != p) return 0;  // 0 * inf, only when 1/d overflowed for a block of tiny values
  return (int)fminf(fmaxf(roundf(p), -127.0f), 127.0f);
}

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float4* __restrict__ x,
                                                            uint32_t* __restrict__ qs,
                                                            uint32_t* __restrict__ ds,
                                                            float* __restrict__ da_plane,
                                                            uint16_t* __restrict__ pieces,
                                                            int64_t nblocks, int M, int kb) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 3;      // all 8 lanes of a group share blk
  const bool ok = blk < nblocks;
  const float4 v = ok ? x[t] : make_float4(0.f, 0.f, 0.f, 0.f);

  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 8));

  const float d = amax / 127.0f;                 // IEEE division
  const float id = d > 0.0f ? 1.0f / d : 0.0f;   // IEEE reciprocal (division)
  const int q0 = quant1(v.x, id), q1 = quant1(v.y, id);
  const int q2 = quant1(v.z, id), q3 = quant1(v.w, id);

  int sum = q0 + q1 + q2 + q3;
  sum += __shfl_xor(sum, 1, 8);
  sum += __shfl_xor(sum, 2, 8);
  sum += __shfl_xor(sum, 4, 8);

  if (ok) {
    qs[t] = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) |
            ((uint32_t)(q2 & 0xFF) << 16) | ((uint32_t)(q3 & 0xFF) << 24);
    if ((threadIdx.x & 7) == 0) {
      const _Float16 dh = (_Float16)d;  // RNE
      const uint32_t hbits = __builtin_bit_cast(uint16_t, dh);
      ds[blk] = hbits | ((uint32_t)(sum & 0xFFFF) << 16);
      // the GEMM's planes: da block-major, and da * sa (exact in f32) as bf16 pieces
      const int64_t row = blk / kb, b = blk - row * kb;
      const float da = (float)dh;
      da_plane[b * M + row] = da;
      uint16_t p[3];
      bf16_split3(da * (float)sum, p[0], p[1], p[2]);
      uint16_t* dst = pieces + ((b >> 3) * 3 * (int64_t)M + row) * 8 + (b & 7);
#pragma unroll
      for (int j = 0; j < 3; ++j) dst[j * (int64_t)M * 8] = p[j];
    }
  }
}

}  // namespace

hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, void* q8, hipStream_t s) {
  const int64_t nblocks = M * (K / 32);
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  uint8_t* base = static_cast<uint8_t*>(q8);
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(x), reinterpret_cast<uint32_t*>(base),
                     reinterpret_cast<uint32_t*>(base + M * K),
                     reinterpret_cast<float*>(base + q8_planes_offset(M, K)),
                     reinterpret_cast<uint16_t*>(base + q8_pieces_offset(M, K)), nblocks,
                     (int)M, (int)(K / 32));
  return hipGetLastError();
}

}  // namespace mmq

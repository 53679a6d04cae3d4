// Offline q4_K repack: GGUF-layout super-blocks -> one 6656-byte record per (32-row weight
// tile, super-block) laid out for the GEMM's operand loads (layout in include/mmq.h).
// The q4_K fields are those of the r15 page ("f32-accumulate mma probe + rank-1 term2
// rescale", section 2.1); the scale expansion dsv = d*sc, dmv = -(dmin*m) is the B-staging
// step quoted there, moved to load time. dmv is stored as three bf16 pieces that sum to it
// exactly, the operand form of the GEMM's bf16 matrix instruction for term2.
#include "mmq_internal.h"

namespace mmq {
namespace {

__device__ __forceinline__ float f16_to_f32(uint32_t lo, uint32_t hi) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(lo | (hi << 8)));
}

// 6-bit scale and min of sub-block b from the 12 packed scale bytes (GGUF q4_K packing).
__device__ __forceinline__ void scale_min(const uint8_t* s, int b, int& sc, int& m) {
  if (b < 4) {
    sc = s[b] & 63;
    m = s[b + 4] & 63;
  } else {
    sc = (s[b + 4] & 15) | ((s[b - 4] >> 6) << 4);
    m = (s[b + 4] >> 4) | ((s[b] >> 6) << 4);
  }
}

// One workgroup per (tile, super-block); 256 threads.
__global__ __launch_bounds__(256) void repack_q4_K_kernel(const uint8_t* __restrict__ w,
                                                          uint8_t* __restrict__ out, int N,
                                                          int nsb) {
  const int tile = blockIdx.x / nsb;
  const int sb = blockIdx.x % nsb;
  const int tid = threadIdx.x;
  uint8_t* rec = out + ((size_t)tile * nsb + sb) * kRepTileBytes;

  {  // nibbles: 256 chunks of 16 bytes, chunk c = g*64 + h*32 + j
    const int g = tid >> 6, h = (tid >> 5) & 1, j = tid & 31;
    const int row = tile * kRepTileRows + j;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < N)
      v = *reinterpret_cast<const uint4*>(w + ((size_t)row * nsb + sb) * 144 + 16 + 32 * g +
                                          16 * h);
    reinterpret_cast<uint4*>(rec)[tid] = v;
  }
  {  // scales: thread = (b, j)
    const int b = tid >> 5, j = tid & 31;
    const int row = tile * kRepTileRows + j;
    float dsv = 0.0f, dmv = 0.0f;
    if (row < N) {
      const uint8_t* blk = w + ((size_t)row * nsb + sb) * 144;
      const float d = f16_to_f32(blk[0], blk[1]);
      const float dmin = f16_to_f32(blk[2], blk[3]);
      int sc, m;
      scale_min(blk + 4, b, sc, m);
      dsv = d * (float)sc;
      dmv = -(dmin * (float)m);
    }
    reinterpret_cast<float*>(rec + kRepNibBytes)[b * 32 + j] = dsv;
    uint16_t p[3];
    bf16_split3(dmv, p[0], p[1], p[2]);
    uint16_t* pc = reinterpret_cast<uint16_t*>(rec + kRepNibBytes + kRepDsvBytes);
#pragma unroll
    for (int i = 0; i < 3; ++i) pc[(i * 32 + j) * 8 + b] = p[i];
  }
}

}  // namespace

hipError_t launch_repack_q4_K(const void* w, int64_t N, int64_t K, void* w_rep, hipStream_t s) {
  const int64_t nsb = K / 256;
  const int64_t ntiles = (N + kRepTileRows - 1) / kRepTileRows;
  hipLaunchKernelGGL(repack_q4_K_kernel, dim3((unsigned)(ntiles * nsb)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(w), static_cast<uint8_t*>(w_rep), (int)N,
                     (int)nsb);
  return hipGetLastError();
}

}  // namespace mmq

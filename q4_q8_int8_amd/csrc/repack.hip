// Offline weight repacks: GGUF-layout q4_K (and q6_K, below) super-blocks -> one record per
// (32-row weight tile, super-block) laid out for the kernels' operand loads (layouts in
// include/mmq.h).
// The q4_K record keeps the fields of the r15 page ("f32-accumulate mma probe + rank-1 term2
// rescale", section 2.1) as the GGUF block holds them: the nibbles, regrouped so that one
// 16-byte load per lane feeds a matrix instruction, and each row's 16-byte header (d, dmin
// and the packed 6-bit sc, m), unchanged. The kernels expand dsv = d*sc and dmv = -(dmin*m)
// from the header when they stage a super-block, the B-staging step quoted there, so the
// record is 4.5 bits per weight, the size of the GGUF blocks themselves.
#include "mmq_internal.h"

namespace mmq {
namespace {

__device__ __forceinline__ float f16_to_f32(uint32_t lo, uint32_t hi) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(lo | (hi << 8)));
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
  if (tid < kRepTileRows) {  // headers: thread = row j, the block's first 16 bytes
    const int row = tile * kRepTileRows + tid;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < N) v = *reinterpret_cast<const uint4*>(w + ((size_t)row * nsb + sb) * 144);
    reinterpret_cast<uint4*>(rec + kRepNibBytes)[tid] = v;
  }
}

// q6_K (GGUF layout, 210 bytes per super-block: 128 bytes of low nibbles, 64 bytes of high
// 2-bit pairs, 16 int8 group scales, f16 d) -> one 10240-byte record per (32-row tile,
// super-block): the signed values u - 32 as int8 in the GEMM's operand order, then the group
// scales expanded to dsv = d * sc (f32, exact: an f16 times an 8-bit integer).
// Value v of the super-block (v = 128*half + 32*q + l) keeps its low 4 bits in byte
// 64*half + 32*(q % 2) + l (the high nibble when q >= 2) and its high 2 bits in bits 2q..2q+1
// of byte 128 + 32*half + l.
__global__ __launch_bounds__(256) void repack_q6_K_kernel(const uint8_t* __restrict__ w,
                                                          uint8_t* __restrict__ out, int N,
                                                          int nsb) {
  const int tile = blockIdx.x / nsb;
  const int sb = blockIdx.x % nsb;
  const int tid = threadIdx.x;
  uint8_t* rec = out + ((size_t)tile * nsb + sb) * kRep6TileBytes;
  // values: 512 chunks of 16 bytes, chunk c = (b*2 + h)*32 + j holds values 32b + 16h + e
  // (e = 0..15) of row 32*tile + j
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = tid + 256 * k;
    const int b = c >> 6, h = (c >> 5) & 1, j = c & 31;
    const int row = tile * kRepTileRows + j;
    uint8_t v[16];
    if (row < N) {
      const uint8_t* blk = w + ((size_t)row * nsb + sb) * kQ6KBlockBytes;
      const int half = b >> 2, q = b & 3;
      const uint8_t* ql = blk + 64 * half + 32 * (q & 1) + 16 * h;
      const uint8_t* qh = blk + 128 + 32 * half + 16 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int lo = q < 2 ? (ql[e] & 15) : (ql[e] >> 4);
        const int hi = (qh[e] >> (2 * q)) & 3;
        v[e] = (uint8_t)(int8_t)((lo | (hi << 4)) - 32);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = 0;
    }
    uint4 o;
    o.x = v[0] | (v[1] << 8) | (v[2] << 16) | ((uint32_t)v[3] << 24);
    o.y = v[4] | (v[5] << 8) | (v[6] << 16) | ((uint32_t)v[7] << 24);
    o.z = v[8] | (v[9] << 8) | (v[10] << 16) | ((uint32_t)v[11] << 24);
    o.w = v[12] | (v[13] << 8) | (v[14] << 16) | ((uint32_t)v[15] << 24);
    reinterpret_cast<uint4*>(rec)[c] = o;
  }
  // scales: dsv[g][j] = d * sc_g of row 32*tile + j, 512 values
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = tid + 256 * k;
    const int g = c >> 5, j = c & 31;
    const int row = tile * kRepTileRows + j;
    float dsv = 0.0f;
    if (row < N) {
      const uint8_t* blk = w + ((size_t)row * nsb + sb) * kQ6KBlockBytes;
      dsv = f16_to_f32(blk[208], blk[209]) * (float)(int8_t)blk[192 + g];
    }
    reinterpret_cast<float*>(rec + kRep6ValBytes)[c] = dsv;
  }
}

}  // namespace

hipError_t launch_repack_q6_K(const void* w, int64_t N, int64_t K, void* w_rep, hipStream_t s) {
  const int64_t nsb = K / 256;
  const int64_t ntiles = (N + kRepTileRows - 1) / kRepTileRows;
  hipLaunchKernelGGL(repack_q6_K_kernel, dim3((unsigned)(ntiles * nsb)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(w), static_cast<uint8_t*>(w_rep), (int)N,
                     (int)nsb);
  return hipGetLastError();
}

hipError_t launch_repack_q4_K(const void* w, int64_t N, int64_t K, void* w_rep, hipStream_t s) {
  const int64_t nsb = K / 256;
  const int64_t ntiles = (N + kRepTileRows - 1) / kRepTileRows;
  hipLaunchKernelGGL(repack_q4_K_kernel, dim3((unsigned)(ntiles * nsb)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(w), static_cast<uint8_t*>(w_rep), (int)N,
                     (int)nsb);
  return hipGetLastError();
}

}  // namespace mmq

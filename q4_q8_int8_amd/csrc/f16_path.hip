// The f16 comparator path's own kernels: the activation conversion f32 -> f16 and the
// dequantization of q4_K weights to an f16 matrix (the dq_f16 step of the audit page "Round 31
// Track C Audit: dq_f16 & DW<F>", sections 1-2, for the q4_K fields of the r15 page, "f32-
// accumulate mma probe + rank-1 term2 rescale", section 2.1). Both are bound by HBM traffic:
// each thread moves whole 16-byte words, and consecutive threads touch consecutive words.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mmq_internal.h"

namespace mmq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kQ4KBlockBytes = 144;  // bytes of one q4_K super-block

// f32 -> f16 with the hardware conversion: round to nearest even in the default float mode,
// f16 subnormals kept, overflow to infinity.
__device__ inline h8 to_h8(float4 a, float4 b) {
  h8 h;
  h[0] = (_Float16)a.x; h[1] = (_Float16)a.y; h[2] = (_Float16)a.z; h[3] = (_Float16)a.w;
  h[4] = (_Float16)b.x; h[5] = (_Float16)b.y; h[6] = (_Float16)b.z; h[7] = (_Float16)b.w;
  return h;
}

// One thread per 8 consecutive values (two 16-byte loads, one 16-byte store), grid-stride over
// the flat array; the last n % 8 values are converted one by one by one thread.
__global__ __launch_bounds__(kThreads) void convert_f32_f16_kernel(
    const float* __restrict__ x, _Float16* __restrict__ y, int64_t n) {
  const int64_t groups = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += stride) {
    const float4* src = reinterpret_cast<const float4*>(x) + 2 * g;
    const float4 a = src[0];
    const float4 b = src[1];
    reinterpret_cast<h8*>(y)[g] = to_h8(a, b);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t i = groups << 3; i < n; ++i) y[i] = (_Float16)x[i];
}

// q4_K super-block (144 bytes): f16 d at byte 0, f16 dmin at byte 2, the 12 bytes of 6-bit
// sub-block scales and mins at bytes 4..15, then 4 groups of 32 nibble bytes: byte e of group
// g holds element e of sub-block 2g in its low nibble and of sub-block 2g+1 in its high one.
// With s[0..11] the scale bytes (block bytes 4..15), the 6-bit fields of sub-block b are
//   b < 4:   sc = s[b] & 63,                          m = s[b+4] & 63
//   b >= 4:  sc = (s[b+4] & 15) | (s[b-4] >> 6) << 4,  m = (s[b+4] >> 4) | (s[b] >> 6) << 4
__device__ inline void scale_min(const uint8_t* s, int b, int& sc, int& m) {
  if (b < 4) {
    sc = s[b] & 63;
    m = s[b + 4] & 63;
  } else {
    sc = (s[b + 4] & 15) | ((s[b - 4] >> 6) << 4);
    m = (s[b + 4] >> 4) | ((s[b] >> 6) << 4);
  }
}

// Per super-block 16 threads; thread t takes the 8 nibble bytes 8(t%4).. of group g = t/4 and
// writes 8 values of sub-block 2g and 8 of sub-block 2g+1 (two 16-byte stores). Every value is
// fma(dsv, v, dmv) in float32 -- dsv*v is exact, so this is the sum rounded once -- then
// rounded to f16.
__global__ __launch_bounds__(kThreads) void dequantize_q4_K_f16_kernel(
    const uint8_t* __restrict__ w, _Float16* __restrict__ out, int64_t nblocks) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < nblocks * 16;
       idx += stride) {
    const int64_t blk = idx >> 4;
    const int t = (int)(idx & 15);
    const int g = t >> 2, e0 = (t & 3) * 8;
    const uint8_t* p = w + blk * kQ4KBlockBytes;
    const uint4 head = *reinterpret_cast<const uint4*>(p);
    const uint2 nib = *reinterpret_cast<const uint2*>(p + 16 + 32 * g + e0);
    uint8_t s[12];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (uint8_t)(head.y >> (8 * i));
      s[4 + i] = (uint8_t)(head.z >> (8 * i));
      s[8 + i] = (uint8_t)(head.w >> (8 * i));
    }
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(head.x & 0xFFFF));
    const float dmin = (float)__builtin_bit_cast(_Float16, (uint16_t)(head.x >> 16));
    int sc0, m0, sc1, m1;
    scale_min(s, 2 * g, sc0, m0);
    scale_min(s, 2 * g + 1, sc1, m1);
    const float dsv0 = d * (float)sc0, dmv0 = -(dmin * (float)m0);
    const float dsv1 = d * (float)sc1, dmv1 = -(dmin * (float)m1);
    h8 lo, hi;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t byte = ((i < 4 ? nib.x : nib.y) >> (8 * (i & 3))) & 0xFF;
      float a = __builtin_fmaf(dsv0, (float)(byte & 15), dmv0);
      float b = __builtin_fmaf(dsv1, (float)(byte >> 4), dmv1);
      // the f32 values exist before their conversion: left to itself the compiler fuses the
      // conversion into a mixed-precision fma with an f16 result, whose rounding of the exact
      // sum is not the two-step rounding defined above
      asm volatile("" : "+v"(a), "+v"(b));
      lo[i] = (_Float16)a;
      hi[i] = (_Float16)b;
    }
    // super-block s of row j starts at element j*K + 256*s = 256*blk
    _Float16* o = out + blk * 256 + 64 * g + e0;
    *reinterpret_cast<h8*>(o) = lo;
    *reinterpret_cast<h8*>(o + 32) = hi;
  }
}

unsigned grid_for(int64_t items) {
  // enough workgroups to cover the items, at most 64 per compute unit of a 256-unit device;
  // the kernels loop over the rest
  const int64_t need = (items + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 64;
  return (unsigned)(need < cap ? (need > 0 ? need : 1) : cap);
}

}  // namespace

hipError_t launch_convert_f32_f16(const float* x, int64_t n, void* y, hipStream_t s) {
  hipLaunchKernelGGL(convert_f32_f16_kernel, dim3(grid_for(n >> 3)), dim3(kThreads), 0, s, x,
                     static_cast<_Float16*>(y), n);
  return hipGetLastError();
}

hipError_t launch_dequantize_q4_K_f16(const void* w, int64_t N, int64_t K, void* out,
                                      hipStream_t s) {
  const int64_t nblocks = N * (K / 256);
  hipLaunchKernelGGL(dequantize_q4_K_f16_kernel, dim3(grid_for(nblocks * 16)), dim3(kThreads), 0,
                     s, static_cast<const uint8_t*>(w), static_cast<_Float16*>(out), nblocks);
  return hipGetLastError();
}

}  // namespace mmq

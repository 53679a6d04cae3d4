// Device-side helpers shared by the GEMM kernels of libmmq (not part of the ABI): vector
// types, raw buffer descriptors, and the direct-to-LDS load.
#pragma once

#include "mmq_internal.h"

namespace mmq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer descriptor over [p, p + bytes): reads at offsets >= bytes return zero.
// The last descriptor word is the gfx9-family default data format (32-bit, untyped).
static __device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
static __device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
static __device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
static __device__ __forceinline__ float2 buf_load_f32x2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
// The same descriptor as four SGPRs, for the direct-to-LDS load below.
static __device__ __forceinline__ v4i make_rsrc_sgpr(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}
// LDS byte address of a pointer into a __shared__ array. Taken once from the array itself it
// is a constant; converting a pointer computed at run time instead costs a null check and
// an aperture lookup at every use.
static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)p);
}
// 16 bytes per lane from the buffer at `off` into LDS at byte address lds + 16 * lane (lds is
// wave-uniform); completion is tracked by the vector-memory counter and waited for
// explicitly before the barrier that ends a stage. The instruction is issued from inline
// assembly on purpose: the compiler cannot tell which LDS bytes such a load writes, so for
// the intrinsic it waits for every outstanding one before the next LDS read, which would
// stall each wavefront on its own prefetch at the start of every stage. The asm declares no
// memory effects on purpose too: it only writes the stage buffer that nothing reads until
// after the explicit wait and the barrier (both ordered with the asm), and so the compiler
// stays free to schedule the current stage's LDS reads around it.
// M0 is declared clobbered rather than saved and restored (two scalar instructions per load).
// The compiler reserves M0 and warns that it need not honour such a clobber, so this relies on
// the compiler never using M0 itself in the kernels that call the helper; a CPU test compiles
// them and checks exactly that. The warning is silenced here and only here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
static __device__ __forceinline__ void dma16(v4i r, uint32_t lds, uint32_t off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(r)
      : "m0");
}
#pragma clang diagnostic pop

// Output tile (ti, tj) of workgroup `tile` in a grid of gm token tiles x gmn / gm weight
// tiles. With xbm > 0 (xcd_block), XCD x = tile % 8 works through its own block of xbm token
// tiles by gmn / 8 / xbm weight tiles, xgm such blocks along the tokens, so that its L2
// fetches each weight tile of its block once; in the plain order (xbm = 0, token tiles
// fastest) the workgroups sharing a weight tile go to different XCDs.
static __device__ __forceinline__ void xcd_tile(int tile, int gm, int gmn, int xbm, int xgm,
                                                int& ti, int& tj) {
  if (xbm > 0) {
    const int x = tile & 7, k = tile >> 3;
    ti = (x % xgm) * xbm + k % xbm;
    tj = (x / xgm) * ((gmn >> 3) / xbm) + k / xbm;
  } else {
    ti = tile % gm;
    tj = tile / gm;
  }
}

// Weight scales of one row's q4_K super-block, from the 16-byte header the repacked record
// keeps per row (word 0: f16 d in bits 0..15, f16 dmin in bits 16..31; words 1..3: the 12
// packed scale bytes s0..s11), for the four sub-blocks 4*half .. 4*half + 3. GGUF packing:
// sub-block b < 4 has sc = s[b] & 63 and m = s[b+4] & 63; b >= 4 has the low four bits of sc
// and m in the low and high nibble of s[b+4] and their top two bits in bits 6..7 of s[b-4]
// and s[b]. Four bytes at a time: dsv[k] = d * sc and dmv[k] = -(dmin * m), each exact in f32
// (an f16 times a 6-bit integer).
static __device__ __forceinline__ void q4k_scales(v4i hdr, bool half, float (&dsv)[4],
                                                  float (&dmv)[4]) {
  const uint32_t w0 = (uint32_t)hdr[0], s0 = (uint32_t)hdr[1], s1 = (uint32_t)hdr[2],
                 s2 = (uint32_t)hdr[3];
  const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 & 0xFFFFu));
  const float dmin = (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 >> 16));
  // both halves' bytes, then a blend (a select of lane-varying operands would branch)
  const uint32_t hm = 0u - (uint32_t)half;
  const uint32_t sc = (((s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u)) & hm) |
                      ((s0 & 0x3F3F3F3Fu) & ~hm);
  const uint32_t mm = ((((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u)) & hm) |
                      ((s1 & 0x3F3F3F3Fu) & ~hm);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    dsv[k] = d * (float)((sc >> (8 * k)) & 0xFFu);
    dmv[k] = -(dmin * (float)((mm >> (8 * k)) & 0xFFu));
  }
}

// Three bfloat16 pieces that sum exactly to a finite float v, by truncation: p0 = the top 16
// bits of v, p1 = the top 16 bits of r = v - p0, p2 = r - p1. Both differences are exact (each
// drops leading bits of the significand), and p2 keeps at most the last 8 of v's 24
// significant bits, so it is a bfloat16 value too. Returned as the float bit patterns whose
// high halves are the pieces (their low halves are not part of the pieces).
static __device__ __forceinline__ void bf16_trunc3(float v, uint32_t& p0, uint32_t& p1,
                                                   uint32_t& p2) {
  p0 = __builtin_bit_cast(uint32_t, v);
  const float r = v - __builtin_bit_cast(float, p0 & 0xFFFF0000u);
  p1 = __builtin_bit_cast(uint32_t, r);
  p2 = __builtin_bit_cast(uint32_t, r - __builtin_bit_cast(float, p1 & 0xFFFF0000u));
}

// The high halves of two float bit patterns as one word: lo's in bits 0..15, hi's above.
static __device__ __forceinline__ uint32_t pack_hi16(uint32_t lo, uint32_t hi) {
  return (lo >> 16) | (hi & 0xFFFF0000u);
}

// The weight scales of sub-blocks 4*half .. 4*half + 3 of row `row` (0..31) of a tile, as the
// MFMA kernels stage them in LDS at sw: dsv f32 [8][32], then the three bf16 pieces of dmv
// [3][32][8] (bf16_trunc3). The header must hold finite d and dmin.
static __device__ __forceinline__ void q4k_stage_scales(v4i hdr, int row, bool half,
                                                        uint8_t* sw) {
  float dsv[4], dmv[4];
  q4k_scales(hdr, half, dsv, dmv);
  const int b0 = 4 * (int)half;
  float* sd = reinterpret_cast<float*>(sw);
#pragma unroll
  for (int k = 0; k < 4; ++k) sd[(b0 + k) * 32 + row] = dsv[k];
  uint32_t p[4][3];
#pragma unroll
  for (int k = 0; k < 4; ++k) bf16_trunc3(dmv[k], p[k][0], p[k][1], p[k][2]);
  uint16_t* pc = reinterpret_cast<uint16_t*>(sw + kWDsvBytes);
#pragma unroll
  for (int i = 0; i < 3; ++i)
    *reinterpret_cast<uint2*>(pc + (i * 32 + row) * 8 + b0) =
        make_uint2(pack_hi16(p[0][i], p[1][i]), pack_hi16(p[2][i], p[3][i]));
}

}  // namespace mmq

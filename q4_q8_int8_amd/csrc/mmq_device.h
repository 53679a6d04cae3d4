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

}  // namespace mmq

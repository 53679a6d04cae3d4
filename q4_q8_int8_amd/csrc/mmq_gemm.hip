// q4_K x q8_1 GEMM on gfx950: integer block dot products on v_mfma_i32_32x32x32_i8 and the
// two-term float rescale, as defined on the r15 page ("f32-accumulate mma probe + rank-1
// term2 rescale", section 2.1) with the row factor da*sa folded once per token row (r16
// page, "Narrow kernel gets the rank-1 fold", section 2.1).
//
// One 32x32x32 int8 MFMA is exactly one q8_1 block against one q4_K sub-block, so its i32
// result is S_ijb for a 32x32 (weight row, token) tile. The instruction has no float
// accumulator form (the integer-MMA fact of the r15 page, section 2.3, holds on gfx950 too),
// so every S is rescaled on the vector ALU:
//
//   D   = MFMA_i8(w, q, bias)       bias = 0x4B400000, so float(D) = 12582912 + S exactly
//   y   = fma(float(D), da, nb)     nb = -12582912 * da (exact), y = RN(S * da)
//   acc = fma(y, dsv, acc)          term1
//
// y equals float(S) * da bit for bit, without an int->float conversion instruction.
// term2 is rank-1 per block: the row factor dma = da * sa (exact in f32, written by the
// quantize prepass) times the column factor dmv. Summed over a pair of blocks it is a K=2
// outer product, which v_mfma_f32_32x32x2_f32 adds into the same accumulator. Per element
// the terms are added in a fixed order (term1 of each block, term2 of each pair of blocks),
// so results are deterministic and identical across tile variants.
//
// Operand orientation: MFMA rows (src0) are weight rows, columns (src1, one per lane) are
// tokens. Lane l holds token l%32 of a tile and, in its 16 accumulator registers r, the
// weight rows 8*(r/4) + 4*(l/32) + r%4. Per block, the token scale da is one float per lane
// and the weight scales dsv 16 floats per lane (lane-half broadcast), both read from LDS;
// dma and dmv for term2 are one float per lane per pair of blocks.
//
// Workgroup: NW wavefronts; wavefront w owns weight tile (32 rows) tn*NW + w for all
// BM = 32*TT tokens of the workgroup. Everything a super-block (256 k) needs from memory is
// staged one super-block ahead, while the current one is computed:
//   - into LDS by direct-to-LDS buffer loads (no registers, no conversion): the int8 token
//     tile in 272-byte rows (16 bytes of padding, so the 16-byte operand reads of 16
//     consecutive rows hit distinct banks and every LDS address is a per-lane base plus a
//     constant), the {da, dma} plane of the token tile, and each wavefront's dsv/dmv;
//   - into registers: the wavefront's nibbles, where the 64 lanes of one load read 1 KiB of
//     contiguous memory.
// Buffer loads take 32-bit offsets off wave-uniform descriptors; reads past the end of an
// operand return zero, which zeroes token rows past M and the padding slots. The stages
// alternate between two LDS buffers; one barrier per super-block separates them.
//
// On gfx950 the MFMA and the vector ALU of a SIMD largely take turns, so every instruction
// counts: the rescale is 2 FMAs per element-block and the int8 MFMA of step n+1 is issued
// before the rescale of step n.
#include "mmq_internal.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer descriptor over [p, p + bytes): reads at offsets >= bytes return zero.
// The last descriptor word is the gfx9-family default data format (32-bit, untyped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// 16 bytes per lane from the buffer at `off` into LDS at lds_base + 16 * lane (lds_base is
// wave-uniform); completion is tracked by the vector-memory counter.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base, 16, (int)off, 0, 0, 0);
}

template <int TT, int NW, bool STORE_S>
__global__ __launch_bounds__(NW * 64, NW >= 8 ? 1 : 2) void mmq_kernel(
    const int8_t* __restrict__ qs, const float2* __restrict__ planes,
    const uint8_t* __restrict__ wrep, void* __restrict__ out, int M, int N, int K, int gm,
    int tm0, int tn0, int i0, int i1, int j0, int j1) {
  constexpr int BM = 32 * TT;
  constexpr int NS = 8 * TT;                      // (block, token tile) steps per super-block
  constexpr int A_BYTES = BM * kRowStride;        // token tile
  constexpr int P_BYTES = BM * 64;                // {da, dma} [8][BM]
  constexpr int STAGE = A_BYTES + P_BYTES + NW * 2048;
  constexpr int A_SLOTS = BM * (kRowStride / 16);  // 16-byte slots of the token tile
  constexpr int A_DMA = (A_SLOTS + 63) / 64;       // wavefront-wide DMA instructions
  constexpr int A_PER_WAVE = (A_DMA + NW - 1) / NW;

  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int tm = tm0 + (int)(blockIdx.x % (unsigned)gm);
  const int tn = tn0 + (int)(blockIdx.x / (unsigned)gm);
  const int m0 = tm * BM;
  const int ntiles = (N + 31) >> 5;
  const int wt_raw = tn * NW + wave;
  const bool wt_ok = wt_raw < ntiles;
  const int wt = wt_ok ? wt_raw : ntiles - 1;  // idle wavefronts still stage and sync
  const int nsb = K >> 8;
  const int kb = K >> 5;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qs, (uint32_t)M * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(planes, (uint32_t)M * (uint32_t)kb * 8u);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wrep + (size_t)wt * nsb * kRepTileBytes, (uint32_t)nsb * kRepTileBytes);

  // Token-tile DMA slots of this lane: slot q = 64*k + lane holds chunk q % 17 of row q / 17;
  // chunk 16 is the row's padding and reads past the end (zero), as do rows past M.
  uint32_t a_off[A_PER_WAVE];
  bool a_act[A_PER_WAVE];
#pragma unroll
  for (int j = 0; j < A_PER_WAVE; ++j) {
    const int k = wave + j * NW;
    const int q = k * 64 + lane;
    const int row = q / 17, c = q - row * 17;
    a_act[j] = k < A_DMA && q < A_SLOTS;
    a_off[j] = c < 16 ? (uint32_t)(m0 + row) * (uint32_t)K + c * 16 : (uint32_t)M * (uint32_t)K;
  }
  auto issue_stage = [&](int s, int p) {
    uint8_t* st = smem + p * STAGE;
#pragma unroll
    for (int j = 0; j < A_PER_WAVE; ++j) {
      const int k = wave + j * NW;
      if (k < A_DMA && a_act[j]) dma16(rq, st + k * 1024, a_off[j] + (uint32_t)s * 256);
    }
    // {da, dma} of blocks 8s..8s+7 for rows m0..m0+BM-1: BM/2 lanes per block
#pragma unroll
    for (int b = wave; b < 8; b += NW)
      if (lane < BM / 2)
        dma16(rp, st + A_BYTES + b * BM * 8,
              (((uint32_t)s * 8 + b) * (uint32_t)M + m0) * 8u + lane * 16);
    // this wavefront's dsv [8][32] and dmv [8][32]
    uint8_t* sw = st + A_BYTES + P_BYTES + wave * 2048;
    dma16(rw, sw, (uint32_t)s * kRepTileBytes + kRepNibBytes + lane * 16);
    dma16(rw, sw + 1024, (uint32_t)s * kRepTileBytes + kRepNibBytes + 1024 + lane * 16);
  };
  auto load_nibbles = [&](int s, v4i (&raw)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      raw[g] = buf_load16(rw, (uint32_t)s * kRepTileBytes + g * 1024 + lane * 16);
  };

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;
  v16f acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  v4i rawn[4];
  issue_stage(0, 0);
  load_nibbles(0, rawn);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int s = 0; s < nsb; ++s) {
    const int p = s & 1;
    v4i raw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) raw[g] = rawn[g];
    if (s + 1 < nsb) {
      issue_stage(s + 1, p ^ 1);
      load_nibbles(s + 1, rawn);
    }

    const uint8_t* st = smem + p * STAGE;
    const uint8_t* sArow = st + l32 * kRowStride + h * 16;
    const float2* sP = reinterpret_cast<const float2*>(st + A_BYTES);
    const float* sWw = reinterpret_cast<const float*>(st + A_BYTES + P_BYTES + wave * 2048);
    auto wop_of = [&](int b) -> v4i {
      const v4i rr = raw[b >> 1];
      return (b & 1) ? ((rr >> 4) & 0x0F0F0F0F) : (rr & 0x0F0F0F0F);
    };
    auto top_of = [&](int n) -> v4i {  // token operand of step n: 16 int8 of row t*32+l32
      const int b = n / TT, t = n % TT;
      return *reinterpret_cast<const v4i*>(sArow + t * 32 * kRowStride + b * 32);
    };
    auto da_of = [&](int n) -> float { return sP[(n / TT) * BM + (n % TT) * 32 + l32].x; };
    auto dsv_of = [&](int b, float (&d)[16]) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = *reinterpret_cast<const float4*>(sWw + b * 32 + 8 * g + 4 * h);
        d[4 * g + 0] = a.x; d[4 * g + 1] = a.y; d[4 * g + 2] = a.z; d[4 * g + 3] = a.w;
      }
    };

    if constexpr (STORE_S) {
      // test path: every S of the window, straight from the MFMA
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const int b = n / TT, t = n % TT;
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(b), top_of(n), bias, 0, 0, 0);
        const int i = m0 + t * 32 + l32;
        if (wt_ok && i >= i0 && i < i1) {
          int32_t* S = static_cast<int32_t*>(out);
          const size_t plane = (size_t)(i1 - i0) * (size_t)(j1 - j0);
          const int bg = s * 8 + b;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = wt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (j >= j0 && j < j1)
              S[(size_t)bg * plane + (size_t)(i - i0) * (j1 - j0) + (j - j0)] = D[r] - kBiasBits;
          }
        }
      }
    } else {
      // Step n = b*TT + t. Entering step n: D(n) has been issued, the token operand of step
      // n+1 and da of step n are in registers; dsv[b & 1] holds block b's weight scales.
      float dsv[2][16];
      dsv_of(0, dsv[0]);
      v4i tnext = top_of(1 % NS);
      float da = da_of(0);
      v16i Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(0), top_of(0), bias, 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const int b = n / TT, t = n % TT;
        const v16i D = Dn;
        const float dac = da;
        if (n + 1 < NS) {
          Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of((n + 1) / TT), tnext, bias, 0, 0, 0);
          da = da_of(n + 1);
        }
        if (n + 2 < NS) tnext = top_of(n + 2);
        if (t == 0 && b + 1 < 8) dsv_of(b + 1, dsv[(b + 1) & 1]);
        const float nb = -kBiasF * dac;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = __builtin_fmaf(__int_as_float(D[r]), dac, nb);
          acc[t][r] = __builtin_fmaf(y, dsv[b & 1][r], acc[t][r]);
        }
        if (b & 1) {
          // term2 of blocks b-1 and b: lane l supplies dmv of weight row l%32 and dma of
          // token l%32 for block b-1+l/32, a K=2 outer product added on the matrix unit
          const float dmv = sWw[256 + (b - 1 + h) * 32 + l32];
          const float dma = sP[(b - 1 + h) * BM + t * 32 + l32].y;
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(dmv, dma, acc[t], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stage s+1 loads have landed
    __syncthreads();                // ... and everyone's; stage s is no longer read
  }

  if constexpr (!STORE_S) {
    if (!wt_ok) return;
    float* C = static_cast<float*>(out);
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int i = m0 + t * 32 + l32;
      if (i >= M) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = wt * 32 + 8 * g + 4 * h;
        float* p = C + (size_t)i * N + j;
        if (vec && j + 3 < N) {
          *reinterpret_cast<float4*>(p) =
              make_float4(acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2], acc[t][4 * g + 3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < N) p[e] = acc[t][4 * g + e];
        }
      }
    }
  }
}

template <int TT, int NW, bool STORE_S>
hipError_t launch_t(const void* q8, const void* w_rep, void* out, int64_t M, int64_t N,
                    int64_t K, int64_t gm, int64_t gn, int64_t tm0, int64_t tn0, int64_t i0,
                    int64_t i1, int64_t j0, int64_t j1, hipStream_t s) {
  constexpr TileShape ts{TT, NW};
  const uint8_t* base = static_cast<const uint8_t*>(q8);
  const int8_t* qs = reinterpret_cast<const int8_t*>(base);
  const float2* planes = reinterpret_cast<const float2*>(base + q8_planes_offset(M, K));
  auto kern = mmq_kernel<TT, NW, STORE_S>;
  if (ts.lds_bytes() > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)ts.lds_bytes());
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(gm * gn)), dim3(ts.threads()), (size_t)ts.lds_bytes(),
                     s, qs, planes, static_cast<const uint8_t*>(w_rep), out, (int)M, (int)N,
                     (int)K, (int)gm, (int)tm0, (int)tn0, (int)i0, (int)i1, (int)j0, (int)j1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mmq(int tile, const void* q8, const void* w_rep, void* out, int64_t M,
                      int64_t N, int64_t K, int64_t gm, int64_t gn, int64_t tm0, int64_t tn0,
                      bool store_s, int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                      hipStream_t s) {
  if (tile == 1) {
    return store_s ? launch_t<kLarge.tt, kLarge.nw, true>(q8, w_rep, out, M, N, K, gm, gn, tm0,
                                                          tn0, i0, i1, j0, j1, s)
                   : launch_t<kLarge.tt, kLarge.nw, false>(q8, w_rep, out, M, N, K, gm, gn,
                                                           tm0, tn0, i0, i1, j0, j1, s);
  }
  return store_s ? launch_t<kSmall.tt, kSmall.nw, true>(q8, w_rep, out, M, N, K, gm, gn, tm0,
                                                        tn0, i0, i1, j0, j1, s)
                 : launch_t<kSmall.tt, kSmall.nw, false>(q8, w_rep, out, M, N, K, gm, gn, tm0,
                                                         tn0, i0, i1, j0, j1, s);
}

}  // namespace mmq

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
//   D   = MFMA(w, q, bias)          bias = 0x4B400000, so float(D) = 12582912 + S exactly
//   y   = fma(float(D), da, nb)     nb = -12582912 * da (exact), y = RN(S * da)
//   acc = fma(y, dsv, acc)          term1
//   acc = fma(dma, dmv, acc)        term2, dma = da * sa formed once per (token, block)
//
// y equals float(S) * da bit for bit, without an int->float conversion instruction.
//
// Operand orientation: MFMA rows (src0) are weight rows, columns (src1, one per lane) are
// tokens. Lane l holds token l%32 of a tile and, in its 16 accumulator registers r, the
// weight rows 8*(r/4) + 4*(l/32) + r%4. Per block, the token scales are one float4 per
// lane and the weight scales 16+16 floats per lane, both read from LDS.
//
// Workgroup: NW wavefronts; wavefront w owns weight tile (32 rows) tn*NW + w for all
// BM = 32*TT tokens of the workgroup. The token tile (int8, 256 k per super-block) and its
// scales are staged in LDS and shared by the wavefronts; the weight nibbles are private to
// a wavefront and loaded straight into registers from the repacked layout, where the 64
// lanes of one load read 1 KiB of contiguous memory.
#include "mmq_internal.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float f16lo_to_f32(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}

template <int TT, int NW, bool STORE_S>
__global__ __launch_bounds__(NW * 64) void mmq_kernel(
    const int8_t* __restrict__ qs, const uint32_t* __restrict__ ds,
    const uint8_t* __restrict__ wrep, void* __restrict__ out, int M, int N, int K, int gm,
    int tm0, int tn0, int i0, int i1, int j0, int j1) {
  constexpr int BM = 32 * TT;
  constexpr int NT = NW * 64;
  static_assert((BM * 16) % NT == 0, "token tile staging must divide evenly");

  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* sA = smem;                                          // [BM][256] int8, swizzled
  float4* sAs = reinterpret_cast<float4*>(smem + BM * 256);    // [8][BM] {da, nb, dma, 0}
  float* sW = reinterpret_cast<float*>(smem + BM * 256 + 8 * BM * 16);  // [NW][2][8][32]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const uint8_t* wtile = wrep + (size_t)wt * nsb * kRepTileBytes;

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;

  float acc[TT][16];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  for (int s = 0; s < nsb; ++s) {
    __syncthreads();  // the previous super-block's LDS reads are done

    // token tile: BM rows x 256 bytes; 16-byte chunk c of row i goes to chunk c ^ (i & 15)
#pragma unroll
    for (int it = 0; it < (BM * 16) / NT; ++it) {
      const int c = it * NT + tid;
      const int row = c >> 4, ch = c & 15;
      const int gi = m0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (gi < M)
        v = *reinterpret_cast<const uint4*>(qs + (size_t)gi * K + (size_t)s * 256 + ch * 16);
      *reinterpret_cast<uint4*>(sA + row * 256 + ((ch ^ (row & 15)) << 4)) = v;
    }
    // token scales: two lanes per row, four blocks each
    for (int c = tid; c < BM * 2; c += NT) {
      const int row = c >> 1, half = c & 1;
      const int gi = m0 + row;
      uint4 w4 = make_uint4(0u, 0u, 0u, 0u);
      if (gi < M)
        w4 = *reinterpret_cast<const uint4*>(ds + (size_t)gi * kb + (size_t)s * 8 + half * 4);
      const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float da = f16lo_to_f32(ws[e]);
        const float sa = (float)(int16_t)(ws[e] >> 16);
        sAs[(half * 4 + e) * BM + row] = make_float4(da, -kBiasF * da, da * sa, 0.0f);
      }
    }
    // this wavefront's weight scales: dsv[8][32], dmv[8][32] (2 KiB)
    {
      const float4* src =
          reinterpret_cast<const float4*>(wtile + (size_t)s * kRepTileBytes + kRepNibBytes);
      float4* dst = reinterpret_cast<float4*>(sW + wave * 512);
      dst[lane] = src[lane];
      dst[lane + 64] = src[lane + 64];
    }
    // this wavefront's weight nibbles: 4 x 16 bytes per lane
    v4i raw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      raw[g] = *reinterpret_cast<const v4i*>(wtile + (size_t)s * kRepTileBytes + g * 1024 +
                                             lane * 16);
    __syncthreads();

#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const v4i rr = raw[b >> 1];
      const v4i wop = (b & 1) ? ((rr >> 4) & 0x0F0F0F0F) : (rr & 0x0F0F0F0F);
      float dsv[16], dmv[16];
      const float* pw = sW + wave * 512 + b * 32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = *reinterpret_cast<const float4*>(pw + 8 * g + 4 * h);
        const float4 m = *reinterpret_cast<const float4*>(pw + 256 + 8 * g + 4 * h);
        dsv[4 * g + 0] = a.x; dsv[4 * g + 1] = a.y; dsv[4 * g + 2] = a.z; dsv[4 * g + 3] = a.w;
        dmv[4 * g + 0] = m.x; dmv[4 * g + 1] = m.y; dmv[4 * g + 2] = m.z; dmv[4 * g + 3] = m.w;
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int row = t * 32 + l32;
        const int ch = 2 * b + h;
        const v4i top = *reinterpret_cast<const v4i*>(sA + row * 256 + ((ch ^ (row & 15)) << 4));
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop, top, bias, 0, 0, 0);
        if constexpr (STORE_S) {
          const int i = m0 + row;
          if (wt_ok && i >= i0 && i < i1) {
            int32_t* S = static_cast<int32_t*>(out);
            const size_t plane = (size_t)(i1 - i0) * (size_t)(j1 - j0);
            const int bg = s * 8 + b;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = wt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
              if (j >= j0 && j < j1)
                S[(size_t)bg * plane + (size_t)(i - i0) * (j1 - j0) + (j - j0)] =
                    D[r] - kBiasBits;
            }
          }
        } else {
          const float4 as = sAs[b * BM + row];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float y = __builtin_fmaf(__int_as_float(D[r]), as.x, as.y);
            acc[t][r] = __builtin_fmaf(y, dsv[r], acc[t][r]);
            acc[t][r] = __builtin_fmaf(as.z, dmv[r], acc[t][r]);
          }
        }
      }
    }
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
  const uint32_t* ds = reinterpret_cast<const uint32_t*>(base + M * K);
  hipLaunchKernelGGL((mmq_kernel<TT, NW, STORE_S>), dim3((unsigned)(gm * gn)),
                     dim3(ts.threads()), (size_t)ts.lds_bytes(), s, qs, ds,
                     static_cast<const uint8_t*>(w_rep), out, (int)M, (int)N, (int)K, (int)gm,
                     (int)tm0, (int)tn0, (int)i0, (int)i1, (int)j0, (int)j1);
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

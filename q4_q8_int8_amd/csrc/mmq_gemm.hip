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
// term2 is rank-1 per block: the row factor dma = da * sa (formed once per token and block,
// exact in f32) times the column factor dmv. Summed over a pair of blocks it is a K=2 outer
// product, which v_mfma_f32_32x32x2_f32 adds into the same accumulator on the matrix unit,
// off the vector ALU. Per element the terms are added in a fixed order (term1 of each block,
// term2 of each pair of blocks), so results are deterministic and identical across tiles.
//
// Operand orientation: MFMA rows (src0) are weight rows, columns (src1, one per lane) are
// tokens. Lane l holds token l%32 of a tile and, in its 16 accumulator registers r, the
// weight rows 8*(r/4) + 4*(l/32) + r%4. Per block, the token scales {da, nb} are one
// float2 per lane and the weight scales dsv 16 floats per lane (lane-half broadcast), both
// read from LDS; dma and dmv are one float per lane per pair of blocks.
//
// Workgroup: NW wavefronts; wavefront w owns weight tile (32 rows) tn*NW + w for all
// BM = 32*TT tokens of the workgroup. The token tile (int8, 256 k per super-block) and its
// scales are staged in LDS and shared by the wavefronts; the weight nibbles are private to
// a wavefront and loaded straight into registers from the repacked layout, where the 64
// lanes of one load read 1 KiB of contiguous memory. Global reads are buffer loads: 32-bit
// offsets off a wave-uniform descriptor, and reads past the end of an operand return zero,
// which masks the token rows past M without any compare. Token rows sit in LDS with a
// 272-byte stride (16 bytes of padding), so the 16-byte operand reads of 16 consecutive
// rows hit distinct banks and every LDS address is a per-lane base plus a constant.
//
// Latency hiding inside a wavefront: the vector ALU is the bottleneck, so the (block,
// token-tile) steps are software-pipelined -- the LDS operand of a step is read two steps
// ahead, its MFMA is issued one step ahead, and the rescale of the current step runs while
// both are in flight. With PF, the global loads of super-block s+1 are also issued before
// super-block s is computed (one wavefront per SIMD holds the extra registers); without PF
// two wavefronts per SIMD cover each other's staging.
#include "mmq_internal.h"

namespace mmq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float f16lo_to_f32(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
[[maybe_unused]] constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;
#ifndef MMQ_SCHED
#define MMQ_SCHED 0
#endif

// Raw buffer descriptor over [p, p + bytes): reads at offsets >= bytes return zero.
// The last descriptor word is the gfx9-family default data format (32-bit, untyped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr int kRowStride = 272;  // LDS bytes per staged token row (256 + 16 padding)

template <int TT, int NW, bool PF, bool STORE_S>
__global__ __launch_bounds__(NW * 64, PF ? 1 : 2) void mmq_kernel(
    const int8_t* __restrict__ qs, const uint32_t* __restrict__ ds,
    const uint8_t* __restrict__ wrep, void* __restrict__ out, int M, int N, int K, int gm,
    int tm0, int tn0, int i0, int i1, int j0, int j1) {
  constexpr int BM = 32 * TT;
  constexpr int NT = NW * 64;
  constexpr int NS = 8 * TT;  // (block, token tile) steps per super-block
  static_assert((BM * 16) % NT == 0, "token tile staging must divide evenly");

  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* sA = smem;                                            // [BM][272] int8 rows
  uint8_t* sS = smem + BM * kRowStride;
  float2* sAs = reinterpret_cast<float2*>(sS);                   // [8][BM] {da, nb}
  float* sAd = reinterpret_cast<float*>(sS + 8 * BM * 8);        // [8][BM] dma
  float* sW = reinterpret_cast<float*>(sS + 8 * BM * 12);        // [NW][2][8][32]

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
  const uint8_t* wtile = wrep + (size_t)wt * nsb * kRepTileBytes;
  float* sWw = sW + wave * 512;  // this wavefront's dsv [8][32] then dmv [8][32]
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qs, (uint32_t)M * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(ds, (uint32_t)M * (uint32_t)kb * 4u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wtile, (uint32_t)nsb * kRepTileBytes);

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;

  v16f acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  // ---- staging of one super-block: all global loads of a super-block are issued together
  constexpr int IT = (BM * 16) / NT;   // 16-byte token chunks per thread
  const int srow = tid >> 1, shalf = tid & 1;
  const bool sact = tid < BM * 2;      // two lanes per token row load its scale words
  struct Stage {
    uint4 va[IT];       // token int8 chunks
    uint4 w4;           // four q8_1 scale words
    uint4 wsc0, wsc1;   // this wavefront's dsv/dmv (2 KiB per wavefront)
    uint4 raw[4];       // this wavefront's nibbles, 4 x 16 B per lane
  };
  auto load_stage = [&](int s, Stage& st) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int c = it * NT + tid;
      const int row = c >> 4, ch = c & 15;
      st.va[it] = buf_load16(rq, (uint32_t)(m0 + row) * (uint32_t)K + (uint32_t)s * 256 + ch * 16);
    }
    st.w4 = make_uint4(0u, 0u, 0u, 0u);
    if (sact)
      st.w4 = buf_load16(rd, ((uint32_t)(m0 + srow) * (uint32_t)kb + (uint32_t)s * 8 + shalf * 4) * 4u);
    const uint32_t wsb = (uint32_t)s * kRepTileBytes;
    st.wsc0 = buf_load16(rw, wsb + kRepNibBytes + lane * 16);
    st.wsc1 = buf_load16(rw, wsb + kRepNibBytes + 1024 + lane * 16);
#pragma unroll
    for (int g = 0; g < 4; ++g) st.raw[g] = buf_load16(rw, wsb + g * 1024 + lane * 16);
  };
  auto store_stage = [&](const Stage& st) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int c = it * NT + tid;
      const int row = c >> 4, ch = c & 15;
      *reinterpret_cast<uint4*>(sA + row * kRowStride + ch * 16) = st.va[it];
    }
    if (sact) {
      const uint32_t ws[4] = {st.w4.x, st.w4.y, st.w4.z, st.w4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float da = f16lo_to_f32(ws[e]);
        const float sa = (float)(int16_t)(ws[e] >> 16);
        sAs[(shalf * 4 + e) * BM + srow] = make_float2(da, -kBiasF * da);
        sAd[(shalf * 4 + e) * BM + srow] = da * sa;
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(sWw);
    dst[lane] = st.wsc0;
    dst[lane + 64] = st.wsc1;
  };

  // ---- operands from LDS
  const uint8_t* sArow = sA + l32 * kRowStride + h * 16;
  auto top_of = [&](int n) -> v4i {  // token operand of step n: 16 int8 of row t*32+l32
    const int b = n / TT, t = n % TT;
    return *reinterpret_cast<const v4i*>(sArow + t * 32 * kRowStride + b * 32);
  };
  auto as_of = [&](int n) -> float2 { return sAs[(n / TT) * BM + (n % TT) * 32 + l32]; };
  auto dsv_of = [&](int b, float (&d)[16]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 a = *reinterpret_cast<const float4*>(sWw + b * 32 + 8 * g + 4 * h);
      d[4 * g + 0] = a.x; d[4 * g + 1] = a.y; d[4 * g + 2] = a.z; d[4 * g + 3] = a.w;
    }
  };

  Stage stg;
  if constexpr (PF) load_stage(0, stg);
  for (int s = 0; s < nsb; ++s) {
    __syncthreads();  // the previous super-block's LDS reads are done
    if constexpr (!PF) load_stage(s, stg);
    store_stage(stg);
    v4i raw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) raw[g] = __builtin_bit_cast(v4i, stg.raw[g]);
    auto wop_of = [&](int b) -> v4i {
      const v4i rr = raw[b >> 1];
      return (b & 1) ? ((rr >> 4) & 0x0F0F0F0F) : (rr & 0x0F0F0F0F);
    };
    __syncthreads();
    if constexpr (PF) {
      if (s + 1 < nsb) load_stage(s + 1, stg);
    }

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
      // n+1 and the scales of step n are in registers; dsv[b & 1] holds block b's scales.
      float dsv[2][16];
      dsv_of(0, dsv[0]);
      v4i tnext = top_of(1 % NS);
      float2 as = as_of(0);
      v16i Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(0), top_of(0), bias, 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const int b = n / TT, t = n % TT;
#if MMQ_SCHED >= 1
        __builtin_amdgcn_sched_barrier(0);
#endif
        const v16i D = Dn;
        const float2 asc = as;
        if (n + 1 < NS) {
          Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of((n + 1) / TT), tnext, bias, 0, 0, 0);
          as = as_of(n + 1);
        }
        if (n + 2 < NS) tnext = top_of(n + 2);
        if (t == 0 && b + 1 < 8) dsv_of(b + 1, dsv[(b + 1) & 1]);
#if MMQ_SCHED >= 2
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 6, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, 32, 0);
#endif
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = __builtin_fmaf(__int_as_float(D[r]), asc.x, asc.y);
          acc[t][r] = __builtin_fmaf(y, dsv[b & 1][r], acc[t][r]);
        }
        if (b & 1) {
          // term2 of blocks b-1 and b: lane l supplies dmv of weight row l%32 and dma of
          // token l%32 for block b-1+l/32, a K=2 outer product added on the matrix unit
          const float dmv = sWw[256 + (b - 1 + h) * 32 + l32];
          const float dma = sAd[(b - 1 + h) * BM + t * 32 + l32];
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(dmv, dma, acc[t], 0, 0, 0);
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

template <int TT, int NW, bool PF, bool STORE_S>
hipError_t launch_t(const void* q8, const void* w_rep, void* out, int64_t M, int64_t N,
                    int64_t K, int64_t gm, int64_t gn, int64_t tm0, int64_t tn0, int64_t i0,
                    int64_t i1, int64_t j0, int64_t j1, hipStream_t s) {
  constexpr TileShape ts{TT, NW};
  const uint8_t* base = static_cast<const uint8_t*>(q8);
  const int8_t* qs = reinterpret_cast<const int8_t*>(base);
  const uint32_t* ds = reinterpret_cast<const uint32_t*>(base + M * K);
  hipLaunchKernelGGL((mmq_kernel<TT, NW, PF, STORE_S>), dim3((unsigned)(gm * gn)),
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
    return store_s ? launch_t<kLarge.tt, kLarge.nw, kLargePF, true>(
                         q8, w_rep, out, M, N, K, gm, gn, tm0, tn0, i0, i1, j0, j1, s)
                   : launch_t<kLarge.tt, kLarge.nw, kLargePF, false>(
                         q8, w_rep, out, M, N, K, gm, gn, tm0, tn0, i0, i1, j0, j1, s);
  }
  return store_s ? launch_t<kSmall.tt, kSmall.nw, kSmallPF, true>(
                       q8, w_rep, out, M, N, K, gm, gn, tm0, tn0, i0, i1, j0, j1, s)
                 : launch_t<kSmall.tt, kSmall.nw, kSmallPF, false>(
                       q8, w_rep, out, M, N, K, gm, gn, tm0, tn0, i0, i1, j0, j1, s);
}

}  // namespace mmq

// q4_K x q8_1 GEMM for few tokens (M <= 32 per token tile): the same arithmetic as the main
// GEMM (the two-term rescale of the r15 page, "f32-accumulate mma probe + rank-1 term2
// rescale", section 2.1, with the rank-1 fold of the r16 page, "Narrow kernel gets the
// rank-1 fold", section 2.1), organised for the memory-bound regime.
//
// With few tokens the product is bound by streaming the weights once, and the main kernel's
// workgroups, which each walk the whole K dimension one super-block at a time, leave HBM
// mostly idle (at M = 1, K = N = 4096 only 64 workgroups). Here a workgroup owns one 32 x 32
// output tile (32 weight rows, one token tile) and its KW wavefronts split K: wavefront w
// takes the contiguous super-blocks [w*nsb/KW, (w+1)*nsb/KW), so all of K is in flight at
// once. The per-wavefront results are summed through LDS in wavefront order.
//
// Per super-block a wavefront loads everything it needs with single instructions: the
// token operand of each block straight into registers (16 bytes per lane; token rows past
// M read past the end of the buffer, which returns zero), (da, nb) of each block, the three bf16
// pieces of da*sa, its four 16-byte nibble words and the 16-byte header of row l % 32. From
// the header lane l expands the weight scales dsv and the dmv pieces of its row's sub-blocks
// 4 (l / 32) .. + 3 into the wavefront's own 2560-byte LDS region (every lane half needs
// them in a different pattern). Per block: D = MFMA_i8(w, q, bias), y = fma(D, da, nb) with nb = -12582912*da,
// acc = fma(y, dsv, acc) exactly as in the main kernel; one third of the super-block's
// term2 is added by a bf16 MFMA after blocks 1, 3 and 5.
//
// Summation order per output element: within a wavefront as in the main kernel, then the
// wavefronts' partial sums in increasing wavefront order. Deterministic, but not the same
// association as the main kernel's (the results agree within the f32 tolerance).
//
// The FUSED instantiation takes the f32 activations instead of the q8 buffer. Each wavefront
// quantizes the real token rows of its own super-blocks itself (8 lanes per block, one row of
// 1 KiB per pass, with the prepass's arithmetic from quant_device.h) into its own LDS tile:
// int8 values in 272-byte rows, (da, nb), and the three bf16 pieces of da*sa, all in the layout the
// token operands are then read in. Rows past M stay zero. So with few tokens the q8 buffer
// never goes through HBM and the prepass launch disappears, and the result is bit for bit the
// one of the prepass followed by the unfused kernel: the same bytes, the same arithmetic in
// the same order.
#include "mmq_device.h"
#include "quant_device.h"

namespace mmq {
namespace {

// Per-wavefront LDS region of the fused kernel: the weight scales (as in the unfused one),
// then the quantized token tile of one super-block.
constexpr int kFQRow = 272;                        // int8 row: 256 values + 16 bytes padding
constexpr int kFQBytes = 32 * kFQRow;              // [32 rows][272]
constexpr int kFDaBytes = 8 * 32 * 8;              // (da, nb) [8 blocks][32 rows]
constexpr int kFPcBytes = 3 * 32 * 16;             // pieces [3][32 rows][8 bf16]
constexpr int kFRegion = kWDsvBytes + kWPieceBytes + kFQBytes + kFDaBytes + kFPcBytes;
constexpr int kRedStride = 65;                     // floats per row of the partial sums

// LAZY (unfused only): the token operands and (da, nb) of each block are loaded two blocks
// ahead of their MFMA instead of with the super-block, with no MFMA pipelining, so that the
// kernel fits 128 registers and two workgroups share a compute unit (four wavefronts per SIMD
// cover each other's loads); chosen when the grid has more workgroups than the device has
// compute units. Otherwise (PIPE below) everything a super-block needs is loaded into
// registers while the previous one is computed, and the MFMA of block b+1 is issued before
// block b's rescale (238 registers, one workgroup per compute unit).
template <int KW, bool FUSED, bool LAZY>
__global__ __launch_bounds__(KW * 64, LAZY ? 4 : 1) void mmq_skinny_kernel(
    const int8_t* __restrict__ qs, const float* __restrict__ da_plane,
    const uint16_t* __restrict__ tpieces, const float4* __restrict__ x,
    const uint8_t* __restrict__ wrep, float* __restrict__ C, int M, int N, int K, int gm,
    int gmn, int xbm, int xgm) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int W_BYTES = kWDsvBytes + kWPieceBytes;
  constexpr int REGION = FUSED ? kFRegion : W_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  int tm, tn;  // the workgroups of one weight tile on one XCD (xcd_tile)
  xcd_tile((int)blockIdx.x, gm, gmn, xbm, xgm, tm, tn);
  const int m0 = tm * 32;
  const int nsb = K >> 8;
  const int kb = K >> 5;
  const int s0 = wave * nsb / KW, s1 = (wave + 1) * nsb / KW;

  const uint8_t* wtile = wrep + (size_t)tn * nsb * kRepTileBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qs, (uint32_t)M * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rda = make_rsrc(da_plane, (uint32_t)M * (uint32_t)kb * 8u);
  const __amdgpu_buffer_rsrc_t rtp = make_rsrc(tpieces, (uint32_t)M * (uint32_t)nsb * 48u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wtile, (uint32_t)nsb * kRepTileBytes);

  uint8_t* sW = smem + wave * REGION;
  const float* sWw = reinterpret_cast<const float*>(sW);
  uint8_t* sQ = sW + W_BYTES;                                      // fused: token tile
  float2* sDa = reinterpret_cast<float2*>(sQ + kFQBytes);
  uint8_t* sPc = sQ + kFQBytes + kFDaBytes;
  const int mt = M - m0 < 32 ? M - m0 : 32;  // real token rows of this tile
  if constexpr (FUSED) {
    // rows past M stay zero: q = 0, da = 0, pieces 0
    for (int o = lane * 16; o < kFQBytes + kFDaBytes + kFPcBytes; o += 64 * 16)
      *reinterpret_cast<v4i*>(sQ + o) = v4i{0, 0, 0, 0};
  }
  // token row of this lane: every offset inside the row is below K, so rows past M read
  // past the end of the buffer (zero)
  const uint32_t tok_row = (uint32_t)(m0 + l32) * (uint32_t)K + h * 16;

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  // PIPE (unfused, one workgroup per compute unit): everything super-block s needs is loaded
  // into registers while super-block s-1 is computed (two register sets)
  constexpr bool PIPE = !FUSED && !LAZY;
  struct SbRegs {
    v4i hdr, raw[4], tok[8], tp[3];
    float2 da[8];
  };
  auto load_sb = [&](int s, SbRegs& r) {
    r.hdr = buf_load16(rw, (uint32_t)s * kRepTileBytes + kRepNibBytes + l32 * 16);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      r.raw[g] = buf_load16(rw, (uint32_t)s * kRepTileBytes + g * 1024 + lane * 16);
#pragma unroll
    for (int b = 0; b < 8; ++b) r.tok[b] = buf_load16(rq, tok_row + (uint32_t)s * 256 + b * 32);
#pragma unroll
    for (int b = 0; b < 8; ++b)
      r.da[b] = buf_load_f32x2(rda, (((uint32_t)s * 8 + b) * (uint32_t)M + m0 + l32) * 8u);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      r.tp[j] = buf_load16(rtp, (((uint32_t)s * 3 + j) * (uint32_t)M + m0 + l32) * 16u);
  };
  SbRegs nxt;
  if constexpr (PIPE) {
    if (s0 < s1) load_sb(s0, nxt);
  }

  for (int s = s0; s < s1; ++s) {
    // this wavefront's earlier LDS reads of its region are done before the weight scales
    // (and, fused, the quantized tile of this super-block) overwrite it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), the other counters unconstrained
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    v4i hdr, raw[4], tok[LAZY ? 1 : 8], tp[3];
    float2 da[LAZY ? 1 : 8];  // (da, nb) per block
    if constexpr (PIPE) {
      const SbRegs cur = nxt;
      if (s + 1 < s1) load_sb(s + 1, nxt);
      hdr = cur.hdr;
#pragma unroll
      for (int g = 0; g < 4; ++g) raw[g] = cur.raw[g];
#pragma unroll
      for (int b = 0; b < 8; ++b) { tok[b] = cur.tok[b]; da[b] = cur.da[b]; }
#pragma unroll
      for (int j = 0; j < 3; ++j) tp[j] = cur.tp[j];
    } else {
      hdr = buf_load16(rw, (uint32_t)s * kRepTileBytes + kRepNibBytes + l32 * 16);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        raw[g] = buf_load16(rw, (uint32_t)s * kRepTileBytes + g * 1024 + lane * 16);
    }
    if constexpr (FUSED) {
      // quantize rows 0..mt-1 of super-block s: lane = 8 * block + chunk, one float4 each.
      // Rows go in unrolled chunks of 8, 4, 2 or 1 (no early exit inside a chunk), so the
      // loads of a chunk are in flight together and its rows' dependent chains interleave.
      const int b = lane >> 3, c = lane & 7;
      auto rows = [&](const int r0, auto count) {
        constexpr int R = decltype(count)::value;
        float4 vr[R];
#pragma unroll
        for (int i = 0; i < R; ++i)
          vr[i] = x[((uint32_t)(m0 + r0 + i) * (uint32_t)K + (uint32_t)s * 256) / 4 + lane];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int r = r0 + i;
          const float4 v = vr[i];
          const float amax =
              group_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
          const float d = amax / 127.0f;                 // IEEE division
          const float id = d > 0.0f ? 1.0f / d : 0.0f;   // IEEE reciprocal (division)
          const int q0 = quant1(v.x, id), q1 = quant1(v.y, id);
          const int q2 = quant1(v.z, id), q3 = quant1(v.w, id);
          const int sum = group_sum(q0 + q1 + q2 + q3);
          const _Float16 dh = (_Float16)d;  // RNE
          *reinterpret_cast<uint32_t*>(sQ + r * kFQRow + lane * 4) =
              (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
              ((uint32_t)(q3 & 0xFF) << 24);
          if (c == 0) sDa[b * 32 + r] = make_float2((float)dh, -kBiasF * (float)dh);
          // da*sa (exact in f32) as three bf16 pieces: lane c < 3 of the block's group
          // writes piece c into slot b of the row's 16 bytes for that piece
          uint16_t pc[3];
          bf16_split3((float)dh * (float)sum, pc[0], pc[1], pc[2]);
          if (c < 3)
            reinterpret_cast<uint16_t*>(sPc)[(c * 32 + r) * 8 + b] =
                c == 0 ? pc[0] : (c == 1 ? pc[1] : pc[2]);
        }
      };
      int r0 = 0;
      for (; r0 + 8 <= mt; r0 += 8) rows(r0, std::integral_constant<int, 8>{});
      if (r0 + 4 <= mt) { rows(r0, std::integral_constant<int, 4>{}); r0 += 4; }
      if (r0 + 2 <= mt) { rows(r0, std::integral_constant<int, 2>{}); r0 += 2; }
      if (r0 < mt) rows(r0, std::integral_constant<int, 1>{});
      // the tile is complete: other lanes' writes are visible to this wavefront's reads
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int b2 = 0; b2 < 8; ++b2)
        tok[b2] = *reinterpret_cast<const v4i*>(sQ + l32 * kFQRow + b2 * 32 + h * 16);
#pragma unroll
      for (int b2 = 0; b2 < 8; ++b2) da[b2] = sDa[b2 * 32 + l32];
#pragma unroll
      for (int j = 0; j < 3; ++j) tp[j] = *reinterpret_cast<const v4i*>(sPc + (j * 32 + l32) * 16);
    } else if constexpr (LAZY) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        tp[j] = buf_load16(rtp, (((uint32_t)s * 3 + j) * (uint32_t)M + m0 + l32) * 16u);
    }
    q4k_stage_scales(hdr, l32, h != 0, sW);
    // the region is written (and, unless LAZY, every load of the super-block has landed);
    // the fence and the barrier keep the compiler from moving the region's reads above the
    // writes of the other lanes
    if constexpr (FUSED)
      __builtin_amdgcn_s_waitcnt(0);
    else
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); register operands wait on their own
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    auto wop_of = [&](int b) -> v4i {
      const v4i rr = raw[b >> 1];
      return (b & 1) ? ((rr >> 4) & 0x0F0F0F0F) : (rr & 0x0F0F0F0F);
    };
    v16i Dn;
    if constexpr (!LAZY) Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(0), tok[0], bias, 0, 0, 0);
    // LAZY: the token operand and (da, nb) of block b are loaded PF blocks ahead
    constexpr int PF = 2;
    v4i tq[PF + 1];
    float2 dq[PF + 1];
    auto lazy_load = [&](int b) {
      tq[b % (PF + 1)] = buf_load16(rq, tok_row + (uint32_t)s * 256 + b * 32);
      dq[b % (PF + 1)] = buf_load_f32x2(rda, (((uint32_t)s * 8 + b) * (uint32_t)M + m0 + l32) * 8u);
    };
    if constexpr (LAZY) {
#pragma unroll
      for (int b = 0; b < PF; ++b) lazy_load(b);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      v16i D;
      float2 dab;
      if constexpr (LAZY) {
        if (b + PF < 8) lazy_load(b + PF);
        const v4i tb = tq[b % (PF + 1)];
        dab = dq[b % (PF + 1)];
        D = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(b), tb, bias, 0, 0, 0);
      } else {
        D = Dn;
        dab = da[b];
        if (b + 1 < 8)
          Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(b + 1), tok[b + 1], bias, 0, 0, 0);
      }
      float dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = *reinterpret_cast<const float4*>(sWw + b * 32 + 8 * g + 4 * h);
        dsv[4 * g + 0] = a.x; dsv[4 * g + 1] = a.y; dsv[4 * g + 2] = a.z; dsv[4 * g + 3] = a.w;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y = __builtin_fmaf(__int_as_float(D[r]), dab.x, dab.y);
        acc[r] = __builtin_fmaf(y, dsv[r], acc[r]);
      }
      if (b == 1 || b == 3 || b == 5) {
        // one third of term2: the piece pairs (0,0) (0,1) | (1,0) (0,2) | (1,1) (2,0)
        const int u = b >> 1;
        const int ia = u == 0 ? 0 : (u == 1 ? 1 - h : 1 + h);
        const int jb = u == 0 ? h : (u == 1 ? 2 * h : 1 - h);
        const v8bf wa = *reinterpret_cast<const v8bf*>(sW + kWDsvBytes + (ia * 32 + l32) * 16);
        const v4i t0 = tp[0], t1 = tp[1], t2 = tp[2];
        const v4i tsel = jb == 0 ? t0 : (jb == 1 ? t1 : t2);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, __builtin_bit_cast(v8bf, tsel), acc,
                                                       0, 0, 0);
      }
    }
  }

  // partial sums: [wave][register][lane], rows of kRedStride floats, then summed in
  // wavefront order. The read below takes, per wavefront, 16 registers x 2 lanes of each of
  // 2 tokens; with 64-float rows all of them fell on 4 of the LDS banks, with 65 they spread.
  __syncthreads();  // every wavefront is done with its LDS region
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * kRedStride + lane] = acc[r];
  __syncthreads();
  // element e = 32 * token + row of the 32 x 32 tile, so consecutive threads store
  // consecutive output features
  for (int e = tid; e < 1024; e += KW * 64) {
    const int il = e >> 5, jl = e & 31;
    const int r = 4 * (jl >> 3) + (jl & 3), ln = 32 * ((jl >> 2) & 1) + il;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < KW; ++w) v += red[(w * 16 + r) * kRedStride + ln];
    const int i = m0 + il, j = tn * 32 + jl;
    if (i < M && j < N) C[(size_t)i * N + j] = v;
  }
}

}  // namespace

// XCD blocks of the skinny grid (one 32 x 32 output tile per workgroup): a token tile is its
// rows of the q8 buffer, a weight tile its records, per super-block column
static XcdBlock skinny_xcd_block(int64_t gm, int64_t gn, int64_t K) {
  return xcd_block(gm, gn, 32.0 * (double)(K / 256) * 400.0, (double)(K / 256) * kRepTileBytes);
}

int64_t skinny_lds_bytes() {
  const int64_t regions = (int64_t)kSkinnyWaves * (kWDsvBytes + kWPieceBytes);
  const int64_t reduce = (int64_t)kSkinnyWaves * 16 * kRedStride * 4;
  return regions > reduce ? regions : reduce;
}

int64_t fused_lds_bytes() {
  const int64_t regions = (int64_t)kSkinnyWaves * kFRegion;
  const int64_t reduce = (int64_t)kSkinnyWaves * 16 * kRedStride * 4;
  return regions > reduce ? regions : reduce;
}

hipError_t launch_mmq_skinny(const void* q8, const void* w_rep, float* C, int64_t M, int64_t N,
                             int64_t K, int64_t compute_units, hipStream_t s) {
  const uint8_t* base = static_cast<const uint8_t*>(q8);
  const int8_t* qs = reinterpret_cast<const int8_t*>(base);
  const float* da_plane = reinterpret_cast<const float*>(base + q8_planes_offset(M, K));
  const uint16_t* tpieces = reinterpret_cast<const uint16_t*>(base + q8_pieces_offset(M, K));
  const int64_t gm = (M + 31) / 32, gn = (N + 31) / 32;
  const XcdBlock xb = skinny_xcd_block(gm, gn, K);
  auto kern = gm * gn > compute_units ? mmq_skinny_kernel<kSkinnyWaves, false, true>
                                      : mmq_skinny_kernel<kSkinnyWaves, false, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(gm * gn)), dim3(kSkinnyWaves * 64),
                     (size_t)skinny_lds_bytes(), s, qs, da_plane, tpieces, nullptr,
                     static_cast<const uint8_t*>(w_rep), C, (int)M, (int)N, (int)K, (int)gm,
                     (int)(gm * gn), xb.bm, xb.xgm);
  return hipGetLastError();
}

hipError_t launch_mmq_fused(const float* x, const void* w_rep, float* C, int64_t M, int64_t N,
                            int64_t K, hipStream_t s) {
  auto kern = mmq_skinny_kernel<kSkinnyWaves, true, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)fused_lds_bytes());
  if (e != hipSuccess) return e;
  const int64_t gm = (M + 31) / 32, gn = (N + 31) / 32;
  const XcdBlock xb = skinny_xcd_block(gm, gn, K);
  hipLaunchKernelGGL(kern, dim3((unsigned)(gm * gn)), dim3(kSkinnyWaves * 64),
                     (size_t)fused_lds_bytes(), s, nullptr, nullptr, nullptr,
                     reinterpret_cast<const float4*>(x), static_cast<const uint8_t*>(w_rep), C,
                     (int)M, (int)N, (int)K, (int)gm, (int)(gm * gn), xb.bm, xb.xgm);
  return hipGetLastError();
}

}  // namespace mmq

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
// M read past the end of the buffer, which returns zero), da of each block, the three bf16
// pieces of da*sa, its four 16-byte nibble words, and, into its own 2560-byte LDS region,
// the weight scales dsv and the dmv pieces (which every lane half needs in a different
// pattern). Per block: D = MFMA_i8(w, q, bias), y = fma(D, da, -12582912*da),
// acc = fma(y, dsv, acc) exactly as in the main kernel; one third of the super-block's
// term2 is added by a bf16 MFMA after blocks 1, 3 and 5.
//
// Summation order per output element: within a wavefront as in the main kernel, then the
// wavefronts' partial sums in increasing wavefront order. Deterministic, but not the same
// association as the main kernel's (the results agree within the f32 tolerance).
#include "mmq_device.h"

namespace mmq {
namespace {

template <int KW>
__global__ __launch_bounds__(KW * 64, 1) void mmq_skinny_kernel(
    const int8_t* __restrict__ qs, const float* __restrict__ da_plane,
    const uint16_t* __restrict__ tpieces, const uint8_t* __restrict__ wrep,
    float* __restrict__ C, int M, int N, int K, int gm) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int W_BYTES = kRepDsvBytes + kRepPieceBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int tm = (int)(blockIdx.x % (unsigned)gm);
  const int tn = (int)(blockIdx.x / (unsigned)gm);
  const int m0 = tm * 32;
  const int nsb = K >> 8;
  const int kb = K >> 5;
  const int s0 = wave * nsb / KW, s1 = (wave + 1) * nsb / KW;

  const uint8_t* wtile = wrep + (size_t)tn * nsb * kRepTileBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qs, (uint32_t)M * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rda = make_rsrc(da_plane, (uint32_t)M * (uint32_t)kb * 4u);
  const __amdgpu_buffer_rsrc_t rtp = make_rsrc(tpieces, (uint32_t)M * (uint32_t)nsb * 48u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wtile, (uint32_t)nsb * kRepTileBytes);
  const v4i rwd = make_rsrc_sgpr(wtile, (uint32_t)nsb * kRepTileBytes);

  uint8_t* sW = smem + wave * W_BYTES;
  const uint32_t sWa = lds_addr(smem) + (uint32_t)(wave * W_BYTES);  // its LDS address
  const float* sWw = reinterpret_cast<const float*>(sW);
  // token row of this lane: every offset inside the row is below K, so rows past M read
  // past the end of the buffer (zero)
  const uint32_t tok_row = (uint32_t)(m0 + l32) * (uint32_t)K + h * 16;

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  for (int s = s0; s < s1; ++s) {
    // this wavefront's earlier LDS reads of its region are done before the loads overwrite it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), the other counters unconstrained
    const uint32_t wo = (uint32_t)s * kRepTileBytes + kRepNibBytes + lane * 16;
    dma16(rwd, sWa, wo);
    dma16(rwd, sWa + 1024, wo + 1024);
    if (lane < 32) dma16(rwd, sWa + 2048, wo + 2048);
    v4i raw[4], tok[8], tp[3];
    float da[8];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      raw[g] = buf_load16(rw, (uint32_t)s * kRepTileBytes + g * 1024 + lane * 16);
#pragma unroll
    for (int b = 0; b < 8; ++b) tok[b] = buf_load16(rq, tok_row + (uint32_t)s * 256 + b * 32);
#pragma unroll
    for (int b = 0; b < 8; ++b)
      da[b] = buf_load_f32(rda, (((uint32_t)s * 8 + b) * (uint32_t)M + m0 + l32) * 4u);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      tp[j] = buf_load16(rtp, (((uint32_t)s * 3 + j) * (uint32_t)M + m0 + l32) * 16u);
    // everything, the LDS region included, has landed; the fence keeps the compiler from
    // moving the region's reads above the wait
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    auto wop_of = [&](int b) -> v4i {
      const v4i rr = raw[b >> 1];
      return (b & 1) ? ((rr >> 4) & 0x0F0F0F0F) : (rr & 0x0F0F0F0F);
    };
    v16i Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(0), tok[0], bias, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const v16i D = Dn;
      if (b + 1 < 8) Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(b + 1), tok[b + 1], bias, 0, 0, 0);
      float dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = *reinterpret_cast<const float4*>(sWw + b * 32 + 8 * g + 4 * h);
        dsv[4 * g + 0] = a.x; dsv[4 * g + 1] = a.y; dsv[4 * g + 2] = a.z; dsv[4 * g + 3] = a.w;
      }
      const float nb = -kBiasF * da[b];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y = __builtin_fmaf(__int_as_float(D[r]), da[b], nb);
        acc[r] = __builtin_fmaf(y, dsv[r], acc[r]);
      }
      if (b == 1 || b == 3 || b == 5) {
        // one third of term2: the piece pairs (0,0) (0,1) | (1,0) (0,2) | (1,1) (2,0)
        const int u = b >> 1;
        const int ia = u == 0 ? 0 : (u == 1 ? 1 - h : 1 + h);
        const int jb = u == 0 ? h : (u == 1 ? 2 * h : 1 - h);
        const v8bf wa = *reinterpret_cast<const v8bf*>(sW + kRepDsvBytes + (ia * 32 + l32) * 16);
        const v4i t0 = tp[0], t1 = tp[1], t2 = tp[2];
        const v4i tsel = jb == 0 ? t0 : (jb == 1 ? t1 : t2);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, __builtin_bit_cast(v8bf, tsel), acc,
                                                       0, 0, 0);
      }
    }
  }

  // partial sums: [wave][register][lane], then summed in wavefront order
  __syncthreads();  // every wavefront is done with its LDS region
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
  __syncthreads();
  // element e = 32 * token + row of the 32 x 32 tile, so consecutive threads store
  // consecutive output features
  for (int e = tid; e < 1024; e += KW * 64) {
    const int il = e >> 5, jl = e & 31;
    const int r = 4 * (jl >> 3) + (jl & 3), ln = 32 * ((jl >> 2) & 1) + il;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < KW; ++w) v += red[(w * 16 + r) * 64 + ln];
    const int i = m0 + il, j = tn * 32 + jl;
    if (i < M && j < N) C[(size_t)i * N + j] = v;
  }
}

}  // namespace

int64_t skinny_lds_bytes() {
  const int64_t regions = (int64_t)kSkinnyWaves * (kRepDsvBytes + kRepPieceBytes);
  const int64_t reduce = (int64_t)kSkinnyWaves * 16 * 64 * 4;
  return regions > reduce ? regions : reduce;
}

hipError_t launch_mmq_skinny(const void* q8, const void* w_rep, float* C, int64_t M, int64_t N,
                             int64_t K, hipStream_t s) {
  const uint8_t* base = static_cast<const uint8_t*>(q8);
  const int8_t* qs = reinterpret_cast<const int8_t*>(base);
  const float* da_plane = reinterpret_cast<const float*>(base + q8_planes_offset(M, K));
  const uint16_t* tpieces = reinterpret_cast<const uint16_t*>(base + q8_pieces_offset(M, K));
  const int64_t gm = (M + 31) / 32, gn = (N + 31) / 32;
  hipLaunchKernelGGL(mmq_skinny_kernel<kSkinnyWaves>, dim3((unsigned)(gm * gn)),
                     dim3(kSkinnyWaves * 64), (size_t)skinny_lds_bytes(), s, qs, da_plane,
                     tpieces, static_cast<const uint8_t*>(w_rep), C, (int)M, (int)N, (int)K,
                     (int)gm);
  return hipGetLastError();
}

}  // namespace mmq

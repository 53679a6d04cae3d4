// q4_K x q8_1 product for a handful of tokens (decode), on the vector ALU.
//
// The arithmetic is the GEMM's: for token m, weight row n and 32-block b,
//   S = sum over the block of nibble * q  (exact integer),
//   C[m][n] += da * (dsv * S + dmv * sa)
// which is term1 (da * dsv * S) plus term2 (dmv times the row factor da * sa) of the r15 page
// ("f32-accumulate mma probe + rank-1 term2 rescale", section 2.1), with dsv = d*sc and
// dmv = -dmin*m expanded from the row's header in the repacked record.
//
// With one to sixteen tokens the product streams the weights once and does little else, so
// matrix instructions buy nothing: the MFMA tiles of the other kernels are 32 tokens wide and
// would be mostly padding. Here a workgroup of eight wavefronts owns 16 weight rows (half of a
// repacked 32-row tile), all of K and a group of at most MT (1, 2, 4 or 8) tokens. Lane l of
// wavefront w has row l % 16 and K-slice 4 (w % 4) + l / 16; slice ks takes the super-blocks
// ks, ks + 16, ks + 32, ..., of which wavefronts 0-3 take blocks 0-3 and wavefronts 4-7 blocks
// 4-7. So at K = 4096 every lane owns half a super-block, the grid has N/16 workgroups (256 at
// N = 4096) per token group, and two wavefronts per SIMD overlap one's loads with the other's
// dot products. Token groups are separate workgroups, so that more tokens bring more
// workgroups rather than longer wavefronts; the groups of one row block read the same weights,
// mostly from L2.
//
// Per step a lane loads its row's 64 nibble bytes of its half and its row's 16-byte header,
// from which it expands the 4 scales dsv and 4 mins dmv of its half (buffer loads; the 16
// lanes of a slice read 256 contiguous bytes); in the same burst the lanes of a wavefront load its four slices' token bytes of that
// half and their (da, sa) words, and put them in the wavefront's own LDS region, which each
// slice's lanes then read at one address (broadcast). When a slice has another super-block,
// its loads are issued before this one is computed. Read instead one token at a time with
// scalar loads, each waited for before its dot products, the token data cost an L2 round trip
// per token and pair of blocks. Per block, S is eight v_dot4_i32_i8 over 4 bytes each (both
// operands signed; nibbles are 0..15) started at the bias word 0x4B400000, then
//   u = fma(dmv, float(sa), fma(float(D), dsv, -1.5 * 2^23 * dsv)),  acc = fma(u, da, acc),
// the inner fma being RN(S * dsv) (the biased sum is 1.5 * 2^23 + S exactly).
//
// Summation order per output: blocks in order within a half, super-blocks in order within a
// (slice, half), then the 32 (slice, half) partial sums in order through LDS. Deterministic;
// not the GEMM's association (the two agree within the f32 tolerance).
//
// The FUSED instantiation takes the f32 activations instead of the q8 buffer: each wavefront
// loads the f32 values of its half of its four slices' super-blocks (with the weights) and
// quantizes them into its LDS region, one pass per token: lane l takes 8 values of block
// (l % 16) / 4 of the half of slice l / 16, and the four lanes of a block combine their max
// and integer sum with two lane swaps. The arithmetic per value and per block is the
// prepass's (quant1, IEEE divisions, f16 rounding), and max and integer sum do not depend on
// the order of their terms, so the region holds exactly the bytes and (da, sa) the unfused
// kernel stages: C is bit for bit that of quantize_q8_1 followed by the unfused kernel, from
// one launch.
#include "mmq_device.h"
#include "quant_device.h"

namespace mmq {
namespace {

constexpr int kGemvSlices = 64 / kGemvRows;              // K-slices per wavefront
constexpr int kGemvMfmaScaleBytes = 1280;                // 9-16 tokens: scales per wavefront
// 9-16 tokens, per wavefront: its super-block's token bytes [16][256], (da, nda) [8][16] and
// da*sa pieces [3][16][16 bytes]
constexpr int kGemvTq = 16 * 256, kGemvTda = 8 * 16 * 8, kGemvTpc = 3 * 16 * 16;
constexpr int kGemvMfmaTokBytes = kGemvTq + kGemvTda + kGemvTpc;
constexpr int kGemvKS = kGemvSlices * (kGemvWaves / 2);  // K-slices per workgroup (16)

// ONE: K fits one step per slice (at most kGemvKS super-blocks), so no next step is ever
// loaded; without the second stage's registers (79-80 VGPRs for 1-2 tokens, fused 1) three
// workgroups share a compute unit, which matters most when the grid has more than two per
// unit (N > 8192 rows).
template <int MT, bool FUSED, bool ONE>
__global__ __launch_bounds__(kGemvWaves * 64, ONE ? 6 : 1) void mmq_gemv_kernel(
    const int8_t* __restrict__ qs, const uint32_t* __restrict__ words,
    const float* __restrict__ da_plane, const float4* __restrict__ x,
    const uint8_t* __restrict__ wrep, float* __restrict__ C, int M, int N, int K, int groups) {
  // Wavefronts 0-3 take blocks 0-3 of their slices' super-blocks, wavefronts 4-7 blocks 4-7.
  // Per wavefront and slice: its half of the token bytes [MT][128], then (da, float(sa))
  // [MT][4]; 16 bytes of padding per slice. After the loop the same memory holds the partial
  // sums [kGemvKS][2][MT][kGemvRows].
  constexpr int kTokBytes = MT * 128;
  constexpr int kSlice = kTokBytes + MT * 32 + 16;
  constexpr int kRegion = kGemvSlices * kSlice;
  static_assert(kGemvWaves * kRegion >= kGemvKS * 2 * MT * kGemvRows * 4, "partial sums fit");
  __shared__ __align__(16) uint8_t smem[kGemvWaves * kRegion];
  // Row block rb (rows 16rb..16rb+15). Workgroups go to the 8 XCDs in turn, so slot u runs on
  // XCD (u * groups + group) % 8; pairing slots u and u + 8 with the two halves of one 32-row
  // tile puts both on one XCD, whose L2 then serves the cache lines the halves share (their
  // dsv rows) once. A last partial run of 16 slots keeps the plain order.
  const int u = (int)(blockIdx.x / (unsigned)groups);
  const int nrb = (N + kGemvRows - 1) / kGemvRows;
  int rb = u;
  if (u < nrb / 16 * 16) rb = (u & ~15) + 2 * (u & 7) + ((u >> 3) & 1);
  const int m0 = (int)(blockIdx.x % (unsigned)groups) * MT;  // first token of the group
  const int mc = M - m0 < MT ? M - m0 : MT;                    // tokens in the group
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int hf = wave >> 2;                                    // half of the super-block
  const int wq = wave & 3;                                     // slice group
  const int jj = lane % kGemvRows;
  const int q = lane / kGemvRows;                              // slice within the wavefront
  const int ks = wq * kGemvSlices + q;
  const int j = (rb & 1) * kGemvRows + jj;                     // row within the 32-row tile
  const int nsb = K >> 8, kb = K >> 5;
  // steps of this wavefront: its first slice has the most super-blocks
  const int steps = (nsb - wq * kGemvSlices + kGemvKS - 1) / kGemvKS;
  uint8_t* region = smem + wave * kRegion;

  const uint8_t* wtile = wrep + (size_t)(rb >> 1) * (size_t)nsb * kRepTileBytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wtile, (uint32_t)nsb * (uint32_t)kRepTileBytes);

  // token staging of this lane (unfused): chunk c = (slice * MT + m) * 8 + part of the
  // wavefront's half, and (da, sa) c = (slice * MT + m) * 4 + block
  constexpr int kTokChunks = kGemvSlices * MT * 8;
  constexpr int kTokPerLane = (kTokChunks + 63) / 64;
  constexpr int kSc = kGemvSlices * MT * 4;
  constexpr int kScPerLane = (kSc + 63) / 64;
  // fused: lane l quantizes 8 values of block (l % 16) / 4 of the half, quarter l % 4, of
  // slice l / 16
  const int fq = lane >> 4, fb = (lane & 15) >> 2, fc = lane & 3;

  struct Stage {
    v4i nib[4];      // chunk (g, h) of the half at 2 (g - 2 hf) + h
    v4i hdr;         // the row's super-block header (d, dmin, packed sc and m)
    v4i tok[FUSED ? 1 : kTokPerLane];
    float2 sc[kScPerLane];  // (da, float(sa)) of entries lane + 64 t (below kSc)
    float4 xv[FUSED ? MT : 1][2];
  };
  auto load = [&](int i, Stage& st) {
    const int s = ks + i * kGemvKS;
    const uint32_t rec = (uint32_t)s * kRepTileBytes;  // an idle slice reads past the tile: 0
#pragma unroll
    for (int t = 0; t < 4; ++t)
      st.nib[t] = buf_load16(rw, rec + (2 * hf + (t >> 1)) * 1024 + (t & 1) * 512 + j * 16);
    st.hdr = buf_load16(rw, rec + kRepNibBytes + j * 16);
    if constexpr (FUSED) {
      const int cs = wq * kGemvSlices + fq + i * kGemvKS;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const size_t base =
            ((size_t)(m0 + m) * K + (size_t)cs * 256 + hf * 128 + fb * 32 + fc * 8) / 4;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          st.xv[m][e] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (m < mc && cs < nsb) st.xv[m][e] = x[base + e];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kTokPerLane; ++t) {
        const int c = lane + 64 * t;
        const int cq = c / (8 * MT), cm = (c / 8) % MT, part = c % 8;
        const int cs = wq * kGemvSlices + cq + i * kGemvKS;
        st.tok[t] = v4i{0, 0, 0, 0};
        if (c < kTokChunks && cm < mc && cs < nsb)
          st.tok[t] = *reinterpret_cast<const v4i*>(qs + (size_t)(m0 + cm) * K +
                                                    (size_t)cs * 256 + hf * 128 + part * 16);
      }
#pragma unroll
      for (int t = 0; t < kScPerLane; ++t) {
        const int c = lane + 64 * t;
        const int cq = c / (4 * MT), cm = (c / 4) % MT, b = 4 * hf + c % 4;
        const int cs = wq * kGemvSlices + cq + i * kGemvKS;
        st.sc[t] = make_float2(0.0f, 0.0f);
        if (c < kSc && cm < mc && cs < nsb) {
          const uint32_t w = words[(size_t)(m0 + cm) * kb + (size_t)cs * 8 + b];
          st.sc[t] = make_float2(da_plane[((size_t)(cs * 8 + b) * M + m0 + cm) * 2],
                                 (float)((int)w >> 16));
        }
      }
    }
  };

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

  Stage cur, nxt;
  if (steps > 0) load(0, cur);
  for (int i = 0; i < steps; ++i) {
    // the next step's loads go out before this step's compute
    if (!ONE && i + 1 < steps) load(i + 1, nxt);
    const int s = ks + i * kGemvKS;
    const bool act = s < nsb;
    // the region's reads of the previous step are done before it is overwritten
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if constexpr (FUSED) {
      uint8_t* sl = region + fq * kSlice;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mc) {
          float a = 0.0f;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float4 v = cur.xv[m][e];
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
          }
          a = fmaxf(a, __int_as_float(dpp<kSwap1>(__float_as_int(a))));
          const float amax = fmaxf(a, __int_as_float(dpp<kSwap2>(__float_as_int(a))));
          const float d = amax / 127.0f;                // IEEE division
          const float id = d > 0.0f ? 1.0f / d : 0.0f;  // IEEE reciprocal (division)
          uint2 packed;
          int sum = 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float4 v = cur.xv[m][e];
            const int q0 = quant1(v.x, id), q1 = quant1(v.y, id);
            const int q2 = quant1(v.z, id), q3 = quant1(v.w, id);
            sum += q0 + q1 + q2 + q3;
            const uint32_t pw = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) |
                                ((uint32_t)(q2 & 0xFF) << 16) | ((uint32_t)(q3 & 0xFF) << 24);
            if (e == 0) packed.x = pw; else packed.y = pw;
          }
          sum += dpp<kSwap1>(sum);
          sum += dpp<kSwap2>(sum);
          const _Float16 dh = (_Float16)d;  // RNE
          *reinterpret_cast<uint2*>(sl + m * 128 + fb * 32 + fc * 8) = packed;
          if (fc == 0)
            *reinterpret_cast<float2*>(sl + kTokBytes + (m * 4 + fb) * 8) =
                make_float2((float)dh, (float)sum);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kTokPerLane; ++t) {
        const int c = lane + 64 * t;
        if (c < kTokChunks)
          *reinterpret_cast<v4i*>(region + (c / (8 * MT)) * kSlice + (c % (8 * MT)) * 16) =
              cur.tok[t];
      }
#pragma unroll
      for (int t = 0; t < kScPerLane; ++t) {
        const int c = lane + 64 * t;
        if (c < kSc)
          *reinterpret_cast<float2*>(region + (c / (4 * MT)) * kSlice + kTokBytes +
                                     (c % (4 * MT)) * 8) = cur.sc[t];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (act) {
      const uint8_t* sl = region + q * kSlice;
      float dsv[4], dmv[4];
      q4k_scales(cur.hdr, hf != 0, dsv, dmv);
      // nds = -1.5 * 2^23 * dsv (exact): with the dot products started at the bias word
      // 0x4B400000, whose float value is 1.5 * 2^23, fma(D, dsv, nds) = RN(S * dsv) in one
      // instruction, as float(S) * dsv would be in two (|S| < 2^22 keeps D in one binade)
      float nds[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) nds[b] = -kBiasF * dsv[b];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        int lo[8], hi[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const uint32_t w = (uint32_t)cur.nib[2 * gg + (d >> 2)][d & 3];
          lo[d] = (int)(w & 0x0F0F0F0Fu);
          hi[d] = (int)((w >> 4) & 0x0F0F0F0Fu);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < mc) {
            // blocks 2gg and 2gg+1 of the half for token m0 + m, and their (da, sa) pairs
            const v4i* tq = reinterpret_cast<const v4i*>(sl + m * 128 + gg * 64);
            const float4 sc =
                *reinterpret_cast<const float4*>(sl + kTokBytes + (m * 4 + 2 * gg) * 8);
            int S0 = kBiasBits, S1 = kBiasBits;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const v4i a = tq[h], c = tq[2 + h];
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                S0 = __builtin_amdgcn_sdot4(lo[4 * h + d], a[d], S0, false);
                S1 = __builtin_amdgcn_sdot4(hi[4 * h + d], c[d], S1, false);
              }
            }
            const float t0 = __builtin_fmaf(__int_as_float(S0), dsv[2 * gg], nds[2 * gg]);
            acc[m] = __builtin_fmaf(__builtin_fmaf(dmv[2 * gg], sc.y, t0), sc.x, acc[m]);
            const float t1 =
                __builtin_fmaf(__int_as_float(S1), dsv[2 * gg + 1], nds[2 * gg + 1]);
            acc[m] = __builtin_fmaf(__builtin_fmaf(dmv[2 * gg + 1], sc.w, t1), sc.z, acc[m]);
          }
        }
      }
    }
    if constexpr (!ONE) cur = nxt;
  }

  __syncthreads();  // every wavefront is done with its region
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int m = 0; m < MT; ++m) red[((ks * 2 + hf) * MT + m) * kGemvRows + jj] = acc[m];
  __syncthreads();
  for (int e = threadIdx.x; e < MT * kGemvRows; e += kGemvWaves * 64) {
    const int m = e / kGemvRows, r = e % kGemvRows;
    const int n = rb * kGemvRows + r;
    if (m < mc && n < N) {
      float v = 0.0f;
#pragma unroll
      for (int k2 = 0; k2 < 2 * kGemvKS; ++k2) v += red[(k2 * MT + m) * kGemvRows + r];
      C[(size_t)(m0 + m) * N + n] = v;
    }
  }
}

// The matrix-unit form (from 5 tokens to 16): the vector ALU's dot products set the time
// there, so one 32-block of 16 weight rows x 16 tokens becomes one v_mfma_i32_16x16x32_i8 (no
// padding at 16 tokens; the columns of tokens past M are computed from in-bounds or zero reads
// and never stored). A workgroup of NW wavefronts owns RT 16-row halves of a repacked tile
// (with one half, the two halves of a tile go to workgroups on one XCD as above) and all of
// K; wavefront w takes the super-blocks w, w + NW, w + 2 NW, ..., each one's weights in
// registers and its token-side operands in the wavefront's own LDS region (six direct-to-LDS
// loads), then computes it. The weights of the wavefront's next super-block are loaded while
// it computes this one. The shape follows the rows N: where the N / 16 workgroups fit the
// compute units once, 16 wavefronts and one half (128 KiB of LDS, one workgroup per unit);
// where N / 32 fit, 8 wavefronts and both halves (82 KiB); else 4 wavefronts and one half
// (32 KiB, up to five per unit). Every workgroup stages all of K's token operands (5.9 KB per
// super-block, 2.5x the bytes of one half's weights), so two halves halve that traffic per
// weight byte, while more workgroups in flight hide more latency: with 16 wavefronts at
// N = 11008 the grid took three rounds, and there two halves with 4 wavefronts (half the
// workgroups) were slower than one.
// Per block a lane holds, for its token l % 16, the four outputs of rows 4 (l / 16) .. + 3,
// and rescales them as the GEMM does: y = fma(D, da, nda) with D biased by 0x4B400000,
// acc = fma(y, dsv, acc). term2 of a super-block is a K = 8 product of dmv and da*sa; as in
// the GEMM it runs on the bf16 matrix unit from exact three-piece splits, those of da*sa
// stored in the q8 buffer, those of dmv (bf16_trunc3) expanded from the row headers into the
// wavefront's LDS region (with dsv) per super-block, lane (c, g) taking sub-blocks 2g and
// 2g + 1 of row c: two v_mfma_f32_16x16x32_bf16 whose 4 k-groups of 8 blocks carry the piece
// pairs (0,0) (0,1) (1,0) (0,2) | (1,1) (2,0) (and two zero groups), added into the same
// accumulator. The NW wavefronts' partial sums are added in wavefront order through LDS.
// Operand layout of both instructions: A row l % 16 and B column l % 16 take the 8 k values
// 8 (l / 16) .. + 7; the result of row 4 (l / 16) + r, column l % 16 is register r of lane l.
template <int NW, int RT>
__global__ __launch_bounds__(64 * NW) void mmq_gemv_mfma_kernel(
    const int8_t* __restrict__ qs, const float* __restrict__ da_plane,
    const uint16_t* __restrict__ tpieces, const uint8_t* __restrict__ wrep,
    float* __restrict__ C, int M, int N, int K) {
  static_assert(NW >= 4, "the final sum takes 256 work-items");
  static_assert(RT == 1 || RT == 2, "one or two 16-row halves of a tile per workgroup");
  constexpr int kRows = RT * 16;  // weight rows per workgroup
  // LDS: per wavefront its expanded weight scales, per half (dsv f32 [8 blocks][16 rows],
  // then the dmv pieces bf16 [3][16 rows][8]); the partial sums [wavefront][token][row]; per
  // wavefront its super-block's token-side operands (kGemvMfmaTokBytes)
  constexpr int kWsDsv = 8 * 16 * 4;
  static_assert(kWsDsv + 3 * 16 * 8 * 2 == kGemvMfmaScaleBytes, "scale region");
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int kRedOff = NW * RT * kGemvMfmaScaleBytes;
  constexpr int kTokOff = kRedOff + NW * 16 * kRows * 4;
  float(*red)[16][kRows] = reinterpret_cast<float(*)[16][kRows]>(smem + kRedOff);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int u = (int)blockIdx.x;
  // row block rb of kRows rows; with 16 rows, halves of one tile paired on one XCD
  int rb = u;
  if (RT == 1) {
    const int nrb = (N + kGemvRows - 1) / kGemvRows;
    if (u < nrb / 16 * 16) rb = (u & ~15) + 2 * (u & 7) + ((u >> 3) & 1);
  }
  const int nsb = K >> 8;
  const int c16 = lane & 15, kg = lane >> 4;   // operand row / token column, k-group
  // A operand row within the 32-row tile, of half h
  auto j_op = [&](int h) { return (RT == 2 ? h : (rb & 1)) * 16 + c16; };
  // term2 piece pairs of this lane's k-group: (ia1, jb1) in the first instruction, (ia2, jb2)
  // in the second (k-groups 2 and 3 of the second are zero)
  const int ia1 = kg == 2 ? 1 : 0, jb1 = kg == 1 ? 1 : (kg == 3 ? 2 : 0);
  const int ia2 = kg == 1 ? 2 : 1, jb2 = kg == 0 ? 1 : 0;
  const bool t2 = kg < 2;
  const uint8_t* wtile = wrep + (size_t)(RT == 2 ? rb : rb >> 1) * (size_t)nsb * kRepTileBytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wtile, (uint32_t)nsb * (uint32_t)kRepTileBytes);
  const v4i rq = make_rsrc_sgpr(qs, (uint32_t)M * (uint32_t)K);
  const v4i rda = make_rsrc_sgpr(da_plane, (uint32_t)M * (uint32_t)(K >> 5) * 8u);
  const v4i rtp = make_rsrc_sgpr(tpieces, (uint32_t)M * (uint32_t)nsb * 48u);
  v4i bias = {kBiasBits, kBiasBits, kBiasBits, kBiasBits};
  asm volatile("" : "+v"(bias));

  // The wavefront's token-side operands of super-block s go to its LDS region by
  // direct-to-LDS loads, 6 instructions instead of one 8-byte load per block and lane:
  //   tokens [16][256]: 16-byte chunk c of token t at chunk position c ^ t (token t's row
  //     starts at bank 0 like every other, so the XOR spreads the operand reads of the 16
  //     tokens over all banks); tokens past M read past the end of q and are zero;
  //   (da, nda) [8 blocks][16 tokens]; the da*sa pieces [3][16 tokens][8 blocks].
  // Tokens past M get other rows' scales or zeros: finite, and their columns are not stored.
  const uint32_t tok = lds_addr(smem) + (uint32_t)(kTokOff + wave * kGemvMfmaTokBytes);
  const uint8_t* stok = smem + kTokOff + wave * kGemvMfmaTokBytes;
  auto stage_tokens = [&](int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 64 * i + lane, t = q >> 4, c = (q & 15) ^ t;
      dma16(rq, tok + i * 1024,
            (uint32_t)t * (uint32_t)K + (uint32_t)s * 256u + (uint32_t)c * 16u);
    }
    dma16(rda, tok + kGemvTq, (((uint32_t)s * 8 + (lane >> 3)) * (uint32_t)M + 2 * (lane & 7)) * 8u);
    if (lane < 48)
      dma16(rtp, tok + kGemvTq + kGemvTda,
            (((uint32_t)s * 3 + (lane >> 4)) * (uint32_t)M + (lane & 15)) * 16u);
  };
  // weights of super-block s, per half: the nibble bytes of A row j_op(h), k-group kg, of
  // block pairs 0..3, and the row's header (kWLoads loads in all)
  constexpr int kWLoads = 5 * RT;
  auto load_weights = [&](int s, uint2 (*nb)[4], v4i* hdr) {
    const uint32_t rec = (uint32_t)s * kRepTileBytes;
#pragma unroll
    for (int h = 0; h < RT; ++h) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        nb[h][g] = __builtin_bit_cast(
            uint2, buf_load_f32x2(rw, rec + g * 1024 + (kg >> 1) * 512 + j_op(h) * 16 + (kg & 1) * 8));
      hdr[h] = buf_load16(rw, rec + kRepNibBytes + j_op(h) * 16);
    }
  };
  auto sdsv = [&](int h) {
    return reinterpret_cast<float*>(smem + (wave * RT + h) * kGemvMfmaScaleBytes);
  };
  auto spc = [&](int h) {
    return reinterpret_cast<uint32_t*>(smem + (wave * RT + h) * kGemvMfmaScaleBytes + kWsDsv);
  };
  // weight scales of a super-block: lane (c16, kg) expands sub-blocks 2kg, 2kg + 1 of row c16
  // of each half into the region, after the previous super-block's reads
  auto expand_scales = [&](const v4i* hdr) {
    float dsv_a[RT], dsv_b[RT];
    uint32_t pa_[RT][3], pb_[RT][3];
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      float dsv4[4], dmv4[4];
      q4k_scales(hdr[h], kg >= 2, dsv4, dmv4);
      const bool odd = (kg & 1) != 0;
      dsv_a[h] = odd ? dsv4[2] : dsv4[0];
      dsv_b[h] = odd ? dsv4[3] : dsv4[1];
      const float dmv_a = odd ? dmv4[2] : dmv4[0], dmv_b = odd ? dmv4[3] : dmv4[1];
      bf16_trunc3(dmv_a, pa_[h][0], pa_[h][1], pa_[h][2]);
      bf16_trunc3(dmv_b, pb_[h][0], pb_[h][1], pb_[h][2]);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      sdsv(h)[(2 * kg) * 16 + c16] = dsv_a[h];
      sdsv(h)[(2 * kg + 1) * 16 + c16] = dsv_b[h];
#pragma unroll
      for (int i = 0; i < 3; ++i) spc(h)[(i * 16 + c16) * 4 + kg] = pack_hi16(pa_[h][i], pb_[h][i]);
    }
  };

  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f acc[RT];
#pragma unroll
  for (int h = 0; h < RT; ++h) acc[h] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // One super-block s whose weights are in nb / hdr; the next one's go to nbn / hdrn.
  auto step = [&](int s, uint2 (*nb)[4], const v4i* hdr, uint2 (*nbn)[4], v4i* hdrn) {
    expand_scales(hdr);
    stage_tokens(s);
    const bool next = s + NW < nsb;
    // the next weights are issued after the token loads (the asm keeps them there), so that
    // waiting for all but the last kWLoads vector loads waits for exactly the token loads
    asm volatile("" ::: "memory");
    if (next) load_weights(s + NW, nbn, hdrn);
    // this wavefront's direct-to-LDS loads have landed, and the scale writes are ordered
    // before the reads below: s_waitcnt vmcnt(kWLoads) lgkmcnt(0), or vmcnt(0) lgkmcnt(0)
    static_assert(kWLoads < 16, "vmcnt in the low field");
    if (next) __builtin_amdgcn_s_waitcnt(0x0070 | kWLoads);
    else __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    v4i pa0[RT], pa1[RT];
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      pa0[h] = *reinterpret_cast<const v4i*>(spc(h) + (ia1 * 16 + c16) * 4);
      pa1[h] = t2 ? *reinterpret_cast<const v4i*>(spc(h) + (ia2 * 16 + c16) * 4)
                  : v4i{0, 0, 0, 0};
    }
    const float2* sdap = reinterpret_cast<const float2*>(stok + kGemvTq);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint2 tb = *reinterpret_cast<const uint2*>(
          stok + c16 * 256 + (((2 * b + (kg >> 1)) ^ c16) << 4) + (kg & 1) * 8);
      const float2 dap = sdap[b * 16 + c16];
#pragma unroll
      for (int h = 0; h < RT; ++h) {
        const uint2 w = nb[h][b >> 1];
        const uint2 a = (b & 1) ? make_uint2((w.x >> 4) & 0x0F0F0F0Fu, (w.y >> 4) & 0x0F0F0F0Fu)
                                : make_uint2(w.x & 0x0F0F0F0Fu, w.y & 0x0F0F0F0Fu);
        const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, a),
                                                            __builtin_bit_cast(long, tb), bias,
                                                            0, 0, 0);
        const float4 dq = *reinterpret_cast<const float4*>(sdsv(h) + b * 16 + 4 * kg);
        const float dsvb[4] = {dq.x, dq.y, dq.z, dq.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float y = __builtin_fmaf(__int_as_float(D[r]), dap.x, dap.y);
          acc[h][r] = __builtin_fmaf(y, dsvb[r], acc[h][r]);
        }
      }
    }
    const v4i pb0 = *reinterpret_cast<const v4i*>(stok + kGemvTq + kGemvTda + (jb1 * 16 + c16) * 16);
    const v4i pb1 = *reinterpret_cast<const v4i*>(stok + kGemvTq + kGemvTda + (jb2 * 16 + c16) * 16);
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, pa0[h]),
                                                       __builtin_bit_cast(v8bf, pb0), acc[h], 0,
                                                       0, 0);
      acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, pa1[h]),
                                                       __builtin_bit_cast(v8bf, pb1), acc[h], 0,
                                                       0, 0);
    }
    // every LDS read of this super-block is done before the next one's loads overwrite the
    // region (the scales are rewritten after the fence in the next expansion): lgkmcnt(0),
    // the next weights may still be in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);
  };
  // two register sets for the weights, used in turn (a copy from one to the other would wait
  // for the loads at the end of every step)
  uint2 nbA[RT][4], nbB[RT][4];
  v4i hdrA[RT], hdrB[RT];
  if (wave < nsb) load_weights(wave, nbA, hdrA);
  for (int s = wave; s < nsb; s += 2 * NW) {
    step(s, nbA, hdrA, nbB, hdrB);
    if (s + NW < nsb) step(s + NW, nbB, hdrB, nbA, hdrA);
  }
  // (a wavefront without a super-block issued no load)

#pragma unroll
  for (int h = 0; h < RT; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][c16][h * 16 + 4 * kg + r] = acc[h][r];
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * kRows; e += 64 * NW) {
    const int t = e / kRows, rr = e % kRows;
    const int n = rb * kRows + rr;
    if (t < M && n < N) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][t][rr];
      C[(size_t)t * N + n] = v;
    }
  }
}

template <int MT, bool ONE>
hipError_t launch_mt(const void* q8, const void* w_rep, float* C, int64_t M, int64_t N, int64_t K,
                     hipStream_t s) {
  const uint8_t* base = static_cast<const uint8_t*>(q8);
  const int64_t groups = (M + MT - 1) / MT;
  hipLaunchKernelGGL((mmq_gemv_kernel<MT, false, ONE>),
                     dim3((unsigned)((N + kGemvRows - 1) / kGemvRows * groups)),
                     dim3(kGemvWaves * 64), 0, s, reinterpret_cast<const int8_t*>(base),
                     reinterpret_cast<const uint32_t*>(base + M * K),
                     reinterpret_cast<const float*>(base + q8_planes_offset(M, K)), nullptr,
                     static_cast<const uint8_t*>(w_rep), C, (int)M, (int)N, (int)K, (int)groups);
  return hipGetLastError();
}

template <int MT, bool ONE>
hipError_t launch_fused_mt(const float* x, const void* w_rep, float* C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s) {
  const int64_t groups = (M + MT - 1) / MT;
  hipLaunchKernelGGL((mmq_gemv_kernel<MT, true, ONE>),
                     dim3((unsigned)((N + kGemvRows - 1) / kGemvRows * groups)),
                     dim3(kGemvWaves * 64), 0, s, nullptr, nullptr, nullptr,
                     reinterpret_cast<const float4*>(x), static_cast<const uint8_t*>(w_rep), C,
                     (int)M, (int)N, (int)K, (int)groups);
  return hipGetLastError();
}

}  // namespace

bool gemv_mfma_form(int64_t M) { return M >= kGemvMfmaMinM; }

int gemv_mfma_waves(int64_t N, int64_t compute_units) {
  if ((N + kGemvRows - 1) / kGemvRows <= compute_units) return 16;
  return (N + 31) / 32 <= compute_units ? 8 : 4;
}

int gemv_mfma_rows(int64_t N, int64_t compute_units) {
  // 32 rows only with 8 wavefronts: with 4 (N / 32 above the compute units) the halved grid
  // left too few wavefronts in flight
  return gemv_mfma_waves(N, compute_units) == 8 ? 2 * kGemvRows : kGemvRows;
}

// tokens per workgroup of the vector-ALU form: 1, 2, 4, then groups of 8
static int64_t gemv_dot_group(int64_t M) { return M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8)); }

int64_t gemv_group(int64_t M, int mfma_waves) { return mfma_waves ? kGemvMaxM : gemv_dot_group(M); }

int64_t gemv_lds_bytes(int64_t M, int mfma_waves, int rows) {
  // the matrix-unit form: per wavefront its expanded weight scales (per 16-row half), its
  // partial sums and its super-block's token-side operands
  if (mfma_waves)
    return mfma_waves * (rows / 16 * kGemvMfmaScaleBytes + 16 * rows * 4 + kGemvMfmaTokBytes);
  const int64_t mt = gemv_dot_group(M);
  return (int64_t)kGemvWaves * kGemvSlices * (mt * 160 + 16);
}

int64_t gemv_grid(int64_t M, int64_t N, int mfma_waves, int rows) {
  const int64_t g = gemv_group(M, mfma_waves);
  return (N + rows - 1) / rows * ((M + g - 1) / g);
}

namespace {
template <int NW, int RT>
hipError_t launch_mfma(const void* q8, const void* w_rep, float* C, int64_t M, int64_t N,
                       int64_t K, hipStream_t s) {
  const uint8_t* base = static_cast<const uint8_t*>(q8);
  const int64_t lds = gemv_lds_bytes(M, NW, RT * 16);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mmq_gemv_mfma_kernel<NW, RT>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mmq_gemv_mfma_kernel<NW, RT>), dim3((unsigned)gemv_grid(M, N, NW, RT * 16)),
                     dim3(64 * NW), (size_t)lds, s, reinterpret_cast<const int8_t*>(base),
                     reinterpret_cast<const float*>(base + q8_planes_offset(M, K)),
                     reinterpret_cast<const uint16_t*>(base + q8_pieces_offset(M, K)),
                     static_cast<const uint8_t*>(w_rep), C, (int)M, (int)N, (int)K);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_mmq_gemv(const void* q8, const void* w_rep, float* C, int64_t M, int64_t N,
                           int64_t K, int mfma_waves, int rows, hipStream_t s) {
  if (M < 1 || M > kGemvMaxM || (!mfma_waves && M > kGemvDotMaxM)) return hipErrorInvalidValue;
  if (mfma_waves) {  // the shapes the guard takes (gemv_mfma_waves, gemv_mfma_rows)
    if (rows == 16 && mfma_waves == 16) return launch_mfma<16, 1>(q8, w_rep, C, M, N, K, s);
    if (rows == 32 && mfma_waves == 8) return launch_mfma<8, 2>(q8, w_rep, C, M, N, K, s);
    if (rows == 16 && mfma_waves == 4) return launch_mfma<4, 1>(q8, w_rep, C, M, N, K, s);
    return hipErrorInvalidValue;
  }
  // one step per slice: the single-stage form for 1 and 2 tokens (at 4 and 8 tokens it would
  // spill)
  const bool one = K / 256 <= kGemvKS;
  switch (gemv_dot_group(M)) {
    case 1: return one ? launch_mt<1, true>(q8, w_rep, C, M, N, K, s)
                       : launch_mt<1, false>(q8, w_rep, C, M, N, K, s);
    case 2: return one ? launch_mt<2, true>(q8, w_rep, C, M, N, K, s)
                       : launch_mt<2, false>(q8, w_rep, C, M, N, K, s);
    case 4: return launch_mt<4, false>(q8, w_rep, C, M, N, K, s);
    default: return launch_mt<8, false>(q8, w_rep, C, M, N, K, s);
  }
}

hipError_t launch_mmq_gemv_fused(const float* x, const void* w_rep, float* C, int64_t M,
                                 int64_t N, int64_t K, hipStream_t s) {
  if (M < 1 || M > kGemvFusedMaxM) return hipErrorInvalidValue;
  // the single-stage form for one token (80 VGPRs; at two tokens it would spill)
  switch (gemv_dot_group(M)) {
    case 1: return K / 256 <= kGemvKS ? launch_fused_mt<1, true>(x, w_rep, C, M, N, K, s)
                                      : launch_fused_mt<1, false>(x, w_rep, C, M, N, K, s);
    case 2: return launch_fused_mt<2, false>(x, w_rep, C, M, N, K, s);
    case 4: return launch_fused_mt<4, false>(x, w_rep, C, M, N, K, s);
    default: return launch_fused_mt<8, false>(x, w_rep, C, M, N, K, s);
  }
}

}  // namespace mmq

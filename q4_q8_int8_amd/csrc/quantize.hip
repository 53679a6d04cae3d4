// q8_1 quantize prepass: f32 activations -> int8 blocks of 32 with an f16 scale and the
// integer block sum, the format of the r15 page ("f32-accumulate mma probe + rank-1 term2
// rescale", section 2.1), computed "for free" by the prepass as on that page (section 2.1).
// It also writes the GEMM's planes, so that the GEMM stages them with direct-to-LDS loads
// and never converts: da as f32 in block-major order, paired with nda = -1.5*2^23*da (the
// constant of the GEMM's rescale of an integer result offset by 1.5*2^23, exact), and the
// folded row factor da*sa of
// term2 (r16 page, "Narrow kernel gets the rank-1 fold", section 2.1) as three bf16 pieces
// that sum to it exactly, grouped per super-block of 8 blocks for the GEMM's bf16 matrix
// instruction. HBM-bound: 4 bytes read and about 1.56 bytes written per element.
//
// Mapping: every load instruction of a wavefront reads 1 KiB of contiguous input, 8
// consecutive blocks with 8 lanes per block and one float4 per lane; block maxima and sums
// are reduced with lane moves inside each group of lanes that owns a block. Two kernels:
// - K % 256 == 0 (whole super-blocks): a workgroup takes a tile of kTileRows rows x one
//   super-block, and a lane-exchange gives each lane 8 values of one block (4 lanes per
//   block). The int8 values and scale words of each row go out directly (256 and 32
//   contiguous bytes); the da plane and the pieces are staged in LDS and written after a
//   barrier as runs of 8*kTileRows and 16*kTileRows contiguous bytes, not as one 8- or
//   16-byte store per row scattered M entries apart;
// - any other K: each wavefront takes 2 groups of 8 consecutive blocks, 8 lanes per block,
//   and stores every block's plane entries where they fall.
#include "quant_device.h"

namespace mmq {
namespace {

// One group of 8 lanes and one block (row, b): quantize, then store q, the scale word, da
// and the pieces of da*sa. gathered: the wavefront's 8 blocks are blocks 8s..8s+7 of one
// row, so lanes 0..2 gather the pieces of all 8 and store 16 bytes each.
__device__ __forceinline__ void quantize_block(const float4 v, const uint32_t blk, const bool ok,
                                               const uint32_t row, const uint32_t b,
                                               const bool gathered, const int lane,
                                               uint32_t* __restrict__ qs,
                                               uint32_t* __restrict__ ds,
                                               float* __restrict__ da_plane,
                                               uint16_t* __restrict__ pieces, uint32_t M) {
  const float amax =
      group_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  const float d = amax / 127.0f;                 // IEEE division
  const float id = d > 0.0f ? 1.0f / d : 0.0f;   // IEEE reciprocal (division)
  const int q0 = quant1(v.x, id), q1 = quant1(v.y, id);
  const int q2 = quant1(v.z, id), q3 = quant1(v.w, id);
  const int sum = group_sum(q0 + q1 + q2 + q3);

  const _Float16 dh = (_Float16)d;  // RNE
  if (ok) {
    qs[blk * 8u + (lane & 7)] = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) |
                                ((uint32_t)(q2 & 0xFF) << 16) | ((uint32_t)(q3 & 0xFF) << 24);
    if ((lane & 7) == 0) {
      ds[blk] = (uint32_t)__builtin_bit_cast(uint16_t, dh) | ((uint32_t)(sum & 0xFFFF) << 16);
      reinterpret_cast<float2*>(da_plane)[b * M + row] =  // the GEMM's plane, block-major
          make_float2((float)dh, -kBiasF * (float)dh);
    }
  }

  // da*sa (exact in f32) as three bf16 pieces, [K/256][3][M][8]
  uint16_t p[3];
  bf16_split3((float)dh * (float)sum, p[0], p[1], p[2]);
  if (gathered) {
    // lane j < 3 gathers piece j of the 8 blocks and stores 16 bytes
    const int j = lane & 7;
    const uint32_t offer = j < 3 ? p[j] : 0u;
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (uint32_t)__shfl((int)offer, 8 * e + j, 64);
    if (ok && lane < 3)
      *reinterpret_cast<uint4*>(pieces + (((b >> 3) * 3 + j) * M + row) * 8) =
          make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                     w[6] | (w[7] << 16));
  } else if (ok && (lane & 7) == 0) {
    uint16_t* dst = pieces + ((b >> 3) * 3 * M + row) * 8 + (b & 7);
#pragma unroll
    for (int j = 0; j < 3; ++j) dst[j * M * 8] = p[j];
  }
}

// A wavefront quantizes kGroups groups of 8 consecutive blocks (1 KiB of input each); all
// its loads are issued before the first block is processed. Indices fit in 32 bits
// (M*K < 2^31).
constexpr int kGroups = 2;

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float4* __restrict__ x,
                                                            uint32_t* __restrict__ qs,
                                                            uint32_t* __restrict__ ds,
                                                            float* __restrict__ da_plane,
                                                            uint16_t* __restrict__ pieces,
                                                            uint32_t nblocks, uint32_t M,
                                                            uint32_t kb) {
  const int lane = threadIdx.x & 63;
  const uint32_t wid = __builtin_amdgcn_readfirstlane((blockIdx.x * 256u + threadIdx.x) >> 6);
  const bool aligned = (kb & 7) == 0;  // then a group of 8 blocks lies in one row
  float4 v[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const uint32_t blk = (wid * kGroups + g) * 8 + (lane >> 3);
    v[g] = blk < nblocks ? x[blk * 8u + (lane & 7)] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const uint32_t blk0 = (wid * kGroups + g) * 8;  // wave-uniform
    const uint32_t blk = blk0 + (lane >> 3);
    uint32_t row, b;
    if (aligned) {
      row = blk0 / kb;
      b = blk0 - row * kb + (lane >> 3);
    } else {
      row = blk / kb;
      b = blk - row * kb;
    }
    quantize_block(v[g], blk, blk < nblocks, row, b, aligned, lane, qs, ds, da_plane, pieces,
                   M);
  }
}

// Whole super-blocks: tile of kTileRows rows x one super-block, kTileWaves wavefronts of
// kTileRows/kTileWaves rows each; 4 lanes own one block, 8 values each, so the per-block
// work (the max, two divisions, the sum, the f16 and bf16 conversions) is shared by 8
// values. Indices fit in 32 bits: 16-byte words of the input below M*K/4 < 2^32.
constexpr int kTileRows = 8;
constexpr int kTileWaves = 4;
constexpr int kRowsPerWave = kTileRows / kTileWaves;
static_assert(kRowsPerWave == 2, "a wavefront's two halves take one row each");
static_assert(kTileRows % 2 == 0 && 7 * kTileRows <= 64 * kTileWaves, "store phase mapping");

// roundf (half away from zero) of p, converted and clamped to [-127, 127], in three
// instructions: for every finite float p, trunc(RN(p + copysign(0.5 - 2^-25, p))) equals
// roundf(p), and v_cvt_i32_f32 truncates, saturates +-inf to the int range and maps NaN to
// 0 (the 0 * inf of a block whose reciprocal overflowed). p must be the rounded product
// x * id: the barrier keeps the compiler from fusing it into the add.
__device__ __forceinline__ int quant_round(float x, float id) {
  float p = x * id;
  asm volatile("" : "+v"(p));
  const float t = p + __builtin_copysignf(0.49999997f, p);
  int r;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(r) : "v"(t));
  return min(max(r, -127), 127);
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)d << 24);
}

__global__ __launch_bounds__(64 * kTileWaves) void quantize_q8_1_tiled_kernel(
    const float4* __restrict__ x, uint32_t* __restrict__ qs, uint32_t* __restrict__ ds,
    float* __restrict__ da_plane, uint16_t* __restrict__ pieces, uint32_t M, uint32_t K,
    uint32_t nsb) {
  __shared__ __align__(16) float2 sDa[8][kTileRows];     // [block of the super-block][row]
  __shared__ __align__(16) uint16_t sPc[3][kTileRows][8];  // [piece][row][block]
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint32_t s = blockIdx.x % nsb;
  const uint32_t r0 = (blockIdx.x / nsb) * kTileRows;
  // Loads: lane l reads 16-byte chunk l of row A (= row 2w of the tile) and of row B, one
  // contiguous KiB per instruction; chunk l is chunk c = l % 8 of block l / 8. A half-mirror
  // swap inside each 8-lane group then gives lanes c < 4 chunks c and 7-c of row A, and
  // lanes c >= 4 chunks c and 7-c of row B: every lane holds 8 values of one block.
  const int c = lane & 7;
  const bool lo = c < 4;
  const int b = lane >> 3;         // block within the super-block
  const int rl = kRowsPerWave * w + (lo ? 0 : 1);  // row of this lane's block
  const uint32_t rowA = r0 + kRowsPerWave * w, rowB = rowA + 1;
  const uint32_t row = lo ? rowA : rowB;
  const bool ok = row < M;
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  const uint32_t seg = 64 * s + lane;  // 16-byte word of chunk l within a row
  // Rows past M load row M-1 (in bounds) and are zeroed after: a load under a condition
  // would be split into four 4-byte loads, each behind its own branch.
  const uint32_t rA = rowA < M ? rowA : M - 1, rB = rowB < M ? rowB : M - 1;
  float4 uA = x[rA * (K / 4) + seg];
  float4 uB = x[rB * (K / 4) + seg];
  if (rowA >= M) uA = zero;
  if (rowB >= M) uB = zero;
  const float4 snd = lo ? uB : uA;
  const float4 u = lo ? uA : uB;
  float4 v;
  v.x = __int_as_float(dpp<kHalfMirror>(__float_as_int(snd.x)));
  v.y = __int_as_float(dpp<kHalfMirror>(__float_as_int(snd.y)));
  v.z = __int_as_float(dpp<kHalfMirror>(__float_as_int(snd.z)));
  v.w = __int_as_float(dpp<kHalfMirror>(__float_as_int(snd.w)));
  const float m = fmaxf(fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w))),
                        fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  float amax = fmaxf(m, __int_as_float(dpp<kSwap1>(__float_as_int(m))));
  amax = fmaxf(amax, __int_as_float(dpp<kSwap2>(__float_as_int(amax))));
  const float d = amax / 127.0f;                 // IEEE division
  const float id = d > 0.0f ? 1.0f / d : 0.0f;   // IEEE reciprocal (division)
  const int q0 = quant_round(u.x, id), q1 = quant_round(u.y, id);
  const int q2 = quant_round(u.z, id), q3 = quant_round(u.w, id);
  const int q4 = quant_round(v.x, id), q5 = quant_round(v.y, id);
  const int q6 = quant_round(v.z, id), q7 = quant_round(v.w, id);
  int sum = (q0 + q1) + (q2 + q3) + ((q4 + q5) + (q6 + q7));
  sum += dpp<kSwap1>(sum);
  sum += dpp<kSwap2>(sum);
  const _Float16 dh = (_Float16)d;  // RNE
  // q words back to chunk order: lane l stores word l of row A and of row B
  const uint32_t own = pack4(q0, q1, q2, q3), oth = pack4(q4, q5, q6, q7);
  const uint32_t got = (uint32_t)dpp<kHalfMirror>((int)oth);
  if (rowA < M) qs[rowA * (K / 4) + seg] = lo ? own : got;
  if (rowB < M) qs[rowB * (K / 4) + seg] = lo ? got : own;
  if (ok && (c & 3) == 0)
    ds[row * (K / 32) + 8 * s + b] =
        (uint32_t)__builtin_bit_cast(uint16_t, dh) | ((uint32_t)(sum & 0xFFFF) << 16);
  // da, and da*sa (exact in f32) as three bf16 pieces: lane j < 3 stages piece j
  uint16_t pc[3];
  bf16_split3((float)dh * (float)sum, pc[0], pc[1], pc[2]);
  const int j = c & 3;
  if (j == 0) sDa[b][rl] = make_float2((float)dh, -kBiasF * (float)dh);
  if (j < 3) sPc[j][rl][b] = j == 0 ? pc[0] : (j == 1 ? pc[1] : pc[2]);
  __syncthreads();
  const int t = threadIdx.x;
  constexpr int kDaThreads = 4 * kTileRows;  // 8 blocks x kTileRows/2 row pairs
  if (t < kDaThreads) {
    const int bb = t / (kTileRows / 2), cc = t % (kTileRows / 2);
    const uint32_t r = r0 + 2 * cc;
    float2* dst = reinterpret_cast<float2*>(da_plane) + (8 * s + bb) * M + r;
    if ((M & 1) == 0 && r + 1 < M) {  // 16-byte aligned: the plane starts on 256 bytes
      *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(&sDa[bb][2 * cc]);
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (r + e < M) dst[e] = sDa[bb][2 * cc + e];
    }
  } else if (t < kDaThreads + 3 * kTileRows) {  // piece pp of row rr of the tile
    const int pp = (t - kDaThreads) / kTileRows, rr = (t - kDaThreads) % kTileRows;
    const uint32_t r = r0 + rr;
    if (r < M)
      *reinterpret_cast<uint4*>(pieces + ((s * 3 + pp) * M + r) * 8) =
          *reinterpret_cast<const uint4*>(&sPc[pp][rr][0]);
  }
}

}  // namespace

hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, void* q8, hipStream_t s) {
  uint8_t* base = static_cast<uint8_t*>(q8);
  if (K % 256 == 0) {
    // ceil(M/8) * K/256 workgroups of 256 work-items: below 2^31 work-items for M*K < 2^34
    const int64_t nsb = K / 256;
    const int64_t grid = (M + kTileRows - 1) / kTileRows * nsb;
    hipLaunchKernelGGL(quantize_q8_1_tiled_kernel, dim3((unsigned)grid), dim3(64 * kTileWaves),
                       0, s, reinterpret_cast<const float4*>(x), reinterpret_cast<uint32_t*>(base),
                       reinterpret_cast<uint32_t*>(base + M * K),
                       reinterpret_cast<float*>(base + q8_planes_offset(M, K)),
                       reinterpret_cast<uint16_t*>(base + q8_pieces_offset(M, K)),
                       (uint32_t)M, (uint32_t)K, (uint32_t)nsb);
    return hipGetLastError();
  }
  const int64_t nblocks = M * (K / 32);
  const int64_t waves = (nblocks + 8 * kGroups - 1) / (8 * kGroups);
  const int64_t grid = (waves + 3) / 4;
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(x), reinterpret_cast<uint32_t*>(base),
                     reinterpret_cast<uint32_t*>(base + M * K),
                     reinterpret_cast<float*>(base + q8_planes_offset(M, K)),
                     reinterpret_cast<uint16_t*>(base + q8_pieces_offset(M, K)),
                     (uint32_t)nblocks, (uint32_t)M, (uint32_t)(K / 32));
  return hipGetLastError();
}

}  // namespace mmq

// Internal declarations shared by the HIP translation units of libmmq (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmq {

// Bias word fed to the integer MFMA as its accumulator input: the bit pattern of the float
// 1.5 * 2^23. With |S| < 2^22 the integer sum 0x4B400000 + S read as a float is exactly
// 12582912 + S, which one FMA turns into S * da (see the GEMM epilogue).
constexpr int32_t kBiasBits = 0x4B400000;
constexpr float kBiasF = 12582912.0f;

constexpr int kRepTileRows = 32;
constexpr int kRepTileBytes = 6144;
constexpr int kRepNibBytes = 4096;

constexpr int kRowStride = 272;  // LDS bytes per staged token row (256 + 16 padding)

// GEMM tile shapes: TT token tiles of 32 per wavefront, NW wavefronts (one 32-row weight
// tile each) per workgroup.
struct TileShape {
  int tt, nw;
  constexpr int block_m() const { return 32 * tt; }
  constexpr int block_n() const { return 32 * nw; }
  constexpr int threads() const { return 64 * nw; }
  // LDS: two stages, each: int8 token tile [BM][272], {da, dma} float2 [8][BM], and per
  // wavefront its dsv/dmv float [2][8][32]
  constexpr int64_t lds_bytes() const {
    return 2 * ((int64_t)block_m() * kRowStride + (int64_t)block_m() * 64 + (int64_t)nw * 2048);
  }
};
constexpr TileShape kLarge{4, 8};
constexpr TileShape kSmall{1, 2};

// q8 buffer: int8 q [M][K], u32 scale words [M][K/32], then (at a 256-byte boundary) the
// GEMM's scale plane float2 {da, da*sa} [K/32][M].
__host__ __device__ constexpr int64_t q8_planes_offset(int64_t M, int64_t K) {
  return ((M * K + 4 * M * (K / 32)) + 255) / 256 * 256;
}
__host__ __device__ constexpr int64_t q8_total_bytes(int64_t M, int64_t K) {
  return q8_planes_offset(M, K) + 8 * M * (K / 32);
}

hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, void* q8, hipStream_t s);
hipError_t launch_repack_q4_K(const void* w, int64_t N, int64_t K, void* w_rep, hipStream_t s);

// GEMM launch: a 1-D grid of gm*gn workgroups covering token tiles [tm0, tm0+gm) and
// weight-tile groups [tn0, tn0+gn). store_s selects the store-S epilogue (S written to
// out as int32 [K/32][i1-i0][j1-j0]); otherwise out is C.
hipError_t launch_mmq(int tile, const void* q8, const void* w_rep, void* out, int64_t M,
                      int64_t N, int64_t K, int64_t gm, int64_t gn, int64_t tm0, int64_t tn0,
                      bool store_s, int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                      hipStream_t s);

}  // namespace mmq

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
// Repacked weight record per (32-row tile, super-block): nibbles [4][2][32][16] (4096 B),
// then each row's 16-byte q4_K header [32][16] (f16 d, f16 dmin, the 12 packed 6-bit scale
// and min bytes; 512 B): 4608 B per 8192 weights, 4.5 bits per weight.
constexpr int kRepNibBytes = 4096;
constexpr int kRepHdrBytes = 512;
constexpr int kRepTileBytes = kRepNibBytes + kRepHdrBytes;  // 4608
// The weight scales as the kernels stage them in LDS, expanded from the headers: dsv = d*sc
// f32 [8][32] (1024 B), then dmv = -(dmin*m) as three bf16 pieces [3][32][8] (1536 B).
constexpr int kWDsvBytes = 1024;
constexpr int kWPieceBytes = 1536;

constexpr int kRowStride = 272;  // LDS bytes per staged token row (256 + 16 padding)

// q6_K: the GGUF block (210 bytes) and the repacked record per (32-row tile, super-block):
// int8 values u - 32 [b 0..7][h 0..1][j 0..31][16] (8192 B), then dsv = d*sc f32 [16][32]
// (2048 B).
constexpr int kQ6KBlockBytes = 210;
constexpr int kRep6ValBytes = 8192;
constexpr int kRep6DsvBytes = 2048;
constexpr int kRep6TileBytes = kRep6ValBytes + kRep6DsvBytes;  // 10240

// Weight formats of the GEMM template.
constexpr int kFmtQ4K = 0;
constexpr int kFmtQ6K = 1;

// GEMM tile shapes: TT token tiles of 32 per wavefront, NW wavefronts (one 32-row weight
// tile each) per workgroup.
struct TileShape {
  int tt, nw;
  constexpr int block_m() const { return 32 * tt; }
  constexpr int block_n() const { return 32 * nw; }
  constexpr int threads() const { return 64 * nw; }
  // LDS: two stages, each: the int8 token tile [BM][272], the (da, nda) pairs f32 [8][BM][2],
  // and per wavefront its weight scales. q4_K also stages the token pieces bf16 [3][BM][8],
  // and its weight scales are dsv and the dmv pieces (2560 bytes) with the 32 row headers
  // they are expanded from (512 bytes); q6_K's are dsv [16][32] (2048 bytes).
  constexpr int64_t stage_bytes(int fmt = kFmtQ4K) const {
    return fmt == kFmtQ4K
               ? (int64_t)block_m() * (kRowStride + 64 + 48) + (int64_t)nw * (kWDsvBytes + kWPieceBytes + kRepHdrBytes)
               : (int64_t)block_m() * (kRowStride + 64) + (int64_t)nw * kRep6DsvBytes;
  }
  constexpr int64_t lds_bytes(int fmt = kFmtQ4K) const { return 2 * stage_bytes(fmt); }
};
// The XCD blocks of a gm x gn grid of output tiles. Workgroups go to the 8 XCDs in turn
// (workgroup i to XCD i % 8), each XCD with its own L2. Of the shapes that split the grid into
// 8 equal blocks (bm token tiles by gm*gn/8/bm weight tiles; xgm = gm/bm blocks along the
// tokens, 8/xgm along the weights), the one whose tiles are the fewest bytes, a token tile
// being tok_bytes and a weight tile w_bytes; {0, 0} (the plain order) when none does.
struct XcdBlock {
  int bm, xgm;
};
inline XcdBlock xcd_block(int64_t gm, int64_t gn, double tok_bytes, double w_bytes) {
  XcdBlock best{0, 0};
  if (gm * gn < 16 || (gm * gn) % 8) return best;
  double cost = 0.0;
  for (int64_t xgm = 1; xgm <= 8; xgm *= 2) {
    const int64_t xgn = 8 / xgm;
    if (gm % xgm || gn % xgn) continue;
    const double c = (double)(gm / xgm) * tok_bytes + (double)(gn / xgn) * w_bytes;
    if (best.bm == 0 || c < cost) {
      cost = c;
      best = {(int)(gm / xgm), (int)xgm};
    }
  }
  return best;
}

constexpr TileShape kLarge{4, 8};
constexpr TileShape kSmall{1, 2};
// 32 tokens x 256 weight rows, 8 wavefronts: the tile that splits K over workgroups
constexpr TileShape kMedium{1, 8};
// 64 tokens x 256 weight rows, 8 wavefronts: half the large tile's token rows
constexpr TileShape kHalf{2, 8};

// q8 buffer: int8 q [M][K], u32 scale words [M][K/32], then (each at a 256-byte boundary)
// the GEMM's planes: f32 pairs (da, nda = -kBiasF * da) [K/32][M][2], and dma = da*sa as
// three bf16 pieces per value, [ceil(K/256)][3][M][8].
__host__ __device__ constexpr int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }
__host__ __device__ constexpr int64_t q8_planes_offset(int64_t M, int64_t K) {
  return round256(M * K + 4 * M * (K / 32));
}
__host__ __device__ constexpr int64_t q8_pieces_offset(int64_t M, int64_t K) {
  return round256(q8_planes_offset(M, K) + 8 * M * (K / 32));
}
__host__ __device__ constexpr int64_t q8_total_bytes(int64_t M, int64_t K) {
  return q8_pieces_offset(M, K) + 48 * M * ((K / 32 + 7) / 8);
}

// Split of a finite float into three bfloat16 values with p1 + p2 + p3 == v exactly (each
// piece is the top 16 bits of a float): p1 = RNE_bf16(v), p2 = RNE_bf16(v - p1),
// p3 = v - p1 - p2. Both subtractions are exact (Sterbenz), and p3 is exact in bf16 for
// every value of at most 23 significant bits, which covers every da*sa (an f16 times an
// integer below 2^12) and every dmin*m (an f16 times an integer below 2^6). A non-finite
// v gives {top 16 bits of v, 0, 0}.
__host__ __device__ inline uint32_t bf16_rne_bits(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
}
__host__ __device__ inline void bf16_split3(float v, uint16_t& p1, uint16_t& p2, uint16_t& p3) {
  const uint32_t vb = __builtin_bit_cast(uint32_t, v);
  if ((vb & 0x7F800000u) == 0x7F800000u) {
    p1 = (uint16_t)(vb >> 16);
    p2 = p3 = 0;
    return;
  }
  const uint32_t a = bf16_rne_bits(v);
  const float r = v - __builtin_bit_cast(float, a);
  const uint32_t b = bf16_rne_bits(r);
  const float c = r - __builtin_bit_cast(float, b);
  p1 = (uint16_t)(a >> 16);
  p2 = (uint16_t)(b >> 16);
  p3 = (uint16_t)(__builtin_bit_cast(uint32_t, c) >> 16);
}

// Skinny GEMM (few tokens): one 32 x 32 output tile per workgroup, K split over
// kSkinnyWaves wavefronts and summed through LDS in wavefront order.
constexpr int kSkinnyWaves = 8;
int64_t skinny_lds_bytes();
// compute_units: the device's, which picks the kernel's form (more workgroups than compute
// units: the form that fits two workgroups per compute unit)
hipError_t launch_mmq_skinny(const void* q8, const void* w_rep, float* C, int64_t M, int64_t N,
                             int64_t K, int64_t compute_units, hipStream_t s);
// The same kernel quantizing its own f32 activations (few tokens; per-wavefront LDS tile).
int64_t fused_lds_bytes();
hipError_t launch_mmq_fused(const float* x, const void* w_rep, float* C, int64_t M, int64_t N,
                            int64_t K, hipStream_t s);

// Product for a handful of tokens (decode), M <= kGemvMaxM, 16 weight rows per workgroup, in
// two forms. The vector-ALU form (kGemvWaves wavefronts, up to 8 tokens): integer dot
// products on the vector ALU, up to 8 tokens per workgroup, K split over 16 slices and each
// super-block over two wavefronts. The matrix-unit form (16 wavefronts and 16 rows, 8 and 32,
// or 4 and 16; up to 16 tokens): one 16 x 16 x 32 int8 MFMA per block and 16 rows, all tokens
// in one workgroup, K split over the wavefronts by super-block.
constexpr int kGemvWaves = 8;
constexpr int kGemvRows = 16;  // weight rows per workgroup (the matrix-unit form: 16 or 32)
constexpr int kGemvMaxM = 16;
// The guard's choice up to here (at 16 tokens, K = N = 4096: 5.6 against the skinny
// kernel's 9.4 us).
constexpr int kGemvAutoMaxM = 16;
// The vector-ALU form serves at most this many tokens.
constexpr int kGemvDotMaxM = 8;
// From this many tokens the guard takes the matrix-unit form, at any N. Graph-replayed over
// weights that do not stay in cache, at 5 to 8 tokens it takes 5.5-5.6 us at K = N = 4096
// (16 wavefronts), 7.6-8.1 us at N = 5120-8192 (8) and 10.0 us at N = 11008 (4), against the
// vector-ALU form's 6.7-7.5, 9.9-10.7 (8 tokens) and 12.6-14.2 us. At 3 and 4 tokens the two
// are within 11 % of each other either way (the vector-ALU form ahead at 5120-8192 rows, behind
// at 4096 and 11008), and the vector-ALU form is kept.
constexpr int kGemvMfmaMinM = 5;
// The variant that quantizes its activations itself: vector-ALU form only.
constexpr int kGemvFusedMaxM = kGemvDotMaxM;
// Whether the guard takes the matrix-unit form for M tokens, and that form's wavefronts and
// weight rows per workgroup for N rows on a device of compute_units (16 and 16 where N / 16
// workgroups run in one round, 8 and 32 where N / 32 do, else 4 and 16). The helpers below
// take mfma_waves = 0 (and 16 rows) for the vector-ALU form.
bool gemv_mfma_form(int64_t M);
int gemv_mfma_waves(int64_t N, int64_t compute_units);
int gemv_mfma_rows(int64_t N, int64_t compute_units);  // weight rows per workgroup, 16 or 32
int64_t gemv_group(int64_t M, int mfma_waves);  // tokens per workgroup
int64_t gemv_lds_bytes(int64_t M, int mfma_waves, int rows);
int64_t gemv_grid(int64_t M, int64_t N, int mfma_waves, int rows);
hipError_t launch_mmq_gemv(const void* q8, const void* w_rep, float* C, int64_t M, int64_t N,
                           int64_t K, int mfma_waves, int rows, hipStream_t s);
// The same kernel quantizing its own f32 activations (same LDS, grid and threads).
hipError_t launch_mmq_gemv_fused(const float* x, const void* w_rep, float* C, int64_t M,
                                 int64_t N, int64_t K, hipStream_t s);

hipError_t launch_quantize_q8_1(const float* x, int64_t M, int64_t K, void* q8, hipStream_t s);
hipError_t launch_repack_q4_K(const void* w, int64_t N, int64_t K, void* w_rep, hipStream_t s);
hipError_t launch_repack_q6_K(const void* w, int64_t N, int64_t K, void* w_rep, hipStream_t s);

// GEMM launch: a 1-D grid of gm*gn*splits workgroups covering token tiles [tm0, tm0+gm),
// weight-tile groups [tn0, tn0+gn) and `splits` contiguous ranges of super-blocks. store_s
// selects the store-S epilogue (S written to out as int32 [K/32][i1-i0][j1-j0], one split);
// otherwise out is C when splits == 1, else the partial planes [splits][M][N] f32 that
// launch_reduce_splits adds into C. tile: 1 large, 2 small, 5 medium (kMedium), 6 half
// (kHalf).
hipError_t launch_mmq(int tile, const void* q8, const void* w_rep, void* out, int64_t M,
                      int64_t N, int64_t K, int64_t gm, int64_t gn, int64_t splits, int64_t tm0,
                      int64_t tn0, bool store_s, int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                      hipStream_t s, int fmt = kFmtQ4K);
hipError_t launch_reduce_splits(const float* ws, float* C, int64_t M, int64_t N, int64_t splits,
                                hipStream_t s);

// Host-side helpers of the C ABI (api.cpp) for the other entry-point source: record an error
// for mmq_last_error, the GEMM entry points' argument checks, and the device check (0 when the
// current device is a gfx950).
int api_fail(int status, const char* msg);
int api_check_gemm_call(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                        const float* C, const struct mmq_options* opt);
int api_current_device();

// The f16 comparator path: f32 -> f16 conversion of n values, q4_K -> f16 dequantization,
// and the f16 GEMM (K % 8 == 0, 2*M*K and 2*N*K below 2^31).
hipError_t launch_convert_f32_f16(const float* x, int64_t n, void* y, hipStream_t s);
hipError_t launch_dequantize_q4_K_f16(const void* w, int64_t N, int64_t K, void* out,
                                      hipStream_t s);
hipError_t launch_gemm_f16(const void* x, const void* w, float* C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s);
int64_t gemm_f16_lds_bytes();

}  // namespace mmq

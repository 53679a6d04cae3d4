// The f16 comparator path's GEMM: C[M][N] = x[M][K] * w[N][K]^T for row-major f16 operands,
// float32 accumulation and output, on v_mfma_f32_32x32x16_f16. The comparator is the f16
// default prefill path of the r15 page ("f32-accumulate mma probe + rank-1 term2 rescale",
// section 5) and the r12 page ("16-chain warp tile + ldmatrix", sections 1 and 5).
//
// Workgroup tile: 256 tokens x 128 output features, 4 wavefronts in a 2 x 2 arrangement, each
// owning 128 tokens x 64 features (4 x 2 tiles of 32 x 32, 128 accumulator registers). K is
// staged 64 at a time through LDS, double-buffered: while a stage is multiplied, the next
// one is loaded straight from global memory into the other LDS buffer (direct-to-LDS loads,
// 16 bytes per lane). A tile row of 64 halves is 8 chunks of 16 bytes; chunk c of row r sits
// in slot c ^ ((r >> 1) & 7) of its 128-byte LDS row, so that the fragment reads (32 rows
// at one chunk, per half-wavefront) hit 16 distinct 16-byte bank groups per 16 lanes, while
// each group of 8 lanes of a load still reads one row's 128 contiguous bytes.
//
// MFMA operands: A = 32 token rows x 16 k (lane l holds row l % 32, 8 halves of k), B = 32
// weight rows x 16 k (the same k mapping), so the k order inside an instruction is the same
// for both and the product is the plain sum over k. D: lane l holds output feature l % 32 and
// tokens 8 * (r / 4) + 4 * (l / 32) + r % 4 in register r, so a store of one register writes
// 2 x 32 consecutive floats of C.
//
// Rows past M or N and chunks past K read as zero (their offsets fall outside the buffer
// descriptors), so ragged tiles need no other masking than the store's.
#include "mmq_device.h"

namespace mmq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 128, kBK = 64;
constexpr int kThreads = 256;
constexpr int kAStage = kBM * kBK * 2;        // 32 KiB
constexpr int kBStage = kBN * kBK * 2;        // 16 KiB
constexpr int kStage = kAStage + kBStage;     // 48 KiB
constexpr int kLds = 2 * kStage;              // 96 KiB
constexpr uint32_t kOob = 0x80000000u;        // an offset past every buffer (all < 2^31 bytes)
constexpr int kGroupM = 4;                    // token tiles per group of the tile order

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// One workgroup per compute unit (96 KiB of LDS), so one wavefront per SIMD: the register
// budget is the whole file, which the fragment prefetch below uses.
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_f16_kernel(
    const _Float16* __restrict__ X, const _Float16* __restrict__ W, float* __restrict__ C, int M,
    int N, int K, int gm, int gn) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // Tile order. Workgroups are dealt to the 8 XCDs in turn; when the grid is a multiple of 8
  // the logical index L makes each XCD's workgroups consecutive in L. L then walks groups of
  // kGroupM token tiles, all feature tiles of a group, so that an XCD's workgroups share few
  // token and feature tiles (in its L2) at any time.
  const int G = gm * gn;
  const int b = blockIdx.x;
  const int L = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int per_group = kGroupM * gn;
  const int group = L / per_group;
  const int first = group * kGroupM;
  const int gsz = min(gm - first, kGroupM);
  const int in = L - group * per_group;
  const int tm = first + in % gsz, tn = in / gsz;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const v4i rx = make_rsrc_sgpr(X, (uint32_t)M * (uint32_t)K * 2u);
  const v4i rw = make_rsrc_sgpr(W, (uint32_t)N * (uint32_t)K * 2u);

  // Loads of one stage by this wavefront: A rows [64w, 64w + 64) in 8 instructions of 8 rows,
  // B rows [32w, 32w + 32) in 4. Lane l of instruction d writes LDS row 8d + l/8 (of its
  // block), slot l % 8, which holds chunk (l % 8) ^ swz(row).
  uint32_t offa[8], offb[4];
  int chka[8], chkb[4];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int r = 64 * wave + 8 * d + (lane >> 3);
    chka[d] = (lane & 7) ^ swz(r);
    offa[d] = (m0 + r < M) ? ((uint32_t)(m0 + r) * (uint32_t)K + 8u * chka[d]) * 2u : kOob;
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int r = 32 * wave + 8 * d + (lane >> 3);
    chkb[d] = (lane & 7) ^ swz(r);
    offb[d] = (n0 + r < N) ? ((uint32_t)(n0 + r) * (uint32_t)K + 8u * chkb[d]) * 2u : kOob;
  }
  auto issue = [&](int s) {
    uint8_t* buf = smem + (s & 1) * kStage;
    const int k0 = s * kBK;
    const bool tail = k0 + kBK > K;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t o = offa[d] == kOob ? kOob : offa[d] + 2u * (uint32_t)k0;
      if (tail && k0 + 8 * chka[d] >= K) o = kOob;
      dma16(rx, buf + (64 * wave + 8 * d) * 128, o);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t o = offb[d] == kOob ? kOob : offb[d] + 2u * (uint32_t)k0;
      if (tail && k0 + 8 * chkb[d] >= K) o = kOob;
      dma16(rw, buf + kAStage + (32 * wave + 8 * d) * 128, o);
    }
  };

  // fragment rows of this wavefront: tokens 128 * wm + 32a + l32, features 64 * wn + 32b + l32
  const int wm = wave & 1, wn = wave >> 1;
  int rowa[4], rowb[2];
#pragma unroll
  for (int a = 0; a < 4; ++a) rowa[a] = 128 * wm + 32 * a + l32;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) rowb[bb] = 64 * wn + 32 * bb + l32;

  v16f acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][bb][r] = 0.0f;

  const int S = (K + kBK - 1) / kBK;
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // fragments of step t (16 k) of the stage in buffer `buf`: chunk 2t + h of each row
  auto load_frags = [&](const uint8_t* buf, int t, v8h (&fa)[4], v8h (&fb)[2]) {
    const int c = 2 * t + h;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      fa[a] = *reinterpret_cast<const v8h*>(buf + rowa[a] * 128 + ((c ^ swz(rowa[a])) << 4));
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
      fb[bb] = *reinterpret_cast<const v8h*>(buf + kAStage + rowb[bb] * 128 +
                                             ((c ^ swz(rowb[bb])) << 4));
  };
  v8h fa[2][4], fb[2][2];
  load_frags(smem, 0, fa[0], fb[0]);
  for (int s = 0; s < S; ++s) {
    if (s + 1 < S) issue(s + 1);
    const uint8_t* buf = smem + (s & 1) * kStage;
    // steps 0..3 of the stage; the fragments of step t + 1 are read while step t multiplies
#pragma unroll
    for (int t = 0; t < kBK / 16; ++t) {
      if (t + 1 < kBK / 16) load_frags(buf, t + 1, fa[(t + 1) & 1], fb[(t + 1) & 1]);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
          acc[a][bb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[t & 1][a], fb[t & 1][bb],
                                                             acc[a][bb], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads of stage s + 1 have landed
    __syncthreads();                // ... and everyone's; stage s is no longer read
    if (s + 1 < S) load_frags(smem + ((s + 1) & 1) * kStage, 0, fa[0], fb[0]);
  }

  // store: register r of tile (a, b) holds token 8(r/4) + 4h + r%4 of the tile, feature l32
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int j = n0 + 64 * wn + 32 * bb + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + 128 * wm + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
        if (i < M && j < N) C[(size_t)i * N + j] = acc[a][bb][r];
      }
    }
}

}  // namespace

hipError_t launch_gemm_f16(const void* x, const void* w, float* C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s) {
  const int64_t gm = (M + kBM - 1) / kBM, gn = (N + kBN - 1) / kBN;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_f16_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_f16_kernel, dim3((unsigned)(gm * gn)), dim3(kThreads), (size_t)kLds, s,
                     static_cast<const _Float16*>(x), static_cast<const _Float16*>(w), C, (int)M,
                     (int)N, (int)K, (int)gm, (int)gn);
  return hipGetLastError();
}

int64_t gemm_f16_lds_bytes() { return kLds; }

}  // namespace mmq

// The f16 comparator path's GEMM: C[M][N] = x[M][K] * w[N][K]^T for row-major f16 operands,
// float32 accumulation and output, on v_mfma_f32_32x32x16_f16. The comparator is the f16
// default prefill path of the r15 page ("f32-accumulate mma probe + rank-1 term2 rescale",
// section 5) and the r12 page ("16-chain warp tile + ldmatrix", sections 1 and 5).
//
// Workgroup tile: 256 tokens x 128 output features, 4 wavefronts in a 2 x 2 arrangement, each
// owning 128 tokens x 64 features (4 x 2 tiles of 32 x 32, 128 accumulator registers). K is
// staged 64 at a time through a ring of kStages LDS buffers: while a stage is multiplied,
// the next kStages - 1 are in flight, loaded straight from global memory into LDS
// (direct-to-LDS loads, 16 bytes per lane). A stage is 0.5 us of matrix work per compute
// unit, shorter than a load's latency under full load, so one stage in flight (double
// buffering) leaves the matrix units waiting for memory; two cover it. A tile row of 64 halves is 8 chunks of 16 bytes; chunk c of row r sits
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
constexpr uint32_t kAStage = kBM * kBK * 2;   // 32 KiB
constexpr uint32_t kBStage = kBN * kBK * 2;   // 16 KiB
constexpr uint32_t kStage = kAStage + kBStage;  // 48 KiB
constexpr int kStages = 3;                     // LDS ring: 1 stage multiplied, 2 in flight
constexpr int kLds = kStages * kStage;        // 144 KiB
constexpr uint32_t kOob = 0x80000000u;        // an offset past every buffer (all < 2^31 bytes)
constexpr int kGroupM = 4;                    // token tiles per group of the tile order
// s_waitcnt immediate: vector-memory count <= 12 (one stage of this wavefront's loads), the
// other counters unconstrained
constexpr int kWaitOneStage = 0x0F7C;
static_assert(kStages == 3, "the ring indexing and the waits assume three buffers");

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// One stage's 12 direct-to-LDS loads of this wavefront, issued back to back: 8 of A (LDS
// blocks of 1 KiB from `ma` on) and 4 of B (from `mb` on). Each lane's byte offset within
// its operand (`va`, `vb`) is fixed for the whole K loop; the stage's k offset is the
// instruction's scalar offset `so`. m0 holds the LDS address of each load; it is restored
// afterwards (the compiler reserves it).
__device__ __forceinline__ void issue_stage(v4i rx, v4i rw, uint32_t ma, uint32_t mb,
                                            uint32_t so, const uint32_t (&va)[8],
                                            const uint32_t (&vb)[4]) {
  int saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_add_u32 m0, %[ma], 0\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a0], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[ma], 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a1], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[ma], 0x800\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a2], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[ma], 0xc00\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a3], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[ma], 0x1000\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a4], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[ma], 0x1400\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a5], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[ma], 0x1800\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a6], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[ma], 0x1c00\n\ts_nop 0\n\tbuffer_load_dwordx4 %[a7], %[rx], %[so] offen lds\n\t"
      "s_add_u32 m0, %[mb], 0\n\ts_nop 0\n\tbuffer_load_dwordx4 %[b0], %[rw], %[so] offen lds\n\t"
      "s_add_u32 m0, %[mb], 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %[b1], %[rw], %[so] offen lds\n\t"
      "s_add_u32 m0, %[mb], 0x800\n\ts_nop 0\n\tbuffer_load_dwordx4 %[b2], %[rw], %[so] offen lds\n\t"
      "s_add_u32 m0, %[mb], 0xc00\n\ts_nop 0\n\tbuffer_load_dwordx4 %[b3], %[rw], %[so] offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [ma] "s"(ma), [mb] "s"(mb), [rx] "s"(rx), [rw] "s"(rw), [so] "s"(so), [a0] "v"(va[0]),
        [a1] "v"(va[1]), [a2] "v"(va[2]), [a3] "v"(va[3]), [a4] "v"(va[4]), [a5] "v"(va[5]),
        [a6] "v"(va[6]), [a7] "v"(va[7]), [b0] "v"(vb[0]), [b1] "v"(vb[1]), [b2] "v"(vb[2]),
        [b3] "v"(vb[3])
      : "scc");
}

// One wavefront per SIMD (a 144 KiB workgroup per compute unit): the whole register file is
// this wavefront's.
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
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)smem);

  // Loads of one stage by this wavefront: A rows [64w, 64w + 64) in 8 instructions of 8 rows,
  // B rows [32w, 32w + 32) in 4. Lane l of instruction d writes LDS row 8d + l/8 (of its
  // block), slot l % 8, which holds chunk (l % 8) ^ swz(row).
  uint32_t va[8], vb[4];
  int chka[8], chkb[4];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int r = 64 * wave + 8 * d + (lane >> 3);
    chka[d] = (lane & 7) ^ swz(r);
    va[d] = (m0 + r < M) ? ((uint32_t)(m0 + r) * (uint32_t)K + 8u * chka[d]) * 2u : kOob;
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int r = 32 * wave + 8 * d + (lane >> 3);
    chkb[d] = (lane & 7) ^ swz(r);
    vb[d] = (n0 + r < N) ? ((uint32_t)(n0 + r) * (uint32_t)K + 8u * chkb[d]) * 2u : kOob;
  }
  const uint32_t ma0 = lds0 + (uint32_t)(64 * wave) * 128u;
  const uint32_t mb0 = lds0 + kAStage + (uint32_t)(32 * wave) * 128u;
  // stage s into ring buffer bi
  auto issue = [&](int s, int bi) {
    const int k0 = s * kBK;
    const uint32_t off = (uint32_t)bi * kStage;
    if (k0 + kBK <= K) {
      issue_stage(rx, rw, __builtin_amdgcn_readfirstlane(ma0 + off),
                  __builtin_amdgcn_readfirstlane(mb0 + off), 2u * (uint32_t)k0, va, vb);
    } else {  // the last, partial stage: chunks past K read as zero
      uint32_t ta[8], tb[4];
#pragma unroll
      for (int d = 0; d < 8; ++d) ta[d] = (k0 + 8 * chka[d] < K) ? va[d] : kOob;
#pragma unroll
      for (int d = 0; d < 4; ++d) tb[d] = (k0 + 8 * chkb[d] < K) ? vb[d] : kOob;
      issue_stage(rx, rw, __builtin_amdgcn_readfirstlane(ma0 + off),
                  __builtin_amdgcn_readfirstlane(mb0 + off), 2u * (uint32_t)k0, ta, tb);
    }
  };

  // Fragment reads. Tile row r = (base) + l32 has swz(r) = (l32 >> 1) & 7 for every fragment
  // of this wavefront (the bases are multiples of 32), so in step t (16 k: chunk 2t + h) every
  // fragment's lane offset within its 32-row block is the same, lo[t]; the 32-row blocks are
  // 4 KiB apart (an immediate offset of the read).
  const int wm = wave & 1, wn = wave >> 1;
  uint32_t lo[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) lo[t] = (uint32_t)l32 * 128u + ((uint32_t)((2 * t + h) ^ ((l32 >> 1) & 7)) << 4);
  const uint32_t fa0 = (uint32_t)(128 * wm) * 128u;             // this wavefront's A rows
  const uint32_t fb0 = kAStage + (uint32_t)(64 * wn) * 128u;    // and B rows
  auto load_frags = [&](uint32_t base_a, uint32_t base_b, v8h (&fa)[4], v8h (&fb)[2]) {
#pragma unroll
    for (int a = 0; a < 4; ++a) fa[a] = *reinterpret_cast<const v8h*>(smem + base_a + a * 4096);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
      fb[bb] = *reinterpret_cast<const v8h*>(smem + base_b + bb * 4096);
  };

  v16f acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][bb][r] = 0.0f;
  auto mfmas = [&](const v8h (&fa)[4], const v8h (&fb)[2]) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
        acc[a][bb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[a], fb[bb], acc[a][bb], 0, 0, 0);
  };

  const int S = (K + kBK - 1) / kBK;
  issue(0, 0);
  if (S > 1) issue(1, 1);
  // stage 0 has landed when at most stage 1's loads are pending
  if (S > 1) __builtin_amdgcn_s_waitcnt(kWaitOneStage);
  else __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  v8h f0a[4], f0b[2], f1a[4], f1b[2];
  load_frags(fa0 + lo[0], fb0 + lo[0], f0a, f0b);
  int bi = 0;  // ring buffer of stage s
  for (int s = 0; s < S; ++s) {
    const uint32_t st = (uint32_t)bi * kStage;
    const int bn = bi == 2 ? 0 : bi + 1;       // buffer of stage s + 1
    // the buffer of stage s + 2 was last read in iteration s - 1, which every wavefront
    // finished before that iteration's barrier
    if (s + 2 < S) issue(s + 2, bn == 2 ? 0 : bn + 1);
    // steps 0..2; each reads the next step's fragments while it multiplies
    load_frags(st + fa0 + lo[1], st + fb0 + lo[1], f1a, f1b);
    mfmas(f0a, f0b);
    load_frags(st + fa0 + lo[2], st + fb0 + lo[2], f0a, f0b);
    mfmas(f1a, f1b);
    load_frags(st + fa0 + lo[3], st + fb0 + lo[3], f1a, f1b);
    mfmas(f0a, f0b);
    // stage s + 1 has landed for this wavefront (stage s + 2's 12 loads may be pending) ...
    if (s + 2 < S) __builtin_amdgcn_s_waitcnt(kWaitOneStage);
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // ... and for every wavefront, all of whose reads of stage s are done
    // step 3 multiplies while the first fragments of stage s + 1 are read
    if (s + 1 < S) {
      const uint32_t sn = (uint32_t)bn * kStage;
      load_frags(sn + fa0 + lo[0], sn + fb0 + lo[0], f0a, f0b);
    }
    mfmas(f1a, f1b);
    bi = bn;
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

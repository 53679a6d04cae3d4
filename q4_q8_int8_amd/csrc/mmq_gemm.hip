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
//   y   = fma(float(D), da, nb)     nb = -12582912 * da (exact, written by the prepass beside
//                                   da), y = RN(S * da)
//   acc = fma(y, dsv, acc)          term1
//
// y equals float(S) * da bit for bit, without an int->float conversion instruction.
// term2 is rank-1 per block: the row factor dma = da * sa (exact in f32, written by the
// quantize prepass) times the column factor dmv (exact in f32). Both come as three bf16
// pieces that sum to them exactly (those of dma from the prepass, those of dmv expanded in
// the kernel), so over the 8 blocks of a super-block term2 is a K = 8 product of pieces; three v_mfma_f32_32x32x16_bf16 per token tile and super-block
// (each lane half supplying one piece pair) add the six largest of the nine piece products
// into the same accumulator, every product exact in f32. Per element the terms are added
// in a fixed order (term1 of each block, a third of term2 after blocks 1, 3 and 5), so
// results are deterministic and identical across tile variants.
//
// Operand orientation: MFMA rows (src0) are weight rows, columns (src1, one per lane) are
// tokens. Lane l holds token l%32 of a tile and, in its 16 accumulator registers r, the
// weight rows 8*(r/4) + 4*(l/32) + r%4. Per block, the token scale da and its nb are one
// float pair per lane and the weight scales dsv 16 floats per lane (lane-half broadcast),
// all read from LDS; the term2 operands are one 16-byte bf16 read each (8 blocks' pieces)
// per token tile and third of a super-block.
//
// Workgroup: NW wavefronts; wavefront w owns weight tile (32 rows) tn*NW + w for all
// BM = 32*TT tokens of the workgroup. Everything a super-block (256 k) needs from memory is
// staged one super-block ahead, while the current one is computed:
//   - into LDS by direct-to-LDS buffer loads (no registers, no conversion): the int8 token
//     tile in 272-byte rows (16 bytes of padding, so the 16-byte operand reads of 16
//     consecutive rows hit distinct banks and every LDS address is a per-lane base plus a
//     constant), the (da, nb) pairs and the dma pieces of the token tile, and the 16-byte
//     q4_K headers of each wavefront's 32 weight rows (d, dmin, the packed sc and m), from
//     which the wavefront expands dsv = d*sc and the dmv = -(dmin*m) pieces into its LDS
//     region when the stage begins, while its first MFMA runs (q4k_stage_scales);
//   - into registers: the wavefront's nibbles, where the 64 lanes of one load read 1 KiB of
//     contiguous memory.
// Buffer loads take 32-bit offsets off wave-uniform descriptors; reads past the end of an
// operand return zero, which zeroes token rows past M and the padding slots. The stages
// alternate between two LDS buffers; one barrier per super-block separates them.
//
// On gfx950 the MFMA and the vector ALU of a SIMD largely take turns, so every instruction
// counts: the rescale is 2 FMAs per element-block and the int8 MFMA of step n+1 is issued
// before the rescale of step n.
#include "mmq_device.h"

namespace mmq {
namespace {

// s_setprio takes an immediate: one call per value, selected at compile time once unrolled.
__device__ __forceinline__ void set_priority(int p) {
  if (p >= 3) __builtin_amdgcn_s_setprio(3);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

template <int TT, int NW, bool STORE_S, int FMT>
__global__ __launch_bounds__(NW * 64, NW >= 8 ? 1 : 2) void mmq_kernel(
    const int8_t* __restrict__ qs, const float* __restrict__ da_plane,
    const uint16_t* __restrict__ tpieces,
    const uint8_t* __restrict__ wrep, void* __restrict__ out, int M, int N, int K, int gm,
    int gmn, int splits, int tm0, int tn0, int i0, int i1, int j0, int j1, int xbm, int xgm) {
  constexpr int BM = 32 * TT;
  constexpr int NS = 8 * TT;                      // (block, token tile) steps per super-block
  constexpr int A_BYTES = BM * kRowStride;        // token tile
  constexpr int DA_BYTES = BM * 64;               // (da, nb) pairs [8][BM][2]
  constexpr bool Q6 = FMT == kFmtQ6K;
  // q4_K: token pieces of da*sa [3][BM][8] for term2; q6_K has no term2
  constexpr int TP_BYTES = Q6 ? 0 : BM * 48;
  // per wavefront in LDS: q4_K dsv and the dmv pieces, expanded at the start of the stage
  // from the tile's 32 row headers loaded behind them; q6_K dsv of its 16 groups
  constexpr int W_BYTES = Q6 ? kRep6DsvBytes : kWDsvBytes + kWPieceBytes + kRepHdrBytes;
  constexpr int W_OPS = Q6 ? 2 : 1;  // direct-to-LDS loads of the record's scales or headers
  constexpr int REC = Q6 ? kRep6TileBytes : kRepTileBytes;   // record per (tile, super-block)
  constexpr int REC_W = Q6 ? kRep6ValBytes : kRepNibBytes;   // where its scales start
  constexpr int NG = Q6 ? 8 : 4;   // 16-byte operand loads per lane and super-block
  constexpr int STAGE = A_BYTES + DA_BYTES + TP_BYTES + NW * W_BYTES;
  static_assert(STAGE == TileShape{TT, NW}.stage_bytes(FMT), "LDS stage layout");
  constexpr int A_SLOTS = BM * (kRowStride / 16);  // 16-byte slots of the token tile
  constexpr int A_DMA = (A_SLOTS + 63) / 64;       // wavefront-wide DMA instructions
  constexpr int A_PER_WAVE = (A_DMA + NW - 1) / NW;
  constexpr int TP_SLOTS = Q6 ? 0 : 3 * BM;        // 16-byte slots of the token pieces
  constexpr int TP_DMA = (TP_SLOTS + 63) / 64;
  constexpr int TP_PER_WAVE = (TP_DMA + NW - 1) / NW;

  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup (tile, split): split sp walks super-blocks [sb0, sb1) of K and writes its partial
  // sums to plane sp of out ([splits][M][N]); with one split the plane is C itself.
  const int sp = (int)(blockIdx.x / (unsigned)gmn);
  const int tile_id = (int)(blockIdx.x - (unsigned)sp * (unsigned)gmn);
  int ti, tj;
  xcd_tile(tile_id, gm, gmn, xbm, xgm, ti, tj);
  const int tm = tm0 + ti;
  const int tn = tn0 + tj;
  const int m0 = tm * BM;
  const int ntiles = (N + 31) >> 5;
  const int wt_raw = tn * NW + wave;
  const bool wt_ok = wt_raw < ntiles;
  const int wt = wt_ok ? wt_raw : ntiles - 1;  // idle wavefronts still stage and sync
  const int nsb = K >> 8;
  const int kb = K >> 5;
  const int sb0 = sp * nsb / splits, sb1 = (sp + 1) * nsb / splits;
  const v4i rq = make_rsrc_sgpr(qs, (uint32_t)M * (uint32_t)K);
  const v4i rda = make_rsrc_sgpr(da_plane, (uint32_t)M * (uint32_t)kb * 8u);
  const v4i rtp = make_rsrc_sgpr(tpieces, (uint32_t)M * (uint32_t)nsb * 48u);
  const uint8_t* wtile = wrep + (size_t)wt * nsb * REC;
  const v4i rwd = make_rsrc_sgpr(wtile, (uint32_t)nsb * REC);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wtile, (uint32_t)nsb * REC);

  // Token-tile DMA slots of this lane: slot q = 64*k + lane holds chunk q % 17 of row q / 17;
  // chunk 16 is the row's padding and reads past the end (zero), as do rows past M.
  uint32_t a_off[A_PER_WAVE];
  bool a_act[A_PER_WAVE];
#pragma unroll
  for (int j = 0; j < A_PER_WAVE; ++j) {
    const int k = wave + j * NW;
    const int q = k * 64 + lane;
    const int row = q / 17, c = q - row * 17;
    a_act[j] = k < A_DMA && q < A_SLOTS;
    a_off[j] = c < 16 ? (uint32_t)(m0 + row) * (uint32_t)K + c * 16 : (uint32_t)M * (uint32_t)K;
  }
  // Token-piece DMA slots: slot q = 64*k + lane holds piece q / BM of token m0 + q % BM; the
  // pieces of super-block s sit at [s][piece][M][8] in memory and [piece][BM][8] in LDS.
  uint32_t tp_off[TP_PER_WAVE > 0 ? TP_PER_WAVE : 1];
  bool tp_act[TP_PER_WAVE > 0 ? TP_PER_WAVE : 1];
#pragma unroll
  for (int j = 0; j < TP_PER_WAVE; ++j) {
    const int k = wave + j * NW;
    const int q = k * 64 + lane;
    const int pc = q / BM, r = q - pc * BM;
    tp_act[j] = k < TP_DMA && q < TP_SLOTS;
    tp_off[j] = ((uint32_t)pc * (uint32_t)M + (uint32_t)(m0 + r)) * 16u;
  }
  // What stage s of the pipeline loads into LDS, as NOPS single DMA instructions of this
  // wavefront (its token-tile DMAs, its da DMAs, its token-piece DMA (q4_K), its weight
  // scales: q4_K the 32 row headers, q6_K 2 KiB of dsv), followed by op NOPS: the last
  // weight-operand load (q4_K nibble group 3, q6_K block 7) into registers. Op v is a
  // compile-time constant wherever it is issued, so each call folds to one instruction. The
  // other operand loads are issued separately, in place (load_nib).
  constexpr int DA_PER_WAVE = (8 + NW - 1) / NW;
  // The next stage's ops are issued three at a time at the first step of every other
  // sub-block (the last ones at the last step at the latest), so that the wavefronts of a
  // workgroup do not queue all their memory instructions at once. Finer spreading costs
  // registers: each issue point constrains how far ahead the compiler schedules LDS reads.
  constexpr int NOPS = A_PER_WAVE + DA_PER_WAVE + TP_PER_WAVE + W_OPS + 1;
  auto op_step = [](int v) { return ((v / 3) * 2 * TT < NS - 1) ? (v / 3) * 2 * TT : NS - 1; };
  auto load_nib = [&](int s, int g) -> v4i {
    return buf_load16(rw, (uint32_t)s * REC + g * 1024 + lane * 16);
  };
  const uint32_t lds0 = lds_addr(smem);
  auto issue_op = [&](int v, int s, int p, v4i& nib3) {
    const uint32_t st = lds0 + (uint32_t)(p * STAGE);
    if (v < A_PER_WAVE) {
      const int k = wave + v * NW;
      if (k < A_DMA && a_act[v]) dma16(rq, st + k * 1024, a_off[v] + (uint32_t)s * 256);
      return;
    }
    v -= A_PER_WAVE;
    if (v < DA_PER_WAVE) {  // (da, nb) of block b for rows m0..m0+BM-1: BM/2 lanes
      const int b = wave + v * NW;
      if (b < 8 && lane < BM / 2)
        dma16(rda, st + A_BYTES + b * BM * 8,
              (((uint32_t)s * 8 + b) * (uint32_t)M + m0) * 8u + lane * 16);
      return;
    }
    v -= DA_PER_WAVE;
    if (v < TP_PER_WAVE) {
      const int k = wave + v * NW;
      if (k < TP_DMA && tp_act[v])
        dma16(rtp, st + A_BYTES + DA_BYTES + k * 1024,
              tp_off[v] + (uint32_t)s * 3u * (uint32_t)M * 16u);
      return;
    }
    v -= TP_PER_WAVE;
    if (v < W_OPS) {  // q4_K: the row headers [32][16] (lanes 0..31); q6_K: dsv [16][32]
      const uint32_t sw = st + A_BYTES + DA_BYTES + TP_BYTES + wave * W_BYTES;
      const uint32_t wo = (uint32_t)s * REC + REC_W + lane * 16;
      if (Q6) dma16(rwd, sw + v * 1024, wo + v * 1024);
      else if (lane < 32) dma16(rwd, sw + kWDsvBytes + kWPieceBytes, wo);
      return;
    }
    nib3 = load_nib(s, NG - 1);
  };

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;
  // Opaque to the compiler from here on, so the tuple stays resident in VGPRs: as a known
  // constant it was kept in SGPRs and copied back (8 moves) before one MFMA in seven.
  asm volatile("" : "+v"(bias));
  v16f acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  // raw[g]: q4_K: the nibbles of sub-blocks 2g and 2g+1 of the current stage; q6_K: the
  // values of block g. Loads 0..NG-2 of the next stage go into raw[g] as soon as the last
  // MFMA that reads them has been issued; the last one is still in use at the end of the
  // stage, so it goes through nib3.
  // EARLY (the q4_K small tile, one token tile and two wavefronts): a super-block is too
  // short to cover the next stage's load latency with loads spread over its steps, so every
  // load of stage s+1 is issued at the first step of super-block s, the nibbles into a second
  // register set (rawB) that becomes raw when the stage ends. ENIB (the medium tile, eight
  // wavefronts): only the nibbles go early (all of a stage's loads at once from eight
  // wavefronts stall on issue); the other loads stay spread over the steps. (Measured: the
  // small tile 8-10 % faster at 128..2048 tokens, the medium tile 1-8 %; the half tile is
  // slower with either, so it keeps the in-place reloads.)
  constexpr bool EARLY = !STORE_S && !Q6 && TT == 1 && NW == 2;
  constexpr bool ENIB = !STORE_S && !Q6 && TT == 1 && NW == 8;
  v4i raw[NG], nib3, rawB[(EARLY || ENIB) ? NG : 1];
  if constexpr (EARLY || ENIB) {
#pragma unroll
    for (int v = 0; v < NOPS - 1; ++v) issue_op(v, sb0, 0, nib3);
#pragma unroll
    for (int g = 0; g < NG; ++g) raw[g] = load_nib(sb0, g);
  } else {
#pragma unroll
    for (int v = 0; v < NOPS; ++v) issue_op(v, sb0, 0, nib3);
#pragma unroll
    for (int g = 0; g < NG - 1; ++g) raw[g] = load_nib(sb0, g);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int s = sb0; s < sb1; ++s) {
    const int p = (s - sb0) & 1;
    if constexpr (!EARLY && !ENIB) raw[NG - 1] = nib3;
    const bool more = s + 1 < sb1;

    const uint8_t* st = smem + p * STAGE;
    const uint8_t* sArow = st + l32 * kRowStride + h * 16;
    const float2* sDa = reinterpret_cast<const float2*>(st + A_BYTES);
    const uint8_t* sTp = st + A_BYTES + DA_BYTES;
    const uint8_t* sW = st + A_BYTES + DA_BYTES + TP_BYTES + wave * W_BYTES;
    const float* sWw = reinterpret_cast<const float*>(sW);
    // q4_K, before the stage's first read of dsv or the dmv pieces: lane (l32, h) expands
    // sub-blocks 4h .. 4h+3 of row l32 from its header, loaded behind the region. Only this
    // wavefront reads the region, so a wavefront-scope fence orders the other lanes' writes
    // before those reads.
    auto expand_scales = [&]() {
      uint8_t* sWm = smem + p * STAGE + A_BYTES + DA_BYTES + TP_BYTES + wave * W_BYTES;
      const v4i hdr =
          *reinterpret_cast<const v4i*>(sWm + kWDsvBytes + kWPieceBytes + l32 * 16);
      q4k_stage_scales(hdr, l32, h != 0, sWm);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    };
    auto wop_of = [&](int b) -> v4i {
      const v4i rr = raw[b >> 1];
      return (b & 1) ? ((rr >> 4) & 0x0F0F0F0F) : (rr & 0x0F0F0F0F);
    };
    // q6_K: the weight operand of group gi (0, 1) of block b: lane half h carries the values
    // 16h..16h+15 of the block, so keeping only half gi's lanes makes the MFMA sum one group
    auto wop6_of = [&](int b, int gi) -> v4i { return h == gi ? raw[b] : v4i{0, 0, 0, 0}; };
    auto top_of = [&](int n) -> v4i {  // token operand of step n: 16 int8 of row t*32+l32
      const int b = n / TT, t = n % TT;
      return *reinterpret_cast<const v4i*>(sArow + t * 32 * kRowStride + b * 32);
    };
    auto da_of = [&](int n) -> float2 { return sDa[(n / TT) * BM + (n % TT) * 32 + l32]; };
    auto dsv_of = [&](int b, float (&d)[16]) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 a = *reinterpret_cast<const float4*>(sWw + b * 32 + 8 * g + 4 * h);
        d[4 * g + 0] = a.x; d[4 * g + 1] = a.y; d[4 * g + 2] = a.z; d[4 * g + 3] = a.w;
      }
    };

    if constexpr (STORE_S) {
      // test path: every S of the window, straight from the MFMA (q4_K: one per 32-block,
      // plane index s*8 + b; q6_K: one per 16-value group, plane index s*16 + 2b + gi)
      v4i nxt[NG - 1];
#pragma unroll
      for (int g = 0; g < NG - 1; ++g) nxt[g] = raw[g];
      if (more) {
#pragma unroll
        for (int v = 0; v < NOPS; ++v) issue_op(v, s + 1, p ^ 1, nib3);
#pragma unroll
        for (int g = 0; g < NG - 1; ++g) nxt[g] = load_nib(s + 1, g);
      }
      auto store = [&](const v16i& D, int bg, int t) {
        const int i = m0 + t * 32 + l32;
        if (wt_ok && i >= i0 && i < i1) {
          int32_t* S = static_cast<int32_t*>(out);
          const size_t plane = (size_t)(i1 - i0) * (size_t)(j1 - j0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = wt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (j >= j0 && j < j1)
              S[(size_t)bg * plane + (size_t)(i - i0) * (j1 - j0) + (j - j0)] = D[r] - kBiasBits;
          }
        }
      };
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const int b = n / TT, t = n % TT;
        if constexpr (Q6) {
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
            store(__builtin_amdgcn_mfma_i32_32x32x32_i8(wop6_of(b, gi), top_of(n), bias, 0, 0, 0),
                  s * 16 + 2 * b + gi, t);
        } else {
          store(__builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(b), top_of(n), bias, 0, 0, 0),
                s * 8 + b, t);
        }
      }
#pragma unroll
      for (int g = 0; g < NG - 1; ++g) raw[g] = nxt[g];
    } else if constexpr (Q6) {
      // q6_K, step n = b*TT + t: per 16-value group gi of block b, one MFMA on the lane half
      // that holds it, then y = RN(S * da) and acc += dsv_g * y, groups in increasing order.
      // The two groups' dsv (32 floats per lane) are read from LDS once per block.
      float dsv[2][16];
      v4i w6[2];
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const int b = n / TT, t = n % TT;
        if (n % 2 == 0) set_priority(3 - (n % 8) / 2);
        if (more) {
#pragma unroll
          for (int v = 0; v < NOPS; ++v)
            if (op_step(v) == n) issue_op(v, s + 1, p ^ 1, nib3);
          // block g's MFMAs were issued by step (g+1)*TT - 1
#pragma unroll
          for (int g = 0; g < NG - 1; ++g)
            if (n == (g + 1) * TT) raw[g] = load_nib(s + 1, g);
        }
        if (t == 0) {
          w6[0] = wop6_of(b, 0);
          w6[1] = wop6_of(b, 1);
          dsv_of(2 * b, dsv[0]);
          dsv_of(2 * b + 1, dsv[1]);
        }
        // The empty asm statements keep the steps in order (they are ordered among
        // themselves): the step's MFMAs cannot be issued before its token operand passes one,
        // nor its FMAs sink past the next. Left free, the compiler issued all the
        // super-block's MFMAs first and spilled their results.
        v4i top = top_of(n);
        asm volatile("" : "+v"(top));
        const v16i D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(w6[0], top, bias, 0, 0, 0);
        const v16i D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(w6[1], top, bias, 0, 0, 0);
        const float2 dac = da_of(n);  // (da, nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = __builtin_fmaf(__int_as_float(D0[r]), dac.x, dac.y);
          acc[t][r] = __builtin_fmaf(y, dsv[0][r], acc[t][r]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = __builtin_fmaf(__int_as_float(D1[r]), dac.x, dac.y);
          acc[t][r] = __builtin_fmaf(y, dsv[1][r], acc[t][r]);
        }
        asm volatile("" : "+v"(acc[t]));
      }
    } else {
      // Step n = b*TT + t. Entering step n: D(n) has been issued, the token operand of step
      // n+1 and da of step n are in registers; dsv[b & 1] holds block b's weight scales.
      // the first MFMA needs no weight scales: issued first, it runs while they are expanded
      v16i Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of(0), top_of(0), bias, 0, 0, 0);
      asm volatile("" : "+v"(Dn));  // issued here, not sunk below the expansion
      v4i tnext = top_of(1 % NS);
      float2 da = da_of(0);
      expand_scales();
      float dsv[2][16];
      dsv_of(0, dsv[0]);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const int b = n / TT, t = n % TT;
        // Issue priority falls by one every two steps within each group of eight, so of the
        // two wavefronts sharing a SIMD the one that is ahead yields to the other: the pair
        // keeps step rather than one running ahead and the other finishing the super-block
        // alone (a lone wavefront issues at well under half the rate of a pair).
        if (n % 2 == 0) set_priority(3 - (n % 8) / 2);
        if (more) {
          if constexpr (EARLY) {
            if (n == 0) {
#pragma unroll
              for (int v = 0; v < NOPS - 1; ++v) issue_op(v, s + 1, p ^ 1, nib3);
#pragma unroll
              for (int g = 0; g < NG; ++g) rawB[g] = load_nib(s + 1, g);
            }
          } else if constexpr (ENIB) {
            if (n == 0) {
#pragma unroll
              for (int g = 0; g < NG; ++g) rawB[g] = load_nib(s + 1, g);
            }
#pragma unroll
            for (int v = 0; v < NOPS - 1; ++v)
              if (op_step(v) == n) issue_op(v, s + 1, p ^ 1, nib3);
          } else {
#pragma unroll
            for (int v = 0; v < NOPS; ++v)
              if (op_step(v) == n) issue_op(v, s + 1, p ^ 1, nib3);
            // the MFMAs of sub-blocks 2g, 2g+1 were issued by step (2g+2)*TT - 2
#pragma unroll
            for (int g = 0; g < 3; ++g)
              if (n == (2 * g + 2) * TT) raw[g] = load_nib(s + 1, g);
          }
        }
        const v16i D = Dn;
        const float2 dac = da;  // (da, nb)
        if (n + 1 < NS) {
          Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(wop_of((n + 1) / TT), tnext, bias, 0, 0, 0);
          da = da_of(n + 1);
        }
        if (n + 2 < NS) tnext = top_of(n + 2);
        if (t == 0 && b + 1 < 8) dsv_of(b + 1, dsv[(b + 1) & 1]);
        // the next stage's weight scales, from the header issued at its step 0, into the
        // other stage buffer (read by no one before the barrier that ends this stage)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = __builtin_fmaf(__int_as_float(D[r]), dac.x, dac.y);
          acc[t][r] = __builtin_fmaf(y, dsv[b & 1][r], acc[t][r]);
        }
        if (b == 1 || b == 3 || b == 5) {
          // one third of term2 of the super-block: products of bf16 pieces (dmv piece ia,
          // da*sa piece jb) over its 8 blocks, lane half h supplying one pair; the three
          // instructions cover the pairs (0,0) (0,1) | (1,0) (0,2) | (1,1) (2,0)
          const int u = b >> 1;
          const int ia = u == 0 ? 0 : (u == 1 ? 1 - h : 1 + h);
          const int jb = u == 0 ? h : (u == 1 ? 2 * h : 1 - h);
          const v8bf wa = *reinterpret_cast<const v8bf*>(sW + kWDsvBytes + (ia * 32 + l32) * 16);
          const v8bf tb = *reinterpret_cast<const v8bf*>(sTp + (jb * BM + t * 32 + l32) * 16);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, tb, acc[t], 0, 0, 0);
        }
      }
    }

    if constexpr (!STORE_S) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stage s+1 loads have landed
    __syncthreads();                // ... and everyone's; stage s is no longer read
    if constexpr (EARLY || ENIB) {
#pragma unroll
      for (int g = 0; g < NG; ++g) raw[g] = rawB[g];
    }
  }

  if constexpr (!STORE_S) {
    // Output tile by tile through LDS (the stage buffers are free now: every wavefront has
    // passed the last stage's barrier): lane (l32, h) holds 16 columns of one token row, which
    // would make every store instruction touch 64 rows; after the transpose 8 consecutive
    // lanes write one token row's 128 contiguous bytes. Each wavefront uses its own 32 x 36
    // float regions (two, alternating over t), so only its own writes and reads need
    // ordering, and a wavefront that finishes its last super-block early starts storing
    // without waiting for the others (0.5-0.7 us at q-proj, interleaved A/B).
    constexpr int TS = 36;  // row stride in floats: rows 36 dwords apart hit distinct banks
    float* C = static_cast<float*>(out) + (size_t)sp * (size_t)M * (size_t)N;
    const int j0c = wt * 32;
    const int rr = lane >> 3, c4 = lane & 7;  // read-back: rows rr + 8k, columns 4*c4..+3
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float* tile = reinterpret_cast<float*>(smem) + ((t & 1) * NW + wave) * (32 * TS);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(tile + l32 * TS + 8 * g + 4 * h) =
            make_float4(acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2], acc[t][4 * g + 3]);
      // the region is this wavefront's own: its writes need only be ordered before its reads
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (wt_ok) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int row = rr + 8 * k;
          const int i = m0 + t * 32 + row;
          const int j = j0c + 4 * c4;
          if (i >= M) continue;
          const float4 v = *reinterpret_cast<const float4*>(tile + row * TS + 4 * c4);
          float* p = C + (size_t)i * N + j;
          if ((N & 3) == 0 && j + 3 < N) {
            *reinterpret_cast<float4*>(p) = v;
          } else {
            if (j + 0 < N) p[0] = v.x;
            if (j + 1 < N) p[1] = v.y;
            if (j + 2 < N) p[2] = v.z;
            if (j + 3 < N) p[3] = v.w;
          }
        }
      }
    }
  }
}

template <int TT, int NW, bool STORE_S, int FMT>
hipError_t launch_t(const void* q8, const void* w_rep, void* out, int64_t M, int64_t N,
                    int64_t K, int64_t gm, int64_t gn, int64_t splits, int64_t tm0, int64_t tn0,
                    int64_t i0, int64_t i1, int64_t j0, int64_t j1, hipStream_t s) {
  constexpr TileShape ts{TT, NW};
  constexpr int64_t lds = ts.lds_bytes(FMT);
  const uint8_t* base = static_cast<const uint8_t*>(q8);
  const int8_t* qs = reinterpret_cast<const int8_t*>(base);
  const float* da_plane = reinterpret_cast<const float*>(base + q8_planes_offset(M, K));
  const uint16_t* tpieces = reinterpret_cast<const uint16_t*>(base + q8_pieces_offset(M, K));
  auto kern = mmq_kernel<TT, NW, STORE_S, FMT>;
  // bytes of one token tile (its rows of the q8 buffer) and of one weight-tile group (its
  // records) per super-block column, for the XCD blocks
  const double tok_tile = (double)ts.block_m() * (K / 256) * 400.0;
  const double w_tile = (double)NW * (K / 256) * (FMT == kFmtQ6K ? kRep6TileBytes : kRepTileBytes);
  const XcdBlock xb = xcd_block(gm, gn, tok_tile, w_tile);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(gm * gn * splits)), dim3(ts.threads()),
                     (size_t)lds, s, qs, da_plane, tpieces,
                     static_cast<const uint8_t*>(w_rep), out, (int)M, (int)N, (int)K, (int)gm,
                     (int)(gm * gn), (int)splits, (int)tm0, (int)tn0, (int)i0, (int)i1, (int)j0,
                     (int)j1, xb.bm, xb.xgm);
  return hipGetLastError();
}

// C = the sum of the partial planes ws[0..splits), added in increasing split order (so the
// result is deterministic), four consecutive elements per thread when N % 4 == 0.
template <bool VEC4>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ ws,
                                                            float* __restrict__ C, int64_t n,
                                                            int splits) {
  const int64_t plane = n;
  if constexpr (VEC4) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    float4 a = *reinterpret_cast<const float4*>(ws + i);
    for (int sp = 1; sp < splits; ++sp) {
      const float4 b = *reinterpret_cast<const float4*>(ws + sp * plane + i);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    *reinterpret_cast<float4*>(C + i) = a;
  } else {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float a = ws[i];
    for (int sp = 1; sp < splits; ++sp) a += ws[sp * plane + i];
    C[i] = a;
  }
}

template <int FMT>
hipError_t launch_fmt(int tile, const void* q8, const void* w_rep, void* out, int64_t M,
                      int64_t N, int64_t K, int64_t gm, int64_t gn, int64_t splits, int64_t tm0,
                      int64_t tn0, bool store_s, int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                      hipStream_t s) {
  constexpr TileShape L = kLarge, S = kSmall, D = kMedium, H = kHalf;
  if (tile == 1) {
    return store_s ? launch_t<L.tt, L.nw, true, FMT>(q8, w_rep, out, M, N, K, gm, gn, 1, tm0,
                                                     tn0, i0, i1, j0, j1, s)
                   : launch_t<L.tt, L.nw, false, FMT>(q8, w_rep, out, M, N, K, gm, gn, splits,
                                                      tm0, tn0, i0, i1, j0, j1, s);
  }
  if (tile == 6) {
    return store_s ? launch_t<H.tt, H.nw, true, FMT>(q8, w_rep, out, M, N, K, gm, gn, 1, tm0,
                                                     tn0, i0, i1, j0, j1, s)
                   : launch_t<H.tt, H.nw, false, FMT>(q8, w_rep, out, M, N, K, gm, gn, splits,
                                                      tm0, tn0, i0, i1, j0, j1, s);
  }
  if (tile == 5) {
    return store_s ? launch_t<D.tt, D.nw, true, FMT>(q8, w_rep, out, M, N, K, gm, gn, 1, tm0,
                                                     tn0, i0, i1, j0, j1, s)
                   : launch_t<D.tt, D.nw, false, FMT>(q8, w_rep, out, M, N, K, gm, gn, splits,
                                                      tm0, tn0, i0, i1, j0, j1, s);
  }
  return store_s ? launch_t<S.tt, S.nw, true, FMT>(q8, w_rep, out, M, N, K, gm, gn, 1, tm0, tn0,
                                                   i0, i1, j0, j1, s)
                 : launch_t<S.tt, S.nw, false, FMT>(q8, w_rep, out, M, N, K, gm, gn, splits, tm0,
                                                    tn0, i0, i1, j0, j1, s);
}

}  // namespace

hipError_t launch_mmq(int tile, const void* q8, const void* w_rep, void* out, int64_t M,
                      int64_t N, int64_t K, int64_t gm, int64_t gn, int64_t splits, int64_t tm0,
                      int64_t tn0, bool store_s, int64_t i0, int64_t i1, int64_t j0, int64_t j1,
                      hipStream_t s, int fmt) {
  return fmt == kFmtQ6K
             ? launch_fmt<kFmtQ6K>(tile, q8, w_rep, out, M, N, K, gm, gn, splits, tm0, tn0,
                                   store_s, i0, i1, j0, j1, s)
             : launch_fmt<kFmtQ4K>(tile, q8, w_rep, out, M, N, K, gm, gn, splits, tm0, tn0,
                                   store_s, i0, i1, j0, j1, s);
}

hipError_t launch_reduce_splits(const float* ws, float* C, int64_t M, int64_t N, int64_t splits,
                                hipStream_t s) {
  const int64_t n = M * N;
  if (N % 4 == 0) {
    const int64_t blocks = (n / 4 + 255) / 256;
    hipLaunchKernelGGL(reduce_splits_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, ws, C,
                       n, (int)splits);
  } else {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(reduce_splits_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, ws,
                       C, n, (int)splits);
  }
  return hipGetLastError();
}

}  // namespace mmq

/*
 * mmq.h -- C ABI of the q4_K x q8_1 quantized matrix multiply (MMQ) for LLM prefill
 * on AMD Instinct MI355X (gfx950, CDNA4).
 *
 *   C[M][N] = sum_k (da_i,b(k) * q_ik) * (dsv_j,b(k) * v_jk + dmv_j,b(k))
 *           = sum_b ( da_ib * dsv_jb * S_ijb  +  dmv_jb * (da_ib * sa_ib) )
 *
 * Activations are quantized to q8_1 blocks of 32 (int8 values q, an f16 scale da and the
 * integer block sum sa); weights are q4_K super-blocks of 256 (f16 d and dmin, 6-bit
 * sub-block scale sc and min m, unsigned nibbles v). S_ijb is the integer dot product of
 * one 32-block, dsv = d*sc, dmv = -dmin*m. Definitions: the r15 page ("f32-accumulate mma
 * probe + rank-1 term2 rescale", section 2.1, the two-term rescale), its section 3.2 (the
 * packed da/sa word) and the r16 page ("Narrow kernel gets the rank-1 fold", section 2.1,
 * the rank-1 term2 fold).
 *
 * Conventions for every entry point below:
 *   - Pointers named x, q8, w, w_rep, C, S are DEVICE pointers owned by the caller; the
 *     library never frees, keeps or allocates device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream). Kernels are enqueued on it and the
 *     call returns without synchronizing.
 *   - All arguments are validated on the host before anything is launched; on any error
 *     nothing is launched and nothing is written. Return value: an mmq_status code.
 *   - Buffers may not overlap. Device pointers must be 16-byte aligned.
 *   - Thread-safe: the per-device property cache is initialized once under a lock;
 *     mmq_last_kernel and mmq_last_error report the calling thread's last call.
 */
#ifndef MMQ_H
#define MMQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum mmq_status {
  MMQ_OK = 0,
  MMQ_E_ARG = 1,     /* null or misaligned pointer, non-positive size, bad option value */
  MMQ_E_SHAPE = 2,   /* K not a multiple of the block length, size overflow, bad window */
  MMQ_E_LDS = 3,     /* no tile fits the LDS budget: refused, nothing launched */
  MMQ_E_DEVICE = 4,  /* current device is not gfx950, or no device */
  MMQ_E_HIP = 5      /* a HIP runtime call or the kernel launch failed (see mmq_last_error) */
};

#define MMQ_QK8 32               /* q8_1 block length */
#define MMQ_QK_K 256             /* q4_K super-block length */
#define MMQ_Q4K_BLOCK_BYTES 144  /* bytes of one q4_K super-block */
#define MMQ_REP_TILE_ROWS 32     /* weight rows per repacked tile */
#define MMQ_REP_TILE_BYTES 4608  /* bytes per (repacked tile, super-block) */
#define MMQ_Q6K_BLOCK_BYTES 210  /* bytes of one q6_K super-block */
#define MMQ_REP6_TILE_BYTES 10240 /* bytes per (repacked q6_K tile, super-block) */

/* Tile variants of the GEMM: one template in four instantiations (large, half, medium,
 * small), a skinny kernel for few tokens that splits K over the wavefronts of a workgroup,
 * and a decode kernel for a handful of tokens in a vector-ALU and a matrix-unit form. */
enum mmq_tile {
  MMQ_TILE_AUTO = 0,   /* let the guard choose */
  MMQ_TILE_LARGE = 1,  /* 128 tokens x 256 output features per workgroup, 8 wavefronts */
  MMQ_TILE_SMALL = 2,  /* 32 tokens x 64 output features per workgroup, 2 wavefronts */
  MMQ_TILE_SKINNY = 3, /* 32 tokens x 32 output features per workgroup, K split over 8
                          wavefronts and summed in wavefront order (no block-dot output) */
  MMQ_TILE_GEMV = 4,   /* M <= 16 only (decode), 16 output features per workgroup, partial
                          sums added in a fixed order, no block-dot output, in two forms.
                          Vector-ALU form (threads = 512, block_m <= 8): 8 wavefronts, up to 8
                          tokens per workgroup, integer dot products on the vector ALU
                          (v_dot4_i32_i8), K split over 16 slices x 2 halves of each
                          super-block; taken for M <= 4, and for 5 <= M <= 8 when the LDS budget
                          is below the other form's. Matrix-unit form (block_m = 16): all tokens
                          in one workgroup, one v_mfma_i32_16x16x32_i8 per block, K split over
                          the wavefronts by super-block, each loading its next super-block's
                          weights while it computes one: 16 wavefronts and 16 rows per
                          workgroup (threads = 1024, block_n = 16, 128 KiB of LDS) when
                          ceil(N/16) workgroups fit the compute units once, 8 wavefronts and
                          32 rows (512, 32, 82 KiB) when ceil(N/32) fit, else 4 wavefronts and
                          16 rows (256, 16, 32 KiB); taken for 5 <= M <= 16 */
  MMQ_TILE_MEDIUM = 5, /* 32 tokens x 256 output features per workgroup, 8 wavefronts (the
                          template of the large and small tiles); with a workspace, K may be
                          split over workgroups (split-K, see mmq_options) */
  MMQ_TILE_HALF = 6    /* 64 tokens x 256 output features per workgroup, 8 wavefronts (the
                          same template): half the large tile's token rows, for grids the
                          large tile would leave short of compute units; split-K as medium */
};

/* Why the guard chose what it chose. */
enum mmq_reason {
  MMQ_REASON_NONE = 0,
  MMQ_REASON_LARGE = 1,         /* large tile fits the LDS budget and M is large enough */
  MMQ_REASON_SMALL_GRID = 2,    /* the large tile's grid would leave compute units idle */
  MMQ_REASON_LDS_FALLBACK = 3,  /* the large tile does not fit the LDS budget: small tile */
  MMQ_REASON_FORCED = 4,        /* the caller's options asked for this tile */
  MMQ_REASON_NO_FIT = 5,        /* nothing fits the budget: refused with MMQ_E_LDS */
  MMQ_REASON_FEW_TOKENS = 6,    /* 16 < M <= 256, K >= 2048, and the large grid would leave compute
                                   units idle:
                                   the skinny kernel, which splits K over wavefronts */
  MMQ_REASON_FUSED = 7,         /* mmq_q4K_f32: the vector-ALU (M <= 8) or skinny kernel quantizing
                                   its own activations */
  MMQ_REASON_DECODE = 8,        /* M <= 16: the decode tile, which streams the weights once
                                   without the large MFMA tiles' 32-token padding */
  MMQ_REASON_SPLIT_K = 9        /* the large grid would leave compute units idle and a workspace
                                   was given: a tile of the template, K split over
                                   workgroups */
};

/* Optional knobs for the _ex entry points (NULL = defaults). */
typedef struct mmq_options {
  int32_t force_tile;   /* enum mmq_tile. A forced tile that does not fit is refused (MMQ_E_LDS);
                           MMQ_TILE_GEMV with M > 16 is refused with MMQ_E_SHAPE */
  int32_t min_workgroups; /* > 0: choose the large tile only when its grid has at least this many
                             workgroups; 0: the device's compute-unit count (256 in mmq_plan) */
  int64_t lds_budget;   /* > 0: check tiles against this many bytes of LDS instead of the
                           device's per-workgroup limit (lets a caller force the fallback) */
  void* workspace;      /* device scratch for split-K partial sums, caller-owned, 16-byte
                           aligned, or NULL: with workspace_bytes > 0 the guard may split K over
                           workgroups (a tile of the template) when the large tile's grid would leave
                           compute units idle. Its contents on entry do not matter; on return
                           they are undefined. The library allocates nothing */
  int64_t workspace_bytes; /* usable bytes at workspace (0: no split-K) */
  int32_t splits;       /* > 0: split K into exactly this many super-block ranges (1 <= splits
                           <= K/256; more than 1 needs force_tile LARGE, HALF, MEDIUM or SMALL and a
                           workspace of splits*M*N*4 bytes); 0: the guard decides */
  int32_t reserved;     /* must be 0 */
} mmq_options;

/* What the guard decided for a product (filled by mmq_plan and by every GEMM call). */
typedef struct mmq_kernel_info {
  int32_t tile;         /* enum mmq_tile actually chosen; MMQ_TILE_AUTO (0) when none */
  int32_t reason;       /* enum mmq_reason */
  int32_t block_m;      /* tokens per workgroup */
  int32_t block_n;      /* output features per workgroup */
  int32_t threads;      /* threads per workgroup */
  int32_t fallback;     /* 1 when the large tile was rejected by the LDS budget */
  int64_t lds_bytes;    /* LDS the chosen kernel uses (0 when none) */
  int64_t lds_budget;   /* budget the guard checked against */
  int64_t grid;         /* workgroups launched by the GEMM kernel (1-D grid) */
  int32_t splits;       /* K ranges the GEMM is split into (1: no split-K) */
  int32_t reserved;
  int64_t workspace_bytes; /* workspace the split-K partial sums use: splits*M*N*4 when
                              splits > 1, else 0 */
} mmq_kernel_info;

/* ---------------------------------------------------------------- sizes (host only) */

/* Bytes of a q8_1 buffer for M x K activations (layout at quantize_q8_1): M*K int8 values,
 * M*(K/32) 32-bit scale words, padding to 256 bytes, M*(K/32) floats, padding to 256 bytes,
 * 48*M*ceil(K/256) bytes of bf16 pieces. K must be a positive multiple of 32. */
int mmq_q8_1_bytes(int64_t M, int64_t K, size_t* bytes);

/* Bytes of q4_K weights N x K in the GGUF layout: N*(K/256)*144. K % 256 == 0. */
int mmq_q4K_bytes(int64_t N, int64_t K, size_t* bytes);

/* Bytes of repacked q4_K weights: ceil(N/32)*(K/256)*4608 (4.5 bits per weight, the size
 * of the GGUF blocks). K % 256 == 0. */
int mmq_q4K_repacked_bytes(int64_t N, int64_t K, size_t* bytes);

/* ---------------------------------------------------------------- the hot path */

/*
 * quantize_q8_1: f32 activations x[M][K] (row-major, leading dimension K) -> q8_1.
 * Defined on the r15 page, section 2.1 (blocks of 32 with scale da and integer in-block sum
 * sa, computed by the quantize prepass). Per block of 32 values, in float32:
 *   amax = max|x|, d = amax/127 (IEEE division), id = d > 0 ? 1/d : 0,
 *   q = roundf(x*id) clamped to [-127, 127] (a NaN product, which only a block whose 1/d
 *   overflows can produce from x = 0, gives 0), sa = sum of q, da = f16(d) (nearest even).
 * Output layout of q8 (mmq_q8_1_bytes(M, K) bytes):
 *   bytes [0, M*K):          int8 q, row-major [M][K]
 *   bytes [M*K, M*K*9/8):    uint32 words [M][K/32]: bits 0..15 = f16 bits of da,
 *                            bits 16..31 = sa as a signed 16-bit integer (|sa| <= 4064)
 *                            (the packed da/sa word of the r15 page, section 3.2)
 *   up to P = the next multiple of 256: padding (not written)
 *   bytes [P, P + 8*M*K/32): float pairs (da, nda) [K/32][M] (block-major): da, the token
 *                            factor of term1, and nda = -1.5 * 2^23 * da (exact), the
 *                            constant of the GEMM's rescale of its integer results, which
 *                            come offset by 1.5 * 2^23
 *   up to Q = the next multiple of 256: padding (not written)
 *   bytes [Q, Q + 48*M*ceil(K/256)): uint16 bf16 pieces [K/256 rounded up][3][M][8]: piece
 *                            i of da*sa of row r, block 8s+e at [s][i][r][e]. da*sa is the
 *                            folded row factor of term2 (r16 page, section 2.1), exact in
 *                            float32; the pieces are p0 = bf16_rne(v), p1 = bf16_rne(v - p0),
 *                            p2 = v - p0 - p1, which sum to v exactly (a non-finite v is
 *                            stored as {top 16 bits of v, 0, 0}). Slots of blocks past K/32
 *                            are not written.
 * Preconditions: finite x with |x| <= 8.3e6 (so that amax/127 fits f16). K % 32 == 0;
 * M*K < 2^34 (the GEMM takes M*K < 2^31).
 * Errors: MMQ_E_ARG (null pointer, M or K <= 0), MMQ_E_SHAPE (K % 32, M*K too large),
 *         MMQ_E_DEVICE, MMQ_E_HIP.
 */
int quantize_q8_1(const float* x, int64_t M, int64_t K, void* q8, void* stream);

/*
 * repack_q4_K: q4_K weights (GGUF layout, [N][K/256] super-blocks of 144 bytes, the fields of
 * the r15 page, section 2.1) -> the kernels' layout. Run once per weight matrix.
 * Output (mmq_q4K_repacked_bytes(N, K) bytes): one 4608-byte record per (tile t of 32 weight
 * rows, super-block s), records ordered [t][s]; rows N..32*ceil(N/32)-1 are zero. Record:
 *   bytes [0, 4096):   nibbles, [g 0..3][h 0..1][j 0..31][16 bytes] = bytes 32g+16h .. +15 of
 *                      the 128 nibble bytes of row 32t+j (low nibble: sub-block 2g, element
 *                      16h+e; high nibble: sub-block 2g+1, element 16h+e)
 *   bytes [4096, 4608): [j 0..31][16 bytes] = bytes 0..15 of row 32t+j's block, unchanged:
 *                       f16 d, f16 dmin, the 12 bytes of packed 6-bit sc and m
 * The kernels expand the scales of sub-block b from the header as they stage it:
 * dsv = d*sc and dmv = -(dmin*m), both exact in float32 (and dmv for the matrix unit as the
 * three bf16 pieces that sum to it exactly: the top 16 bits of dmv, the top 16 bits of what
 * is left, and the rest). Precondition of the products: finite d and dmin in every block
 * (a non-finite one leaves its row's outputs unspecified).
 * Errors: MMQ_E_ARG, MMQ_E_SHAPE (K % 256; ceil(N/32)*(K/256) >= 2^31), MMQ_E_DEVICE,
 *         MMQ_E_HIP.
 */
int repack_q4_K(const void* w_q4K, int64_t N, int64_t K, void* w_rep, void* stream);

/*
 * mmq_q4K_q8_1: C[M][N] (float32, row-major, leading dimension N; overwritten) =
 *   sum over 32-blocks b of  da_ib*dsv_jb*S_ijb  +  dmv_jb*(da_ib*sa_ib)
 * (the two-term rescale of the r15 page, section 2.1, with the row factor da*sa folded once
 * per token row as on the r16 page, section 2.1). q8 comes from quantize_q8_1 (M x K), w_rep
 * from repack_q4_K (N x K). S_ijb is computed exactly with int8 MFMA and term1 of each block
 * is added to a float32 accumulator in increasing b. term2 of each super-block is added as
 * three bf16 matrix products of the pieces of dmv and da*sa (six of the nine piece pairs:
 * every product is exact, the three dropped pairs are below 2^-17 of |dmv*da*sa| per
 * block), after the term1 of its blocks 1, 3 and 5. The order is fixed, so the result is
 * deterministic and the same for every tile variant.
 * M, N >= 1 (any value; ragged tiles are masked), K % 256 == 0, K <= 2^24, M*K < 2^31.
 * Errors: MMQ_E_ARG, MMQ_E_SHAPE, MMQ_E_LDS (no tile fits), MMQ_E_DEVICE, MMQ_E_HIP.
 */
int mmq_q4K_q8_1(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                 float* C, void* stream);

/*
 * As mmq_q4K_q8_1, with options (tile choice, LDS budget, split-K workspace); opt may be NULL.
 * With a workspace (opt->workspace, opt->workspace_bytes) and a product whose large-tile grid
 * would leave compute units idle (few tokens or few output features: M = 128..1024 at
 * N = 4096, one GPU's share of a column-split layer), the guard may choose a tile
 * with K split into `splits` ranges of super-blocks: each workgroup writes the partial sums
 * of its range to plane [split] of the workspace ([splits][M][N] float32), and a second kernel
 * adds the planes into C in increasing split order. The result is deterministic (the same
 * bits on every call) and within the same bound as the unsplit product, but it associates
 * the sum differently. Both kernels run on `stream`; the workspace must not be used by other
 * work until the call's kernels have finished.
 * Errors: as mmq_q4K_q8_1; MMQ_E_ARG for a bad option (a null or misaligned workspace with
 * workspace_bytes > 0, a forced split the workspace cannot hold, reserved != 0).
 */
int mmq_q4K_q8_1_ex(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                    float* C, void* stream, const mmq_options* opt);

/* Bytes of split-K workspace the guard would use for an M x N x K product given an unlimited
 * workspace (0 when it would not split K). Host only. */
int mmq_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);

/*
 * mmq_q4K_q8_1_static: for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). The same product, kernels
 * and guard as mmq_q4K_q8_1_ex, with the split-K workspace taken from a 32 MiB array of device
 * memory that the library's code object holds (one per GPU, for the life of the process)
 * instead of the caller's buffer; the guard plans its splits within those 32 MiB. The call
 * allocates nothing. opt may be NULL and must carry no workspace. Every call on a GPU uses
 * that GPU's one array, so calls that overlap on one GPU (on different streams, or from
 * several threads) race and must be serialized by the caller; the array's contents between
 * calls do not matter (each split-K call writes every partial sum it reads).
 * Errors: as mmq_q4K_q8_1_ex; MMQ_E_ARG for a workspace in opt, or forced splits whose
 * partial planes (splits*M*N*4 bytes) exceed 32 MiB; MMQ_E_HIP if the array's device address
 * cannot be found.
 */
int mmq_q4K_q8_1_static(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                        float* C, void* stream, const mmq_options* opt);

/*
 * mmq_q4K_f32: the product for few tokens straight from float32 activations x[M][K]
 * (row-major, leading dimension K), quantizing them inside the GEMM. C is bit for bit what
 * quantize_q8_1 followed by mmq_q4K_q8_1_ex writes with MMQ_TILE_GEMV in its vector-ALU form
 * (M <= 8; the form mmq_q4K_q8_1_ex takes under an LDS budget below the matrix-unit form's)
 * or with MMQ_TILE_SKINNY (8 < M <= 128), but no q8 buffer goes through memory and there is
 * one launch instead of two. Each workgroup quantizes, into LDS, the activations of the
 * super-blocks it works on (the quantization of quantize_q8_1: the r15 page, section 2.1),
 * then runs the unfused kernel's arithmetic on them. Every workgroup that needs a token's
 * super-block repeats that quantization, so the call is limited to few tokens:
 * 1 <= M <= 128. It pays for the fewest: at K = N = 4096, replayed from a graph over weights
 * that do not stay in cache, one call takes 5.3, 6.2 and 8.3 us at M = 1, 2 and 4, against
 * 7.5, 7.9 and 8.9 us for quantize_q8_1 followed by the decode tile; from M = 5 the two
 * kernels are faster (8.8 against 9.7 us, at M = 8 8.7 against 12.3).
 * w_rep from repack_q4_K (N x K); C overwritten as for mmq_q4K_q8_1; mmq_last_kernel reports
 * the tile (MMQ_TILE_GEMV or MMQ_TILE_SKINNY) with reason MMQ_REASON_FUSED.
 * Errors: MMQ_E_ARG, MMQ_E_SHAPE (as mmq_q4K_q8_1, or M > 128), MMQ_E_LDS (the kernel's LDS
 * does not fit the device's per-workgroup limit), MMQ_E_DEVICE, MMQ_E_HIP.
 */
int mmq_q4K_f32(int64_t M, int64_t N, int64_t K, const float* x, const void* w_rep,
                float* C, void* stream);

/*
 * mmq_q4K_q8_1_blockdots: the per-block integer dot products S_ijb = sum_{k in block b}
 * q_ik * v_jk (the r15 page, section 2.1) for a window of tokens [i0, i1) and output
 * features [j0, j1), through the same GEMM kernel template with a store-S epilogue.
 * S (int32, device) has layout [K/32][i1-i0][j1-j0]. For testing bit-exactness.
 * Errors: as mmq_q4K_q8_1; MMQ_E_SHAPE for an empty or out-of-range window.
 */
int mmq_q4K_q8_1_blockdots(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                           int64_t i0, int64_t i1, int64_t j0, int64_t j1, int32_t* S,
                           void* stream, const mmq_options* opt);

/* ---------------------------------------------------------------- the q6_K variant */

/*
 * The q6_K weight format (the r16 page, sections 2.3 and 5, names the q6_K kernel family that
 * the rank-1 fold was carried over to; the pages give no layout, and the GGUF q6_K layout is
 * the reading taken): 256 values per 210-byte super-block, each a 6-bit u whose weight value
 * is the signed integer u - 32, one int8 scale sc per 16 consecutive values and one f16 d:
 *   bytes 0..127   low 4 bits: value 128h + 32q + l (h = 0..1, q = 0..3, l = 0..31) in byte
 *                  64h + 32(q mod 2) + l, the low nibble for q < 2, the high one for q >= 2
 *   bytes 128..191 high 2 bits: bits 2q..2q+1 of byte 128 + 32h + l
 *   bytes 192..207 the 16 scales (int8), scale g for values 16g..16g+15
 *   bytes 208..209 d (f16, little endian)
 * so w = d * sc * (u - 32). The product with q8_1 activations is one term per group of 16:
 *   C_ij = sum_g da_i,b(g) * dsv_jg * S_ijg,  S_ijg = sum_{k in g} q_ik (u_jk - 32), dsv = d*sc.
 * The int8 MFMA is signed, so it takes the values u - 32 directly and the offset needs no
 * rank-1 correction (the fold form on the pages computes the same S from u and the group
 * sums of q).
 */
int mmq_q6K_bytes(int64_t N, int64_t K, size_t* bytes);          /* N*(K/256)*210 */
int mmq_q6K_repacked_bytes(int64_t N, int64_t K, size_t* bytes); /* ceil(N/32)*(K/256)*10240 */

/*
 * repack_q6_K: q6_K blocks [N][K/256] of 210 bytes -> one 10240-byte record per (tile t of 32
 * weight rows, super-block s), records ordered [t][s]; rows N..32*ceil(N/32)-1 are zero:
 *   bytes [0, 8192):     int8 u - 32, [b 0..7][h 0..1][j 0..31][16 bytes] = values
 *                        32b + 16h .. +15 of the super-block of row 32t+j
 *   bytes [8192, 10240): float dsv[g 0..15][j 0..31] = d*sc_g of row 32t+j (exact in f32)
 * Errors: MMQ_E_ARG (null pointer, w_rep not 16-byte aligned, N or K <= 0), MMQ_E_SHAPE (K %
 * 256; ceil(N/32)*(K/256) >= 2^31), MMQ_E_DEVICE, MMQ_E_HIP.
 */
int repack_q6_K(const void* w_q6K, int64_t N, int64_t K, void* w_rep, void* stream);

/*
 * mmq_q6K_q8_1: C[M][N] (float32, row-major, overwritten) = the product above, from q8 of
 * quantize_q8_1 (M x K) and w_rep of repack_q6_K (N x K). The GEMM template of the q4_K
 * product (large, half, medium and small tiles, the same guard, split-K with a workspace through
 * the _ex options): per 32-block two int8 MFMAs, each keeping one 16-value group (the lane half
 * that holds it), S_ijg exact; per group y = RN(S * da), acc += dsv * y, groups in increasing
 * order (deterministic). There is no skinny or decode kernel for q6_K.
 * Same preconditions and errors as mmq_q4K_q8_1 (forcing MMQ_TILE_SKINNY or MMQ_TILE_GEMV is
 * MMQ_E_ARG).
 */
int mmq_q6K_q8_1(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                 float* C, void* stream);
int mmq_q6K_q8_1_ex(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                    float* C, void* stream, const mmq_options* opt);

/* The q6_K group dot products S_ijg for a window, S int32 [K/16][i1-i0][j1-j0] (test path). */
int mmq_q6K_q8_1_blockdots(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                           int64_t i0, int64_t i1, int64_t j0, int64_t j1, int32_t* S,
                           void* stream, const mmq_options* opt);

/* ---------------------------------------------------------------- the guard (host only) */

/*
 * mmq_plan: the LDS-budget guard as a pure host function (no device access). Chooses the
 * tile for an M x N x K product given `lds_budget` bytes per workgroup (opt->lds_budget,
 * when set, takes precedence): for M <= 16 the decode tile (MMQ_TILE_GEMV, reason
 * MMQ_REASON_DECODE, in the form that enum entry describes, with the compute-unit count as
 * below); else, with no workspace, the large tile when it fits and its grid has
 * at least opt->min_workgroups workgroups (default 256, the MI355X compute-unit count; a GEMM
 * call uses the device's count); else the cheapest choice under a cost model (rounds of the
 * grid over the compute units times a per-tile cost per super-block, plus the partial
 * planes' traffic of a split) among the large, half, medium and small tiles that fit (with a
 * workspace, each with K split into 1, 2, 4, 8 or 16 ranges: MMQ_REASON_SPLIT_K; see
 * mmq_q4K_q8_1_ex) and, for M <= 256 and K >= 2048 (at least one super-block for each of its
 * wavefronts), the skinny kernel (MMQ_REASON_FEW_TOKENS); an unsplit half, medium or small tile is
 * reported as MMQ_REASON_SMALL_GRID. When the large tile does not fit the budget, the small
 * tile (fallback = 1, MMQ_REASON_LDS_FALLBACK); when nothing fits, MMQ_E_LDS. A
 * kernel that does not fit the budget is never launched: on the r16 page
 * (section 1) an over-budget launch failed silently and produced wrong numbers, so here
 * the fallback is explicit and reported (fallback, reason), and a refusal is an error.
 */
int mmq_plan(int64_t M, int64_t N, int64_t K, const mmq_options* opt, int64_t lds_budget,
             mmq_kernel_info* out);

/* The guard decision of the calling thread's last GEMM or blockdots call. */
int mmq_last_kernel(mmq_kernel_info* out);

/* Static text for a status code. */
const char* mmq_status_str(int status);

/* Detail of the calling thread's last error (empty string when the last call succeeded). */
const char* mmq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MMQ_H */

// Host side of the C ABI declared in include/mmq.h: argument validation, the LDS-budget
// guard, the per-device property cache and the launches. Nothing here touches the device
// before every argument has been validated, so the validation and the guard can be
// exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mmq.h"
#include "mmq_f16.h"
#include "mmq_internal.h"

namespace {

thread_local mmq_kernel_info g_last = {};
thread_local char g_err[512] = {0};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return MMQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every in-kernel 32-bit index in range
constexpr int64_t kMaxK = (int64_t)1 << 24;

constexpr int64_t kDefaultComputeUnits = 256;  // MI355X; mmq_plan assumes it
constexpr int64_t kDefaultLdsBudget = 160 * 1024;  // MI355X per-workgroup LDS
// The guard considers the skinny kernel (K split over the wavefronts of a workgroup) up to
// this many tokens: at K = N = 4096 it takes 10.5 / 16.3 / 22.1 / 27.7 us for M = 32 / 128 /
// 192 / 256 against 31.0 / 31.1 / 32.3 / 32.9 us for the small tile, ties it at 320 and
// loses from 384 (38.9 against 33.7 us for the medium tile).
constexpr int64_t kSkinnyGuardMaxM = 256;
// mmq_q4K_f32 (the skinny kernel quantizing its own token tile in every workgroup) takes up
// to this many tokens.
constexpr int64_t kFusedMaxM = 128;
struct DeviceInfo {
  std::once_flag once;
  int status = MMQ_OK;
  int64_t lds_budget = 0;
  int64_t compute_units = kDefaultComputeUnits;
  char msg[256] = {0};
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];

// Checks the current device once: it must be gfx950; records its per-workgroup LDS limit.
int current_device(DeviceInfo** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(MMQ_E_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(MMQ_E_DEVICE, "device index %d out of range", dev);
  DeviceInfo& di = g_dev[dev];
  std::call_once(di.once, [&di, dev]() {
    hipDeviceProp_t prop;
    hipError_t pe = hipGetDeviceProperties(&prop, dev);
    if (pe != hipSuccess) {
      di.status = MMQ_E_DEVICE;
      snprintf(di.msg, sizeof(di.msg), "hipGetDeviceProperties: %s", hipGetErrorString(pe));
      return;
    }
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      di.status = MMQ_E_DEVICE;
      snprintf(di.msg, sizeof(di.msg), "device %d is %s, this library is built for gfx950", dev,
               prop.gcnArchName);
      return;
    }
    // the per-workgroup LDS limit: the default one, or the larger one a kernel may opt in to
    // (the GEMM launch opts in with hipFuncSetAttribute when it needs more than 64 KiB)
    int lds = 0, lds_optin = 0;
    pe = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (pe != hipSuccess || lds <= 0) {
      di.status = MMQ_E_DEVICE;
      snprintf(di.msg, sizeof(di.msg), "cannot read the LDS limit: %s", hipGetErrorString(pe));
      return;
    }
    if (hipDeviceGetAttribute(&lds_optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) !=
        hipSuccess)
      lds_optin = 0;
    (void)hipGetLastError();  // an unsupported attribute query leaves no sticky error
    di.lds_budget = lds_optin > lds ? lds_optin : lds;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = kDefaultComputeUnits;
    (void)hipGetLastError();
    di.compute_units = cus;
  });
  if (di.status != MMQ_OK) return fail(di.status, "%s", di.msg);
  *out = &di;
  return MMQ_OK;
}

int check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(MMQ_E_ARG, "M, N, K must be positive (%lld, %lld, %lld)",
                                              (long long)M, (long long)N, (long long)K);
  if (K % MMQ_QK_K) return fail(MMQ_E_SHAPE, "K = %lld is not a multiple of 256", (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxK)
    return fail(MMQ_E_SHAPE, "M or N above 2^30, or K above 2^24");
  // the GEMM addresses its operands with 32-bit buffer offsets
  if ((__int128)M * K >= ((__int128)1 << 31) || (__int128)M * N > ((__int128)1 << 40))
    return fail(MMQ_E_SHAPE, "activations of M*K >= 2^31 bytes, or an output above 2^40 elements");
  return MMQ_OK;
}

int check_options(const mmq_options* opt) {
  if (!opt) return MMQ_OK;
  if (opt->force_tile < MMQ_TILE_AUTO || opt->force_tile > MMQ_TILE_HALF)
    return fail(MMQ_E_ARG, "force_tile %d is not an mmq_tile", opt->force_tile);
  if (opt->lds_budget < 0) return fail(MMQ_E_ARG, "negative lds_budget");
  if (opt->min_workgroups < 0) return fail(MMQ_E_ARG, "negative min_workgroups");
  if (opt->workspace_bytes < 0) return fail(MMQ_E_ARG, "negative workspace_bytes");
  if (opt->splits < 0) return fail(MMQ_E_ARG, "negative splits");
  if (opt->reserved != 0) return fail(MMQ_E_ARG, "mmq_options.reserved must be 0");
  return MMQ_OK;
}

// Split-K: at most this many super-block ranges (the partial planes cost 8*M*N bytes of
// memory traffic each, written and read back).
constexpr int64_t kMaxSplits = 16;

// The guard's cost model of the template's tiles, fitted to graph-replayed timings of 22
// few-token and few-feature shapes (M = 32..2048 at N = 4096 and 11008, K = 4096 and 11008;
// one GPU's share of an 8-way column split of the 7B projections) under every tile and split
// count 1..16, with and without a workspace: a workgroup spends c microseconds per
// super-block, `occ` workgroups share a compute unit, and each split adds its partial
// plane's traffic. The model's pick is 0.6 % above the fastest measured choice on average
// over the 44 cases (14 % at worst: 32 x 11008 x 4096 with a workspace, the skinny kernel
// where the small tile with 4 splits was fastest).
struct TileCost {
  int tile;
  double us_per_sb;  // per super-block and round of workgroups
  double occ;        // workgroups per compute unit (registers and LDS)
};
constexpr TileCost kTileCosts[] = {{MMQ_TILE_LARGE, 3.4, 1.0},
                                   {MMQ_TILE_HALF, 2.6, 1.0},
                                   {MMQ_TILE_MEDIUM, 2.1, 1.0},
                                   {MMQ_TILE_SMALL, 1.7, 2.5}};
constexpr double kUsPerPartialMB = 0.45;
// The skinny kernel in the same model: one workgroup per 32 x 32 output tile, its 8
// wavefronts each walking K/8 super-blocks; one workgroup per compute unit at a time when
// the grid fits the device in one round, else the form that shares a compute unit between
// two (an effective 1.2 per compute unit).
constexpr double kSkinnyUsPerSb = 3.6;
constexpr double kSkinnyOccLargeGrid = 1.2;

// the tiles of the GEMM template, which can split K
bool template_tile(int tile) {
  return tile == MMQ_TILE_LARGE || tile == MMQ_TILE_HALF || tile == MMQ_TILE_MEDIUM ||
         tile == MMQ_TILE_SMALL;
}

mmq::TileShape tile_shape(int tile) {
  return tile == MMQ_TILE_LARGE    ? mmq::kLarge
         : tile == MMQ_TILE_HALF   ? mmq::kHalf
         : tile == MMQ_TILE_MEDIUM ? mmq::kMedium
                                   : mmq::kSmall;
}

// The guard: which tile, given the LDS budget and the compute units the grid should fill.
int plan(int64_t M, int64_t N, int64_t K, const mmq_options* opt, int64_t budget,
         int64_t compute_units, mmq_kernel_info* info, int fmt = mmq::kFmtQ4K) {
  const bool q6 = fmt == mmq::kFmtQ6K;
  memset(info, 0, sizeof(*info));
  if (opt && opt->lds_budget > 0) budget = opt->lds_budget;
  const int64_t min_wg = opt && opt->min_workgroups > 0 ? opt->min_workgroups : compute_units;
  auto grid_of = [&](const mmq::TileShape& ts) {
    const int64_t gm = (M + ts.block_m() - 1) / ts.block_m();
    const int64_t gn = ((N + 31) / 32 + ts.nw - 1) / ts.nw;
    return gm * gn;
  };
  info->lds_budget = budget;
  const int64_t need_large = mmq::kLarge.lds_bytes(fmt);
  const int64_t need_small = mmq::kSmall.lds_bytes(fmt);
  const int64_t need_medium = mmq::kMedium.lds_bytes(fmt);
  const int64_t need_half = mmq::kHalf.lds_bytes(fmt);
  const int forced = opt ? opt->force_tile : MMQ_TILE_AUTO;
  if (q6 && (forced == MMQ_TILE_SKINNY || forced == MMQ_TILE_GEMV))
    return fail(MMQ_E_ARG, "the q6_K product has no skinny or decode kernel: force large, medium "
                           "or small");
  const int64_t nsb = K / 256;
  const int64_t ws_bytes = opt ? opt->workspace_bytes : 0;
  const int64_t forced_splits = opt ? opt->splits : 0;
  auto plane_bytes = [&](int64_t sp) { return sp > 1 ? sp * M * N * 4 : 0; };
  if (forced_splits > 0) {
    if (forced_splits > nsb)
      return fail(MMQ_E_ARG, "splits = %lld is more than the %lld super-blocks of K",
                  (long long)forced_splits, (long long)nsb);
    if (forced_splits > 1 && !template_tile(forced))
      return fail(MMQ_E_ARG, "split-K needs force_tile LARGE, HALF, MEDIUM or SMALL");
    if (plane_bytes(forced_splits) > ws_bytes)
      return fail(MMQ_E_ARG, "%lld splits need %lld bytes of workspace, %lld given",
                  (long long)forced_splits, (long long)plane_bytes(forced_splits),
                  (long long)ws_bytes);
  }
  int64_t splits = forced_splits > 0 ? forced_splits : 1;

  int tile = 0, reason = MMQ_REASON_NONE, fallback = 0;
  // the decode tile's form (0: vector ALU, else the matrix-unit form's wavefronts): up to
  // kGemvDotMaxM tokens the matrix-unit form only where it fits the budget (the vector-ALU
  // form needs far less LDS)
  const int mfma_waves = mmq::gemv_mfma_waves(N, compute_units);
  const int mfma_rows = mmq::gemv_mfma_rows(N, compute_units);
  const int gemv_form =
      mmq::gemv_mfma_form(M) &&
              (M > mmq::kGemvDotMaxM || mmq::gemv_lds_bytes(M, mfma_waves, mfma_rows) <= budget)
          ? mfma_waves
          : 0;
  const int gemv_rows = gemv_form ? mfma_rows : mmq::kGemvRows;
  if (forced == MMQ_TILE_LARGE) {
    if (need_large <= budget) { tile = MMQ_TILE_LARGE; reason = MMQ_REASON_FORCED; }
  } else if (forced == MMQ_TILE_SMALL) {
    if (need_small <= budget) { tile = MMQ_TILE_SMALL; reason = MMQ_REASON_FORCED; }
  } else if (forced == MMQ_TILE_MEDIUM) {
    if (need_medium <= budget) { tile = MMQ_TILE_MEDIUM; reason = MMQ_REASON_FORCED; }
  } else if (forced == MMQ_TILE_HALF) {
    if (need_half <= budget) { tile = MMQ_TILE_HALF; reason = MMQ_REASON_FORCED; }
  } else if (forced == MMQ_TILE_SKINNY) {
    if (mmq::skinny_lds_bytes() <= budget) { tile = MMQ_TILE_SKINNY; reason = MMQ_REASON_FORCED; }
  } else if (forced == MMQ_TILE_GEMV) {
    if (M > mmq::kGemvMaxM)
      return fail(MMQ_E_SHAPE, "the decode tile takes M <= %d (M = %lld)", mmq::kGemvMaxM,
                  (long long)M);
    if (mmq::gemv_lds_bytes(M, gemv_form, gemv_rows) <= budget) {
      tile = MMQ_TILE_GEMV; reason = MMQ_REASON_FORCED;
    }
  } else if (!q6 && M <= mmq::kGemvAutoMaxM && mmq::gemv_lds_bytes(M, gemv_form, gemv_rows) <= budget) {
    tile = MMQ_TILE_GEMV; reason = MMQ_REASON_DECODE;
  } else if (need_large <= budget) {
    // the cheapest (tile, splits) under the cost model: splits only with a workspace that
    // holds their planes, each split at least one super-block
    const double cus = (double)compute_units;
    double best = 1e300;
    int best_tile = 0;
    int64_t best_sp = 1;
    if (!q6 && M <= kSkinnyGuardMaxM && nsb >= mmq::kSkinnyWaves &&
        mmq::skinny_lds_bytes() <= budget) {
      // (below 8 super-blocks some of the skinny kernel's wavefronts get none, and the small
      // tile is faster: 5.5 against 7.6 us at 128 x 256 x 512)
      const double grid = (double)(((M + 31) / 32) * ((N + 31) / 32));
      const double occ = grid > cus ? kSkinnyOccLargeGrid : 1.0;
      const double rounds = grid / (cus * occ) > 1.0 ? grid / (cus * occ) : 1.0;
      best = kSkinnyUsPerSb * rounds * (double)((nsb + mmq::kSkinnyWaves - 1) / mmq::kSkinnyWaves);
      best_tile = MMQ_TILE_SKINNY;
    }
    for (const TileCost& c : kTileCosts) {
      if (tile_shape(c.tile).lds_bytes(fmt) > budget) continue;
      for (int64_t sp = 1; sp <= kMaxSplits && sp <= nsb; sp *= 2) {
        if (sp > 1 && plane_bytes(sp) > ws_bytes) break;
        // the large tile only with a grid of at least min_wg workgroups
        if (c.tile == MMQ_TILE_LARGE && grid_of(mmq::kLarge) * sp < min_wg) continue;
        const double grid = (double)grid_of(tile_shape(c.tile)) * (double)sp;
        const double rounds = grid / (cus * c.occ) > 1.0 ? grid / (cus * c.occ) : 1.0;
        const double per_wg = (double)((nsb + sp - 1) / sp);
        double cost = c.us_per_sb * rounds * per_wg;
        if (sp > 1) cost += kUsPerPartialMB * (double)(8 * sp + 4) * (double)M * (double)N * 1e-6;
        if (cost < best) { best = cost; best_tile = c.tile; best_sp = sp; }
      }
    }
    if ((grid_of(mmq::kLarge) >= min_wg && ws_bytes == 0) || best_tile == MMQ_TILE_LARGE) {
      tile = MMQ_TILE_LARGE;
      reason = best_sp > 1 ? MMQ_REASON_SPLIT_K : MMQ_REASON_LARGE;
      splits = grid_of(mmq::kLarge) >= min_wg && ws_bytes == 0 ? 1 : best_sp;
    } else if (best_sp > 1) {
      tile = best_tile; reason = MMQ_REASON_SPLIT_K; splits = best_sp;
    } else if (best_tile == MMQ_TILE_SKINNY) {
      tile = MMQ_TILE_SKINNY; reason = MMQ_REASON_FEW_TOKENS;
    } else {
      tile = best_tile ? best_tile : MMQ_TILE_SMALL; reason = MMQ_REASON_SMALL_GRID;
    }
  } else if (need_small <= budget) {
    tile = MMQ_TILE_SMALL; reason = MMQ_REASON_LDS_FALLBACK; fallback = 1;
  }
  if (!tile) {
    info->reason = MMQ_REASON_NO_FIT;
    return fail(MMQ_E_LDS, "no GEMM tile fits %lld bytes of LDS (large needs %lld, small %lld)",
                (long long)budget, (long long)need_large, (long long)need_small);
  }
  info->tile = tile;
  info->reason = reason;
  info->fallback = fallback;
  info->splits = 1;
  if (splits > 1 && !template_tile(tile))
    splits = 1;  // (an LDS fallback to another kind of kernel drops a forced split)
  if (tile == MMQ_TILE_GEMV) {
    info->block_m = (int32_t)mmq::gemv_group(M, gemv_form);
    info->block_n = gemv_rows;
    info->threads = 64 * (gemv_form ? gemv_form : mmq::kGemvWaves);
    info->lds_bytes = mmq::gemv_lds_bytes(M, gemv_form, gemv_rows);
    info->grid = mmq::gemv_grid(M, N, gemv_form, gemv_rows);
    return MMQ_OK;
  }
  if (tile == MMQ_TILE_SKINNY) {
    info->block_m = 32;
    info->block_n = 32;
    info->threads = 64 * mmq::kSkinnyWaves;
    info->lds_bytes = mmq::skinny_lds_bytes();
    info->grid = ((M + 31) / 32) * ((N + 31) / 32);
    return MMQ_OK;
  }
  const mmq::TileShape ts = tile_shape(tile);
  const int64_t gm = (M + ts.block_m() - 1) / ts.block_m();
  const int64_t ntiles = (N + 31) / 32;
  const int64_t gn = (ntiles + ts.nw - 1) / ts.nw;
  info->block_m = ts.block_m();
  info->block_n = ts.block_n();
  info->threads = ts.threads();
  info->lds_bytes = ts.lds_bytes(fmt);
  info->grid = gm * gn * splits;
  info->splits = (int32_t)splits;
  info->workspace_bytes = plane_bytes(splits);
  return MMQ_OK;
}

int hip_fail(const char* what, hipError_t e) {
  return fail(MMQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Argument checks of the GEMM entry points, before any device access.
int check_gemm_call(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                    const float* C, const mmq_options* opt) {
  int st = check_gemm_shape(M, N, K);
  if (st) return st;
  if ((st = check_options(opt))) return st;
  if (!q8 || !w_rep || !C) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(q8) || !aligned16(w_rep) || !aligned16(C))
    return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  return MMQ_OK;
}

// Launch what the guard planned; with split-K the GEMM writes the partial planes into ws and
// a second kernel adds them into C, both on the stream.
int launch_planned(const mmq_kernel_info& info, int64_t M, int64_t N, int64_t K, const void* q8,
                   const void* w_rep, float* C, void* ws, int64_t compute_units,
                   hipStream_t stream, int fmt = mmq::kFmtQ4K) {
  hipError_t e;
  if (info.tile == MMQ_TILE_GEMV) {
    // the form the guard chose: the matrix-unit form takes all tokens in one workgroup, with
    // threads / 64 wavefronts and block_n weight rows
    e = mmq::launch_mmq_gemv(q8, w_rep, C, M, N, K,
                             info.block_m == mmq::kGemvMaxM ? info.threads / 64 : 0,
                             info.block_n, stream);
  } else if (info.tile == MMQ_TILE_SKINNY) {
    e = mmq::launch_mmq_skinny(q8, w_rep, C, M, N, K, compute_units, stream);
  } else {
    const mmq::TileShape ts = tile_shape(info.tile);
    const int64_t gm = (M + ts.block_m() - 1) / ts.block_m();
    const int64_t gn = ((N + 31) / 32 + ts.nw - 1) / ts.nw;
    const int64_t sp = info.splits;
    e = mmq::launch_mmq(info.tile, q8, w_rep, sp > 1 ? ws : C, M, N, K, gm, gn, sp, 0, 0, false,
                        0, 0, 0, 0, stream, fmt);
    if (e == hipSuccess && sp > 1)
      e = mmq::launch_reduce_splits(static_cast<const float*>(ws), C, M, N, sp, stream);
  }
  if (e != hipSuccess) return hip_fail("mmq_q4K_q8_1 launch", e);
  return ok();
}

// The GEMM entry points of both weight formats: validate, plan, launch.
int gemm_ex(int fmt, int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
            float* C, void* stream, const mmq_options* opt) {
  int st = check_gemm_call(M, N, K, q8, w_rep, C, opt);
  if (st) return st;
  if (opt && opt->workspace_bytes > 0 && (!opt->workspace || !aligned16(opt->workspace)))
    return fail(MMQ_E_ARG, "workspace_bytes > 0 needs a 16-byte aligned workspace");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  mmq_kernel_info info;
  st = plan(M, N, K, opt, di->lds_budget, di->compute_units, &info, fmt);
  g_last = info;
  if (st) return st;
  return launch_planned(info, M, N, K, q8, w_rep, C, opt ? opt->workspace : nullptr,
                        di->compute_units, static_cast<hipStream_t>(stream), fmt);
}

int blockdots(int fmt, int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
              int64_t i0, int64_t i1, int64_t j0, int64_t j1, int32_t* S, void* stream,
              const mmq_options* opt) {
  int st = check_gemm_shape(M, N, K);
  if (st) return st;
  if ((st = check_options(opt))) return st;
  if (!q8 || !w_rep || !S) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(q8) || !aligned16(w_rep) || !aligned16(S))
    return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  if (!(0 <= i0 && i0 < i1 && i1 <= M && 0 <= j0 && j0 < j1 && j1 <= N))
    return fail(MMQ_E_SHAPE, "window [%lld,%lld) x [%lld,%lld) is empty or outside %lld x %lld",
                (long long)i0, (long long)i1, (long long)j0, (long long)j1, (long long)M,
                (long long)N);
  if (opt && (opt->force_tile == MMQ_TILE_SKINNY || opt->force_tile == MMQ_TILE_GEMV))
    return fail(MMQ_E_ARG, "the skinny and vector-ALU tiles have no block-dot output; force "
                           "large, half, medium or small");
  if (opt && opt->splits > 1)
    return fail(MMQ_E_ARG, "the block dots are written without split-K");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  mmq_kernel_info info;
  st = plan(M, N, K, opt, di->lds_budget, di->compute_units, &info, fmt);
  if (!st && (info.tile == MMQ_TILE_SKINNY || info.tile == MMQ_TILE_GEMV || info.splits > 1)) {
    // the block dots come from the small tile, unsplit
    mmq_options o = opt ? *opt : mmq_options{};
    o.force_tile = MMQ_TILE_SMALL;
    o.workspace_bytes = 0;
    o.splits = 0;
    st = plan(M, N, K, &o, di->lds_budget, di->compute_units, &info, fmt);
  }
  g_last = info;
  if (st) return st;
  const mmq::TileShape ts = tile_shape(info.tile);
  const int64_t tm0 = i0 / ts.block_m();
  const int64_t tm1 = (i1 + ts.block_m() - 1) / ts.block_m();
  const int64_t tn0 = j0 / ts.block_n();
  const int64_t tn1 = (j1 + ts.block_n() - 1) / ts.block_n();
  const int64_t gm = tm1 - tm0, gn = tn1 - tn0;
  g_last.grid = gm * gn;
  g_last.splits = 1;
  g_last.workspace_bytes = 0;
  hipError_t e = mmq::launch_mmq(info.tile, q8, w_rep, S, M, N, K, gm, gn, 1, tm0, tn0, true,
                                 i0, i1, j0, j1, static_cast<hipStream_t>(stream), fmt);
  if (e != hipSuccess) return hip_fail("blockdots launch", e);
  return ok();
}

}  // namespace

namespace mmq {
int api_fail(int status, const char* msg) { return fail(status, "%s", msg); }
int api_check_gemm_call(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                        const float* C, const mmq_options* opt) {
  return check_gemm_call(M, N, K, q8, w_rep, C, opt);
}
int api_current_device() {
  DeviceInfo* di;
  return current_device(&di);
}
}  // namespace mmq

extern "C" {

int mmq_q8_1_bytes(int64_t M, int64_t K, size_t* bytes) {
  if (!bytes) return fail(MMQ_E_ARG, "bytes is NULL");
  if (M <= 0 || K <= 0) return fail(MMQ_E_ARG, "M and K must be positive");
  if (K % MMQ_QK8) return fail(MMQ_E_SHAPE, "K = %lld is not a multiple of 32", (long long)K);
  if (M > kMaxDim || K > kMaxDim || (__int128)M * K > ((__int128)1 << 40))
    return fail(MMQ_E_SHAPE, "activation matrix too large");
  *bytes = (size_t)mmq::q8_total_bytes(M, K);
  return ok();
}

int mmq_q4K_bytes(int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(MMQ_E_ARG, "bytes is NULL");
  if (N <= 0 || K <= 0) return fail(MMQ_E_ARG, "N and K must be positive");
  if (K % MMQ_QK_K) return fail(MMQ_E_SHAPE, "K = %lld is not a multiple of 256", (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(MMQ_E_SHAPE, "weight matrix too large");
  *bytes = (size_t)N * (size_t)(K / MMQ_QK_K) * MMQ_Q4K_BLOCK_BYTES;
  return ok();
}

int mmq_q4K_repacked_bytes(int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(MMQ_E_ARG, "bytes is NULL");
  if (N <= 0 || K <= 0) return fail(MMQ_E_ARG, "N and K must be positive");
  if (K % MMQ_QK_K) return fail(MMQ_E_SHAPE, "K = %lld is not a multiple of 256", (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(MMQ_E_SHAPE, "weight matrix too large");
  static_assert(MMQ_REP_TILE_BYTES == mmq::kRepTileBytes, "repacked record size");
  *bytes = (size_t)((N + 31) / 32) * (size_t)(K / MMQ_QK_K) * MMQ_REP_TILE_BYTES;
  return ok();
}

int quantize_q8_1(const float* x, int64_t M, int64_t K, void* q8, void* stream) {
  size_t nb;
  int st = mmq_q8_1_bytes(M, K, &nb);
  if (st) return st;
  // the prepass indexes the input in 16-byte words with 32-bit offsets
  if ((__int128)M * K >= ((__int128)1 << 34))
    return fail(MMQ_E_SHAPE, "quantize_q8_1 takes M*K below 2^34 (M=%lld, K=%lld)",
                (long long)M, (long long)K);
  if (!x || !q8) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(x) || !aligned16(q8)) return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  hipError_t e = mmq::launch_quantize_q8_1(x, M, K, q8, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("quantize_q8_1 launch", e);
  return ok();
}

int repack_q4_K(const void* w_q4K, int64_t N, int64_t K, void* w_rep, void* stream) {
  size_t nb;
  int st = mmq_q4K_repacked_bytes(N, K, &nb);
  if (st) return st;
  // one workgroup per (32-row tile, super-block), on a 1-D grid
  if ((__int128)((N + 31) / 32) * (K / MMQ_QK_K) >= ((__int128)1 << 31))
    return fail(MMQ_E_SHAPE, "repack_q4_K takes ceil(N/32)*(K/256) below 2^31");
  if (!w_q4K || !w_rep) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(w_q4K) || !aligned16(w_rep)) return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  hipError_t e = mmq::launch_repack_q4_K(w_q4K, N, K, w_rep, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("repack_q4_K launch", e);
  return ok();
}

int mmq_plan(int64_t M, int64_t N, int64_t K, const mmq_options* opt, int64_t lds_budget,
             mmq_kernel_info* out) {
  if (!out) return fail(MMQ_E_ARG, "out is NULL");
  int st = check_gemm_shape(M, N, K);
  if (st) return st;
  if ((st = check_options(opt))) return st;
  if (lds_budget <= 0 && !(opt && opt->lds_budget > 0)) return fail(MMQ_E_ARG, "lds_budget must be positive");
  if ((st = plan(M, N, K, opt, lds_budget, kDefaultComputeUnits, out))) return st;
  return ok();
}

int mmq_q4K_q8_1_ex(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                    float* C, void* stream, const mmq_options* opt) {
  return gemm_ex(mmq::kFmtQ4K, M, N, K, q8, w_rep, C, stream, opt);
}

int mmq_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(MMQ_E_ARG, "bytes is NULL");
  int st = check_gemm_shape(M, N, K);
  if (st) return st;
  mmq_options o = {};
  o.workspace_bytes = INT64_MAX;
  mmq_kernel_info info;
  if ((st = plan(M, N, K, &o, kDefaultLdsBudget, kDefaultComputeUnits, &info))) return st;
  *bytes = (size_t)info.workspace_bytes;
  return ok();
}

int mmq_q4K_q8_1(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep, float* C,
                 void* stream) {
  return mmq_q4K_q8_1_ex(M, N, K, q8, w_rep, C, stream, nullptr);
}

int mmq_q4K_f32(int64_t M, int64_t N, int64_t K, const float* x, const void* w_rep, float* C,
                void* stream) {
  int st = check_gemm_shape(M, N, K);
  if (st) return st;
  if (M > kFusedMaxM)
    return fail(MMQ_E_SHAPE, "mmq_q4K_f32 is for few tokens: M = %lld is above %lld",
                (long long)M, (long long)kFusedMaxM);
  if (!x || !w_rep || !C) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(x) || !aligned16(w_rep) || !aligned16(C))
    return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  // up to kGemvFusedMaxM tokens the vector-ALU kernel, else the skinny one, each quantizing
  // the activations itself
  const bool gemv = M <= mmq::kGemvFusedMaxM;
  mmq_kernel_info info = {};
  info.reason = MMQ_REASON_FUSED;
  info.lds_budget = di->lds_budget;
  if (gemv) {
    info.tile = MMQ_TILE_GEMV;
    info.block_m = (int32_t)mmq::gemv_group(M, 0);
    info.block_n = mmq::kGemvRows;
    info.threads = 64 * mmq::kGemvWaves;
    info.lds_bytes = mmq::gemv_lds_bytes(M, 0, mmq::kGemvRows);
    info.grid = mmq::gemv_grid(M, N, 0, mmq::kGemvRows);
  } else {
    info.tile = MMQ_TILE_SKINNY;
    info.block_m = 32;
    info.block_n = 32;
    info.threads = 64 * mmq::kSkinnyWaves;
    info.lds_bytes = mmq::fused_lds_bytes();
    info.grid = ((M + 31) / 32) * ((N + 31) / 32);
  }
  if (info.lds_bytes > di->lds_budget) {
    info.tile = MMQ_TILE_AUTO;
    info.reason = MMQ_REASON_NO_FIT;
    g_last = info;
    return fail(MMQ_E_LDS, "mmq_q4K_f32 needs %lld bytes of LDS, the device allows %lld",
                (long long)info.lds_bytes, (long long)di->lds_budget);
  }
  g_last = info;
  hipError_t e = gemv ? mmq::launch_mmq_gemv_fused(x, w_rep, C, M, N, K,
                                                   static_cast<hipStream_t>(stream))
                      : mmq::launch_mmq_fused(x, w_rep, C, M, N, K, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("mmq_q4K_f32 launch", e);
  return ok();
}

int mmq_q4K_q8_1_blockdots(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                           int64_t i0, int64_t i1, int64_t j0, int64_t j1, int32_t* S,
                           void* stream, const mmq_options* opt) {
  return blockdots(mmq::kFmtQ4K, M, N, K, q8, w_rep, i0, i1, j0, j1, S, stream, opt);
}

// ---------------------------------------------------------------- q6_K

int mmq_q6K_bytes(int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(MMQ_E_ARG, "bytes is NULL");
  if (N <= 0 || K <= 0) return fail(MMQ_E_ARG, "N and K must be positive");
  if (K % MMQ_QK_K) return fail(MMQ_E_SHAPE, "K = %lld is not a multiple of 256", (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(MMQ_E_SHAPE, "weight matrix too large");
  *bytes = (size_t)N * (size_t)(K / MMQ_QK_K) * MMQ_Q6K_BLOCK_BYTES;
  return ok();
}

int mmq_q6K_repacked_bytes(int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(MMQ_E_ARG, "bytes is NULL");
  if (N <= 0 || K <= 0) return fail(MMQ_E_ARG, "N and K must be positive");
  if (K % MMQ_QK_K) return fail(MMQ_E_SHAPE, "K = %lld is not a multiple of 256", (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(MMQ_E_SHAPE, "weight matrix too large");
  static_assert(MMQ_REP6_TILE_BYTES == mmq::kRep6TileBytes, "repacked q6_K record size");
  static_assert(MMQ_Q6K_BLOCK_BYTES == mmq::kQ6KBlockBytes, "q6_K block size");
  *bytes = (size_t)((N + 31) / 32) * (size_t)(K / MMQ_QK_K) * MMQ_REP6_TILE_BYTES;
  return ok();
}

int repack_q6_K(const void* w_q6K, int64_t N, int64_t K, void* w_rep, void* stream) {
  size_t nb;
  int st = mmq_q6K_repacked_bytes(N, K, &nb);
  if (st) return st;
  if ((__int128)((N + 31) / 32) * (K / MMQ_QK_K) >= ((__int128)1 << 31))
    return fail(MMQ_E_SHAPE, "repack_q6_K takes ceil(N/32)*(K/256) below 2^31");
  if (!w_q6K || !w_rep) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(w_rep)) return fail(MMQ_E_ARG, "w_rep must be 16-byte aligned");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  hipError_t e = mmq::launch_repack_q6_K(w_q6K, N, K, w_rep, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("repack_q6_K launch", e);
  return ok();
}

int mmq_q6K_q8_1_ex(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                    float* C, void* stream, const mmq_options* opt) {
  return gemm_ex(mmq::kFmtQ6K, M, N, K, q8, w_rep, C, stream, opt);
}

int mmq_q6K_q8_1(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep, float* C,
                 void* stream) {
  return mmq_q6K_q8_1_ex(M, N, K, q8, w_rep, C, stream, nullptr);
}

int mmq_q6K_q8_1_blockdots(int64_t M, int64_t N, int64_t K, const void* q8, const void* w_rep,
                           int64_t i0, int64_t i1, int64_t j0, int64_t j1, int32_t* S,
                           void* stream, const mmq_options* opt) {
  return blockdots(mmq::kFmtQ6K, M, N, K, q8, w_rep, i0, i1, j0, j1, S, stream, opt);
}

// ---------------------------------------------------------------- f16 comparator path

int mmq_f16_bytes(int64_t rows, int64_t K, size_t* bytes) {
  if (!bytes) return fail(MMQ_E_ARG, "bytes is NULL");
  if (rows <= 0 || K <= 0) return fail(MMQ_E_ARG, "rows and K must be positive");
  if (rows > kMaxDim || K > kMaxDim || (__int128)rows * K > ((__int128)1 << 40))
    return fail(MMQ_E_SHAPE, "f16 matrix too large");
  *bytes = (size_t)rows * (size_t)K * 2;
  return ok();
}

int convert_f32_f16(const float* x, int64_t M, int64_t K, void* x_f16, void* stream) {
  size_t nb;
  int st = mmq_f16_bytes(M, K, &nb);
  if (st) return st;
  if (!x || !x_f16) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(x) || !aligned16(x_f16))
    return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  hipError_t e = mmq::launch_convert_f32_f16(x, M * K, x_f16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("convert_f32_f16 launch", e);
  return ok();
}

int dequantize_q4_K_f16(const void* w_q4K, int64_t N, int64_t K, void* w_f16, void* stream) {
  size_t nb;
  int st = mmq_q4K_bytes(N, K, &nb);
  if (st) return st;
  if ((st = mmq_f16_bytes(N, K, &nb))) return st;
  if (!w_q4K || !w_f16) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(w_q4K) || !aligned16(w_f16))
    return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  DeviceInfo* di;
  if ((st = current_device(&di))) return st;
  hipError_t e =
      mmq::launch_dequantize_q4_K_f16(w_q4K, N, K, w_f16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("dequantize_q4_K_f16 launch", e);
  return ok();
}

int gemm_f16(int64_t M, int64_t N, int64_t K, const void* x_f16, const void* w_f16, float* C,
             void* stream) {
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(MMQ_E_ARG, "M, N, K must be positive (%lld, %lld, %lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 8) return fail(MMQ_E_SHAPE, "K = %lld is not a multiple of 8", (long long)K);
  // the kernel addresses each operand with 32-bit byte offsets below 2^31
  if (M > kMaxDim || N > kMaxDim || (__int128)M * K >= ((__int128)1 << 30) ||
      (__int128)N * K >= ((__int128)1 << 30))
    return fail(MMQ_E_SHAPE, "an f16 operand of 2^30 or more elements");
  if (!x_f16 || !w_f16 || !C) return fail(MMQ_E_ARG, "null device pointer");
  if (!aligned16(x_f16) || !aligned16(w_f16) || !aligned16(C))
    return fail(MMQ_E_ARG, "device pointers must be 16-byte aligned");
  DeviceInfo* di;
  int st;
  if ((st = current_device(&di))) return st;
  if (mmq::gemm_f16_lds_bytes() > di->lds_budget)
    return fail(MMQ_E_LDS, "the f16 GEMM needs %lld bytes of LDS, the device allows %lld",
                (long long)mmq::gemm_f16_lds_bytes(), (long long)di->lds_budget);
  hipError_t e = mmq::launch_gemm_f16(x_f16, w_f16, C, M, N, K, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gemm_f16 launch", e);
  return ok();
}

int mmq_last_kernel(mmq_kernel_info* out) {
  if (!out) return fail(MMQ_E_ARG, "out is NULL");
  *out = g_last;
  return MMQ_OK;
}

const char* mmq_status_str(int status) {
  switch (status) {
    case MMQ_OK: return "MMQ_OK";
    case MMQ_E_ARG: return "MMQ_E_ARG: invalid argument";
    case MMQ_E_SHAPE: return "MMQ_E_SHAPE: unsupported shape";
    case MMQ_E_LDS: return "MMQ_E_LDS: no tile fits the LDS budget";
    case MMQ_E_DEVICE: return "MMQ_E_DEVICE: no gfx950 device";
    case MMQ_E_HIP: return "MMQ_E_HIP: HIP runtime error";
    default: return "unknown mmq status";
  }
}

const char* mmq_last_error(void) { return g_err; }

}  // extern "C"

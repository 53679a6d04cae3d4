// mmq_q4K_q8_1_static: the GEMM entry point for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It is
// mmq_q4K_q8_1_ex with the split-K workspace in a file-scope device array instead of the
// caller's buffer, so such callers get the split-K path too. The array is part of the code
// object: every GPU the library runs on holds one copy of it until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mmq.h"
#include "mmq_internal.h"

namespace {

constexpr int64_t kScratchBytes = (int64_t)32 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchAddress {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddress g_scratch[kMaxDevices];

}  // namespace

extern "C" int mmq_q4K_q8_1_static(int64_t M, int64_t N, int64_t K, const void* q8,
                                   const void* w_rep, float* C, void* stream,
                                   const mmq_options* opt) {
  int st = mmq::api_check_gemm_call(M, N, K, q8, w_rep, C, opt);
  if (st) return st;
  if (opt && (opt->workspace || opt->workspace_bytes))
    return mmq::api_fail(MMQ_E_ARG, "mmq_q4K_q8_1_static uses its own scratch: pass no workspace");
  if (opt && opt->splits > K / 256)
    return mmq::api_fail(MMQ_E_ARG, "splits is more than the super-blocks of K");
  // at most K/256 <= 2^16 splits of an output below 2^40 elements: the product fits 64 bits
  if (opt && opt->splits > 1 && opt->splits * M * N * 4 > kScratchBytes)
    return mmq::api_fail(MMQ_E_ARG, "the forced splits' partial planes exceed the 32 MiB scratch "
                                    "of mmq_q4K_q8_1_static");
  if ((st = mmq::api_current_device())) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return mmq::api_fail(MMQ_E_DEVICE, "no usable current device");
  // The array's name is a host-side stand-in: its device address, which differs per device,
  // is looked up once per device, with that device current, and used everywhere after.
  ScratchAddress& sa = g_scratch[dev];
  std::call_once(sa.once, [&sa]() {
    sa.err = hipGetSymbolAddress(&sa.ptr, HIP_SYMBOL(scratch));
  });
  if (sa.err != hipSuccess || !sa.ptr)
    return mmq::api_fail(MMQ_E_HIP, "hipGetSymbolAddress of the scratch array failed");
  mmq_options o = opt ? *opt : mmq_options{};
  o.workspace = sa.ptr;
  o.workspace_bytes = kScratchBytes;
  return mmq_q4K_q8_1_ex(M, N, K, q8, w_rep, C, stream, &o);
}

// bsp_plan into the library's own device scratch, for callers that cannot
// allocate device memory (code under graph capture, serving loops, harnesses
// that forbid allocation). The scratch is a file-scope device array; its
// address is looked up once per device, with that device current, on the
// first call there, and only that address is ever handed to the runtime or a
// kernel. Every plan planned this way on one device shares that device's
// array: calls (and the steps that read the plan) that overlap on one device
// race, and each call rewrites everything a step reads, including the error
// word and the split counters, so nothing is inherited from an earlier call.
#include <mutex>

#include "bsp_internal.h"

namespace {

constexpr size_t kScratchBytes = bsp::kStaticWorkspaceBytes;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

extern "C" bsp_status_t bsp_plan_static(bsp_plan_t plan, int32_t B, int32_t W, int32_t q_len,
                                        const int32_t* prefix_len_h, const int32_t* seq_len_h,
                                        const int32_t* block_tables_h, hipStream_t stream) {
  if (plan == nullptr) return bsp::set_error(BSP_ERR_ARG, "null plan");
  const size_t need = bsp_plan_workspace_bytes(plan);
  if (need > kScratchBytes)
    return bsp::set_error(BSP_ERR_WORKSPACE,
                          "plan needs a workspace of %zu bytes; the library's static scratch "
                          "holds %zu bytes (use bsp_plan with a caller workspace)",
                          need, kScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return bsp::set_error(BSP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return bsp::set_error(BSP_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                          kMaxDevices);
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
      e = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch[dev] = nullptr;
        return bsp::set_error(BSP_ERR_HIP, "hipGetSymbolAddress (static scratch): %s",
                              hipGetErrorString(e));
      }
    }
    ptr = g_scratch[dev];
  }
  // the array keeps the last call's contents: copy the whole header again
  bsp::forget_workspace(plan);
  return bsp_plan(plan, B, W, q_len, prefix_len_h, seq_len_h, block_tables_h, ptr, kScratchBytes,
                  stream);
}

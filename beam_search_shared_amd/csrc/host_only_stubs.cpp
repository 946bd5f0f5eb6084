// Kernel launchers for the host-only build of the planner (bsp_host.cpp built
// with a plain C++ compiler and the address and undefined-behaviour
// sanitizers). That build serves the CPU tests of the host logic only: every
// launcher here reports that no GPU code is linked, and plans created with
// BSP_PLAN_HOST_ONLY never reach them.
#include "bsp_internal.h"
#include "merge_row.h"

namespace bsp {

hipError_t launch_write_kv(const WriteKvParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefix(const PrefixParams&, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_cached_decode(const PrefixParams&, const FusedParams&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
bool cached_decode_supported(int, int) { return false; }
bool decode_uses_slot_table(int, int, int, int, int) { return false; }
hipError_t launch_prefix_two(const PrefixParams&, const PrefixParams&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode_step(const PrefixParams&, const FusedParams&, int, int, int, int, int,
                              hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_prefill(const PrefixParams&, const FusedParams&, int, int, int, int,
                          hipStream_t) {
  return hipErrorNotSupported;
}
bool mixed_step_supported(const PrefixParams&, const FusedParams&, int, int, int, int, int) {
  return false;
}
hipError_t launch_mixed_step(const PrefixParams&, const FusedParams&, const PrefixParams&,
                             const FusedParams&, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_tail(const TailParams&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_tail_slots(const TailParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_merge(const MergeParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_merge_row(const MergeRowParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_naive(const TailParams&, void*, float*, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace bsp

// The static scratch is GPU code: the host-only build has none.
extern "C" bsp_status_t bsp_plan_static(bsp_plan_t, int32_t, int32_t, int32_t, const int32_t*,
                                        const int32_t*, const int32_t*, hipStream_t) {
  return bsp::set_error(BSP_ERR_UNSUPPORTED, "host-only build: no static scratch");
}

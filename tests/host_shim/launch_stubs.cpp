// Host-only stand-ins for the kernel launchers of the retention library.
//
// Linked with the library's validation and planning sources (api.cpp,
// plan.cpp) into a shared object built with a host compiler and the address
// and undefined-behaviour sanitizers, so the C ABI's argument checks and
// planning arithmetic run under the sanitizers on a machine without a GPU.
// Every launcher records the call and returns success without touching any
// pointer; retention_shim_launches() reports how many were made.
#include <atomic>

#include "kernels.h"

namespace {
std::atomic<int> g_launches{0};
hipError_t record() {
  g_launches.fetch_add(1, std::memory_order_relaxed);
  return hipSuccess;
}
}  // namespace

extern "C" int retention_shim_launches(void) { return g_launches.load(std::memory_order_relaxed); }

namespace ret {

hipError_t launch_decode_step(int, const void*, const void*, const void*, float*, void*, int, int, int, int,
                              const HeadDecay&, const GnArgs&, hipStream_t) {
  return record();
}
hipError_t launch_generic_state_walk(int, const void*, const void*, const float*, float*, float*, const Dims&, int,
                                     const HeadDecay&, hipStream_t) {
  return record();
}
hipError_t launch_generic_chunk_out(int, const void*, const void*, const void*, const float*, bool, void*,
                                    const Dims&, int, const HeadDecay&, const GnArgs&, bool, hipStream_t) {
  return record();
}
hipError_t launch_mfma_state_walk(const uint16_t*, const uint16_t*, const float*, float*, uint16_t*, float*, int,
                                  const Dims&, int, const HeadDecay&, hipStream_t) {
  return record();
}
hipError_t launch_mfma_chunk_out(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, bool, uint16_t*,
                                 const Dims&, int, const HeadDecay&, const GnArgs&, bool, hipStream_t) {
  return record();
}
hipError_t launch_split_rows(int, const void*, const SplitTarget*, int, const Dims&, int, hipStream_t) {
  return record();
}
hipError_t launch_sum_parts(int, const void*, void*, const Dims&, int, int, int64_t, bool, hipStream_t) {
  return record();
}
hipError_t launch_state_prep(const float*, float*, int, int, int, int, bool, int, int64_t, const float*,
                             hipStream_t) {
  return record();
}

hipError_t launch_fused_chunkwise(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, const float*, float*,
                                  void*, const Dims&, int, const HeadDecay&, const GnArgs&, bool, hipStream_t, int,
                                  const float*, const FusedLayout*) {
  return record();
}
hipError_t copy_device(void*, const void*, size_t, hipStream_t) { return record(); }
hipError_t launch_segment_ends(const uint16_t*, const uint16_t*, const float*, float*, int, const Dims&, int,
                               const HeadDecay&, hipStream_t) {
  return record();
}

hipError_t launch_xpos_rotate(int, const void*, const void*, void*, void*, const float*, int, int, int, int64_t,
                              hipStream_t) {
  return record();
}

// The scratch lookup hands out a fake address (never dereferenced: the
// launchers above touch nothing).
hipError_t scratch_pointer(void** out) {
  *out = reinterpret_cast<void*>(uintptr_t{1} << 40);
  return hipSuccess;
}

}  // namespace ret

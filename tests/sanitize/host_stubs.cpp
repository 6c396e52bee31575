// Host-only build of libpagedattn for the sanitizer run of the CPU tests:
// the kernel launchers, which live in the HIP sources, are replaced by stubs
// that refuse every launch.  The CPU tests reach the C ABI's argument checks,
// host validators and block manager, never a launch.
#include <hip/hip_runtime.h>

#include "launch.h"
#include "pagedattn.h"

namespace pa {

hipError_t launch_reshape_and_cache(const void*, const void*, void*, void*, const int64_t*, int,
                                    int, int, int, int, int64_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_copy_blocks(void*, void*, const int32_t*, int, int64_t, int64_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_swap_blocks(const void*, void*, const int64_t*, int, int64_t, int64_t, int64_t,
                              hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_decode_valu(const DecodeArgs&, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_decode_mfma(const DecodeArgs&, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
bool decode_mfma_streams(const DecodeArgs&) { return false; }
hipError_t launch_prefix(const DecodeArgs&, const PrefixOut&, const KvWrite&, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_multi_query(const MultiQueryArgs&, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_reduce(const ReduceArgs&, int, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace pa

extern "C" int pa_reshape_and_decode_static(void*, const void*, const void*, const void*, void*,
                                            void*, const int64_t*, const int32_t*,
                                            const int32_t*, int32_t, int32_t, int32_t, int32_t,
                                            int32_t, int32_t, int64_t, float, int32_t, int32_t,
                                            int32_t, void*) {
  return PA_ERR_LAUNCH;
}

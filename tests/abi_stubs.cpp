// Stand-ins for the library's kernel launchers, so that the host-side C-ABI
// layer (ra_abi.cpp) can be built for the CPU alone, with AddressSanitizer,
// and driven by the ABI tests: each launcher counts its calls and launches
// nothing. Test infrastructure only; never part of libra.so.

#include "ra_bwd.h"
#include "ra_launch.h"
#include "ra_stream_launch.h"

static int g_launches = 0;

extern "C" int ra_test_launch_count(void) { return g_launches; }

namespace ra {

static hipError_t counted() {
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_step_bf16(const StepArgs&, hipStream_t) { return counted(); }
hipError_t launch_step_last_bf16(const StepArgs&, void*, float*, hipStream_t) { return counted(); }
hipError_t launch_step_f32(const StepArgs&, hipStream_t) { return counted(); }
hipError_t launch_attend_bf16(const void*, const void*, const void*, int32_t, int32_t, int32_t, float, void*,
                              float*, hipStream_t) {
  return counted();
}
hipError_t launch_finalize(const float*, const float*, const float*, int64_t, int32_t, void*, bool, float*,
                           hipStream_t) {
  return counted();
}
hipError_t launch_merge(const void*, const float*, const void*, const float*, bool, int64_t, int32_t, void*,
                        float*, hipStream_t) {
  return counted();
}
hipError_t launch_temporal_bf16(const void*, const void*, const void*, int32_t, int32_t, int32_t, int32_t, float,
                                void*, float*, hipStream_t) {
  return counted();
}
hipError_t launch_temporal_long_bf16(const void*, const void*, const void*, int32_t, int32_t, int32_t, int32_t,
                                     float, void*, float*, hipStream_t) {
  return counted();
}
hipError_t launch_add_rows(const float*, int64_t, int64_t, float*, int64_t, int64_t, int64_t, int64_t, int32_t,
                           hipStream_t) {
  return counted();
}
hipError_t launch_kv_pass(const void*, void*, const void*, void*, int64_t, hipStream_t) { return counted(); }
hipError_t launch_step_bwd_bf16(const BwdArgs&, hipStream_t) { return counted(); }
hipError_t launch_bwd_prep_bf16(const void*, const void*, int64_t, int32_t, float*, hipStream_t) {
  return counted();
}

}  // namespace ra

// Host-side launchers of the gfx950 kernels. Arguments are validated by the
// C-ABI layer (ra_abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

struct HostSegs {
  int32_t start0, start1, len0, len;
};

// One problem of the step kernels: `nb` independent (batch*head) query slices,
// each with Lq query rows, against nb / group K/V slices of Lk key rows:
// query slice p reads K/V slice p / group.
struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  int32_t nb, Lq, Lk, d;
  int32_t group;  // query heads per K/V head (1: one K/V head per query head)
  HostSegs qs, ks;
  bool causal;
  bool init;
  float scale;
  float* o_acc;
  float* m;
  float* l;
};

hipError_t launch_step_bf16(const StepArgs& a, hipStream_t s);
// The last ring step with the finalize folded in: out [nb, Lq, d] bf16 and
// lse (may be null) from the state (read unless a.init) and the block; the
// state is not written.
hipError_t launch_step_last_bf16(const StepArgs& a, void* out, float* lse, hipStream_t s);
hipError_t launch_step_f32(const StepArgs& a, hipStream_t s);

// Fused single-block attention (init + finalize): batched, unmasked, Lq = Lk.
hipError_t launch_attend_bf16(const void* q, const void* k, const void* v, int32_t nb,
                              int32_t L, int32_t d, float scale, void* out, float* lse,
                              hipStream_t s);

hipError_t launch_finalize(const float* o_acc, const float* m, const float* l, int64_t rows,
                           int32_t d, void* out, bool out_bf16, float* lse, hipStream_t s);

hipError_t launch_merge(const void* oa, const float* la, const void* ob, const float* lb,
                        bool bf16, int64_t rows, int32_t d, void* oo, float* lo, hipStream_t s);

hipError_t launch_temporal_bf16(const void* q, const void* k, const void* v, int32_t nb,
                                int32_t T, int32_t S_sp, int32_t d, float scale, void* out,
                                float* lse, hipStream_t s);

}  // namespace ra

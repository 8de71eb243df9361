// Host-side launchers of the backward ring-step kernels. Arguments are
// validated by the C-ABI layer (ra_abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_launch.h"

namespace ra {

// One backward step: `nb` (batch*head) query slices of Lq local rows against
// nb / group K/V slices of an Lk-row block (query slice p reads K/V slice
// p / group), with the final forward lse and delta = <dO, O> per query row.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* delta;
  int32_t nb, Lq, Lk, d;
  int32_t group;  // query heads per K/V head
  HostSegs qs, ks;
  bool causal;
  bool init_dq;   // dq starts at zero (not read)
  bool init_dkv;  // dk, dv start at zero (not read)
  bool run_dq;    // launch the dQ kernel
  bool run_dkv;   // launch the dK/dV kernel
  float scale;
  float* dq;
  float* dk;
  float* dv;
};

hipError_t launch_step_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_prep_bf16(const void* out, const void* dout, int64_t rows, int32_t d,
                                float* delta, hipStream_t s);

}  // namespace ra

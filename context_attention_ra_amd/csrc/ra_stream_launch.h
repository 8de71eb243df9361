// Host-side launchers of the HBM-stream kernels added beside the ring step:
// factored temporal attention of clips longer than 16 frames, the row
// accumulate of the reduce-scatter, and the ring's block pass. Arguments are
// validated by the C-ABI layer (ra_abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// factored temporal attention for 16 < T <= 128 frames (bf16 in and out)
hipError_t launch_temporal_long_bf16(const void* q, const void* k, const void* v, int32_t nb,
                                     int32_t T, int32_t S_sp, int32_t d, float scale, void* out,
                                     float* lse, hipStream_t s);

// dst rows [dst_row0, +nrows) += src rows [src_row0, +nrows) of each of
// nslices fp32 slices of d values per row
hipError_t launch_add_rows(const float* src, int64_t src_slice_rows, int64_t src_row0, float* dst,
                           int64_t dst_slice_rows, int64_t dst_row0, int64_t nslices, int64_t nrows,
                           int32_t d, hipStream_t s);

// the ring's block pass: a and c (n16 16-byte pieces each, 16-byte aligned)
// copied to b and d by a kernel small enough to run beside a ring step;
// n16 <= 2^30
hipError_t launch_kv_pass(const void* a, void* b, const void* c, void* d, int64_t n16, hipStream_t s);

}  // namespace ra

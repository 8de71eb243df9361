// Row-wise accumulate for the reduce-scatter that returns the gathered K/V's
// gradients to the ranks that own them (Ultralytics glossary, "How Context
// Parallelism Works": reduce-scatter next to all-gather): dst rows += src
// rows, over nslices slices. One thread per 16 bytes; rows of a slice are
// contiguous, so each wave streams whole rows (an HBM stream: 12 bytes moved
// per fp32 value added).

#include "ra_device.h"
#include "ra_stream_launch.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void add_rows_kernel(
    const float* __restrict__ src, int64_t src_slice_rows, int64_t src_row0, float* __restrict__ dst,
    int64_t dst_slice_rows, int64_t dst_row0, int64_t nrows, int32_t c4_per_row, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const int64_t per_slice = nrows * c4_per_row;
  const int64_t sl = idx / per_slice;
  const int64_t rem = idx - sl * per_slice;
  const int64_t row = rem / c4_per_row;
  const int64_t c = rem - row * c4_per_row;
  const f32x4 a = *(const f32x4*)(src + ((sl * src_slice_rows + src_row0 + row) * c4_per_row + c) * 4);
  f32x4* dp = (f32x4*)(dst + ((sl * dst_slice_rows + dst_row0 + row) * c4_per_row + c) * 4);
  const f32x4 b = *dp;
  *dp = f32x4{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
}

}  // namespace

hipError_t launch_add_rows(const float* src, int64_t src_slice_rows, int64_t src_row0, float* dst,
                           int64_t dst_slice_rows, int64_t dst_row0, int64_t nslices, int64_t nrows,
                           int32_t d, hipStream_t st) {
  const int32_t c4 = d / 4;
  const int64_t total = nslices * nrows * c4;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(add_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, src,
                     src_slice_rows, src_row0, dst, dst_slice_rows, dst_row0, nrows, c4, total);
  return hipGetLastError();
}

}  // namespace ra

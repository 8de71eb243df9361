// Row-wise accumulate for the reduce-scatter that returns the gathered K/V's
// gradients to the ranks that own them (Ultralytics glossary, "How Context
// Parallelism Works": reduce-scatter next to all-gather): dst rows += src
// rows, over nslices slices. One thread per 16 bytes; rows of a slice are
// contiguous, so each wave streams whole rows (an HBM stream: 12 bytes moved
// per fp32 value added).
//
// The ring's block pass (Day 83 post, "The communication pattern"; k8ai ring
// figure: the next block moves while the current one is computed on): K and V
// of the source copied into the receive buffers. A device-to-device copy runs
// on the compute units, and a ring step fills every SIMD's registers but for
// 16 per lane (two waves of 248), so the copy is written to fit there: one
// wave per workgroup, at most 16 VGPRs (two 16-byte pieces in flight per
// lane), 1024 workgroups: one per SIMD, which the step kernel's workgroups
// still fit beside (with more, a CU whose SIMDs hold two copy waves has no
// room for a step workgroup until they finish). Alone it moves about 3 TB/s
// of copy traffic, half the runtime's blit; beside a step it is hidden.

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

constexpr int kPassWaves = 1024;

__global__ __launch_bounds__(64) void kv_pass_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b,
                                                     const u32x4* __restrict__ c, u32x4* __restrict__ d,
                                                     int32_t n16, int32_t per_wave) {
  // this wave's pieces [lo, hi); per_wave is a multiple of 128
  const int32_t lo = (int32_t)blockIdx.x * per_wave;
  const int32_t hi = min(lo + per_wave, n16);
  for (int32_t i = lo + (int32_t)threadIdx.x; i < hi; i += 128) {
    const u32x4 x0 = __builtin_nontemporal_load(a + i);
    const u32x4 x1 = __builtin_nontemporal_load(a + min(i + 64, hi - 1));
    __builtin_nontemporal_store(x0, b + i);
    if (i + 64 < hi) __builtin_nontemporal_store(x1, b + i + 64);
  }
  for (int32_t i = lo + (int32_t)threadIdx.x; i < hi; i += 128) {
    const u32x4 x0 = __builtin_nontemporal_load(c + i);
    const u32x4 x1 = __builtin_nontemporal_load(c + min(i + 64, hi - 1));
    __builtin_nontemporal_store(x0, d + i);
    if (i + 64 < hi) __builtin_nontemporal_store(x1, d + i + 64);
  }
}

}  // namespace

hipError_t launch_kv_pass(const void* a, void* b, const void* c, void* d, int64_t n16, hipStream_t st) {
  const int64_t per = ((n16 + kPassWaves - 1) / kPassWaves + 127) / 128 * 128;
  hipLaunchKernelGGL(kv_pass_kernel, dim3(kPassWaves), dim3(64), 0, st, (const u32x4*)a, (u32x4*)b,
                     (const u32x4*)c, (u32x4*)d, (int32_t)n16, (int32_t)per);
  return hipGetLastError();
}

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

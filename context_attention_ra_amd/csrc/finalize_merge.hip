// Finalize and log-sum-exp merge: the two HBM-streaming epilogues of the ring.
//
// Finalize turns the running state into the output once every block has been
// folded in (Day 83 post on skandtandon.pages.dev, "Context parallelism:
// splitting the sequence": after P steps the device holds the correct output
// for its queries): out = O_acc / l, lse = m + ln l.
// Merge combines two normalised partial outputs over disjoint key sets with
// softmax weights e^{lse_x - lse}, lse = ln(e^{lse_a} + e^{lse_b}) — the
// "accumulate partial attention outputs" rule of the same section in its
// normalised form.
// Both kernels are pure streams: each thread moves 16-32 contiguous bytes per
// tensor and a row's per-row scalars are read by the threads of that row,
// which always sit in one wave (the row's thread count divides 64).

#include "ra_device.h"
#include "ra_launch.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void finalize_kernel(
    const float* __restrict__ O, const float* __restrict__ M, const float* __restrict__ L,
    int64_t rows, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int TPR = D / 8;  // threads per row, 8 values each
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = idx / TPR;
  if (row >= rows) return;
  const int c = (int)(idx % TPR);
  const float l = L[row];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const f32x4 a = *(const f32x4*)(O + row * D + 8 * c);
  const f32x4 b = *(const f32x4*)(O + row * D + 8 * c + 4);
  if (OUT_BF16) {
    bf16x8 y = {to_bf16(a[0] * inv), to_bf16(a[1] * inv), to_bf16(a[2] * inv), to_bf16(a[3] * inv),
                to_bf16(b[0] * inv), to_bf16(b[1] * inv), to_bf16(b[2] * inv), to_bf16(b[3] * inv)};
    *(bf16x8*)((bf16*)out + row * D + 8 * c) = y;
  } else {
    float* op = (float*)out + row * D + 8 * c;
    *(f32x4*)op = f32x4{a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv};
    *(f32x4*)(op + 4) = f32x4{b[0] * inv, b[1] * inv, b[2] * inv, b[3] * inv};
  }
  if (lse && c == 0) lse[row] = l > 0.f ? M[row] + fast_log2(l) * kLn2 : kNegInf;
}

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void merge_kernel(
    const void* oa, const float* la, const void* ob, const float* lb, int64_t rows, void* oo,
    float* lo) {
  constexpr int TPR = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = idx / TPR;
  if (row >= rows) return;
  const int c = (int)(idx % TPR);
  const float xa = la[row], xb = lb[row];
  const float hi = fmaxf(xa, xb);
  const bool empty = hi == kNegInf;
  const float ref = empty ? 0.f : hi;
  const float ea = fast_exp2((xa - ref) * kLog2e);
  const float eb = fast_exp2((xb - ref) * kLog2e);
  const float tot = ea + eb;
  const float inv = empty ? 0.f : 1.f / tot;
  const float wa = ea * inv, wb = eb * inv;
  const int64_t off = row * D + 8 * c;
  if (BF16) {
    const bf16x8 a = *(const bf16x8*)((const bf16*)oa + off);
    const bf16x8 b = *(const bf16x8*)((const bf16*)ob + off);
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      y[e] = to_bf16(__builtin_fmaf(wa, from_bf16(a[e]), wb * from_bf16(b[e])));
    *(bf16x8*)((bf16*)oo + off) = y;
  } else {
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      const f32x4 a = *(const f32x4*)((const float*)oa + off + 4 * hlf);
      const f32x4 b = *(const f32x4*)((const float*)ob + off + 4 * hlf);
      f32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(wa, a[e], wb * b[e]);
      *(f32x4*)((float*)oo + off + 4 * hlf) = y;
    }
  }
  if (c == 0) lo[row] = empty ? kNegInf : ref + fast_log2(tot) * kLn2;
}

}  // namespace

hipError_t launch_finalize(const float* o, const float* m, const float* l, int64_t rows, int32_t d,
                           void* out, bool out_bf16, float* lse, hipStream_t st) {
  const int64_t threads = rows * (d / 8);
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
  if (d == 128) {
    if (out_bf16) hipLaunchKernelGGL((finalize_kernel<128, true>), grid, dim3(kThreads), 0, st, o, m, l, rows, out, lse);
    else hipLaunchKernelGGL((finalize_kernel<128, false>), grid, dim3(kThreads), 0, st, o, m, l, rows, out, lse);
  } else {
    if (out_bf16) hipLaunchKernelGGL((finalize_kernel<64, true>), grid, dim3(kThreads), 0, st, o, m, l, rows, out, lse);
    else hipLaunchKernelGGL((finalize_kernel<64, false>), grid, dim3(kThreads), 0, st, o, m, l, rows, out, lse);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const void* oa, const float* la, const void* ob, const float* lb, bool bf16,
                        int64_t rows, int32_t d, void* oo, float* lo, hipStream_t st) {
  const int64_t threads = rows * (d / 8);
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
  if (d == 128) {
    if (bf16) hipLaunchKernelGGL((merge_kernel<128, true>), grid, dim3(kThreads), 0, st, oa, la, ob, lb, rows, oo, lo);
    else hipLaunchKernelGGL((merge_kernel<128, false>), grid, dim3(kThreads), 0, st, oa, la, ob, lb, rows, oo, lo);
  } else {
    if (bf16) hipLaunchKernelGGL((merge_kernel<64, true>), grid, dim3(kThreads), 0, st, oa, la, ob, lb, rows, oo, lo);
    else hipLaunchKernelGGL((merge_kernel<64, false>), grid, dim3(kThreads), 0, st, oa, la, ob, lb, rows, oo, lo);
  }
  return hipGetLastError();
}

}  // namespace ra

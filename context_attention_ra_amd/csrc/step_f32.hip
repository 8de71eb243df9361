// Ring-step attention in fp32 on the vector ALUs (the fp32 dtype path).
//
// Same operation as the bf16 matrix-core step (Day 83 post on
// skandtandon.pages.dev, "Context parallelism: splitting the sequence": fold
// one K/V block into the running online-softmax state), kept in fp32
// end to end. D/32 lanes share one query row, each holding 32 of its
// dimensions; dot products are finished with lane shuffles. Keys stream
// through LDS in tiles of 32 rows. The running maximum is exact here.

#include "ra_device.h"
#include "ra_launch.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void step_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    int32_t Lq, int32_t Lk, DevSegs qs, DevSegs ks, float c_log2, int32_t init,
    float* __restrict__ Oacc, float* __restrict__ Mst, float* __restrict__ Lst, int32_t nqt,
    int32_t group) {
  constexpr int TPR = D / 32;                 // lanes per query row
  constexpr int RPB = kThreads / TPR;         // query rows per workgroup
  __shared__ f32x4 kt[kBK * D / 4];
  __shared__ f32x4 vt[kBK * D / 4];

  const int32_t prob = blockIdx.x / nqt;
  const int32_t qt = blockIdx.x - prob * nqt;
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int32_t qrow = qt * RPB + tid / TPR;
  const bool qvalid = qrow < Lq;
  const int32_t qrow_c = qvalid ? qrow : Lq - 1;
  const int32_t qpos = seg_pos(qs, qrow_c);
  const size_t qoff = ((size_t)prob * Lq + qrow_c) * D + 32 * part;
  // query heads h*group .. h*group+group-1 share K/V head h (batch-major slices)
  const size_t kbase = (size_t)(prob / group) * Lk * D;

  float q[32], o[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 x = *(const f32x4*)(Q + qoff + 4 * i);
    q[4 * i] = x[0]; q[4 * i + 1] = x[1]; q[4 * i + 2] = x[2]; q[4 * i + 3] = x[3];
  }
  float mu = kNegInf, lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = 0.f;
  if (!init && qvalid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 x = *(const f32x4*)(Oacc + qoff + 4 * i);
      o[4 * i] = x[0]; o[4 * i + 1] = x[1]; o[4 * i + 2] = x[2]; o[4 * i + 3] = x[3];
    }
    mu = Mst[(size_t)prob * Lq + qrow] * kLog2e;
    lsum = Lst[(size_t)prob * Lq + qrow];
  }

  int32_t wg_lo, wg_hi;
  seg_range(qs, qt * RPB, min(qt * RPB + RPB, Lq), wg_lo, wg_hi);

  for (int32_t kt0 = 0; kt0 < Lk; kt0 += kBK) {
    const int32_t kend = min(kt0 + kBK, Lk);
    if (CAUSAL) {
      int32_t klo, khi;
      seg_range(ks, kt0, kend, klo, khi);
      if (klo > wg_hi) continue;  // uniform across the workgroup
    }
    __syncthreads();
    for (int idx = tid; idx < kBK * D / 4; idx += kThreads) {
      const int row = idx / (D / 4);
      const int32_t kr = kt0 + row;
      f32x4 zk = {0.f, 0.f, 0.f, 0.f}, zv = zk;
      if (kr < Lk) {
        zk = *(const f32x4*)(K + kbase + (size_t)kr * D + 4 * (idx % (D / 4)));
        zv = *(const f32x4*)(V + kbase + (size_t)kr * D + 4 * (idx % (D / 4)));
      }
      kt[idx] = zk;
      vt[idx] = zv;
    }
    __syncthreads();

    float s[kBK];
#pragma unroll
    for (int j = 0; j < kBK; ++j) {
      const f32x4* kr = kt + j * (D / 4) + 8 * part;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f32x4 x = kr[i];
        acc = __builtin_fmaf(q[4 * i], x[0], acc);
        acc = __builtin_fmaf(q[4 * i + 1], x[1], acc);
        acc = __builtin_fmaf(q[4 * i + 2], x[2], acc);
        acc = __builtin_fmaf(q[4 * i + 3], x[3], acc);
      }
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
      const int32_t krow = kt0 + j;
      bool masked = krow >= Lk;
      if (CAUSAL && !masked) masked = seg_pos(ks, krow) > qpos;
      s[j] = masked ? kNegInf : acc * c_log2;
    }
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < kBK; ++j) mx = fmaxf(mx, s[j]);
    const float mnew = fmaxf(mu, mx);
    const float mref = mnew == kNegInf ? 0.f : mnew;
    const float alpha = fast_exp2(mu - mref);
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kBK; ++j) {
      const float p = fast_exp2(s[j] - mref);
      lsum += p;
      const f32x4* vr = vt + j * (D / 4) + 8 * part;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f32x4 x = vr[i];
        o[4 * i] = __builtin_fmaf(p, x[0], o[4 * i]);
        o[4 * i + 1] = __builtin_fmaf(p, x[1], o[4 * i + 1]);
        o[4 * i + 2] = __builtin_fmaf(p, x[2], o[4 * i + 2]);
        o[4 * i + 3] = __builtin_fmaf(p, x[3], o[4 * i + 3]);
      }
    }
    mu = mnew;
  }

  if (!qvalid) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 y = {o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
    *(f32x4*)(Oacc + qoff + 4 * i) = y;
  }
  if (part == 0) {
    Mst[(size_t)prob * Lq + qrow] = mu * kLn2;
    Lst[(size_t)prob * Lq + qrow] = lsum;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const StepArgs& a, hipStream_t st) {
  constexpr int RPB = kThreads / (D / 32);
  const int32_t nqt = (a.Lq + RPB - 1) / RPB;
  hipLaunchKernelGGL((step_f32_kernel<D, CAUSAL>), dim3(nqt * a.nb), dim3(kThreads), 0, st,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, a.Lq, a.Lk,
                     DevSegs{a.qs.start0, a.qs.start1, a.qs.len0, a.qs.len},
                     DevSegs{a.ks.start0, a.ks.start1, a.ks.len0, a.ks.len}, a.scale * kLog2e,
                     (int32_t)a.init, a.o_acc, a.m, a.l, nqt, a.group);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_f32(const StepArgs& a, hipStream_t st) {
  if (a.d == 128) return a.causal ? launch<128, true>(a, st) : launch<128, false>(a, st);
  return a.causal ? launch<64, true>(a, st) : launch<64, false>(a, st);
}

}  // namespace ra

// Temporal half of factored video attention (Day 83 post on
// skandtandon.pages.dev, "The spatial-temporal twist"): tokens are
// frame-major (index t*S_sp + s) and the query at (t, s) attends, without a
// mask, to the T tokens {t'*S_sp + s} at its spatial position.
//
// Each problem is a T x T (T <= 16) attention with d = 64 or 128, far too
// small to be compute-bound: the kernel is an HBM stream that must move
// Q, K, V in and O out once. Design:
// * One wave per (batch*head, spatial position); the four waves of a
//   workgroup take consecutive positions, so for every frame a workgroup
//   touches one contiguous run of 4 rows.
// * Scores S^T = K Q^T come from v_mfma_f32_16x16x32_bf16 with Q and K loaded
//   straight from HBM in operand layout (16-byte loads); each lane then holds 4
//   keys of one query, and the row max / row sum finish with two lane swaps.
// * Probabilities are normalised in registers and used as the B operand of
//   O^T = V^T P^T (v_mfma_f32_16x16x16_bf16); V goes through a 4 KiB
//   per-wave LDS slot so its transpose comes from ds_read_b64_tr_b16, and the
//   output goes back out through the same slot as whole rows.
// * Frames t >= T (when T < 16) are zero-filled and masked.

#include "ra_device.h"
#include "ra_launch.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 16;  // frames per problem slot

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D>
__device__ __forceinline__ int tswz(int t, int c) {
  return D == 128 ? c ^ (2 * (t & 7)) : c ^ (2 * ((t >> 1) & 3));
}

template <int D>
__global__ __launch_bounds__(kThreads) void temporal_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    int32_t nb, int32_t T, int32_t S_sp, float c_log2, bf16* __restrict__ Out,
    float* __restrict__ Lse) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int KS = D / 32;  // k-steps of the score MFMA
  constexpr int DT = D / 16;  // 16-wide output tiles
  __shared__ bf16x8 vs[kWaves][kT * CPR];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + w;
  if (gw >= (int64_t)nb * S_sp) return;  // whole-wave exit; no workgroup barrier below
  const int64_t prob = gw / S_sp;
  const int32_t s = (int32_t)(gw - prob * S_sp);
  const int64_t N = (int64_t)T * S_sp;
  const size_t base = (size_t)prob * N * D;
  auto row_off = [&](int t) { return base + ((size_t)t * S_sp + s) * D; };

  // Every global load is issued before any result is used, so a wave waits
  // for memory once. Rows of frames t >= T are clamped to a valid row and
  // zeroed after the load.
  constexpr int NV = kT * CPR / 64;  // 16-byte V chunks per lane
  u32x4 vx[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int id = lane + 64 * i;
    const int t = id / CPR, c = id % CPR;
    vx[i] = *(const u32x4*)(V + row_off(t < T ? t : T - 1) + 8 * c);
  }
  // scores: S^T[t'][t] with A = K (row t' = lane%16), B = Q^T (column t = lane%16)
  const int t16 = lane & 15, g = lane >> 4;
  const bool ok = t16 < T;
  bf16x8 kf[KS], qf[KS];
  {
    const bf16* kp = K + row_off(ok ? t16 : 0) + 8 * g;
    const bf16* qp = Q + row_off(ok ? t16 : 0) + 8 * g;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      kf[k] = *(const bf16x8*)(kp + 32 * k);
      qf[k] = *(const bf16x8*)(qp + 32 * k);
    }
  }
  // V rows -> LDS (swizzled), zero for frames t >= T
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int id = lane + 64 * i;
    const int t = id / CPR, c = id % CPR;
    *(u32x4*)&vs[w][t * CPR + tswz<D>(t, c)] = t < T ? vx[i] : u32x4{0, 0, 0, 0};
  }
  // the slot is private to this wave: a wave-scope fence orders the writes
  // above before the transposed reads below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
  if (!ok) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      kf[k] = bf16x8{};
      qf[k] = bf16x8{};
    }
  }
#pragma unroll
  for (int k = 0; k < KS; ++k) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[k], sc, 0, 0, 0);
  // lane holds keys t' = 4g + j of query t16
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = (4 * g + j) < T ? sc[j] * c_log2 : kNegInf;
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float p[4], sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = fast_exp2(x[j] - mx);
    sum += p[j];
  }
  sum += __shfl_xor(sum, 16, 64);
  sum += __shfl_xor(sum, 32, 64);
  const float inv = 1.f / sum;
  bf16x4 pb = {to_bf16(p[0] * inv), to_bf16(p[1] * inv), to_bf16(p[2] * inv), to_bf16(p[3] * inv)};
  const s16x4 pf = __builtin_bit_cast(s16x4, pb);

  // O^T = V^T P^T, 16 output dims at a time
  const int rr = t16 >> 2, cc = t16 & 3;
  const int vrow = 4 * g + rr;
  const bool store = t16 < T;
  // The output goes out through the wave's LDS slot, so that each store
  // instruction writes four whole rows instead of 32-byte pieces of sixteen.
  // Lane (t16, g) holds dims 16dt+4g..+3 of frame t16; it overwrites V
  // columns that only this iteration reads, after its reads (a wave's LDS
  // operations run in order).
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int ncol = 16 * dt + 4 * cc;
    const char* pa = (const char*)vs[w] + 16 * (vrow * CPR + tswz<D>(vrow, ncol >> 3)) + 2 * (ncol & 7);
    const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pa);
    const f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(s16x4, va), pf, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    *(bf16x4*)((char*)vs[w] + 16 * (t16 * CPR + tswz<D>(t16, 2 * dt + (g >> 1))) + 8 * (g & 1)) =
        bf16x4{to_bf16(acc[0]), to_bf16(acc[1]), to_bf16(acc[2]), to_bf16(acc[3])};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int id = lane + 64 * i;
    const int t = id / CPR, c = id % CPR;
    const u32x4 x = *(const u32x4*)&vs[w][t * CPR + tswz<D>(t, c)];
    if (t < T) *(u32x4*)(Out + row_off(t) + 8 * c) = x;
  }
  if (Lse && g == 0 && store) Lse[(size_t)prob * N + (size_t)t16 * S_sp + s] = (mx + fast_log2(sum)) * kLn2;
}

}  // namespace

hipError_t launch_temporal_bf16(const void* q, const void* k, const void* v, int32_t nb, int32_t T,
                                int32_t S_sp, int32_t d, float scale, void* out, float* lse,
                                hipStream_t st) {
  const int64_t waves = (int64_t)nb * S_sp;
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
  const float c = scale * kLog2e;
  if (d == 128)
    hipLaunchKernelGGL((temporal_kernel<128>), grid, dim3(kThreads), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, nb, T, S_sp, c, (bf16*)out, lse);
  else
    hipLaunchKernelGGL((temporal_kernel<64>), grid, dim3(kThreads), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, nb, T, S_sp, c, (bf16*)out, lse);
  return hipGetLastError();
}

}  // namespace ra

// Temporal half of factored video attention for clips longer than 16 frames
// (Day 83 post on skandtandon.pages.dev, "The spatial-temporal twist": the
// query at (t, s) attends, without a mask, to the T tokens {t'*S_sp + s} at
// its spatial position; the opening paragraph's 48-frame clip and the
// 120-frame clip of "What the numbers look like" need more than 16).
//
// One workgroup per (batch*head, 4 adjacent spatial positions taken one after
// another; one position beyond 64 frames), T <= 128 frames:
// * K and V of the T frames (one 2*d-byte row each, S_sp rows apart in HBM)
//   are staged once in LDS, rows padded with zeros to a multiple of 16, each
//   row's 16-byte chunks XOR-swizzled by the row index so that the 16-row
//   operand reads and the transposing V reads spread over the banks.
// * Wave w takes the 16-frame query block w (4 waves up to 64 frames, 8 up to
//   128). Q rows
//   come straight from HBM as the B operand of S^T = K Q^T
//   (v_mfma_f32_16x16x32_bf16, K from LDS), so every lane holds 4 keys of one
//   query per 16-key block: the row max and row sum are in-lane reductions
//   plus two lane swaps. At T <= 128 all scores of a query fit in registers,
//   so the softmax is exact in one pass (no running rescale).
// * The weights 2^(s - max), rounded to bf16, are already the B operand of
//   O^T = V^T P^T (16x16x32, two 16-key blocks per product; V^T from the
//   transposing LDS read ds_read_b64_tr_b16 in the matching key order); the
//   output is divided by the fp32 row sum at the end.
// * Two phases split by a workgroup barrier: every wave first forms the
//   scores and weights of its query block, then the products with V;
//   between them K is no longer needed, and each wave's 16 output rows go out
//   through its own 16 rows of the K area, so that every store instruction
//   writes four whole rows rather than 8-byte pieces of 16. The lse values of
//   a frame row's positions are written together at the end (one 4-byte
//   value alone would still move a whole memory segment).
// * Arithmetic intensity is T/2 FLOP per byte (60 at T = 120), still far
//   below the matrix cores' ridge: the kernel is an HBM stream of Q, K, V in
//   and O out, and the LDS size follows T so that short clips keep several
//   workgroups per CU in flight.

#include "ra_device.h"
#include "ra_stream_launch.h"
#include "ra_tiles.h"

namespace ra {
namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;


// position of 16-byte chunk c within LDS row t (rows of D bf16); an XOR, so
// also the chunk held at position c
template <int D>
__device__ __forceinline__ int swz(int t, int c) {
  return D == 128 ? (c ^ (2 * (t & 7))) : (c ^ (2 * ((t >> 1) & 3)));
}
template <int D>
__device__ __forceinline__ int chunk_at(int t, int c) {
  return t * (D / 8) + swz<D>(t, c);
}

// kMaxT frames at most (a multiple of 16 * kWaves): every wave holds one
// 16-frame query block; kPos adjacent spatial positions per workgroup, one
// after another
template <int D, int kWaves, int kMaxT, int kPos>
__global__ __launch_bounds__(64 * kWaves) void temporal_long_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    int32_t T, int32_t S_sp, float c_log2, bf16* __restrict__ Out, float* __restrict__ Lse) {
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int KS = D / 32;   // k-steps of the score product
  constexpr int DB = D / 16;   // 16-wide output blocks
  extern __shared__ __attribute__((aligned(16))) u32x4 lds[];
  const int TP = (T + 15) & ~15;  // frames padded to whole 16-row blocks
  u32x4* ks = lds;                // [TP][CPR]
  u32x4* vs = lds + TP * CPR;     // [TP][CPR]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // this workgroup's kPos adjacent spatial positions s0 .. s0 + npos - 1
  const int32_t ngrp = (S_sp + kPos - 1) / kPos;
  const int64_t prob = blockIdx.x / ngrp;
  const int32_t s0 = (int32_t)(blockIdx.x - prob * ngrp) * kPos;
  const int npos = min(kPos, S_sp - s0);
  const int64_t N = (int64_t)T * S_sp;
  const size_t base = (size_t)prob * N * D;
  auto row_off = [&](int t, int32_t s) { return base + ((size_t)t * S_sp + s) * D; };
  const int t16 = lane & 15, g = lane >> 4;
  const int nqb = TP / 16;
  const int qb = w;  // this wave's 16-frame query block (none if w >= nqb)
  const int t = 16 * qb + t16;
  const char* kb8 = (const char*)ks;
  const char* vb8 = (const char*)vs;
  constexpr int NKP = kMaxT / 32;  // 32-key pairs of blocks
  // transposing read of V: lane (t16 = 4rr + cc, g) points at row 4g + rr of
  // a 16-key block, d columns 16db + 4cc .. +4
  const int rr = t16 >> 2, cc = t16 & 3;
  float lse_keep[kPos];

#pragma unroll
  for (int j = 0; j < kPos; ++j) {
    if (j >= npos) break;
    const int32_t s = s0 + j;
    // every wave is done with the previous position's K, V and staging rows
    if (j > 0) __syncthreads();
    // ---- stage K and V: bounds-checked buffer loads straight into LDS. A
    // record ends after row T-1 of this position, so rows T..TP-1 read as
    // zero. One load instruction fills 64 consecutive LDS chunks; lane i
    // brings the HBM chunk that the swizzle puts at LDS chunk 64u + i.
    {
      const int32_t rec = (int32_t)((((int64_t)(T - 1) * S_sp + s) * D + D) * 2);
      const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), 0, rec, 0x00020000);
      const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), 0, rec, 0x00020000);
      const int units = TP * CPR / 64;
      for (int u = w; u < units; u += kWaves) {
        const int P = 64 * u + lane, tt = P / CPR, pp = P % CPR;
        const int c = swz<D>(tt, pp);  // the swizzle is its own inverse
        const int voff = (int)(((int64_t)tt * S_sp + s) * D * 2 + 16 * c);
        tiles::bload_lds16(krs, (const char*)(ks + 64 * u), voff, 0);
        tiles::bload_lds16(vrs, (const char*)(vs + 64 * u), voff, 0);
      }
    }
    // B operand of S^T: lane (t16, g) holds d 32k + 8g .. +8 of query row t
    bf16x8 qf[KS];
    if (qb < nqb) {
      const bf16* qp = Q + row_off(t < T ? t : T - 1, s) + 8 * g;
#pragma unroll
      for (int k = 0; k < KS; ++k) qf[k] = *(const bf16x8*)(qp + 32 * k);
    }
    __builtin_amdgcn_s_waitcnt(tiles::kVmcnt0);
    __syncthreads();

    // ---- phase 1: scores and weights of the wave's query block. Weights
    // 2^(s - max), summed in fp32 and rounded to bf16, are kept as the B
    // operands of O^T = V^T P^T over 32-key pairs of blocks (a missing second
    // block of an odd count is zero in both operands).
    bf16x8 pb[NKP];
    float inv = 0.f;
    if (qb < nqb) {
      // scores, log2 units; lane holds keys 16kb + 4g + jj of query t16
      f32x4 sc[kMaxT / 16];
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < kMaxT / 16; ++kb) {
        if (kb < nqb) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            const bf16x8 kf = *(const bf16x8*)(kb8 + 16 * chunk_at<D>(16 * kb + t16, 4 * k + g));
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[k], a, 0, 0, 0);
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            a[jj] = (16 * kb + 4 * g + jj) < T ? a[jj] * c_log2 : kNegInf;
            mx = max2_nn(mx, a[jj]);
          }
          sc[kb] = a;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float sum = 0.f;
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp)
        if (2 * kp < nqb) {
          const bool two = 2 * kp + 1 < nqb;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float e0 = fast_exp2(sc[2 * kp][jj] - mx);
            const float e1 = two ? fast_exp2(sc[2 * kp + 1][jj] - mx) : 0.f;
            sum += e0 + e1;
            pb[kp][jj] = to_bf16(e0);
            pb[kp][4 + jj] = to_bf16(e1);
          }
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      inv = 1.f / sum;
      lse_keep[j] = (mx + fast_log2(sum)) * kLn2;
    }
    // every wave is done with K: its LDS rows 16w .. 16w + 15 become this
    // wave's output staging slot (chunk c of slot row r at c ^ (r % CPR)), so
    // that the stores write whole rows. A wave with a block has such rows:
    // w < nqb means 16w + 16 <= TP.
    __syncthreads();
    if (qb < nqb) {
      u32x4* os = ks + 16 * w * CPR;
      char* ob8 = (char*)os;
      // ---- phase 2: O^T = V^T P^T; lane (t16, g) ends with d 16db + 4g .. +4
      // of query t
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        const int col = 16 * db + 4 * cc;
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp) {
          if (2 * kp < nqb) {
            const int r0 = 32 * kp + 4 * g + rr;
            const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4_t*)(vb8 + 16 * chunk_at<D>(r0, col >> 3) + 2 * (col & 7)));
            bf16x4 vb = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            if (2 * kp + 1 < nqb)
              vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (lds_bf16x4_t*)(vb8 + 16 * chunk_at<D>(r0 + 16, col >> 3) + 2 * (col & 7)));
            const bf16x8 vf = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[kp], o, 0, 0, 0);
          }
        }
        const int oc = (2 * db + (g >> 1)) ^ (t16 % CPR);
        *(bf16x4*)(ob8 + 16 * (t16 * CPR + oc) + 8 * (g & 1)) =
            bf16x4{to_bf16(o[0] * inv), to_bf16(o[1] * inv), to_bf16(o[2] * inv), to_bf16(o[3] * inv)};
        // keep each block's operand reads next to its products
        __builtin_amdgcn_sched_barrier(0);
      }
      // the slot is this wave's own: a wave-scope fence orders the writes
      // above before the row reads below
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < 16 * CPR / 64; ++i) {
        const int id = lane + 64 * i, r = id / CPR, c = id % CPR;
        const u32x4 x = os[r * CPR + (c ^ (r % CPR))];
        if (16 * qb + r < T) *(u32x4*)(Out + row_off(16 * qb + r, s) + 8 * c) = x;
      }
    }
  }
  // the lse of a frame row's kPos adjacent positions go out together, so
  // that they share their memory segments
  if (Lse && qb < nqb && g == 0 && t < T) {
    float* lp = Lse + (size_t)prob * N + (size_t)t * S_sp + s0;
#pragma unroll
    for (int j = 0; j < kPos; ++j)
      if (j < npos) lp[j] = lse_keep[j];
  }
}

}  // namespace

hipError_t launch_temporal_long_bf16(const void* q, const void* k, const void* v, int32_t nb,
                                     int32_t T, int32_t S_sp, int32_t d, float scale, void* out,
                                     float* lse, hipStream_t st) {
  const int TP = (T + 15) & ~15;
  const size_t lds = (size_t)2 * TP * d * 2;
  const float c = scale * kLog2e;
  // up to 64 frames 4 waves (several workgroups fit a CU's LDS) and 4
  // positions per workgroup (their lse values go out together); beyond, 8
  // waves, one 16-frame query block each, so that a workgroup's compute
  // between its loads takes half as long, and one position per workgroup, so
  // that of the 2 workgroups that fit a CU's LDS one loads while the other
  // computes
  const bool wide = TP > 64;
  const int kpos = wide ? 1 : 4;
  const dim3 grid((unsigned)((int64_t)nb * ((S_sp + kpos - 1) / kpos)));
  const dim3 block(wide ? 512 : 256);
  if (d == 128) {
    if (wide)
      hipLaunchKernelGGL((temporal_long_kernel<128, 8, 128, 1>), grid, block, lds, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, T, S_sp, c, (bf16*)out, lse);
    else
      hipLaunchKernelGGL((temporal_long_kernel<128, 4, 64, 4>), grid, block, lds, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, T, S_sp, c, (bf16*)out, lse);
  } else {
    if (wide)
      hipLaunchKernelGGL((temporal_long_kernel<64, 8, 128, 1>), grid, block, lds, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, T, S_sp, c, (bf16*)out, lse);
    else
      hipLaunchKernelGGL((temporal_long_kernel<64, 4, 64, 4>), grid, block, lds, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, T, S_sp, c, (bf16*)out, lse);
  }
  return hipGetLastError();
}

}  // namespace ra

// Ring-step attention on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// One ring step folds the attention of a device's local queries against the
// K/V block it currently holds into a running online-softmax state; after the
// last block the state holds the exact attention output (Day 83 post on
// skandtandon.pages.dev, "Context parallelism: splitting the sequence"; k8ai
// "Sequence and Context Parallel", "How context parallel works"). Causal
// masking compares global token positions, so the balanced chunk pattern of
// the k8ai page needs no special casing here.
//
// Design (CDNA4-first; FlashAttention is prior art, not the template):
// * A workgroup is 4 waves; each wave owns 32 query rows, so a workgroup
//   covers 128 rows. Keys stream through LDS in tiles of 64 rows, double
//   buffered: the next tile is fetched into registers with 16-byte loads while
//   the current one is consumed, then written to the other LDS buffer.
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   the 32x32 accumulator layout gives every lane one query column and 16 of
//   the 32 keys, so a row maximum is an in-lane reduction plus one 32-lane swap
//   (v_permlane32_swap), and the per-query rescale factor is a lane scalar.
// * The probabilities stay in registers as the B operand of O^T += V^T P^T.
//   The key order inside each 16-key MFMA slice is permuted to match the
//   accumulator layout; the matching V^T operand is read with the gfx950
//   transposing LDS load ds_read_b64_tr_b16, so no LDS round trip of P and no
//   shuffles are needed.
// * LDS rows are XOR-swizzled in 16-byte chunks (different patterns for K and
//   V) so that both the 16-byte K reads and the transposed V reads are free
//   of bank conflicts.
// * The running maximum is only moved when a tile's maximum exceeds it by more
//   than 2^8 in weight (lazy rescale); the state stays exact because O and l
//   are always expressed relative to the same reference value m.
// * Tiles whose keys all lie after the last query (causal) are never loaded;
//   tiles straddling the diagonal, and ragged tails, are masked per element.
// * Workgroup ids are remapped so that each of the 8 XCDs works through whole
//   (batch, head) slices, keeping a slice's K/V block in that XCD's L2, and
//   within a slice the query tiles at the end of the block (the heaviest under
//   a causal mask and the zigzag split) start first.

#include "ra_device.h"
#include "ra_launch.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;  // query rows per workgroup
constexpr int kBK = 64;           // key rows per tile
constexpr float kTau = 8.0f;      // lazy-rescale threshold, log2 units

// XOR swizzle of the 16-byte chunk `c` of LDS row `row`.
template <int D>
struct Swz;
template <>
struct Swz<128> {
  static __device__ __forceinline__ int k(int row, int c) { return c ^ (row & 15); }
  static __device__ __forceinline__ int v(int row, int c) {
    return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  }
};
template <>
struct Swz<64> {
  static __device__ __forceinline__ int k(int row, int c) { return c ^ ((row >> 1) & 7); }
  static __device__ __forceinline__ int v(int row, int c) {
    return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D>
struct Tile {
  static constexpr int kChunksPerRow = D / 8;                      // 16-byte chunks
  static constexpr int kChunks = kBK * kChunksPerRow;              // per tensor
  static constexpr int kPerThread = kChunks / kThreads;            // 4 (D=128) or 2
};

template <int D, bool CAUSAL, bool FUSED>
__global__ __launch_bounds__(kThreads, 2) void step_mfma_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    int32_t nb, int32_t Lq, int32_t Lk, DevSegs qs, DevSegs ks, float c_log2, int32_t init,
    float* __restrict__ Oacc, float* __restrict__ Mst, float* __restrict__ Lst,
    bf16* __restrict__ Out, float* __restrict__ Lse, int32_t nqt, int32_t per_xcd) {
  constexpr int CPR = Tile<D>::kChunksPerRow;
  constexpr int NPT = Tile<D>::kPerThread;
  constexpr int KS = D / 16;  // k-steps of the score MFMA
  constexpr int DT = D / 32;  // 32-wide output tiles
  __shared__ bf16x8 smem[2][2][Tile<D>::kChunks];  // [buffer][K/V][row*CPR + chunk]

  // ---- which (slice, query tile) this workgroup owns
  const int32_t total = nb * nqt;
  const int32_t p = blockIdx.x;
  const int32_t logical = (p & 7) * per_xcd + (p >> 3);
  if (logical >= total) return;
  const int32_t prob = logical / nqt;
  const int32_t qtile = nqt - 1 - (logical - prob * nqt);
  const int32_t qt0 = qtile * kBQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const size_t qbase = (size_t)prob * Lq * D;
  const size_t kbase = (size_t)prob * Lk * D;

  const int32_t qrow = qt0 + 32 * w + l32;
  const bool qvalid = qrow < Lq;
  const int32_t qrow_c = qvalid ? qrow : Lq - 1;
  const int32_t qpos = seg_pos(qs, qrow_c);

  const int32_t wg_r1 = min(qt0 + kBQ, Lq);
  int32_t wg_qlo, wg_qhi;
  seg_range(qs, qt0, wg_r1, wg_qlo, wg_qhi);
  const int32_t w_r0 = qt0 + 32 * w;
  const bool wave_active = w_r0 < Lq;
  int32_t w_qlo = 0, w_qhi = -1;
  if (wave_active) seg_range(qs, w_r0, min(w_r0 + 32, Lq), w_qlo, w_qhi);

  // ---- query fragments: B operand of S^T = K Q^T (lane: query l32, d 16ks+8h..+8)
  bf16x8 qf[KS];
  {
    const bf16* qp = Q + qbase + (size_t)qrow_c * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
  }

  // ---- running state: O^T accumulators (lane: query l32, d 32dt+8i+4h+j)
  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};
  float mu = kNegInf;  // reference value in log2 units of the weights
  float lrun = 0.f;    // this lane's share of the row sum
  if (!FUSED && !init && qvalid) {
    const float* op = Oacc + qbase + (size_t)qrow * D + 4 * h;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 x = *(const f32x4*)(op + 32 * t + 8 * i);
        o[t][4 * i + 0] = x[0];
        o[t][4 * i + 1] = x[1];
        o[t][4 * i + 2] = x[2];
        o[t][4 * i + 3] = x[3];
      }
    const size_t r = (size_t)prob * Lq + qrow;
    mu = Mst[r] * kLog2e;
    lrun = h == 0 ? Lst[r] : 0.f;
  }

  // ---- key rows this workgroup can see: at most two row ranges
  int32_t ra0 = 0, rb0 = Lk, ra1 = 0, rb1 = 0;
  if (CAUSAL) {
    auto vis = [&](int32_t start, int32_t n) {
      int32_t x = wg_qhi - start + 1;
      return x < 0 ? 0 : (x > n ? n : x);
    };
    ra0 = 0;
    rb0 = vis(ks.start0, ks.len0);
    ra1 = ks.len0;
    rb1 = ks.len0 + (ks.len > ks.len0 ? vis(ks.start1, ks.len - ks.len0) : 0);
  }
  const int32_t t0a = ra0 / kBK, t0b = (rb0 + kBK - 1) / kBK;
  const int32_t n0 = rb0 > ra0 ? t0b - t0a : 0;
  int32_t t1a = ra1 / kBK;
  const int32_t t1b = (rb1 + kBK - 1) / kBK;
  if (n0 > 0 && t1a < t0b) t1a = t0b;
  const int32_t n1 = rb1 > ra1 && t1b > t1a ? t1b - t1a : 0;
  const int32_t ntiles = n0 + n1;
  auto tile_of = [&](int32_t n) { return n < n0 ? t0a + n : t1a + (n - n0); };

  u32x4 pk[NPT], pv[NPT];
  auto gload = [&](int32_t kt0) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int id = tid + kThreads * i;
      const int row = id / CPR, c = id % CPR;
      const int32_t kr = kt0 + row;
      if (kr < Lk) {
        const size_t off = kbase + (size_t)kr * D + 8 * c;
        pk[i] = *(const u32x4*)(K + off);
        pv[i] = *(const u32x4*)(V + off);
      } else {
        pk[i] = u32x4{0, 0, 0, 0};
        pv[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int id = tid + kThreads * i;
      const int row = id / CPR, c = id % CPR;
      *(u32x4*)&smem[buf][0][row * CPR + Swz<D>::k(row, c)] = pk[i];
      *(u32x4*)&smem[buf][1][row * CPR + Swz<D>::v(row, c)] = pv[i];
    }
  };

  if (ntiles > 0) {
    gload(tile_of(0) * kBK);
    sstore(0);
    __syncthreads();
  }

  for (int32_t n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    const int32_t kt0 = tile_of(n) * kBK;
    const bool has_next = n + 1 < ntiles;
    if (has_next) gload(tile_of(n + 1) * kBK);

    bool run = wave_active;
    bool need_mask = kt0 + kBK > Lk;
    if (CAUSAL && run) {
      int32_t klo, khi;
      seg_range(ks, kt0, min(kt0 + kBK, Lk), klo, khi);
      if (klo > w_qhi) run = false;
      if (khi > w_qlo) need_mask = true;
    }
    if (run) {
      const bf16x8* Kt = smem[buf][0];
      const bf16x8* Vt = smem[buf][1];
      // S^T for two 32-key slices
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s[st] = f32x16{};
        const int row = 32 * st + l32;
#pragma unroll
        for (int ksi = 0; ksi < KS; ++ksi) {
          const bf16x8 kf = Kt[row * CPR + Swz<D>::k(row, 2 * ksi + h)];
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ksi], s[st], 0, 0, 0);
        }
      }
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int32_t kr = kt0 + 32 * st + 8 * i + 4 * h + j;
              bool masked = kr >= Lk;
              if (CAUSAL && !masked) masked = seg_pos(ks, kr) > qpos;
              if (masked) s[st][4 * i + j] = kNegInf;
            }
      }
      // online softmax with lazy rescale
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = partner32_max(mx);
      const float mt = mx * c_log2;
      const bool need = mt > mu + kTau;
      if (__builtin_amdgcn_ballot_w64(need)) {
        // lanes that keep their reference (including rows with no visible key
        // yet, mu = -inf) must get exactly 1, not exp2(-inf - -inf)
        const float mnew = need ? mt : mu;
        const float alpha = need ? fast_exp2(mu - mnew) : 1.f;
        lrun *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
        mu = mnew;
      }
      const float mus = mu == kNegInf ? 0.f : mu;
      bf16x8 pf[4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(__builtin_fmaf(s[st][r], c_log2, -mus));
          lrun += pr;
          pf[2 * st + r / 8][r % 8] = to_bf16(pr);
        }
      // O^T += V^T P^T over four 16-key slices
      const int g = lane >> 4, jj = lane & 15, rr = jj >> 2, cc = jj & 3;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const int ncol = 32 * t + 16 * (g & 1) + 4 * cc;  // first of 4 columns this lane loads
          const int ra = 16 * kc + 4 * (g >> 1) + rr;       // key row, first half
          const int rb = ra + 8;                            // key row, second half
          const char* base = (const char*)Vt;
          const char* pa = base + 16 * (ra * CPR + Swz<D>::v(ra, ncol >> 3)) + 2 * (ncol & 7);
          const char* pb = base + 16 * (rb * CPR + Swz<D>::v(rb, ncol >> 3)) + 2 * (ncol & 7);
          const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pa);
          const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pb);
          const bf16x8 vf = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kc], o[t], 0, 0, 0);
        }
      }
    }
    if (has_next) sstore(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float lsum = partner32_sum(lrun);
  if (FUSED) {
    if (!qvalid) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    bf16* op = Out + qbase + (size_t)qrow * D + 4 * h;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 y = {to_bf16(o[t][4 * i + 0] * inv), to_bf16(o[t][4 * i + 1] * inv),
                    to_bf16(o[t][4 * i + 2] * inv), to_bf16(o[t][4 * i + 3] * inv)};
        *(bf16x4*)(op + 32 * t + 8 * i) = y;
      }
    if (Lse && h == 0)
      Lse[(size_t)prob * Lq + qrow] = lsum > 0.f ? (mu + fast_log2(lsum)) * kLn2 : kNegInf;
  } else {
    if (!qvalid) return;
    float* op = Oacc + qbase + (size_t)qrow * D + 4 * h;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 y = {o[t][4 * i + 0], o[t][4 * i + 1], o[t][4 * i + 2], o[t][4 * i + 3]};
        *(f32x4*)(op + 32 * t + 8 * i) = y;
      }
    if (h == 0) {
      const size_t r = (size_t)prob * Lq + qrow;
      Mst[r] = mu * kLn2;
      Lst[r] = lsum;
    }
  }
}

DevSegs dev(const HostSegs& s) { return DevSegs{s.start0, s.start1, s.len0, s.len}; }

template <int D, bool CAUSAL, bool FUSED>
hipError_t launch(const StepArgs& a, bf16* out, float* lse, hipStream_t st) {
  const int32_t nqt = (a.Lq + kBQ - 1) / kBQ;
  const int64_t total = (int64_t)a.nb * nqt;
  const int32_t per_xcd = (int32_t)((total + 7) / 8);
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((step_mfma_kernel<D, CAUSAL, FUSED>), dim3(8 * per_xcd), dim3(kThreads), 0,
                     st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.nb, a.Lq, a.Lk,
                     dev(a.qs), dev(a.ks), c, (int32_t)a.init, a.o_acc, a.m, a.l, out, lse, nqt,
                     per_xcd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& a, hipStream_t st) {
  if (a.d == 128)
    return a.causal ? launch<128, true, false>(a, nullptr, nullptr, st)
                    : launch<128, false, false>(a, nullptr, nullptr, st);
  return a.causal ? launch<64, true, false>(a, nullptr, nullptr, st)
                  : launch<64, false, false>(a, nullptr, nullptr, st);
}

hipError_t launch_attend_bf16(const void* q, const void* k, const void* v, int32_t nb, int32_t L,
                              int32_t d, float scale, void* out, float* lse, hipStream_t st) {
  StepArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.nb = nb;
  a.Lq = L;
  a.Lk = L;
  a.d = d;
  a.qs = HostSegs{0, 0, L, L};
  a.ks = HostSegs{0, 0, L, L};
  a.causal = false;
  a.init = true;
  a.scale = scale;
  if (d == 128) return launch<128, false, true>(a, (bf16*)out, lse, st);
  return launch<64, false, true>(a, (bf16*)out, lse, st);
}

}  // namespace ra

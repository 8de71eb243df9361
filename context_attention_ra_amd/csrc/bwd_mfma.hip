// Backward ring step on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// The ring moves K/V blocks in the backward pass as in the forward one (k8ai
// "Sequence and Context Parallel", "Communication profile"); the Ultralytics
// glossary's example trains through the attention ("Practical Use and
// Tradeoffs"). For one block held at a ring step, this adds the block's share
// of the gradients of softmax attention, taken with the final forward
// normaliser lse_i and delta_i = <dO_i, O_i>:
//   P_ij  = exp(scale <q_i, k_j> - lse_i)   (visible pairs only)
//   dS_ij = P_ij (<dO_i, v_j> - delta_i)
//   dQ_i += scale sum_j dS_ij k_j      (local queries: dQ stays on the device)
//   dK_j += scale sum_i dS_ij q_i      (the block's accumulators travel with it)
//   dV_j += sum_i P_ij dO_i
//
// Two kernels, no atomics, so the result is deterministic:
// * bwd_dq: each wave owns 32 query rows and streams 64-key K/V tiles:
//   S^T = K Q^T and dP^T = V dO^T (A from LDS, B = the wave's Q and dO rows
//   in registers), dS^T formed in registers (every lane owns one query, so
//   lse and delta are lane scalars), dQ^T += K^T dS^T with the transposing
//   LDS read for K^T and dS^T as the B operand straight from the registers.
//   Eight waves (256 queries) share a 4-deep LDS ring of K/V tiles; as in the
//   forward ring step, the two halves of the workgroup (one wave of each on
//   every SIMD) run the same per-tile program one phase apart, so one wave
//   of a SIMD issues the products (dQ of tile n, S and dP of tile n+1) while
//   the other forms the weights of its next tile. Without that offset the
//   barrier of every tile keeps both waves of a SIMD in the same phase, and
//   products and exponentials take turns instead of overlapping.
// * bwd_dkdv: each wave owns 32 key rows and streams 64-row Q/dO tiles:
//   S = Q K^T and dP = dO V^T (every lane owns one key; the per-row lse and
//   delta of the tile come from LDS), then dV^T += dO^T P and dK^T += Q^T dS.
// With fewer K/V heads than query heads (G consecutive query heads per K/V
// head), the dQ kernel reads K/V slice p / G and the dK/dV kernel walks the
// Q/dO tiles of all G query heads of its K/V head, so their contributions sum
// in one accumulator.
// Both recompute S and dP, so the matrix cores run 14*d FLOP per visible
// pair against the 8*d of the four products the gradients need.
// The LDS tile layout, the operand reads and the key permutation inside each
// 16-row MFMA slice are those of the forward ring step: tiles are stored
// column-major in 16-byte columns (runs of 64 rows padded to 1088 bytes),
// filled by bounds-checked buffer loads that write LDS directly.

#include "ra_bwd.h"
#include "ra_device.h"
#include "ra_tiles.h"

namespace ra {
namespace {

constexpr int kQW = 8;                // waves per workgroup of the dQ kernel
constexpr int kQThreads = 64 * kQW;
constexpr int kQOwn = 32 * kQW;       // owned query rows per workgroup of the dQ kernel
constexpr int kQStages = 4;           // LDS ring depth of the dQ kernel
constexpr int kQAhead = 3;            // LDS operands read ahead of their MFMA (dQ kernel)
constexpr int kKW = 8;                // waves per workgroup of the dK/dV kernel
constexpr int kKThreads = 64 * kKW;
constexpr int kKOwn = 32 * kKW;       // owned keys per workgroup of the dK/dV kernel
constexpr int kKAhead = 4;            // LDS operands read ahead of their MFMA (dK/dV kernel)
using namespace tiles;
static_assert(BLay<128>::NRUN % kKW == 0 && BLay<64>::NRUN % kKW == 0 && kQW == kKW,
              "load runs must split evenly over the waves");

// s_waitcnt encodings (gfx9): wait until at most n vector-memory ops are pending
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// The dQ kernel body is written as lambdas; with two copies of its schedule
// the inliner would otherwise turn some of them into calls with stack frames.
#define RA_BINLINE __attribute__((always_inline))

template <bool B>
struct GroupC {
  static constexpr bool value = B;
};

// ---------------------------------------------------------------------------
// dQ: owned queries, streamed K/V tiles, two wave groups in ping-pong

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kQThreads, 1) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ Dlt,
    int32_t nb, int32_t Lq, int32_t Lk, DevSegs qs, DevSegs ks, float c_log2, float scale,
    int32_t init, float* __restrict__ dQ, int32_t nqt, int32_t per_xcd, int32_t group) {
  using L = BLay<D>;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int TB = 2 * L::TBYTES;          // K tile, then V tile
  constexpr int NDMA = 2 * (L::NRUN / kQW);  // load instructions per wave per tile
  __shared__ __attribute__((aligned(16))) char smem[kQStages * TB];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: the group branch is scalar
  const int32_t logical = xcd_logical(per_xcd);
  if (logical >= nb * nqt) return;
  const int32_t prob = logical / nqt;
  // causal: the last query tiles of a slice see the most keys, so they are
  // dispatched first and the light ones fill the tail (the workgroups of an
  // XCD start in logical order as CUs free up)
  const int32_t qt = logical - prob * nqt;
  const int32_t q0 = (CAUSAL ? nqt - 1 - qt : qt) * kQOwn;

  const int32_t w_r0 = q0 + 32 * w;
  const int32_t qrow = w_r0 + l32;
  const bool qvalid = qrow < Lq;
  const int32_t qrow_c = qvalid ? qrow : Lq - 1;
  const int32_t qpos = seg_pos(qs, qrow_c);
  int32_t w_qlo = INT32_MAX, w_qhi;
  if (w_r0 < Lq) seg_range(qs, w_r0, min(w_r0 + 32, Lq), w_qlo, w_qhi);
  w_qlo = __builtin_amdgcn_readfirstlane(w_qlo);

  // key tiles some owned query can see
  TileRuns tr{0, 0, 0, 0};
  if (CAUSAL) {
    int32_t lo, hi;
    seg_range(qs, q0, min(q0 + kQOwn, Lq), lo, hi);
    tr = tiles_from(ks, Lk, 0, hi, false);
  } else {
    tr.n0 = tr.n = (Lk + kT - 1) / kT;
  }
  const size_t rbase = (size_t)prob * Lq;
  float* dqp = dQ + (rbase + qrow) * D + 4 * h;
  if (tr.n == 0) {
    if (init && qvalid) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) *(f32x4*)(dqp + 32 * t + 8 * i) = f32x4{};
    }
    return;
  }
  const int32_t nt = tr.n;

  // this lane's query and upstream-gradient rows (B operands), lse and delta
  bf16x8 qf[KS], df[KS];
  const bf16* qp = Q + (rbase + qrow_c) * D + 8 * h;
  const bf16* dp = dO + (rbase + qrow_c) * D + 8 * h;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = *(const bf16x8*)(qp + 16 * s);
    df[s] = *(const bf16x8*)(dp + 16 * s);
  }
  const float lse = Lse[rbase + qrow_c];
  // rows with no visible key (lse = -inf) and rows past the end get P = 0
  const float lse2 = (qvalid && lse != kNegInf) ? lse * kLog2e : __builtin_inff();
  const float dlt = Dlt[rbase + qrow_c];

  const size_t kvbase = (size_t)(prob / group) * Lk * D;  // the K/V head of this query head
  const __amdgpu_buffer_rsrc_t krs = slice_rsrc(K + kvbase, Lk, D);
  const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(V + kvbase, Lk, D);
  int32_t fg = 0;  // next tile to request; tile n sits in stage n % kQStages
  auto fetch_next = [&]() RA_BINLINE {
    char* st = smem + (fg % kQStages) * TB;
    const int32_t r0 = __builtin_amdgcn_readfirstlane(tile_row0(tr, fg));
    load_tile<D, kQW>(krs, st, r0, w, lane);
    load_tile<D, kQW>(vrs, st + L::TBYTES, r0, w, lane);
    ++fg;
  };
#pragma unroll
  for (int i = 0; i < kQStages; ++i)
    if (i < nt) fetch_next();

  f32x16 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x16{};
  f32x16 s[2], dpv[2];  // S^T, dP^T of the tile whose weights come next
  bf16x8 dsb[4];        // dS^T of the tile whose dQ products come next (16-key slices)
  const int trb = tr_base<D>(lane);

  // step i of S^T = K Q^T and dP^T = V dO^T (k-step i/4, 32-key half (i/2)%2,
  // K or V): its A operand from the tile at kt, and its product
  auto m1_operand = [&](const char* kt, int i) RA_BINLINE -> bf16x8 {
    const int ksi = i / 4, st = (i / 2) % 2, tens = i % 2;
    return row_operand<D>(kt + tens * L::TBYTES, st, ksi, l32, h);
  };
  auto m1_step = [&](int i, const bf16x8& op) RA_BINLINE {
    const int ksi = i / 4, st = (i / 2) % 2, tens = i % 2;
    if (tens == 0)
      s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[ksi], s[st], 0, 0, 0);
    else
      dpv[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, df[ksi], dpv[st], 0, 0, 0);
  };
  // S^T and dP^T of tile n alone (the first tile of each group)
  auto scores = [&](int32_t n) RA_BINLINE {
    const char* kt = smem + (n % kQStages) * TB;
#pragma unroll
    for (int st = 0; st < 2; ++st) s[st] = dpv[st] = f32x16{};
#pragma unroll
    for (int i = 0; i < 4 * KS; ++i) m1_step(i, m1_operand(kt, i));
  };
  // weights of tile n: P = exp(S - lse) on visible pairs, dS = P (dP - delta)
  auto vector_phase = [&](int32_t n) RA_BINLINE {
    const int32_t kt0 = tile_row0(tr, n);
    bool need_mask = kt0 + kT > Lk;
    if (CAUSAL) {
      int32_t klo, khi;
      seg_range(ks, kt0, min(kt0 + kT, Lk), klo, khi);
      (void)klo;
      need_mask = need_mask || khi > w_qlo;
    }
    if (need_mask) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t kr = kt0 + 32 * st + acc_row(r, h);
          const bool vis = kr < Lk && (!CAUSAL || seg_pos(ks, kr) <= qpos);
          s[st][r] = vis ? s[st][r] : kNegInf;
        }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[st][r], c_log2, -lse2));
        ds[r] = p * (dpv[st][r] - dlt);
      }
      pack_b(ds, dsb[2 * st], dsb[2 * st + 1]);
    }
    // the weights are complete here: without this use the compiler sinks part
    // of the exponentials into the next phase, between the same wave's products
    asm volatile("" ::"v"(dsb[0]), "v"(dsb[1]), "v"(dsb[2]), "v"(dsb[3]));
  };
  // matrix phase n: S^T, dP^T of tile n+1, then dQ^T += K^T dS^T of tile n;
  // every LDS operand is read kQAhead steps before its MFMA, and scheduling
  // barriers keep that order
  auto matrix = [&](int32_t n) RA_BINLINE {
    __builtin_amdgcn_s_setprio(1);
    // past the last tile the S^T, dP^T products read a stage that holds no
    // tile of this workgroup; their results are never used
    const char* kn = smem + ((n + 1) % kQStages) * TB;
    const char* kc = smem + (n % kQStages) * TB;
    constexpr int N1 = 4 * KS, N2 = 4 * DT;
    auto operand = [&](int i) RA_BINLINE -> bf16x8 {
      if (i < N1) return m1_operand(kn, i);
      const int j = i - N1;
      return tr_operand<D>(kc, trb, j / DT, j % DT);
    };
#pragma unroll
    for (int st = 0; st < 2; ++st) s[st] = dpv[st] = f32x16{};
    bf16x8 op[kQAhead];
#pragma unroll
    for (int j = 0; j < kQAhead; ++j) op[j] = operand(j);
#pragma unroll
    for (int i = 0; i < N1 + N2; ++i) {
      const bf16x8 cur = op[i % kQAhead];
      if (i < N1) {
        m1_step(i, cur);
      } else {
        const int j = i - N1, t = j % DT;
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, dsb[j / DT], acc[t], 0, 0, 0);
      }
      if (i + kQAhead < N1 + N2) op[i % kQAhead] = operand(i + kQAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Ping-pong as in the forward ring step: waves 0..3 (group A) and 4..7
  // (group B, one of each on every SIMD) run the same per-tile program one
  // slot apart, so one wave of a SIMD issues products while the other forms
  // weights. Group A: slot 0 = scores and weights of tile 0, slot 2n+1 =
  // matrix phase n, slot 2n+2 = weights of tile n+1; group B one slot later.
  // Tile n is read from matrix phase n-1 to matrix phase n of group B (slot
  // 2n+2); at the start of slot 2n+3 tile n+4 is requested into its stage.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  auto run = [&](auto grp) RA_BINLINE {
    constexpr bool late = decltype(grp)::value;
    // end of slot 2n: tile n+1 must be in LDS; tiles requested after it may
    // stay in flight
    auto slot_end = [&](int32_t n) RA_BINLINE {
      const int32_t in_flight = fg - (n + 2);
      if (in_flight >= 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NDMA));
      else if (in_flight == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NDMA));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
    };
    if (!late) {
      scores(0);
      vector_phase(0);
    }
    slot_end(0);
    for (int32_t n = 0; n < nt; ++n) {
      if (fg == n + kQStages - 1 && fg < nt) fetch_next();
      if (!late) {
        matrix(n);
      } else {
        if (n == 0) scores(0);
        vector_phase(n);
      }
      __syncthreads();
      if (!late) {
        if (n + 1 < nt) vector_phase(n + 1);
      } else {
        matrix(n);
      }
      slot_end(n + 1);
    }
  };
  if (w >= kQW / 2)
    run(GroupC<true>{});
  else
    run(GroupC<false>{});

  if (!qvalid) return;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 y = {scale * acc[t][4 * i], scale * acc[t][4 * i + 1], scale * acc[t][4 * i + 2],
                 scale * acc[t][4 * i + 3]};
      if (!init) y += *(const f32x4*)(dqp + 32 * t + 8 * i);
      *(f32x4*)(dqp + 32 * t + 8 * i) = y;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: owned keys, streamed Q/dO tiles. Eight waves (256 owned keys): the
// owned V rows sit in LDS (four 64-row tiles of the same layout) and are read
// as B operands, which keeps a wave within 256 registers, so two waves share
// each SIMD. Every LDS operand of a tile is read kKAhead products before the
// product that uses it (one stream per tile through a ring of registers, its
// order held by scheduling barriers): the compiler by itself keeps one or two
// reads in flight and waits on the LDS before almost every product. (The dQ
// kernel's ping-pong does not pay here: the scores of a whole next tile do not
// fit beside the two accumulators, and with half-tile units each matrix phase
// reads about as many LDS bytes per product as the LDS delivers.)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kKThreads, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ Dlt,
    int32_t nb, int32_t Lq, int32_t Lk, DevSegs qs, DevSegs ks, float c_log2, float scale,
    int32_t init, float* __restrict__ dK, float* __restrict__ dV, int32_t nkt, int32_t per_xcd,
    int32_t group) {
  using L = BLay<D>;
  constexpr int KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::STAGE + (kKOwn / kT) * L::TBYTES];
  char* const vown = smem + 2 * L::STAGE;  // the owned V rows, 64 per tile
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int32_t logical = xcd_logical(per_xcd);
  if (logical >= nb * nkt) return;  // nb counts K/V slices here
  const int32_t prob = logical / nkt;  // K/V slice; its query slices are prob*group ..
  const int32_t k0 = (logical - prob * nkt) * kKOwn;

  const int32_t w_r0 = k0 + 32 * w;
  const int32_t krow = w_r0 + l32;
  const bool kvalid = krow < Lk;
  const int32_t krow_c = kvalid ? krow : Lk - 1;
  const int32_t kpos = seg_pos(ks, krow_c);
  int32_t w_klo, w_khi = INT32_MIN;
  if (w_r0 < Lk) seg_range(ks, w_r0, min(w_r0 + 32, Lk), w_klo, w_khi);
  w_khi = __builtin_amdgcn_readfirstlane(w_khi);

  // query tiles holding a query that can see some owned key
  TileRuns tr{0, 0, 0, 0};
  if (CAUSAL) {
    int32_t lo, hi;
    seg_range(ks, k0, min(k0 + kKOwn, Lk), lo, hi);
    tr = tiles_from(qs, Lq, lo, 0, true);
  } else {
    tr.n0 = tr.n = (Lq + kT - 1) / kT;
  }
  const size_t kb = (size_t)prob * Lk;
  float* dkp = dK + (kb + krow) * D + 4 * h;
  float* dvp = dV + (kb + krow) * D + 4 * h;
  // the stream: tr.n tiles of each of the group's query heads in turn
  const int32_t ntiles = tr.n * group;
  if (tr.n == 0) {
    if (init && kvalid) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *(f32x4*)(dkp + 32 * t + 8 * i) = f32x4{};
          *(f32x4*)(dvp + 32 * t + 8 * i) = f32x4{};
        }
    }
    return;
  }

  // query slice and tile of stream tile m
  auto qslice = [&](int32_t m) { return (size_t)prob * group + m / tr.n; };
  auto qtile = [&](int32_t m) { return tile_row0(tr, m % tr.n); };
  // lse (log2 units) and delta of the tile's rows: thread i < 64 brings the
  // lse of row i, thread 64 + i its delta; rows past the end get lse = +inf
  // (so P = 0) and delta = 0
  float rowv = 0.f;
  auto fetch_rowv = [&](int32_t n) {
    const size_t rbase = qslice(n) * Lq;
    const int32_t r = qtile(n) + (tid & 63);
    if (tid < 64) {
      const float x = r < Lq ? Lse[rbase + r] : kNegInf;
      rowv = x != kNegInf ? x * kLog2e : __builtin_inff();
    } else if (tid < 128) {
      rowv = r < Lq ? Dlt[rbase + r] : 0.f;
    }
  };
  auto store_rowv = [&](int32_t n) {
    if (tid < 128) *(float*)(smem + (n & 1) * L::STAGE + 2 * L::TBYTES + 4 * tid) = rowv;
  };
  auto fetch = [&](int32_t n) {
    char* st = smem + (n & 1) * L::STAGE;
    const size_t rbase = qslice(n) * Lq;
    const int32_t r0 = qtile(n);
    load_tile<D, kKW>(slice_rsrc(Q + rbase * D, Lq, D), st, r0, w, lane);
    load_tile<D, kKW>(slice_rsrc(dO + rbase * D, Lq, D), st + L::TBYTES, r0, w, lane);
  };
  fetch_rowv(0);
  fetch(0);
  {
    const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(V + kb * D, Lk, D);
#pragma unroll
    for (int j = 0; j < kKOwn / kT; ++j) load_tile<D, kKW>(vrs, vown + j * L::TBYTES, k0 + kT * j, w, lane);
  }
  // this wave's 32 owned V rows: rows 32(w%2).. of owned tile w/2
  const char* vw = vown + (w >> 1) * L::TBYTES;

  bf16x8 kf[KS];
  const bf16* kp = K + (kb + krow_c) * D + 8 * h;
#pragma unroll
  for (int s = 0; s < KS; ++s) kf[s] = *(const bf16x8*)(kp + 16 * s);
  f32x16 ak[DT], av[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) ak[t] = av[t] = f32x16{};
  const int trb = tr_base<D>(lane);

  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  store_rowv(0);
  __syncthreads();
  // the LDS operand stream of a tile, each read AH products ahead: for each
  // 32-row half st, the S and dP products' operands (per k-step: Q rows, dO
  // rows, this wave's owned V rows), then the accumulation products'
  // (transposing reads of dO and Q)
  constexpr int AH = kKAhead;
  constexpr int NE1 = 3 * KS, NE2 = 4 * DT, NEH = NE1 + NE2, NE = 2 * NEH;
  for (int32_t n = 0; n < ntiles; ++n) {
    if (n + 1 < ntiles) {
      fetch_rowv(n + 1);
      fetch(n + 1);
    }
    const char* qt = smem + (n & 1) * L::STAGE;
    const char* dt = qt + L::TBYTES;
    const float* lsev = (const float*)(qt + 2 * L::TBYTES);
    const float* dltv = lsev + kT;
    const int32_t qt0 = qtile(n);
    bool need_mask = false;
    if (CAUSAL) {
      int32_t qlo, qhi;
      seg_range(qs, qt0, min(qt0 + kT, Lq), qlo, qhi);
      (void)qhi;
      need_mask = w_khi > qlo;
    }
    auto entry = [&](int e) RA_BINLINE -> bf16x8 {
      const int st = e / NEH, j = e % NEH;
      if (j < NE1) {
        const int ksi = j / 3, which = j % 3;
        if (which == 0) return row_operand<D>(qt, st, ksi, l32, h);
        if (which == 1) return row_operand<D>(dt, st, ksi, l32, h);
        return row_operand<D>(vw, w & 1, ksi, l32, h);
      }
      // accumulation product k: operand u (dO slice 2st, 2st+1, Q slice 2st,
      // 2st+1) of output tile t, t varying fastest, so that the two products
      // into one accumulator have three others between them
      const int k = j - NE1, u = k / DT, t = k % DT;
      return tr_operand<D>(u < 2 ? dt : qt, trb, 2 * st + (u & 1), t);
    };
    bf16x8 ring[AH];
#pragma unroll
    for (int e = 0; e < AH; ++e) ring[e] = entry(e);
    auto refill = [&](int e) RA_BINLINE {
      if (e + AH < NE) ring[e % AH] = entry(e + AH);
    };
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 s = f32x16{}, dpv = f32x16{};
#pragma unroll
      for (int ksi = 0; ksi < KS; ++ksi) {
        const int e = st * NEH + 3 * ksi;
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[e % AH], kf[ksi], s, 0, 0, 0);
        refill(e);
        __builtin_amdgcn_sched_barrier(0);
        dpv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[(e + 1) % AH], ring[(e + 2) % AH], dpv, 0, 0, 0);
        refill(e + 1);
        refill(e + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      // masked scores become -inf (weight exactly 0) in one block, so that
      // the exponentials below are straight-line code
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t q = qt0 + 32 * st + acc_row(r, h);
          const bool vis = q < Lq && seg_pos(qs, q) >= kpos;
          s[r] = vis ? s[r] : kNegInf;
        }
      }
      f32x16 p, ds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rb = 32 * st + 8 * i + 4 * h;  // rows rb..rb+3 of the tile
        const f32x4 l4 = *(const f32x4*)(lsev + rb);
        const f32x4 d4 = *(const f32x4*)(dltv + rb);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * i + j;
          // c_log2 > 0 and the row's lse is finite or +inf: a -inf score gives 0
          const float pv = fast_exp2(__builtin_fmaf(s[r], c_log2, -l4[j]));
          p[r] = pv;
          ds[r] = pv * (dpv[r] - d4[j]);
        }
      }
      bf16x8 pk[4];
      pack_b(p, pk[0], pk[1]);
      pack_b(ds, pk[2], pk[3]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NE2; ++k) {
        const int e = st * NEH + NE1 + k, u = k / DT, t = k % DT;
        if (u < 2)
          av[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[e % AH], pk[u], av[t], 0, 0, 0);
        else
          ak[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[e % AH], pk[u], ak[t], 0, 0, 0);
        refill(e);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    if (n + 1 < ntiles) store_rowv(n + 1);
    __syncthreads();
  }
  if (!kvalid) return;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 yk = {scale * ak[t][4 * i], scale * ak[t][4 * i + 1], scale * ak[t][4 * i + 2],
                  scale * ak[t][4 * i + 3]};
      f32x4 yv = {av[t][4 * i], av[t][4 * i + 1], av[t][4 * i + 2], av[t][4 * i + 3]};
      if (!init) {
        yk += *(const f32x4*)(dkp + 32 * t + 8 * i);
        yv += *(const f32x4*)(dvp + 32 * t + 8 * i);
      }
      *(f32x4*)(dkp + 32 * t + 8 * i) = yk;
      *(f32x4*)(dvp + 32 * t + 8 * i) = yv;
    }
}

// delta_i = <dO_i, O_i> in fp32; D/8 lanes per row, 8 elements each
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const bf16* __restrict__ O,
                                                       const bf16* __restrict__ dO, int64_t rows,
                                                       float* __restrict__ Dlt) {
  constexpr int LPR = D / 8;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / LPR;
  const int part = (int)(g % LPR);
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *(const bf16x8*)(O + row * D + 8 * part);
    const bf16x8 b = *(const bf16x8*)(dO + row * D + 8 * part);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_fmaf(from_bf16(a[j]), from_bf16(b[j]), acc);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) Dlt[row] = acc;
}

DevSegs bdev(const HostSegs& s) { return DevSegs{s.start0, s.start1, s.len0, s.len}; }

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  const float c = a.scale * kLog2e;
  const int32_t nqt = (a.Lq + kQOwn - 1) / kQOwn, nkt = (a.Lk + kKOwn - 1) / kKOwn;
  const int32_t nkv = a.nb / a.group;
  const int32_t pq = (int32_t)(((int64_t)a.nb * nqt + kXcdsB - 1) / kXcdsB);
  const int32_t pk = (int32_t)(((int64_t)nkv * nkt + kXcdsB - 1) / kXcdsB);
  if (a.run_dq) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(kXcdsB * pq), dim3(kQThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dout,
                       a.lse, a.delta, a.nb, a.Lq, a.Lk, bdev(a.qs), bdev(a.ks), c, a.scale,
                       (int32_t)a.init_dq, a.dq, nqt, pq, a.group);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.run_dkv) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(kXcdsB * pk), dim3(kKThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dout,
                       a.lse, a.delta, nkv, a.Lq, a.Lk, bdev(a.qs), bdev(a.ks), c, a.scale,
                       (int32_t)a.init_dkv, a.dk, a.dv, nkt, pk, a.group);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_step_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  if (a.d == 128) return a.causal ? launch_bwd<128, true>(a, st) : launch_bwd<128, false>(a, st);
  return a.causal ? launch_bwd<64, true>(a, st) : launch_bwd<64, false>(a, st);
}

hipError_t launch_bwd_prep_bf16(const void* out, const void* dout, int64_t rows, int32_t d,
                                float* delta, hipStream_t st) {
  const int64_t threads = rows * (d / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (d == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, grid, dim3(256), 0, st, (const bf16*)out, (const bf16*)dout, rows, delta);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, grid, dim3(256), 0, st, (const bf16*)out, (const bf16*)dout, rows, delta);
  return hipGetLastError();
}

}  // namespace ra

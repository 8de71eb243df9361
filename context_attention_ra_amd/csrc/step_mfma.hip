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
// * A workgroup is eight waves of 32 query rows (256 rows). Each K or V
//   fragment a wave reads from LDS feeds one MFMA; on gfx950 the transposed
//   LDS read of V runs at about half the rate of a plain 16-byte read.
// * Keys stream through a kStages-deep LDS ring in tiles of kBK rows, fetched
//   by bounds-checked buffer loads that write LDS directly (no staging
//   registers; rows past the block read as zero). A tile is requested about
//   three slots before it is consumed and waited for only just before, so
//   global latency hides behind several slots.
// * LDS holds each tile column-major in 16-byte columns; one load instruction
//   fills a 1 KiB run (one or two columns), runs padded to 1088 bytes. Both the
//   16-byte K reads and the transposed V reads are then free of bank
//   conflicts, and every LDS address is a per-lane base plus an immediate.
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   the 32x32 accumulator layout gives every lane one query column and 16 of
//   each 32 keys, so a row maximum is an in-lane reduction plus one 32-lane
//   swap (v_permlane32_swap), and the per-query rescale factor is a lane scalar.
// * Ping-pong: the two halves of the workgroup (one wave of each on every
//   SIMD) alternate, one slot apart, between a matrix phase (scores of tile
//   n+1 and PV of tile n) and a vector phase (mask, row maximum, rescale and
//   exponentials), so one wave feeds the matrix core while the other computes
//   exponentials; a workgroup barrier ends every slot.
// * The probabilities stay in registers as the B operand of O^T += V^T P^T.
//   The key order inside each 16-key MFMA slice is permuted to match the
//   accumulator layout; the matching V^T operand is read with the gfx950
//   transposing LDS load ds_read_b64_tr_b16, so P never leaves registers.
// * The running maximum only moves when a tile's maximum exceeds it by more
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

constexpr int kWaves = 8;               // waves per workgroup
constexpr int kQB = 1;                  // 32-row query blocks per wave
constexpr int kBK = 64;                 // key rows per tile (32 or 64)
constexpr int kStages = 4;              // LDS ring depth
constexpr int kAhead = 3;               // LDS operands read ahead of their MFMA
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kQB * kWaves;  // query rows per workgroup
constexpr int kNST = kBK / 32;          // 32-key halves per tile
constexpr int kRun = 1088;              // LDS bytes per 1 KiB load run, padded
constexpr float kTau = 8.0f;            // lazy-rescale threshold, log2 units
static_assert(kBK == 32 || kBK == 64, "tile of 32 or 64 keys");

template <int D>
struct Lay {
  static constexpr int CPR = D / 8;               // 16-byte columns per row
  static constexpr int COLS_PER_RUN = 64 / kBK;   // columns one load instruction fills
  static constexpr int NRUN = CPR / COLS_PER_RUN; // runs per tensor tile
  static constexpr int TBYTES = NRUN * kRun;      // one tensor's tile in LDS
  static constexpr int STAGE = 2 * TBYTES;        // K tile then V tile
  static constexpr int RUNS_PER_WAVE = NRUN / kWaves;
  static_assert(RUNS_PER_WAVE >= 1 && NRUN % kWaves == 0, "runs must split evenly over waves");
  static_assert(NRUN % 4 == 0, "layout assumes at least four runs");
  // byte offset of (row, column) inside a tensor tile
  static constexpr int at(int row, int col) { return (col % NRUN) * kRun + (col / NRUN) * 16 * kBK + 16 * row; }
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

// 16 bytes per lane from a bounds-checked buffer straight into LDS at
// m0 + 16*lane (gfx950 buffer_load_dwordx4 ... lds). Written as inline asm so
// that the compiler does not treat these loads as pending LDS writes: it would
// otherwise wait for every one of them before each transposed LDS read. The
// kernel orders them itself with explicit vmcnt waits before its barriers.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, const char* lds, int voff,
                                           int soff) {
  const unsigned m0 = (unsigned)(size_t)(const lds_char*)lds;
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs), "s"(soff), "{m0}"(m0)
               : "memory");
}

__device__ __forceinline__ bf16x8 lds_b128(const char* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ bf16x4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// s_waitcnt encodings (gfx9): wait until at most N vector-memory ops are pending
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int D, bool CAUSAL, bool FUSED>
__global__ __launch_bounds__(kThreads, 1) void step_mfma_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    int32_t nb, int32_t Lq, int32_t Lk, DevSegs qs, DevSegs ks, float c_log2, int32_t init,
    float* __restrict__ Oacc, float* __restrict__ Mst, float* __restrict__ Lst,
    bf16* __restrict__ Out, float* __restrict__ Lse, int32_t nqt, int32_t per_xcd) {
  using L = Lay<D>;
  constexpr int KS = D / 16;  // k-steps of the score MFMA
  constexpr int DT = D / 32;  // 32-wide output tiles
  constexpr int NDMA = 2 * L::RUNS_PER_WAVE;  // load instructions per wave per tile
  __shared__ __attribute__((aligned(16))) char smem[kStages * L::STAGE];

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

  // this wave's query rows: block b covers rows w_r0 + 32b .. +31
  const int32_t w_r0 = qt0 + 32 * kQB * w;
  int32_t qrow[kQB], qpos[kQB];
  bool qvalid[kQB];
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    qrow[b] = w_r0 + 32 * b + l32;
    qvalid[b] = qrow[b] < Lq;
    qpos[b] = seg_pos(qs, qvalid[b] ? qrow[b] : Lq - 1);
  }

  const int32_t wg_r1 = min(qt0 + kBQ, Lq);
  int32_t wg_qlo, wg_qhi;
  seg_range(qs, qt0, wg_r1, wg_qlo, wg_qhi);
  const bool wave_active = w_r0 < Lq;
  int32_t w_qlo = 0, w_qhi = -1;
  if (wave_active) seg_range(qs, w_r0, min(w_r0 + 32 * kQB, Lq), w_qlo, w_qhi);

  // ---- key rows this workgroup can see: at most two row ranges
  int32_t ra0 = 0, rb0 = Lk, ra1 = 0, rb1 = 0;
  if (CAUSAL) {
    auto vis = [&](int32_t start, int32_t n) {
      int32_t x = wg_qhi - start + 1;
      return x < 0 ? 0 : (x > n ? n : x);
    };
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
  auto tile_kt0 = [&](int32_t n) { return (n < n0 ? t0a + n : t1a + (n - n0)) * kBK; };

  // ---- a query tile that sees no key of this block keeps its state: no
  // loads and no stores, except that a first step stores the empty state
  // (and a fused call the empty output: zeros, lse -inf)
  if (ntiles == 0) {
    if ((!FUSED && !init) || !wave_active) return;
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      if (!qvalid[b]) continue;
      const size_t r = (size_t)prob * Lq + qrow[b];
      if (FUSED) {
        bf16* op = Out + qbase + (size_t)qrow[b] * D + 4 * h;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) *(bf16x4*)(op + 32 * t + 8 * i) = bf16x4{};
        if (Lse && h == 0) Lse[r] = kNegInf;
      } else {
        float* op = Oacc + qbase + (size_t)qrow[b] * D + 4 * h;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) *(f32x4*)(op + 32 * t + 8 * i) = f32x4{};
        if (h == 0) {
          Mst[r] = kNegInf;
          Lst[r] = 0.f;
        }
      }
    }
    return;
  }

  // ---- K/V tiles: bounds-checked buffer loads straight into LDS. Load run r
  // of a tile holds columns r, r+NRUN, ... of rows 0..kBK-1; lane i brings
  // row i % kBK of column r + NRUN * (i / kBK). A wave owns RUNS_PER_WAVE runs.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + kbase), 0, Lk * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + kbase), 0, Lk * D * 2, 0x00020000);
  auto fetch = [&](int32_t n, int stage) {
    const int32_t soff = tile_kt0(n) * D * 2;
    char* sb = smem + stage * L::STAGE;
#pragma unroll
    for (int i = 0; i < L::RUNS_PER_WAVE; ++i) {
      const int r = w * L::RUNS_PER_WAVE + i;
      const int voff = (lane % kBK) * D * 2 + 16 * (r + L::NRUN * (lane / kBK));
      load_lds16(krs, sb + r * kRun, voff, soff);
      load_lds16(vrs, sb + L::TBYTES + r * kRun, voff, soff);
    }
  };

  // the first tiles are requested before the Q and state loads
#pragma unroll
  for (int i = 0; i < kStages; ++i)
    if (ntiles > i) fetch(i, i);

  // ---- query fragments: B operand of S^T = K Q^T (lane: query l32, d 16ks+8h..+8)
  bf16x8 qf[kQB][KS];
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    const bf16* qp = Q + qbase + (size_t)(qvalid[b] ? qrow[b] : Lq - 1) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[b][s] = *(const bf16x8*)(qp + 16 * s);
  }

  // ---- running state: O^T accumulators (lane: query l32, d 32dt+8i+4h+j)
  f32x16 o[kQB][DT];
  float mu[kQB];        // reference value in log2 units of the weights
  float lpart[kQB][2];  // this lane's share of the row sum, two partial sums
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
#pragma unroll
    for (int t = 0; t < DT; ++t) o[b][t] = f32x16{};
    mu[b] = kNegInf;
    lpart[b][0] = lpart[b][1] = 0.f;
    if (!FUSED && !init && qvalid[b]) {
      const float* op = Oacc + qbase + (size_t)qrow[b] * D + 4 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 x = *(const f32x4*)(op + 32 * t + 8 * i);
          o[b][t][4 * i + 0] = x[0];
          o[b][t][4 * i + 1] = x[1];
          o[b][t][4 * i + 2] = x[2];
          o[b][t][4 * i + 3] = x[3];
        }
      const size_t r = (size_t)prob * Lq + qrow[b];
      mu[b] = Mst[r] * kLog2e;
      lpart[b][0] = h == 0 ? Lst[r] : 0.f;
    }
  }

  // per-lane LDS read bases within a stage; the rest are immediate offsets.
  // K (A operand): row 32st+l32, column 2ksi+h.
  // V^T (transposed reads): row 16kc+4(g>>1)+rr(+8), columns 32t+16(g&1)+4cc..+3
  // (16-byte column 4t+2(g&1)+(cc>>1), byte 8(cc&1)).
  const int g = lane >> 4, jj = lane & 15, rr = jj >> 2, cc = jj & 3;
  const int kread = L::at(l32, h);
  const int vread = L::TBYTES + L::at(4 * (g >> 1) + rr, 2 * (g & 1) + (cc >> 1)) + 8 * (cc & 1);

  // per-tile facts for this wave
  struct TileInfo {
    int32_t kt0;
    bool mask;       // element mask needed (diagonal, ragged tail, or fully after the queries)
    bool straddle;   // tile crosses the K segment boundary
    int32_t kpos0;   // global position of the tile's first row (if not straddling)
  };
  auto tile_info = [&](int32_t n) {
    TileInfo ti;
    ti.kt0 = tile_kt0(n);
    const int32_t kend = min(ti.kt0 + kBK, Lk);
    ti.mask = ti.kt0 + kBK > Lk;
    ti.straddle = ti.kt0 < ks.len0 && kend > ks.len0;
    ti.kpos0 = seg_pos(ks, ti.kt0);
    if (CAUSAL) {
      int32_t klo, khi;
      seg_range(ks, ti.kt0, kend, klo, khi);
      (void)klo;
      if (khi > w_qlo) ti.mask = true;
    }
    return ti;
  };

  typedef f32x16 Scores[kQB][kNST];  // [query block][32-key part of the tile]

  auto scores = [&](int stage, Scores& s) {
    const char* kb = smem + stage * L::STAGE + kread;
#pragma unroll
    for (int b = 0; b < kQB; ++b)
#pragma unroll
      for (int st = 0; st < kNST; ++st) s[b][st] = f32x16{};
#pragma unroll
    for (int ksi = 0; ksi < KS; ++ksi)
#pragma unroll
      for (int st = 0; st < kNST; ++st) {
        // rows 32st+l32, column 2ksi+h: the lane base covers l32 and h
        const bf16x8 kf = lds_b128(kb + L::at(32 * st, 2 * ksi));
#pragma unroll
        for (int b = 0; b < kQB; ++b)
          s[b][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[b][ksi], s[b][st], 0, 0, 0);
      }
  };

  auto apply_mask = [&](const TileInfo& ti, Scores& s) {
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      if (!ti.straddle) {
        // key offset e in the tile is visible iff e <= lim
        int32_t lim = Lk - 1 - ti.kt0;
        if (CAUSAL) lim = min(lim, qpos[b] - ti.kpos0);
#pragma unroll
        for (int st = 0; st < kNST; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int e = 32 * st + 8 * i + 4 * h + j;
              s[b][st][4 * i + j] = e > lim ? kNegInf : s[b][st][4 * i + j];
            }
      } else {
#pragma unroll
        for (int st = 0; st < kNST; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int32_t kr = ti.kt0 + 32 * st + 8 * i + 4 * h + j;
              const bool m = kr >= Lk || (CAUSAL && seg_pos(ks, kr) > qpos[b]);
              s[b][st][4 * i + j] = m ? kNegInf : s[b][st][4 * i + j];
            }
      }
    }
  };

  // row maxima of one tile's scores, log2 units (both lanes of a query agree)
  auto rowmax = [&](const Scores& s, float (&mt)[kQB]) {
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      // 16*kNST values: chains of v_max3, two values per instruction
      float a[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        a[c] = max2_nn(s[b][0][4 * c], s[b][0][4 * c + 1]);
        a[c] = max3_nn(a[c], s[b][0][4 * c + 2], s[b][0][4 * c + 3]);
#pragma unroll
        for (int st = 1; st < kNST; ++st) {
          a[c] = max3_nn(a[c], s[b][st][4 * c], s[b][st][4 * c + 1]);
          a[c] = max3_nn(a[c], s[b][st][4 * c + 2], s[b][st][4 * c + 3]);
        }
      }
      mt[b] = partner32_max(max3_nn(max2_nn(a[0], a[1]), a[2], a[3])) * c_log2;
    }
  };

  // the (rare) rescale of the state when a tile's maximum outgrows the
  // reference value by more than kTau
  auto rescale = [&](const float (&mt)[kQB]) {
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const bool need = mt[b] > mu[b] + kTau;
      if (__builtin_amdgcn_ballot_w64(need)) {
        // lanes keeping their reference (also rows with no visible key yet,
        // mu = -inf) must get exactly 1, not exp2(-inf - -inf)
        const float mnew = need ? mt[b] : mu[b];
        const float alpha = need ? fast_exp2(mu[b] - mnew) : 1.f;
        lpart[b][0] *= alpha;
        lpart[b][1] *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[b][t][r] *= alpha;
        mu[b] = mnew;
      }
    }
  };

  typedef bf16x8 Probs[kQB][2 * kNST];  // [query block][16-key slice]

  // exponentials of one tile into bf16 B operands (and the row-sum shares,
  // summed in fp32 before rounding so that lse keeps full precision)
  auto exps = [&](const Scores& s, Probs& pf) {
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const float mus = mu[b] == kNegInf ? 0.f : mu[b];
#pragma unroll
      for (int st = 0; st < kNST; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(__builtin_fmaf(s[b][st][r], c_log2, -mus));
          lpart[b][r & 1] += pr;
          pf[b][2 * st + r / 8][r % 8] = to_bf16(pr);
        }
    }
  };



  // The matrix phase of one tile in a fixed order: the score MFMAs of the next
  // tile, then the PV MFMAs of this one. Each step's LDS operand is read
  // kAhead steps earlier and scheduling barriers keep that order, so no MFMA
  // waits on a just-issued LDS read.
  Scores sc;
  Probs pf;
  auto mfma_phase = [&](int kstage, int vstage) {
    constexpr int NSC = KS * kNST;      // score steps
    constexpr int NPV = 2 * kNST * DT;  // PV steps
    const char* kb = smem + kstage * L::STAGE + kread;
    const char* vb = smem + vstage * L::STAGE + vread;
#pragma unroll
    for (int b = 0; b < kQB; ++b)
#pragma unroll
      for (int st = 0; st < kNST; ++st) sc[b][st] = f32x16{};
    auto operand = [&](int i) -> bf16x8 {
      if (i < NSC) return lds_b128(kb + L::at(32 * (i % kNST), 2 * (i / kNST)));
      const int j = i - NSC, off = L::at(16 * (j / DT), 4 * (j % DT));
      const bf16x4 va = lds_tr16(vb + off);
      const bf16x4 vbb = lds_tr16(vb + off + 16 * 8);
      return bf16x8{va[0], va[1], va[2], va[3], vbb[0], vbb[1], vbb[2], vbb[3]};
    };
    bf16x8 op[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) op[j] = operand(j);
#pragma unroll
    for (int i = 0; i < NSC + NPV; ++i) {
      const bf16x8 cur = op[i % kAhead];
      if (i < NSC) {
        const int st = i % kNST, ksi = i / kNST;
#pragma unroll
        for (int b = 0; b < kQB; ++b)
          sc[b][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[b][ksi], sc[b][st], 0, 0, 0);
      } else {
        const int j = i - NSC, kc = j / DT, t = j % DT;
#pragma unroll
        for (int b = 0; b < kQB; ++b)
          o[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pf[b][kc], o[b][t], 0, 0, 0);
      }
      if (i + kAhead < NSC + NPV) op[i % kAhead] = operand(i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- ping-pong schedule. The two halves of the workgroup (waves 0..W/2-1
  // and W/2..W-1, one of each on every SIMD) run the same per-tile program
  // shifted by half an iteration: while one wave of a SIMD issues its matrix
  // work (scores of tile n+1 and PV of tile n), the other does its vector
  // work (mask, row maximum, rescale and exponentials of its next tile), so
  // the matrix core always has a wave feeding it. Time advances in slots that
  // end with a workgroup barrier:
  //   group A: slot 0 = start (scores + softmax of tile 0), then slot 2n+1 =
  //            matrix phase n, slot 2n+2 = vector phase n;
  //   group B: the same, one slot later.
  // The matrix phase n reads K of tile n+1 and V of tile n, so tile m is
  // needed from slot 2m-1 and free after slot 2m+2: tile m+kStages is
  // requested at the start of slot 2m+3 into m's stage, and tile n+1 is
  // waited for at the end of slot 2n.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // group B: waves w and w + 4 share a SIMD
  const bool late = w >= kWaves / 2;
  auto vector_phase = [&](int32_t n) {  // softmax of tile n (scores in sc)
    const TileInfo ti = tile_info(n);
    if (ti.mask) apply_mask(ti, sc);
    float mt[kQB];
    rowmax(sc, mt);
    rescale(mt);
    exps(sc, pf);
  };
  const int32_t nslots = ntiles > 0 ? 2 * ntiles + 1 : 0;
  for (int32_t s = 0; s < nslots; ++s) {
    if ((s & 1) && s >= 3) {
      const int32_t m = (s - 3) >> 1;
      if (m + kStages < ntiles) fetch(m + kStages, m % kStages);
    }
    const int32_t a = late ? s - 1 : s;  // this group's own slot number
    if (a == 0) {
      scores(0, sc);
      vector_phase(0);
    } else if (a > 0 && (a & 1)) {
      const int32_t n = (a - 1) >> 1;
      if (n < ntiles) {
        __builtin_amdgcn_s_setprio(1);
        // past the last tile the scores read a stale stage and are never used
        mfma_phase((n + 1) % kStages, n % kStages);
        __builtin_amdgcn_s_setprio(0);
      }
    } else if (a > 0) {
      const int32_t n = (a - 2) >> 1;
      if (n + 1 < ntiles) vector_phase(n + 1);
    }
    if (!(s & 1)) {
      // end of slot 2n: tile n+1 must be in LDS; tiles requested later may
      // stay in flight
      const int32_t n = s >> 1;
      const int32_t latest = min(ntiles - 1, n + kStages - 2);  // requested so far
      const int32_t in_flight = latest - (n + 1);
      if (in_flight >= 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NDMA));
      else if (in_flight == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NDMA));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
  }


  if (!wave_active) return;
#pragma unroll
  for (int b = 0; b < kQB; ++b) {
    const float lsum = partner32_sum(lpart[b][0] + lpart[b][1]);
    if (!qvalid[b]) continue;
    if (FUSED) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      bf16* op = Out + qbase + (size_t)qrow[b] * D + 4 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 y = {to_bf16(o[b][t][4 * i + 0] * inv), to_bf16(o[b][t][4 * i + 1] * inv),
                      to_bf16(o[b][t][4 * i + 2] * inv), to_bf16(o[b][t][4 * i + 3] * inv)};
          *(bf16x4*)(op + 32 * t + 8 * i) = y;
        }
      if (Lse && h == 0)
        Lse[(size_t)prob * Lq + qrow[b]] = lsum > 0.f ? (mu[b] + fast_log2(lsum)) * kLn2 : kNegInf;
    } else {
      float* op = Oacc + qbase + (size_t)qrow[b] * D + 4 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 y = {o[b][t][4 * i + 0], o[b][t][4 * i + 1], o[b][t][4 * i + 2], o[b][t][4 * i + 3]};
          *(f32x4*)(op + 32 * t + 8 * i) = y;
        }
      if (h == 0) {
        const size_t r = (size_t)prob * Lq + qrow[b];
        Mst[r] = mu[b] * kLn2;
        Lst[r] = lsum;
      }
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

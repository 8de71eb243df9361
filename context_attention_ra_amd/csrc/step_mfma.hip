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
// * Work items are (batch*head slice, 256-row query tile). Workgroups are
//   persistent, one per CU: each walks a list of items as one continuous
//   stream of 64-key K/V tiles, so the loads of the next item's first tiles,
//   and its queries, are in flight while the current item finishes. A
//   workgroup that ran one item and exited would wait for its queries, state
//   and first tiles with the CU idle, and all CUs would do so at the same
//   time, contending for HBM.
// * Eight waves of 32 query rows. Keys stream through a 4-deep LDS ring,
//   fetched by bounds-checked buffer loads that write LDS directly (no
//   staging registers; rows past the block read as zero).
// * LDS holds each tile column-major in 16-byte columns; one load instruction
//   fills a 1 KiB run, runs padded to 1088 bytes. Both the 16-byte K reads and
//   the transposed V reads are then free of bank conflicts, and every LDS
//   address is a per-lane base plus an immediate.
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   the 32x32 accumulator layout gives every lane one query column and 16 of
//   each 32 keys, so a row maximum is an in-lane reduction plus one 32-lane
//   swap (v_permlane32_swap), and the per-query rescale factor is a lane scalar.
// * The probabilities stay in registers as the B operand of O^T += V^T P^T.
//   The key order inside each 16-key MFMA slice is permuted to match the
//   accumulator layout; the matching V^T operand is read with the gfx950
//   transposing LDS load ds_read_b64_tr_b16, so P never leaves registers.
// * Ping-pong: the two halves of the workgroup (one wave of each on every
//   SIMD) alternate between a matrix phase and a vector phase, so one wave
//   feeds the matrix core while the other computes exponentials.
// * The running maximum only moves when a tile's maximum exceeds it by more
//   than 2^8 in weight (lazy rescale); the state stays exact because O and l
//   are always expressed relative to the same reference value m. The tile's
//   row maxima are only formed when a lane's share of the tile sum shows that
//   such a move may be due.
// * Tiles whose keys all lie after the last query (causal) are never loaded;
//   tiles straddling the diagonal, and ragged tails, are masked per element.
// * Each of the 8 XCDs owns a contiguous range of items (whole slices), so a
//   slice's K/V block stays in that XCD's L2; within a slice the query tiles
//   at the end (the heaviest under a causal mask and the zigzag split) come
//   first, dealt to the XCD's workgroups in snake order to even out the work.

#include "ra_device.h"
#include "ra_launch.h"

namespace ra {
namespace {

constexpr int kWaves = 8;               // waves per workgroup
constexpr int kBK = 64;                 // key rows per tile
constexpr int kStages = 4;              // LDS ring depth
constexpr int kAhead = 3;               // LDS operands read ahead of their MFMA
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;        // query rows per work item
constexpr int kNST = kBK / 32;          // 32-key halves per tile
constexpr int kRun = 1088;              // LDS bytes per 1 KiB load run, padded
constexpr float kTau = 8.0f;            // lazy-rescale threshold, log2 units
// A weight above 2^kTau (a tile maximum more than kTau above the reference,
// when the rescale rule moves it) makes its lane's share of the tile sum
// exceed 2^kTau; while every lane's share stays within it, no rescale is due
// and the row maximum is not needed.
constexpr float kSumMax = 256.0f;       // 2^kTau
constexpr int kXcds = 8;

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

// The kernel body is written as lambdas; with two copies of the schedule the
// inliner would otherwise turn some of them into calls with stack frames.
#define RA_INLINE __attribute__((always_inline))

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// One work item: query tile qt0.. of slice prob, the K/V slice kvp it reads,
// and the K/V tiles it sees (two runs of tile indices: t0a.. (n0 tiles) and
// t1a.. (the rest)).
struct Item {
  int32_t prob, kvp, qt0, n0, t0a, t1a, ntiles;
};

// A position in a workgroup's stream of tiles: item number i of the
// workgroup, the item, and the stream indices [g0, g1) of its tiles.
struct Cursor {
  int32_t i, g0, g1;
  Item it;
};

// What a launch reads and writes besides the queries and the block:
//   kStep   running state in (unless init) and out;
//   kAttend no state (a single block, init implied), final output out;
//   kLast   running state in (unless init), final output out: the last ring
//           step with the finalize folded in (the state is left unchanged).
enum Mode { kStep = 0, kAttend = 1, kLast = 2 };

#define RA_STEP_PARAMS                                                                        \
  const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,         \
      int32_t nb, int32_t Lq, int32_t Lk, DevSegs qs, DevSegs ks, float c_log2, int32_t init, \
      float *__restrict__ Oacc, float *__restrict__ Mst, float *__restrict__ Lst,             \
      bf16 *__restrict__ Out, float *__restrict__ Lse, int32_t nqt, int32_t per_xcd,          \
      int32_t nwg_x, int32_t group
#define RA_STEP_ARGS \
  Q, K, V, nb, Lq, Lk, qs, ks, c_log2, init, Oacc, Mst, Lst, Out, Lse, nqt, per_xcd, nwg_x, group

template <int D, bool CAUSAL, int MODE>
__device__ __forceinline__ void step_mfma_body(RA_STEP_PARAMS) {
  using L = Lay<D>;
  constexpr int KS = D / 16;  // k-steps of the score MFMA
  constexpr int DT = D / 32;  // 32-wide output tiles
  constexpr int NDMA = 2 * L::RUNS_PER_WAVE;  // load instructions per wave per tile
  __shared__ __attribute__((aligned(16))) char smem[kStages * L::STAGE];

  constexpr bool FUSED = MODE != kStep;  // writes the final output
  const bool state_in = MODE != kAttend && !init;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;

  // ---- this workgroup's items: XCD x owns logical items [x*per_xcd, ...);
  // its nwg_x workgroups take them round by round, in snake order
  const int32_t total = nb * nqt;
  const int32_t xcd = blockIdx.x % kXcds, wj = blockIdx.x / kXcds;
  const int32_t x_lo = xcd * per_xcd;
  const int32_t x_cnt = max(0, min(per_xcd, total - x_lo));
  const int32_t nrounds = (x_cnt + nwg_x - 1) / nwg_x;
  auto item_logical = [&](int32_t i) RA_INLINE -> int32_t {
    const int32_t pos = (i & 1) ? (i + 1) * nwg_x - 1 - wj : i * nwg_x + wj;
    return pos < x_cnt ? x_lo + pos : -1;
  };
  auto decode = [&](int32_t logical) RA_INLINE {
    Item it;
    it.prob = logical / nqt;
    // query heads h*group .. h*group+group-1 of a batch share K/V head h;
    // slices are batch-major, so the K/V slice is the query slice / group
    it.kvp = it.prob / group;
    const int32_t qtile = nqt - 1 - (logical - it.prob * nqt);
    it.qt0 = qtile * kBQ;
    // key rows this item can see: at most two row ranges
    int32_t ra0 = 0, rb0 = Lk, ra1 = 0, rb1 = 0;
    if (CAUSAL) {
      int32_t qlo, qhi;
      seg_range(qs, it.qt0, min(it.qt0 + kBQ, Lq), qlo, qhi);
      (void)qlo;
      auto vis = [&](int32_t start, int32_t n) RA_INLINE {
        int32_t x = qhi - start + 1;
        return x < 0 ? 0 : (x > n ? n : x);
      };
      rb0 = vis(ks.start0, ks.len0);
      ra1 = ks.len0;
      rb1 = ks.len0 + (ks.len > ks.len0 ? vis(ks.start1, ks.len - ks.len0) : 0);
    }
    it.t0a = ra0 / kBK;
    const int32_t t0b = (rb0 + kBK - 1) / kBK;
    it.n0 = rb0 > ra0 ? t0b - it.t0a : 0;
    it.t1a = ra1 / kBK;
    const int32_t t1b = (rb1 + kBK - 1) / kBK;
    if (it.n0 > 0 && it.t1a < t0b) it.t1a = t0b;
    const int32_t n1 = rb1 > ra1 && t1b > it.t1a ? t1b - it.t1a : 0;
    it.ntiles = it.n0 + n1;
    return it;
  };
  auto tile_kt0 = [&](const Item& it, int32_t n) RA_INLINE {
    return (n < it.n0 ? it.t0a + n : it.t1a + (n - it.n0)) * kBK;
  };
  // the next item with at least one tile; g0 continues the stream
  auto advance = [&](Cursor& c) RA_INLINE {
    c.g0 = c.g1;
    for (++c.i; c.i < nrounds; ++c.i) {
      const int32_t lg = item_logical(c.i);
      if (lg < 0) continue;
      c.it = decode(lg);
      if (c.it.ntiles > 0) break;
    }
    c.g1 = c.g0 + (c.i < nrounds ? c.it.ntiles : 0);
  };

  // ---- items that see no key of the block keep their state: no loads and
  // no stores, except that a first step stores the empty state (and a fused
  // call the empty output: zeros, lse -inf; a last step with a state in
  // finalizes that state once the stream is done). NT counts the stream's tiles.
  int32_t NT = 0;
  for (int32_t i = 0; i < nrounds; ++i) {
    const int32_t lg = item_logical(i);
    if (lg < 0) continue;
    const Item it = decode(lg);
    NT += it.ntiles;
    if (it.ntiles > 0 || state_in) continue;
    const int32_t qrow = it.qt0 + 32 * w + l32;
    if (qrow >= Lq) continue;
    const size_t r = (size_t)it.prob * Lq + qrow;
    if (FUSED) {
      bf16* op = Out + r * D + 4 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) *(bf16x4*)(op + 32 * t + 8 * i4) = bf16x4{};
      if (Lse && h == 0) Lse[r] = kNegInf;
    } else {
      float* op = Oacc + r * D + 4 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) *(f32x4*)(op + 32 * t + 8 * i4) = f32x4{};
      if (h == 0) {
        Mst[r] = kNegInf;
        Lst[r] = 0.f;
      }
    }
  }
  // the output of the rows whose items see no key of a last block: the
  // state they carry in, normalised (as the separate finalize does)
  auto finalize_empty_items = [&]() RA_INLINE {
    for (int32_t i = 0; i < nrounds; ++i) {
      const int32_t lg = item_logical(i);
      if (lg < 0) continue;
      const Item it = decode(lg);
      if (it.ntiles > 0) continue;
      const int32_t qrow = it.qt0 + 32 * w + l32;
      if (qrow >= Lq) continue;
      const size_t r = (size_t)it.prob * Lq + qrow;
      const float l = Lst[r];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float* ip = Oacc + r * D + 4 * h;
      bf16* op = Out + r * D + 4 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 x = *(const f32x4*)(ip + 32 * t + 8 * i4);
          *(bf16x4*)(op + 32 * t + 8 * i4) =
              bf16x4{to_bf16(x[0] * inv), to_bf16(x[1] * inv), to_bf16(x[2] * inv), to_bf16(x[3] * inv)};
        }
      if (Lse && h == 0) Lse[r] = l > 0.f ? Mst[r] + fast_log2(l) * kLn2 : kNegInf;
    }
  };
  if (NT == 0) {
    if (MODE == kLast && state_in) finalize_empty_items();
    return;
  }

  Cursor first;
  first.i = -1;
  first.g1 = 0;
  advance(first);

  // ---- K/V tiles of the stream: tile g goes to stage g % kStages. Load run
  // r of a tile holds columns r, r+NRUN, ... of rows 0..kBK-1; lane i brings
  // row i % kBK of column r + NRUN * (i / kBK). A wave owns RUNS_PER_WAVE runs.
  Cursor fc = first;  // item of the next tile to request
  int32_t fg = 0;     // stream index of the next tile to request
  auto fetch_next = [&]() RA_INLINE {
    if (fg == fc.g1) advance(fc);
    const size_t kbase = (size_t)fc.it.kvp * Lk * D;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + kbase), 0, Lk * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + kbase), 0, Lk * D * 2, 0x00020000);
    const int32_t soff = tile_kt0(fc.it, fg - fc.g0) * D * 2;
    char* sb = smem + (fg % kStages) * L::STAGE;
#pragma unroll
    for (int i = 0; i < L::RUNS_PER_WAVE; ++i) {
      const int r = w * L::RUNS_PER_WAVE + i;
      const int voff = (lane % kBK) * D * 2 + 16 * (r + L::NRUN * (lane / kBK));
      load_lds16(krs, sb + r * kRun, voff, soff);
      load_lds16(vrs, sb + L::TBYTES + r * kRun, voff, soff);
    }
    ++fg;
  };

  // the first tiles are requested before the query and state loads
#pragma unroll
  for (int i = 0; i < kStages; ++i)
    if (i < NT) fetch_next();

  // ---- query fragments: B operand of S^T = K Q^T (lane: query l32, d 16ks+8h..+8)
  bf16x8 qf[KS];
  auto load_q = [&](const Item& it) RA_INLINE {
    const int32_t row = min(it.qt0 + 32 * w + l32, Lq - 1);
    // in the non-final steps the lane's part as a 32-bit offset (a slice of Q
    // is under 2 GiB), one VGPR instead of a 64-bit lane pointer kept across
    // the item loop; the other modes keep the form they were tuned with
    const bf16* qp = MODE == kStep ? (Q + (size_t)it.prob * Lq * D) + (row * D + 8 * h)
                                   : Q + ((size_t)it.prob * Lq + row) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
  };
  load_q(first.it);

  // ---- running state of the current item: O^T accumulators (lane: query
  // l32, d 32dt+8i+4h+j), reference value mu (log2 units), row-sum shares
  f32x16 o[DT];
  float mu;
  float lpart[2];
  Cursor cc = first;  // item whose state is in registers
  int32_t qrow, qpos, w_qlo;
  bool qvalid, wave_active;
  auto begin_item = [&]() RA_INLINE {
    const Item& it = cc.it;
    const int32_t w_r0 = it.qt0 + 32 * w;
    qrow = w_r0 + l32;
    qvalid = qrow < Lq;
    qpos = seg_pos(qs, qvalid ? qrow : Lq - 1);
    wave_active = w_r0 < Lq;
    int32_t w_qhi;
    w_qlo = 0;
    if (wave_active) seg_range(qs, w_r0, min(w_r0 + 32, Lq), w_qlo, w_qhi);
    w_qlo = __builtin_amdgcn_readfirstlane(w_qlo);  // the same in every lane
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = f32x16{};
    mu = kNegInf;
    lpart[0] = lpart[1] = 0.f;
    if (state_in && qvalid) {
      const size_t r = (size_t)it.prob * Lq + qrow;
      const float* op = Oacc + r * D + 4 * h;
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
      mu = Mst[r] * kLog2e;
      lpart[0] = h == 0 ? Lst[r] : 0.f;
    }
  };
  auto end_item = [&]() RA_INLINE {
    const float lsum = partner32_sum(lpart[0] + lpart[1]);
    if (!wave_active) return;
    const size_t r = (size_t)cc.it.prob * Lq + qrow;
    if (FUSED) {
      // lane h holds d = 32t + 8i + 4h + (0..3) of its query; one 32-lane swap
      // per pair of i gives it 8 consecutive values instead, so each store
      // writes 16 whole bytes (d = 32t + 16p + 8h ..) of the row. The swap
      // needs both lanes of a row, which are valid or not together.
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      bf16* op = Out + r * D + 8 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const bf16x4 ya = {to_bf16(o[t][8 * pp + 0] * inv), to_bf16(o[t][8 * pp + 1] * inv),
                             to_bf16(o[t][8 * pp + 2] * inv), to_bf16(o[t][8 * pp + 3] * inv)};
          const bf16x4 yb = {to_bf16(o[t][8 * pp + 4] * inv), to_bf16(o[t][8 * pp + 5] * inv),
                             to_bf16(o[t][8 * pp + 6] * inv), to_bf16(o[t][8 * pp + 7] * inv)};
          const u32x2 a = __builtin_bit_cast(u32x2, ya), b = __builtin_bit_cast(u32x2, yb);
          const auto s0 = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
          const u32x4 chunk = {s0[0], s1[0], s0[1], s1[1]};
          if (qvalid) *(u32x4*)(op + 32 * t + 16 * pp) = chunk;
        }
      if (qvalid && Lse && h == 0) Lse[r] = lsum > 0.f ? (mu + fast_log2(lsum)) * kLn2 : kNegInf;
    } else {
      if (!qvalid) return;
      float* op = Oacc + r * D + 4 * h;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 y = {o[t][4 * i + 0], o[t][4 * i + 1], o[t][4 * i + 2], o[t][4 * i + 3]};
          *(f32x4*)(op + 32 * t + 8 * i) = y;
        }
      if (h == 0) {
        Mst[r] = mu * kLn2;
        Lst[r] = lsum;
      }
    }
  };
  begin_item();

  // per-lane LDS read bases within a stage; the rest are immediate offsets.
  // K (A operand): row 32st+l32, column 2ksi+h.
  // V^T (transposed reads): row 16kc+4(g>>1)+rr(+8), columns 32t+16(g&1)+4cc..+3
  // (16-byte column 4t+2(g&1)+(c4>>1), byte 8(c4&1)).
  const int g = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  const int kread = L::at(l32, h);
  const int vread = L::TBYTES + L::at(4 * (g >> 1) + rr, 2 * (g & 1) + (c4 >> 1)) + 8 * (c4 & 1);

  // per-tile facts for this wave (stream tile m of the current item)
  struct TileInfo {
    int32_t kt0;
    bool mask;       // element mask needed (diagonal, ragged tail, or fully after the queries)
    bool straddle;   // tile crosses the K segment boundary
    int32_t kpos0;   // global position of the tile's first row (if not straddling)
  };
  auto tile_info = [&](int32_t m) RA_INLINE {
    TileInfo ti;
    ti.kt0 = tile_kt0(cc.it, m - cc.g0);
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

  typedef f32x16 Scores[kNST];   // [32-key part of the tile]
  typedef bf16x8 Probs[2 * kNST];  // [16-key slice]
  Scores sc;
  Probs pf;
  Scores pw;  // the weights in fp32, rounded to pf inside the matrix phase

  auto scores = [&](int stage) RA_INLINE {
    const char* kb = smem + stage * L::STAGE + kread;
#pragma unroll
    for (int st = 0; st < kNST; ++st) sc[st] = f32x16{};
#pragma unroll
    for (int ksi = 0; ksi < KS; ++ksi)
#pragma unroll
      for (int st = 0; st < kNST; ++st) {
        // rows 32st+l32, column 2ksi+h: the lane base covers l32 and h
        const bf16x8 kf = lds_b128(kb + L::at(32 * st, 2 * ksi));
        sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ksi], sc[st], 0, 0, 0);
      }
  };

  auto apply_mask = [&](const TileInfo& ti) RA_INLINE {
    if (!ti.straddle) {
      // key offset e in the tile is visible iff e <= lim
      int32_t lim = Lk - 1 - ti.kt0;
      if (CAUSAL) lim = min(lim, qpos - ti.kpos0);
      // compare the lane-independent part of e with a per-lane limit, so that
      // the 32 offsets are immediates rather than registers
      const int32_t limh = lim - 4 * h;
      // in place (each select is tied to its score register), so that the
      // masked and unmasked paths leave the scores in the same registers and
      // the unmasked path needs no copies
      const float ninf = kNegInf;
#pragma unroll
      for (int st = 0; st < kNST; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 32 * st + 8 * i + j;  // + 4h
            asm volatile("v_cmp_lt_i32 vcc, %2, %3\n\tv_cndmask_b32 %0, %0, %1, vcc"
                         : "+v"(sc[st][4 * i + j])
                         : "v"(ninf), "v"(limh), "n"(e)
                         : "vcc");
          }
    } else {
      // only the tile holding the segment boundary straddles it; an opaque
      // copy of its start keeps the compiler from computing this tile's 32
      // masks ahead for every item and holding them in scalar registers
      int32_t kt0 = ti.kt0;
      asm volatile("" : "+v"(kt0));
#pragma unroll
      for (int st = 0; st < kNST; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int32_t kr = kt0 + 32 * st + 8 * i + 4 * h + j;
            const bool m = kr >= Lk || (CAUSAL && seg_pos(ks, kr) > qpos);
            sc[st][4 * i + j] = m ? kNegInf : sc[st][4 * i + j];
          }
    }
  };

  // row maximum of one tile's scores, log2 units (both lanes of a query agree)
  auto rowmax = [&]() RA_INLINE {
    // 16*kNST values: chains of v_max3, two values per instruction
    float a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[c] = max2_nn(sc[0][4 * c], sc[0][4 * c + 1]);
      a[c] = max3_nn(a[c], sc[0][4 * c + 2], sc[0][4 * c + 3]);
#pragma unroll
      for (int st = 1; st < kNST; ++st) {
        a[c] = max3_nn(a[c], sc[st][4 * c], sc[st][4 * c + 1]);
        a[c] = max3_nn(a[c], sc[st][4 * c + 2], sc[st][4 * c + 3]);
      }
    }
    return partner32_max(max3_nn(max2_nn(a[0], a[1]), a[2], a[3])) * c_log2;
  };

  // the (rare) rescale of the state when a tile's maximum outgrows the
  // reference value by more than kTau
  auto rescale = [&](float mt) RA_INLINE {
    const bool need = mt > mu + kTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // lanes keeping their reference (also rows with no visible key yet,
      // mu = -inf) must get exactly 1, not exp2(-inf - -inf)
      const float mnew = need ? mt : mu;
      const float alpha = need ? fast_exp2(mu - mnew) : 1.f;
      lpart[0] *= alpha;
      lpart[1] *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      mu = mnew;
    }
  };

  // exponentials of one tile against the current reference, into the fp32
  // weights pw (rounded to the bf16 B operands pf in the next matrix phase);
  // tsum gets this lane's share of the tile's row sum (in fp32, before the
  // rounding, so that lse keeps full precision)
  auto exps = [&](float& tsum) RA_INLINE {
    const float mus = mu == kNegInf ? 0.f : mu;
    float pr[16 * kNST];
#pragma unroll
    for (int st = 0; st < kNST; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[16 * st + r] = fast_exp2(__builtin_fmaf(sc[st][r], c_log2, -mus));
        pw[st][r] = pr[16 * st + r];
      }
    // pairwise sum: five dependent adds instead of a chain of sixteen
#pragma unroll
    for (int n = 8 * kNST; n >= 1; n /= 2)
#pragma unroll
      for (int i = 0; i < n; ++i) pr[i] = pr[2 * i] + pr[2 * i + 1];
    tsum = pr[0];
  };

  // The matrix phase of one tile in a fixed order: the score MFMAs of the next
  // tile, then the PV MFMAs of this one. Each step's LDS operand is read
  // kAhead steps earlier and scheduling barriers keep that order, so no MFMA
  // waits on a just-issued LDS read.
  auto mfma_phase = [&](int kstage, int vstage) RA_INLINE {
    constexpr int NSC = KS * kNST;      // score steps
    constexpr int NPV = 2 * kNST * DT;  // PV steps
    const char* kb = smem + kstage * L::STAGE + kread;
    const char* vb = smem + vstage * L::STAGE + vread;
#pragma unroll
    for (int st = 0; st < kNST; ++st) sc[st] = f32x16{};
    auto operand = [&](int i) RA_INLINE -> bf16x8 {
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
        sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[ksi], sc[st], 0, 0, 0);
      } else {
        const int j = i - NSC, kc = j / DT, t = j % DT;
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pf[kc], o[t], 0, 0, 0);
      }
      if (i + kAhead < NSC + NPV) op[i % kAhead] = operand(i + kAhead);
      // the bf16 weights of slice kc, rounded between the first score products
      // (the matrix wave has issue slots to spare there; the vector phase
      // of the other wave does not)
      if (i >= 1 && i < 1 + 2 * kNST) {
        const int kc = i - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[kc][e] = to_bf16(pw[kc / 2][8 * (kc % 2) + e]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // softmax of stream tile m of the current item (scores in sc). The weights
  // are taken against the current reference first: the row maxima are only
  // formed, and the rescale rule applied, when some lane's share of the tile
  // sum exceeds kSumMax (or is not finite), or a row that had no visible key
  // yet meets one; then the weights are taken again. The row maximum is a
  // fifth of the vector work, and this way it is skipped on almost every tile.
  auto vector_phase = [&](int32_t m) RA_INLINE {
    const TileInfo ti = tile_info(m);
    if (ti.mask) apply_mask(ti);
    float tsum;
    exps(tsum);
    // bitwise, so that the test is two compares and lane-mask logic, not branches
    const bool check = (!(tsum <= kSumMax)) | ((mu == kNegInf) & (tsum > 0.f));
    if (__builtin_amdgcn_ballot_w64(check)) {
      rescale(rowmax());
      exps(tsum);
    }
    lpart[0] += tsum;
    // the weights are complete here: without this use the compiler sinks part
    // of the exponentials and conversions past the barrier into the other
    // phase, where the same wave then issues them between its products
    asm volatile("" ::"v"(pw[0]), "v"(pw[1]), "v"(lpart[0]), "v"(lpart[1]));
  };

  // ---- ping-pong schedule, one item at a time. The two halves of the
  // workgroup (waves 0..3 and 4..7, one of each on every SIMD) run the same
  // per-tile program shifted by one slot: while one wave of a SIMD issues its
  // matrix work (scores of tile n+1 and PV of tile n), the other does its
  // vector work (mask, row maximum, rescale and exponentials of its next
  // tile). Time advances in slots that end with a workgroup barrier:
  //   group A: slot 0 = start (scores + softmax of tile 0), then slot 2n+1 =
  //            matrix phase n, slot 2n+2 = vector phase of tile n+1;
  //   group B: the same, one slot later.
  // Tiles are numbered along the stream (g = g0 + n) and tile g sits in
  // stage g % kStages. The matrix phase n reads K of tile n+1 and V of tile n,
  // so tile g is needed from slot 2n-1 and free after slot 2n+2 of its item:
  // at the start of odd slot 2m+3 (m >= -1) the stream tile g0+m+4 is
  // requested into the stage of tile g0+m, which may already belong to the
  // next item, so the next item's first tiles land while this one finishes.
  // Tile n+1 is waited for at the end of slot 2n; at an item boundary
  // everything in flight (queries, state, tiles) is waited for.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // One copy of the schedule per group, the group a compile-time constant: a
  // group is made of whole waves, but the compiler cannot prove it, and a group
  // flag known only at run time would put the slot arithmetic on the vector
  // unit.
  auto run = [&](auto group) RA_INLINE {
  constexpr bool late = decltype(group)::value;  // group B
  for (;;) {
    const int32_t g0 = cc.g0, nt = cc.g1 - cc.g0;
    // end of slot 2n: stream tile g0+n+1 must be in LDS; tiles requested
    // after it may stay in flight
    auto slot_end = [&](int32_t n) RA_INLINE {
      const int32_t in_flight = fg - (g0 + n + 2);
      if (in_flight >= 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NDMA));
      else if (in_flight == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NDMA));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
    };
    auto matrix = [&](int32_t n) RA_INLINE {
      __builtin_amdgcn_s_setprio(1);
      mfma_phase((g0 + n + 1) % kStages, (g0 + n) % kStages);
      __builtin_amdgcn_s_setprio(0);
    };
    // slot 0: group A starts
    if (!late) {
      scores(g0 % kStages);
      vector_phase(g0);
    }
    slot_end(0);
    // slots 2n+1 and 2n+2. The slot arithmetic is the same for both groups;
    // only the choice of phase depends on the group, a whole wave.
    for (int32_t n = 0; n < nt; ++n) {
      if (fg == g0 + n - 1 + kStages && fg < NT) fetch_next();
      if (!late) {
        // past the item's last tile the scores read a stage that is not
        // this item's and are never used
        matrix(n);
      } else {
        if (n == 0) scores(g0 % kStages);  // group B starts
        vector_phase(g0 + n);
      }
      __syncthreads();
      if (!late) {
        if (n + 1 < nt) vector_phase(g0 + n + 1);
      } else {
        matrix(n);
      }
      slot_end(n + 1);
    }
    // queries first (theirs is the longest wait), then this item's results,
    // then the next item's state
    const bool more = cc.g1 < NT;
    Cursor nx = cc;
    if (more) {
      advance(nx);
      load_q(nx.it);
      // the compiler cannot tell which iteration reloaded the query
      // registers: without this wait it would wait for every outstanding load
      // before each score product
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    end_item();
    if (!more) break;
    cc = nx;
    begin_item();
    // the state just requested must be in. Without state nothing is pending
    // but the output stores, which no wait here needs: the counter is in
    // order, so the first tile wait of the next item covers them, a slot or
    // two after they were issued
    if (MODE != kAttend) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }
  };
  if (w >= kWaves / 2)
    run(BoolC<true>{});
  else
    run(BoolC<false>{});
  if (MODE == kLast && state_in) finalize_empty_items();
}

template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(kThreads, 1) void step_mfma_kernel(RA_STEP_PARAMS) {
  step_mfma_body<D, CAUSAL, MODE>(RA_STEP_ARGS);
}

// The steps before the last one of a ring run while the next block is passed
// on a side stream. Two waves of 248 VGPRs leave 16 registers per SIMD lane,
// where one wave of the block-pass copy kernel fits beside the step kernel;
// with 251-256 the SIMD's register file is full and the copy only runs in the
// step kernel's tail, after its workgroups finish. On gfx950 the attribute
// counts the unified VGPR/AGPR file in pairs: 124 caps the kernel at 248.
// (At d = 64 the kernel needs about 200.)
template <>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_num_vgpr(124))) void
step_mfma_kernel<128, true, kStep>(RA_STEP_PARAMS) {
  step_mfma_body<128, true, kStep>(RA_STEP_ARGS);
}
template <>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_num_vgpr(124))) void
step_mfma_kernel<128, false, kStep>(RA_STEP_PARAMS) {
  step_mfma_body<128, false, kStep>(RA_STEP_ARGS);
}

#undef RA_STEP_PARAMS
#undef RA_STEP_ARGS

DevSegs dev(const HostSegs& s) { return DevSegs{s.start0, s.start1, s.len0, s.len}; }

// workgroups per XCD: one per CU (a workgroup's LDS ring fills a CU)
int32_t cus_per_xcd() {
  static int32_t n = 0;
  if (n == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < kXcds)
      cus = 256;
    n = cus / kXcds;
  }
  return n;
}

template <int D, bool CAUSAL, int MODE>
hipError_t launch(const StepArgs& a, bf16* out, float* lse, hipStream_t st) {
  const int32_t nqt = (a.Lq + kBQ - 1) / kBQ;
  const int64_t total = (int64_t)a.nb * nqt;
  const int32_t per_xcd = (int32_t)((total + kXcds - 1) / kXcds);
  const int32_t nwg_x = min(per_xcd, cus_per_xcd());
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((step_mfma_kernel<D, CAUSAL, MODE>), dim3(kXcds * nwg_x), dim3(kThreads), 0,
                     st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.nb, a.Lq, a.Lk,
                     dev(a.qs), dev(a.ks), c, (int32_t)a.init, a.o_acc, a.m, a.l, out, lse, nqt,
                     per_xcd, nwg_x, a.group);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& a, hipStream_t st) {
  if (a.d == 128)
    return a.causal ? launch<128, true, kStep>(a, nullptr, nullptr, st)
                    : launch<128, false, kStep>(a, nullptr, nullptr, st);
  return a.causal ? launch<64, true, kStep>(a, nullptr, nullptr, st)
                  : launch<64, false, kStep>(a, nullptr, nullptr, st);
}

hipError_t launch_step_last_bf16(const StepArgs& a, void* out, float* lse, hipStream_t st) {
  bf16* o = (bf16*)out;
  if (a.d == 128)
    return a.causal ? launch<128, true, kLast>(a, o, lse, st) : launch<128, false, kLast>(a, o, lse, st);
  return a.causal ? launch<64, true, kLast>(a, o, lse, st) : launch<64, false, kLast>(a, o, lse, st);
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
  a.group = 1;
  a.causal = false;
  a.init = true;
  a.scale = scale;
  if (d == 128) return launch<128, false, kAttend>(a, (bf16*)out, lse, st);
  return launch<64, false, kAttend>(a, (bf16*)out, lse, st);
}

}  // namespace ra

// LDS tiles and matrix-core operands shared by the short-loop attention
// kernels (backward ring step, attention of short independent problems).
//
// A tile is 64 rows of a [rows, D] bf16 slice, stored column-major in 16-byte
// columns: one buffer load instruction (64 lanes x 16 bytes, lane i = row i)
// fills the 1 KiB run of one column, runs padded to 1088 bytes so that the
// 16-byte row reads and the transposing reads are free of bank conflicts.
// Operands follow the 32x32x16 bf16 MFMA: a row operand gives lane (l32, h)
// rows 32st + l32 and d columns 16ksi + 8h..+8; a transposed operand gives the
// A operand of X^T for the 16 rows of slice kc in the permuted order that
// matches a 32x32 accumulator packed by pack_b (lane half h of register r
// holds row 8(r/4) + 4h + r%4), so a score accumulator feeds the next product
// straight from the registers.
#pragma once

#include "ra_device.h"

namespace ra {
namespace tiles {

constexpr int kT = 64;                // streamed rows per tile
constexpr int kRunB = 1088;           // LDS bytes per 64-row run of one 16-byte column
constexpr int kXcdsB = 8;

template <int D>
struct BLay {
  static constexpr int NRUN = D / 8;               // 16-byte columns = load runs per tile
  static constexpr int TBYTES = NRUN * kRunB;      // one tensor's tile
  static constexpr int ROWV = 2 * kT * 4;          // lse (log2 units) and delta of a tile's rows
  static constexpr int STAGE = 2 * TBYTES + ROWV;
  static constexpr int at(int row, int col) { return col * kRunB + 16 * row; }
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;
typedef __attribute__((address_space(3))) char lds_char_b;

// 16 bytes per lane from a bounds-checked buffer straight into LDS at
// m0 + 16*lane; out-of-range rows read as zero. Ordered by explicit vmcnt
// waits before the barriers that publish a tile.
__device__ __forceinline__ void bload_lds16(__amdgpu_buffer_rsrc_t rs, const char* lds, int voff,
                                            int soff) {
  const unsigned m0 = (unsigned)(size_t)(const lds_char_b*)lds;
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs), "s"(soff), "{m0}"(m0)
               : "memory");
}

__device__ __forceinline__ bf16x8 bl_b128(const char* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ bf16x4 bl_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)p);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const bf16* base, int32_t rows, int d) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, rows * d * 2, 0x00020000);
}

// rows row0.. of a [rows, D] slice into a tile of the layout above; wave w of
// W fills runs (16-byte columns) w*NRUN/W.., lane i brings row i
template <int D, int W>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, char* dst, int32_t row0, int w,
                                          int lane) {
  constexpr int RUNS = BLay<D>::NRUN / W;
#pragma unroll
  for (int i = 0; i < RUNS; ++i) {
    const int r = w * RUNS + i;
    bload_lds16(rs, dst + r * kRunB, lane * D * 2 + 16 * r, row0 * D * 2);
  }
}

// A operand of rows 32st+l32 of a tile, d columns 16ksi+8h..+8
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char* tile, int st, int ksi, int l32, int h) {
  return bl_b128(tile + BLay<D>::at(32 * st + l32, 2 * ksi + h));
}

// A operand of the transposed tile: d rows 32t.. and the 16 tile rows of
// slice kc, in the permuted order that matches a score accumulator packed by
// pack_b (lane base `tr` from tr_base)
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int tr, int kc, int t) {
  const int off = tr + BLay<D>::at(16 * kc, 4 * t);
  const bf16x4 a = bl_tr16(tile + off);
  const bf16x4 b = bl_tr16(tile + off + 16 * 8);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <int D>
__device__ __forceinline__ int tr_base(int lane) {
  const int g = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  return BLay<D>::at(4 * (g >> 1) + rr, 2 * (g & 1) + (c4 >> 1)) + 8 * (c4 & 1);
}

// the 16 values of one 32x32 accumulator as two bf16 B operands (16-row slices)
__device__ __forceinline__ void pack_b(const f32x16& x, bf16x8& lo, bf16x8& hi) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    lo[r] = to_bf16(x[r]);
    hi[r] = to_bf16(x[8 + r]);
  }
}

// row of register r of a 32x32 accumulator (within its 32-row block), for lane half h
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

// logical workgroup index: each XCD takes a contiguous range, so the
// workgroups of one slice share that XCD's L2
__device__ __forceinline__ int32_t xcd_logical(int32_t per_xcd) {
  return (int32_t)(blockIdx.x % kXcdsB) * per_xcd + (int32_t)(blockIdx.x / kXcdsB);
}

// Tiles [first, last) of `rows` streamed rows (segments `ss`) holding rows
// whose position is >= lo (causal: rows that some owned row can see, or that
// can see some owned row), as at most two runs of tile indices.
struct TileRuns {
  int32_t t0a, n0, t1a, n;
};
__device__ __forceinline__ TileRuns tiles_from(const DevSegs& ss, int32_t rows, int32_t lo_pos,
                                               int32_t hi_pos, bool after) {
  // after: keep rows with pos >= lo_pos (queries seen by keys);
  // otherwise keep rows with pos <= hi_pos (keys seen by queries)
  int32_t ra0, rb0, ra1 = 0, rb1 = 0;
  const int32_t len1 = rows - ss.len0;
  auto clampi = [](int32_t x, int32_t n) { return x < 0 ? 0 : (x > n ? n : x); };
  if (after) {
    ra0 = clampi(lo_pos - ss.start0, ss.len0);
    rb0 = ss.len0;
    if (len1 > 0) {
      ra1 = ss.len0 + clampi(lo_pos - ss.start1, len1);
      rb1 = rows;
    }
  } else {
    ra0 = 0;
    rb0 = clampi(hi_pos - ss.start0 + 1, ss.len0);
    if (len1 > 0) {
      ra1 = ss.len0;
      rb1 = ss.len0 + clampi(hi_pos - ss.start1 + 1, len1);
    }
  }
  TileRuns tr;
  const int32_t t0b = (rb0 + kT - 1) / kT;
  tr.t0a = ra0 / kT;
  tr.n0 = rb0 > ra0 ? t0b - tr.t0a : 0;
  tr.t1a = ra1 / kT;
  const int32_t t1b = (rb1 + kT - 1) / kT;
  if (tr.n0 > 0 && tr.t1a < t0b) tr.t1a = t0b;
  const int32_t n1 = rb1 > ra1 && t1b > tr.t1a ? t1b - tr.t1a : 0;
  tr.n = tr.n0 + n1;
  return tr;
}
__device__ __forceinline__ int32_t tile_row0(const TileRuns& tr, int32_t n) {
  return (n < tr.n0 ? tr.t0a + n : tr.t1a + (n - tr.n0)) * kT;
}

// s_waitcnt vmcnt(0) (gfx9 encoding, other counters left alone)
constexpr int kVmcnt0 = (7 << 4) | (15 << 8);

}  // namespace tiles
}  // namespace ra

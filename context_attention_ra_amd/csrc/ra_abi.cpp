// C-ABI boundary of libra: host-side validation, then launch on the caller's
// stream. The declarations and their contracts are in include/ra.h.

#include "ra.h"

#include <math.h>
#include <stdint.h>

#include "ra_bwd.h"
#include "ra_launch.h"
#include "ra_stream_launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

ra_status hip_fail(hipError_t e) {
  if (e == hipSuccess) return RA_OK;
  g_last_hip_error = (int32_t)e;
  return RA_ERR_HIP;
}

size_t esize(ra_dtype dt) { return dt == RA_BF16 ? 2 : 4; }
bool known_dtype(ra_dtype dt) { return dt == RA_F32 || dt == RA_BF16; }
bool supported_d(int32_t d) { return d == 64 || d == 128; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range span(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks a segment table against the row count it describes.
bool segs_ok(const ra_segs* s, int32_t rows, ra::HostSegs* out) {
  if (!s || (s->n != 1 && s->n != 2) || s->reserved != 0) return false;
  int64_t total = 0;
  for (int k = 0; k < s->n; ++k) {
    if (s->start[k] < 0 || s->len[k] < 1) return false;
    if (s->start[k] + s->len[k] > (int64_t)INT32_MAX) return false;
    total += s->len[k];
  }
  if (total != rows) return false;
  out->start0 = (int32_t)s->start[0];
  out->len0 = (int32_t)s->len[0];
  out->start1 = s->n == 2 ? (int32_t)s->start[1] : 0;
  out->len = rows;
  return true;
}

bool dims_ok(int32_t B, int32_t H, int32_t L) {
  if (B <= 0 || H <= 0 || L <= 0) return false;
  return (int64_t)B * H <= (int64_t)INT32_MAX;
}

}  // namespace

extern "C" {

namespace {

// Checks shared by ra_step and ra_step_final; fills the launch arguments.
ra_status step_args(const void* q, const void* k, const void* v, ra_dtype dt, int32_t B,
                    int32_t H, int32_t H_kv, int32_t Lq, int32_t Lk, int32_t d,
                    const ra_segs* q_segs, const ra_segs* kv_segs, ra_mask mask, float scale,
                    uint32_t flags, float* o_acc, float* m, float* l, ra::StepArgs* out_args) {
  if (!q || !k || !v || !o_acc || !m || !l || !q_segs || !kv_segs) return RA_ERR_INVALID_ARG;
  if (!known_dtype(dt) || !dims_ok(B, H, Lq) || Lk <= 0 || d <= 0) return RA_ERR_INVALID_ARG;
  if (H_kv <= 0 || H % H_kv != 0) return RA_ERR_INVALID_ARG;
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return RA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return RA_ERR_INVALID_ARG;
  if (flags & ~RA_STEP_INIT) return RA_ERR_INVALID_ARG;
  ra::HostSegs qs, ks;
  if (!segs_ok(q_segs, Lq, &qs) || !segs_ok(kv_segs, Lk, &ks)) return RA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_acc, 16) ||
      !aligned(m, 4) || !aligned(l, 4))
    return RA_ERR_INVALID_ARG;
  const size_t nb = (size_t)B * H, nkv = (size_t)B * H_kv, es = esize(dt);
  const Range rq = span(q, nb * Lq * d * es), rk = span(k, nkv * Lk * d * es),
              rv = span(v, nkv * Lk * d * es), ro = span(o_acc, nb * Lq * d * 4),
              rm = span(m, nb * Lq * 4), rl = span(l, nb * Lq * 4);
  for (Range st : {ro, rm, rl})
    for (Range in : {rq, rk, rv})
      if (overlap(st, in)) return RA_ERR_INVALID_ARG;
  if (overlap(ro, rm) || overlap(ro, rl) || overlap(rm, rl)) return RA_ERR_INVALID_ARG;
  if (!supported_d(d)) return RA_ERR_UNSUPPORTED;
  const int64_t tiles = (int64_t)nb * ((Lq + 127) / 128);
  if (tiles > (int64_t)INT32_MAX / 2) return RA_ERR_UNSUPPORTED;
  // one (batch, head) slice of Q, K or V must be addressable by a 32-bit offset
  if ((int64_t)Lk * d * (int64_t)es > (int64_t)INT32_MAX) return RA_ERR_UNSUPPORTED;
  if ((int64_t)Lq * d * (int64_t)es > (int64_t)INT32_MAX) return RA_ERR_UNSUPPORTED;

  ra::StepArgs& a = *out_args;
  a = ra::StepArgs{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.nb = (int32_t)nb;
  a.Lq = Lq;
  a.Lk = Lk;
  a.d = d;
  a.group = H / H_kv;
  a.qs = qs;
  a.ks = ks;
  a.causal = mask == RA_MASK_CAUSAL;
  a.init = (flags & RA_STEP_INIT) != 0;
  a.scale = scale;
  a.o_acc = o_acc;
  a.m = m;
  a.l = l;
  return RA_OK;
}

}  // namespace

ra_status ra_step_gqa(const void* q, const void* k, const void* v, ra_dtype dt, int32_t B,
                      int32_t H, int32_t H_kv, int32_t Lq, int32_t Lk, int32_t d,
                      const ra_segs* q_segs, const ra_segs* kv_segs, ra_mask mask, float scale,
                      uint32_t flags, float* o_acc, float* m, float* l, hipStream_t stream) {
  ra::StepArgs a;
  const ra_status st = step_args(q, k, v, dt, B, H, H_kv, Lq, Lk, d, q_segs, kv_segs, mask, scale,
                                 flags, o_acc, m, l, &a);
  if (st != RA_OK) return st;
  return hip_fail(dt == RA_BF16 ? ra::launch_step_bf16(a, stream) : ra::launch_step_f32(a, stream));
}

ra_status ra_step(const void* q, const void* k, const void* v, ra_dtype dt, int32_t B, int32_t H,
                  int32_t Lq, int32_t Lk, int32_t d, const ra_segs* q_segs,
                  const ra_segs* kv_segs, ra_mask mask, float scale, uint32_t flags,
                  float* o_acc, float* m, float* l, hipStream_t stream) {
  return ra_step_gqa(q, k, v, dt, B, H, H, Lq, Lk, d, q_segs, kv_segs, mask, scale, flags, o_acc,
                     m, l, stream);
}

ra_status ra_step_final_gqa(const void* q, const void* k, const void* v, ra_dtype dt, int32_t B,
                            int32_t H, int32_t H_kv, int32_t Lq, int32_t Lk, int32_t d,
                            const ra_segs* q_segs, const ra_segs* kv_segs, ra_mask mask,
                            float scale, uint32_t flags, float* o_acc, float* m, float* l,
                            void* out, float* lse, hipStream_t stream) {
  if (!out) return RA_ERR_INVALID_ARG;
  ra::StepArgs a;
  const ra_status st = step_args(q, k, v, dt, B, H, H_kv, Lq, Lk, d, q_segs, kv_segs, mask, scale,
                                 flags, o_acc, m, l, &a);
  if (st != RA_OK) return st;
  if (!aligned(out, 16) || (lse && !aligned(lse, 4))) return RA_ERR_INVALID_ARG;
  const size_t nb = (size_t)B * H, nkv = (size_t)B * H_kv, es = esize(dt), rows = nb * Lq;
  const Range rout = span(out, rows * d * es);
  const Range others[] = {span(q, rows * d * es), span(k, nkv * Lk * d * es), span(v, nkv * Lk * d * es),
                          span(o_acc, rows * d * 4), span(m, rows * 4), span(l, rows * 4)};
  for (Range x : others) {
    if (overlap(rout, x)) return RA_ERR_INVALID_ARG;
    if (lse && overlap(span(lse, rows * 4), x)) return RA_ERR_INVALID_ARG;
  }
  if (lse && overlap(span(lse, rows * 4), rout)) return RA_ERR_INVALID_ARG;
  if (dt == RA_BF16) return hip_fail(ra::launch_step_last_bf16(a, out, lse, stream));
  // fp32: the step, then the finalize of the updated state
  const hipError_t e = ra::launch_step_f32(a, stream);
  if (e != hipSuccess) return hip_fail(e);
  return hip_fail(ra::launch_finalize(o_acc, m, l, (int64_t)rows, d, out, false, lse, stream));
}

ra_status ra_step_final(const void* q, const void* k, const void* v, ra_dtype dt, int32_t B,
                        int32_t H, int32_t Lq, int32_t Lk, int32_t d, const ra_segs* q_segs,
                        const ra_segs* kv_segs, ra_mask mask, float scale, uint32_t flags,
                        float* o_acc, float* m, float* l, void* out, float* lse,
                        hipStream_t stream) {
  return ra_step_final_gqa(q, k, v, dt, B, H, H, Lq, Lk, d, q_segs, kv_segs, mask, scale, flags,
                           o_acc, m, l, out, lse, stream);
}

ra_status ra_bwd_prep(const void* out, const void* dout, ra_dtype dt, int32_t B, int32_t H,
                      int32_t L, int32_t d, float* delta, hipStream_t stream) {
  if (!out || !dout || !delta) return RA_ERR_INVALID_ARG;
  if (!known_dtype(dt) || !dims_ok(B, H, L) || d <= 0) return RA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(delta, 4)) return RA_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * L;
  const Range rd = span(delta, rows * 4);
  if (overlap(rd, span(out, rows * d * esize(dt))) || overlap(rd, span(dout, rows * d * esize(dt))))
    return RA_ERR_INVALID_ARG;
  if (dt != RA_BF16 || !supported_d(d)) return RA_ERR_UNSUPPORTED;
  return hip_fail(ra::launch_bwd_prep_bf16(out, dout, (int64_t)rows, d, delta, stream));
}

ra_status ra_step_bwd(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, const float* delta, ra_dtype dt, int32_t B, int32_t H,
                      int32_t H_kv, int32_t Lq, int32_t Lk, int32_t d, const ra_segs* q_segs,
                      const ra_segs* kv_segs, ra_mask mask, float scale, uint32_t flags,
                      float* dq_acc, float* dk_acc, float* dv_acc, hipStream_t stream) {
  if (!dout || !lse || !delta || !dq_acc || !dk_acc || !dv_acc) return RA_ERR_INVALID_ARG;
  if (flags & ~(RA_STEP_INIT | RA_BWD_KV_INIT | RA_BWD_NO_DQ | RA_BWD_NO_DKV)) return RA_ERR_INVALID_ARG;
  if ((flags & RA_BWD_NO_DQ) && (flags & RA_BWD_NO_DKV)) return RA_ERR_INVALID_ARG;
  // the forward checks cover q, k, v, the sizes, segments, mask and scale; dq_acc
  // and the two per-row vectors take the places of o_acc, m and l
  ra::StepArgs sa;
  const ra_status st = step_args(q, k, v, dt, B, H, H_kv, Lq, Lk, d, q_segs, kv_segs, mask, scale,
                                 flags & RA_STEP_INIT, dq_acc, (float*)lse, (float*)delta, &sa);
  if (st != RA_OK) return st;
  if (!aligned(dout, 16) || !aligned(dk_acc, 16) || !aligned(dv_acc, 16)) return RA_ERR_INVALID_ARG;
  const size_t nb = (size_t)B * H, nkv = (size_t)B * H_kv, es = esize(dt);
  const Range in[] = {span(q, nb * Lq * d * es), span(k, nkv * Lk * d * es), span(v, nkv * Lk * d * es),
                      span(dout, nb * Lq * d * es), span(lse, nb * Lq * 4), span(delta, nb * Lq * 4)};
  const Range acc[] = {span(dq_acc, nb * Lq * d * 4), span(dk_acc, nkv * Lk * d * 4),
                       span(dv_acc, nkv * Lk * d * 4)};
  for (int i = 0; i < 3; ++i) {
    for (Range x : in)
      if (overlap(acc[i], x)) return RA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(acc[i], acc[j])) return RA_ERR_INVALID_ARG;
  }
  if (dt != RA_BF16) return RA_ERR_UNSUPPORTED;
  // the dK/dV kernel streams the query and dO slices through buffer resources
  // whose byte size is a 32-bit value, as the step kernels do for K/V
  if ((int64_t)Lq * d * (int64_t)es > (int64_t)INT32_MAX) return RA_ERR_UNSUPPORTED;
  // the dK/dV kernel numbers its workgroups (K/V slice, 256-key tile) in 32 bits
  if ((int64_t)B * H_kv * ((Lk + 255) / 256) > (int64_t)INT32_MAX / 2) return RA_ERR_UNSUPPORTED;
  ra::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.nb = sa.nb;
  a.Lq = Lq;
  a.Lk = Lk;
  a.d = d;
  a.group = sa.group;
  a.qs = sa.qs;
  a.ks = sa.ks;
  a.causal = sa.causal;
  a.init_dq = (flags & RA_STEP_INIT) != 0;
  a.init_dkv = (flags & RA_BWD_KV_INIT) != 0;
  a.run_dq = (flags & RA_BWD_NO_DQ) == 0;
  a.run_dkv = (flags & RA_BWD_NO_DKV) == 0;
  a.scale = scale;
  a.dq = dq_acc;
  a.dk = dk_acc;
  a.dv = dv_acc;
  return hip_fail(ra::launch_step_bwd_bf16(a, stream));
}

ra_status ra_finalize(const float* o_acc, const float* m, const float* l, int32_t B, int32_t H,
                      int32_t L, int32_t d, void* out, ra_dtype out_dt, float* lse,
                      hipStream_t stream) {
  if (!o_acc || !m || !l || !out) return RA_ERR_INVALID_ARG;
  if (!known_dtype(out_dt) || !dims_ok(B, H, L) || d <= 0) return RA_ERR_INVALID_ARG;
  if (!aligned(o_acc, 16) || !aligned(out, 16) || !aligned(m, 4) || !aligned(l, 4) ||
      (lse && !aligned(lse, 4)))
    return RA_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * L;
  const Range ro = span(o_acc, rows * d * 4), rm = span(m, rows * 4), rl = span(l, rows * 4),
              rout = span(out, rows * d * esize(out_dt));
  for (Range st : {ro, rm, rl}) {
    if (overlap(rout, st)) return RA_ERR_INVALID_ARG;
    if (lse && overlap(span(lse, rows * 4), st)) return RA_ERR_INVALID_ARG;
  }
  if (lse && overlap(span(lse, rows * 4), rout)) return RA_ERR_INVALID_ARG;
  if (!supported_d(d)) return RA_ERR_UNSUPPORTED;
  return hip_fail(ra::launch_finalize(o_acc, m, l, (int64_t)rows, d, out, out_dt == RA_BF16, lse, stream));
}

ra_status ra_merge_lse(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                       ra_dtype dt, int32_t B, int32_t H, int32_t L, int32_t d, void* o_out,
                       float* lse_out, hipStream_t stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return RA_ERR_INVALID_ARG;
  if (!known_dtype(dt) || !dims_ok(B, H, L) || d <= 0) return RA_ERR_INVALID_ARG;
  if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o_out, 16) || !aligned(lse_a, 4) ||
      !aligned(lse_b, 4) || !aligned(lse_out, 4))
    return RA_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * L, ob = rows * d * esize(dt), lb = rows * 4;
  const Range ra_ = span(o_a, ob), rb = span(o_b, ob), ro = span(o_out, ob);
  const Range la = span(lse_a, lb), lbr = span(lse_b, lb), lo = span(lse_out, lb);
  // the output may be exactly one of the inputs; partial overlaps are refused
  auto same_or_disjoint = [](Range x, Range y) { return (x.lo == y.lo && x.hi == y.hi) || !overlap(x, y); };
  if (!same_or_disjoint(ro, ra_) || !same_or_disjoint(ro, rb)) return RA_ERR_INVALID_ARG;
  if (!same_or_disjoint(lo, la) || !same_or_disjoint(lo, lbr)) return RA_ERR_INVALID_ARG;
  for (Range x : {ra_, rb, ro})
    for (Range y : {la, lbr, lo})
      if (overlap(x, y)) return RA_ERR_INVALID_ARG;
  if (!supported_d(d)) return RA_ERR_UNSUPPORTED;
  return hip_fail(ra::launch_merge(o_a, lse_a, o_b, lse_b, dt == RA_BF16, (int64_t)rows, d, o_out, lse_out, stream));
}

static ra_status factored_check(const void* q, const void* k, const void* v, ra_dtype dt,
                                int32_t B, int32_t H, int32_t T, int32_t S_sp, int32_t d,
                                float scale, void* out, float* lse) {
  if (!q || !k || !v || !out) return RA_ERR_INVALID_ARG;
  if (!known_dtype(dt) || B <= 0 || H <= 0 || T <= 0 || S_sp <= 0 || d <= 0) return RA_ERR_INVALID_ARG;
  if ((int64_t)T * S_sp > (int64_t)INT32_MAX || (int64_t)B * H * T > (int64_t)INT32_MAX)
    return RA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return RA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return RA_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * T * S_sp, tb = rows * d * esize(dt);
  const Range ro = span(out, tb);
  for (Range in : {span(q, tb), span(k, tb), span(v, tb)}) {
    if (overlap(ro, in)) return RA_ERR_INVALID_ARG;
    if (lse && overlap(span(lse, rows * 4), in)) return RA_ERR_INVALID_ARG;
  }
  if (lse && overlap(span(lse, rows * 4), ro)) return RA_ERR_INVALID_ARG;
  if (dt != RA_BF16 || !supported_d(d)) return RA_ERR_UNSUPPORTED;
  return RA_OK;
}

ra_status ra_factored_spatial(const void* q, const void* k, const void* v, ra_dtype dt, int32_t B,
                              int32_t H, int32_t T, int32_t S_sp, int32_t d, float scale,
                              void* out, float* lse, hipStream_t stream) {
  const ra_status st = factored_check(q, k, v, dt, B, H, T, S_sp, d, scale, out, lse);
  if (st != RA_OK) return st;
  // one frame of K or V must be addressable by a 32-bit offset
  if ((int64_t)S_sp * d * (int64_t)esize(dt) > (int64_t)INT32_MAX) return RA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * T * ((S_sp + 255) / 256) > (int64_t)INT32_MAX / 2) return RA_ERR_UNSUPPORTED;
  // every frame is an independent unmasked S_sp x S_sp problem: rows of frame t
  // of slice (b, h) are contiguous, so the frames are simply B*H*T slices
  return hip_fail(ra::launch_attend_bf16(q, k, v, B * H * T, S_sp, d, scale, out, lse, stream));
}

ra_status ra_factored_temporal(const void* q, const void* k, const void* v, ra_dtype dt, int32_t B,
                               int32_t H, int32_t T, int32_t S_sp, int32_t d, float scale,
                               void* out, float* lse, hipStream_t stream) {
  const ra_status st = factored_check(q, k, v, dt, B, H, T, S_sp, d, scale, out, lse);
  if (st != RA_OK) return st;
  if (T > 128) return RA_ERR_UNSUPPORTED;
  // the long-clip kernel addresses the T rows of a position from the start of
  // its (batch, head) slice with 32-bit byte offsets
  if (T > 16 && (int64_t)T * S_sp * d * (int64_t)esize(dt) > (int64_t)INT32_MAX) return RA_ERR_UNSUPPORTED;
  // up to 16 frames: one wave per problem; longer clips: one workgroup per
  // problem with the K/V frames staged in LDS
  if (T <= 16)
    return hip_fail(ra::launch_temporal_bf16(q, k, v, B * H, T, S_sp, d, scale, out, lse, stream));
  return hip_fail(ra::launch_temporal_long_bf16(q, k, v, B * H, T, S_sp, d, scale, out, lse, stream));
}

ra_status ra_kv_pass(const void* k_src, const void* v_src, void* k_dst, void* v_dst, size_t bytes,
                     hipStream_t stream) {
  if (bytes == 0) return RA_OK;
  if (!k_src || !v_src || !k_dst || !v_dst) return RA_ERR_INVALID_ARG;
  const Range a = span(k_src, bytes), b = span(v_src, bytes), c = span(k_dst, bytes),
              e = span(v_dst, bytes);
  if (overlap(c, e) || overlap(c, a) || overlap(c, b) || overlap(e, a) || overlap(e, b))
    return RA_ERR_INVALID_ARG;
  // the pass kernel (sized to run beside a ring step) for 16-byte aligned
  // buffers of whole 16-byte pieces; the runtime's copy otherwise
  if (aligned(k_src, 16) && aligned(v_src, 16) && aligned(k_dst, 16) && aligned(v_dst, 16) &&
      bytes % 16 == 0 && bytes / 16 <= ((size_t)1 << 30))
    return hip_fail(ra::launch_kv_pass(k_src, k_dst, v_src, v_dst, (int64_t)(bytes / 16), stream));
  hipError_t err = hipMemcpyAsync(k_dst, k_src, bytes, hipMemcpyDeviceToDevice, stream);
  if (err == hipSuccess) err = hipMemcpyAsync(v_dst, v_src, bytes, hipMemcpyDeviceToDevice, stream);
  return hip_fail(err);
}

ra_status ra_copy_rows(const void* src, int64_t src_slice_rows, int64_t src_row0, void* dst,
                       int64_t dst_slice_rows, int64_t dst_row0, int64_t nslices, int64_t nrows,
                       int64_t row_bytes, hipStream_t stream) {
  if (nrows == 0) return RA_OK;
  if (!src || !dst || nslices <= 0 || nrows < 0 || row_bytes <= 0) return RA_ERR_INVALID_ARG;
  if (src_row0 < 0 || dst_row0 < 0 || src_row0 + nrows > src_slice_rows ||
      dst_row0 + nrows > dst_slice_rows)
    return RA_ERR_INVALID_ARG;
  const size_t sp = (size_t)src_slice_rows * row_bytes, dp = (size_t)dst_slice_rows * row_bytes;
  const Range rs = span((const char*)src + src_row0 * row_bytes, sp * (nslices - 1) + nrows * row_bytes);
  const Range rd = span((const char*)dst + dst_row0 * row_bytes, dp * (nslices - 1) + nrows * row_bytes);
  if (overlap(rs, rd)) return RA_ERR_INVALID_ARG;
  return hip_fail(hipMemcpy2DAsync((char*)dst + dst_row0 * row_bytes, dp,
                                   (const char*)src + src_row0 * row_bytes, sp,
                                   (size_t)nrows * row_bytes, (size_t)nslices,
                                   hipMemcpyDeviceToDevice, stream));
}

ra_status ra_add_rows(const float* src, int64_t src_slice_rows, int64_t src_row0, float* dst,
                      int64_t dst_slice_rows, int64_t dst_row0, int64_t nslices, int64_t nrows,
                      int32_t d, hipStream_t stream) {
  if (nrows == 0) return RA_OK;
  if (!src || !dst || nslices <= 0 || nrows < 0 || d <= 0 || d % 4 != 0) return RA_ERR_INVALID_ARG;
  if (src_row0 < 0 || dst_row0 < 0 || src_row0 + nrows > src_slice_rows ||
      dst_row0 + nrows > dst_slice_rows)
    return RA_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return RA_ERR_INVALID_ARG;
  const size_t rb = (size_t)d * 4;
  const Range rs = span((const char*)src + src_row0 * rb, (size_t)src_slice_rows * rb * (nslices - 1) + nrows * rb);
  const Range rd = span((const char*)dst + dst_row0 * rb, (size_t)dst_slice_rows * rb * (nslices - 1) + nrows * rb);
  if (overlap(rs, rd)) return RA_ERR_INVALID_ARG;
  return hip_fail(ra::launch_add_rows(src, src_slice_rows, src_row0, dst, dst_slice_rows, dst_row0,
                                      nslices, nrows, d, stream));
}

const char* ra_status_string(ra_status s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARG: return "RA_ERR_INVALID_ARG";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_HIP: return "RA_ERR_HIP";
  }
  return "RA_UNKNOWN_STATUS";
}

int32_t ra_last_hip_error(void) { return g_last_hip_error; }

int32_t ra_version(void) { return 200; }

}  // extern "C"

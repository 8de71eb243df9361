/*
 * ra.h — one device's share of ring attention on MI355X (gfx950).
 *
 * What the library computes. Under context parallelism each device keeps its
 * chunk of queries while K/V blocks travel around a ring; at every step the
 * device attends its local queries to the block it holds and folds the result
 * into a running online-softmax state, and after P steps it holds the exact
 * attention output for its queries (Day 83 post on skandtandon.pages.dev,
 * "Context parallelism: splitting the sequence"; k8ai "Sequence and Context
 * Parallel", "How context parallel works"). Causal masking compares global
 * token positions, so any balanced chunk assignment works (k8ai, same section).
 * For video tokens, the factored spatial/temporal attention of the Day 83
 * post, "The spatial-temporal twist", is provided as two batched kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout: every tensor is a contiguous row-major [B, H, rows, d] array
 *   ("BHSD": the sequence is dimension 2), base address 16-byte aligned.
 *   Per-row vectors (m, l, lse) are contiguous [B, H, rows] float arrays.
 *   d must be 64 or 128, otherwise RA_ERR_UNSUPPORTED.
 * Ownership: all tensor pointers are device pointers owned by the caller.
 *   The library allocates no device memory and keeps no state between calls,
 *   so calls from several host threads are safe.
 * Streams: every call only enqueues work on `stream` (a hipStream_t; 0 is the
 *   null stream) and returns; it never synchronises. Ordering against other
 *   streams is the caller's job (hipEventRecord / hipStreamWaitEvent).
 * Errors: arguments are validated on the host before anything is enqueued; on
 *   RA_ERR_INVALID_ARG / RA_ERR_UNSUPPORTED nothing is launched and no output
 *   is touched. A failed launch returns RA_ERR_HIP and records the hipError_t,
 *   readable with ra_last_hip_error() on the same thread.
 * Numerics: bf16 inputs are multiplied on the matrix cores with fp32
 *   accumulation; the softmax, the running state and lse are fp32. Outputs are
 *   rounded to the output dtype with round-to-nearest-even. Logarithms are
 *   natural logarithms of the scaled scores.
 */
#ifndef RA_H_
#define RA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ra_status {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent segments, aliasing */
  RA_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement (d, dtype) */
  RA_ERR_HIP = 3           /* a HIP call failed; see ra_last_hip_error() */
} ra_status;

typedef enum ra_dtype { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

typedef enum ra_mask { RA_MASK_NONE = 0, RA_MASK_CAUSAL = 1 } ra_mask;

/*
 * Global token positions of the rows of a local tensor: up to two runs of
 * consecutive positions, stored one after the other. Row i of the local
 * tensor lies in segment k with rows_before_k <= i < rows_before_k + len[k]
 * and has global position start[k] + (i - rows_before_k).
 * Zigzag (balanced causal) split of k8ai "How context parallel works", as read
 * here: rank r of P holds chunk r then chunk 2P-1-r of 2P equal chunks, i.e.
 * n = 2. A contiguous or temporal-first split is n = 1.
 * Requirements: n in {1, 2}; start[k] >= 0; len[k] >= 1; the lengths sum to
 * the row count of the tensor they describe. Host memory, read during the call.
 */
typedef struct ra_segs {
  int32_t n;
  int32_t reserved; /* must be 0 */
  int64_t start[2];
  int64_t len[2];
} ra_segs;

/* ra_step flag: the incoming state is (O_acc = 0, m = -inf, l = 0); it is not
 * read, only written. Use it on the first ring step. */
#define RA_STEP_INIT 1u

/*
 * ra_step — one ring step: fold the attention of the local queries against one
 * K/V block into the running online-softmax state (Day 83 post, "Context
 * parallelism: splitting the sequence": each device accumulates partial
 * outputs with the online-softmax rule, the trick FlashAttention uses).
 *
 * q        [B,H,Lq,d] local queries (dt)
 * k, v     [B,H,Lk,d] the K/V block held at this step (dt)
 * q_segs   global positions of the Lq query rows
 * kv_segs  global positions of the Lk key rows
 * mask     RA_MASK_CAUSAL: key j is visible to query i iff pos(j) <= pos(i);
 *          RA_MASK_NONE: every key is visible
 * scale    score multiplier (finite, > 0), typically 1/sqrt(d)
 * flags    0 or RA_STEP_INIT
 * o_acc    [B,H,Lq,d] fp32, in/out: unnormalised output sum_j e^{s_ij - m_i} v_j
 * m        [B,H,Lq]   fp32, in/out: per-row reference value (natural-log units)
 * l        [B,H,Lq]   fp32, in/out: sum_j e^{s_ij - m_i}
 * The state (o_acc, m, l) after a step satisfies the two sums above over all
 * keys seen so far; m need not equal the running row maximum (the kernels may
 * keep it a bounded amount below it to skip rescaling), and m = -inf with
 * l = 0 means no visible key yet. A row with no visible key in this block is
 * left unchanged. The result does not depend on the order of the blocks
 * beyond rounding.
 * dt: RA_BF16 (matrix-core path) or RA_F32 (fp32 vector path).
 * Errors: RA_ERR_INVALID_ARG for null pointers, B/H/Lq/Lk <= 0, bad segments,
 *   a non-finite or non-positive scale, unknown flags or mask, or o_acc/m/l
 *   overlapping q/k/v; RA_ERR_UNSUPPORTED for d not in {64, 128}, a Q
 *   slice (Lq * d elements) or K/V slice (Lk * d elements) of more than
 *   INT32_MAX bytes, or more than 2^30 (batch x head, 128-row query tile)
 *   pairs.
 */
ra_status ra_step(const void* q, const void* k, const void* v, ra_dtype dt,
                  int32_t B, int32_t H, int32_t Lq, int32_t Lk, int32_t d,
                  const ra_segs* q_segs, const ra_segs* kv_segs, ra_mask mask,
                  float scale, uint32_t flags, float* o_acc, float* m, float* l,
                  hipStream_t stream);

/*
 * ra_finalize — turn the running state into the attention output after the
 * last ring step (Day 83 post, same section: after P steps the device holds
 * the correct output for its queries).
 *   out = o_acc / l (rounded to out_dt), lse = m + ln l.
 * A row with l = 0 (no visible key) gets out = 0 and lse = -inf.
 * o_acc [B,H,L,d] fp32, m, l [B,H,L] fp32; out [B,H,L,d] of out_dt;
 * lse [B,H,L] fp32 or NULL.
 * Errors: RA_ERR_INVALID_ARG for null required pointers, sizes <= 0, or out /
 *   lse overlapping the state; RA_ERR_UNSUPPORTED for d not in {64, 128}.
 */
ra_status ra_finalize(const float* o_acc, const float* m, const float* l,
                      int32_t B, int32_t H, int32_t L, int32_t d,
                      void* out, ra_dtype out_dt, float* lse, hipStream_t stream);

/*
 * ra_step_final — the last ring step with the finalize folded in: the result
 * of ra_step on this block followed by ra_finalize (Day 83 post, "Context
 * parallelism: splitting the sequence": after the last block the device
 * holds the exact output of its queries).
 * Arguments as for ra_step, plus
 *   out  [B,H,Lq,d] of dt: (o_acc' / l') with the state after this block;
 *   lse  [B,H,Lq] fp32 (m' + ln l'), or NULL.
 * A row with no visible key in any block gets out = 0 and lse = -inf.
 * The state (o_acc, m, l) is an input (not read with RA_STEP_INIT); its
 * contents afterwards are unspecified (the bf16 path leaves it unchanged and
 * never writes the updated state: the output is written straight from the
 * registers; the fp32 path runs the step and the finalize).
 * Errors: those of ra_step, and RA_ERR_INVALID_ARG for a null out or out /
 *   lse overlapping the inputs or the state.
 */
ra_status ra_step_final(const void* q, const void* k, const void* v, ra_dtype dt,
                        int32_t B, int32_t H, int32_t Lq, int32_t Lk, int32_t d,
                        const ra_segs* q_segs, const ra_segs* kv_segs, ra_mask mask,
                        float scale, uint32_t flags, float* o_acc, float* m, float* l,
                        void* out, float* lse, hipStream_t stream);

/*
 * ra_step_gqa, ra_step_final_gqa — ra_step and ra_step_final with fewer K/V
 * heads than query heads. The k8ai page ("Communication profile") notes that
 * the bytes a ring moves per step grow with the number of K/V heads, so a
 * model that shares each K/V head among several query heads passes
 * proportionally smaller blocks.
 * H_kv  K/V heads, 1 <= H_kv <= H and H % H_kv == 0. Query head h of batch b
 *       attends to K/V head h / (H / H_kv) of batch b (consecutive query heads
 *       form a group).
 * k, v  [B,H_kv,Lk,d]; every other argument, the state and the result are as
 *       for ra_step / ra_step_final (q, o_acc, m, l, out, lse have H heads).
 * With H_kv == H these are exactly ra_step and ra_step_final.
 * Errors: those of ra_step / ra_step_final, and RA_ERR_INVALID_ARG for
 *   H_kv <= 0 or H not a multiple of H_kv.
 */
ra_status ra_step_gqa(const void* q, const void* k, const void* v, ra_dtype dt,
                      int32_t B, int32_t H, int32_t H_kv, int32_t Lq, int32_t Lk, int32_t d,
                      const ra_segs* q_segs, const ra_segs* kv_segs, ra_mask mask,
                      float scale, uint32_t flags, float* o_acc, float* m, float* l,
                      hipStream_t stream);
ra_status ra_step_final_gqa(const void* q, const void* k, const void* v, ra_dtype dt,
                            int32_t B, int32_t H, int32_t H_kv, int32_t Lq, int32_t Lk,
                            int32_t d, const ra_segs* q_segs, const ra_segs* kv_segs,
                            ra_mask mask, float scale, uint32_t flags, float* o_acc,
                            float* m, float* l, void* out, float* lse, hipStream_t stream);

/* ra_step_bwd flag: the block's gradient accumulators dk_acc, dv_acc start at
 * zero; they are not read, only written. (RA_STEP_INIT does the same for
 * dq_acc.) */
#define RA_BWD_KV_INIT 2u

/* ra_step_bwd flags that run half of a step: RA_BWD_NO_DQ launches only the
 * dK/dV kernel (dq_acc is neither read nor written), RA_BWD_NO_DKV only the
 * dQ kernel (dk_acc, dv_acc are neither read nor written). The two halves
 * read the same inputs and write disjoint accumulators, so a caller may issue
 * them on two streams; the accumulators of a skipped half are still checked
 * as arguments. Setting both is an invalid argument. */
#define RA_BWD_NO_DQ 4u
#define RA_BWD_NO_DKV 8u

/*
 * ra_bwd_prep — per-row delta_i = <dO_i, O_i> (fp32) of the final forward
 * output O and its upstream gradient dO, needed by every backward ring step.
 * out, dout [B,H,L,d] of dt (RA_BF16); delta [B,H,L] fp32.
 * Errors: RA_ERR_INVALID_ARG for null pointers, sizes <= 0 or delta
 *   overlapping the inputs; RA_ERR_UNSUPPORTED for dt != RA_BF16 or d not in
 *   {64, 128}.
 */
ra_status ra_bwd_prep(const void* out, const void* dout, ra_dtype dt, int32_t B, int32_t H,
                      int32_t L, int32_t d, float* delta, hipStream_t stream);

/*
 * ra_step_bwd — one backward ring step. The ring passes K/V blocks in the
 * backward pass as well (k8ai "Communication profile"); at each step the
 * device adds the gradient contributions of its local queries against the
 * block it holds: with P_ij = exp(scale <q_i, k_j> - lse_i) over the visible
 * pairs and dS_ij = P_ij (<dO_i, v_j> - delta_i),
 *   dq_acc_i += scale sum_j dS_ij k_j   (stays with the local queries)
 *   dk_acc_j += scale sum_i dS_ij q_i   (travels with the block)
 *   dv_acc_j += sum_i P_ij dO_i         (travels with the block)
 * Summed over the P blocks (dq) and over the P ranks' queries (dk, dv) these
 * are the exact gradients of the attention, whatever the order.
 * q, dout  [B,H,Lq,d] local queries and the upstream gradient of their output
 * k, v     [B,H_kv,Lk,d] the block held at this step; H_kv K/V heads as for
 *          ra_step_gqa (query head h reads K/V head h / (H / H_kv); H_kv == H
 *          is one K/V head per query head); the dk_acc and dv_acc rows of a
 *          K/V head sum the contributions of the H / H_kv query heads that
 *          share it
 * lse      [B,H,Lq] fp32, the final forward lse of the local queries
 *          (ra_step_final / ra_finalize); -inf rows contribute nothing
 * delta    [B,H,Lq] fp32 from ra_bwd_prep
 * q_segs, kv_segs, mask, scale: as for ra_step (the same mask and scale as
 *          the forward pass)
 * flags    0, RA_STEP_INIT (dq_acc starts at zero), RA_BWD_KV_INIT (dk_acc,
 *          dv_acc start at zero), or both; with at most one of RA_BWD_NO_DQ,
 *          RA_BWD_NO_DKV to run half of the step
 * dq_acc   [B,H,Lq,d] fp32 in/out; dk_acc, dv_acc [B,H_kv,Lk,d] fp32 in/out
 * dt must be RA_BF16 (inputs bf16, products on the matrix cores, fp32
 * accumulation). The two kernels run one after the other on `stream`.
 * Errors: those of ra_step_gqa, RA_ERR_INVALID_ARG for a null dout, lse, delta or
 *   accumulator, unknown flags, both RA_BWD_NO_DQ and RA_BWD_NO_DKV, or an
 *   accumulator overlapping an input or another accumulator;
 *   RA_ERR_UNSUPPORTED for dt != RA_BF16, a local query slice (Lq * d
 *   elements) of more than INT32_MAX bytes, or more than 2^30 (K/V head,
 *   256-key tile) pairs.
 */
ra_status ra_step_bwd(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, const float* delta, ra_dtype dt,
                      int32_t B, int32_t H, int32_t H_kv, int32_t Lq, int32_t Lk, int32_t d,
                      const ra_segs* q_segs, const ra_segs* kv_segs, ra_mask mask,
                      float scale, uint32_t flags, float* dq_acc, float* dk_acc,
                      float* dv_acc, hipStream_t stream);

/*
 * ra_merge_lse — combine two normalised partial attentions of the same queries
 * over disjoint key sets (the partial outputs the Day 83 post's devices
 * accumulate, "Context parallelism: splitting the sequence"):
 *   lse = ln(e^{lse_a} + e^{lse_b})
 *   o   = e^{lse_a - lse} o_a + e^{lse_b - lse} o_b
 * A side with lse = -inf has weight 0; if both are -inf, o = 0, lse = -inf.
 * o_a, o_b, o_out [B,H,L,d] of dt; lse_a, lse_b, lse_out [B,H,L] fp32.
 * o_out may be o_a or o_b exactly (in place) and lse_out may be lse_a or
 * lse_b exactly; any other overlap is RA_ERR_INVALID_ARG.
 */
ra_status ra_merge_lse(const void* o_a, const float* lse_a,
                       const void* o_b, const float* lse_b, ra_dtype dt,
                       int32_t B, int32_t H, int32_t L, int32_t d,
                       void* o_out, float* lse_out, hipStream_t stream);

/*
 * ra_factored_spatial — spatial half of factored video attention (Day 83 post,
 * "The spatial-temporal twist"): tokens are frame-major, index t*S_sp + s, and
 * each query attends without a mask to the S_sp keys of its own frame.
 * q, k, v, out [B,H,T*S_sp,d] of dt (RA_BF16); lse [B,H,T*S_sp] fp32 or NULL.
 * Under a temporal-first split this is fully local to a device.
 * Errors: RA_ERR_INVALID_ARG for null required pointers, sizes <= 0,
 *   T*S_sp > INT32_MAX, bad scale or out/lse overlapping inputs;
 *   RA_ERR_UNSUPPORTED for dt != RA_BF16, d not in {64, 128}, or one frame
 *   of K/V larger than INT32_MAX bytes.
 */
ra_status ra_factored_spatial(const void* q, const void* k, const void* v, ra_dtype dt,
                              int32_t B, int32_t H, int32_t T, int32_t S_sp, int32_t d,
                              float scale, void* out, float* lse, hipStream_t stream);

/*
 * ra_factored_temporal — temporal half of factored video attention (same
 * section): each query at (t, s) attends without a mask to the T keys
 * {t'*S_sp + s : t' < T} at its spatial position. T must be 1..128 (the
 * page's clips run to 48 and 120 frames, "What the numbers look like"); up
 * to 16 frames one wave serves a spatial position, longer clips one
 * workgroup with the position's K and V frames staged in LDS.
 * Arguments and errors as ra_factored_spatial (without the per-frame size
 * limit); T > 128 is RA_ERR_UNSUPPORTED, and so is T > 16 when one (batch,
 * head) slice, T * S_sp * d elements, exceeds 2^31 - 1 bytes.
 */
ra_status ra_factored_temporal(const void* q, const void* k, const void* v, ra_dtype dt,
                               int32_t B, int32_t H, int32_t T, int32_t S_sp, int32_t d,
                               float scale, void* out, float* lse, hipStream_t stream);

/*
 * ra_kv_pass — the ring's K/V hand-off (Day 83 post, same section: blocks are
 * passed to the next device; k8ai ring figure: send the next block while
 * computing on the current one). On one GPU the transfer from the source rank
 * is simulated by an asynchronous device-to-device copy of its K and V blocks
 * into the receive buffers, enqueued on `stream` (normally a side stream, so
 * the copy overlaps the current step's compute). For 16-byte aligned buffers
 * of a multiple of 16 bytes (up to 16 GiB) the copy is the library's pass
 * kernel, whose waves are small enough (16 VGPRs) to run on every SIMD beside
 * the kernel of ra_step and ra_step_gqa, which leaves room for one; other
 * buffers take the runtime's device-to-device copy.
 * k_src, v_src -> k_dst, v_dst: `bytes` each, device memory; source and
 * destination must not overlap. bytes == 0 is a no-op.
 */
ra_status ra_kv_pass(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                     size_t bytes, hipStream_t stream);

/*
 * ra_copy_rows — the exchanges of the two alternatives to the ring that the
 * k8ai page names ("An alternative: all-to-all on heads"; gathering every K/V
 * block), simulated on one GPU: an asynchronous strided device-to-device copy
 * of `nrows` consecutive rows from each of `nslices` slices of a source
 * tensor into the same number of slices of a destination tensor.
 *   dst[s][dst_row0 + i] = src[s][src_row0 + i] for s < nslices, i < nrows
 * where slice s of src starts at src + s * src_slice_rows * row_bytes (and
 * likewise for dst). row_bytes is the size of one row (d * element size).
 * Used to place blocks at their global positions (all-gather) and to move a
 * head group between sequence-sharded and head-sharded layouts (all-to-all).
 * Errors: RA_ERR_INVALID_ARG for null pointers, nslices / nrows / row_bytes
 *   <= 0, a row range outside its slice, or source and destination ranges
 *   that overlap. nrows == 0 is a no-op.
 */
ra_status ra_copy_rows(const void* src, int64_t src_slice_rows, int64_t src_row0,
                       void* dst, int64_t dst_slice_rows, int64_t dst_row0,
                       int64_t nslices, int64_t nrows, int64_t row_bytes, hipStream_t stream);

/*
 * ra_add_rows — the reduce-scatter that the Ultralytics glossary lists next to
 * all-gather ("How Context Parallelism Works"), in the form the backward pass
 * of the all-gather variant needs: every rank's gradient of the gathered K/V
 * covers all positions, and the rows a rank owns must be summed over the
 * ranks. One GPU simulates the exchange; this call is its arithmetic:
 *   dst[s][dst_row0 + i][c] += src[s][src_row0 + i][c]
 * for s < nslices, i < nrows, c < d, fp32, with slice s of src starting at
 * src + s * src_slice_rows * d floats (likewise dst). Device pointers, 16-byte
 * aligned; d a multiple of 4. Asynchronous on `stream`.
 * Errors: RA_ERR_INVALID_ARG for null pointers, nslices <= 0, nrows < 0,
 *   d <= 0 or not a multiple of 4, a row range outside its slice, misaligned
 *   pointers, or source and destination ranges that overlap. nrows == 0 is a
 *   no-op.
 */
ra_status ra_add_rows(const float* src, int64_t src_slice_rows, int64_t src_row0,
                      float* dst, int64_t dst_slice_rows, int64_t dst_row0,
                      int64_t nslices, int64_t nrows, int32_t d, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* ra_status_string(ra_status s);

/* hipError_t of the last RA_ERR_HIP returned on the calling thread (0 if none). */
int32_t ra_last_hip_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H_ */

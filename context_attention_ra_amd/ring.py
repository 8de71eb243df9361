"""One rank's ring, simulated on one GPU: P block steps with a side-stream prefetch.

Ring attention as the pages describe it (Day 83 post, "Context parallelism:
splitting the sequence"; k8ai "How context parallel works", ring figure): the
rank keeps its queries; at step s it holds the K/V block of rank (r - s) mod P,
folds it into the running state with ``ra_step``, and meanwhile the block for
step s+1 is being passed to it. Here every rank's block already sits in this
GPU's memory, so the pass is ``ra_kv_pass`` (a device-to-device copy) enqueued
on a side stream into one half of a double buffer, ordered against the compute
stream with events exactly as a network receive would be. The last step is
``ra_step_final``: the same kernel folds in the last block and writes the
output and its log-sum-exp (no separate finalize pass over the state).

This module is host control only: every byte of the path moves in libra.
"""

from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib, layout


class RingState:
    """The running (O_acc, m, l) state of one rank's queries (fp32)."""

    def __init__(self, B, H, L, d, device):
        self.o = torch.empty((B, H, L, d), dtype=torch.float32, device=device)
        self.m = torch.empty((B, H, L), dtype=torch.float32, device=device)
        self.l = torch.empty((B, H, L), dtype=torch.float32, device=device)


def run(q: torch.Tensor,
        q_segs: Sequence[Tuple[int, int]],
        kv_blocks: Sequence[Tuple[torch.Tensor, torch.Tensor]],
        kv_segs: Sequence[Sequence[Tuple[int, int]]],
        rank: int,
        causal: bool,
        scale: Optional[float] = None,
        order: Optional[List[int]] = None,
        prefetch: bool = True,
        out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None,
        state: Optional[RingState] = None,
        bufs: Optional[List[Tuple[torch.Tensor, torch.Tensor]]] = None,
        copy_stream: Optional[torch.cuda.Stream] = None,
        step_events: Optional[List[Tuple[torch.cuda.Event, torch.cuda.Event]]] = None,
        finalize: bool = True):
    """Run rank `rank`'s share of ring attention on the current stream.

    q          [B, H, Lq, d] local queries; q_segs their global positions
    kv_blocks  P pairs (k_t, v_t), rank t's local K/V [B, H, Lk, d]
    kv_segs    P segment lists, the global positions of each rank's block
    order      source rank per step (default: the ring, (rank - s) mod P)
    prefetch   True: pass the next block on `copy_stream` while the current
               step computes; False: pass it on the compute stream first
    finalize   True: the last step writes out and lse (the state is then left
               as it was before the last block); False: every step updates the
               state and out / lse are not written
    returns (out [B, H, Lq, d] in q's dtype, lse [B, H, Lq] fp32, state)
    """
    P = len(kv_blocks)
    if order is None:
        order = layout.ring_order(rank, P)
    if sorted(order) != list(range(P)):
        raise ValueError("order must visit every block once")
    B, H, Lq, d = q.shape
    dev = q.device
    if scale is None:
        scale = 1.0 / d ** 0.5
    compute = torch.cuda.current_stream(dev)
    if state is None:
        state = RingState(B, H, Lq, d, dev)
    if out is None and finalize:
        out = torch.empty_like(q)
    if lse is None and finalize:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)

    needs_pass = [t != rank for t in order]
    if any(needs_pass) and bufs is None:
        k0, v0 = kv_blocks[0]
        bufs = [(torch.empty_like(k0), torch.empty_like(v0)) for _ in range(2)]
    if prefetch and any(needs_pass):
        if copy_stream is None:
            copy_stream = torch.cuda.Stream(dev)
        copy_stream.wait_stream(compute)  # inputs written on the compute stream
        for kb, vb in bufs:
            kb.record_stream(copy_stream)
            vb.record_stream(copy_stream)
    ev_ready = [torch.cuda.Event(), torch.cuda.Event()]
    ev_free = [torch.cuda.Event(), torch.cuda.Event()]
    used = [False, False]

    def pass_block(s):
        slot = s % 2
        src_k, src_v = kv_blocks[order[s]]
        dst_k, dst_v = bufs[slot]
        if prefetch:
            if used[slot]:
                copy_stream.wait_event(ev_free[slot])
            _lib.ra_kv_pass(src_k, src_v, dst_k, dst_v, stream=copy_stream)
            ev_ready[slot].record(copy_stream)
        else:
            _lib.ra_kv_pass(src_k, src_v, dst_k, dst_v, stream=compute)

    if prefetch and needs_pass[0]:
        pass_block(0)
    for s in range(P):
        if prefetch and s + 1 < P and needs_pass[s + 1]:
            pass_block(s + 1)
        if needs_pass[s]:
            if prefetch:
                compute.wait_event(ev_ready[s % 2])
            else:
                pass_block(s)
            k, v = bufs[s % 2]
        else:
            k, v = kv_blocks[order[s]]
        if step_events is not None:
            step_events[s][0].record(compute)
        if finalize and s == P - 1:
            # the last block: the output is written straight from the kernel
            # (the state is left as the previous steps wrote it)
            _lib.ra_step_final(q, k, v, q_segs, kv_segs[order[s]], causal, scale,
                               state.o, state.m, state.l, out, lse, init=(s == 0), stream=compute)
        else:
            _lib.ra_step(q, k, v, q_segs, kv_segs[order[s]], causal, scale,
                         state.o, state.m, state.l, init=(s == 0), stream=compute)
        if step_events is not None:
            step_events[s][1].record(compute)
        # the slot is free again after this step; only a later block passed
        # into the same slot waits for that (an event record costs a queue packet)
        if prefetch and needs_pass[s] and any(needs_pass[s + 2::2]):
            ev_free[s % 2].record(compute)
            used[s % 2] = True
    return out, lse, state


def group_half(x: torch.Tensor, H_kv: int, p: int) -> torch.Tensor:
    """Half p (0 or 1) of every K/V head's query heads of x [B, H, ...], as a
    contiguous [B, H/2, ...] tensor. Query head h belongs to K/V head h // G
    (G = H / H_kv, even); half p holds heads j*G + p*G/2 .. j*G + (p+1)*G/2 - 1
    of every group j, so that K/V head j of the half serves its heads
    j*G/2 .. (j+1)*G/2 - 1, the grouping the kernels assume."""
    B, H = x.shape[:2]
    G = H // H_kv
    if G * H_kv != H or G % 2:
        raise ValueError("group_half needs an even number of query heads per K/V head")
    g = x.reshape(B, H_kv, G, *x.shape[2:])[:, :, p * (G // 2):(p + 1) * (G // 2)]
    return g.reshape(B, H // 2, *x.shape[2:]).contiguous()


def run_bwd(q: torch.Tensor,
            q_segs: Sequence[Tuple[int, int]],
            kv_blocks: Sequence[Tuple[torch.Tensor, torch.Tensor]],
            kv_segs: Sequence[Sequence[Tuple[int, int]]],
            rank: int,
            causal: bool,
            out: torch.Tensor,
            lse: torch.Tensor,
            dout: torch.Tensor,
            scale: Optional[float] = None,
            order: Optional[List[int]] = None,
            dkv: Optional[List[Tuple[torch.Tensor, torch.Tensor]]] = None,
            overlap: Optional[bool] = None,
            split: bool = False):
    """Backward pass of rank `rank`'s share: P backward block steps.

    The ring passes the K/V blocks again in the backward pass (k8ai
    "Communication profile"), each now travelling with its dK/dV
    accumulators. At step s the rank adds its queries' contributions to the
    block of rank order[s] with ``ra_step_bwd``; dQ stays local.

    out, lse   the final forward output and lse of the local queries
    dout       upstream gradient of `out`
    dkv        optional per-block (dk, dv) fp32 accumulators [B, H, Lk, d] that
               already hold other ranks' contributions (they are added to);
               None: fresh accumulators holding this rank's contributions only
    overlap    run the dK/dV half of every step on a second stream, beside the
               chain of dQ halves on the current stream (each block's dK/dV
               depends on no other step), and make the current stream wait for
               it before returning; the gradients are bitwise the same. None
               (the default): only when the blocks have fewer K/V heads than
               q has heads. Then the dK/dV kernel is a single round of
               workgroups whose causal imbalance leaves CUs idle, which the
               other stream's dQ workgroups fill; with one K/V head per query
               head the two kernels only trade CUs and the second stream is
               slower
    split      on the step against the rank's own block (the diagonal: under
               the causal mask its key tiles see very different numbers of
               queries), run the dK/dV half as two launches on two streams,
               each over half of every K/V head's query heads (the group,
               H / H_kv, must be even), the second into a partial accumulator
               that is then added in. With grouped heads the dK/dV grid has
               one workgroup per key tile and K/V head, as many as there are
               CUs at the 32K share, so the diagonal's heaviest tiles set that
               kernel's time, and the halves cut it by 28%; but the whole pass
               is not faster, since the dQ kernels on the other stream already
               fill the CUs that the light tiles leave idle, and the copies of
               the halves cost more than is left. Off by default. The
               gradients equal the unsplit ones up to the order of the fp32
               sums. Refused under graph capture: a captured pass with it (a
               third stream forked from the dK/dV stream and joined back into
               it) ended in a crash inside the runtime's end of capture whose
               cause is not known
    returns (dq [B, H, Lq, d] fp32, dkv)
    """
    P = len(kv_blocks)
    if order is None:
        order = layout.ring_order(rank, P)
    if sorted(order) != list(range(P)):
        raise ValueError("order must visit every block once")
    B, H, Lq, d = q.shape
    dev = q.device
    if scale is None:
        scale = 1.0 / d ** 0.5
    H_kv = kv_blocks[0][0].shape[1]
    G = H // H_kv
    if split and (G % 2 != 0 or G * H_kv != H):
        raise ValueError("split needs an even number of query heads per K/V head")
    stream = torch.cuda.current_stream(dev)
    if split and torch.cuda.is_current_stream_capturing():
        raise RuntimeError("the split diagonal step is not supported under graph capture")
    if overlap is None:
        overlap = H_kv < H
    fresh = dkv is None
    if fresh:
        dkv = [(torch.empty(k.shape, dtype=torch.float32, device=dev),
                torch.empty(k.shape, dtype=torch.float32, device=dev)) for k, _ in kv_blocks]
    delta = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    _lib.ra_bwd_prep(out, dout, delta, stream=stream)
    dq = torch.empty((B, H, Lq, d), dtype=torch.float32, device=dev)
    halves = None
    if split and rank in order:
        halves = [tuple(group_half(x, H_kv, p) for x in (q, dout, lse, delta)) for p in (0, 1)]
        # a stand-in of the right shape for the halves' dq argument, which the
        # dK/dV-only launches neither read nor write
        dq_unused = dq.view(-1)[:dq.numel() // 2].view(B, H // 2, Lq, d)
        part = (torch.empty(kv_blocks[rank][0].shape, dtype=torch.float32, device=dev),
                torch.empty(kv_blocks[rank][0].shape, dtype=torch.float32, device=dev))
        split_stream = torch.cuda.Stream(dev)
        for x in (*halves[1], *part, *kv_blocks[rank], dq):
            x.record_stream(split_stream)
    side = None
    if overlap:
        side = torch.cuda.Stream(dev)
        ready = torch.cuda.Event()
        ready.record(stream)  # delta and every input are in place
        side.wait_event(ready)
        for x in (q, dout, lse, delta):
            x.record_stream(side)
        for (k, v), (dk, dv) in zip(kv_blocks, dkv):
            for x in (k, v, dk, dv):
                x.record_stream(side)
        if halves is not None:
            for x in (*halves[0], *part, dq):
                x.record_stream(side)
    for s in range(P):
        t = order[s]
        k, v = kv_blocks[t]
        dk, dv = dkv[t]
        args = (q, k, v, dout, lse, delta, q_segs, kv_segs[t], causal, scale, dq, dk, dv)
        if halves is not None and t == rank:
            kv_stream = stream if side is None else side
            split_stream.wait_stream(kv_stream)  # the halves, and earlier steps' writes to dk, dv
            _lib.ra_step_bwd(*args, init_dq=(s == 0), init_dkv=fresh, stream=stream, parts="dq")
            for p, (qh, doh, lh, dh) in enumerate(halves):
                acc = (dk, dv) if p == 0 else part
                _lib.ra_step_bwd(qh, k, v, doh, lh, dh, q_segs, kv_segs[t], causal, scale, dq_unused, *acc,
                                 init_dkv=(fresh if p == 0 else True), parts="dkv",
                                 stream=(kv_stream if p == 0 else split_stream))
            kv_stream.wait_stream(split_stream)
            _lib.ra_add_rows(part[0], 0, dk, 0, k.shape[2], stream=kv_stream)
            _lib.ra_add_rows(part[1], 0, dv, 0, k.shape[2], stream=kv_stream)
        elif side is None:
            _lib.ra_step_bwd(*args, init_dq=(s == 0), init_dkv=fresh, stream=stream)
        else:
            _lib.ra_step_bwd(*args, init_dq=(s == 0), init_dkv=fresh, stream=side, parts="dkv")
            _lib.ra_step_bwd(*args, init_dq=(s == 0), init_dkv=fresh, stream=stream, parts="dq")
    if side is not None:
        done = torch.cuda.Event()
        done.record(side)
        stream.wait_event(done)
    return dq, dkv

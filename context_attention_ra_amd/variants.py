"""The alternatives to the ring that the pages name, one rank's share on one GPU.

* All-gather: the Ultralytics glossary ("How Context Parallelism Works") lists
  all-gather and reduce-scatter next to ring-based exchange of K/V blocks.
  Every rank gathers all K/V blocks at their global positions, then attends
  its local queries to the whole sequence in one step. In the backward pass
  each rank's gradient of the gathered K/V covers every position; a
  reduce-scatter sums those over the ranks into the rows each rank owns.
* All-to-all on heads: in the scheme of the k8ai page ("An alternative:
  all-to-all on heads") the ranks trade their token ranges for head groups
  before the attention and trade back after it, so the number of heads bounds
  how many ranks can take part. Rank g holds every position of heads
  [g*H/P, (g+1)*H/P) and runs plain attention on them.

The exchanges are simulated by ``ra_copy_rows`` (strided device-to-device
copies on the current stream); the attention itself is the library's step
kernel with the finalize folded in (``ra_step_final``) over one block that
covers the whole sequence. Host control only: every byte moves in libra.
"""

from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib
from .ring import RingState

Segs = Sequence[Tuple[int, int]]


def _global_length(segs: Sequence[Segs]) -> int:
    """Length of the sequence the segments of all ranks tile exactly once."""
    runs = sorted((s, n) for sg in segs for s, n in sg)
    pos = 0
    for s, n in runs:
        if s != pos:
            raise ValueError("the ranks' segments must cover 0..S-1 exactly once")
        pos += n
    return pos


def gather_kv(kv_blocks: Sequence[Tuple[torch.Tensor, torch.Tensor]], kv_segs: Sequence[Segs],
              stream=None):
    """All-gather of K/V: every rank's block placed at its global positions.

    kv_blocks  P pairs (k_t, v_t) [B, H_kv, L_t, d]; kv_segs their global positions
    returns (k, v) [B, H_kv, S, d] in global position order
    """
    S = _global_length(kv_segs)
    k0, v0 = kv_blocks[0]
    B, Hkv, _, d = k0.shape
    kg = torch.empty((B, Hkv, S, d), dtype=k0.dtype, device=k0.device)
    vg = torch.empty_like(kg)
    for (k, v), segs in zip(kv_blocks, kv_segs):
        off = 0
        for start, n in segs:
            _lib.ra_copy_rows(k, off, kg, start, n, stream=stream)
            _lib.ra_copy_rows(v, off, vg, start, n, stream=stream)
            off += n
    return kg, vg


def run_allgather(q: torch.Tensor, q_segs: Segs,
                  kv_blocks: Sequence[Tuple[torch.Tensor, torch.Tensor]], kv_segs: Sequence[Segs],
                  causal: bool, scale: Optional[float] = None):
    """One rank's share under all-gather: its queries against the gathered K/V.

    returns (out [B, H, Lq, d] in q's dtype, lse [B, H, Lq] fp32)
    """
    B, H, Lq, d = q.shape
    if scale is None:
        scale = 1.0 / d ** 0.5
    stream = torch.cuda.current_stream(q.device)
    kg, vg = gather_kv(kv_blocks, kv_segs, stream=stream)
    S = kg.shape[2]
    st = RingState(B, H, Lq, d, q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    _lib.ra_step_final(q, kg, vg, q_segs, [(0, S)], causal, scale, st.o, st.m, st.l, out, lse,
                       init=True, stream=stream)
    return out, lse


def allgather_bwd(q: torch.Tensor, q_segs: Segs,
                  kv_blocks: Sequence[Tuple[torch.Tensor, torch.Tensor]], kv_segs: Sequence[Segs],
                  causal: bool, out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                  scale: Optional[float] = None):
    """Backward pass of one rank's share under all-gather.

    The rank's queries saw the gathered K/V, so its backward step yields dQ
    for its own rows and this rank's contribution to dK and dV at every global
    position; ``reduce_scatter`` then sums those contributions over the ranks
    into the rows each rank owns (the adjoint of the gather).

    out, lse   the rank's forward output and lse (``run_allgather``)
    dout       upstream gradient of `out`
    returns (dq [B, H, Lq, d] fp32, dk, dv [B, H_kv, S, d] fp32, global order)
    """
    B, H, Lq, d = q.shape
    if scale is None:
        scale = 1.0 / d ** 0.5
    stream = torch.cuda.current_stream(q.device)
    kg, vg = gather_kv(kv_blocks, kv_segs, stream=stream)
    S = kg.shape[2]
    delta = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    _lib.ra_bwd_prep(out, dout, delta, stream=stream)
    dq = torch.empty((B, H, Lq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty(kg.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    _lib.ra_step_bwd(q, kg, vg, dout, lse, delta, q_segs, [(0, S)], causal, scale, dq, dk, dv,
                     init_dq=True, init_dkv=True, stream=stream)
    return dq, dk, dv


def reduce_scatter(partials: Sequence[torch.Tensor], segs: Sequence[Segs], stream=None) -> List[torch.Tensor]:
    """Reduce-scatter over the ranks: rank t receives the sum of every rank's
    partial at the global positions it owns.

    partials  P fp32 tensors [B, Hb, S, d] in global position order (one per rank)
    segs      the ranks' global positions
    returns   P fp32 tensors [B, Hb, L_t, d], rows in rank t's storage order
    """
    B, Hb, S, d = partials[0].shape
    if _global_length(segs) != S:
        raise ValueError("the segments must tile the partials' sequence")
    outs = []
    for sg in segs:
        L = sum(n for _, n in sg)
        y = torch.empty((B, Hb, L, d), dtype=torch.float32, device=partials[0].device)
        off = 0
        for start, n in sg:
            _lib.ra_copy_rows(partials[0], start, y, off, n, stream=stream)
            for p in partials[1:]:
                _lib.ra_add_rows(p, start, y, off, n, stream=stream)
            off += n
        outs.append(y)
    return outs


def heads_to_group(blocks: Sequence[torch.Tensor], segs: Sequence[Segs], g: int, P: int, stream=None):
    """All-to-all from the sequence split to the head split: group g's heads
    [g*Hb/P, (g+1)*Hb/P) at every position, in global order.

    blocks  P tensors [B, Hb, L_t, d], rank t's rows at segs[t]
    returns [B, Hb/P, S, d]
    """
    B, Hb, _, d = blocks[0].shape
    if Hb % P:
        raise ValueError(f"the head count {Hb} must be a multiple of the group count {P}")
    hg = Hb // P
    S = _global_length(segs)
    dst = torch.empty((B, hg, S, d), dtype=blocks[0].dtype, device=blocks[0].device)
    for x, sg in zip(blocks, segs):
        off = 0
        for start, n in sg:
            for b in range(B):
                _lib.ra_copy_rows(x, off, dst, start, n, src_slice0=b * Hb + g * hg,
                                  dst_slice0=b * hg, nslices=hg, stream=stream)
            off += n
    return dst


def group_to_ranks(y: torch.Tensor, g: int, P: int, segs: Sequence[Segs], outs: List[torch.Tensor],
                   stream=None):
    """The all-to-all back: rows of head group g (y [B, H/P, S, d], global order)
    into every rank's sequence-split tensor outs[t] [B, H, L_t, d] (heads g*H/P..)."""
    B, hg, _, d = y.shape
    H = outs[0].shape[1]
    for x, sg in zip(outs, segs):
        off = 0
        for start, n in sg:
            for b in range(B):
                _lib.ra_copy_rows(y, start, x, off, n, src_slice0=b * hg, dst_slice0=b * H + g * hg,
                                  nslices=hg, stream=stream)
            off += n


def run_head_group(q_blocks: Sequence[torch.Tensor],
                   kv_blocks: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                   segs: Sequence[Segs], g: int, causal: bool, scale: Optional[float] = None):
    """Rank g's share under the all-to-all on heads: its head group over the
    whole sequence (grouped K/V heads split over the ranks the same way).

    q_blocks   P sequence-split query tensors [B, H, L_t, d]
    kv_blocks  P sequence-split (k, v) [B, H_kv, L_t, d]
    returns (out [B, H/P, S, d], lse [B, H/P, S]) in global position order
    """
    P = len(q_blocks)
    d = q_blocks[0].shape[3]
    if scale is None:
        scale = 1.0 / d ** 0.5
    stream = torch.cuda.current_stream(q_blocks[0].device)
    qh = heads_to_group(q_blocks, segs, g, P, stream=stream)
    kh = heads_to_group([k for k, _ in kv_blocks], segs, g, P, stream=stream)
    vh = heads_to_group([v for _, v in kv_blocks], segs, g, P, stream=stream)
    B, hg, S, _ = qh.shape
    st = RingState(B, hg, S, d, qh.device)
    out = torch.empty_like(qh)
    lse = torch.empty((B, hg, S), dtype=torch.float32, device=qh.device)
    _lib.ra_step_final(qh, kh, vh, [(0, S)], [(0, S)], causal, scale, st.o, st.m, st.l, out, lse,
                       init=True, stream=stream)
    return out, lse

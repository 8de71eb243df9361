"""Context-parallel attention over a whole sequence, every rank simulated on one GPU.

The Ultralytics glossary's example ("Practical Use and Tradeoffs") shards the
query, key and value buffers along the sequence dimension and lets each rank
run its attention; the pages' ring then hands every rank the K/V blocks of the
others (Day 83 post, "Context parallelism: splitting the sequence"; k8ai "How
context parallel works"). ``context_parallel_attention`` does the same on one
GPU: it splits full-sequence [B, H, S, d] tensors into the ranks' shares
(contiguous, zigzag or temporal-first), runs every rank's ring with
``ring.run``, and puts the outputs back in global order. The splitting and
reassembly are ``ra_copy_rows`` copies; the attention is the library's ring
step. Host control only.
"""

from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib, layout, ring

Segs = Sequence[Tuple[int, int]]


def shard(x: torch.Tensor, segs: Sequence[Segs]) -> List[torch.Tensor]:
    """The ranks' shares of a full-sequence tensor x [..., S, w]: rank r's rows
    are the positions of segs[r], in segment order."""
    parts = []
    for sg in segs:
        L = sum(n for _, n in sg)
        part = torch.empty((*x.shape[:-2], L, x.shape[-1]), dtype=x.dtype, device=x.device)
        off = 0
        for start, n in sg:
            _lib.ra_copy_rows(x, start, part, off, n)
            off += n
        parts.append(part)
    return parts


def unshard(parts: Sequence[torch.Tensor], segs: Sequence[Segs], S: int) -> torch.Tensor:
    """Inverse of ``shard``: the ranks' rows put back at their global positions."""
    x = torch.empty((*parts[0].shape[:-2], S, parts[0].shape[-1]), dtype=parts[0].dtype,
                    device=parts[0].device)
    for part, sg in zip(parts, segs):
        off = 0
        for start, n in sg:
            _lib.ra_copy_rows(part, off, x, start, n)
            off += n
    return x


def context_parallel_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: int,
                               split: str = "zigzag", causal: bool = True,
                               scale: Optional[float] = None, S_sp: int = 0):
    """Attention of a whole sequence computed as P ranks' ring shares.

    q [B, H, S, d], k, v [B, H_kv, S, d] (H a multiple of H_kv); split is
    "contiguous", "zigzag" or "temporal" (frames of S_sp tokens).
    returns (out [B, H, S, d] in q's dtype, lse [B, H, S] fp32), both in
    global position order: the same result as attention over the whole
    sequence, up to rounding.
    """
    S = q.shape[2]
    segs = [layout.split(split, S, P, r, S_sp=S_sp) for r in range(P)]
    qs = shard(q, segs)
    kv = list(zip(shard(k, segs), shard(v, segs)))
    outs, lses = [], []
    for r in range(P):
        out, lse, _ = ring.run(qs[r], segs[r], kv, segs, r, causal, scale=scale)
        outs.append(out)
        lses.append(lse.unsqueeze(-1))
    return unshard(outs, segs, S), unshard(lses, segs, S)[..., 0]


class _Shard(torch.autograd.Function):
    """``shard`` with the reassembly of the shares' gradients as its backward."""

    @staticmethod
    def forward(ctx, x, segs):
        ctx.segs, ctx.S = segs, x.shape[-2]
        return tuple(shard(x, segs))

    @staticmethod
    def backward(ctx, *grads):
        parts = [g.contiguous() for g in grads]
        return unshard(parts, ctx.segs, ctx.S), None


class _Unshard(torch.autograd.Function):
    """``unshard`` with the split of the output gradient as its backward."""

    @staticmethod
    def forward(ctx, segs, S, *parts):
        ctx.segs = segs
        return unshard(parts, segs, S)

    @staticmethod
    def backward(ctx, g):
        return (None, None, *shard(g.contiguous(), ctx.segs))


def cp_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: int, split: str = "zigzag",
                 causal: bool = True, scale: Optional[float] = None, S_sp: int = 0) -> torch.Tensor:
    """``context_parallel_attention`` as a differentiable operation (bf16).

    Returns the output [B, H, S, d] in global order; ``backward`` runs every
    rank's backward ring and returns whole-sequence gradients of q, k and v
    (the K/V block gradients of all ranks added, as the travelling dK/dV of a
    real ring are).
    """
    from .autograd import ring_attention

    S = q.shape[2]
    segs = [layout.split(split, S, P, r, S_sp=S_sp) for r in range(P)]
    qs = _Shard.apply(q, segs)
    ks = _Shard.apply(k, segs)
    vs = _Shard.apply(v, segs)
    kv = list(zip(ks, vs))
    outs = [ring_attention(qs[r], segs[r], kv, segs, r, causal, scale=scale) for r in range(P)]
    return _Unshard.apply(segs, S, *outs)

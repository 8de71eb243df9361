"""One rank's ring attention as a differentiable PyTorch operation.

The Ultralytics glossary's example ("Practical Use and Tradeoffs") trains
through the attention, and the k8ai page ("Communication profile") has the
ring pass K/V blocks in the backward pass as well. ``ring_attention`` runs the
forward ring (``ring.run``) and, on ``backward``, the backward ring
(``ring.run_bwd``): the gradient of the local queries, and this rank's
contributions to the gradients of every K/V block it attended to. When several
ranks' shares are computed on one GPU from the same block tensors, autograd
adds the ranks' contributions to each block's gradient, which is what the
travelling dK/dV accumulators of a real ring produce.

Host control only: the forward and backward arithmetic runs in libra.
"""

from typing import Optional, Sequence, Tuple

import torch

from . import ring


class _RingAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, q_segs, kv_segs, rank, causal, scale, order, *kv_flat):
        kv = [(kv_flat[2 * i], kv_flat[2 * i + 1]) for i in range(len(kv_flat) // 2)]
        out, lse, _ = ring.run(q, q_segs, kv, kv_segs, rank, causal, scale=scale, order=order)
        ctx.save_for_backward(q, out, lse, *kv_flat)
        ctx.meta = (q_segs, kv_segs, rank, causal, scale, order)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, out, lse, *kv_flat = ctx.saved_tensors
        q_segs, kv_segs, rank, causal, scale, order = ctx.meta
        kv = [(kv_flat[2 * i], kv_flat[2 * i + 1]) for i in range(len(kv_flat) // 2)]
        dq, dkv = ring.run_bwd(q, q_segs, kv, kv_segs, rank, causal, out, lse, dout.contiguous(),
                               scale=scale, order=order)
        # fp32 gradients; autograd converts them to each input's dtype
        grads = [g for pair in dkv for g in pair]
        return (dq, None, None, None, None, None, None, *grads)


def ring_attention(q: torch.Tensor, q_segs: Sequence[Tuple[int, int]],
                   kv_blocks: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                   kv_segs: Sequence[Sequence[Tuple[int, int]]], rank: int, causal: bool,
                   scale: Optional[float] = None, order=None) -> torch.Tensor:
    """Rank `rank`'s share of ring attention, differentiable in q and every K/V block.

    Arguments as ``ring.run`` (bf16 tensors for the backward pass). Returns the
    output [B, H, Lq, d]; its backward gives q.grad and each block's k.grad and
    v.grad (this rank's contributions, added to what autograd already holds).
    """
    if scale is None:
        scale = 1.0 / q.shape[-1] ** 0.5
    flat = [t for pair in kv_blocks for t in pair]
    return _RingAttention.apply(q, q_segs, kv_segs, rank, causal, scale, order, *flat)

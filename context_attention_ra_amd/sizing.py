"""Algorithmic work and the pages' sizing arithmetic.

Work is counted per unmasked (query, key) pair: 2*d FLOP for the score and
2*d FLOP for the value product, so 4*d FLOP per pair. Masked pairs, skipped
tiles, padding and the softmax itself are not counted.
"""

from typing import Sequence, Tuple

import numpy as np

Segs = Sequence[Tuple[int, int]]


def causal_pairs(q_segs: Segs, k_segs: Segs) -> int:
    """Number of (q, k) pairs with global pos(k) <= pos(q)."""
    total = 0
    for qa, qn in q_segs:
        qpos = np.arange(qa, qa + qn, dtype=np.int64)
        for kb, km in k_segs:
            total += int(np.clip(qpos - kb + 1, 0, km).sum())
    return total


def pairs(q_segs: Segs, k_segs: Segs, causal: bool) -> int:
    if not causal:
        return sum(n for _, n in q_segs) * sum(m for _, m in k_segs)
    return causal_pairs(q_segs, k_segs)


def attention_flop(n_pairs: int, d: int, batch_heads: int) -> float:
    return 4.0 * d * n_pairs * batch_heads


# ---- the pages' own back-of-envelope figures (Day 83 post) -------------------

def video_tokens(frames: int, spatial_tokens: int) -> int:
    """Frame-major token count (Day 83 post, intro and "What the numbers look like")."""
    return frames * spatial_tokens


def spatial_tokens_720p_vae() -> int:
    """720p frame after 16x16 downsampling: (720//16) * (1280//16)."""
    return (720 // 16) * (1280 // 16)


def attn_matrix_bytes(tokens: int, bytes_per_el: int = 2) -> int:
    """Bytes of a materialised tokens x tokens score matrix for one head."""
    return tokens * tokens * bytes_per_el


def kv_bytes_per_step_per_head(L: int, d: int, bytes_per_el: int = 2) -> int:
    """K and V of one local block for one head (Day 83 post, "The communication pattern")."""
    return 2 * L * d * bytes_per_el


def ring_comm_bytes(L: int, d: int, heads: int, P: int, bytes_per_el: int = 2) -> int:
    """K/V bytes one rank sends over the P-1 ring transfers of one layer."""
    return kv_bytes_per_step_per_head(L, d, bytes_per_el) * heads * (P - 1)


def comm_seconds(nbytes: float, link_bytes_per_s: float) -> float:
    return nbytes / link_bytes_per_s

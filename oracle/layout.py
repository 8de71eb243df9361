"""Which global token positions a rank holds, and which block it sees per ring step.

Integer bookkeeping of the pages' partitions, written from their prose
(test infrastructure; see the package docstring for who may use it).
"""

import numpy as np


def contiguous_positions(S, P, r):
    """Plain sequence split: rank r holds tokens [r*S/P, (r+1)*S/P).

    Day 83 post, "Context parallelism: splitting the sequence" (each GPU holds
    about S/P tokens); Ultralytics glossary, "How Context Parallelism Works".
    """
    if S % P:
        raise ValueError("S must be divisible by P")
    L = S // P
    return np.arange(r * L, (r + 1) * L, dtype=np.int64)


def zigzag_positions(S, P, r):
    """Balanced causal split.

    k8ai, "How context parallel works": under a causal mask the sequence is cut
    into chunks handed out in a balanced pattern so that every GPU gets a
    similar amount of work. Reading taken: 2P equal chunks of C = S/(2P)
    tokens; rank r stores chunk r followed by chunk 2P-1-r (an early chunk
    paired with its mirror-image late chunk).
    """
    if S % (2 * P):
        raise ValueError("S must be divisible by 2P")
    C = S // (2 * P)
    early = np.arange(r * C, (r + 1) * C, dtype=np.int64)
    late_chunk = 2 * P - 1 - r
    late = np.arange(late_chunk * C, (late_chunk + 1) * C, dtype=np.int64)
    return np.concatenate([early, late])


def temporal_first_positions(T, S_sp, P, r):
    """Temporal-first video split: rank r holds whole consecutive frames.

    Day 83 post, "The spatial-temporal twist": each GPU gets a contiguous run
    of frames rather than scattered patches. Tokens are frame-major
    (index = t * S_sp + s), so rank r holds frames [r*T/P, (r+1)*T/P).
    """
    if T % P:
        raise ValueError("T must be divisible by P")
    F = T // P
    return np.arange(r * F * S_sp, (r + 1) * F * S_sp, dtype=np.int64)


def ring_source(r, s, P):
    """Rank whose K/V block rank r holds at ring step s.

    k8ai, "How context parallel works" (ring figure): at step 0 every GPU uses
    its own block; at step 1 GPU0 has block 3, GPU1 block 0, and so on — each
    GPU receives from its predecessor. Hence the block at step s comes from
    rank (r - s) mod P.
    """
    return (r - s) % P

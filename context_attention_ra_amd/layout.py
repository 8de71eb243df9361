"""Segment maps of one rank's share, in the form the library's ``ra_segs`` takes.

A rank stores its tokens as up to two runs of consecutive global positions;
row i of a local tensor sits at global position start[k] + (i - rows before
segment k). These maps feed the causal mask, which compares global positions,
so the kernels never need to know which split produced them.

* contiguous: Day 83 post, "Context parallelism: splitting the sequence".
* zigzag: k8ai, "How context parallel works" — under a causal mask the chunks
  are handed out in a balanced pattern. Reading: 2P chunks of S/(2P) tokens;
  rank r holds chunk r, then chunk 2P-1-r.
* temporal-first: Day 83 post, "The spatial-temporal twist" — each rank holds a
  run of whole frames of a frame-major token sequence.
* ring order: k8ai ring figure — at step s rank r holds the block of rank
  (r - s) mod P.
"""

from typing import List, Tuple

Segs = List[Tuple[int, int]]  # [(global start, length), ...]


def contiguous(S: int, P: int, r: int) -> Segs:
    if S % P or not 0 <= r < P:
        raise ValueError(f"contiguous split needs S % P == 0 and 0 <= r < P (S={S}, P={P}, r={r})")
    L = S // P
    return [(r * L, L)]


def zigzag(S: int, P: int, r: int) -> Segs:
    if S % (2 * P) or not 0 <= r < P:
        raise ValueError(f"zigzag split needs S % 2P == 0 and 0 <= r < P (S={S}, P={P}, r={r})")
    C = S // (2 * P)
    return [(r * C, C), ((2 * P - 1 - r) * C, C)]


def temporal_first(T: int, S_sp: int, P: int, r: int) -> Segs:
    if T % P or not 0 <= r < P:
        raise ValueError(f"temporal-first split needs T % P == 0 (T={T}, P={P}, r={r})")
    F = T // P
    return [(r * F * S_sp, F * S_sp)]


def split(kind: str, S: int, P: int, r: int, S_sp: int = 0) -> Segs:
    if kind == "contiguous":
        return contiguous(S, P, r)
    if kind == "zigzag":
        return zigzag(S, P, r)
    if kind == "temporal":
        if S_sp <= 0 or S % S_sp:
            raise ValueError("temporal-first split needs S_sp dividing S")
        return temporal_first(S // S_sp, S_sp, P, r)
    raise ValueError(f"unknown split {kind!r}")


def ring_order(r: int, P: int) -> List[int]:
    """Source rank of the K/V block used at each step s = 0..P-1."""
    return [(r - s) % P for s in range(P)]


def rows(segs: Segs) -> int:
    return sum(n for _, n in segs)


def local_rows_of(segs: Segs, global_positions):
    """Local row indices of the given global positions (each must be held)."""
    out = []
    for g in global_positions:
        off = 0
        for st, n in segs:
            if st <= g < st + n:
                out.append(off + g - st)
                break
            off += n
        else:
            raise ValueError(f"position {g} not held by these segments")
    return out

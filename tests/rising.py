"""Inputs whose scores rise along the key sequence, and a check that they make
the matrix-core kernels move their running maximum part-way.

The online-softmax accumulation of the Day 83 post ("Context parallelism:
splitting the sequence") rescales the running output and sum by
alpha = exp(m_old - m_new) whenever a new block raises a row's maximum. The
bf16 ring-step kernel moves its reference value only when a 64-key tile's row
maximum exceeds it by more than 8 (log2 units of the scaled scores); with
N(0,1) inputs at scale 1/sqrt(d) that almost never happens after the first
tile, so alpha is 0 (first tile) or 1 in every other test. These inputs make
it happen many times per row:

* queries are N(0,1) times `q_gain`;
* the key at global position p is N(0,1) times lo * (hi / lo) ** (p / S), so
  the typical score grows geometrically along the sequence;
* values are N(0,1).

All draws come from ``seeded``; the gains are applied in float32 before the
rounding to bf16, and both the GPU and the oracle see the same bf16 values.

``partial_rescales`` replays the kernel's trigger on the CPU (per row: the
maximum of every 64-key tile of every block in ring order, against the
reference value carried across steps) and counts the triggers with a finite
previous reference, i.e. 0 < alpha < 1. It only checks that the inputs do
what they are meant to do; expected outputs come from the oracle alone.
"""

import numpy as np
import torch

import seeded

LOG2E = 1.4426950408889634
TAU = 8.0      # the kernel's rescale threshold, log2 units
TILE = 64      # keys per tile of the kernel


def key_gain(pos, S, lo, hi):
    return (lo * (hi / lo) ** (np.asarray(pos, dtype=np.float64) / S)).astype(np.float32)


def rising_global(wid, B, H, Hkv, S, d, q_gain=4.0, lo=0.25, hi=4.0, key_pos=None, span=None,
                  gains=None, dtype=torch.bfloat16):
    """CPU tensors q [B,H,S,d], k, v [B,Hkv,S,d] of the rising recipe. Key row p
    is scaled by the gain at key_pos[p] of `span` (default: p of S); factored
    spatial inputs pass the position inside the frame and the frame size.
    `gains` (S,) replaces the geometric gains by explicit ones."""
    key_pos = np.arange(S) if key_pos is None else np.asarray(key_pos)
    if gains is None:
        g = key_gain(key_pos, S if span is None else span, lo, hi)[:, None]
    else:
        g = np.asarray(gains, dtype=np.float32)[:, None]
    q = torch.empty((B, H, S, d), dtype=dtype)
    k = torch.empty((B, Hkv, S, d), dtype=dtype)
    v = torch.empty((B, Hkv, S, d), dtype=dtype)
    for b in range(B):
        for h in range(H):
            q[b, h] = seeded.to_dtype(q_gain * seeded.normal_rows(wid, seeded.Q, b, h, 0, S, d), dtype)
        for h in range(Hkv):
            k[b, h] = seeded.to_dtype(g * seeded.normal_rows(wid, seeded.K, b, h, 0, S, d), dtype)
            v[b, h] = seeded.to_dtype(seeded.normal_rows(wid, seeded.V, b, h, 0, S, d), dtype)
    return q, k, v


def partial_rescales(q, qpos, blocks, scale, causal, mu0=None):
    """Count, per query row, the kernel's rescales with 0 < alpha < 1.

    q       (n, d) float64 query rows; qpos (n,) their global positions
    blocks  [(k (Lk, d) float64, kpos (Lk,)), ...] in the order the kernel
            sees them (one entry per ring step)
    mu0     reference value carried in (log2 units), default -inf
    returns (counts (n,), mu (n,) the reference after the last block)
    """
    n = q.shape[0]
    mu = np.full(n, -np.inf) if mu0 is None else np.array(mu0, dtype=np.float64)
    count = np.zeros(n, dtype=np.int64)
    for k, kpos in blocks:
        s = (q @ k.T) * (scale * LOG2E)
        if causal:
            s = np.where(np.asarray(kpos)[None, :] <= np.asarray(qpos)[:, None], s, -np.inf)
        Lk = k.shape[0]
        nt = (Lk + TILE - 1) // TILE
        pad = np.full((n, nt * TILE - Lk), -np.inf)
        tmax = np.concatenate([s, pad], axis=1).reshape(n, nt, TILE).max(axis=2)
        for t in range(nt):
            mt = tmax[:, t]
            need = mt > mu + TAU
            with np.errstate(invalid="ignore"):
                count += need & np.isfinite(mu) & (mt - mu < 120.0)
            mu = np.where(need, mt, mu)
    return count, mu


def emulate_lazy_softmax(q, qpos, blocks, scale, causal, bug=None):
    """The bf16 kernels' accumulation order in fp64, optionally with a planted mistake.

    Per row: for each block (ring step) and each 64-key tile in order, the
    reference value mu moves to the tile maximum only when that exceeds it by
    more than TAU; O and l are then multiplied by alpha = 2^(mu_old - mu_new);
    the tile's weights are 2^(s - mu). ``bug`` plants one mistake in the
    rescale: "l_not_rescaled", "o_not_rescaled", "alpha_natural" (e^ instead
    of 2^) or "mu_not_carried" (the reference is forgotten between steps while
    O and l are kept). Used only to show that the rising inputs tell a correct
    rescale from a wrong one; expected outputs come from the oracle.

    blocks: [(k (Lk, d), v (Lk, d), kpos (Lk,)), ...]; returns (o, lse).
    """
    n = q.shape[0]
    mu = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, blocks[0][1].shape[1]))
    for k, v, kpos in blocks:
        if bug == "mu_not_carried":
            mu = np.full(n, -np.inf)
        s = (q @ k.T) * (scale * LOG2E)
        if causal:
            s = np.where(np.asarray(kpos)[None, :] <= np.asarray(qpos)[:, None], s, -np.inf)
        for t0 in range(0, k.shape[0], TILE):
            st = s[:, t0:t0 + TILE]
            mt = st.max(axis=1)
            need = mt > mu + TAU
            mnew = np.where(need, mt, mu)
            with np.errstate(invalid="ignore"):
                diff = np.where(np.isfinite(mu), mu - mnew, -np.inf)
            alpha = np.where(need, np.exp(diff) if bug == "alpha_natural" else np.exp2(diff), 1.0)
            if bug != "l_not_rescaled":
                l = l * alpha
            if bug != "o_not_rescaled":
                o = o * alpha[:, None]
            mu = mnew
            ref = np.where(np.isfinite(mu), mu, 0.0)
            p = np.exp2(st - ref[:, None])
            l = l + p.sum(axis=1)
            o = o + p @ v[t0:t0 + TILE]
    has = l > 0
    out = np.where(has[:, None], o / np.where(has, l, 1.0)[:, None], 0.0)
    lse = np.where(has, (mu + np.log2(np.where(has, l, 1.0))) / LOG2E, -np.inf)
    return out, lse


def stair_gains(S, P, first=0.02, step=0.55):
    """Key gains of a contiguous P-block split: nearly flat scores in block 0
    (every key weighs about the same, so the state it leaves is large), then
    block t at gain step * t, each block's top scores about 10 log2 units
    above the previous ones: every row rescales at every later step with an
    alpha small enough to matter and large enough that the old state still
    counts."""
    L = S // P
    return np.concatenate([np.full(L, first)] + [np.full(L, step * t) for t in range(1, P)])

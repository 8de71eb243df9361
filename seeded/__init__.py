"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module only draws numbers; it holds none of the attention arithmetic, so
both the CPU oracle and the GPU path may use it without sharing method code.

Recipe: every tensor of a workload is a set of per-(batch, head) matrices of
shape (rows, d) drawn from N(0, 1) in float32 with numpy's PCG64 generator.
Rows are drawn in blocks of ROW_BLOCK rows; block j of tensor `tid` for
(b, h) of workload `wid` is seeded with [wid, tid, b, h, j]. Any row range can
thus be regenerated without drawing the whole sequence. bfloat16 inputs are
the float32 draws rounded to nearest even (torch's conversion); the oracle
reads those exact bfloat16 values back as float64.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ROW_BLOCK = 1024

# numpy's generators release the GIL while filling large arrays, so blocks are
# drawn concurrently; the values do not depend on the thread count.
_POOL = ThreadPoolExecutor(max_workers=max(1, min(16, len(os.sched_getaffinity(0)))))

# tensor ids (DO: the upstream gradient of the attention output)
Q, K, V, DO = 0, 1, 2, 3


def normal_rows(wid, tid, b, h, r0, r1, d):
    """float32 N(0,1) rows [r0, r1) of the (wid, tid, b, h) matrix (width d)."""
    if r1 <= r0:
        return np.zeros((0, d), dtype=np.float32)
    out = np.empty((r1 - r0, d), dtype=np.float32)
    j0, j1 = r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK

    def fill(j):
        blk = np.random.default_rng([wid, tid, b, h, j]).standard_normal(
            (ROW_BLOCK, d), dtype=np.float32)
        a = max(r0, j * ROW_BLOCK)
        z = min(r1, (j + 1) * ROW_BLOCK)
        out[a - r0:z - r0] = blk[a - j * ROW_BLOCK:z - j * ROW_BLOCK]

    list(_POOL.map(fill, range(j0, j1 + 1)))
    return out


def normal_rows_at(wid, tid, b, h, rows, d):
    """float32 N(0,1) rows at an arbitrary (sorted or not) index array."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), dtype=np.float32)
    blocks = rows // ROW_BLOCK
    for j in np.unique(blocks):
        blk = np.random.default_rng([wid, tid, b, h, int(j)]).standard_normal(
            (ROW_BLOCK, d), dtype=np.float32)
        sel = blocks == j
        out[sel] = blk[rows[sel] - int(j) * ROW_BLOCK]
    return out


def to_dtype(x, dtype):
    """float32 numpy -> CPU torch tensor of `dtype` (bf16 rounds to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype) if dtype != torch.float32 else t


def exact_f64(t):
    """The exact values of a CPU torch tensor as a float64 numpy array."""
    return t.to(torch.float64).numpy()


def gen_bhsd(wid, tid, B, H, r0, r1, d, dtype, device="cpu"):
    """A [B, H, r1-r0, d] tensor of rows [r0, r1) of every (b, h) matrix."""
    out = torch.empty((B, H, r1 - r0, d), dtype=dtype, device=device)
    for b in range(B):
        for h in range(H):
            out[b, h] = to_dtype(normal_rows(wid, tid, b, h, r0, r1, d), dtype).to(device)
    return out


def gen_bhsd_at(wid, tid, B, H, rows, d, dtype, device="cpu"):
    """A [B, H, len(rows), d] tensor of the given rows of every (b, h) matrix."""
    rows = np.asarray(rows, dtype=np.int64)
    out = torch.empty((B, H, rows.size, d), dtype=dtype, device=device)
    for b in range(B):
        for h in range(H):
            out[b, h] = to_dtype(normal_rows_at(wid, tid, b, h, rows, d), dtype).to(device)
    return out


def uniform_sample(seed, n, k):
    """k distinct indices from range(n), uniform without replacement, sorted."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(k, n), replace=False)).astype(np.int64)

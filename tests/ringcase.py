"""Shared set-up for the GPU parity tests: seeded inputs on the GPU, oracle rows on the CPU.

The GPU side gets each simulated rank's K/V block laid out contiguously, as a
rank would hold it; the oracle side sees only global positions and the global
K/V, and takes its positions from oracle.layout (never from the package).
"""

import numpy as np
import torch

import oracle
import seeded
from context_attention_ra_amd import layout


def oracle_positions(w, r):
    if w.split == "zigzag":
        return oracle.zigzag_positions(w.S, w.P, r)
    if w.split == "temporal":
        return oracle.temporal_first_positions(w.S // w.S_sp, w.S_sp, w.P, r)
    return oracle.contiguous_positions(w.S, w.P, r)


def pkg_segs(w, r):
    return layout.split(w.split, w.S, w.P, r, S_sp=w.S_sp)


class RingCase:
    """Inputs of rank `rank` of ring workload `w`, plus every rank's K/V block."""

    def __init__(self, w, rank, device="cuda"):
        self.w, self.rank = w, rank
        B, H, Hkv, d, P = w.B, w.H, w.Hkv, w.d, w.P
        self.q_segs = pkg_segs(w, rank)
        self.kv_segs = [pkg_segs(w, t) for t in range(P)]
        qpos = oracle_positions(w, rank)
        self.q = seeded.gen_bhsd_at(w.wid, seeded.Q, B, H, qpos, d, w.dtype, device)
        L = w.L
        self.kv = [(torch.empty((B, Hkv, L, d), dtype=w.dtype, device=device),
                    torch.empty((B, Hkv, L, d), dtype=w.dtype, device=device)) for _ in range(P)]
        pos_t = [torch.as_tensor(oracle_positions(w, t), device=device) for t in range(P)]
        for b in range(B):
            for h in range(Hkv):
                for tid, slot in ((seeded.K, 0), (seeded.V, 1)):
                    g = seeded.to_dtype(seeded.normal_rows(w.wid, tid, b, h, 0, w.S, d), w.dtype).to(device)
                    for t in range(P):
                        self.kv[t][slot][b, h] = g.index_select(0, pos_t[t])

    def expected(self, rows=None):
        """Oracle (o, lse) for local rows `rows` (default all), per (b, h): [B,H,n,d], [B,H,n]."""
        w = self.w
        qpos_all = oracle_positions(w, self.rank)
        rows = np.arange(qpos_all.size) if rows is None else np.asarray(rows)
        qpos = qpos_all[rows]
        o = np.zeros((w.B, w.H, rows.size, w.d))
        lse = np.zeros((w.B, w.H, rows.size))
        ex = lambda tid, b, h, r: seeded.exact_f64(seeded.to_dtype(
            seeded.normal_rows_at(w.wid, tid, b, h, r, w.d), w.dtype))
        if w.Hkv != w.H:
            # grouped K/V heads: the oracle decides which K/V head a query head reads
            for b in range(w.B):
                q = np.stack([ex(seeded.Q, b, h, qpos) for h in range(w.H)])
                k = np.stack([ex(seeded.K, b, h, np.arange(w.S)) for h in range(w.Hkv)])
                v = np.stack([ex(seeded.V, b, h, np.arange(w.S)) for h in range(w.Hkv)])
                o[b], lse[b] = oracle.grouped_attention(q, qpos, k, v, np.arange(w.S), w.scale, w.causal)
            return o, lse
        for b in range(w.B):
            for h in range(w.H):
                q = seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, seeded.Q, b, h, qpos, w.d), w.dtype))
                k = seeded.exact_f64(seeded.to_dtype(seeded.normal_rows(w.wid, seeded.K, b, h, 0, w.S, w.d), w.dtype))
                v = seeded.exact_f64(seeded.to_dtype(seeded.normal_rows(w.wid, seeded.V, b, h, 0, w.S, w.d), w.dtype))
                o[b, h], lse[b, h] = oracle.attention_rows(q, qpos, k, v, np.arange(w.S), w.scale, w.causal)
        return o, lse


def sample_rows(w, rank, n_total=4096, seed=1234):
    """Stratified sample: n_total/(B*H) rows per (b, h) head... the same local rows for every head,
    drawn uniformly without replacement, always including the first and last row of each local run."""
    L = w.L
    segs = pkg_segs(w, rank)
    must = []
    off = 0
    for _, n in segs:
        must += [off, off + n - 1]
        off += n
    per_head = max(1, n_total // (w.B * w.H))
    rest = seeded.uniform_sample([seed, w.wid, rank], L, per_head)
    rows = np.unique(np.concatenate([np.array(must), rest]))
    return rows


def compare(gpu, ref):
    """(max |gpu-ref|, sum|gpu-ref| / sum|ref|) over all compared elements."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(gpu - ref)
    return float(diff.max()), float(diff.sum() / max(np.abs(ref).sum(), 1e-300))


# tolerances stated for the method's outputs: fp32 path 1e-4 max-abs; bf16
# outputs 2e-2 max-abs and 1e-2 mean-relative (fp32 accumulation)
TOL = {torch.float32: dict(max_abs=1e-4, mean_rel=1e-4, lse_abs=1e-5),
       torch.bfloat16: dict(max_abs=2e-2, mean_rel=1e-2, lse_abs=1e-3)}


def assert_close(gpu_o, ref_o, gpu_lse, ref_lse, dtype, what=""):
    tol = TOL[dtype]
    mx, mr = compare(gpu_o, ref_o)
    lmx, _ = compare(gpu_lse, ref_lse)
    msg = f"{what}: max_abs={mx:.3e} mean_rel={mr:.3e} lse_max_abs={lmx:.3e}"
    print(msg, flush=True)
    assert mx <= tol["max_abs"], msg
    assert mr <= tol["mean_rel"], msg
    assert lmx <= tol["lse_abs"], msg
    return mx, mr, lmx

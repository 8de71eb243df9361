"""Benchmark: attention TFLOP/s of one rank's ring-attention share on one MI355X.

One "step" is one full pass of the hot path over the workload: the P ring steps
(``ra_step`` on the compute stream, the next K/V block passed on a side stream
with ``ra_kv_pass``) and ``ra_finalize``. Inputs are seeded synthetic tensors
already resident in HBM before the timed region. The default workload is the
32K-token causal LLM context, share of rank 0 of 4 (zigzag split).

Printed: one JSON line. ``value`` is whole-pass throughput (algorithmic FLOP =
4*d per unmasked query/key pair) over the wall time of the timed steps.
``roofline`` is the ring-step kernel's algorithmic FLOP per launch over its
mean launch time (HIP events on the compute stream) against the bf16 dense
matrix-core peak. ``legs`` times the remaining kernels of the path on their
own workloads (merge on this workload's shapes; factored spatial/temporal on
the 16x900 video workload). ``cpu_baseline`` times the CPU oracle on a bounded
sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import seeded  # noqa: E402
from context_attention_ra_amd import _lib, configs, layout, ring, sizing, variants  # noqa: E402

PEAK_BF16_DENSE = 2.5e15    # MI355X bf16 dense matrix-core FLOP/s (published)
PEAK_HBM = 8.0e12           # MI355X HBM3E bytes/s (published)
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def positions(segs):
    return np.concatenate([np.arange(s, s + n, dtype=np.int64) for s, n in segs])


def make_ring_inputs(w, rank, dev):
    segs = [layout.split(w.split, w.S, w.P, t, S_sp=w.S_sp) for t in range(w.P)]
    pos = [torch.as_tensor(positions(s), device=dev) for s in segs]
    q = seeded.gen_bhsd_at(w.wid, seeded.Q, w.B, w.H, positions(segs[rank]), w.d, w.dtype, dev)
    kv = [(torch.empty((w.B, w.Hkv, w.L, w.d), dtype=w.dtype, device=dev),
           torch.empty((w.B, w.Hkv, w.L, w.d), dtype=w.dtype, device=dev)) for _ in range(w.P)]
    for b in range(w.B):
        for h in range(w.Hkv):
            for tid, slot in ((seeded.K, 0), (seeded.V, 1)):
                g = seeded.to_dtype(seeded.normal_rows(w.wid, tid, b, h, 0, w.S, w.d), w.dtype).to(dev)
                for t in range(w.P):
                    kv[t][slot][b, h] = g.index_select(0, pos[t])
    return q, segs, kv


def ring_flop(w, rank, segs):
    order = layout.ring_order(rank, w.P)
    per_step = [sizing.pairs(segs[rank], segs[t], w.causal) for t in order]
    return [sizing.attention_flop(p, w.d, w.B * w.H) for p in per_step]


# Sources that define the ring-step kernel; a change to any of them makes the
# committed HBM counter figures stale (traffic is then reported as null).
STEP_SOURCES = {
    torch.bfloat16: ["step_mfma.hip", "ra_device.h", "ra_launch.h"],
    torch.float32: ["step_f32.hip", "ra_device.h", "ra_launch.h"],
}


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "context_attention_ra_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch from committed counter summaries, if still current."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


EVENT_EVERY = 4


def time_ring(w, rank, q, segs, kv, steps, warmup, prefetch):
    dev = q.device
    st = ring.RingState(w.B, w.H, w.L, w.d, dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
    bufs = [(torch.empty_like(kv[0][0]), torch.empty_like(kv[0][1])) for _ in range(2)]
    side = torch.cuda.Stream(dev)
    # events around every launch add queue packets between the kernels (about
    # 15 us per launch, 2-3% of a pass), so they are recorded in every
    # EVENT_EVERY-th timed pass only
    timed_with_events = [i for i in range(steps) if i % EVENT_EVERY == 0]
    ev = {i: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(w.P)] for i in timed_with_events}

    def one(events=None):
        ring.run(q, segs[rank], kv, segs, rank, w.causal, scale=w.scale, prefetch=prefetch,
                 out=out, lse=lse, state=st, bufs=bufs, copy_stream=side, step_events=events)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(ev.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([[a.elapsed_time(b) for a, b in ev[i]] for i in timed_with_events])  # [passes, P] ms
    return wall, kms, out, lse


def time_kernel(fn, reps, warmup=3):
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for i in range(reps):
        e0[i].record()
        fn()
        e1[i].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in zip(e0, e1)]))


def plain_gemm(dev, n=8192, reps=20):
    """A plain bf16 GEMM through PyTorch (hipBLASLt), n x n x n, timed with HIP
    events: what the matrix cores sustain for a large dense product on this
    chip, the counterpart of the plain stream beside the HBM-bound legs."""
    g = torch.Generator(device=dev).manual_seed(20262)
    a = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    ms = time_kernel(lambda: torch.matmul(a, b, out=c), reps, warmup=20)
    fl = 2.0 * n ** 3
    return {"TFLOP/s": fl / ms / 1e9, "frac_of_peak": fl / ms / 1e-3 / PEAK_BF16_DENSE,
            "shape": f"bf16 [{n},{n}] x [{n},{n}] -> bf16, fp32 accumulate (torch.matmul)", "ms": ms}


def time_backward(w, rank, q, segs, kv, out, lse, reps, warmup=3):
    """The backward pass of the same share: ra_bwd_prep and P ra_step_bwd
    launches (dQ kernel, then dK/dV kernel), timed with HIP events on the
    stream they run on."""
    dev = q.device
    do = seeded.gen_bhsd_at(w.wid, seeded.DO, w.B, w.H, positions(segs[rank]), w.d, w.dtype, dev)
    dkv = [(torch.empty(k.shape, dtype=torch.float32, device=dev),
            torch.empty(k.shape, dtype=torch.float32, device=dev)) for k, _ in kv]
    box = {}

    def one():
        # fresh accumulators each pass: every block's dK/dV holds this rank's share
        box["dq"], _ = ring.run_bwd(q, segs[rank], kv, segs, rank, w.causal, out, lse, do, scale=w.scale)

    ms = time_kernel(one, reps, warmup)
    assert torch.isfinite(box["dq"]).all(), "non-finite dq"
    fl = 2.0 * sum(ring_flop(w, rank, segs))
    return {"workload": f"{w.name} rank {rank}, {w.P} backward ring steps", "ms": ms,
            "TFLOP/s": fl / ms / 1e9, "mfma_frac": fl / ms / 1e-3 / PEAK_BF16_DENSE,
            "flop": fl, "flop_convention": "8*d per visible pair (the dV, dP, dQ and dK products); "
            "the kernels execute 14*d (scores and dP are formed in both the dQ and the dK/dV kernel)"}


def time_variants(w, rank, q, segs, kv, reps, warmup=2):
    """The alternatives to the ring on the same workload: the rank's queries
    against the all-gathered K/V (gather copies plus one step launch), and
    head group `rank` of the all-to-all on heads (the re-layout copies plus
    one step launch over the whole sequence). Same algorithmic FLOP per rank
    as the ring pass."""
    dev = q.device
    res = {}
    fl = sum(ring_flop(w, rank, segs))
    ms = time_kernel(lambda: variants.run_allgather(q, segs[rank], kv, segs, w.causal, scale=w.scale),
                     reps, warmup)
    res["all_gather"] = {"ms": ms, "TFLOP/s": fl / ms / 1e9, "flop": fl}
    if w.H % w.P == 0 and w.Hkv % w.P == 0:
        qb = [q if t == rank else seeded.gen_bhsd_at(w.wid, seeded.Q, w.B, w.H, positions(segs[t]), w.d,
                                                     w.dtype, dev) for t in range(w.P)]
        full = [(0, w.S)]
        flh = sizing.attention_flop(sizing.pairs(full, full, w.causal), w.d, w.B * (w.H // w.P))
        ms = time_kernel(lambda: variants.run_head_group(qb, kv, segs, rank, w.causal, scale=w.scale),
                         reps, warmup)
        res["all_to_all_heads"] = {"ms": ms, "TFLOP/s": flh / ms / 1e9, "flop": flh,
                                   "heads": f"{w.H // w.P} of {w.H} over all {w.S} positions"}
    res["workload"] = f"{w.name} rank {rank}; exchanges simulated by device copies inside the timing"
    return res


def time_small_ring(dev, reps=50):
    """Whole ring pass of the causal 4K two-rank share (rank 0): two steps and
    the block pass, too small to fill the chip (launch-bound); reported for
    completeness beside the 32K share."""
    w = configs.CAUSAL_2RANK
    q, segs, kv = make_ring_inputs(w, 0, dev)
    bufs = [(torch.empty_like(kv[0][0]), torch.empty_like(kv[0][1])) for _ in range(2)]
    side = torch.cuda.Stream(dev)
    st = ring.RingState(w.B, w.H, w.L, w.d, dev)
    out, lse = torch.empty_like(q), torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
    ms = time_kernel(lambda: ring.run(q, segs[0], kv, segs, 0, w.causal, scale=w.scale, out=out, lse=lse,
                                      state=st, bufs=bufs, copy_stream=side), reps, warmup=10)
    fl = float(sum(ring_flop(w, 0, segs)))
    return {"workload": f"{w.name} rank 0, whole ring pass ({w.P} steps)", "ms": ms, "TFLOP/s": fl / ms / 1e9,
            "mfma_frac": fl / ms / 1e-3 / PEAK_BF16_DENSE, "flop": fl}


def time_video_steps(dev, reps=2):
    """Two ring steps of the video DiT share (rank 0: 54,000 local queries,
    two non-causal 54,000-token K/V blocks, 32 heads, d = 128): the first with
    RA_STEP_INIT, the second reading the state back, as in the ring. Inputs
    are seeded N(0,1) draws made on the GPU (timing only; the parity tests use
    the oracle's seeded rows)."""
    w = configs.VIDEO_DIT_CP8
    g = torch.Generator(device=dev).manual_seed(20263)
    L = w.L
    q = torch.randn((w.B, w.H, L, w.d), generator=g, device=dev).to(w.dtype)
    blocks = [tuple(torch.randn((w.B, w.H, L, w.d), generator=g, device=dev).to(w.dtype) for _ in range(2))
              for _ in range(2)]
    st = ring.RingState(w.B, w.H, L, w.d, dev)
    segs = [layout.split(w.split, w.S, w.P, t, S_sp=w.S_sp) for t in range(w.P)]
    order = layout.ring_order(0, w.P)[:2]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * reps)]

    def two_steps(events):
        for s, t in enumerate(order):
            k, v = blocks[s]
            events[s][0].record()
            _lib.ra_step(q, k, v, segs[0], segs[t], False, w.scale, st.o, st.m, st.l, init=(s == 0))
            events[s][1].record()

    two_steps(ev[:2])  # warm-up
    torch.cuda.synchronize()
    for r in range(reps):
        two_steps(ev[2 * r:2 * r + 2])
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.mean(per))
    fl = sizing.attention_flop(L * L, w.d, w.B * w.H)
    assert torch.isfinite(st.l).all()
    return {"workload": f"{w.name} rank 0, ring steps 0 and 1 (init, then state read back)", "ms_per_step": ms,
            "ms_per_step_each": per, "TFLOP/s": fl / ms / 1e9, "mfma_frac": fl / ms / 1e-3 / PEAK_BF16_DENSE,
            "flop_per_step": fl, "timing": f"HIP events around each ra_step launch, {reps} reps after one warm-up"}


def legs(w, q, dev, reps):
    out = {}
    # LSE merge of two normalised partials of this workload's shape (bf16)
    B, H, L, d = q.shape
    g = torch.Generator(device=dev).manual_seed(20261)
    oa = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
    ob = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
    la = torch.randn((B, H, L), generator=g, device=dev)
    lb = torch.randn((B, H, L), generator=g, device=dev)
    oo, lo = torch.empty_like(q), torch.empty_like(la)
    # the HBM-bound legs evict their inputs from L2 and the last-level cache
    # before each rep by reading a 1 GiB buffer (a read leaves clean lines
    # behind, so no write-back of the flush data lands inside the timed call),
    # and are set against a plain PyTorch elementwise stream of the same bytes
    # timed the same way
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def evicted_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tms = []
        for i in range(reps + 2):
            torch.sum(flush, dim=0, out=sink)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                tms.append(e0.elapsed_time(e1))
        return float(np.mean(tms))

    ms = evicted_ms(lambda: _lib.ra_merge_lse(oa, la, ob, lb, oo, lo))
    plain = evicted_ms(lambda: torch.add(oa, ob, out=oo))  # 2 reads + 1 write of O
    nbytes = 3 * q.numel() * q.element_size() + 3 * la.numel() * 4
    pbytes = 3 * q.numel() * q.element_size()
    out["merge_lse"] = {"workload": f"{w.name} rank share [B,H,L,d]={list(q.shape)} bf16",
                        "ms": ms, "GB/s": nbytes / ms / 1e6, "hbm_frac": nbytes / ms / 1e-3 / PEAK_HBM,
                        "plain_stream_GB/s": pbytes / plain / 1e6,
                        "plain_stream": "torch.add of the two O inputs (2 reads + 1 write)",
                        "caches": "evicted by reading 1 GiB before each rep"}
    # factored video attention, 16 frames x 900 tokens
    v = configs.VIDEO_FACTORED
    qv, kvv, vv = (seeded.gen_bhsd(v.wid, tid, v.B, v.H, 0, v.N, v.d, v.dtype, dev)
                   for tid in (seeded.Q, seeded.K, seeded.V))
    ov = torch.empty_like(qv)
    lv = torch.empty((v.B, v.H, v.N), dtype=torch.float32, device=dev)
    # about 20 ms of calls first: the clock takes that long to settle under MFMA load
    ms = time_kernel(lambda: _lib.ra_factored_spatial(qv, kvv, vv, v.T, v.S_sp, v.scale, ov, lv), reps, warmup=60)
    fl = sizing.attention_flop(v.T * v.S_sp * v.S_sp, v.d, v.B * v.H)
    out["factored_spatial"] = {"workload": v.name, "ms": ms, "TFLOP/s": fl / ms / 1e9,
                               "mfma_frac": fl / ms / 1e-3 / PEAK_BF16_DENSE}
    # temporal: one (b, h, spatial position) problem reads 16 strided rows of
    # each input; the plain stream reads and writes the same bytes contiguously
    ms = evicted_ms(lambda: _lib.ra_factored_temporal(qv, kvv, vv, v.T, v.S_sp, v.scale, ov, lv))
    plain = evicted_ms(lambda: torch.addcmul(qv, kvv, vv, out=ov))  # 3 reads + 1 write
    nbytes = 4 * qv.numel() * qv.element_size() + lv.numel() * 4
    pbytes = 4 * qv.numel() * qv.element_size()
    out["factored_temporal"] = {"workload": v.name, "ms": ms, "GB/s": nbytes / ms / 1e6,
                                "hbm_frac": nbytes / ms / 1e-3 / PEAK_HBM,
                                "algorithmic_bytes": nbytes,
                                "plain_stream_GB/s": pbytes / plain / 1e6,
                                "plain_stream": "torch.addcmul of q, k, v (3 reads + 1 write)",
                                "caches": "evicted by reading 1 GiB before each rep"}
    # longer clips (Day 83 post: 48 frames of 900 tokens; 120 frames, one of
    # 8 devices' 450 spatial positions after the re-split), 32 heads, d = 128
    g2 = torch.Generator(device=dev).manual_seed(20264)
    for T, S_sp in ((48, 900), (120, 450)):
        shape = (1, 32, T * S_sp, 128)
        ql, kl, vl = (torch.randn(shape, generator=g2, device=dev).to(torch.bfloat16) for _ in range(3))
        ol = torch.empty_like(ql)
        ll = torch.empty(shape[:3], dtype=torch.float32, device=dev)
        ms = evicted_ms(lambda: _lib.ra_factored_temporal(ql, kl, vl, T, S_sp, 128 ** -0.5, ol, ll))
        plain = evicted_ms(lambda: torch.addcmul(ql, kl, vl, out=ol))
        nbytes = 4 * ql.numel() * 2 + ll.numel() * 4
        out[f"factored_temporal_{T}x{S_sp}"] = {
            "workload": f"{T} frames x {S_sp} positions, H=32, d=128, bf16", "ms": ms,
            "GB/s": nbytes / ms / 1e6, "hbm_frac": nbytes / ms / 1e-3 / PEAK_HBM,
            "plain_stream_GB/s": 4 * ql.numel() * 2 / plain / 1e6,
            "TFLOP/s": sizing.attention_flop(T * T * S_sp, 128, 32) / ms / 1e9,
            "caches": "evicted by reading 1 GiB before each rep"}
        del ql, kl, vl, ol, ll
    return out


def cpu_baseline(w, rank, segs, budget_s):
    """The oracle, as it stands, on a bounded sample of this workload's rows."""
    import oracle
    from threadpoolctl import threadpool_info
    qpos_all = positions(segs[rank])
    chunk = 256
    rng = np.random.default_rng(7)
    done_rows, flop, elapsed = 0, 0.0, 0.0
    heads = set()
    kv = {}
    i = 0
    while elapsed < budget_s:
        h = i % (w.B * w.H)
        b, hh = divmod(h, w.H)
        if h not in kv:  # the global K and V this head reads, kept for later runs of that head
            hk = hh // (w.H // w.Hkv)  # consecutive query heads share a K/V head
            kv[h] = tuple(seeded.exact_f64(seeded.to_dtype(
                seeded.normal_rows(w.wid, t, b, hk, 0, w.S, w.d), w.dtype)) for t in (seeded.K, seeded.V))
        kf, vf = kv[h]
        r0 = int(rng.integers(0, max(1, qpos_all.size - chunk)))
        qp = qpos_all[r0:r0 + chunk]
        qf = seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, seeded.Q, b, hh, qp, w.d), w.dtype))
        t0 = time.perf_counter()
        oracle.attention_rows(qf, qp, kf, vf, np.arange(w.S), w.scale, w.causal)
        elapsed += time.perf_counter() - t0
        pairs = int(np.minimum(qp + 1, w.S).sum()) if w.causal else qp.size * w.S
        flop += sizing.attention_flop(pairs, w.d, 1)
        done_rows += qp.size
        heads.add(h)
        i += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    rows_per_s = done_rows / elapsed
    full_rows = w.B * w.H * qpos_all.size
    return {"value": flop / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "rows_per_s": rows_per_s,
            "extrapolated_full_s": full_rows / rows_per_s,
            "extrapolation": f"{full_rows} query rows of the rank's share (B*H*local rows) at the sampled "
                             f"rows/s; extrapolated, not measured",
            "sample": f"{done_rows} query rows ({i} runs of {chunk} rows from {len(heads)} heads) of rank {rank} "
                      f"against the full {w.S}-token K/V, fp64 numpy; {elapsed:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_full_configs():
    """The oracle, as it stands, on the three small configurations in full:
    the tiny fp32 ring and the causal two-rank share (every rank's queries
    against the whole sequence, the result their rings reach), and factored
    spatial and temporal attention of the 16 x 900 video workload."""
    import oracle
    out = []
    for w in (configs.TINY_F32, configs.CAUSAL_2RANK):
        pos = np.arange(w.S)
        t0 = time.perf_counter()
        for b in range(w.B):
            for h in range(w.H):
                q, k, v = (seeded.exact_f64(seeded.to_dtype(seeded.normal_rows(w.wid, t, b, h, 0, w.S, w.d), w.dtype))
                           for t in (seeded.Q, seeded.K, seeded.V))
                oracle.attention_rows(q, pos, k, v, pos, w.scale, w.causal)
        el = time.perf_counter() - t0
        pairs = w.S * (w.S + 1) // 2 if w.causal else w.S * w.S
        fl = sizing.attention_flop(pairs, w.d, w.B * w.H)
        out.append({"workload": f"{w.name}, all {w.P} ranks' queries", "s": el, "TFLOP/s": fl / el / 1e12})
    v = configs.VIDEO_FACTORED
    for name, fn, pairs in (("spatial", oracle.factored_spatial, v.T * v.S_sp * v.S_sp),
                            ("temporal", oracle.factored_temporal, v.S_sp * v.T * v.T)):
        t0 = time.perf_counter()
        for b in range(v.B):
            for h in range(v.H):
                q, k, vv = (seeded.exact_f64(seeded.to_dtype(seeded.normal_rows(v.wid, t, b, h, 0, v.N, v.d), v.dtype))
                            for t in (seeded.Q, seeded.K, seeded.V))
                fn(q, k, vv, v.T, v.S_sp, v.scale)
        el = time.perf_counter() - t0
        fl = sizing.attention_flop(pairs, v.d, v.B * v.H)
        out.append({"workload": f"{v.name} {name}", "s": el, "TFLOP/s": fl / el / 1e12})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=configs.LLM_32K_CP4.name, choices=sorted(configs.RING_WORKLOADS))
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-prefetch", action="store_true", help="pass each block on the compute stream")
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--legs-only", action="store_true",
                    help="time only the merge / factored legs (for profiling those kernels) and exit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain 'copy_' of this many MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _lib.load()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 18
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4}))
        return

    w = configs.RING_WORKLOADS[args.workload]
    if args.legs_only:
        q = torch.empty((w.B, w.H, w.L, w.d), dtype=w.dtype, device=dev)
        print(json.dumps({"legs": legs(w, q, dev, reps=args.steps)}), flush=True)
        return
    log(f"[bench] workload {w.name} rank {args.rank}: generating inputs")
    q, segs, kv = make_ring_inputs(w, args.rank, dev)
    flops = ring_flop(w, args.rank, segs)
    total = float(sum(flops))
    log(f"[bench] {w.P} ring steps, {total:.4e} algorithmic FLOP per pass; timing {args.steps} passes")
    wall, kms, out, lse = time_ring(w, args.rank, q, segs, kv, args.steps, args.warmup, not args.no_prefetch)
    assert torch.isfinite(lse).all(), "non-finite lse"
    ms_per_step = wall / args.steps * 1e3
    value = total * args.steps / wall / 1e12
    k_mean_ms = float(kms.mean())
    achieved = (total / w.P) / (k_mean_ms * 1e-3)
    src_hash = kernel_source_hash(STEP_SOURCES[w.dtype])
    gemm = plain_gemm(dev)
    traffic = load_traffic("ra_step:" + w.name, src_hash)
    rec = {
        "metric": "attention TFLOP/s per MI355X (and % bf16 MFMA peak), ring-step kernel",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded N(0,1), rounded to bf16)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.Hkv, "d": w.d, "global_seq": w.S,
                   "ring_P": w.P, "rank": args.rank, "local_q": w.L, "split": w.split,
                   "causal": w.causal, "prefetch": not args.no_prefetch,
                   "parallelism": "one rank's share, ring simulated on 1 GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16_DENSE / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_DENSE,
                     "traffic": traffic, "kernel": "ra_step (step_mfma_kernel)",
                     "kernel_ms_mean": k_mean_ms,
                     "kernel_timing": f"HIP events around each ra_step launch on its stream, in every "
                                      f"{EVENT_EVERY}th timed pass ({kms.shape[0]} of {args.steps})",
                     "kernel_ms_per_ring_step": [float(x) for x in kms.mean(axis=0)],
                     "flop_per_launch_mean": total / w.P,
                     "plain_gemm": gemm, "vs_plain_gemm": achieved / 1e12 / gemm["TFLOP/s"]},
        "ring_ms_per_pass": ms_per_step,
        "kernel_share_of_pass": float(kms.sum(axis=1).mean()) / ms_per_step,
    }
    # the same pass with each block passed on the compute stream before its
    # step (no overlap), so that the side stream's effect is in the record
    cmp_prefetch = args.no_prefetch  # the mode the main measurement did not use
    log(f"[bench] ring pass with prefetch={cmp_prefetch} for comparison")
    n2 = max(4, args.steps // 2)
    wall2, kms2, _, _ = time_ring(w, args.rank, q, segs, kv, n2, 3, cmp_prefetch)
    ms2 = wall2 / n2 * 1e3
    tag = "prefetch" if cmp_prefetch else "no_prefetch"
    rec["ring_ms_per_pass_" + tag] = ms2
    rec["ring_kernel_ms_mean_" + tag] = float(kms2.mean())
    with_pf, without_pf = (ms2, ms_per_step) if cmp_prefetch else (ms_per_step, ms2)
    # share of the serial pass time that passing the blocks on the side stream saves
    rec["prefetch_saving"] = (without_pf - with_pf) / without_pf
    if not args.no_prefetch:
        # in the timed passes the block copy runs beside the step kernels and
        # shares the GPU with them; the comparison passes run each kernel alone
        alone = (total / w.P) / (float(kms2.mean()) * 1e-3)
        rec["roofline"]["frac_kernel_alone"] = alone / PEAK_BF16_DENSE
        rec["roofline"]["kernel_alone_timing"] = ("the same launches in the comparison passes (blocks passed on the "
                                                  "compute stream, no copy beside the kernel)")
    if not args.no_legs:
        log("[bench] legs: merge, factored spatial, factored temporal")
        rec["legs"] = legs(w, q, dev, reps=20)
        if w.dtype == torch.bfloat16:
            log("[bench] leg: backward ring pass")
            rec["legs"]["backward"] = time_backward(w, args.rank, q, segs, kv, out, lse, reps=10)
        log("[bench] leg: all-gather and all-to-all on heads")
        rec["legs"]["variants"] = time_variants(w, args.rank, q, segs, kv, reps=5)
        log("[bench] legs: the other ring workloads (4K two-rank ring, video DiT share steps)")
        rec["legs"]["ring_causal_4k_cp2"] = time_small_ring(dev)
        rec["legs"]["video_dit_432k_cp8_steps"] = time_video_steps(dev)
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle for ~{args.cpu_budget:.0f} s")
        rec["cpu_baseline"] = cpu_baseline(w, args.rank, segs, args.cpu_budget)
        rec["cpu_baseline"]["full_configs"] = cpu_full_configs()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

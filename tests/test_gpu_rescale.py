"""GPU parity on inputs that force the online-softmax rescale part-way (0 < alpha < 1).

Day 83 post, "Context parallelism: splitting the sequence": the running output
and sum are rescaled whenever a new block raises a row's maximum. The bf16
kernels move their reference value lazily (only past a threshold), so N(0,1)
inputs never take that branch after the first tile. The inputs here (see
``rising``) make scores grow along the key sequence; each case first checks on
the CPU, by replaying the kernel's tile order, that a large share of its rows
really rescale with a finite previous reference, then compares the GPU
result with the oracle at the stated bf16 tolerances.

Cases: the causal two-rank zigzag ring (both ranks, ring order and reversed),
a non-causal ring whose blocks arrive in rising order (every rescale after the
first step starts from a state read back from memory), ragged causal single
steps with and without a state carried in, factored spatial attention, and
the 32K causal share (sampled rows, blocks in rising order).
"""

import numpy as np
import pytest
import torch

import oracle
import rising
import seeded
from context_attention_ra_amd import _lib, configs, layout, ring
from ringcase import assert_close, sample_rows

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def _f64(t):
    return seeded.exact_f64(t)


def _ring_rescale_case(w, rank, q, k, v, order, min_frac, rows=None):
    """Ring of rank `rank` over global CPU inputs, checked against the oracle."""
    segs = [layout.split(w.split, w.S, w.P, t, S_sp=w.S_sp) for t in range(w.P)]
    pos = [np.concatenate([np.arange(s, s + n) for s, n in sg]) for sg in segs]
    qpos = pos[rank]
    rows = np.arange(qpos.size) if rows is None else np.asarray(rows)
    # the inputs must make the kernel's reference value move part-way
    frac = []
    for b in range(w.B):
        for h in range(w.H):
            hk = h // (w.H // w.Hkv)
            kf = _f64(k[b, hk])
            blocks = [(kf[pos[t]], pos[t]) for t in order]
            cnt, _ = rising.partial_rescales(_f64(q[b, h])[qpos[rows]], qpos[rows], blocks, w.scale, w.causal)
            frac.append((cnt > 0).mean())
    print(f"rows with a partial rescale: min {min(frac):.3f} mean {np.mean(frac):.3f} over heads", flush=True)
    assert np.mean(frac) >= min_frac, f"inputs rescale too rarely: {np.mean(frac):.3f}"
    dev = "cuda"
    qd = q[:, :, torch.as_tensor(qpos)].contiguous().to(dev)
    kv = [(k[:, :, torch.as_tensor(p)].contiguous().to(dev), v[:, :, torch.as_tensor(p)].contiguous().to(dev))
          for p in pos]
    out, lse, _ = ring.run(qd, segs[rank], kv, segs, rank, w.causal, scale=w.scale, order=order)
    torch.cuda.synchronize()
    ro = np.zeros((w.B, w.H, rows.size, w.d))
    rl = np.zeros((w.B, w.H, rows.size))
    allk = np.arange(w.S)
    for b in range(w.B):
        for h in range(w.H):
            hk = h // (w.H // w.Hkv)
            ro[b, h], rl[b, h] = oracle.attention_rows(_f64(q[b, h])[qpos[rows]], qpos[rows], _f64(k[b, hk]),
                                                       _f64(v[b, hk]), allk, w.scale, w.causal)
    idx = torch.as_tensor(rows, device=dev)
    go = out.index_select(2, idx).float().cpu().double().numpy()
    gl = lse.index_select(2, idx).cpu().double().numpy()
    assert_close(go, ro, gl, rl, w.dtype, f"{w.name} rising r{rank} order {order}")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("rank", [0, 1])
@pytest.mark.parametrize("reverse", [False, True])
def test_rescale_causal_2rank_ring(gpu_lib, rank, reverse):
    w = configs.CAUSAL_2RANK
    order = layout.ring_order(rank, w.P)
    if reverse:
        order = order[::-1]
    banner(f"{w.name} rising scores, rank {rank}, order {order}")
    q, k, v = rising.rising_global(900, w.B, w.H, w.Hkv, w.S, w.d, q_gain=6.0, lo=0.2, hi=5.0)
    _ring_rescale_case(w, rank, q, k, v, order, min_frac=0.45)


def test_rescale_across_steps_noncausal_ring(gpu_lib):
    # blocks visited in rising order: each step's scores outgrow the reference
    # value the previous step stored, so the rescale starts from a state read
    # back from memory (the checkpointed m of the last step)
    w = configs.RingWorkload(903, "stair-noncausal-4k-cp4", B=1, H=2, d=128, S=4096, P=4,
                             split="contiguous", causal=False, dtype=torch.bfloat16)
    order = [0, 1, 2, 3]
    banner(f"{w.name}: rank 0, blocks in rising order {order}")
    q, k, v = rising.rising_global(w.wid, w.B, w.H, w.Hkv, w.S, w.d, q_gain=4.0,
                                   gains=rising.stair_gains(w.S, w.P))
    segs = [layout.split(w.split, w.S, w.P, t) for t in range(w.P)]
    pos = [np.arange(s, s + n) for sg in segs for s, n in sg]
    # every row must rescale at some step after the first
    for h in range(w.H):
        kf = _f64(k[0, h])
        qf = _f64(q[0, h])[pos[0]]
        _, mu = rising.partial_rescales(qf, pos[0], [(kf[pos[0]], pos[0])], w.scale, False)
        cnt, _ = rising.partial_rescales(qf, pos[0], [(kf[pos[t]], pos[t]) for t in order[1:]], w.scale, False,
                                         mu0=mu)
        print(f"head {h}: rows rescaled after step 0: {(cnt > 0).mean():.3f}", flush=True)
        assert (cnt > 0).mean() >= 0.9
    _ring_rescale_case(w, 0, q, k, v, order, min_frac=0.9)


RESCALE_STEP_CASES = [
    # (B, H, Lq, q_runs, Lk, k_runs, d)
    (2, 3, 300, [(40, 137), (1000, 163)], 333, [(0, 250), (900, 83)], 128),
    (1, 2, 517, [(600, 517)], 999, [(0, 999)], 64),
    (1, 2, 700, [(0, 700)], 700, [(0, 700)], 128),
]


@pytest.mark.parametrize("ci", range(len(RESCALE_STEP_CASES)))
def test_rescale_single_steps_and_resumed_state(gpu_lib, ci):
    B, H, Lq, qr, Lk, kr, d = RESCALE_STEP_CASES[ci]
    banner(f"rising scores, causal step case {ci}: B{B} H{H} Lq{Lq} {qr} Lk{Lk} {kr} d{d}")
    qp = np.concatenate([np.arange(s, s + n) for s, n in qr])
    kp = np.concatenate([np.arange(s, s + n) for s, n in kr])
    span = int(max(qp.max(), kp.max())) + 1
    # two blocks at the same positions: the second one's keys have higher gains
    qa, ka, va = rising.rising_global(910 + ci, B, H, H, Lk, d, q_gain=6.0, lo=0.2, hi=3.0, key_pos=kp, span=span)
    _, kb, vb = rising.rising_global(920 + ci, B, H, H, Lk, d, q_gain=6.0, lo=1.0, hi=6.0, key_pos=kp, span=span)
    q = seeded.gen_bhsd(930 + ci, seeded.Q, B, H, 0, Lq, d, torch.float32, "cpu")
    q = (6.0 * q).to(torch.bfloat16)
    scale = d ** -0.5
    qf, kaf, vaf, kbf, vbf = (_f64(t) for t in (q, ka, va, kb, vb))
    frac1, frac2 = [], []
    for b in range(B):
        for h in range(H):
            c1, mu = rising.partial_rescales(qf[b, h], qp, [(kaf[b, h], kp)], scale, True)
            c2, _ = rising.partial_rescales(qf[b, h], qp, [(kbf[b, h], kp)], scale, True, mu0=mu)
            frac1.append((c1 > 0).mean())
            frac2.append((c2 > 0).mean())
    print(f"partial rescales: first step {np.mean(frac1):.3f}, resumed step {np.mean(frac2):.3f}", flush=True)
    assert np.mean(frac1) >= 0.3 and np.mean(frac2) >= 0.3
    dev = "cuda"
    qd, kad, vad, kbd, vbd = (t.to(dev) for t in (q, ka, va, kb, vb))
    st = ring.RingState(B, H, Lq, d, dev)
    # step 1 alone (init), finalised
    _lib.ra_step(qd, kad, vad, qr, kr, True, scale, st.o, st.m, st.l, init=True)
    o1 = torch.empty_like(qd)
    l1 = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    _lib.ra_finalize(st.o, st.m, st.l, o1, l1)
    # checkpoint the state, resume it in a fresh buffer with the second block
    saved = [x.clone() for x in (st.o, st.m, st.l)]
    st2 = ring.RingState(B, H, Lq, d, dev)
    for x, y in zip((st2.o, st2.m, st2.l), saved):
        x.copy_(y)
    o2 = torch.empty_like(qd)
    l2 = torch.empty_like(l1)
    # the second block sits at the same positions; the oracle sees both as one
    # key set (the union of the two blocks' keys)
    _lib.ra_step_final(qd, kbd, vbd, qr, kr, True, scale, st2.o, st2.m, st2.l, o2, l2)
    o3 = torch.empty_like(qd)
    l3 = torch.empty_like(l1)
    _lib.ra_step(qd, kbd, vbd, qr, kr, True, scale, st.o, st.m, st.l)
    _lib.ra_finalize(st.o, st.m, st.l, o3, l3)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3)
    ro1, rl1 = np.zeros((B, H, Lq, d)), np.zeros((B, H, Lq))
    ro2, rl2 = np.zeros((B, H, Lq, d)), np.zeros((B, H, Lq))
    kk = np.concatenate([kp, kp])
    for b in range(B):
        for h in range(H):
            ro1[b, h], rl1[b, h] = oracle.attention_rows(qf[b, h], qp, kaf[b, h], vaf[b, h], kp, scale, True)
            ro2[b, h], rl2[b, h] = oracle.attention_rows(qf[b, h], qp, np.concatenate([kaf[b, h], kbf[b, h]]),
                                                         np.concatenate([vaf[b, h], vbf[b, h]]), kk, scale, True)
    for go, gl, ro, rl, name in ((o1, l1, ro1, rl1, "first step"), (o2, l2, ro2, rl2, "resumed step")):
        go, gl = go.float().cpu().double().numpy(), gl.cpu().double().numpy()
        empty = ~np.isfinite(rl)
        assert np.array_equal(empty, ~np.isfinite(gl))
        assert np.all(go[empty] == 0.0)
        assert_close(go, ro, np.where(empty, 0.0, gl), np.where(empty, 0.0, rl), torch.bfloat16,
                     f"rising step case {ci} {name}")


@pytest.mark.parametrize("T,S_sp,d", [(3, 900, 128), (4, 517, 64)])
def test_rescale_factored_spatial(gpu_lib, T, S_sp, d):
    banner(f"rising scores inside each frame, factored spatial T={T} S_sp={S_sp} d={d}")
    B, H = 1, 4
    N = T * S_sp
    sp = np.arange(N) % S_sp  # position inside the frame
    q, k, v = rising.rising_global(940 + d, B, H, H, N, d, q_gain=6.0, lo=0.1, hi=5.0, key_pos=sp, span=S_sp)
    scale = d ** -0.5
    qf, kf, vf = (_f64(t) for t in (q, k, v))
    frac = []
    for h in range(H):
        for t in range(T):
            r = slice(t * S_sp, (t + 1) * S_sp)
            cnt, _ = rising.partial_rescales(qf[0, h, r], np.arange(S_sp), [(kf[0, h, r], np.arange(S_sp))],
                                             scale, False)
            frac.append((cnt > 0).mean())
    print(f"rows with a partial rescale: {np.mean(frac):.3f}", flush=True)
    assert np.mean(frac) >= 0.9
    qd, kd, vd = (t.to("cuda") for t in (q, k, v))
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    _lib.ra_factored_spatial(qd, kd, vd, T, S_sp, scale, out, lse)
    torch.cuda.synchronize()
    ro, rl = np.zeros((B, H, N, d)), np.zeros((B, H, N))
    for h in range(H):
        ro[0, h], rl[0, h] = oracle.factored_spatial(qf[0, h], kf[0, h], vf[0, h], T, S_sp, scale)
    assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, torch.bfloat16,
                 f"rising factored spatial T{T} S{S_sp} d{d}")


def test_rescale_llm_32k_rank0_sampled(gpu_lib):
    w = configs.LLM_32K_CP4
    # blocks in rising order: the late chunk's rows see higher scores at every step
    order = [3, 2, 1, 0]
    banner(f"{w.name} rising scores, rank 0, order {order}, sampled rows")
    q, k, v = rising.rising_global(902, w.B, w.H, w.Hkv, w.S, w.d, q_gain=8.0, lo=0.25, hi=4.0)
    rows = sample_rows(w, 0)
    _ring_rescale_case(w, 0, q, k, v, order, min_frac=0.4, rows=rows)

"""GPU parity with NaN right after the last row of every input tensor.

The kernels read ragged tails (K/V tiles past Lk, query and dO tiles past Lq,
the dK/dV kernel's owned rows past Lk) through bounds-checked buffer loads
whose record size is one slice and whose row offset is a scalar operand; the
hardware returns zero for every byte past the record. If the scalar offset
were not part of that check, the last slice's tail would read whatever
follows the tensor, and a NaN there would turn P = 0 into 0 * NaN = NaN in
the output or the gradients. Here every input is a view at the start of a
larger allocation whose remaining bytes are NaN (every read stays inside the
allocation), and the results are checked against the oracle: the forward
output and lse, dq, dk and dv (the derivative of the definition the Day 83
post's ring computes), factored spatial and temporal attention.
"""

import numpy as np
import pytest
import torch

import oracle
import seeded
from context_attention_ra_amd import _lib, ring
from ringcase import assert_close, compare

pytestmark = pytest.mark.gpu

PAD_ROWS = 512  # more than any tile or owned-row block runs past a slice


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def nan_tailed(x):
    """A GPU copy of CPU tensor x at the start of a buffer whose remaining
    PAD_ROWS * d elements are NaN; returns the (contiguous) view."""
    n = x.numel()
    buf = torch.full((n + PAD_ROWS * x.shape[-1],), float("nan"), dtype=x.dtype, device="cuda")
    buf[:n].copy_(x.reshape(-1).to("cuda"))
    v = buf[:n].view(x.shape)
    assert v.is_contiguous() and torch.isnan(buf[n:]).all()
    return v


def grad_close(gpu, ref, what):
    mx, mr = compare(gpu, ref)
    scale = max(float(np.abs(ref).max()), 1e-30)
    msg = f"{what}: max_abs={mx:.3e} (max|ref|={scale:.3e}) mean_rel={mr:.3e}"
    print(msg, flush=True)
    assert mx <= 2e-2 * scale and mr <= 1e-2, msg


TAIL_CASES = [
    # (B, H, Lq, q_runs, Lk, k_runs, d, causal)
    (1, 2, 300, [(0, 300)], 333, [(0, 333)], 128, False),
    (1, 3, 517, [(600, 517)], 999, [(0, 999)], 64, True),
    (2, 1, 190, [(40, 100), (1000, 90)], 161, [(0, 100), (950, 61)], 128, True),
    (1, 1, 33, [(0, 33)], 65, [(0, 65)], 64, False),
]


@pytest.mark.parametrize("ci", range(len(TAIL_CASES)))
def test_nan_after_last_row_forward_and_backward(gpu_lib, ci):
    B, H, Lq, qr, Lk, kr, d, causal = TAIL_CASES[ci]
    banner(f"NaN-tailed inputs, case {ci}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} causal={causal}")
    dt = torch.bfloat16
    qc = seeded.gen_bhsd(700 + ci, seeded.Q, B, H, 0, Lq, d, dt)
    kc = seeded.gen_bhsd(700 + ci, seeded.K, B, H, 0, Lk, d, dt)
    vc = seeded.gen_bhsd(700 + ci, seeded.V, B, H, 0, Lk, d, dt)
    dc = seeded.gen_bhsd(700 + ci, seeded.DO, B, H, 0, Lq, d, dt)
    q, k, v, do = (nan_tailed(t) for t in (qc, kc, vc, dc))
    scale = d ** -0.5
    st = ring.RingState(B, H, Lq, d, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    _lib.ra_step_final(q, k, v, qr, kr, causal, scale, st.o, st.m, st.l, out, lse, init=True)
    # the step form too: state written, then finalised
    st2 = ring.RingState(B, H, Lq, d, "cuda")
    _lib.ra_step(q, k, v, qr, kr, causal, scale, st2.o, st2.m, st2.l, init=True)
    out2 = torch.empty_like(q)
    _lib.ra_finalize(st2.o, st2.m, st2.l, out2)
    delta = torch.empty_like(lse)
    _lib.ra_bwd_prep(out, do, delta)
    dq = torch.empty((B, H, Lq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((B, H, Lk, d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    _lib.ra_step_bwd(q, k, v, do, lse, delta, qr, kr, causal, scale, dq, dk, dv, init_dq=True, init_dkv=True)
    torch.cuda.synchronize()
    for name, t in (("out", out), ("out (step + finalize)", out2), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(t.float()).any(), f"NaN from past the tensor in {name}"
    assert torch.equal(out, out2)
    qp = np.concatenate([np.arange(s, s + n) for s, n in qr])
    kp = np.concatenate([np.arange(s, s + n) for s, n in kr])
    qf, kf, vf, df = (seeded.exact_f64(t) for t in (qc, kc, vc, dc))
    ro, rl = np.zeros((B, H, Lq, d)), np.zeros((B, H, Lq))
    rq, rk, rv = np.zeros((B, H, Lq, d)), np.zeros((B, H, Lk, d)), np.zeros((B, H, Lk, d))
    for b in range(B):
        for h in range(H):
            ro[b, h], rl[b, h] = oracle.attention_rows(qf[b, h], qp, kf[b, h], vf[b, h], kp, scale, causal)
            rq[b, h], rk[b, h], rv[b, h] = oracle.attention_grads(qf[b, h], qp, kf[b, h], vf[b, h], kp, scale,
                                                                  causal, df[b, h])
    go, gl = out.float().cpu().double().numpy(), lse.cpu().double().numpy()
    empty = ~np.isfinite(rl)
    assert np.array_equal(empty, ~np.isfinite(gl))
    assert_close(go, ro, np.where(empty, 0.0, gl), np.where(empty, 0.0, rl), dt, f"NaN-tailed case {ci}")
    for g, r, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        grad_close(g.cpu().double().numpy(), r, f"NaN-tailed case {ci} {n}")


@pytest.mark.parametrize("kind", ["spatial", "temporal"])
@pytest.mark.parametrize("T,S_sp,d", [(3, 130, 128), (5, 37, 64)])
def test_nan_after_last_row_factored(gpu_lib, kind, T, S_sp, d):
    banner(f"NaN-tailed inputs, factored {kind} T={T} S_sp={S_sp} d={d}")
    B, H, N = 1, 2, T * S_sp
    qc, kc, vc = (seeded.gen_bhsd(720 + d, tid, B, H, 0, N, d, torch.bfloat16) for tid in range(3))
    q, k, v = (nan_tailed(t) for t in (qc, kc, vc))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = d ** -0.5
    fn = _lib.ra_factored_spatial if kind == "spatial" else _lib.ra_factored_temporal
    fn(q, k, v, T, S_sp, scale, out, lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    ofn = oracle.factored_spatial if kind == "spatial" else oracle.factored_temporal
    qf, kf, vf = (seeded.exact_f64(t) for t in (qc, kc, vc))
    ro, rl = np.zeros((B, H, N, d)), np.zeros((B, H, N))
    for h in range(H):
        ro[0, h], rl[0, h] = ofn(qf[0, h], kf[0, h], vf[0, h], T, S_sp, scale)
    assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, torch.bfloat16,
                 f"NaN-tailed factored {kind}")

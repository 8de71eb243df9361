"""GPU parity of a ring step at the largest query slice the boundary accepts.

ra_step takes one (batch, head) slice of Q of up to INT32_MAX bytes; the
non-final step kernel addresses a lane's query row as a 32-bit element offset
inside the slice, so the rows at the end of the largest slice are where an
overflow would show. One head of 2^23 - 64 query rows (just under 2 GiB of
bf16) attends to one 64-key block; the first and last rows of the slice are
checked against the oracle (the definition of attention, Day 83 post,
"Context parallelism: splitting the sequence"), with and without the causal
mask. Further tests run the largest K/V slice (2^23 - 64 keys) against a
closed form, the backward step over the largest query slice, and factored
temporal attention over the largest long-clip slice. Inputs are
drawn on the GPU with a seeded generator; the checked rows are read back and
given to the oracle as they are.
"""

import numpy as np
import pytest
import torch

import oracle
import seeded
from context_attention_ra_amd import _lib, ring
from ringcase import assert_close, compare

pytestmark = pytest.mark.gpu

LQ = (1 << 23) - 64  # 2^31 - 2^14 bytes of bf16 at d = 128
LK, D = 64, 128
EDGE = 96


def banner(msg):
    print(f"\n[limits] {msg}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_largest_query_slice_step(gpu_lib, causal):
    banner(f"ra_step over {LQ} query rows, causal={causal}")
    assert LQ * D * 2 <= 2**31 - 1
    g = torch.Generator(device="cuda")
    g.manual_seed(2024 + causal)
    q = torch.randn((1, 1, LQ, D), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((1, 1, LK, D), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((1, 1, LK, D), device="cuda", generator=g).to(torch.bfloat16)
    # causal: queries at positions 0.., keys at 0..63, so the first rows see
    # part of the block and the rest all of it
    q_runs, k_runs = [(0, LQ)], [(0, LK)]
    st = ring.RingState(1, 1, LQ, D, "cuda")
    scale = D ** -0.5
    _lib.ra_step(q, k, v, q_runs, k_runs, causal, scale, st.o, st.m, st.l, init=True)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(EDGE), np.arange(LQ - EDGE, LQ)])
    ri = torch.as_tensor(rows, device="cuda")
    o = st.o[0, 0].index_select(0, ri).double().cpu().numpy()
    m = st.m[0, 0].index_select(0, ri).double().cpu().numpy()
    l = st.l[0, 0].index_select(0, ri).double().cpu().numpy()
    out = o / l[:, None]
    lse = m + np.log(l)
    qc = seeded.exact_f64(q[0, 0].index_select(0, ri).cpu())
    kc, vc = (seeded.exact_f64(t[0, 0].cpu()) for t in (k, v))
    ro, rl = oracle.attention_rows(qc, rows, kc, vc, np.arange(LK), scale, causal)
    assert np.all(np.isfinite(rl)), "every checked row sees a key"
    assert_close(out, ro, lse, rl, torch.bfloat16, f"largest slice causal={causal}")
    del q, st
    torch.cuda.empty_cache()


def test_largest_kv_slice_step(gpu_lib):
    """One block of 2^23 - 64 keys (just under 2 GiB of bf16 per tensor): all
    keys are zero (score 0) except the last 64, which are small random
    directions, so the expected output has a closed form that a chunked fp64
    sum over V computes: out_i = (sum_j w_ij v_j) / (sum_j w_ij) with w_ij = 1
    for the plain keys and exp(s_ij) for the last 64."""
    LKB, LQB = (1 << 23) - 64, 64
    banner(f"ra_step over a block of {LKB} keys")
    assert LKB * D * 2 <= 2**31 - 1
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    q = torch.randn((1, 1, LQB, D), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((1, 1, LKB, D), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.zeros((1, 1, LKB, D), device="cuda", dtype=torch.bfloat16)
    # the last 64 keys: small random directions (scores of about a quarter)
    k[0, 0, LKB - 64:] = (0.25 * torch.randn((64, D), device="cuda", generator=g)).to(torch.bfloat16)
    st = ring.RingState(1, 1, LQB, D, "cuda")
    scale = D ** -0.5
    _lib.ra_step(q, k, v, [(0, LQB)], [(0, LKB)], False, scale, st.o, st.m, st.l, init=True)
    torch.cuda.synchronize()
    o = st.o[0, 0].double().cpu().numpy()
    m = st.m[0, 0].double().cpu().numpy()
    l = st.l[0, 0].double().cpu().numpy()
    out, lse = o / l[:, None], m + np.log(l)
    # closed form: the plain keys contribute weight 1 each and their V rows' sum
    qc = seeded.exact_f64(q[0, 0].cpu())
    kt = seeded.exact_f64(k[0, 0, LKB - 64:].cpu())
    vt = seeded.exact_f64(v[0, 0, LKB - 64:].cpu())
    vsum = np.zeros(D)
    step = 1 << 20
    for r0 in range(0, LKB - 64, step):
        r1 = min(r0 + step, LKB - 64)
        vsum += seeded.exact_f64(v[0, 0, r0:r1].cpu()).sum(axis=0)
    s = scale * (qc @ kt.T)                       # [LQB, 64]
    smax = np.maximum(s.max(axis=1), 0.0)
    wt = np.exp(s - smax[:, None])
    w0 = np.exp(-smax) * (LKB - 64)               # the plain keys' total weight
    den = w0 + wt.sum(axis=1)
    ro = (np.exp(-smax)[:, None] * vsum[None, :] + wt @ vt) / den[:, None]
    rl = smax + np.log(den)
    assert_close(out, ro, lse, rl, torch.bfloat16, "largest block")
    del k, v, st
    torch.cuda.empty_cache()


def grad_close(gpu, ref, what):
    """Gradients relative to their own scale (max |ref|) and in aggregate."""
    mx, mr = compare(gpu, ref)
    sc = max(float(np.abs(ref).max()), 1e-30)
    msg = f"{what}: max_abs={mx:.3e} (max|ref|={sc:.3e}) mean_rel={mr:.3e}"
    print(msg, flush=True)
    assert mx <= 2e-2 * sc and mr <= 1e-2, msg


def test_largest_query_slice_backward(gpu_lib):
    """The backward step over the largest query slice against one 64-key
    block. The upstream gradient is zero except on the first and last rows, so
    dk and dv, sums over all 2^23 - 64 queries that the dK/dV kernel streams
    to the end of the slice, equal the oracle's gradients of those rows alone;
    dq of those rows is checked too, and dq of a row with zero upstream
    gradient must be exactly zero."""
    banner(f"ra_step_bwd over {LQ} query rows")
    g = torch.Generator(device="cuda")
    g.manual_seed(4048)
    q = torch.randn((1, 1, LQ, D), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((1, 1, LK, D), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((1, 1, LK, D), device="cuda", generator=g).to(torch.bfloat16)
    rows = np.concatenate([np.arange(EDGE), np.arange(LQ - EDGE, LQ)])
    ri = torch.as_tensor(rows, device="cuda")
    do = torch.zeros((1, 1, LQ, D), device="cuda", dtype=torch.bfloat16)
    do[0, 0].index_copy_(0, ri, torch.randn((len(rows), D), device="cuda", generator=g).to(torch.bfloat16))
    runs_q, runs_k = [(0, LQ)], [(0, LK)]
    scale = D ** -0.5
    st = ring.RingState(1, 1, LQ, D, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((1, 1, LQ), dtype=torch.float32, device="cuda")
    _lib.ra_step_final(q, k, v, runs_q, runs_k, False, scale, st.o, st.m, st.l, out, lse, init=True)
    del st
    delta = torch.empty_like(lse)
    _lib.ra_bwd_prep(out, do, delta)
    del out
    dq = torch.empty((1, 1, LQ, D), dtype=torch.float32, device="cuda")
    dk = torch.empty((1, 1, LK, D), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    _lib.ra_step_bwd(q, k, v, do, lse, delta, runs_q, runs_k, False, scale, dq, dk, dv, init_dq=True, init_dkv=True)
    torch.cuda.synchronize()
    kc, vc = (seeded.exact_f64(t[0, 0].cpu()) for t in (k, v))
    qs, dos = (seeded.exact_f64(t[0, 0].index_select(0, ri).cpu()) for t in (q, do))
    rq, rk, rv = oracle.attention_grads(qs, rows, kc, vc, np.arange(LK), scale, False, dos)
    grad_close(dq[0, 0].index_select(0, ri).double().cpu().numpy(), rq, "largest slice dq")
    grad_close(dk[0, 0].double().cpu().numpy(), rk, "largest slice dk")
    grad_close(dv[0, 0].double().cpu().numpy(), rv, "largest slice dv")
    mid = torch.as_tensor([EDGE, LQ // 2, LQ - EDGE - 1], device="cuda")
    assert bool((dq[0, 0].index_select(0, mid) == 0).all()), "rows with zero upstream gradient"
    del q, do, dq
    torch.cuda.empty_cache()


def test_largest_temporal_slice(gpu_lib):
    """Factored temporal attention of the longest clip (128 frames) with the
    largest slice the long-clip kernel accepts (T * S_sp * d bf16 values just
    under 2 GiB): the temporal attention at a spatial position is plain
    attention among its T tokens, so each checked position's rows are taken
    out and given to the oracle as a clip of one position."""
    T = 128
    S_sp = (2**31 - 1) // (T * D * 2)
    N = T * S_sp
    banner(f"ra_factored_temporal, T={T} S_sp={S_sp} ({N} tokens)")
    g = torch.Generator(device="cuda")
    g.manual_seed(128)
    q, k, v = (torch.randn((1, 1, N, D), device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    out = torch.empty_like(q)
    lse = torch.empty((1, 1, N), dtype=torch.float32, device="cuda")
    scale = D ** -0.5
    _lib.ra_factored_temporal(q, k, v, T, S_sp, scale, out, lse)
    torch.cuda.synchronize()
    for s in (0, 1, S_sp // 2, S_sp - 2, S_sp - 1):
        ri = torch.arange(T, device="cuda") * S_sp + s
        qc, kc, vc = (seeded.exact_f64(t[0, 0].index_select(0, ri).cpu()) for t in (q, k, v))
        ro, rl = oracle.factored_temporal(qc, kc, vc, T, 1, scale)
        assert_close(out[0, 0].index_select(0, ri).double().cpu().numpy(), ro,
                     lse[0, 0].index_select(0, ri).double().cpu().numpy(), rl, torch.bfloat16,
                     f"largest temporal slice, position {s}")
    del q, k, v, out
    torch.cuda.empty_cache()

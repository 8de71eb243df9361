"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name and shape before touching the GPU. Tolerances are
the ones stated for the method's outputs (see ringcase.TOL).
"""

import numpy as np
import pytest
import torch

import oracle
import seeded
from context_attention_ra_amd import _lib, configs, ring
from ringcase import RingCase, assert_close, compare, sample_rows

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def run_case(case, **kw):
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, case.rank, case.w.causal,
                           scale=case.w.scale, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_tiny_f32_ring(gpu_lib, rank):
    w = configs.TINY_F32
    banner(f"{w.name} rank {rank}")
    case = RingCase(w, rank)
    out, lse = run_case(case)
    ro, rl = case.expected()
    assert_close(out.cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, w.dtype, w.name)


@pytest.mark.parametrize("rank", [0, 1])
def test_causal_2rank_full(gpu_lib, rank):
    w = configs.CAUSAL_2RANK
    banner(f"{w.name} rank {rank}")
    case = RingCase(w, rank)
    out, lse = run_case(case)
    ro, rl = case.expected()
    assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, w.dtype, w.name)


def _sampled(w, rank, **kw):
    banner(f"{w.name} rank {rank} (sampled rows)")
    case = RingCase(w, rank)
    out, lse = run_case(case, **kw)
    rows = sample_rows(w, rank)
    ro, rl = case.expected(rows)
    idx = torch.as_tensor(rows, device=out.device)
    go = out.index_select(2, idx).float().cpu().double().numpy()
    gl = lse.index_select(2, idx).cpu().double().numpy()
    assert_close(go, ro, gl, rl, w.dtype, f"{w.name} r{rank} {rows.size} rows/head")
    # properties that hold for every row: finite output, finite lse
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    return case, out, lse


def test_llm_32k_rank0_sampled(gpu_lib):
    _sampled(configs.LLM_32K_CP4, 0)


@pytest.mark.slow
@pytest.mark.parametrize("rank", [1, 2, 3])
def test_llm_32k_other_ranks_sampled(gpu_lib, rank):
    _sampled(configs.LLM_32K_CP4, rank)


@pytest.mark.slow
def test_video_dit_432k_sampled(gpu_lib):
    _sampled(configs.VIDEO_DIT_CP8, 3)


def _video_inputs(v, device="cuda"):
    qkv = [seeded.gen_bhsd(v.wid, tid, v.B, v.H, 0, v.N, v.d, v.dtype, device)
           for tid in (seeded.Q, seeded.K, seeded.V)]
    return qkv


@pytest.mark.parametrize("kind", ["spatial", "temporal"])
def test_video_factored_full(gpu_lib, kind):
    v = configs.VIDEO_FACTORED
    banner(f"{v.name} {kind}")
    q, k, vv = _video_inputs(v)
    out = torch.empty_like(q)
    lse = torch.empty((v.B, v.H, v.N), dtype=torch.float32, device=q.device)
    fn = _lib.ra_factored_spatial if kind == "spatial" else _lib.ra_factored_temporal
    fn(q, k, vv, v.T, v.S_sp, v.scale, out, lse)
    torch.cuda.synchronize()
    ofn = oracle.factored_spatial if kind == "spatial" else oracle.factored_temporal
    ro = np.zeros((v.B, v.H, v.N, v.d))
    rl = np.zeros((v.B, v.H, v.N))
    qc, kc, vc = (seeded.exact_f64(t.cpu()) for t in (q, k, vv))
    for b in range(v.B):
        for h in range(v.H):
            ro[b, h], rl[b, h] = ofn(qc[b, h], kc[b, h], vc[b, h], v.T, v.S_sp, v.scale)
    assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, v.dtype,
                 f"{v.name} {kind}")


@pytest.mark.parametrize("kind", ["spatial", "temporal"])
@pytest.mark.parametrize("d,T,S_sp", [(64, 5, 37), (128, 16, 7), (128, 3, 130), (64, 16, 257)])
def test_factored_ragged(gpu_lib, kind, d, T, S_sp):
    banner(f"factored {kind} d={d} T={T} S_sp={S_sp}")
    B, H = 2, 3
    N = T * S_sp
    q, k, v = (seeded.gen_bhsd(90 + d, tid, B, H, 0, N, d, torch.bfloat16, "cuda") for tid in range(3))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = d ** -0.5
    fn = _lib.ra_factored_spatial if kind == "spatial" else _lib.ra_factored_temporal
    fn(q, k, v, T, S_sp, scale, out, lse)
    torch.cuda.synchronize()
    ofn = oracle.factored_spatial if kind == "spatial" else oracle.factored_temporal
    qc, kc, vc = (seeded.exact_f64(t.cpu()) for t in (q, k, v))
    ro = np.zeros((B, H, N, d))
    rl = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            ro[b, h], rl[b, h] = ofn(qc[b, h], kc[b, h], vc[b, h], T, S_sp, scale)
    assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl,
                 torch.bfloat16, f"{kind} d{d} T{T} S{S_sp}")


# ---- single-step cases with ragged tails and arbitrary segment tables ---------

STEP_CASES = [
    # (B, H, Lq, q_runs, Lk, k_runs, d, causal, dtype)
    (1, 1, 128, [(0, 128)], 64, [(0, 64)], 128, False, torch.bfloat16),
    (2, 3, 300, [(0, 300)], 200, [(100, 200)], 128, True, torch.bfloat16),
    (2, 3, 300, [(40, 137), (1000, 163)], 333, [(0, 250), (900, 83)], 128, True, torch.bfloat16),
    (1, 2, 517, [(0, 517)], 999, [(0, 999)], 64, False, torch.bfloat16),
    (1, 2, 257, [(500, 129), (2000, 128)], 700, [(300, 350), (1900, 350)], 64, True, torch.bfloat16),
    (2, 2, 190, [(64, 190)], 161, [(0, 161)], 64, True, torch.float32),
    (1, 3, 77, [(10, 40), (300, 37)], 250, [(0, 120), (200, 130)], 128, True, torch.float32),
    (1, 1, 96, [(0, 96)], 33, [(5, 33)], 128, False, torch.float32),
    # degenerate sizes: one query against one key, one query against a block
    # one key longer than a tile, and a single key seen by every query (the
    # output is that key's value row)
    (1, 2, 1, [(5, 1)], 1, [(3, 1)], 128, True, torch.bfloat16),
    (1, 1, 1, [(0, 1)], 65, [(0, 65)], 64, False, torch.bfloat16),
    (3, 1, 33, [(100, 33)], 1, [(50, 1)], 128, True, torch.float32),
]


def _runs_pos(runs):
    return np.concatenate([np.arange(s, s + n) for s, n in runs])


@pytest.mark.parametrize("ci", range(len(STEP_CASES)))
def test_single_step_ragged(gpu_lib, ci):
    B, H, Lq, qr, Lk, kr, d, causal, dt = STEP_CASES[ci]
    banner(f"step case {ci}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} causal={causal} {dt}")
    q = seeded.gen_bhsd(70 + ci, 0, B, H, 0, Lq, d, dt, "cuda")
    k = seeded.gen_bhsd(70 + ci, 1, B, H, 0, Lk, d, dt, "cuda")
    v = seeded.gen_bhsd(70 + ci, 2, B, H, 0, Lk, d, dt, "cuda")
    st = ring.RingState(B, H, Lq, d, "cuda")
    scale = d ** -0.5
    _lib.ra_step(q, k, v, qr, kr, causal, scale, st.o, st.m, st.l, init=True)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    _lib.ra_finalize(st.o, st.m, st.l, out, lse)
    torch.cuda.synchronize()
    qp, kp = _runs_pos(qr), _runs_pos(kr)
    qc, kc, vc = (seeded.exact_f64(t.cpu()) for t in (q, k, v))
    ro = np.zeros((B, H, Lq, d))
    rl = np.zeros((B, H, Lq))
    for b in range(B):
        for h in range(H):
            ro[b, h], rl[b, h] = oracle.attention_rows(qc[b, h], qp, kc[b, h], vc[b, h], kp, scale, causal)
    go, gl = out.float().cpu().double().numpy(), lse.cpu().double().numpy()
    empty = ~np.isfinite(rl)
    assert np.array_equal(empty, ~np.isfinite(gl)), "rows without visible keys must give lse = -inf"
    assert np.all(go[empty] == 0.0)
    rl_f = np.where(empty, 0.0, rl)
    gl_f = np.where(empty, 0.0, gl)
    assert_close(go, ro, gl_f, rl_f, dt, f"step case {ci}")


def test_rows_without_visible_keys(gpu_lib):
    banner("causal rows that see no key: out = 0, lse = -inf, state untouched")
    d, B, H = 128, 1, 2
    q = seeded.gen_bhsd(81, 0, B, H, 0, 64, d, torch.bfloat16, "cuda")
    k = seeded.gen_bhsd(81, 1, B, H, 0, 128, d, torch.bfloat16, "cuda")
    v = seeded.gen_bhsd(81, 2, B, H, 0, 128, d, torch.bfloat16, "cuda")
    st = ring.RingState(B, H, 64, d, "cuda")
    # queries at positions 0..63, keys at 1000.. : nothing visible
    _lib.ra_step(q, k, v, [(0, 64)], [(1000, 128)], True, d ** -0.5, st.o, st.m, st.l, init=True)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, 64), dtype=torch.float32, device="cuda")
    _lib.ra_finalize(st.o, st.m, st.l, out, lse)
    torch.cuda.synchronize()
    assert torch.all(st.l == 0) and torch.all(st.o == 0) and torch.all(torch.isneginf(st.m))
    assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))


def test_block_after_every_query_leaves_state_untouched(gpu_lib):
    banner("causal step whose block lies after every local query: state bitwise unchanged")
    d, B, H, L = 128, 1, 3, 700
    q = seeded.gen_bhsd(82, 0, B, H, 0, L, d, torch.bfloat16, "cuda")
    k = seeded.gen_bhsd(82, 1, B, H, 0, L, d, torch.bfloat16, "cuda")
    v = seeded.gen_bhsd(82, 2, B, H, 0, L, d, torch.bfloat16, "cuda")
    st = ring.RingState(B, H, L, d, "cuda")
    _lib.ra_step(q, k, v, [(0, L)], [(0, L)], True, d ** -0.5, st.o, st.m, st.l, init=True)
    before = (st.o.clone(), st.m.clone(), st.l.clone())
    # the second block starts after the last query: no query tile sees any key
    _lib.ra_step(q, k, v, [(0, L)], [(L, L)], True, d ** -0.5, st.o, st.m, st.l)
    torch.cuda.synchronize()
    for a, b in zip(before, (st.o, st.m, st.l)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,dt", [(128, torch.bfloat16), (64, torch.bfloat16), (64, torch.float32)])
@pytest.mark.parametrize("init", [False, True])
def test_step_final_equals_step_then_finalize(gpu_lib, d, dt, init):
    banner(f"ra_step_final vs ra_step + ra_finalize: d{d} {dt} init={init}")
    B, H, L, Lk = 1, 3, 700, 300
    q = seeded.gen_bhsd(83, 0, B, H, 0, L, d, dt, "cuda")
    ka = seeded.gen_bhsd(83, 1, B, H, 0, L, d, dt, "cuda")
    va = seeded.gen_bhsd(83, 2, B, H, 0, L, d, dt, "cuda")
    kb = seeded.gen_bhsd(83, 3, B, H, 0, Lk, d, dt, "cuda")
    vb = seeded.gen_bhsd(83, 4, B, H, 0, Lk, d, dt, "cuda")
    scale = d ** -0.5
    qr = [(0, L)]
    # block b at positions 600..899: the query rows before 600 (the first two
    # 256-row tiles) see none of it, the third tile straddles the diagonal
    kbr = [(600, Lk)]
    st = ring.RingState(B, H, L, d, "cuda")
    if not init:
        _lib.ra_step(q, ka, va, qr, [(0, L)], True, scale, st.o, st.m, st.l, init=True)
    before = (st.o.clone(), st.m.clone(), st.l.clone())
    out2 = torch.empty_like(q)
    lse2 = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    _lib.ra_step_final(q, kb, vb, qr, kbr, True, scale, st.o, st.m, st.l, out2, lse2, init=init)
    torch.cuda.synchronize()
    if dt == torch.bfloat16:
        # the state is an input only on the matrix-core path
        for a, b in zip(before, (st.o, st.m, st.l)):
            assert torch.equal(a, b)
    ref = ring.RingState(B, H, L, d, "cuda")
    for x, y in zip((ref.o, ref.m, ref.l), before):
        x.copy_(y)
    _lib.ra_step(q, kb, vb, qr, kbr, True, scale, ref.o, ref.m, ref.l, init=init)
    out1 = torch.empty_like(q)
    lse1 = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    _lib.ra_finalize(ref.o, ref.m, ref.l, out1, lse1)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(torch.isneginf(lse1), torch.isneginf(lse2))
    fin = torch.isfinite(lse1)
    assert torch.all(torch.isfinite(lse2) == fin)
    assert (lse1[fin] - lse2[fin]).abs().max().item() <= 1e-5
    if init:
        # rows before position 600 see no key at all
        assert torch.all(out2[:, :, :600].float() == 0) and torch.all(torch.isneginf(lse2[:, :, :600]))


# ---- invariants on the GPU --------------------------------------------------------

@pytest.fixture(scope="module")
def c2_case(gpu_lib):
    return RingCase(configs.CAUSAL_2RANK, 0)


def test_block_order_independence(c2_case):
    banner("block order: ring order vs reversed (causal 4k, P=2) and 4-block orders")
    w = c2_case.w
    o1, l1 = run_case(c2_case)
    o2, l2 = run_case(c2_case, order=[1, 0])
    ro, rl = c2_case.expected()
    for o, l, name in ((o1, l1, "ring"), (o2, l2, "reversed")):
        assert_close(o.float().cpu().double().numpy(), ro, l.cpu().double().numpy(), rl, w.dtype, name)


@pytest.mark.parametrize("order", [[2, 1, 0, 3], [3, 2, 1, 0], [0, 3, 1, 2]])
def test_tiny_f32_any_order(gpu_lib, order):
    w = configs.TINY_F32
    banner(f"{w.name} rank 2 order {order}")
    case = RingCase(w, 2)
    out, lse = run_case(case, order=order)
    ro, rl = case.expected()
    assert_close(out.cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, w.dtype, str(order))


def test_running_state_equals_merge_of_partials(c2_case):
    banner("running state vs per-step partials merged with ra_merge_lse")
    case = c2_case
    w = case.w
    order = [0, 1]
    parts = []
    for t in order:
        st = ring.RingState(w.B, w.H, w.L, w.d, "cuda")
        k, v = case.kv[t]
        _lib.ra_step(case.q, k, v, case.q_segs, case.kv_segs[t], True, w.scale, st.o, st.m, st.l, init=True)
        o = torch.empty_like(case.q)
        lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device="cuda")
        _lib.ra_finalize(st.o, st.m, st.l, o, lse)
        parts.append((o, lse))
    om = torch.empty_like(case.q)
    lm = torch.empty_like(parts[0][1])
    _lib.ra_merge_lse(parts[0][0], parts[0][1], parts[1][0], parts[1][1], om, lm)
    torch.cuda.synchronize()
    ro, rl = case.expected()
    assert_close(om.float().cpu().double().numpy(), ro, lm.cpu().double().numpy(), rl, w.dtype, "merged")


def test_init_flag_equals_explicit_empty_state(c2_case):
    banner("RA_STEP_INIT vs an explicit (0, -inf, 0) state: bitwise")
    case, w = c2_case, c2_case.w
    k, v = case.kv[0]
    a = ring.RingState(w.B, w.H, w.L, w.d, "cuda")
    b = ring.RingState(w.B, w.H, w.L, w.d, "cuda")
    _lib.ra_step(case.q, k, v, case.q_segs, case.kv_segs[0], True, w.scale, a.o, a.m, a.l, init=True)
    b.o.zero_()
    b.m.fill_(float("-inf"))
    b.l.zero_()
    _lib.ra_step(case.q, k, v, case.q_segs, case.kv_segs[0], True, w.scale, b.o, b.m, b.l, init=False)
    torch.cuda.synchronize()
    assert torch.equal(a.o, b.o) and torch.equal(a.m, b.m) and torch.equal(a.l, b.l)


def test_deterministic_and_prefetch_modes_bitwise(c2_case):
    banner("run-to-run determinism; prefetch vs serial pass; delayed side stream")
    o1, l1 = run_case(c2_case)
    o2, l2 = run_case(c2_case)
    o3, l3 = run_case(c2_case, prefetch=False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    # a copy stream held back by a spin kernel must not change the result
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(50_000_000)
    o4, l4, _ = ring.run(c2_case.q, c2_case.q_segs, c2_case.kv, c2_case.kv_segs, 1, True,
                         scale=c2_case.w.scale, copy_stream=side)
    torch.cuda.synchronize()
    o5, l5, _ = ring.run(c2_case.q, c2_case.q_segs, c2_case.kv, c2_case.kv_segs, 1, True,
                         scale=c2_case.w.scale, prefetch=False)
    torch.cuda.synchronize()
    assert torch.equal(o4, o5) and torch.equal(l4, l5)


def test_checkpoint_resume_bitwise(gpu_lib):
    banner("checkpoint the state after step 1, resume: bitwise equal")
    case = RingCase(configs.TINY_F32, 0)
    w = case.w
    full_o, full_l, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, 0, False, scale=w.scale)
    order = [0, 3, 2, 1]
    st = ring.RingState(w.B, w.H, w.L, w.d, "cuda")
    for s in range(2):
        k, v = case.kv[order[s]]
        _lib.ra_step(case.q, k, v, case.q_segs, case.kv_segs[order[s]], False, w.scale, st.o, st.m, st.l, init=s == 0)
    saved = [x.clone() for x in (st.o, st.m, st.l)]
    st2 = ring.RingState(w.B, w.H, w.L, w.d, "cuda")
    st2.o.copy_(saved[0]), st2.m.copy_(saved[1]), st2.l.copy_(saved[2])
    for s in range(2, 4):
        k, v = case.kv[order[s]]
        _lib.ra_step(case.q, k, v, case.q_segs, case.kv_segs[order[s]], False, w.scale, st2.o, st2.m, st2.l)
    out = torch.empty_like(case.q)
    lse = torch.empty_like(full_l)
    _lib.ra_finalize(st2.o, st2.m, st2.l, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, full_o) and torch.equal(lse, full_l)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_lse_parity(gpu_lib, dt, d):
    banner(f"ra_merge_lse {dt} d={d}, with empty rows and in-place output")
    B, H, L = 2, 3, 333
    oa = seeded.gen_bhsd(60, 0, B, H, 0, L, d, dt, "cuda")
    ob = seeded.gen_bhsd(60, 1, B, H, 0, L, d, dt, "cuda")
    la = (3.0 * seeded.gen_bhsd(60, 2, B, H, 0, L, 1, torch.float32, "cuda"))[..., 0].contiguous()
    lb = (3.0 * seeded.gen_bhsd(60, 3, B, H, 0, L, 1, torch.float32, "cuda"))[..., 0].contiguous()
    la[:, :, :7] = float("-inf")
    lb[:, :, 3:11] = float("-inf")
    oa[:, :, :7] = 0
    ob[:, :, 3:11] = 0
    ref_o, ref_l = [], []
    oac, obc, lac, lbc = (seeded.exact_f64(t.cpu()) for t in (oa, ob, la, lb))
    ro = np.zeros((B, H, L, d))
    rl = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            ro[b, h], rl[b, h] = oracle.merge_lse(oac[b, h], lac[b, h], obc[b, h], lbc[b, h])
    oo = torch.empty_like(oa)
    lo = torch.empty_like(la)
    _lib.ra_merge_lse(oa, la, ob, lb, oo, lo)
    _lib.ra_merge_lse(oa, la, ob, lb, oa, la)  # in place
    torch.cuda.synchronize()
    assert torch.equal(oo, oa) and torch.equal(lo, la)
    go, gl = oo.float().cpu().double().numpy(), lo.cpu().double().numpy()
    both = ~np.isfinite(rl)
    assert np.array_equal(both, ~np.isfinite(gl))
    # the stated output bounds: bf16 2e-2 max-abs and 1e-2 mean-relative; fp32
    # 1e-5 max-abs (tighter than 1e-4: one rescale and one add per element)
    tol, rel_tol = (2e-2, 1e-2) if dt == torch.bfloat16 else (1e-5, 1e-4)
    mx, mr = compare(go, ro)
    lm, _ = compare(np.where(both, 0, gl), np.where(both, 0, rl))
    print(f"merge {dt} d{d}: max_abs={mx:.3e} mean_rel={mr:.3e} lse={lm:.3e}", flush=True)
    assert mx <= tol and mr <= rel_tol and lm <= 1e-5


def test_invalid_arguments_raise_before_launch(gpu_lib):
    banner("argument errors are reported, nothing launched")
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    st = ring.RingState(1, 1, 64, 128, "cuda")
    with pytest.raises(_lib.RaError) as e:
        _lib.ra_step(q, q, q, [(0, 63)], [(0, 64)], True, 0.1, st.o, st.m, st.l, init=True)
    assert e.value.status == _lib.RA_ERR_INVALID_ARG
    with pytest.raises(_lib.RaError) as e:
        _lib.ra_step(q, q, q, [(0, 64)], [(0, 64)], True, float("nan"), st.o, st.m, st.l)
    assert e.value.status == _lib.RA_ERR_INVALID_ARG
    q96 = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device="cuda")
    st96 = ring.RingState(1, 1, 64, 96, "cuda")
    with pytest.raises(_lib.RaError) as e:
        _lib.ra_step(q96, q96, q96, [(0, 64)], [(0, 64)], True, 0.1, st96.o, st96.m, st96.l)
    assert e.value.status == _lib.RA_ERR_UNSUPPORTED


# ---- grouped K/V heads (fewer K/V heads than query heads) -------------------------

GQA_CASES = [
    # (B, H, H_kv, Lq, q_runs, Lk, k_runs, d, causal, dtype)
    (2, 6, 2, 300, [(40, 137), (1000, 163)], 333, [(0, 250), (900, 83)], 128, True, torch.bfloat16),
    (1, 4, 1, 517, [(0, 517)], 999, [(0, 999)], 64, False, torch.bfloat16),
    (1, 8, 4, 640, [(0, 640)], 640, [(0, 640)], 128, True, torch.bfloat16),
    (2, 4, 2, 190, [(64, 190)], 161, [(0, 161)], 64, True, torch.float32),
    (1, 3, 1, 77, [(10, 40), (300, 37)], 250, [(0, 120), (200, 130)], 128, True, torch.float32),
]


def _gqa_inputs(ci, B, H, Hkv, Lq, Lk, d, dt):
    q = seeded.gen_bhsd(200 + ci, 0, B, H, 0, Lq, d, dt, "cuda")
    k = seeded.gen_bhsd(200 + ci, 1, B, Hkv, 0, Lk, d, dt, "cuda")
    v = seeded.gen_bhsd(200 + ci, 2, B, Hkv, 0, Lk, d, dt, "cuda")
    return q, k, v


@pytest.mark.parametrize("ci", range(len(GQA_CASES)))
def test_gqa_single_step(gpu_lib, ci):
    B, H, Hkv, Lq, qr, Lk, kr, d, causal, dt = GQA_CASES[ci]
    banner(f"gqa step case {ci}: B{B} H{H} H_kv{Hkv} Lq{Lq} Lk{Lk} d{d} causal={causal} {dt}")
    q, k, v = _gqa_inputs(ci, B, H, Hkv, Lq, Lk, d, dt)
    st = ring.RingState(B, H, Lq, d, "cuda")
    scale = d ** -0.5
    _lib.ra_step(q, k, v, qr, kr, causal, scale, st.o, st.m, st.l, init=True)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    _lib.ra_finalize(st.o, st.m, st.l, out, lse)
    torch.cuda.synchronize()
    qp, kp = _runs_pos(qr), _runs_pos(kr)
    qc, kc, vc = (seeded.exact_f64(t.cpu()) for t in (q, k, v))
    ro = np.zeros((B, H, Lq, d))
    rl = np.zeros((B, H, Lq))
    for b in range(B):
        ro[b], rl[b] = oracle.grouped_attention(qc[b], qp, kc[b], vc[b], kp, scale, causal)
    go, gl = out.float().cpu().double().numpy(), lse.cpu().double().numpy()
    empty = ~np.isfinite(rl)
    assert np.array_equal(empty, ~np.isfinite(gl))
    assert np.all(go[empty] == 0.0)
    assert_close(go, ro, np.where(empty, 0.0, gl), np.where(empty, 0.0, rl), dt, f"gqa case {ci}")


@pytest.mark.parametrize("ci", [0, 3])
def test_gqa_step_final_equals_step_then_finalize(gpu_lib, ci):
    B, H, Hkv, Lq, qr, Lk, kr, d, causal, dt = GQA_CASES[ci]
    banner(f"gqa ra_step_final vs ra_step + ra_finalize, case {ci}")
    q, k, v = _gqa_inputs(ci, B, H, Hkv, Lq, Lk, d, dt)
    scale = d ** -0.5
    a = ring.RingState(B, H, Lq, d, "cuda")
    out1 = torch.empty_like(q)
    lse1 = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    _lib.ra_step(q, k, v, qr, kr, causal, scale, a.o, a.m, a.l, init=True)
    _lib.ra_finalize(a.o, a.m, a.l, out1, lse1)
    b = ring.RingState(B, H, Lq, d, "cuda")
    out2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse1)
    _lib.ra_step_final(q, k, v, qr, kr, causal, scale, b.o, b.m, b.l, out2, lse2, init=True)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    fin = torch.isfinite(lse1)
    assert torch.equal(fin, torch.isfinite(lse2))
    assert (lse1[fin] - lse2[fin]).abs().max().item() <= 1e-5


def test_gqa_with_one_kv_head_per_query_head_is_ra_step(gpu_lib):
    banner("ra_step_gqa with H_kv = H vs ra_step: bitwise")
    import ctypes
    B, H, L, d = 1, 4, 300, 128
    q, k, v = _gqa_inputs(9, B, H, H, L, L, d, torch.bfloat16)
    a = ring.RingState(B, H, L, d, "cuda")
    b = ring.RingState(B, H, L, d, "cuda")
    _lib.ra_step(q, k, v, [(0, L)], [(0, L)], True, d ** -0.5, a.o, a.m, a.l, init=True)
    qs, ks = _lib.segs([(0, L)]), _lib.segs([(0, L)])
    st = _lib.load().ra_step_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), _lib.RA_BF16, B, H, H, L, L, d,
                                 ctypes.byref(qs), ctypes.byref(ks), _lib.RA_MASK_CAUSAL, d ** -0.5,
                                 _lib.RA_STEP_INIT, b.o.data_ptr(), b.m.data_ptr(), b.l.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == _lib.RA_OK
    torch.cuda.synchronize()
    assert torch.equal(a.o, b.o) and torch.equal(a.m, b.m) and torch.equal(a.l, b.l)


@pytest.mark.parametrize("rank", [0, 1])
def test_gqa_causal_2rank_full(gpu_lib, rank):
    w = configs.CAUSAL_2RANK_GQA
    banner(f"{w.name} rank {rank} (H={w.H}, H_kv={w.Hkv})")
    case = RingCase(w, rank)
    assert case.kv[0][0].shape[1] == w.Hkv
    out, lse = run_case(case)
    ro, rl = case.expected()
    assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, w.dtype, w.name)


def test_gqa_llm_32k_rank0_sampled(gpu_lib):
    _sampled(configs.LLM_32K_CP4_GQA, 0)


# ---- backward ring step -------------------------------------------------------------

DOUT = seeded.DO  # seeded tensor id of the upstream gradient


def grad_close(gpu, ref, what):
    """Gradients are not bounded like outputs: errors are taken relative to the
    gradient's own scale (max |ref|) and in aggregate (sum |diff| / sum |ref|)."""
    mx, mr = compare(gpu, ref)
    scale = max(float(np.abs(ref).max()), 1e-30)
    msg = f"{what}: max_abs={mx:.3e} (max|ref|={scale:.3e}, ratio {mx / scale:.3e}) mean_rel={mr:.3e}"
    print(msg, flush=True)
    assert mx <= 2e-2 * scale and mr <= 1e-2, msg


BWD_CASES = [
    # (B, H, Lq, q_runs, Lk, k_runs, d, causal)
    (1, 2, 256, [(0, 256)], 256, [(0, 256)], 128, True),
    (2, 3, 300, [(40, 137), (1000, 163)], 333, [(0, 250), (900, 83)], 128, True),
    (1, 2, 517, [(0, 517)], 999, [(0, 999)], 64, False),
    (1, 2, 257, [(500, 129), (2000, 128)], 700, [(300, 350), (1900, 350)], 64, True),
    (1, 1, 96, [(0, 96)], 33, [(5, 33)], 128, False),
]


@pytest.mark.parametrize("ci", range(len(BWD_CASES)))
def test_bwd_single_block(gpu_lib, ci):
    B, H, Lq, qr, Lk, kr, d, causal = BWD_CASES[ci]
    banner(f"bwd case {ci}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} causal={causal}")
    dt = torch.bfloat16
    q = seeded.gen_bhsd(300 + ci, 0, B, H, 0, Lq, d, dt, "cuda")
    k = seeded.gen_bhsd(300 + ci, 1, B, H, 0, Lk, d, dt, "cuda")
    v = seeded.gen_bhsd(300 + ci, 2, B, H, 0, Lk, d, dt, "cuda")
    do = seeded.gen_bhsd(300 + ci, DOUT, B, H, 0, Lq, d, dt, "cuda")
    scale = d ** -0.5
    st = ring.RingState(B, H, Lq, d, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    _lib.ra_step_final(q, k, v, qr, kr, causal, scale, st.o, st.m, st.l, out, lse, init=True)
    delta = torch.empty_like(lse)
    _lib.ra_bwd_prep(out, do, delta)
    dq = torch.empty((B, H, Lq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((B, H, Lk, d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    _lib.ra_step_bwd(q, k, v, do, lse, delta, qr, kr, causal, scale, dq, dk, dv, init_dq=True, init_dkv=True)
    torch.cuda.synchronize()
    # delta against the exact values handed to the kernel
    ref_delta = (out.double() * do.double()).sum(-1)
    assert (delta.double() - ref_delta).abs().max().item() <= 1e-4 * max(1.0, ref_delta.abs().max().item())
    qp, kp = _runs_pos(qr), _runs_pos(kr)
    qc, kc, vc, dc = (seeded.exact_f64(t.cpu()) for t in (q, k, v, do))
    rq, rk, rv = (np.zeros((B, H, L, d)) for L in (Lq, Lk, Lk))
    for b in range(B):
        for h in range(H):
            rq[b, h], rk[b, h], rv[b, h] = oracle.attention_grads(qc[b, h], qp, kc[b, h], vc[b, h], kp, scale,
                                                                  causal, dc[b, h])
    for g, r, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        assert torch.isfinite(g).all(), n
        grad_close(g.cpu().double().numpy(), r, f"bwd case {ci} {n}")


def test_bwd_accumulates(gpu_lib):
    banner("ra_step_bwd without the init flags adds to the accumulators")
    B, H, L, d = 1, 2, 200, 64
    dt = torch.bfloat16
    q, k, v, do = (seeded.gen_bhsd(320, t, B, H, 0, L, d, dt, "cuda") for t in range(4))
    lse = torch.full((B, H, L), 5.0, device="cuda")
    delta = torch.full((B, H, L), 0.25, device="cuda")
    acc = [torch.empty((B, H, L, d), dtype=torch.float32, device="cuda") for _ in range(3)]
    _lib.ra_step_bwd(q, k, v, do, lse, delta, [(0, L)], [(0, L)], True, 0.125, *acc, init_dq=True, init_dkv=True)
    once = [a.clone() for a in acc]
    _lib.ra_step_bwd(q, k, v, do, lse, delta, [(0, L)], [(0, L)], True, 0.125, *acc)
    torch.cuda.synchronize()
    for a, o in zip(acc, once):
        assert torch.allclose(a, 2 * o, rtol=1e-6, atol=1e-6)


def test_bwd_halves_touch_only_their_accumulators(gpu_lib):
    banner("ra_step_bwd halves: parts='dq' and parts='dkv' against the whole step")
    B, H, L, d = 1, 2, 200, 128
    dt = torch.bfloat16
    q, k, v, do = (seeded.gen_bhsd(321, t, B, H, 0, L, d, dt, "cuda") for t in range(4))
    lse = torch.full((B, H, L), 5.0, device="cuda")
    delta = torch.full((B, H, L), 0.25, device="cuda")
    new = lambda: [torch.full((B, H, L, d), float("nan"), device="cuda") for _ in range(3)]
    both, dq_only, dkv_only = new(), new(), new()
    args = (q, k, v, do, lse, delta, [(0, L)], [(0, L)], True, 0.125)
    _lib.ra_step_bwd(*args, *both, init_dq=True, init_dkv=True)
    _lib.ra_step_bwd(*args, *dq_only, init_dq=True, init_dkv=True, parts="dq")
    _lib.ra_step_bwd(*args, *dkv_only, init_dq=True, init_dkv=True, parts="dkv")
    torch.cuda.synchronize()
    assert torch.equal(dq_only[0], both[0]) and torch.isnan(dq_only[1]).all() and torch.isnan(dq_only[2]).all()
    assert torch.isnan(dkv_only[0]).all()
    assert torch.equal(dkv_only[1], both[1]) and torch.equal(dkv_only[2], both[2])


@pytest.mark.parametrize("wname", ["causal-bf16-4k-cp2", "causal-bf16-4k-cp2-gqa4", "llm-32k-causal-cp4-gqa4"])
def test_bwd_ring_overlap_matches_one_stream(gpu_lib, wname):
    # the dK/dV halves on a second stream are the same launches on the same
    # inputs: every gradient is bitwise the one of the single-stream ring
    w = configs.RING_WORKLOADS[wname]
    rank = 0
    banner(f"backward ring, {w.name} rank {rank}: dK/dV halves on a second stream vs one stream")
    case = RingCase(w, rank)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, rank, w.causal, scale=w.scale)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, ringcase_positions(w, rank), w.d, w.dtype, "cuda")
    res = [ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, rank, w.causal, out, lse, do,
                        scale=w.scale, overlap=ov) for ov in (False, True)]
    torch.cuda.synchronize()
    (dq1, kv1), (dq2, kv2) = res
    assert torch.equal(dq1, dq2)
    for (a, b), (c, e) in zip(kv1, kv2):
        assert torch.equal(a, c) and torch.equal(b, e)


def _bwd_ring_case(w):
    """Forward and backward of every rank of ring workload w; dK/dV accumulators
    travel over the ranks. Returns the GPU gradients and the per-rank cases."""
    cases = [RingCase(w, r) for r in range(w.P)]
    dkv = None
    dqs, dos = [], []
    for r, case in enumerate(cases):
        out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, r, w.causal, scale=w.scale)
        do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, ringcase_positions(w, r), w.d, w.dtype, "cuda")
        dq, dkv = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, r, w.causal, out, lse, do,
                               scale=w.scale, dkv=dkv)
        dqs.append(dq)
        dos.append(do)
    torch.cuda.synchronize()
    return cases, dqs, dkv


def ringcase_positions(w, r):
    from ringcase import oracle_positions
    return oracle_positions(w, r)


def test_bwd_ring_causal_2rank_all_ranks(gpu_lib):
    w = configs.CAUSAL_2RANK
    banner(f"backward ring, {w.name}, both ranks; dK/dV accumulated over the ranks")
    cases, dqs, dkv = _bwd_ring_case(w)
    S = w.S
    allpos = np.arange(S)
    for b in range(w.B):
        for h in range(w.H):
            ex = lambda tid, rows: seeded.exact_f64(seeded.to_dtype(
                seeded.normal_rows_at(w.wid, tid, b, h, rows, w.d), w.dtype))
            gq, gk, gv, gdo = ex(seeded.Q, allpos), ex(seeded.K, allpos), ex(seeded.V, allpos), ex(DOUT, allpos)
            rq, rk, rv = oracle.attention_grads(gq, allpos, gk, gv, allpos, w.scale, w.causal, gdo)
            for r in range(w.P):
                pos = ringcase_positions(w, r)
                grad_close(dqs[r][b, h].cpu().double().numpy(), rq[pos], f"dq rank {r} h{h}")
                grad_close(dkv[r][0][b, h].cpu().double().numpy(), rk[pos], f"dk block {r} h{h}")
                grad_close(dkv[r][1][b, h].cpu().double().numpy(), rv[pos], f"dv block {r} h{h}")


def test_bwd_ring_block_order_independent(gpu_lib):
    w = configs.CAUSAL_2RANK
    banner(f"backward ring, {w.name} rank 1: ring order vs reversed")
    case = RingCase(w, 1)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, 1, True, scale=w.scale)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, ringcase_positions(w, 1), w.d, w.dtype, "cuda")
    dq1, kv1 = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, 1, True, out, lse, do, scale=w.scale)
    dq2, kv2 = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, 1, True, out, lse, do, scale=w.scale,
                            order=[0, 1])
    torch.cuda.synchronize()
    # dq sums the blocks in another order: equal up to fp32 rounding; dk/dv do not depend on it
    assert torch.allclose(dq1, dq2, rtol=1e-5, atol=1e-5 * dq1.abs().max().item())
    for (a, b), (c, e) in zip(kv1, kv2):
        assert torch.equal(a, c) and torch.equal(b, e)


def test_bwd_llm_32k_rank0_sampled_dq(gpu_lib):
    w = configs.LLM_32K_CP4
    banner(f"backward ring, {w.name} rank 0: dq on sampled rows")
    case = RingCase(w, 0)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, scale=w.scale)
    qpos = ringcase_positions(w, 0)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, qpos, w.d, w.dtype, "cuda")
    dq, dkv = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, out, lse, do, scale=w.scale)
    torch.cuda.synchronize()
    rows = sample_rows(w, 0)
    allpos = np.arange(w.S)
    gpu = dq.index_select(2, torch.as_tensor(rows, device=dq.device)).cpu().double().numpy()
    ref = np.zeros_like(gpu)
    for h in range(w.H):
        ex = lambda tid, r: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, 0, h, r, w.d), w.dtype))
        # dq_i depends on row i alone (and on every key), so a row sample is exact
        ref[0, h], _, _ = oracle.attention_grads(ex(seeded.Q, qpos[rows]), qpos[rows], ex(seeded.K, allpos),
                                                 ex(seeded.V, allpos), allpos, w.scale, True,
                                                 ex(DOUT, qpos[rows]))
    grad_close(gpu, ref, f"{w.name} dq, {rows.size} rows/head")
    for dk, dv in dkv:
        assert torch.isfinite(dk).all() and torch.isfinite(dv).all()


@pytest.mark.slow
def test_bwd_video_dit_432k_sampled_dq(gpu_lib):
    # the backward ring at the video share (54,000 local queries against eight
    # non-causal 54,000-token blocks: ragged 256-key tiles), dq of the sampled
    # rows of three heads against the oracle; dk, dv must be finite
    w = configs.VIDEO_DIT_CP8
    rank = 3
    banner(f"backward ring, {w.name} rank {rank}: dq on sampled rows of heads 0, 15, 31")
    case = RingCase(w, rank)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, rank, w.causal, scale=w.scale)
    qpos = ringcase_positions(w, rank)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, qpos, w.d, w.dtype, "cuda")
    dq, dkv = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, rank, w.causal, out, lse, do,
                           scale=w.scale)
    torch.cuda.synchronize()
    rows = sample_rows(w, rank)
    allpos = np.arange(w.S)
    for h in (0, 15, 31):
        ex = lambda tid, r: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, 0, h, r, w.d), w.dtype))
        ref, _, _ = oracle.attention_grads(ex(seeded.Q, qpos[rows]), qpos[rows], ex(seeded.K, allpos),
                                           ex(seeded.V, allpos), allpos, w.scale, False, ex(DOUT, qpos[rows]))
        gpu = dq[0, h].index_select(0, torch.as_tensor(rows, device=dq.device)).cpu().double().numpy()
        grad_close(gpu, ref, f"{w.name} dq head {h}, {rows.size} rows")
    for dk, dv in dkv:
        assert torch.isfinite(dk).all() and torch.isfinite(dv).all()


@pytest.mark.slow
def test_bwd_video_dit_432k_sampled_dkdv(gpu_lib):
    # dK/dV at the video share: rank 3's contributions to every block, on
    # sampled key rows of head 7 (each needs the lse and output of all 54,000
    # local queries against the 432,000 keys: about 1.2e13 fp64 FLOP, computed
    # in pieces with progress lines)
    w = configs.VIDEO_DIT_CP8
    rank, h = 3, 7
    banner(f"backward ring, {w.name} rank {rank}: dk, dv of sampled key rows of head {h}")
    case = RingCase(w, rank)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, rank, w.causal, scale=w.scale)
    qpos = ringcase_positions(w, rank)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, qpos, w.d, w.dtype, "cuda")
    _, dkv = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, rank, w.causal, out, lse, do,
                          scale=w.scale)
    torch.cuda.synchronize()
    for dk, dv in dkv:
        assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
    allpos = np.arange(w.S)
    ex = lambda tid, r: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, 0, h, r, w.d), w.dtype))
    qf, kf, vf, dof = ex(seeded.Q, qpos), ex(seeded.K, allpos), ex(seeded.V, allpos), ex(DOUT, qpos)
    n = qf.shape[0]
    o, lse_ref = np.zeros((n, w.d)), np.zeros(n)
    step = 6000
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        o[r0:r1], lse_ref[r0:r1] = oracle.attention_rows(qf[r0:r1], qpos[r0:r1], kf, vf, allpos, w.scale, False)
        print(f"  oracle forward rows {r1}/{n}", flush=True)
    # per block: its first and last local row and 30 more, uniform from a seed
    rng = np.random.default_rng([77, rank, h])
    for t in range(w.P):
        kpos = ringcase_positions(w, t)
        local = np.unique(np.concatenate([[0, kpos.size - 1], rng.choice(kpos.size, 30, replace=False)]))
        rk, rv = oracle.attention_kv_grads_rows(qf, qpos, kf, vf, allpos, w.scale, False, dof, kpos[local],
                                                fwd=(o, lse_ref))
        idx = torch.as_tensor(local, device=dkv[t][0].device)
        grad_close(dkv[t][0][0, h].index_select(0, idx).cpu().double().numpy(), rk, f"dk block {t}, {local.size} rows")
        grad_close(dkv[t][1][0, h].index_select(0, idx).cpu().double().numpy(), rv, f"dv block {t}, {local.size} rows")


def test_bwd_llm_32k_rank0_dkdv_two_heads(gpu_lib):
    # dK/dV of every block at the full share: rank 0's contributions, all key
    # rows of heads 0 and H-1 (the oracle's full gradient costs about 10 s per head)
    w = configs.LLM_32K_CP4
    banner(f"backward ring, {w.name} rank 0: dk, dv of every block, heads 0 and {w.H - 1}")
    case = RingCase(w, 0)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, scale=w.scale)
    qpos = ringcase_positions(w, 0)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, qpos, w.d, w.dtype, "cuda")
    _, dkv = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, out, lse, do, scale=w.scale)
    torch.cuda.synchronize()
    allpos = np.arange(w.S)
    for h in (0, w.H - 1):
        ex = lambda tid, r: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, 0, h, r, w.d), w.dtype))
        _, rk, rv = oracle.attention_grads(ex(seeded.Q, qpos), qpos, ex(seeded.K, allpos), ex(seeded.V, allpos),
                                           allpos, w.scale, True, ex(DOUT, qpos))
        for t in range(w.P):
            kpos = ringcase_positions(w, t)
            grad_close(dkv[t][0][0, h].cpu().double().numpy(), rk[kpos], f"dk block {t} h{h}")
            grad_close(dkv[t][1][0, h].cpu().double().numpy(), rv[kpos], f"dv block {t} h{h}")


@pytest.mark.parametrize("ci", [0, 1, 2])  # the bf16 cases (the backward step is bf16 only)
def test_bwd_gqa_single_block(gpu_lib, ci):
    B, H, Hkv, Lq, qr, Lk, kr, d, causal, dt = GQA_CASES[ci]
    banner(f"bwd gqa case {ci}: B{B} H{H} H_kv{Hkv} Lq{Lq} Lk{Lk} d{d} causal={causal}")
    q, k, v = _gqa_inputs(ci, B, H, Hkv, Lq, Lk, d, dt)
    do = seeded.gen_bhsd(200 + ci, DOUT, B, H, 0, Lq, d, dt, "cuda")
    scale = d ** -0.5
    st = ring.RingState(B, H, Lq, d, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    _lib.ra_step_final(q, k, v, qr, kr, causal, scale, st.o, st.m, st.l, out, lse, init=True)
    delta = torch.empty_like(lse)
    _lib.ra_bwd_prep(out, do, delta)
    dq = torch.empty((B, H, Lq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((B, Hkv, Lk, d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    _lib.ra_step_bwd(q, k, v, do, lse, delta, qr, kr, causal, scale, dq, dk, dv, init_dq=True, init_dkv=True)
    torch.cuda.synchronize()
    qp, kp = _runs_pos(qr), _runs_pos(kr)
    qc, kc, vc, dc = (seeded.exact_f64(t.cpu()) for t in (q, k, v, do))
    rq, rk, rv = np.zeros((B, H, Lq, d)), np.zeros((B, Hkv, Lk, d)), np.zeros((B, Hkv, Lk, d))
    for b in range(B):
        rq[b], rk[b], rv[b] = oracle.grouped_attention_grads(qc[b], qp, kc[b], vc[b], kp, scale, causal, dc[b])
    for g, r, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        grad_close(g.cpu().double().numpy(), r, f"bwd gqa case {ci} {n}")


def test_bwd_gqa_ring_causal_2rank_all_ranks(gpu_lib):
    w = configs.CAUSAL_2RANK_GQA
    banner(f"backward ring, {w.name} (H={w.H}, H_kv={w.Hkv}), both ranks")
    cases, dqs, dkv = _bwd_ring_case(w)
    allpos = np.arange(w.S)
    for b in range(w.B):
        ex = lambda tid, h: seeded.exact_f64(seeded.to_dtype(
            seeded.normal_rows_at(w.wid, tid, b, h, allpos, w.d), w.dtype))
        gq = np.stack([ex(seeded.Q, h) for h in range(w.H)])
        gdo = np.stack([ex(DOUT, h) for h in range(w.H)])
        gk = np.stack([ex(seeded.K, h) for h in range(w.Hkv)])
        gv = np.stack([ex(seeded.V, h) for h in range(w.Hkv)])
        rq, rk, rv = oracle.grouped_attention_grads(gq, allpos, gk, gv, allpos, w.scale, w.causal, gdo)
        for r in range(w.P):
            pos = ringcase_positions(w, r)
            grad_close(dqs[r][b].cpu().double().numpy(), rq[:, pos], f"dq rank {r}")
            grad_close(dkv[r][0][b].cpu().double().numpy(), rk[:, pos], f"dk block {r}")
            grad_close(dkv[r][1][b].cpu().double().numpy(), rv[:, pos], f"dv block {r}")


def test_bwd_gqa_llm_32k_rank0_last_kv_head(gpu_lib):
    # grouped backward at the full 32K share (32 query heads over 8 K/V heads):
    # dq of query heads 28..31 and dk, dv of K/V head 7, which they share, for
    # every block; rank 0's contributions, exact from the oracle's gradients
    w = configs.LLM_32K_CP4_GQA
    G = w.H // w.Hkv
    g = w.Hkv - 1
    heads = list(range(g * G, (g + 1) * G))
    banner(f"backward ring, {w.name} rank 0: query heads {heads[0]}..{heads[-1]} and their K/V head {g}")
    case = RingCase(w, 0)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, scale=w.scale)
    qpos = ringcase_positions(w, 0)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, qpos, w.d, w.dtype, "cuda")
    dq, dkv = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, out, lse, do, scale=w.scale)
    torch.cuda.synchronize()
    allpos = np.arange(w.S)
    ex = lambda tid, h, r: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, 0, h, r, w.d), w.dtype))
    gq = np.stack([ex(seeded.Q, h, qpos) for h in heads])
    gdo = np.stack([ex(DOUT, h, qpos) for h in heads])
    gk, gv = ex(seeded.K, g, allpos)[None], ex(seeded.V, g, allpos)[None]
    rq, rk, rv = oracle.grouped_attention_grads(gq, qpos, gk, gv, allpos, w.scale, True, gdo)
    grad_close(dq[0, heads[0]:heads[-1] + 1].cpu().double().numpy(), rq, f"dq heads {heads[0]}..{heads[-1]}")
    for t in range(w.P):
        kpos = ringcase_positions(w, t)
        grad_close(dkv[t][0][0, g].cpu().double().numpy(), rk[0, kpos], f"dk block {t} kv head {g}")
        grad_close(dkv[t][1][0, g].cpu().double().numpy(), rv[0, kpos], f"dv block {t} kv head {g}")


@pytest.mark.parametrize("G,B,L", [(2, 2, 1000), (4, 1, 777), (8, 1, 513)])
def test_bwd_split_diagonal_step(gpu_lib, G, B, L):
    # the causal diagonal step with its dK/dV half split over the two halves
    # of every K/V head's query heads (two streams, the second half into a
    # partial accumulator that is added in), against the unsplit step and the
    # oracle, with fresh accumulators and with accumulators that already hold
    # other ranks' sums; the dQ launches are the same, so dq is bitwise equal
    Hkv, d, dt = 2, 128, torch.bfloat16
    H = G * Hkv
    banner(f"backward diagonal step split in head halves: B{B} H{H} H_kv{Hkv} L{L}")
    wid = 600 + G
    q = seeded.gen_bhsd(wid, seeded.Q, B, H, 0, L, d, dt, "cuda")
    k = seeded.gen_bhsd(wid, seeded.K, B, Hkv, 0, L, d, dt, "cuda")
    v = seeded.gen_bhsd(wid, seeded.V, B, Hkv, 0, L, d, dt, "cuda")
    do = seeded.gen_bhsd(wid, DOUT, B, H, 0, L, d, dt, "cuda")
    segs = [(0, L)]
    scale = d ** -0.5
    out, lse, _ = ring.run(q, segs, [(k, v)], [segs], 0, True, scale=scale)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wid)
    held = [torch.randn(k.shape, device="cuda", generator=gen) for _ in range(2)]
    res = {}
    for sp in (False, True):
        for acc in (None, [tuple(t.clone() for t in held)]):
            res[sp, acc is None] = ring.run_bwd(q, segs, [(k, v)], [segs], 0, True, out, lse, do, scale=scale,
                                                dkv=acc, split=sp)
    torch.cuda.synchronize()
    for fresh in (True, False):
        (dq0, kv0), (dq1, kv1) = res[False, fresh], res[True, fresh]
        assert torch.equal(dq0, dq1)
        for a, b in zip(kv0[0], kv1[0]):
            assert torch.allclose(b, a, rtol=1e-5, atol=1e-5 * a.abs().max().item()), f"fresh={fresh}"
    dq, kv = res[True, True]
    qc, kc, vc, dc = (seeded.exact_f64(t.cpu()) for t in (q, k, v, do))
    pos = np.arange(L)
    for b in range(B):
        rq, rk, rv = oracle.grouped_attention_grads(qc[b], pos, kc[b], vc[b], pos, scale, True, dc[b])
        grad_close(dq[b].cpu().double().numpy(), rq, f"split dq b{b}")
        grad_close(kv[0][0][b].cpu().double().numpy(), rk, f"split dk b{b}")
        grad_close(kv[0][1][b].cpu().double().numpy(), rv, f"split dv b{b}")
        # with accumulators that held other sums, those sums plus the same gradients
        _, kva = res[True, False]
        grad_close(kva[0][0][b].cpu().double().numpy() - held[0][b].cpu().double().numpy(), rk, f"split dk+held b{b}")
        grad_close(kva[0][1][b].cpu().double().numpy() - held[1][b].cpu().double().numpy(), rv, f"split dv+held b{b}")


def test_bwd_split_at_the_32k_share(gpu_lib):
    # the opt-in split diagonal step at the grouped 32K share (32 query heads
    # over 8 K/V heads, rank 0), with and without the second dK/dV stream:
    # dq is bitwise the unsplit one and dk, dv agree with it up to the order
    # of the fp32 sums (only the diagonal block's accumulators differ at all)
    w = configs.LLM_32K_CP4_GQA
    banner(f"backward ring, {w.name} rank 0: split diagonal step against the unsplit one")
    case = RingCase(w, 0)
    out, lse, _ = ring.run(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, scale=w.scale)
    do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, ringcase_positions(w, 0), w.d, w.dtype, "cuda")
    ref = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, out, lse, do, scale=w.scale)
    for ov in (True, False):
        dq, dkv = ring.run_bwd(case.q, case.q_segs, case.kv, case.kv_segs, 0, True, out, lse, do, scale=w.scale,
                               split=True, overlap=ov)
        torch.cuda.synchronize()
        assert torch.equal(dq, ref[0])
        for t, ((a, b), (c, e)) in enumerate(zip(ref[1], dkv)):
            for x, y in ((a, c), (b, e)):
                if t != 0:
                    assert torch.equal(x, y), f"block {t}"
                else:
                    assert torch.allclose(y, x, rtol=1e-5, atol=1e-5 * x.abs().max().item()), f"overlap={ov}"


# ---- the alternatives to the ring: all-gather and all-to-all on heads ------------------

from context_attention_ra_amd import variants  # noqa: E402


@pytest.mark.parametrize("wname", ["causal-bf16-4k-cp2", "causal-bf16-4k-cp2-gqa4"])
def test_allgather_every_rank(gpu_lib, wname):
    w = configs.RING_WORKLOADS[wname]
    for rank in range(w.P):
        banner(f"all-gather variant, {w.name} rank {rank}")
        case = RingCase(w, rank)
        out, lse = variants.run_allgather(case.q, case.q_segs, case.kv, case.kv_segs, w.causal, scale=w.scale)
        torch.cuda.synchronize()
        ro, rl = case.expected()
        assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, w.dtype,
                     f"all-gather {w.name} r{rank}")


def test_add_rows_is_an_fp32_add(gpu_lib):
    banner("ra_add_rows: strided row accumulate over slices, bitwise against an fp32 add")
    g = torch.Generator(device="cuda").manual_seed(5)
    src = torch.randn((2, 3, 300, 128), generator=g, device="cuda")
    dst = torch.randn((2, 3, 100, 128), generator=g, device="cuda")
    ref = dst.clone()
    ref[:, 1:3, 7:7 + 61] += src[:, 0:2, 200:200 + 61].clone()
    # slices 1..2 of every batch of dst: slices are the flattened leading dims
    for b in range(2):
        _lib.ra_add_rows(src, 200, dst, 7, 61, src_slice0=3 * b, dst_slice0=3 * b + 1, nslices=2)
    torch.cuda.synchronize()
    assert torch.equal(dst, ref)


@pytest.mark.parametrize("wname", ["causal-bf16-4k-cp2", "causal-bf16-4k-cp2-gqa4"])
def test_allgather_backward_reduce_scatter(gpu_lib, wname):
    # backward of the all-gather variant: every rank's dK/dV of the gathered
    # K/V, reduce-scattered to the owning ranks, equals the gradient of
    # full-sequence attention at each rank's positions (the ranks' queries
    # together are the whole sequence)
    w = configs.RING_WORKLOADS[wname]
    banner(f"all-gather backward + reduce-scatter, {w.name}, all ranks")
    cases = [RingCase(w, r) for r in range(w.P)]
    dqs, pk, pv = [], [], []
    for r, case in enumerate(cases):
        out, lse = variants.run_allgather(case.q, case.q_segs, case.kv, case.kv_segs, w.causal, scale=w.scale)
        do = seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, ringcase_positions(w, r), w.d, w.dtype, "cuda")
        dq, dk, dv = variants.allgather_bwd(case.q, case.q_segs, case.kv, case.kv_segs, w.causal, out, lse, do,
                                            scale=w.scale)
        dqs.append(dq)
        pk.append(dk)
        pv.append(dv)
    segs = cases[0].kv_segs
    dks = variants.reduce_scatter(pk, segs)
    dvs = variants.reduce_scatter(pv, segs)
    torch.cuda.synchronize()
    allpos = np.arange(w.S)
    G = w.H // w.Hkv
    for b in range(w.B):
        ex = lambda tid, h: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, b, h, allpos, w.d),
                                                             w.dtype))
        q = np.stack([ex(seeded.Q, h) for h in range(w.H)])
        do = np.stack([ex(DOUT, h) for h in range(w.H)])
        k = np.stack([ex(seeded.K, h) for h in range(w.Hkv)])
        v = np.stack([ex(seeded.V, h) for h in range(w.Hkv)])
        rq, rk, rv = oracle.grouped_attention_grads(q, allpos, k, v, allpos, w.scale, w.causal, do)
        for r in range(w.P):
            pos = ringcase_positions(w, r)
            grad_close(dqs[r][b].cpu().double().numpy(), rq[:, pos], f"dq rank {r} (G={G})")
            grad_close(dks[r][b].cpu().double().numpy(), rk[:, pos], f"dk rank {r} after reduce-scatter")
            grad_close(dvs[r][b].cpu().double().numpy(), rv[:, pos], f"dv rank {r} after reduce-scatter")


@pytest.mark.parametrize("wname", ["causal-bf16-4k-cp2", "causal-bf16-4k-cp2-gqa4"])
def test_head_all_to_all_every_group(gpu_lib, wname):
    w = configs.RING_WORKLOADS[wname]
    cases = [RingCase(w, r) for r in range(w.P)]
    segs = [c.q_segs for c in cases]
    qb = [c.q for c in cases]
    kvb = cases[0].kv  # every rank's K/V block, as each case holds them all
    hg = w.H // w.P
    outs = [torch.empty_like(c.q) for c in cases]
    for g in range(w.P):
        banner(f"all-to-all on heads, {w.name} group {g} (heads {g * hg}..{(g + 1) * hg - 1})")
        out, lse = variants.run_head_group(qb, kvb, segs, g, w.causal, scale=w.scale)
        variants.group_to_ranks(out, g, w.P, segs, outs)
        torch.cuda.synchronize()
        # head group g at every position, against the oracle at positions 0..S-1
        allpos = np.arange(w.S)
        G = w.H // w.Hkv
        for j in range(hg):
            h = g * hg + j
            ex = lambda tid, hh: seeded.exact_f64(seeded.to_dtype(
                seeded.normal_rows_at(w.wid, tid, 0, hh, allpos, w.d), w.dtype))
            ro, rl = oracle.grouped_attention(ex(seeded.Q, h)[None], allpos, ex(seeded.K, h // G)[None],
                                              ex(seeded.V, h // G)[None], allpos, w.scale, w.causal)
            assert_close(out[0, j].float().cpu().double().numpy(), ro[0], lse[0, j].cpu().double().numpy(),
                         rl[0], w.dtype, f"group {g} head {h}")
    # the all-to-all back gives every rank its sequence-split output of all heads
    for r, c in enumerate(cases):
        ro, rl = c.expected()
        mx, mr = compare(outs[r].float().cpu().double().numpy(), ro)
        print(f"rank {r} reassembled: max_abs={mx:.3e} mean_rel={mr:.3e}", flush=True)
        assert mx <= 2e-2 and mr <= 1e-2


def test_variants_llm_32k_sampled(gpu_lib):
    # the configuration the bench times: rank 0 / head group 0 of the 32K causal share
    w = configs.LLM_32K_CP4
    banner(f"all-gather and all-to-all on heads, {w.name}, sampled rows")
    case = RingCase(w, 0)
    out, lse = variants.run_allgather(case.q, case.q_segs, case.kv, case.kv_segs, True, scale=w.scale)
    torch.cuda.synchronize()
    rows = sample_rows(w, 0)
    ro, rl = case.expected(rows)
    idx = torch.as_tensor(rows, device=out.device)
    assert_close(out.index_select(2, idx).float().cpu().double().numpy(), ro,
                 lse.index_select(2, idx).cpu().double().numpy(), rl, w.dtype, "all-gather 32K r0")
    del out, lse
    segs = [case.kv_segs[t] for t in range(w.P)]
    qb = [case.q] + [seeded.gen_bhsd_at(w.wid, seeded.Q, w.B, w.H, ringcase_positions(w, t), w.d, w.dtype, "cuda")
                     for t in range(1, w.P)]
    og, lg = variants.run_head_group(qb, case.kv, segs, 0, True, scale=w.scale)
    torch.cuda.synchronize()
    hg = w.H // w.P
    pos = np.unique(np.concatenate([np.array([0, w.S - 1]), seeded.uniform_sample([77, w.wid], w.S, 128)]))
    allpos = np.arange(w.S)
    gpu_o = og.index_select(2, torch.as_tensor(pos, device=og.device)).float().cpu().double().numpy()
    gpu_l = lg.index_select(2, torch.as_tensor(pos, device=lg.device)).cpu().double().numpy()
    ref_o, ref_l = np.zeros_like(gpu_o), np.zeros_like(gpu_l)
    for j in range(hg):
        ex = lambda tid, r: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, 0, j, r, w.d), w.dtype))
        ref_o[0, j], ref_l[0, j] = oracle.attention_rows(ex(seeded.Q, pos), pos, ex(seeded.K, allpos),
                                                         ex(seeded.V, allpos), allpos, w.scale, True)
    assert_close(gpu_o, ref_o, gpu_l, ref_l, w.dtype, f"head group 0 (heads 0..{hg - 1}), {pos.size} positions")


# ---- seeded random segment tables: tile classification and masks -------------------

def _random_runs(rng, n_rows, max_start):
    """One or two runs of global positions that tile n_rows local rows."""
    if n_rows >= 2 and rng.random() < 0.6:
        n0 = int(rng.integers(1, n_rows))
        s0 = int(rng.integers(0, max_start))
        s1 = int(rng.integers(0, max_start))
        return [(s0, n0), (s1, n_rows - n0)]
    return [(int(rng.integers(0, max_start)), n_rows)]


def _random_case(seed):
    rng = np.random.default_rng([4242, seed])
    d = int(rng.choice([64, 128]))
    H_kv = int(rng.choice([1, 2]))
    H = H_kv * int(rng.choice([1, 2, 3]))
    B = int(rng.choice([1, 2]))
    Lq = int(rng.integers(1, 700))
    Lk = int(rng.integers(1, 700))
    causal = bool(rng.random() < 0.7)
    return B, H, H_kv, Lq, _random_runs(rng, Lq, 1500), Lk, _random_runs(rng, Lk, 1500), d, causal


@pytest.mark.parametrize("seed", range(12))
def test_random_segments_forward_and_backward(gpu_lib, seed):
    B, H, Hkv, Lq, qr, Lk, kr, d, causal = _random_case(seed)
    banner(f"random case {seed}: B{B} H{H} H_kv{Hkv} Lq{Lq} {qr} Lk{Lk} {kr} d{d} causal={causal}")
    dt = torch.bfloat16
    q = seeded.gen_bhsd(500 + seed, 0, B, H, 0, Lq, d, dt, "cuda")
    k = seeded.gen_bhsd(500 + seed, 1, B, Hkv, 0, Lk, d, dt, "cuda")
    v = seeded.gen_bhsd(500 + seed, 2, B, Hkv, 0, Lk, d, dt, "cuda")
    do = seeded.gen_bhsd(500 + seed, DOUT, B, H, 0, Lq, d, dt, "cuda")
    scale = d ** -0.5
    st = ring.RingState(B, H, Lq, d, "cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    _lib.ra_step_final(q, k, v, qr, kr, causal, scale, st.o, st.m, st.l, out, lse, init=True)
    delta = torch.empty_like(lse)
    _lib.ra_bwd_prep(out, do, delta)
    dq = torch.empty((B, H, Lq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((B, Hkv, Lk, d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    _lib.ra_step_bwd(q, k, v, do, lse, delta, qr, kr, causal, scale, dq, dk, dv, init_dq=True, init_dkv=True)
    torch.cuda.synchronize()
    qp, kp = _runs_pos(qr), _runs_pos(kr)
    qc, kc, vc, dc = (seeded.exact_f64(t.cpu()) for t in (q, k, v, do))
    ro, rl = np.zeros((B, H, Lq, d)), np.zeros((B, H, Lq))
    rq, rk, rv = np.zeros((B, H, Lq, d)), np.zeros((B, Hkv, Lk, d)), np.zeros((B, Hkv, Lk, d))
    for b in range(B):
        ro[b], rl[b] = oracle.grouped_attention(qc[b], qp, kc[b], vc[b], kp, scale, causal)
        rq[b], rk[b], rv[b] = oracle.grouped_attention_grads(qc[b], qp, kc[b], vc[b], kp, scale, causal, dc[b])
    go, gl = out.float().cpu().double().numpy(), lse.cpu().double().numpy()
    empty = ~np.isfinite(rl)
    assert np.array_equal(empty, ~np.isfinite(gl)), "rows without visible keys must give lse = -inf"
    assert np.all(go[empty] == 0.0)
    assert_close(go, ro, np.where(empty, 0.0, gl), np.where(empty, 0.0, rl), dt, f"random {seed} forward")
    for g, r, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        assert torch.isfinite(g).all(), n
        if np.abs(r).max() == 0.0:  # nothing visible at all: the gradient is exactly zero
            assert torch.all(g == 0), n
        else:
            grad_close(g.cpu().double().numpy(), r, f"random {seed} {n}")


# ---- the ring as a differentiable PyTorch operation ----------------------------------

def test_autograd_ring_attention_both_ranks(gpu_lib):
    from context_attention_ra_amd.autograd import ring_attention
    w = configs.CAUSAL_2RANK
    banner(f"autograd ring attention, {w.name}, both ranks through one loss")
    cases = [RingCase(w, r) for r in range(w.P)]
    kv = [(k.clone().requires_grad_(True), v.clone().requires_grad_(True)) for k, v in cases[0].kv]
    qs = [c.q.clone().requires_grad_(True) for c in cases]
    dos = [seeded.gen_bhsd_at(w.wid, DOUT, w.B, w.H, ringcase_positions(w, r), w.d, w.dtype, "cuda")
           for r in range(w.P)]
    loss = 0.0
    for r, c in enumerate(cases):
        out = ring_attention(qs[r], c.q_segs, kv, c.kv_segs, r, w.causal, scale=w.scale)
        loss = loss + (out.float() * dos[r].float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    allpos = np.arange(w.S)
    for h in range(w.H):
        ex = lambda tid: seeded.exact_f64(seeded.to_dtype(seeded.normal_rows_at(w.wid, tid, 0, h, allpos, w.d),
                                                          w.dtype))
        rq, rk, rv = oracle.attention_grads(ex(seeded.Q), allpos, ex(seeded.K), ex(seeded.V), allpos, w.scale,
                                            w.causal, ex(DOUT))
        for r in range(w.P):
            pos = ringcase_positions(w, r)
            grad_close(qs[r].grad[0, h].float().cpu().double().numpy(), rq[pos], f"q.grad rank {r} h{h}")
            grad_close(kv[r][0].grad[0, h].float().cpu().double().numpy(), rk[pos], f"k.grad block {r} h{h}")
            grad_close(kv[r][1].grad[0, h].float().cpu().double().numpy(), rv[pos], f"v.grad block {r} h{h}")


@pytest.mark.parametrize("split,P,causal,dtype", [("zigzag", 2, True, torch.bfloat16),
                                                  ("zigzag", 4, True, torch.bfloat16),
                                                  ("contiguous", 3, False, torch.bfloat16),
                                                  ("contiguous", 4, True, torch.float32),
                                                  ("temporal", 4, False, torch.bfloat16)])
def test_context_parallel_attention_whole_sequence(gpu_lib, split, P, causal, dtype):
    from context_attention_ra_amd.cp import context_parallel_attention
    B, H, H_kv, d = 1, 4, 2, 64
    S_sp = 96 if split == "temporal" else 0
    S = 8 * 96 if split == "temporal" else (768 if P == 3 else 1024)
    banner(f"context-parallel attention of a whole sequence: {split} P={P} causal={causal} {dtype} S={S}")
    q = seeded.gen_bhsd(600, 0, B, H, 0, S, d, dtype, "cuda")
    k = seeded.gen_bhsd(600, 1, B, H_kv, 0, S, d, dtype, "cuda")
    v = seeded.gen_bhsd(600, 2, B, H_kv, 0, S, d, dtype, "cuda")
    out, lse = context_parallel_attention(q, k, v, P, split=split, causal=causal, S_sp=S_sp)
    torch.cuda.synchronize()
    pos = np.arange(S)
    qc, kc, vc = (seeded.exact_f64(t.cpu()) for t in (q, k, v))
    ro, rl = oracle.grouped_attention(qc[0], pos, kc[0], vc[0], pos, d ** -0.5, causal)
    assert_close(out[0].float().cpu().double().numpy(), ro, lse[0].cpu().double().numpy(), rl, dtype,
                 f"whole sequence {split} P={P}")


def test_cp_attention_gradients_whole_sequence(gpu_lib):
    from context_attention_ra_amd.cp import cp_attention
    B, H, H_kv, d, S, P = 1, 4, 2, 64, 1024, 2
    banner(f"differentiable whole-sequence attention: zigzag P={P}, H={H}, H_kv={H_kv}, S={S}")
    dt = torch.bfloat16
    q, k, v = (seeded.gen_bhsd(610, t, B, hh, 0, S, d, dt, "cuda").requires_grad_(True)
               for t, hh in ((0, H), (1, H_kv), (2, H_kv)))
    do = seeded.gen_bhsd(610, DOUT, B, H, 0, S, d, dt, "cuda")
    out = cp_attention(q, k, v, P, split="zigzag", causal=True)
    (out.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    pos = np.arange(S)
    qc, kc, vc, dc = (seeded.exact_f64(t.detach().cpu()) for t in (q, k, v, do))
    ro, _ = oracle.grouped_attention(qc[0], pos, kc[0], vc[0], pos, d ** -0.5, True)
    rq, rk, rv = oracle.grouped_attention_grads(qc[0], pos, kc[0], vc[0], pos, d ** -0.5, True, dc[0])
    mx, mr = compare(out[0].detach().float().cpu().double().numpy(), ro)
    assert mx <= 2e-2 and mr <= 1e-2, (mx, mr)
    for t, r, n in ((q, rq, "q"), (k, rk, "k"), (v, rv, "v")):
        grad_close(t.grad[0].float().cpu().double().numpy(), r, f"whole-sequence {n}.grad")

"""Pins for the CPU oracle: brute force, closed forms, invariants, a library routine.

None of these re-types the oracle's formula: brute force uses pure-Python loops
with math.exp / math.fsum, closed forms come from the mathematics, and the
library cross-check is PyTorch's scaled dot-product attention in float64 on the
CPU (the routine the Ultralytics glossary's example calls).
"""

import math

import numpy as np
import pytest
import torch

from oracle import (attention_grads, attention_kv_grads_rows, attention_rows, factored_spatial,
                    factored_temporal, grouped_attention, grouped_attention_grads, merge_lse)


def brute_attention(q, q_pos, k, v, k_pos, scale, causal):
    """Pure-Python softmax attention (no numpy arithmetic)."""
    n, d = len(q), len(q[0])
    out, lses = [], []
    for i in range(n):
        vis = [j for j in range(len(k)) if (not causal) or k_pos[j] <= q_pos[i]]
        if not vis:
            out.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in vis}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in vis}
        z = math.fsum(w.values())
        out.append([math.fsum(w[j] * v[j][c] for j in vis) / z for c in range(len(v[0]))])
        lses.append(mx + math.log(z))
    return out, lses


def rnd(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed, causal):
    rng = np.random.default_rng(100 + seed)
    n, S, d = rng.integers(1, 6), rng.integers(1, 9), rng.integers(1, 5)
    q, k, v = rnd(seed, n, d, scale=2.0), rnd(seed + 50, S, d, scale=2.0), rnd(seed + 99, S, d)
    q_pos = rng.integers(0, S, size=n)
    k_pos = rng.permutation(S)
    scale = float(rng.uniform(0.1, 1.5))
    o, lse = attention_rows(q, q_pos, k, v, k_pos, scale, causal)
    bo, blse = brute_attention(q.tolist(), q_pos.tolist(), k.tolist(), v.tolist(),
                               k_pos.tolist(), scale, causal)
    np.testing.assert_allclose(o, np.array(bo), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(blse), rtol=1e-12, atol=1e-12)


def test_brute_force_adversarial_scores():
    # huge score gaps: exp without the max shift would overflow
    q = np.array([[300.0, -200.0], [-1e3, 1e3]])
    k = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    v = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    pos = np.arange(3)
    o, lse = attention_rows(q, [2, 2], k, v, pos, 1.0, False)
    bo, blse = brute_attention(q.tolist(), [2, 2], k.tolist(), v.tolist(), pos.tolist(), 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(o, bo, rtol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    S, d = 11, 3
    k, v = rnd(1, S, d), rnd(2, S, d)
    q = np.zeros((S, d))
    pos = np.arange(S)
    o, lse = attention_rows(q, pos, k, v, pos, 0.7, True)
    for i in range(S):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert lse[i] == pytest.approx(math.log(i + 1), rel=1e-13)


def test_single_visible_key():
    # causal global row 0 sees only key 0: o = v_0, lse = s_00
    k, v, q = rnd(3, 5, 4), rnd(4, 5, 4), rnd(5, 1, 4)
    o, lse = attention_rows(q, [0], k, v, np.arange(5), 0.5, True)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-14)
    assert lse[0] == pytest.approx(0.5 * float(q[0] @ k[0]), rel=1e-13)


def test_identical_keys_give_uniform_weights():
    k = np.tile(rnd(6, 1, 4), (7, 1))
    v, q = rnd(7, 7, 4), rnd(8, 3, 4)
    o, _ = attention_rows(q, np.zeros(3, int), k, v, np.arange(7), 0.3, False)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (3, 1)), rtol=1e-12)


def test_constant_values():
    k, q = rnd(9, 13, 4), rnd(10, 5, 4)
    c = np.array([1.5, -2.0, 0.25, 7.0])
    o, _ = attention_rows(q, np.arange(5) + 8, k, np.tile(c, (13, 1)), np.arange(13), 1.0, True)
    np.testing.assert_allclose(o, np.tile(c, (5, 1)), rtol=1e-13)


def test_two_keys_sigmoid():
    q, k, v = rnd(11, 1, 3), rnd(12, 2, 3), rnd(13, 2, 3)
    scale = 0.8
    o, lse = attention_rows(q, [5], k, v, [0, 1], scale, True)
    s1, s2 = scale * float(q[0] @ k[0]), scale * float(q[0] @ k[1])
    sig = 1.0 / (1.0 + math.exp(-(s1 - s2)))
    np.testing.assert_allclose(o[0], sig * v[0] + (1 - sig) * v[1], rtol=1e-12)
    assert lse[0] == pytest.approx(max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))), rel=1e-13)


def test_dominant_score_selects_its_value():
    k = np.eye(4)
    v = rnd(14, 4, 2)
    q = np.array([[0.0, 0.0, 60.0, 0.0]])
    o, _ = attention_rows(q, [0], k, v, np.arange(4), 1.0, False)
    np.testing.assert_allclose(o[0], v[2], rtol=0, atol=1e-20)


def test_no_visible_key_row():
    o, lse = attention_rows(rnd(15, 1, 2), [0], rnd(16, 3, 2), rnd(17, 3, 2), [1, 2, 3], 1.0, True)
    assert np.all(o == 0.0) and lse[0] == -np.inf


def test_key_shift_invariance():
    q, k, v = rnd(18, 6, 5), rnd(19, 9, 5), rnd(20, 9, 5)
    u = rnd(21, 5)
    scale = 0.37
    pos = np.arange(9)
    o1, l1 = attention_rows(q, pos[3:], k, v, pos, scale, True)
    o2, l2 = attention_rows(q, pos[3:], k + u[None, :], v, pos, scale, True)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, scale * (q @ u), rtol=1e-10, atol=1e-12)


def test_joint_permutation_invariance_unmasked():
    q, k, v = rnd(22, 4, 3), rnd(23, 10, 3), rnd(24, 10, 3)
    perm = np.random.default_rng(25).permutation(10)
    pos = np.arange(10)
    o1, l1 = attention_rows(q, pos[:4], k, v, pos, 1.1, False)
    o2, l2 = attention_rows(q, pos[:4], k[perm], v[perm], pos[perm], 1.1, False)
    np.testing.assert_allclose(o1, o2, rtol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    # causal: permuting rows together with their positions changes nothing either
    o3, l3 = attention_rows(q, pos[5:9], k, v, pos, 1.1, True)
    o4, l4 = attention_rows(q, pos[5:9], k[perm], v[perm], pos[perm], 1.1, True)
    np.testing.assert_allclose(o3, o4, rtol=1e-12)
    np.testing.assert_allclose(l3, l4, rtol=1e-13)


def test_value_affine_map():
    q, k, v = rnd(26, 4, 3), rnd(27, 8, 3), rnd(28, 8, 3)
    pos = np.arange(8)
    o1, _ = attention_rows(q, pos[4:], k, v, pos, 0.9, True)
    o2, _ = attention_rows(q, pos[4:], k, 2.5 * v - 1.25, pos, 0.9, True)
    np.testing.assert_allclose(o2, 2.5 * o1 - 1.25, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    L, d = 96, 16
    q, k, v = rnd(29, L, d), rnd(30, L, d), rnd(31, L, d)
    pos = np.arange(L)
    o, _ = attention_rows(q, pos, k, v, pos, 1.0 / math.sqrt(d), causal)
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-11, atol=1e-12)


# ---- backward -----------------------------------------------------------------

def _loss(q, qp, k, v, kp, scale, causal, do):
    o, _ = attention_rows(q, qp, k, v, kp, scale, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_grads_match_central_differences(causal):
    # the derivative of the forward definition, taken numerically: no formula shared
    n, S, d = 4, 6, 3
    q, k, v, do = rnd(60, n, d), rnd(61, S, d), rnd(62, S, d), rnd(63, n, d)
    qp, kp = np.array([1, 3, 4, 5]), np.random.default_rng(64).permutation(S)
    scale = 0.8
    dq, dk, dv = attention_grads(q, qp, k, v, kp, scale, causal, do)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            lp = _loss(**{**args, name: xp}, qp=qp, kp=kp, scale=scale, causal=causal, do=do)
            lm = _loss(**{**args, name: xm}, qp=qp, kp=kp, scale=scale, causal=causal, do=do)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_grads_match_torch_autograd_float64(causal):
    # library routine: autograd through PyTorch's scaled dot-product attention
    L, d = 48, 16
    q, k, v, do = rnd(65, L, d), rnd(66, L, d), rnd(67, L, d), rnd(68, L, d)
    pos = np.arange(L)
    dq, dk, dv = attention_grads(q, pos, k, v, pos, 1.0 / math.sqrt(d), causal, do)
    tq, tk, tv = (torch.from_numpy(a)[None, None].requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.from_numpy(do)[None, None])
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, ref.grad[0, 0].numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_grads_of_selected_rows(causal):
    # the selected-rows form against numerical derivatives of the forward
    # definition (for the chosen key rows) and against PyTorch autograd
    n, S, d = 5, 9, 3
    q, k, v, do = rnd(70, n, d), rnd(71, S, d), rnd(72, S, d), rnd(73, n, d)
    qp, kp = np.array([0, 2, 5, 7, 8]), np.random.default_rng(74).permutation(S)
    rows = np.array([7, 0, 4])
    scale = 0.7
    dk, dv = attention_kv_grads_rows(q, qp, k, v, kp, scale, causal, do, rows)
    eps = 1e-6
    for name, x, g in (("k", k, dk), ("v", v, dv)):
        num = np.zeros((rows.size, d))
        for a, r in enumerate(rows):
            for c in range(d):
                xp, xm = x.copy(), x.copy()
                xp[r, c] += eps
                xm[r, c] -= eps
                args = {"k": k, "v": v}
                lp = _loss(q=q, **{**args, name: xp}, qp=qp, kp=kp, scale=scale, causal=causal, do=do)
                lm = _loss(q=q, **{**args, name: xm}, qp=qp, kp=kp, scale=scale, causal=causal, do=do)
                num[a, c] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)
    L = 40
    q, k, v, do = rnd(75, L, 8), rnd(76, L, 8), rnd(77, L, 8), rnd(78, L, 8)
    pos = np.arange(L)
    rows = np.array([0, 13, 39, 21])
    dk, dv = attention_kv_grads_rows(q, pos, k, v, pos, 8 ** -0.5, causal, do, rows)
    tq, tk, tv = (torch.from_numpy(a)[None, None].requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.from_numpy(do)[None, None])
    np.testing.assert_allclose(dk, tk.grad[0, 0].numpy()[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad[0, 0].numpy()[rows], rtol=1e-10, atol=1e-12)


def test_grads_invariants():
    n, S, d = 7, 20, 4
    q, k, v, do = rnd(69, n, d), rnd(70, S, d), rnd(71, S, d), rnd(72, n, d)
    qp, kp = np.array([0, 4, 9, 11, 15, 18, 19]), np.arange(S)
    dq, dk, dv = attention_grads(q, qp, k, v, kp, 0.6, True, do)
    # linear in the upstream gradient
    dq2, dk2, dv2 = attention_grads(q, qp, k, v, kp, 0.6, True, -2.5 * do)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_allclose(b, -2.5 * a, rtol=1e-12, atol=1e-13)
    # keys after the last query are never visible, so they receive no gradient
    assert np.all(dk[kp > qp.max()] == 0) and np.all(dv[kp > qp.max()] == 0)
    # adding one vector to every key shifts each row's scores by a constant, so
    # the weights and dq do not change
    u = rnd(73, d)
    dq3, _, _ = attention_grads(q, qp, k + u, v, kp, 0.6, True, do)
    np.testing.assert_allclose(dq3, dq, rtol=1e-9, atol=1e-11)
    # unmasked: every row of ds sums to zero (softmax Jacobian), so sum_j dk_j = 0
    _, dk4, _ = attention_grads(q, qp, k, v, kp, 0.6, False, do)
    np.testing.assert_allclose(dk4.sum(axis=0), np.zeros(d), atol=1e-12)


# ---- grouped K/V heads ---------------------------------------------------------

def test_grouped_constant_values_name_the_shared_head():
    # closed form: if every value row of K/V head g equals g, each output row of
    # query head h equals the index of the K/V head it reads, floor(h / G)
    H, H_kv, n, S, d = 12, 3, 5, 9, 4
    q, k = rnd(40, H, n, d, scale=2.0), rnd(41, H_kv, S, d, scale=2.0)
    v = np.broadcast_to(np.arange(H_kv, dtype=np.float64)[:, None, None], (H_kv, S, 3)).copy()
    pos = np.arange(S)
    for causal in (False, True):
        o, _ = grouped_attention(q, pos[-n:], k, v, pos, 0.7, causal)
        for h in range(H):
            np.testing.assert_allclose(o[h], np.full((n, 3), float(h * H_kv // H)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(8, 2), (6, 3), (4, 1), (5, 5)])
def test_grouped_matches_torch_sdpa_gqa_float64(causal, H, H_kv):
    # library routine: PyTorch's scaled dot-product attention with enable_gqa,
    # which shares each K/V head among consecutive query heads
    L, d = 40, 8
    q, k, v = rnd(42, H, L, d), rnd(43, H_kv, L, d), rnd(44, H_kv, L, d)
    pos = np.arange(L)
    o, _ = grouped_attention(q, pos, k, v, pos, 1.0 / math.sqrt(d), causal)
    t = lambda a: torch.from_numpy(a)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal,
                                                           enable_gqa=True)
    np.testing.assert_allclose(o, ref[0].numpy(), rtol=1e-11, atol=1e-12)


def test_grouped_with_one_group_per_head_is_per_head_attention():
    H, n, S, d = 3, 6, 11, 5
    q, k, v = rnd(45, H, n, d), rnd(46, H, S, d), rnd(47, H, S, d)
    qp, kp = np.arange(5, 5 + n), np.arange(S)
    o, lse = grouped_attention(q, qp, k, v, kp, 0.4, True)
    for h in range(H):
        bo, bl = brute_attention(q[h].tolist(), qp.tolist(), k[h].tolist(), v[h].tolist(),
                                 kp.tolist(), 0.4, True)
        np.testing.assert_allclose(o[h], bo, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[h], bl, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_grads_match_torch_autograd_gqa_float64(causal):
    # library routine: autograd through SDPA with enable_gqa (shared K/V heads)
    H, H_kv, L, d = 6, 2, 24, 8
    q, k, v, do = rnd(74, H, L, d), rnd(75, H_kv, L, d), rnd(76, H_kv, L, d), rnd(77, H, L, d)
    pos = np.arange(L)
    dq, dk, dv = grouped_attention_grads(q, pos, k, v, pos, 1.0 / math.sqrt(d), causal, do)
    tq, tk, tv = (torch.from_numpy(a)[None].requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, enable_gqa=True)
    out.backward(torch.from_numpy(do)[None])
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, ref.grad[0].numpy(), rtol=1e-10, atol=1e-12)


def test_grouped_rejects_heads_that_do_not_divide():
    with pytest.raises(ValueError):
        grouped_attention(rnd(48, 6, 2, 3), [0, 1], rnd(49, 4, 2, 3), rnd(50, 4, 2, 3), [0, 1], 1.0, False)


def test_merge_identity_union_of_disjoint_key_sets():
    q, k, v = rnd(32, 7, 4), rnd(33, 20, 4), rnd(34, 20, 4)
    pos = np.arange(20)
    qp = np.array([0, 3, 7, 10, 13, 18, 19])
    a = np.random.default_rng(35).permutation(20)[:9]
    b = np.setdiff1d(pos, a)
    for causal in (False, True):
        of, lf = attention_rows(q, qp, k, v, pos, 0.6, causal)
        oa, la = attention_rows(q, qp, k[a], v[a], pos[a], 0.6, causal)
        ob, lb = attention_rows(q, qp, k[b], v[b], pos[b], 0.6, causal)
        om, lm = merge_lse(oa, la, ob, lb)
        np.testing.assert_allclose(om, of, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(lm, lf, rtol=1e-12, atol=1e-13)


def test_merge_empty_sides():
    o = rnd(36, 3, 2)
    lse = np.array([0.5, -1.0, 2.0])
    ninf = np.full(3, -np.inf)
    z = np.zeros((3, 2))
    om, lm = merge_lse(o, lse, z, ninf)
    np.testing.assert_allclose(om, o, rtol=1e-15)
    np.testing.assert_allclose(lm, lse, rtol=1e-15)
    om, lm = merge_lse(z, ninf, o, lse)
    np.testing.assert_allclose(om, o, rtol=1e-15)
    om, lm = merge_lse(z, ninf, z, ninf)
    assert np.all(om == 0) and np.all(lm == -np.inf)


def test_merge_equal_halves():
    # two identical partials: same output, lse + ln 2
    o, lse = rnd(37, 4, 3), rnd(38, 4)
    om, lm = merge_lse(o, lse, o, lse)
    np.testing.assert_allclose(om, o, rtol=1e-14)
    np.testing.assert_allclose(lm, lse + math.log(2.0), rtol=1e-14)


def _brute_factored(q, k, v, T, S, scale, kind):
    q, k, v = q.tolist(), k.tolist(), v.tolist()
    out, lses = [None] * (T * S), [None] * (T * S)
    for t in range(T):
        for s in range(S):
            i = t * S + s
            keys = [t * S + s2 for s2 in range(S)] if kind == "spatial" else [t2 * S + s for t2 in range(T)]
            o, l = brute_attention([q[i]], [0], [k[j] for j in keys], [v[j] for j in keys],
                                   [0] * len(keys), scale, False)
            out[i], lses[i] = o[0], l[0]
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("kind", ["spatial", "temporal"])
def test_factored_brute_force(kind):
    T, S, d = 3, 4, 2
    q, k, v = rnd(40, T * S, d), rnd(41, T * S, d), rnd(42, T * S, d)
    fn = factored_spatial if kind == "spatial" else factored_temporal
    o, lse = fn(q, k, v, T, S, 0.75)
    bo, bl = _brute_factored(q, k, v, T, S, 0.75, kind)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12)


def test_factored_degenerate_shapes_reduce_to_full_attention():
    d = 5
    q, k, v = rnd(43, 6, d), rnd(44, 6, d), rnd(45, 6, d)
    pos = np.arange(6)
    full_o, full_l = attention_rows(q, pos, k, v, pos, 0.4, False)
    o, l = factored_spatial(q, k, v, 1, 6, 0.4)   # one frame: spatial = full
    np.testing.assert_allclose(o, full_o, rtol=1e-12)
    np.testing.assert_allclose(l, full_l, rtol=1e-12)
    o, l = factored_temporal(q, k, v, 6, 1, 0.4)  # one position: temporal = full
    np.testing.assert_allclose(o, full_o, rtol=1e-12)
    np.testing.assert_allclose(l, full_l, rtol=1e-12)
    # one position per frame: spatial attention of a token sees only itself
    o, l = factored_spatial(q, k, v, 6, 1, 0.4)
    np.testing.assert_allclose(o, v, rtol=1e-14)


def test_temporal_ignores_other_positions():
    T, S, d = 4, 5, 3
    q, k, v = rnd(46, T * S, d), rnd(47, T * S, d), rnd(48, T * S, d)
    o1, _ = factored_temporal(q, k, v, T, S, 0.5)
    k2, v2 = k.copy(), v.copy()
    other = [t * S + s for t in range(T) for s in range(S) if s != 2]
    k2[other] += 3.0
    v2[other] -= 1.0
    o2, _ = factored_temporal(q, k2, v2, T, S, 0.5)
    idx = [t * S + 2 for t in range(T)]
    np.testing.assert_allclose(o1[idx], o2[idx], rtol=1e-14)

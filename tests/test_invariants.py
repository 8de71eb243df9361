"""The pages' invariants, checked on a CPU emulation of the ring against the oracle.

The emulation below is a test-only fp64 online softmax (running max, running
sum, rescaled accumulator) fed one K/V block per ring step. It is not the
oracle and not the GPU path; it checks the pages' claims about the method:
* Day 83 post, "Context parallelism: splitting the sequence": after P steps the
  running online-softmax state holds the correct output for the local queries;
* Ultralytics glossary, "How Context Parallelism Works": equal to full-sequence
  attention up to rounding;
* k8ai ring figure: the block order is (r - s) mod P, and any order gives the
  same result since the final state does not depend on it;
* k8ai, causal balance: all ranks of the zigzag split together reproduce
  global causal attention.
"""

import numpy as np
import pytest

import oracle
from oracle import attention_rows, merge_lse


def online_softmax_ring(q, q_pos, blocks, scale, causal):
    n, d = q.shape
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, d))
    for k, v, k_pos in blocks:
        s = scale * (q @ k.T)
        if causal:
            s = np.where(k_pos[None, :] <= q_pos[:, None], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - ref)
        p = np.exp(s - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v
        m = m_new
    o = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def make(S, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((S, d)), rng.standard_normal((S, d)), rng.standard_normal((S, d))


@pytest.mark.parametrize("split,causal", [("contiguous", False), ("zigzag", True), ("zigzag", False)])
def test_ring_equals_full_attention(split, causal):
    S, P, d = 64, 4, 8
    q, k, v = make(S, d, 1)
    posfn = oracle.zigzag_positions if split == "zigzag" else oracle.contiguous_positions
    for r in range(P):
        qp = posfn(S, P, r)
        blocks = []
        for s in range(P):
            t = oracle.ring_source(r, s, P)
            kp = posfn(S, P, t)
            blocks.append((k[kp], v[kp], kp))
        o, lse = online_softmax_ring(q[qp], qp, blocks, 0.35, causal)
        of, lf = attention_rows(q[qp], qp, k, v, np.arange(S), 0.35, causal)
        np.testing.assert_allclose(o, of, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, lf, rtol=1e-12, atol=1e-12)


def test_block_order_does_not_matter():
    S, P, d = 48, 3, 5
    q, k, v = make(S, d, 2)
    r = 1
    qp = oracle.zigzag_positions(S, P, r)
    orders = [[oracle.ring_source(r, s, P) for s in range(P)], [2, 1, 0], [0, 2, 1]]
    outs = []
    for order in orders:
        blocks = [(k[oracle.zigzag_positions(S, P, t)], v[oracle.zigzag_positions(S, P, t)],
                   oracle.zigzag_positions(S, P, t)) for t in order]
        outs.append(online_softmax_ring(q[qp], qp, blocks, 0.5, True))
    for o, lse in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, outs[0][1], rtol=1e-12, atol=1e-13)


def test_zigzag_ranks_reproduce_global_causal_attention():
    S, P, d = 96, 3, 6
    q, k, v = make(S, d, 3)
    out = np.zeros((S, d))
    for r in range(P):
        qp = oracle.zigzag_positions(S, P, r)
        blocks = [(k[oracle.zigzag_positions(S, P, t)], v[oracle.zigzag_positions(S, P, t)],
                   oracle.zigzag_positions(S, P, t)) for t in range(P)]
        o, _ = online_softmax_ring(q[qp], qp, blocks, 0.4, True)
        out[qp] = o
    pos = np.arange(S)
    full, _ = attention_rows(q, pos, k, v, pos, 0.4, True)
    np.testing.assert_allclose(out, full, rtol=1e-11, atol=1e-12)


def test_running_state_equals_merge_of_per_step_partials():
    S, P, d = 64, 4, 4
    q, k, v = make(S, d, 4)
    r = 2
    qp = oracle.zigzag_positions(S, P, r)
    o_run, l_run = None, None
    for s in range(P):
        t = oracle.ring_source(r, s, P)
        kp = oracle.zigzag_positions(S, P, t)
        o_s, l_s = attention_rows(q[qp], qp, k[kp], v[kp], kp, 0.3, True)
        if o_run is None:
            o_run, l_run = o_s, l_s
        else:
            o_run, l_run = merge_lse(o_run, l_run, o_s, l_s)
    blocks = [(k[oracle.zigzag_positions(S, P, t)], v[oracle.zigzag_positions(S, P, t)],
               oracle.zigzag_positions(S, P, t)) for t in range(P)]
    o, lse = online_softmax_ring(q[qp], qp, blocks, 0.3, True)
    np.testing.assert_allclose(o_run, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l_run, lse, rtol=1e-12, atol=1e-12)


def test_dropping_a_block_is_detected():
    # a lost ring step must change the result (the check has teeth)
    S, P, d = 32, 4, 4
    q, k, v = make(S, d, 5)
    qp = oracle.contiguous_positions(S, P, 0)
    blocks = [(k[oracle.contiguous_positions(S, P, t)], v[oracle.contiguous_positions(S, P, t)],
               oracle.contiguous_positions(S, P, t)) for t in range(P)]
    o, _ = online_softmax_ring(q[qp], qp, blocks[:-1], 0.5, False)
    of, _ = attention_rows(q[qp], qp, k, v, np.arange(S), 0.5, False)
    assert np.abs(o - of).max() > 1e-3

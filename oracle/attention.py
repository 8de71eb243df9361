"""Plain fp64 softmax attention: the result the ring reaches (test infrastructure).

The ring of the pages ends with every device holding "the correct output for its
local Q tokens", and the Ultralytics glossary ("How Context Parallelism Works")
states that the result equals full-sequence attention up to ordinary rounding.
Neither page writes the formula out; the Ultralytics example ("Practical Use and
Tradeoffs") names it as PyTorch's scaled dot-product attention with
``is_causal=True``. So this module is that textbook definition, computed
directly over the whole global key set. It never sees blocks, ring steps, chunk
assignments or running state.

For a query row i at global position g(i), with visible key set V(i):
    s_ij  = scale * <q_i, k_j>
    M_i   = max_{j in V(i)} s_ij
    o_i   = sum_j exp(s_ij - M_i) v_j / sum_j exp(s_ij - M_i)
    lse_i = M_i + ln sum_j exp(s_ij - M_i)
V(i) is every key for the unmasked case and {j : g(j) <= g(i)} for the causal
case (the diagonal is visible). A row with no visible key has o_i = 0 and
lse_i = -inf.

Only tests/, the smoke check and the CPU-baseline leg of the benchmark use this.
"""

import numpy as np

_NEG_INF = -np.inf


def attention_rows(q, q_pos, k, v, k_pos, scale, causal, row_chunk=256):
    """Softmax attention of query rows against a global key/value set.

    Definition: Day 83 post, "Context parallelism: splitting the sequence"
    (the ring's end state is full attention for the local queries); Ultralytics
    glossary, "How Context Parallelism Works" (equivalence with full-sequence
    attention) and "Practical Use and Tradeoffs" (scaled dot-product attention,
    causal).

    q      (n, d)  query rows; upcast to fp64 from the exact values given
    q_pos  (n,)    global token position of each query row
    k, v   (S, d)  keys and values of the global sequence
    k_pos  (S,)    global position of each key row
    scale  float   multiplier on the dot products
    causal bool    if True, key j is visible to query i iff k_pos[j] <= q_pos[i]
    returns (o (n, d) fp64, lse (n,) fp64, natural log)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    n, d = q.shape
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), _NEG_INF, dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        s = float(scale) * (q[r0:r1] @ k.T)
        if causal:
            visible = k_pos[None, :] <= q_pos[r0:r1, None]
            s = np.where(visible, s, _NEG_INF)
        row_max = s.max(axis=1)
        has_key = np.isfinite(row_max)
        shift = np.where(has_key, row_max, 0.0)
        w = np.exp(s - shift[:, None])  # exp(-inf) = 0 for masked keys
        denom = w.sum(axis=1)
        num = w @ v
        safe = np.where(has_key, denom, 1.0)
        o[r0:r1] = np.where(has_key[:, None], num / safe[:, None], 0.0)
        lse[r0:r1] = np.where(has_key, shift + np.log(safe), _NEG_INF)
    return o, lse


def attention_grads(q, q_pos, k, v, k_pos, scale, causal, do):
    """Gradients of softmax attention with respect to its queries, keys and values.

    The ring exchanges of the k8ai page ("Communication profile") happen in the
    backward pass as well as the forward one, and the Ultralytics example
    ("Practical Use and Tradeoffs") trains through the attention. The backward
    pass computes the derivative of the same definition as ``attention_rows``;
    for an upstream gradient do_i of each output row o_i (loss L with
    dL/do_i = do_i):
        P_ij  = exp(s_ij - lse_i) for visible j, 0 otherwise
        dv_j  = sum_i P_ij do_i
        dP_ij = <do_i, v_j>
        ds_ij = P_ij (dP_ij - <do_i, o_i>)      (the softmax Jacobian)
        dq_i  = scale * sum_j ds_ij k_j
        dk_j  = scale * sum_i ds_ij q_i
    Rows with no visible key contribute nothing.

    q, do (n, d); k, v (S, d); other arguments as ``attention_rows``.
    returns (dq (n, d), dk (S, d), dv (S, d)) in fp64
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    o, lse = attention_rows(q, q_pos, k, v, k_pos, scale, causal)
    s = float(scale) * (q @ k.T)
    visible = np.ones_like(s, dtype=bool)
    if causal:
        visible = k_pos[None, :] <= q_pos[:, None]
    has_key = np.isfinite(lse)
    lse_safe = np.where(has_key, lse, 0.0)
    P = np.where(visible & has_key[:, None], np.exp(np.where(visible, s, 0.0) - lse_safe[:, None]), 0.0)
    dv = P.T @ do
    dP = do @ v.T
    delta = np.sum(do * o, axis=1)
    ds = P * (dP - delta[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_kv_grads_rows(q, q_pos, k, v, k_pos, scale, causal, do, key_rows, fwd=None):
    """dk and dv of selected key rows, for sequences too long for the full
    probability matrix of ``attention_grads``.

    The same derivative (k8ai "Communication profile": the ring also runs
    backward): with lse_i and o_i of every query row from ``attention_rows``
    and delta_i = <do_i, o_i>, for each selected key j
        P_ij  = exp(s_ij - lse_i) (0 if j is not visible to i)
        dv_j  = sum_i P_ij do_i
        dk_j  = scale * sum_i P_ij (<do_i, v_j> - delta_i) q_i
    Only the selected columns of P are formed.

    key_rows: indices into k, v, k_pos; other arguments as ``attention_grads``.
    fwd: optional (o, lse) of these query rows from ``attention_rows`` (a long
    forward can then be computed in pieces by the caller)
    returns (dk (m, d), dv (m, d)) in fp64
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    key_rows = np.asarray(key_rows, dtype=np.int64)
    o, lse = attention_rows(q, q_pos, k, v, k_pos, scale, causal) if fwd is None else fwd
    delta = np.sum(do * o, axis=1)
    kj, vj, pj = k[key_rows], v[key_rows], k_pos[key_rows]
    s = float(scale) * (q @ kj.T)
    visible = np.ones_like(s, dtype=bool)
    if causal:
        visible = pj[None, :] <= q_pos[:, None]
    has_key = np.isfinite(lse)
    lse_safe = np.where(has_key, lse, 0.0)
    P = np.where(visible & has_key[:, None], np.exp(np.where(visible, s, 0.0) - lse_safe[:, None]), 0.0)
    dP = do @ vj.T
    ds = P * (dP - delta[:, None])
    return float(scale) * (ds.T @ q), P.T @ do


def grouped_attention(q, q_pos, k, v, k_pos, scale, causal):
    """Attention of H query heads when groups of query heads share a K/V head.

    The k8ai page ("Communication profile") ties the bytes a ring moves per
    step to the number of K/V heads; a model with fewer K/V heads than query
    heads lets each K/V head serve a group of query heads. The pages do not
    say which query heads form a group; the reading taken here is consecutive
    groups: with G = H / H_kv, query head h attends to K/V head floor(h / G).
    Each head is then the plain attention of ``attention_rows``.

    q      (H, n, d)     query rows of every head
    k, v   (H_kv, S, d)  keys and values of every K/V head, H % H_kv == 0
    other arguments as ``attention_rows``
    returns (o (H, n, d) fp64, lse (H, n) fp64)
    """
    H, n, d = np.shape(q)
    H_kv = np.shape(k)[0]
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("the query head count must be a multiple of the K/V head count")
    G = H // H_kv
    o = np.zeros((H, n, np.shape(v)[2]), dtype=np.float64)
    lse = np.zeros((H, n), dtype=np.float64)
    for h in range(H):
        o[h], lse[h] = attention_rows(q[h], q_pos, k[h // G], v[h // G], k_pos, scale, causal)
    return o, lse


def grouped_attention_grads(q, q_pos, k, v, k_pos, scale, causal, do):
    """Gradients of ``grouped_attention``: query head h reads K/V head
    floor(h / G), so each K/V head's gradient is the sum of the gradients of
    the G query heads that share it (the chain rule for a shared input).

    q, do (H, n, d); k, v (H_kv, S, d).
    returns (dq (H, n, d), dk (H_kv, S, d), dv (H_kv, S, d)) in fp64
    """
    H, n, d = np.shape(q)
    H_kv = np.shape(k)[0]
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("the query head count must be a multiple of the K/V head count")
    G = H // H_kv
    dq = np.zeros((H, n, d), dtype=np.float64)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for h in range(H):
        a, b, c = attention_grads(q[h], q_pos, k[h // G], v[h // G], k_pos, scale, causal, do[h])
        dq[h] = a
        dk[h // G] += b
        dv[h // G] += c
    return dq, dk, dv


def factored_spatial(q, k, v, T, S_sp, scale):
    """Spatial attention of a frame-major video token sequence.

    Day 83 post, "The spatial-temporal twist": factored video attention runs
    spatial attention inside each frame. Token index = t * S_sp + s. Each query
    at (t, s) attends, without a mask, to the S_sp keys of its own frame t.

    q, k, v (T*S_sp, d); returns (o (T*S_sp, d), lse (T*S_sp,)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.zeros_like(v, dtype=np.float64)
    lse = np.zeros((T * S_sp,), dtype=np.float64)
    pos = np.arange(S_sp)
    for t in range(T):
        rows = slice(t * S_sp, (t + 1) * S_sp)
        o[rows], lse[rows] = attention_rows(q[rows], pos, k[rows], v[rows], pos,
                                            scale, causal=False)
    return o, lse


def factored_temporal(q, k, v, T, S_sp, scale):
    """Temporal attention of a frame-major video token sequence.

    Day 83 post, "The spatial-temporal twist": temporal attention runs across
    frames. A query at (t, s) attends, without a mask, to the T keys
    {t' * S_sp + s : t' < T} at the same spatial position s.

    q, k, v (T*S_sp, d); returns (o (T*S_sp, d), lse (T*S_sp,)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[1]
    # (T, S_sp, d) -> (S_sp, T, d): one length-T problem per spatial position.
    qs = q.reshape(T, S_sp, d).transpose(1, 0, 2)
    ks = k.reshape(T, S_sp, d).transpose(1, 0, 2)
    vs = v.reshape(T, S_sp, d).transpose(1, 0, 2)
    s = float(scale) * np.matmul(qs, ks.transpose(0, 2, 1))  # (S_sp, T, T)
    row_max = s.max(axis=2, keepdims=True)
    w = np.exp(s - row_max)
    denom = w.sum(axis=2, keepdims=True)
    o = np.matmul(w, vs) / denom  # (S_sp, T, d)
    lse = (row_max + np.log(denom))[..., 0]  # (S_sp, T)
    return (o.transpose(1, 0, 2).reshape(T * S_sp, d),
            lse.transpose(1, 0).reshape(T * S_sp))


def merge_lse(o_a, lse_a, o_b, lse_b):
    """Combine two normalised partial attentions over disjoint key sets.

    Day 83 post, "Context parallelism: splitting the sequence": each device
    accumulates partial attention outputs with the online-softmax rule. For
    partial results over disjoint key sets A and B, the softmax weights of the
    union are the partial weights rescaled by exp(lse_part - lse_union):
        lse = ln(exp(lse_a) + exp(lse_b))
        o   = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b
    A side with lse = -inf (no keys) has weight 0; if both sides are empty the
    result is o = 0, lse = -inf.

    o_* (n, d), lse_* (n,); returns (o (n, d), lse (n,)) in fp64.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    hi = np.maximum(lse_a, lse_b)
    empty = ~np.isfinite(hi)
    ref = np.where(empty, 0.0, hi)
    ea = np.exp(lse_a - ref)  # exp(-inf) = 0 for an empty side
    eb = np.exp(lse_b - ref)
    tot = ea + eb
    safe = np.where(empty, 1.0, tot)
    lse = np.where(empty, _NEG_INF, ref + np.log(safe))
    wa = np.where(empty, 0.0, ea / safe)
    wb = np.where(empty, 0.0, eb / safe)
    o = wa[:, None] * o_a + wb[:, None] * o_b
    return o, lse

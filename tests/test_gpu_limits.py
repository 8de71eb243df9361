"""GPU parity of a ring step at the largest query slice the boundary accepts.

ra_step takes one (batch, head) slice of Q of up to INT32_MAX bytes; the
non-final step kernel addresses a lane's query row as a 32-bit element offset
inside the slice, so the rows at the end of the largest slice are where an
overflow would show. One head of 2^23 - 64 query rows (just under 2 GiB of
bf16) attends to one 64-key block; the first and last rows of the slice are
checked against the oracle (the definition of attention, Day 83 post,
"Context parallelism: splitting the sequence"), with and without the causal
mask. Inputs are drawn on the GPU with a seeded generator; the checked rows
are read back and given to the oracle as they are.
"""

import numpy as np
import pytest
import torch

import oracle
import seeded
from context_attention_ra_amd import _lib, ring
from ringcase import assert_close

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

"""GPU parity of factored temporal attention for clips longer than 16 frames.

Day 83 post: the opening paragraph's 48-frame clip and the 120-frame clip of
"What the numbers look like"; "The spatial-temporal twist" defines the
temporal half (each query attends to the T tokens at its spatial position).
Ragged shapes around the 16-frame block size, the largest supported T, and
two workloads of the pages' shapes, all against oracle.factored_temporal.
"""

import numpy as np
import pytest
import torch

import oracle
import seeded
from context_attention_ra_amd import _lib
from ringcase import assert_close

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def _run(wid, B, H, T, S_sp, d):
    N = T * S_sp
    q, k, v = (seeded.gen_bhsd(wid, tid, B, H, 0, N, d, torch.bfloat16, "cuda") for tid in range(3))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = d ** -0.5
    _lib.ra_factored_temporal(q, k, v, T, S_sp, scale, out, lse)
    torch.cuda.synchronize()
    qc, kc, vc = (seeded.exact_f64(t.cpu()) for t in (q, k, v))
    ro, rl = np.zeros((B, H, N, d)), np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            ro[b, h], rl[b, h] = oracle.factored_temporal(qc[b, h], kc[b, h], vc[b, h], T, S_sp, scale)
    assert_close(out.float().cpu().double().numpy(), ro, lse.cpu().double().numpy(), rl, torch.bfloat16,
                 f"temporal T={T} S_sp={S_sp} d={d}")


@pytest.mark.parametrize("T,S_sp,d", [(17, 29, 128), (31, 5, 64), (32, 13, 128), (48, 37, 128), (48, 23, 64),
                                      (64, 10, 128), (65, 9, 64), (80, 6, 128),
                                      (100, 7, 128), (120, 19, 128), (128, 11, 64), (128, 3, 128)])
def test_temporal_long_ragged(gpu_lib, T, S_sp, d):
    banner(f"factored temporal, long clip: T={T} S_sp={S_sp} d={d}")
    _run(800 + T, 2, 3, T, S_sp, d)


def test_temporal_48_frames_of_900(gpu_lib):
    # the opening paragraph's clip: 48 frames of 900 tokens, 32 heads
    banner("factored temporal: 48 frames x 900 tokens, H=32, d=128")
    _run(811, 1, 32, 48, 900, 128)


def test_temporal_120_frames_share(gpu_lib):
    # the 120-frame clip, one of 8 devices' shares after the re-split to
    # spatial positions (3600 / 8 = 450 positions, every frame)
    banner("factored temporal: 120 frames x 450 positions, H=32, d=128")
    _run(812, 1, 32, 120, 450, 128)

"""The synthetic workloads, by name.

Each ring workload describes one rank's share: the global sequence S, the ring
size P, the split that decides which global positions the rank holds, the mask
and the dtype. The video workload describes factored attention over a
frame-major [T * S_sp] token sequence.
"""

from dataclasses import dataclass
from typing import Optional

import torch


@dataclass(frozen=True)
class RingWorkload:
    wid: int            # seed id of the workload's inputs
    name: str
    B: int
    H: int
    d: int
    S: int              # global sequence length
    P: int              # ring size (simulated ranks)
    split: str          # "contiguous" | "zigzag" | "temporal"
    causal: bool
    dtype: torch.dtype
    S_sp: int = 0       # spatial tokens per frame (temporal split only)
    sample_rows: Optional[int] = None  # rows the oracle checks (None = all)
    H_kv: int = 0       # K/V heads (0: one per query head); H % H_kv == 0

    @property
    def L(self) -> int:
        return self.S // self.P

    @property
    def Hkv(self) -> int:
        return self.H_kv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5


@dataclass(frozen=True)
class VideoWorkload:
    wid: int
    name: str
    B: int
    H: int
    d: int
    T: int
    S_sp: int
    dtype: torch.dtype

    @property
    def N(self) -> int:
        return self.T * self.S_sp

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5


# 1: tiny fp32, unmasked, 256-token blocks, P=4
TINY_F32 = RingWorkload(1, "tiny-f32-ring", B=1, H=1, d=64, S=1024, P=4,
                        split="contiguous", causal=False, dtype=torch.float32)
# 2: causal bf16, share of 1 of 2 ranks, zigzag chunks of 1024 (shape of the
#    Ultralytics example: (1, 4, 4096, 64))
CAUSAL_2RANK = RingWorkload(2, "causal-bf16-4k-cp2", B=1, H=4, d=64, S=4096, P=2,
                            split="zigzag", causal=True, dtype=torch.bfloat16)
# 3: 32K causal LLM context, share of 1 of 4 ranks
LLM_32K_CP4 = RingWorkload(3, "llm-32k-causal-cp4", B=1, H=32, d=128, S=32768, P=4,
                           split="zigzag", causal=True, dtype=torch.bfloat16,
                           sample_rows=4096)
# 4: factored video attention, 16 frames x 900 tokens
VIDEO_FACTORED = VideoWorkload(4, "video-factored-16x900", B=1, H=32, d=128, T=16,
                               S_sp=900, dtype=torch.bfloat16)
# 5: video DiT share of 1 of 8 ranks, 120 frames x 3600 tokens, temporal-first
VIDEO_DIT_CP8 = RingWorkload(5, "video-dit-432k-cp8", B=1, H=32, d=128, S=432000, P=8,
                             split="temporal", causal=False, dtype=torch.bfloat16,
                             S_sp=3600, sample_rows=4096)

# Grouped K/V heads (fewer K/V heads than query heads; the k8ai page ties the
# ring's bytes per step to the K/V head count): the causal 4K share with 8
# query heads over 2 K/V heads, and the 32K share with 32 over 8.
CAUSAL_2RANK_GQA = RingWorkload(6, "causal-bf16-4k-cp2-gqa4", B=1, H=8, d=64, S=4096, P=2,
                                split="zigzag", causal=True, dtype=torch.bfloat16, H_kv=2)
LLM_32K_CP4_GQA = RingWorkload(7, "llm-32k-causal-cp4-gqa4", B=1, H=32, d=128, S=32768, P=4,
                               split="zigzag", causal=True, dtype=torch.bfloat16,
                               sample_rows=4096, H_kv=8)

RING_WORKLOADS = {w.name: w for w in (TINY_F32, CAUSAL_2RANK, LLM_32K_CP4, VIDEO_DIT_CP8,
                                      CAUSAL_2RANK_GQA, LLM_32K_CP4_GQA)}
ALL = {**RING_WORKLOADS, VIDEO_FACTORED.name: VIDEO_FACTORED}

"""CPU oracle for the ring-attention hot path (test infrastructure only).

This package is the reference against which the HIP kernels are checked. It is
plain, slow and written to be checked by eye against the pages that describe
the method. It shares no code with ``context_attention_ra_amd`` and imports
nothing from it; only the seeded input generator (``seeded``) serves both.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package. The product
path never routes through it.

Sources (cited by page title and section):
* "Day 83" post on skandtandon.pages.dev (context parallelism for video
  diffusion): sections "Context parallelism: splitting the sequence",
  "The spatial-temporal twist", "What the numbers look like",
  "The communication pattern".
* Ultralytics glossary, "Context Parallelism": "How Context Parallelism Works",
  "Practical Use and Tradeoffs".
* k8ai concepts, "Sequence and Context Parallel": "How context parallel works"
  (the ring figure and the causal balance remark), "Communication profile"
  (ring volume and the number of K/V heads; exchanges in the forward and
  the backward pass).
"""

from .attention import (  # noqa: F401
    attention_grads,
    attention_kv_grads_rows,
    attention_rows,
    factored_spatial,
    factored_temporal,
    grouped_attention,
    grouped_attention_grads,
    merge_lse,
)
from .layout import (  # noqa: F401
    contiguous_positions,
    ring_source,
    temporal_first_positions,
    zigzag_positions,
)

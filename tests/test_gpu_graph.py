"""Whole ring passes captured in a HIP graph replay bitwise like eager passes.

The ring driver launches every kernel on the caller's current stream and the
block pass on a side stream forked from it and joined back through events,
and nothing on the path clears memory with a memset, so one pass of
`ring.run` can be captured (torch.cuda.CUDAGraph) and replayed. The replays
are compared with the eager pass on the same inputs, with eager passes run
between them (the causal two-rank share, rank 0, and the same share with
grouped K/V heads), for the forward pass and for the backward pass (where the
grouped case runs the dK/dV halves on a second stream; the accumulators are
cleared by torch's fill kernel, not a memset). The backward pass's opt-in
split diagonal step is not captured: run_bwd refuses it under capture.
"""

import pytest
import torch

from context_attention_ra_amd import configs, layout, ring
import seeded

pytestmark = pytest.mark.gpu


def _inputs(w, dev):
    import numpy as np
    segs = [layout.split(w.split, w.S, w.P, t) for t in range(w.P)]
    pos = [np.concatenate([np.arange(s, s + n) for s, n in sg]) for sg in segs]
    q = seeded.gen_bhsd_at(w.wid, seeded.Q, w.B, w.H, pos[0], w.d, w.dtype, dev)
    kv = [(seeded.gen_bhsd_at(w.wid, seeded.K, w.B, w.Hkv, pos[t], w.d, w.dtype, dev),
           seeded.gen_bhsd_at(w.wid, seeded.V, w.B, w.Hkv, pos[t], w.d, w.dtype, dev)) for t in range(w.P)]
    return q, segs, kv


@pytest.mark.parametrize("wname", ["causal-bf16-4k-cp2", "causal-bf16-4k-cp2-gqa4"])
def test_ring_pass_in_a_graph(gpu_lib, wname):
    print(f"\n[graph] {wname}: one ring pass captured and replayed", flush=True)
    w = configs.RING_WORKLOADS[wname]
    dev = torch.device("cuda")
    q, segs, kv = _inputs(w, dev)
    st = ring.RingState(w.B, w.H, w.L, w.d, dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
    bufs = [(torch.empty_like(kv[0][0]), torch.empty_like(kv[0][1])) for _ in range(2)]
    side = torch.cuda.Stream(dev)

    def one():
        ring.run(q, segs[0], kv, segs, 0, w.causal, scale=w.scale, out=out, lse=lse, state=st, bufs=bufs,
                 copy_stream=side)

    one()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        one()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {rep}"
        one()  # an eager pass between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"eager after replay {rep}"


@pytest.mark.parametrize("wname", ["causal-bf16-4k-cp2", "causal-bf16-4k-cp2-gqa4"])
def test_backward_ring_pass_in_a_graph(gpu_lib, wname):
    # the grouped case runs the dK/dV halves on a second stream (joined back
    # before the pass returns)
    print(f"\n[graph] {wname}: one backward ring pass captured and replayed", flush=True)
    w = configs.RING_WORKLOADS[wname]
    dev = torch.device("cuda")
    q, segs, kv = _inputs(w, dev)
    import numpy as np
    pos0 = np.concatenate([np.arange(s, s + n) for s, n in segs[0]])
    do = seeded.gen_bhsd_at(w.wid, seeded.DO, w.B, w.H, pos0, w.d, w.dtype, dev)
    out, lse, _ = ring.run(q, segs[0], kv, segs, 0, w.causal, scale=w.scale)
    dkv = [(torch.empty(k.shape, dtype=torch.float32, device=dev), torch.empty(k.shape, dtype=torch.float32, device=dev))
           for k, _ in kv]
    res = {}

    def one():
        for dk, dv in dkv:
            dk.zero_()
            dv.zero_()
        res["dq"], _ = ring.run_bwd(q, segs[0], kv, segs, 0, w.causal, out, lse, do, scale=w.scale, dkv=dkv)

    one()
    torch.cuda.synchronize()
    ref = [res["dq"].clone()] + [t.clone() for pair in dkv for t in pair]
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        one()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    dq_graph = res["dq"]  # the graph's own output tensor
    torch.cuda.synchronize()
    for rep in range(3):
        dq_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [dq_graph] + [t for pair in dkv for t in pair]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep}"
        one()
        torch.cuda.synchronize()


@pytest.mark.skip(reason="a captured backward pass with the split diagonal step (a third stream forked "
                         "from the dK/dV stream and joined back into it) crashed the host process inside "
                         "the runtime's end of capture; run_bwd refuses the split under capture until the "
                         "cause is shown")
def test_backward_split_diagonal_in_a_graph(gpu_lib):
    w = configs.RING_WORKLOADS["causal-bf16-4k-cp2-gqa4"]
    dev = torch.device("cuda")
    q, segs, kv = _inputs(w, dev)
    out, lse, _ = ring.run(q, segs[0], kv, segs, 0, w.causal, scale=w.scale)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ring.run_bwd(q, segs[0], kv, segs, 0, w.causal, out, lse, q, scale=w.scale, split=True)


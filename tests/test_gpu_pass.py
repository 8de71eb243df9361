"""The ring's block pass (ra_kv_pass) moves K and V byte for byte.

For 16-byte aligned buffers of whole 16-byte pieces the library uses its own
pass kernel (sized to run beside a ring step); otherwise the runtime's copy.
Both are checked against the source bytes, with guard bytes around every
destination that must stay untouched, for sizes that do not divide evenly
over the kernel's waves, a single piece, and unaligned or ragged buffers.
The ring's own tests check that passing the blocks on a side stream beside
the steps gives bitwise the same output as passing them on the compute stream.
"""

import ctypes

import pytest
import torch

from context_attention_ra_amd import _lib

pytestmark = pytest.mark.gpu

GUARD = 4096


def banner(msg):
    print(f"\n[kv_pass] {msg}", flush=True)


def pass_bytes(nbytes, offset, seed):
    """Copy nbytes from two random buffers at byte `offset` into two guarded ones."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    total = offset + nbytes + GUARD
    src = [torch.randint(0, 256, (total,), dtype=torch.uint8, device="cuda", generator=g) for _ in range(2)]
    dst = [torch.full((GUARD + total,), 0xA5, dtype=torch.uint8, device="cuda") for _ in range(2)]
    lib = _lib.load()
    p = lambda t, off: ctypes.c_void_p(t.data_ptr() + off)
    st = lib.ra_kv_pass(p(src[0], offset), p(src[1], offset), p(dst[0], GUARD + offset), p(dst[1], GUARD + offset),
                        nbytes, None)
    assert st == _lib.RA_OK, _lib.status_name(st)
    torch.cuda.synchronize()
    for s, d in zip(src, dst):
        assert torch.equal(d[GUARD + offset:GUARD + offset + nbytes], s[offset:offset + nbytes])
        assert bool((d[:GUARD + offset] == 0xA5).all())
        assert bool((d[GUARD + offset + nbytes:] == 0xA5).all())


@pytest.mark.parametrize("nbytes", [16, 16 * 127, 16 * 128 * 2048 + 16 * 37, 64 << 20])
def test_pass_kernel_copies_exactly(gpu_lib, nbytes):
    banner(f"aligned, {nbytes} bytes")
    pass_bytes(nbytes, 0, seed=nbytes % 1000)


@pytest.mark.parametrize("nbytes,offset", [(16 * 1000 + 2, 0), (16 * 1000, 2), (6, 8)])
def test_unaligned_or_ragged_pass_uses_the_runtime_copy(gpu_lib, nbytes, offset):
    banner(f"unaligned or ragged, {nbytes} bytes at offset {offset}")
    pass_bytes(nbytes, offset, seed=7)


def test_pass_of_block_tensors(gpu_lib):
    banner("bf16 block tensors through the binding")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    k, v = (torch.randn((1, 4, 1000, 128), device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
    kd, vd = torch.empty_like(k), torch.empty_like(v)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    _lib.ra_kv_pass(k, v, kd, vd, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(kd, k) and torch.equal(vd, v)

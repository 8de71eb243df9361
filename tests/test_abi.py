"""C-ABI contract checks that need no GPU: the library loads, exports every
declared entry point, and rejects bad arguments before any HIP call.

The pointers used here are fake (never dereferenced): every call below fails
validation on the host, which is the behaviour under test.
"""

import ctypes
import os
import re

import pytest

from context_attention_ra_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")


@pytest.fixture(scope="module")
def lib():
    # RA_TEST_ABI_LIB: the host-only build of the ABI layer with
    # AddressSanitizer and counting launcher stand-ins (tests/test_abi_asan.py)
    path = os.environ.get("RA_TEST_ABI_LIB", _lib.LIB_PATH)
    if not os.path.exists(path):
        from context_attention_ra_amd import build
        build.build()
    return _lib.load(path)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert _lib.status_name(0) == "RA_OK"
    assert _lib.status_name(1) == "RA_ERR_INVALID_ARG"
    assert _lib.status_name(2) == "RA_ERR_UNSUPPORTED"
    assert _lib.status_name(3) == "RA_ERR_HIP"
    assert lib.ra_version() >= 100
    assert lib.ra_last_hip_error() == 0


FAKE = 0x10000  # 16-byte aligned, never touched


def ptr(i):
    return FAKE * (i + 1) << 20  # far apart: no accidental overlap


def step(lib, q=None, k=None, v=None, dt=1, B=1, H=1, Lq=64, Lk=64, d=128, qs=((0, 64),),
         ks=((0, 64),), mask=1, scale=0.1, flags=1, o=None, m=None, l=None):
    q = ptr(0) if q is None else q
    k = ptr(1) if k is None else k
    v = ptr(2) if v is None else v
    o = ptr(3) if o is None else o
    m = ptr(4) if m is None else m
    l = ptr(5) if l is None else l
    a, b = _lib.segs(list(qs)), _lib.segs(list(ks))
    return lib.ra_step(q, k, v, dt, B, H, Lq, Lk, d, ctypes.byref(a), ctypes.byref(b), mask,
                       scale, flags, o, m, l, None)


INV, UNS = _lib.RA_ERR_INVALID_ARG, _lib.RA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), INV), (dict(k=0), INV), (dict(v=0), INV), (dict(o=0), INV), (dict(m=0), INV),
    (dict(l=0), INV), (dict(B=0), INV), (dict(H=-1), INV), (dict(Lq=0, qs=()), INV),
    (dict(Lk=-5), INV), (dict(dt=7), INV), (dict(mask=2), INV), (dict(scale=0.0), INV),
    (dict(scale=float("inf")), INV), (dict(scale=float("nan")), INV), (dict(scale=-1.0), INV),
    (dict(flags=2), INV), (dict(qs=((0, 63),)), INV), (dict(qs=((0, 32), (-4, 32))), INV),
    (dict(ks=((0, 32), (100, 33))), INV), (dict(ks=((0, 0), (10, 64))), INV),
    (dict(qs=((2**31 - 10, 64),)), INV), (dict(q=ptr(0) + 8), INV),
    (dict(o=ptr(0)), INV),  # state overlapping the queries
    (dict(m=ptr(3)), INV),  # m overlapping o_acc
    (dict(d=96), UNS), (dict(d=256), UNS),
    # a query slice past 32-bit byte offsets (2^23 rows of 128 bf16 values)
    (dict(Lq=1 << 23, qs=((0, 1 << 23),)), UNS),
])
def test_step_rejects_bad_arguments(lib, kw, expect):
    assert step(lib, **kw) == expect


def test_segs_with_three_runs_is_rejected(lib):
    s = _lib.RaSegs()
    s.n = 3
    t = _lib.segs([(0, 64)])
    assert lib.ra_step(ptr(0), ptr(1), ptr(2), 1, 1, 1, 64, 64, 128, ctypes.byref(s),
                       ctypes.byref(t), 1, 0.1, 0, ptr(3), ptr(4), ptr(5), None) == INV
    s = _lib.segs([(0, 64)])
    s.reserved = 1
    assert lib.ra_step(ptr(0), ptr(1), ptr(2), 1, 1, 1, 64, 64, 128, ctypes.byref(s),
                       ctypes.byref(t), 1, 0.1, 0, ptr(3), ptr(4), ptr(5), None) == INV


def test_finalize_and_merge_validation(lib):
    f = lib.ra_finalize
    assert f(None, ptr(1), ptr(2), 1, 1, 64, 128, ptr(3), 1, ptr(4), None) == INV
    assert f(ptr(0), ptr(1), ptr(2), 1, 1, 64, 128, ptr(0), 1, None, None) == INV  # out == state
    assert f(ptr(0), ptr(1), ptr(2), 1, 1, 64, 128, ptr(3), 9, None, None) == INV
    assert f(ptr(0), ptr(1), ptr(2), 1, 1, 64, 80, ptr(3), 1, None, None) == UNS
    mg = lib.ra_merge_lse
    assert mg(ptr(0), ptr(1), ptr(2), ptr(3), 1, 1, 1, 64, 128, None, ptr(5), None) == INV
    # output partially overlapping an input is refused; exact aliasing is allowed (not launched here)
    assert mg(ptr(0), ptr(1), ptr(2), ptr(3), 1, 1, 1, 64, 128, ptr(0) + 256, ptr(5), None) == INV
    assert mg(ptr(0), ptr(1), ptr(2), ptr(3), 1, 1, 1, 64, 64 + 1, ptr(4), ptr(5), None) == UNS


def test_factored_validation(lib):
    for fn in (lib.ra_factored_spatial, lib.ra_factored_temporal):
        assert fn(None, ptr(1), ptr(2), 1, 1, 1, 4, 9, 128, 0.1, ptr(3), None, None) == INV
        assert fn(ptr(0), ptr(1), ptr(2), 1, 1, 1, 0, 9, 128, 0.1, ptr(3), None, None) == INV
        assert fn(ptr(0), ptr(1), ptr(2), 1, 1, 1, 4, 9, 128, 0.1, ptr(1), None, None) == INV
        assert fn(ptr(0), ptr(1), ptr(2), 0, 1, 1, 4, 9, 128, 0.1, ptr(3), None, None) == UNS
        assert fn(ptr(0), ptr(1), ptr(2), 1, 1, 1, 4, 9, 32, 0.1, ptr(3), None, None) == UNS
    # a long clip's slice must be addressable with 32-bit byte offsets
    assert lib.ra_factored_temporal(ptr(0), ptr(1), ptr(2), 1, 1, 1, 120, 1 << 17, 128, 0.1, ptr(3),
                                    None, None) == UNS
    # clips longer than 128 frames are not supported (the pages' longest is 120)
    assert lib.ra_factored_temporal(ptr(0), ptr(1), ptr(2), 1, 1, 1, 129, 9, 128, 0.1, ptr(3),
                                    None, None) == UNS
    # offsets inside one frame of the spatial kernel are 32-bit
    assert lib.ra_factored_spatial(ptr(0), ptr(1), ptr(2), 1, 1, 1, 1, 1 << 23, 128, 0.1, ptr(3),
                                   None, None) == UNS


def test_kv_pass_validation(lib):
    assert lib.ra_kv_pass(ptr(0), ptr(1), ptr(2), ptr(3), 0, None) == _lib.RA_OK  # no-op
    assert lib.ra_kv_pass(None, ptr(1), ptr(2), ptr(3), 64, None) == INV
    assert lib.ra_kv_pass(ptr(0), ptr(1), ptr(0), ptr(3), 64, None) == INV
    assert lib.ra_kv_pass(ptr(0), ptr(1), ptr(2), ptr(2) + 32, 64, None) == INV


def step_gqa(lib, H=4, H_kv=2, d=128, final=False, out=None):
    a, b = _lib.segs([(0, 64)]), _lib.segs([(0, 64)])
    args = (ptr(0), ptr(1), ptr(2), 1, 1, H, H_kv, 64, 64, d, ctypes.byref(a), ctypes.byref(b), 1,
            0.1, 1, ptr(3), ptr(4), ptr(5))
    if final:
        return lib.ra_step_final_gqa(*args, out, None, None)
    return lib.ra_step_gqa(*args, None)


@pytest.mark.parametrize("H,H_kv", [(4, 0), (4, -2), (6, 4), (4, 8), (3, 2)])
def test_gqa_rejects_heads_that_do_not_divide(lib, H, H_kv):
    assert step_gqa(lib, H=H, H_kv=H_kv) == INV
    assert step_gqa(lib, H=H, H_kv=H_kv, final=True, out=ptr(6)) == INV


def test_gqa_valid_heads_reach_the_later_checks(lib):
    # a valid grouping passes the head check and stops at the unsupported head size
    for H, H_kv in ((4, 2), (8, 1), (5, 5)):
        assert step_gqa(lib, H=H, H_kv=H_kv, d=96) == UNS
        assert step_gqa(lib, H=H, H_kv=H_kv, d=96, final=True, out=ptr(6)) == UNS
    assert step_gqa(lib, final=True, out=None) == INV
    assert step_gqa(lib, final=True, out=ptr(0)) == INV  # out overlapping the queries


def test_gqa_spans_use_the_kv_head_count(lib):
    # one K/V head of 64 x 96 bf16 is 12 KiB: a state placed right after it does not
    # overlap K with one K/V head, but would with four (d = 96 stops the call after the
    # overlap checks)
    a, b = _lib.segs([(0, 64)]), _lib.segs([(0, 64)])
    k = ptr(1)
    o_after_one_head = k + 64 * 96 * 2
    args = lambda H_kv: (ptr(0), k, ptr(2), 1, 1, 4, H_kv, 64, 64, 96, ctypes.byref(a),
                         ctypes.byref(b), 1, 0.1, 1, o_after_one_head, ptr(4), ptr(5), None)
    assert lib.ra_step_gqa(*args(1)) == UNS
    assert lib.ra_step_gqa(*args(4)) == INV


def step_bwd(lib, dt=1, d=128, flags=3, q=None, dout=None, lse=None, delta=None, dq=None, dk=None, dv=None,
             H=1, H_kv=1):
    a, b = _lib.segs([(0, 64)]), _lib.segs([(0, 64)])
    pick = lambda x, i: ptr(i) if x is None else x
    return lib.ra_step_bwd(pick(q, 0), ptr(1), ptr(2), pick(dout, 3), pick(lse, 4), pick(delta, 5), dt,
                           1, H, H_kv, 64, 64, d, ctypes.byref(a), ctypes.byref(b), 1, 0.1, flags,
                           pick(dq, 6), pick(dk, 7), pick(dv, 8), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dout=0), INV), (dict(lse=0), INV), (dict(delta=0), INV), (dict(dq=0), INV),
    (dict(dk=0), INV), (dict(dv=0), INV), (dict(flags=16), INV),
    (dict(flags=4 | 8), INV),          # both halves skipped
    (dict(flags=4 | 3, d=96), UNS), (dict(flags=8 | 3, d=96), UNS),  # one half: valid flags
    (dict(flags=4, dq=0), INV),        # a skipped half's accumulator is still checked
    (dict(dk=ptr(1)), INV),            # dk accumulator over the keys
    (dict(dv=ptr(7) + 256), INV),      # dv overlapping dk
    (dict(dq=ptr(3)), INV),            # dq over the upstream gradient
    (dict(dt=0), UNS), (dict(d=96), UNS),
    (dict(flags=0, d=96), UNS), (dict(flags=1, d=96), UNS), (dict(flags=2, d=96), UNS),
    (dict(H=4, H_kv=3), INV), (dict(H=4, H_kv=0), INV), (dict(H=4, H_kv=2, d=96), UNS),
])
def test_step_bwd_rejects_bad_arguments(lib, kw, expect):
    assert step_bwd(lib, **kw) == expect


def test_step_bwd_refuses_grids_past_32_bits(lib):
    # 2^15 heads of 2^24 keys at d=64 pass every other check (fake pointers 2^48 apart, so
    # no span overlaps) but give 2^31 (K/V head, 256-key tile) pairs
    H, Lk = 1 << 15, 1 << 24
    a, b = _lib.segs([(0, 64)]), _lib.segs([(0, Lk)])
    p = [(i + 1) << 48 for i in range(9)]
    st = lib.ra_step_bwd(p[0], p[1], p[2], p[3], p[4], p[5], 1, 1, H, H, 64, Lk, 64, ctypes.byref(a),
                         ctypes.byref(b), 1, 0.1, 3, p[6], p[7], p[8], None)
    assert st == UNS
    # an invalid grouping is refused first, as an argument error
    assert lib.ra_step_bwd(p[0], p[1], p[2], p[3], p[4], p[5], 1, 1, H, 3, 64, Lk, 64, ctypes.byref(a),
                           ctypes.byref(b), 1, 0.1, 3, p[6], p[7], p[8], None) == INV


def test_step_bwd_refuses_query_slices_past_32_bit_bytes(lib):
    # 2^23 local queries at d=128 bf16 are 2^31 bytes per slice: past the
    # 32-bit byte size of the buffer resource the dK/dV kernel streams them with
    Lq = 1 << 23
    a, b = _lib.segs([(0, Lq)]), _lib.segs([(0, 64)])
    p = [(i + 1) << 48 for i in range(9)]
    assert lib.ra_step_bwd(p[0], p[1], p[2], p[3], p[4], p[5], 1, 1, 1, 1, Lq, 64, 128,
                           ctypes.byref(a), ctypes.byref(b), 1, 0.1, 3, p[6], p[7], p[8], None) == UNS


def test_bwd_prep_validation(lib):
    p = lib.ra_bwd_prep
    assert p(None, ptr(1), 1, 1, 1, 64, 128, ptr(2), None) == INV
    assert p(ptr(0), ptr(1), 1, 1, 1, 64, 128, None, None) == INV
    assert p(ptr(0), ptr(1), 1, 1, 1, 0, 128, ptr(2), None) == INV
    assert p(ptr(0), ptr(1), 1, 1, 1, 64, 128, ptr(1) + 64, None) == INV  # delta inside dout
    assert p(ptr(0), ptr(1), 0, 1, 1, 64, 128, ptr(2), None) == UNS       # fp32 inputs
    assert p(ptr(0), ptr(1), 1, 1, 1, 64, 80, ptr(2), None) == UNS


def test_binding_checks_shapes_before_calling():
    # the binding refuses tensors whose shapes do not match what the C call
    # would assume (CPU tensors: the check fires before any pointer is used)
    import torch
    q = torch.zeros((1, 4, 64, 64), dtype=torch.bfloat16)
    k2 = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)
    k3 = torch.zeros((1, 3, 64, 64), dtype=torch.bfloat16)
    st = [torch.zeros((1, 4, 64, 64)), torch.zeros((1, 4, 64)), torch.zeros((1, 4, 64))]
    with pytest.raises(ValueError):
        _lib.ra_step(q, k3, k3, [(0, 64)], [(0, 64)], True, 0.1, *st)
    with pytest.raises(ValueError):
        _lib.ra_step(q, k2, k3, [(0, 64)], [(0, 64)], True, 0.1, *st)
    with pytest.raises(ValueError):  # dk/dv accumulators shaped like the K/V block
        _lib.ra_step_bwd(q, k2, k2, q, st[1], st[2], [(0, 64)], [(0, 64)], True, 0.1, st[0],
                         torch.zeros((1, 4, 64, 64)), torch.zeros((1, 4, 64, 64)))
    with pytest.raises(ValueError):  # a half of the step that does not exist
        _lib.ra_step_bwd(q, k2, k2, q, st[1], st[2], [(0, 64)], [(0, 64)], True, 0.1, st[0],
                         torch.zeros((1, 2, 64, 64)), torch.zeros((1, 2, 64, 64)), parts="dk")
    with pytest.raises(ValueError):
        _lib.ra_finalize(st[0], st[1], st[2], torch.zeros((1, 4, 63, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        _lib.ra_factored_spatial(q, q, q[:, :, :32], 4, 16, 0.1, torch.empty_like(q))


def test_copy_rows_validation(lib):
    c = lib.ra_copy_rows
    assert c(ptr(0), 64, 0, ptr(1), 64, 0, 4, 0, 256, None) == _lib.RA_OK  # no rows: no-op
    assert c(None, 64, 0, ptr(1), 64, 0, 4, 8, 256, None) == INV
    assert c(ptr(0), 64, 0, ptr(1), 64, 0, 0, 8, 256, None) == INV          # no slices
    assert c(ptr(0), 64, 60, ptr(1), 64, 0, 4, 8, 256, None) == INV         # past the source slice
    assert c(ptr(0), 64, 0, ptr(1), 64, 60, 4, 8, 256, None) == INV         # past the destination slice
    assert c(ptr(0), 64, -1, ptr(1), 64, 0, 4, 8, 256, None) == INV
    assert c(ptr(0), 64, 0, ptr(0) + 256 * 8, 64, 0, 4, 8, 256, None) == INV  # overlapping ranges


def test_add_rows_validation(lib):
    a = lib.ra_add_rows
    assert a(ptr(0), 64, 0, ptr(1), 64, 0, 4, 0, 128, None) == _lib.RA_OK  # no rows: no-op
    assert a(None, 64, 0, ptr(1), 64, 0, 4, 8, 128, None) == INV
    assert a(ptr(0), 64, 0, ptr(1), 64, 0, 0, 8, 128, None) == INV          # no slices
    assert a(ptr(0), 64, 0, ptr(1), 64, 0, 4, 8, 126, None) == INV          # d not a multiple of 4
    assert a(ptr(0), 64, 60, ptr(1), 64, 0, 4, 8, 128, None) == INV         # past the source slice
    assert a(ptr(0), 64, 0, ptr(1), 64, 60, 4, 8, 128, None) == INV         # past the destination slice
    assert a(ptr(0), 64, -1, ptr(1), 64, 0, 4, 8, 128, None) == INV
    assert a(ptr(0) + 4, 64, 0, ptr(1), 64, 0, 4, 8, 128, None) == INV      # misaligned
    assert a(ptr(0), 64, 0, ptr(0) + 512 * 8, 64, 0, 4, 8, 128, None) == INV  # overlapping ranges


def test_variants_refuse_segments_that_do_not_tile_the_sequence():
    from context_attention_ra_amd import variants
    with pytest.raises(ValueError):
        variants._global_length([[(0, 10)], [(12, 10)]])
    with pytest.raises(ValueError):
        variants._global_length([[(0, 10)], [(5, 10)]])
    assert variants._global_length([[(0, 4), (12, 4)], [(4, 8)]]) == 16


def test_ring_drivers_refuse_bad_block_orders():
    # the order is checked on the host before any buffer is made or any call is made
    import torch
    from context_attention_ra_amd import ring
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    kv = [(torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16),) * 2 for _ in range(3)]
    segs = [[(64 * t, 64)] for t in range(3)]
    for order in ([0, 1, 1], [0, 1], [2, 1, 0, 3]):
        with pytest.raises(ValueError):
            ring.run(q, segs[0], kv, segs, 0, True, order=order)
        with pytest.raises(ValueError):
            ring.run_bwd(q, segs[0], kv, segs, 0, True, q, torch.zeros((1, 1, 64)), q, order=order)


def test_backward_split_needs_an_even_group():
    # splitting the diagonal step's query heads in two halves per K/V head is
    # refused on the host for an odd group (3 query heads per K/V head)
    import torch
    from context_attention_ra_amd import ring
    q = torch.zeros((1, 3, 64, 64), dtype=torch.bfloat16)
    kv = [(torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16),) * 2]
    with pytest.raises(ValueError):
        ring.run_bwd(q, [(0, 64)], kv, [[(0, 64)]], 0, True, q, torch.zeros((1, 3, 64)), q, split=True)


def test_group_halves_partition_every_group():
    # the split diagonal step's head halves: together they hold every query
    # head once, and head i of half p is query head (i // (G/2)) * G +
    # p * G/2 + i % (G/2), which belongs to K/V head i // (G/2) of the half
    import torch
    from context_attention_ra_amd import ring
    for B, H_kv, G in ((1, 1, 2), (2, 3, 4), (1, 8, 4), (2, 2, 8)):
        H = H_kv * G
        x = torch.arange(B * H * 5 * 3, dtype=torch.float32).reshape(B, H, 5, 3)
        halves = [ring.group_half(x, H_kv, p) for p in (0, 1)]
        seen = []
        for p, hx in enumerate(halves):
            assert hx.shape == (B, H // 2, 5, 3) and hx.is_contiguous()
            for i in range(H // 2):
                src = (i // (G // 2)) * G + p * (G // 2) + i % (G // 2)
                assert src // G == i // (G // 2)  # the same K/V head
                assert torch.equal(hx[:, i], x[:, src])
                seen.append(src)
        assert sorted(seen) == list(range(H))
        lse = torch.randn(B, H, 5)
        assert torch.equal(torch.cat([ring.group_half(lse, H_kv, p).reshape(B, H_kv, G // 2, 5)
                                      for p in (0, 1)], dim=2).reshape(B, H, 5), lse)
    with pytest.raises(ValueError):
        ring.group_half(torch.zeros(1, 3, 4), 1, 0)


def test_backward_split_refused_under_graph_capture(monkeypatch):
    # the split diagonal step is refused while the current stream captures a
    # graph (checked on the host before any buffer is made or call is made)
    import torch
    from context_attention_ra_amd import ring
    monkeypatch.setattr(torch.cuda, "current_stream", lambda dev=None: None)
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    monkeypatch.setattr(_lib, "load", lambda: (_ for _ in ()).throw(AssertionError("the library was reached")))
    q = torch.zeros((1, 4, 64, 64), dtype=torch.bfloat16)
    kv = [(torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16),) * 2]
    with pytest.raises(RuntimeError):
        ring.run_bwd(q, [(0, 64)], kv, [[(0, 64)]], 0, True, q, torch.zeros((1, 4, 64)), q, split=True)


def test_binding_checks_dtypes_and_devices_before_any_library_call(monkeypatch):
    # The C calls derive every byte count from one dtype argument and cannot
    # tell host pointers from device ones: the binding must refuse mismatched
    # dtypes and tensors off the GPU before the library is even loaded.
    import torch

    def no_call(*a, **k):
        raise AssertionError("the library was reached")

    monkeypatch.setattr(_lib, "load", no_call)
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros((1, 2, 64, 64), dtype=bf)
    st = [torch.zeros((1, 2, 64, 64)), torch.zeros((1, 2, 64)), torch.zeros((1, 2, 64))]
    segs = ([(0, 64)], [(0, 64)], True, 0.1)
    with pytest.raises(TypeError):  # fp32 queries with bf16 keys: K/V read at twice their size
        _lib.ra_step(q.float(), q, q, *segs, *st)
    with pytest.raises(TypeError):
        _lib.ra_step(q, q, q.float(), *segs, *st)
    with pytest.raises(TypeError):  # a bf16 running state would take fp32 stores
        _lib.ra_step(q, q, q, *segs, st[0].to(bf), st[1], st[2])
    with pytest.raises(TypeError):
        _lib.ra_step(q, q, q, *segs, st[0], st[1].to(bf), st[2])
    with pytest.raises(TypeError):  # fp16 is not a library dtype
        _lib.ra_step(q.half(), q.half(), q.half(), *segs, *st)
    with pytest.raises(ValueError, match="GPU"):  # right dtypes, host memory
        _lib.ra_step(q, q, q, *segs, *st)
    with pytest.raises(TypeError):
        _lib.ra_step_final(q, q, q, *segs, *st, q.float(), st[1])
    with pytest.raises(TypeError):
        _lib.ra_step_final(q, q, q, *segs, *st, q, st[1].to(bf))
    with pytest.raises(ValueError, match="GPU"):
        _lib.ra_step_final(q, q, q, *segs, *st, q, st[1])
    lse, delta = st[1], st[2]
    with pytest.raises(TypeError):  # gradient accumulators are fp32
        _lib.ra_step_bwd(q, q, q, q, lse, delta, *segs, st[0], st[0].to(bf), st[0])
    with pytest.raises(TypeError):
        _lib.ra_step_bwd(q, q, q, q.float(), lse, delta, *segs, st[0], st[0], st[0])
    with pytest.raises(TypeError):
        _lib.ra_step_bwd(q, q, q, q, lse, delta, *segs, st[0].to(bf), st[0], st[0])
    with pytest.raises(ValueError, match="GPU"):
        _lib.ra_step_bwd(q, q, q, q, lse, delta, *segs, st[0], st[0], st[0])
    with pytest.raises(TypeError):
        _lib.ra_bwd_prep(q, q.float(), delta)
    with pytest.raises(TypeError):
        _lib.ra_bwd_prep(q, q, delta.to(bf))
    with pytest.raises(ValueError, match="GPU"):
        _lib.ra_bwd_prep(q, q, delta)
    with pytest.raises(TypeError):
        _lib.ra_finalize(st[0], st[1], st[2], q.half())
    with pytest.raises(TypeError):
        _lib.ra_finalize(st[0].to(bf), st[1], st[2], q)
    with pytest.raises(ValueError, match="GPU"):
        _lib.ra_finalize(st[0], st[1], st[2], q, lse)
    with pytest.raises(TypeError):
        _lib.ra_merge_lse(q, lse, q.float(), lse, q, lse)
    with pytest.raises(TypeError):
        _lib.ra_merge_lse(q, lse, q, lse.to(bf), q, lse)
    with pytest.raises(ValueError, match="GPU"):
        _lib.ra_merge_lse(q, lse, q, lse, torch.empty_like(q), torch.empty_like(lse))
    for fn in (_lib.ra_factored_spatial, _lib.ra_factored_temporal):
        with pytest.raises(TypeError):
            fn(q, q.float(), q, 4, 16, 0.1, torch.empty_like(q))
        with pytest.raises(TypeError):
            fn(q, q, q, 4, 16, 0.1, torch.empty_like(q), lse.to(bf))
        with pytest.raises(ValueError, match="GPU"):
            fn(q, q, q, 4, 16, 0.1, torch.empty_like(q), lse)
    with pytest.raises(ValueError, match="GPU"):
        _lib.ra_kv_pass(q, q, torch.empty_like(q), torch.empty_like(q))
    with pytest.raises(ValueError, match="GPU"):
        _lib.ra_copy_rows(q, 0, torch.empty_like(q), 0, 8)


def test_rejected_calls_launch_nothing(lib):
    # only the host build with counting launcher stand-ins can see launches
    if not hasattr(lib, "ra_test_launch_count"):
        pytest.skip("needs the host build of the ABI layer with counting launchers")
    count = lib.ra_test_launch_count
    count.restype = ctypes.c_int32
    before = count()
    for kw in (dict(q=0), dict(scale=float("nan")), dict(qs=((0, 63),)), dict(o=ptr(0)), dict(d=96)):
        assert step(lib, **kw) != _lib.RA_OK
    for kw in (dict(dout=0), dict(flags=4 | 8), dict(dk=ptr(1)), dict(d=96)):
        assert step_bwd(lib, **kw) != _lib.RA_OK
    assert lib.ra_factored_temporal(ptr(0), ptr(1), ptr(2), 1, 1, 1, 129, 9, 128, 0.1, ptr(3), None,
                                    None) != _lib.RA_OK
    assert lib.ra_add_rows(ptr(0), 64, 60, ptr(1), 64, 0, 4, 8, 128, None) != _lib.RA_OK
    assert count() == before
    # and valid calls do reach their launchers
    assert step(lib) == _lib.RA_OK
    assert lib.ra_add_rows(ptr(0), 64, 0, ptr(1), 64, 0, 4, 8, 128, None) == _lib.RA_OK
    assert count() == before + 2

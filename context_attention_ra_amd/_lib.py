"""ctypes binding of libra.so: the C-ABI entry points under the same names.

Argument marshalling only: shapes are read off the tensors, pointers and the
stream handle are passed through, and a non-OK status raises. Every operation
runs in the library's HIP kernels. If the library is missing the import of an
entry point fails loudly; there is no fallback.
"""

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP = 0, 1, 2, 3
RA_F32, RA_BF16 = 0, 1
RA_MASK_NONE, RA_MASK_CAUSAL = 0, 1
RA_STEP_INIT = 1
RA_BWD_KV_INIT = 2
RA_BWD_NO_DQ = 4
RA_BWD_NO_DKV = 8

# every symbol include/ra.h declares
EXPORTS = ("ra_step", "ra_finalize", "ra_step_final", "ra_step_gqa", "ra_step_final_gqa",
           "ra_bwd_prep", "ra_step_bwd", "ra_copy_rows", "ra_add_rows",
           "ra_merge_lse", "ra_factored_spatial",
           "ra_factored_temporal", "ra_kv_pass", "ra_status_string",
           "ra_last_hip_error", "ra_version")


class RaSegs(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("start", ctypes.c_int64 * 2), ("len", ctypes.c_int64 * 2)]


class RaError(RuntimeError):
    def __init__(self, name, status, hip_error):
        self.status = status
        self.hip_error = hip_error
        super().__init__(f"{name} failed: {status_name(status)} (hipError {hip_error})")


_lib = None

_vp, _i32, _f32, _u32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_uint32, ctypes.c_size_t
_SIGS = {
    "ra_step": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                       ctypes.POINTER(RaSegs), ctypes.POINTER(RaSegs), _i32, _f32, _u32,
                       _vp, _vp, _vp, _vp]),
    "ra_step_gqa": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                           ctypes.POINTER(RaSegs), ctypes.POINTER(RaSegs), _i32, _f32, _u32,
                           _vp, _vp, _vp, _vp]),
    "ra_step_final_gqa": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 ctypes.POINTER(RaSegs), ctypes.POINTER(RaSegs), _i32, _f32, _u32,
                                 _vp, _vp, _vp, _vp, _vp, _vp]),
    "ra_bwd_prep": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "ra_step_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                           ctypes.POINTER(RaSegs), ctypes.POINTER(RaSegs), _i32, _f32, _u32,
                           _vp, _vp, _vp, _vp]),
    "ra_finalize": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp]),
    "ra_step_final": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                             ctypes.POINTER(RaSegs), ctypes.POINTER(RaSegs), _i32, _f32, _u32,
                             _vp, _vp, _vp, _vp, _vp, _vp]),
    "ra_merge_lse": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "ra_factored_spatial": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                   _vp, _vp, _vp]),
    "ra_factored_temporal": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                    _vp, _vp, _vp]),
    "ra_kv_pass": (_i32, [_vp, _vp, _vp, _vp, _sz, _vp]),
    "ra_copy_rows": (_i32, [_vp, ctypes.c_int64, ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int64,
                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp]),
    "ra_add_rows": (_i32, [_vp, ctypes.c_int64, ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int64,
                           ctypes.c_int64, ctypes.c_int64, _i32, _vp]),
    "ra_status_string": (ctypes.c_char_p, [_i32]),
    "ra_last_hip_error": (_i32, []),
    "ra_version": (_i32, []),
}


def load(path: str = LIB_PATH):
    """Load libra.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m context_attention_ra_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load().ra_status_string(status).decode()


def _check(name: str, status: int):
    if status != RA_OK:
        raise RaError(name, status, load().ra_last_hip_error())


def segs(runs: Sequence[Tuple[int, int]]) -> RaSegs:
    """[(global start, length), ...] -> ra_segs (one or two runs)."""
    s = RaSegs()
    s.n = len(runs)
    s.reserved = 0
    for i, (st, n) in enumerate(runs[:2]):
        s.start[i] = int(st)
        s.len[i] = int(n)
    return s


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libra must be contiguous")
    return t.data_ptr()


def _s(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shape(name, t, want):
    if t is not None and tuple(t.shape) != tuple(want):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(want)}")


F32 = torch.float32


def _dtypes(ref, *named):
    """Every tensor must have the dtype the C call assumes.

    The C ABI sees bare pointers and derives every byte count from one dtype
    argument, so a tensor of another dtype would be read or written past its
    end. named: (name, tensor or None, required dtype)."""
    _dtype(ref)
    for name, t, dt in named:
        if t is not None and t.dtype != dt:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dt}")


def _on_gpu(ref, *tensors):
    """Every tensor must sit on `ref`'s GPU: the kernels would take a host
    pointer, or another device's, for one of their own."""
    if ref.device.type != "cuda":
        raise ValueError(f"tensors passed to libra must be on a GPU, got {ref.device}")
    for t in tensors:
        if t is not None and t.device != ref.device:
            raise ValueError(f"tensor on {t.device}, expected {ref.device}")


def _check_step(q, k, v, o_acc, m, l, grouped=True):
    """The sizes the C call derives from q and k must describe every buffer it touches."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, L, d]")
    _dtypes(q, ("k", k, q.dtype), ("v", v, q.dtype), ("o_acc", o_acc, F32), ("m", m, F32), ("l", l, F32))
    B, H, Lq, d = q.shape
    H_kv, Lk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d or H_kv < 1 or H % H_kv != 0 or (not grouped and H_kv != H):
        raise ValueError(f"k: shape {tuple(k.shape)} does not fit q {tuple(q.shape)}")
    _shape("v", v, k.shape)
    _shape("o_acc", o_acc, (B, H, Lq, d))
    _shape("m", m, (B, H, Lq))
    _shape("l", l, (B, H, Lq))


def ra_step(q, k, v, q_segs, kv_segs, causal, scale, o_acc, m, l, init=False, stream=None):
    """ra_step; with fewer K/V heads than query heads (k.shape[1] < q.shape[1]) ra_step_gqa."""
    _check_step(q, k, v, o_acc, m, l)
    _on_gpu(q, k, v, o_acc, m, l)
    B, H, Lq, d = q.shape
    H_kv, Lk = k.shape[1], k.shape[2]
    qs, ks = segs(q_segs), segs(kv_segs)
    args = (ctypes.byref(qs), ctypes.byref(ks), RA_MASK_CAUSAL if causal else RA_MASK_NONE,
            float(scale), RA_STEP_INIT if init else 0, _p(o_acc), _p(m), _p(l), _s(stream))
    if H_kv == H:
        _check("ra_step", load().ra_step(_p(q), _p(k), _p(v), _dtype(q), B, H, Lq, Lk, d, *args))
    else:
        _check("ra_step_gqa", load().ra_step_gqa(_p(q), _p(k), _p(v), _dtype(q), B, H, H_kv, Lq,
                                                 Lk, d, *args))


def ra_step_final(q, k, v, q_segs, kv_segs, causal, scale, o_acc, m, l, out, lse=None,
                  init=False, stream=None):
    """ra_step_final; with fewer K/V heads than query heads ra_step_final_gqa."""
    _check_step(q, k, v, o_acc, m, l)
    _dtypes(q, ("out", out, q.dtype), ("lse", lse, F32))
    _shape("out", out, q.shape)
    _shape("lse", lse, q.shape[:3])
    _on_gpu(q, k, v, o_acc, m, l, out, lse)
    B, H, Lq, d = q.shape
    H_kv, Lk = k.shape[1], k.shape[2]
    qs, ks = segs(q_segs), segs(kv_segs)
    args = (ctypes.byref(qs), ctypes.byref(ks), RA_MASK_CAUSAL if causal else RA_MASK_NONE,
            float(scale), RA_STEP_INIT if init else 0, _p(o_acc), _p(m), _p(l), _p(out),
            _p(lse), _s(stream))
    if H_kv == H:
        _check("ra_step_final", load().ra_step_final(_p(q), _p(k), _p(v), _dtype(q), B, H, Lq,
                                                     Lk, d, *args))
    else:
        _check("ra_step_final_gqa", load().ra_step_final_gqa(_p(q), _p(k), _p(v), _dtype(q), B, H,
                                                             H_kv, Lq, Lk, d, *args))


def ra_bwd_prep(out, dout, delta, stream=None):
    B, H, L, d = out.shape
    _dtypes(out, ("dout", dout, out.dtype), ("delta", delta, F32))
    _shape("dout", dout, out.shape)
    _shape("delta", delta, (B, H, L))
    _on_gpu(out, dout, delta)
    _check("ra_bwd_prep", load().ra_bwd_prep(_p(out), _p(dout), _dtype(out), B, H, L, d, _p(delta),
                                             _s(stream)))


def ra_step_bwd(q, k, v, dout, lse, delta, q_segs, kv_segs, causal, scale, dq, dk, dv,
                init_dq=False, init_dkv=False, stream=None, parts="both"):
    """parts: "both", "dq" (only the dQ kernel) or "dkv" (only the dK/dV kernel)."""
    if parts not in ("both", "dq", "dkv"):
        raise ValueError(f"parts must be 'both', 'dq' or 'dkv', not {parts!r}")
    _check_step(q, k, v, dq, lse, delta)
    _dtypes(q, ("dout", dout, q.dtype), ("dk", dk, F32), ("dv", dv, F32))
    _shape("dout", dout, q.shape)
    _shape("dk", dk, k.shape)
    _shape("dv", dv, k.shape)
    _on_gpu(q, k, v, dout, lse, delta, dq, dk, dv)
    B, H, Lq, d = q.shape
    H_kv, Lk = k.shape[1], k.shape[2]
    qs, ks = segs(q_segs), segs(kv_segs)
    flags = (RA_STEP_INIT if init_dq else 0) | (RA_BWD_KV_INIT if init_dkv else 0)
    flags |= {"both": 0, "dq": RA_BWD_NO_DKV, "dkv": RA_BWD_NO_DQ}[parts]
    _check("ra_step_bwd", load().ra_step_bwd(
        _p(q), _p(k), _p(v), _p(dout), _p(lse), _p(delta), _dtype(q), B, H, H_kv, Lq, Lk, d,
        ctypes.byref(qs), ctypes.byref(ks), RA_MASK_CAUSAL if causal else RA_MASK_NONE,
        float(scale), flags, _p(dq), _p(dk), _p(dv), _s(stream)))


def ra_finalize(o_acc, m, l, out, lse=None, stream=None):
    B, H, L, d = o_acc.shape
    _dtypes(out, ("o_acc", o_acc, F32), ("m", m, F32), ("l", l, F32), ("lse", lse, F32))
    for n, t, want in (("m", m, (B, H, L)), ("l", l, (B, H, L)), ("out", out, o_acc.shape),
                       ("lse", lse, (B, H, L))):
        _shape(n, t, want)
    _on_gpu(o_acc, m, l, out, lse)
    _check("ra_finalize", load().ra_finalize(_p(o_acc), _p(m), _p(l), B, H, L, d, _p(out),
                                             _dtype(out), _p(lse), _s(stream)))


def ra_merge_lse(o_a, lse_a, o_b, lse_b, o_out, lse_out, stream=None):
    B, H, L, d = o_a.shape
    _dtypes(o_a, ("o_b", o_b, o_a.dtype), ("o_out", o_out, o_a.dtype), ("lse_a", lse_a, F32),
            ("lse_b", lse_b, F32), ("lse_out", lse_out, F32))
    for n, t, want in (("o_b", o_b, o_a.shape), ("o_out", o_out, o_a.shape), ("lse_a", lse_a, (B, H, L)),
                       ("lse_b", lse_b, (B, H, L)), ("lse_out", lse_out, (B, H, L))):
        _shape(n, t, want)
    _on_gpu(o_a, lse_a, o_b, lse_b, o_out, lse_out)
    _check("ra_merge_lse", load().ra_merge_lse(_p(o_a), _p(lse_a), _p(o_b), _p(lse_b),
                                               _dtype(o_a), B, H, L, d, _p(o_out),
                                               _p(lse_out), _s(stream)))


def ra_factored_spatial(q, k, v, T, S_sp, scale, out, lse=None, stream=None):
    B, H, N, d = q.shape
    _dtypes(q, ("k", k, q.dtype), ("v", v, q.dtype), ("out", out, q.dtype), ("lse", lse, F32))
    if N != T * S_sp:
        raise ValueError("q.shape[2] must equal T * S_sp")
    for n, t, want in (("k", k, q.shape), ("v", v, q.shape), ("out", out, q.shape), ("lse", lse, (B, H, N))):
        _shape(n, t, want)
    _on_gpu(q, k, v, out, lse)
    _check("ra_factored_spatial", load().ra_factored_spatial(
        _p(q), _p(k), _p(v), _dtype(q), B, H, T, S_sp, d, float(scale), _p(out), _p(lse), _s(stream)))


def ra_factored_temporal(q, k, v, T, S_sp, scale, out, lse=None, stream=None):
    B, H, N, d = q.shape
    _dtypes(q, ("k", k, q.dtype), ("v", v, q.dtype), ("out", out, q.dtype), ("lse", lse, F32))
    if N != T * S_sp:
        raise ValueError("q.shape[2] must equal T * S_sp")
    for n, t, want in (("k", k, q.shape), ("v", v, q.shape), ("out", out, q.shape), ("lse", lse, (B, H, N))):
        _shape(n, t, want)
    _on_gpu(q, k, v, out, lse)
    _check("ra_factored_temporal", load().ra_factored_temporal(
        _p(q), _p(k), _p(v), _dtype(q), B, H, T, S_sp, d, float(scale), _p(out), _p(lse), _s(stream)))


def ra_kv_pass(k_src, v_src, k_dst, v_dst, stream=None):
    nbytes = k_src.numel() * k_src.element_size()
    for t in (v_src, k_dst, v_dst):
        if t.numel() * t.element_size() != nbytes:
            raise ValueError("ra_kv_pass: all four buffers must have the same size")
    _on_gpu(k_src, v_src, k_dst, v_dst)
    _check("ra_kv_pass", load().ra_kv_pass(_p(k_src), _p(v_src), _p(k_dst), _p(v_dst),
                                           nbytes, _s(stream)))


def ra_copy_rows(src, src_row0, dst, dst_row0, nrows, src_slice0=0, dst_slice0=0, nslices=None,
                 stream=None):
    """Rows [src_row0, +nrows) of slices src_slice0.. of a [..., rows, d] tensor into rows
    [dst_row0, +nrows) of slices dst_slice0.. of another (slices = the flattened leading dims)."""
    if src.dtype != dst.dtype or src.shape[-1] != dst.shape[-1]:
        raise ValueError("ra_copy_rows: source and destination need the same dtype and row width")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("tensors passed to libra must be contiguous")
    _on_gpu(src, dst)
    sr, dr = src.shape[-2], dst.shape[-2]
    ns, nd = src.numel() // (sr * src.shape[-1]), dst.numel() // (dr * dst.shape[-1])
    if nslices is None:
        nslices = ns - src_slice0
    if src_slice0 < 0 or dst_slice0 < 0 or src_slice0 + nslices > ns or dst_slice0 + nslices > nd:
        raise ValueError("ra_copy_rows: slice range outside a tensor")
    row_bytes = src.shape[-1] * src.element_size()
    sp = src.data_ptr() + src_slice0 * sr * row_bytes
    dp = dst.data_ptr() + dst_slice0 * dr * row_bytes
    _check("ra_copy_rows", load().ra_copy_rows(sp, sr, src_row0, dp, dr, dst_row0, nslices, nrows,
                                               row_bytes, _s(stream)))


def ra_add_rows(src, src_row0, dst, dst_row0, nrows, src_slice0=0, dst_slice0=0, nslices=None,
                stream=None):
    """dst rows [dst_row0, +nrows) += src rows [src_row0, +nrows) of slices
    src_slice0.. / dst_slice0.. of two fp32 [..., rows, d] tensors."""
    _dtypes(src, ("src", src, F32), ("dst", dst, F32))
    if src.shape[-1] != dst.shape[-1]:
        raise ValueError("ra_add_rows: source and destination need the same row width")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("tensors passed to libra must be contiguous")
    sr, dr, d = src.shape[-2], dst.shape[-2], src.shape[-1]
    ns, nd = src.numel() // (sr * d), dst.numel() // (dr * d)
    if nslices is None:
        nslices = ns - src_slice0
    if src_slice0 < 0 or dst_slice0 < 0 or src_slice0 + nslices > ns or dst_slice0 + nslices > nd:
        raise ValueError("ra_add_rows: slice range outside a tensor")
    _on_gpu(src, dst)
    sp = src.data_ptr() + src_slice0 * sr * d * 4
    dp = dst.data_ptr() + dst_slice0 * dr * d * 4
    _check("ra_add_rows", load().ra_add_rows(sp, sr, src_row0, dp, dr, dst_row0, nslices, nrows, d,
                                             _s(stream)))

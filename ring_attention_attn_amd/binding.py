"""ctypes binding of libringattn.so: the C ABI's calls under the same names.

Argument marshalling only: tensors are passed as device pointers
(``tensor.data_ptr()``) with the caller's current HIP stream; every computation
runs in the library's kernels. A non-RA_OK status raises :class:`RaError`.
Loading fails loudly if the library has not been built (``build()`` in
``__graft_entry__`` or ``python -m ring_attention_attn_amd.build``); there is no
fallback.
"""
import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libringattn.so")

RA_OK, RA_EINVAL, RA_EUNSUPPORTED, RA_EALIGN, RA_EDEVICE = 0, 1, 2, 3, 4
RA_BF16, RA_F32 = 0, 1
RA_MAX_CHUNKS = 32   # include/ring_attn.h

EXPORTS = ("ring_attn_step_fwd", "ring_attn_step_fwd_merge", "ring_attn_fwd_chunks",
           "ring_attn_step_bwd", "ring_attn_bwd_chunks", "lse_merge",
           "ra_bwd_delta",
           "head_permute", "ra_fill_f32", "ra_zigzag_positions", "ra_zigzag_segments",
           "ra_double_ring_order", "ra_validate_step", "ra_status_str")


class RaStepDesc(ctypes.Structure):
    """Mirror of ``ra_step_desc`` in include/ring_attn.h (same field order)."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("q_nseg", ctypes.c_int32), ("k_nseg", ctypes.c_int32),
        ("q_seg_len", ctypes.c_int64), ("k_seg_len", ctypes.c_int64),
        ("q_seg_pos", ctypes.c_int64 * 2), ("k_seg_pos", ctypes.c_int64 * 2),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q_ss", ctypes.c_int64), ("q_hs", ctypes.c_int64),
        ("k_ss", ctypes.c_int64), ("k_hs", ctypes.c_int64),
        ("v_ss", ctypes.c_int64), ("v_hs", ctypes.c_int64),
        ("o_ss", ctypes.c_int64), ("o_hs", ctypes.c_int64),
        ("do_ss", ctypes.c_int64), ("do_hs", ctypes.c_int64),
        ("dk_ss", ctypes.c_int64), ("dk_hs", ctypes.c_int64),
        ("dkv_accumulate", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class RaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


_lib = None


def lib():
    """The loaded library (loads on first use; raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python -m ring_attention_attn_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        pd = ctypes.POINTER(RaStepDesc)
        sig = {
            "ring_attn_step_fwd": [pd, vp, vp, vp, vp, vp, vp],
            "ring_attn_step_fwd_merge": [pd, vp, vp, vp, vp, vp, vp],
            "ring_attn_fwd_chunks": [pd, i32, vp, vp, vp, vp, vp, vp],
            "ring_attn_bwd_chunks": [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "ring_attn_step_bwd": [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "lse_merge": [i64, i32, i32, i64, i64, vp, vp, vp, vp, vp],
            "ra_bwd_delta": [i64, i32, i32, i32, vp, vp, vp, vp, vp],
            "head_permute": [vp, vp, i64, i32, i32, i32, i32, i32, vp],
            "ra_fill_f32": [vp, i64, f32, vp],
            "ra_zigzag_positions": [i64, i32, i32, vp],
            "ra_zigzag_segments": [i64, i32, i32, vp, vp],
            "ra_double_ring_order": [i32, i32, i32, vp],
            "ra_validate_step": [pd, i32],
            "ra_status_str": [i32],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "ra_status_str" else ctypes.c_int
        _lib = L
    return _lib


def status_str(status):
    return lib().ra_status_str(int(status)).decode()


def _check(status, where):
    if status != RA_OK:
        raise RaError(status, where)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensors passed to libringattn must be contiguous "
                         "(layouts are given by the descriptor's strides, not the tensor's)")
    return x.data_ptr()


def _extent(rows, heads, ss, hs, d, eb):
    """Bytes from the base pointer that a [rows][heads][d] tensor with element
    strides (ss, hs) spans."""
    if rows <= 0 or heads <= 0:
        return 0
    return ((rows - 1) * ss + (heads - 1) * hs + d) * eb


def _arg(x, name, nbytes, dtype=None, elem_bytes=None):
    """Check a tensor argument before its pointer reaches a kernel: on the GPU,
    of the expected dtype ("bf16" / "f32") or element size, holding at least
    ``nbytes`` from its data pointer. Raw integer pointers pass unchecked."""
    if x is None or isinstance(x, int) or nbytes <= 0:
        return
    import torch
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {x.device})")
    if dtype is not None:
        want = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
        if x.dtype != want:
            raise ValueError(f"{name} must be {want} (got {x.dtype})")
    if elem_bytes is not None and x.element_size() != elem_bytes:
        raise ValueError(f"{name} must have {elem_bytes}-byte elements (got {x.dtype})")
    have = x.untyped_storage().nbytes() - x.storage_offset() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: the call addresses {nbytes} bytes from its data pointer, "
                         f"the tensor holds {have}")


def _step_args(desc, for_bwd, q, k, v, o, lse, dout=None, delta=None, dk=None, dv=None):
    """Tensor checks of the step calls, done only for a descriptor the library
    accepts (an invalid one is left to the library's own status)."""
    if lib().ra_validate_step(ctypes.byref(desc), int(for_bwd)) != RA_OK:
        return
    dt = "bf16" if desc.dtype == RA_BF16 else "f32"
    eb = 2 if dt == "bf16" else 4
    D, lq, lk = desc.head_dim, desc.q_nseg * desc.q_seg_len, desc.k_nseg * desc.k_seg_len
    _arg(q, "q", _extent(lq, desc.hq, desc.q_ss, desc.q_hs, D, eb), dt)
    _arg(k, "k", _extent(lk, desc.hkv, desc.k_ss, desc.k_hs, D, eb), dt)
    _arg(v, "v", _extent(lk, desc.hkv, desc.v_ss, desc.v_hs, D, eb), dt)
    _arg(o, "o", _extent(lq, desc.hq, desc.o_ss, desc.o_hs, D, 4), "f32")
    _arg(lse, "lse", desc.hq * lq * 4, "f32")
    if for_bwd:
        _arg(dout, "dout", _extent(lq, desc.hq, desc.do_ss, desc.do_hs, D, eb), dt)
        _arg(delta, "delta", desc.hq * lq * 4, "f32")
        _arg(dk, "dk_acc", _extent(lk, desc.hkv, desc.dk_ss, desc.dk_hs, D, 4), "f32")
        _arg(dv, "dv_acc", _extent(lk, desc.hkv, desc.dk_ss, desc.dk_hs, D, 4), "f32")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- device calls

def ring_attn_step_fwd(desc, q, k, v, o_step, lse_step, stream=None):
    _step_args(desc, 0, q, k, v, o_step, lse_step)
    _check(lib().ring_attn_step_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o_step),
                                    _ptr(lse_step), _stream(stream)), "ring_attn_step_fwd")


def ring_attn_step_fwd_merge(desc, q, k, v, o_acc, lse_acc, stream=None):
    _step_args(desc, 0, q, k, v, o_acc, lse_acc)
    _check(lib().ring_attn_step_fwd_merge(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(o_acc), _ptr(lse_acc), _stream(stream)),
           "ring_attn_step_fwd_merge")


def ring_attn_fwd_chunks(descs, q, ks, vs, o, lse, stream=None):
    """All ring steps of the forward in one launch: descs, ks, vs are sequences
    (chunk i's descriptor, K and V); o, lse are written."""
    n = len(descs)
    if len(ks) != n or len(vs) != n:
        raise ValueError("ring_attn_fwd_chunks: descs, ks and vs must have the same length")
    arr = (RaStepDesc * max(n, 1))(*descs)
    for d, k, v in zip(descs, ks, vs):
        _step_args(d, 0, q, k, v, o, lse)
    kp = (ctypes.c_void_p * max(n, 1))(*[_ptr(k) for k in ks])
    vp_ = (ctypes.c_void_p * max(n, 1))(*[_ptr(v) for v in vs])
    _check(lib().ring_attn_fwd_chunks(arr, n, _ptr(q), kp, vp_, _ptr(o), _ptr(lse),
                                      _stream(stream)), "ring_attn_fwd_chunks")


def ring_attn_bwd_chunks(descs, q, ks, vs, dout, lse, delta, dq, dks, dvs, stream=None):
    """All ring steps of the backward: descs, ks, vs, dks, dvs are sequences
    (chunk i's descriptor, K, V, dK, dV); dq is written."""
    n = len(descs)
    if not (len(ks) == len(vs) == len(dks) == len(dvs) == n):
        raise ValueError("ring_attn_bwd_chunks: descs, ks, vs, dks and dvs must have the same length")
    arr = (RaStepDesc * max(n, 1))(*descs)
    for d, k, v, dk, dv in zip(descs, ks, vs, dks, dvs):
        _step_args(d, 1, q, k, v, dq, lse, dout, delta, dk, dv)

    def parr(xs):
        return (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in xs])
    _check(lib().ring_attn_bwd_chunks(arr, n, _ptr(q), parr(ks), parr(vs), _ptr(dout), _ptr(lse),
                                      _ptr(delta), _ptr(dq), parr(dks), parr(dvs),
                                      _stream(stream)), "ring_attn_bwd_chunks")


def ring_attn_step_bwd(desc, q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, stream=None):
    _step_args(desc, 1, q, k, v, dq_acc, lse, dout, delta, dk_acc, dv_acc)
    _check(lib().ring_attn_step_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                    _ptr(lse), _ptr(delta), _ptr(dq_acc), _ptr(dk_acc),
                                    _ptr(dv_acc), _stream(stream)), "ring_attn_step_bwd")


def lse_merge(rows, hq, head_dim, o_acc, lse_acc, o_step, lse_step, stream=None, row_begin=0,
              row_count=None):
    """Merge rows [row_begin, row_begin + row_count) (default: all rows)."""
    if row_count is None:
        row_count = rows - row_begin
    if rows > 0 and hq > 0:
        for x, name, n in ((o_acc, "o_acc", rows * hq * head_dim), (o_step, "o_step", rows * hq * head_dim),
                           (lse_acc, "lse_acc", hq * rows), (lse_step, "lse_step", hq * rows)):
            _arg(x, name, 4 * n, "f32")
    _check(lib().lse_merge(rows, hq, head_dim, row_begin, row_count, _ptr(o_acc), _ptr(lse_acc),
                           _ptr(o_step), _ptr(lse_step), _stream(stream)), "lse_merge")


def ra_bwd_delta(rows, hq, head_dim, dtype, o, dout, delta, o_out=None, stream=None):
    if rows > 0 and hq > 0 and dtype in (RA_BF16, RA_F32):
        n = rows * hq * head_dim
        _arg(o, "o", 4 * n, "f32")
        _arg(dout, "dout", (2 if dtype == RA_BF16 else 4) * n, "bf16" if dtype == RA_BF16 else "f32")
        _arg(delta, "delta", 4 * hq * rows, "f32")
        _arg(o_out, "o_out", 2 * n, "bf16")
    _check(lib().ra_bwd_delta(rows, hq, head_dim, dtype, _ptr(o), _ptr(dout), _ptr(delta),
                              _ptr(o_out), _stream(stream)), "ra_bwd_delta")


def head_permute(src, dst, s, h, d, p, elem_bytes, inverse=0, stream=None):
    if s > 0 and h > 0 and d > 0 and elem_bytes in (2, 4):  # a bit copy: any dtype of that size
        _arg(src, "src", s * h * d * elem_bytes, elem_bytes=elem_bytes)
        _arg(dst, "dst", s * h * d * elem_bytes, elem_bytes=elem_bytes)
    _check(lib().head_permute(_ptr(src), _ptr(dst), s, h, d, p, elem_bytes, int(inverse),
                              _stream(stream)), "head_permute")


def ra_fill_f32(dst, n, value, stream=None):
    _arg(dst, "dst", 4 * n, "f32")
    _check(lib().ra_fill_f32(_ptr(dst), n, float(value), _stream(stream)), "ra_fill_f32")


# ---------------------------------------------------------------- host helpers

def ra_zigzag_positions(S, P, rank):
    b = S // (2 * P) if P > 0 else 0
    out = np.zeros(max(2 * b, 1), dtype=np.int64)
    _check(lib().ra_zigzag_positions(S, P, rank, out.ctypes.data), "ra_zigzag_positions")
    return out[:2 * b]


def ra_zigzag_segments(S, P, rank):
    pos = np.zeros(2, dtype=np.int64)
    ln = np.zeros(1, dtype=np.int64)
    _check(lib().ra_zigzag_segments(S, P, rank, pos.ctypes.data, ln.ctypes.data),
           "ra_zigzag_segments")
    return (int(pos[0]), int(pos[1])), int(ln[0])


def ra_double_ring_order(inner, outer, rank):
    out = np.zeros(max(inner * outer, 1), dtype=np.int32)
    _check(lib().ra_double_ring_order(inner, outer, rank, out.ctypes.data), "ra_double_ring_order")
    return out[:inner * outer]


def ra_validate_step(desc, for_bwd=0):
    return lib().ra_validate_step(ctypes.byref(desc), int(for_bwd))


def make_desc(*, dtype, head_dim, hq, hkv, q_segments, k_segments, scale, causal=1,
              q_strides, k_strides, v_strides, o_strides, do_strides=(0, 0), dk_strides=(0, 0),
              dkv_accumulate=0):
    """Fill a :class:`RaStepDesc`. ``*_segments`` = ((pos0[, pos1]), seg_len);
    ``*_strides`` = (seq stride, head stride) in elements."""
    d = RaStepDesc()
    d.dtype, d.head_dim, d.hq, d.hkv = dtype, head_dim, hq, hkv
    (qp, ql), (kp, kl) = q_segments, k_segments
    d.q_nseg, d.k_nseg = len(qp), len(kp)
    d.q_seg_len, d.k_seg_len = ql, kl
    for i, x in enumerate(qp):
        d.q_seg_pos[i] = x
    for i, x in enumerate(kp):
        d.k_seg_pos[i] = x
    d.causal, d.scale = causal, scale
    d.q_ss, d.q_hs = q_strides
    d.k_ss, d.k_hs = k_strides
    d.v_ss, d.v_hs = v_strides
    d.o_ss, d.o_hs = o_strides
    d.do_ss, d.do_hs = do_strides
    d.dk_ss, d.dk_hs = dk_strides
    d.dkv_accumulate = dkv_accumulate
    return d

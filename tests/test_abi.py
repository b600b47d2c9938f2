"""The C ABI without a GPU: the library loads, exports every function that
include/ring_attn.h declares, its host index maps equal the oracle's bit for
bit, and invalid arguments are rejected with the documented codes before any
device work."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from ring_attention_attn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libringattn.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    L = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_struct_layout_matches_header_sizes():
    # 6 int32 + 2 int64 + 4 int64 + (int32, float) + 12 int64 + 2 int32
    assert ctypes.sizeof(B.RaStepDesc) == 6 * 4 + 2 * 8 + 4 * 8 + 8 + 12 * 8 + 8


@pytest.mark.parametrize("S,P", [(512, 4), (96, 3), (131072, 8), (1 << 20, 16), (524288, 32)])
def test_zigzag_positions_bit_exact(S, P):
    for r in sorted({0, 1, P // 2, P - 1}):
        np.testing.assert_array_equal(B.ra_zigzag_positions(S, P, r), oracle.zigzag_positions(S, P, r))
        (p0, p1), b = B.ra_zigzag_segments(S, P, r)
        assert (p0, p1, b) == (r * b, (2 * P - 1 - r) * b, S // (2 * P))


@pytest.mark.parametrize("inner,outer", [(4, 1), (8, 1), (4, 4), (8, 4), (3, 5), (1, 7)])
def test_double_ring_order_bit_exact(inner, outer):
    for r in range(inner * outer):
        np.testing.assert_array_equal(B.ra_double_ring_order(inner, outer, r),
                                      oracle.double_ring_order(inner, outer, r))


def test_index_map_errors():
    for args in [(100, 8, 0), (512, 4, 4), (512, 0, 0), (512, 4, -1)]:
        with pytest.raises(B.RaError) as e:
            B.ra_zigzag_positions(*args)
        assert e.value.status == B.RA_EINVAL
    with pytest.raises(B.RaError):
        B.ra_double_ring_order(0, 4, 0)
    with pytest.raises(B.RaError):
        B.ra_double_ring_order(4, 2, 8)


def good_desc(**kw):
    args = dict(dtype=B.RA_BF16, head_dim=128, hq=8, hkv=2, q_segments=((0, 448), 64),
                k_segments=((64, 384), 64), scale=1 / math.sqrt(128), q_strides=(1024, 128),
                k_strides=(256, 128), v_strides=(256, 128), o_strides=(1024, 128),
                do_strides=(1024, 128), dk_strides=(256, 128))
    args.update(kw)
    return B.make_desc(**args)


def test_validation_accepts_good_descriptor():
    assert B.ra_validate_step(good_desc(), 0) == B.RA_OK
    assert B.ra_validate_step(good_desc(), 1) == B.RA_OK
    # head-major layout is a valid nesting too
    assert B.ra_validate_step(good_desc(q_strides=(128, 128 * 128), o_strides=(128, 128 * 128)), 0) == B.RA_OK
    # padded strides in either nesting; any head stride
    assert B.ra_validate_step(good_desc(q_strides=(1024 + 64, 128)), 0) == B.RA_OK
    assert B.ra_validate_step(good_desc(q_strides=(128, 2**62)), 0) == B.RA_OK
    # the largest row stride whose 64-row tile stays within 32-bit byte offsets
    big = 2**31 // 128 - 256
    assert B.ra_validate_step(good_desc(q_strides=(big, 128)), 0) == B.RA_OK
    assert B.ra_validate_step(good_desc(q_strides=(big + 8, 128)), 0) == B.RA_EUNSUPPORTED
    assert B.ra_validate_step(good_desc(q_strides=(2**62, 128)), 0) == B.RA_EUNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), B.RA_EUNSUPPORTED),
    (dict(dtype=7), B.RA_EINVAL),
    (dict(hq=6, hkv=4), B.RA_EINVAL),
    (dict(hkv=0), B.RA_EINVAL),
    (dict(q_segments=((0, 1, 2), 64)), None),       # 3 segments: rejected by make_desc
    (dict(k_segments=((0, 448), -1)), B.RA_EINVAL),
    (dict(scale=float("nan")), B.RA_EINVAL),
    (dict(scale=-0.1), B.RA_EINVAL),
    (dict(scale=0.0), B.RA_EINVAL),
    (dict(causal=2), B.RA_EINVAL),
    (dict(q_strides=(1024, 100)), B.RA_EINVAL),     # heads overlap (head stride < d)
    (dict(q_strides=(1028, 128)), B.RA_EALIGN),     # rows not 16-byte aligned
    (dict(o_strides=(1026, 128)), B.RA_EALIGN),
    (dict(q_strides=(512, 128)), B.RA_EINVAL),      # rows overlap heads
    (dict(q_strides=(2**60, 2**58)), B.RA_EINVAL),  # overlap; rows * ss would overflow int64
])
def test_validation_rejects(kw, code):
    if code is None:
        with pytest.raises(IndexError):
            good_desc(**kw)
        return
    assert B.ra_validate_step(good_desc(**kw), 0) == code


def test_backward_stride_checks():
    assert B.ra_validate_step(good_desc(do_strides=(1024, 3)), 1) == B.RA_EINVAL
    assert B.ra_validate_step(good_desc(dk_strides=(258, 128)), 1) == B.RA_EALIGN
    # the forward ignores backward-only strides
    assert B.ra_validate_step(good_desc(do_strides=(1024, 3)), 0) == B.RA_OK


def test_calls_reject_before_device_work():
    """Invalid arguments come back as status codes without touching a device."""
    d = good_desc(head_dim=96)
    with pytest.raises(B.RaError) as e:
        B.ring_attn_step_fwd(d, 16, 16, 16, 16, 16, stream=0)
    assert e.value.status == B.RA_EUNSUPPORTED
    with pytest.raises(B.RaError) as e:
        B.ring_attn_step_fwd(good_desc(), 0, 16, 16, 16, 16, stream=0)   # null q
    assert e.value.status == B.RA_EINVAL
    with pytest.raises(B.RaError) as e:
        B.ring_attn_step_fwd(good_desc(), 8, 16, 16, 16, 16, stream=0)   # misaligned q
    assert e.value.status == B.RA_EALIGN
    with pytest.raises(B.RaError) as e:
        B.ring_attn_step_bwd(good_desc(), 16, 16, 16, 0, 16, 16, 16, 16, 16, stream=0)
    assert e.value.status == B.RA_EINVAL
    for args, code in [((d, 16, 16, 16, 16, 16), B.RA_EUNSUPPORTED),
                       ((good_desc(), 16, 16, 16, 0, 16), B.RA_EINVAL),      # null o_acc
                       ((good_desc(), 16, 16, 16, 16, 8), B.RA_EALIGN)]:     # misaligned lse_acc
        with pytest.raises(B.RaError) as e:
            B.ring_attn_step_fwd_merge(*args, stream=0)
        assert e.value.status == code
    for call, code in [
        (lambda: B.lse_merge(-1, 4, 128, 16, 16, 16, 16, stream=0), B.RA_EINVAL),
        (lambda: B.lse_merge(8, 4, 80, 16, 16, 16, 16, stream=0), B.RA_EUNSUPPORTED),
        (lambda: B.lse_merge(1 << 28, 32, 128, 16, 16, 16, 16, stream=0), B.RA_EUNSUPPORTED),
        (lambda: B.lse_merge(8, 4, 128, 16, 16, 16, 8, stream=0), B.RA_EALIGN),
        (lambda: B.lse_merge(8, 4, 128, 16, 16, 16, 16, stream=0, row_begin=-1), B.RA_EINVAL),
        (lambda: B.lse_merge(8, 4, 128, 16, 16, 16, 16, stream=0, row_begin=4, row_count=5),
         B.RA_EINVAL),                                                   # past the last row
        (lambda: B.ra_bwd_delta(8, 4, 128, 5, 16, 16, 16, stream=0), B.RA_EINVAL),
        (lambda: B.ra_bwd_delta(1 << 28, 32, 128, B.RA_BF16, 16, 16, 16, stream=0),
         B.RA_EUNSUPPORTED),
        (lambda: B.head_permute(16, 4096, 8, 6, 128, 4, 2, stream=0), B.RA_EINVAL),   # H % P
        (lambda: B.head_permute(16, 4096, 8, 8, 4, 8, 2, stream=0), B.RA_EALIGN),     # 8-byte runs
        (lambda: B.head_permute(16, 32, 8, 8, 128, 4, 2, stream=0), B.RA_EINVAL),     # overlap
        (lambda: B.head_permute(16, 1 << 20, 8, 8, 128, 4, 3, stream=0), B.RA_EINVAL),
        (lambda: B.head_permute(16, 1 << 30, 8, 65536, 8, 65536, 2, stream=0),     # p > 65535
         B.RA_EUNSUPPORTED),
        (lambda: B.ra_fill_f32(8, 10, 0.0, stream=0), B.RA_EALIGN),
        (lambda: B.ra_fill_f32(16, -1, 0.0, stream=0), B.RA_EINVAL),
    ]:
        with pytest.raises(B.RaError) as e:
            call()
        assert e.value.status == code


def test_zero_size_calls_are_noops():
    B.lse_merge(0, 4, 128, 0, 0, 0, 0, stream=0)
    B.lse_merge(8, 4, 128, 0, 0, 0, 0, stream=0, row_begin=8, row_count=0)
    B.ra_fill_f32(0, 0, 1.0, stream=0)
    B.head_permute(0, 0, 0, 8, 128, 4, 2, stream=0)
    B.ring_attn_step_fwd(good_desc(q_segments=((0, 448), 0)), 0, 0, 0, 0, 0, stream=0)
    B.ring_attn_step_fwd_merge(good_desc(k_segments=((0, 448), 0)), 0, 0, 0, 0, 0, stream=0)
    B.ring_attn_step_bwd(good_desc(k_segments=((0, 448), 0)), 0, 0, 0, 0, 0, 0, 0, 0, 0, stream=0)


def test_status_strings():
    for s in range(5):
        assert B.status_str(s).startswith("RA_")


def test_binding_rejects_non_contiguous_tensors():
    import torch
    t = torch.zeros((4, 6)).t()
    with pytest.raises(ValueError):
        B._ptr(t)
    assert B._ptr(torch.zeros(4)) != 0


def test_binding_rejects_host_tensors():
    """A host tensor never reaches a kernel: the binding refuses it before the call."""
    import torch
    d = good_desc()
    q = torch.zeros((128, 8, 128), dtype=torch.bfloat16)
    k = torch.zeros((128, 2, 128), dtype=torch.bfloat16)
    o = torch.zeros((128, 8, 128))
    lse = torch.zeros((8, 128))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.ring_attn_step_fwd(d, q, k, k, o, lse, stream=0)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.ring_attn_step_fwd_merge(d, q, k, k, o, lse, stream=0)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.ra_fill_f32(o, o.numel(), 0.0, stream=0)
    # an invalid descriptor is reported by the library's own status, as before
    with pytest.raises(B.RaError) as e:
        B.ring_attn_step_fwd(good_desc(head_dim=96), q, k, k, o, lse, stream=0)
    assert e.value.status == B.RA_EUNSUPPORTED


@pytest.mark.parametrize("layout,S,inner,outer,r", [("zigzag", 512, 4, 1, 1), ("zigzag", 4096, 4, 2, 6),
                                                     ("contiguous", 512, 4, 1, 2)])
@pytest.mark.parametrize("kv_rings", ["one", "ab"])
def test_ring_merge_rows_are_the_rows_that_see_a_key(layout, S, inner, outer, r, kv_rings):
    """The separate merge's row range of each launch: exactly the query rows
    with a visible key in the launch's key set (host logic of the ring driver)."""
    from ring_attention_attn_amd.ring import ShareRing
    if layout == "contiguous" and kv_rings == "ab":
        return
    P = inner * outer
    ring = ShareRing(S, inner, outer, r, 1, 1, 64, "f32", device="cpu", merge="separate",
                     layout=layout, kv_rings=kv_rings)
    posf = oracle.zigzag_positions if layout == "zigzag" else oracle.contiguous_positions
    pos_q = posf(S, P, r)
    for j, off, desc in ring.launches:
        pos_k = posf(S, P, j)
        n = desc.k_nseg * desc.k_seg_len
        pos_k = pos_k[off:off + n]
        sees = (pos_q[:, None] >= pos_k[None, :]).any(axis=1)
        r0, cnt = ring.merge_rows(desc)
        want = np.zeros(len(pos_q), bool)
        want[r0:r0 + cnt] = True
        assert np.array_equal(sees, want), (j, off)


def test_fwd_chunks_rejects_before_device_work():
    """The one-launch forward of all ring steps: argument errors come back as
    status codes with no device work."""
    g = good_desc()

    def call(descs, ks=None, vs=None, q=16, o=16, lse=16):
        n = len(descs)
        ks = [16] * n if ks is None else ks
        vs = [16] * n if vs is None else vs
        with pytest.raises(B.RaError) as e:
            B.ring_attn_fwd_chunks(descs, q, ks, vs, o, lse, stream=0)
        return e.value.status

    assert call([]) == B.RA_EINVAL                                   # no chunk
    assert call([g] * 33) == B.RA_EUNSUPPORTED                       # more than 32 chunks
    assert call([g, good_desc(hq=4)]) == B.RA_EINVAL                 # query side differs
    assert call([g, good_desc(q_segments=((64, 448), 64))]) == B.RA_EINVAL
    assert call([g, good_desc(k_strides=(384, 128))]) == B.RA_EINVAL  # K strides differ
    assert call([g, good_desc(head_dim=96)]) == B.RA_EUNSUPPORTED    # invalid chunk
    f32 = dict(dtype=B.RA_F32)
    assert call([good_desc(**f32), good_desc(**f32)]) == B.RA_EUNSUPPORTED  # bf16 only
    assert call([g], q=0) == B.RA_EINVAL                             # null q
    assert call([g], o=8) == B.RA_EALIGN                             # misaligned o
    assert call([g, g], ks=[16, 0]) == B.RA_EINVAL                   # null K of a chunk
    assert call([g, g], vs=[16, 24]) == B.RA_EALIGN                  # misaligned V of a chunk
    with pytest.raises(ValueError):
        B.ring_attn_fwd_chunks([g, g], 16, [16], [16, 16], 16, 16, stream=0)


def test_bwd_chunks_rejects_before_device_work():
    """The backward of all ring steps in one call: argument errors come back as
    status codes with no device work."""
    g = good_desc()

    def call(descs, ks=None, vs=None, dks=None, dvs=None, q=16, dout=16, dq=16):
        n = len(descs)
        f = lambda x: [16] * n if x is None else x
        with pytest.raises(B.RaError) as e:
            B.ring_attn_bwd_chunks(descs, q, f(ks), f(vs), dout, 16, 16, dq, f(dks), f(dvs),
                                   stream=0)
        return e.value.status

    assert call([]) == B.RA_EINVAL
    assert call([g] * 33) == B.RA_EUNSUPPORTED
    assert call([g, good_desc(hkv=4)]) == B.RA_EINVAL                 # query side differs
    assert call([g, good_desc(do_strides=(2048, 128))]) == B.RA_EINVAL  # dout strides differ
    assert call([g, good_desc(dk_strides=(384, 128))]) == B.RA_EINVAL   # dK strides differ
    f32 = dict(dtype=B.RA_F32)
    assert call([good_desc(**f32)]) == B.RA_EUNSUPPORTED               # bf16 only
    assert call([g], dout=0) == B.RA_EINVAL
    assert call([g], dq=8) == B.RA_EALIGN
    assert call([g, g], dks=[16, 0]) == B.RA_EINVAL                    # null dK of a chunk
    assert call([g, g], dvs=[16, 40]) == B.RA_EALIGN
    with pytest.raises(ValueError):
        B.ring_attn_bwd_chunks([g, g], 16, [16, 16], [16, 16], 16, 16, 16, 16, [16], [16, 16],
                               stream=0)


def test_chunk_limit_constant_and_driver_check():
    """The binding's RA_MAX_CHUNKS is the header's; the ring driver refuses a
    chunks-mode ring with more launches than one call takes (32 chunks as
    block A / block B rings are 64 launches), and accepts 32."""
    from ring_attention_attn_amd.ring import ShareRing
    m = re.search(r"#define\s+RA_MAX_CHUNKS\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == B.RA_MAX_CHUNKS
    with pytest.raises(ValueError, match="at most 32"):
        ShareRing(2048, 32, 1, 0, 1, 1, 64, "bf16", device="cpu", merge="chunks", kv_rings="ab")
    ring = ShareRing(2048, 32, 1, 0, 1, 1, 64, "bf16", device="cpu", merge="chunks")
    assert len(ring.launches) == 32
    # a call with one descriptor more than the limit is refused before device work
    with pytest.raises(B.RaError) as e:
        B.ring_attn_fwd_chunks([good_desc()] * (B.RA_MAX_CHUNKS + 1), 16, [16] * 33, [16] * 33,
                               16, 16, stream=0)
    assert e.value.status == B.RA_EUNSUPPORTED

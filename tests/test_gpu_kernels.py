"""Kernel-level parity on the GPU: each C-ABI call against the fp64 oracle on
the same seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles and ragged tails."""
import math

import numpy as np
import pytest

import oracle
from ring_attention_attn_amd import synth
from tests.helpers import share_inputs, widen, to_device, assert_close, max_abs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ring_attention_attn_amd import binding
    binding.lib()
    yield
    torch.cuda.synchronize()


def B():
    from ring_attention_attn_amd import binding
    return binding


# ------------------------------------------------------------------ guard bands
# Every output of a call under test sits inside a larger buffer, with guard
# bands of a fixed bit pattern before and after it; a write past either end of
# an output changes a band.
GUARD = 4096                       # elements on each side
_PATTERN = {torch.float32: (torch.int32, 0x5A5A5A5A), torch.bfloat16: (torch.int16, 0x5A5A),
            torch.int16: (torch.int16, 0x5A5A), torch.int32: (torch.int32, 0x5A5A5A5A)}
_guarded = []                      # (buffer, n) of the current test


def guarded(shape, dtype=torch.float32, fill=float("nan")):
    """A contiguous tensor of ``shape`` between two guard bands."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda")
    idt, pat = _PATTERN[dtype]
    buf.view(idt).fill_(pat)
    t = buf[GUARD:GUARD + n].view(shape)
    if fill is not None:
        t.fill_(fill)
    _guarded.append((buf, n))
    return t


def check_guards():
    torch.cuda.synchronize()
    for buf, n in _guarded:
        idt, pat = _PATTERN[buf.dtype]
        ib = buf.view(idt)
        assert bool((ib[:GUARD] == pat).all()), "write before the start of an output"
        assert bool((ib[GUARD + n:] == pat).all()), "write past the end of an output"
    _guarded.clear()


@pytest.fixture(autouse=True)
def _guards_checked():
    _guarded.clear()
    yield
    check_guards()


# ------------------------------------------------------------------ head permute

@pytest.mark.parametrize("s,h,d,p,eb", [(37, 8, 128, 4, 2), (64, 32, 128, 4, 2), (5, 6, 16, 3, 4),
                                        (100, 8, 64, 8, 2), (16, 4, 128, 1, 2),
                                        (97, 9, 16, 3, 2),     # 6-vector runs: 42 runs per block
                                        (3, 32, 128, 1, 4)])   # 1024-vector runs: a block loops
def test_head_permute_bit_exact(s, h, d, p, eb):
    rng = np.random.default_rng(s + h)
    dt = np.uint16 if eb == 2 else np.uint32
    x = rng.integers(0, np.iinfo(dt).max, size=(s, h, d), dtype=dt)
    tdt = torch.int16 if eb == 2 else torch.int32
    src = torch.from_numpy(x.view(np.int16 if eb == 2 else np.int32)).cuda()
    dst = guarded((p, s, h // p, d), tdt, fill=None)
    B().head_permute(src, dst, s, h, d, p, eb, 0)
    back = guarded((s, h, d), tdt, fill=None)
    B().head_permute(dst, back, s, h, d, p, eb, 1)
    torch.cuda.synchronize()
    want = oracle.head_permute(x, p)
    assert np.array_equal(dst.cpu().numpy().view(dt), want)
    assert np.array_equal(back.cpu().numpy().view(dt), x)


def test_head_permute_full_size_2d_attention_share():
    """The 2D-Attention share's permute: 65,536 tokens x 32 heads x 128 bf16 into
    4 head groups (and back), bit-exact."""
    s, h, d, p = 65536, 32, 128, 4
    x = synth.blocks_tensor(1003, synth.T_Q, [0], s, h, d, "bf16")
    src = torch.from_numpy(x.view(np.int16)).cuda()
    dst = torch.empty((p, s, h // p, d), dtype=torch.int16, device="cuda")
    B().head_permute(src, dst, s, h, d, p, 2, 0)
    back = torch.empty_like(src)
    B().head_permute(dst, back, s, h, d, p, 2, 1)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint16), oracle.head_permute(x, p))
    assert torch.equal(back, src)


# ------------------------------------------------------------------ merge / delta / fill

@pytest.mark.parametrize("rows,hq,d", [(37, 3, 128), (256, 8, 64), (1, 1, 128)])
def test_lse_merge(rows, hq, d):
    rng = np.random.default_rng(rows)
    oa = rng.standard_normal((rows, hq, d)).astype(np.float32)
    os_ = rng.standard_normal((rows, hq, d)).astype(np.float32)
    la = (rng.standard_normal((hq, rows)) * 3).astype(np.float32)
    ls = (rng.standard_normal((hq, rows)) * 3).astype(np.float32)
    # empty rows: one side, the other side, both
    la[:, ::5] = -np.inf
    ls[:, ::7] = -np.inf
    oa[::5] = 0.0
    os_[::7] = 0.0
    want_o, want_l = oracle.lse_merge(oa, la, os_, ls)
    t = [torch.from_numpy(a.copy()).cuda() for a in (oa, la, os_, ls)]
    for i in (0, 1):
        g = guarded(t[i].shape, fill=None)
        g.copy_(t[i])
        t[i] = g
    B().lse_merge(rows, hq, d, t[0], t[1], t[2], t[3])
    torch.cuda.synchronize()
    got_o, got_l = t[0].cpu().numpy(), t[1].cpu().numpy()
    assert not np.isnan(got_o).any() and not np.isnan(got_l).any()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l))
    assert max_abs(got_o, want_o) < 2e-6
    assert max_abs(got_l, want_l) < 2e-6


def test_lse_merge_row_range():
    """Only rows [row_begin, row_begin + row_count) are merged; every other row
    of O and LSE keeps its bits."""
    rows, hq, d, r0, n = 300, 4, 128, 117, 90
    rng = np.random.default_rng(5)
    oa, os_ = (rng.standard_normal((rows, hq, d)).astype(np.float32) for _ in range(2))
    la, ls = ((rng.standard_normal((hq, rows)) * 2).astype(np.float32) for _ in range(2))
    want_o, want_l = oracle.lse_merge(oa, la, os_, ls)
    to, tl = guarded((rows, hq, d), fill=None), guarded((hq, rows), fill=None)
    to.copy_(torch.from_numpy(oa))
    tl.copy_(torch.from_numpy(la))
    B().lse_merge(rows, hq, d, to, tl, torch.from_numpy(os_).cuda(), torch.from_numpy(ls).cuda(),
                  row_begin=r0, row_count=n)
    torch.cuda.synchronize()
    go, gl = to.cpu().numpy(), tl.cpu().numpy()
    inside = slice(r0, r0 + n)
    assert max_abs(go[inside], want_o[inside]) < 2e-6
    assert max_abs(gl[:, inside], want_l[:, inside]) < 2e-6
    for outside in (slice(0, r0), slice(r0 + n, rows)):
        assert np.array_equal(go[outside], oa[outside])
        assert np.array_equal(gl[:, outside], la[:, outside])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_bwd_delta_and_cast(dtype, d):
    rows, hq = 301, 5
    rng = np.random.default_rng(d)
    o = rng.standard_normal((rows, hq, d)).astype(np.float32)
    g = synth.blocks_tensor(9, synth.T_DO, [0], rows, hq, d, dtype)
    want = np.einsum("lhd,lhd->hl", widen(g, dtype), o.astype(np.float64))
    to = torch.from_numpy(o).cuda()
    tg = to_device(g, dtype)
    delta = guarded((hq, rows))
    ob = guarded((rows, hq, d), torch.bfloat16)
    B().ra_bwd_delta(rows, hq, d, B().RA_BF16 if dtype == "bf16" else B().RA_F32, to, tg, delta, ob)
    torch.cuda.synchronize()
    assert max_abs(delta.cpu().numpy(), want) < 1e-4
    ref_bits = synth.f32_to_bf16_bits(o)
    assert np.array_equal(ob.cpu().view(torch.int16).numpy().view(np.uint16), ref_bits)


def test_fill():
    x = guarded((1000003,))
    B().ra_fill_f32(x, x.numel(), -2.5)
    torch.cuda.synchronize()
    assert bool((x == -2.5).all())


# ------------------------------------------------------------------ step forward / backward

STEP_CASES = [
    # dtype, d, hq, hkv, b, P, r, causal
    ("bf16", 128, 8, 2, 200, 4, 1, 1),    # GQA 4, ragged rows (400 local rows)
    ("bf16", 64, 4, 4, 96, 3, 2, 1),      # MHA, d=64
    ("bf16", 128, 8, 1, 256, 2, 0, 1),    # GQA 8
    ("bf16", 128, 4, 2, 130, 2, 1, 1),    # GQA 2, tiles crossing the segment boundary
    ("bf16", 128, 4, 1, 72, 2, 0, 0),     # non-causal
    ("bf16", 128, 6, 2, 130, 2, 1, 1),    # GQA 3 (one head per row block), ragged
    ("bf16", 64, 8, 1, 100, 3, 1, 1),     # GQA 8 at d=64, ragged
    ("f32", 64, 1, 1, 64, 4, 3, 1),       # the fp32 workload's shape
    ("f32", 128, 4, 2, 40, 2, 1, 1),
]


def _desc(dtype, d, hq, hkv, S, P, r, j, causal, dkv_acc=0):
    (qp, b) = B().ra_zigzag_segments(S, P, r)
    (kp, _) = B().ra_zigzag_segments(S, P, j)
    return B().make_desc(dtype=B().RA_BF16 if dtype == "bf16" else B().RA_F32, head_dim=d, hq=hq,
                         hkv=hkv, q_segments=(qp, b), k_segments=(kp, b), scale=1 / math.sqrt(d),
                         causal=causal, q_strides=(hq * d, d), k_strides=(hkv * d, d),
                         v_strides=(hkv * d, d), o_strides=(hq * d, d), do_strides=(hq * d, d),
                         dk_strides=(hkv * d, d), dkv_accumulate=dkv_acc)


def _oracle_step_fwd(x, S, P, r, j, d, dtype, causal):
    pos_q = oracle.zigzag_positions(S, P, r)
    pos_k = oracle.zigzag_positions(S, P, j)
    if not causal:
        pos_q = np.full_like(pos_q, S)   # every key visible
    return oracle.step_forward(widen(x["q"], dtype), widen(x["k_ch"][j], dtype),
                               widen(x["v_ch"][j], dtype), pos_q, pos_k, 1 / math.sqrt(d))


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_step_forward(case):
    dtype, d, hq, hkv, b, P, r, causal = case
    S = 2 * P * b
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=77)
    L = 2 * b
    q = to_device(x["q"], dtype)
    kc = to_device(x["k_ch"], dtype)
    vc = to_device(x["v_ch"], dtype)
    for j in range(P):
        o = guarded((L, hq, d))
        lse = guarded((hq, L))
        desc = _desc(dtype, d, hq, hkv, S, P, r, j, causal)
        B().ring_attn_step_fwd(desc, q, kc[j], vc[j], o, lse)
        o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
        B().ring_attn_step_fwd(desc, q, kc[j], vc[j], o2, lse2)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2), f"chunk {j}: not deterministic"
        want_o, want_l = _oracle_step_fwd(x, S, P, r, j, d, dtype, causal)
        got_l = lse.cpu().numpy()
        assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l)), f"chunk {j}: empty rows"
        assert_close(f"O chunk {j}", o.cpu().numpy(), want_o, dtype)
        assert_close(f"LSE chunk {j}", got_l, want_l, dtype, is_lse=True)


def test_step_forward_empty_chunk():
    d, hq, hkv, S, P, r = 128, 4, 2, 512, 2, 0
    desc = _desc("bf16", d, hq, hkv, S, P, r, 1, 1)
    desc.k_seg_len = 0
    L = S // P
    q = torch.zeros((L, hq, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full((L, hq, d), float("nan"), device="cuda")
    lse = torch.zeros((hq, L), device="cuda")
    B().ring_attn_step_fwd(desc, q, 0, 0, o, lse)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_binding_checks_tensor_arguments():
    """Wrong dtype or too few bytes for what the descriptor addresses: the
    binding raises before any launch."""
    d, hq, hkv, S, P, r = 128, 4, 2, 512, 2, 0
    desc = _desc("bf16", d, hq, hkv, S, P, r, 1, 1)
    L = S // P
    q = torch.zeros((L, hq, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((L, hkv, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((L, hq, d), device="cuda")
    lse = torch.zeros((hq, L), device="cuda")
    with pytest.raises(ValueError, match="must be torch.float32"):
        B().ring_attn_step_fwd(desc, q, kv, kv, o.to(torch.bfloat16), lse)
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        B().ring_attn_step_fwd(desc, q.float(), kv, kv, o, lse)
    # (fresh tensors: a view is checked against the memory of its whole storage)
    with pytest.raises(ValueError, match="the call addresses"):
        B().ring_attn_step_fwd(desc, q[: L // 2].clone(), kv, kv, o, lse)
    dk = torch.zeros((L, hkv, d), device="cuda")
    with pytest.raises(ValueError, match="the call addresses"):
        B().ring_attn_step_bwd(desc, q, kv, kv, q, lse, lse[:, 1:].clone(), o, dk, dk)
    with pytest.raises(ValueError, match="the call addresses"):
        B().ring_attn_step_bwd(desc, q, kv, kv, q, lse, lse, o, dk, dk[1:].clone())
    with pytest.raises(ValueError, match="the call addresses"):
        B().ra_fill_f32(lse, lse.numel() + 1, 0.0)
    # the same call with matching tensors runs
    B().ring_attn_step_fwd(desc, q, kv, kv, o, lse)
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_step_forward_merge(case):
    """The fused step + merge, folded over every chunk of the ring, against the
    oracle's steps merged in fp64, and against the separate GPU calls."""
    dtype, d, hq, hkv, b, P, r, causal = case
    S = 2 * P * b
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=79)
    L = 2 * b
    q = to_device(x["q"], dtype)
    kc = to_device(x["k_ch"], dtype)
    vc = to_device(x["v_ch"], dtype)
    o_f = guarded((L, hq, d), fill=0.0)
    l_f = guarded((hq, L), fill=float("-inf"))
    o_u = torch.zeros((L, hq, d), device="cuda")
    l_u = torch.full((hq, L), float("-inf"), device="cuda")
    o_s = torch.empty((L, hq, d), device="cuda")
    l_s = torch.empty((hq, L), device="cuda")
    want_o = np.zeros((L, hq, d))
    want_l = np.full((hq, L), -np.inf)
    for j in oracle.double_ring_order(P, 1, r):
        desc = _desc(dtype, d, hq, hkv, S, P, r, int(j), causal)
        B().ring_attn_step_fwd_merge(desc, q, kc[j], vc[j], o_f, l_f)
        B().ring_attn_step_fwd(desc, q, kc[j], vc[j], o_s, l_s)
        B().lse_merge(L, hq, d, o_u, l_u, o_s, l_s)
        so, sl = _oracle_step_fwd(x, S, P, r, int(j), d, dtype, causal)
        want_o, want_l = oracle.lse_merge(want_o, want_l, so, sl)
    torch.cuda.synchronize()
    got_o, got_l = o_f.cpu().numpy(), l_f.cpu().numpy()
    assert not np.isnan(got_o).any() and not np.isnan(got_l).any()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l))
    assert_close("merged O", got_o, want_o, dtype)
    assert_close("merged LSE", got_l, want_l, dtype, is_lse=True)
    # the fused epilogue applies the separate merge's formula to the same values
    fin = np.isfinite(want_l)
    assert max_abs(got_o, o_u.cpu().numpy()) < 1e-5
    assert max_abs(got_l[fin], l_u.cpu().numpy()[fin]) < 1e-5


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_step_backward(case):
    dtype, d, hq, hkv, b, P, r, causal = case
    S = 2 * P * b
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=78)
    L = 2 * b
    scale = 1 / math.sqrt(d)
    pos_q = oracle.zigzag_positions(S, P, r)
    if not causal:
        pos_q = np.full_like(pos_q, S)
    q64, do64 = widen(x["q"], dtype), widen(x["do"], dtype)
    full = oracle.share_backward(q64, widen(x["k_nat"], dtype), widen(x["v_nat"], dtype), do64,
                                 pos_q, scale)
    q = to_device(x["q"], dtype)
    do = to_device(x["do"], dtype)
    kc = to_device(x["k_ch"], dtype)
    vc = to_device(x["v_ch"], dtype)
    lse = torch.from_numpy(np.ascontiguousarray(full["LSE"], dtype=np.float32)).cuda()
    delta = torch.from_numpy(np.ascontiguousarray(full["D"], dtype=np.float32)).cuda()
    for j in range(P):
        pos_k = oracle.zigzag_positions(S, P, j)
        want_dq, want_dk, want_dv = oracle.step_backward(
            q64, widen(x["k_ch"][j], dtype), widen(x["v_ch"][j], dtype), do64, full["LSE"],
            full["D"], pos_q, pos_k, scale)
        dq = guarded((L, hq, d), fill=0.0)
        dk = guarded((L, hkv, d))
        dv = guarded((L, hkv, d))
        desc = _desc(dtype, d, hq, hkv, S, P, r, j, causal)
        B().ring_attn_step_bwd(desc, q, kc[j], vc[j], do, lse, delta, dq, dk, dv)
        # deterministic: a second run from the same state gives the same bits
        dq2 = torch.zeros_like(dq)
        dk2, dv2 = torch.full_like(dk, float("nan")), torch.full_like(dv, float("nan"))
        B().ring_attn_step_bwd(desc, q, kc[j], vc[j], do, lse, delta, dq2, dk2, dv2)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), \
            f"chunk {j}: backward not deterministic"
        assert_close(f"dQ chunk {j}", dq.cpu().numpy(), want_dq, dtype)
        assert_close(f"dK chunk {j}", dk.cpu().numpy(), want_dk, dtype)
        assert_close(f"dV chunk {j}", dv.cpu().numpy(), want_dv, dtype)
        # accumulate mode adds the same contribution again: dK, dV have one writer per
        # element, so the second pass doubles them exactly (a + a = 2a in fp32)
        dk1, dv1 = dk.clone(), dv.clone()
        B().ring_attn_step_bwd(_desc(dtype, d, hq, hkv, S, P, r, j, causal, dkv_acc=1), q, kc[j],
                               vc[j], do, lse, delta, dq, dk, dv)
        torch.cuda.synchronize()
        assert torch.equal(dk, 2 * dk1) and torch.equal(dv, 2 * dv1), f"accumulate chunk {j}"


# ------------------------------------------------------------------ strided layouts

def _in_layout(x_dev, layout, pad=64):
    """A [L][H][d] device tensor copied into a buffer of another layout; returns
    (buffer, (seq stride, head stride), view of the buffer as [L][H][d])."""
    L, H, d = x_dev.shape
    if layout == "padded_rows":          # [L][H*d + pad]
        buf = torch.zeros((L, H * d + pad), dtype=x_dev.dtype, device="cuda")
        view = buf.as_strided((L, H, d), (H * d + pad, d, 1))
        strides = (H * d + pad, d)
    elif layout == "head_major":         # [H][L][d]
        buf = torch.zeros((H, L, d), dtype=x_dev.dtype, device="cuda")
        view = buf.permute(1, 0, 2)
        strides = (d, L * d)
    elif layout == "padded_heads":       # [L][H][d + 32]
        buf = torch.zeros((L, H, d + 32), dtype=x_dev.dtype, device="cuda")
        view = buf[:, :, :d]
        strides = (H * (d + 32), d + 32)
    else:
        raise ValueError(layout)
    view.copy_(x_dev)
    return buf, strides, view


@pytest.mark.parametrize("layout", ["padded_rows", "head_major", "padded_heads"])
def test_step_strided_layouts(layout):
    """The descriptor's strides are honoured: forward and backward of a ring step
    with every tensor in a padded or head-major layout, against the oracle."""
    dtype, d, hq, hkv, b, P, r, j = "bf16", 128, 8, 2, 200, 4, 2, 1
    S, L = 2 * P * b, 2 * b
    scale = 1 / math.sqrt(d)
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=81)
    pos_q = oracle.zigzag_positions(S, P, r)
    pos_k = oracle.zigzag_positions(S, P, j)
    q64, do64 = widen(x["q"], dtype), widen(x["do"], dtype)
    k64, v64 = widen(x["k_ch"][j], dtype), widen(x["v_ch"][j], dtype)
    full = oracle.share_backward(q64, widen(x["k_nat"], dtype), widen(x["v_nat"], dtype), do64,
                                 pos_q, scale)
    want_o, want_l = oracle.step_forward(q64, k64, v64, pos_q, pos_k, scale)
    want_dq, want_dk, want_dv = oracle.step_backward(q64, k64, v64, do64, full["LSE"], full["D"],
                                                     pos_q, pos_k, scale)
    q, qs, _ = _in_layout(to_device(x["q"], dtype), layout)
    k, ks, _ = _in_layout(to_device(x["k_ch"][j], dtype), layout)
    v, vs, _ = _in_layout(to_device(x["v_ch"][j], dtype), layout)
    do, dos, _ = _in_layout(to_device(x["do"], dtype), layout)
    o, os_, o_view = _in_layout(torch.full((L, hq, d), float("nan"), device="cuda"), layout)
    dq, _, dq_view = _in_layout(torch.zeros((L, hq, d), device="cuda"), layout)
    dk, dks, dk_view = _in_layout(torch.full((L, hkv, d), float("nan"), device="cuda"), layout)
    dv, _, dv_view = _in_layout(torch.full((L, hkv, d), float("nan"), device="cuda"), layout)
    (qp, _), (kp, _) = B().ra_zigzag_segments(S, P, r), B().ra_zigzag_segments(S, P, j)
    desc = B().make_desc(dtype=B().RA_BF16, head_dim=d, hq=hq, hkv=hkv, q_segments=(qp, b),
                         k_segments=(kp, b), scale=scale, q_strides=qs, k_strides=ks,
                         v_strides=vs, o_strides=os_, do_strides=dos, dk_strides=dks)
    lse = torch.empty((hq, L), device="cuda")
    B().ring_attn_step_fwd(desc, q, k, v, o, lse)
    lse_f = torch.from_numpy(np.ascontiguousarray(full["LSE"], dtype=np.float32)).cuda()
    delta = torch.from_numpy(np.ascontiguousarray(full["D"], dtype=np.float32)).cuda()
    B().ring_attn_step_bwd(desc, q, k, v, do, lse_f, delta, dq, dk, dv)
    torch.cuda.synchronize()
    assert_close("O", o_view.cpu().numpy(), want_o, dtype)
    assert_close("LSE", lse.cpu().numpy(), want_l, dtype, is_lse=True)
    assert_close("dQ", dq_view.cpu().numpy(), want_dq, dtype)
    assert_close("dK", dk_view.cpu().numpy(), want_dk, dtype)
    assert_close("dV", dv_view.cpu().numpy(), want_dv, dtype)
    if layout != "head_major":
        # the padding is never written
        pad_o = o.view(L, -1)[:, hq * d:] if layout == "padded_rows" else o[:, :, d:]
        assert bool((pad_o == 0).all())

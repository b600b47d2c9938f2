"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against a printed worked example, a closed form, an
invariant of the mathematics, a library routine in a special case, brute force
on tiny inputs, or finite differences, chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import index_maps as im
from oracle import attention as att

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- index maps

def test_paired_blocks_worked_example():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "paired_blocks_p4.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    for S, P, b, r, ba, bb, pa, pb, work in (map(int, x) for x in rows):
        assert im.chunk_blocks(P, r) == (ba, bb)
        pos = im.zigzag_positions(S, P, r)
        assert len(pos) == 2 * b
        assert pos[0] == pa and pos[b] == pb
        assert np.array_equal(pos[:b], np.arange(pa, pa + b))
        assert np.array_equal(pos[b:], np.arange(pb, pb + b))
        assert ba + bb == work  # Workload(r) proportional to r + (2P-1-r)


@pytest.mark.parametrize("S,P", [(512, 4), (64, 1), (96, 3), (4096, 8), (1 << 16, 16)])
def test_paired_positions_partition_sequence(S, P):
    allpos = np.concatenate([im.zigzag_positions(S, P, r) for r in range(P)])
    assert np.array_equal(np.sort(allpos), np.arange(S))


@pytest.mark.parametrize("S,P", [(512, 4), (96, 3), (4096, 8), (131072, 8), (524288, 32)])
def test_paired_workload_is_rank_independent(S, P):
    b = S // (2 * P)
    for r in range(P):
        assert im.causal_pair_count(im.zigzag_positions(S, P, r), S) == b * (S + 1)
    # the contiguous split is NOT balanced (so the invariant above is not vacuous)
    if P > 1:
        L = S // P
        first = im.causal_pair_count(np.arange(0, L), S)
        last = im.causal_pair_count(np.arange(S - L, S), S)
        assert first < last


def test_pair_count_brute_force():
    S, P = 24, 3
    for r in range(P):
        pos = im.zigzag_positions(S, P, r)
        brute = sum(1 for p in pos for k in range(S) if k <= p)
        assert im.causal_pair_count(pos, S) == brute


def test_zigzag_rejects_bad_shapes():
    with pytest.raises(ValueError):
        im.zigzag_positions(100, 8, 0)
    with pytest.raises(ValueError):
        im.chunk_blocks(4, 4)


@pytest.mark.parametrize("inner,outer", [(4, 1), (8, 1), (4, 4), (8, 4), (2, 3), (1, 5)])
def test_double_ring_order_properties(inner, outer):
    P = inner * outer
    for r in range(P):
        order = im.double_ring_order(inner, outer, r)
        assert order[0] == r
        assert sorted(order.tolist()) == list(range(P))
        g = r // inner
        for t, j in enumerate(order.tolist()):
            o = t // inner
            # the outer ring moves one group back every `inner` steps
            assert j // inner == (g - o) % outer
        if outer == 1:
            assert order.tolist() == [(r - t) % P for t in range(P)]


def test_double_ring_each_step_is_a_ring_shift():
    """At every step the chunks held by all ranks are a permutation (each chunk is
    somewhere), and within the inner ring each rank holds what its predecessor
    held one step earlier (receive from rank i-1)."""
    inner, outer = 4, 4
    P = inner * outer
    orders = np.stack([im.double_ring_order(inner, outer, r) for r in range(P)])
    for t in range(P):
        assert sorted(orders[:, t].tolist()) == list(range(P))
        if t % inner != 0:
            for r in range(P):
                g, l = divmod(r, inner)
                pred = g * inner + (l - 1) % inner
                assert orders[r, t] == orders[pred, t - 1]


def test_head_permute_brute_force_and_roundtrip():
    x = rng(1).integers(0, 1 << 16, size=(6, 8, 3), dtype=np.uint16)
    for P in (1, 2, 4, 8):
        y = im.head_permute(x, P)
        assert y.shape == (P, 6, 8 // P, 3)
        for p in range(P):
            for s in range(6):
                for hh in range(8 // P):
                    for e in range(3):
                        assert y[p, s, hh, e] == x[s, p * (8 // P) + hh, e]
        assert np.array_equal(im.head_permute(y, P, inverse=True), x)
    assert np.array_equal(im.head_permute(x, 1)[0], x)
    with pytest.raises(ValueError):
        im.head_permute(x, 3)


def _strided_head_permute(src, P):
    """The other plausible grouping (destination p gets heads p, p+P, p+2P, ...),
    kept here only as the negative case of the GQA-invariant pin below."""
    S, H, d = src.shape
    return np.stack([src[:, p::P, :] for p in range(P)])


@pytest.mark.parametrize("H, Hkv, P", [(8, 4, 2), (8, 2, 2), (12, 4, 4), (32, 8, 4)])
def test_head_permute_grouping_keeps_gqa_groups(H, Hkv, P):
    """Pin of the head grouping by what the head-parallel split must preserve
    ("Guide to LoongTrain", "The Scalability Limits of DeepSpeed Ulysses": every
    head-parallel rank must receive whole KV heads, with their query heads).

    Attention of the full-head tensors restricted to the query heads of group p
    must equal attention of the p-th permuted Q/K/V run on its own (query head
    h uses KV head h div (H/Hkv) before and after the permute). The strided
    grouping, which passes the round trip and P = 1, must fail this."""
    S, Pr, r, d = 64, 2, 1, 8
    g = rng(H * 100 + Hkv * 10 + P)
    pos = im.zigzag_positions(S, Pr, r)
    q = g.standard_normal((len(pos), H, d))
    k = g.standard_normal((S, Hkv, d))
    v = g.standard_normal((S, Hkv, d))
    full, _ = att.share_forward(q, k, v, pos, 0.3)
    Hp = H // P
    qp, kp, vp = im.head_permute(q, P), im.head_permute(k, P), im.head_permute(v, P)
    for p in range(P):
        o, _ = att.share_forward(qp[p], kp[p], vp[p], pos, 0.3)
        np.testing.assert_allclose(o, full[:, p * Hp:(p + 1) * Hp], rtol=0, atol=1e-12)
    if Hkv > 1 and H // Hkv > 1:
        qs, ks, vs = (_strided_head_permute(x, P) for x in (q, k, v))
        worst = max(np.abs(att.share_forward(qs[p], ks[p], vs[p], pos, 0.3)[0]
                           - full[:, p::P]).max() for p in range(P))
        assert worst > 1e-3


# ----------------------------------------------------------------------------- forward

def make_share(S, P, r, hq, hkv, d, seed):
    g = rng(seed)
    q_full = g.standard_normal((S, hq, d))
    k = g.standard_normal((S, hkv, d))
    v = g.standard_normal((S, hkv, d))
    do_full = g.standard_normal((S, hq, d))
    pos = im.zigzag_positions(S, P, r)
    return q_full[pos], k, v, do_full[pos], pos


def torch_causal(q, k, v, scale, grad_out=None):
    """torch fp64 SDPA on the whole sequence (P = 1 special case); GQA heads
    expanded with KV head h // (Hq/Hkv)."""
    G = q.shape[1] // k.shape[1]
    tq = torch.tensor(q).permute(1, 0, 2)[None].requires_grad_(True)
    tk = torch.tensor(k).permute(1, 0, 2)[None].requires_grad_(True)
    tv = torch.tensor(v).permute(1, 0, 2)[None].requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1),
        is_causal=True, scale=scale)
    out = {"O": o[0].permute(1, 0, 2).detach().numpy()}
    if grad_out is not None:
        o.backward(torch.tensor(grad_out).permute(1, 0, 2)[None])
        out["dQ"] = tq.grad[0].permute(1, 0, 2).numpy()
        out["dK"] = tk.grad[0].permute(1, 0, 2).numpy()
        out["dV"] = tv.grad[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("hq,hkv,d", [(1, 1, 16), (4, 2, 8), (8, 2, 32)])
def test_forward_matches_torch_sdpa_whole_sequence(hq, hkv, d):
    S = 96
    q, k, v, _, pos = make_share(S, 1, 0, hq, hkv, d, 3)
    scale = 1 / math.sqrt(d)
    O, LSE = oracle.share_forward(q, k, v, pos, scale)
    ref = torch_causal(q, k, v, scale)
    np.testing.assert_allclose(O, ref["O"], rtol=0, atol=1e-12)
    # LSE against torch.logsumexp of the masked score matrix
    G = hq // hkv
    for h in range(hq):
        s = scale * torch.tensor(q[:, h]) @ torch.tensor(k[:, h // G]).T
        s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
        np.testing.assert_allclose(LSE[h], torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


def test_forward_diagonal_block_matches_sdpa():
    """A square, position-aligned block against itself is the masked local
    attention of the pages' reference code: torch SDPA with is_causal."""
    S, P, d = 256, 2, 16
    g = rng(5)
    k = g.standard_normal((S, 1, d)); v = g.standard_normal((S, 1, d))
    qf = g.standard_normal((S, 1, d))
    blk = slice(64, 128)
    pos = np.arange(64, 128)
    O, _ = oracle.step_forward(qf[blk], k[blk], v[blk], pos, pos, 0.25)
    ref = torch_causal(qf[blk], k[blk], v[blk], 0.25)
    np.testing.assert_allclose(O, ref["O"], atol=1e-12)


def brute_forward(q, k, v, pos_q, pos_k, scale):
    L, Hq, d = q.shape
    G = Hq // k.shape[1]
    O = np.zeros_like(q); LSE = np.full((Hq, L), -np.inf)
    for h in range(Hq):
        for i in range(L):
            ss = [(scale * sum(q[i, h, x] * k[j, h // G, x] for x in range(d)), j)
                  for j in range(len(pos_k)) if pos_k[j] <= pos_q[i]]
            if not ss:
                continue
            z = sum(math.exp(s) for s, _ in ss)
            LSE[h, i] = math.log(z)
            for s, j in ss:
                for x in range(d):
                    O[i, h, x] += math.exp(s) / z * v[j, h // G, x]
    return O, LSE


def test_forward_brute_force_tiny():
    S, P = 16, 2
    for r in range(P):
        q, k, v, _, pos = make_share(S, P, r, 4, 2, 3, 11 + r)
        O, LSE = oracle.share_forward(q, k, v, pos, 0.7)
        Ob, Lb = brute_forward(q, k, v, pos, np.arange(S), 0.7)
        np.testing.assert_allclose(O, Ob, atol=1e-13)
        np.testing.assert_allclose(LSE, Lb, atol=1e-13)
        # one chunk only, with empty rows
        kpos = im.zigzag_positions(S, P, (r + 1) % P)
        O, LSE = oracle.step_forward(q, k[kpos], v[kpos], pos, kpos, 0.7)
        Ob, Lb = brute_forward(q, k[kpos], v[kpos], pos, kpos, 0.7)
        np.testing.assert_allclose(O, Ob, atol=1e-13)
        assert np.array_equal(np.isneginf(LSE), np.isneginf(Lb))
        fin = np.isfinite(Lb)
        np.testing.assert_allclose(LSE[fin], Lb[fin], atol=1e-13)


def test_forward_closed_forms():
    S, P, r, hq, hkv, d = 128, 4, 1, 4, 2, 8
    q, k, v, _, pos = make_share(S, P, r, hq, hkv, d, 21)
    scale = 1 / math.sqrt(d)
    # (i) uniform V -> O = c
    c = rng(2).standard_normal(d)
    vu = np.broadcast_to(c, v.shape).copy()
    O, _ = oracle.share_forward(q, k, vu, pos, scale)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), atol=1e-13)
    # (ii) the row at position 0 sees only key 0
    q0, k0, v0, _, pos0 = make_share(S, P, 0, hq, hkv, d, 22)
    O, LSE = oracle.share_forward(q0, k0, v0, pos0, scale)
    assert pos0[0] == 0
    for h in range(hq):
        np.testing.assert_allclose(O[0, h], v0[0, h // 2], atol=1e-14)
        np.testing.assert_allclose(LSE[h, 0], scale * q0[0, h] @ k0[0, h // 2], atol=1e-14)
    # (iii) Q = 0 -> uniform weights: LSE = ln(pos + 1), O = prefix mean of V
    O, LSE = oracle.share_forward(np.zeros_like(q), k, v, pos, scale)
    for h in range(hq):
        np.testing.assert_allclose(LSE[h], np.log(pos + 1.0), atol=1e-12)
        pm = np.cumsum(v[:, h // 2, :], axis=0) / np.arange(1, S + 1)[:, None]
        np.testing.assert_allclose(O[:, h, :], pm[pos], atol=1e-12)


def test_forward_key_shift_metamorphic():
    S, P, r, d = 64, 2, 1, 8
    q, k, v, _, pos = make_share(S, P, r, 2, 1, d, 31)
    u = rng(4).standard_normal(d)
    O1, L1 = oracle.share_forward(q, k, v, pos, 0.3)
    O2, L2 = oracle.share_forward(q, k + u, v, pos, 0.3)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(L2 - L1, 0.3 * np.einsum("lhd,d->hl", q, u), atol=1e-12)


@pytest.mark.parametrize("inner,outer,r", [(4, 1, 0), (4, 1, 3), (2, 2, 1), (4, 2, 5)])
def test_chunked_merged_equals_whole(inner, outer, r):
    P = inner * outer
    S = 32 * 2 * P
    q, k, v, _, pos = make_share(S, P, r, 4, 1, 8, 41 + r)
    scale = 0.35
    O_ref, L_ref = oracle.share_forward(q, k, v, pos, scale)
    for order in (im.double_ring_order(inner, outer, r), np.arange(P)[::-1], rng(r).permutation(P)):
        acc_o = np.zeros_like(q); acc_l = np.full((4, len(pos)), -np.inf)
        for j in order:
            kp = im.zigzag_positions(S, P, int(j))
            o_s, l_s = oracle.step_forward(q, k[kp], v[kp], pos, kp, scale)
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, o_s, l_s)
        np.testing.assert_allclose(acc_o, O_ref, atol=1e-12)
        np.testing.assert_allclose(acc_l, L_ref, atol=1e-12)


def test_step_empty_rows():
    S, P, r = 64, 4, 0
    q, k, v, _, pos = make_share(S, P, r, 1, 1, 4, 51)
    kp = im.zigzag_positions(S, P, 2)      # chunk 2 > r: block-A rows of rank 0 see nothing
    O, L = oracle.step_forward(q, k[kp], v[kp], pos, kp, 0.5)
    b = S // (2 * P)
    assert np.all(np.isneginf(L[:, :b])) and np.all(O[:b] == 0)
    assert np.all(np.isfinite(L[:, b:]))


def test_merge_truth_table_and_hand_case():
    o1 = np.ones((1, 1, 2)); o2 = 2 * np.ones((1, 1, 2)); z = np.zeros((1, 1, 2))
    ninf = np.array([[-np.inf]])
    o, l = oracle.lse_merge(z, ninf, z, ninf)
    assert np.isneginf(l).all() and not np.isnan(o).any() and (o == 0).all()
    o, l = oracle.lse_merge(z, ninf, o2, np.array([[0.5]]))
    assert l[0, 0] == 0.5 and np.all(o == 2)
    o, l = oracle.lse_merge(o1, np.array([[0.5]]), z, ninf)
    assert l[0, 0] == 0.5 and np.all(o == 1)
    # two single-key chunks with scores a, b: L = log(e^a + e^b), weights softmax
    a, bb = 1.3, -0.4
    o, l = oracle.lse_merge(o1, np.array([[a]]), o2, np.array([[bb]]))
    np.testing.assert_allclose(l[0, 0], math.log(math.exp(a) + math.exp(bb)), atol=1e-15)
    wa = math.exp(a) / (math.exp(a) + math.exp(bb))
    np.testing.assert_allclose(o[0, 0], wa * 1 + (1 - wa) * 2, atol=1e-15)


# ----------------------------------------------------------------------------- backward

def test_backward_matches_torch_autograd_whole_sequence():
    S, hq, hkv, d = 80, 4, 2, 16
    q, k, v, do, pos = make_share(S, 1, 0, hq, hkv, d, 61)
    scale = 1 / math.sqrt(d)
    res = oracle.share_backward(q, k, v, do, pos, scale)
    ref = torch_causal(q, k, v, scale, grad_out=do)
    for name in ("O", "dQ", "dK", "dV"):
        np.testing.assert_allclose(res[name], ref[name], atol=1e-11, err_msg=name)


def test_backward_finite_differences():
    S, P, r, hq, hkv, d = 12, 2, 1, 2, 1, 3
    q, k, v, do, pos = make_share(S, P, r, hq, hkv, d, 71)
    scale = 0.6
    res = oracle.share_backward(q, k, v, do, pos, scale)

    def loss(qq, kk, vv):
        O, _ = oracle.share_forward(qq, kk, vv, pos, scale)
        return float(np.sum(do * O))

    eps = 1e-6
    for name, arr, idx in (("dQ", q, 0), ("dK", k, 1), ("dV", v, 2)):
        g = np.zeros_like(arr)
        for ix in np.ndindex(arr.shape):
            args = [q, k, v]
            a_p = arr.copy(); a_p[ix] += eps
            a_m = arr.copy(); a_m[ix] -= eps
            args[idx] = a_p; lp = loss(*args)
            args[idx] = a_m; lm = loss(*args)
            g[ix] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(res[name], g, atol=2e-8, err_msg=name)


def test_backward_closed_forms_and_invariants():
    S, P, r, hq, hkv, d = 128, 4, 0, 4, 2, 8
    q, k, v, do, pos = make_share(S, P, r, hq, hkv, d, 81)
    scale = 1 / math.sqrt(d)
    # uniform V -> dQ = dK = 0
    c = rng(9).standard_normal(d)
    res = oracle.share_backward(q, k, np.broadcast_to(c, v.shape).copy(), do, pos, scale)
    assert np.abs(res["dQ"]).max() < 1e-12 and np.abs(res["dK"]).max() < 1e-12
    res = oracle.share_backward(q, k, v, do, pos, scale)
    # the row at position 0 has a single key: dQ_0 = 0
    assert pos[0] == 0 and np.abs(res["dQ"][0]).max() < 1e-13
    # sum over keys of dK is 0; sum over keys of dV is the sum of dO over the group
    for g in range(hkv):
        assert np.abs(res["dK"][:, g].sum(axis=0)).max() < 1e-11
        np.testing.assert_allclose(res["dV"][:, g].sum(axis=0),
                                   do[:, 2 * g:2 * g + 2].sum(axis=(0, 1)), atol=1e-11)
    # D = rowsum(dO * O)
    np.testing.assert_allclose(res["D"], np.einsum("lhd,lhd->hl", do, res["O"]), atol=1e-13)


@pytest.mark.parametrize("inner,outer,r", [(4, 1, 2), (2, 2, 3)])
def test_backward_steps_sum_to_whole(inner, outer, r):
    P = inner * outer
    S = 16 * 2 * P
    q, k, v, do, pos = make_share(S, P, r, 4, 2, 8, 91)
    scale = 0.3
    res = oracle.share_backward(q, k, v, do, pos, scale)
    dq = np.zeros_like(q)
    for j in im.double_ring_order(inner, outer, r):
        kp = im.zigzag_positions(S, P, int(j))
        dq_s, dk_s, dv_s = oracle.step_backward(q, k[kp], v[kp], do, res["LSE"], res["D"],
                                                pos, kp, scale)
        dq += dq_s
        np.testing.assert_allclose(dk_s, res["dK"][kp], atol=1e-12)
        np.testing.assert_allclose(dv_s, res["dV"][kp], atol=1e-12)
    np.testing.assert_allclose(dq, res["dQ"], atol=1e-12)


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x7F80, 0x4049], dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0 and np.isposinf(vals[3])
    assert vals[4] == 3.140625


@pytest.mark.parametrize("S,P", [(64, 4), (96, 3), (4096, 8)])
def test_contiguous_layout_pairs_and_imbalance(S, P):
    """Contiguous chunks partition the sequence; rank r's pair count is
    L (r L) + L (L + 1) / 2 (brute force), so the latest rank does (2P - 1)
    times the earliest one's work up to O(1/L) -- the imbalance the paired
    blocks remove (every paired-block rank has b (S + 1))."""
    from ring_attention_attn_amd.configs import ShareConfig
    L = S // P
    allpos = np.concatenate([oracle.contiguous_positions(S, P, r) for r in range(P)])
    assert np.array_equal(np.sort(allpos), np.arange(S))
    cfg = ShareConfig("t", S=S, inner=P, outer=1, hq=1, hkv=1, d=64, dtype="f32", seed=0)
    counts = []
    for r in range(P):
        pos = oracle.contiguous_positions(S, P, r)
        brute = sum(1 for p in pos for k in range(S) if k <= p)
        assert oracle.causal_pair_count(pos, S) == brute == cfg.pairs_per_head("contiguous", r)
        counts.append(brute)
        assert cfg.pairs_per_head("zigzag", r) == oracle.causal_pair_count(
            oracle.zigzag_positions(S, P, r), S)
    assert counts[-1] * (L + 1) == counts[0] * (2 * (P - 1) * L + L + 1)
    assert sum(counts) == S * (S + 1) // 2

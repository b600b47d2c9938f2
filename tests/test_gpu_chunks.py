"""ring_attn_fwd_chunks / ring_attn_bwd_chunks at their edges: the largest
chunk count (32), chunks of different lengths with an empty one among them,
and no key or no query row at all. Each case runs against the fp64 oracle over the union of
the chunks' keys (softmax over a union of key sets is what the ring's merges
compute) and against the per-step entry points on the same descriptors."""
import math

import numpy as np
import pytest

import oracle
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


def B():
    from ring_attention_attn_amd import binding
    return binding


def chunk_set(S, P, r, hq, hkv, d, shape, seed):
    """Rank r's zigzag share with its P chunks reshaped by `shape`: "full"
    keeps them; "ragged" shortens both runs of chunk 1 by 13 rows, keeps only
    the first run of chunk 2 and empties chunk 3; "empty" empties them all.
    Returns descriptors, host inputs (bf16 bits), the chunks' key rows and
    positions, and the query positions."""
    x = share_inputs(S, P, r, hq, hkv, d, "bf16", seed=seed)
    b = x["b"]
    (qp, _) = B().ra_zigzag_segments(S, P, r)
    pos_q = np.concatenate([np.arange(p, p + b) for p in qp])
    descs, ks, vs, kpos = [], [], [], []
    for j in range(P):
        (kp, _) = B().ra_zigzag_segments(S, P, j)
        runs, kl = list(kp), b
        if shape == "empty" or (shape == "ragged" and j == 3):
            kl = 0
        elif shape == "ragged" and j == 1:
            kl = b - 13
        elif shape == "ragged" and j == 2:
            runs = runs[:1]
        rows = np.concatenate([np.arange(i * b, i * b + kl) for i in range(len(runs))])
        ks.append(x["k_ch"][j][rows])
        vs.append(x["v_ch"][j][rows])
        kpos.append(np.concatenate([np.arange(p, p + kl) for p in runs]))
        descs.append(B().make_desc(dtype=B().RA_BF16, head_dim=d, hq=hq, hkv=hkv,
                                   q_segments=(qp, b), k_segments=(runs, kl),
                                   scale=1 / math.sqrt(d), causal=1, q_strides=(hq * d, d),
                                   k_strides=(hkv * d, d), v_strides=(hkv * d, d),
                                   o_strides=(hq * d, d), do_strides=(hq * d, d),
                                   dk_strides=(hkv * d, d), dkv_accumulate=0))
    return descs, x, ks, vs, kpos, pos_q


def dev_chunks(arrs, hkv, d):
    # an empty chunk still gets a (one-row) buffer: the calls skip it unread
    return [to_device(a if len(a) else np.zeros((1, hkv, d), np.uint16), "bf16") for a in arrs]


CASES = [
    # name, S, P, r, hq, hkv, d, shape
    ("ring32_max_chunks", 2048, 32, 5, 4, 2, 128, "full"),
    ("ragged_and_empty_chunks", 1024, 4, 1, 8, 2, 128, "ragged"),
    ("ragged_d64_mha", 1408, 4, 2, 4, 4, 64, "ragged"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_chunks_edges(case):
    name, S, P, r, hq, hkv, d, shape = case
    descs, x, ks, vs, kpos, pos_q = chunk_set(S, P, r, hq, hkv, d, shape, seed=7000 + S + P)
    L = len(pos_q)
    q, do = to_device(x["q"], "bf16"), to_device(x["do"], "bf16")
    K, V = dev_chunks(ks, hkv, d), dev_chunks(vs, hkv, d)
    f32 = dict(device="cuda", dtype=torch.float32)

    # forward: all chunks in one launch, and step by step with the fused merge
    o = torch.full((L, hq, d), float("nan"), **f32)
    lse = torch.full((hq, L), float("nan"), **f32)
    B().ring_attn_fwd_chunks(descs, q, K, V, o, lse)
    o1 = torch.zeros((L, hq, d), **f32)
    l1 = torch.full((hq, L), float("-inf"), **f32)
    for dsc, k, v in zip(descs, K, V):
        B().ring_attn_step_fwd_merge(dsc, q, k, v, o1, l1)
    # D and the bf16 O for the backward, from the chunks forward
    delta = torch.empty((hq, L), **f32)
    o_bf = torch.empty((L, hq, d), dtype=torch.bfloat16, device="cuda")
    B().ra_bwd_delta(L, hq, d, B().RA_BF16, o, do, delta, o_bf)

    # backward: one call, and step by step (dq accumulated from zero)
    dq = torch.full((L, hq, d), float("nan"), **f32)
    dk = [torch.full((len(a), hkv, d), float("nan"), **f32) for a in ks]
    dv = [torch.full((len(a), hkv, d), float("nan"), **f32) for a in ks]
    dkd = [t if len(t) else torch.zeros((1, hkv, d), **f32) for t in dk]
    dvd = [t if len(t) else torch.zeros((1, hkv, d), **f32) for t in dv]
    B().ring_attn_bwd_chunks(descs, q, K, V, do, lse, delta, dq, dkd, dvd)
    dq1 = torch.zeros((L, hq, d), **f32)
    dk1 = [torch.full_like(t, float("nan")) for t in dkd]
    dv1 = [torch.full_like(t, float("nan")) for t in dvd]
    for dsc, k, v, a, c in zip(descs, K, V, dk1, dv1):
        B().ring_attn_step_bwd(dsc, q, k, v, do, lse, delta, dq1, a, c)
    torch.cuda.synchronize()

    got = dict(O=o.cpu().numpy(), LSE=lse.cpu().numpy(), dQ=dq.cpu().numpy())
    fin = np.isfinite(l1.cpu().numpy())
    assert np.array_equal(np.isneginf(got["LSE"]), ~fin)
    assert max_abs(got["O"], o1.cpu().numpy()) < 1e-2
    assert max_abs(got["LSE"][fin], l1.cpu().numpy()[fin]) < 1e-4
    for j in range(P):
        if len(ks[j]):
            assert torch.equal(dkd[j], dk1[j]) and torch.equal(dvd[j], dv1[j]), f"chunk {j}"
    scale_dq = float(dq1.abs().max())
    assert float((dq - dq1).abs().max()) <= 1e-5 * scale_dq + 1e-30

    # the oracle over the union of the chunks' keys
    kcat = np.concatenate([widen(a, "bf16") for a in ks])
    vcat = np.concatenate([widen(a, "bf16") for a in vs])
    pk = np.concatenate(kpos)
    qd, dod = widen(x["q"], "bf16"), widen(x["do"], "bf16")
    want_o, want_l = oracle.step_forward(qd, kcat, vcat, pos_q, pk, 1 / math.sqrt(d))
    want_delta = np.einsum("lhd,lhd->hl", dod, want_o)
    wdq, wdk, wdv = oracle.step_backward(qd, kcat, vcat, dod, want_l, want_delta, pos_q, pk,
                                         1 / math.sqrt(d))
    assert_close("O", got["O"], want_o, "bf16")
    assert_close("LSE", got["LSE"], want_l, "bf16", is_lse=True)
    assert_close("dQ", got["dQ"], wdq, "bf16")
    off = 0
    for j in range(P):
        n = len(ks[j])
        if n:
            assert_close(f"dK[{j}]", dkd[j].cpu().numpy(), wdk[off:off + n], "bf16")
            assert_close(f"dV[{j}]", dvd[j].cpu().numpy(), wdv[off:off + n], "bf16")
        off += n


def test_chunks_without_keys():
    """Every chunk empty: the forward writes O = 0 and LSE = -inf (no key is
    visible), the backward writes dQ = 0 and touches no dK/dV."""
    S, P, r, hq, hkv, d = 1024, 4, 1, 4, 2, 128
    descs, x, ks, vs, kpos, pos_q = chunk_set(S, P, r, hq, hkv, d, "empty", seed=11)
    L = len(pos_q)
    q, do = to_device(x["q"], "bf16"), to_device(x["do"], "bf16")
    K, V = dev_chunks(ks, hkv, d), dev_chunks(vs, hkv, d)
    f32 = dict(device="cuda", dtype=torch.float32)
    o = torch.full((L, hq, d), float("nan"), **f32)
    lse = torch.full((hq, L), float("nan"), **f32)
    B().ring_attn_fwd_chunks(descs, q, K, V, o, lse)
    dq = torch.full((L, hq, d), float("nan"), **f32)
    dk = [torch.full((1, hkv, d), 3.5, **f32) for _ in range(P)]
    dv = [torch.full((1, hkv, d), 3.5, **f32) for _ in range(P)]
    delta = torch.zeros((hq, L), **f32)
    B().ring_attn_bwd_chunks(descs, q, K, V, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())
    assert bool((dq == 0).all())
    assert all(bool((t == 3.5).all()) for t in dk + dv)


def test_chunks_without_queries():
    """No query row (lq = 0): the forward does nothing, the backward writes
    every chunk's dK/dV as zeros and reads no query-side argument."""
    S, P, r, hq, hkv, d = 1024, 4, 1, 4, 2, 128
    descs, x, ks, vs, kpos, pos_q = chunk_set(S, P, r, hq, hkv, d, "full", seed=12)
    for dsc in descs:
        dsc.q_seg_len = 0
    K, V = dev_chunks(ks, hkv, d), dev_chunks(vs, hkv, d)
    f32 = dict(device="cuda", dtype=torch.float32)
    dummy_q = torch.zeros((1, hq, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full((1, hq, d), 5.0, **f32)
    lse = torch.full((hq, 1), 5.0, **f32)
    B().ring_attn_fwd_chunks(descs, dummy_q, K, V, o, lse)
    dq = torch.full((1, hq, d), 5.0, **f32)
    dk = [torch.full((len(a), hkv, d), float("nan"), **f32) for a in ks]
    dv = [torch.full((len(a), hkv, d), float("nan"), **f32) for a in ks]
    B().ring_attn_bwd_chunks(descs, dummy_q, K, V, dummy_q, lse, lse, dq, dk, dv)
    torch.cuda.synchronize()
    assert bool((o == 5.0).all()) and bool((lse == 5.0).all()) and bool((dq == 5.0).all())
    assert all(bool((t == 0).all()) for t in dk + dv)

"""Whole-share parity on the GPU: the virtual ring (P forward steps + merges,
backward preprocess, P backward steps) against the fp64 oracle of full-sequence
causal attention restricted to the share's rows.

Small shares are compared element by element; the full-size workload that the
benchmark times is compared on sampled rows and keys that the oracle computes
one by one, plus identities that hold at any size."""
import math

import numpy as np
import pytest

import oracle
from ring_attention_attn_amd.configs import CONFIGS
from tests.helpers import share_inputs, widen, to_device, assert_close, max_abs, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ring_attention_attn_amd import binding
    binding.lib()
    yield


def run_share(S, inner, outer, r, hq, hkv, d, dtype, x, merge="fused", layout="zigzag"):
    from ring_attention_attn_amd.ring import ShareRing
    ring = ShareRing(S, inner, outer, r, hq, hkv, d, dtype, merge=merge, layout=layout)
    q, do = to_device(x["q"], dtype), to_device(x["do"], dtype)
    K, V = to_device(x["k_ch"], dtype), to_device(x["v_ch"], dtype)
    o, lse = ring.forward(q, K, V)
    dq, dk, dv = ring.backward(q, K, V, do)
    torch.cuda.synchronize()
    return ring, dict(O=o.cpu().numpy(), LSE=lse.cpu().numpy(), dQ=dq.cpu().numpy(),
                      dK=dk.cpu().numpy(), dV=dv.cpu().numpy(), Obf=ring.o_lowp)


SHARE_CASES = [
    # name, S, inner, outer, rank, hq, hkv, d, dtype
    ("tiny_f32_r0", 512, 4, 1, 0, 1, 1, 64, "f32"),
    ("tiny_f32_r1", 512, 4, 1, 1, 1, 1, 64, "f32"),
    ("tiny_f32_r2", 512, 4, 1, 2, 1, 1, 64, "f32"),
    ("tiny_f32_r3", 512, 4, 1, 3, 1, 1, 64, "f32"),
    ("gqa4_ring4_r0", 8192, 4, 1, 0, 8, 2, 128, "bf16"),
    ("gqa4_ring4_r3", 8192, 4, 1, 3, 8, 2, 128, "bf16"),
    ("gqa8_double_ring_4x2_r5", 4096, 4, 2, 5, 8, 1, 128, "bf16"),
    ("mha_ring8_ragged_r6", 8 * 2 * 88, 8, 1, 6, 4, 4, 64, "bf16"),
    # a ring of one rank: the whole causal sequence in one (diagonal) step
    ("single_rank_p1", 1024, 1, 1, 0, 8, 2, 128, "bf16"),
    ("single_rank_p1_ragged_d64", 600, 1, 1, 0, 4, 4, 64, "bf16"),
]


@pytest.mark.parametrize("case", SHARE_CASES, ids=lambda c: c[0])
def test_share_matches_oracle(case):
    name, S, inner, outer, r, hq, hkv, d, dtype = case
    P = inner * outer
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=1000 + S + r)
    _, got = run_share(S, inner, outer, r, hq, hkv, d, dtype, x)
    pos = oracle.zigzag_positions(S, P, r)
    want = oracle.share_backward(widen(x["q"], dtype), widen(x["k_nat"], dtype),
                                 widen(x["v_nat"], dtype), widen(x["do"], dtype), pos, 1 / math.sqrt(d))
    assert_close("O", got["O"], want["O"], dtype)
    assert_close("LSE", got["LSE"], want["LSE"], dtype, is_lse=True)
    assert_close("dQ", got["dQ"], want["dQ"], dtype)
    b = S // (2 * P)
    for j in range(P):
        kp = oracle.zigzag_positions(S, P, j)
        assert_close(f"dK[{j}]", got["dK"][j], want["dK"][kp], dtype)
        assert_close(f"dV[{j}]", got["dV"][j], want["dV"][kp], dtype)
    if dtype == "bf16":
        # per zigzag half, so that a wrong short-row block cannot hide in the average
        for half in (slice(0, b), slice(b, 2 * b)):
            assert rel_l2(got["O"][half], want["O"][half]) < 1e-2
            assert rel_l2(got["dQ"][half], want["dQ"][half]) < 1e-2


@pytest.mark.parametrize("case", [SHARE_CASES[1], SHARE_CASES[6]], ids=lambda c: c[0])
def test_share_separate_merge_matches_fused(case):
    """The forward with separate lse_merge launches gives the fused result (the
    same merge formula on the same values, up to fp32 rounding)."""
    name, S, inner, outer, r, hq, hkv, d, dtype = case
    x = share_inputs(S, inner * outer, r, hq, hkv, d, dtype, seed=2000 + S + r)
    _, fused = run_share(S, inner, outer, r, hq, hkv, d, dtype, x, "fused")
    _, sep = run_share(S, inner, outer, r, hq, hkv, d, dtype, x, "separate")
    fin = np.isfinite(sep["LSE"])
    assert np.array_equal(np.isneginf(fused["LSE"]), np.isneginf(sep["LSE"]))
    assert max_abs(fused["O"], sep["O"]) < 1e-5
    assert max_abs(fused["LSE"][fin], sep["LSE"][fin]) < 1e-5


@pytest.mark.parametrize("case", [c for c in SHARE_CASES if c[8] == "bf16"], ids=lambda c: c[0])
def test_share_chunks_matches_oracle(case):
    """The forward of all steps in one launch (running max, sum and output kept
    in registers across chunks) and the backward of all steps in one call (dQ
    summed in registers over the chunks and written once) against the oracle,
    and close to the per-step path (the same arithmetic; only the rounding of
    the intermediate normalisation and dQ's summation order differ)."""
    name, S, inner, outer, r, hq, hkv, d, dtype = case
    P = inner * outer
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=3000 + S + r)
    _, got = run_share(S, inner, outer, r, hq, hkv, d, dtype, x, "chunks")
    pos = oracle.zigzag_positions(S, P, r)
    want = oracle.share_backward(widen(x["q"], dtype), widen(x["k_nat"], dtype),
                                 widen(x["v_nat"], dtype), widen(x["do"], dtype), pos, 1 / math.sqrt(d))
    assert_close("O", got["O"], want["O"], dtype)
    assert_close("LSE", got["LSE"], want["LSE"], dtype, is_lse=True)
    assert_close("dQ", got["dQ"], want["dQ"], dtype)
    for j in range(P):
        kp = oracle.zigzag_positions(S, P, j)
        assert_close(f"dK[{j}]", got["dK"][j], want["dK"][kp], dtype)
        assert_close(f"dV[{j}]", got["dV"][j], want["dV"][kp], dtype)
    _, fused = run_share(S, inner, outer, r, hq, hkv, d, dtype, x, "fused")
    fin = np.isfinite(fused["LSE"])
    assert np.array_equal(np.isneginf(fused["LSE"]), np.isneginf(got["LSE"]))
    assert max_abs(fused["O"], got["O"]) < 1e-2
    assert max_abs(fused["LSE"][fin], got["LSE"][fin]) < 1e-4
    for t in ("dQ", "dK", "dV"):
        assert max_abs(fused[t], got[t]) < 1e-2, t


@pytest.mark.parametrize("r", [0, 1, 3])
def test_contiguous_layout_share(r):
    """One contiguous chunk per rank (the layout whose causal imbalance the
    paired blocks remove): same kernels, one segment per map."""
    S, inner, outer, hq, hkv, d, dtype = 4096, 4, 1, 8, 2, 128, "bf16"
    P = inner * outer
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=3000 + r, layout="contiguous")
    _, got = run_share(S, inner, outer, r, hq, hkv, d, dtype, x, layout="contiguous")
    pos = oracle.contiguous_positions(S, P, r)
    want = oracle.share_backward(widen(x["q"], dtype), widen(x["k_nat"], dtype),
                                 widen(x["v_nat"], dtype), widen(x["do"], dtype), pos, 1 / math.sqrt(d))
    assert_close("O", got["O"], want["O"], dtype)
    assert_close("LSE", got["LSE"], want["LSE"], dtype, is_lse=True)
    assert_close("dQ", got["dQ"], want["dQ"], dtype)
    for j in range(P):
        kp = oracle.contiguous_positions(S, P, j)
        assert_close(f"dK[{j}]", got["dK"][j], want["dK"][kp], dtype)
        assert_close(f"dV[{j}]", got["dV"][j], want["dV"][kp], dtype)
    assert rel_l2(got["O"], want["O"]) < 1e-2
    assert rel_l2(got["dQ"], want["dQ"]) < 1e-2


@pytest.mark.parametrize("merge", ["fused", "chunks"])
@pytest.mark.parametrize("case", [SHARE_CASES[4], SHARE_CASES[7]], ids=lambda c: c[0])
def test_ab_rings_share(case, merge):
    """Each step as two launches, one per block of the KV chunk (the block A and
    block B rings), per step or all in one call, against the oracle and the
    one-launch steps."""
    name, S, inner, outer, r, hq, hkv, d, dtype = case
    P = inner * outer
    x = share_inputs(S, P, r, hq, hkv, d, dtype, seed=4000 + S + r)
    from ring_attention_attn_amd.ring import ShareRing
    q, do = to_device(x["q"], dtype), to_device(x["do"], dtype)
    K, V = to_device(x["k_ch"], dtype), to_device(x["v_ch"], dtype)
    ring = ShareRing(S, inner, outer, r, hq, hkv, d, dtype, kv_rings="ab", merge=merge)
    assert len(ring.launches) == 2 * P
    o, lse = ring.forward(q, K, V)
    dq, dk, dv = ring.backward(q, K, V, do)
    torch.cuda.synchronize()
    pos = oracle.zigzag_positions(S, P, r)
    want = oracle.share_backward(widen(x["q"], dtype), widen(x["k_nat"], dtype),
                                 widen(x["v_nat"], dtype), widen(x["do"], dtype), pos, 1 / math.sqrt(d))
    assert_close("O", o.cpu().numpy(), want["O"], dtype)
    assert_close("LSE", lse.cpu().numpy(), want["LSE"], dtype, is_lse=True)
    assert_close("dQ", dq.cpu().numpy(), want["dQ"], dtype)
    for j in range(P):
        kp = oracle.zigzag_positions(S, P, j)
        assert_close(f"dK[{j}]", dk[j].cpu().numpy(), want["dK"][kp], dtype)
        assert_close(f"dV[{j}]", dv[j].cpu().numpy(), want["dV"][kp], dtype)
    # against the one-launch steps: a half-chunk step rounds P to bf16 under its
    # own exponent shift, so O (and, through D, the gradients) differ at the
    # level of that rounding, not of fp32
    _, one = run_share(S, inner, outer, r, hq, hkv, d, dtype, x)
    assert max_abs(o.cpu().numpy(), one["O"]) < 2e-3
    assert max_abs(dk.cpu().numpy(), one["dK"]) < 2e-3


@pytest.mark.parametrize("case", [c for c in SHARE_CASES if c[8] == "bf16"], ids=lambda c: c[0])
def test_bwd_chunks_matches_per_step(case):
    """ring_attn_bwd_chunks from the same forward (O, LSE, D) as the per-step
    backward: dK and dV come from the same key-block computation (bit for bit,
    whatever the outputs held before, since each chunk's first visit writes);
    dQ is written, not accumulated, and equals the per-step sum up to its
    fp32 summation order."""
    from ring_attention_attn_amd import binding as B
    from ring_attention_attn_amd.ring import ShareRing
    name, S, inner, outer, r, hq, hkv, d, dtype = case
    x = share_inputs(S, inner * outer, r, hq, hkv, d, dtype, seed=4000 + S + r)
    q, do = to_device(x["q"], dtype), to_device(x["do"], dtype)
    K, V = to_device(x["k_ch"], dtype), to_device(x["v_ch"], dtype)
    ring = ShareRing(S, inner, outer, r, hq, hkv, d, dtype)
    ring.forward(q, K, V)
    dq1, dk1, dv1 = (t.clone() for t in ring.backward(q, K, V, do))
    dq2, dk2, dv2 = (torch.full_like(t, float("nan")) for t in (dq1, dk1, dv1))
    L = ring.launches
    B.ring_attn_bwd_chunks([dsc for _, _, dsc in L], q, [ring._kv(K, j, o) for j, o, _ in L],
                           [ring._kv(V, j, o) for j, o, _ in L], do, ring.lse_acc, ring.delta, dq2,
                           [ring._kv(dk2, j, o) for j, o, _ in L],
                           [ring._kv(dv2, j, o) for j, o, _ in L])
    torch.cuda.synchronize()
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    assert torch.isfinite(dq2).all()
    assert (dq1 - dq2).abs().max().item() <= 1e-5 * dq1.abs().max().item()


def test_ring_order_invariance():
    """The merged result does not depend on the order the chunks are visited in
    (up to fp32 rounding of the merge)."""
    from ring_attention_attn_amd import binding as B
    from ring_attention_attn_amd.ring import ShareRing
    S, inner, outer, r, hq, hkv, d = 4096, 4, 2, 3, 8, 2, 128
    x = share_inputs(S, inner * outer, r, hq, hkv, d, "bf16", seed=5)
    q, do = to_device(x["q"], "bf16"), to_device(x["do"], "bf16")
    K, V = to_device(x["k_ch"], "bf16"), to_device(x["v_ch"], "bf16")
    ring = ShareRing(S, inner, outer, r, hq, hkv, d, "bf16")
    o1 = ring.forward(q, K, V)[0].clone()
    ring.launches = ring.launches[::-1]
    o2 = ring.forward(q, K, V)[0].clone()
    torch.cuda.synchronize()
    assert max_abs(o1.cpu().numpy(), o2.cpu().numpy()) < 1e-5


HP_CASES = [
    # name, S, inner, outer, rank, H, Hkv, d, hp, group
    ("hp4_gqa4_2x2_g2", 4096, 2, 2, 1, 16, 4, 128, 4, 2),
    ("hp2_gqa2_ragged_d64_g1", 1600, 4, 1, 3, 8, 4, 64, 2, 1),
    ("hp4_mha_g0", 2048, 4, 1, 0, 8, 8, 128, 4, 0),
]


def head_parallel_inputs(S, P, r, H, Hkv, d, hp, g, seed):
    """All-head Q/dO of the rank's rows, all-KV-head K/V of its own chunk, and
    the other chunks' K/V in head-group g layout (as the ring would deliver
    them); plus the oracle's view of head group g (natural-order K/V)."""
    from ring_attention_attn_amd import synth
    b = S // (2 * P)
    hq, hkv = H // hp, Hkv // hp
    gk = range(g * hkv, (g + 1) * hkv)
    mine = synth.paired_blocks(P, r)
    x = dict(b=b)
    x["q_full"] = synth.blocks_tensor(seed, synth.T_Q, mine, b, H, d, "bf16")
    x["do_full"] = synth.blocks_tensor(seed, synth.T_DO, mine, b, H, d, "bf16")
    x["k_own"] = synth.blocks_tensor(seed, synth.T_K, mine, b, Hkv, d, "bf16")
    x["v_own"] = synth.blocks_tensor(seed, synth.T_V, mine, b, Hkv, d, "bf16")
    x["k_rest"] = [None if j == r else synth.blocks_tensor(seed, synth.T_K, synth.paired_blocks(P, j),
                                                           b, gk, d, "bf16") for j in range(P)]
    x["v_rest"] = [None if j == r else synth.blocks_tensor(seed, synth.T_V, synth.paired_blocks(P, j),
                                                           b, gk, d, "bf16") for j in range(P)]
    x["k_nat"] = synth.blocks_tensor(seed, synth.T_K, range(2 * P), b, gk, d, "bf16")
    x["v_nat"] = synth.blocks_tensor(seed, synth.T_V, range(2 * P), b, gk, d, "bf16")
    x["q"] = x["q_full"][:, g * hq:(g + 1) * hq]
    x["do"] = x["do_full"][:, g * hq:(g + 1) * hq]
    return x


def run_head_parallel(S, inner, outer, r, H, Hkv, d, hp, g, x, sentinel=7.25, merge="fused"):
    """The 2D-Attention share through HeadParallelShare. Exchange slots other
    than g are filled with ``sentinel`` first: they stand for the other
    head-parallel ranks' data and must come back bit for bit."""
    from ring_attention_attn_amd.ring import HeadParallelShare
    hp_share = HeadParallelShare(S, inner, outer, r, H, Hkv, d, hp, group=g, merge=merge)
    for t in (hp_share.o_x, hp_share.dq_x, hp_share.dk_x, hp_share.dv_x):
        t.fill_(sentinel)
    dev = lambda a: to_device(a, "bf16")
    k_rest = [None if a is None else dev(a) for a in x["k_rest"]]
    v_rest = [None if a is None else dev(a) for a in x["v_rest"]]
    o, lse = hp_share.forward(dev(x["q_full"]), dev(x["k_own"]), dev(x["v_own"]), k_rest, v_rest)
    dq, dk_own, dv_own = hp_share.backward(dev(x["do_full"]))
    torch.cuda.synchronize()
    hq, hkv = H // hp, Hkv // hp
    P = inner * outer
    got = dict(O_full=o.cpu().numpy(), LSE=lse.cpu().numpy(), dQ_full=dq.cpu().numpy(),
               dK_own=dk_own.cpu().numpy(), dV_own=dv_own.cpu().numpy())
    got["O"] = got["O_full"][:, g * hq:(g + 1) * hq]
    got["dQ"] = got["dQ_full"][:, g * hq:(g + 1) * hq]
    # per-chunk dK/dV of this head group, in the chunk order of the ring buffers
    got["dK"] = np.stack([got["dK_own"][:, g * hkv:(g + 1) * hkv] if j == r else
                          hp_share.dk_chunks[j].cpu().numpy() for j in range(P)])
    got["dV"] = np.stack([got["dV_own"][:, g * hkv:(g + 1) * hkv] if j == r else
                          hp_share.dv_chunks[j].cpu().numpy() for j in range(P)])
    other_q = np.ones(H, bool)
    other_q[g * hq:(g + 1) * hq] = False
    other_k = np.ones(Hkv, bool)
    other_k[g * hkv:(g + 1) * hkv] = False
    for name, arr, mask in (("O", got["O_full"], other_q), ("dQ", got["dQ_full"], other_q),
                            ("dK", got["dK_own"], other_k), ("dV", got["dV_own"], other_k)):
        assert bool((arr[:, mask] == np.float32(sentinel)).all()), \
            f"{name}: the other head groups' slots were not carried through unchanged"
    return hp_share, got


@pytest.mark.parametrize("merge", ["fused", "chunks"])
@pytest.mark.parametrize("case", HP_CASES, ids=lambda c: c[0])
def test_head_parallel_share_matches_oracle(case, merge):
    """2D-Attention: head permute of Q/dO and of the own K/V chunk, the ring on
    head group g, inverse permute of O/dQ and of the own chunk's dK/dV. Outputs
    in the all-head layout against the oracle on the full-head tensors
    restricted to group g (query head h uses KV head h div (H/Hkv) throughout)."""
    name, S, inner, outer, r, H, Hkv, d, hp, g = case
    P = inner * outer
    x = head_parallel_inputs(S, P, r, H, Hkv, d, hp, g, seed=6000 + S + r)
    _, got = run_head_parallel(S, inner, outer, r, H, Hkv, d, hp, g, x, merge=merge)
    pos = oracle.zigzag_positions(S, P, r)
    w = lambda a: widen(a, "bf16")
    want = oracle.share_backward(w(x["q"]), w(x["k_nat"]), w(x["v_nat"]), w(x["do"]), pos,
                                 1 / math.sqrt(d))
    assert_close("O", got["O"], want["O"], "bf16")
    assert_close("LSE", got["LSE"], want["LSE"], "bf16", is_lse=True)
    assert_close("dQ", got["dQ"], want["dQ"], "bf16")
    for j in range(P):
        kp = oracle.zigzag_positions(S, P, j)
        assert_close(f"dK[{j}]", got["dK"][j], want["dK"][kp], "bf16")
        assert_close(f"dV[{j}]", got["dV"][j], want["dV"][kp], "bf16")


def _sample_rows(b, n_rand, seed):
    fixed = [0, 1, 31, 32, 63, 64, 127, b - 1, b, b + 1, b + 63, 2 * b - 64, 2 * b - 1]
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([fixed, rng.integers(0, 2 * b, n_rand)]))


def _sample_keys(b, seed):
    """Key rows of a chunk: both blocks, the 32- and 128-key workgroup edges,
    the first and last rows, and a few random ones."""
    fixed = [0, 1, 31, 32, 127, 128, b - 1, b, b + 1, b + 127, b + 128, 2 * b - 1]
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([fixed, rng.integers(0, 2 * b, 4)]))


FULL_SIZE = ["llama3_8b_cp8_128k", "llama3_70b_hp2_cp32_512k", "hp4_cp16_1m", "mha7b_hp8_cp8_1m"]
FULL_CASES = [(c, rank) for c in FULL_SIZE for rank in ("first", "last")]


@pytest.mark.parametrize("cfg_name,which", FULL_CASES, ids=lambda v: str(v))
def test_full_size_share_sampled(cfg_name, which):
    """Each bf16 workload at full size, in the benchmark's launch configuration,
    for the first and the last ring rank.

    Sampled query rows (both zigzag halves, tile edges) of several heads: O,
    LSE, D and dQ from the oracle row by row. Sampled keys of chunks 0, 1 and
    P-1 (both blocks, workgroup edges): dK and dV from the oracle over every
    local row, driven by the GPU's final LSE and D (which the row samples pin).
    Identities over all keys: sum_k dV_k = sum of dO over the group's rows and
    heads, and sum_k dK_k = 0. The 2D-Attention workload runs through the head
    permutes (all-head inputs and outputs, head group 0). The 128K workload
    also runs its backward a second time and must give the same bits."""
    cfg = CONFIGS[cfg_name]
    S, P, hq, hkv, d = cfg.S, cfg.P, cfg.hq, cfg.hkv, cfg.d
    r = 0 if which == "first" else P - 1
    G = hq // hkv
    scale = 1 / math.sqrt(d)
    b = S // (2 * P)
    print(f"[full-size] {cfg_name}: S={S} P={P} rank={r} hq={hq} hkv={hkv}", flush=True)
    if cfg.permute_heads:
        H, Hkv, hp = cfg.permute_heads, hkv * (cfg.permute_heads // hq), cfg.permute_heads // hq
        x = head_parallel_inputs(S, P, r, H, Hkv, d, hp, 0, seed=cfg.seed)
        ring, got = run_head_parallel(S, cfg.inner, cfg.outer, r, H, Hkv, d, hp, 0, x)
        ring = ring.ring
    else:
        x = share_inputs(S, P, r, hq, hkv, d, "bf16", seed=cfg.seed)
        ring, got = run_share(S, cfg.inner, cfg.outer, r, hq, hkv, d, "bf16", x)
    print("[full-size] GPU share done; oracle samples", flush=True)
    pos = oracle.zigzag_positions(S, P, r)
    rows = _sample_rows(b, 16, cfg.seed + r)
    heads = sorted({0, G - 1, hq // 2, hq - 1})
    delta = ring.delta.cpu().numpy()
    for h in heads:
        g = h // G
        kg = widen(x["k_nat"][:, g:g + 1], "bf16")
        vg = widen(x["v_nat"][:, g:g + 1], "bf16")
        qr = widen(x["q"][rows][:, h:h + 1], "bf16")
        dor = widen(x["do"][rows][:, h:h + 1], "bf16")
        res = oracle.share_backward(qr, kg, vg, dor, pos[rows], scale, row_block=16)
        assert_close(f"O h{h}", got["O"][rows][:, h:h + 1], res["O"], "bf16")
        assert_close(f"LSE h{h}", got["LSE"][h:h + 1, rows], res["LSE"], "bf16", is_lse=True)
        assert_close(f"D h{h}", delta[h:h + 1, rows], res["D"], "bf16")
        assert_close(f"dQ h{h}", got["dQ"][rows][:, h:h + 1], res["dQ"], "bf16")
    # dK/dV of sampled keys: every local row of the group's heads contributes
    lse_all = got["LSE"].astype(np.float64)
    for j in sorted({0, 1, P - 1}):
        kp_all = oracle.zigzag_positions(S, P, j)
        keys = _sample_keys(b, cfg.seed + 31 * j)
        for g in sorted({0, hkv - 1}):
            hs_ = slice(g * G, (g + 1) * G)
            kg = widen(x["k_nat"][kp_all[keys]][:, g:g + 1], "bf16")
            vg = widen(x["v_nat"][kp_all[keys]][:, g:g + 1], "bf16")
            _, dk, dv = oracle.step_backward(widen(x["q"][:, hs_], "bf16"), kg, vg,
                                             widen(x["do"][:, hs_], "bf16"), lse_all[hs_],
                                             delta[hs_].astype(np.float64), pos, kp_all[keys],
                                             scale, row_block=2048)
            assert_close(f"dK chunk {j} g{g}", got["dK"][j][keys][:, g:g + 1], dk, "bf16")
            assert_close(f"dV chunk {j} g{g}", got["dV"][j][keys][:, g:g + 1], dv, "bf16")
    do64 = widen(x["do"], "bf16")
    for g in range(hkv):
        dv_sum = got["dV"][:, :, g].astype(np.float64).sum(axis=(0, 1))
        want_sum = do64[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        np.testing.assert_allclose(dv_sum, want_sum, atol=1e-3 * np.abs(want_sum).max() + 1e-2)
        dk_g = got["dK"][:, :, g].astype(np.float64)
        assert np.abs(dk_g.sum(axis=(0, 1))).max() <= 1e-3 * np.abs(dk_g).sum(axis=(0, 1)).max()
    if cfg_name == "llama3_8b_cp8_128k":
        q, do = to_device(x["q"], "bf16"), to_device(x["do"], "bf16")
        K, V = to_device(x["k_ch"], "bf16"), to_device(x["v_ch"], "bf16")
        dq2, dk2, dv2 = ring.backward(q, K, V, do)
        torch.cuda.synchronize()
        assert np.array_equal(dq2.cpu().numpy(), got["dQ"]), "dQ not bitwise repeatable"
        assert np.array_equal(dk2.cpu().numpy(), got["dK"]), "dK not bitwise repeatable"
        assert np.array_equal(dv2.cpu().numpy(), got["dV"]), "dV not bitwise repeatable"

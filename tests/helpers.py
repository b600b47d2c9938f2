"""Shared test helpers: seeded share inputs (numpy + device), error reports.

Every GPU-vs-oracle comparison made through :func:`assert_close` is appended,
with its test id, error and bar, to the JSON-lines file named by the
RA_PARITY_LOG environment variable (if set), so that the margins of a run can
be tabulated (tests/parity_margins.py).
"""
import json
import os

import numpy as np

from ring_attention_attn_amd import synth


def share_inputs(S, P, r, hq, hkv, d, dtype, seed, layout="zigzag"):
    """Seeded inputs of rank r's share.

    Returns a dict of host arrays in the input dtype (uint16 bf16 bits or
    float32): q, dout [L][hq][d] (rows of blocks r, 2P-1-r), K/V chunks
    [P][L][hkv][d] (chunk j = blocks j, 2P-1-j), and the natural-order K/V
    [S][hkv][d]; plus fp64 widenings (exact) for the oracle."""
    b = S // (2 * P)
    blocks_of = synth.paired_blocks if layout == "zigzag" else synth.contiguous_blocks
    mine = blocks_of(P, r)
    q = synth.blocks_tensor(seed, synth.T_Q, mine, b, hq, d, dtype)
    do = synth.blocks_tensor(seed, synth.T_DO, mine, b, hq, d, dtype)
    k_nat = synth.blocks_tensor(seed, synth.T_K, range(2 * P), b, hkv, d, dtype)
    v_nat = synth.blocks_tensor(seed, synth.T_V, range(2 * P), b, hkv, d, dtype)

    # chunk j = its blocks in order, gathered in one copy per tensor
    idx = np.array([blocks_of(P, j) for j in range(P)])

    def chunks(nat):
        return nat.reshape(2 * P, b, hkv, d)[idx].reshape(P, 2 * b, hkv, d)

    return dict(q=q, do=do, k_nat=k_nat, v_nat=v_nat, k_ch=chunks(k_nat), v_ch=chunks(v_nat), b=b)


def widen(x, dtype):
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def to_device(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    both_ninf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):  # -inf - -inf: masked by both_ninf
        diff = np.where(both_ninf, 0.0, np.abs(a - b))
    return float(np.nanmax(np.where(np.isnan(diff), np.inf, diff)))


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))


# parity bars: max abs error on O/dQ/dK/dV and on LSE, per input dtype
TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}
REL_L2_BAR = 1e-2   # non-triviality check beside the absolute bar (bf16)


CURRENT_TEST = None   # set per test by tests/conftest.py


def _record(name, dtype, is_lse, err, atol, rl):
    path = os.environ.get("RA_PARITY_LOG")
    if not path:
        return
    rec = dict(test=CURRENT_TEST, tensor=name, dtype=dtype, kind="lse" if is_lse else "value",
               max_abs=err, bar=atol, rel_l2=rl)
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def assert_close(name, got, want, dtype, is_lse=False):
    atol = TOL[dtype][1 if is_lse else 0]
    err = max_abs(got, want)
    rl = rel_l2(got, want) if not is_lse else None
    _record(name, dtype, is_lse, err, atol, rl)
    assert err <= atol, f"{name}: max abs err {err:.3e} > {atol:.1e}"
    if dtype == "bf16" and not is_lse:
        assert rl <= REL_L2_BAR, f"{name}: rel L2 {rl:.3e} > {REL_L2_BAR:.0e}"
    return err

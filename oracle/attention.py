"""Forward and backward of causal softmax attention for one GPU's query rows, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed is the plain definition, written out directly:

* "Guide to LoongTrain", "Step 3" reference code: scores = Q K^T * scale with
  scale = 1/sqrt(head_dim), masked keys get -inf, probabilities = softmax over
  keys, output = probabilities @ V.
* Causal rule ("The Communication Overhead and Causal Imbalance of Ring
  Attention"): the query at global position p sees the key at position p' iff
  p' <= p. Positions come from the paired-block map (``index_maps``).
* A ring step ("rank i receives (K_j, V_j) from rank i-1 and attends with its
  local Q_i", same section) is the same definition restricted to the keys of
  one chunk; the pages give no merge and no log-sum-exp, so the readings taken
  are: LSE in natural log, a row with no visible key in the chunk has O = 0 and
  LSE = -inf, and partial results combine by the max-shifted log-sum-exp rule
  (:func:`lse_merge`).
* Backward: the exact gradient of sum(dO * O) with respect to Q, K, V, written
  out with P = exp(s - LSE) and D = rowsum(dO * O) (the pages give no backward;
  this is calculus, pinned by finite differences). K/V heads are shared by
  Hq/Hkv query heads (grouped-query attention, "The Scalability Limits of
  DeepSpeed Ulysses"); query head h uses KV head h // (Hq/Hkv), so dK/dV sum over
  the group.

Layouts (token-major, as the head transpose of the Ulysses section has them):
Q, O, dO, dQ are [L][Hq][d]; K, V, dK, dV are [Lk][Hkv][d]; LSE and D are [Hq][L].
The arithmetic is a straightforward two-pass softmax per block of query rows;
row blocking only bounds memory and does not change any sum.
"""
import numpy as np

NEG_INF = -np.inf


def bf16_bits_to_f64(bits):
    """Widen bfloat16 bit patterns (uint16) to fp64 exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _kv_head(h, Hq, Hkv):
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _check(q, k, v, pos_q, pos_k):
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape:
        raise ValueError("expected q [L][Hq][d], k/v [Lk][Hkv][d]")
    if q.shape[2] != k.shape[2]:
        raise ValueError("head_dim mismatch")
    if len(pos_q) != q.shape[0] or len(pos_k) != k.shape[0]:
        raise ValueError("positions do not match rows")


def _row_blocks(L, rb):
    for i0 in range(0, L, rb):
        yield i0, min(L, i0 + rb)


def step_forward(q, k, v, pos_q, pos_k, scale, row_block=128):
    """Attention of query rows (positions ``pos_q``) against one key set (positions
    ``pos_k``), causal. Returns (O [L][Hq][d], LSE [Hq][L]) in fp64.

    Rows with no visible key: O = 0, LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    _check(q, k, v, pos_q, pos_k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    O = np.zeros((L, Hq, d), dtype=np.float64)
    LSE = np.full((Hq, L), NEG_INF, dtype=np.float64)
    for h in range(Hq):
        g = _kv_head(h, Hq, Hkv)
        kg = k[:, g, :]
        vg = v[:, g, :]
        for i0, i1 in _row_blocks(L, row_block):
            s = scale * (q[i0:i1, h, :] @ kg.T)
            visible = pos_k[None, :] <= pos_q[i0:i1, None]
            s = np.where(visible, s, NEG_INF)
            any_vis = visible.any(axis=1)
            m = np.where(any_vis, s.max(axis=1, initial=NEG_INF), 0.0)
            e = np.where(visible, np.exp(s - m[:, None]), 0.0)
            tot = e.sum(axis=1)
            lse = np.where(any_vis, m + np.log(np.where(any_vis, tot, 1.0)), NEG_INF)
            p = np.where(visible, np.exp(s - np.where(any_vis, lse, 0.0)[:, None]), 0.0)
            O[i0:i1, h, :] = p @ vg
            LSE[h, i0:i1] = lse
    return O, LSE


def share_forward(q, k_full, v_full, pos_q, scale, row_block=128):
    """Full-sequence causal attention for this share's rows: the keys are the
    whole sequence in natural token order (key row t is position t)."""
    S = np.asarray(k_full).shape[0]
    return step_forward(q, k_full, v_full, pos_q, np.arange(S, dtype=np.int64), scale,
                        row_block=row_block)


def step_backward(q, k, v, dout, lse, delta, pos_q, pos_k, scale, row_block=128):
    """Gradient pieces of one key set, driven by the FINAL per-row LSE and D.

    P_ik = exp(s_ik - LSE_i) on visible pairs (0 elsewhere); dP_ik = dO_i . v_k;
    dS_ik = P_ik (dP_ik - D_i); dQ_i = scale sum_k dS_ik k_k;
    dK_k = scale sum_i dS_ik q_i; dV_k = sum_i P_ik dO_i; dK, dV summed over the
    query heads sharing the KV head. Returns (dQ [L][Hq][d], dK, dV [Lk][Hkv][d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    _check(q, k, v, pos_q, pos_k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for h in range(Hq):
        g = _kv_head(h, Hq, Hkv)
        kg = k[:, g, :]
        vg = v[:, g, :]
        for i0, i1 in _row_blocks(L, row_block):
            s = scale * (q[i0:i1, h, :] @ kg.T)
            visible = pos_k[None, :] <= pos_q[i0:i1, None]
            lrow = lse[h, i0:i1]
            p = np.where(visible, np.exp(np.where(visible, s, 0.0) - lrow[:, None]), 0.0)
            dp = dout[i0:i1, h, :] @ vg.T
            ds = p * (dp - delta[h, i0:i1, None])
            dQ[i0:i1, h, :] = scale * (ds @ kg)
            dK[:, g, :] += scale * (ds.T @ q[i0:i1, h, :])
            dV[:, g, :] += p.T @ dout[i0:i1, h, :]
    return dQ, dK, dV


def share_backward(q, k_full, v_full, dout, pos_q, scale, row_block=128):
    """Forward plus exact backward over the whole sequence for this share's rows.

    Returns a dict with O, LSE, D (= rowsum(dO * O), [Hq][L]), dQ, and dK, dV over
    all S key positions (natural order): this share's contribution only.
    """
    S = np.asarray(k_full).shape[0]
    pos_k = np.arange(S, dtype=np.int64)
    O, LSE = step_forward(q, k_full, v_full, pos_q, pos_k, scale, row_block=row_block)
    dout = np.asarray(dout, dtype=np.float64)
    D = np.einsum("lhd,lhd->hl", dout, O)
    dQ, dK, dV = step_backward(q, k_full, v_full, dout, LSE, D, pos_q, pos_k, scale,
                               row_block=row_block)
    return {"O": O, "LSE": LSE, "D": D, "dQ": dQ, "dK": dK, "dV": dV}


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial results over disjoint key sets (online-softmax rescale).

    m = max(L_a, L_b); if m = -inf both are empty and the result is (0, -inf);
    else L = m + ln(e^(L_a - m) + e^(L_b - m)) and O = e^(L_a - L) O_a + e^(L_b - L) O_b.
    O: [L][H][d]; LSE: [H][L]. Reading of "merged by online-softmax rescaling";
    the pages print no formula.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    ms = np.where(empty, 0.0, m)
    wa = np.exp(lse_a - ms)
    wb = np.exp(lse_b - ms)
    tot = wa + wb
    lse = np.where(empty, NEG_INF, ms + np.log(np.where(empty, 1.0, tot)))
    ls = np.where(empty, 0.0, lse)
    ca = np.where(empty, 0.0, np.exp(lse_a - ls))  # [H][L]
    cb = np.where(empty, 0.0, np.exp(lse_b - ls))
    o = ca.T[:, :, None] * o_a + cb.T[:, :, None] * o_b
    return o, lse

"""Integer index maps of the share (oracle side; test infrastructure only).

Written from the definitions, with plain Python loops where sizes are small.
"""
import numpy as np


def chunk_blocks(P, r):
    """Blocks held by ring rank ``r`` of ``P``.

    "Guide to LoongTrain", section "2. Paired-Block Allocation for Causal Load
    Balancing": the sequence is cut into 2P blocks and rank r keeps block A_r = r
    (front) and block B_r = 2P - 1 - r (back), in that order.
    """
    if not (0 <= r < P):
        raise ValueError("rank out of range")
    return (r, 2 * P - 1 - r)


def zigzag_positions(S, P, r):
    """Global token positions of the 2b local rows of rank ``r`` (b = S / 2P).

    Row i < b is token r*b + i (block A); row b + i is token (2P-1-r)*b + i
    (block B). Same section as :func:`chunk_blocks`. A KV chunk j uses the same
    map with r := j.
    """
    if S % (2 * P) != 0:
        raise ValueError("S must be a multiple of 2P")
    b = S // (2 * P)
    out = []
    for blk in chunk_blocks(P, r):
        for i in range(b):
            out.append(blk * b + i)
    return np.array(out, dtype=np.int64)


def contiguous_positions(S, P, r):
    """Global token positions of rank ``r``'s rows when the sequence is sliced
    into P consecutive chunks and rank r holds chunk r (the layout whose causal
    load imbalance the paired blocks remove): tokens r*S/P .. (r+1)*S/P - 1.

    "Guide to LoongTrain", section "The Communication Overhead and Causal
    Imbalance of Ring Attention" (P chunks, GPU 0 holding the earliest chunk and
    GPU P-1 the latest). A KV chunk j uses the same map with r := j.
    """
    if not (0 <= r < P):
        raise ValueError("rank out of range")
    if S % P != 0:
        raise ValueError("S must be a multiple of P")
    L = S // P
    return np.array([r * L + i for i in range(L)], dtype=np.int64)


def causal_pair_count(pos_q, S):
    """Number of visible (query, key) pairs for query rows ``pos_q`` against the
    whole sequence of length S: query at position p sees keys 0..p.

    "Guide to LoongTrain", section "The Communication Overhead and Causal
    Imbalance of Ring Attention" (q_i sees k_j iff j <= i); the "Workload(r)"
    equation of the paired-block section says this is the same for every rank.
    """
    total = 0
    for p in pos_q.tolist():
        if not (0 <= p < S):
            raise ValueError("position out of range")
        total += p + 1
    return total


def double_ring_order(inner, outer, r):
    """Source chunk id visited by rank ``r`` at each step t = 0 .. inner*outer-1.

    The ring moves K/V one hop per step from the predecessor (rank i receives
    (K_j, V_j) from rank i-1: "Guide to LoongTrain", section "The Communication
    Overhead and Causal Imbalance of Ring Attention"), so at step t a plain ring
    of P ranks holds chunk (r - t) mod P. The double ring (abstract of the
    LoongTrain paper; "3. Double-Ring Asynchronous Communication Pipeline")
    nests two such rings: ranks form groups of ``inner`` consecutive ids; the
    inner ring turns fastest inside a group, the outer ring moves between
    groups once every ``inner`` steps. Reading taken: t = o*inner + i,
    r = g*inner + l, chunk = ((g - o) mod outer)*inner + ((l - i) mod inner).

    parity unpinned by the pages beyond: step 0 is the rank's own chunk, each
    order is a permutation of 0..P-1, and outer == 1 is the plain ring.
    """
    P = inner * outer
    if inner < 1 or outer < 1 or not (0 <= r < P):
        raise ValueError("bad ring shape")
    g, l = divmod(r, inner)
    order = []
    for o in range(outer):
        for i in range(inner):
            order.append(((g - o) % outer) * inner + ((l - i) % inner))
    return np.array(order, dtype=np.int32)


def head_permute(src, P, inverse=False):
    """Local layout of the head-parallel (Ulysses) all-to-all.

    "Guide to LoongTrain", section "The Scalability Limits of DeepSpeed Ulysses":
    the all-to-all turns (S/P, H) into (S, H/P) before attention and back after.
    On one device it is a pure permutation: forward maps src[s][h][x] (shape
    [S][H][d]) to dst[p][s][h'][x] (shape [P][S][H/P][d]) with h = p*(H/P) + h',
    i.e. destination p gets the contiguous head group p. ``inverse`` undoes it.
    The caps of the same section (each of the P destinations needs whole heads)
    give the check H % P == 0.
    """
    if inverse:
        Pn, S, Hp, d = src.shape
        if Pn != P:
            raise ValueError("leading dim must be P")
        H = Hp * P
        dst = np.empty((S, H, d), dtype=src.dtype)
        for p in range(P):
            for hh in range(Hp):
                dst[:, p * Hp + hh, :] = src[p, :, hh, :]
        return dst
    S, H, d = src.shape
    if H % P != 0:
        raise ValueError("H must be a multiple of P")
    Hp = H // P
    dst = np.empty((P, S, Hp, d), dtype=src.dtype)
    for p in range(P):
        for hh in range(Hp):
            dst[p, :, hh, :] = src[:, p * Hp + hh, :]
    return dst

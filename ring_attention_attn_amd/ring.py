"""Virtual ring over one GPU's share: the step sequence of ring attention with
every step run by the library's kernels.

On one device the ring is a loop over the KV chunks (all resident in HBM) in
the double-ring visit order, where a multi-GPU ring would receive chunk j from
its predecessor at step t ("Guide to LoongTrain", "The Communication Overhead
and Causal Imbalance of Ring Attention"; "3. Double-Ring Asynchronous
Communication Pipeline"). Forward: the first step writes the running (O, LSE)
directly; every later step is folded into it, either by the fused
ring_attn_step_fwd_merge (default) or by ring_attn_step_fwd then lse_merge
(merge="separate"). Backward: ra_bwd_delta (D = rowsum(dO O) and O in bf16), dq
cleared with ra_fill_f32, then ring_attn_step_bwd per step with the final LSE.

PyTorch only allocates device memory and provides the stream.
"""
import torch

from . import binding as B

_RA_DTYPE = {"bf16": B.RA_BF16, "f32": B.RA_F32}


class ShareRing:
    """Buffers and precomputed step descriptors of one rank's share.

    kv_rings="ab" runs each step as two launches, one per block of the chunk
    (the two rings of the double-ring pipeline, one carrying block A and one
    block B; "3. Double-Ring Asynchronous Communication Pipeline").

    Inputs (caller-owned, contiguous): q [L][hq][d], K/V [P][L][hkv][d] (chunk j
    = rows of blocks j and 2P-1-j), dout [L][hq][d]; L = 2b rows, b = S/(2P).
    layout="contiguous" instead gives rank r (and chunk j) the L consecutive
    tokens r*L .. r*L+L-1, the layout whose causal imbalance the paired blocks
    remove; the kernels are the same (one segment instead of two).
    """

    def __init__(self, S, inner, outer, rank, hq, hkv, d, dtype="bf16", scale=None,
                 device="cuda", causal=1, merge="fused", layout="zigzag", kv_rings="one"):
        if merge not in ("fused", "separate"):
            raise ValueError(f"merge must be 'fused' or 'separate', not {merge!r}")
        if layout not in ("zigzag", "contiguous"):
            raise ValueError(f"layout must be 'zigzag' or 'contiguous', not {layout!r}")
        if kv_rings not in ("one", "ab") or (kv_rings == "ab" and layout != "zigzag"):
            raise ValueError("kv_rings must be 'one', or 'ab' with the paired-block layout")
        self.merge, self.layout, self.kv_rings = merge, layout, kv_rings
        self.S, self.inner, self.outer, self.rank = S, inner, outer, rank
        self.P = inner * outer
        self.hq, self.hkv, self.d, self.dtype = hq, hkv, d, dtype
        self.scale = scale if scale is not None else d ** -0.5
        def segments(r):
            # zigzag: two paired blocks of b rows; contiguous: one chunk of 2b rows
            if layout == "zigzag":
                return B.ra_zigzag_segments(S, self.P, r)
            L = S // self.P
            return (r * L,), L

        q_seg, b = segments(rank)
        self.L = 2 * b if layout == "zigzag" else b
        self.order = [int(j) for j in B.ra_double_ring_order(inner, outer, rank)]
        f32 = dict(dtype=torch.float32, device=device)
        L = self.L
        self.o_acc = torch.empty((L, hq, d), **f32)
        self.lse_acc = torch.empty((hq, L), **f32)
        self.o_step = torch.empty((L, hq, d), **f32)
        self.lse_step = torch.empty((hq, L), **f32)
        self.delta = torch.empty((hq, L), **f32)
        self.dq = torch.empty((L, hq, d), **f32)
        self.dk = torch.empty((self.P, L, hkv, d), **f32)
        self.dv = torch.empty((self.P, L, hkv, d), **f32)
        self.o_lowp = torch.empty((L, hq, d), dtype=torch.bfloat16, device=device)
        def desc(k_seg, kb, acc):
            return B.make_desc(dtype=_RA_DTYPE[dtype], head_dim=d, hq=hq, hkv=hkv,
                               q_segments=(q_seg, b), k_segments=(k_seg, kb), scale=self.scale,
                               causal=causal, q_strides=(hq * d, d), k_strides=(hkv * d, d),
                               v_strides=(hkv * d, d), o_strides=(hq * d, d),
                               do_strides=(hq * d, d), dk_strides=(hkv * d, d),
                               dkv_accumulate=acc)

        # launches in order: (chunk j, row offset of the K/V rows in the chunk, desc)
        self.launches = []
        for j in self.order:
            k_seg, kb = segments(j)
            if kv_rings == "one":
                self.launches.append((j, 0, desc(k_seg, kb, 0)))
            else:
                # two rings, one carrying block A and one block B of each chunk
                # (each a one-segment key map; each launch writes dK/dV of its
                # own block's rows, which no other launch touches)
                self.launches.append((j, 0, desc((k_seg[0],), kb, 0)))
                self.launches.append((j, kb, desc((k_seg[1],), kb, 0)))

    def _kv(self, X, j, off):
        return X[j] if off == 0 else X[j][off:]

    def forward(self, q, K, V, stream=None):
        """Running (O fp32 [L][hq][d], LSE fp32 [hq][L]) after all P steps."""
        for t, (j, off, desc) in enumerate(self.launches):
            k, v = self._kv(K, j, off), self._kv(V, j, off)
            if t == 0:
                B.ring_attn_step_fwd(desc, q, k, v, self.o_acc, self.lse_acc, stream)
            elif self.merge == "fused":
                B.ring_attn_step_fwd_merge(desc, q, k, v, self.o_acc, self.lse_acc, stream)
            else:
                B.ring_attn_step_fwd(desc, q, k, v, self.o_step, self.lse_step, stream)
                B.lse_merge(self.L, self.hq, self.d, self.o_acc, self.lse_acc, self.o_step,
                            self.lse_step, stream)
        return self.o_acc, self.lse_acc

    def backward(self, q, K, V, dout, stream=None):
        """dQ fp32 [L][hq][d] and per-chunk dK, dV fp32 [P][L][hkv][d] of this share,
        using the forward's final O and LSE (call forward first)."""
        B.ra_bwd_delta(self.L, self.hq, self.d, _RA_DTYPE[self.dtype], self.o_acc, dout,
                       self.delta, self.o_lowp if self.dtype == "bf16" else None, stream)
        B.ra_fill_f32(self.dq, self.dq.numel(), 0.0, stream)
        for j, off, desc in self.launches:
            B.ring_attn_step_bwd(desc, q, self._kv(K, j, off), self._kv(V, j, off), dout,
                                 self.lse_acc, self.delta, self.dq, self._kv(self.dk, j, off),
                                 self._kv(self.dv, j, off), stream)
        return self.dq, self.dk, self.dv

    def step(self, q, K, V, dout, stream=None):
        """One pass of the whole path: forward over all steps, then backward."""
        self.forward(q, K, V, stream)
        return self.backward(q, K, V, dout, stream)

"""Virtual ring over one GPU's share: the step sequence of ring attention with
every step run by the library's kernels.

On one device the ring is a loop over the KV chunks (all resident in HBM) in
the double-ring visit order, where a multi-GPU ring would receive chunk j from
its predecessor at step t ("Guide to LoongTrain", "The Communication Overhead
and Causal Imbalance of Ring Attention"; "3. Double-Ring Asynchronous
Communication Pipeline"). Forward: the first step writes the running (O, LSE)
directly; every later step is folded into it, either by the fused
ring_attn_step_fwd_merge (default) or by ring_attn_step_fwd then lse_merge
(merge="separate", over the rows the step gave any visible key); merge="chunks"
runs all steps in one ring_attn_fwd_chunks launch and the backward as one
ring_attn_bwd_chunks call (bf16). Backward:
ra_bwd_delta (D = rowsum(dO O) and O in bf16), dq cleared with ra_fill_f32,
then ring_attn_step_bwd per step with the final LSE.

HeadParallelShare wraps the ring in the local layout change of the head
all-to-all of 2D-Attention ("The Scalability Limits of DeepSpeed Ulysses":
(S/P, H) -> (S, H/P) before attention, back after it), so that the share takes
and returns tensors with every head.

PyTorch only allocates device memory and provides the stream.
"""
import contextlib

import torch

from . import binding as B

_RA_DTYPE = {"bf16": B.RA_BF16, "f32": B.RA_F32}
_UNTIMED = contextlib.nullcontext()


class _Timed:
    """``timer``: None, or a callable kind -> context manager that a caller
    (a benchmark) wraps around each launch of that kind; it sees the launches
    the library makes, in order, and changes nothing about them."""
    timer = None

    def _t(self, kind):
        return self.timer(kind) if self.timer is not None else _UNTIMED


class ShareRing(_Timed):
    """Buffers and precomputed step descriptors of one rank's share.

    kv_rings="ab" runs each step as two launches, one per block of the chunk
    (the two rings of the double-ring pipeline, one carrying block A and one
    block B; "3. Double-Ring Asynchronous Communication Pipeline").

    Inputs (caller-owned, contiguous): q [L][hq][d], K/V [P][L][hkv][d] (chunk j
    = rows of blocks j and 2P-1-j; a sequence of P [L][hkv][d] tensors works as
    well), dout [L][hq][d]; L = 2b rows, b = S/(2P).
    layout="contiguous" instead gives rank r (and chunk j) the L consecutive
    tokens r*L .. r*L+L-1, the layout whose causal imbalance the paired blocks
    remove; the kernels are the same (one segment instead of two).

    ``buffers`` may supply the output buffers (o_acc, dq: [L][hq][d] fp32;
    dk, dv: P-sequences of [L][hkv][d] fp32 or [P][L][hkv][d]) so that the
    results land where a caller wants them, e.g. in an exchange buffer.
    """

    def __init__(self, S, inner, outer, rank, hq, hkv, d, dtype="bf16", scale=None,
                 device="cuda", causal=1, merge="fused", layout="zigzag", kv_rings="one",
                 buffers=None):
        if merge not in ("fused", "separate", "chunks"):
            raise ValueError(f"merge must be 'fused', 'separate' or 'chunks', not {merge!r}")
        if merge == "chunks" and dtype != "bf16":
            raise ValueError("merge='chunks' (all steps in one launch) runs the bf16 kernels only")
        if layout not in ("zigzag", "contiguous"):
            raise ValueError(f"layout must be 'zigzag' or 'contiguous', not {layout!r}")
        if kv_rings not in ("one", "ab") or (kv_rings == "ab" and layout != "zigzag"):
            raise ValueError("kv_rings must be 'one', or 'ab' with the paired-block layout")
        self.merge, self.layout, self.kv_rings = merge, layout, kv_rings
        self.S, self.inner, self.outer, self.rank = S, inner, outer, rank
        self.P = inner * outer
        self.hq, self.hkv, self.d, self.dtype = hq, hkv, d, dtype
        self.scale = scale if scale is not None else d ** -0.5
        self.causal = causal

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
        buffers = dict(buffers or {})
        self.o_acc = buffers.pop("o_acc", None)
        if self.o_acc is None:
            self.o_acc = torch.empty((L, hq, d), **f32)
        self.dq = buffers.pop("dq", None)
        if self.dq is None:
            self.dq = torch.empty((L, hq, d), **f32)
        self.dk = buffers.pop("dk", None)
        if self.dk is None:
            self.dk = torch.empty((self.P, L, hkv, d), **f32)
        self.dv = buffers.pop("dv", None)
        if self.dv is None:
            self.dv = torch.empty((self.P, L, hkv, d), **f32)
        if buffers:
            raise ValueError(f"unknown buffers: {sorted(buffers)}")
        self.lse_acc = torch.empty((hq, L), **f32)
        self.o_step = torch.empty((L, hq, d), **f32)
        self.lse_step = torch.empty((hq, L), **f32)
        self.delta = torch.empty((hq, L), **f32)
        self.o_lowp = torch.empty((L, hq, d), dtype=torch.bfloat16, device=device)

        def desc(k_seg, kb, acc):
            return B.make_desc(dtype=_RA_DTYPE[dtype], head_dim=d, hq=hq, hkv=hkv,
                               q_segments=(q_seg, b), k_segments=(k_seg, kb), scale=self.scale,
                               causal=causal, q_strides=(hq * d, d), k_strides=(hkv * d, d),
                               v_strides=(hkv * d, d), o_strides=(hq * d, d),
                               do_strides=(hq * d, d), dk_strides=(hkv * d, d),
                               dkv_accumulate=acc)

        # query positions in row order (increasing along the rows in both
        # layouts: block A precedes block B), for the merge's row range
        q_first = [p for p in q_seg]
        self._q_runs = [(q_first[i], i * b, b) for i in range(len(q_first))]

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
        if merge == "chunks" and len(self.launches) > B.RA_MAX_CHUNKS:
            raise ValueError(f"merge='chunks' takes at most {B.RA_MAX_CHUNKS} launches per call, "
                             f"this ring has {len(self.launches)}")

    def _kv(self, X, j, off):
        return X[j] if off == 0 else X[j][off:]

    def merge_rows(self, desc):
        """(row_begin, row_count): the query rows with a visible key in the
        launch's key set (all rows when not causal). Causally a row sees a key
        of the set iff its position is at or after the set's first position; the
        rows' positions increase along the buffer, so these rows are a suffix."""
        if not self.causal:
            return 0, self.L
        k_min = min(desc.k_seg_pos[i] for i in range(desc.k_nseg))
        first = 0
        for pos0, row0, n in self._q_runs:
            if pos0 + n - 1 < k_min:
                first = row0 + n           # the whole run is earlier than every key
            elif pos0 < k_min:
                first = row0 + (k_min - pos0)
        return first, self.L - first

    def forward(self, q, K, V, stream=None):
        """Running (O fp32 [L][hq][d], LSE fp32 [hq][L]) after all P steps."""
        if self.merge == "chunks":
            ks = [self._kv(K, j, off) for j, off, _ in self.launches]
            vs = [self._kv(V, j, off) for j, off, _ in self.launches]
            with self._t("step_fwd"):
                B.ring_attn_fwd_chunks([d for _, _, d in self.launches], q, ks, vs, self.o_acc,
                                       self.lse_acc, stream)
            return self.o_acc, self.lse_acc
        for t, (j, off, desc) in enumerate(self.launches):
            k, v = self._kv(K, j, off), self._kv(V, j, off)
            if t == 0:
                with self._t("step_fwd"):
                    B.ring_attn_step_fwd(desc, q, k, v, self.o_acc, self.lse_acc, stream)
            elif self.merge == "fused":
                with self._t("step_fwd"):
                    B.ring_attn_step_fwd_merge(desc, q, k, v, self.o_acc, self.lse_acc, stream)
            else:
                with self._t("step_fwd"):
                    B.ring_attn_step_fwd(desc, q, k, v, self.o_step, self.lse_step, stream)
                r0, n = self.merge_rows(desc)
                with self._t("lse_merge"):
                    B.lse_merge(self.L, self.hq, self.d, self.o_acc, self.lse_acc, self.o_step,
                                self.lse_step, stream, row_begin=r0, row_count=n)
        return self.o_acc, self.lse_acc

    def backward(self, q, K, V, dout, stream=None):
        """dQ fp32 [L][hq][d] and per-chunk dK, dV fp32 [L][hkv][d] of this share,
        using the forward's final O and LSE (call forward first)."""
        with self._t("bwd_delta"):
            B.ra_bwd_delta(self.L, self.hq, self.d, _RA_DTYPE[self.dtype], self.o_acc, dout,
                           self.delta, self.o_lowp if self.dtype == "bf16" else None, stream)
        if self.merge == "chunks":
            L = self.launches
            with self._t("step_bwd"):
                B.ring_attn_bwd_chunks([d for _, _, d in L], q, [self._kv(K, j, o) for j, o, _ in L],
                                       [self._kv(V, j, o) for j, o, _ in L], dout, self.lse_acc,
                                       self.delta, self.dq, [self._kv(self.dk, j, o) for j, o, _ in L],
                                       [self._kv(self.dv, j, o) for j, o, _ in L], stream)
            return self.dq, self.dk, self.dv
        with self._t("fill"):
            B.ra_fill_f32(self.dq, self.dq.numel(), 0.0, stream)
        for j, off, desc in self.launches:
            with self._t("step_bwd"):
                B.ring_attn_step_bwd(desc, q, self._kv(K, j, off), self._kv(V, j, off), dout,
                                     self.lse_acc, self.delta, self.dq, self._kv(self.dk, j, off),
                                     self._kv(self.dv, j, off), stream)
        return self.dq, self.dk, self.dv

    def step(self, q, K, V, dout, stream=None):
        """One pass of the whole path: forward over all steps, then backward."""
        self.forward(q, K, V, stream)
        return self.backward(q, K, V, dout, stream)


class HeadParallelShare(_Timed):
    """One GPU's share of 2D-Attention: head group ``group`` of ``hp`` and ring
    rank ``rank``, taking and returning tensors with all heads.

    "Guide to LoongTrain", "The Scalability Limits of DeepSpeed Ulysses": the
    head all-to-all turns (S/P, H) into (S, H/P) before attention and back after
    it. On one GPU the all-to-all's data movement is the local permute
    head_permute: [L][H][d] -> [hp][L][H/hp][d], slot p being what head-parallel
    rank p receives (the head group p, all of the chunk's tokens), and its
    inverse [hp][L][H/hp][d] -> [L][H][d] on the way back. This share fills slot
    ``group`` of each exchange buffer; the other slots stand for what the other
    head-parallel ranks would deliver (left as they are on one GPU).

    Permuted here: the local rows' Q and dO ([L][H][d]) and the ring rank's own
    K/V chunk ([L][Hkv][d]); the other chunks arrive through the ring already in
    head-group layout ([L][Hkv/hp][d]), as their owners permuted them.
    Inverse-permuted: O and dQ ([L][H][d] fp32) and the own chunk's dK/dV
    ([L][Hkv][d] fp32). Head h of group p is local head h - p*H/hp; KV head
    numbering follows the same grouping, so the query-to-KV head map stays local.
    """

    def __init__(self, S, inner, outer, rank, H, Hkv, d, hp, group=0, dtype="bf16",
                 device="cuda", **ring_kw):
        if H % hp or Hkv % hp:
            raise ValueError("the head-parallel degree must divide the query and KV heads")
        if not (0 <= group < hp):
            raise ValueError("head group out of range")
        self.H, self.Hkv, self.hp, self.group, self.d = H, Hkv, hp, group, d
        self.hq, self.hkv = H // hp, Hkv // hp
        self.eb = 2 if dtype == "bf16" else 4
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        P = inner * outer
        b = S // (2 * P)
        L = 2 * b if ring_kw.get("layout", "zigzag") == "zigzag" else S // P
        self.L, self.P, self.rank = L, P, rank
        f32 = dict(dtype=torch.float32, device=device)
        low = dict(dtype=tdt, device=device)
        # exchange buffers: [hp][...] with slot `group` this share's
        self.q_x = torch.empty((hp, L, self.hq, d), **low)
        self.do_x = torch.empty((hp, L, self.hq, d), **low)
        self.k_x = torch.empty((hp, L, self.hkv, d), **low)
        self.v_x = torch.empty((hp, L, self.hkv, d), **low)
        self.o_x = torch.empty((hp, L, self.hq, d), **f32)
        self.dq_x = torch.empty((hp, L, self.hq, d), **f32)
        self.dk_x = torch.empty((hp, L, self.hkv, d), **f32)
        self.dv_x = torch.empty((hp, L, self.hkv, d), **f32)
        # outputs with all heads
        self.o = torch.empty((L, H, d), **f32)
        self.dq = torch.empty((L, H, d), **f32)
        self.dk_own = torch.empty((L, Hkv, d), **f32)
        self.dv_own = torch.empty((L, Hkv, d), **f32)
        # dK/dV of the other chunks stay in head-group layout (they go back to
        # their owners through the ring)
        dk = [self.dk_x[group] if j == rank else torch.empty((L, self.hkv, d), **f32)
              for j in range(P)]
        dv = [self.dv_x[group] if j == rank else torch.empty((L, self.hkv, d), **f32)
              for j in range(P)]
        self.ring = ShareRing(S, inner, outer, rank, self.hq, self.hkv, d, dtype, device=device,
                              buffers=dict(o_acc=self.o_x[group], dq=self.dq_x[group], dk=dk,
                                           dv=dv), **ring_kw)
        self.dk_chunks, self.dv_chunks = dk, dv

    @property
    def timer(self):
        return self.ring.timer

    @timer.setter
    def timer(self, t):
        self.ring.timer = t

    def _permute(self, src, dst, heads, inverse, eb, stream):
        with self._t("head_permute"):
            B.head_permute(src, dst, self.L, heads, self.d, self.hp, eb, inverse, stream)

    def step(self, q_full, K_own, V_own, K_rest, V_rest, dout_full, stream=None):
        """One pass of the whole path: permutes, forward ring, backward ring,
        inverse permutes."""
        self.forward(q_full, K_own, V_own, K_rest, V_rest, stream)
        return self.backward(dout_full, stream)

    def _chunks(self, K_own, K_rest, x):
        """The ring's K (or V) chunk list: the own chunk from the exchange slot."""
        return [x[self.group] if j == self.rank else K_rest[j] for j in range(self.P)]

    def forward(self, q_full, K_own, V_own, K_rest, V_rest, stream=None):
        """q_full [L][H][d], K_own/V_own [L][Hkv][d] (the rank's chunk, all KV
        heads), K_rest/V_rest: P-sequences whose entry j != rank is chunk j in
        head-group layout [L][Hkv/hp][d]. Returns (O [L][H][d] fp32 with this
        share's heads filled in, LSE [H/hp][L] of the share)."""
        g = self.group
        self._permute(q_full, self.q_x, self.H, 0, self.eb, stream)
        self._permute(K_own, self.k_x, self.Hkv, 0, self.eb, stream)
        self._permute(V_own, self.v_x, self.Hkv, 0, self.eb, stream)
        self._K = self._chunks(K_own, K_rest, self.k_x)
        self._V = self._chunks(V_own, V_rest, self.v_x)
        _, lse = self.ring.forward(self.q_x[g], self._K, self._V, stream)
        self._permute(self.o_x, self.o, self.H, 1, 4, stream)
        return self.o, lse

    def backward(self, dout_full, stream=None):
        """dout_full [L][H][d]. Returns (dQ [L][H][d], dK and dV of the own chunk
        [L][Hkv][d], fp32, with this share's heads filled in); the other chunks'
        dK/dV are in ``dk_chunks`` / ``dv_chunks`` (head-group layout)."""
        g = self.group
        self._permute(dout_full, self.do_x, self.H, 0, self.eb, stream)
        self.ring.backward(self.q_x[g], self._K, self._V, self.do_x[g], stream)
        self._permute(self.dq_x, self.dq, self.H, 1, 4, stream)
        self._permute(self.dk_x, self.dk_own, self.Hkv, 1, 4, stream)
        self._permute(self.dv_x, self.dv_own, self.Hkv, 1, 4, stream)
        return self.dq, self.dk_own, self.dv_own

    def permute_bytes(self):
        """HBM bytes the permutes of one forward + backward move (read + write)."""
        lh, lk = self.L * self.H * self.d, self.L * self.Hkv * self.d
        fwd = 2 * (lh * self.eb + 2 * lk * self.eb) + 2 * lh * 4
        bwd = 2 * lh * self.eb + 2 * (lh * 4 + 2 * lk * 4)
        return fwd + bwd

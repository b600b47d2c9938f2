"""Named workloads: one GPU's share of context-parallel causal attention.

Shapes follow the pages' workloads (LLaMA-3-8B/70B-shaped heads, 128K-1M
token sequences; "Guide to LoongTrain", section "Evaluation"). Heads are the
LOCAL heads after the head-parallel split. ``inner * outer`` is the ring size P
(the context degree); the sequence is cut into 2P blocks of b = S / 2P tokens.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class ShareConfig:
    name: str
    S: int          # global sequence length
    inner: int      # inner ring size
    outer: int      # outer ring size
    hq: int         # local query heads
    hkv: int        # local KV heads
    d: int          # head dim
    dtype: str      # "bf16" | "f32"
    seed: int
    hp: int = 1     # head-parallel degree (Ulysses group size)
    permute_heads: int = 0   # heads of the pre-permute tensor (0: no permute)

    @property
    def P(self):
        return self.inner * self.outer

    @property
    def b(self):
        return self.S // (2 * self.P)

    @property
    def rows(self):
        return 2 * self.b

    @property
    def scale(self):
        return 1.0 / (self.d ** 0.5)

    def pairs_per_head(self, layout="zigzag", rank=0):
        """Visible (q, k) pairs per query head of a rank's share: b (S + 1) for
        every rank with paired blocks; with contiguous chunks of L = S/P rows,
        rank r's rows r*L .. r*L+L-1 see L (r L) + L (L + 1) / 2 pairs."""
        if layout == "zigzag":
            return self.b * (self.S + 1)
        L = self.S // self.P
        return L * rank * L + L * (L + 1) // 2

    def flops(self, layout="zigzag", rank=0):
        """Algorithmic fwd+bwd flops of the share: 4 d Hq N (fwd) + 10 d Hq N (bwd)."""
        n = self.pairs_per_head(layout, rank)
        return 4 * self.d * self.hq * n, 10 * self.d * self.hq * n


CONFIGS = {
    "tiny_f32": ShareConfig("tiny_f32", S=512, inner=4, outer=1, hq=1, hkv=1, d=64,
                            dtype="f32", seed=1001),
    "llama3_8b_cp8_128k": ShareConfig("llama3_8b_cp8_128k", S=131072, inner=8, outer=1,
                                      hq=32, hkv=8, d=128, dtype="bf16", seed=1002),
    "hp4_cp16_1m": ShareConfig("hp4_cp16_1m", S=1048576, inner=4, outer=4, hq=8, hkv=2,
                               d=128, dtype="bf16", seed=1003, hp=4, permute_heads=32),
    "mha7b_hp8_cp8_1m": ShareConfig("mha7b_hp8_cp8_1m", S=1048576, inner=8, outer=1, hq=4,
                                    hkv=4, d=128, dtype="bf16", seed=1004, hp=8),
    "llama3_70b_hp2_cp32_512k": ShareConfig("llama3_70b_hp2_cp32_512k", S=524288, inner=8,
                                            outer=4, hq=32, hkv=4, d=128, dtype="bf16",
                                            seed=1005, hp=2),
}

"""Plain fp64 CPU oracle for one GPU's share of ring (context-parallel) causal attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code with the HIP library; the only module
both sides use is the seeded input generator, which holds none of the method's
arithmetic.

Sources (the pages' text; cited by page title and section):
  * "LoongTrain: Efficient Training of Long-Sequence LLMs with Head-Context
    Parallelism" (arXiv 2406.18485), abstract: 2D-Attention = head-parallel x
    context-parallel attention; Double-Ring-Attention.
  * "Guide to LoongTrain: 2D Head-Context Parallelism for LLMs", sections
    "The Scalability Limits of DeepSpeed Ulysses" (the (S/P,H) <-> (S,H/P) head
    transpose and the P_ulysses <= H_kv cap), "The Communication Overhead and
    Causal Imbalance of Ring Attention" (rank i receives (K_j,V_j) from rank i-1
    and attends with its local Q_i; causal rule: q_i sees k_j iff j <= i),
    "2. Paired-Block Allocation for Causal Load Balancing" (2P blocks, rank r
    holds blocks r and 2P-1-r; the Workload(r) equation), and the "Step 3"
    reference code (scale 1/sqrt(head_dim), softmax(QK^T*scale + mask) V).

Modules:
  index_maps  -- paired-block positions, double-ring visit order, head permute
  attention   -- forward/backward of the share, per-step restriction, LSE merge

Every function is pinned by ``tests/test_oracle.py`` (closed forms, invariants,
a library special case, brute force, finite differences) except where its
docstring says "parity unpinned".
"""
from .index_maps import (zigzag_positions, contiguous_positions, chunk_blocks,
                         double_ring_order, head_permute, causal_pair_count)
from .attention import (share_forward, share_backward, step_forward, step_backward,
                        lse_merge, bf16_bits_to_f64, NEG_INF)

__all__ = ["zigzag_positions", "contiguous_positions", "chunk_blocks", "double_ring_order", "head_permute",
           "causal_pair_count", "share_forward", "share_backward", "step_forward",
           "step_backward", "lse_merge", "bf16_bits_to_f64", "NEG_INF"]

"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds none of the attention arithmetic: it only draws N(0,1) values
and rounds them to bfloat16 bit patterns. Values are drawn per natural sequence
block, so any rank's rows (blocks r and 2P-1-r) exist without materialising the
rest of the sequence:

    values(T, block) = Generator(PCG64(SeedSequence([seed, T, block])))
                         .standard_normal((b, H_T, d), float32)

then rounded to bf16 with round-to-nearest-even on the fp32 bit pattern
(u + 0x7FFF + ((u >> 16) & 1)) >> 16. fp32 configurations keep the fp32 draw.
"""
import numpy as np

# tensor ids in the seed sequence
T_Q, T_K, T_V, T_DO, T_QPRE = 1, 2, 3, 4, 5


def block_normal(seed, tensor_id, block, shape):
    """fp32 N(0,1) values of one natural block of one tensor."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id), int(block)])))
    return g.standard_normal(shape, dtype=np.float32)


def f32_to_bf16_bits(x):
    """Round fp32 values to bfloat16 (nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def blocks_tensor(seed, tensor_id, blocks, b, H, d, dtype):
    """Rows of the given natural blocks, concatenated in the order given.

    dtype "bf16" -> uint16 bit patterns [len(blocks)*b][H][d];
    dtype "f32"  -> float32 values of the same shape.
    """
    parts = [block_normal(seed, tensor_id, blk, (b, H, d)) for blk in blocks]
    x = np.concatenate(parts, axis=0) if parts else np.zeros((0, H, d), np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError("dtype must be 'bf16' or 'f32'")


def contiguous_blocks(P, r):
    """Natural block ids (2P blocks of S/2P rows) whose rows rank r holds when
    the sequence is cut into P consecutive chunks: blocks 2r and 2r+1. Pure
    bookkeeping of which draws to take, as for paired_blocks."""
    return [2 * r, 2 * r + 1]


def paired_blocks(P, r):
    """Natural block ids (2P blocks in all) whose rows a ring chunk r holds, in
    row order: the front block r, then the back block 2P-1-r. Pure bookkeeping
    of which draws to take; the positions themselves are computed by each side."""
    return [r, 2 * P - 1 - r]

"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds none of the attention arithmetic: it only draws N(0,1) values
and rounds them to bfloat16 bit patterns. Values are drawn per natural sequence
block, so any rank's rows (blocks r and 2P-1-r) exist without materialising the
rest of the sequence, and per head, so that the heads of one head-parallel
group exist without the others:

    values(T, block, head) = Generator(PCG64(SeedSequence([seed, T, block, head])))
                               .standard_normal((b, d), float32)

then rounded to bf16 with round-to-nearest-even on the fp32 bit pattern
(u + 0x7FFF + ((u >> 16) & 1)) >> 16. fp32 configurations keep the fp32 draw.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids in the seed sequence
T_Q, T_K, T_V, T_DO = 1, 2, 3, 4


def block_normal(seed, tensor_id, block, head, shape):
    """fp32 N(0,1) values of one natural block of one head of one tensor."""
    ss = np.random.SeedSequence([int(seed), int(tensor_id), int(block), int(head)])
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(shape, dtype=np.float32)


def f32_to_bf16_bits(x):
    """Round fp32 values to bfloat16 (nearest even); returns uint16 bit patterns.
    NaNs stay NaN (quiet, sign kept). Works in slices to bound temporaries."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 22
    for i in range(0, u.size, step):
        v = u[i:i + step]
        r = (v >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += v                       # no wrap for finite values or infinities
        r >>= np.uint32(16)
        nan = (v & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r[nan] = (v[nan] >> np.uint32(16)) | np.uint32(0x0040)
        out[i:i + step] = r
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def blocks_tensor(seed, tensor_id, blocks, b, heads, d, dtype):
    """Rows of the given natural blocks, concatenated in the order given, for the
    given heads (an int H means heads 0 .. H-1; a sequence names head ids).

    dtype "bf16" -> uint16 bit patterns [len(blocks)*b][len(heads)][d];
    dtype "f32"  -> float32 values of the same shape.
    """
    heads = list(range(heads)) if isinstance(heads, (int, np.integer)) else list(heads)
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    x = np.empty((len(blocks) * b, len(heads), d), np.uint16 if dtype == "bf16" else np.float32)

    def fill(ij):
        i, j = ij
        v = block_normal(seed, tensor_id, blocks[i], heads[j], (b, d))
        x[i * b:(i + 1) * b, j] = f32_to_bf16_bits(v) if dtype == "bf16" else v

    jobs = [(i, j) for i in range(len(blocks)) for j in range(len(heads))]
    if len(jobs) * b * d < (1 << 22):
        for ij in jobs:
            fill(ij)
    else:   # independent draws: numpy releases the GIL while it fills them
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, jobs))
    return x


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

"""Philox4x32-10 counter-based generator and the dropout keep mask built from it (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/attention.py).  The HIP library has its own implementation
of the same published generator; the two share no code.

Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3" (SC'11): a 4 x 32-bit counter, a 2 x 32-bit key, ten rounds.  Each round multiplies
counter words 0 and 2 by the constants 0xD2511F53 and 0xCD9E8D57 into 64-bit products, and the
new counter is (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); after each round
the key is bumped by the Weyl constants (0x9E3779B9, 0xBB67AE85).

Dropout on the attention probabilities is a step of the pages' attention chain ("Why attention is
memory-bound, not compute-bound", promptingindex page: matmul, scaling, masking, softmax,
dropout, matmul); fusing it means the mask is regenerated, never stored (the recomputation idea
of NOTE-005, "Method").  The pages fix no generator or mask layout; the reading taken here:
  * keep probability t/256 with t = round((1 - p) 256), 1 <= t <= 256; kept probabilities are
    multiplied by 256/t (so the dropped attention is unbiased);
  * element (b, h, i, j) draws one byte: Philox4x32-10 with key (seed low word, seed high word) and
    counter (i, j // 32, b H + h, 2 offset + (j // 4) % 2); the four output words x_0..x_3 hold the
    bytes of keys 32 (j // 32) + 8 g + 4 ((j // 4) % 2) + e in byte e (little end first) of x_g;
  * the element is kept when its byte is below t.
"""
from __future__ import annotations

import numpy as np
import torch

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10: counter words c0..c3 and key words k0, k1 (uint32 arrays or
    scalars, broadcast); returns the four uint32 output words."""
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3)]
    k = [np.asarray(x, dtype=np.uint64) & MASK32 for x in (k0, k1)]
    for _ in range(10):
        p0 = c[0] * M0  # exact: both factors < 2^32
        p1 = c[2] * M1
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k[0], p1 & MASK32, (p0 >> np.uint64(32)) ^ c[3] ^ k[1], p0 & MASK32]
        k = [(k[0] + W0) & MASK32, (k[1] + W1) & MASK32]
    return [x.astype(np.uint32) for x in c]


def keep_threshold(p: float) -> int:
    """t = round((1 - p) 256), half to even, with p taken as a float32 (the C ABI's type); the keep
    probability is t / 256."""
    t = int(round((1.0 - float(np.float32(p))) * 256.0))
    if not 1 <= t <= 256:
        raise ValueError("dropout probability must leave a keep threshold of 1..256 (0 <= p < 1 - 1/512)")
    return t


def dropout_keep(B: int, H: int, N: int, p: float, seed: int, offset: int) -> torch.Tensor:
    """Boolean keep mask [B, H, N, N] (query, key) of the reading in this module's docstring."""
    t = keep_threshold(p)
    nb = (N + 31) // 32
    i = np.arange(N, dtype=np.uint64)[:, None, None]          # query
    jb = np.arange(nb, dtype=np.uint64)[None, :, None]        # 32-key block
    h = np.arange(2, dtype=np.uint64)[None, None, :]          # (j // 4) % 2
    k0, k1 = seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF
    keep = torch.empty(B, H, N, N, dtype=torch.bool)
    for b in range(B):
        for hh in range(H):
            bh = np.uint64(b * H + hh)
            words = philox4x32_10(i, jb, bh, (np.uint64(2 * offset) + h) & MASK32, k0, k1)  # each [N, nb, 2]
            byte = np.empty((N, nb, 2, 4, 4), dtype=np.uint32)   # [i, jb, h, g, e]
            for g in range(4):
                for e in range(4):
                    byte[:, :, :, g, e] = (words[g] >> np.uint32(8 * e)) & np.uint32(0xFF)
            # key within the 32-block: 8 g + 4 h + e
            full = byte.transpose(0, 1, 3, 2, 4).reshape(N, nb * 32)  # [i, jb, g, h, e] -> key order
            keep[b, hh] = torch.from_numpy(full[:, :N] < t)
    return keep

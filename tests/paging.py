"""Test-side helpers that lay logical per-sequence K/V out into a paged pool.

Pure data movement (no arithmetic of the method), used to build the same
logical contents under different block sizes, permutations and sharing, for
the invariance checks the PageServe page lists ("Correctness comes first").
"""

from __future__ import annotations

import numpy as np


def page_out(logical_k, logical_v, block_size, perm_seed=None, extra_blocks=0, poison=None,
             shared_prefix_blocks=0):
    """Lay ``logical_k[s]`` / ``logical_v[s]`` (``[n_s, H, D]`` storage) into a pool.

    Returns ``(k_pool, v_pool, tables)``.  Blocks are handed out in sequence
    order; ``perm_seed`` shuffles the physical ids; ``shared_prefix_blocks``
    makes every sequence list the same first blocks (their contents are taken
    from sequence 0, so callers pass identical prefixes).
    """
    B = len(logical_k)
    h, d = logical_k[0].shape[1:]
    dtype = logical_k[0].dtype
    counts = [-(-x.shape[0] // block_size) for x in logical_k]
    sb = shared_prefix_blocks
    nblocks = sb + sum(c - sb for c in counts) + extra_blocks
    ids = np.arange(nblocks)
    if perm_seed is not None:
        ids = np.random.default_rng(perm_seed).permutation(nblocks)
    if poison is None:
        poison = np.nan if dtype == np.float32 else (0x7FC0 if dtype == np.uint16 else 0x7F)
    kp = np.full((nblocks, block_size, h, d), poison, dtype=dtype)
    vp = np.full((nblocks, block_size, h, d), poison, dtype=dtype)
    tables = np.full((B, max(counts)), -1, dtype=np.int32)
    cursor = sb
    for s in range(B):
        own = counts[s] - sb
        row = np.concatenate([ids[:sb], ids[cursor:cursor + own]]).astype(np.int32)
        cursor += own
        tables[s, :counts[s]] = row
        n = logical_k[s].shape[0]
        for p in range(n):
            blk, off = row[p // block_size], p % block_size
            kp[blk, off] = logical_k[s][p]
            vp[blk, off] = logical_v[s][p]
    return kp, vp, tables


def logical_from_pool(pool, table_row, n):
    """Read a sequence back as ``[n, H, D]`` by walking its table token by token."""
    bs = pool.shape[1]
    return np.stack([pool[table_row[p // bs], p % bs] for p in range(n)]) if n else pool[:0, 0]

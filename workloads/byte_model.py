"""Algorithmic byte and flop counts of one layer-call (measurement only).

The achieved-bandwidth figures divide these counts by measured time.  They
count what the method must move at least once, not what a kernel happens to
move: every valid K and V element once, every query and output element once,
the block-table entries that cover the context, and the per-sequence lengths.

* KV bytes per token and layer: ``2 x H_kv x D x bytes`` (K and V); the
  whole-model form ``2 x layers x H_kv x D x bytes`` is the formula on "How to
  design an LLM serving system" ("Two phases and the KV cache").
* A single-token page of one of K or V at 8 kv heads x 128 dims x 2 bytes is a
  2 KB read ("How Easy Is It to Start Serving LLMs?", Phase 4 §1 key results).
* Index entries per batch are ``sum ceil(n / page)`` (the same key results:
  262K entries at page 1 against 16K at page 16 for 64 x 4K tokens).

Under a sliding window of W keys (a row at position p sees p - W < j <= p)
a sequence whose last L rows attend reads keys max(0, n - L - W + 1) .. n - 1
only, and a row sees min(p + 1, W) keys.

Pinned by tests/test_byte_model.py against the numbers those pages print.
"""

from __future__ import annotations

import numpy as np


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return 2 * int(num_layers) * int(num_kv_heads) * int(head_dim) * int(dtype_bytes)


def index_entries(context_lens, block_size: int) -> int:
    lens = np.asarray(context_lens, dtype=np.int64)
    return int(((lens + block_size - 1) // block_size).sum())


def first_read_key(context_lens, q_lens, window: int = 0) -> np.ndarray:
    """First key any row of each sequence sees (0 without a window)."""
    lens = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    if window <= 0:
        return np.zeros_like(lens)
    return np.maximum(0, lens - ql - int(window) + 1)


def attention_bytes(context_lens, q_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                    kv_bytes, q_bytes, out_bytes=None, window: int = 0) -> int:
    """Bytes of one attention layer-call (decode or mixed)."""
    if out_bytes is None:
        out_bytes = q_bytes
    lens = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    first = first_read_key(lens, ql, window)
    kv = int((lens - first).sum()) * kv_bytes_per_token(1, num_kv_heads, head_dim, kv_bytes)
    rows = int(ql.sum())
    qo = rows * int(num_q_heads) * int(head_dim) * (int(q_bytes) + int(out_bytes))
    # table entries of the pages that hold keys first .. n - 1
    bs = int(block_size)
    tables = int(np.where(lens > 0, (lens + bs - 1) // bs - first // bs, 0).sum()) * 4
    meta = lens.shape[0] * 4 * 2  # context_lens and cu_seqlens entries
    return kv + qo + tables + meta


def write_bytes(num_tokens, num_kv_heads, head_dim, new_bytes, cache_bytes) -> int:
    """Bytes of one paged_kv_write: read new K and V, write them into the cache, read slots."""
    per = 2 * int(num_kv_heads) * int(head_dim)
    return int(num_tokens) * (per * (int(new_bytes) + int(cache_bytes)) + 4)


def attention_flops(context_lens, q_lens, num_q_heads, head_dim, window: int = 0) -> int:
    """Multiply-adds x 2 of QK^T and PV over the visible (causal) keys."""
    lens = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    if window <= 0:
        # row i of a chunk of L rows over n keys sees n - L + i + 1 keys
        pairs = int((ql * lens - ql * (ql - 1) // 2).sum())
    else:
        pairs = 0
        for n, L in zip(lens.tolist(), ql.tolist()):
            seen = np.arange(n - L + 1, n + 1, dtype=np.int64)  # keys row i sees without a window
            pairs += int(np.minimum(seen, int(window)).sum())
    return 4 * pairs * int(num_q_heads) * int(head_dim)

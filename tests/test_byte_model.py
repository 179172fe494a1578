"""Pins of the measurement byte model against numbers the pages print."""

import os

import numpy as np

from workloads import byte_model as bm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    out = {}
    with open(os.path.join(GOLDEN, "byte_model.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, value = line.split()[:2]
                out[name] = int(value)
    return out


def test_printed_numbers():
    g = _golden()
    # one of K or V for one token at 8 kv heads x 128 x 2 bytes is half the
    # per-token K+V bytes of one layer
    assert bm.kv_bytes_per_token(1, 8, 128, 2) // 2 == g["single_token_page_bytes"]
    lens = np.full(64, 4096)
    assert bm.index_entries(lens, 1) == g["index_entries_page1"]
    assert bm.index_entries(lens, 16) == g["index_entries_page16"]
    assert bm.kv_bytes_per_token(32, 8, 128, 2) == g["llama3_8b_bytes_per_token"]
    assert bm.kv_bytes_per_token(32, 8, 128, 2) * 2048 == g["llama3_8b_2048_tokens"]


def test_decode_workload_bytes_and_mixed_flops():
    # 147,456 tokens x 4096 B is the decode workload's nominal size; check the formula's parts
    lens = np.full(64, 2304)
    b = bm.attention_bytes(lens, np.ones(64), 32, 8, 128, 16, 2, 2)
    kv = 64 * 2304 * 4096
    assert b == kv + 64 * 32 * 128 * 4 + 64 * 144 * 4 + 64 * 8
    # one 512-row chunk over 2560 keys: 1,179,904 visible (q, k) pairs per head
    f = bm.attention_flops([2560], [512], 32, 128)
    assert f == 4 * 1179904 * 32 * 128
    # a decode row sees every key
    assert bm.attention_flops([100], [1], 1, 1) == 400


def test_window_byte_and_flop_counts():
    lens, ql = np.array([100, 5000, 17, 2560]), np.array([1, 1, 1, 512])
    args = (32, 8, 128, 16, 2, 2)
    # a window at least as long as every context changes nothing
    assert bm.attention_bytes(lens, ql, *args, window=5000) == bm.attention_bytes(lens, ql, *args)
    assert bm.attention_flops(lens, ql, 32, 128, window=5000) == bm.attention_flops(lens, ql, 32, 128)
    # window 1: a decode row reads its last key only, a chunk row its own key
    # (the chunk reads its 512 new keys); pages: one per decode row, and the
    # 32 pages of keys 2048 .. 2559
    b = bm.attention_bytes(lens, ql, *args, window=1)
    kv = (1 + 1 + 1 + 512) * 2 * 8 * 128 * 2
    qo = (1 + 1 + 1 + 512) * 32 * 128 * 4
    assert b == kv + qo + (1 + 1 + 1 + 32) * 4 + 4 * 8
    assert bm.attention_flops(lens, ql, 1, 1, window=1) == 4 * (1 + 1 + 1 + 512)
    # brute force over (row, key) pairs for a chunk under a window of 100
    n, L, W = 700, 300, 100
    pairs = sum(1 for r in range(L) for j in range(n) if j <= n - L + r and j > n - L + r - W)
    assert bm.attention_flops([n], [L], 1, 1, window=W) == 4 * pairs
    keys = len({j for r in range(L) for j in range(n) if n - L + r - W < j <= n - L + r})
    # one-byte K and V of one head and dim, pages of one key, no q/out bytes:
    # K + V, one table entry per key, the two length entries
    assert bm.attention_bytes([n], [L], 1, 1, 1, 1, 1, 0, window=W) == 2 * keys + 4 * keys + 8

"""Seeded synthetic inputs for the paged-KV attention path.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.  This module
holds no arithmetic of the method: it draws random numbers, rounds them to the
storage dtype of the inputs, builds block tables, slot lists and packed-token
offsets, and nothing else.  Neither the oracle nor the GPU library imports it.

Shapes follow the pages' workloads:

* ``tiny``      - 4 sequences of 7/16/33/100 keys, 4 q / 2 kv heads, D=64,
  page 16, a 64-block pool in seeded random order, fp32.
* ``decode``    - 64 sequences with context uniform in [512, 4096], 32 q / 8 kv
  heads, D=128, page 16, shuffled pool, bf16 (Qwen3-4B attention shape: "How
  Easy Is It to Start Serving LLMs?", Phase 4 setup; 64 x 4K batch of §1).
* ``long``      - 16 sequences at 32768 keys, same heads, three layouts: page 1
  shuffled, page 16 shuffled, page 16 in order (a contiguous slab), bf16.
* ``mixed``     - 63 decodes (context uniform in [256, 2048]) then one
  512-token chunk over 2048 cached tokens, packed in [T], bf16 ("nanoserve":
  512-token chunked-prefill budget, 2,048-token prompts).
* ``fp8prefix`` - 128 sequences whose tables start with the same 256 blocks
  (a 4096-token shared prefix) plus 256 private tokens each, fp8 E4M3 cache
  filled from bf16 N(0,1) values with one scale per tensor.

* ``skew``      - length mixes at an equal total of tokens for the load-balance
  study (batch 4/16/64/128): ``uniform`` (all equal), ``one-long`` (one
  sequence holds half the tokens, the others share the rest) and ``heavy``
  (Pareto(1.2)-tailed draws scaled to the total), same heads and page 16.

Random streams: ``numpy.random.default_rng([config_id, stream])`` with stream
0 = lengths, 1 = pool permutation, 2 = K pool, 3 = V pool, 4 = Q, 5 = new K,
6 = new V.  Values are N(0, 1) in fp32, rounded to the storage dtype (bf16 by
round-to-nearest-even through torch).  Pool slots that hold no token, and the
slots this step's tokens will be written to, are poisoned with NaN; table
entries past a sequence's last block are -1.  A stray read therefore shows up
as NaN in the output.

For an fp8 cache the generator cannot produce codes (quantising is the
method's work): it returns the bf16 values of every valid slot as a *fill* list
(``fill_slots``, ``k_fill``, ``v_fill``) and a cache of NaN codes; the caller
writes the fill through the write path under test (kernel or oracle).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CONFIG_IDS = {"tiny": 0, "decode": 1, "long": 2, "mixed": 3, "fp8prefix": 4, "skew": 5}

STORAGE_NP = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
STORAGE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
POISON = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}


def rng_for(config_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(stream)])


def to_storage(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 draws to an input storage dtype (f32 or bf16)."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        import torch

        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"inputs are drawn as f32 or bf16, not {dtype}")


def draw(config_id: int, stream: int, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, 1) fp32 draws of one random stream, rounded to ``dtype`` chunk by
    chunk straight into the output array (no full-size fp32 temporary)."""
    rng = rng_for(config_id, stream)
    out = np.empty(shape, dtype=STORAGE_NP[dtype])
    flat = out.reshape(-1)
    for i in range(0, flat.size, chunk):
        n = min(chunk, flat.size - i)
        flat[i:i + n] = to_storage(rng.standard_normal(n, dtype=np.float32), dtype)
    return out


@dataclasses.dataclass
class Case:
    """One batch of paged-attention inputs (storage arrays, host side)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    new_dtype: str
    context_lens: np.ndarray      # int32 [B], keys after this step's write
    q_lens: np.ndarray            # int32 [B], new tokens (query rows) this step
    cu_seqlens: np.ndarray        # int32 [B+1]
    block_tables: np.ndarray      # int32 [B, max_blocks], -1 past the end
    k_cache: np.ndarray           # storage [N, bs, Hkv, D]
    v_cache: np.ndarray
    slot_mapping: np.ndarray      # int32 [T], slot of each new token
    k_new: np.ndarray             # storage (new_dtype) [T, Hkv, D]
    v_new: np.ndarray
    q: np.ndarray                 # storage (q_dtype) [T, Hq, D]
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    fill_slots: Optional[np.ndarray] = None   # fp8 only: slots of the old tokens
    k_fill: Optional[np.ndarray] = None       # fp8 only: their bf16 values
    v_fill: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])


def _tables(block_counts, shared_blocks: int, num_blocks: int, perm: np.ndarray):
    """Block tables: sequences take consecutive entries of the permuted pool.

    The first ``shared_blocks`` entries of the pool are listed first by every
    sequence (a shared prompt prefix); private blocks follow in sequence order.
    """
    B = len(block_counts)
    max_blocks = max(block_counts) if B else 0
    tables = np.full((B, max(max_blocks, 1)), -1, dtype=np.int32)
    cursor = shared_blocks
    for s, nb in enumerate(block_counts):
        own = nb - shared_blocks
        ids = np.concatenate([perm[:shared_blocks], perm[cursor:cursor + own]])
        cursor += own
        tables[s, :nb] = ids
    if cursor > num_blocks:
        raise ValueError("pool too small")
    return tables


def build_case(
    name: str,
    config_id: int,
    context_lens,
    q_lens,
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    q_dtype: str = "bf16",
    kv_dtype: str = "bf16",
    new_dtype: Optional[str] = None,
    layout: str = "shuffle",
    shared_prefix_tokens: int = 0,
    pool_blocks: Optional[int] = None,
    scale: Optional[float] = None,
) -> Case:
    """Draw one case.  ``layout`` is ``"shuffle"`` (seeded permutation of the
    pool) or ``"identity"`` (blocks in order: one contiguous slab)."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    B = ctx.shape[0]
    if np.any(ql > ctx):
        raise ValueError("a sequence has more new tokens than keys")
    bs = int(block_size)
    hkv, d = int(num_kv_heads), int(head_dim)
    if new_dtype is None:
        new_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    if shared_prefix_tokens % bs:
        raise ValueError("shared prefix must be whole blocks")
    shared = shared_prefix_tokens // bs
    counts = [int(-(-n // bs)) for n in ctx]
    needed = shared + sum(c - shared for c in counts)
    nblocks = int(pool_blocks) if pool_blocks is not None else max(needed, 1)

    perm = rng_for(config_id, 1).permutation(nblocks) if layout == "shuffle" else np.arange(nblocks)
    tables = _tables(counts, shared, nblocks, perm.astype(np.int32))

    # Which physical slots hold an old token, and which receive a new one.
    valid = np.zeros(nblocks * bs, dtype=bool)
    new_slots = []
    for s in range(B):
        n, L = int(ctx[s]), int(ql[s])
        pos = np.arange(n)
        slots = tables[s, pos // bs].astype(np.int64) * bs + pos % bs
        valid[slots[: n - L]] = True
        new_slots.append(slots[n - L:])
    slot_mapping = (np.concatenate(new_slots) if B else np.zeros(0, np.int64)).astype(np.int32)
    T = int(ql.sum())
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)

    shape = (nblocks, bs, hkv, d)
    src_dtype = new_dtype if kv_dtype == "fp8" else kv_dtype
    k_pool = draw(config_id, 2, shape, src_dtype)
    v_pool = draw(config_id, 3, shape, src_dtype)
    q = draw(config_id, 4, (T, int(num_q_heads), d), q_dtype)
    k_new = draw(config_id, 5, (T, hkv, d), new_dtype)
    v_new = draw(config_id, 6, (T, hkv, d), new_dtype)

    fill_slots = k_fill = v_fill = None
    k_scale = v_scale = 1.0
    if kv_dtype == "fp8":
        fill_slots = np.nonzero(valid)[0].astype(np.int32)
        k_fill = k_pool.reshape(nblocks * bs, hkv, d)[fill_slots].copy()
        v_fill = v_pool.reshape(nblocks * bs, hkv, d)[fill_slots].copy()
        k_scale = amax_scale([k_fill, k_new], new_dtype)
        v_scale = amax_scale([v_fill, v_new], new_dtype)
        k_cache = np.full(shape, POISON["fp8"], dtype=np.uint8)
        v_cache = np.full(shape, POISON["fp8"], dtype=np.uint8)
    else:
        k_cache, v_cache = k_pool, v_pool
        flat_k = k_cache.reshape(nblocks * bs, hkv, d)
        flat_v = v_cache.reshape(nblocks * bs, hkv, d)
        flat_k[~valid] = POISON[kv_dtype]
        flat_v[~valid] = POISON[kv_dtype]

    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    return Case(
        name=name, num_q_heads=int(num_q_heads), num_kv_heads=hkv, head_dim=d, block_size=bs,
        q_dtype=q_dtype, kv_dtype=kv_dtype, new_dtype=new_dtype,
        context_lens=ctx.astype(np.int32), q_lens=ql.astype(np.int32), cu_seqlens=cu,
        block_tables=tables, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping,
        k_new=k_new, v_new=v_new, q=q, scale=float(scale), k_scale=k_scale, v_scale=v_scale,
        fill_slots=fill_slots, k_fill=k_fill, v_fill=v_fill,
    )


def amax_scale(parts, dtype: str) -> float:
    """Per-tensor fp8 scale chosen by the caller: fp32(max |x|) / 448 in fp32."""
    amax = np.float32(0.0)
    for p in parts:
        if p.size:
            if dtype == "bf16":
                vals = (p.astype(np.uint32) << np.uint32(16)).view(np.float32)
            else:
                vals = p.astype(np.float32)
            amax = max(amax, np.float32(np.max(np.abs(vals))))
    if amax == 0:
        return 1.0
    return float(np.float32(amax) / np.float32(448.0))


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------


def decode_lengths(config: str) -> np.ndarray:
    cid = CONFIG_IDS[config]
    if config == "tiny":
        return np.array([7, 16, 33, 100], dtype=np.int32)
    if config == "decode":
        return rng_for(cid, 0).integers(512, 4096, size=64, endpoint=True).astype(np.int32)
    if config == "long":
        return np.full(16, 32768, dtype=np.int32)
    if config == "fp8prefix":
        return np.full(128, 4096 + 256, dtype=np.int32)
    raise ValueError(config)


def make_case(config: str, layout: str = "page16") -> Case:
    """One of the five workloads at full size."""
    cid = CONFIG_IDS[config]
    if config == "tiny":
        lens = decode_lengths("tiny")
        return build_case("tiny", cid, lens, np.ones(4, np.int32), num_q_heads=4, num_kv_heads=2,
                          head_dim=64, block_size=16, q_dtype="f32", kv_dtype="f32",
                          pool_blocks=64, scale=1.0 / 8.0)
    if config == "decode":
        lens = decode_lengths("decode")
        return build_case("decode", cid, lens, np.ones(64, np.int32), num_q_heads=32, num_kv_heads=8,
                          head_dim=128, block_size=16)
    if config == "long":
        lens = decode_lengths("long")
        bs = 1 if layout == "page1" else 16
        lay = "identity" if layout == "contig" else "shuffle"
        return build_case(f"long-{layout}", cid, lens, np.ones(16, np.int32), num_q_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=bs, layout=lay)
    if config == "mixed":
        dec = rng_for(cid, 0).integers(256, 2048, size=63, endpoint=True).astype(np.int32)
        lens = np.concatenate([dec, [2048 + 512]]).astype(np.int32)
        ql = np.concatenate([np.ones(63, np.int32), [512]]).astype(np.int32)
        return build_case("mixed", cid, lens, ql, num_q_heads=32, num_kv_heads=8, head_dim=128,
                          block_size=16)
    if config == "fp8prefix":
        lens = decode_lengths("fp8prefix")
        return build_case("fp8prefix", cid, lens, np.ones(128, np.int32), num_q_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=16, kv_dtype="fp8",
                          new_dtype="bf16", shared_prefix_tokens=4096)
    raise ValueError(config)


SKEW_MIXES = ("uniform", "one-long", "heavy")
SKEW_TOTAL = 64 * 2304  # the decode workload's expected total of context tokens


def skew_lengths(mix: str, batch: int, total: int = SKEW_TOTAL, min_len: int = 16) -> np.ndarray:
    """Context lengths of one skew case: ``batch`` sequences summing to
    ``total`` tokens (each at least ``min_len``)."""
    if batch < 1 or total < batch * min_len:
        raise ValueError("batch and total do not fit")
    if mix == "uniform":
        w = np.ones(batch)
    elif mix == "one-long":
        w = np.ones(batch) if batch == 1 else np.concatenate([[batch - 1.0], np.ones(batch - 1)])
    elif mix == "heavy":
        w = 1.0 + rng_for(CONFIG_IDS["skew"], 0 + 16 * batch).pareto(1.2, size=batch)
    else:
        raise ValueError(mix)
    spare = total - batch * min_len
    lens = min_len + np.floor(spare * w / w.sum()).astype(np.int64)
    lens[np.argmax(w)] += total - int(lens.sum())  # the rounding remainder goes to the longest
    return lens.astype(np.int32)


def structure_for_lengths(config_id: int, context_lens, q_lens=None, block_size: int = 16, layout: str = "shuffle"):
    """Tables, slots and offsets for given lengths (the pool holds exactly the
    sequences' blocks, in seeded random order or in order), no values."""
    lens = np.asarray(context_lens, dtype=np.int32)
    ql = np.ones(lens.shape[0], np.int32) if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    bs = int(block_size)
    counts = [int(-(-int(n) // bs)) for n in lens]
    nblocks = max(1, sum(counts))
    perm = rng_for(config_id, 1).permutation(nblocks) if layout == "shuffle" else np.arange(nblocks)
    tables = _tables(counts, 0, nblocks, perm.astype(np.int32))
    slots = []
    for s in range(lens.shape[0]):
        n, L = int(lens[s]), int(ql[s])
        pos = np.arange(n - L, n)
        slots.append(tables[s, pos // bs].astype(np.int64) * bs + pos % bs)
    cu = np.zeros(lens.shape[0] + 1, np.int32)
    cu[1:] = np.cumsum(ql)
    return dict(context_lens=lens, q_lens=ql, cu_seqlens=cu, block_tables=tables,
                slot_mapping=np.concatenate(slots).astype(np.int32), num_blocks=nblocks, block_size=bs)


def structure_only(config: str, layout: str = "page16"):
    """Lengths, tables and slots of a workload without drawing any values."""
    cid = CONFIG_IDS[config]
    if config == "mixed":
        dec = rng_for(cid, 0).integers(256, 2048, size=63, endpoint=True).astype(np.int32)
        lens = np.concatenate([dec, [2560]]).astype(np.int32)
        ql = np.concatenate([np.ones(63, np.int32), [512]]).astype(np.int32)
        bs, lay, shared = 16, "shuffle", 0
    else:
        lens = decode_lengths(config)
        ql = np.ones(lens.shape[0], np.int32)
        bs = 1 if (config == "long" and layout == "page1") else 16
        lay = "identity" if (config == "long" and layout == "contig") else "shuffle"
        shared = 4096 if config == "fp8prefix" else 0
    counts = [int(-(-int(n) // bs)) for n in lens]
    sb = shared // bs
    nblocks = 64 if config == "tiny" else max(1, sb + sum(c - sb for c in counts))
    perm = rng_for(cid, 1).permutation(nblocks) if lay == "shuffle" else np.arange(nblocks)
    tables = _tables(counts, sb, nblocks, perm.astype(np.int32))
    slots = []
    for s in range(lens.shape[0]):
        n, L = int(lens[s]), int(ql[s])
        pos = np.arange(n - L, n)
        slots.append(tables[s, pos // bs].astype(np.int64) * bs + pos % bs)
    cu = np.zeros(lens.shape[0] + 1, np.int32)
    cu[1:] = np.cumsum(ql)
    return dict(context_lens=lens, q_lens=ql, cu_seqlens=cu, block_tables=tables,
                slot_mapping=np.concatenate(slots).astype(np.int32), num_blocks=nblocks,
                block_size=bs)

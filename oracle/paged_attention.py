"""Paged KV write and attention, plain fp64 (TEST INFRASTRUCTURE ONLY).

What the GPU library computes, stated as the definition and nothing more.

Layout (the pages' block pool; "nanoserve", "Paged KV cache" bullet and the
architecture diagram; "How to design an LLM serving system", "PagedAttention"):

* ``k_cache``, ``v_cache``: ``[num_blocks, block_size, H_kv, D]`` storage arrays.
* ``block_tables``: int32 ``[B, max_blocks]``; row ``s`` lists the physical
  block of each logical block of sequence ``s``.  Or, in the CSR form of
  "How Easy Is It to Start Serving LLMs?" (Phase 4 §1: ``kv_indptr`` and
  ``kv_indices``), a flat int32 ``kv_indices`` array whose slice
  ``kv_indptr[s]:kv_indptr[s+1]`` is the row of sequence ``s``.
* ``slot_mapping``: int32 ``[T]``; token ``t`` of this step goes to physical
  slot ``slot_mapping[t]`` = ``block * block_size + offset``.
* ``q``: ``[T, Hq, D]`` packed tokens; sequence ``s`` owns rows
  ``cu_seqlens[s]:cu_seqlens[s+1]`` ("nanoserve", "Packed batches" bullet).
* ``context_lens[s]``: number of keys of sequence ``s`` *after* this step's
  write (each layer writes first, then attends over the whole context:
  "nanoserve", "One engine step", step 3).

Readings of points the pages leave open:

* GQA groups are consecutive: q head ``h`` reads kv head ``h // (Hq / H_kv)``.
* A chunk of ``L`` new rows over a context of ``n`` keys is aligned at the
  bottom right: row ``i`` sits at position ``n - L + i`` and sees keys
  ``0 .. n - L + i``.
* ``n == 0`` gives a zero output row and ``lse = -inf``.
* ``slot < 0`` and slots past the pool are skipped by the write.
* The fp32 ``scale`` multiplies ``q . k`` before the maximum is taken.
* Variants ("How Easy Is It to Start Serving LLMs?", Phase 4 §2 names logit
  soft-capping and sliding windows as template parameters of one kernel
  family, without formulas).  Read as: a soft-cap ``c > 0`` replaces each
  scaled logit ``S`` by ``c * tanh(S / c)`` before the softmax; a window
  ``W > 0`` lets the row at position ``p`` see keys ``p - W < j <= p``
  (its last ``W`` keys, itself included).  ``0`` turns either off.
"""

from __future__ import annotations

import numpy as np

from .numerics import decode_storage, encode_storage


def kv_write(
    k_cache: np.ndarray,
    v_cache: np.ndarray,
    cache_dtype: str,
    k_new: np.ndarray,
    v_new: np.ndarray,
    new_dtype: str,
    slot_mapping: np.ndarray,
    k_scale: float = 1.0,
    v_scale: float = 1.0,
    inplace: bool = False,
):
    """Return the caches after writing this step's K/V by slot (copies unless
    ``inplace``, which writes into the given arrays).

    ``cache.reshape(num_blocks * block_size, H_kv, D)[slot[t]] = enc(new[t])``
    for every token with ``0 <= slot[t] < num_blocks * block_size``; every
    other slot keeps its bytes ("nanoserve", "One engine step", steps 2-3;
    "How to design an LLM serving system", "PagedAttention": slot_mapping).
    ``enc`` converts the stored new values into the cache dtype (bit copy when
    they match, fp8 quantisation with the per-tensor scale otherwise).
    """
    kc = k_cache if inplace else np.array(k_cache, copy=True)
    vc = v_cache if inplace else np.array(v_cache, copy=True)
    nb, bs, hkv, d = kc.shape
    flat_k = kc.reshape(nb * bs, hkv, d)
    flat_v = vc.reshape(nb * bs, hkv, d)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s < 0 or s >= nb * bs:
            continue
        flat_k[s] = encode_storage(k_new[t], new_dtype, cache_dtype, k_scale)
        flat_v[s] = encode_storage(v_new[t], new_dtype, cache_dtype, v_scale)
    return kc, vc


def gather_kv(cache: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Logical ``[n, H_kv, D]`` storage of one sequence, read through its table.

    Logical token ``p`` lives in physical block ``table_row[p // block_size]``
    at offset ``p % block_size`` ("nanoserve", "Paged KV cache" bullet;
    "How Easy Is It to Start Serving LLMs?", Phase 4 §1: a request reads the
    pool at the page ids its row lists).  Table entries past ``ceil(n/bs)``
    are never touched.
    """
    bs = cache.shape[1]
    nblk = -(-n // bs)
    pages = np.asarray(table_row[:nblk], dtype=np.int64)
    return cache[pages].reshape(nblk * bs, cache.shape[2], cache.shape[3])[:n]


def attention_over_range(qf: np.ndarray, kf: np.ndarray, vf: np.ndarray, positions: np.ndarray,
                         scale: float, key_begin: int, key_end: int, soft_cap: float = 0.0, window: int = 0):
    """Exact softmax attention of rows ``qf`` over keys ``[key_begin, key_end)``.

    ``qf`` is ``[L, D]`` fp64, ``kf``/``vf`` are ``[n, D]`` fp64 for one kv head,
    ``positions[i]`` is row ``i``'s position; key ``j`` is visible to row ``i``
    when ``j <= positions[i]`` (and, with a window ``W > 0``, ``j >
    positions[i] - W``); a soft-cap ``c > 0`` maps every scaled logit ``S``
    to ``c * tanh(S / c)``.  Returns ``(o, lse)``: ``o`` ``[L, D]`` is the
    normalised output over the visible keys of the range and ``lse`` ``[L]``
    is ``log(sum_j exp(S_ij))`` (``-inf`` and a zero row when no key of the
    range is visible).
    """
    L = qf.shape[0]
    d = vf.shape[1]
    o = np.zeros((L, d), dtype=np.float64)
    lse = np.full((L,), -np.inf, dtype=np.float64)
    if key_end <= key_begin:
        return o, lse
    s = np.float64(np.float32(scale)) * (qf @ kf[key_begin:key_end].T)
    if soft_cap > 0:
        c = np.float64(np.float32(soft_cap))
        s = c * np.tanh(s / c)
    keys = np.arange(key_begin, key_end)[None, :]
    visible = keys <= np.asarray(positions)[:, None]
    if window > 0:
        visible &= keys > np.asarray(positions)[:, None] - int(window)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    w = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    l = w.sum(axis=1)
    num = w @ vf[key_begin:key_end]
    o[has] = num[has] / l[has, None]
    lse[has] = m[has] + np.log(l[has])
    return o, lse


def lse_merge(parts_o: np.ndarray, parts_lse: np.ndarray):
    """Merge partial attention results over disjoint key ranges.

    For partials ``(o_c, lse_c)``: ``L = log sum_c exp(lse_c)`` and
    ``o = sum_c exp(lse_c - L) * o_c``.  Partials with ``lse = -inf`` carry no
    weight; all of them empty gives a zero row and ``-inf``.  This is the
    merge step that stitches the chunks of a split request back together
    ("How Easy Is It to Start Serving LLMs?", Phase 4 §3).
    ``parts_o``: ``[C, ..., D]``; ``parts_lse``: ``[C, ...]``.
    """
    po = np.asarray(parts_o, dtype=np.float64)
    pl = np.asarray(parts_lse, dtype=np.float64)
    m = pl.max(axis=0)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    w = np.exp(pl - m_safe)                     # [C, ...]
    tot = w.sum(axis=0)
    L = np.where(has, m_safe + np.log(np.where(has, tot, 1.0)), -np.inf)
    wn = np.where(has, w / np.where(has, tot, 1.0), 0.0)
    o = (wn[..., None] * po).sum(axis=0)
    return o, L


def paged_attention(
    q: np.ndarray,
    q_dtype: str,
    k_cache: np.ndarray,
    v_cache: np.ndarray,
    kv_dtype: str,
    block_tables: np.ndarray,
    context_lens: np.ndarray,
    cu_seqlens: np.ndarray,
    scale: float,
    k_scale: float = 1.0,
    v_scale: float = 1.0,
    seqs=None,
    kv_indptr=None,
    soft_cap: float = 0.0,
    window: int = 0,
):
    """Exact attention over a paged cache; returns ``(out, lse)`` in fp64.

    With ``kv_indptr`` given, ``block_tables`` is the flat ``kv_indices``
    array and sequence ``s`` reads its pages from
    ``kv_indices[kv_indptr[s]:kv_indptr[s+1]]`` (the CSR page table).
    ``soft_cap`` and ``window`` select the variants described in the module
    notes (both off at 0).

    For every sequence ``s`` (or only those listed in ``seqs``): gather its
    ``n = context_lens[s]`` keys and values through the block table, decode
    them exactly to fp64 (fp8 codes times their scale), and for every row
    ``i`` of its ``L = cu_seqlens[s+1] - cu_seqlens[s]`` packed query rows and
    every q head ``h`` compute

        S_j = scale * sum_d q[i, h, d] * K[j, h // G, d]    for j <= n - L + i
        out[i, h] = sum_j exp(S_j - m) V[j, h // G] / sum_j exp(S_j - m)

    with ``m = max_j S_j`` and ``G = Hq / H_kv``.  This is the gather-then-
    softmax path ("nanoserve" file table, torch gather + SDPA; "PageServe",
    batched decode over gathered KV) evaluated in fp64; the paged kernel is a
    faster way to the same numbers ("nanoserve", Triton paged-decode bullet:
    online softmax over the block table instead of a padded gather).
    ``out`` is ``[T, Hq, D]``, ``lse`` is ``[T, Hq]`` (natural log).  Rows of
    sequences not in ``seqs`` are left as zeros / ``-inf``.
    """
    T, hq, d = q.shape
    hkv = k_cache.shape[2]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of H_kv")
    group = hq // hkv
    qf = decode_storage(q, q_dtype)
    out = np.zeros((T, hq, d), dtype=np.float64)
    lse = np.full((T, hq), -np.inf, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    nseq = ctx.shape[0]
    todo = range(nseq) if seqs is None else seqs
    for s in todo:
        n = int(ctx[s])
        r0, r1 = int(cu[s]), int(cu[s + 1])
        L = r1 - r0
        if L == 0:
            continue
        if L > n:
            raise ValueError(f"sequence {s}: {L} query rows but only {n} keys")
        if kv_indptr is None:
            row = block_tables[s]
        else:
            row = np.asarray(block_tables)[int(kv_indptr[s]):int(kv_indptr[s + 1])]
        ks = decode_storage(gather_kv(k_cache, row, n), kv_dtype, k_scale)
        vs = decode_storage(gather_kv(v_cache, row, n), kv_dtype, v_scale)
        pos = n - L + np.arange(L)
        for h in range(hq):
            g = h // group
            o, l = attention_over_range(qf[r0:r1, h, :], ks[:, g, :], vs[:, g, :], pos, scale, 0, n, soft_cap,
                                        window)
            out[r0:r1, h, :] = o
            lse[r0:r1, h] = l
    return out, lse

"""Pins of the oracle's write, gather, attention and merge (CPU).

Each check is independent of the oracle's own code path:

* brute force: a pure-Python triple loop over *logical* per-sequence K/V
  (no pages, no tables, math.exp), including multi-row causal chunks;
* a library routine: torch's fp64 ``scaled_dot_product_attention`` on the
  gathered K/V with an explicit bottom-right mask;
* closed forms: one key, zero query, zero scale, constant V, a dominant key,
  MQA / MHA head mappings;
* the invariants of "PageServe" ("Correctness comes first"): block size
  1/3/7/16/32, table permutation, prefix sharing vs private copies, batch
  size, neighbour independence, incremental decode = full recompute;
* the merge identity: attention over a split key range, LSE-merged, equals
  attention over the whole range ("How Easy Is It to Start Serving LLMs?",
  Phase 4 §3: pieces of a split request are merged back together).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import numerics as nx
from paging import page_out, logical_from_pool


def _rand_logical(rng, lens, h, d, dtype="f32"):
    ks, vs = [], []
    for n in lens:
        k = rng.standard_normal((n, h, d)).astype(np.float32)
        v = rng.standard_normal((n, h, d)).astype(np.float32)
        if dtype == "bf16":
            k, v = nx.f32_to_bf16_bits(k), nx.f32_to_bf16_bits(v)
        ks.append(k)
        vs.append(v)
    return ks, vs


def _val(x, dtype):
    return x.astype(np.float64) if dtype == "f32" else nx.bf16_bits_to_f64(x)


def brute_force(q_rows, K, V, n, scale, hq, hkv, soft_cap=0.0, window=0):
    """softmax(scale * q K^T) V with plain loops; q_rows[i][h][d], K[j][g][d].

    Only the keys a row sees are visited at all: keys 0 .. pos, and with a
    window W > 0 only the last W of them (pos - W < j <= pos).  With a cap
    c > 0 each visited key's scaled score s becomes c * tanh(s / c)."""
    L = len(q_rows)
    g_size = hq // hkv
    d = len(K[0][0]) if n else len(q_rows[0][0])
    out = []
    for i in range(L):
        pos = n - L + i
        first = max(0, pos - window + 1) if window > 0 else 0
        keys = range(first, pos + 1)
        row = []
        for h in range(hq):
            g = h // g_size
            scores = []
            for j in keys:
                acc = 0.0
                for e in range(d):
                    acc += q_rows[i][h][e] * K[j][g][e]
                sc = scale * acc
                if soft_cap > 0:
                    sc = soft_cap * math.tanh(sc / soft_cap)
                scores.append(sc)
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            tot = sum(w)
            row.append([sum(w[k] * V[j][g][e] for k, j in enumerate(keys)) / tot for e in range(d)])
        out.append(row)
    return np.array(out)


def _run_oracle(q, pool, lens, q_lens, scale, kv_dtype="f32", q_dtype="f32"):
    kp, vp, tables = pool
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return oracle.paged_attention(q, q_dtype, kp, vp, kv_dtype, tables, np.asarray(lens, np.int32), cu, scale)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [1, 3, 4, 16])
def test_oracle_matches_brute_force(kv_dtype, bs):
    rng = np.random.default_rng(100 + bs)
    lens, q_lens = [1, 5, 19, 8], [1, 2, 5, 8]
    hq, hkv, d = 6, 2, 8
    K, V = _rand_logical(rng, lens, hkv, d, kv_dtype)
    kp, vp, tables = page_out(K, V, bs, perm_seed=bs, extra_blocks=3)
    T = sum(q_lens)
    q = rng.standard_normal((T, hq, d)).astype(np.float32)
    scale = 0.37
    out, lse = _run_oracle(q, (kp, vp, tables), lens, q_lens, scale, kv_dtype)
    assert np.all(np.isfinite(out))
    r = 0
    s64 = float(np.float32(scale))
    for s, (n, L) in enumerate(zip(lens, q_lens)):
        Kl = _val(K[s], kv_dtype).tolist()
        Vl = _val(V[s], kv_dtype).tolist()
        ref = brute_force(q[r:r + L].astype(np.float64).tolist(), Kl, Vl, n, s64, hq, hkv)
        np.testing.assert_allclose(out[r:r + L], ref, rtol=0, atol=1e-12)
        r += L


def test_oracle_matches_torch_sdpa_bottom_right_causal():
    rng = np.random.default_rng(9)
    lens, q_lens = [40, 17, 64], [9, 1, 64]
    hq, hkv, d = 8, 2, 16
    K, V = _rand_logical(rng, lens, hkv, d)
    kp, vp, tables = page_out(K, V, 16, perm_seed=4)
    q = rng.standard_normal((sum(q_lens), hq, d)).astype(np.float32)
    scale = 0.25
    out, lse = _run_oracle(q, (kp, vp, tables), lens, q_lens, scale)
    r = 0
    for s, (n, L) in enumerate(zip(lens, q_lens)):
        qs = torch.from_numpy(q[r:r + L].astype(np.float64)).transpose(0, 1)          # [hq, L, d]
        ks = torch.from_numpy(K[s].astype(np.float64)).transpose(0, 1)
        vs = torch.from_numpy(V[s].astype(np.float64)).transpose(0, 1)
        ks = ks.repeat_interleave(hq // hkv, dim=0).contiguous()
        vs = vs.repeat_interleave(hq // hkv, dim=0).contiguous()
        pos = torch.arange(n - L, n)[:, None]
        mask = torch.arange(n)[None, :] <= pos                                         # bottom-right
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(out[r:r + L], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
        # lse from the definition, recomputed independently with torch
        sc = scale * (qs @ ks.transpose(1, 2))
        sc = sc.masked_fill(~mask, float("-inf"))
        np.testing.assert_allclose(lse[r:r + L], torch.logsumexp(sc, dim=-1).transpose(0, 1).numpy(),
                                   rtol=0, atol=1e-12)
        r += L


def _single(lens, hq, hkv, d, bs, seed=0, kv_dtype="f32"):
    rng = np.random.default_rng(seed)
    K, V = _rand_logical(rng, lens, hkv, d, kv_dtype)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    return K, V, q


@pytest.mark.parametrize("bs", [1, 3, 7, 16, 32])
def test_invariant_block_size_bit_identical(bs):
    lens = [5, 37, 100, 64]
    K, V, q = _single(lens, 4, 2, 16, bs, seed=1, kv_dtype="bf16")
    ref_k, ref_v, ref_t = page_out(K, V, 16, perm_seed=None)
    ref, _ = _run_oracle(q, (ref_k, ref_v, ref_t), lens, [1] * 4, 0.3, "bf16")
    kp, vp, t = page_out(K, V, bs, perm_seed=bs * 13, extra_blocks=5)
    got, _ = _run_oracle(q, (kp, vp, t), lens, [1] * 4, 0.3, "bf16")
    assert np.array_equal(got, ref)


def test_invariant_permutation_and_poisoned_tail():
    lens = [23, 50, 9]
    K, V, q = _single(lens, 8, 8, 8, 4, seed=2)
    a = page_out(K, V, 4, perm_seed=None)
    b = page_out(K, V, 4, perm_seed=77, extra_blocks=11)
    ra, _ = _run_oracle(q, a, lens, [1] * 3, 0.5)
    rb, _ = _run_oracle(q, b, lens, [1] * 3, 0.5)
    assert np.array_equal(ra, rb)
    assert np.all(np.isfinite(rb))  # NaN poison in unused slots / blocks is never read


def test_invariant_prefix_sharing_identical_to_private_copies():
    rng = np.random.default_rng(3)
    prefix_k = rng.standard_normal((32, 2, 8)).astype(np.float32)
    prefix_v = rng.standard_normal((32, 2, 8)).astype(np.float32)
    K, V = [], []
    for n_priv in (5, 17, 0):
        K.append(np.concatenate([prefix_k, rng.standard_normal((n_priv, 2, 8)).astype(np.float32)]))
        V.append(np.concatenate([prefix_v, rng.standard_normal((n_priv, 2, 8)).astype(np.float32)]))
    lens = [k.shape[0] for k in K]
    q = rng.standard_normal((3, 4, 8)).astype(np.float32)
    shared = page_out(K, V, 8, perm_seed=5, shared_prefix_blocks=4)
    private = page_out(K, V, 8, perm_seed=6)
    assert shared[0].shape[0] < private[0].shape[0]
    for s in range(3):  # the shared table really reads the same logical data
        assert np.array_equal(logical_from_pool(shared[0], shared[2][s], lens[s]), K[s])
    rs, _ = _run_oracle(q, shared, lens, [1] * 3, 0.3)
    rp, _ = _run_oracle(q, private, lens, [1] * 3, 0.3)
    assert np.array_equal(rs, rp)


def test_invariant_neighbour_independence_and_batch_size():
    lens = [3, 250, 40, 1]
    K, V, q = _single(lens, 4, 1, 8, 16, seed=4)
    full, _ = _run_oracle(q, page_out(K, V, 16, perm_seed=1), lens, [1] * 4, 0.2)
    for subset in ([0], [1, 3], [0, 2, 3], [2, 0, 1, 3]):
        Ks = [K[i] for i in subset]
        Vs = [V[i] for i in subset]
        got, _ = _run_oracle(q[subset], page_out(Ks, Vs, 16, perm_seed=9), [lens[i] for i in subset],
                             [1] * len(subset), 0.2)
        assert np.array_equal(got, full[subset])


def test_invariant_incremental_decode_equals_recompute():
    rng = np.random.default_rng(5)
    n, L = 30, 6
    K, V = _rand_logical(rng, [n], 2, 8)
    q = rng.standard_normal((L, 4, 8)).astype(np.float32)
    pool = page_out(K, V, 4, perm_seed=2)
    chunk, _ = _run_oracle(q, pool, [n], [L], 0.4)
    for i in range(L):
        # row i of the chunk == a decode of that token over the first n-L+i+1 keys
        # (equal up to fp64 rounding order: BLAS sums rows of different lengths)
        dec, _ = _run_oracle(q[i:i + 1], pool, [n - L + i + 1], [1], 0.4)
        np.testing.assert_allclose(dec[0], chunk[i], rtol=0, atol=1e-13)
    # splitting the chunk into two consecutive chunks gives the same rows
    a, _ = _run_oracle(q[:2], pool, [n - L + 2], [2], 0.4)
    b, _ = _run_oracle(q[2:], pool, [n], [L - 2], 0.4)
    np.testing.assert_allclose(np.concatenate([a, b]), chunk, rtol=0, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(6)
    d = 8
    # one key -> out = v0 exactly
    K, V = _rand_logical(rng, [1], 2, d)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    out, lse = _run_oracle(q, page_out(K, V, 16), [1], [1], 0.7)
    assert np.array_equal(out[0], np.repeat(V[0][0].astype(np.float64), 2, axis=0))
    # q = 0 (or scale = 0) -> mean of V over the context
    K, V = _rand_logical(rng, [13], 2, d)
    pool = page_out(K, V, 4, perm_seed=3)
    z, _ = _run_oracle(np.zeros((1, 4, d), np.float32), pool, [13], [1], 0.7)
    s0, _ = _run_oracle(q, pool, [13], [1], 0.0)
    mean = np.repeat(V[0].astype(np.float64).mean(axis=0), 2, axis=0)
    np.testing.assert_allclose(z[0], mean, rtol=0, atol=1e-14)
    np.testing.assert_allclose(s0[0], mean, rtol=0, atol=1e-14)
    # all V rows equal c -> c
    Vc = [np.full_like(V[0], 0.625)]
    c, _ = _run_oracle(q, page_out(K, Vc, 4), [13], [1], 0.7)
    np.testing.assert_allclose(c, 0.625, rtol=0, atol=1e-15)
    # a key far above the rest -> its value
    Kd = [K[0].copy()]
    Kd[0][7] = 50.0 * q[0, 0].reshape(1, d).repeat(2, axis=0)
    dom, _ = _run_oracle(q, page_out(Kd, V, 4), [13], [1], 1.0)
    np.testing.assert_allclose(dom[0, 0], V[0][7][0], rtol=0, atol=1e-12)


def test_gqa_mapping_mqa_and_mha():
    rng = np.random.default_rng(8)
    n, d = 11, 8
    # MQA: every q head reads kv head 0
    K, V = _rand_logical(rng, [n], 1, d)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    mqa, _ = _run_oracle(q, page_out(K, V, 4), [n], [1], 0.3)
    for h in range(4):
        one, _ = _run_oracle(q[:, h:h + 1], page_out(K, V, 4), [n], [1], 0.3)
        assert np.array_equal(mqa[0, h], one[0, 0])
    # GQA group of 2: q heads 2,3 read kv head 1 (consecutive groups)
    K2, V2 = _rand_logical(rng, [n], 2, d)
    gqa, _ = _run_oracle(q, page_out(K2, V2, 4), [n], [1], 0.3)
    only1 = [K2[0][:, 1:2]], [V2[0][:, 1:2]]
    for h in (2, 3):
        one, _ = _run_oracle(q[:, h:h + 1], page_out(*only1, 4), [n], [1], 0.3)
        assert np.array_equal(gqa[0, h], one[0, 0])
    # MHA: head h reads kv head h
    K4, V4 = _rand_logical(rng, [n], 4, d)
    mha, _ = _run_oracle(q, page_out(K4, V4, 4), [n], [1], 0.3)
    for h in range(4):
        one, _ = _run_oracle(q[:, h:h + 1], page_out([K4[0][:, h:h + 1]], [V4[0][:, h:h + 1]], 4),
                             [n], [1], 0.3)
        assert np.array_equal(mha[0, h], one[0, 0])


@pytest.mark.parametrize("cuts", [[0, 16, 37], [0, 1, 2, 37], [0, 30, 36, 37], [0, 37]])
def test_merge_identity(cuts):
    rng = np.random.default_rng(10)
    n, L, d = 37, 4, 8
    qf = rng.standard_normal((L, d))
    kf = rng.standard_normal((n, d))
    vf = rng.standard_normal((n, d))
    pos = n - L + np.arange(L)
    whole_o, whole_l = oracle.attention_over_range(qf, kf, vf, pos, 0.5, 0, n)
    parts = [oracle.attention_over_range(qf, kf, vf, pos, 0.5, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    mo, ml = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(mo, whole_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, whole_l, rtol=0, atol=1e-12)


def test_merge_skips_empty_parts_and_all_empty():
    o = np.array([[[1.0, 2.0]], [[5.0, 7.0]]])
    l = np.array([[0.3], [-np.inf]])
    mo, ml = oracle.lse_merge(o, l)
    assert np.array_equal(mo, [[1.0, 2.0]]) and ml[0] == 0.3
    mo, ml = oracle.lse_merge(o, np.full((2, 1), -np.inf))
    assert np.array_equal(mo, [[0.0, 0.0]]) and ml[0] == -np.inf


def test_write_places_by_slot_and_leaves_everything_else():
    rng = np.random.default_rng(12)
    nb, bs, h, d = 6, 4, 2, 8
    kc = rng.standard_normal((nb, bs, h, d)).astype(np.float32)
    vc = rng.standard_normal((nb, bs, h, d)).astype(np.float32)
    kn = rng.standard_normal((5, h, d)).astype(np.float32)
    vn = rng.standard_normal((5, h, d)).astype(np.float32)
    slots = np.array([0, 23, -1, 9, 24], dtype=np.int32)   # 24 is past the pool: skipped
    k2, v2 = oracle.kv_write(kc, vc, "f32", kn, vn, "f32", slots)
    changed = np.zeros((nb, bs), bool)
    for t, s in enumerate(slots):
        if 0 <= s < nb * bs:
            assert np.array_equal(k2[s // bs, s % bs], kn[t]) and np.array_equal(v2[s // bs, s % bs], vn[t])
            changed[s // bs, s % bs] = True
    assert np.array_equal(k2[~changed], kc[~changed]) and np.array_equal(v2[~changed], vc[~changed])


def test_write_fp8_quantises_with_scale():
    rng = np.random.default_rng(13)
    kn = nx.f32_to_bf16_bits(rng.standard_normal((3, 2, 8)).astype(np.float32))
    vn = nx.f32_to_bf16_bits(rng.standard_normal((3, 2, 8)).astype(np.float32))
    kc = np.full((2, 2, 2, 8), 0x7F, np.uint8)
    ks, vs = 0.01, 0.0037
    k2, v2 = oracle.kv_write(kc, kc, "fp8", kn, vn, "bf16", np.array([3, 0, 1], np.int32), ks, vs)
    wk = nx.e4m3_encode(nx.bf16_bits_to_f64(kn).astype(np.float32), ks)
    wv = nx.e4m3_encode(nx.bf16_bits_to_f64(vn).astype(np.float32), vs)
    for cache, want in ((k2, wk), (v2, wv)):
        assert np.array_equal(cache[1, 1], want[0]) and np.array_equal(cache[0, 0], want[1])
        assert np.array_equal(cache[0, 1], want[2]) and np.all(cache[1, 0] == 0x7F)


def test_fp8_attention_reads_dequantised_values():
    rng = np.random.default_rng(14)
    n, h, d = 20, 2, 8
    Kb, Vb = _rand_logical(rng, [n], h, d)
    ks, vs = np.float32(0.011), np.float32(0.009)
    Kq = [nx.e4m3_encode(Kb[0], float(ks))]
    Vq = [nx.e4m3_encode(Vb[0], float(vs))]
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    kp, vp, t = page_out(Kq, Vq, 8, perm_seed=1)
    got = oracle.paged_attention(q, "f32", kp, vp, "fp8", t, np.array([n], np.int32),
                                 np.array([0, 1], np.int32), 0.3, float(ks), float(vs))[0]
    Kd = [nx.e4m3_decode(Kq[0], float(ks)).astype(np.float32)]
    Vd = [nx.e4m3_decode(Vq[0], float(vs)).astype(np.float32)]
    # the dequantised values are exact in fp32 here only up to the scale product; compare in fp64
    ref = brute_force(q.astype(np.float64).tolist(), nx.e4m3_decode(Kq[0], float(ks)).tolist(),
                      nx.e4m3_decode(Vq[0], float(vs)).tolist(), n, float(np.float32(0.3)), 4, h)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    assert Kd[0].shape == Kb[0].shape


def _to_csr(tables, lens, bs, extra=0, seed=0):
    """CSR page table of dense rows: each sequence's first ceil(n/bs) entries,
    plus ``extra`` unused entries (-1) after them."""
    rows = []
    for s, n in enumerate(lens):
        nb = -(-int(n) // bs)
        rows.append(np.concatenate([tables[s, :nb], np.full(extra, -1, np.int32)]).astype(np.int32))
    indptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    return indptr, np.concatenate(rows).astype(np.int32)


@pytest.mark.parametrize("bs,extra", [(1, 0), (4, 2), (16, 0), (16, 3)])
def test_csr_page_table_equals_dense(bs, extra):
    """The CSR form of the page table ("How Easy Is It to Start Serving LLMs?",
    Phase 4 §1) reads the same pages as the dense rows: bit-identical outputs,
    also with unused entries after a row's last page and an empty sequence."""
    lens = [5, 37, 100, 0, 64]
    q_lens = [1, 1, 3, 0, 1]
    K, V, _ = _single(lens, 4, 2, 16, bs, seed=9, kv_dtype="bf16")
    kp, vp, t = page_out(K, V, bs, perm_seed=bs * 7, extra_blocks=4)
    rng = np.random.default_rng(10)
    q = rng.standard_normal((sum(q_lens), 4, 16)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    ref, ref_lse = oracle.paged_attention(q, "f32", kp, vp, "bf16", t, np.asarray(lens, np.int32), cu, 0.25)
    indptr, indices = _to_csr(t, lens, bs, extra)
    got, got_lse = oracle.paged_attention(q, "f32", kp, vp, "bf16", indices, np.asarray(lens, np.int32), cu, 0.25,
                                          kv_indptr=indptr)
    assert np.array_equal(got, ref) and np.array_equal(got_lse, ref_lse)


# --- variants: logit soft-cap and sliding window (readings of Phase 4 §2) ---

def _variant_case(seed, lens, q_lens, hq=4, hkv=2, d=16, bs=4):
    K, V, _ = _single(lens, hq, hkv, d, bs, seed=seed, kv_dtype="bf16")
    kp, vp, t = page_out(K, V, bs, perm_seed=seed + 1)
    rng = np.random.default_rng(seed + 2)
    q = rng.standard_normal((sum(q_lens), hq, d)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return q, kp, vp, t, np.asarray(lens, np.int32), cu


def _attn(q, kp, vp, t, lens, cu, scale, **kw):
    return oracle.paged_attention(q, "f32", kp, vp, "bf16", t, lens, cu, scale, **kw)


def test_soft_cap_large_cap_is_plain_attention():
    q, kp, vp, t, lens, cu = _variant_case(20, [37, 100, 5], [1, 4, 2])
    plain, plain_lse = _attn(q, kp, vp, t, lens, cu, 0.3)
    capped, capped_lse = _attn(q, kp, vp, t, lens, cu, 0.3, soft_cap=1e7)
    assert np.allclose(capped, plain, rtol=0, atol=1e-9) and np.allclose(capped_lse, plain_lse, rtol=0, atol=1e-9)


def test_soft_cap_equal_scores_give_the_mean_of_v():
    """Identical keys give identical logits whatever the cap: a plain mean."""
    rng = np.random.default_rng(21)
    n, hkv, d = 9, 1, 8
    k = np.tile(rng.standard_normal((1, hkv, d)).astype(np.float32), (n, 1, 1))
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    kp, vp, t = page_out([k], [v], 4, perm_seed=3)
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    cu = np.array([0, 1], np.int32)
    out, _ = oracle.paged_attention(q, "f32", kp, vp, "f32", t, np.array([n], np.int32), cu, 2.0, soft_cap=0.7)
    assert np.allclose(out[0, 0], v[:, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)


def test_soft_cap_saturation_closed_form():
    """With the cap fixed and the scale huge, every capped logit is +c or -c
    (by the sign of q.k), so the output is (e^c sum V+ + e^-c sum V-) /
    (e^c N+ + e^-c N-)."""
    rng = np.random.default_rng(22)
    n, d, c = 12, 8, 1.5
    k = rng.standard_normal((n, 1, d)).astype(np.float32)
    v = rng.standard_normal((n, 1, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    kp, vp, t = page_out([k], [v], 4, perm_seed=5)
    out, _ = oracle.paged_attention(q, "f32", kp, vp, "f32", t, np.array([n], np.int32), np.array([0, 1], np.int32),
                                    1e9, soft_cap=c)
    dots = (k[:, 0, :].astype(np.float64) @ q[0, 0].astype(np.float64))
    pos, neg = dots > 0, dots < 0
    vv = v[:, 0, :].astype(np.float64)
    cf = float(np.float32(c))
    expect = (np.exp(cf) * vv[pos].sum(0) + np.exp(-cf) * vv[neg].sum(0)) / (np.exp(cf) * pos.sum() + np.exp(-cf) * neg.sum())
    assert np.allclose(out[0, 0], expect, rtol=0, atol=1e-9)


def test_window_at_least_the_context_is_plain_attention():
    q, kp, vp, t, lens, cu = _variant_case(23, [37, 100, 5], [1, 4, 2])
    plain, _ = _attn(q, kp, vp, t, lens, cu, 0.3)
    wide, _ = _attn(q, kp, vp, t, lens, cu, 0.3, window=100)
    assert np.array_equal(plain, wide)


def test_window_of_one_returns_the_rows_own_value():
    q, kp, vp, t, lens, cu = _variant_case(24, [37, 100, 5], [1, 4, 2])
    out, _ = _attn(q, kp, vp, t, lens, cu, 0.3, window=1)
    for s in range(3):
        n, L = int(lens[s]), int(cu[s + 1] - cu[s])
        vs = nx.bf16_bits_to_f64(oracle.gather_kv(vp, t[s], n))
        for i in range(L):
            for h in range(4):
                assert np.array_equal(out[cu[s] + i, h], vs[n - L + i, h // 2])


@pytest.mark.parametrize("w", [2, 7, 30])
def test_window_equals_attention_over_the_last_keys(w):
    """A window W is plain attention over the truncated sequence that starts
    at the first visible key: for a decode row (one row at position n - 1),
    keys n - W .. n - 1 re-paged as a sequence of their own."""
    lens = [37, 100, 5]
    q, kp, vp, t, lens_a, cu = _variant_case(25, lens, [1, 1, 1])
    got, _ = _attn(q, kp, vp, t, lens_a, cu, 0.3, window=w)
    K = [oracle.gather_kv(kp, t[s], n)[max(0, n - w):] for s, n in enumerate(lens)]
    V = [oracle.gather_kv(vp, t[s], n)[max(0, n - w):] for s, n in enumerate(lens)]
    k2, v2, t2 = page_out(K, V, 4, perm_seed=11)
    ref, _ = oracle.paged_attention(q, "f32", k2, v2, "bf16", t2, np.array([len(x) for x in K], np.int32), cu, 0.3)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("soft_cap,window", [(2.0, 0), (0.0, 5), (2.0, 5), (0.75, 3), (2.0, 1)])
@pytest.mark.parametrize("bs", [1, 4])
def test_soft_cap_and_window_match_brute_force_on_causal_chunks(soft_cap, window, bs):
    """Multi-row causal chunks with 1 < W < n and a moderate cap, against the
    brute force that never visits a key its row cannot see: a cap applied to
    masked keys (which would then carry weight e^(-c - m)) or a window off by
    one fails here, unlike with decode rows or a cap large enough that -c
    underflows."""
    rng = np.random.default_rng(700 + bs + int(10 * soft_cap) + window)
    lens, q_lens = [6, 13, 9, 20], [1, 6, 9, 7]
    hq, hkv, d = 4, 2, 8
    K, V = _rand_logical(rng, lens, hkv, d)
    kp, vp, tables = page_out(K, V, bs, perm_seed=bs + 1, extra_blocks=2)
    q = (2.0 * rng.standard_normal((sum(q_lens), hq, d))).astype(np.float32)
    scale = 0.5
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    out, _ = oracle.paged_attention(q, "f32", kp, vp, "f32", tables, np.asarray(lens, np.int32), cu, scale,
                                    soft_cap=soft_cap, window=window)
    c64 = float(np.float32(soft_cap))
    r = 0
    for s, (n, L) in enumerate(zip(lens, q_lens)):
        ref = brute_force(q[r:r + L].astype(np.float64).tolist(), K[s].astype(np.float64).tolist(),
                          V[s].astype(np.float64).tolist(), n, 0.5, hq, hkv, soft_cap=c64, window=window)
        np.testing.assert_allclose(out[r:r + L], ref, rtol=0, atol=1e-12)
        r += L

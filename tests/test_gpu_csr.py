"""GPU parity of the CSR page-table forms (paged_attn_decode_csr,
paged_attn_mixed_csr) against the fp64 oracle's CSR gather, and bit for bit
against the dense-table calls reading the same pages.

CSR rows ("How Easy Is It to Start Serving LLMs?", Phase 4 §1) are built from
the generator's dense rows: each sequence's pages, optionally followed by
unused entries, optionally sharing another row's first pages.
"""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_caches, to_dev

pytestmark = pytest.mark.gpu


def _csr(case, extra=0):
    bs = case.block_size
    rows = []
    for s, n in enumerate(case.context_lens):
        nb = -(-int(n) // bs)
        rows.append(np.concatenate([case.block_tables[s, :nb], np.full(extra, -1, np.int32)]).astype(np.int32))
    indptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    indices = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return indptr, indices


def _oracle_csr(case, kr, vr, indptr, indices):
    return oracle.paged_attention(case.q, case.q_dtype, kr, vr, case.kv_dtype, indices, case.context_lens,
                                  case.cu_seqlens, case.scale, case.k_scale, case.v_scale, kv_indptr=indptr)


def _run(case, gpu, mixed, extra=0, num_queues=0):
    import torch
    import paged_kv_attention_write_amd as pkv

    dc = DeviceCase(case, gpu)
    dc.write()
    plan = dc.plan(num_queues, mixed=mixed)
    indptr, indices = _csr(case, extra)
    ip, ix = to_dev(indptr, gpu), to_dev(indices, gpu)
    out = torch.empty_like(dc.q)
    if mixed:
        pkv.paged_attn_mixed_csr(out, dc.q, dc.kc, dc.vc, ip, ix, dc.cu, dc.ctx, case.scale, plan, case.k_scale,
                                 case.v_scale)
    else:
        pkv.paged_attn_decode_csr(out, dc.q, dc.kc, dc.vc, ip, ix, dc.ctx, case.scale, plan, case.k_scale,
                                  case.v_scale)
    dense = dc.mixed(plan) if mixed else dc.decode(plan)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), dense.view(torch.int16)), "CSR and dense rows differ"
    kr, vr = oracle_caches(case)
    ref, _ = _oracle_csr(case, kr, vr, indptr, indices)
    return as_f64(out), ref, plan


def test_csr_decode_full_size(gpu):
    log("csr decode full size")
    case = workloads.make_case("decode")
    got, ref, plan = _run(case, gpu, mixed=False)
    check_close(got, ref, "bf16", f"csr decode merges={plan.desc.num_merges}")


@pytest.mark.parametrize("bs,extra", [(16, 0), (16, 3), (1, 0), (3, 2), (4, 0), (32, 1), (48, 1), (64, 2)])
def test_csr_decode_page_sizes(gpu, bs, extra):
    log(f"csr decode bs={bs} extra={extra}")
    lens = [1, 17, 100, 250, 513, 64, 2000]
    case = workloads.build_case(f"csr{bs}", 140 + bs, lens, [1] * len(lens), num_q_heads=16, num_kv_heads=4,
                                head_dim=128, block_size=bs)
    got, ref, _ = _run(case, gpu, mixed=False, extra=extra, num_queues=9)
    check_close(got, ref, "bf16", f"csr bs={bs}")


@pytest.mark.parametrize("bs", [16, 32, 3, 4, 48, 64])
def test_csr_mixed(gpu, bs):
    """Chunks and decodes through the CSR rows: page 16/32 run the
    direct-to-LDS prefill ring, page 3 the register-staged tiles."""
    log(f"csr mixed bs={bs}")
    lens = [40, 900, 600, 1300, 77]
    ql = [1, 1, 96, 1, 33]
    case = workloads.build_case(f"csrm{bs}", 150 + bs, lens, ql, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=bs)
    got, ref, _ = _run(case, gpu, mixed=True, extra=1, num_queues=11)
    check_close(got, ref, "bf16", f"csr mixed bs={bs}")


@pytest.mark.parametrize("shape", ["shared-prefix", "empty-row"])
def test_csr_shared_prefix_and_empty_row(gpu, shape):
    """Rows naming the same first pages (a shared prompt), or a sequence of
    length 0 with an empty row, against the oracle's CSR gather."""
    import torch
    import paged_kv_attention_write_amd as pkv

    log(f"csr {shape}")
    if shape == "shared-prefix":
        case = workloads.build_case("csrsh", 160, [300, 260, 145], [1, 1, 1], num_q_heads=8, num_kv_heads=2,
                                    head_dim=128, block_size=16, shared_prefix_tokens=128)
    else:
        case = workloads.build_case("csrem", 162, [300, 0, 45], [1, 0, 1], num_q_heads=8, num_kv_heads=2,
                                    head_dim=128, block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = dc.plan(7, mixed=True)
    indptr, indices = _csr(case, extra=0)
    if shape == "empty-row":
        assert indptr[2] == indptr[1]
    else:
        assert np.array_equal(indices[indptr[0]:indptr[0] + 8], indices[indptr[1]:indptr[1] + 8])
    out = torch.empty_like(dc.q)
    pkv.paged_attn_mixed_csr(out, dc.q, dc.kc, dc.vc, to_dev(indptr, gpu), to_dev(indices, gpu), dc.cu, dc.ctx,
                             case.scale, plan)
    kr, vr = oracle_caches(case)
    ref, _ = _oracle_csr(case, kr, vr, indptr, indices)
    check_close(as_f64(out), ref, "bf16", f"csr {shape}")


def test_csr_bad_entry_gives_nan_rows_only_for_that_sequence(gpu):
    import torch
    import paged_kv_attention_write_amd as pkv

    log("csr bad entry")
    case = workloads.build_case("csrbad", 161, [50, 700, 33], [1, 1, 1], num_q_heads=8, num_kv_heads=2,
                                head_dim=128, block_size=16)
    dc = DeviceCase(case, gpu)
    dc.write()
    plan = dc.plan(5)
    indptr, indices = _csr(case)
    kr, vr = oracle_caches(case)
    ref, _ = _oracle_csr(case, kr, vr, indptr, indices)
    bad = indices.copy()
    bad[indptr[1] + 20] = case.num_blocks + 99
    out = torch.empty_like(dc.q)
    pkv.paged_attn_decode_csr(out, dc.q, dc.kc, dc.vc, to_dev(indptr, gpu), to_dev(bad, gpu), dc.ctx, case.scale,
                              plan)
    got = as_f64(out)
    assert np.all(np.isnan(got[1]))
    check_close(got[[0, 2]], ref[[0, 2]], "bf16", "neighbours of the bad CSR row")

"""paged_attn_decode_noalloc through the C ABI: the entry point that
allocates nothing (its workspace is the library's own per-device array)
against paged_attn_decode with a caller workspace, on two calls in a row,
the second with a smaller batch: outputs byte-identical (same plan, same
kernels), and within the bf16 bound of the fp64 oracle."""

import ctypes

import numpy as np
import pytest

import workloads
from gpu_helpers import DeviceCase, as_f64, check_close, log, oracle_attention, oracle_caches, to_host

pytestmark = pytest.mark.gpu


def _noalloc(dc, out):
    """Plan on the host (paged_attn_plan_host) and call the entry point that
    allocates nothing, through the C ABI."""
    import torch

    import paged_kv_attention_write_amd as pkv
    from paged_kv_attention_write_amd import _abi

    c = dc.case
    p, image = pkv.plan_host(c.context_lens, None, c.num_q_heads, c.num_kv_heads, c.head_dim, pkv.default_queues())
    staging = torch.from_numpy(image).pin_memory()  # the copy is asynchronous from pinned memory
    nb, bs, hkv, d = dc.kc.shape
    B, hq = dc.q.shape[0], dc.q.shape[1]
    st = pkv.lib().paged_attn_decode_noalloc(
        out.data_ptr(), dc.q.data_ptr(), _abi.dtype_code(dc.q), dc.q.stride(0), dc.kc.data_ptr(), dc.vc.data_ptr(),
        _abi.dtype_code(dc.kc), dc.tables.data_ptr(), dc.tables.shape[1], dc.ctx.data_ptr(), B, hq, hkv, d, nb, bs,
        float(c.scale), float(c.k_scale), float(c.v_scale), ctypes.byref(p), staging.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, pkv.strerror(st)
    torch.cuda.synchronize()  # the staging buffer stays alive until the copy has run
    return p


@pytest.mark.parametrize("order", ["large-then-small"])
def test_noalloc_decode_matches_the_workspace_call(gpu, order):
    import torch

    cases = [
        workloads.build_case("noalloc-a", 400, [3000, 512, 4096, 900, 77, 2500], [1] * 6, num_q_heads=32,
                             num_kv_heads=8, head_dim=128, block_size=16),
        workloads.build_case("noalloc-b", 401, [200, 1500, 33], [1] * 3, num_q_heads=32, num_kv_heads=8,
                             head_dim=128, block_size=16),
    ]
    for case in cases:
        log(f"noalloc {case.name}: B={len(case.context_lens)} keys={int(case.context_lens.sum())}")
        dc = DeviceCase(case, gpu)
        dc.write()
        ref_out = dc.decode(dc.plan(0))
        out = torch.full_like(dc.q, float("nan"))
        p = _noalloc(dc, out)
        assert p.num_merges >= 1  # rows cut into pieces: the merge reads partials from the array
        assert np.array_equal(to_host(out), to_host(ref_out)), "entry point without allocation differs"
        kr, vr = oracle_caches(case)
        ref, _ = oracle_attention(case, kr, vr)
        check_close(as_f64(out), ref, "bf16", f"noalloc {case.name}")


def test_noalloc_rejects_a_plan_larger_than_its_array(gpu):
    """A plan whose workspace exceeds the 32 MiB array is refused before any
    device work, with the workspace status."""
    import paged_kv_attention_write_amd as pkv
    from paged_kv_attention_write_amd import _abi

    lens = np.full(64, 60000, np.int32)
    p, image = pkv.plan_host(lens, None, 32, 8, 128, 4096)
    assert p.workspace_bytes > 32 << 20
    st = pkv.lib().paged_attn_decode_noalloc(None, None, 1, 32 * 128, None, None, 1, None, 1, None, 64, 32, 8, 128,
                                             1, 16, 0.1, 1.0, 1.0, ctypes.byref(p), image.ctypes.data, None)
    assert st == _abi.PKV_ERR_WORKSPACE

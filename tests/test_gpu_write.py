"""GPU parity of paged_kv_write against the oracle: bit-exact, every dtype pair.

The write is byte work, so the bar is bit equality of the whole pool after the
write (targeted slots hold the converted rows, every other byte is unchanged).
"""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _pool(rng, nb, bs, h, d, dtype):
    if dtype == "fp8":
        return rng.integers(0, 256, size=(nb, bs, h, d), dtype=np.uint8)
    x = rng.standard_normal((nb, bs, h, d)).astype(np.float32)
    return workloads.to_storage(x, dtype)


@pytest.mark.parametrize("new_dt,cache_dt", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"),
                                              ("bf16", "fp8"), ("f32", "fp8")])
def test_write_bit_exact_every_pair(gpu, new_dt, cache_dt):
    import paged_kv_attention_write_amd as pkv

    log(f"write {new_dt}->{cache_dt}")
    rng = np.random.default_rng(21)
    nb, bs, h, d, T = 37, 16, 8, 128, 300
    kc0, vc0 = _pool(rng, nb, bs, h, d, cache_dt), _pool(rng, nb, bs, h, d, cache_dt)
    kn = workloads.to_storage((rng.standard_normal((T, h, d)) * 3).astype(np.float32), new_dt)
    vn = workloads.to_storage((rng.standard_normal((T, h, d)) * 0.01).astype(np.float32), new_dt)
    slots = rng.permutation(nb * bs)[:T].astype(np.int32)
    slots[::17] = -1                       # skipped
    slots[5] = nb * bs + 3                 # past the pool: skipped
    ks, vs = 0.0123, 0.000071
    kd, vd = to_dev(kc0, gpu), to_dev(vc0, gpu)
    pkv.paged_kv_write(to_dev(kn, gpu), to_dev(vn, gpu), to_dev(slots, gpu), kd, vd, ks, vs)
    kr, vr = oracle.kv_write(kc0, vc0, cache_dt, kn, vn, new_dt, slots, ks, vs)
    assert np.array_equal(to_host(kd).view(np.uint8), kr.view(np.uint8))
    assert np.array_equal(to_host(vd).view(np.uint8), vr.view(np.uint8))


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [1.0, 0.0478, 3.5])
def test_fp8_quantise_exhaustive_bf16_inputs(gpu, src, scale):
    """All 65,536 bf16 bit patterns (fp32 copies of them for src=f32) through the quantising write."""
    import paged_kv_attention_write_amd as pkv

    log(f"fp8 exhaustive src={src} scale={scale}")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.reshape(64, 1, 1024)                        # 64 tokens x 1 head x 1024 dims
    if src == "f32":
        vals = (vals.astype(np.uint32) << np.uint32(16)).view(np.float32)
    nb, bs = 4, 16
    kc0 = np.full((nb, bs, 1, 1024), 0x7F, np.uint8)
    slots = np.arange(64, dtype=np.int32)
    kd, vd = to_dev(kc0, gpu), to_dev(kc0, gpu)
    pkv.paged_kv_write(to_dev(vals, gpu), to_dev(vals, gpu), to_dev(slots, gpu), kd, vd, scale, scale)
    kr, _ = oracle.kv_write(kc0, kc0, "fp8", vals, vals, src, slots, scale, scale)
    got = to_host(kd)
    bad = np.nonzero(got.reshape(-1) != kr.reshape(-1))[0]
    assert bad.size == 0, f"{bad.size} mismatches, first inputs {bits[bad[:8] % 65536]}"


def test_write_strided_new_rows(gpu):
    """K/V rows taken from a fused [T, (Hq + 2 H_kv) D] projection output."""
    import paged_kv_attention_write_amd as pkv

    rng = np.random.default_rng(4)
    T, hq, h, d, nb, bs = 40, 16, 4, 64, 20, 8
    qkv = workloads.to_storage(rng.standard_normal((T, (hq + 2 * h) * d)).astype(np.float32), "bf16")
    qkv_d = to_dev(qkv, gpu)
    k_new = qkv_d[:, hq * d:(hq + h) * d].view(T, h, d)
    v_new = qkv_d[:, (hq + h) * d:].view(T, h, d)
    kc0 = _pool(rng, nb, bs, h, d, "bf16")
    slots = rng.permutation(nb * bs)[:T].astype(np.int32)
    kd, vd = to_dev(kc0, gpu), to_dev(kc0, gpu)
    pkv.paged_kv_write(k_new, v_new, to_dev(slots, gpu), kd, vd)
    kn = qkv[:, hq * d:(hq + h) * d].reshape(T, h, d)
    vn = qkv[:, (hq + h) * d:].reshape(T, h, d)
    kr, vr = oracle.kv_write(kc0, kc0, "bf16", kn, vn, "bf16", slots)
    assert np.array_equal(to_host(kd), kr) and np.array_equal(to_host(vd), vr)


@pytest.mark.parametrize("config", ["tiny", "decode", "mixed"])
def test_write_of_each_workload(gpu, config):
    """This step's write of each workload at full size: the whole pool compared."""
    import paged_kv_attention_write_amd as pkv

    log(f"write workload {config}")
    c = workloads.make_case(config)
    kd, vd = to_dev(c.k_cache, gpu), to_dev(c.v_cache, gpu)
    pkv.paged_kv_write(to_dev(c.k_new, gpu), to_dev(c.v_new, gpu), to_dev(c.slot_mapping, gpu), kd, vd)
    kr, vr = oracle.kv_write(c.k_cache, c.v_cache, c.kv_dtype, c.k_new, c.v_new, c.new_dtype, c.slot_mapping)
    assert np.array_equal(to_host(kd).view(np.uint8), kr.view(np.uint8))
    assert np.array_equal(to_host(vd).view(np.uint8), vr.view(np.uint8))


def test_write_empty_is_a_no_op(gpu):
    import torch

    import paged_kv_attention_write_amd as pkv

    kc = torch.zeros((2, 16, 2, 64), dtype=torch.bfloat16, device=gpu)
    e = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device=gpu)
    pkv.paged_kv_write(e, e, torch.zeros(0, dtype=torch.int32, device=gpu), kc, kc)
    torch.cuda.synchronize()
    assert int(kc.float().abs().sum().item()) == 0

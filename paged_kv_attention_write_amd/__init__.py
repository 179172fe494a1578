"""Paged-KV attention for AMD MI355X (gfx950): write, decode and mixed step.

The computation lives in ``libpkv.so`` (hand-written HIP kernels behind the C
ABI of include/pkv.h); this package only passes torch tensors to it.

    from paged_kv_attention_write_amd import paged_kv_write, Plan, paged_attn_decode
    paged_kv_write(k_new, v_new, slot_mapping, k_cache, v_cache)
    plan = Plan(context_lens_host, num_q_heads=32, num_kv_heads=8, head_dim=128)
    paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, plan)
"""

from ._abi import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    DTYPE_FP8_E4M3,
    EXPORTS,
    LIB_PATH,
    Plan,
    PkvError,
    PkvPlan,
    decode_plan_image,
    default_queues,
    lib,
    paged_attn_decode,
    paged_attn_decode_write,
    paged_attn_mixed,
    paged_attn_decode_csr,
    paged_attn_mixed_csr,
    paged_kv_write,
    plan_host,
    set_split_event,
    strerror,
)

"""GPU-test plumbing: move generator cases to the device, run the library
through its binding, run the oracle on the same inputs, compare."""

from __future__ import annotations

import sys

import numpy as np

import oracle
import paged_kv_attention_write_amd as pkv

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}  # max-abs error against the fp64 oracle
# A second, scale-aware bound: the error may not exceed REL x the largest
# |output| (plus a small floor).  bf16 output rounding alone is 2^-9
# relative; fp32 accumulation adds far less.  Long contexts have outputs of
# ~0.01-0.04, where the absolute bar alone would pass a 20 % error.
REL = {"f32": 2.0 ** -16, "bf16": 2.0 ** -7, "fp8": 2.0 ** -7}
FLOOR = {"f32": 1e-6, "bf16": 1e-4, "fp8": 1e-4}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dev):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a).copy()).to(dev)


def to_host(t) -> np.ndarray:
    import torch

    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class DeviceCase:
    """A generator case on the GPU after the fill (fp8) and this step's write."""

    def __init__(self, case, dev):
        self.case = case
        self.dev = dev
        self.kc = to_dev(case.k_cache, dev)
        self.vc = to_dev(case.v_cache, dev)
        if case.fill_slots is not None:
            pkv.paged_kv_write(to_dev(case.k_fill, dev), to_dev(case.v_fill, dev), to_dev(case.fill_slots, dev),
                               self.kc, self.vc, case.k_scale, case.v_scale)
        self.k_new = to_dev(case.k_new, dev)
        self.v_new = to_dev(case.v_new, dev)
        self.slots = to_dev(case.slot_mapping, dev)
        self.q = to_dev(case.q, dev)
        self.tables = to_dev(case.block_tables, dev)
        self.ctx = to_dev(case.context_lens, dev)
        self.cu = to_dev(case.cu_seqlens, dev)

    def write(self):
        c = self.case
        pkv.paged_kv_write(self.k_new, self.v_new, self.slots, self.kc, self.vc, c.k_scale, c.v_scale)

    def plan(self, num_queues: int = 0, mixed: bool = False):
        c = self.case
        return pkv.Plan(c.context_lens, c.q_lens if mixed else None, num_q_heads=c.num_q_heads,
                        num_kv_heads=c.num_kv_heads, head_dim=c.head_dim, device=self.dev, num_queues=num_queues)

    def decode(self, plan, out=None):
        import torch

        c = self.case
        out = torch.empty_like(self.q) if out is None else out
        pkv.paged_attn_decode(out, self.q, self.kc, self.vc, self.tables, self.ctx, c.scale, plan, c.k_scale,
                              c.v_scale)
        return out

    def mixed(self, plan, out=None):
        import torch

        c = self.case
        out = torch.empty_like(self.q) if out is None else out
        pkv.paged_attn_mixed(out, self.q, self.kc, self.vc, self.tables, self.cu, self.ctx, c.scale, plan,
                             c.k_scale, c.v_scale)
        return out


def oracle_caches(case, inplace: bool = False):
    """Oracle side of the fill (fp8) and this step's write.  ``inplace`` writes
    into the case's own arrays (large cases, once they are on the device)."""
    kc, vc = case.k_cache, case.v_cache
    if case.fill_slots is not None:
        kc, vc = oracle.kv_write(kc, vc, case.kv_dtype, case.k_fill, case.v_fill, case.new_dtype, case.fill_slots,
                                 case.k_scale, case.v_scale, inplace=inplace)
    return oracle.kv_write(kc, vc, case.kv_dtype, case.k_new, case.v_new, case.new_dtype, case.slot_mapping,
                           case.k_scale, case.v_scale, inplace=inplace)


def oracle_attention(case, kc, vc, seqs=None):
    return oracle.paged_attention(case.q, case.q_dtype, kc, vc, case.kv_dtype, case.block_tables,
                                  case.context_lens, case.cu_seqlens, case.scale, case.k_scale, case.v_scale,
                                  seqs=seqs)


def rows_of(case, seqs):
    cu = case.cu_seqlens
    return np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]) if len(seqs) else np.zeros(0, int)


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)))


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """Assert finite outputs within TOL[dtype] and within the scale-aware bound; return the error."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = max_err(got, ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = min(TOL[dtype], FLOOR[dtype] + REL[dtype] * scale)
    log(f"  {what} max abs err {err:.3e} (bound {bound:.3e}, max|ref| {scale:.3e})")
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e} (max|ref| {scale:.3e})"
    return err

"""ctypes binding of ``libpkv.so`` (the C ABI declared in include/pkv.h).

Argument marshalling only: shapes and dtypes of torch tensors become the
sizes, dtype codes and device pointers the C functions take; every step of
the computation runs in the library's HIP kernels.  The library must be
built (``python -m paged_kv_attention_write_amd.build``); nothing here falls
back to another implementation.
"""

from __future__ import annotations

import ctypes
import os
import time
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_NULL = -1
PKV_ERR_SHAPE = -2
PKV_ERR_DTYPE = -3
PKV_ERR_UNSUPPORTED = -4
PKV_ERR_WORKSPACE = -5
PKV_ERR_PLAN = -6
PKV_ERR_HIP = -7

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_FP8_E4M3 = 2

PLAN_MAGIC = 0x504B5635  # "PKV5", PKV_PLAN_MAGIC in include/pkv.h

# Symbols include/pkv.h declares (checked by the CPU tests).
EXPORTS = (
    "paged_attn_strerror",
    "pkv_abi_version",
    "pkv_set_split_event",
    "paged_kv_write",
    "paged_attn_workspace_size",
    "paged_attn_default_queues",
    "paged_attn_plan_host",
    "paged_attn_plan",
    "paged_attn_plan_capacity",
    "paged_attn_plan_variant",
    "paged_attn_decode",
    "paged_attn_mixed",
    "paged_attn_decode_csr",
    "paged_attn_mixed_csr",
    "paged_attn_decode_noalloc",
    "paged_attn_decode_write",
)


class PkvPlan(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_queues", ctypes.c_int32),
        ("num_units", ctypes.c_int32),
        ("num_merges", ctypes.c_int32),
        ("num_partial_rows", ctypes.c_int32),
        ("target_tiles", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("num_prefill_queues", ctypes.c_int32),
        ("num_prefill_units", ctypes.c_int32),
        ("num_wide_merges", ctypes.c_int32),
        ("num_block_merges", ctypes.c_int32),
        ("max_row_merges", ctypes.c_int32),
        ("max_block_merges", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("logits_soft_cap", ctypes.c_float),
        ("num_tail_queues", ctypes.c_int32),
        ("off_units", ctypes.c_int64),
        ("off_queues", ctypes.c_int64),
        ("off_merges", ctypes.c_int64),
        ("off_partial_o", ctypes.c_int64),
        ("off_partial_lse", ctypes.c_int64),
        ("image_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
    ]


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_attention_write_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        P = ctypes.POINTER
        L.paged_attn_strerror.argtypes = [ctypes.c_int]
        L.paged_attn_strerror.restype = ctypes.c_char_p
        L.pkv_abi_version.argtypes = []
        L.pkv_abi_version.restype = ctypes.c_int
        L.pkv_set_split_event.argtypes = [ctypes.c_void_p]
        L.pkv_set_split_event.restype = ctypes.c_int
        L.paged_kv_write.argtypes = [vp, vp, i32, i64, vp, i64, vp, vp, i32, i64, i32, i32, i32, f32, f32, vp]
        L.paged_kv_write.restype = ctypes.c_int
        L.paged_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, P(sz), P(sz)]
        L.paged_attn_workspace_size.restype = ctypes.c_int
        L.paged_attn_default_queues.argtypes = [P(i32)]
        L.paged_attn_default_queues.restype = ctypes.c_int
        L.paged_attn_plan_host.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, sz, P(PkvPlan)]
        L.paged_attn_plan_host.restype = ctypes.c_int
        L.paged_attn_plan.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, sz, vp, sz, P(PkvPlan), vp]
        L.paged_attn_plan.restype = ctypes.c_int
        L.paged_attn_plan_capacity.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp, sz,
                                               P(PkvPlan), vp]
        L.paged_attn_plan_capacity.restype = ctypes.c_int
        L.paged_attn_plan_variant.argtypes = [vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp, sz, vp, sz,
                                              P(PkvPlan), vp]
        L.paged_attn_plan_variant.restype = ctypes.c_int
        L.paged_attn_decode.argtypes = [vp, vp, i32, i64, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i64, i32,
                                        f32, f32, f32, P(PkvPlan), vp, sz, vp]
        L.paged_attn_decode.restype = ctypes.c_int
        # decode with the step's write: out, q, q_dtype, q stride, k_new, v_new, new_dtype, new stride,
        # slot_mapping, then the decode arguments from k_cache on
        L.paged_attn_decode_write.argtypes = [vp, vp, i32, i64, vp, vp, i32, i64, vp, vp, vp, i32, vp, i32, vp, i32,
                                              i32, i32, i32, i64, i32, f32, f32, f32, P(PkvPlan), vp, sz, vp]
        L.paged_attn_decode_write.restype = ctypes.c_int
        L.paged_attn_mixed.argtypes = [vp, vp, i32, i64, vp, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, i64,
                                       i32, f32, f32, f32, P(PkvPlan), vp, sz, vp]
        L.paged_attn_mixed.restype = ctypes.c_int
        # CSR forms: kv_indptr, kv_indices in place of block_tables, max_blocks
        L.paged_attn_decode_csr.argtypes = [vp, vp, i32, i64, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i64, i32,
                                            f32, f32, f32, P(PkvPlan), vp, sz, vp]
        L.paged_attn_decode_csr.restype = ctypes.c_int
        L.paged_attn_mixed_csr.argtypes = [vp, vp, i32, i64, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                           i64, i32, f32, f32, f32, P(PkvPlan), vp, sz, vp]
        L.paged_attn_mixed_csr.restype = ctypes.c_int
        # the entry point that allocates nothing: the plan image (host) in place of the workspace
        L.paged_attn_decode_noalloc.argtypes = [vp, vp, i32, i64, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i64,
                                                i32, f32, f32, f32, P(PkvPlan), vp, vp]
        L.paged_attn_decode_noalloc.restype = ctypes.c_int
        _lib = L
    return _lib


def set_split_event(event) -> None:
    """Timing hook (pkv_set_split_event): while ``event`` (a ``torch.cuda.Event``
    that has been recorded once, or a raw hipEvent_t as an int) is not None,
    every attention call records it on its stream between its attention
    kernel and its merge kernel.  Process-wide; keep it None during capture."""
    handle = None
    if event is not None:
        handle = int(event.cuda_event) if hasattr(event, "cuda_event") else int(event)
        if handle == 0:
            raise ValueError("set_split_event: the event has no HIP event yet (record it once first)")
    _check(lib().pkv_set_split_event(handle), "pkv_set_split_event")


def strerror(status: int) -> str:
    return lib().paged_attn_strerror(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where)


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------


def _torch():
    import torch

    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _inner_contiguous(t, inner: int, name: str) -> None:
    if t.dim() < 2 or t.shape[1:].numel() != inner:
        raise ValueError(f"{name}: expected [T, ...] with {inner} elements per token")
    if t.shape[0] and (not t[0].is_contiguous() or t.stride(-1) != 1):
        raise ValueError(f"{name}: the per-token [heads, dim] block must be contiguous")


def paged_kv_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale: float = 1.0, v_scale: float = 1.0,
                   stream=None) -> None:
    """Write ``k_new``/``v_new`` ``[T, H_kv, D]`` into the pools by ``slot_mapping`` ``[T]`` (int32)."""
    torch = _torch()
    nb, bs, hkv, d = k_cache.shape
    T = k_new.shape[0]
    _inner_contiguous(k_new, hkv * d, "k_new")
    _inner_contiguous(v_new, hkv * d, "v_new")
    if v_new.stride(0) != k_new.stride(0) or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must have the same shape, dtype and token stride")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if slot_mapping.dtype != torch.int32 or slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must be int32 [T]")
    if not k_cache.is_contiguous() or not v_cache.is_contiguous() or not slot_mapping.is_contiguous():
        raise ValueError("caches and slot_mapping must be contiguous")
    with torch.cuda.device(k_cache.device):
        st = lib().paged_kv_write(_ptr(k_new), _ptr(v_new), dtype_code(k_new), k_new.stride(0) if T else hkv * d,
                                  _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), nb, bs, hkv,
                                  d, float(k_scale), float(v_scale), _stream(stream, k_cache.device))
    _check(st, "paged_kv_write")


def plan_host(context_lens, q_lens, num_q_heads: int, num_kv_heads: int, head_dim: int, num_queues: int, *,
              soft_cap: float = 0.0, window: int = 0):
    """Run the host planner only; returns ``(PkvPlan, image bytes as np.uint8)``.
    A soft-cap or window plans through ``paged_attn_plan_variant`` (host only)."""
    ctx = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    ql = None if q_lens is None else np.ascontiguousarray(np.asarray(q_lens, dtype=np.int32))
    p = PkvPlan()
    ql_ptr = None if ql is None else ql.ctypes.data

    def run(buf, nbytes):
        if soft_cap != 0.0 or window != 0:
            _check(lib().paged_attn_plan_variant(ctx.ctypes.data, ql_ptr, ctx.shape[0], num_q_heads, num_kv_heads,
                                                 head_dim, num_queues, float(soft_cap), int(window), -1, -1, buf,
                                                 nbytes, None, 0, ctypes.byref(p), None), "paged_attn_plan_variant")
        else:
            _check(lib().paged_attn_plan_host(ctx.ctypes.data, ql_ptr, ctx.shape[0], num_q_heads, num_kv_heads,
                                              head_dim, num_queues, buf, nbytes, ctypes.byref(p)),
                   "paged_attn_plan_host")

    run(None, 0)
    image = np.zeros(max(int(p.image_bytes), 1), dtype=np.uint8)
    run(image.ctypes.data, image.nbytes)
    return p, image


UNIT_FIELDS = ("seq", "kv_begin", "kv_end", "row0", "nrows", "pos0", "prow", "kind")
MERGE_FIELDS = ("row0", "nrows", "prow0", "parts")


def decode_plan_image(p: PkvPlan, image: np.ndarray):
    """Split a plan image into (units [U, 8], queue offsets [Q + Qp + 1], merges [M, 4])
    int32 arrays; decode queues come first, then the Qp prefill queues."""
    b = np.asarray(image, dtype=np.uint8)
    units = b[p.off_units:p.off_units + 32 * p.num_units].view(np.int32).reshape(-1, 8)
    queues = b[p.off_queues:p.off_queues + 4 * (p.num_queues + p.num_prefill_queues + 1)].view(np.int32)
    merges = b[p.off_merges:p.off_merges + 16 * p.num_merges].view(np.int32).reshape(-1, 4)
    return units, queues, merges


def default_queues() -> int:
    n = ctypes.c_int32(0)
    _check(lib().paged_attn_default_queues(ctypes.byref(n)), "paged_attn_default_queues")
    return int(n.value)


class Plan:
    """A split-KV plan in a device workspace, reusable by every layer of a step.

    Holds the plan descriptor, two pinned host staging buffers used in turn
    for the upload (so a new plan never waits for the previous upload) and
    the device workspace (all allocated through torch).  ``update`` re-plans
    for new lengths into the same buffers when they are large enough.  The
    upload is ordered on the stream like any kernel, so a re-plan issued
    after the previous step's attention calls on the same stream is safe.
    ``last_plan_s`` is the host time of the last planner call (plan and
    upload issue) and ``last_wait_s`` the time spent waiting for a staging
    buffer to come free before it.

    ``capacity=(max_seqs, max_tokens)`` makes every plan of this object use
    ``paged_attn_plan_capacity``: buffers sized for the capacity are allocated
    once and never replaced, and the image keeps the same offsets, so attention
    calls captured into a HIP graph (e.g. ``torch.cuda.CUDAGraph``) stay valid
    across updates with the same q_lens.

    ``soft_cap`` (> 0: scores pass through ``c * tanh(s / c)``) and ``window``
    (> 0: a row at position p sees keys p - window < j <= p) select an
    attention variant through ``paged_attn_plan_variant``; every attention
    call made with the plan computes that variant.
    """

    def __init__(self, context_lens, q_lens=None, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 device=None, num_queues: int = 0, stream=None, capacity=None, soft_cap: float = 0.0,
                 window: int = 0):
        torch = _torch()
        self.soft_cap, self.window = float(soft_cap), int(window)
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        with torch.cuda.device(self.device):
            self.num_queues = int(num_queues) if num_queues and num_queues > 0 else default_queues()
        self._staging = [None, None]
        self._uploaded = [None, None]
        self._turn = 0
        self.workspace = None
        self.desc = PkvPlan()
        self.capacity = None
        if capacity is not None:
            max_seqs, max_tokens = (int(x) for x in capacity)
            ws_b, host_b = ctypes.c_size_t(0), ctypes.c_size_t(0)
            _check(lib().paged_attn_workspace_size(max_seqs, max_tokens, num_q_heads, head_dim, self.num_queues,
                                                   ctypes.byref(ws_b), ctypes.byref(host_b)),
                   "paged_attn_workspace_size")
            self._staging = [torch.empty(max(int(host_b.value), 256), dtype=torch.uint8, pin_memory=True)
                             for _ in range(2)]
            self.workspace = torch.empty(max(int(ws_b.value), 256), dtype=torch.uint8, device=self.device)
            self.capacity = (max_seqs, max_tokens)
        self.update(context_lens, q_lens, stream=stream)

    def update(self, context_lens, q_lens=None, stream=None) -> "Plan":
        torch = _torch()
        ctx = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
        ql = None if q_lens is None else np.ascontiguousarray(np.asarray(q_lens, dtype=np.int32))
        ql_ptr = None if ql is None else ql.ctypes.data
        i = self._turn
        self._turn ^= 1
        t0 = time.perf_counter()
        if self._uploaded[i] is not None:
            self._uploaded[i].synchronize()  # this staging buffer's last upload (two updates ago) has run
        self.last_wait_s = time.perf_counter() - t0
        with torch.cuda.device(self.device):
            st_ptr = _stream(stream, self.device)
            for attempt in range(2):
                staging, ws = self._staging[i], self.workspace
                t1 = time.perf_counter()
                variant = self.soft_cap != 0.0 or self.window != 0
                if variant:
                    max_seqs, max_tokens = self.capacity if self.capacity is not None else (-1, -1)
                    st = lib().paged_attn_plan_variant(ctx.ctypes.data, ql_ptr, ctx.shape[0], self.num_q_heads,
                                                       self.num_kv_heads, self.head_dim, self.num_queues,
                                                       self.soft_cap, self.window, max_seqs, max_tokens,
                                                       staging.data_ptr() if staging is not None else None,
                                                       staging.numel() if staging is not None else 0,
                                                       ws.data_ptr() if ws is not None else None,
                                                       ws.numel() if ws is not None else 0, ctypes.byref(self.desc),
                                                       st_ptr)
                    if st == PKV_OK and ws is None:  # a host-only call: no workspace yet
                        st = PKV_ERR_WORKSPACE
                elif self.capacity is not None:
                    st = lib().paged_attn_plan_capacity(ctx.ctypes.data, ql_ptr, ctx.shape[0], self.num_q_heads,
                                                        self.num_kv_heads, self.head_dim, self.num_queues,
                                                        self.capacity[0], self.capacity[1], staging.data_ptr(),
                                                        staging.numel(), ws.data_ptr(), ws.numel(),
                                                        ctypes.byref(self.desc), st_ptr)
                else:
                    st = lib().paged_attn_plan(ctx.ctypes.data, ql_ptr, ctx.shape[0], self.num_q_heads,
                                               self.num_kv_heads, self.head_dim, self.num_queues,
                                               staging.data_ptr() if staging is not None else None,
                                               staging.numel() if staging is not None else 0,
                                               ws.data_ptr() if ws is not None else None,
                                               ws.numel() if ws is not None else 0, ctypes.byref(self.desc), st_ptr)
                self.last_plan_s = time.perf_counter() - t1
                if st in (PKV_ERR_WORKSPACE, PKV_ERR_NULL) and attempt == 0 and self.capacity is None:
                    probe = PkvPlan()
                    if variant:
                        _check(lib().paged_attn_plan_variant(ctx.ctypes.data, ql_ptr, ctx.shape[0], self.num_q_heads,
                                                             self.num_kv_heads, self.head_dim, self.num_queues,
                                                             self.soft_cap, self.window, -1, -1, None, 0, None, 0,
                                                             ctypes.byref(probe), None), "paged_attn_plan_variant")
                    else:
                        _check(lib().paged_attn_plan_host(ctx.ctypes.data, ql_ptr, ctx.shape[0], self.num_q_heads,
                                                          self.num_kv_heads, self.head_dim, self.num_queues, None, 0,
                                                          ctypes.byref(probe)), "paged_attn_plan_host")
                    if staging is None or staging.numel() < probe.image_bytes:
                        self._staging[i] = torch.empty(max(int(probe.image_bytes), 256), dtype=torch.uint8,
                                                       pin_memory=True)
                    if ws is None or ws.numel() < probe.workspace_bytes:
                        self.workspace = torch.empty(max(int(probe.workspace_bytes), 256), dtype=torch.uint8,
                                                     device=self.device)
                    continue
                break
            _check(st, "paged_attn_plan")
            ev = torch.cuda.Event()
            ev.record(torch.cuda.current_stream(self.device) if stream is None else stream)
            self._uploaded[i] = ev
        self.context_lens = ctx
        self.q_lens = ql
        return self


def _attn_common(q, k_cache, v_cache, block_tables, context_lens, plan):
    torch = _torch()
    nb, bs, hkv, d = k_cache.shape
    if q.dim() != 3 or q.shape[2] != d or q.stride(-1) != 1 or (q.shape[0] and not q[0].is_contiguous()):
        raise ValueError("q must be [T, Hq, D] with contiguous heads")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    if block_tables.dtype != torch.int32 or not block_tables.is_contiguous() or block_tables.dim() != 2:
        raise ValueError("block_tables must be contiguous int32 [B, max_blocks]")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    return nb, bs, hkv, d


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, plan: Plan,
                      k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """One query row per sequence: ``out[B, Hq, D] = attention(q[B, Hq, D], paged K/V)``."""
    torch = _torch()
    nb, bs, hkv, d = _attn_common(q, k_cache, v_cache, block_tables, context_lens, plan)
    B, hq = q.shape[0], q.shape[1]
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    with torch.cuda.device(q.device):
        st = lib().paged_attn_decode(_ptr(out), _ptr(q), dtype_code(q), q.stride(0) if B else hq * d, _ptr(k_cache),
                                     _ptr(v_cache), dtype_code(k_cache), _ptr(block_tables), block_tables.shape[1],
                                     _ptr(context_lens), B, hq, hkv, d, nb, bs, float(scale), float(k_scale),
                                     float(v_scale), ctypes.byref(plan.desc), _ptr(plan.workspace),
                                     plan.workspace.numel(), _stream(stream, q.device))
    _check(st, "paged_attn_decode")


def paged_attn_decode_write(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                            scale: float, plan: Plan, k_scale: float = 1.0, v_scale: float = 1.0,
                            stream=None) -> None:
    """A decode step's write and attention in one call: ``paged_kv_write(k_new, v_new,
    slot_mapping, ...)`` then ``paged_attn_decode(...)``, where token ``s`` of ``k_new`` /
    ``v_new`` ``[B, H_kv, D]`` is sequence ``s``'s new key and value and ``slot_mapping[s]``
    the slot of its key ``context_lens[s] - 1`` (or < 0: nothing written)."""
    torch = _torch()
    nb, bs, hkv, d = _attn_common(q, k_cache, v_cache, block_tables, context_lens, plan)
    B, hq = q.shape[0], q.shape[1]
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    _inner_contiguous(k_new, hkv * d, "k_new")
    _inner_contiguous(v_new, hkv * d, "v_new")
    if k_new.shape[0] != B or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype or \
            v_new.stride(0) != k_new.stride(0):
        raise ValueError("k_new and v_new must be [B, H_kv, D] with one dtype and token stride")
    if slot_mapping.dtype != torch.int32 or slot_mapping.shape[0] != B or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int32 [B]")
    with torch.cuda.device(q.device):
        st = lib().paged_attn_decode_write(_ptr(out), _ptr(q), dtype_code(q), q.stride(0) if B else hq * d,
                                           _ptr(k_new), _ptr(v_new), dtype_code(k_new),
                                           k_new.stride(0) if B else hkv * d, _ptr(slot_mapping), _ptr(k_cache),
                                           _ptr(v_cache), dtype_code(k_cache), _ptr(block_tables),
                                           block_tables.shape[1], _ptr(context_lens), B, hq, hkv, d, nb, bs,
                                           float(scale), float(k_scale), float(v_scale), ctypes.byref(plan.desc),
                                           _ptr(plan.workspace), plan.workspace.numel(), _stream(stream, q.device))
    _check(st, "paged_attn_decode_write")


def _csr_check(kv_indptr, kv_indices, B):
    torch = _torch()
    if kv_indptr.dtype != torch.int32 or kv_indptr.dim() != 1 or kv_indptr.shape[0] != B + 1 or \
            not kv_indptr.is_contiguous():
        raise ValueError("kv_indptr must be contiguous int32 [B+1]")
    if kv_indices.dtype != torch.int32 or kv_indices.dim() != 1 or not kv_indices.is_contiguous():
        raise ValueError("kv_indices must be contiguous int32 [nnz]")


def paged_attn_decode_csr(out, q, k_cache, v_cache, kv_indptr, kv_indices, context_lens, scale: float, plan: Plan,
                          k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """``paged_attn_decode`` with the page table in CSR form: sequence ``s``
    reads its pages from ``kv_indices[kv_indptr[s]:kv_indptr[s+1]]``."""
    torch = _torch()
    B, hq = q.shape[0], q.shape[1]
    dummy = kv_indices.view(1, -1) if kv_indices.numel() else kv_indices.new_zeros((1, 1))
    nb, bs, hkv, d = _attn_common(q, k_cache, v_cache, dummy, context_lens, plan)
    _csr_check(kv_indptr, kv_indices, B)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    with torch.cuda.device(q.device):
        st = lib().paged_attn_decode_csr(_ptr(out), _ptr(q), dtype_code(q), q.stride(0) if B else hq * d,
                                         _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), _ptr(kv_indptr),
                                         _ptr(dummy), _ptr(context_lens), B, hq, hkv, d, nb, bs, float(scale),
                                         float(k_scale), float(v_scale), ctypes.byref(plan.desc),
                                         _ptr(plan.workspace), plan.workspace.numel(), _stream(stream, q.device))
    _check(st, "paged_attn_decode_csr")


def paged_attn_mixed_csr(out, q, k_cache, v_cache, kv_indptr, kv_indices, cu_seqlens, context_lens, scale: float,
                         plan: Plan, k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """``paged_attn_mixed`` with the page table in CSR form."""
    torch = _torch()
    T, hq = q.shape[0], q.shape[1]
    B = context_lens.shape[0]
    dummy = kv_indices.view(1, -1) if kv_indices.numel() else kv_indices.new_zeros((1, 1))
    nb, bs, hkv, d = _attn_common(q, k_cache, v_cache, dummy, context_lens, plan)
    _csr_check(kv_indptr, kv_indices, B)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.shape[0] != B + 1:
        raise ValueError("cu_seqlens must be int32 [B+1]")
    with torch.cuda.device(q.device):
        st = lib().paged_attn_mixed_csr(_ptr(out), _ptr(q), dtype_code(q), q.stride(0) if T else hq * d,
                                        _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), _ptr(kv_indptr),
                                        _ptr(dummy), _ptr(cu_seqlens), _ptr(context_lens), B, T, hq, hkv, d, nb, bs,
                                        float(scale), float(k_scale), float(v_scale), ctypes.byref(plan.desc),
                                        _ptr(plan.workspace), plan.workspace.numel(), _stream(stream, q.device))
    _check(st, "paged_attn_mixed_csr")


def paged_attn_mixed(out, q, k_cache, v_cache, block_tables, cu_seqlens, context_lens, scale: float, plan: Plan,
                     k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Packed batch: ``out[T, Hq, D]`` for rows ``cu_seqlens[s]..cu_seqlens[s+1]`` of each sequence."""
    torch = _torch()
    nb, bs, hkv, d = _attn_common(q, k_cache, v_cache, block_tables, context_lens, plan)
    T, hq = q.shape[0], q.shape[1]
    B = context_lens.shape[0]
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.shape[0] != B + 1:
        raise ValueError("cu_seqlens must be int32 [B+1]")
    with torch.cuda.device(q.device):
        st = lib().paged_attn_mixed(_ptr(out), _ptr(q), dtype_code(q), q.stride(0) if T else hq * d, _ptr(k_cache),
                                    _ptr(v_cache), dtype_code(k_cache), _ptr(block_tables), block_tables.shape[1],
                                    _ptr(cu_seqlens), _ptr(context_lens), B, T, hq, hkv, d, nb, bs, float(scale),
                                    float(k_scale), float(v_scale), ctypes.byref(plan.desc), _ptr(plan.workspace),
                                    plan.workspace.numel(), _stream(stream, q.device))
    _check(st, "paged_attn_mixed")

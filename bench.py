#!/usr/bin/env python3
"""Benchmark: paged KV attention on one MI355X.

Default workload (``--config decode``): one decode step of a Qwen3-4B-shaped
model's attention: the split-KV plan once on the host, then for each of the
36 layers the write of this step's K/V (64 new tokens) and the paged decode
over that layer's own pool (64 sequences, context uniform in [512, 4096], 32
query / 8 KV heads, head dim 128, page 16, bf16).  The plan is made once per
step and reused by every layer, as the planner's description on "How Easy Is
It to Start Serving LLMs?" (Phase 4 §3) has it.  Other workloads:
``long-page1`` / ``long-page16`` / ``long-contig`` (16 x 32768 keys, the
scattered-vs-contiguous comparison), ``fp8prefix`` (128 sequences over a
shared 4096-token prefix, fp8 cache; ``bf16prefix`` the same with a bf16
cache, for the comparison), ``mixed`` (63 decodes and one 512-row
prefill chunk packed in one step; "nanoserve" chunked prefill) and
``mixed-chunk`` (that chunk alone, to read the matrix-core tile against its
peak), ``specverify`` (64 sequences with 4 new rows each, a speculative
verify step, through the mixed path).  ``--study skew``, ``--study
plan-cost``, ``--study pages``, ``--study read-peak`` and ``--study gather``
print, instead of the bench line, one JSON line per case of the load-balance
study (length mixes of equal total tokens at batch 4-128), the planner-cost
sweep (batch 8-512), the page-size sweep (pages of 1/4/16/64 tokens and a
contiguous slab at 64 x 4K, 16 x 16K and 256 x 1K keys, each case's layer 0
checked against the oracle on sampled sequences), the measured read ceilings
of the streaming-read probe, and the decode call against the gather path it
replaces (K/V gathered into a padded contiguous copy, then dense attention
in torch; a comparator only, never part of the library).

Inputs are synthetic: block tables, lengths and slots come from the seeded
generator in workloads/; K/V/Q values are N(0, 1) drawn on the GPU from a
seeded torch generator per layer and rounded to bf16 (fp8: quantised by the
library's own write).  They are resident in HBM before timing starts.

Printed: one JSON line.  ``value`` is the step's algorithmic bytes (every
valid K/V element, q, out, table entries, lengths, and the write's bytes) over
its wall time, in TB/s.  The step is timed twice: as eager launches (with HIP
events around every attention call, which feed ``roofline``) and, unless
``--no-graph``, as one captured HIP graph of all the layers' writes and
attention calls, replayed after each step's re-plan into a fixed-capacity
workspace; ``value`` and ``ms_per_step`` come from the faster of the two
forms then (both step times, and which one was used, are in ``graph``), and
layer 0's output of the last replay is the one checked against the oracle.  A decode step over bf16 pages of whole
16-token tiles calls ``paged_attn_decode_write`` (the new tokens written
inside the decode launch, one call per layer); other steps, and
``--separate-write``, call ``paged_kv_write`` and then the attention.
``roofline`` covers the dominant kernel: the attention kernel of the
attention call (or of the call that writes and attends), timed with HIP
events on its stream from before the call to the event the library records
between that kernel and the merge kernel (``pkv_set_split_event``, set on
every other timed step: the record costs its call about 3 us), against the
call's algorithmic bytes (and the new tokens' when it writes them);
``roofline.call`` gives the same for the whole call, merge kernel included,
from the timed steps without the split event.
With prefill chunks in the step it reads the chunk's flops against the bf16
matrix-core peak when that fraction is the larger.
``cpu_baseline`` is the fp64 CPU oracle (write + attention of layer 0) timed
on this host's cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_TBS = 8.0
METRIC = "paged-decode attn achieved HBM TB/s (% of peak) + µs/layer, Qwen3-4B shape"
LAYERS = 36  # Qwen3-4B decoder layers

CONFIGS = {
    "decode": dict(config="decode", layout="page16", desc="64 seqs, ctx U[512,4096], 32q/8kv heads, D=128, page 16, bf16 KV"),
    "long-page1": dict(config="long", layout="page1", desc="16 seqs x 32768, 32q/8kv, D=128, page 1 shuffled, bf16"),
    "long-page16": dict(config="long", layout="page16", desc="16 seqs x 32768, 32q/8kv, D=128, page 16 shuffled, bf16"),
    "long-contig": dict(config="long", layout="contig", desc="16 seqs x 32768, 32q/8kv, D=128, contiguous slab, bf16"),
    "fp8prefix": dict(config="fp8prefix", layout="page16", kv="fp8",
                      desc="128 seqs, 4096 shared + 256 private tokens, fp8 E4M3 KV"),
    "bf16prefix": dict(config="fp8prefix", layout="page16",
                       desc="the fp8prefix sequences and shared pages with a bf16 KV cache (the fp8 cache's "
                            "comparison)"),
    "mixed": dict(config="mixed", layout="page16",
                  desc="63 decodes (ctx U[256,2048]) + one 512-row chunk over 2048 cached tokens, packed T=575, "
                       "32q/8kv, D=128, page 16, bf16"),
    "specverify": dict(config="decode", layout="page16", q_len=4,
                       desc="64 seqs x 4 new rows each (speculative verify), ctx U[512,4096], 32q/8kv, D=128, "
                            "page 16, bf16; all rows through the mixed path"),
    "mixed-chunk": dict(config="mixed", layout="page16", only_chunk=True,
                        desc="the 512-row chunk of the mixed step alone (2560 keys, causal), 32q/8kv, D=128, bf16"),
}
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_layers(torch, st, cfg, layers, dev):
    """Per-layer pools, queries and new K/V on the GPU (seeded)."""
    import workloads

    hq, hkv, d = 32, 8, 128
    nb, bs = st["num_blocks"], st["block_size"]
    B = int(st["q_lens"].sum())  # query rows (one per sequence for decode)
    fp8 = cfg.get("kv") == "fp8"
    out = []
    for l in range(layers):
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + l)
        layer = {}
        if fp8:
            kc = torch.empty((nb, bs, hkv, d), dtype=torch.uint8, device=dev)
            vc = torch.empty_like(kc)
        else:
            kc = torch.randn((nb, bs, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            vc = torch.randn((nb, bs, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        layer["kc"], layer["vc"] = kc, vc
        layer["q"] = torch.randn((B, hq, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        layer["k_new"] = torch.randn((B, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        layer["v_new"] = torch.randn((B, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        layer["out"] = torch.empty_like(layer["q"])
        out.append(layer)
    return out


def fill_fp8(torch, pkv, layers, st, dev):
    """Fill every fp8 pool by the quantising write from N(0,1) bf16 values."""
    nb, bs = st["num_blocks"], st["block_size"]
    hkv, d = 8, 128
    slots_all = torch.arange(nb * bs, dtype=torch.int32, device=dev)
    scales = []
    for i, layer in enumerate(layers):
        g = torch.Generator(device=dev)
        g.manual_seed(5000 + i)
        k = torch.randn((nb * bs, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        v = torch.randn((nb * bs, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        ks = float(np.float32(k.float().abs().max().item()) / np.float32(448.0))
        vs = float(np.float32(v.float().abs().max().item()) / np.float32(448.0))
        pkv.paged_kv_write(k, v, slots_all, layer["kc"], layer["vc"], ks, vs)
        scales.append((ks, vs))
        del k, v
    return scales


def cpu_baseline(torch, st, layer, kv_dtype, scales, budget_s=10.0, soft_cap=0.0, window=0):
    """The fp64 oracle on layer 0 (write + attention), repeated up to ~budget_s."""
    import oracle
    from workloads import byte_model

    def host(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    kc, vc = host(layer["kc"]), host(layer["vc"])
    q, kn, vn = host(layer["q"]), host(layer["k_new"]), host(layer["v_new"])
    ks, vs = scales
    B = st["context_lens"].shape[0]
    T = int(st["q_lens"].sum())
    cu = st["cu_seqlens"]
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    reps, t0 = 0, time.perf_counter()
    while True:
        k2, v2 = oracle.kv_write(kc, vc, kv_dtype, kn, vn, "bf16", st["slot_mapping"], ks, vs)
        out, _ = oracle.paged_attention(q, "bf16", k2, v2, kv_dtype, st["block_tables"], st["context_lens"], cu,
                                        scale, ks, vs, soft_cap=soft_cap, window=window)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    kvb = 1 if kv_dtype == "fp8" else 2
    nbytes = byte_model.attention_bytes(st["context_lens"], st["q_lens"], 32, 8, 128, st["block_size"], kvb, 2,
                                        window=window) + byte_model.write_bytes(T, 8, 128, 2, kvb)
    try:
        from threadpoolctl import threadpool_info

        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    cores = len(os.sched_getaffinity(0))
    return {"value": nbytes / per / 1e12, "unit": "TB/s", "cores": int(blas or cores),
            "kind": "oracle", "host_cores": cores, "seconds_per_layer_call": per,
            "sample": f"layer 0 of the step (write of {T} tokens + attention of all {B} sequences), "
                      f"{reps} repetition(s), fp64 NumPy oracle", "out": out}


COPY_BYTES = 1 << 30

# Sources that define the kernels of one paged_attn_decode call (decode and
# merge kernels, the plan they walk); a paged_attn_mixed call also runs the
# prefill, mixed and few-row kernels.  A traffic record taken from the byte
# counters is reported only while the sources of its call are unchanged.
DECODE_SOURCES = ["pkv_decode.hip", "pkv_decode_unit.h", "pkv_device.h", "pkv_attention.h", "pkv_internal.h", "pkv_plan.cpp"]
MIXED_SOURCES = DECODE_SOURCES + ["pkv_prefill.hip"]
# configs whose calls go through paged_attn_mixed, or through the few-row
# kernel (fp8 decode)
PREFILL_CONFIGS = ("mixed", "mixed-chunk", "specverify", "fp8prefix")


def decode_source_digest(sources=None):
    import hashlib

    h = hashlib.sha256()
    for f in sources or DECODE_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_attention_write_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(config):
    """HBM bytes per call from a committed counter summary (profiles/*.md,
    a line 'traffic-record: {json}'), or None if there is none for this
    config or the kernels changed since it was taken."""
    d = os.path.join(ROOT, "profiles")
    if not os.path.isdir(d):
        return None
    digest = decode_source_digest(MIXED_SOURCES if config.split("+")[0] in PREFILL_CONFIGS else DECODE_SOURCES)
    for name in sorted(os.listdir(d)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(d, name)) as fh:
            for line in fh:
                if line.startswith("traffic-record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("config") == config and rec.get("source_sha256") == digest:
                        return rec
    return None


def copy_calibration(torch):
    """A plain 1 GiB device-to-device copy, three times: under a counter run
    its FETCH_SIZE / WRITE_SIZE per dispatch against 1 GiB read / written
    gives the factor that turns those counters into bytes."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for i in range(3):
        dst.copy_(src)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "dispatches": 3,
                      "copy_ms": ms, "copy_read_plus_write_TBps": [2 * COPY_BYTES / (m * 1e-3) / 1e12 for m in ms]}),
          flush=True)


PROBE_LIB = os.path.join(ROOT, "paged_kv_attention_write_amd", "libpkv_probe.so")


def probe_read_GBps(torch, nbytes, reps=20, pages=None, page_bytes=0, pool=None):
    """HBM read rate of the streaming probe (libpkv_probe.so): one persistent
    8-wave workgroup per CU reading 16 bytes per lane, non-temporal.  Without
    ``pages`` it reads ``nbytes`` contiguous bytes, rotating over four
    disjoint windows of a buffer four times that size so that no launch finds
    its bytes in the last-level cache; with ``pages`` (a device int32 list of
    page ids into ``pool``, a uint8 device buffer of whole pages) it reads
    those pages whole, in list order.  Median over ``reps`` launches timed
    with HIP events on the current stream, in GB/s."""
    import ctypes

    L = ctypes.CDLL(PROBE_LIB)
    L.pkv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.pkv_probe_read.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    blocks = int(props.multi_processor_count)
    sink = torch.empty(blocks, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if pages is None:
        nbytes = nbytes // 16 * 16
        buf = torch.ones(4 * nbytes, dtype=torch.uint8, device=dev)
        args = [(buf.data_ptr() + (i % 4) * nbytes, nbytes, None, 0, 0, 0) for i in range(reps + 4)]
        moved = nbytes
    else:
        args = [(pool.data_ptr(), 0, pages.data_ptr(), pages.numel(), page_bytes, pool.numel() // page_bytes)] * (reps + 4)
        moved = pages.numel() * page_bytes
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(args))]
    for i, a in enumerate(args):
        ev[2 * i].record(stream)
        st = L.pkv_probe_read(*a, sink.data_ptr(), blocks, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"pkv_probe_read failed ({st})")
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(4, len(args))])
    return moved / (float(np.median(ms)) * 1e-3) / 1e9


def study_read_peak(args, torch, workloads):
    """Measured read ceilings: the streaming probe over contiguous buffers of
    the decode call's size and of 2 GiB, and over the K and V pages of the
    decode workload's and the long workload's shuffled page-16 tables (each
    page of 16 tokens x 8 kv heads x 128 x bf16 = 32 KiB read whole)."""
    dev = torch.device("cuda:0")
    from workloads import byte_model

    st = workloads.structure_only("decode", "page16")
    call = byte_model.attention_bytes(st["context_lens"], st["q_lens"], 32, 8, 128, 16, 2, 2)
    for nbytes in (call, 2 << 30):
        gbs = probe_read_GBps(torch, nbytes)
        print(json.dumps({"study": "read-peak", "pattern": "contiguous", "bytes": int(nbytes // 16 * 16),
                          "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / 8000.0, 4)}), flush=True)
    page_bytes = 16 * 8 * 128 * 2
    for config, layout in (("decode", "page16"), ("long", "page16")):
        st = workloads.structure_only(config, layout)
        nb = int(st["num_blocks"])
        used = np.concatenate([st["block_tables"][s, :-(-int(n) // 16)]
                               for s, n in enumerate(st["context_lens"])]).astype(np.int64)
        ids = np.stack([used, used + nb], axis=1).reshape(-1).astype(np.int32)  # K page, then its V page
        pool = torch.ones(2 * nb * page_bytes, dtype=torch.uint8, device=dev)
        pages = torch.from_numpy(ids).to(dev)
        gbs = probe_read_GBps(torch, 0, pages=pages, page_bytes=page_bytes, pool=pool)
        print(json.dumps({"study": "read-peak", "pattern": f"{config} K/V pages (page 16, shuffled)",
                          "pages": int(ids.size), "bytes": int(ids.size * page_bytes), "GBps": round(gbs, 1),
                          "frac_of_8TBps": round(gbs / 8000.0, 4)}), flush=True)
        del pool, pages
        torch.cuda.empty_cache()


def queue_balance(pkv, st, num_queues):
    """Largest over mean decode-queue load of the host plan, in 16-key tiles."""
    from paged_kv_attention_write_amd import _abi

    p, image = _abi.plan_host(st["context_lens"], None, 32, 8, 128, num_queues)
    units, qoff, _ = _abi.decode_plan_image(p, image)
    ctx = st["context_lens"]
    ends = np.minimum(units[:, 2], ctx[units[:, 0]])
    tiles = np.maximum(0, -(-(ends - units[:, 1]) // 16))
    loads = np.array([tiles[qoff[q]:qoff[q + 1]].sum() for q in range(int(p.num_queues))], dtype=np.float64)
    return float(loads.max() / loads.mean()) if loads.mean() > 0 else 1.0


def study_skew(args, torch, pkv, workloads, byte_model):
    """Load-balance study: decode calls over length mixes of equal total
    tokens (uniform, one long sequence holding half, Pareto-tailed) at batch
    4 / 16 / 64 / 128, one JSON line per case."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    for batch in (4, 16, 64, 128):
        for mix in workloads.SKEW_MIXES:
            lens = workloads.skew_lengths(mix, batch)
            st = workloads.structure_for_lengths(workloads.CONFIG_IDS["skew"], lens)
            layers = build_layers(torch, st, {"config": "decode"}, args.layers, dev)
            tables = torch.from_numpy(st["block_tables"]).to(dev)
            ctx = torch.from_numpy(st["context_lens"]).to(dev)
            plan = pkv.Plan(lens, None, num_q_heads=32, num_kv_heads=8, head_dim=128, device=dev,
                            num_queues=args.queues)
            n = args.steps * len(layers)
            ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            plan_s = []
            for it in range(args.warmup + args.steps):
                plan.update(lens, None)
                plan_s.append(plan.last_plan_s)
                for l, layer in enumerate(layers):
                    k = (it - args.warmup) * len(layers) + l
                    if k >= 0:
                        ev_a[k].record(stream)
                    pkv.paged_attn_decode(layer["out"], layer["q"], layer["kc"], layer["vc"], tables, ctx, scale, plan)
                    if k >= 0:
                        ev_b[k].record(stream)
            torch.cuda.synchronize()
            ms = np.array([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)])
            nbytes = byte_model.attention_bytes(lens, st["q_lens"], 32, 8, 128, st["block_size"], 2, 2)
            p50 = float(np.median(ms)) * 1e-3
            print(json.dumps({
                "study": "skew", "mix": mix, "batch": batch, "total_tokens": int(lens.sum()),
                "longest": int(lens.max()), "shortest": int(lens.min()),
                "call_us": {"p10": round(float(np.percentile(ms, 10)) * 1e3, 2), "p50": round(p50 * 1e6, 2),
                            "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)},
                "TBps": round(nbytes / p50 / 1e12, 4), "frac_of_8TBps": round(nbytes / p50 / 8e12, 4),
                "plan": {"queues": int(plan.desc.num_queues), "units": int(plan.desc.num_units),
                         "merges": int(plan.desc.num_merges),
                         "max_over_mean_queue_tiles": round(queue_balance(pkv, st, int(plan.desc.num_queues)), 4),
                         "plan_us_per_step": round(float(np.median(plan_s)) * 1e6, 2)},
                "layers": len(layers)}), flush=True)
            del layers, plan
            torch.cuda.empty_cache()


def study_pages(args, torch, pkv, workloads, byte_model):
    """Page-size sweep: decode over equal-length batches of the pages' three
    shapes (64 x 4096, 16 x 16384, 256 x 1024 keys), pages of 1, 4, 16 and 64
    tokens in shuffled order and one contiguous slab (page 16 in order), one
    JSON line per case.  The five layouts of a shape are resident together
    and their calls alternate (the starting layout rotating every step), so
    that the ratios to the contiguous slab compare calls made under the same
    conditions."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    layouts = (("contiguous", 16), ("shuffled", 1), ("shuffled", 4), ("shuffled", 16), ("shuffled", 64))
    for batch, n in ((64, 4096), (16, 16384), (256, 1024)):
        lens = np.full(batch, n, np.int32)
        cases = []
        for layout, bs in layouts:
            st = workloads.structure_for_lengths(workloads.CONFIG_IDS["skew"], lens, block_size=bs,
                                                 layout="identity" if layout == "contiguous" else "shuffle")
            layers = build_layers(torch, st, {"config": "decode"}, args.layers, dev)
            tables = torch.from_numpy(st["block_tables"]).to(dev)
            ctx = torch.from_numpy(st["context_lens"]).to(dev)
            plan = pkv.Plan(lens, None, num_q_heads=32, num_kv_heads=8, head_dim=128, device=dev,
                            num_queues=args.queues)
            cases.append(dict(layout=layout, bs=bs, st=st, layers=layers, tables=tables, ctx=ctx, plan=plan, ev=[]))
        for it in range(args.warmup + args.steps):
            k = it % len(cases)
            for c in cases[k:] + cases[:k]:
                for layer in c["layers"]:
                    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a_.record(stream)
                    pkv.paged_attn_decode(layer["out"], layer["q"], layer["kc"], layer["vc"], c["tables"], c["ctx"],
                                          scale, c["plan"])
                    b_.record(stream)
                    if it >= args.warmup:
                        c["ev"].append((a_, b_))
        torch.cuda.synchronize()
        ref_us = None
        for c in cases:
            ms = np.array([a_.elapsed_time(b_) for a_, b_ in c["ev"]])
            nbytes = byte_model.attention_bytes(lens, c["st"]["q_lens"], 32, 8, 128, c["bs"], 2, 2)
            p50 = float(np.median(ms)) * 1e-3
            if c["layout"] == "contiguous":
                ref_us = p50
            cb = pages_cpu_baseline(torch, c["st"], c["layers"][0], scale)
            print(json.dumps({
                "study": "pages", "batch": batch, "context": n, "layout": c["layout"], "block_size": c["bs"],
                "table_entries": int(c["st"]["block_tables"].size),
                "call_us": {"p10": round(float(np.percentile(ms, 10)) * 1e3, 2), "p50": round(p50 * 1e6, 2),
                            "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)},
                "TBps": round(nbytes / p50 / 1e12, 4), "frac_of_8TBps": round(nbytes / p50 / 8e12, 4),
                "vs_contiguous": round(ref_us / p50, 4), "layers": len(c["layers"]), "cpu_baseline": cb}),
                  flush=True)
            if not cb["parity"]["ok"]:
                raise SystemExit(f"page-size sweep: layer 0 differs from the oracle at {c['layout']} page {c['bs']}")
        del cases
        torch.cuda.empty_cache()


def pages_cpu_baseline(torch, st, layer, scale, samples=6):
    """The cpu_baseline leg of a page-size sweep case: the fp64 oracle timed
    on a sample of sequences of layer 0 (first, last and evenly spaced ones),
    and layer 0's output of the timed calls compared with it under the
    library's bf16 bound (max-abs 2e-2 and 2^-7 of the largest |output|)."""
    import oracle

    def host(t):
        t = t.detach().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    B = st["context_lens"].shape[0]
    seqs = sorted(set(np.linspace(0, B - 1, samples).round().astype(int).tolist()))
    kc, vc, q = host(layer["kc"]), host(layer["vc"]), host(layer["q"])
    t0 = time.perf_counter()
    ref, _ = oracle.paged_attention(q, "bf16", kc, vc, "bf16", st["block_tables"], st["context_lens"],
                                    st["cu_seqlens"], scale, seqs=seqs)
    el = time.perf_counter() - t0
    got = layer["out"].float().cpu().numpy().astype(np.float64)
    rows = np.asarray(seqs)
    err = float(np.max(np.abs(got[rows] - ref[rows])))
    bound = min(2e-2, 1e-4 + 2.0 ** -7 * float(np.max(np.abs(ref[rows]))))
    toks = int(st["context_lens"][rows].sum())
    return {"kind": "oracle", "sample": f"sequences {seqs} of layer 0", "seconds": round(el, 3),
            "TBps": toks * 4096 / el / 1e12, "cores": len(os.sched_getaffinity(0)),
            "parity": {"max_abs_err": err, "bound": bound, "ok": bool(np.all(np.isfinite(got[rows])) and err <= bound)}}


def gather_attention(torch, layer, tables, lens, bs, scale, hq=32, hkv=8, d=128):
    """The gather path the paged kernel replaces: every sequence's pages
    gathered into a padded contiguous K/V copy ([B, L] keys, L = the table's
    width in keys), then dense attention by batched products (bf16 operands,
    each one contiguous; scores and softmax in fp32, keys past a sequence's
    length masked).  Returns (out [B, hq, d], seconds of the gather, of the
    products) from HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    B, mb = tables.shape
    L = mb * bs
    g = hq // hkv
    e0.record(stream)
    idx = tables.clamp(min=0).long()
    kt = layer["kc"][idx].reshape(B, L, hkv, d).permute(0, 2, 3, 1).contiguous().reshape(B * hkv, d, L)
    vv = layer["vc"][idx].reshape(B, L, hkv, d).permute(0, 2, 1, 3).contiguous().reshape(B * hkv, L, d)
    e1.record(stream)
    q = layer["q"].reshape(B * hkv, g, d).contiguous()
    s = torch.bmm(q, kt).float() * scale
    live = (torch.arange(L, device=s.device)[None, :] < lens[:, None]).repeat_interleave(hkv, dim=0)
    s = s.masked_fill(~live[:, None, :], float("-inf"))
    p = torch.softmax(s, dim=-1).to(torch.bfloat16).contiguous()
    out = torch.bmm(p, vv).reshape(B, hq, d)
    e2.record(stream)
    torch.cuda.synchronize()
    return out, e0.elapsed_time(e1) * 1e-3, e1.elapsed_time(e2) * 1e-3


def study_gather(args, torch, pkv, workloads, byte_model):
    """The paged decode call against the gather path it replaces ("nanoserve"
    reports its Triton paged decode 13.7-18.5x faster than gathering K/V and
    running dense attention): the decode workload, one layer, p50 of the
    timed calls of each, and the two outputs compared."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    st = workloads.structure_only("decode", "page16")
    layer = build_layers(torch, st, {"config": "decode"}, 1, dev)[0]
    tables = torch.from_numpy(st["block_tables"]).to(dev)
    ctx = torch.from_numpy(st["context_lens"]).to(dev)
    plan = pkv.Plan(st["context_lens"], None, num_q_heads=32, num_kv_heads=8, head_dim=128, device=dev,
                    num_queues=args.queues)
    paged_ms, gather_s, attn_s = [], [], []
    for it in range(args.warmup + args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        pkv.paged_attn_decode(layer["out"], layer["q"], layer["kc"], layer["vc"], tables, ctx, scale, plan)
        b.record(stream)
        ref, gs, ats = gather_attention(torch, layer, tables, ctx, st["block_size"], scale)
        if it >= args.warmup:
            paged_ms.append(a.elapsed_time(b))
            gather_s.append(gs)
            attn_s.append(ats)
    torch.cuda.synchronize()
    nbytes = byte_model.attention_bytes(st["context_lens"], st["q_lens"], 32, 8, 128, st["block_size"], 2, 2)
    paged = float(np.median(paged_ms)) * 1e-3
    gath = float(np.median(np.array(gather_s) + np.array(attn_s)))
    print(json.dumps({
        "study": "gather", "workload": "decode: 64 seqs, ctx U[512,4096], 32q/8kv, D=128, page 16, bf16",
        "paged_call_us": round(paged * 1e6, 2),
        "gather_path_us": round(gath * 1e6, 2),
        "gather_us": round(float(np.median(gather_s)) * 1e6, 2),
        "dense_attention_us": round(float(np.median(attn_s)) * 1e6, 2),
        "paged_speedup": round(gath / paged, 2),
        "paged_TBps": round(nbytes / paged / 1e12, 4),
        "max_abs_diff_paged_vs_gather": float((layer["out"].float() - ref.float()).abs().max()),
        "calls": len(paged_ms)}), flush=True)


def study_plan_cost(args, torch, pkv, workloads):
    """Host planner cost per step (reused by all layers) for batch 8..512 with
    context uniform in [512, 4096], one JSON line per batch."""
    dev = torch.device("cuda:0")
    for batch in (8, 16, 32, 64, 128, 256, 512):
        lens = workloads.rng_for(workloads.CONFIG_IDS["skew"], 100 + batch).integers(
            512, 4096, size=batch, endpoint=True).astype(np.int32)
        plan = pkv.Plan(lens, None, num_q_heads=32, num_kv_heads=8, head_dim=128, device=dev,
                        num_queues=args.queues)
        ts = []
        for _ in range(50):
            plan.update(lens, None)
            ts.append(plan.last_plan_s)
        torch.cuda.synchronize()
        med = float(np.median(ts[5:]))
        print(json.dumps({"study": "plan-cost", "batch": batch, "plan_us_per_step": round(med * 1e6, 2),
                          "plan_us_per_layer": round(med * 1e6 / LAYERS, 3), "units": int(plan.desc.num_units),
                          "merges": int(plan.desc.num_merges)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--config", default="decode", choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--queues", type=int, default=0, help="planner decode queues (0: the library default, one per CU)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (scales the HBM byte counters)")
    ap.add_argument("--separate-write", action="store_true",
                    help="decode steps call paged_kv_write and then paged_attn_decode instead of "
                         "paged_attn_decode_write (the new tokens written inside the decode launch)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time the step only as eager launches (by default the step is also captured once as a "
                         "HIP graph of every layer's write + attention, the plan made for a fixed capacity, and "
                         "replayed after each step's re-plan; value and ms_per_step then come from the replays)")
    ap.add_argument("--soft-cap", type=float, default=0.0,
                    help="attention variant: logit soft-cap c (scores through c * tanh(s / c)); 0: off")
    ap.add_argument("--window", type=int, default=0,
                    help="attention variant: sliding window of W keys (a row at p sees p - W < j <= p); 0: off")
    ap.add_argument("--study", choices=["skew", "plan-cost", "pages", "read-peak", "gather"],
                    help="instead of the bench line: the load-balance study over length mixes (skew), the "
                         "planner cost over batch sizes (plan-cost), the page-size sweep with its parity check "
                         "(pages), the streaming-read ceilings of the read probe (read-peak) or the paged decode "
                         "call against a gather + dense attention path in torch (gather), one JSON line per case")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); sharding across GPUs is not built",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return

    import paged_kv_attention_write_amd as pkv
    import workloads
    from workloads import byte_model

    if args.study == "skew":
        study_skew(args, torch, pkv, workloads, byte_model)
        return
    if args.study == "plan-cost":
        study_plan_cost(args, torch, pkv, workloads)
        return
    if args.study == "pages":
        study_pages(args, torch, pkv, workloads, byte_model)
        return
    if args.study == "read-peak":
        study_read_peak(args, torch, workloads)
        return
    if args.study == "gather":
        study_gather(args, torch, pkv, workloads, byte_model)
        return

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    st = workloads.structure_only(cfg["config"], cfg["layout"])
    if cfg.get("q_len"):
        lens = st["context_lens"]
        st = workloads.structure_for_lengths(workloads.CONFIG_IDS[cfg["config"]], lens,
                                             q_lens=np.full(lens.shape[0], cfg["q_len"], np.int32))
    if cfg.get("only_chunk"):
        s_ = int(np.argmax(st["q_lens"]))
        L = int(st["q_lens"][s_])
        cu0 = int(st["cu_seqlens"][s_])
        st = dict(st, context_lens=st["context_lens"][s_:s_ + 1], q_lens=st["q_lens"][s_:s_ + 1],
                  cu_seqlens=np.array([0, L], np.int32), block_tables=st["block_tables"][s_:s_ + 1],
                  slot_mapping=st["slot_mapping"][cu0:cu0 + L])
    B = st["context_lens"].shape[0]
    T = int(st["q_lens"].sum())
    mixed = bool(np.any(st["q_lens"] > 1))
    kv_dtype = cfg.get("kv", "bf16")
    kvb = 1 if kv_dtype == "fp8" else 2
    log(f"building {args.layers} layers of {args.config}")
    layers = build_layers(torch, st, cfg, args.layers, dev)
    scales = [(1.0, 1.0)] * args.layers
    if kv_dtype == "fp8":
        scales = fill_fp8(torch, pkv, layers, st, dev)
    tables = torch.from_numpy(st["block_tables"]).to(dev)
    ctx = torch.from_numpy(st["context_lens"]).to(dev)
    slots = torch.from_numpy(st["slot_mapping"]).to(dev)
    cu = torch.from_numpy(st["cu_seqlens"]).to(dev)
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    q_lens = st["q_lens"] if mixed else None
    variant = dict(soft_cap=args.soft_cap, window=args.window)
    # a decode step over bf16 pages of whole 16-token tiles writes its new
    # tokens inside the decode launch (one call per layer); other steps, and
    # --separate-write, call the write, then the attention
    fused = not args.separate_write and not mixed and kv_dtype == "bf16" and st["block_size"] % 16 == 0
    plan = pkv.Plan(st["context_lens"], q_lens, num_q_heads=32, num_kv_heads=8, head_dim=128, device=dev,
                    num_queues=args.queues, **variant)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    attn_bytes = byte_model.attention_bytes(st["context_lens"], st["q_lens"], 32, 8, 128, st["block_size"], kvb, 2,
                                            window=args.window)
    chunk = st["q_lens"] > 1
    chunk_flops = byte_model.attention_flops(st["context_lens"][chunk], st["q_lens"][chunk], 32, 128,
                                             window=args.window)
    wr_bytes = byte_model.write_bytes(T, 8, 128, 2, kvb)
    step_bytes = args.layers * (attn_bytes + wr_bytes)

    n_events = args.steps * args.layers
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    # recorded by the library between each timed call's attention kernel and
    # its merge kernel (pkv_set_split_event); each is recorded once here so
    # that its HIP event exists
    ev_m = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    for e in ev_m:
        e.record(stream)
    torch.cuda.synchronize()
    # before each separate paged_kv_write call (its time: to ev_a)
    ev_w = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    plan_s = []
    wait_s = []

    # the split event costs its call about 3 us (a record between the two
    # kernels), so with two or more timed steps it is set on the odd ones
    # only: those give the attention kernel's time, the even ones the call's
    def split_step(i):
        return args.steps < 2 or i % 2 == 1

    def step(timed_index=None):
        plan.update(st["context_lens"], q_lens)
        plan_s.append(plan.last_plan_s)
        wait_s.append(plan.last_wait_s)
        for l, layer in enumerate(layers):
            ks, vs = scales[l]
            if timed_index is not None and split_step(timed_index):
                pkv.set_split_event(ev_m[timed_index * args.layers + l])
            if fused:
                if timed_index is not None:
                    ev_a[timed_index * args.layers + l].record(stream)
                pkv.paged_attn_decode_write(layer["out"], layer["q"], layer["k_new"], layer["v_new"], slots,
                                            layer["kc"], layer["vc"], tables, ctx, scale, plan, ks, vs)
                if timed_index is not None:
                    ev_b[timed_index * args.layers + l].record(stream)
                    pkv.set_split_event(None)
                continue
            if timed_index is not None:
                ev_w[timed_index * args.layers + l].record(stream)
            pkv.paged_kv_write(layer["k_new"], layer["v_new"], slots, layer["kc"], layer["vc"], ks, vs)
            if timed_index is not None:
                ev_a[timed_index * args.layers + l].record(stream)
            if mixed:
                pkv.paged_attn_mixed(layer["out"], layer["q"], layer["kc"], layer["vc"], tables, cu, ctx, scale, plan,
                                     ks, vs)
            else:
                pkv.paged_attn_decode(layer["out"], layer["q"], layer["kc"], layer["vc"], tables, ctx, scale, plan,
                                      ks, vs)
            if timed_index is not None:
                ev_b[timed_index * args.layers + l].record(stream)
                pkv.set_split_event(None)

    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    plan_s.clear()
    wait_s.clear()
    log("timed")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pkv.set_split_event(None)
    split = np.array([split_step(i) for i in range(args.steps) for _ in range(args.layers)])
    all_call_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)])
    # call times from the steps without the split event (all of them when
    # there is a single timed step), kernel times from those with it
    decode_ms = all_call_ms[~split] if np.any(~split) else all_call_ms
    kernel_ms = np.array([a.elapsed_time(m) for a, m, sp in zip(ev_a, ev_m, split) if sp])
    # the separate write call (HIP events around it), or a note that the
    # decode launch writes the tokens
    if fused:
        write_us = {"note": "written inside the decode launch (paged_attn_decode_write)"}
    else:
        wms = np.array([w.elapsed_time(a) for w, a in zip(ev_w, ev_a)])
        write_us = {"p50": round(float(np.median(wms)) * 1e3, 3), "mean": round(float(wms.mean()) * 1e3, 3),
                    "bytes": int(wr_bytes)}
    eager_ms_step = wall * 1e3 / args.steps
    graph_info = None
    if args.graph:
        # the same step captured once (writes and attention calls of every
        # layer) with a plan of fixed capacity; each timed step re-plans into
        # that plan's workspace, then replays it
        plan = pkv.Plan(st["context_lens"], q_lens, num_q_heads=32, num_kv_heads=8, head_dim=128, device=dev,
                        num_queues=args.queues, capacity=(B, T), **variant)

        def layers_only():
            for l, layer in enumerate(layers):
                ks, vs = scales[l]
                if fused:
                    pkv.paged_attn_decode_write(layer["out"], layer["q"], layer["k_new"], layer["v_new"], slots,
                                                layer["kc"], layer["vc"], tables, ctx, scale, plan, ks, vs)
                    continue
                pkv.paged_kv_write(layer["k_new"], layer["v_new"], slots, layer["kc"], layer["vc"], ks, vs)
                if mixed:
                    pkv.paged_attn_mixed(layer["out"], layer["q"], layer["kc"], layer["vc"], tables, cu, ctx, scale,
                                         plan, ks, vs)
                else:
                    pkv.paged_attn_decode(layer["out"], layer["q"], layer["kc"], layer["vc"], tables, ctx, scale,
                                          plan, ks, vs)

        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            layers_only()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layers_only()
        torch.cuda.synchronize()
        log("graph timed")
        for _ in range(args.warmup):
            plan.update(st["context_lens"], q_lens)
            graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(args.steps):
            plan.update(st["context_lens"], q_lens)
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - g0
        graph_info = {"ms_per_step_graph": round(wall * 1e3 / args.steps, 4),
                      "ms_per_step_eager": round(eager_ms_step, 4),
                      "captured_per_step": (f"{args.layers} x paged_attn_decode_write" if fused else
                                            f"{args.layers} x (paged_kv_write + attention call)")}
    # the step's time: the faster of its two complete forms (eager launches,
    # or the captured graph replayed after each re-plan); which one is named
    # in graph.value_from
    if graph_info is not None:
        graph_info["value_from"] = "graph" if wall * 1e3 / args.steps <= eager_ms_step else "eager"
        wall = min(wall, eager_ms_step * args.steps / 1e3)
    ms_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e12
    # mean over the timed calls, leaving out calls above 3x the median (a
    # host-side gap between the events and the launch, milliseconds long,
    # once in hundreds of calls; the kernels' rocprofv3 averages never
    # contain it)
    def kept_mean_s(ms):
        kept_ = ms[ms <= 3.0 * float(np.median(ms))]
        return float(kept_.mean()) / 1e3, int(ms.size - kept_.size)

    kept = decode_ms[decode_ms <= 3.0 * float(np.median(decode_ms))]
    call_s, _ = kept_mean_s(decode_ms)
    # the roofline's kernel: the call's attention kernel, from the event
    # before the call to the event the library records between that kernel
    # and the merge kernel
    kern_s, kern_left_out = kept_mean_s(kernel_ms)
    # the algorithmic bytes of the call (all read or written by its
    # attention kernel): the attention's, and the new tokens' when the call
    # writes them
    call_bytes = attn_bytes + (wr_bytes if fused else 0)
    hbm_frac = call_bytes / kern_s / (PEAK_HBM_TBS * 1e12)
    mfma_tflops = chunk_flops / kern_s / 1e12
    mfma_frac = mfma_tflops / PEAK_BF16_TFLOPS
    few_rows = mixed and int(st["q_lens"].max()) * 4 <= 16  # 32 q / 8 kv heads: G = 4
    decode_rows_in_step = bool(np.any(st["q_lens"] == 1))
    mixed_kern = ("fewrow_kernel" if few_rows else "mixed_kernel" if decode_rows_in_step else "prefill kernel")
    kern_name = (f"{mixed_kern} (the attention kernel of paged_attn_mixed)" if mixed else
                 "decode_kernel writing the step's tokens (the attention kernel of paged_attn_decode_write)"
                 if fused else "fewrow_kernel (the attention kernel of paged_attn_decode on an fp8 cache)"
                 if kv_dtype == "fp8" else "decode_kernel (the attention kernel of paged_attn_decode)")
    call_name = (f"paged_attn_mixed ({mixed_kern} + merge kernel)" if mixed else
                 "paged_attn_decode (few-row kernel + merge kernel)" if kv_dtype == "fp8" and not fused else
                 "paged_attn_decode_write (decode kernel writing the step's tokens + merge kernel)"
                 if fused else "paged_attn_decode (decode kernel + merge kernel)")
    mfma_bound = mixed and mfma_frac > hbm_frac
    if mfma_bound:
        roofline = {"bound": "mfma", "kernel": kern_name, "achieved": round(mfma_tflops, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(mfma_frac, 4),
                    "flops_per_launch": int(chunk_flops), "traffic": None}
    else:
        roofline = {"bound": "hbm", "kernel": kern_name, "achieved": round(call_bytes / kern_s / 1e9, 2),
                    "peak": PEAK_HBM_TBS * 1e3, "unit": "GB/s", "frac": round(hbm_frac, 4),
                    "bytes_per_launch": int(call_bytes), "traffic": None}
    roofline["kernel_us"] = round(kern_s * 1e6, 3)
    roofline["kernel_left_out_above_3x_median"] = kern_left_out
    # the whole call (its merge kernel and the gap before it included)
    call_rate = chunk_flops / call_s / 1e12 if mfma_bound else call_bytes / call_s / 1e9
    call_peak = PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_TBS * 1e3
    roofline["call"] = {"what": call_name, "us": round(call_s * 1e6, 3), "achieved": round(call_rate, 2),
                        "frac": round(call_rate / call_peak, 4)}
    if mixed:
        roofline["other"] = {"hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4),
                             "chunk_tflops": round(mfma_tflops, 2)}
    # the device's measured streaming-read rate for as many bytes as one call
    # reads, beside the published peak (an HBM-bound call only: the probe
    # measures bytes, not matrix-core flops)
    if roofline["bound"] == "hbm":
        peak_gbs = probe_read_GBps(torch, call_bytes)
        roofline["measured_peak"] = {"value": round(peak_gbs, 1), "unit": "GB/s",
                                     "what": "streaming-read probe (libpkv_probe.so): contiguous, 16 B per lane, "
                                             "non-temporal, one 8-wave workgroup per CU, as many bytes as one call"}
        roofline["frac_of_measured_peak"] = round(call_bytes / kern_s / 1e9 / peak_gbs, 4)
        roofline["call"]["frac_of_measured_peak"] = round(call_bytes / call_s / 1e9 / peak_gbs, 4)

    variant_desc = "".join([f", soft-cap {args.soft_cap:g}" if args.soft_cap else "",
                            f", window {args.window}" if args.window else ""])
    result = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": kv_dtype,
        "data": "synthetic: seeded N(0,1) K/V/Q, seeded lengths and shuffled block tables",
        "config": {
            "workload": f"{args.config}: {cfg['desc']}{variant_desc}; one step = plan + {args.layers} layers x "
                        f"(write + attention{', in one call' if fused else ''})",
            "num_seqs": int(B),
            "query_rows": int(T),
            "total_context_tokens": int(st["context_lens"].sum()),
            "layers": args.layers,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_TBS, 2),
        "us_per_layer": round(ms_step * 1e3 / args.layers, 3),
        "attention_call_us": {"mean": round(float(decode_ms.mean()) * 1e3, 3),
                              "p10": round(float(np.percentile(decode_ms, 10)) * 1e3, 3),
                              "p50": round(float(np.median(decode_ms)) * 1e3, 3),
                              "p90": round(float(np.percentile(decode_ms, 90)) * 1e3, 3),
                              "p99": round(float(np.percentile(decode_ms, 99)) * 1e3, 3),
                              "max": round(float(decode_ms.max()) * 1e3, 3),
                              "roofline_mean": round(call_s * 1e6, 3),
                              "left_out_above_3x_median": int(decode_ms.size - kept.size)},
        "write_call_us": write_us,
        "plan_us_per_step": round(float(np.median(plan_s)) * 1e6, 2),
        "plan_us_per_layer": round(float(np.median(plan_s)) * 1e6 / args.layers, 3),
        "plan_staging_wait_us_per_step": round(float(np.median(wait_s)) * 1e6, 2),
        "roofline": roofline,
        "plan": {"queues": int(plan.desc.num_queues), "units": int(plan.desc.num_units),
                 "merges": int(plan.desc.num_merges), "target_tiles": int(plan.desc.target_tiles)},
    }
    if graph_info is not None:
        result["graph"] = graph_info
    rec = recorded_traffic(args.config + ("+write" if fused else "")) if not variant_desc else None
    if rec is not None:
        result["roofline"]["traffic"] = int(rec["kernel_read_bytes"] + rec["kernel_written_bytes"])
        result["roofline"]["call"]["traffic"] = int(rec["read_bytes"] + rec["written_bytes"])
        result["roofline"]["traffic_source"] = rec["profile"]
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cb = cpu_baseline(torch, st, layers[0], kv_dtype, scales[0], args.cpu_budget, **variant)
        # parity of layer 0's last timed output against the oracle run above
        got = layers[0]["out"].float().cpu().numpy().astype(np.float64)
        cb_out = cb.pop("out")
        result["parity_max_abs_layer0"] = float(np.max(np.abs(got - cb_out)))
        # the oracle's time per layer-call (write + attention) over the GPU's
        # (the attention call, and the separate write when there is one)
        gpu_layer_s = call_s + (0.0 if fused else float(write_us["mean"]) * 1e-6)
        cb["oracle_s_over_gpu_s_per_layer_call"] = round(float(cb["seconds_per_layer_call"]) / gpu_layer_s, 1)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

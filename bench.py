"""Benchmark of the batched paged-attention decode step on one MI355X.

One step is the whole hot path over one synthetic batch: for every layer,
the new token of each sequence is appended to that layer's block pool (the
slot-mapped cache write, at position context_len - 1) and the layer is then
decoded over its block tables; both happen in one launch per layer
(photon_paged_attn_decode_step), with split contexts merged inside it.  The
same step with a separate cache-write launch per layer is timed too, for
comparison.  Inputs are generated once, copied to HBM, and stay resident;
every layer owns its own K/V pool, so a 16-layer step touches about 1.1 GB
and the 256 MiB Infinity Cache cannot serve repeated reads.

Printed: one JSON line.  ``value`` is whole-step throughput in algorithmic
GB/s (bytes the method must move: valid K/V rows, q, out, table entries and
lengths, and the new K/V rows read and written) per measured step time
(HIP-graph replay of the step).  ``roofline`` describes the decode kernel:
its average launch time is the event-timed run of one step's launches
(events recorded on the launch stream) divided by the number of launches.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload.  The fused rotary + cache-write kernel, the multi-query kernel and
the host scheduler are timed after the step and reported in their own
objects.

``ceiling`` holds two bandwidth probes timed like the step's launches (HIP
graph replay over the same pools): a bare gather of every valid K/V row of
the call through the same block tables, with no arithmetic, and a plain
streaming read of as many bytes; ``roofline.frac_of_ceiling`` is the
gather's time over the decode's.  ``workloads`` gives one line per other
configuration (batch 1, the ragged fp16 batch of 64, the Qwen3-shaped long
context, bf16 at batch 16): time per fused call, algorithmic GB/s, fraction
of 8 TB/s and of the gather ceiling of its own tables.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload llama1b_b16]
    python bench.py --summarize trace|pmc DIR --summary-command CMD   (no GPU: rocprofv3
                                                                      output -> markdown)
"""
from __future__ import annotations

import argparse
import ctypes
import functools
import hashlib
import json
import os
import re
import statistics
import sys
import time
import warnings

import numpy as np

import decode_inputs as di

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["paged_attention_decode_photon_amd/csrc/paged_decode.hip",
                  "paged_attention_decode_photon_amd/csrc/lane_ops.h",
                  "paged_attention_decode_photon_amd/csrc/launch.h",
                  "paged_attention_decode_photon_amd/csrc/elem.h",
                  "paged_attention_decode_photon_amd/csrc/arrival.h"]
# workloads reported one line each next to the headline
SECONDARY_WORKLOADS = ["llama1b_b1", "cb_b64", "qwen3_long", "llama1b_b16_bf16"]
TYPE_NAMES = {"f32": "float", "f16": "_Float16", "bf16": "__bf16"}


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


PMC_SUMMARY = os.path.join(ROOT, "profiles", "paged_decode_all_workloads_pmc.md")


def measured_traffic(workload: str, path: str = PMC_SUMMARY):
    """HBM bytes per decode launch of ``workload`` from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(re.escape(workload) + r" hbm_bytes_per_launch:\s*([0-9.]+)", text)
    if not sha or not val or sha.group(1) != kernel_source_sha256():
        return None
    return float(val.group(1))


def decode_bytes(cfg: di.DecodeConfig, ctx: np.ndarray) -> int:
    """Algorithmic bytes of one decode call: valid K/V rows, q, out, table entries, lengths."""
    ctx = np.asarray(ctx, dtype=np.int64)
    eb = cfg.elem_bytes
    kv = int(ctx.sum()) * cfg.num_kv_heads * cfg.head_dim * eb * 2
    qo = 2 * len(ctx) * cfg.num_q_heads * cfg.head_dim * eb
    tables = int(di.blocks_needed(ctx, cfg.block_size).sum()) * 4
    return kv + qo + tables + 4 * len(ctx)


def write_bytes(cfg: di.DecodeConfig, num_tokens: int, num_written: int) -> int:
    """Algorithmic bytes of one cache-write call: read k/v rows and slots, write the rows."""
    row = cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
    return 2 * num_tokens * row + 2 * num_written * row + 4 * num_tokens


def rope_write_bytes(cfg: di.DecodeConfig, num_tokens: int, num_written: int) -> int:
    """Algorithmic bytes of one fused rotary + cache-write call.

    Reads q, k, v, positions and slots; writes rotated q and, for written
    tokens, the rotated k and raw v rows.
    """
    qrow = cfg.num_q_heads * cfg.head_dim * cfg.elem_bytes
    kvrow = cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
    return num_tokens * (2 * qrow + 2 * kvrow + 8) + 2 * num_written * kvrow


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama1b_b16", choices=sorted(di.CONFIGS))
    ap.add_argument("--partition-tokens", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the oracle baseline (0 disables it)")
    ap.add_argument("--rope-prefill-tokens", type=int, default=4096,
                    help="tokens of the large fused rotary + cache-write call timed after the "
                         "step (0 skips the rotary measurements)")
    ap.add_argument("--no-multi-query", action="store_true",
                    help="skip the multi-query (speculative verify / chunked prefill) timings")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the continuous-batching serving run")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (default: the step is also captured in a "
                         "HIP graph and replayed, and value uses the replays)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB once (a plain "
                         "device copy of known size, used to scale HBM byte counters)")
    ap.add_argument("--copy-bw-mib", type=int, default=1024,
                    help="size of the device-to-device copy timed for context (0 disables)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the bandwidth ceiling (streaming read and bare gather probes)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-workload lines of the other configurations")
    ap.add_argument("--workloads", default=",".join(SECONDARY_WORKLOADS),
                    help="comma-separated workloads measured besides the headline one")
    ap.add_argument("--summarize", nargs=2, metavar=("KIND", "DIR"), default=None,
                    help="no GPU work: summarise the rocprofv3 output under DIR (KIND 'trace' for "
                         "a --kernel-trace --stats run, 'pmc' for counter runs, DIR may hold "
                         "several) into markdown on stdout")
    ap.add_argument("--summary-command", default="",
                    help="the command that produced the rocprofv3 output (quoted in the summary)")
    ap.add_argument("--summary-workload", default=None, choices=sorted(di.CONFIGS),
                    help="with --summarize trace: the run measured only this workload, so its "
                         "probe launches are this workload's ceiling")
    ap.add_argument("--min-step-gib", type=float, default=1.0,
                    help="the workload's layers are replicated (fresh pools) until one step "
                         "reads at least this much distinct K/V, so no layer is served from "
                         "the 256 MiB Infinity Cache")
    return ap.parse_args(argv)


def cpu_baseline(cfg, lay, host_layers, budget_s: float):
    """Time the fp64 oracle on whole layers of the workload until the budget is used:
    with every host thread (the reported value), then single-threaded on a
    fifth of the budget."""
    import oracle
    threads = oracle.max_threads()
    per_layer = decode_bytes(cfg, lay.context_lens)

    def timed(num_threads, budget):
        done, t_total = 0, 0.0
        while t_total < budget:
            t = host_layers[done % len(host_layers)]
            t0 = time.perf_counter()
            oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables,
                                     lay.context_lens, cfg.scale, num_threads=num_threads)
            t_total += time.perf_counter() - t0
            done += 1
        return done, t_total

    done, t_total = timed(threads, budget_s)
    done1, t1 = timed(1, budget_s / 5)
    return {
        "value": round(per_layer * done / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} decode calls (whole layers, all {len(lay.context_lens)} sequences) of "
                  f"the {cfg.name} workload, {t_total:.1f} s wall; cache write not included",
        "ms_per_layer": round(t_total / done * 1e3, 3),
        "single_thread": {"value": round(per_layer * done1 / t1 / 1e9, 4), "unit": "GB/s",
                          "cores": 1, "ms_per_layer": round(t1 / done1 * 1e3, 3),
                          "sample": f"{done1} decode calls, {t1:.1f} s wall"},
        "host_cpu": _host_cpu(),
    }


def _host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rope_measurements(args, cfg, lay, layers, slots, device, stream):
    """Time the fused rotary + cache-write kernel, outside the step.

    Two sizes: the decode step's T = batch tokens, one call per layer,
    replayed from a HIP graph (this size is launch-bound); and one
    prefill-sized call of ``--rope-prefill-tokens`` tokens at consecutive
    positions into distinct slots of the first layer's pools, repeated.
    """
    import paged_attention_decode_photon_amd as pa
    import torch

    def event():
        return torch.cuda.Event(enable_timing=True)

    positions = di.to_torch(lay.positions).to(device)
    for L in layers:
        L["qr"] = torch.empty_like(L["q"])

    def burst():
        for L in layers:
            pa.rope_kv_cache_write(L["q"], L["k"], L["v"], positions, slots, L["kc"], L["vc"],
                                   cfg.rope_base, q_out=L["qr"])

    # A call this small takes less GPU time than its Python launch, so the
    # layers' calls are captured once in a HIP graph and the replays timed.
    burst()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        burst()
    graph.replay()
    torch.cuda.synchronize()
    a, b = event(), event()
    a.record(stream)
    for _ in range(args.steps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del graph
    decode_us = a.elapsed_time(b) * 1e3 / (args.steps * len(layers))
    t_dec = len(lay.positions)
    n_written = int((lay.slot_mapping >= 0).sum())

    t = args.rope_prefill_tokens
    L = layers[0]
    nslots = L["kc"].shape[0] * L["kc"].shape[2]
    if t > nslots:
        t = nslots
    rng = np.random.default_rng(cfg.seed + 1000)
    q = di.to_torch(di.cast(rng.standard_normal((t, cfg.num_q_heads, cfg.head_dim)),
                            cfg.np_dtype)).to(device)
    k = di.to_torch(di.cast(rng.standard_normal((t, cfg.num_kv_heads, cfg.head_dim)),
                            cfg.np_dtype)).to(device)
    v = torch.empty_like(k).copy_(k)
    pos = torch.arange(t, dtype=torch.int32, device=device)
    sl = di.to_torch(rng.permutation(nslots)[:t].astype(np.int32)).to(device)
    qr = torch.empty_like(q)
    kc, vc = L["kc"].clone(), L["vc"].clone()
    for _ in range(2):
        pa.rope_kv_cache_write(q, k, v, pos, sl, kc, vc, cfg.rope_base, q_out=qr)
    torch.cuda.synchronize()
    reps = max(args.steps, 5)
    a.record(stream)
    for _ in range(reps):
        pa.rope_kv_cache_write(q, k, v, pos, sl, kc, vc, cfg.rope_base, q_out=qr)
    b.record(stream)
    torch.cuda.synchronize()
    prefill_us = a.elapsed_time(b) * 1e3 / reps
    nbytes = rope_write_bytes(cfg, t, t)
    return {
        "kernel": "rope_kv_cache_write_kernel (rotate-half pairs)",
        "rope_base": cfg.rope_base,
        "decode_tokens": t_dec,
        "decode_us_per_call": round(decode_us, 3),
        "decode_bytes_per_call": rope_write_bytes(cfg, t_dec, n_written),
        "prefill_tokens": t,
        "prefill_us_per_call": round(prefill_us, 3),
        "prefill_bytes_per_call": nbytes,
        "prefill_gbps": round(nbytes / (prefill_us * 1e-6) / 1e9, 1),
    }


MFMA_PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0, "bf16": 2500.0}  # dense, MI355X


def multi_query_measurements(args, cfg, lay, layers, device, stream):
    """Time the multi-query (causal tail) kernel at two shapes.

    Speculative verification: every sequence of the workload verifies 4
    tokens against its whole context, one call per layer pool (HBM-bound;
    algorithmic bytes as for decode, with 4 query rows per sequence).
    Chunked prefill: 4 sequences computing 512-token chunks (bf16, contexts
    2048, 512, 1500 and 4000 tokens; matrix-core-bound; algorithmic flops
    4 * D * Hq * (p + 1) per query row at position p).
    """
    import paged_attention_decode_photon_amd as pa
    import torch

    def event():
        return torch.cuda.Event(enable_timing=True)

    rng = np.random.default_rng(cfg.seed + 2000)
    n = 4
    b = len(lay.context_lens)
    qs = torch.arange(0, b * n + 1, n, dtype=torch.int32, device=device)
    tables = di.to_torch(lay.block_tables).to(device)
    lens = di.to_torch(lay.context_lens).to(device)
    qv = [di.to_torch(di.cast(rng.standard_normal((b * n, cfg.num_q_heads, cfg.head_dim)),
                              cfg.np_dtype)).to(device) for _ in range(2)]
    outs = [torch.empty_like(qv[0]) for _ in range(2)]
    max_ctx = lay.max_context_len
    mqd = pa.multi_query_desc(qv[0], layers[0]["kc"], tables, b, n, max_ctx)
    mq_ws = pa.new_workspace(pa.multi_query_workspace_bytes(mqd), device)

    def verify_burst():
        for i, L in enumerate(layers):
            pa.paged_attn_multi_query(qv[i % 2], L["kc"], L["vc"], tables, lens, qs, cfg.scale,
                                      max_query_len=n, max_context_len=max_ctx, out=outs[i % 2],
                                      workspace=mq_ws)

    verify_burst()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        verify_burst()
    graph.replay()
    torch.cuda.synchronize()
    a, z = event(), event()
    a.record(stream)
    for _ in range(args.steps):
        graph.replay()
    z.record(stream)
    torch.cuda.synchronize()
    del graph
    verify_us = a.elapsed_time(z) * 1e3 / (args.steps * len(layers))
    eb = cfg.elem_bytes
    verify_bytes = (int(lay.context_lens.sum()) * cfg.num_kv_heads * cfg.head_dim * eb * 2
                    + 2 * b * n * cfg.num_q_heads * cfg.head_dim * eb
                    + int(di.blocks_needed(lay.context_lens).sum()) * 4 + 4 * b + 4 * (b + 1))

    # chunked prefill, bf16, its own pool
    qlens, ctx = [512, 512, 300, 512], [2048, 512, 1500, 4000]
    hq, hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    need = [-(-c // 16) for c in ctx]
    nb = sum(need)
    perm = rng.permutation(nb).astype(np.int32)
    tab = np.full((4, max(need)), -1, np.int32)
    p0 = 0
    for i, k in enumerate(need):
        tab[i, :k] = perm[p0:p0 + k]
        p0 += k
    qstart = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    bf = di.BF16
    kc = di.to_torch(di.cast(rng.standard_normal((nb, hkv, 16, d)), bf)).to(device)
    vc = di.to_torch(di.cast(rng.standard_normal((nb, hkv, 16, d)), bf)).to(device)
    q = di.to_torch(di.cast(rng.standard_normal((int(qstart[-1]), hq, d)), bf)).to(device)
    out = torch.empty_like(q)
    tab_t, ctx_t = di.to_torch(tab).to(device), torch.tensor(ctx, dtype=torch.int32, device=device)
    qs_t = di.to_torch(qstart).to(device)
    pf_kw = dict(max_query_len=512, max_context_len=max(ctx), out=out)
    pfd = pa.multi_query_desc(q, kc, tab_t, 4, 512, max(ctx))
    pf_kw["workspace"] = pa.new_workspace(pa.multi_query_workspace_bytes(pfd), device)
    for _ in range(2):
        pa.paged_attn_multi_query(q, kc, vc, tab_t, ctx_t, qs_t, cfg.scale, **pf_kw)
    torch.cuda.synchronize()
    reps = max(args.steps, 5)
    a.record(stream)
    for _ in range(reps):
        pa.paged_attn_multi_query(q, kc, vc, tab_t, ctx_t, qs_t, cfg.scale, **pf_kw)
    z.record(stream)
    torch.cuda.synchronize()
    prefill_us = a.elapsed_time(z) * 1e3 / reps
    flops = sum(4 * d * hq * (c - nq + j + 1) for c, nq in zip(ctx, qlens) for j in range(nq))
    tflops = flops / (prefill_us * 1e-6) / 1e12
    return {
        "kernel": "paged_mq_kernel (16x16 MFMA, causal tail)",
        "verify": {"dtype": cfg.dtype, "query_tokens_per_seq": n, "seqs": b,
                   "us_per_call": round(verify_us, 3), "bytes_per_call": verify_bytes,
                   "gbps": round(verify_bytes / (verify_us * 1e-6) / 1e9, 1),
                   "frac_of_hbm_peak": round(verify_bytes / (verify_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
        "chunked_prefill": {"dtype": "bf16", "query_lens": qlens, "context_lens": ctx,
                            "us_per_call": round(prefill_us, 3), "flops_per_call": flops,
                            "tflops": round(tflops, 2),
                            "frac_of_mfma_peak": round(tflops / MFMA_PEAK_TFLOPS["bf16"], 4)},
    }


def serving_measurements(cfg, device, stream, trace_name: str = "serving"):
    """A continuous-batching run of the attention path, one layer.

    The native scheduler turns a seeded request trace into steps; each step
    uploads its positions, slots, tables, context lengths and query starts
    (pinned host buffers, asynchronous copies), then runs the fused rotary +
    cache write over the step's new tokens and the multi-query kernel over
    all of them (prefill chunks and decode tokens in one launch), or the
    decode kernel when every sequence has one new token.  q/k/v of
    the new tokens are synthetic (no model).  Reported: attention-path GPU
    time per step (events around the two launches) and new tokens per
    second, over all steps and over the decode-only steps.  Each step's
    launches are enqueued behind a short GPU sleep, so the events time the
    kernels back to back rather than the host's launch overhead between them.
    """
    import paged_attention_decode_photon_amd as pa
    import torch
    from paged_attention_decode_photon_amd.sched import Scheduler

    tc = di.TRACES[trace_name]
    trace = di.make_request_trace(tc)
    hq, hkv, d, bs = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, tc.block_size
    rng = np.random.default_rng(cfg.seed + 3000)
    dt = cfg.np_dtype
    kc = di.to_torch(di.cast(rng.standard_normal((tc.num_blocks, hkv, bs, d)), dt)).to(device)
    vc = torch.empty_like(kc).copy_(kc)
    mt = tc.max_tokens_per_step
    q = di.to_torch(di.cast(rng.standard_normal((mt, hq, d)), dt)).to(device)
    k = di.to_torch(di.cast(rng.standard_normal((mt, hkv, d)), dt)).to(device)
    v = torch.empty_like(k).copy_(k)
    qr, out = torch.empty_like(q), torch.empty_like(q)
    ms, mb = tc.max_seqs, tc.max_blocks_per_seq
    host = {"pos": torch.zeros(mt, dtype=torch.int32).pin_memory(),
            "slot": torch.zeros(mt, dtype=torch.int32).pin_memory(),
            "tables": torch.zeros(ms * mb, dtype=torch.int32).pin_memory(),
            "ctx": torch.zeros(ms, dtype=torch.int32).pin_memory(),
            "qs": torch.zeros(ms + 1, dtype=torch.int32).pin_memory()}
    devb = {n: torch.empty_like(t, device=device) for n, t in host.items()}
    ws = pa.new_workspace(1 << 20, device)
    # decode workspace for the largest decode-only step this trace allows
    dd = pa.decode_desc(q[:ms], kc, torch.empty((ms, mb), dtype=torch.int32), mb * bs)
    dec_ws = pa.new_workspace(pa.workspace_bytes(dd), device)
    sched = Scheduler(**tc.sched_config())

    def event():
        return torch.cuda.Event(enable_timing=True)

    # cycles of torch.cuda._sleep per microsecond, to hold the GPU about
    # 200 us while a step's launches are enqueued
    torch.cuda.synchronize()
    c0, c1 = event(), event()
    c0.record(stream)
    torch.cuda._sleep(1_000_000)
    c1.record(stream)
    torch.cuda.synchronize()
    hold_cycles = int(1_000_000 * 200.0 / max(c0.elapsed_time(c1) * 1e3, 1.0))

    records = []
    i, done, step = 0, 0, 0
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    while done < len(trace):
        while i < len(trace) and trace[i][0] <= step:
            sched.add_request(*trace[i][1:])
            i += 1
        o = sched.schedule()
        t, b = len(o["slot_mapping"]), len(o["request_ids"])
        if t:
            host["pos"][:t].numpy()[:] = o["positions"]
            host["slot"][:t].numpy()[:] = o["slot_mapping"]
            host["tables"][:b * mb].numpy()[:] = o["block_tables"].ravel()
            host["ctx"][:b].numpy()[:] = o["context_lens"]
            host["qs"][:b + 1].numpy()[:] = o["query_start"]
            for n in host:
                devb[n].copy_(host[n], non_blocking=True)
            maxq = int(np.diff(o["query_start"]).max())
            maxc = int(o["context_lens"].max())
            tables = devb["tables"][:b * mb].view(b, mb)
            desc = pa.multi_query_desc(q[:t], kc, tables, b, maxq, maxc)
            need = pa.multi_query_workspace_bytes(desc)
            if need > ws.numel():
                ws = pa.new_workspace(need, device)
            e0, e1 = event(), event()
            torch.cuda._sleep(hold_cycles)
            e0.record(stream)
            pa.rope_kv_cache_write(q[:t], k[:t], v[:t], devb["pos"][:t], devb["slot"][:t], kc, vc,
                                   cfg.rope_base, q_out=qr[:t])
            if maxq == 1:  # decode-only step: the balanced decode kernel
                pa.paged_attn_decode(qr[:t], kc, vc, tables, devb["ctx"][:b], cfg.scale,
                                     max_context_len=maxc, out=out[:t], workspace=dec_ws)
            else:
                pa.paged_attn_multi_query(qr[:t], kc, vc, tables, devb["ctx"][:b],
                                          devb["qs"][:b + 1], cfg.scale, max_query_len=maxq,
                                          max_context_len=maxc, out=out[:t], workspace=ws)
            e1.record(stream)
            records.append((e0, e1, t, b, maxq))
            # the host buffers are rewritten next step: wait for this step's copies
            e1.synchronize()
        done += len(sched.update())
        step += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_us = [a.elapsed_time(z) * 1e3 for a, z, _, _, _ in records]
    toks = sum(r[2] for r in records)
    dec = [(us, r[2]) for us, r in zip(gpu_us, records) if r[4] == 1]
    return {
        "trace": trace_name, "dtype": cfg.dtype, "requests": len(trace), "steps": step,
        "kernels": "rope_kv_cache_write, then paged_decode_kernel (decode-only steps) or "
                   "paged_mq_kernel (steps with prompt chunks), one layer",
        "new_tokens": toks,
        "gpu_us_per_step_mean": round(statistics.fmean(gpu_us), 2),
        "tokens_per_s_gpu": round(toks / (sum(gpu_us) * 1e-6), 1),
        "decode_only_steps": len(dec),
        "decode_only_us_per_step_mean": round(statistics.fmean(u for u, _ in dec), 2) if dec else None,
        "decode_only_tokens_per_s_gpu": round(sum(n for _, n in dec) / (sum(u for u, _ in dec) * 1e-6), 1)
        if dec else None,
        "wall_s": round(wall, 3),
        "note": "wall time includes scheduling, uploads and a wait per step (the host buffers are reused)",
    }


def scheduler_measurements(trace_name: str = "serving"):
    """Host cost of the native block manager + scheduler over a seeded request
    trace (every step: admit arrivals, schedule, update), next to the plain
    Python reference scheduler on the same trace."""
    from paged_attention_decode_photon_amd.sched import Scheduler
    from oracle.scheduler import OracleScheduler

    tc = di.TRACES[trace_name]
    trace = di.make_request_trace(tc)

    def drive(s):
        per_step, i, done, tokens = [], 0, 0, 0
        step = 0
        while done < len(trace):
            t0 = time.perf_counter()
            while i < len(trace) and trace[i][0] <= step:
                s.add_request(*trace[i][1:])
                i += 1
            out = s.schedule()
            done += len(s.update())
            per_step.append(time.perf_counter() - t0)
            tokens += len(out["slot_mapping"])
            step += 1
        return per_step, tokens

    nat, tokens = drive(Scheduler(**tc.sched_config()))
    ref, _ = drive(OracleScheduler(**tc.sched_config()))
    return {
        "trace": trace_name,
        "requests": len(trace),
        "steps": len(nat),
        "tokens_scheduled": tokens,
        "native_us_per_step_mean": round(1e6 * statistics.fmean(nat), 2),
        "native_us_per_step_p99": round(1e6 * float(np.percentile(nat, 99)), 2),
        "reference_us_per_step_mean": round(1e6 * statistics.fmean(ref), 2),
        "note": "host time per step, Python binding included; max_seqs 64, 2048-token budget",
    }


def time_graph(calls, stream, steps: int, warmup: int) -> dict:
    """Per-call GPU time of ``calls`` (launch functions taking the HIP stream
    to launch on).

    The calls are captured once in a HIP graph (launched on the capturing
    stream); each of ``steps`` replays is bracketed by events on ``stream``,
    and the time per call is the replay's time over the number of calls
    (host launch overhead excluded, back-to-back gaps included).
    """
    import torch
    for c in calls:  # any first-use set-up happens outside the capture
        c(stream.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with warnings.catch_warnings(record=True) as caught:
        warnings.simplefilter("always")
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for c in calls:
                c(cap)
    if any("empty" in str(w.message) for w in caught):
        raise RuntimeError("nothing was captured: the launches did not go to the capturing stream")
    for _ in range(max(warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    del graph
    per = [a.elapsed_time(b) * 1e3 / len(calls) for a, b in ev]
    p10, p90 = (float(x) for x in np.percentile(per, [10, 90]))
    return {"us_mean": round(statistics.fmean(per), 3), "us_median": round(statistics.median(per), 3),
            "us_p10_p90": [round(p10, 3), round(p90, 3)]}


PROBE_WAVES = (1024, 2048, 4096, 8192)
# LDS-staged gather settings: (workgroups of four wavefronts, tiles in flight
# per wavefront); those whose ring does not fit the row size are skipped.
STAGED_PROBES = ((256, 2), (256, 4), (512, 2), (512, 4), (1024, 2))
# queue-driven gather: wavefronts, thousandths split statically, tiles per piece
QUEUE_PROBE = (1024, 900, 4)


def gather_ceiling(pools, tables, lens, max_ctx: int, kv_bytes: int, stream, steps, warmup) -> dict:
    """Bare gather of the decode call's K/V rows through its tables (no
    arithmetic), over every (k_cache, v_cache) pair in ``pools``, one call
    each per replay: from register sets at several wavefront counts and
    from LDS rings at several workgroup counts and depths; the fastest is the
    ceiling.  Also times one queue-driven setting (part of the work handed
    out at run time), which is not a ceiling candidate."""
    import paged_attention_decode_photon_amd as pa
    import torch
    lib = pa.get_lib()
    sink = torch.empty(max(max(PROBE_WAVES), 4 * max(w for w, _ in STAGED_PROBES)),
                       dtype=torch.int32, device=tables.device)
    queue = torch.zeros(1, dtype=torch.int64, device=tables.device)
    desc = pa.DecodeDesc(lens.shape[0], pools[0][0].shape[1], tables.shape[1], max_ctx, 0,
                         pa.kv_desc(pools[0][0]), 0)
    dref = ctypes.byref(desc)
    row_bytes = pools[0][0].shape[3] * pools[0][0].element_size()

    def timed(fn, *args):
        calls = [functools.partial(_checked, fn, kc.data_ptr(), vc.data_ptr(), tables.data_ptr(),
                                   lens.data_ptr(), dref, *args) for kc, vc in pools]
        return time_graph(calls, stream, steps, warmup)["us_median"]

    by_waves = {w: timed(lib.photon_probe_gather, w, sink.data_ptr()) for w in PROBE_WAVES}
    staged = {f"{w}x{r}": timed(lib.photon_probe_gather_staged, w, r, sink.data_ptr())
              for w, r in STAGED_PROBES if r * row_bytes <= 1024}
    qw, qs, qp = QUEUE_PROBE
    queued = timed(lib.photon_probe_gather_queue, qw, qs, qp, queue.data_ptr(), sink.data_ptr())
    cands = {f"register sets, {w} waves": v for w, v in by_waves.items()}
    cands.update({f"LDS ring, {k.replace('x', ' workgroups x ')} tiles": v for k, v in staged.items()})
    best = min(cands, key=cands.get)
    us = cands[best]
    return {"kernel": "gather_kernel / gather_staged_kernel (photon_probe_gather, "
                      "photon_probe_gather_staged)",
            "bytes_per_call": kv_bytes,
            "us_per_call_by_waves": {str(k): v for k, v in by_waves.items()},
            "staged_us_by_workgroups_x_ring": staged,
            "queue_us": {f"{qw} waves, {qs}/1000 static, {qp}-tile pieces": queued},
            "best": best, "us_per_call": us, "gbps": round(kv_bytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(kv_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def stream_ceiling(nbytes: int, device, stream, steps, warmup, total_gib: float = 1.0) -> dict:
    """Plain streaming read of ``nbytes`` per call, each call on a fresh
    window of a buffer of at least ``total_gib`` GiB (so no window is served
    from the 256 MiB Infinity Cache); the fastest wavefront count counts."""
    import paged_attention_decode_photon_amd as pa
    import torch
    lib = pa.get_lib()
    nbytes = (nbytes + 15) // 16 * 16
    win = (nbytes + 4095) // 4096 * 4096
    nwin = max(4, -(-int(total_gib * 2**30) // win))
    buf = torch.zeros(nwin * win, dtype=torch.uint8, device=device)
    sink = torch.empty(max(PROBE_WAVES), dtype=torch.int32, device=device)
    by_waves = {}
    for waves in PROBE_WAVES:
        calls = [functools.partial(_checked, lib.photon_probe_stream_read, buf.data_ptr() + i * win,
                                   nbytes, waves, sink.data_ptr()) for i in range(nwin)]
        by_waves[waves] = time_graph(calls, stream, steps, warmup)["us_median"]
    del buf
    best = min(by_waves, key=by_waves.get)
    us = by_waves[best]
    return {"kernel": "stream_read_kernel (photon_probe_stream_read)", "bytes_per_call": nbytes,
            "us_per_call_by_waves": {str(k): v for k, v in by_waves.items()}, "best_waves": best,
            "us_per_call": us, "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def _checked(fn, *args):
    import paged_attention_decode_photon_amd as pa
    pa.check(fn(*args))


def kv_read_bytes(cfg: di.DecodeConfig, ctx: np.ndarray) -> int:
    """Bytes of the valid K and V rows of one decode call (what the probes read)."""
    return int(np.asarray(ctx, dtype=np.int64).sum()) * cfg.num_kv_heads * cfg.head_dim \
        * cfg.elem_bytes * 2


def workload_line(name: str, device, stream, steps: int, warmup: int, min_gib: float,
                  ceiling: bool = True) -> dict:
    """One workload's fused decode step (append + decode, one launch per
    call), timed per call by HIP-graph replay over copies of its pools that
    add up to ``min_gib`` GiB (fresh data every call), next to the bare
    gather of the same rows through the same tables.  The pools, q and new
    rows are N(0,1) draws made on the GPU (torch, seeded with the
    workload's seed); tables and contexts are the workload's own."""
    import paged_attention_decode_photon_amd as pa
    import torch
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    b, hq, hkv, d = len(lay.context_lens), cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    pool_shape = (lay.num_blocks, hkv, cfg.block_size, d)
    pool_bytes = 2 * lay.num_blocks * hkv * cfg.block_size * d * cfg.elem_bytes
    copies = int(min(512, max(2, -(-int(min_gib * 2**30) // pool_bytes))))

    def draw(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(tdt)

    layers = [{"q": draw((b, hq, d)), "kc": draw(pool_shape), "vc": draw(pool_shape),
               "k": draw((b, hkv, d)), "v": draw((b, hkv, d))} for _ in range(copies)]
    for L in layers:
        L["out"] = torch.empty_like(L["q"])
    tables = di.to_torch(lay.block_tables).to(device)
    lens = di.to_torch(lay.context_lens).to(device)
    max_ctx = lay.max_context_len
    desc = pa.decode_desc(layers[0]["q"], layers[0]["kc"], tables, max_ctx)
    ws_bytes = pa.workspace_bytes(desc)
    ws = pa.new_workspace(ws_bytes, device)
    lib, dref = pa.get_lib(), ctypes.byref(desc)
    calls = [functools.partial(_checked, lib.photon_paged_attn_decode_step, L["q"].data_ptr(),
                               L["k"].data_ptr(), L["v"].data_ptr(), L["kc"].data_ptr(),
                               L["vc"].data_ptr(), tables.data_ptr(), lens.data_ptr(), cfg.scale,
                               dref, L["out"].data_ptr(), ws.data_ptr(), ws_bytes)
             for L in layers]
    t = time_graph(calls, stream, steps, warmup)
    n_written = int((lay.slot_mapping >= 0).sum())
    nbytes = decode_bytes(cfg, lay.context_lens) + 4 * n_written * hkv * d * cfg.elem_bytes
    us = t["us_median"]
    line = {"config": {"batch": b, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                       "kv_dtype": cfg.dtype, "context_sum": int(lay.context_lens.sum()),
                       "context_max": max_ctx, "pool_copies": copies},
            "kernel": f"paged_decode_kernel<{TYPE_NAMES[cfg.dtype]}, {TYPE_NAMES[cfg.dtype]}, {d}, "
                      f"{cfg.group}> (photon_paged_attn_decode_step)",
            "bytes_per_call": nbytes, **t,
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "tokens_per_s": round(b / (us * 1e-6), 1)}
    if ceiling:
        g = gather_ceiling([(L["kc"], L["vc"]) for L in layers], tables, lens, max_ctx,
                           kv_read_bytes(cfg, lay.context_lens), stream, steps, warmup)
        line["gather_ceiling"] = g
        line["frac_of_gather_ceiling"] = round(g["us_per_call"] / us, 4)
    del layers, ws
    torch.cuda.empty_cache()
    return line


# ----------------------------------------------------------- profile summaries

_MANGLED_TYPES = {"f": "float", "DF16_": "_Float16", "DF16b": "__bf16"}


def decode_kernel_sig(name: str):
    """(storage, output, head_dim, group) of a paged_decode_kernel dispatch
    name, mangled or demangled; None for other kernels."""
    m = re.search(r"paged_decode_kernel<\s*(\w+),\s*(\w+),\s*(\d+),\s*(\d+)\s*>", name)
    if m:
        return m.group(1), m.group(2), int(m.group(3)), int(m.group(4))
    m = re.search(r"paged_decode_kernelI(f|DF16_|DF16b)(f|DF16_|DF16b)Li(\d+)ELi(\d+)E", name)
    if m:
        return (_MANGLED_TYPES[m.group(1)], _MANGLED_TYPES[m.group(2)], int(m.group(3)),
                int(m.group(4)))
    return None


def short_kernel_name(name: str) -> str:
    sig = decode_kernel_sig(name)
    if sig:
        return "paged_decode_kernel<%s, %s, %d, %d>" % sig
    # longer names first: "rope_kv_cache_write_kernel" contains "kv_cache_write_kernel"
    for key in ("gather_staged_kernel", "gather_queue_kernel", "gather_kernel",
                "stream_read_kernel", "paged_mq_wide_kernel", "paged_mq_kernel",
                "rope_kv_cache_write_kernel", "kv_cache_write_kernel", "__amd_rocclr_copyBuffer"):
        if key in name:
            m = re.search(key + r"<([^>]*)>", name)
            if m:
                return f"{key}<{m.group(1)}>"
            m = re.search(key + r"I((?:Li\d+E)+)E", name)  # mangled integer template arguments
            if m:
                args = re.findall(r"Li(\d+)E", m.group(1))
                return key + "<" + ", ".join(args) + ">"
            return key
    return name[:60]


def workload_dispatch_keys(names) -> dict:
    """(decode kernel signature, grid threads) of each workload's fused-step
    launch with automatic partitioning, from the library's own plan."""
    import paged_attention_decode_photon_amd as pa
    keys = {}
    for name in names:
        cfg = di.CONFIGS[name]
        lay = di.make_layout(cfg)
        desc = pa.DecodeDesc(len(lay.context_lens), cfg.num_q_heads, lay.max_blocks_per_seq,
                             lay.max_context_len, 0,
                             pa.KvDesc(lay.num_blocks, cfg.num_kv_heads, cfg.block_size,
                                       cfg.head_dim, {"f32": pa.F32, "f16": pa.F16,
                                                      "bf16": pa.BF16}[cfg.dtype]), 0)
        t = TYPE_NAMES[cfg.dtype]
        keys[name] = ((t, t, cfg.head_dim, cfg.group), planned_waves(desc) * 64)
    return keys


def planned_waves(desc) -> int:
    """Wavefronts the library launches for ``desc`` with automatic
    partitioning: one per unit of the largest batch the descriptor allows,
    but no more than 256 compute units x max(4, 64 KiB / bytes in flight per
    wave), in whole workgroups of four (the rule include/photon_decode.h
    states for partition_tokens = 0; a CPU test checks it against the
    workspace size).  A wave keeps two chunks in flight, one with eight
    query heads per KV head."""
    import paged_attention_decode_photon_amd as pa
    quantum = pa.partition_quantum(desc)
    eb = 4 if desc.kv.dtype == pa.F32 else 2
    chunks = -(-desc.max_context_len // quantum)
    upper = desc.num_seqs * desc.kv.num_kv_heads * chunks
    in_flight = 2 if desc.num_q_heads // desc.kv.num_kv_heads < 8 else 1
    per_cu = max(4, (64 * 1024) // (2 * quantum * desc.kv.head_dim * eb * in_flight))
    waves = max(1, min(upper, 256 * per_cu))
    return -(-waves // 4) * 4


def _read_csvs(root: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _col(row: dict, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names)


def probe_rows(groups: dict) -> list:
    """(design, setting, median us, ceiling candidate) of every probe kernel
    in a trace's (kernel, grid threads) -> durations groups."""
    rows = []
    for (name, grid), v in sorted(groups.items()):
        med = statistics.median(v)
        if name.startswith("gather_kernel"):
            rows.append(("gather, register sets", f"{grid // 64} waves", med, True))
        elif name.startswith("gather_staged_kernel"):
            ring = name.split(",")[-1].strip(" >")
            rows.append(("gather, LDS ring", f"{grid // 256} workgroups x {ring} tiles", med, True))
        elif name.startswith("gather_queue_kernel"):
            w, st, pc = QUEUE_PROBE
            rows.append(("gather, queue-driven", f"{grid // 64} waves, {st}/1000 static, "
                         f"{pc}-tile pieces", med, False))
        elif name.startswith("stream_read"):
            rows.append(("stream read", f"{grid // 64} waves", med, False))
    return rows


def summarize_trace(root: str, command: str, workload: str | None = None) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace run: per-kernel
    durations, the decode kernel split by workload (signature and grid) with
    its algorithmic GB/s; for a run of one ``workload``, also its bandwidth
    probes and the decode's fraction of the fastest gather."""
    rows = _read_csvs(root, "kernel_trace.csv")
    if not rows:
        raise SystemExit(f"no *kernel_trace.csv under {root}")
    groups: dict = {}
    for r in rows:
        name = _col(r, "Kernel_Name")
        grid = int(_col(r, "Grid_Size_X", "Grid_Size"))
        dur = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3
        groups.setdefault((short_kernel_name(name), grid), []).append(dur)
    total = sum(sum(v) for v in groups.values())
    title = (f"the {workload} workload: its decode kernel, its bandwidth probes and the other "
             "kernels of the run") if workload else "every kernel of the run"
    out = [f"# Kernel durations (rocprofv3 kernel trace), {title}", "",
           "Command ($REPO is the repository root):", "",
           "```", command, "```", "",
           "| kernel | grid (threads) | calls | average (us) | median (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {name} | {grid} | {len(v)} | {statistics.fmean(v):.2f} | "
                   f"{statistics.median(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                   f"{100 * sum(v) / total:.1f}% |")
    out.append("")
    keys = workload_dispatch_keys(list(di.CONFIGS))
    out += ["Decode kernel by workload (fused append + decode launches; algorithmic bytes as in "
            "`bench.decode_bytes` plus the new rows read and appended):", "",
            "| workload | launches | average (us) | median (us) | bytes per launch | GB/s at the average "
            "| % of 8 TB/s |", "|---|---|---|---|---|---|---|"]
    for wl, (sig, grid) in keys.items():
        v = [d for (n, g), ds in groups.items() for d in ds
             if g == grid and n == "paged_decode_kernel<%s, %s, %d, %d>" % sig]
        if not v:
            continue
        cfg = di.CONFIGS[wl]
        lay = di.make_layout(cfg)
        nbytes = decode_bytes(cfg, lay.context_lens) + 4 * int((lay.slot_mapping >= 0).sum()) \
            * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
        avg = statistics.fmean(v)
        gbps = nbytes / (avg * 1e-6) / 1e9
        out.append(f"| {wl} | {len(v)} | {avg:.2f} | {statistics.median(v):.2f} | {nbytes} | "
                   f"{gbps:.1f} | {100 * gbps / HBM_PEAK_GBPS:.1f}% |")
        out.append(f"<!-- {wl} decode_avg_us: {avg:.3f} -->")
    # several workloads' probes share kernels and grids: probes only for a one-workload run
    probes = probe_rows(groups) if workload is not None else []
    ceiling = [p for p in probes if p[3]]
    if ceiling:
        cfg = di.CONFIGS[workload]
        lay = di.make_layout(cfg)
        kvb = kv_read_bytes(cfg, lay.context_lens)
        sig, grid = keys[workload]
        dec = [d for (n, g), ds in groups.items() for d in ds
               if g == grid and n == "paged_decode_kernel<%s, %s, %d, %d>" % sig]
        best = min(ceiling, key=lambda p: p[2])
        out += ["", f"Bandwidth probes of this run ({workload}: {kvb} bytes of valid K/V rows per "
                "call; the gathers read exactly those rows through the same tables, the stream "
                "read as many contiguous bytes), median us:", "",
                "| probe | setting | median (us) | GB/s |", "|---|---|---|---|"]
        for design, setting, med, _ in probes:
            out.append(f"| {design} | {setting} | {med:.2f} | {kvb / (med * 1e-6) / 1e9:.1f} |")
        if dec:
            avg = statistics.fmean(dec)
            out += ["", f"Fastest gather: {best[0]}, {best[1]}: {best[2]:.2f} us = "
                    f"{kvb / (best[2] * 1e-6) / 1e9:.1f} GB/s "
                    f"({100 * kvb / (best[2] * 1e-6) / 1e9 / HBM_PEAK_GBPS:.1f}% of 8 TB/s). "
                    f"Decode average {avg:.2f} us: {100 * best[2] / avg:.1f}% of the gather's rate.",
                    f"<!-- {workload} gather_best_us: {best[2]:.3f} -->"]
    out += ["", f"kernel_source_sha256: {kernel_source_sha256()}"]
    return "\n".join(out) + "\n"


def summarize_pmc(root: str, command: str) -> str:
    """Markdown summary of rocprofv3 --pmc runs under ``root`` (one
    subdirectory per pass): every counter's mean per dispatch for the decode
    kernel of each workload, and HBM bytes from FETCH_SIZE / WRITE_SIZE
    scaled by what the same counters read for a copy of known size."""
    rows = _read_csvs(root, "counter_collection.csv")
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {root}")
    per: dict = {}
    for r in rows:
        name = short_kernel_name(_col(r, "Kernel_Name"))
        grid = int(_col(r, "Grid_Size", "Grid_Size_X"))
        key = (name, grid, _col(r, "Counter_Name"))
        disp = _col(r, "Dispatch_Id", "Correlation_Id")
        per.setdefault(key, {}).setdefault(disp, 0.0)
        per[key][disp] += float(_col(r, "Counter_Value"))
    mean = {k: statistics.fmean(v.values()) for k, v in per.items()}
    ndisp = {k: len(v) for k, v in per.items()}
    counters = sorted({k[2] for k in per})
    out = ["# Decode kernel counters on every workload (rocprofv3 --pmc)", "",
           "Counter passes, one run each ($REPO is the repository root); the passes were "
           "FETCH_SIZE | WRITE_SIZE | TCC_HIT_sum TCC_MISS_sum | OccupancyPercent "
           "MeanOccupancyPerCU LDSBankConflict | SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
           "SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_VMEM_RD | "
           "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_INSTS_SALU "
           "SQ_INSTS_MFMA SQ_ACTIVE_INST_LDS SQ_INSTS_SMEM:", "", "```", command, "```", ""]
    # copy calibration: the largest copyBuffer dispatch is the known-size copy
    scale = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        cands = [(g, mean[(n, g, c)]) for (n, g, c) in mean if n == "__amd_rocclr_copyBuffer"
                 and c == cname]
        if cands:
            g, kib = max(cands)
            copy_bytes = COPY_CALIBRATION_BYTES
            scale[cname] = copy_bytes / (kib * 1024.0)
            out.append(f"Calibration: a copy of {copy_bytes} bytes reads {cname} = {kib:.1f} KiB "
                       f"per dispatch; scale {scale[cname]:.5f}.")
    out.append("")
    keys = workload_dispatch_keys(list(di.CONFIGS))
    for wl, (sig, grid) in keys.items():
        name = "paged_decode_kernel<%s, %s, %d, %d>" % sig
        have = [c for c in counters if (name, grid, c) in mean]
        if not have:
            continue
        cfg = di.CONFIGS[wl]
        lay = di.make_layout(cfg)
        nbytes = decode_bytes(cfg, lay.context_lens) + 4 * int((lay.slot_mapping >= 0).sum()) \
            * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
        out += [f"### {wl}: {name}, {grid // 64} wavefronts", "",
                "| counter | mean per dispatch | dispatches |", "|---|---|---|"]
        for c in have:
            out.append(f"| {c} | {mean[(name, grid, c)]:.1f} | {ndisp[(name, grid, c)]} |")
        if all((name, grid, c) in mean for c in ("FETCH_SIZE", "WRITE_SIZE")) and len(scale) == 2:
            hbm = mean[(name, grid, "FETCH_SIZE")] * 1024 * scale["FETCH_SIZE"] + \
                mean[(name, grid, "WRITE_SIZE")] * 1024 * scale["WRITE_SIZE"]
            out += ["", f"Algorithmic bytes per launch {nbytes}; HBM bytes per launch (scaled) "
                    f"{hbm:.0f} = {hbm / nbytes:.3f} x algorithmic.",
                    f"<!-- {wl} hbm_bytes_per_launch: {hbm:.0f} -->"]
        if (name, grid, "TCC_HIT_sum") in mean and (name, grid, "TCC_MISS_sum") in mean:
            h, m = mean[(name, grid, "TCC_HIT_sum")], mean[(name, grid, "TCC_MISS_sum")]
            out.append(f"L2 hit rate {100 * h / max(h + m, 1):.1f}%.")
        if (name, grid, "SQ_WAVE_CYCLES") in mean:
            # SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* count per-wave
            # quad-cycles, so their ratios are fractions of wave lifetime
            wc = mean[(name, grid, "SQ_WAVE_CYCLES")]
            for c, what in (("SQ_ACTIVE_INST_VALU", "issuing VALU instructions"),
                            ("SQ_WAIT_INST_ANY", "waiting for a dependency (s_waitcnt)"),
                            ("SQ_WAIT_ANY", "waiting for anything")):
                if (name, grid, c) in mean:
                    out.append(f"{c} / SQ_WAVE_CYCLES = {mean[(name, grid, c)] / wc:.3f} "
                               f"(share of wave time {what}).")
            if (name, grid, "SQ_WAVES") in mean:
                nw = mean[(name, grid, "SQ_WAVES")]
                out.append(f"Mean wave lifetime {4 * wc / nw / 2.4e3:.2f} us at 2.4 GHz "
                           f"({nw:.0f} waves).")
                if (name, grid, "SQ_INSTS_VALU") in mean:
                    out.append(f"VALU instructions per wave {mean[(name, grid, 'SQ_INSTS_VALU')] / nw:.0f}.")
        if (name, grid, "SQ_LDS_BANK_CONFLICT") in mean and (name, grid, "SQ_LDS_IDX_ACTIVE") in mean:
            out.append("LDS bank conflict cycles / LDS active cycles = "
                       f"{mean[(name, grid, 'SQ_LDS_BANK_CONFLICT')] / max(mean[(name, grid, 'SQ_LDS_IDX_ACTIVE')], 1):.3f}.")
        out.append("")
    out += [f"kernel_source_sha256: {kernel_source_sha256()}"]
    return "\n".join(out) + "\n"


COPY_CALIBRATION_BYTES = 256 << 20  # --calibrate-copy-mib 256 in the counter runs


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.summarize:
        kind, root = args.summarize
        if kind not in ("trace", "pmc"):
            print("--summarize KIND must be 'trace' or 'pmc'", file=sys.stderr)
            return 2
        if kind == "trace":
            sys.stdout.write(summarize_trace(root, args.summary_command, args.summary_workload))
        else:
            sys.stdout.write(summarize_pmc(root, args.summary_command))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every (sequence, KV head) pair is independent, see the sharding notes)",
              file=sys.stderr)
        return 2

    import torch
    import paged_attention_decode_photon_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    device = torch.device("cuda:0")
    cfg = di.CONFIGS[args.workload]
    lay = di.make_layout(cfg)
    n_layers = max(cfg.layers, 1)
    host_layers = [di.make_layer(cfg, lay, layer) for layer in range(n_layers)]
    pool_bytes = 2 * host_layers[0].k_cache.nbytes * n_layers
    copies = int(min(512 // n_layers, max(1, -(-int(args.min_step_gib * 2**30) // pool_bytes))))

    def up(a):
        return di.to_torch(a).to(device)

    tables, lens, slots = up(lay.block_tables), up(lay.context_lens), up(lay.slot_mapping)
    layers = []
    for _ in range(copies):
        for t in host_layers:
            layers.append({"q": up(t.q), "kc": up(t.k_cache), "vc": up(t.v_cache),
                           "k": up(t.k_new), "v": up(t.v_new), "out": torch.empty_like(up(t.q))})
    max_ctx = lay.max_context_len
    desc = pa.decode_desc(layers[0]["q"], layers[0]["kc"], tables, max_ctx, args.partition_tokens)
    part = pa.partition_tokens(desc)
    ws_bytes = pa.workspace_bytes(desc)
    workspace = pa.new_workspace(ws_bytes, device)
    stream = torch.cuda.current_stream(device)
    sptr = stream.cuda_stream
    kvd = pa.kv_desc(layers[0]["kc"])
    lib = pa.lib
    import ctypes
    descref, kvref = ctypes.byref(desc), ctypes.byref(kvd)
    T = lay.slot_mapping.shape[0]
    scale = cfg.scale

    def write(L, st=sptr):
        pa.check(lib.photon_kv_cache_write(L["k"].data_ptr(), L["v"].data_ptr(), slots.data_ptr(),
                                           T, L["kc"].data_ptr(), L["vc"].data_ptr(), kvref, st))

    def decode(L, st=sptr):
        pa.check(lib.photon_paged_attn_decode(L["q"].data_ptr(), L["kc"].data_ptr(),
                                              L["vc"].data_ptr(), tables.data_ptr(),
                                              lens.data_ptr(), scale, descref, L["out"].data_ptr(),
                                              workspace.data_ptr(), ws_bytes, st))

    def fused(L, st=sptr):
        pa.check(lib.photon_paged_attn_decode_step(L["q"].data_ptr(), L["k"].data_ptr(),
                                                   L["v"].data_ptr(), L["kc"].data_ptr(),
                                                   L["vc"].data_ptr(), tables.data_ptr(),
                                                   lens.data_ptr(), scale, descref,
                                                   L["out"].data_ptr(), workspace.data_ptr(),
                                                   ws_bytes, st))

    def step(st=sptr):
        # one launch per layer: the new token's K/V append fused with decode
        for L in layers:
            fused(L, st)

    def step_unfused(st=sptr):
        for L in layers:
            write(L, st)
        for L in layers:
            decode(L, st)

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    copy_gbps = None
    if args.copy_bw_mib > 0:
        # achievable read+write rate of a plain device copy, for context
        n = args.copy_bw_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * n * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
        del src, dst

    def event():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region.  A step appends every layer's new tokens and decodes
    # every layer, one fused launch per layer; one event pair brackets each
    # step's run of launches, on the launch stream.
    burst = [(event(), event()) for _ in range(args.steps)]
    start, stop = event(), event()
    start.record(stream)
    for i in range(args.steps):
        burst[i][0].record(stream)
        step()
        burst[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(stop) / args.steps
    burst_us = [a.elapsed_time(b) * 1e3 / len(layers) for a, b in burst]
    call_mean = statistics.fmean(burst_us)
    call_med = statistics.median(burst_us)
    call_p10, call_p90 = (float(x) for x in np.percentile(burst_us, [10, 90]))

    eager_step_ms = step_ms
    graph_step_ms = None
    unfused_step_ms = None

    def replay_ms(fn):
        # fn captured once in a HIP graph and replayed.  The kernels issue no
        # memsets and the workspace counters return to zero on their own, so
        # replays are safe.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn(torch.cuda.current_stream(device).cuda_stream)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            graph.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        del graph
        return start.elapsed_time(stop) / args.steps

    if not args.no_graph:
        graph_step_ms = replay_ms(step)
        step_ms = graph_step_ms
        # for comparison: the same step with the separate cache-write kernel
        unfused_step_ms = replay_ms(step_unfused)

    # Secondary: events around every single decode call (adds the event
    # packets' own overhead to each launch).
    single = [(event(), event()) for _ in layers]
    for (a, b), L in zip(single, layers):
        a.record(stream)
        fused(L)
        b.record(stream)
    torch.cuda.synchronize()
    single_us = statistics.fmean(a.elapsed_time(b) * 1e3 for a, b in single)

    ceiling = None
    if not args.no_ceiling:
        kvb = kv_read_bytes(cfg, lay.context_lens)
        ceiling = {"gather": gather_ceiling([(L["kc"], L["vc"]) for L in layers], tables, lens,
                                            max_ctx, kvb, stream, args.steps, args.warmup),
                   "stream_read": stream_ceiling(kvb, device, stream, args.steps, args.warmup)}
    rope = rope_measurements(args, cfg, lay, layers, slots, device, stream) \
        if args.rope_prefill_tokens > 0 else None
    mq = None if args.no_multi_query else \
        multi_query_measurements(args, cfg, lay, layers, device, stream)

    workloads = None
    if not args.no_workloads:
        del layers[:]  # free the headline pools before the other workloads'
        torch.cuda.empty_cache()
        workloads = {}
        for name in [w for w in args.workloads.split(",") if w and w != cfg.name]:
            workloads[name] = workload_line(name, device, stream, args.steps, args.warmup,
                                            args.min_step_gib, ceiling=not args.no_ceiling)
            print(f"workload {name}: {workloads[name]['us_median']} us per call", file=sys.stderr,
                  flush=True)

    per_decode = decode_bytes(cfg, lay.context_lens)
    n_written = int((lay.slot_mapping >= 0).sum())
    # the fused launch also reads each new K/V row and writes it to the pool
    per_append = 4 * n_written * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
    per_launch = per_decode + per_append
    n_launch = len(host_layers) * copies
    step_bytes = n_launch * per_launch
    value = step_bytes / (step_ms * 1e-3) / 1e9
    achieved = per_launch / (call_mean * 1e-6) / 1e9
    tok_per_layer = len(lay.context_lens) / (step_ms * 1e-3 / n_launch)

    result = {
        "metric": "decode attention KV GB/s (% of HBM peak) + tokens/s per layer at batch 16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled block pool)",
        "config": {
            "workload": cfg.name,
            "batch": len(lay.context_lens),
            "layers_per_step": n_launch,
            "num_q_heads": cfg.num_q_heads,
            "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim,
            "block_size": cfg.block_size,
            "kv_dtype": cfg.dtype,
            "context_sum": int(lay.context_lens.sum()),
            "context_max": max_ctx,
            "partition_tokens": part,
            "parallelism": "single GPU",
        },
        "timing": "hip-graph replay of the step" if graph_step_ms else "eager launches",
        "ms_per_step_eager": round(eager_step_ms, 5),
        "ms_per_step_unfused_write_then_decode": round(unfused_step_ms, 5) if unfused_step_ms else None,
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s_per_layer": round(tok_per_layer, 1),
        "decode_call_us_mean": round(call_mean, 3),
        "decode_call_us_median": round(call_med, 3),
        "decode_call_us_p10_p90": [round(call_p10, 3), round(call_p90, 3)],
        "decode_call_us_single_event_pair": round(single_us, 3),
        "decode_gbps_event_timed": round(achieved, 2),
        "copy_gbps_read_plus_write": round(copy_gbps, 1) if copy_gbps else None,
        # the step's algorithmic rate against that copy's (reads plus writes
        # of a >= 1 GiB device copy, the achievable-bandwidth reference)
        "pct_of_copy_bandwidth": round(100 * value / copy_gbps, 2) if copy_gbps else None,
        "kernel_source_sha256": kernel_source_sha256(),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(cfg.name),
            "kernel": "paged_decode_kernel (one launch per photon_paged_attn_decode_step call: "
                      "new-token append + decode)",
            "bytes_per_launch": per_launch,
        },
    }
    if ceiling is not None:
        # decode against the bare gather of the same rows through the same
        # tables, both timed per call by graph replay over the same pools
        dec_us = step_ms * 1e3 / n_launch
        g = ceiling["gather"]
        ceiling["decode_us_per_call_graph"] = round(dec_us, 3)
        ceiling["decode_frac_of_gather_ceiling"] = round(g["us_per_call"] / dec_us, 4)
        ceiling["note"] = ("gather: every valid K/V row of the call through the block tables, "
                           "no arithmetic; stream_read: the same number of bytes from one "
                           "contiguous buffer; fraction = gather time / decode time per call")
        result["roofline"]["ceiling_gbps"] = g["gbps"]
        result["roofline"]["frac_of_ceiling"] = round(g["us_per_call"] / dec_us, 4)
        result["ceiling"] = ceiling
    if workloads is not None:
        result["workloads"] = workloads
    if rope is not None:
        result["rope_kv_cache_write"] = rope
    if mq is not None:
        result["multi_query"] = mq
    result["scheduler"] = scheduler_measurements()
    if not args.no_serving:
        result["serving"] = serving_measurements(cfg, device, stream)
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, lay, host_layers, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

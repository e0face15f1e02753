#!/usr/bin/env python3
"""Benchmark of one decode step of Parallel Prompting attention on one MI355X.

A step is one call of pp_attn_decode: the visibility plan, the document part
(read once for all P streams, MFMA), the per-stream own-slot gather and the
merge.  Workload (default): CodeLlama-7B attention shape, H=32 heads of
d=128, bf16, a 16384-token document, P=256 streams with questions uniform
8-48 tokens and 31 prior answer tokens each, answers interleaved by step,
seeded N(0,1) inputs resident in HBM before timing starts.

Prints ONE JSON line (the headline number is answer tokens per second of
one layer's attention) with: effective KV bandwidth and its fraction of the
8 TB/s HBM peak, the per-kernel durations measured with HIP events recorded
by the library on the stream its kernels run on, the roofline of the
dominant kernel, the per-question baseline's time on the same inputs, and
the fp64 CPU oracle timed on a bounded sample of streams.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --read-calibration   # 1 GiB streaming read, to scale PMC byte counters
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "answer tok/s & effective doc-KV GB/s (% HBM peak), doc=16k P=256 H=32 d=128"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """Hash of the HIP sources: PMC byte counts in profiles/ are only used
    while the kernels are unchanged since they were taken."""
    csrc = os.path.join(ROOT, "shared_prefix_stream_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def read_pmc_traffic(stage: str, workload: str):
    """HBM bytes per launch from profiles/pmc_<stage>_<workload>.txt
    (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by the read and write
    calibration factor), or None if absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, f"pmc_{stage}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def step_bytes(case):
    """Algorithmic bytes: the document's K/V once, each stream's own slots
    once (read by their owner only), Q, out and the stream ids."""
    es = case.q.element_size()
    row = case.H * case.D * es
    tail = sum(len(o) for o in case.own_slots)
    return {
        "doc_kv": 2 * case.doc_len * row,
        "tail_kv": 2 * tail * row,
        "q": case.P * row,
        "out": case.P * row,
        "ids": 4 * case.seq_len,
        "tail_slots": tail,
        "doc_flops": 4 * case.D * case.H * case.P * case.doc_len,
        "tail_flops": 4 * case.D * case.H * tail,
    }


def cpu_baseline(case, target_s: float):
    """The fp64 oracle as it stands, timed on a bounded sample of streams of
    the same inputs (all heads each)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import oracle_decode

    ids = case.stream_id.numpy()
    rng = np.random.default_rng(0)
    order = rng.permutation(case.P).tolist()

    def timed(n):
        t = time.perf_counter()
        oracle_decode(case.q, case.k, case.v, ids, case.seq_len, case.scale, streams=order[:n])
        return time.perf_counter() - t

    # each call also converts the cache to fp64: fit t(n) = a + b*n from two
    # small calls, then size the timed sample to about target_s
    n1, n2 = 2, min(case.P, 8)
    t1, t2 = timed(n1), timed(n2)
    b = max((t2 - t1) / max(n2 - n1, 1), 1e-4)
    a = max(t1 - b * n1, 0.0)
    n = int(max(n2, min(case.P, (target_s - a) / b)))
    dt = timed(n)
    passes = 1
    # a whole step shorter than the target: repeat it (whole steps) up to about the target
    while n == case.P and dt * (passes + 1) / passes <= target_s:
        dt += timed(n)
        passes += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    what = f"{n} of {case.P} streams" if passes == 1 else f"the whole step ({n} streams) {passes} times"
    return {
        "value": n * passes / dt,
        "unit": "answer tok/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what} x all {case.H} heads, fp64 NumPy, {dt:.1f} s "
                  f"(includes the oracle's fp64 conversion of the KV cache)",
        "seconds": dt,
        "cpu_model": _cpu_model(),
    }


def _blas_threads() -> int:
    from threadpoolctl import threadpool_info

    return int(max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1]))


def oracle_rate(fn, units: float, unit: str, sample: str):
    """Time one call of an oracle function on a bounded sample: `units` of
    `unit` done in that call -> rate (the oracle as it stands, CPU only)."""
    t = time.perf_counter()
    fn()
    dt = time.perf_counter() - t
    return {"value": units / dt, "unit": unit, "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{sample}, fp64 NumPy, {dt:.1f} s", "seconds": dt}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def decode_loop(torch, pp, dev, layers=32, steps=32, doc=12000, P=256, H=32, D=128, seed=1003, rope_base=1e6,
                with_oracle=True, Hkv=None, model="codellama7b"):
    """The answer loop of a 12000-token document with 256 streams: 32 steps of
    32 layers, each step appending one slot per stream (ids and plan once per
    step, then per layer: rotary embedding at the shared positions, append,
    attention).  Timed eagerly and as one captured HIP graph of the step
    replayed every step (the step's start lives on the device).  The q/k/v
    inputs of a layer are reused from step to step here (values do not change
    the work); the parity tests use fresh ones.  Hkv < H: query heads in
    groups sharing a key/value head."""
    from workloads import decode_loop_layout

    Hkv = H if Hkv is None else Hkv
    ids_full, q_lens, base0 = decode_loop_layout(doc, P, steps, seed)
    cap = len(ids_full)
    ids = ids_full.copy()
    ids[base0:] = 0
    sid = torch.from_numpy(ids).to(dev)
    g = torch.Generator(device=dev).manual_seed(seed)
    K = torch.randn(layers, cap, Hkv, D, generator=g, device=dev, dtype=torch.bfloat16)
    V = torch.randn(layers, cap, Hkv, D, generator=g, device=dev, dtype=torch.bfloat16)
    qs = torch.randn(layers, P, H, D, generator=g, device=dev, dtype=torch.bfloat16)
    kvn = torch.randn(layers, 2, P, Hkv, D, generator=g, device=dev, dtype=torch.bfloat16)
    outs = torch.empty(layers, P, H, D, device=dev, dtype=torch.bfloat16)
    base = torch.tensor([base0], dtype=torch.int32, device=dev)
    plan = (torch.zeros(2, dtype=torch.int32, device=dev), torch.zeros(P, dtype=torch.int32, device=dev),
            torch.zeros(P, 256, dtype=torch.int32, device=dev))
    ws = torch.empty(pp.multi_workspace_bytes(cap, 1, P, H, Hkv, D, torch.bfloat16), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)

    def one_step():
        pp.pp_step_plan(sid, base, P, max_seq_len=cap, plan=plan)
        for i in range(layers):
            pp.pp_attn_decode_append(qs[i], kvn[i, 0], kvn[i, 1], K[i], V[i], sid, plan, scale=scale,
                                     rope_base=rope_base, out=outs[i], workspace=ws, max_seq_len=cap)
        base.add_(P)

    def timed(fn):
        base.fill_(base0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        assert int(base.item()) == base0 + steps * P
        return a.elapsed_time(b)

    timed(one_step)  # warm-up pass over the whole loop
    eager_ms = timed(one_step)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        one_step()
    torch.cuda.synchronize()
    timed(graph.replay)
    graph_ms = timed(graph.replay)
    cpu = None
    if with_oracle:
        from oracle import oracle_append_step

        b_last = base0 + (steps - 1) * P
        kc, vc = K[0, :b_last + P].cpu(), V[0, :b_last + P].cpu()
        qi, ki, vi = (x.cpu() for x in (qs[0], kvn[0, 0], kvn[0, 1]))
        cpu = oracle_rate(lambda: oracle_append_step(qi, ki, vi, kc, vc, ids_full, b_last, scale, rope_base,
                                                     streams=[0, 85, 170, 255]),
                          4 / layers, "answer tok/s",
                          f"one layer of the last step ({layers} per answer token) for 4 of {P} streams, all heads, "
                          "including the append, rotation and fp64 conversion of that layer's cache")
    # KV bytes the loop reads: every layer-step reads the document and each
    # stream's own slots (its question and the answers so far, new one included)
    tail_slots = sum(sum(q_lens) + P * (t + 1) for t in range(steps))
    kv_bytes = layers * (steps * doc + tail_slots) * Hkv * D * 2 * 2
    attn_flops = layers * (steps * P * doc + tail_slots) * H * D * 4
    return {
        "workload": f"{model}_doc12k_p{P}_{layers}layers_{steps}steps",
        "layers": layers, "steps": steps, "P": P, "doc_len": doc, "rope_base": rope_base, "Hq": H, "Hkv": Hkv,
        "seq_len_first_last": [base0 + P, base0 + steps * P],
        "graph_ms_total": graph_ms, "eager_ms_total": eager_ms,
        "graph_ms_per_step": graph_ms / steps, "eager_ms_per_step": eager_ms / steps,
        "graph_us_per_layer_step": graph_ms / steps / layers * 1e3,
        "answer_tok_s_graph": P * steps / (graph_ms / 1e3),
        "effective_kv_gbs_graph": kv_bytes / (graph_ms / 1e3) / 1e9,
        "effective_kv_hbm_frac_graph": kv_bytes / (graph_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        # with grouped heads every K/V row meets Hq / Hkv queries, so the
        # loop leans on the matrix cores: its attention flops (QK and PV,
        # 2 flops per multiply-add) against the dense bf16 peak
        "attn_tflops_graph": attn_flops / (graph_ms / 1e3) / 1e12,
        "attn_mfma_frac_graph": attn_flops / (graph_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "inputs": "per-layer q/k/v reused across steps; caches N(0,1) bf16 from a seeded device generator",
        "cpu_oracle": cpu,
    }


def answer_sweep(torch, pp, dev, lengths=(128, 256, 512, 1024), doc=8192, P=128, H=32, D=128, seed=1005,
                 with_oracle=True):
    """Long answers: an 8k-token document with 128 questions (16-32 tokens)
    and 128-1,024 answer tokens per stream already cached; one step through
    pp_attn_decode and through the per-question baseline."""
    import numpy as np

    from workloads import canonical_layout

    rows = []
    for a in lengths:
        rng = np.random.Generator(np.random.PCG64(seed ^ a))
        q_lens = [int(x) for x in rng.integers(16, 33, size=P)]
        ids, _ = canonical_layout(doc, q_lens, [a] * P)
        T = len(ids)
        g = torch.Generator(device=dev).manual_seed(seed + a)
        q = torch.randn(P, H, D, generator=g, device=dev, dtype=torch.bfloat16)
        k = torch.randn(T, H, D, generator=g, device=dev, dtype=torch.bfloat16)
        v = torch.randn(T, H, D, generator=g, device=dev, dtype=torch.bfloat16)
        sid = torch.from_numpy(ids).to(dev)
        out = torch.empty_like(q)
        ws = torch.empty(pp.workspace_bytes(T, P, H, D, torch.bfloat16), dtype=torch.uint8, device=dev)

        def t(fn, n, warm):
            for _ in range(warm):
                fn(q, k, v, sid, seq_len=T, out=out, workspace=ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn(q, k, v, sid, seq_len=T, out=out, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        dm = t(pp.pp_attn_decode, 10, 2)
        bm = t(pp.pp_attn_decode_batched, 3, 1)
        kv = T * H * D * 2 * 2
        row = {"answer_len": a, "seq_len": T, "decode_ms": dm, "batched_ms": bm, "speedup": bm / dm,
               "effective_kv_gbs": kv / (dm / 1e3) / 1e9}
        if with_oracle and a == lengths[-1]:
            from oracle import oracle_decode

            qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
            row["cpu_oracle"] = oracle_rate(lambda: oracle_decode(qc, kc, vc, ids, T, 1.0 / math.sqrt(D),
                                                                  streams=[0, P - 1]),
                                            2, "answer tok/s", f"2 of {P} streams, all heads, one step")
        rows.append(row)
        del q, k, v, sid, out, ws
        torch.cuda.empty_cache()
    return {"workload": f"codellama7b_doc8k_p{P}_answers{lengths[0]}-{lengths[-1]}", "P": P, "doc_len": doc,
            "questions": "uniform 16-32", "rows": rows}


def prefill_bench(torch, pp, dev, doc=16384, P=256, H=32, D=128, seed=1006, runs=5, with_oracle=True, Hkv=None):
    """Prefill of the packed request (the 16k-token document and 256
    questions of 8-48 tokens, one sequence): every slot attends causally
    under the stream rule."""
    import numpy as np

    from workloads import _uniform_ints, canonical_layout

    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED))
    q_lens = _uniform_ints(rng, 8, 48, P)
    ids, _ = canonical_layout(doc, q_lens, [0] * P)
    T = len(ids)
    g = torch.Generator(device=dev).manual_seed(seed)
    hk = H if Hkv is None else Hkv
    q = torch.randn(T, H, D, generator=g, device=dev, dtype=torch.bfloat16)
    k, v = (torch.randn(T, hk, D, generator=g, device=dev, dtype=torch.bfloat16) for _ in range(2))
    sid = torch.from_numpy(ids).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(pp.prefill_workspace_bytes(T, H, D, torch.bfloat16), dtype=torch.uint8, device=dev)
    pp.pp_attn_prefill(q, k, v, sid, out=out, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(runs):
        pp.pp_attn_prefill(q, k, v, sid, out=out, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / runs
    # visible (query, key) pairs: the document causally, each question slot
    # the whole document and its own question up to itself
    pairs = doc * (doc + 1) // 2 + sum(n * doc + n * (n + 1) // 2 for n in q_lens)
    flops = 4 * D * H * pairs
    cpu = None
    if with_oracle:
        from oracle import oracle_prefill

        qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
        rows = [0, doc // 2, doc - 1, doc, (doc + T) // 2, T - 1, T - 2, T - 3]
        cpu = oracle_rate(lambda: oracle_prefill(qc, kc, vc, ids, T, 1.0 / math.sqrt(D), rows=rows), len(rows),
                          "prefilled tok/s", f"{len(rows)} of {T} slots (half of them question slots), all heads, "
                          "including the fp64 conversion of q, k, v")
    name = f"codellama7b_prefill_doc16k_p{P}" if Hkv is None else f"qwen2.5-7b-heads_prefill_doc16k_p{P}"
    return {"workload": name, "seq_len": T, "doc_len": doc, "P": P, "Hq": H, "Hkv": hk,
            "questions": "uniform 8-48", "ms": ms, "prefill_tok_s": T / (ms / 1e3),
            "visible_pairs_per_head": pairs, "tflops": flops / (ms / 1e3) / 1e12,
            "mfma_frac": flops / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, "cpu_oracle": cpu}


def multi_bench(torch, pp, dev, B=4, P=64, Hq=28, Hkv=4, D=128, doc=16384, a_len=31, seed=1007, steps=20,
                with_oracle=True):
    """Several requests per launch with grouped key/value heads: 4 requests of
    64 streams (the pages' best streams per request is 16-64), each on its
    own 16k-token document, 28 query heads sharing 4 key/value heads (the
    pages' real-benchmark model family); one decode step, and the
    per-question baseline on the same inputs."""
    import numpy as np

    from workloads import _uniform_ints, canonical_layout

    rng = np.random.Generator(np.random.PCG64(seed))
    layouts, q_total = [], 0
    for _ in range(B):
        ql = _uniform_ints(rng, 8, 48, P)
        q_total += sum(ql)
        layouts.append(canonical_layout(doc, ql, [a_len] * P)[0])
    T = max(len(x) for x in layouts)
    sid_np = np.full((B, T), -5, dtype=np.int32)
    for b, ids in enumerate(layouts):
        sid_np[b, : len(ids)] = ids
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn(B, P, Hq, D, generator=g, device=dev, dtype=torch.bfloat16)
    k = torch.randn(B, T, Hkv, D, generator=g, device=dev, dtype=torch.bfloat16)
    v = torch.randn(B, T, Hkv, D, generator=g, device=dev, dtype=torch.bfloat16)
    sid = torch.from_numpy(sid_np).to(dev)
    lens = torch.tensor([len(x) for x in layouts], dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(pp.multi_workspace_bytes(T, B, P, Hq, Hkv, D, torch.bfloat16), dtype=torch.uint8, device=dev)

    def t(batched, n):
        for _ in range(2):
            pp.pp_attn_decode_multi(q, k, v, sid, lens, out=out, workspace=ws, batched=batched)
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            pp.pp_attn_decode_multi(q, k, v, sid, lens, out=out, workspace=ws, batched=batched)
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e) / n

    ms = t(False, steps)
    bms = t(True, max(3, steps // 4))
    cpu = None
    if with_oracle:
        from oracle import oracle_decode

        n0 = len(layouts[0])
        qc, kc, vc = q[0].cpu(), k[0, :n0].cpu(), v[0, :n0].cpu()
        cpu = oracle_rate(lambda: oracle_decode(qc, kc, vc, layouts[0], n0, 1.0 / math.sqrt(D), streams=[0, 21, 42, 63]),
                          4, "answer tok/s", f"4 of the {P} streams of one request, all {Hq} query heads, one step")
    slot_bytes = Hkv * D * 2 * 2  # K + V of one slot, all key/value heads
    kv = (B * doc + q_total + B * P * a_len) * slot_bytes
    return {"workload": f"qwen2.5-7b-heads_{B}x{P}streams_doc16k", "B": B, "P": P, "Hq": Hq, "Hkv": Hkv, "d": D,
            "doc_len": doc, "questions": "uniform 8-48", "answers": a_len, "ms_per_step": ms,
            "answer_tok_s": B * P / (ms / 1e3), "effective_kv_gbs": kv / (ms / 1e3) / 1e9,
            "effective_kv_hbm_frac": kv / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "tflops": 4 * D * Hq * B * P * doc / (ms / 1e3) / 1e12,
            "mfma_frac": 4 * D * Hq * B * P * doc / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "batched_baseline_ms": bms, "speedup_of_decode": bms / ms, "cpu_oracle": cpu}


def serving_bench(torch, pp, dev, R=16, B=4, P=16, Hq=28, Hkv=4, D=128, seed=1008):
    """Continuous against static batching of request slots: 16 requests of
    16 streams on 4k-8k-token documents, every other one asking for long
    answers (128 tokens against 8), 4 slots of one pp_attn_decode_multi
    launch per step.  Refilling a slot copies the request's cache in (a
    stand-in for its prefill) and is inside the timed loop.  The continuous
    schedule is also run through the appending step (one plan of all slots,
    then append with rotation and attend), one layer per step as above."""
    import numpy as np

    from shared_prefix_stream_amd.batching import continuous_schedule, static_schedule
    from workloads import _uniform_ints, canonical_layout

    answer = [8, 128] * (R // 2)
    rng = np.random.Generator(np.random.PCG64(seed))
    reqs = []
    for a in answer:
        doc = int(rng.integers(4096, 8193))
        ql = _uniform_ints(rng, 16, 32, P)
        reqs.append((canonical_layout(doc, ql, [a] * P)[0], doc + sum(ql)))
    T = max(len(ids) for ids, _ in reqs)
    g = torch.Generator(device=dev).manual_seed(seed)
    pool_k = [torch.randn(len(ids), Hkv, D, generator=g, device=dev, dtype=torch.bfloat16) for ids, _ in reqs]
    pool_v = [torch.randn(len(ids), Hkv, D, generator=g, device=dev, dtype=torch.bfloat16) for ids, _ in reqs]
    pool_ids = [torch.from_numpy(ids).to(dev) for ids, _ in reqs]
    K = torch.zeros(B, T, Hkv, D, device=dev, dtype=torch.bfloat16)
    V = torch.zeros_like(K)
    sid = torch.full((B, T), -1, dtype=torch.int32, device=dev)
    q = torch.randn(B, P, Hq, D, generator=g, device=dev, dtype=torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.empty(pp.multi_workspace_bytes(T, B, P, Hq, Hkv, D, torch.bfloat16), dtype=torch.uint8, device=dev)

    def run(steps):
        lens = torch.tensor([[0 if x is None else reqs[x[0]][1] + (x[1] + 1) * P for x in st] for st in steps],
                            dtype=torch.int32, device=dev)
        placed = [None] * B
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i, st in enumerate(steps):
            for b, x in enumerate(st):
                if x is not None and placed[b] != x[0]:
                    r = x[0]
                    n = pool_ids[r].shape[0]
                    K[b, :n].copy_(pool_k[r])
                    V[b, :n].copy_(pool_v[r])
                    sid[b, :n].copy_(pool_ids[r])
                    placed[b] = r
            pp.pp_attn_decode_multi(q, K, V, sid, lens[i], out=out, workspace=ws)
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e)

    kn = torch.randn(B, P, Hkv, D, generator=g, device=dev, dtype=torch.bfloat16)
    vn = torch.randn_like(kn)
    plan = (torch.zeros(2 * B, dtype=torch.int32, device=dev), torch.zeros(B, P, dtype=torch.int32, device=dev),
            torch.zeros(B, P, 256, dtype=torch.int32, device=dev))

    def run_appending(steps):
        # the same schedule through the appending step: per step one plan of
        # all slots (idle slots at base -1), then append + rotate + attend
        bases = torch.tensor([[-1 if x is None else reqs[x[0]][1] + x[1] * P for x in st] for st in steps],
                             dtype=torch.int32, device=dev)
        placed = [None] * B
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i, st in enumerate(steps):
            for b, x in enumerate(st):
                if x is not None and placed[b] != x[0]:
                    r = x[0]
                    n = pool_ids[r].shape[0]
                    K[b, :n].copy_(pool_k[r])
                    V[b, :n].copy_(pool_v[r])
                    sid[b, :n].copy_(pool_ids[r])
                    placed[b] = r
            pp.pp_step_plan_multi(sid, bases[i], P, plan=plan)
            pp.pp_attn_decode_append_multi(q, kn, vn, K, V, sid, plan, rope_base=1e6, out=out, workspace=ws)
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e)

    res = {}
    for name, fn, runner in (("static", static_schedule, run), ("continuous", continuous_schedule, run),
                             ("continuous_appending", continuous_schedule, run_appending)):
        steps = fn(answer, B)
        runner(steps)  # warm-up pass
        ms = runner(steps)
        res[name] = {"decode_steps": len(steps), "ms": ms, "answer_tok_s": P * sum(answer) / (ms / 1e3)}
    return {"workload": f"qwen2.5-7b-heads_{R}requests_x{P}streams_{B}slots_answers8-128",
            "requests": R, "slots": B, "P": P, "Hq": Hq, "Hkv": Hkv, "doc_len": "uniform 4096-8192",
            "answers": "8 and 128 tokens, alternating", **res,
            "steps_saved_frac": 1 - res["continuous"]["decode_steps"] / res["static"]["decode_steps"],
            "speedup": res["static"]["ms"] / res["continuous"]["ms"]}


# stage of pp_attn_decode_profiled -> kernel-name prefixes in a rocprofv3 kernel trace
STAGE_KERNELS = {
    "plan": ("plan_kernel",),
    "document": ("doc_mfma_bf16_kernel", "doc_valu_f32_kernel"),
    "own_slots_merge": ("tail_merge_kernel",),
}
SLEEP_CYCLES = 1_000_000  # a GPU spin of ~0.5 ms: the host enqueues a timed call before the GPU reaches it


def read_trace_avg_us(stage: str, workload: str):
    """Average duration of a stage's kernel in profiles/kernels_<workload>.txt
    (a rocprofv3 --kernel-trace --stats summary), or None if absent or taken
    on other kernel sources."""
    path = os.path.join(PROFILES, f"kernels_{workload}.txt")
    if not os.path.exists(path):
        return None
    lines = open(path).read().splitlines()
    digest = next((ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("kernel_source_digest:")), None)
    if digest != kernel_source_digest():
        return None
    for ln in lines:
        if ln.startswith(STAGE_KERNELS[stage]):
            name, rest = ln.split(">", 1) if ">" in ln else (ln.split()[0], " ".join(ln.split()[1:]))
            cols = rest.split()
            try:
                return float(cols[1])  # calls, avg_us, ...
            except (IndexError, ValueError):
                return None
    return None


def read_sq_counters(stage: str, workload: str):
    """Matrix-core busy and LDS utilisation of a stage's kernel from
    profiles/pmc_sq_<workload>.txt (rocprofv3 SQ counters), or None if absent
    or taken on other kernel sources."""
    path = os.path.join(PROFILES, f"pmc_sq_{workload}.txt")
    if not os.path.exists(path):
        return None
    lines = open(path).read().splitlines()
    digest = next((ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("kernel_source_digest:")), None)
    if digest != kernel_source_digest():
        return None
    out, inside = {}, False
    for ln in lines:
        if ln and not ln.startswith(" ") and not ln.startswith("#"):
            inside = ln.startswith(stage + " (")
            continue
        if inside and "%" in ln and "=" in ln:
            key = ln.split("=")[0].strip()
            if key in ("MfmaUtil", "LdsUtil"):
                out[key] = float(ln.rsplit(None, 2)[-2]) / 100.0
    if not out:
        return None
    out["source"] = os.path.relpath(path, ROOT)
    return out


def median_ci(xs, n_boot: int = 2000, seed: int = 0):
    """Median of xs and a 95 % bootstrap interval of the median."""
    import numpy as np

    a = np.asarray(xs, dtype=np.float64)
    rng = np.random.default_rng(seed)
    boots = np.median(a[rng.integers(0, a.size, (n_boot, a.size))], axis=1)
    return float(np.median(a)), [float(np.percentile(boots, 2.5)), float(np.percentile(boots, 97.5))]


def geomean_ci(xs, n_boot: int = 2000, seed: int = 1):
    """Geometric mean of xs and a 95 % bootstrap interval of it."""
    import numpy as np

    la = np.log(np.asarray(xs, dtype=np.float64))
    rng = np.random.default_rng(seed)
    boots = np.exp(la[rng.integers(0, la.size, (n_boot, la.size))].mean(axis=1))
    return float(np.exp(la.mean())), [float(np.percentile(boots, 2.5)), float(np.percentile(boots, 97.5))]


def timed_call(torch, fn, flush=None):
    """GPU time (ms) of one call, bracketed by events on the current stream.
    The GPU is kept busy (a spin, or the cache-evicting write) while the host
    enqueues the call, so host launch latency is not inside the interval."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if flush is not None:
        flush.fill_(1)
    else:
        torch.cuda._sleep(SLEEP_CYCLES)
    a.record()
    fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b)


def paired_protocol(torch, dev, fa, fb, n_warm: int, n_cold: int):
    """Decode step (fa) and per-question baseline (fb) on identical inputs,
    timed as interleaved pairs (order alternating), warm and after a 1 GiB
    cache-evicting write; medians with 95 % bootstrap intervals and the
    geometric mean of the per-pair speedups."""
    warm_a, warm_b, cold_a, cold_b = [], [], [], []
    for _ in range(3):
        fa(), fb()
    torch.cuda.synchronize()
    for i in range(n_warm):
        if i % 2 == 0:
            warm_a.append(timed_call(torch, fa))
            warm_b.append(timed_call(torch, fb))
        else:
            warm_b.append(timed_call(torch, fb))
            warm_a.append(timed_call(torch, fa))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if n_cold else None
    for i in range(n_cold):
        if i % 2 == 0:
            cold_a.append(timed_call(torch, fa, flush))
            cold_b.append(timed_call(torch, fb, flush))
        else:
            cold_b.append(timed_call(torch, fb, flush))
            cold_a.append(timed_call(torch, fa, flush))
    del flush

    def summary(xs, ys):
        out = {}
        if xs:
            m, ci = median_ci(xs)
            out.update({"median_ms": m, "ci95_ms": ci, "n": len(xs)})
        if ys:
            m, ci = median_ci(ys)
            out.update({"cold_median_ms": m, "cold_ci95_ms": ci, "cold_n": len(ys)})
        return out

    res = {"decode": summary(warm_a, cold_a), "batched": summary(warm_b, cold_b),
           "protocol": f"{n_warm} warm and {n_cold} cold interleaved pairs (order alternating) on identical inputs; "
                       "events around each call; cold = after a 1 GiB write; medians with 95 % bootstrap intervals"}
    if warm_a:
        g, ci = geomean_ci([b / a for a, b in zip(warm_a, warm_b)])
        res["speedup_geomean"], res["speedup_ci95"] = g, ci
    if cold_a:
        g, ci = geomean_ci([b / a for a, b in zip(cold_a, cold_b)])
        res["cold_speedup_geomean"], res["cold_speedup_ci95"] = g, ci
    res["batched_summary"] = {"ms_per_step": res["batched"].get("median_ms"),
                              "speedup_of_decode": res.get("speedup_geomean"),
                              "speedup_ci95": res.get("speedup_ci95")}
    return res


def read_ceiling(torch, pp, dev, gib: int = 4, reps: int = 5):
    """Streaming-read rate of this device: a 4 GiB buffer (16x the last-level
    cache) read whole by pp_stream_read, over a few launch widths; the best."""
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    rates = {}
    for bpc in (2, 4, 8, 16):
        for _ in range(2):
            pp.stream_read(buf, sink, bpc)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            pp.stream_read(buf, sink, bpc)
        b.record()
        torch.cuda.synchronize()
        rates[bpc] = reps * n / (a.elapsed_time(b) / 1e3) / 1e9
    del buf
    torch.cuda.empty_cache()
    best = max(rates, key=rates.get)
    return {"gbs": rates[best], "frac_of_nominal": rates[best] / HBM_PEAK_GBS, "bytes_per_launch": n,
            "blocks_per_cu": best, "gbs_by_blocks_per_cu": {str(k): v for k, v in rates.items()},
            "kernel": "stream_read_kernel (include/ppmeasure.h)"}


def read_calibration(torch, pp, steps: int):
    """A 1 GiB buffer read `steps` times, for scaling PMC byte counters."""
    n = 1 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        pp.stream_read(buf, sink, 8)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"read_bytes": n, "write_bytes": 0, "ms": ms, "gbs": n / ms / 1e6}), flush=True)


def kernel_durations(torch, pp, case, q, k, v, sid, out, ws, n: int):
    """Mean and median duration (us) of each stage's kernel over n profiled
    steps, from events bound to the kernel's own start and end."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(pp.PP_PROFILE_EVENTS)]
    for e in evs:
        e.record()  # (torch creates the hipEvent_t on first record)
    torch.cuda.synchronize()
    handles = [e.cuda_event for e in evs]
    per = {name: [] for name in pp.PROFILE_STAGES}
    for _ in range(n):
        pp.pp_attn_decode_profiled(handles, q, k, v, sid, seq_len=case.seq_len, scale=case.scale, out=out,
                                   workspace=ws)
        torch.cuda.synchronize()
        for i, name in enumerate(pp.PROFILE_STAGES):
            per[name].append(evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e3)
    mean = {name: sum(x) / len(x) for name, x in per.items()}
    med = {name: sorted(x)[len(x) // 2] for name, x in per.items()}
    return mean, med


def stage_algorithmic_bytes(by):
    """Bytes each kernel must move (the split partials, workspace traffic, are
    not counted)."""
    return {
        "plan": by["ids"],
        "document": by["doc_kv"] + by["q"],
        "own_slots_merge": by["tail_kv"] + by["q"] + by["out"],
    }


def kernel_table(stage_us, stage_med_us, stage_bytes, by):
    kernels = {}
    for name, us in stage_us.items():
        gbs = stage_bytes[name] / (us * 1e-6) / 1e9
        kernels[name] = {"us": us, "median_us": stage_med_us[name], "algorithmic_bytes": stage_bytes[name],
                         "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    doc_tflops = by["doc_flops"] / (stage_us["document"] * 1e-6) / 1e12
    kernels["document"]["flops"] = by["doc_flops"]
    kernels["document"]["mfma_tflops"] = doc_tflops
    kernels["document"]["mfma_frac"] = doc_tflops / MFMA_BF16_PEAK_TFLOPS
    return kernels


def roofline_entry(dom, kernels, workload, ceiling):
    """Roofline of the dominant kernel: algorithmic bytes per launch over its
    mean duration (kernel-bound events over the profiled steps).  Its roof is
    HBM when its flops per byte sit below the ridge of the two published
    peaks (2.5 PFLOP/s / 8 TB/s = 312.5), else the matrix cores."""
    kern = kernels[dom]
    flops = kern.get("flops", 0)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "mfma" if flops / kern["algorithmic_bytes"] > ridge else "hbm"
    if bound == "hbm":
        achieved, peak, unit = kern["gbs"], HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = kern["mfma_tflops"], MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    trace_us = read_trace_avg_us(dom, workload)
    entry = {
        "bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
        "traffic": read_pmc_traffic(dom, workload),
        "algorithmic_bytes": kern["algorithmic_bytes"], "flops": flops,
        "intensity_flop_per_byte": flops / kern["algorithmic_bytes"], "ridge_flop_per_byte": ridge,
        "duration_us": kern["us"],
        "achieved_from": "algorithmic bytes / mean kernel duration, HIP events bound to the kernel's start and end "
                         "(hipExtLaunchKernel) over the profiled steps",
        "kernel_trace_avg_us": trace_us,
        "frac_from_kernel_trace": (kern["algorithmic_bytes"] / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS
                                   if trace_us and bound == "hbm" else None),
    }
    if flops:
        entry["mfma_frac"] = kern["mfma_frac"]
    # what the counters say binds it below both roofs (the roofline's bound is
    # the lower roof at this intensity)
    entry["counters"] = read_sq_counters(dom, workload)
    if ceiling and bound == "hbm":
        entry["measured_read_ceiling_gbs"] = ceiling["gbs"]
        entry["frac_vs_measured"] = achieved / ceiling["gbs"]
    return entry


def other_config(torch, pp, dev, name, seed, steps, warmup, ceiling):
    """One more single-step configuration, timed like the headline."""
    from workloads import named_workload

    case = named_workload(name, seed=seed)
    q, k, v, sid = (t.to(dev) for t in (case.q, case.k, case.v, case.stream_id))
    out = torch.empty_like(q)
    ws = torch.empty(pp.workspace_bytes(case.seq_len, case.P, case.H, case.D, q.dtype), dtype=torch.uint8, device=dev)
    by = step_bytes(case)

    def step():
        pp.pp_attn_decode(q, k, v, sid, seq_len=case.seq_len, scale=case.scale, out=out, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    us, med = kernel_durations(torch, pp, case, q, k, v, sid, out, ws, max(20, min(steps, 100)))
    kv = by["doc_kv"] + by["tail_kv"]
    step_b = kv + by["q"] + by["out"] + by["ids"]
    res = {
        "workload": name, "H": case.H, "d": case.D, "doc_len": case.doc_len, "P": case.P, "seq_len": case.seq_len,
        "ms_per_step": ms, "answer_tok_s": case.P / (ms / 1e3),
        "effective_kv_gbs": kv / (ms / 1e3) / 1e9, "effective_kv_hbm_frac": kv / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "step_algorithmic_bytes": step_b, "hbm_floor_us": step_b / (HBM_PEAK_GBS * 1e9) * 1e6,
        "kernels": kernel_table(us, med, stage_algorithmic_bytes(by), by),
    }
    if ceiling:
        res["effective_kv_frac_vs_measured_ceiling"] = res["effective_kv_gbs"] / ceiling["gbs"]
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="codellama7b_doc16k_p256")
    ap.add_argument("--seed", type=int, default=1002)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true")
    ap.add_argument("--no-decode-loop", action="store_true",
                    help="skip the 32-step x 32-layer appending loop (eager and graph-replayed)")
    ap.add_argument("--decode-loop-heads", choices=("both", "mha", "grouped"), default="both",
                    help="which appending loops to run: 32 heads, 28 query heads on 4 key/value heads, or both")
    ap.add_argument("--no-answer-sweep", action="store_true",
                    help="skip the long-answer sweep (8k document, 128 streams, 128-1024 answer tokens)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill of the 16k-token document with 256 questions")
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the 4-request, grouped-head (28/4) decode step")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip continuous against static batching of 16 requests in 4 slots")
    ap.add_argument("--pairs", type=int, default=50,
                    help="warm (decode step, per-question baseline) pairs timed interleaved")
    ap.add_argument("--cold-pairs", type=int, default=20,
                    help="the same pairs, each step after a 1 GiB cache-evicting write")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the streaming-read HBM ceiling")
    ap.add_argument("--no-c2", action="store_true", help="skip the doc 8k, P = 64 step")
    ap.add_argument("--read-calibration", action="store_true",
                    help="only stream-read a 1 GiB buffer --steps times (to scale PMC byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the decode step of one "
              "request runs on one MI355X; multi-GPU sharding is not part of this library.", file=sys.stderr)
        sys.exit(2)

    import torch

    import shared_prefix_stream_amd as pp
    from workloads import named_workload

    if args.read_calibration:
        read_calibration(torch, pp, args.steps)
        return

    dev = torch.device("cuda:0")
    log(f"bench: generating {args.workload} seed {args.seed}")
    case = named_workload(args.workload, seed=args.seed)
    q, k, v, sid = (t.to(dev) for t in (case.q, case.k, case.v, case.stream_id))
    out = torch.empty_like(q)
    ws = torch.empty(pp.workspace_bytes(case.seq_len, case.P, case.H, case.D, q.dtype), dtype=torch.uint8, device=dev)
    by = step_bytes(case)

    def step():
        pp.pp_attn_decode(q, k, v, sid, seq_len=case.seq_len, scale=case.scale, out=out, workspace=ws)

    outb = torch.empty_like(q)

    def batched_step():
        pp.pp_attn_decode_batched(q, k, v, sid, seq_len=case.seq_len, scale=case.scale, out=outb, workspace=ws)

    # The legs that need no exact step count run first: after the seconds of
    # host-side input generation the GPU idles at low clocks, and a few
    # warm-up steps do not bring it back (measured: 153 us per step right
    # after the inputs were made, 134 us with the GPU busy before).  The
    # headline below is timed on a busy GPU, as a serving loop runs it.
    # ---- the HBM read ceiling of this device --------------------------------------
    ceiling = None
    if not args.no_read_ceiling:
        log("bench: streaming-read ceiling")
        ceiling = read_ceiling(torch, pp, dev)

    # ---- paired protocol: decode step and per-question baseline interleaved --
    paired = None
    if not args.no_batched:
        log(f"bench: {args.pairs} warm and {args.cold_pairs} cold pairs (decode step, per-question baseline)")
        paired = paired_protocol(torch, dev, step, batched_step, args.pairs, args.cold_pairs)

    # ---- per-kernel durations: events bound to each kernel's start and end ---
    stage_us, stage_med_us = kernel_durations(torch, pp, case, q, k, v, sid, out, ws, max(20, min(args.steps, 100)))

    # ---- headline: K back-to-back steps, inputs resident in HBM --------------
    log(f"bench: warmup {args.warmup}, timed {args.steps}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    t_s = ms / 1e3

    # ---- numbers ----------------------------------------------------------------
    kv = by["doc_kv"] + by["tail_kv"]
    kv_gbs = kv / t_s / 1e9
    doc_gbs = by["doc_kv"] / t_s / 1e9
    stage_bytes = stage_algorithmic_bytes(by)
    kernels = kernel_table(stage_us, stage_med_us, stage_bytes, by)
    dom = max(stage_us, key=stage_us.get)
    roofline = roofline_entry(dom, kernels, args.workload, ceiling)

    c2 = None
    if not args.no_c2:
        log("bench: doc 8k, P = 64 step")
        c2 = other_config(torch, pp, dev, "codellama7b_doc8k_p64", 1001, args.steps, args.warmup, ceiling)
        torch.cuda.empty_cache()

    loop = None
    if not args.no_decode_loop:
        log("bench: 32-step x 32-layer appending loop")
        loop = {}
        if args.decode_loop_heads != "grouped":
            loop = decode_loop(torch, pp, dev, with_oracle=not args.no_cpu_baseline)
            torch.cuda.empty_cache()
        if args.decode_loop_heads != "mha":
            log("bench: appending loop, 28 query heads sharing 4 key/value heads")
            loop["grouped_heads"] = decode_loop(torch, pp, dev, layers=28, H=28, Hkv=4, with_oracle=False,
                                                model="qwen7b_shape")
            torch.cuda.empty_cache()

    sweep = None
    if not args.no_answer_sweep:
        log("bench: long-answer sweep")
        sweep = answer_sweep(torch, pp, dev, with_oracle=not args.no_cpu_baseline)

    prefill = None
    if not args.no_prefill:
        log("bench: prefill")
        prefill = prefill_bench(torch, pp, dev, with_oracle=not args.no_cpu_baseline)
        prefill["grouped_heads"] = prefill_bench(torch, pp, dev, H=28, Hkv=4, with_oracle=False)
        torch.cuda.empty_cache()

    multi = None
    if not args.no_multi:
        log("bench: several requests, grouped heads")
        multi = multi_bench(torch, pp, dev, with_oracle=not args.no_cpu_baseline)
        torch.cuda.empty_cache()

    serving = None
    if not args.no_serving:
        log("bench: continuous against static batching")
        serving = serving_bench(torch, pp, dev)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(case, args.cpu_seconds)

    result = {
        "metric": METRIC,
        "value": case.P / t_s,
        "unit": "answer tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16, canonical layout (document, questions, answers "
                "interleaved by step); one layer's attention, no model weights",
        "config": {"workload": args.workload, "H": case.H, "d": case.D, "doc_len": case.doc_len, "P": case.P,
                   "seq_len": case.seq_len, "tail_slots": by["tail_slots"], "seed": args.seed},
        "steps_per_s": 1 / t_s,
        "wall_ms_per_step": wall_ms,
        "cold_ms_per_step": paired["decode"].get("cold_median_ms") if paired else None,
        "effective_kv_gbs": kv_gbs,
        "effective_kv_hbm_frac": kv_gbs / HBM_PEAK_GBS,
        "doc_kv_gbs": doc_gbs,
        "doc_kv_hbm_frac": doc_gbs / HBM_PEAK_GBS,
        "step_algorithmic_bytes": kv + by["q"] + by["out"] + by["ids"],
        "step_flops": by["doc_flops"] + by["tail_flops"],
        "kernels": kernels,
        "roofline": roofline,
        "batched_baseline": paired["batched_summary"] if paired else None,
        "paired": paired,
        "hbm_read_ceiling": ceiling,
        "effective_kv_frac_vs_measured_ceiling": (kv_gbs / ceiling["gbs"]) if ceiling else None,
        "config_doc8k_p64": c2,
        "decode_loop": loop,
        "answer_sweep": sweep,
        "prefill": prefill,
        "multi_request_gqa": multi,
        "continuous_batching": serving,
        "cpu_baseline": cpu,
        "kernel_source_digest": kernel_source_digest(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

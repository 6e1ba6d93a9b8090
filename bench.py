#!/usr/bin/env python3
"""Throughput of the TurboQuant KV-cache hot path on one MI355X.

Default workload (32K-context decode config): 16 sequences x 8 kv heads x
32768 cached tokens, head_dim 128, bf16 keys encoded as turbo3 (2-bit
Lloyd-Max + 128 QJL signs, 56-byte records), 32 bf16 query heads (grouped
4:1) scored from the compressed keys.  One step = encode the whole key cache
+ score every query head against a whole (previously encoded) cache.

Inputs are resident in HBM before timing.  Buffers rotate (2 input caches,
3 record caches) so that neither kernel reads data the 256 MB memory-side
cache still holds from the previous launch.  Kernel durations come from HIP
events on the stream the kernels are launched on.

Prints ONE JSON line.  `--config c2|c4|c5|haar|paged|gram` measures the
prefill-encode, the long-context attend, the mixed-precision layer, the
Haar-rotation, the paged-cache decode and the Gram-table scoring rows instead
(also one line each).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-K score tokens/s + encode GB/s at 32K ctx; % of HBM roofline"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def _kernel_sources_sha(kernel: str) -> str:
    from kv_cache_vector_diag_amd.rocprof_summary import kernel_sources_sha
    return kernel_sources_sha(ROOT, kernel)


def _traffic(kernel_key: str, launches_bytes: float):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data[kernel_key]
    except (KeyError, ValueError):
        return None
    if "kernel" not in ent or ent.get("source_sha") != _kernel_sources_sha(ent["kernel"]):
        return None
    return ent.get("hbm_bytes_per_launch")


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def cpu_baseline_c3(budget_s: float = 15.0) -> dict:
    """The oracle (as it stands) on a bounded sample of the same workload:
    whole (sequence, kv-head) groups of 32768 keys, encode + score of the 4
    query heads of each group, single thread (BLAS limited to 1)."""
    from threadpoolctl import threadpool_limits

    from kv_cache_vector_diag_amd import inputs
    from oracle import turboquant as tq
    T, d, Hkv, Hq_per = 32768, 128, 8, 4
    with threadpool_limits(1):
        qzs = tq.quantizers(Hkv, d, 3, 128, 3, tq.ROLE_KEY)
        q = inputs.exact_values(inputs.to_torch(inputs.queries(3, 16, 32, d), "bf16"))
        done = 0
        spent = 0.0
        while done < 128 and spent < budget_s:
            g = done
            K = inputs.exact_values(inputs.to_torch(inputs.kv_normal(3, 128, T, d, groups=[g]), "bf16"))[0]
            t0 = time.perf_counter()
            enc = tq.encode(qzs[g % Hkv], K)
            b, h = divmod(g, Hkv)
            tq.scores([qzs[g % Hkv]], enc.records[None, None], q[b:b + 1, h * Hq_per:(h + 1) * Hq_per])
            spent += time.perf_counter() - t0
            done += 1
    tokens = done / Hkv * T   # sequence positions fully processed (all kv heads of a position)
    return {"value": tokens / spent, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of 128 (sequence, kv-head) groups x {T} keys: encode + score of 4 query "
                      f"heads each, float64 NumPy, 1 thread, {spent:.1f} s"}


def bench_c3(args, torch, b):
    from kv_cache_vector_diag_amd import inputs
    dev = "cuda:0"
    B, Hkv, Hq, T, d, bits, m, seed = 16, 8, 32, 32768, 128, 3, 128, 3
    G = B * Hkv
    words = b.tq_record_bytes(d, bits, m, b.ROLE_KEY) // 4
    kcb = b.make_codebooks(Hkv, d, bits, m, seed, b.ROLE_KEY, device=dev)
    K0 = inputs.to_torch(inputs.kv_normal(seed, G, T, d), "bf16", dev)
    K1 = inputs.to_torch(inputs.kv_normal(seed + 1000, G, T, d), "bf16", dev)
    Ks = [K0, K1]
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", dev)
    recs = [torch.empty((G, T, words), dtype=torch.int32, device=dev) for _ in range(3)]
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for i in range(3):
        b.tq_encode_keys(kcb, Hkv, Ks[i % 2], d, bits, m, rec=recs[i], status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0

    def step(i, ev=None):
        if ev:
            ev[0].record()
        b.tq_encode_keys(kcb, Hkv, Ks[i % 2], d, bits, m, rec=recs[i % 3], status=status)
        if ev:
            ev[1].record()
        b.tq_scores(kcb, Hkv, recs[(i + 1) % 3].view(B, Hkv, T, words), q, d, bits, m, out=scores)
        if ev:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [_events(torch, 3) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0
    enc_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    sc_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_step = wall * 1e3 / args.steps

    enc_bytes = G * T * d * 2 + G * T * words * 4 + kcb.numel()           # 312 B per key + codebooks
    sc_bytes = G * T * words * 4 + B * Hq * T * 4 + q.numel() * 2 + kcb.numel()  # 56 B + 4 scores per key
    enc_gbps = enc_bytes / (enc_ms * 1e-3) / 1e9
    sc_gbps = sc_bytes / (sc_ms * 1e-3) / 1e9
    tokens = B * T
    dominant = "encode" if enc_ms >= sc_ms else "score"
    dom_gbps, dom_bytes = (enc_gbps, enc_bytes) if dominant == "encode" else (sc_gbps, sc_bytes)
    tr = _traffic(f"{dominant}_c3", dom_bytes)
    line = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "32K-context decode step: encode turbo3 keys + score from compressed keys",
                   "batch": B, "kv_heads": Hkv, "q_heads": Hq, "ctx": T, "head_dim": d, "key_bits": bits,
                   "projections": m, "input": "bf16 N(0,1), seed 3", "record_bytes": words * 4},
        "encode_ms": enc_ms, "encode_GBps": enc_gbps, "encode_frac_hbm": enc_gbps / HBM_PEAK_GBPS,
        "encode_keys_per_s": G * T / (enc_ms * 1e-3),
        "score_ms": sc_ms, "score_GBps": sc_gbps, "score_frac_hbm": sc_gbps / HBM_PEAK_GBPS,
        "score_tokens_per_s": tokens / (sc_ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": dom_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dom_gbps / HBM_PEAK_GBPS, "traffic": tr, "kernel": dominant,
                     "algorithmic_bytes_per_launch": dom_bytes},
        "roofline_score": {"bound": "hbm", "achieved": sc_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": sc_gbps / HBM_PEAK_GBPS, "traffic": _traffic("score_c3", sc_bytes),
                           "algorithmic_bytes_per_launch": sc_bytes},
    }
    return line


def bench_c2(args, torch, b):
    from kv_cache_vector_diag_amd import inputs
    dev = "cuda:0"
    L, Hkv, T, d, seed = 32, 8, 4096, 128, 1
    G = L * Hkv
    kw = b.tq_record_bytes(d, 4, 128, b.ROLE_KEY) // 4
    vw = b.tq_record_bytes(d, 4, 0, b.ROLE_VALUE) // 4
    kcb = b.make_codebooks(G, d, 4, 128, seed, b.ROLE_KEY, device=dev)
    vcb = b.make_codebooks(G, d, 4, 0, seed, b.ROLE_VALUE, device=dev)
    Kf, Vf, _ = inputs.kv_outliers(seed, G, T, d)
    K = inputs.to_torch(Kf, "bf16", dev)
    V = inputs.to_torch(Vf, "bf16", dev)
    krec = [torch.empty((G, T, kw), dtype=torch.int32, device=dev) for _ in range(2)]
    vrec = [torch.empty((G, T, vw), dtype=torch.int32, device=dev) for _ in range(2)]

    def step(i, ev=None):
        if ev:
            ev[0].record()
        b.tq_encode_keys(kcb, G, K, d, 4, 128, rec=krec[i % 2])
        if ev:
            ev[1].record()
        b.tq_encode_values(vcb, G, V, d, 4, rec=vrec[i % 2])
        if ev:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    evs = [_events(torch, 3) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    v_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_step = wall * 1e3 / args.steps
    kb = G * T * (d * 2 + kw * 4) + kcb.numel()
    vb = G * T * (d * 2 + vw * 4) + vcb.numel()
    return {"metric": "prefill encode GB/s (K turbo4 + V 4-bit)", "value": (kb + vb) / (ms_step * 1e-3) / 1e9,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "prefill encode: 32 layers x 8 kv heads x 4096 tokens, d=128, bf16 with "
                                   "4 outlier channels x8, K b=4 + V 4-bit"},
            "encode_keys_ms": k_ms, "encode_keys_GBps": kb / (k_ms * 1e-3) / 1e9,
            "encode_values_ms": v_ms, "encode_values_GBps": vb / (v_ms * 1e-3) / 1e9,
            "roofline": {"bound": "hbm", "achieved": kb / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": kb / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "traffic": _traffic("encode_c2", kb), "kernel": "encode_keys"}}


def bench_c4(args, torch, b):
    from kv_cache_vector_diag_amd import inputs
    dev = "cuda:0"
    B, Hkv, Hq, T, d, seed = 4, 8, 8, 131072, 128, 4
    G = B * Hkv
    kw = b.tq_record_bytes(d, 2, 128, b.ROLE_KEY) // 4
    vw = b.tq_record_bytes(d, 2, 0, b.ROLE_VALUE) // 4
    kcb = b.make_codebooks(Hkv, d, 2, 128, seed, b.ROLE_KEY, device=dev)
    vcb = b.make_codebooks(Hkv, d, 2, 0, seed, b.ROLE_VALUE, device=dev)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), "bf16", dev)
    V = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_V), "bf16", dev)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", dev)
    krecs = [b.tq_encode_keys(kcb, Hkv, K, d, 2, 128).view(B, Hkv, T, kw) for _ in range(2)]
    vrecs = [b.tq_encode_values(vcb, Hkv, V, d, 2).view(B, Hkv, T, vw) for _ in range(2)]
    del K, V
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    work = torch.empty(b.load().tq_attend_workspace_bytes(d, B, Hq, T), dtype=torch.uint8, device=dev)

    def step(i):
        b.tq_attend(kcb, Hkv, vcb, Hkv, krecs[i % 2], vrecs[i % 2], q, d, 2, 2, 128, out=out, work=work)

    for i in range(args.warmup):
        step(i)
    ev = _events(torch, 2)
    torch.cuda.synchronize()
    ev[0].record()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    ev[1].record()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_eager_dev = ev[0].elapsed_time(ev[1]) / args.steps
    # the call's three launches captured in a HIP graph per cache and replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
        step(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = [torch.cuda.CUDAGraph() for _ in range(2)]
    for i in range(2):
        with torch.cuda.graph(graphs[i]):
            step(i)
    for i in range(args.warmup):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    ev[0].record()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % 2].replay()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    fused_bytes = G * T * (kw + vw) * 4 + q.numel() * 2 + out.numel() * 4
    return {"metric": "long-context decode step tokens/s (scores -> softmax -> V from compressed K, V)",
            "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "long-context step: B=4, 8 kv heads, 8 q heads, 131072 tokens, d=128, "
                                   "turbo2 K + 2-bit V",
                       "launch": "HIP graph per step (eager launches: ms_per_step_eager)"},
            "ms_per_step_eager": ms_eager, "ms_per_step_eager_device": ms_eager_dev,
            "roofline": {"bound": "hbm", "achieved": fused_bytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": fused_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "traffic": _traffic("attend_c4", fused_bytes), "kernel": "attend"}}


def bench_c5(args, torch, b):
    """Mixed-precision layers: 32 layers x 8 kv heads x 16384 tokens, d=256, bf16 K and V
    with per-channel std log-uniform in [0.5, 8] (seed 5).  Layers 0, 1, 30, 31: K b=8
    (7-bit Lloyd-Max + 256 QJL signs) and V 8-bit; other layers: 32 outlier channels by
    variance at b+1 = 4 bits (Walsh-Hadamard), 224 normal channels at b = 3 bits (Haar)."""
    from kv_cache_vector_diag_amd import inputs
    dev = "cuda:0"
    L, Hkv, T, d, n_out, seed = 32, 8, 16384, 256, 32, 5
    G = L * Hkv
    Kd = torch.empty((G, T, d), dtype=torch.bfloat16, device=dev)
    Vd = torch.empty((G, T, d), dtype=torch.bfloat16, device=dev)
    for l in range(L):
        gl = list(range(l * Hkv, (l + 1) * Hkv))
        Kd[gl[0]:gl[-1] + 1] = inputs.to_torch(inputs.kv_channel_std(seed, G, T, d, stream=inputs.STREAM_K,
                                                                     groups=gl)[0], "bf16", dev)
        Vd[gl[0]:gl[-1] + 1] = inputs.to_torch(inputs.kv_channel_std(seed, G, T, d, stream=inputs.STREAM_V,
                                                                     groups=gl)[0], "bf16", dev)
    edges = [(0, 2 * Hkv), ((L - 2) * Hkv, L * Hkv)]          # boundary layers 0,1 and 30,31
    s0, s1 = 2 * Hkv, (L - 2) * Hkv                            # split layers 2..29
    GS = s1 - s0
    kcb8 = [b.make_codebooks(e1 - e0, d, 8, d, seed, b.ROLE_KEY, dev, seeds=[seed + g for g in range(e0, e1)])
            for e0, e1 in edges]
    vcb8 = [b.make_codebooks(e1 - e0, d, 8, 0, seed, b.ROLE_VALUE, dev, seeds=[seed + g for g in range(e0, e1)])
            for e0, e1 in edges]
    kcbn, kcbo = b.split_codebooks(GS, d, n_out, 3, seed + s0, b.ROLE_KEY, device=dev)
    vcbn, vcbo = b.split_codebooks(GS, d, n_out, 3, seed + s0, b.ROLE_VALUE, device=dev)
    kw8 = b.tq_record_bytes(d, 8, d, b.ROLE_KEY) // 4
    vw8 = b.tq_record_bytes(d, 8, 0, b.ROLE_VALUE) // 4
    kwn, kwo = b.split_record_words(d, n_out, 3, b.ROLE_KEY)
    vwn, vwo = b.split_record_words(d, n_out, 3, b.ROLE_VALUE)
    krec8 = [torch.empty((e1 - e0, T, kw8), dtype=torch.int32, device=dev) for e0, e1 in edges]
    vrec8 = [torch.empty((e1 - e0, T, vw8), dtype=torch.int32, device=dev) for e0, e1 in edges]
    krn = torch.empty((GS, T, kwn), dtype=torch.int32, device=dev)
    kro = torch.empty((GS, T, kwo), dtype=torch.int32, device=dev)
    vrn = torch.empty((GS, T, vwn), dtype=torch.int32, device=dev)
    vro = torch.empty((GS, T, vwo), dtype=torch.int32, device=dev)
    kchan = torch.empty((GS, d), dtype=torch.int32, device=dev)
    vchan = torch.empty((GS, d), dtype=torch.int32, device=dev)
    work = torch.empty(b.load().tq_outlier_workspace_bytes(d, GS, T), dtype=torch.uint8, device=dev)
    kwork = torch.empty(b.tq_encode_split_workspace_bytes(b.ROLE_KEY, d, n_out, 3, GS), dtype=torch.uint8, device=dev)
    vwork = torch.empty(b.tq_encode_split_workspace_bytes(b.ROLE_VALUE, d, n_out, 3, GS), dtype=torch.uint8,
                        device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        b.tq_outlier_channels(Kd[s0:s1], d, n_out, chan=kchan, work=work)
        b.tq_encode_split(b.ROLE_KEY, kcbn, kcbo, GS, Kd[s0:s1], d, n_out, 3, kchan, krn, kro, status, work=kwork)
        for (e0, e1), cb, rec in zip(edges, kcb8, krec8):
            b.tq_encode_keys(cb, e1 - e0, Kd[e0:e1], d, 8, d, rec=rec, status=status)
        if ev:
            ev[1].record()
        b.tq_outlier_channels(Vd[s0:s1], d, n_out, chan=vchan, work=work)
        b.tq_encode_split(b.ROLE_VALUE, vcbn, vcbo, GS, Vd[s0:s1], d, n_out, 3, vchan, vrn, vro, status,
                          work=vwork)
        for (e0, e1), cb, rec in zip(edges, vcb8, vrec8):
            b.tq_encode_values(cb, e1 - e0, Vd[e0:e1], d, 8, rec=rec, status=status)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    evs = [_events(torch, 3) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0
    k_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    v_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_step = wall * 1e3 / args.steps
    GB = G - GS
    row = T * d * 2
    cbk = sum(c.numel() for c in kcb8) + kcbn.numel() + kcbo.numel()
    cbv = sum(c.numel() for c in vcb8) + vcbn.numel() + vcbo.numel()
    # algorithmic bytes: boundary layers read once; split layers read twice (variance pass + encode)
    kb = GB * row + 2 * GS * row + GB * T * kw8 * 4 + GS * T * (kwn + kwo) * 4 + cbk
    vb = GB * row + 2 * GS * row + GB * T * vw8 * 4 + GS * T * (vwn + vwo) * 4 + cbv
    return {"metric": "mixed-precision encode GB/s (K and V, 32 layers)", "value": (kb + vb) / (ms_step * 1e-3) / 1e9,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
            "config": {"workload": "mixed-precision layers: 32 layers x 8 kv heads x 16384 tokens, d=256, bf16 "
                                   "with per-channel std log-U[0.5,8]; layers 0,1,30,31 b=8; others b=3 with 32 "
                                   "outlier channels at 4 bits (Walsh-Hadamard) + 224 at 3 bits (Haar)"},
            "encode_keys_ms": k_ms, "encode_keys_GBps": kb / (k_ms * 1e-3) / 1e9,
            "encode_values_ms": v_ms, "encode_values_GBps": vb / (v_ms * 1e-3) / 1e9,
            "roofline": {"bound": "hbm", "achieved": kb / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": kb / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "traffic": _traffic("encode_c5", kb), "kernel": "encode_keys (all layers)"}}


def bench_paged(args, torch, b):
    """Paged decode step at the 32K-context shape: append one token (key and
    value, every kv head of every sequence) into pages of 256 tokens, then score
    32 query heads against the 32768 paged keys of each sequence.  The kernel
    breakdown comes from an eager loop with HIP events; the step time from the
    same step captured in a HIP graph and replayed."""
    from kv_cache_vector_diag_amd import inputs
    dev = "cuda:0"
    B, Hkv, Hq, T, d, kb, vb, m, P, seed = 16, 8, 32, 32768, 128, 3, 3, 128, 256, 3
    G = B * Hkv
    kw = b.tq_record_bytes(d, kb, m, b.ROLE_KEY) // 4
    vw = b.tq_record_bytes(d, vb, 0, b.ROLE_VALUE) // 4
    kcb = b.make_codebooks(Hkv, d, kb, m, seed, b.ROLE_KEY, device=dev)
    vcb = b.make_codebooks(Hkv, d, vb, 0, seed + 1, b.ROLE_VALUE, device=dev)
    max_pages = T // P + 1
    num_pages = B * max_pages
    # pool pages in a shuffled order; the cached keys placed by batch encode (set-up, untimed)
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
    table = perm.view(B, max_pages).to(dev)
    # two pools, alternated, so that the memory-side cache cannot serve one step from the previous
    kpools = [torch.empty((num_pages, Hkv, P, kw), dtype=torch.int32, device=dev) for _ in range(2)]
    vpools = [torch.empty((num_pages, Hkv, P, vw), dtype=torch.int32, device=dev) for _ in range(2)]
    for i in range(2):
        K = inputs.to_torch(inputs.kv_normal(seed + i, G, T, d), "bf16", dev)
        krec = b.tq_encode_keys(kcb, Hkv, K, d, kb, m).view(B, Hkv, T // P, P, kw)
        del K
        kpools[i][table[:, : T // P].reshape(-1).long()] = krec.permute(0, 2, 1, 3, 4).reshape(-1, Hkv, P, kw)
        del krec
    kn = inputs.to_torch(inputs.kv_normal(seed + 5, B, Hkv, d), "bf16", dev).contiguous()
    vn = inputs.to_torch(inputs.kv_normal(seed + 6, B, Hkv, d), "bf16", dev).contiguous()
    pos = torch.full((B,), T, dtype=torch.int32, device=dev)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", dev)
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    work = torch.empty(b.load().tq_append_workspace_bytes(d, kb, vb, m, B, Hkv), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(i, ev=None):
        if ev:
            ev[0].record()
        b.tq_append_kv(kcb, Hkv, vcb, Hkv, kn, vn, d, kb, vb, m, pos, table, P, kpools[i % 2], vpools[i % 2],
                       work=work, status=status)
        if ev:
            ev[1].record()
        b.tq_scores_paged(kcb, Hkv, kpools[i % 2], table, P, T, q, d, kb, m, out=scores, status=status)
        if ev:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    evs = [_events(torch, 3) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0
    ap_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    sc_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_eager = wall * 1e3 / args.steps
    # the step as a decode loop runs it: captured once per pool in a HIP graph
    # and replayed, so the launches cost no host time between kernels
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
        step(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = [torch.cuda.CUDAGraph() for _ in range(2)]
    for i in range(2):
        with torch.cuda.graph(graphs[i]):
            step(i)
    for i in range(args.warmup):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    assert int(status.item()) == 0
    sc_bytes = G * T * kw * 4 + B * Hq * T * 4 + q.numel() * 2 + kcb.numel()
    ap_bytes = G * (2 * d * 2 + (kw + vw) * 4)            # vectors in, records written into their page slots
    return {"metric": "paged decode step tokens/s (append one token per sequence + score the paged 32K context)",
            "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "paged cache: 16 seq x 8 kv heads x 32768 tokens in pages of 256, d=128, turbo3 "
                                   "keys + 3-bit values appended, 32 bf16 query heads scored",
                       "launch": "HIP graph per step (eager launches: ms_per_step_eager)"},
            "ms_per_step_eager": ms_eager,
            "append_us": ap_ms * 1e3, "append_tokens_per_s": G / (ap_ms * 1e-3), "append_bytes": ap_bytes,
            "score_ms": sc_ms,
            "roofline": {"bound": "hbm", "achieved": sc_bytes / (sc_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": sc_bytes / (sc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                         "kernel": "score (paged)", "algorithmic_bytes_per_launch": sc_bytes}}


BF16_MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak


def bench_haar(args, torch, b):
    """Haar-QR rotation (dense R = sqrt(d) Q): encode turbo3 keys + score, d=128,
    on a 4K-context slice of the decode-step shape.  The encode runs the rotation
    R x on bf16 MFMA (R in three exact bf16 terms, fp32 sums) and the projection
    S rho as in the Walsh-Hadamard kernel; the roofline is its algorithmic
    arithmetic (2 d^2 + 2 m d flops per key) against the dense bf16 MFMA peak.
    The score kernel rotates each query by R and is otherwise the Walsh-Hadamard
    one."""
    from kv_cache_vector_diag_amd import inputs
    dev = "cuda:0"
    B, Hkv, Hq, T, d, bits, m, seed = 16, 8, 32, 4096, 128, 3, 128, 3
    G = B * Hkv
    rot = b.ROT_HAAR
    words = b.tq_record_bytes_ex(d, bits, m, b.ROLE_KEY, rot) // 4
    kcb = b.make_codebooks(Hkv, d, bits, m, seed, b.ROLE_KEY, device=dev, rotation=rot)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d), "bf16", dev)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", dev)
    recs = [torch.empty((G, T, words), dtype=torch.int32, device=dev) for _ in range(2)]
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    b.tq_encode_keys(kcb, Hkv, K, d, bits, m, rec=recs[1], status=status, rotation=rot)

    def step(i, ev=None):
        if ev:
            ev[0].record()
        b.tq_encode_keys(kcb, Hkv, K, d, bits, m, rec=recs[i % 2], status=status, rotation=rot)
        if ev:
            ev[1].record()
        b.tq_scores(kcb, Hkv, recs[(i + 1) % 2].view(B, Hkv, T, words), q, d, bits, m, out=scores, rotation=rot)
        if ev:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    evs = [_events(torch, 3) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0
    enc_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    sc_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_step = wall * 1e3 / args.steps
    flops = G * T * (2 * d * d + 2 * m * d)
    tflops = flops / (enc_ms * 1e-3) / 1e12
    enc_bytes = G * T * (d * 2 + words * 4) + kcb.numel()
    sc_bytes = G * T * words * 4 + B * Hq * T * 4
    return {"metric": "Haar-rotation encode + score tokens/s", "value": B * T / (ms_step * 1e-3),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "Haar-QR rotation: 16 seq x 8 kv heads x 4096 tokens, d=128, bf16 N(0,1) "
                                   "keys b=3 (128 projections), 32 query heads"},
            "encode_ms": enc_ms, "encode_GBps": enc_bytes / (enc_ms * 1e-3) / 1e9,
            "encode_keys_per_s": G * T / (enc_ms * 1e-3), "score_ms": sc_ms,
            "score_GBps": sc_bytes / (sc_ms * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": None, "kernel": "encode",
                         "algorithmic_flops_per_launch": flops}}


def bench_gram(args, torch, b):
    """Gram-table scoring of block-codebook codes at the 32K-context decode
    shape: head_dim 128 cut into blocks of 4, a 32-codeword codebook (5-bit
    indices, 24-byte records).  The key cache is encoded once before timing;
    one step = encode the 32 query heads of every sequence + score them against
    the whole cache from the Gram table.  Three record caches rotate so that no
    launch reads what the memory-side cache kept from the previous one."""
    from kv_cache_vector_diag_amd import inputs
    dev = "cuda:0"
    B, Hkv, Hq, T, d, k, N, seed = 16, 8, 32, 32768, 128, 4, 32, 3
    G = B * Hkv
    words = b.tq_gram_record_bytes(d, k, N) // 4
    C = torch.from_numpy(inputs.block_codebook(seed, N, k, d)).to(dev)
    signs = torch.from_numpy(inputs.sign_bits(seed, d).view("int32")).to(dev)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d), "bf16", dev)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    krec = b.tq_gram_encode(C, signs, K, d, status=status)
    recs = [krec.view(B, Hkv, T, words)] + [krec.clone().view(B, Hkv, T, words) for _ in range(2)]
    del K
    table = b.tq_gram_table(C)
    qrec = torch.empty((B, Hq, words), dtype=torch.int32, device=dev)
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    assert int(status.item()) == 0

    def step(i, ev=None):
        b.tq_gram_encode(C, signs, q, d, rec=qrec, status=status)
        if ev:
            ev[0].record()
        b.tq_gram_scores(table, qrec, recs[i % 3], d, k, out=scores)
        if ev:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    evs = [_events(torch, 2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0
    sc_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_eager = wall * 1e3 / args.steps
    # the step captured in a HIP graph per record cache and replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = [torch.cuda.CUDAGraph() for _ in range(3)]
    for i in range(3):
        with torch.cuda.graph(graphs[i]):
            step(i)
    for i in range(args.warmup):
        graphs[i % 3].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % 3].replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    assert int(status.item()) == 0
    sc_bytes = G * T * words * 4 + B * Hq * T * 4 + qrec.numel() * 4 + table.numel() * 4
    sc_gbps = sc_bytes / (sc_ms * 1e-3) / 1e9
    return {"metric": "Gram-table score tokens/s (block-codebook codes, no decode)", "value": B * T / (ms_step * 1e-3),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "Gram-table scoring: 16 seq x 8 kv heads x 32768 tokens, d=128, blocks of 4, "
                                   "32 codewords (24-byte records), 32 bf16 query heads encoded per step",
                       "launch": "HIP graph per step (eager launches: ms_per_step_eager)"},
            "ms_per_step_eager": ms_eager, "score_ms": sc_ms, "score_GBps": sc_gbps, "score_tokens_per_s": B * T / (sc_ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": sc_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": sc_gbps / HBM_PEAK_GBPS, "traffic": _traffic("score_gram", sc_bytes),
                         "kernel": "gram_scores", "algorithmic_bytes_per_launch": sc_bytes}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3", choices=["c2", "c3", "c4", "c5", "haar", "paged", "gram"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path runs on a single MI355X); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from kv_cache_vector_diag_amd import binding as b
    b.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        reps = max(args.steps, 1)
        ev = _events(torch, 2)
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": reps + 1,
                                               "ms_per_copy": ms, "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}}))
        return
    fn = {"c2": bench_c2, "c3": bench_c3, "c4": bench_c4, "c5": bench_c5, "haar": bench_haar,
          "paged": bench_paged, "gram": bench_gram}[args.config]
    line = fn(args, torch, b)
    if args.config == "c3":
        line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_c3()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

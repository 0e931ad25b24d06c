#!/usr/bin/env python3
"""Decode attention over a transform-coded KV cache on one MI355X.

Workload (default): a Qwen2.5-7B-shaped attention layer at 128K context -- 28 q heads,
4 KV heads, d=128, bf16 K/V with Student-t(3) marginals, Walsh-Hadamard rotation,
1.33 bits/elem (170 bits per vector, 12.05x vs bf16).  A step is one decode token through
all 28 layers' attention, each layer reading its own compressed cache (624 MB in total,
above the 256 MB last-level cache, so reads come from HBM).  Inputs are resident in HBM
before the timed region.

Prints one JSON line.  `value` = algorithmic compressed-cache bytes per step / step time.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=4)
    p.add_argument("--layers", type=int, default=0, help="independent layer caches (0 = config default)")
    p.add_argument("--tokens", type=int, default=0, help="override context length")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-dense", action="store_true", help="skip the dense bf16 comparator")
    p.add_argument("--no-tiers", action="store_true", help="skip the tiered-layer measurement")
    p.add_argument("--quiet", action="store_true")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run one plain 256 MiB device copy (scales HBM counters of a profiler run)")
    return p.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def build_layer(cfg, layer, n_tokens, device):
    """Calibrate (host), draw the context on the GPU, encode it; returns (cache, q, host key sample)."""
    import torch
    import synth
    from compressed_decode_attention_head_amd import api
    kb, vb = [], []
    for h in range(cfg.n_kv_heads):
        for t, dst in ((synth.K, kb), (synth.V, vb)):
            cal = synth.draw(cfg.idx, layer, h, t, "calib", cfg.n_calib, dtype=cfg.dtype, marginal=cfg.marginal)
            dst.append(api.calibrate(cal if cfg.dtype == "f32" else synth.bf16_bits(cal), cfg.rotation, cfg.bits_per_elem))
    cap = -(-n_tokens // 64) * 64
    cache = api.CompressedKVCache(kb, vb, cfg.batch, cap, device=device)
    ksample = []
    for t in (synth.K, synth.V):
        x = torch.empty((cfg.batch, cfg.n_kv_heads, n_tokens, 128), dtype=synth.torch_dtype(cfg.dtype),
                        device=device)
        for b in range(cfg.batch):
            for h in range(cfg.n_kv_heads):
                x[b, h] = synth.draw_device(cfg.idx, layer, h, t, n_tokens, dtype=cfg.dtype, marginal=cfg.marginal,
                                            device=device, extra=b)
        cache.encode(t, x)
        if t == synth.K:
            ksample = [x[0, h, :4096].float().cpu().numpy() for h in range(cfg.n_kv_heads)]
        del x
    q = synth.queries(cfg.idx, layer, cfg.n_q_heads, cfg.n_kv_heads, ksample)
    qt = torch.from_numpy(np.broadcast_to(q, (cfg.batch,) + q.shape).copy()).to(device)
    return cache, qt, ksample


KERNEL_SRC = os.path.join(ROOT, "compressed_decode_attention_head_amd", "csrc", "aatc_attn_kernel.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_main_qwen7b_128k_wht133_hbm_traffic.txt")


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(cfg, n_tokens):
    """HBM bytes per launch of the cache pass from the committed counter summary, or None when
    the summary is missing, was taken on another version of the kernel source, or covers
    another workload (it covers the 128K Qwen-shaped layer)."""
    if cfg.idx != 4 or n_tokens != cfg.n_tokens:
        return None
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_bytes(cfg, n_tokens, cache):
    codes = cfg.batch * cfg.n_kv_heads * n_tokens * (cache.k_bits + cache.v_bits) / 8.0
    tables = cfg.n_kv_heads * 2 * (128 * 128 * 4 + 3 * 128 * 4)     # fp32 R_K, R_V + per-channel tables
    qo = cfg.batch * cfg.n_q_heads * 128 * 4 * 2
    return codes, codes + tables + qo


def cpu_baseline(cfg, n_tokens):
    """The oracle on a bounded sample: one KV head's decode attention over a token sample."""
    import oracle as O
    import synth
    sample = min(n_tokens, 16384)
    h = 0
    arts = [O.calibrate(synth.draw(cfg.idx, 0, h, t, "calib", cfg.n_calib, dtype=cfg.dtype, marginal=cfg.marginal),
                        cfg.rotation, cfg.bits_per_elem) for t in (synth.K, synth.V)]
    xs = [synth.draw(cfg.idx, 0, h, t, "context", sample, dtype=cfg.dtype, marginal=cfg.marginal)
          for t in (synth.K, synth.V)]
    codes = [O.encode_codes(xs[i], arts[i]) for i in range(2)]
    q = synth.queries(cfg.idx, 0, cfg.group, 1, [xs[0]])
    t0 = time.perf_counter()
    reps = 0
    while True:
        O.decode_attention(q, [codes[0]], [codes[1]], [arts[0]], [arts[1]])
        reps += 1
        if time.perf_counter() - t0 > 10.0:
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes = sample * (arts[0]["B"] + arts[1]["B"]) / 8.0
    t1 = time.perf_counter()
    for t in range(2):
        O.encode_codes(xs[t], arts[t])
    enc = time.perf_counter() - t1
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": "1 KV head x %d tokens x %d q heads (decode attention = reconstruct + fp64 softmax "
                      "attention), %d reps; encode %.0f tokens/s (K+V, 1 head)" % (sample, cfg.group, reps,
                                                                                 sample / enc)}


def dense_comparator(args, cfg, n_tokens, qs, dev, st, ms_compressed_step):
    """The same decode step over an uncompressed bf16 cache (aatc_decode_attn_dense): one call per
    layer, same queries, timed the same way (graph replay, inputs resident in HBM)."""
    import torch
    import synth
    from compressed_decode_attention_head_amd import api
    lays = []
    for l in range(len(qs)):
        k = torch.empty((cfg.batch, cfg.n_kv_heads, n_tokens, 128), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        for b in range(cfg.batch):
            for h in range(cfg.n_kv_heads):
                k[b, h] = synth.draw_device(cfg.idx, l, h, synth.K, n_tokens, dtype="bf16", marginal=cfg.marginal,
                                            device=dev, extra=b)
                v[b, h] = synth.draw_device(cfg.idx, l, h, synth.V, n_tokens, dtype="bf16", marginal=cfg.marginal,
                                            device=dev, extra=b)
        lays.append((k, v))
    ws = torch.empty(api.decode_attn_dense_workspace_bytes(cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, n_tokens),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(qs[0])
    lse = torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device=dev)

    def dstep():
        for (k, v), q in zip(lays, qs):
            api.decode_attn_dense(k, v, q, n_tokens, workspace=ws, out=out, lse=lse)

    runner = dstep
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(st)
        with torch.cuda.stream(s2):
            dstep()
        st.wait_stream(s2)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            dstep()
        runner = g.replay
    for _ in range(args.warmup):
        runner()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        runner()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    layer_bytes = 2 * cfg.batch * cfg.n_kv_heads * n_tokens * 128 * 2
    gbs = layer_bytes * len(qs) / (ms * 1e-3) / 1e9
    del lays
    return {"kernels": "k_dense_attn + k_merge_states (aatc_decode_attn_dense, one call per layer)",
            "bytes_per_layer": layer_bytes, "ms_per_step": round(ms, 4),
            "us_per_layer": round(ms * 1e3 / len(qs), 3), "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "speedup_compressed_vs_dense": round(ms / ms_compressed_step, 3)}


def tiered_segments(args, dev, st):
    """One decode step over the 128K tiered Llama-shaped layers: token tiers (0 evicted, 2 and 4
    bits coded, 16 raw bf16) from each KV head's Zipf attention mass at the workload's 2.76 bits
    per element on average (the library's solver), tier-2 and tier-4 caches with their own bits
    and the same rotation, one aatc_decode_attn_segments call per layer; graph replay over
    n_layers independent layers.  Bytes are the compressed codes and raw rows the call reads."""
    import torch
    import synth
    from compressed_decode_attention_head_amd import api
    cfg = synth.CONFIGS[5]
    n, n_kv, n_q, n_layers = cfg.n_tokens, cfg.n_kv_heads, cfg.n_q_heads, cfg.n_layers
    K, V = synth.K, synth.V
    calls, keep = [], []
    total_bytes, pop = 0, {0: 0, 2: 0, 4: 0, 16: 0}
    for l in range(n_layers):
        blobs = {(tau, t): [api.calibrate(synth.bf16_bits(synth.draw(cfg.idx, l, h, t, "calib", cfg.n_calib)), "klt",
                                          float(tau)) for h in range(n_kv)] for tau in (2, 4) for t in (K, V)}
        tiers = []
        for h in range(n_kv):
            s2 = [api.calib_view(blobs[(2, t)][h])["sigma2"] for t in (K, V)]
            tiers.append(api.token_tiers(synth.zipf_mass(cfg.idx, l, h, n), api.tier_distortions(s2),
                                         cfg.bits_per_elem))
        ctx = {t: [synth.draw_device(cfg.idx, l, h, t, n, device=dev) for h in range(n_kv)] for t in (K, V)}
        ksample = [ctx[K][h][:4096].float().cpu().numpy() for h in range(n_kv)]
        segs = []
        for tau in (0, 2, 4, 16):
            pop[tau] += int(sum((tr == tau).sum() for tr in tiers))
        for tau in (2, 4, 16):
            idx = [torch.from_numpy(np.nonzero(tiers[h] == tau)[0]).to(dev) for h in range(n_kv)]
            counts = [int(i.numel()) for i in idx]
            cap = max(64, -(-max(counts) // 64) * 64)
            sl = torch.tensor([counts], dtype=torch.int32, device=dev)
            xt = {}
            for t in (K, V):
                xt[t] = torch.zeros((1, n_kv, cap, 128), dtype=torch.bfloat16, device=dev)
                for h in range(n_kv):
                    xt[t][0, h, :counts[h]] = ctx[t][h].index_select(0, idx[h])
            if tau == 16:
                segs.append({"k_raw": xt[K], "v_raw": xt[V], "seq_lens": sl, "max_seq_len": max(counts)})
                keep += [xt[K], xt[V], sl]
                total_bytes += sum(counts) * 2 * 128 * 2
            else:
                cache = api.CompressedKVCache(blobs[(tau, K)], blobs[(tau, V)], 1, cap, device=dev)
                for t in (K, V):
                    cache.encode(t, xt[t])
                segs.append({"cache": cache, "seq_lens": sl, "max_seq_len": max(counts)})
                keep += [cache, sl]
                total_bytes += sum(counts) * (cache.k_bits + cache.v_bits) // 8
                del xt
        del ctx
        q = torch.from_numpy(synth.queries(cfg.idx, l, n_q, n_kv, ksample)[None]).to(dev)
        ws = torch.empty(api.decode_attn_segments_workspace_bytes(segs, 1, n_kv, n_q), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty((1, n_q), dtype=torch.float32, device=dev)
        calls.append((segs, q, ws, out, lse))
    torch.cuda.synchronize()

    def tstep():
        for segs, q, ws, out, lse in calls:
            api.decode_attn_segments(segs, q, 1, n_kv, workspace=ws, out=out, lse=lse)

    runner = tstep
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(st)
        with torch.cuda.stream(s2):
            tstep()
        st.wait_stream(s2)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            tstep()
        runner = g.replay
    for _ in range(args.warmup):
        runner()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        runner()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tot = sum(pop.values())
    return {"workload": cfg.name, "layers_per_step": n_layers, "avg_bits": cfg.bits_per_elem,
            "tier_fractions": {str(t): round(pop[t] / tot, 4) for t in (0, 2, 4, 16)},
            "bytes_per_step": total_bytes, "ms_per_step": round(ms, 4),
            "us_per_layer": round(ms * 1e3 / n_layers, 3), "gbs": round(total_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "calls": "aatc_decode_attn_segments: cache pass + merge per coded tier, dense pass for raw, "
                     "one state merge"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        sys.exit(1)
    cfg = synth.CONFIGS[args.config]
    n_tokens = args.tokens or cfg.n_tokens
    n_layers = args.layers or cfg.n_layers
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(args, "building %d layers of %s, %d tokens" % (n_layers, cfg.name, n_tokens))
    layers = []
    for l in range(n_layers):
        cache, q, _ = build_layer(cfg, l, n_tokens, dev)
        ws = cache.new_workspace(cfg.n_q_heads, n_tokens)
        out = torch.empty_like(q)
        lse = torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device=dev)
        layers.append((cache, q, ws, out, lse))
        log(args, "layer %d ready" % l)
    torch.cuda.synchronize()
    codes_b, alg_b = algorithmic_bytes(cfg, n_tokens, layers[0][0])

    def step():
        for cache, q, ws, out, lse in layers:
            cache.decode_attn(q, n_tokens, workspace=ws, out=out, lse=lse)

    # --- per-call durations (eager, HIP events on the launch stream)
    st = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
    call_ms = []
    for _ in range(max(3, args.steps // 4)):
        for (e0, e1), (cache, q, ws, out, lse) in zip(evs, layers):
            e0.record(st)
            cache.decode_attn(q, n_tokens, workspace=ws, out=out, lse=lse)
            e1.record(st)
        torch.cuda.synchronize()
        call_ms += [e0.elapsed_time(e1) for e0, e1 in evs]
    call_ms = float(np.mean(call_ms))
    log(args, "decode_attn call: %.2f us per layer" % (call_ms * 1e3))

    # --- timed steps (graph replay of the whole step unless --no-graph)
    runner = step
    graph_used = False
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            s2 = torch.cuda.Stream()
            s2.wait_stream(st)
            with torch.cuda.stream(s2):
                step()
            st.wait_stream(s2)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step()
            runner = g.replay
            graph_used = True
        except Exception as e:  # pragma: no cover
            log(args, "graph capture failed (%s); timing eager launches" % e)
    for _ in range(args.warmup):
        runner()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        runner()
    e1.record(st)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    gbs = codes_b * n_layers / (ms_step * 1e-3) / 1e9

    # --- encode throughput (prefill of one layer: all heads, K and V)
    cache0 = layers[0][0]
    x = torch.empty((cfg.batch, cfg.n_kv_heads, n_tokens, 128), dtype=synth.torch_dtype(cfg.dtype), device=dev)
    for h in range(cfg.n_kv_heads):
        x[0, h] = synth.draw_device(cfg.idx, 0, h, synth.K, n_tokens, dtype=cfg.dtype, marginal=cfg.marginal,
                                    device=dev)
    cache0.encode(0, x)
    torch.cuda.synchronize()
    ee0, ee1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    ee0.record(st)
    for _ in range(reps):
        cache0.encode(0, x)
        cache0.encode(1, x)
    ee1.record(st)
    torch.cuda.synchronize()
    enc_ms = ee0.elapsed_time(ee1) / reps
    enc_tok_s = n_tokens * cfg.batch / (enc_ms * 1e-3)
    del x

    # --- the dominant kernel alone: the cache pass (aatc_decode_attn_partial -> k_attn_main),
    # HIP events around each launch on the stream it runs on; then the merge kernel the same way
    def time_each(fn):
        for cache, q, ws, out, lse in layers:
            fn(cache, q, ws, out, lse)
        torch.cuda.synchronize()
        ms = []
        for _ in range(max(3, args.steps // 4)):
            for (e0, e1), lay in zip(evs, layers):
                e0.record(st)
                fn(*lay)
                e1.record(st)
            torch.cuda.synchronize()
            ms += [e0.elapsed_time(e1) for e0, e1 in evs]
        return float(np.mean(ms))

    def time_graph(fn):
        # one launch per layer captured back to back in a graph, replayed between events: the
        # average launch duration without per-launch event and host overheads
        if not graph_used:
            return None
        g2 = torch.cuda.CUDAGraph()
        s3 = torch.cuda.Stream()
        s3.wait_stream(st)
        with torch.cuda.stream(s3):
            for lay in layers:
                fn(*lay)
        st.wait_stream(s3)
        torch.cuda.synchronize()
        with torch.cuda.graph(g2):
            for lay in layers:
                fn(*lay)
        g2.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(5, args.steps)
        e0.record(st)
        for _ in range(reps):
            g2.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(layers))

    part_fn = lambda cache, q, ws, out, lse: cache.decode_attn_partial(q, n_tokens, ws)
    merge_fn = lambda cache, q, ws, out, lse: cache.decode_attn_merge(q.shape[1], n_tokens, ws, out, lse)
    part_eager_ms = time_each(part_fn)
    merge_eager_ms = time_each(merge_fn)
    part_graph_ms = time_graph(part_fn)
    merge_graph_ms = time_graph(merge_fn)
    part_ms = part_graph_ms if part_graph_ms is not None else part_eager_ms
    merge_ms = merge_graph_ms if merge_graph_ms is not None else merge_eager_ms
    log(args, "cache pass %.2f us, merge %.2f us per layer (%s); eager with an event pair per launch: %.2f, %.2f us" % (
        part_ms * 1e3, merge_ms * 1e3, "graph of back-to-back launches" if part_graph_ms is not None else "eager",
        part_eager_ms * 1e3, merge_eager_ms * 1e3))
    achieved = codes_b / (part_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg, n_tokens)
    if args.copy_calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res = {
        "metric": "decode-attn compressed-KV GB/s & % HBM peak at 128K ctx; encode tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8-mfma/fp32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers_per_step": n_layers, "batch": cfg.batch,
                   "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads, "context": n_tokens,
                   "rotation": cfg.rotation, "bits_per_elem": cfg.bits_per_elem,
                   "k_bits": cache0.k_bits, "v_bits": cache0.v_bits,
                   "compression_vs_bf16": round(16 * 128 * 2 / (cache0.k_bits + cache0.v_bits), 3),
                   "graph": graph_used},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "encode_tokens_per_s": round(enc_tok_s, 1),
        "encode_note": "one layer prefill, all KV heads, K and V, fp64 rotation+quantize",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_attn_main (the cache pass, one launch per layer)",
                     "bytes_per_launch": codes_b, "launch_us": round(part_ms * 1e3, 3),
                     "launch_timing": "graph of back-to-back launches" if part_graph_ms is not None else "eager events",
                     "launch_us_eager_events": round(part_eager_ms * 1e3, 3),
                     "merge_kernel_us": round(merge_ms * 1e3, 3), "call_us": round(call_ms * 1e3, 3)},
    }
    if not args.no_dense:
        log(args, "timing the dense bf16 comparator")
        res["dense_bf16"] = dense_comparator(args, cfg, n_tokens, [lay[1] for lay in layers], dev, st, ms_step)
        log(args, "dense bf16: %.2f us per layer, %.0f GB/s; compressed step is %.2fx faster" % (
            res["dense_bf16"]["us_per_layer"], res["dense_bf16"]["gbs"], res["dense_bf16"]["speedup_compressed_vs_dense"]))
    if not args.no_tiers:
        log(args, "timing the tiered 128K layer")
        res["tiers"] = tiered_segments(args, dev, st)
        log(args, "tiers: %.2f us per layer, %.0f GB/s, tier fractions %s" % (
            res["tiers"]["us_per_layer"], res["tiers"]["gbs"], res["tiers"]["tier_fractions"]))
    if not args.no_cpu_baseline:
        log(args, "timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(cfg, n_tokens)
    print(json.dumps(res))


if __name__ == "__main__":
    main()

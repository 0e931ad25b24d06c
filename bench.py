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
FP64_PEAK_TFLOPS = 78.6


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
    p.add_argument("--no-encode", action="store_true", help="skip the encode rooflines")
    p.add_argument("--no-folded", action="store_true", help="skip the folded all-layers launch")
    p.add_argument("--no-loops", action="store_true", help="skip the append + decode loops")
    p.add_argument("--no-lloyd-max", action="store_true", help="skip the Lloyd-Max caches")
    p.add_argument("--only-headline", action="store_true", help="headline step and roofline only")
    p.add_argument("--only", choices=["encode", "lloyd-max", "append-loop"], default=None,
                   help="one side measurement alone (its JSON object only), for profiling")
    return p.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def build_layer(cfg, layer, n_tokens, device, capacity=None, quantizer="uniform", heads=None, batch=None):
    """Calibrate (host), draw the context on the GPU, encode it; returns (cache, q, host key sample)."""
    import torch
    import synth
    from compressed_decode_attention_head_amd import api
    from dataclasses import replace
    if heads is not None or batch is not None:
        cfg = replace(cfg, n_kv_heads=heads or cfg.n_kv_heads, batch=batch or cfg.batch,
                      n_q_heads=(heads or cfg.n_kv_heads) * cfg.group)
    kb, vb = [], []
    for h in range(cfg.n_kv_heads):
        for t, dst in ((synth.K, kb), (synth.V, vb)):
            cal = synth.draw(cfg.idx, layer, h, t, "calib", cfg.n_calib, dtype=cfg.dtype, marginal=cfg.marginal)
            dst.append(api.calibrate(cal if cfg.dtype == "f32" else synth.bf16_bits(cal), cfg.rotation, cfg.bits_per_elem,
                                     quantizer=quantizer))
    cap = -(-max(n_tokens, capacity or 0) // 64) * 64
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count()


# token samples of the oracle per workload: about 3-5 s of host work each
CPU_SAMPLE = {1: 4096, 2: 8192, 3: 8192, 4: 16384}


def cpu_baseline_config(idx, min_s=2.0):
    """The oracle on one KV head of one workload: calibrate (K and V), encode a token sample (K and
    V), and decode attention of the head's q-head group over the sample, repeated for min_s."""
    import oracle as O
    import synth
    cfg = synth.CONFIGS[idx]
    sample = min(cfg.n_tokens, CPU_SAMPLE[idx])
    cals = [synth.draw(cfg.idx, 0, 0, t, "calib", cfg.n_calib, dtype=cfg.dtype, marginal=cfg.marginal)
            for t in (synth.K, synth.V)]
    t0 = time.perf_counter()
    arts = [O.calibrate(c, cfg.rotation, cfg.bits_per_elem) for c in cals]
    cal_s = (time.perf_counter() - t0) / 2
    xs = [synth.draw(cfg.idx, 0, 0, t, "context", sample, dtype=cfg.dtype, marginal=cfg.marginal)
          for t in (synth.K, synth.V)]
    t0 = time.perf_counter()
    codes = [O.encode_codes(xs[i], arts[i]) for i in range(2)]
    enc_s = time.perf_counter() - t0
    q = synth.queries(cfg.idx, 0, cfg.group, 1, [xs[0]])
    t0 = time.perf_counter()
    reps = 0
    while True:
        O.decode_attention(q, [codes[0]], [codes[1]], [arts[0]], [arts[1]])
        reps += 1
        if time.perf_counter() - t0 > min_s:
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes = sample * (arts[0]["B"] + arts[1]["B"]) / 8.0
    return {"workload": cfg.name, "sample": "1 KV head x %d tokens x %d q heads" % (sample, cfg.group),
            "calibrate_s_per_tensor": round(cal_s, 4),
            "encode_tokens_per_s": round(sample / enc_s, 1),
            "decode_attn_s": round(dt, 5), "decode_attn_gbs": round(nbytes / dt / 1e9, 5), "reps": reps}


def cpu_baseline(cfg, n_tokens):
    """The oracle as it stands on the host cores: the headline workload's decode attention in the
    metric's unit, plus calibrate / encode / decode figures for each of the four workloads."""
    per = {str(i): cpu_baseline_config(i) for i in (1, 2, 3, 4)}
    head = per[str(cfg.idx)] if str(cfg.idx) in per else per["4"]
    return {"value": head["decode_attn_gbs"], "unit": "GB/s", "cores": oracle_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%s: %s (decode attention = reconstruct + fp64 softmax attention; the same "
                      "algorithmic compressed bytes per second as the GPU figure)" % (head["workload"], head["sample"]),
            "per_workload": per}


def gpu_info():
    """Device name and the shader / memory clocks rocm-smi reports (None where unavailable)."""
    import re
    import subprocess
    import torch
    info = {"name": torch.cuda.get_device_name(0), "sclk_mhz": None, "mclk_mhz": None}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        for line in r.stdout.splitlines():
            m = re.search(r"(sclk|mclk) clock level: \d+: \((\d+)Mhz\)", line)
            if m and info[m.group(1) + "_mhz"] is None:
                info[m.group(1) + "_mhz"] = int(m.group(2))
    except Exception:  # pragma: no cover
        pass
    return info


USE_GRAPHS = True


def timed_graph(fn, reps, st):
    """Capture fn() in a graph, replay it reps times between HIP events on stream st; returns ms
    per replay (the launches back to back, without host overheads).  With --no-graph: eager
    calls between the events."""
    import torch
    if not USE_GRAPHS:
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    g = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    s2.wait_stream(st)
    with torch.cuda.stream(s2):
        fn()
    st.wait_stream(s2)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def read_probe(dev, st, nbytes=1 << 30, reps=20):
    """Plain streaming read of a 1 GiB buffer (aatc_probe_read): the read bandwidth this GPU
    delivers to a kernel that does nothing else."""
    import torch
    from compressed_decode_attention_head_amd import api
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(2048 * 16, dtype=torch.uint8, device=dev)
    ms = timed_graph(lambda: api.probe_read(buf, sink), reps, st)
    del buf
    return {"kernel": "k_read_probe (aatc_probe_read: 16-byte non-temporal loads, nothing else)",
            "bytes": nbytes, "us": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def cold_layer_latency(dev, st, cache, q, n_tokens, ws, out, lse, reps=7):
    """One layer's decode step (aatc_decode_attn: cache pass + merge) right after writing 512 MB of
    other memory, so that neither the cache nor the tables sit in the last-level cache; the median
    of reps, with an event pair around the call on its stream."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ms = []
    for r in range(reps):
        flush.fill_(r & 255)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        cache.decode_attn(q, n_tokens, workspace=ws, out=out, lse=lse)
        e1.record(st)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del flush
    return float(np.median(ms))


def encode_rooflines(args, dev, st):
    """Encode (aatc_encode: rotate, quantize, pack) against its roofline, inputs above the 256 MB
    last-level cache: four independent 128K-token layers' keys (4 x 134 MB of bf16) of the
    Walsh-Hadamard 1.33-bit workload against HBM bandwidth, and four 32K-token layers' keys
    (4 x 67 MB) of the KLT 2.76-bit workload against the fp64 peak (2 d^2 flops per vector)."""
    import torch
    import synth
    from compressed_decode_attention_head_amd import api
    res = {}
    for idx, n_lay in ((4, 4), (2, 4)):
        cfg = synth.CONFIGS[idx]
        n = cfg.n_tokens
        caches, xs = [], []
        for l in range(n_lay):
            kb, vb = [], []
            for h in range(cfg.n_kv_heads):
                for t, dst in ((synth.K, kb), (synth.V, vb)):
                    cal = synth.draw(cfg.idx, l, h, t, "calib", cfg.n_calib, dtype=cfg.dtype, marginal=cfg.marginal)
                    dst.append(api.calibrate(synth.bf16_bits(cal), cfg.rotation, cfg.bits_per_elem))
            caches.append(api.CompressedKVCache(kb, vb, 1, n, device=dev))
            x = torch.empty((1, cfg.n_kv_heads, n, 128), dtype=torch.bfloat16, device=dev)
            for h in range(cfg.n_kv_heads):
                x[0, h] = synth.draw_device(cfg.idx, l, h, synth.K, n, dtype="bf16", marginal=cfg.marginal, device=dev)
            xs.append(x)
        torch.cuda.synchronize()

        def enc():
            for c, x in zip(caches, xs):
                c.encode(synth.K, x)

        ms = timed_graph(enc, max(3, args.steps // 4), st) / n_lay
        vectors = cfg.n_kv_heads * n
        kbits = caches[0].k_bits
        nbytes = vectors * (128 * 2 + kbits / 8.0)
        flops = vectors * 2.0 * 128 * 128
        ent = {"workload": cfg.name, "rotation": cfg.rotation, "kernel": "k_encode",
               "vectors_per_launch": vectors, "us_per_launch": round(ms * 1e3, 2),
               "vectors_per_s": round(vectors / (ms * 1e-3), 1),
               "tokens_per_s_k_and_v": round(n / (ms * 1e-3) / 2, 1),
               "bytes_per_launch": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "layers_cycled": n_lay, "input_mb_cycled": round(n_lay * vectors * 256 / 1e6, 1)}
        if cfg.rotation == "wht":
            ent["roofline"] = {"bound": "hbm", "achieved": ent["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(ent["gbs"] / HBM_PEAK_GBS, 4)}
        else:
            tf = flops / (ms * 1e-3) / 1e12
            ent["roofline"] = {"bound": "fp64", "achieved": round(tf, 2), "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(tf / FP64_PEAK_TFLOPS, 4), "flops_per_launch": flops}
        res[cfg.rotation] = ent
        del caches, xs
        torch.cuda.synchronize()
    return res


def folded_launch(args, cfg, layers, dev, st, n_tokens):
    """Every layer's cache in one launch: the 28 layers' KV heads folded into the head axis of a
    single cache (112 KV heads, 784 q heads), so one cache pass streams all 624 MB.  The queries of
    different layers are not available together during real decoding; this separates the
    stream rate of the pass from the fixed costs of a launch."""
    import torch
    from compressed_decode_attention_head_amd import api
    kb = [b for lay in layers for b in lay[0].k_blobs_host]
    vb = [b for lay in layers for b in lay[0].v_blobs_host]
    big = api.CompressedKVCache(kb, vb, cfg.batch, layers[0][0].capacity, device=dev)
    kw = layers[0][0].k_codes.numel() - 4
    vw = layers[0][0].v_codes.numel() - 4
    for l, lay in enumerate(layers):
        big.k_codes[l * kw:(l + 1) * kw].copy_(lay[0].k_codes[:kw])
        big.v_codes[l * vw:(l + 1) * vw].copy_(lay[0].v_codes[:vw])
    q = torch.cat([lay[1] for lay in layers], dim=1).contiguous()
    ws = big.new_workspace(q.shape[1], n_tokens)
    out = torch.empty_like(q)
    lse = torch.empty((cfg.batch, q.shape[1]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    # the folded call gives every layer's result of the per-layer calls (up to the order of the
    # split merge, which depends on the number of splits)
    ref = []
    for lay in layers:
        o, _ = lay[0].decode_attn(lay[1], n_tokens)
        ref.append(o)
    big.decode_attn(q, n_tokens, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    diff = float((torch.cat(ref, dim=1) - out).abs().max())
    reps = max(5, args.steps)
    part = timed_graph(lambda: big.decode_attn_partial(q, n_tokens, ws), reps, st)
    call = timed_graph(lambda: big.decode_attn(q, n_tokens, workspace=ws, out=out, lse=lse), reps, st)
    nbytes = len(layers) * cfg.batch * cfg.n_kv_heads * n_tokens * (big.k_bits + big.v_bits) / 8.0
    del big
    return {"layers_folded": len(layers), "kv_heads": len(kb), "q_heads": int(q.shape[1]),
            "bytes_per_launch": nbytes, "cache_pass_us": round(part * 1e3, 2), "call_us": round(call * 1e3, 2),
            "cache_pass_gbs": round(nbytes / (part * 1e-3) / 1e9, 1),
            "cache_pass_frac_of_peak": round(nbytes / (part * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "call_gbs": round(nbytes / (call * 1e-3) / 1e9, 1),
            "max_abs_diff_vs_per_layer_calls": diff}


def append_decode_loop(args, dev, st):
    """The batch-16 workload as a decode loop: 4 layers of 16 sequences x 8 KV heads with 8192
    prefill tokens (KLT, 4 bits per element), then 64 steps; each step appends one encoded K and V
    token per sequence and head to every layer (aatc_encode_kv at the next offset) and runs every
    layer's decode attention over the grown cache.  Eager launches, timed with HIP events."""
    import torch
    import synth
    cfg = synth.CONFIGS[3]
    steps, n0 = cfg.decode_steps, cfg.n_tokens
    cap = n0 + steps
    lays = []
    for l in range(cfg.n_layers):
        cache, q, _ = build_layer(cfg, l, n0, dev, capacity=cap)
        new = {}
        for t in (synth.K, synth.V):
            x = torch.empty((cfg.batch, cfg.n_kv_heads, steps, 128), dtype=torch.bfloat16, device=dev)
            for b in range(cfg.batch):
                for h in range(cfg.n_kv_heads):
                    x[b, h] = synth.draw_device(cfg.idx, l, h, t, steps, dtype="bf16", device=dev, extra=1000 + b)
            new[t] = x
        ws = cache.new_workspace(cfg.n_q_heads, cap)
        out = torch.empty_like(q)
        lse = torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device=dev)
        lays.append((cache, q, new, ws, out, lse))
    torch.cuda.synchronize()

    def run(s):
        for cache, q, new, ws, out, lse in lays:
            cache.encode_kv(new[synth.K][:, :, s:s + 1], new[synth.V][:, :, s:s + 1], token_offset=n0 + s)
            cache.decode_attn(q, n0 + s + 1, workspace=ws, out=out, lse=lse)

    run(0)                                         # warm: the first step's encode rewrites the same token
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for s_ in range(steps):
        run(s_)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the appends alone (the same tokens written again: encoding is idempotent)
    e0.record(st)
    for s_ in range(steps):
        for cache, q, new, ws, out, lse in lays:
            cache.encode_kv(new[synth.K][:, :, s_:s_ + 1], new[synth.V][:, :, s_:s_ + 1], token_offset=n0 + s_)
    e1.record(st)
    torch.cuda.synchronize()
    ms_enc = e0.elapsed_time(e1) / steps
    kb, vb = lays[0][0].k_bits, lays[0][0].v_bits
    avg_tokens = n0 + (steps + 1) / 2.0
    nbytes = cfg.n_layers * cfg.batch * cfg.n_kv_heads * avg_tokens * (kb + vb) / 8.0
    del lays
    return {"workload": cfg.name, "layers": cfg.n_layers, "steps": steps, "prefill_tokens": n0,
            "ms_per_step": round(ms, 4), "us_per_layer_step": round(ms * 1e3 / cfg.n_layers, 2),
            "append_us_per_layer_step": round(ms_enc * 1e3 / cfg.n_layers, 2),
            "decode_tokens_per_s": round(cfg.batch * 1e3 / ms, 1),
            "cache_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "calls_per_layer_step": "aatc_encode_kv (K and V, 1 token per sequence and head) + aatc_decode_attn",
            "timing": "eager launches, HIP events around all steps"}


def lloyd_max_pass(args, dev, st):
    """Lloyd-Max caches (K and V) of the 32K-token 2.76-bit layer (12 layers, 277 MB) and of the
    batch-16 x 8K 4-bit layer (4 layers, 537 MB): one aatc_decode_attn per layer (the level pass
    k_attn_lm + the merge), graph replay over the layers, beside the reconstruction MSE of the
    same context under the uniform and the Lloyd-Max quantizer (aatc_decode on the GPU, one head)."""
    import torch
    import synth
    res = {}
    for idx, n_lay in ((2, 12), (3, 4)):
        cfg = synth.CONFIGS[idx]
        n = cfg.n_tokens
        lays = []
        for l in range(n_lay):
            cache, q, _ = build_layer(cfg, l, n, dev, quantizer="lloyd-max")
            ws = cache.new_workspace(cfg.n_q_heads, n)
            lays.append((cache, q, ws, torch.empty_like(q),
                         torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        reps = max(5, args.steps)
        ms = timed_graph(lambda: [c.decode_attn(q, n, workspace=w, out=o, lse=e) for c, q, w, o, e in lays], reps, st)
        part = timed_graph(lambda: [c.decode_attn_partial(q, n, w) for c, q, w, o, e in lays], reps, st)
        kb, vb = lays[0][0].k_bits, lays[0][0].v_bits
        nbytes = cfg.batch * cfg.n_kv_heads * n * (kb + vb) / 8.0
        # reconstruction error of head 0's keys, both quantizers, same context
        mse = {}
        x = torch.empty((1, 1, n, 128), dtype=torch.bfloat16, device=dev)
        x[0, 0] = synth.draw_device(cfg.idx, 0, 0, synth.K, n, dtype="bf16", device=dev)
        for qz in ("uniform", "lloyd-max"):
            c1, _, _ = build_layer(cfg, 0, 64, dev, quantizer=qz, heads=1, batch=1, capacity=n)
            c1.encode(synth.K, x)
            xh = c1.decode(synth.K, 0, n)
            mse[qz] = float(((xh.float() - x.float()) ** 2).mean())
        res["config%d" % idx] = {
            "workload": cfg.name, "layers": n_lay, "kernel": "k_attn_lm (level pass) + k_attn_combine",
            "bytes_per_layer": nbytes, "us_per_layer": round(ms * 1e3 / n_lay, 2),
            "cache_pass_us": round(part * 1e3 / n_lay, 2),
            "cache_pass_gbs": round(nbytes / (part * 1e-3 / n_lay) / 1e9, 1),
            "cache_pass_frac_of_peak": round(nbytes / (part * 1e-3 / n_lay) / 1e9 / HBM_PEAK_GBS, 4),
            "step_gbs": round(nbytes / (ms * 1e-3 / n_lay) / 1e9, 1),
            "key_reconstruction_mse": {"uniform": mse["uniform"], "lloyd-max": mse["lloyd-max"],
                                       "reduction": round(1 - mse["lloyd-max"] / mse["uniform"], 4)}}
        del lays
        torch.cuda.synchronize()
    return res


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
    calls, keep, raws = [], [], []
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
            # the raw tier has room for the tokens the decode loop appends
            cap = max(64, -(-(max(counts) + (cfg.decode_steps if tau == 16 else 0)) // 64) * 64)
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
                raw = (xt[K], xt[V], counts)
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
        raws.append(raw)
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
    res = {"workload": cfg.name, "layers_per_step": n_layers, "avg_bits": cfg.bits_per_elem,
           "tier_fractions": {str(t): round(pop[t] / tot, 4) for t in (0, 2, 4, 16)},
           "bytes_per_step": total_bytes, "ms_per_step": round(ms, 4),
           "us_per_layer": round(ms * 1e3 / n_layers, 3), "gbs": round(total_bytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_peak": round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "calls": "aatc_decode_attn_segments: cache pass + merge per coded tier, dense pass for raw, "
                    "one state merge"}
    if not args.no_loops:
        res["decode_loop"] = tiered_append_loop(cfg, calls, raws, dev, st)
    return res


def tiered_append_loop(cfg, calls, raws, dev, st):
    """The tiered workload's decode loop: 256 steps, each appending one token per KV head to every
    layer's raw bf16 tier (tokens after prefill are kept at full precision) and running every
    layer's multi-segment decode attention over the grown raw tier.  Eager launches, HIP events."""
    import torch
    import synth
    from compressed_decode_attention_head_amd import api
    steps = cfg.decode_steps
    n_kv, n_q = cfg.n_kv_heads, cfg.n_q_heads
    loop = []
    for l, ((segs, q, ws, out, lse), (rk, rv, counts)) in enumerate(zip(calls, raws)):
        sl = torch.tensor([counts], dtype=torch.int32, device=dev)
        segs2 = [dict(sg) for sg in segs]
        segs2[-1]["seq_lens"] = sl                 # the raw tier is the last segment
        segs2[-1]["max_seq_len"] = max(counts) + steps
        ws2 = torch.empty(api.decode_attn_segments_workspace_bytes(segs2, 1, n_kv, n_q), dtype=torch.uint8,
                          device=dev)
        new = [torch.stack([synth.draw_device(cfg.idx, l, h, t, steps, device=dev, extra=2000) for h in range(n_kv)])
               for t in (synth.K, synth.V)]      # [n_kv, steps, 128] each
        base = torch.tensor(counts, dtype=torch.int64, device=dev)
        loop.append((segs2, q, ws2, out, lse, rk, rv, new, base, sl))
    heads = torch.arange(n_kv, device=dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for s_ in range(steps):
        for segs2, q, ws2, out, lse, rk, rv, new, base, sl in loop:
            pos = base + s_
            rk[0, heads, pos] = new[0][:, s_]
            rv[0, heads, pos] = new[1][:, s_]
            sl += 1
            api.decode_attn_segments(segs2, q, 1, n_kv, workspace=ws2, out=out, lse=lse)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"steps": steps, "layers": len(loop), "ms_per_step": round(ms, 4),
            "us_per_layer_step": round(ms * 1e3 / len(loop), 2), "decode_tokens_per_s": round(1e3 / ms, 1),
            "calls_per_layer_step": "2 row writes into the raw tier, a length increment, aatc_decode_attn_segments",
            "timing": "eager launches, HIP events around all steps"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        sys.exit(1)
    global USE_GRAPHS
    USE_GRAPHS = not args.no_graph
    if args.only:
        dev = torch.device("cuda", 0)
        torch.cuda.set_device(dev)
        st = torch.cuda.current_stream()
        part = {"encode": encode_rooflines, "lloyd-max": lloyd_max_pass,
                "append-loop": append_decode_loop}[args.only](args, dev, st)
        print(json.dumps({"only": args.only, "result": part}))
        return
    if args.only_headline:
        args.no_dense = args.no_tiers = args.no_cpu_baseline = args.no_encode = args.no_folded = args.no_loops = True
        args.no_lloyd_max = True
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
    log(args, "%d layers ready" % n_layers)
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

    # --- timed steps (graph replay of the whole step unless --no-graph), an event per step
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
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record(st)
    for i in range(args.steps):
        runner()
        marks[i + 1].record(st)
    torch.cuda.synchronize()
    ms_step = marks[0].elapsed_time(marks[-1]) / args.steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    gbs = codes_b * n_layers / (ms_step * 1e-3) / 1e9

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
        return timed_graph(lambda: [fn(*lay) for lay in layers], max(5, args.steps), st) / len(layers)

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
    c0, q0, ws0, out0, lse0 = layers[0]
    cold_ms = cold_layer_latency(dev, st, c0, q0, n_tokens, ws0, out0, lse0)
    probe = read_probe(dev, st)
    log(args, "cold layer %.2f us; read probe %.0f GB/s" % (cold_ms * 1e3, probe["gbs"]))
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
                   "k_bits": layers[0][0].k_bits, "v_bits": layers[0][0].v_bits,
                   "compression_vs_bf16": round(16 * 128 * 2 / (layers[0][0].k_bits + layers[0][0].v_bits), 3),
                   "graph": graph_used},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "step_ms_percentiles": {"p10": round(float(np.percentile(per_step, 10)), 4),
                                "p50": round(float(np.percentile(per_step, 50)), 4),
                                "p90": round(float(np.percentile(per_step, 90)), 4)},
        "cold_layer_us": round(cold_ms * 1e3, 2),
        "cold_layer_note": "one layer's aatc_decode_attn right after a 512 MB write (median of 7)",
        "read_probe": probe,
        "pct_of_read_probe": round(100.0 * gbs / probe["gbs"], 2),
        "gpu": gpu_info(),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "frac_of_read_probe": round(achieved / probe["gbs"], 4),
                     "kernel": "k_attn_main (the cache pass, one launch per layer)",
                     "bytes_per_launch": codes_b, "launch_us": round(part_ms * 1e3, 3),
                     "launch_timing": "graph of back-to-back launches" if part_graph_ms is not None else "eager events",
                     "launch_us_eager_events": round(part_eager_ms * 1e3, 3),
                     "merge_kernel_us": round(merge_ms * 1e3, 3), "call_us": round(call_ms * 1e3, 3)},
    }
    if not args.no_folded and cfg.batch == 1:
        log(args, "timing the folded all-layers launch")
        res["folded_layers"] = folded_launch(args, cfg, layers, dev, st, n_tokens)
        log(args, "folded: %.1f us, %.0f GB/s cache pass" % (res["folded_layers"]["cache_pass_us"],
                                                           res["folded_layers"]["cache_pass_gbs"]))
    if not args.no_dense:
        log(args, "timing the dense bf16 comparator")
        res["dense_bf16"] = dense_comparator(args, cfg, n_tokens, [lay[1] for lay in layers], dev, st, ms_step)
        log(args, "dense bf16: %.2f us per layer, %.0f GB/s; compressed step is %.2fx faster" % (
            res["dense_bf16"]["us_per_layer"], res["dense_bf16"]["gbs"], res["dense_bf16"]["speedup_compressed_vs_dense"]))
    del layers
    torch.cuda.synchronize()
    if not args.no_encode:
        log(args, "timing encode")
        enc = encode_rooflines(args, dev, st)
        res["encode_tokens_per_s"] = enc["wht"]["tokens_per_s_k_and_v"]
        res["encode_note"] = ("tokens/s of one 128K layer's prefill, all KV heads, K and V (k_encode over inputs "
                              "cycled through 4 layers, above the last-level cache)")
        res["encode_roofline"] = enc
        log(args, "encode: WHT %.0f GB/s, KLT %.1f TFLOP/s" % (enc["wht"]["gbs"], enc["klt"]["roofline"]["achieved"]))
    if not args.no_tiers:
        log(args, "timing the tiered 128K layer")
        res["tiers"] = tiered_segments(args, dev, st)
        log(args, "tiers: %.2f us per layer, %.0f GB/s, tier fractions %s" % (
            res["tiers"]["us_per_layer"], res["tiers"]["gbs"], res["tiers"]["tier_fractions"]))
    if not args.no_lloyd_max:
        log(args, "timing Lloyd-Max caches")
        res["lloyd_max"] = lloyd_max_pass(args, dev, st)
        log(args, "Lloyd-Max: %s" % {k: (v["us_per_layer"], v["key_reconstruction_mse"]["reduction"])
                                     for k, v in res["lloyd_max"].items()})
    if not args.no_loops:
        log(args, "timing the batch-16 append + decode loop")
        res["append_decode_loop"] = append_decode_loop(args, dev, st)
        log(args, "loop: %.3f ms per step" % res["append_decode_loop"]["ms_per_step"])
    if not args.no_cpu_baseline:
        log(args, "timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(cfg, n_tokens)
    print(json.dumps(res))


if __name__ == "__main__":
    main()

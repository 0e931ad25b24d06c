"""GPU parity at the workloads' full sizes, on sampled outputs the oracle computes one by one.

Each case builds a whole layer at its real shape (every KV head, the full context) through the
same C-ABI calls the benchmark times, then checks sampled KV heads against the fp64 oracle:
packed codes (bit-exact up to the bin-edge excuse) and decode attention for every q head of the
sampled KV heads (max abs error <= 2e-3, lse <= 5e-3).  Inputs are the seeded host draws, so
both sides see identical values.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_helpers import assert_codes_match, unpack_all

pytestmark = pytest.mark.gpu

ATOL_ATTN = 2e-3


def _layer(cfg, n_tokens, sampled, n_encode=None, quantizer="uniform"):
    """Calibrate every KV head (library and oracle), encode the first n_encode (default all)
    context tokens on the GPU.  Returns (cache, q [batch, n_q, d] float32, host contexts of the
    sampled (b, h), oracle arts, tails: tokens n_encode.. of every (tensor, b, h))."""
    import torch
    from compressed_decode_attention_head_amd import api
    batch = cfg.batch
    blobs, arts = {}, {}
    for t in (synth.K, synth.V):
        cal = [synth.draw(cfg.idx, 0, h, t, "calib", cfg.n_calib, dtype=cfg.dtype, marginal=cfg.marginal)
               for h in range(cfg.n_kv_heads)]
        blobs[t] = [api.calibrate(synth.bf16_bits(c), cfg.rotation, cfg.bits_per_elem, quantizer=quantizer)
                    for c in cal]
        arts[t] = {h: O.calibrate(cal[h], cfg.rotation, cfg.bits_per_elem, quantizer=quantizer)
                   for h in {s[1] for s in sampled}}
    cap = -(-n_tokens // 64) * 64
    cache = api.CompressedKVCache(blobs[synth.K], blobs[synth.V], batch, cap)
    n_enc = n_tokens if n_encode is None else n_encode
    host, tails = {}, {}
    keys_for_q = {}
    for t in (synth.K, synth.V):
        x = torch.empty((batch, cfg.n_kv_heads, n_enc, 128), dtype=torch.bfloat16, device="cuda")
        for b in range(batch):
            for h in range(cfg.n_kv_heads):
                xh = synth.draw(cfg.idx, 0, h, t, "context", n_tokens, dtype=cfg.dtype, marginal=cfg.marginal,
                                extra=b)
                x[b, h] = torch.from_numpy(xh[:n_enc].astype(np.float32)).to(torch.bfloat16)
                tails[(t, b, h)] = xh[n_enc:]
                if (b, h) in sampled:
                    host[(t, b, h)] = xh
                if t == synth.K and b == 0:
                    keys_for_q[h] = xh[:4096]
        cache.encode(t, x)
        del x
    q = synth.queries(cfg.idx, 0, cfg.n_q_heads, cfg.n_kv_heads, [keys_for_q[h] for h in range(cfg.n_kv_heads)])
    q = np.broadcast_to(q, (batch,) + q.shape).copy()
    torch.cuda.synchronize()
    return cache, q, host, arts, tails


def _check_head(cfg, cache, q, host, arts, b, h, n, out, lse, check_codes, more=()):
    """Codes (if check_codes) and decode attention of (b, h) against the oracle; `more` holds
    further (label, q, out, lse) results of the same cache for other queries."""
    group = cfg.n_q_heads // cfg.n_kv_heads
    codes = {}
    for t in (synth.K, synth.V):
        codes[t] = O.encode_codes(host[(t, b, h)][:n], arts[t][h])
        if check_codes:
            # tiles are packed independently: the first 8192 tokens and the last tile (which
            # holds appended tokens) stand for the whole sequence; unpacking in the oracle is slow
            words = cache.codes(t)[b, h].cpu().numpy().view(np.uint32)
            bits = arts[t][h]["bits"]
            wpt = 2 * int(bits.sum())                       # words per 64-token tile
            last = (n - 1) // 64
            for t0, nt in ((0, min(n, 8192)), (64 * last, n - 64 * last)):
                w = words[(t0 // 64) * wpt:(t0 // 64) * wpt + O.packed_words(int(bits.sum()), nt)]
                got = unpack_all(w, bits, nt, t)
                want = codes[t][t0:t0 + nt]
                assert_codes_match(host[(t, b, h)][t0:t0 + nt], arts[t][h], got, want, cfg.dtype, (t, b, h, t0))
    kh = O.reconstruct(codes[synth.K], arts[synth.K][h])
    vh = O.reconstruct(codes[synth.V], arts[synth.V][h])
    for label, qq, oo, ll in (("std 2", q, out, lse),) + tuple(more):
        errs = []
        for g in range(h * group, (h + 1) * group):
            ref, lref = O.attention(qq[b, g], kh, vh)
            errs.append((float(np.abs(oo[b, g] - ref).max()), abs(float(ll[b, g]) - lref)))
        err, lerr = max(e[0] for e in errs), max(e[1] for e in errs)
        print("config %d (b=%d, h=%d, n=%d, queries %s): max abs err %.2e, lse err %.2e"
              % (cfg.idx, b, h, n, label, err, lerr), flush=True)
        assert err <= ATOL_ATTN and lerr <= 5e-3, (label, err, lerr)


@pytest.mark.parametrize("idx,sampled", [(4, [(0, 0), (0, 3)]), (2, [(0, 0), (0, 7)])])
def test_fullsize_layer_sampled_heads(idx, sampled):
    """128K-token WHT 1.33-bit layer (4 KV heads, 28 q heads) and 32K-token KLT 2.76-bit layer
    (8 KV heads, 32 q heads): whole layer on the GPU, two KV heads checked against the oracle."""
    import torch
    cfg = synth.CONFIGS[idx]
    n = cfg.n_tokens
    cache, q, host, arts, _ = _layer(cfg, n, set(sampled))
    qt = torch.from_numpy(q).cuda()
    ws = cache.new_workspace(cfg.n_q_heads, n)
    out = torch.empty_like(qt)
    lse = torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device="cuda")
    cache.decode_attn(qt, n, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    # the same cache at other query temperatures: score std 0.5, 4 and 8 over the context, and
    # near one-hot queries (each q head along one key, 12 above every other score)
    more = []
    keys = [host[(synth.K, 0, h)] if (0, h) in sampled else
            synth.draw(cfg.idx, 0, h, synth.K, "context", n, dtype=cfg.dtype, marginal=cfg.marginal)
            for h in range(cfg.n_kv_heads)]
    for mode in (0.5, 4.0, 8.0, "peaked"):
        if mode == "peaked":
            qm = synth.peaked_queries(cfg.idx, 0, cfg.n_q_heads, cfg.n_kv_heads, keys)
        else:
            qm = synth.queries(cfg.idx, 0, cfg.n_q_heads, cfg.n_kv_heads, [k[:4096] for k in keys], target_std=mode)
        qm = np.broadcast_to(qm, (cfg.batch,) + qm.shape).copy()
        om, lm = cache.decode_attn(torch.from_numpy(qm).cuda(), n, workspace=ws)
        torch.cuda.synchronize()
        more.append(("std %s" % mode if mode != "peaked" else "peaked", qm, om.cpu().numpy(), lm.cpu().numpy()))
    for i, (b, h) in enumerate(sampled):
        _check_head(cfg, cache, q, host, arts, b, h, n, o, l, check_codes=(i == 0), more=more)


@pytest.mark.parametrize("idx,sampled", [(2, [(0, 0), (0, 7)]), (3, [(0, 0), (9, 5), (15, 7)])])
def test_fullsize_lloyd_max_layer(idx, sampled):
    """Lloyd-Max caches at full size: the 32K-token 2.76-bit layer (8 KV heads) and the
    batch-16 x 8K 4-bit layer, K and V Lloyd-Max, whole layer on the GPU (the level pass), sampled
    sequences' codes and attention against the oracle."""
    import torch
    cfg = synth.CONFIGS[idx]
    n = cfg.n_tokens
    cache, q, host, arts, _ = _layer(cfg, n, set(sampled), quantizer="lloyd-max")
    assert cache.quantizer == 3
    out, lse = cache.decode_attn(torch.from_numpy(q).cuda(), n)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for i, (b, h) in enumerate(sampled):
        _check_head(cfg, cache, q, host, arts, b, h, n, o, l, check_codes=(i == 0))


def test_fullsize_append_loop_64_steps():
    """The batch-16 workload's decode loop for all of its 64 steps on two sequences' worth of
    cache: each step encodes one new K and V token per (b, h) at the next offset and runs decode
    attention over the grown cache; the codes of every appended token and the attention of steps
    1, 17, 33 and 64 are checked against the oracle."""
    import torch
    cfg = synth.CONFIGS[3]
    n0, steps = cfg.n_tokens, cfg.decode_steps
    sampled = {(0, 0), (1, 3)}
    batch = 2
    from dataclasses import replace
    cfg2 = replace(cfg, batch=batch)
    cache, q, host, arts, tails = _layer(cfg2, n0 + steps, sampled, n_encode=n0)
    qt = torch.from_numpy(q).cuda()
    group = cfg.n_q_heads // cfg.n_kv_heads
    for s_ in range(steps):
        for t in (synth.K, synth.V):
            x = np.stack([np.stack([tails[(t, b, h)][s_] for h in range(cfg.n_kv_heads)]) for b in range(batch)])
            cache.encode(t, torch.from_numpy(x[:, :, None, :].astype(np.float32)).to(torch.bfloat16).cuda(),
                         token_offset=n0 + s_)
        n = n0 + s_ + 1
        if s_ + 1 in (1, 17, 33, 64):
            out, lse = cache.decode_attn(qt, n)
            torch.cuda.synchronize()
            o, l = out.cpu().numpy(), lse.cpu().numpy()
            for b, h in sorted(sampled):
                ref, lref = O.decode_attention(q[b, h * group:(h + 1) * group],
                                               [O.encode_codes(host[(synth.K, b, h)][:n], arts[synth.K][h])],
                                               [O.encode_codes(host[(synth.V, b, h)][:n], arts[synth.V][h])],
                                               [arts[synth.K][h]], [arts[synth.V][h]])
                err = float(np.abs(o[b, h * group:(h + 1) * group] - ref).max())
                lerr = float(np.abs(l[b, h * group:(h + 1) * group] - lref).max())
                print("append step %d (b=%d, h=%d, %d tokens): max abs err %.2e, lse err %.2e" % (s_ + 1, b, h, n, err, lerr),
                      flush=True)
                assert err <= ATOL_ATTN and lerr <= 5e-3
    # every appended token's codes (the last two tiles hold them)
    n = n0 + steps
    for t in (synth.K, synth.V):
        for b, h in sorted(sampled):
            art = arts[t][h]
            B = int(art["bits"].sum())
            words = cache.codes(t)[b, h].cpu().numpy().view(np.uint32)
            first = n0 // 64
            w = words[first * 2 * B:first * 2 * B + O.packed_words(B, n - n0)]
            got = unpack_all(w, art["bits"], n - n0, t)
            want = O.encode_codes(host[(t, b, h)][n0:n], art)
            assert_codes_match(host[(t, b, h)][n0:n], art, got, want, cfg.dtype, ("append", t, b, h))


def test_fullsize_batch16_append_sampled():
    """Batch 16 x 8 KV heads x 8192 tokens, KLT 4.0 bits, then decode steps that each append one
    encoded token per (b, h): sampled sequences checked after the appends."""
    import torch
    cfg = synth.CONFIGS[3]
    n0, steps = cfg.n_tokens, 3
    sampled = {(0, 0), (9, 5), (15, 7)}
    cache, q, host, arts, tails = _layer(cfg, n0 + steps, sampled, n_encode=n0)
    # decode steps: each appends one encoded token per (b, h) to the prefill
    for s in range(steps):
        for t in (synth.K, synth.V):
            x = np.stack([np.stack([tails[(t, b, h)][s] for h in range(cfg.n_kv_heads)]) for b in range(cfg.batch)])
            xt = torch.from_numpy(x[:, :, None, :].astype(np.float32)).to(torch.bfloat16).cuda()
            cache.encode(t, xt, token_offset=n0 + s)
    n = n0 + steps
    qt = torch.from_numpy(q).cuda()
    out, lse = cache.decode_attn(qt, n)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for i, (b, h) in enumerate(sorted(sampled)):
        _check_head(cfg, cache, q, host, arts, b, h, n, o, l, check_codes=(i == 0))


def test_fullsize_nova_keys_joint_split():
    """The 128K-token Qwen-shaped layer with the non-orthogonal key transform on K (query
    second moments from 2048 calibration queries per head, scaled like the decode queries) and
    the joint K/V split of 2 x 170 bits: library split equal to the oracle's, whole layer on the
    GPU, KV heads 0 and 3 checked against the oracle (codes of head 0 too)."""
    import torch
    from compressed_decode_attention_head_amd import api
    cfg = synth.CONFIGS[4]
    n, n_kv = cfg.n_tokens, cfg.n_kv_heads
    sampled = [(0, 0), (0, 3)]
    cal = {t: [synth.draw(cfg.idx, 0, h, t, "calib", cfg.n_calib, dtype=cfg.dtype, marginal=cfg.marginal)
               for h in range(n_kv)] for t in (synth.K, synth.V)}
    q_cal = []
    for h in range(n_kv):
        qr = synth.draw(cfg.idx, 0, h, synth.K, "query", 2048, dtype="f64", extra=50000)
        q_cal.append(qr * (2.0 / (cal[synth.K][h] @ qr.T / np.sqrt(128)).std(axis=0))[:, None])
    moments = [api.query_moment(qc) for qc in q_cal]
    total = 2 * O.bits_budget(cfg.bits_per_elem, 128)
    kb0 = [api.calibrate(synth.bf16_bits(cal[synth.K][h]), "nova", cfg.bits_per_elem, query_moment=moments[h])
           for h in range(n_kv)]
    vb0 = [api.calibrate(synth.bf16_bits(c), cfg.rotation, cfg.bits_per_elem) for c in cal[synth.V]]
    bk, bv = api.joint_kv_split(kb0, vb0, total)
    ka0 = [O.calibrate(cal[synth.K][h], "nova", cfg.bits_per_elem, q_cal=q_cal[h]) for h in range(n_kv)]
    va0 = [O.calibrate(c, cfg.rotation, cfg.bits_per_elem) for c in cal[synth.V]]
    want = O.joint_kv_split([a["sigma2"] for a in ka0], [a["sigma2"] for a in va0],
                            [O.value_term_weight(a["C"]) for a in va0], total, tensor_cap=512)
    assert (bk, bv) == want[:2], ((bk, bv), want)
    blobs = {synth.K: [api.calibrate(synth.bf16_bits(cal[synth.K][h]), "nova", bk / 128, query_moment=moments[h])
                       for h in range(n_kv)],
             synth.V: [api.calibrate(synth.bf16_bits(c), cfg.rotation, bv / 128) for c in cal[synth.V]]}
    arts = {synth.K: {h: O.calibrate(cal[synth.K][h], "nova", bk / 128, q_cal=q_cal[h]) for h in (0, 3)},
            synth.V: {h: O.calibrate(cal[synth.V][h], cfg.rotation, bv / 128) for h in (0, 3)}}
    cache = api.CompressedKVCache(blobs[synth.K], blobs[synth.V], 1, n)
    host, keys_for_q = {}, {}
    for t in (synth.K, synth.V):
        x = torch.empty((1, n_kv, n, 128), dtype=torch.bfloat16, device="cuda")
        for h in range(n_kv):
            xh = synth.draw(cfg.idx, 0, h, t, "context", n, dtype=cfg.dtype, marginal=cfg.marginal)
            x[0, h] = torch.from_numpy(xh.astype(np.float32)).to(torch.bfloat16)
            if h in (0, 3):
                host[(t, 0, h)] = xh
            if t == synth.K:
                keys_for_q[h] = xh[:4096]
        cache.encode(t, x)
        del x
    q = synth.queries(cfg.idx, 0, cfg.n_q_heads, n_kv, [keys_for_q[h] for h in range(n_kv)])[None]
    out, lse = cache.decode_attn(torch.from_numpy(q).cuda(), n)
    torch.cuda.synchronize()
    print("nova keys, joint split", bk, bv, flush=True)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for i, (b, h) in enumerate(sampled):
        _check_head(cfg, cache, q, host, arts, b, h, n, o, l, check_codes=(i == 0))


@pytest.mark.parametrize("avg_bits", [2.76, 2.0])
def test_fullsize_token_tiers_segments(avg_bits):
    """The 128K-token tiered Llama-shaped layer (8 KV heads, 32 q heads) at its 2.76 bits per
    element on average, and at 2.0, where tokens are also evicted: tiers from the library's solver on each head's Zipf attention mass (equal to the
    oracle's for the sampled heads), tier-2 and tier-4 coded caches with their own bits and the
    same rotation, raw bf16 tier-16 tokens, evicted tier-0 tokens; one multi-segment decode step
    on the GPU, KV heads 0 and 5 (all 4 q heads each) against the oracle's segment attention."""
    import torch
    from compressed_decode_attention_head_amd import api
    cfg = synth.CONFIGS[5]
    n, n_kv, n_q = cfg.n_tokens, cfg.n_kv_heads, cfg.n_q_heads
    group = n_q // n_kv
    sampled = (0, 5)
    cal = {t: [synth.draw(cfg.idx, 0, h, t, "calib", cfg.n_calib) for h in range(n_kv)] for t in (synth.K, synth.V)}
    blobs = {(tau, t): [api.calibrate(synth.bf16_bits(c), "klt", float(tau)) for c in cal[t]]
             for tau in (2, 4) for t in (synth.K, synth.V)}
    x = {t: [synth.draw(cfg.idx, 0, h, t, "context", n) for h in range(n_kv)] for t in (synth.K, synth.V)}
    tiers = []
    for h in range(n_kv):
        s2 = [api.calib_view(blobs[(2, t)][h])["sigma2"] for t in (synth.K, synth.V)]
        tiers.append(api.token_tiers(synth.zipf_mass(cfg.idx, 0, h, n), api.tier_distortions(s2), avg_bits))
    arts = {(tau, t): {h: O.calibrate(cal[t][h], "klt", float(tau)) for h in sampled} for tau in (2, 4)
            for t in (synth.K, synth.V)}
    for h in sampled:
        dist = O.tier_distortions([arts[(2, synth.K)][h]["sigma2"], arts[(2, synth.V)][h]["sigma2"]], 128)
        assert np.array_equal(tiers[h], O.token_tiers(synth.zipf_mass(cfg.idx, 0, h, n), dist, 128, avg_bits)), h
    idx = {tau: [np.nonzero(tiers[h] == tau)[0] for h in range(n_kv)] for tau in (0, 2, 4, 16)}
    assert all(len(idx[tau][h]) > 0 for tau in (2, 4, 16) for h in sampled)
    assert (avg_bits >= 2.5) == all(len(idx[0][h]) == 0 for h in sampled)     # eviction at 2.0 only
    q = synth.queries(cfg.idx, 0, n_q, n_kv, [x[synth.K][h][:4096] for h in range(n_kv)])
    segs, keep = [], []
    for tau in (2, 4, 16):
        counts = [len(idx[tau][h]) for h in range(n_kv)]
        cap = max(64, -(-max(counts) // 64) * 64)
        sl = torch.tensor([counts], dtype=torch.int32, device="cuda")
        xt = {}
        for t in (synth.K, synth.V):
            xt[t] = torch.zeros((1, n_kv, cap, 128), dtype=torch.bfloat16, device="cuda")
            for h in range(n_kv):
                xt[t][0, h, :counts[h]] = torch.from_numpy(x[t][h][idx[tau][h]].astype(np.float32)).to(torch.bfloat16)
        if tau == 16:
            keep += [xt[synth.K], xt[synth.V], sl]
            segs.append({"k_raw": xt[synth.K], "v_raw": xt[synth.V], "seq_lens": sl, "max_seq_len": max(counts)})
        else:
            cache = api.CompressedKVCache(blobs[(tau, synth.K)], blobs[(tau, synth.V)], 1, cap)
            for t in (synth.K, synth.V):
                cache.encode(t, xt[t])
            keep += [cache, sl]
            segs.append({"cache": cache, "seq_lens": sl, "max_seq_len": max(counts)})
        del xt
    # the default queries (score std 2) and sharper ones (std 4) over the same segments
    q4 = synth.queries(cfg.idx, 0, n_q, n_kv, [x[synth.K][h][:4096] for h in range(n_kv)], target_std=4.0)
    res = []
    for label, qq in (("std 2", q), ("std 4", q4)):
        out, lse = api.decode_attn_segments(segs, torch.from_numpy(qq[None]).cuda(), 1, n_kv)
        torch.cuda.synchronize()
        res.append((label, qq, out[0].cpu().numpy(), lse[0].cpu().numpy()))
    for h in sampled:
        parts = []
        for tau in (2, 4):
            ii = idx[tau][h]
            rec = [O.reconstruct(O.encode_codes(x[t][h][ii], arts[(tau, t)][h]), arts[(tau, t)][h])
                   for t in (synth.K, synth.V)]
            parts.append((rec[0], rec[1]))
        parts.append((x[synth.K][h][idx[16][h]], x[synth.V][h][idx[16][h]]))
        for label, qq, o, l in res:
            for g in range(h * group, (h + 1) * group):
                ref, lref = O.segment_attention(qq[g], parts)
                err, lerr = float(np.abs(o[g] - ref).max()), abs(float(l[g]) - lref)
                print("tiers 128K head %d q %d (%s): tokens per tier %s, max abs err %.2e, lse err %.2e"
                      % (h, g, label, [len(idx[tau][h]) for tau in (0, 2, 4, 16)], err, lerr), flush=True)
                assert err <= ATOL_ATTN and lerr <= 5e-3, (h, g, label, err, lerr)

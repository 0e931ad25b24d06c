"""GPU parity of the dense bf16 decode attention (aatc_decode_attn_dense), the full-cache
comparator, against the oracle's plain fp64 softmax attention on the same bf16 values.

Bar, from the arithmetic: K and V enter the matrix cores exactly (bf16); q and the
probabilities enter as bf16 high plus low parts, which leave a relative error of at most 2^-18
each; sums are fp32.  Output errors are then of order 2^-18 |s| max|v| plus fp32 rounding, so
the bar is max abs error <= 1e-4 * max(1, max|v|) on the output and 1e-4 on the lse.
"""
import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

CFG = 4                      # Qwen2.5-7B-shaped heads: 28 q heads over 4 KV heads, d = 128


def _torch():
    import torch
    return torch


def _inputs(batch, n_kv, group, n_tokens, cap, layer=0):
    """Seeded bf16 keys/values [batch, n_kv, cap, 128] (zero past n_tokens) and fp32 queries."""
    k = np.zeros((batch, n_kv, cap, 128), dtype=np.float32)
    v = np.zeros_like(k)
    for b in range(batch):
        for h in range(n_kv):
            k[b, h, :n_tokens] = synth.draw(CFG, layer, h, synth.K, "context", n_tokens, extra=b)
            v[b, h, :n_tokens] = synth.draw(CFG, layer, h, synth.V, "context", n_tokens, extra=b)
    q = np.stack([synth.queries(CFG, layer, n_kv * group, n_kv, [k[b, h, :max(n_tokens, 1)] for h in range(n_kv)])
                  for b in range(batch)]).astype(np.float32)
    return k, v, q


def _run(k, v, q, max_seq, seq_lens=None):
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    kt = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vt = torch.from_numpy(v).to(torch.bfloat16).cuda()
    qt = torch.from_numpy(q).cuda()
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    out, lse = api.decode_attn_dense(kt, vt, qt, max_seq, seq_lens=sl)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check(k, v, q, out, lse, lens):
    batch, n_kv = k.shape[:2]
    group = q.shape[1] // n_kv
    worst, lworst = 0.0, 0.0
    for b in range(batch):
        for h in range(n_kv):
            n = lens[b][h]
            tol = 1e-4 * max(1.0, float(np.abs(v[b, h, :n]).max()) if n else 1.0)
            for g in range(h * group, (h + 1) * group):
                ref, lref = O.attention(q[b, g].astype(np.float64), k[b, h, :n], v[b, h, :n])
                err = float(np.abs(out[b, g] - ref).max())
                if n == 0:
                    assert np.all(out[b, g] == 0.0) and lse[b, g] == -np.inf, (b, g)
                    continue
                lerr = abs(float(lse[b, g]) - lref)
                assert err <= tol, (b, h, g, n, err, tol)
                assert lerr <= 1e-4, (b, h, g, n, lerr)
                worst, lworst = max(worst, err / tol), max(lworst, lerr)
    return worst, lworst


@pytest.mark.parametrize("batch,n_kv,group,n_tokens,cap,ragged", [
    (1, 2, 7, 5000, 5005, False),        # 20 chunks of 256 tokens, a ragged 32-token block at the end
    (1, 1, 1, 2049, 2049, False),        # one token past a 256-token chunk boundary, group of 1
    (4, 8, 2, 9000, 9000, False),        # 1024-token chunks (2048 would give 160 workgroups)
    (8, 8, 1, 8200, 8256, False),        # 2048-token chunks (320 workgroups), ragged last chunk
    (1, 1, 8, 4096, 4096, False),        # group of 8
    (1, 3, 3, 64, 70, False),
    (2, 2, 4, 2100, 2112, True),         # per-(b,h) lengths 0, 1, 33, 2100
])
def test_dense_matches_oracle(batch, n_kv, group, n_tokens, cap, ragged):
    k, v, q = _inputs(batch, n_kv, group, n_tokens, cap)
    if ragged:
        lens = [[0, 1], [33, n_tokens]]
        out, lse = _run(k, v, q, n_tokens, seq_lens=lens)
    else:
        lens = [[n_tokens] * n_kv for _ in range(batch)]
        out, lse = _run(k, v, q, n_tokens)
    worst, lworst = _check(k, v, q, out, lse, lens)
    print("dense", batch, n_kv, group, n_tokens, "err/tol %.3g lse err %.3g" % (worst, lworst), flush=True)


def test_dense_short_max_seq_len_and_scale():
    """max_seq_len below the capacity limits every head; an explicit softmax scale."""
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    k, v, q = _inputs(1, 2, 4, 700, 768)
    kt = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vt = torch.from_numpy(v).to(torch.bfloat16).cuda()
    out, lse = api.decode_attn_dense(kt, vt, torch.from_numpy(q).cuda(), 333, scale=0.05)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for g in range(8):
        h = g // 4
        ref, lref = O.attention(q[0, g].astype(np.float64), k[0, h, :333], v[0, h, :333], scale=0.05)
        assert np.abs(out[0, g] - ref).max() <= 1e-4 * max(1.0, np.abs(v[0, h, :333]).max())
        assert abs(lse[0, g] - lref) <= 1e-4


def test_dense_fullsize_sampled_heads():
    """The 128K-token, 28-q-head layer the comparator is timed on: every KV head on the GPU,
    KV heads 0 and 3 (all 7 q heads each) checked against the oracle."""
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    cfg = synth.CONFIGS[CFG]
    n, n_kv, n_q = cfg.n_tokens, cfg.n_kv_heads, cfg.n_q_heads
    group = n_q // n_kv
    kt = torch.empty((1, n_kv, n, 128), dtype=torch.bfloat16, device="cuda")
    vt = torch.empty_like(kt)
    host = {}
    for h in range(n_kv):
        for t, dst in ((synth.K, kt), (synth.V, vt)):
            x = synth.draw(CFG, 0, h, t, "context", n)
            dst[0, h] = torch.from_numpy(x).to(torch.bfloat16)
            if h in (0, 3):
                host[(t, h)] = x
            if t == synth.K:
                host[("q", h)] = x[:4096]
    q = synth.queries(CFG, 0, n_q, n_kv, [host[("q", h)] for h in range(n_kv)]).astype(np.float32)
    out, lse = api.decode_attn_dense(kt, vt, torch.from_numpy(q[None]).cuda(), n)
    torch.cuda.synchronize()
    out, lse = out[0].cpu().numpy(), lse[0].cpu().numpy()
    for h in (0, 3):
        tol = 1e-4 * max(1.0, float(np.abs(host[(synth.V, h)]).max()))
        for g in range(h * group, (h + 1) * group):
            ref, lref = O.attention(q[g].astype(np.float64), host[(synth.K, h)], host[(synth.V, h)])
            err = float(np.abs(out[g] - ref).max())
            print("dense 128K head", h, "q", g, "err %.3g tol %.3g lse err %.3g" % (err, tol, abs(lse[g] - lref)),
                  flush=True)
            assert err <= tol
            assert abs(lse[g] - lref) <= 1e-4

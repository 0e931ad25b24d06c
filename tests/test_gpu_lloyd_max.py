"""GPU parity of Lloyd-Max caches: the codes the HIP encoder writes, the reconstruction and the
decode attention (the level pass, k_attn_lm) against the fp64 oracle on the same seeded inputs.

Bars as for the uniform quantizer: codes bit-exact up to the bin-edge excuse (Walsh-Hadamard bf16
rows: no mismatch), reconstruction within 1e-6 max|x_hat|, attention within 2e-3 and lse within
5e-3 of the oracle's fp64 attention over the reconstructed cache.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_helpers import Case, assert_codes_match, unpack_all

pytestmark = pytest.mark.gpu

ATOL_ATTN = 2e-3

CASES = {
    "cfg1-lm": dict(cfg=1, n_kv=1, group=1, n_tokens=4096, dtype="f32", rotation="klt", bpe_k=2.0),
    "cfg2s-lm": dict(cfg=2, n_kv=2, group=4, n_tokens=1000, rotation="klt", bpe_k=2.76),
    "cfg3s-lm": dict(cfg=3, n_kv=2, group=4, n_tokens=300, batch=2, rotation="klt", bpe_k=4.0),
    "cfg4s-lm": dict(cfg=4, n_kv=2, group=7, n_tokens=777, rotation="wht", bpe_k=1.33, marginal="t3"),
    "k-lm-v-uniform": dict(cfg=2, n_kv=2, group=8, n_tokens=500, rotation="klt", bpe_k=2.76, quant_v="uniform"),
    "k-uniform-v-lm": dict(cfg=2, n_kv=2, group=3, n_tokens=500, rotation="klt", bpe_k=2.76, quant_k="uniform"),
}


def _torch():
    import torch
    return torch


@pytest.fixture(scope="module", params=sorted(CASES))
def built(request):
    torch = _torch()
    kw = dict(CASES[request.param])
    kw.setdefault("quant_k", "lloyd-max")
    kw.setdefault("quant_v", "lloyd-max")
    case = Case(**kw)
    cache = case.make_cache()
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    torch.cuda.synchronize()
    return request.param, case, cache


def test_lloyd_max_codes(built):
    name, case, cache = built
    print("case", name, "quantizer bits", cache.quantizer, flush=True)
    for t in (synth.K, synth.V):
        words = cache.codes(t).cpu().numpy().view(np.uint32)
        for b in range(case.batch):
            for h in range(case.n_kv):
                art = case.art[t][h]
                B = int(art["bits"].sum())
                got = unpack_all(words[b, h, :O.packed_words(B, case.n)], art["bits"], case.n, t)
                assert_codes_match(case.x[t][b, h], art, got, case.codes[t][b, h], case.dtype, (name, t, b, h))


def test_lloyd_max_reconstruction(built):
    name, case, cache = built
    for t in (synth.K, synth.V):
        xh = cache.decode(t, 0, case.n).cpu().numpy().astype(np.float64)
        for b in range(case.batch):
            for h in range(case.n_kv):
                ref = O.reconstruct(case.codes[t][b, h], case.art[t][h])
                assert np.abs(xh[b, h] - ref).max() <= 1e-6 * np.abs(ref).max(), (name, t, b, h)


@pytest.mark.parametrize("mode", [None, 4.0, "peaked"])
def test_lloyd_max_decode_attention(built, mode):
    torch = _torch()
    name, case, cache = built
    qh = case.q if mode is None else case.queries(mode)
    out, lse = cache.decode_attn(torch.from_numpy(qh.astype(np.float32)).cuda(), case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention(q=qh)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    lerr = float(np.abs(lse.cpu().numpy() - lref).max())
    print(name, "queries", mode or "std 2", "attn max abs err", err, "lse err", lerr, flush=True)
    assert err <= ATOL_ATTN and lerr <= 5e-3, (err, lerr)


def test_lloyd_max_ragged_and_empty():
    torch = _torch()
    case = Case(cfg=2, n_kv=2, group=4, n_tokens=333, batch=3, rotation="klt", bpe_k=2.76,
                quant_k="lloyd-max", quant_v="lloyd-max")
    cache = case.make_cache(capacity=384)
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    seq = np.array([333, 65, 0], dtype=np.int32)
    out, lse = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), 333,
                                 seq_lens=torch.from_numpy(seq).cuda())
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention(seq_lens=seq)
    o = out.cpu().numpy()
    assert np.abs(o[:2] - ref[:2]).max() <= ATOL_ATTN
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[2]))
    assert np.abs(lse.cpu().numpy()[:2] - lref[:2]).max() <= 5e-3


def test_lloyd_max_lowers_reconstruction_error():
    """On the same context and bits, the Lloyd-Max cache reconstructs closer than the uniform one
    (the gain the codebooks buy at 2.76 and 4 bits per element), measured on the GPU's own
    reconstruction."""
    torch = _torch()
    for cfg, bpe in ((2, 2.76), (3, 4.0)):
        mse = {}
        for qz in ("uniform", "lloyd-max"):
            case = Case(cfg=cfg, n_kv=1, group=4, n_tokens=4096, rotation="klt", bpe_k=bpe, quant_k=qz, quant_v=qz)
            cache = case.make_cache()
            cache.encode(synth.K, case.torch_x(synth.K))
            xh = cache.decode(synth.K, 0, case.n).cpu().numpy().astype(np.float64)[0, 0]
            mse[qz] = float(np.mean((xh - case.x[synth.K][0, 0].astype(np.float64)) ** 2))
        gain = 1 - mse["lloyd-max"] / mse["uniform"]
        print("config %d, %.2f bits: reconstruction MSE uniform %.4g, Lloyd-Max %.4g (%.1f%% lower)"
              % (cfg, bpe, mse["uniform"], mse["lloyd-max"], 100 * gain), flush=True)
        assert gain > 0.01

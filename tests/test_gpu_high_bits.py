"""Decode attention over caches with more than 512 bits per K or V vector (5 to 8 bits per
element, up to the 8d bits that calibration and encoding allow): such caches take the level pass
(uniform blobs' level tables, c - 2^(b-1) + 1/2), which this checks against the fp64 oracle on the
same seeded inputs, with the codes the HIP encoder writes checked first.

Bars as elsewhere: codes bit-exact up to the bin-edge excuse, attention within 2e-3 and lse within
5e-3 of the oracle's fp64 attention over the reconstructed cache.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import Case, assert_codes_match, unpack_all
import oracle as O

pytestmark = pytest.mark.gpu

ATOL_ATTN = 2e-3

CASES = {
    # K 6 bits, V 8 bits per element (768 and 1024 bits per vector: one LDS slot per wave)
    "klt-6-8": dict(cfg=3, n_kv=2, group=4, n_tokens=700, batch=2, rotation="klt", bpe_k=6.0, bpe_v=8.0),
    # K within the summed-code limit, V past it: the whole call takes the level pass
    "klt-2-5": dict(cfg=2, n_kv=2, group=3, n_tokens=1000, rotation="klt", bpe_k=2.0, bpe_v=5.0),
    # Walsh-Hadamard at 5 bits, GQA group 7
    "wht-5": dict(cfg=4, n_kv=1, group=7, n_tokens=1333, rotation="wht", bpe_k=5.0, marginal="t3"),
}


def _torch():
    import torch
    return torch


@pytest.fixture(scope="module", params=sorted(CASES))
def built(request):
    torch = _torch()
    case = Case(**CASES[request.param])
    cache = case.make_cache()
    assert max(cache.k_bits, cache.v_bits) > 512
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    torch.cuda.synchronize()
    return request.param, case, cache


def test_high_bits_codes(built):
    name, case, cache = built
    for t in (synth.K, synth.V):
        words = cache.codes(t).cpu().numpy().view(np.uint32)
        for b in range(case.batch):
            for h in range(case.n_kv):
                art = case.art[t][h]
                B = int(art["bits"].sum())
                got = unpack_all(words[b, h, :O.packed_words(B, case.n)], art["bits"], case.n, t)
                assert_codes_match(case.x[t][b, h], art, got, case.codes[t][b, h], case.dtype, (name, t, b, h))


@pytest.mark.parametrize("mode", [None, 4.0, "peaked"])
def test_high_bits_decode_attention(built, mode):
    torch = _torch()
    name, case, cache = built
    qh = case.q if mode is None else case.queries(mode)
    out, lse = cache.decode_attn(torch.from_numpy(qh.astype(np.float32)).cuda(), case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention(q=qh)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    lerr = float(np.abs(lse.cpu().numpy() - lref).max())
    print(name, (cache.k_bits, cache.v_bits), "queries", mode or "std 2", "attn max abs err", err, "lse err", lerr,
          flush=True)
    assert err <= ATOL_ATTN and lerr <= 5e-3, (err, lerr)


def test_high_bits_ragged_lengths():
    """Per-sequence lengths (a partial last tile, one tile, empty) over a 768 + 1024-bit cache."""
    torch = _torch()
    case = Case(cfg=3, n_kv=2, group=4, n_tokens=300, batch=3, rotation="klt", bpe_k=6.0, bpe_v=8.0)
    cache = case.make_cache(capacity=320)
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    seq = np.array([300, 64, 0], dtype=np.int32)
    out, lse = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), 300,
                                 seq_lens=torch.from_numpy(seq).cuda())
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention(seq_lens=seq)
    o = out.cpu().numpy()
    assert np.abs(o[:2] - ref[:2]).max() <= ATOL_ATTN
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[2]))
    assert np.abs(lse.cpu().numpy()[:2] - lref[:2]).max() <= 5e-3

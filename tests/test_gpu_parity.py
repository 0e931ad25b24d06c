"""GPU parity: libaatc's HIP path against the fp64 oracle on the same seeded inputs.

Bars: codes and packed words bit-exact (a mismatch is allowed only within 1e-5 of a bin edge,
at a rate <= 1e-6); reconstruction within 1e-6 max|x_hat|; decode attention max abs error
<= 2e-3 against the oracle's fp64 attention on the dequantized cache.
"""
import math

import numpy as np
import pytest

import oracle as O
import synth
from gpu_helpers import Case, assert_codes_match, unpack_all

pytestmark = pytest.mark.gpu

ATOL_ATTN = 2e-3


def _torch():
    import torch
    return torch


def _check_codes(case, cache, tensor):
    words = cache.codes(tensor).cpu().numpy().view(np.uint32)
    bits_lib = None
    from compressed_decode_attention_head_amd import api
    blobs = cache.k_blobs_host if tensor == synth.K else cache.v_blobs_host
    for b in range(case.batch):
        for h in range(case.n_kv):
            bits = np.asarray(api.calib_view(blobs[h])["bits"], dtype=np.int64)
            assert np.array_equal(bits, case.art[tensor][h]["bits"])
            B = int(bits.sum())
            nw = O.packed_words(B, case.n)
            got_words = words[b, h, :nw]
            got = unpack_all(got_words, bits, case.n, tensor)
            want = case.codes[tensor][b, h]
            n_bad = assert_codes_match(case.x[tensor][b, h], case.art[tensor][h], got, want, case.dtype, (b, h))
            if n_bad == 0:
                ref_words = (O.pack_k if tensor == synth.K else O.pack_v)(want, bits)
                assert np.array_equal(got_words, ref_words), (b, h)


CASES = {
    "cfg1": dict(cfg=1, n_kv=1, group=1, n_tokens=4096, dtype="f32", rotation="klt", bpe_k=2.0),
    "cfg2s": dict(cfg=2, n_kv=2, group=4, n_tokens=1000, dtype="bf16", rotation="klt", bpe_k=2.76),
    "cfg3s": dict(cfg=3, n_kv=2, group=4, n_tokens=300, batch=2, dtype="bf16", rotation="klt", bpe_k=4.0),
    "cfg4s": dict(cfg=4, n_kv=2, group=7, n_tokens=777, dtype="bf16", rotation="wht", bpe_k=1.33,
                  marginal="t3"),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def built(request):
    torch = _torch()
    case = Case(**CASES[request.param])
    cache = case.make_cache()
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    torch.cuda.synchronize()
    return request.param, case, cache


def test_encode_codes_and_words(built):
    name, case, cache = built
    print("case", name, flush=True)
    for t in (synth.K, synth.V):
        _check_codes(case, cache, t)


def test_decode_reconstruction(built):
    torch = _torch()
    name, case, cache = built
    for t in (synth.K, synth.V):
        xh = cache.decode(t, 0, case.n).cpu().numpy().astype(np.float64)
        for b in range(case.batch):
            for h in range(case.n_kv):
                ref = O.reconstruct(case.codes[t][b, h], case.art[t][h])
                err = np.abs(xh[b, h] - ref).max()
                assert err <= 1e-6 * np.abs(ref).max(), (name, t, b, h, err)


def test_decode_attention(built):
    torch = _torch()
    name, case, cache = built
    q = torch.from_numpy(case.q.astype(np.float32)).cuda()
    out, lse = cache.decode_attn(q, case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention()
    err = np.abs(out.cpu().numpy() - ref).max()
    lerr = np.abs(lse.cpu().numpy() - lref).max()
    print(name, "attn max abs err", err, "lse err", lerr, flush=True)
    assert err <= ATOL_ATTN, err
    assert lerr <= 5e-3, lerr


@pytest.mark.parametrize("mode", [0.5, 4.0, 8.0, "peaked"])
def test_decode_attention_temperature(built, mode):
    """Sharper and flatter attention than the default score std of 2: the fixed-point weights and
    probabilities of the cache pass stay within the bar at score std 0.5, 4 and 8 and for near
    one-hot queries."""
    torch = _torch()
    name, case, cache = built
    qh = case.queries(mode)
    out, lse = cache.decode_attn(torch.from_numpy(qh).cuda(), case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention(q=qh)
    err = np.abs(out.cpu().numpy() - ref).max()
    lerr = np.abs(lse.cpu().numpy() - lref).max()
    print(name, "queries", mode, "attn max abs err", err, "lse err", lerr, flush=True)
    assert err <= ATOL_ATTN, err
    assert lerr <= 5e-3, lerr


def test_partial_then_merge_equals_one_call(built):
    """The two halves called separately give the one-shot result bit for bit."""
    torch = _torch()
    name, case, cache = built
    q = torch.from_numpy(case.q.astype(np.float32)).cuda()
    out1, lse1 = cache.decode_attn(q, case.n)
    ws = cache.new_workspace(q.shape[1], case.n)
    out2 = torch.full_like(q, float("nan"))
    lse2 = torch.full_like(lse1, float("nan"))
    cache.decode_attn_partial(q, case.n, ws)
    cache.decode_attn_merge(q.shape[1], case.n, ws, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2), name


def test_ragged_seq_lens_and_empty():
    torch = _torch()
    case = Case(cfg=2, n_kv=2, group=4, n_tokens=333, batch=3, rotation="klt", bpe_k=2.76)
    cache = case.make_cache(capacity=384)
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    seq = np.array([333, 65, 0], dtype=np.int32)
    q = torch.from_numpy(case.q.astype(np.float32)).cuda()
    out, lse = cache.decode_attn(q, 333, seq_lens=torch.from_numpy(seq).cuda())
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention(seq_lens=seq)
    o = out.cpu().numpy()
    assert np.abs(o[:2] - ref[:2]).max() <= ATOL_ATTN
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[2]))
    assert np.abs(lse.cpu().numpy()[:2] - lref[:2]).max() <= 5e-3


@pytest.mark.parametrize("bpe_k", [1.0, 2.0, 3.0, 4.0])
def test_unit_aligned_k_tiles(bpe_k):
    """K caches of 128, 256, 384 and 512 bits per vector (whole 16-byte units per token, the K
    tiles that the cache pass stores permuted in LDS), over several tiles with a ragged tail and
    per-sequence lengths that end inside a tile."""
    torch = _torch()
    case = Case(cfg=3, n_kv=2, group=4, n_tokens=837, batch=2, rotation="klt", bpe_k=bpe_k, bpe_v=2.0)
    cache = case.make_cache()
    assert cache.k_bits == int(128 * bpe_k)
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    seq = np.array([837, 450], dtype=np.int32)
    q = torch.from_numpy(case.q.astype(np.float32)).cuda()
    out, lse = cache.decode_attn(q, 837, seq_lens=torch.from_numpy(seq).cuda())
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention(seq_lens=seq)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    print("k bits", cache.k_bits, "attn max abs err", err, flush=True)
    assert err <= ATOL_ATTN
    assert np.abs(lse.cpu().numpy() - lref).max() <= 5e-3


@pytest.mark.parametrize("group", [1, 3, 8])
def test_gqa_groups(group):
    torch = _torch()
    case = Case(cfg=2, n_kv=2, group=group, n_tokens=200, rotation="klt", bpe_k=2.0)
    cache = case.make_cache()
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    out, _ = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), case.n)
    ref, _ = case.oracle_attention()
    assert np.abs(out.cpu().numpy() - ref).max() <= ATOL_ATTN


def test_attention_aware_key_allocation():
    """Key bits allocated by the calibration queries' rotated second moments (library: query
    weights, then a weighted calibration): same bits as the oracle's, attention within the bar."""
    torch = _torch()
    case = Case(cfg=2, n_kv=2, group=4, n_tokens=300, rotation="klt", bpe_k=2.76, aware=True)
    plain = Case(cfg=2, n_kv=2, group=4, n_tokens=300, rotation="klt", bpe_k=2.76)
    from compressed_decode_attention_head_amd import api
    for h, blob in enumerate(case.blobs(synth.K)):
        assert np.array_equal(api.calib_view(blob)["bits"].astype(np.int64), case.art[synth.K][h]["bits"])
    assert any(not np.array_equal(case.art[synth.K][h]["bits"], plain.art[synth.K][h]["bits"]) for h in range(2))
    cache = case.make_cache()
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    _check_codes(case, cache, synth.K)
    out, lse = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention()
    err = np.abs(out.cpu().numpy() - ref).max()
    print("attention-aware keys: attn max abs err", err, flush=True)
    assert err <= ATOL_ATTN
    assert np.abs(lse.cpu().numpy() - lref).max() <= 5e-3


@pytest.mark.parametrize("cfg,group,bpe,v_rot,marginal", [(2, 4, 2.76, "klt", "gauss"), (4, 7, 1.33, "wht", "t3")])
def test_nova_key_transform(cfg, group, bpe, v_rot, marginal):
    """Non-orthogonal key transform (library: query moment, then a NOVA calibration): the
    encoder's E x codes, the decoder's E^-1 y_hat, and decode attention through the query
    transform E^-T, all against the oracle."""
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    case = Case(cfg=cfg, n_kv=2, group=group, n_tokens=700, rotation="nova", v_rotation=v_rot, bpe_k=bpe,
                marginal=marginal, n_q_cal=2048)
    for h, blob in enumerate(case.blobs(synth.K)):
        c = api.calib_view(blob)
        assert int(c["rotation"]) == 3
        assert np.array_equal(c["bits"].astype(np.int64), case.art[synth.K][h]["bits"])
    cache = case.make_cache()
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    _check_codes(case, cache, synth.K)
    xh = cache.decode(synth.K, 0, case.n).cpu().numpy().astype(np.float64)
    for h in range(case.n_kv):
        ref = O.reconstruct(case.codes[synth.K][0, h], case.art[synth.K][h])
        assert np.abs(xh[0, h] - ref).max() <= 1e-6 * np.abs(ref).max(), h
    out, lse = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention()
    err = np.abs(out.cpu().numpy() - ref).max()
    lerr = np.abs(lse.cpu().numpy() - lref).max()
    print("nova keys cfg", cfg, "attn max abs err", err, "lse err", lerr, flush=True)
    assert err <= ATOL_ATTN
    assert lerr <= 5e-3


@pytest.mark.parametrize("batch,group", [(1, 4), (3, 8)])
def test_identity_rotation_end_to_end(batch, group):
    """Per-channel coding without a rotation (E = R = I): the encoder's GEMM form, the cache pass
    and both merge forms' identity branch against the oracle.  Batch 3 leaves few splits per
    sequence (the per-KV-head merge); batch 1 with 20K tokens, many (the per-q-head merge)."""
    torch = _torch()
    n = 20000 if batch == 1 else 300
    case = Case(cfg=2, n_kv=2, group=group, n_tokens=n, batch=batch, rotation="identity", bpe_k=2.76)
    cache = case.make_cache()
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    for t in (synth.K, synth.V):
        _check_codes(case, cache, t)
    out, lse = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention()
    err = np.abs(out.cpu().numpy() - ref).max()
    lerr = np.abs(lse.cpu().numpy() - lref).max()
    print("identity rotation batch", batch, "attn max abs err", err, "lse err", lerr, flush=True)
    assert err <= ATOL_ATTN
    assert lerr <= 5e-3


@pytest.mark.parametrize("dtype,cfg", [("bf16", 4), ("f32", 1)])
def test_encode_unaligned_rows_and_wht_appends(dtype, cfg):
    """Encoder paths the other cases do not take: rows that are not 16-byte aligned (a view with
    a 131-element token stride, offset by one element) go through scalar loads; a Walsh-Hadamard
    cache is filled by a prefill and three appends, so partial tiles keep their earlier tokens."""
    torch = _torch()
    case = Case(cfg=cfg, n_kv=2, group=4, n_tokens=300, dtype=dtype, rotation="wht", bpe_k=1.33 if cfg == 4 else 2.0)
    for t in (synth.K, synth.V):
        cache = case.make_cache(capacity=320)
        x = case.torch_x(t)
        big = torch.zeros((case.batch, case.n_kv, case.n, 131), dtype=x.dtype, device=x.device)
        big[..., 1:129] = x
        view = big[..., 1:129]
        assert view.stride(2) == 131 and (view.data_ptr() % 16) != 0
        cache.encode(t, view)
        torch.cuda.synchronize()
        _check_codes(case, cache, t)
        cache2 = case.make_cache(capacity=320)
        off = 0
        for step in (100, 1, 7, 192):
            cache2.encode(t, x[:, :, off:off + step], token_offset=off)
            off += step
        torch.cuda.synchronize()
        assert torch.equal(cache.codes(t), cache2.codes(t))


@pytest.mark.parametrize("cfg,bpe,aware", [(2, 2.0, True), (2, 2.76, True), (3, 4.0, False)])
def test_joint_kv_split_cache(cfg, bpe, aware):
    """A layer calibrated with the joint K/V split (library: query weights, split, calibration at
    B_K and B_V) at 2 x 256, 2 x 353 (attention-aware keys) and 2 x 512 bits: the split equals
    the oracle's (both limited to the 512 bits the summed-code cache pass reads, which binds at
    the last two budgets), and the calibrate -> encode -> decode attention chain matches the
    oracle."""
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    probe = Case(cfg=cfg, n_kv=2, group=4, n_tokens=64, rotation="klt", bpe_k=bpe, aware=aware)
    kb = probe.blobs(synth.K)
    vb = probe.blobs(synth.V)
    w = np.stack([api.query_channel_weights(kb[h], probe.q_cal[h]) for h in range(2)]) if aware else None
    total = 2 * O.bits_budget(bpe, 128)
    bk, bv = api.joint_kv_split(kb, vb, total, k_weight=w)
    want = O.joint_kv_split([a["sigma2"] for a in probe.art[synth.K]], [a["sigma2"] for a in probe.art[synth.V]],
                            [O.value_term_weight(a["C"]) for a in probe.art[synth.V]], total,
                            k_weight=[a["weight"] for a in probe.art[synth.K]] if aware else None, tensor_cap=512)
    assert (bk, bv) == want[:2] and max(bk, bv) <= 512
    case = Case(cfg=cfg, n_kv=2, group=4, n_tokens=500, rotation="klt", bpe_k=bk / 128, bpe_v=bv / 128,
                aware=aware)
    cache = case.make_cache()
    assert (cache.k_bits, cache.v_bits) == (bk, bv)
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    for t in (synth.K, synth.V):
        _check_codes(case, cache, t)
    out, lse = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), case.n)
    torch.cuda.synchronize()
    ref, lref = case.oracle_attention()
    err = np.abs(out.cpu().numpy() - ref).max()
    print("joint split", bk, bv, "attn max abs err", err, flush=True)
    assert err <= ATOL_ATTN
    assert np.abs(lse.cpu().numpy() - lref).max() <= 5e-3


def test_zero_bit_tensors():
    """All K channels at 0 bits: uniform softmax; all V channels at 0 bits: output = mu_V."""
    torch = _torch()
    for bk, bv in ((0.0, 2.0), (2.0, 0.0)):
        case = Case(cfg=2, n_kv=1, group=4, n_tokens=150, rotation="klt", bpe_k=bk, bpe_v=bv)
        cache = case.make_cache()
        for t in (synth.K, synth.V):
            cache.encode(t, case.torch_x(t))
        out, _ = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), case.n)
        ref, _ = case.oracle_attention()
        assert np.abs(out.cpu().numpy() - ref).max() <= ATOL_ATTN, (bk, bv)
        # the fused K+V encode skips the 0-bit tensor the same way
        fused = case.make_cache()
        fused.encode_kv(case.torch_x(synth.K), case.torch_x(synth.V))
        torch.cuda.synchronize()
        for t in (synth.K, synth.V):
            assert torch.equal(fused.codes(t), cache.codes(t)), (bk, bv, t)


def test_append_matches_one_shot_pack():
    """Prefill 100 tokens, then append 1, 7 and 20 tokens: words equal the one-shot pack."""
    torch = _torch()
    case = Case(cfg=3, n_kv=2, group=4, n_tokens=128, batch=2, rotation="klt", bpe_k=4.0)
    cache = case.make_cache(capacity=192)
    for t in (synth.K, synth.V):
        x = case.torch_x(t)
        cache.encode(t, x[:, :, :100])
        off = 100
        for step in (1, 7, 20):
            cache.encode(t, x[:, :, off:off + step], token_offset=off)
            off += step
    torch.cuda.synchronize()
    case.n = 128
    for t in (synth.K, synth.V):
        _check_codes(case, cache, t)
    out, _ = cache.decode_attn(torch.from_numpy(case.q.astype(np.float32)).cuda(), 128)
    ref, _ = case.oracle_attention()
    assert np.abs(out.cpu().numpy() - ref).max() <= ATOL_ATTN


@pytest.mark.parametrize("dtype,rotation,quant", [("bf16", "klt", "uniform"), ("f32", "klt", "uniform"),
                                                  ("bf16", "nova", "uniform"), ("bf16", "klt", "lloyd-max")])
def test_small_appends_cross_half_tiles(dtype, rotation, quant):
    """Appends of 1 to 8 tokens (launches that small transform on the vector ALU instead of the
    fp64 MFMA) that start and end on both sides of half-tile and tile boundaries, onto KLT and
    NOVA caches and Lloyd-Max codes: K and V words equal a one-shot encode of the same rows, and
    the codes match the oracle's."""
    torch = _torch()
    case = Case(cfg=3, n_kv=2, group=4, n_tokens=200, batch=2, dtype=dtype, rotation=rotation, bpe_k=4.0,
                quant_k=quant, quant_v=quant, v_rotation="klt")     # NOVA is a key transform
    steps = [27, 1, 2, 3, 8, 8, 7, 8, 5, 1, 6, 8, 8, 8, 4, 96]
    assert sum(steps) == case.n
    for t in (synth.K, synth.V):
        x = case.torch_x(t)
        whole = case.make_cache(capacity=256)
        whole.encode(t, x)
        parts = case.make_cache(capacity=256)
        off = 0
        for n in steps:
            parts.encode(t, x[:, :, off:off + n], token_offset=off)
            off += n
        torch.cuda.synchronize()
        assert torch.equal(whole.codes(t), parts.codes(t)), t
        _check_codes(case, parts, t)


@pytest.mark.parametrize("rotation,cfg,bpe,marginal", [("klt", 3, 4.0, "gauss"), ("wht", 4, 1.33, "t3")])
def test_encode_kv_equals_two_encodes(rotation, cfg, bpe, marginal):
    """aatc_encode_kv (K and V in one launch) writes the same words as aatc_encode of K and of V,
    through a prefill and appends of 1, 7 and 3 tokens (the small-launch form for KLT) and a
    longer one."""
    torch = _torch()
    case = Case(cfg=cfg, n_kv=2, group=4, n_tokens=300, batch=2, rotation=rotation, bpe_k=bpe, marginal=marginal)
    xk, xv = case.torch_x(synth.K), case.torch_x(synth.V)
    two, one = case.make_cache(capacity=320), case.make_cache(capacity=320)
    off = 0
    for n in (100, 1, 7, 3, 189):
        two.encode(synth.K, xk[:, :, off:off + n], token_offset=off)
        two.encode(synth.V, xv[:, :, off:off + n], token_offset=off)
        one.encode_kv(xk[:, :, off:off + n], xv[:, :, off:off + n], token_offset=off)
        off += n
    torch.cuda.synchronize()
    for t in (synth.K, synth.V):
        assert torch.equal(two.codes(t), one.codes(t)), t
        _check_codes(case, one, t)


def test_device_error_paths():
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    case = Case(cfg=2, n_kv=1, group=4, n_tokens=64, rotation="klt", bpe_k=2.0)
    cache = case.make_cache()
    x = case.torch_x(synth.K)
    with pytest.raises(api.AatcError) as e:
        cache.encode(0, x, token_offset=10)            # beyond capacity
    assert e.value.name == "AATC_ERR_INVALID_ARGUMENT"
    with pytest.raises(api.AatcError) as e:
        cache.encode_kv(x, case.torch_x(synth.V), token_offset=10)
    assert e.value.name == "AATC_ERR_INVALID_ARGUMENT"
    q = torch.zeros((1, 9, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(api.AatcError) as e:
        cache.decode_attn(q, 64)                        # group 9 > 8
    assert e.value.name == "AATC_ERR_UNSUPPORTED"
    q = torch.zeros((1, 4, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.AatcError) as e:
        cache.decode_attn(q, 64, workspace=ws)
    assert e.value.name == "AATC_ERR_BUFFER_TOO_SMALL"
    with pytest.raises(api.AatcError) as e:
        cache.decode_attn(q, 128)                       # longer than capacity
    assert e.value.name == "AATC_ERR_INVALID_ARGUMENT"


@pytest.mark.parametrize("avg_bits", [2.76, 1.0])
def test_segments_tiers_match_oracle(avg_bits):
    """Token tiers -> coded tier-2 and tier-4 caches (own water-filling, same rotation) + raw
    bf16 tier-16 tokens; tier-0 tokens evicted; one softmax over the union."""
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    cfg, n_kv, group, n = 5, 2, 4, 900
    n_q = n_kv * group
    cal = {t: [synth.draw(cfg, 0, h, t, "calib", 1024) for h in range(n_kv)] for t in (synth.K, synth.V)}
    x = {t: np.stack([synth.draw(cfg, 0, h, t, "context", n) for h in range(n_kv)]) for t in (synth.K, synth.V)}
    arts = {(tau, t): [O.calibrate(c, "klt", float(tau)) for c in cal[t]] for tau in (2, 4) for t in (synth.K, synth.V)}
    tiers = []
    for h in range(n_kv):
        dist = O.tier_distortions([arts[(2, synth.K)][h]["sigma2"], arts[(2, synth.V)][h]["sigma2"]], 128)
        tiers.append(O.token_tiers(synth.zipf_mass(cfg, 0, h, n), dist, 128, avg_bits))
    idx = {tau: [np.nonzero(tiers[h] == tau)[0] for h in range(n_kv)] for tau in (0, 2, 4, 16)}
    if avg_bits < 2:
        assert sum(len(i) for i in idx[0]) > 0          # some tokens are evicted
    q = synth.queries(cfg, 0, n_q, n_kv, [x[synth.K][h] for h in range(n_kv)])

    segs, keep = [], []
    for tau in (2, 4, 16):
        counts = [len(idx[tau][h]) for h in range(n_kv)]
        cap = max(64, -(-max(counts) // 64) * 64)
        sl = torch.tensor([counts], dtype=torch.int32, device="cuda")
        xs = {t: np.zeros((1, n_kv, cap, 128), dtype=np.float32) for t in (synth.K, synth.V)}
        for t in (synth.K, synth.V):
            for h in range(n_kv):
                xs[t][0, h, :counts[h]] = x[t][h][idx[tau][h]]
        if tau == 16:
            kr = torch.from_numpy(xs[synth.K]).to(torch.bfloat16).cuda()
            vr = torch.from_numpy(xs[synth.V]).to(torch.bfloat16).cuda()
            keep += [kr, vr, sl]
            segs.append({"k_raw": kr, "v_raw": vr, "seq_lens": sl, "max_seq_len": max(counts)})
        else:
            blobs = {t: [api.calibrate(synth.bf16_bits(c), "klt", float(tau)) for c in cal[t]] for t in (synth.K, synth.V)}
            cache = api.CompressedKVCache(blobs[synth.K], blobs[synth.V], 1, cap)
            for t in (synth.K, synth.V):
                cache.encode(t, torch.from_numpy(xs[t]).to(torch.bfloat16).cuda())
            keep += [cache, sl]
            segs.append({"cache": cache, "seq_lens": sl, "max_seq_len": max(counts)})
    qt = torch.from_numpy(q[None].astype(np.float32)).cuda()
    out, lse = api.decode_attn_segments(segs, qt, 1, n_kv)
    torch.cuda.synchronize()

    ref = np.zeros((n_q, 128))
    lref = np.zeros(n_q)
    for g in range(n_q):
        h = g // group
        parts = []
        for tau in (2, 4):
            ii = idx[tau][h]
            rec = [O.reconstruct(O.encode_codes(x[t][h][ii], arts[(tau, t)][h]), arts[(tau, t)][h])
                   for t in (synth.K, synth.V)]
            parts.append((rec[0], rec[1]))
        parts.append((x[synth.K][h][idx[16][h]], x[synth.V][h][idx[16][h]]))
        ref[g], lref[g] = O.segment_attention(q[g], parts)
    err = np.abs(out[0].cpu().numpy() - ref).max()
    lerr = np.abs(lse[0].cpu().numpy() - lref).max()
    print("segments", avg_bits, [[len(i) for i in idx[tau]] for tau in (0, 2, 4, 16)], "err", err, lerr, flush=True)
    assert err <= ATOL_ATTN, err
    assert lerr <= 5e-3, lerr

    # the same call captured in a graph, replayed with eager work (another call, which reuses
    # nothing of the graph's buffers) between the replays, equals the eager result
    ws = torch.empty(api.decode_attn_segments_workspace_bytes(segs, 1, n_kv, n_q), dtype=torch.uint8, device="cuda")
    go, gl = torch.empty_like(out), torch.empty_like(lse)
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        api.decode_attn_segments(segs, qt, 1, n_kv, workspace=ws, out=go, lse=gl)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.decode_attn_segments(segs, qt, 1, n_kv, workspace=ws, out=go, lse=gl)
    for rep in range(3):
        go.fill_(float("nan"))
        gl.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(go, out) and torch.equal(gl, lse), rep
        api.decode_attn_segments(segs, qt * 0.5, 1, n_kv)
        torch.cuda.synchronize()
    print("segments graph replays equal the eager call", flush=True)


def test_segments_raw_tier_appends_64_steps():
    """The tiered workload's decode loop: after prefill (tiers from the oracle's solver at 2.76
    bits per element), 64 steps each append one token per KV head to the raw bf16 tier (a row
    write and a length increment on the device) and run the multi-segment decode attention; the
    results of steps 1, 32 and 64 match the oracle's segment attention with the appended tokens."""
    torch = _torch()
    from compressed_decode_attention_head_amd import api
    cfg, n_kv, group, n, steps = 5, 2, 4, 600, 64
    n_q = n_kv * group
    cal = {t: [synth.draw(cfg, 0, h, t, "calib", 1024) for h in range(n_kv)] for t in (synth.K, synth.V)}
    x = {t: np.stack([synth.draw(cfg, 0, h, t, "context", n + steps) for h in range(n_kv)]) for t in (synth.K, synth.V)}
    arts = {(tau, t): [O.calibrate(c, "klt", float(tau)) for c in cal[t]] for tau in (2, 4) for t in (synth.K, synth.V)}
    tiers = []
    for h in range(n_kv):
        dist = O.tier_distortions([arts[(2, synth.K)][h]["sigma2"], arts[(2, synth.V)][h]["sigma2"]], 128)
        tiers.append(O.token_tiers(synth.zipf_mass(cfg, 0, h, n), dist, 128, 2.76))
    idx = {tau: [np.nonzero(tiers[h] == tau)[0] for h in range(n_kv)] for tau in (2, 4, 16)}
    q = synth.queries(cfg, 0, n_q, n_kv, [x[synth.K][h][:n] for h in range(n_kv)])
    segs, keep = [], []
    for tau in (2, 4, 16):
        counts = [len(idx[tau][h]) for h in range(n_kv)]
        cap = max(64, -(-(max(counts) + (steps if tau == 16 else 0)) // 64) * 64)
        xs = {t: np.zeros((1, n_kv, cap, 128), dtype=np.float32) for t in (synth.K, synth.V)}
        for t in (synth.K, synth.V):
            for h in range(n_kv):
                xs[t][0, h, :counts[h]] = x[t][h][idx[tau][h]]
        sl = torch.tensor([counts], dtype=torch.int32, device="cuda")
        if tau == 16:
            kr = torch.from_numpy(xs[synth.K]).to(torch.bfloat16).cuda()
            vr = torch.from_numpy(xs[synth.V]).to(torch.bfloat16).cuda()
            keep += [kr, vr, sl]
            raw = (kr, vr, torch.tensor(counts, dtype=torch.int64, device="cuda"), sl)
            segs.append({"k_raw": kr, "v_raw": vr, "seq_lens": sl, "max_seq_len": max(counts) + steps})
        else:
            blobs = {t: [api.calibrate(synth.bf16_bits(c), "klt", float(tau)) for c in cal[t]] for t in (synth.K, synth.V)}
            cache = api.CompressedKVCache(blobs[synth.K], blobs[synth.V], 1, cap)
            for t in (synth.K, synth.V):
                cache.encode(t, torch.from_numpy(xs[t]).to(torch.bfloat16).cuda())
            keep += [cache, sl]
            segs.append({"cache": cache, "seq_lens": sl, "max_seq_len": max(counts)})
    kr, vr, base, sl = raw
    new = {t: torch.from_numpy(np.ascontiguousarray(x[t][:, n:n + steps]).astype(np.float32)).to(torch.bfloat16).cuda()
           for t in (synth.K, synth.V)}
    heads = torch.arange(n_kv, device="cuda")
    qt = torch.from_numpy(q[None].astype(np.float32)).cuda()
    coded = {}
    for h in range(n_kv):
        coded[h] = []
        for tau in (2, 4):
            ii = idx[tau][h]
            rec = [O.reconstruct(O.encode_codes(x[t][h][ii], arts[(tau, t)][h]), arts[(tau, t)][h]) for t in (synth.K, synth.V)]
            coded[h].append((rec[0], rec[1]))
    for s_ in range(steps):
        kr[0, heads, base + s_] = new[synth.K][:, s_]
        vr[0, heads, base + s_] = new[synth.V][:, s_]
        sl += 1
        out, lse = api.decode_attn_segments(segs, qt, 1, n_kv)
        if s_ + 1 in (1, 32, 64):
            torch.cuda.synchronize()
            o, l = out[0].cpu().numpy(), lse[0].cpu().numpy()
            err = lerr = 0.0
            for g in range(n_q):
                h = g // group
                rawk = np.concatenate([x[synth.K][h][idx[16][h]], x[synth.K][h][n:n + s_ + 1]])
                rawv = np.concatenate([x[synth.V][h][idx[16][h]], x[synth.V][h][n:n + s_ + 1]])
                ref, lref = O.segment_attention(q[g], coded[h] + [(rawk, rawv)])
                err, lerr = max(err, float(np.abs(o[g] - ref).max())), max(lerr, abs(float(l[g]) - lref))
            print("raw-tier append step %d: max abs err %.2e, lse err %.2e" % (s_ + 1, err, lerr), flush=True)
            assert err <= ATOL_ATTN and lerr <= 5e-3


@pytest.mark.parametrize("quant", ["uniform", "lloyd-max"])
def test_bf16_queries(quant):
    """q in bf16 (the call widens it to fp32 in its workspace) gives the same outputs, bit for bit,
    as the fp32 widening of the same values, through aatc_decode_attn, the no-alloc entry point and
    partial + merge, on the summed-code pass and on the level pass; and it matches the oracle on
    the bf16 values."""
    torch = _torch()
    case = Case(cfg=4, n_kv=2, group=7, n_tokens=900, rotation="wht", bpe_k=1.33, marginal="t3",
                quant_k=quant, quant_v=quant)
    cache = case.make_cache()
    for t in (synth.K, synth.V):
        cache.encode(t, case.torch_x(t))
    qb = torch.from_numpy(case.q.astype(np.float32)).cuda().to(torch.bfloat16)
    qf = qb.float()
    o1, l1 = cache.decode_attn(qb, case.n)
    o2, l2 = cache.decode_attn(qf, case.n)
    o3 = torch.empty_like(o2)
    l3 = torch.empty_like(l2)
    cache.decode_attn_noalloc(qb, case.n, o3, l3)
    ws = cache.new_workspace(case.n_q, case.n)
    cache.decode_attn_partial(qb, case.n, ws)
    o4, l4 = cache.decode_attn_merge(case.n_q, case.n, ws, torch.empty_like(o2), torch.empty_like(l2))
    torch.cuda.synchronize()
    for o, l in ((o1, l1), (o3, l3), (o4, l4)):
        assert torch.equal(o, o2) and torch.equal(l, l2)
    ref, lref = case.oracle_attention(q=qf.cpu().numpy().astype(np.float64))
    assert np.abs(o1.cpu().numpy() - ref).max() <= ATOL_ATTN
    assert np.abs(l1.cpu().numpy() - lref).max() <= 5e-3

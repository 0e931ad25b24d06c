"""CPU tests of libaatc's host side: exports, calibration parity with the oracle, error paths.

No GPU is touched: only aatc_calibrate / aatc_calib_validate / size helpers are called.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle as O
import synth
from compressed_decode_attention_head_amd import _native as N
from compressed_decode_attention_head_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    return N.lib()


def test_exports_match_header(L):
    hdr = open(os.path.join(ROOT, "include", "aatc.h")).read()
    names = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(aatc_[a-z_0-9]+)\(", hdr, re.M))
    assert names, "no declarations parsed"
    assert names == set(N.EXPORTS), names ^ set(N.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_struct_size_and_sizes(L):
    assert L.aatc_calib_bytes(128) == N.CALIB_DTYPE.itemsize
    assert L.aatc_calib_bytes(64) == 0
    assert [L.aatc_bits_budget(b, 128) for b in (2.0, 2.76, 4.0, 1.33, 0.0, 8.0)] == [256, 353, 512, 170, 0, 1024]
    assert L.aatc_bits_budget(8.01, 128) == -1 and L.aatc_bits_budget(-1.0, 128) == -1
    assert L.aatc_packed_bytes(170, 131072) == 131072 // 64 * 8 * 170
    assert L.aatc_packed_bytes(353, 65) == 2 * 8 * 353


def _cal(cfg, head=0, tensor=synth.K, dtype="bf16", marginal="gauss"):
    return synth.draw(cfg, 0, head, tensor, "calib", 1024, dtype=dtype, marginal=marginal)


def _bits16(x):
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("cfg,rot,bpe,tensor", [(1, "klt", 2.0, synth.K), (2, "klt", 2.76, synth.V),
                                                (3, "klt", 4.0, synth.K), (4, "wht", 1.33, synth.V),
                                                (2, "identity", 2.76, synth.K)])
def test_calibrate_matches_oracle(cfg, rot, bpe, tensor):
    dtype = "f32" if cfg == 1 else "bf16"
    x = _cal(cfg, 1, tensor, dtype=dtype, marginal="t3" if cfg == 4 else "gauss")
    blob = api.calibrate(x if dtype == "f32" else _bits16(x), rot, bpe)
    api.validate(blob)
    c = api.calib_view(blob)
    ref = O.calibrate(x, rot, bpe)
    assert int(c["total_bits"]) == ref["B"]
    assert np.array_equal(c["bits"].astype(np.int64), ref["bits"])
    assert np.abs(c["mu"] - ref["mu"]).max() < 1e-13
    R = c["R"].reshape(128, 128)
    assert np.abs(R - ref["R"]).max() < 1e-9
    assert np.abs(c["sigma2"] - ref["sigma2"]).max() < 1e-12 * ref["sigma2"].max()
    assert np.abs(c["o"] - ref["o"]).max() < 1e-10 * (1 + np.abs(ref["o"]).max())
    coded = ref["bits"] > 0
    assert np.all(np.abs(c["delta"][coded] / ref["delta"][coded] - 1) < 1e-11)
    assert np.array_equal(c["delta"][~coded], np.zeros((~coded).sum()))
    assert np.array_equal(c["inv_delta"][coded], 1.0 / c["delta"][coded])
    assert np.array_equal(c["R32"], R.astype(np.float32).ravel())


@pytest.mark.parametrize("cfg,rot,bpe", [(2, "klt", 2.76), (4, "wht", 1.33)])
def test_attention_aware_calibration_matches_oracle(cfg, rot, bpe):
    """Query weights and the weighted allocation: library (C++) against the oracle."""
    x = _cal(cfg, 1, synth.K, marginal="t3" if cfg == 4 else "gauss")
    rng = np.random.default_rng(cfg)
    ref0 = O.calibrate(x, rot, bpe)
    # calibration queries: a few dominant rotated directions plus a floor
    qw = np.where(np.arange(128) % 7 == 0, 4.0, 0.3)
    q = (rng.standard_normal((256, 128)) * qw) @ ref0["R"]
    ref = O.calibrate(x, rot, bpe, q_cal=q)
    blob0 = api.calibrate(_bits16(x), rot, bpe)
    w = api.query_channel_weights(blob0, q)
    assert np.abs(w - ref["weight"]).max() < 1e-10 * ref["weight"].max()
    blob = api.calibrate(_bits16(x), rot, bpe, channel_weight=w)
    api.validate(blob)
    c = api.calib_view(blob)
    assert np.array_equal(c["bits"].astype(np.int64), ref["bits"])
    assert int(c["total_bits"]) == ref["B"]
    assert not np.array_equal(ref["bits"], ref0["bits"])      # the weights moved bits
    # same statistics and rotation as the unweighted blob; only the allocation differs
    assert np.array_equal(c["R"], api.calib_view(blob0)["R"])


def _nova_queries(seed, n, scales):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 128)) * scales) @ synth.haar_orthogonal(rng, 128)


def test_query_moment_matches_numpy():
    q = _nova_queries(3, 777, np.geomspace(0.05, 3.0, 128))
    for qq in (q, q.astype(np.float32), _bits16(synth.round_bf16(q))):
        want = O.query_moment(qq.astype(np.float64) if qq.dtype != np.uint16
                              else (qq.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        got = api.query_moment(qq)
        assert np.array_equal(got, got.T)
        assert np.abs(got - want).max() < 1e-13 * np.abs(want).max()


@pytest.mark.parametrize("cfg,bpe,scales", [(2, 2.76, "geo"), (4, 1.33, "ramp"), (1, 2.0, "geo")])
def test_nova_calibration_matches_oracle(cfg, bpe, scales):
    """The non-orthogonal key transform: library (C++, Jacobi) against the oracle (LAPACK)."""
    dtype = "f32" if cfg == 1 else "bf16"
    x = _cal(cfg, 1, synth.K, dtype=dtype, marginal="t3" if cfg == 4 else "gauss")
    sc = np.geomspace(0.05, 3.0, 128) if scales == "geo" else np.linspace(0.1, 3.0, 128)
    q = _nova_queries(cfg, 2048, sc)
    ref = O.calibrate(x, "nova", bpe, q_cal=q)
    blob = api.calibrate(x if dtype == "f32" else _bits16(x), "nova", bpe, query_moment=api.query_moment(q))
    api.validate(blob)
    c = api.calib_view(blob)
    assert int(c["rotation"]) == 3 and int(c["total_bits"]) == ref["B"]
    assert np.array_equal(c["bits"].astype(np.int64), ref["bits"])
    E, R = c["E"].reshape(128, 128), c["R"].reshape(128, 128)
    assert np.abs(E - ref["E"]).max() < 1e-8 * np.abs(ref["E"]).max()
    assert np.abs(R - ref["R"]).max() < 1e-8 * np.abs(ref["R"]).max()
    assert np.abs(R @ E.T - np.eye(128)).max() < 1e-9
    assert np.abs(c["sigma2"] - ref["sigma2"]).max() < 1e-10 * ref["sigma2"].max()
    assert np.abs(c["o"] - ref["o"]).max() < 1e-9 * (1 + np.abs(ref["o"]).max())
    coded = ref["bits"] > 0
    assert np.all(np.abs(c["delta"][coded] / ref["delta"][coded] - 1) < 1e-9)
    assert np.array_equal(c["R32"], R.astype(np.float32).ravel())


def test_orthogonal_blobs_encode_with_r():
    """Every other rotation stores E = R."""
    x = _cal(2, 0, synth.K)
    for rot in ("klt", "wht", "identity"):
        c = api.calib_view(api.calibrate(_bits16(x), rot, 2.0))
        assert np.array_equal(c["E"], c["R"])


def test_nova_errors(L):
    x = _bits16(_cal(2, 0, synth.K))
    with pytest.raises(N.AatcError) as e:
        api.calibrate(x, "nova", 2.0)                                   # no query moment
    assert e.value.status == 1
    m = api.query_moment(_nova_queries(1, 300, np.ones(128)))
    bad = m.copy()
    bad[3, 7] += 1e-3
    with pytest.raises(N.AatcError) as e:
        api.calibrate(x, "nova", 2.0, query_moment=bad)                 # not symmetric
    assert e.value.status == 1
    bad = m.copy()
    bad[5, 5] = np.nan
    with pytest.raises(N.AatcError) as e:
        api.calibrate(x, "nova", 2.0, query_moment=bad)
    assert e.value.status == 4
    with pytest.raises(N.AatcError) as e:
        api.calibrate(x, "nova", 2.0, query_moment=np.zeros((128, 128)))
    assert e.value.status == 4
    with pytest.raises(N.AatcError) as e:
        api.query_moment(np.full((3, 128), np.inf, dtype=np.float32))
    assert e.value.status == 4
    out = np.zeros((128, 128))
    qq = np.ones((4, 128), dtype=np.float32)
    assert L.aatc_query_moment(qq.ctypes.data, 0, 0, 128, out.ctypes.data) == 1
    assert L.aatc_query_moment(qq.ctypes.data, 0, 4, 100, out.ctypes.data) == 1
    assert L.aatc_query_moment(None, 0, 4, 128, out.ctypes.data) == 1


@pytest.mark.parametrize("cfg,rot,bpe,aware", [(2, "klt", 2.0, True), (4, "wht", 1.33, True), (3, "klt", 4.0, False),
                                               (2, "klt", 2.76, True), (3, "klt", 4.0, True)])
def test_joint_kv_split_matches_oracle(cfg, rot, bpe, aware):
    """The layer's K/V split: library (C++) against the oracle on the same blobs' statistics,
    both limited to the 512 bits per vector that the summed-code cache pass reads."""
    n_kv = 3
    calk = [_cal(cfg, h, synth.K) for h in range(n_kv)]
    calv = [_cal(cfg, h, synth.V) for h in range(n_kv)]
    kb = [api.calibrate(_bits16(c), rot, bpe) for c in calk]
    vb = [api.calibrate(_bits16(c), rot, bpe) for c in calv]
    ka = [O.calibrate(c, rot, bpe) for c in calk]
    va = [O.calibrate(c, rot, bpe) for c in calv]
    w = None
    if aware:
        rng = np.random.default_rng(cfg)
        qs = [rng.standard_normal((400, 128)) * np.linspace(0.2, 3.0, 128) for _ in range(n_kv)]
        w = np.stack([api.query_channel_weights(kb[h], qs[h]) for h in range(n_kv)])
    T = 2 * O.bits_budget(bpe, 128)
    got = api.joint_kv_split(kb, vb, T, k_weight=w)
    want = O.joint_kv_split([a["sigma2"] for a in ka], [a["sigma2"] for a in va],
                            [O.value_term_weight(a["C"]) for a in va], T,
                            k_weight=None if w is None else list(w), tensor_cap=512)
    assert got == want[:2], (got, want)
    assert sum(got) == T and max(got) <= 512


def test_joint_kv_split_decode_cap_binds():
    """At 4 bits per element the unconstrained split gives V more than the 512 bits per vector
    the summed-code cache pass reads; the library's split is then the cap's corner (512, 512), which the
    oracle's capped split also gives, and a budget past 2 x 512 is refused."""
    n_kv = 3
    calk = [_cal(3, h, synth.K) for h in range(n_kv)]
    calv = [_cal(3, h, synth.V) for h in range(n_kv)]
    ka = [O.calibrate(c, "klt", 4.0) for c in calk]
    va = [O.calibrate(c, "klt", 4.0) for c in calv]
    args = ([a["sigma2"] for a in ka], [a["sigma2"] for a in va], [O.value_term_weight(a["C"]) for a in va], 1024)
    free = O.joint_kv_split(*args)
    assert max(free[:2]) > 512                     # the cap is not idle at this budget
    assert O.joint_kv_split(*args, tensor_cap=512)[:2] == (512, 512)
    kb = [api.calibrate(_bits16(c), "klt", 4.0) for c in calk]
    vb = [api.calibrate(_bits16(c), "klt", 4.0) for c in calv]
    assert api.joint_kv_split(kb, vb, 1024) == (512, 512)
    with pytest.raises(N.AatcError) as e:
        api.joint_kv_split(kb, vb, 1025)
    assert e.value.name == "AATC_ERR_BUDGET"


def test_joint_kv_split_errors(L):
    x = _bits16(_cal(2, 0, synth.K))
    kb = api.calibrate(x, "klt", 2.0)
    with pytest.raises(N.AatcError) as e:
        api.joint_kv_split([kb], [kb], 2049)
    assert e.value.name == "AATC_ERR_BUDGET"
    with pytest.raises(N.AatcError) as e:
        api.joint_kv_split([kb], [kb], 256, k_weight=-np.ones((1, 128)))
    assert e.value.name == "AATC_ERR_INVALID_ARGUMENT"
    with pytest.raises(N.AatcError) as e:
        api.joint_kv_split([kb], [kb], 256, k_weight=np.full((1, 128), np.nan))
    assert e.value.name == "AATC_ERR_NUMERICAL"
    bad = kb.copy()
    bad[300] ^= 1
    with pytest.raises(N.AatcError) as e:
        api.joint_kv_split([kb], [bad], 256)
    assert e.value.name == "AATC_ERR_BAD_ARTEFACT"
    out = ctypes.c_int32()
    assert L.aatc_joint_kv_split(kb.ctypes.data, kb.ctypes.data, 0, None, 0.0, 256, ctypes.byref(out),
                                 ctypes.byref(out)) == 1
    assert api.joint_kv_split([kb], [kb], 0) == (0, 0)


def test_attention_aware_errors(L):
    x = _cal(2, 0, synth.K)
    blob = api.calibrate(_bits16(x), "klt", 2.0)
    w = np.ones(128)
    w[3] = -1.0
    with pytest.raises(N.AatcError) as e:
        api.calibrate(_bits16(x), "klt", 2.0, channel_weight=w)
    assert e.value.status == 1
    w[3] = float("nan")
    with pytest.raises(N.AatcError) as e:
        api.calibrate(_bits16(x), "klt", 2.0, channel_weight=w)
    assert e.value.status == 4
    q = np.ones((4, 128), dtype=np.float32)
    q[2, 5] = np.inf
    with pytest.raises(N.AatcError) as e:
        api.query_channel_weights(blob, q)
    assert e.value.status == 4
    bad = blob.copy()
    bad[200] ^= 1
    with pytest.raises(N.AatcError) as e:
        api.query_channel_weights(bad, np.ones((4, 128), dtype=np.float32))
    assert e.value.status == 5
    wout = np.zeros(128)
    qq = np.ones((4, 128), dtype=np.float32)
    assert L.aatc_query_channel_weights(blob.ctypes.data, blob.nbytes, qq.ctypes.data, 0, 0, 128, wout.ctypes.data) == 1
    assert L.aatc_query_channel_weights(blob.ctypes.data, blob.nbytes, qq.ctypes.data, 0, 4, 100, wout.ctypes.data) == 1


def test_quantizer_step_matches_oracle_all_widths():
    """sigma=1 channels at every width: delta/sigma must equal the oracle's g(b) to 1e-13."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4096, 128))
    x = (x - x.mean(0)) / x.std(0)
    for bpe in (1.0, 2.0, 3.0, 5.0, 8.0):
        blob = api.calibrate(x.astype(np.float64), "identity", bpe)
        c = api.calib_view(blob)
        for i in range(128):
            b = int(c["bits"][i])
            if b:
                assert abs(c["delta"][i] / math.sqrt(c["sigma2"][i]) - O.optimal_step(b)) < 1e-13


def test_noise_free_klt_pin_f64():
    q, lam, _ = synth.basis(1, 0, 0, synth.K)
    d = 128
    cols = [math.sqrt(d) * math.sqrt(lam[i]) * q[:, i] for i in range(d)]
    x = np.array(cols + [-c for c in cols])
    blob = api.calibrate(x, "klt", 2.0)
    c = api.calib_view(blob)
    R = c["R"].reshape(128, 128)
    assert np.abs(R @ R.T - np.eye(128)).max() < 1e-10
    assert np.abs(c["sigma2"] - lam).max() < 1e-12
    assert np.abs(np.abs(R @ q) - np.eye(128)).max() < 1e-10
    hist = {int(k): int(v) for k, v in zip(*np.unique(c["bits"], return_counts=True))}
    assert hist == {6: 1, 5: 4, 4: 7, 3: 19, 2: 48, 1: 49}


def test_layout_tables_match_oracle():
    x = _cal(2, 0, synth.V)
    blob = api.calibrate(_bits16(x), "klt", 2.76)
    c = api.calib_view(blob)
    bits = c["bits"].astype(np.int64)
    fields = O.v_fields(bits)
    nf = int(c["n_fields"])
    assert nf == len(fields)
    got = [(int(c["field_channel"][k]), int(c["field_shift"][k]), int(c["field_width"][k])) for k in range(nf)]
    assert got == fields
    word = np.concatenate([[0], np.cumsum([2 * f[2] for f in fields])])[:-1]
    assert np.array_equal(c["field_word"][:nf], word)
    planes = [(i, k) for i in range(128) for k in range(bits[i])]
    B = int(c["total_bits"])
    assert list(zip(c["plane_channel"][:B].tolist(), c["plane_bit"][:B].tolist())) == planes
    assert api.v_tiles(blob) == sum(-(-n // 16) for n in (int(c["n_fields4"]), int(c["n_fields2"]),
                                                         int(c["n_fields1"])))


def test_zero_variance_channels_get_no_bits():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((512, 128))
    x[:, 5] = 3.0
    x[:, 77] = -1.0
    blob = api.calibrate(x, "identity", 2.0)
    c = api.calib_view(blob)
    assert c["bits"][5] == 0 and c["bits"][77] == 0
    assert c["o"][5] == 3.0 and c["o"][77] == -1.0


def _status(fn):
    with pytest.raises(api.AatcError) as e:
        fn()
    return e.value.name


@pytest.mark.parametrize("cfg,rot,bpe", [(2, "klt", 2.76), (3, "klt", 4.0), (4, "wht", 1.33)])
def test_lloyd_max_calibration_matches_oracle(cfg, rot, bpe):
    """A Lloyd-Max blob: the same bits as the uniform one, scale = the channel's standard
    deviation, and standardized level and threshold tables of every width equal to the oracle's
    Lloyd-Max quantizer (the library solves Lloyd's conditions on its own)."""
    x = _cal(cfg, marginal="t3" if cfg == 4 else "gauss")
    blob = api.calibrate(_bits16(x), rot, bpe, quantizer="lloyd-max")
    api.validate(blob)
    v = api.calib_view(blob)
    art = O.calibrate(x, rot, bpe, quantizer="lloyd-max")
    assert int(v["quantizer"]) == 1
    assert np.array_equal(v["bits"].astype(np.int64), art["bits"])
    coded = art["bits"] > 0
    assert np.allclose(v["scale"][coded], art["scale"][coded], rtol=1e-9, atol=0)
    assert np.all(v["scale"][~coded] == 0)
    assert np.array_equal(v["inv_scale"][coded], 1.0 / v["scale"][coded])
    for b in range(1, 9):
        off, n = 2 ** b - 2, 2 ** b
        lv, th = O.lloyd_max_gaussian(b)
        assert np.allclose(v["level"][off:off + n], lv, rtol=0, atol=2e-12), b
        assert np.allclose(v["thresh"][off:off + n - 1], th, rtol=0, atol=2e-12), b
        assert np.array_equal(v["level32"][off:off + n], v["level"][off:off + n].astype(np.float32))
    u = api.calib_view(api.calibrate(_bits16(x), rot, bpe))
    assert int(u["quantizer"]) == 0 and np.array_equal(u["scale"], u["delta"])
    for b in range(1, 9):
        off, n = 2 ** b - 2, 2 ** b
        assert np.array_equal(u["level"][off:off + n], np.arange(n) - n / 2 + 0.5), b


def test_calibrate_error_paths(L):
    x = np.random.default_rng(0).standard_normal((64, 128))
    assert _status(lambda: api.calibrate(x, "klt", 8.5)) == "AATC_ERR_BUDGET"
    assert _status(lambda: api.calibrate(x, "klt", -0.5)) == "AATC_ERR_BUDGET"
    assert _status(lambda: api.calibrate(x[:1], "klt", 2.0)) == "AATC_ERR_INVALID_ARGUMENT"
    bad = x.copy()
    bad[3, 4] = np.nan
    assert _status(lambda: api.calibrate(bad, "klt", 2.0)) == "AATC_ERR_NUMERICAL"
    bad[3, 4] = np.inf
    assert _status(lambda: api.calibrate(bad, "klt", 2.0)) == "AATC_ERR_NUMERICAL"
    assert _status(lambda: api.calibrate(x[:, :64], "klt", 2.0, d=64)) == "AATC_ERR_UNSUPPORTED"
    p = N.CalibParams(128, 0, 2.0, 8, 0)
    out = np.zeros(100, dtype=np.uint8)
    assert L.aatc_calibrate(ctypes.byref(p), x.ctypes.data, 2, 64, 128, out.ctypes.data, out.nbytes) == 6
    assert L.aatc_calibrate(ctypes.byref(p), None, 2, 64, 128, out.ctypes.data, out.nbytes) == 1
    assert L.aatc_calibrate(ctypes.byref(p), x.ctypes.data, 2, 64, 100, out.ctypes.data, out.nbytes) == 1
    p = N.CalibParams(128, 0, 2.0, 9, 0)
    big = np.zeros(N.CALIB_DTYPE.itemsize, dtype=np.uint8)
    assert L.aatc_calibrate(ctypes.byref(p), x.ctypes.data, 2, 64, 128, big.ctypes.data, big.nbytes) == 3


def test_validate_detects_corruption():
    x = np.random.default_rng(0).standard_normal((256, 128))
    blob = api.calibrate(x, "klt", 2.0)
    api.validate(blob)
    for off in (0, 100, 5000, N.CALIB_DTYPE.itemsize - 70):
        b = blob.copy()
        b[off] ^= 0x40
        assert _status(lambda: api.validate(b)) == "AATC_ERR_BAD_ARTEFACT"
    assert _status(lambda: api.validate(blob[:100])) == "AATC_ERR_BUFFER_TOO_SMALL"


def test_status_strings(L):
    for s in range(8):
        assert L.aatc_status_string(s)


# ---------------------------------------------------------------- token tiers (host)
def _head_sigma2(cfg, h):
    return [O.calibrate(synth.draw(cfg, 0, h, t, "calib", 1024), "klt", 2.76)["sigma2"] for t in (synth.K, synth.V)]


def test_tier_distortions_match_oracle():
    for h in range(2):
        s2 = _head_sigma2(5, h)
        got = api.tier_distortions(s2)
        want = O.tier_distortions(s2, 128)
        assert got[3] == 0.0 and want[3] == 0.0
        assert np.allclose(got, want, rtol=1e-12, atol=0.0), (got, want)
    s2 = synth.spectrum(128)
    assert np.allclose(api.tier_distortions([s2, s2]), O.tier_distortions([s2, s2], 128), rtol=1e-12, atol=0.0)


@pytest.mark.parametrize("n,avg", [(4096, 2.76), (131072, 2.76), (4096, 0.5), (4096, 8.0), (300, 16.0),
                                   (300, 0.0)])
def test_token_tiers_match_oracle(n, avg):
    """Same distortions in, the same tier per token out (both sides follow one bisection)."""
    s2 = synth.spectrum(128)
    dist = O.tier_distortions([s2, s2], 128)
    a = synth.zipf_mass(5, 0, 0, n)
    got = api.token_tiers(a, dist, avg)
    want = O.token_tiers(a, dist, 128, avg)
    assert np.array_equal(got.astype(np.int64), want.astype(np.int64))
    assert got.astype(np.int64).sum() * 128 <= avg * n * 128


def test_token_tiers_errors(L):
    dist = np.array([1.0, 0.1, 0.01, 0.0])
    with pytest.raises(N.AatcError) as e:
        api.token_tiers(np.ones(4) / 4, dist, 17.0)
    assert e.value.name == "AATC_ERR_BUDGET"
    with pytest.raises(N.AatcError) as e:
        api.token_tiers(np.array([0.5, -0.1, 0.3, 0.3]), dist, 2.0)
    assert e.value.name == "AATC_ERR_NUMERICAL"
    with pytest.raises(N.AatcError) as e:
        api.tier_distortions([np.full(128, np.nan)])
    assert e.value.name == "AATC_ERR_NUMERICAL"


def test_dense_workspace_bytes(L):
    """One state per token chunk and q head: [states][batch*n_q][128] fp32 outputs, then
    [states][batch*n_q] fp32 lse, each padded to 256 bytes.  Chunks hold 2048 tokens, halved
    down to 256 while the grid (chunks x batch x KV heads) is below 256 workgroups."""
    def al(x):
        return -(-x // 256) * 256
    for b, n_kv, n_q, n, chunk in ((1, 4, 28, 131072, 2048), (2, 2, 8, 3000, 256), (1, 1, 1, 0, 256),
                                   (3, 1, 8, 2048, 256), (4, 8, 16, 9000, 1024), (8, 8, 8, 8200, 2048),
                                   (1, 8, 32, 3700, 256), (1, 4, 28, 65536, 1024)):
        states, bq = max(1, -(-n // chunk)), b * n_q
        assert L.aatc_decode_attn_dense_workspace_bytes(b, n_kv, n_q, n) == al(states * bq * 512) + al(states * bq * 4)
    assert L.aatc_decode_attn_dense_workspace_bytes(1, 4, 30, 100) == 0      # 30 q heads over 4 KV heads
    assert L.aatc_decode_attn_dense_workspace_bytes(1, 1, 9, 100) == 0       # group of 9
    assert L.aatc_decode_attn_dense_workspace_bytes(1, 1, 1, -1) == 0


def test_dense_argument_errors(L):
    """Every case fails host-side validation before a launch; the fake device addresses are
    never dereferenced."""
    ok = 1 << 20

    def call(k=ok, v=ok, batch=1, n_kv=1, cap=64, max_seq=64, q=ok, n_q=1, out=ok, ws=ok, ws_bytes=1 << 20):
        return N.STATUS[L.aatc_decode_attn_dense(k, v, batch, n_kv, cap, None, max_seq, q, n_q, 0.0, out, None, ws,
                                                 ws_bytes, None)]
    assert call(k=None) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(out=None) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(v=ok + 8) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(q=ok + 4) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(ws=ok + 16) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(max_seq=65) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(cap=-1, max_seq=0) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(batch=0) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(n_q=9) == "AATC_ERR_UNSUPPORTED"
    assert call(n_kv=2, n_q=3) == "AATC_ERR_INVALID_ARGUMENT"
    assert call(batch=70000) == "AATC_ERR_UNSUPPORTED"
    assert call(ws_bytes=16) == "AATC_ERR_BUFFER_TOO_SMALL"

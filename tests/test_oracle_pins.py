"""Pins of the fp64 oracle against what the pages and mathematics fix (CPU only).

Every check here is independent of the oracle's own formulas: closed forms, library
routines the oracle does not call, brute force, literature values and invariants.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy import integrate, linalg, stats

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _noise_free_tokens(q, lam):
    """2d tokens +-sqrt(d) sqrt(lambda_i) q_i: mean 0, covariance exactly Q Lambda Q^T."""
    d = q.shape[0]
    cols = [math.sqrt(d) * math.sqrt(lam[i]) * q[:, i] for i in range(d)]
    return np.array(cols + [-c for c in cols])


# ---------------------------------------------------------------- statistics / rotations
def test_calib_stats_matches_numpy_cov():
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f32")
    mu, c = O.calib_stats(x)
    assert np.allclose(mu, np.mean(x.astype(np.float64), axis=0), rtol=0, atol=1e-13)
    assert np.allclose(c, np.cov(x.astype(np.float64), rowvar=False, bias=True), rtol=1e-12, atol=1e-15)


def test_klt_orthogonal_and_decorrelating():
    x = synth.draw(2, 0, 3, synth.V, "calib", 1024, dtype="bf16")
    mu, c = O.calib_stats(x)
    r, s2 = O.rotation_klt(c)
    d = c.shape[0]
    assert np.abs(r @ r.T - np.eye(d)).max() < 1e-10
    rc = r @ c @ r.T
    assert np.abs(rc - np.diag(np.diag(rc))).max() < 1e-10 * np.abs(c).max()
    assert np.allclose(np.diag(rc), s2, rtol=0, atol=1e-12 * s2.max())
    assert abs(np.trace(c) - s2.sum()) < 1e-12 * np.trace(c)
    assert np.all(np.diff(s2) <= 0)
    # sign rule: largest-magnitude entry of each row is positive
    assert np.all(r[np.arange(d), np.argmax(np.abs(r), axis=1)] > 0)


def test_klt_noise_free_closed_form():
    q, lam, _ = synth.basis(1, 0, 0, synth.K)
    x = _noise_free_tokens(q, lam)
    mu, c = O.calib_stats(x)
    assert np.abs(mu).max() < 1e-14
    r, s2 = O.rotation_klt(c)
    assert np.abs(s2 - lam).max() < 1e-12
    assert np.abs(np.abs(r @ q) - np.eye(128)).max() < 1e-10


def test_wht_matches_scipy_hadamard():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((128, 128))
    c = a @ a.T
    r, s2 = O.rotation_wht(c)
    h = linalg.hadamard(128) / math.sqrt(128)
    assert np.array_equal(r, h)
    assert np.abs(r @ r.T - np.eye(128)).max() < 1e-12
    e0 = np.zeros(128)
    e0[0] = 1.0
    assert np.allclose(r @ e0, np.full(128, 1 / math.sqrt(128)), rtol=0, atol=1e-15)
    assert np.allclose(s2, np.diag(h @ c @ h.T), rtol=1e-12)


def test_wht_encoder_takes_exact_sums():
    """For bf16 rows every +-1 sum of H x is exact in integer units of the row's smallest power of
    two; the encoder's coefficients equal those exact sums times 1/sqrt(d) rounded to fp64, with
    one rounding, while multiplying by the rounded matrix H/sqrt(d) rounds every product and
    differs in some coefficients."""
    x = synth.draw(4, 0, 1, synth.K, "context", 64, dtype="bf16", marginal="t3").astype(np.float64)
    art = O.calibrate(synth.draw(4, 0, 1, synth.K, "calib", 1024, dtype="bf16", marginal="t3"), "wht", 1.33)
    y = O.rotate(x, art)
    h = linalg.hadamard(128).astype(np.int64)
    s = 1.0 / math.sqrt(128)
    for t in range(x.shape[0]):
        m, e = np.frexp(x[t])
        e0 = int(e[x[t] != 0].min()) - 9            # bf16: 8 significant bits
        n = np.array([int(v) for v in np.ldexp(x[t], -e0)], dtype=np.int64)
        assert np.array_equal(np.ldexp(n.astype(np.float64), e0), x[t])
        exact = h @ n                               # integer sums, no rounding
        assert np.abs(exact).max() < 2 ** 53
        want = np.ldexp(exact.astype(np.float64), e0) * s
        assert np.array_equal(y[t], want), t
    rounded = x @ (h / math.sqrt(128)).T
    assert np.any(rounded != y)


def test_wht_flattens_variances_klt_compacts():
    q, lam, _ = synth.basis(4, 0, 0, synth.K)
    c = q @ np.diag(lam) @ q.T
    _, s2w = O.rotation_wht(c)
    _, s2k = O.rotation_klt(c)
    assert s2w.max() / s2w.min() < 50.0          # Hadamard equalises variances
    assert s2k.max() / s2k.min() > 1000.0        # the KLT compacts energy
    assert s2k[:16].sum() / s2k.sum() > 0.85


def test_identity_rotation():
    c = np.diag(np.arange(1.0, 9.0))
    r, s2 = O.rotation_identity(c)
    assert np.array_equal(r, np.eye(8)) and np.array_equal(s2, np.arange(1.0, 9.0))


# ---------------------------------------------------------------- water-filling
def test_budget_integerisation():
    assert [O.bits_budget(b, 128) for b in (2.0, 2.76, 4.0, 1.33)] == [256, 353, 512, 170]


def _check_certificate(s2, bits, max_bits=8):
    d = len(s2)
    for i in range(d):
        if bits[i] == 0:
            continue
        for j in range(d):
            if bits[j] >= max_bits:
                continue
            # moving one bit from i to j cannot help
            gain_j = s2[j] * 4.0 ** (-bits[j])             # marginal value of j's next bit
            loss_i = s2[i] * 4.0 ** (-(bits[i] - 1))       # value of i's last bit
            assert gain_j <= loss_i * (1 + 1e-15)


@pytest.mark.parametrize("budget", [0, 1, 37, 170, 256, 353, 512, 1000, 1024])
def test_waterfill_sum_range_certificate(budget):
    x = synth.draw(2, 0, 0, synth.K, "calib", 1024, dtype="bf16")
    _, c = O.calib_stats(x)
    _, s2 = O.rotation_klt(c)
    b = O.waterfill_bits(s2, budget)
    assert b.sum() == budget and b.min() >= 0 and b.max() <= 8
    assert np.all(np.diff(b) <= 0)       # descending variances -> non-increasing bits
    _check_certificate(s2, b)


def test_waterfill_bruteforce_d4():
    rng = np.random.default_rng(7)
    for trial in range(6):
        s2 = np.sort(rng.lognormal(0, 2, 4))[::-1]
        if trial == 5:
            s2 = np.array([1.0, 0.25, 0.25, 0.0])     # exact ties and a dead channel
        for budget in range(0, 33):
            best = min(
                (a for a in itertools.product(range(9), repeat=4) if sum(a) == budget),
                key=lambda a: sum(s2[i] * 4.0 ** (-a[i]) for i in range(4)))
            got = O.waterfill_bits(s2, budget)
            dist_best = sum(s2[i] * 4.0 ** (-best[i]) for i in range(4))
            dist_got = sum(s2[i] * 4.0 ** (-got[i]) for i in range(4))
            assert dist_got <= dist_best * (1 + 1e-15) + 1e-300


def test_waterfill_tie_rule_prefers_lower_channel():
    s2 = np.array([1.0, 1.0, 1.0])
    assert list(O.waterfill_bits(s2, 4)) == [2, 1, 1]
    s2 = np.array([1.0, 4.0])            # 4 * 4^-1 == 1 * 4^0: ties between (1,1) and (0,0)
    assert list(O.waterfill_bits(s2, 2)) == [1, 1]


def test_waterfill_vs_continuous_closed_form():
    rng = np.random.default_rng(3)
    for _ in range(40):
        d = 128
        s2 = np.sort(rng.lognormal(0, 2.5, d))[::-1]
        budget = int(rng.integers(20, 600))
        theta, dist, rate = O.waterfill_theta(s2, budget)
        assert abs(rate.sum() - budget) < 1e-9
        assert np.allclose(dist, np.minimum(theta, s2), rtol=0, atol=0)
        b = O.waterfill_bits(s2, budget)
        unc = (b < 8) & (b > 0)
        assert np.all(np.abs(b[unc] - rate[unc]) <= 1.0 + 1e-12)


def test_waterfill_noise_free_histograms():
    """Histograms on sigma^2 = i^-1.5 (derived with the tie rule; two budgets hit exact ties)."""
    s2 = synth.spectrum(128)
    want = {256: {6: 1, 5: 4, 4: 7, 3: 19, 2: 48, 1: 49},
            353: {7: 1, 6: 2, 5: 6, 4: 15, 3: 36, 2: 68},
            512: {8: 1, 7: 4, 6: 7, 5: 19, 4: 48, 3: 49},
            170: {6: 1, 5: 1, 4: 4, 3: 10, 2: 25, 1: 63, 0: 24}}
    for budget, hist in want.items():
        b = O.waterfill_bits(s2, budget)
        got = {int(k): int(v) for k, v in zip(*np.unique(b, return_counts=True))}
        assert got == hist, (budget, got)


def test_waterfill_rejects_bad_budget():
    with pytest.raises(ValueError):
        O.waterfill_bits(np.ones(4), 33)
    with pytest.raises(ValueError):
        O.waterfill_bits(np.ones(4), -1)


# ---------------------------------------------------------------- attention-aware allocation
def test_weighted_waterfill_bruteforce_d4():
    """sum_i w_i sigma_i^2 4^-b_i at the allocation equals the exhaustive minimum."""
    rng = np.random.default_rng(11)
    for trial in range(6):
        s2 = rng.lognormal(0, 2, 4)
        w = rng.lognormal(0, 1.5, 4)
        if trial == 5:
            w = np.array([1.0, 0.0, 2.0, 0.5])          # a zero-weight channel
        for budget in range(0, 33, 3):
            best = min(sum(w[i] * s2[i] * 4.0 ** (-a[i]) for i in range(4))
                       for a in itertools.product(range(9), repeat=4) if sum(a) == budget)
            got = O.waterfill_bits(s2, budget, weight=w)
            assert got.sum() == budget and got.max() <= 8
            dist = sum(w[i] * s2[i] * 4.0 ** (-got[i]) for i in range(4))
            assert dist <= best * (1 + 1e-14) + 1e-300


def test_weighted_waterfill_special_cases():
    s2 = synth.spectrum(128)
    for budget in (170, 256, 353):
        # unit weights are the unweighted allocation; power-of-two scaling is exact
        assert np.array_equal(O.waterfill_bits(s2, budget, weight=np.ones(128)), O.waterfill_bits(s2, budget))
        w = np.random.default_rng(budget).lognormal(0, 1, 128)
        assert np.array_equal(O.waterfill_bits(s2, budget, weight=w), O.waterfill_bits(s2, budget, weight=8.0 * w))
    # all weight on two channels: they take max_bits first
    w = np.zeros(128)
    w[[5, 77]] = 1.0
    b = O.waterfill_bits(s2, 16, weight=w)
    assert b[5] == 8 and b[77] == 8 and b.sum() == 16
    with pytest.raises(ValueError):
        O.waterfill_bits(s2, 16, weight=-w)


def test_query_weights_sum_and_identity():
    """sum_i E[(R q)_i^2] = E|q|^2 for orthogonal R; with R = I they are E[q_i^2]."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((500, 128)) * np.linspace(0.1, 3.0, 128)
    x = synth.draw(2, 0, 0, synth.K, "calib", 1024, dtype="bf16")
    _, c = O.calib_stats(x)
    for rot in (O.rotation_klt, O.rotation_wht):
        r, _ = rot(c)
        w = O.query_channel_weights(r, q)
        assert abs(w.sum() - (q * q).sum(axis=1).mean()) < 1e-9 * w.sum()
    assert np.allclose(O.query_channel_weights(np.eye(128), q), (q * q).mean(axis=0), rtol=1e-14, atol=0)


def test_score_error_decomposes_over_key_channels():
    """AATC abstract: under white quantization noise the expected attention-aware (score)
    distortion is additive over channels.  Monte Carlo: with independent zero-mean errors e_i of
    variance D_i in the rotated basis, E[(q.(R^T e))^2] = sum_i E[(R q)_i^2] D_i."""
    rng = np.random.default_rng(9)
    r, _ = O.rotation_wht(np.eye(128))
    q = rng.standard_normal((4000, 128)) * np.linspace(0.2, 2.0, 128)
    dvar = rng.uniform(0.01, 1.0, 128)
    e = rng.uniform(-1.0, 1.0, (4000, 128)) * np.sqrt(3.0 * dvar)    # variance dvar, zero mean
    err = np.einsum("ni,ni->n", q, e @ r)                             # q . (R^T e)
    want = (O.query_channel_weights(r, q) * dvar).sum()
    assert abs((err * err).mean() - want) < 0.05 * want


def test_attention_aware_bits_lower_score_error():
    """Allocation weighted by the queries' rotated second moments gives a smaller score error
    than the cache-MSE allocation at the same budget, on keys and queries whose energy sits in
    different rotated channels (the situation the criterion targets)."""
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f32")
    ctx = synth.draw(1, 0, 0, synth.K, "context", 2048, dtype="f32")
    plain = O.calibrate(x, "klt", 2.0)
    rng = np.random.default_rng(2)
    # queries concentrated on the low-variance key directions
    qw = np.concatenate([np.zeros(96), np.ones(32)]) * 3.0 + 0.05
    q_cal = (rng.standard_normal((512, 128)) * qw) @ plain["R"]
    q_test = (rng.standard_normal((512, 128)) * qw) @ plain["R"]
    aware = O.calibrate(x, "klt", 2.0, q_cal=q_cal)
    assert aware["bits"].sum() == plain["bits"].sum()
    errs = []
    for art in (plain, aware):
        kh = O.reconstruct(O.encode_codes(ctx, art), art)
        d = (q_test @ (ctx - kh).T)
        errs.append(float((d * d).mean()))
    assert errs[1] < 0.8 * errs[0], errs


# ---------------------------------------------------------------- joint K/V budget split
def test_joint_split_brute_force():
    """The split is the exhaustive optimum over every pair of allocations with the same total
    (d = 3 channels per tensor, up to 3 bits each, one head)."""
    rng = np.random.default_rng(31)
    for _ in range(20):
        ks, vs = rng.uniform(0.01, 4.0, 3), rng.uniform(0.01, 4.0, 3)
        lam, total = float(rng.uniform(0.1, 3.0)), int(rng.integers(0, 19))
        best = min(lam * O.allocation_distortion(ks, bk) + O.allocation_distortion(vs, bv)
                   for bk in itertools.product(range(4), repeat=3) for bv in itertools.product(range(4), repeat=3)
                   if sum(bk) + sum(bv) == total)
        bk, bv, dist = O.joint_kv_split([ks], [vs], [lam], total, max_bits=3)
        assert bk + bv == total and abs(dist - best) <= 1e-12 * best


def test_joint_split_limits_symmetry_and_scaling():
    s2 = synth.spectrum(128)
    T = 2 * 256
    # no weight on keys -> every bit to V (up to its cap); a dominant key term -> every bit to K
    assert O.joint_kv_split([s2], [s2], [0.0], T)[:2] == (0, T)
    assert O.joint_kv_split([s2], [s2], [1e12], T)[:2] == (T, 0)
    assert O.joint_kv_split([s2], [s2], [0.0], 1100)[:2] == (1100 - 1024, 1024)
    # identical spectra with unit weight: the even split (353: no tie at the threshold); at 256
    # candidates 256 and 257 tie, so 255 + 257 has the same distortion and the smaller B_K wins
    assert O.joint_kv_split([s2], [s2], [1.0], 2 * 353)[:2] == (353, 353)
    assert O.joint_kv_split([s2], [s2], [1.0], T)[:2] == (255, 257)
    # scaling V's variances and lambda by the same power of two changes nothing
    v2 = s2[::-1].copy() * 0.5
    a = O.joint_kv_split([s2], [v2], [0.3], T)
    b = O.joint_kv_split([s2], [4.0 * v2], [1.2], T)
    assert a[:2] == b[:2] and abs(4.0 * a[2] - b[2]) <= 1e-12 * b[2]
    # key weights act as a per-channel lambda
    w = np.full(128, 2.0)
    assert O.joint_kv_split([s2], [v2], [0.3], T, k_weight=[w])[:2] == O.joint_kv_split([s2], [v2], [0.6], T)[:2]


def test_first_order_output_error_terms():
    """The two error terms behind the split, checked by Monte Carlo on one attention row: small
    independent score errors ds_t move the output by E|d out|^2 = sum_t p_t^2 E[ds^2] |v_t - out|^2,
    small value errors e_t by sum_t p_t^2 E|e|^2."""
    rng = np.random.default_rng(33)
    n, d = 200, 16
    s = rng.standard_normal(n) * 1.5
    v = rng.standard_normal((n, d))
    p = np.exp(s - s.max())
    p /= p.sum()
    out = p @ v
    eps = 1e-4
    ks, vs = [], []
    for _ in range(3000):
        ds = rng.standard_normal(n) * eps
        p2 = np.exp(s + ds - (s + ds).max())
        p2 /= p2.sum()
        ks.append(((p2 @ v - out) ** 2).sum())
        e = rng.standard_normal((n, d)) * eps
        vs.append(((p @ (v + e) - out) ** 2).sum())
    want_k = (p * p * ((v - out) ** 2).sum(axis=1)).sum() * eps * eps
    want_v = (p * p).sum() * d * eps * eps
    assert abs(np.mean(ks) / want_k - 1) < 0.08 and abs(np.mean(vs) / want_v - 1) < 0.08
    assert abs(O.value_term_weight(np.diag(np.arange(1.0, 5.0))) - 10.0 / 4.0) < 1e-15


def test_joint_split_lowers_attention_error():
    """At 2 bits per element, the split from the calibration statistics (attention-aware key
    weights from queries scaled like the decode queries) gives a lower attention-output error than
    the equal split, at the same total bits."""
    cfg, n_kv, group, n, bpe = 2, 2, 4, 2048, 2.0
    B = O.bits_budget(bpe, 128)
    calk = [synth.draw(cfg, 0, h, synth.K, "calib", 1024) for h in range(n_kv)]
    calv = [synth.draw(cfg, 0, h, synth.V, "calib", 1024) for h in range(n_kv)]
    ctxk = [synth.draw(cfg, 0, h, synth.K, "context", n) for h in range(n_kv)]
    ctxv = [synth.draw(cfg, 0, h, synth.V, "context", n) for h in range(n_kv)]
    qcal = []
    for h in range(n_kv):
        qr = synth.draw(cfg, 0, h, synth.K, "query", 2048, dtype="f64", extra=50000)
        qcal.append(qr * (2.0 / (calk[h] @ qr.T / math.sqrt(128)).std(axis=0))[:, None])
    q = synth.queries(cfg, 0, n_kv * group, n_kv, ctxk)
    ka = [O.calibrate(calk[h], "klt", bpe, q_cal=qcal[h]) for h in range(n_kv)]
    va = [O.calibrate(calv[h], "klt", bpe) for h in range(n_kv)]
    bk, bv, _ = O.joint_kv_split([a["sigma2"] for a in ka], [a["sigma2"] for a in va],
                                 [O.value_term_weight(a["C"]) for a in va], 2 * B, k_weight=[a["weight"] for a in ka])
    assert bk + bv == 2 * B and bk != B

    def err(bk_, bv_):
        e = 0.0
        for h in range(n_kv):
            kart = O.calibrate(calk[h], "klt", bk_ / 128, q_cal=qcal[h])
            vart = O.calibrate(calv[h], "klt", bv_ / 128)
            kh = O.reconstruct(O.encode_codes(ctxk[h], kart), kart)
            vh = O.reconstruct(O.encode_codes(ctxv[h], vart), vart)
            for g in range(h * group, (h + 1) * group):
                e += float(((O.attention(q[g], ctxk[h], ctxv[h])[0] - O.attention(q[g], kh, vh)[0]) ** 2).sum())
        return e

    assert err(bk, bv) < 0.7 * err(B, B)


# ---------------------------------------------------------------- non-orthogonal key transform
def _aniso_queries(rng, n, basis, scales):
    return (rng.standard_normal((n, 128)) * scales) @ basis


def test_nova_identity_moment_is_klt():
    """With E[q q^T] = I the attention-aware distortion is the cache MSE, and the transform is the
    KLT itself; with a I it is sqrt(a) times the KLT (same bits)."""
    x = synth.draw(2, 0, 0, synth.K, "calib", 1024, dtype="bf16")
    klt = O.calibrate(x, "klt", 2.76)
    for a in (1.0, 4.0):
        q = np.vstack([math.sqrt(256.0 * a) * np.eye(128), np.zeros((128, 128))])   # moment a I, exactly
        assert np.array_equal(O.query_moment(q), a * np.eye(128))
        nova = O.calibrate(x, "nova", 2.76, q_cal=q)
        sa = math.sqrt(a)
        assert np.abs(nova["E"] - sa * klt["R"]).max() < 1e-9 * sa
        assert np.abs(nova["R"] - klt["R"] / sa).max() < 1e-9
        assert np.allclose(nova["sigma2"], a * klt["sigma2"], rtol=1e-9, atol=1e-12 * a * klt["sigma2"].max())
        assert np.array_equal(nova["bits"], klt["bits"])


def test_nova_generalized_parseval():
    """NOVA abstract: under the key transform the attention-aware distortion is MSE in the
    transform domain: the mean over the calibration queries of (q . T^-1 e)^2 is |e|^2 for every
    coefficient error e (exactly, for the sample second moment)."""
    rng = np.random.default_rng(21)
    x = synth.draw(4, 0, 1, synth.K, "calib", 1024, dtype="bf16")
    _, c = O.calib_stats(x)
    q = _aniso_queries(rng, 3000, synth.haar_orthogonal(rng, 128), np.geomspace(0.05, 3.0, 128))
    t, p, _ = O.transform_nova(c, O.query_moment(q))
    for _ in range(5):
        e = rng.standard_normal(128) * rng.uniform(0.1, 2.0, 128)
        err = q @ (p.T @ e)                              # q . (T^-1 e), with T^-1 = P^T
        assert abs((err * err).mean() - e @ e) < 1e-9 * (e @ e)


def test_nova_transform_properties():
    """P = T^-T; T C T^T is diagonal with the returned variances in descending order; scores
    in the coefficient domain equal the original scores; the artefact's offset is T mu."""
    rng = np.random.default_rng(22)
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f32")
    mu, c = O.calib_stats(x)
    q = _aniso_queries(rng, 2000, synth.haar_orthogonal(rng, 128), np.linspace(0.1, 3.0, 128))
    art = O.calibrate(x, "nova", 2.0, q_cal=q)
    t, p, s2 = art["E"], art["R"], art["sigma2"]
    assert np.abs(p @ t.T - np.eye(128)).max() < 1e-9
    cov_y = t @ c @ t.T
    off = cov_y - np.diag(np.diag(cov_y))
    assert np.abs(off).max() < 1e-9 * s2.max()
    assert np.allclose(np.diag(cov_y), s2, rtol=1e-8, atol=1e-12 * s2.max())
    assert np.all(np.diff(s2) <= 0)
    keys = synth.draw(1, 0, 0, synth.K, "context", 300, dtype="f32")
    for g in range(7):
        s_orig = keys @ q[g]
        s_coef = O.rotated_scores(q[g], p, keys @ t.T)
        assert np.abs(s_orig - s_coef).max() < 1e-9 * np.abs(s_orig).max()
    assert np.allclose(art["o"], t @ mu, rtol=0, atol=1e-12 * np.abs(t @ mu).max())
    # reconstruction is P^T y_hat = T^-1 y_hat
    codes = O.encode_codes(keys, art)
    assert np.allclose(O.reconstruct(codes, art), np.linalg.solve(t, O.dequantize(codes, art).T).T, atol=1e-9)


def test_nova_rank_deficient_queries_floor():
    """Queries confined to a 16-dimensional subspace: eigenvalues of E[q q^T] are raised to
    1e-6 of the largest, so the transform stays finite and invertible."""
    rng = np.random.default_rng(23)
    x = synth.draw(2, 0, 0, synth.K, "calib", 1024, dtype="bf16")
    _, c = O.calib_stats(x)
    basis = synth.haar_orthogonal(rng, 128)[:16]
    q = rng.standard_normal((500, 16)) @ basis
    t, p, s2 = O.transform_nova(c, O.query_moment(q))
    assert np.all(np.isfinite(t)) and np.all(np.isfinite(p)) and np.all(s2 >= 0)
    assert np.abs(p @ t.T - np.eye(128)).max() < 1e-6
    with pytest.raises(ValueError):
        O.transform_nova(c, np.zeros((128, 128)))


def test_nova_lower_score_error_than_orthogonal():
    """Queries whose anisotropy is not aligned with the keys' principal axes: the non-orthogonal
    transform gives a much smaller score error than the KLT, with or without query-weighted bits,
    at the same budget (calibration and test queries are separate draws)."""
    x = synth.draw(4, 0, 0, synth.K, "calib", 1024, dtype="f32")
    ctx = synth.draw(4, 0, 0, synth.K, "context", 2048, dtype="f32")
    rng = np.random.default_rng(5)
    basis = synth.haar_orthogonal(rng, 128)
    for scales in (np.linspace(0.1, 3.0, 128), np.geomspace(0.05, 3.0, 128)):
        q_cal = _aniso_queries(rng, 8192, basis, scales)
        q_test = _aniso_queries(rng, 512, basis, scales)
        arts = [O.calibrate(x, "klt", 2.0), O.calibrate(x, "klt", 2.0, q_cal=q_cal),
                O.calibrate(x, "nova", 2.0, q_cal=q_cal)]
        assert len({int(a["bits"].sum()) for a in arts}) == 1
        errs = []
        for art in arts:
            kh = O.reconstruct(O.encode_codes(ctx, art), art)
            d = q_test @ (ctx - kh).T
            errs.append(float((d * d).mean()))
        assert errs[2] < 0.7 * min(errs[:2]), errs


# ---------------------------------------------------------------- quantizer step g(b)
def test_g1_closed_form():
    assert abs(O.optimal_step(1) - 2 * math.sqrt(2 / math.pi)) < 1e-14
    assert abs(O.uniform_quantizer_mse(1, O.optimal_step(1)) - (1 - 2 / math.pi)) < 1e-14


def test_g_matches_max_1960_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "max1960_uniform_gaussian.txt"))
            if l.strip() and not l.startswith("#")]
    for b, _levels, step in rows:
        assert abs(O.optimal_step(int(b)) - float(step)) <= 6e-4 * float(step)


@pytest.mark.parametrize("b", range(1, 9))
def test_mse_closed_form_vs_quadrature_and_minimum(b):
    g = O.optimal_step(b)
    levels = 2 ** b

    def q(z):
        k = np.clip(np.floor(z / g + levels / 2), 0, levels - 1)
        return (k - levels / 2 + 0.5) * g

    edges = [(k - levels / 2) * g for k in range(1, levels)]
    pts = [-np.inf] + edges + [np.inf]
    quad = sum(integrate.quad(lambda z: (z - q(0.5 * (a + c) if np.isfinite(a) and np.isfinite(c)
                                                   else (a + 1e-9 if np.isfinite(a) else c - 1e-9))) ** 2
                              * stats.norm.pdf(z), a, c, epsabs=1e-14, epsrel=1e-12)[0]
               for a, c in zip(pts[:-1], pts[1:]))
    assert abs(quad - O.uniform_quantizer_mse(b, g)) < 1e-10
    for f in (1 - 1e-3, 1 + 1e-3):
        assert O.uniform_quantizer_mse(b, g * f) > O.uniform_quantizer_mse(b, g)
    h = 1e-6 * g
    fd = (O.uniform_quantizer_mse(b, g + h) - O.uniform_quantizer_mse(b, g - h)) / (2 * h)
    assert abs(fd) < 1e-6


def test_mse_monte_carlo():
    rng = np.random.default_rng(11)
    z = rng.standard_normal(2_000_000)
    for b in (1, 2, 3, 4, 6, 8):
        g = O.optimal_step(b)
        levels = 2 ** b
        k = np.clip(np.floor(z / g + levels / 2), 0, levels - 1)
        e2 = (z - (k - levels / 2 + 0.5) * g) ** 2
        se = e2.std() / math.sqrt(z.size)
        assert abs(e2.mean() - O.uniform_quantizer_mse(b, g)) < 3.5 * se


# ---------------------------------------------------------------- encode / decode
def _max1960_nonuniform():
    rows = {}
    with open(os.path.join(GOLDEN, "max1960_nonuniform_gaussian.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                n, kind, *vals = line.split()
                rows[(int(n), kind)] = [float(v) for v in vals]
    return rows


def test_lloyd_max_matches_max_1960_table():
    """Levels, interval end points and MSE of the 2-, 4-, 8- and 16-level Gaussian Lloyd-Max
    quantizers against Max's 1960 table (four significant digits)."""
    tab = _max1960_nonuniform()
    for b in (1, 2, 3, 4):
        n = 2 ** b
        levels, th = O.lloyd_max_gaussian(b)
        assert levels.shape == (n,) and th.shape == (n - 1,)
        assert np.all(np.diff(levels) > 0) and np.allclose(levels, -levels[::-1], rtol=0, atol=1e-15)
        y = tab[(n, "y")]
        assert np.allclose(levels[n // 2:], y, rtol=6e-4, atol=0), (b, levels[n // 2:], y)
        if (n, "x") in tab:
            assert np.allclose(th[n // 2:], tab[(n, "x")], rtol=6e-4, atol=0), (b, th[n // 2:])
        assert abs(O.lloyd_max_mse(b) - tab[(n, "mse")][0]) <= 6e-4 * tab[(n, "mse")][0], b


@pytest.mark.parametrize("b", [1, 2, 3, 5, 8])
def test_lloyd_max_conditions_by_quadrature(b):
    """The two Lloyd conditions, checked by numerical quadrature (not the closed form the solver
    uses): every level is the mean of N(0,1) over its cell (to 1e-12) and every threshold the
    midpoint of its levels; the MSE by quadrature equals lloyd_max_mse and is below the uniform
    quantizer's (equal at one bit, where both are +-sqrt(2/pi))."""
    levels, th = O.lloyd_max_gaussian(b)
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    mse = 0.0
    for k in range(2 ** b):
        lo, hi = edges[k], edges[k + 1]
        # tail masses from the survival function on the positive side (no cancellation near 1)
        mass = stats.norm.sf(lo) - stats.norm.sf(hi) if lo >= 0 else stats.norm.cdf(hi) - stats.norm.cdf(lo)
        m1 = integrate.quad(lambda z: z * stats.norm.pdf(z), lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        assert abs(m1 / mass - levels[k]) <= 1e-12 * max(1.0, abs(levels[k])), (b, k)
        mse += integrate.quad(lambda z: (z - levels[k]) ** 2 * stats.norm.pdf(z), lo, hi,
                              epsabs=1e-16, epsrel=1e-13, limit=200)[0]
    assert np.allclose(th, 0.5 * (levels[:-1] + levels[1:]), rtol=0, atol=1e-15)
    assert abs(mse - O.lloyd_max_mse(b)) <= 1e-11
    uni = O.uniform_quantizer_mse(b, O.optimal_step(b))
    if b == 1:
        assert abs(levels[1] - math.sqrt(2 / math.pi)) < 1e-15 and abs(mse - uni) < 1e-12
    else:
        assert mse < uni


def test_lloyd_max_encode_decode():
    """Lloyd-Max caches: codes count the thresholds at or below z = (y - o)/s (a value on a
    threshold goes up; NaN -> 0, +-Inf -> the ends), reconstruction is o + s l[c], and on Gaussian
    channels the per-channel MSE is s^2 times the table's MSE (3 standard errors)."""
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f64")
    assert np.array_equal(O.calibrate(x, "klt", 2.76, quantizer="lloyd-max")["bits"], O.calibrate(x, "klt", 2.76)["bits"])
    # identity rotation: y = x exactly, so inputs can sit exactly on a channel's thresholds
    art = O.calibrate(x, "identity", 2.76, quantizer="lloyd-max")
    i = int(np.argmax(art["bits"] == 3))
    levels, th = O.lloyd_max_gaussian(3)
    s, o = art["scale"][i], art["o"][i]
    zz = np.concatenate([th, [np.nan, np.inf, -np.inf, 0.0]])
    xs = np.tile(art["o"], (zz.size, 1))
    xs[:, i] = o + s * zz
    z = (xs[:, i] - o) * art["inv_scale"][i]        # the encoder's fp64 expression
    codes = O.encode_codes(xs, art)
    got = codes[:, i]
    for k in range(7):                               # at (or within rounding of) threshold k
        assert got[k] == (k + 1 if z[k] >= th[k] else k), (k, z[k], th[k])
    assert got[7] == 0 and got[8] == 7 and got[9] == 0 and got[10] == 4
    yh = O.dequantize(codes, art)
    assert np.array_equal(yh[:, i], o + s * levels[got])
    # Monte Carlo on exactly Gaussian rotated coefficients
    rng = np.random.default_rng(11)
    n = 200000
    sig = np.sqrt(art["sigma2"])
    yy = art["o"][None, :] + rng.standard_normal((n, 128)) * sig[None, :]
    cc = O.encode_codes(yy @ art["R"], art)
    err = O.dequantize(cc, art) - O.rotate(yy @ art["R"], art)
    for j in range(128):
        b = int(art["bits"][j])
        if b == 0 or sig[j] == 0:
            continue
        e2 = err[:, j] ** 2
        want = sig[j] ** 2 * O.lloyd_max_mse(b)
        assert abs(e2.mean() - want) <= 3 * e2.std() / math.sqrt(n) + 1e-12 * want, (j, b)


def _art_identity(d, bits, delta, o=None):
    bits = np.asarray(bits)
    o = np.zeros(d) if o is None else np.asarray(o, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    inv = np.where(bits > 0, 1.0 / delta, 0.0)
    return {"R": np.eye(d), "o": o, "delta": np.where(bits > 0, delta, 0.0), "inv_delta": inv,
            "bits": bits}


def test_encode_edges_go_up_and_special_values():
    bits = np.array([2, 3, 1, 0])
    art = _art_identity(4, bits, [0.25, 0.5, 1.0, 1.0])
    # edges of channel 0 (2 bits, step 1/4, offset 0): -0.25, 0, 0.25
    x = np.array([[-0.25, 0.0, 0.0, 5.0], [0.0, -1.0, -1e-3, 0.0], [0.25, 1.5, 7.0, 0.0],
                  [-7.0, -9.0, np.inf, 0.0], [np.nan, np.nan, np.nan, 0.0], [np.inf, -np.inf, 0.0, 0.0]])
    c = O.encode_codes(x, art)
    # row 3: channel 2 sees +inf (clamped to the top code); channels 0/1 see -7 + 0*inf = NaN -> 0.
    # row 5: every channel meets 0*inf = NaN in y = R x, so every code is 0.
    assert c.tolist() == [[1, 4, 1, 0], [2, 2, 0, 0], [3, 7, 1, 0], [0, 0, 1, 0], [0, 0, 0, 0], [0, 0, 0, 0]]


def test_quantization_error_bounded_by_half_step():
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f32")
    art = O.calibrate(x, "klt", 2.0)
    xc = synth.draw(1, 0, 0, synth.K, "context", 2048, dtype="f32")
    codes = O.encode_codes(xc, art)
    y = xc.astype(np.float64) @ art["R"].T
    yh = O.dequantize(codes, art)
    bits = art["bits"]
    top = (1 << bits) - 1
    for i in np.nonzero(bits)[0]:
        inner = (codes[:, i] > 0) & (codes[:, i] < top[i])
        assert np.all(np.abs(yh[inner, i] - y[inner, i]) <= art["delta"][i] / 2 * (1 + 1e-12))
    assert np.allclose(yh[:, bits == 0], art["o"][bits == 0][None, :])
    assert np.allclose(O.reconstruct(codes, art), yh @ art["R"])


def test_per_channel_mse_matches_gaussian_closed_form():
    """On Gaussian data the per-channel MSE is eps(b_i) sigma_i^2 (3.5 SE)."""
    rng = np.random.default_rng(5)
    d = 16
    q = synth.haar_orthogonal(rng, d)
    lam = np.arange(1, d + 1) ** -1.0
    cal = (rng.standard_normal((200_000, d)) * np.sqrt(lam)) @ q.T
    art = O.calibrate(cal, "klt", 3.0)
    x = (rng.standard_normal((200_000, d)) * np.sqrt(lam)) @ q.T
    codes = O.encode_codes(x, art)
    err = (O.dequantize(codes, art) - x @ art["R"].T) ** 2
    for i in range(d):
        b = int(art["bits"][i])
        want = art["sigma2"][i] * (O.uniform_quantizer_mse(b, O.optimal_step(b)) if b else 1.0)
        se = err[:, i].std() / math.sqrt(err.shape[0])
        assert abs(err[:, i].mean() - want) < 3.5 * se + 1e-3 * want


# ---------------------------------------------------------------- packed formats
def test_pack_k_hand_example():
    """d=4 with bits (3,2,1,0): B=6 bits/token; planes (0,0),(0,1),(0,2),(1,0),(1,1),(2,0)."""
    bits = [3, 2, 1, 0]
    codes = np.array([[5, 2, 1, 0], [3, 1, 0, 0]])
    w = O.pack_k(codes, bits)
    assert w.size == 2 * 6
    # token 0: c0=5 -> planes 1,0,1 ; c1=2 -> 0,1 ; c2=1 -> 1  => bits 0..5 = 1,0,1,0,1,1
    # token 1 at bits 6..11: c0=3 -> 1,1,0 ; c1=1 -> 1,0 ; c2=0 -> 0
    expect = (1 << 0) | (1 << 2) | (1 << 4) | (1 << 5) | (1 << 6) | (1 << 7) | (1 << 9)
    assert int(w[0]) == expect and not w[1:].any()


def test_pack_v_hand_example():
    bits = [3, 0, 1]
    # fields: (0,0,w2), (0,2,w1), (2,0,w1) -> words [0,4) w2, [4,6) w1 ch0 bit2, [6,8) w1 ch2
    codes = np.zeros((64, 3), dtype=np.int64)
    codes[5, 0] = 6        # t=5: G=0 r=1 m=1 -> low field value 2 at 8m+2r = 10, bit2 at 8+2+0 = 10
    codes[37, 2] = 1       # t=37: G=2 r=1 m=1 -> w1 offset 32*1 + 8 + 2 + 0 = 42
    codes[31, 0] = 2       # t=31: G=1 r=3 m=3 -> w2 in word 1 rotated by 1: bit 0 at 31, bit 1 wraps to 0
    codes[20, 2] = 1       # t=20: G=1 r=1 m=0 -> w1 offset 0 + 0 + 2 + 1 = 3
    w = O.pack_v(codes, bits)
    assert w.size == 8
    assert int(w[0]) == (2 << 10)
    assert int(w[1]) == 1
    assert int(w[4]) == (1 << 10)
    assert int(w[6]) == (1 << 3)
    assert int(w[6 + 1]) == (1 << (42 - 32))
    assert sum(int(v) != 0 for v in w) == 5


def test_pack_roundtrip_and_sizes():
    rng = np.random.default_rng(1)
    for bits in ([8, 7, 6, 5, 4, 3, 2, 1, 0, 0, 3], [1] * 11, [2, 0, 0, 8]):
        bits = np.array(bits)
        for n in (1, 63, 64, 65, 130):
            codes = rng.integers(0, 1 << bits, size=(n, bits.size))
            wk, wv = O.pack_k(codes, bits), O.pack_v(codes, bits)
            assert wk.size == wv.size == O.packed_words(bits.sum(), n) == -(-n // 64) * 2 * bits.sum()
            assert np.array_equal(O.unpack_k(wk, bits, n), codes)
            assert np.array_equal(O.unpack_v(wv, bits, n), codes)


def test_v_field_positions_are_bijective():
    for w in (1, 2, 4):
        pos = sorted(O.aatc_oracle._v_bit(t, w, b) for t in range(64) for b in range(w))
        assert pos == list(range(64 * w))


def test_v_lane_words_expand_by_uniform_shifts():
    """The decode kernel's operand rule: lane group G of a 16-token block reads one word per
    w<=2 field, rotates it right by G%2, and finds token 16G + 4r + m's value at bit 8m + 2r."""
    rng = np.random.default_rng(3)
    for w in (1, 2):
        vals = rng.integers(0, 1 << w, size=64)
        words = np.zeros(2 * w, dtype=np.uint32)
        for t in range(64):
            for b in range(w):
                if (vals[t] >> b) & 1:
                    s = O.aatc_oracle._v_bit(t, w, b)
                    words[s // 32] |= np.uint32(1 << (s % 32))
        for g in range(4):
            x = int(words[g if w == 2 else g // 2])
            d = ((x >> (g % 2)) | (x << (32 - g % 2))) & 0xFFFFFFFF if g % 2 else x
            for r in range(4):
                for m in range(4):
                    assert (d >> (8 * m + 2 * r)) & ((1 << w) - 1) == vals[16 * g + 4 * r + m]


# ---------------------------------------------------------------- scores and attention
def test_rotated_domain_scores_equal_plain_scores():
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f32")
    art = O.calibrate(x, "klt", 2.0)
    q = np.random.default_rng(2).standard_normal(128)
    y = x.astype(np.float64) @ art["R"].T           # full-precision "codes"
    s_rot = O.rotated_scores(q, art["R"], y)
    s = x.astype(np.float64) @ q
    assert np.abs(s_rot - s).max() <= 1e-12 * np.abs(s).max()


def test_compressed_score_linear_form():
    """sum_i alpha_i c_i + beta == scale q.x_hat with alpha = scale (Rq) Delta (affine dequant)."""
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f32")
    art = O.calibrate(x, "klt", 2.0)
    xc = synth.draw(1, 0, 0, synth.K, "context", 300, dtype="f32")
    codes = O.encode_codes(xc, art)
    q = np.random.default_rng(4).standard_normal(128)
    scale = 1 / math.sqrt(128)
    qt = art["R"] @ q
    bits = art["bits"]
    alpha = scale * qt * art["delta"]
    half = np.where(bits > 0, 2.0 ** (np.maximum(bits, 1) - 1) - 0.5, 0.0)
    beta = scale * np.sum(qt * (art["o"] - art["delta"] * half))
    lhs = codes @ alpha + beta
    rhs = scale * (O.reconstruct(codes, art) @ q)
    assert np.abs(lhs - rhs).max() <= 1e-12 * np.abs(rhs).max()


def test_attention_streaming_equals_direct():
    rng = np.random.default_rng(9)
    for n in (1, 5, 64, 1000):
        q = rng.standard_normal(128) * 3
        k = rng.standard_normal((n, 128))
        v = rng.standard_normal((n, 128))
        o1, l1 = O.attention(q, k, v)
        o2, l2 = O.attention_streaming(q, k, v, chunk=13)
        assert np.abs(o1 - o2).max() < 1e-13 and abs(l1 - l2) < 1e-12


def test_attention_vs_mpmath():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    rng = np.random.default_rng(10)
    for n in (1, 3, 16):
        q = rng.standard_normal(8) * 4
        k = rng.standard_normal((n, 8))
        v = rng.standard_normal((n, 8))
        out, lse = O.attention(q, k, v)
        s = [mpmath.mpf(1) / mpmath.sqrt(8) * mpmath.fsum(mpmath.mpf(float(q[j])) * mpmath.mpf(float(k[t, j]))
                                                          for j in range(8)) for t in range(n)]
        e = [mpmath.e ** st for st in s]
        z = mpmath.fsum(e)
        for j in range(8):
            ref = mpmath.fsum(e[t] * mpmath.mpf(float(v[t, j])) for t in range(n)) / z
            assert abs(float(ref) - out[j]) < 1e-14 * max(1.0, abs(float(ref)))
        assert abs(float(mpmath.log(z)) - lse) < 1e-13


def test_attention_special_cases():
    x = synth.draw(1, 0, 0, synth.K, "calib", 1024, dtype="f32")
    xv = synth.draw(1, 0, 0, synth.V, "calib", 1024, dtype="f32")
    art_k0 = O.calibrate(x, "klt", 0.0)                  # every K channel at 0 bits
    art_v0 = O.calibrate(xv, "klt", 0.0)
    art_v = O.calibrate(xv, "klt", 2.0)
    ck = O.encode_codes(synth.draw(1, 0, 0, synth.K, "context", 50, dtype="f32"), art_k0)
    cv = O.encode_codes(synth.draw(1, 0, 0, synth.V, "context", 50, dtype="f32"), art_v)
    q = np.random.default_rng(1).standard_normal((1, 128))
    out, _ = O.decode_attention(q, [ck], [cv], [art_k0], [art_v])
    assert np.allclose(out[0], O.reconstruct(cv, art_v).mean(0), atol=1e-12)
    cv0 = O.encode_codes(synth.draw(1, 0, 0, synth.V, "context", 50, dtype="f32"), art_v0)
    art_k = O.calibrate(x, "klt", 2.0)
    ck2 = O.encode_codes(synth.draw(1, 0, 0, synth.K, "context", 50, dtype="f32"), art_k)
    out, _ = O.decode_attention(q, [ck2], [cv0], [art_k], [art_v0])
    assert np.allclose(out[0], art_v0["mu"], atol=1e-12)     # R^T o = mu
    out, _ = O.decode_attention(q, [ck2[:1]], [cv[:1]], [art_k], [art_v])
    assert np.allclose(out[0], O.reconstruct(cv[:1], art_v)[0], atol=1e-12)


# ---------------------------------------------------------------- token tiers and segments
def test_token_tiers_budget_monotone_bruteforce():
    d = 128
    s2 = synth.spectrum(d)
    dist = O.tier_distortions([s2, s2], d)
    assert dist[0] > dist[1] > dist[2] > dist[3] == 0.0
    a = synth.zipf_mass(5, 0, 0, 4096)
    tiers = O.token_tiers(a, dist, d, 2.76)
    assert tiers.sum() * d <= 2.76 * a.size * d
    order = np.argsort(a)
    assert np.all(np.diff(tiers[order]) >= 0)        # more attention mass, never fewer bits
    rng = np.random.default_rng(0)
    for _ in range(5):
        a = rng.dirichlet(np.ones(6))
        lam = float(rng.uniform(1e-6, 1e-3))
        got = O.aatc_oracle._tiers_at(a * a, dist, lam, d)
        best = min(itertools.product(O.aatc_oracle.TIERS, repeat=6),
                   key=lambda ts: (sum(a[t] ** 2 * dist[O.aatc_oracle.TIERS.index(ts[t])] + lam * d * ts[t]
                                       for t in range(6))))
        cost = lambda ts: sum(a[t] ** 2 * dist[O.aatc_oracle.TIERS.index(ts[t])] + lam * d * ts[t]
                              for t in range(6))
        assert cost(tuple(got)) <= cost(best) * (1 + 1e-12)


def _bits_from_histogram(hist):
    """Non-increasing bit vector with the given {bits: channels} histogram (KLT channel order)."""
    return np.concatenate([np.full(c, b, dtype=np.int64) for b, c in sorted(hist.items(), reverse=True)])


def test_tier_distortions_closed_form_on_noise_free_spectrum():
    """D(tau) = sum_i s_i 4^-b_i(tau) with b(tau) the allocation of tau*d bits: on s_i = i^-1.5 the
    allocations at 256 and 512 bits are the derived histograms (tie rule included), so D(2) and
    D(4) follow from them alone; D(0) is the total variance, D(16) = 0; several tensors add, and a
    tensor scaled by 4 has the same bits and 4 times the distortion."""
    s2 = synth.spectrum(128)
    b2 = _bits_from_histogram({6: 1, 5: 4, 4: 7, 3: 19, 2: 48, 1: 49})
    b4 = _bits_from_histogram({8: 1, 7: 4, 6: 7, 5: 19, 4: 48, 3: 49})
    assert b2.sum() == 256 and b4.sum() == 512
    want = np.array([math.fsum(s2), math.fsum(s2 * 4.0 ** -b2), math.fsum(s2 * 4.0 ** -b4), 0.0])
    got = O.tier_distortions([s2], 128)
    assert np.allclose(got, want, rtol=1e-14, atol=0.0), (got, want)
    assert got[3] == 0.0
    got2 = O.tier_distortions([s2, 4.0 * s2], 128)
    assert np.allclose(got2, 5.0 * want, rtol=1e-14, atol=0.0)


_TIERS = (0, 2, 4, 16)


def _tiers_by_enumeration(w, dist, d, budget):
    """Brute force over every tier assignment of len(w) tokens: the Lagrangian solutions are the
    vertices of the lower convex hull of (bits, sum_t w_t D(tier_t)); the one with the most bits
    within the budget is what the smallest fitting multiplier picks.  Returns (assignment, bits, cost)."""
    best = {}
    for ts in itertools.product(range(4), repeat=len(w)):
        b = d * sum(_TIERS[k] for k in ts)
        c = sum(w[t] * dist[k] for t, k in enumerate(ts))
        if b not in best or c < best[b][0]:
            best[b] = (c, ts)
    hull = []
    for x in sorted(best):
        p = (x, best[x][0])
        while len(hull) >= 2:
            (x1, y1), (x2, y2) = hull[-2], hull[-1]
            if (x2 - x1) * (p[1] - y1) - (y2 - y1) * (p[0] - x1) <= 0:
                hull.pop()
            else:
                break
        hull.append(p)
    bits, cost = max(p for p in hull if p[0] <= budget)
    return tuple(_TIERS[k] for k in best[bits][1]), bits, cost


def test_token_tiers_match_enumeration():
    """token_tiers against the enumeration of all 4^6 assignments, with weights a_t^2: same tiers
    (hence optimal for the constrained problem at its own bit total, and the largest such total
    within the budget); a multiplier 1e-9 smaller than the returned one overshoots the budget
    (the argmin found by enumeration); and the a_t-weighted enumeration differs in some cases,
    so a_t^2 is what decides."""
    d = 128
    s2 = synth.spectrum(d)
    dist = O.tier_distortions([s2, s2], d)
    rng = np.random.default_rng(5)
    differ = 0
    for trial in range(24):
        a = rng.dirichlet(np.full(6, 0.3))
        avg = float(rng.choice([1.0, 2.0, 2.76, 4.0, 6.0]))
        budget = avg * 6 * d
        want, wbits, _ = _tiers_by_enumeration(a * a, dist, d, budget)
        got, lam = O.token_tiers(a, dist, d, avg, return_lambda=True)
        assert tuple(int(v) for v in got) == want, (trial, got, want)
        if lam > 0:
            lam2 = lam * (1.0 - 1e-9)
            over = min(itertools.product(range(4), repeat=6),
                       key=lambda ts: sum(a[t] ** 2 * dist[k] + lam2 * d * _TIERS[k] for t, k in enumerate(ts)))
            assert d * sum(_TIERS[k] for k in over) > budget, trial
        if _tiers_by_enumeration(a, dist, d, budget)[0] != want:
            differ += 1
    assert differ >= 5


def test_segment_attention_excludes_evicted():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((10, 8))
    v = rng.standard_normal((10, 8))
    q = rng.standard_normal(8)
    keep = np.array([1, 1, 0, 1, 0, 1, 1, 1, 0, 1], dtype=bool)
    out, lse = O.segment_attention(q, [(k[keep][:3], v[keep][:3]), (k[keep][3:], v[keep][3:])])
    ref, lref = O.attention(q, k[keep], v[keep])
    assert np.allclose(out, ref, atol=1e-14) and abs(lse - lref) < 1e-13

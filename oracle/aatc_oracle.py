"""Plain, slow, fp64 definition of the compression path (test infrastructure only).

Sources (cited by page title and section; no line numbers):
  [AATC]    "KV Cache Compression Through the Lens of Transform Coding" -- At a glance,
            Key points, Full text: transform coding plus reverse water-filling that
            allocates bits over a calibration set.
  [SPECTRA] "SPECTRA: Pushing the KV Cache Beyond the 2-Bit Cliff via Spectral Transform
            Coding" -- Abstract: rotate the cache into a coordinate system computed from
            its own statistics (removing channel correlations), then spend the bit budget
            on the few channels that carry the signal.
  [RDKV]    "SPHERICAL KV: ..." page, first abstract (RDKV): each token or channel gets
            a width between uncompressed and none at all, set by reverse water-filling,
            once after prefill; every decode step reads the cache from HBM again.
  [NOVA]    same page, third abstract (NOVA-KV): decode is bandwidth-bound; a fixed
            per-token bit count / fixed-width layout is required; the key transform that
            is optimal for the attention-aware distortion is not orthogonal, and under it
            that distortion becomes plain MSE of the transformed coefficients.
  [ABL]     "Ablation, Statistical Inference, and Validation for KV-Cache Compression",
            first abstract: Walsh-Hadamard transform followed by a scalar MSE quantizer.
  [OCTOPUS] same page, third abstract: keys are reconstructed on the fly inside the
            attention kernel instead of being materialized.

Where the pages are silent the readings below are used:
centred covariance with 1/M, eigenvectors in descending eigenvalue order with a sign
rule, Sylvester-ordered WHT, budget B = floor(b*d + 1/2) bits per vector, greedy integer
water-filling with a fixed tie order, a mid-rise uniform quantizer with the Gaussian
MSE-optimal step, floor with half-open bins, 0-bit channels reconstructed to the mean,
softmax scale 1/sqrt(d), no mask at decode, contiguous GQA groups.

Everything is fp64 NumPy/SciPy.  Inputs in fp32/bf16 are read as their exact fp64 values.
"""
import math

import numpy as np
from scipy import linalg, optimize, special

TILE = 64          # tokens per packed tile
MAX_BITS = 8

__all__ = [
    "TILE", "MAX_BITS", "calib_stats", "rotation_klt", "hadamard_signs", "rotation_wht", "rotation_identity",
    "query_channel_weights", "query_moment", "transform_nova", "NOVA_EIG_FLOOR",
    "allocation_distortion", "value_term_weight", "joint_kv_split",
    "bits_budget", "waterfill_bits", "waterfill_theta", "uniform_quantizer_mse",
    "uniform_quantizer_mse_deriv", "optimal_step", "lloyd_max_gaussian", "lloyd_max_mse",
    "quantizer_tables", "calibrate",
    "rotate", "encode_codes", "dequantize", "reconstruct", "v_fields", "pack_k", "unpack_k",
    "pack_v", "unpack_v", "packed_words", "attention", "attention_streaming",
    "decode_attention", "rotated_scores", "tier_distortions", "token_tiers",
    "segment_attention",
]


# ----------------------------------------------------------------------------------
# Calibration statistics  [AATC Full text: the bit allocation is made on calibration data;
# SPECTRA Abstract: the basis comes from the statistics of the cache itself]
# ----------------------------------------------------------------------------------
def calib_stats(x):
    """Mean and centred covariance (1/M normalisation) of calibration rows x [M, d]."""
    x = np.asarray(x, dtype=np.float64)
    m = x.shape[0]
    mu = x.sum(axis=0) / m
    xc = x - mu[None, :]
    return mu, (xc.T @ xc) / m


# ----------------------------------------------------------------------------------
# Rotations  [SPECTRA Abstract (data-derived, decorrelating); ABL first abstract (WHT)]
# ----------------------------------------------------------------------------------
def _sign_rule(r):
    """Make the largest-magnitude entry of every row positive (first index on ties)."""
    r = r.copy()
    for i in range(r.shape[0]):
        j = int(np.argmax(np.abs(r[i])))
        if r[i, j] < 0:
            r[i] = -r[i]
    return r


def rotation_klt(c):
    """KLT / PCA basis: rows of R are eigenvectors of C in descending eigenvalue order.

    Returns (R, sigma2) with sigma2_i = max(lambda_i, 0) the variance of channel i of R x.
    """
    w, vec = np.linalg.eigh(np.asarray(c, dtype=np.float64))
    order = np.argsort(-w, kind="stable")
    r = _sign_rule(vec[:, order].T)
    return r, np.maximum(w[order], 0.0)


def hadamard_signs(d):
    """Sylvester (natural-order) Hadamard matrix H_ij = (-1)^popcount(i & j), entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("WHT needs a power-of-two dimension")
    i = np.arange(d)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return np.where(par == 1, -1.0, 1.0)


def rotation_wht(c):
    """Walsh-Hadamard rotation in Sylvester (natural) order, scaled to be orthogonal.

    R_ij = (-1)^popcount(i & j) / sqrt(d); sigma2 = diag(R C R^T).  (The encoder applies it as
    the exact +-1 sums H x times one rounded 1/sqrt(d): see rotate.)
    """
    c = np.asarray(c, dtype=np.float64)
    d = c.shape[0]
    r = hadamard_signs(d) / math.sqrt(d)
    return r, np.einsum("ij,jk,ik->i", r, c, r)


def rotation_identity(c):
    """No rotation (per-channel quantization baseline)."""
    c = np.asarray(c, dtype=np.float64)
    return np.eye(c.shape[0]), np.diag(c).copy()


# Non-orthogonal key transform  [NOVA third abstract: closed-form key transform from
# calibration statistics, not orthogonal, with a generalized Parseval relation]
#
# The attention-aware error of a key error e is (q.e)^2, of mean e^T S e with S = E[q q^T].
# A transform y = T x turns it into plain MSE of y exactly when T^-T S T^-1 = I, i.e.
# T = U S^(1/2) with U orthogonal; U is then the KLT of the whitened keys S^(1/2) x, so the
# coefficients are decorrelated with variances the eigenvalues of S^(1/2) C S^(1/2).  Scores
# use q.x = (P q).y with P = T^-T = U S^(-1/2); reconstruction is x = T^-1 y = P^T y.
# ----------------------------------------------------------------------------------
NOVA_EIG_FLOOR = 1e-6   # eigenvalues of S below this fraction of the largest are raised to it


def query_moment(q):
    """Second moment S = E[q q^T] (not centred) of query rows q [n, d]."""
    q = np.asarray(q, dtype=np.float64)
    return (q.T @ q) / q.shape[0]


def transform_nova(c, s):
    """Key transform from the key covariance c and the query second moment s.

    Returns (T, P, sigma2): coefficients y = T x, the query transform P = T^-T (rows of P
    and of T share the KLT sign rule of U), and sigma2_i = var(y_i).
    """
    w, v = np.linalg.eigh(np.asarray(s, dtype=np.float64))
    if not w.max() > 0:
        raise ValueError("query second moment has no positive eigenvalue")
    w = np.maximum(w, NOVA_EIG_FLOOR * w.max())
    s_half = (v * np.sqrt(w)) @ v.T
    s_ihalf = (v / np.sqrt(w)) @ v.T
    m = s_half @ np.asarray(c, dtype=np.float64) @ s_half
    u, lam = rotation_klt(0.5 * (m + m.T))
    return u @ s_half, u @ s_ihalf, lam


# ----------------------------------------------------------------------------------
# Reverse water-filling  [AATC Key points / Full text; SPECTRA Abstract; RDKV abstract]
# ----------------------------------------------------------------------------------
def bits_budget(bits_per_elem, d):
    """Integer bits per vector B = floor(b*d + 1/2)."""
    return int(math.floor(bits_per_elem * d + 0.5))


def waterfill_bits(sigma2, total_bits, max_bits=MAX_BITS, weight=None):
    """Integer reverse water-filling: bits b_i in [0, max_bits] with sum b_i = B that
    minimise sum_i w_i sigma_i^2 4^(-b_i) (high-resolution distortion model; w_i = 1 unless
    per-channel weights are given, as for the attention-aware allocation).

    Greedy on the exact candidates v_ik = (w_i sigma_i^2) 4^-k (k < max_bits): the B largest
    under the order (value desc, channel asc, bit asc) are granted.  The gains of one
    channel fall geometrically, so the greedy choice is optimal.
    """
    s2 = np.asarray(sigma2, dtype=np.float64)
    d = s2.shape[0]
    if total_bits < 0 or total_bits > d * max_bits:
        raise ValueError("budget out of range")
    if weight is not None:
        w = np.asarray(weight, dtype=np.float64)
        if w.shape != s2.shape or not np.all(np.isfinite(w)) or np.any(w < 0):
            raise ValueError("channel weights must be finite and non-negative, one per channel")
        s2 = w * s2
    cands = [(-math.ldexp(float(s2[i]), -2 * k), i, k) for i in range(d) for k in range(max_bits)]
    cands.sort()
    bits = np.zeros(d, dtype=np.int64)
    for _, i, _k in cands[:total_bits]:
        bits[i] += 1
    return bits


def allocation_distortion(sigma2, bits, weight=None):
    """High-resolution distortion sum_i w_i sigma_i^2 4^-b_i of an allocation."""
    s2 = np.asarray(sigma2, dtype=np.float64)
    if weight is not None:
        s2 = np.asarray(weight, dtype=np.float64) * s2
    return float(sum(math.ldexp(float(s2[i]), -2 * int(bits[i])) for i in range(s2.shape[0])))


def value_term_weight(c_v, scale=None):
    """lambda = scale^2 tr(C_V): how much a unit of key score-distortion costs in output error,
    relative to a unit of value distortion, for attention spread over typical tokens.

    First order in the errors, with out = sum_t p_t v_t: a score error ds_t moves the output by
    sum_t p_t ds_t (v_t - out), a value error e_t by sum_t p_t e_t.  With independent zero-mean
    errors the mean squared output errors are sum_t p_t^2 E[ds_t^2] |v_t - out|^2 and
    sum_t p_t^2 E|e_t|^2; E[ds_t^2] = scale^2 x (the attention-aware key distortion), and
    |v_t - out|^2 averages tr(C_V) when out is near the values' mean.
    """
    c_v = np.asarray(c_v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(c_v.shape[0])
    return scale * scale * float(np.trace(c_v))


def joint_kv_split(k_sigma2, v_sigma2, lam, total_bits, max_bits=MAX_BITS, k_weight=None, tensor_cap=None):
    """Split T = total_bits bits per (key, value) vector pair between K and V for a layer whose
    heads all share B_K (and B_V = T - B_K): the B_K minimising
        sum_h lam_h D_K,h(B_K) + D_V,h(T - B_K)
    with D the water-filled distortions (keys with their attention-aware weights).  Among
    values within 1e-12 (relative) of the minimum the smallest B_K is taken.

    k_sigma2, v_sigma2: per-head variance vectors; lam: per-head weights (value_term_weight);
    k_weight: per-head key weights or None; tensor_cap: largest B_K and B_V allowed (None: d
    times max_bits), e.g. the most bits per vector a decode kernel reads.
    Returns (B_K, B_V, distortion).
    """
    heads = len(k_sigma2)
    d = len(k_sigma2[0])
    cap = d * max_bits if tensor_cap is None else min(d * max_bits, int(tensor_cap))
    lo, hi = max(0, total_bits - cap), min(total_bits, cap)
    if lo > hi:
        raise ValueError("budget out of range")
    kw = [None] * heads if k_weight is None else k_weight
    dist = []
    for bk in range(lo, hi + 1):
        tot = 0.0
        for h in range(heads):
            tot += lam[h] * allocation_distortion(k_sigma2[h], waterfill_bits(k_sigma2[h], bk, max_bits, kw[h]), kw[h])
            tot += allocation_distortion(v_sigma2[h], waterfill_bits(v_sigma2[h], total_bits - bk, max_bits))
        dist.append(tot)
    best = min(dist)
    i = next(j for j, v in enumerate(dist) if v <= best * (1.0 + 1e-12))
    return lo + i, total_bits - lo - i, dist[i]


def query_channel_weights(r, q_cal):
    """Attention-aware key weights w_i = E[(R q)_i^2] over calibration queries q.

    [AATC abstract: with quantization errors modelled as white noise, the mean attention-aware
    error is a key part plus a value part, each separable over tokens and channels.]  With a
    zero-mean key error e independent of q and of its other channels, the score error
    q.(k - k_hat) = (R q).(R e) has E[(q.(k - k_hat))^2] = sum_i E[(R q)_i^2] E[(R e)_i^2]:
    the key channels' distortions add with these weights.  The value path has no such factor
    (uniform weights).
    """
    qr = np.asarray(q_cal, dtype=np.float64) @ np.asarray(r, dtype=np.float64).T
    return (qr * qr).mean(axis=0)


def waterfill_theta(sigma2, total_bits):
    """Continuous reverse water-filling: theta with sum_i max(0, 1/2 log2(sigma_i^2/theta)) = B.

    Returns (theta, D, R): D_i = min(theta, sigma_i^2), R_i = 1/2 log2(sigma_i^2 / D_i).
    """
    s2 = np.asarray(sigma2, dtype=np.float64)
    pos = s2[s2 > 0]

    def rate(theta):
        return np.maximum(0.0, 0.5 * np.log2(pos / theta)).sum()

    lo, hi = math.log(pos.max()) - 200.0, math.log(pos.max())
    for _ in range(400):
        mid = 0.5 * (lo + hi)
        if rate(math.exp(mid)) > total_bits:
            lo = mid
        else:
            hi = mid
    theta = math.exp(0.5 * (lo + hi))
    dist = np.minimum(theta, s2)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s2 > 0, 0.5 * np.log2(s2 / dist), 0.0)
    return theta, dist, r


# ----------------------------------------------------------------------------------
# Uniform scalar quantizer  [ABL first abstract ("MSE" scalar quantizer); NOVA abstract
# (fixed-width scalar quantizers); per-channel scale/offset]
# ----------------------------------------------------------------------------------
def _phi(z):
    return np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def _upper_tail(z):
    return special.ndtr(-z)


def _bins_positive(b, step):
    """Positive half of the mid-rise quantizer with 2^b levels and step ``step``.

    Returns per bin: phi and upper-tail mass at both edges, z*phi at both edges, the
    reconstruction point r_k = (k + 1/2) step and the level offset a_k = k + 1/2.
    The last bin extends to +inf (phi, z*phi and the tail are 0 there)."""
    half = 2 ** (b - 1)
    k = np.arange(half, dtype=np.float64)
    lo = k * step
    hi = (k + 1) * step
    last = np.arange(half) == half - 1
    phi_lo, phi_hi = _phi(lo), np.where(last, 0.0, _phi(hi))
    tail_lo, tail_hi = _upper_tail(lo), np.where(last, 0.0, _upper_tail(hi))
    zphi_lo, zphi_hi = lo * phi_lo, np.where(last, 0.0, hi * _phi(hi))
    return phi_lo, phi_hi, tail_lo, tail_hi, zphi_lo, zphi_hi, (k + 0.5) * step, k + 0.5


def uniform_quantizer_mse(b, step):
    """E[(Z - Q(Z))^2], Z ~ N(0,1), mid-rise uniform quantizer with 2^b levels
    (k - 2^(b-1) + 1/2) * step, from the closed form
    int_a^b (z-r)^2 phi = [Phi - z phi]_a^b + 2r[phi]_a^b + r^2 [Phi]_a^b
    summed over bins (twice the positive half, by symmetry)."""
    phi_lo, phi_hi, t_lo, t_hi, zp_lo, zp_hi, r, _ = _bins_positive(b, step)
    mass = t_lo - t_hi                       # int phi
    first = phi_lo - phi_hi                  # int z phi
    second = mass + zp_lo - zp_hi            # int z^2 phi
    return float(2.0 * np.sum(second - 2.0 * r * first + r * r * mass))


def uniform_quantizer_mse_deriv(b, step):
    """d MSE / d step.  Boundary terms cancel at the mid-point thresholds, leaving
    -2 sum_k a_k int_bin (z - r_k) phi(z) dz over all bins (twice the positive half)."""
    phi_lo, phi_hi, t_lo, t_hi, _, _, r, a = _bins_positive(b, step)
    return float(-4.0 * np.sum(a * ((phi_lo - phi_hi) - r * (t_lo - t_hi))))


def optimal_step(b):
    """g(b): the MSE-optimal step of the 2^b-level mid-rise uniform quantizer for N(0,1),
    the root of d MSE / d step (bracketed root finding)."""
    if b < 1:
        raise ValueError("b >= 1")
    return optimize.brentq(lambda s: uniform_quantizer_mse_deriv(b, s), 1e-4, 4.0,
                           xtol=1e-300, rtol=4 * np.finfo(float).eps, maxiter=500)


# ----------------------------------------------------------------------------------
# Lloyd-Max scalar quantizer  [SPHERICAL KV page, NOVA-KV abstract: fixed-width uniform
# scalar quantizers lose at low rates; "Ablation ..." page, OCTOPUS abstract: each coordinate
# is quantized with the Lloyd-Max quantizer of the marginal it follows]
#
# The codebook of a channel with b bits is the MSE-optimal 2^b-level quantizer of N(0,1),
# scaled by the channel's standard deviation and centred on its offset: reconstruction
# y_hat = o + sigma l_c, cell boundaries at o + sigma t_k.  Lloyd's necessary conditions fix it:
# every level is the mean of N(0,1) over its cell, every threshold the midpoint of its two
# levels; for a log-concave density they have one solution.
# ----------------------------------------------------------------------------------
def _lm_centroids(t):
    """Mean of N(0,1) over each cell [t_k, t_(k+1)) of the positive half-line (t_0 = 0, last cell
    unbounded), with the cells' masses and the densities at the boundaries."""
    tt = np.concatenate([t, [np.inf]])
    dens = np.where(np.isinf(tt), 0.0, _phi(np.where(np.isinf(tt), 0.0, tt)))
    tail = np.where(np.isinf(tt), 0.0, _upper_tail(np.where(np.isinf(tt), 0.0, tt)))
    mass = tail[:-1] - tail[1:]
    return (dens[:-1] - dens[1:]) / mass, mass, dens


def lloyd_max_gaussian(b):
    """Levels (2^b, ascending) and thresholds (2^b - 1, ascending) of the 2^b-level Lloyd-Max
    quantizer of N(0,1).  By symmetry only the positive half is solved: h = 2^(b-1) levels
    y_1 < ... < y_h, thresholds t_0 = 0 and t_k = (y_k + y_(k+1)) / 2.  Lloyd iterations
    (levels <- cell means) bring the levels near the fixed point; Newton steps on
    y - centroid(y) = 0, whose Jacobian is tridiagonal, then converge to rounding level."""
    if b < 1:
        raise ValueError("b >= 1")
    h = 2 ** (b - 1)
    if h == 1:
        y = np.array([math.sqrt(2.0 / math.pi)])
    else:
        y = (np.arange(h) + 0.5) * (1.0 + 0.5 * b) / h       # a uniform start

        def thresholds(y):
            return np.concatenate([[0.0], 0.5 * (y[:-1] + y[1:])])

        for _ in range(200):
            y = _lm_centroids(thresholds(y))[0]
        for _ in range(60):
            t = thresholds(y)
            c, mass, dens = _lm_centroids(t)
            # d c_k / d t_k (left edge) and d c_k / d t_(k+1) (right edge)
            dl = dens[:-1] * (c - t) / mass
            dr = dens[1:] * (np.concatenate([t[1:], [0.0]]) - c) / mass
            dl[0] = 0.0                                  # t_0 = 0 is fixed
            # Jacobian of F(y) = y - c(y): t_k (k >= 1) moves with y_(k-1) and y_k by 1/2 each
            diag = 1.0 - 0.5 * (dl + np.concatenate([dr[:-1], [0.0]]))
            sub = -0.5 * dl[1:]                          # F_k with respect to y_(k-1)
            sup = -0.5 * dr[:-1]                         # F_k with respect to y_(k+1)
            ab = np.zeros((3, h))
            ab[0, 1:] = sup
            ab[1] = diag
            ab[2, :-1] = sub
            step = linalg.solve_banded((1, 1), ab, -(y - c))
            y = y + step
            if np.abs(step).max() <= 1e-17 * y.max():
                break
    t_pos = 0.5 * (y[:-1] + y[1:])
    levels = np.concatenate([-y[::-1], y])
    thresholds = np.concatenate([-t_pos[::-1], [0.0], t_pos])
    return levels, thresholds


def lloyd_max_mse(b):
    """E[(Z - Q(Z))^2] of the Lloyd-Max quantizer of N(0,1): by the centroid condition it is
    1 - sum_k P(cell k) l_k^2."""
    levels, th = lloyd_max_gaussian(b)
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    cdf = np.where(np.isinf(edges), (edges > 0).astype(float), special.ndtr(np.where(np.isinf(edges), 0.0, edges)))
    mass = np.diff(cdf)
    return float(1.0 - np.sum(mass * levels * levels))


def quantizer_tables(r, mu, sigma2, bits):
    """Per-channel offset o = R mu, step Delta_i = sigma_i g(b_i) and 1/Delta_i.

    Channels with b_i = 0 get Delta = 0 (no code; they reconstruct to o_i).  A coded
    channel with sigma_i = 0 gets Delta_i = 2^-40 max_j sigma_j (1 if every sigma is 0).
    """
    o = np.asarray(r, dtype=np.float64) @ np.asarray(mu, dtype=np.float64)
    sig = np.sqrt(np.asarray(sigma2, dtype=np.float64))
    ref = sig.max() if sig.max() > 0 else 1.0
    delta = np.zeros_like(sig)
    for i, b in enumerate(bits):
        if b > 0:
            s = sig[i] if sig[i] > 0 else math.ldexp(ref, -40)
            delta[i] = s * optimal_step(int(b))
    with np.errstate(divide="ignore"):
        inv = np.where(delta > 0, 1.0 / np.where(delta > 0, delta, 1.0), 0.0)
    return o, delta, inv


def calibrate(x_cal, rotation="klt", bits_per_elem=2.0, max_bits=MAX_BITS, total_bits=None, q_cal=None,
              quantizer="uniform"):
    """Full calibration of one (head, tensor): statistics, rotation, bits, quantizer tables.

    quantizer="uniform": the mid-rise uniform quantizer with step sigma_i g(b_i);
    quantizer="lloyd-max": channel i's codebook is the Lloyd-Max quantizer of N(0,1) with b_i
    bits scaled by s_i (sigma_i, or the coded-zero-variance substitute of quantizer_tables).

    q_cal (keys only): calibration queries of the head's q heads.  With an orthogonal
    rotation the bits then minimise the attention-aware distortion
    sum_i E[(R q)_i^2] sigma_i^2 4^-b_i instead of the cache MSE.  rotation="nova" needs q_cal:
    the transform is transform_nova(C, query_moment(q_cal)), under which that distortion is
    the plain MSE of the coefficients, so the bits use unit weights.

    The artefact's "E" is the encoder matrix (y = E x) and "R" the matrix of the query
    (q~ = R q) and of reconstruction (x = R^T y); they are the same matrix except for "nova".
    """
    mu, c = calib_stats(x_cal)
    d = c.shape[0]
    b_total = bits_budget(bits_per_elem, d) if total_bits is None else int(total_bits)
    if rotation == "nova":
        if q_cal is None:
            raise ValueError("the nova transform needs calibration queries")
        e, r, s2 = transform_nova(c, query_moment(q_cal))
        weight = None
    else:
        rot = {"klt": rotation_klt, "wht": rotation_wht, "identity": rotation_identity}[rotation]
        r, s2 = rot(c)
        e = r
        weight = None if q_cal is None else query_channel_weights(r, q_cal)
    bits = waterfill_bits(s2, b_total, max_bits, weight)
    o, delta, inv = quantizer_tables(e, mu, s2, bits)
    art = {"R": r, "E": e, "mu": mu, "C": c, "sigma2": s2, "bits": bits, "B": b_total,
           "o": o, "delta": delta, "inv_delta": inv, "rotation": rotation, "weight": weight,
           "quantizer": quantizer}
    if quantizer == "lloyd-max":
        sig = np.sqrt(np.asarray(s2, dtype=np.float64))
        ref = sig.max() if sig.max() > 0 else 1.0
        scale = np.where(bits > 0, np.where(sig > 0, sig, math.ldexp(ref, -40)), 0.0)
        with np.errstate(divide="ignore"):
            inv_scale = np.where(scale > 0, 1.0 / np.where(scale > 0, scale, 1.0), 0.0)
        art["scale"], art["inv_scale"] = scale, inv_scale
        art["lm"] = {int(b): lloyd_max_gaussian(int(b)) for b in set(int(v) for v in bits) if b > 0}
    elif quantizer != "uniform":
        raise ValueError(quantizer)
    return art


# ----------------------------------------------------------------------------------
# Encode / dequantize / reconstruct
# ----------------------------------------------------------------------------------
def rotate(x, art):
    """Transform coefficients y = E x of rows x [N, d] in fp64 (E = R for orthogonal rotations).

    Walsh-Hadamard: y = (H x) * (1/sqrt(d)), the +-1 sums H x taken exactly (fp64 holds every
    partial sum of bf16 inputs exactly) and then one multiply by 1/sqrt(d) rounded to fp64, the
    same definition R x with R = H / sqrt(d) has, without rounding each product separately.
    """
    x = np.asarray(x, dtype=np.float64)
    if art.get("rotation") == "wht":
        d = x.shape[-1]
        with np.errstate(invalid="ignore", over="ignore"):
            return (x @ hadamard_signs(d).T) * (1.0 / math.sqrt(d))
    with np.errstate(invalid="ignore", over="ignore"):
        return x @ np.asarray(art.get("E", art["R"])).T


def encode_codes(x, art):
    """Codes c[N, d] (0 for 0-bit channels) of rows x [N, d].

    y = rotate(x) in fp64; u = (y - o) * (1/Delta) + 2^(b-1) as separately rounded fp64
    operations;
    c = clamp(floor(u), 0, 2^b - 1) (half-open bins: a value on an edge goes up);
    NaN -> 0, +-Inf -> the clamp ends.
    """
    x = np.asarray(x, dtype=np.float64)
    bits = np.asarray(art["bits"])
    y = rotate(x, art)
    if art.get("quantizer") == "lloyd-max":
        # z = (y - o) * (1/s) as separately rounded fp64 operations; the code is the number of
        # thresholds at or below z (a value on a threshold goes up); NaN -> 0
        c = np.zeros(y.shape, dtype=np.int64)
        with np.errstate(invalid="ignore", over="ignore"):
            z = (y - art["o"][None, :]) * art["inv_scale"][None, :]
        for i in range(y.shape[1]):
            b = int(bits[i])
            if b == 0:
                continue
            th = art["lm"][b][1]
            zi = z[:, i]
            ci = np.searchsorted(th, zi, side="right")
            c[:, i] = np.where(np.isnan(zi), 0, ci)
        return c
    with np.errstate(invalid="ignore", over="ignore"):
        half = np.where(bits > 0, np.ldexp(1.0, np.maximum(bits, 1) - 1), 0.0)
        u = (y - art["o"][None, :]) * art["inv_delta"][None, :]
        u = u + half[None, :]
        top = np.where(bits > 0, np.ldexp(1.0, bits) - 1.0, 0.0)
        c = np.floor(u)
        c = np.where(np.isnan(c), 0.0, c)
        c = np.clip(c, 0.0, top[None, :])
    c[:, bits == 0] = 0
    return c.astype(np.int64)


def dequantize(codes, art):
    """y_hat_i = o_i + Delta_i (c_i - 2^(b_i-1) + 1/2) for b_i >= 1, o_i for b_i = 0
    (Lloyd-Max: o_i + s_i l_(b_i)[c_i])."""
    bits = np.asarray(art["bits"])
    if art.get("quantizer") == "lloyd-max":
        codes = np.asarray(codes)
        yh = np.repeat(art["o"][None, :], codes.shape[0], axis=0).astype(np.float64)
        for i in range(codes.shape[1]):
            b = int(bits[i])
            if b:
                yh[:, i] = art["o"][i] + art["scale"][i] * art["lm"][b][0][codes[:, i]]
        return yh
    half = np.where(bits > 0, np.ldexp(1.0, np.maximum(bits, 1) - 1), 0.0)
    yh = art["o"][None, :] + art["delta"][None, :] * (np.asarray(codes, dtype=np.float64) - half[None, :] + 0.5)
    yh[:, bits == 0] = art["o"][bits == 0][None, :]
    return yh


def reconstruct(codes, art):
    """x_hat = R^T y_hat (for "nova", R^T = E^-1)."""
    return dequantize(codes, art) @ np.asarray(art["R"])


# ----------------------------------------------------------------------------------
# Packed formats (fixed per-token bit count, [NOVA] third abstract)
#
# Tiles of 64 tokens; a tile holds exactly 64*B bits = 2B little-endian uint32 words.
# String bit s of a tile is bit (s mod 32) of word floor(s/32).
#
# K tiles -- token-major bit-planes: token t (0..63) owns string bits [tB, tB+B); its
#   plane p sits at bit tB + p, planes ordered by channel ascending, then code bit
#   ascending (plane (i,k) carries bit k of c_i).
#
# V tiles -- field-major: channel i's code is split into fields by the binary expansion of
#   b_i into widths {4,2,1} (8 = 4+4), low code bits in the widest field.  Fields are
#   ordered by width descending, then channel ascending, then shift ascending.  A field of
#   width w owns 2w consecutive words (64 tokens x w bits).  Bit b (LSB first) of the
#   value of token t = 16G + 4r + m (G, r, m in 0..3) sits at bit offset
#     w=1: 32*(G//2) + 8m + 2r + (G%2)
#     w=2: 32G + ((8m + 2r + b + (G%2)) mod 32)      (odd G: the word rotated left by 1)
#     w=4: 64G + 32*(r//2) + 8m + 4*(r%2) + b
#   of the field's bit string.
# ----------------------------------------------------------------------------------
def packed_words(total_bits, n_tokens):
    return -(-int(n_tokens) // TILE) * 2 * int(total_bits)


def _planes(bits):
    return [(i, k) for i in range(len(bits)) for k in range(int(bits[i]))]


def _set_bits(words, start, value, width):
    for k in range(width):
        if (value >> k) & 1:
            s = start + k
            words[s // 32] |= np.uint32(1 << (s % 32))


def _get_bits(words, start, width):
    v = 0
    for k in range(width):
        s = start + k
        v |= ((int(words[s // 32]) >> (s % 32)) & 1) << k
    return v


def pack_k(codes, bits):
    """Token-major bit-plane tiles for K codes [N, d]; returns uint32 words."""
    codes = np.asarray(codes)
    n = codes.shape[0]
    b_total = int(np.sum(bits))
    words = np.zeros(packed_words(b_total, n), dtype=np.uint32)
    planes = _planes(bits)
    for t in range(n):
        base = (t // TILE) * 64 * b_total + (t % TILE) * b_total
        for p, (i, k) in enumerate(planes):
            if (int(codes[t, i]) >> k) & 1:
                s = base + p
                words[s // 32] |= np.uint32(1 << (s % 32))
    return words


def unpack_k(words, bits, n):
    d = len(bits)
    b_total = int(np.sum(bits))
    planes = _planes(bits)
    codes = np.zeros((n, d), dtype=np.int64)
    for t in range(n):
        base = (t // TILE) * 64 * b_total + (t % TILE) * b_total
        for p, (i, k) in enumerate(planes):
            s = base + p
            codes[t, i] |= ((int(words[s // 32]) >> (s % 32)) & 1) << k
    return codes


def v_fields(bits):
    """Field list [(channel, shift, width)] in tile order."""
    fields = []
    for i, b in enumerate(bits):
        rest, shift = int(b), 0
        for w in (4, 2, 1):
            while rest >= w:
                fields.append((i, shift, w))
                shift += w
                rest -= w
    fields.sort(key=lambda f: (-f[2], f[0], f[1]))
    return fields


def _v_bit(t, w, b):
    """Offset of bit b of token t's w-bit value in its field's bit string (layout above)."""
    g, r, m = t // 16, (t // 4) % 4, t % 4
    if w == 1:
        return 32 * (g // 2) + 8 * m + 2 * r + (g % 2)
    if w == 2:
        return 32 * g + (8 * m + 2 * r + b + (g % 2)) % 32
    if w == 4:
        return 64 * g + 32 * (r // 2) + 8 * m + 4 * (r % 2) + b
    raise ValueError(w)


def pack_v(codes, bits):
    """Field-major tiles for V codes [N, d]; returns uint32 words."""
    codes = np.asarray(codes)
    n = codes.shape[0]
    b_total = int(np.sum(bits))
    words = np.zeros(packed_words(b_total, n), dtype=np.uint32)
    fields = v_fields(bits)
    for t in range(n):
        tile_base = (t // TILE) * 2 * b_total * 32
        off = 0
        for (i, shift, w) in fields:
            val = (int(codes[t, i]) >> shift) & ((1 << w) - 1)
            for b in range(w):
                _set_bits(words, tile_base + off * 32 + _v_bit(t % TILE, w, b), (val >> b) & 1, 1)
            off += 2 * w
    return words


def unpack_v(words, bits, n):
    d = len(bits)
    b_total = int(np.sum(bits))
    fields = v_fields(bits)
    codes = np.zeros((n, d), dtype=np.int64)
    for t in range(n):
        tile_base = (t // TILE) * 2 * b_total * 32
        off = 0
        for (i, shift, w) in fields:
            for b in range(w):
                codes[t, i] |= _get_bits(words, tile_base + off * 32 + _v_bit(t % TILE, w, b), 1) << (shift + b)
            off += 2 * w
    return codes


# ----------------------------------------------------------------------------------
# Attention (decode)  -- the plain definition the compressed-domain kernel must match.
# [SPECTRA Abstract / RDKV abstract: the whole cache is read at every generated token;
#  OCTOPUS abstract: attention without materialising the decompressed keys]
# ----------------------------------------------------------------------------------
def attention(q, k, v, scale=None):
    """Softmax attention of one query q [d] over keys k [N, d] and values v [N, d].

    Returns (out [d], lse) with lse = log sum_t exp(s_t).  N = 0 gives (0, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if k.shape[0] == 0:
        return np.zeros(d), -np.inf
    s = scale * (k @ q)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return (e @ v) / z, m + math.log(z)


def attention_streaming(q, k, v, scale=None, chunk=7):
    """Oracle-internal check: the same attention by online softmax over chunks."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m, l, acc = -np.inf, 0.0, np.zeros(d)
    for a in range(0, k.shape[0], chunk):
        s = scale * (np.asarray(k[a:a + chunk], dtype=np.float64) @ q)
        m_new = max(m, s.max())
        f = math.exp(m - m_new) if m > -np.inf else 0.0
        e = np.exp(s - m_new)
        l = l * f + e.sum()
        acc = acc * f + e @ np.asarray(v[a:a + chunk], dtype=np.float64)
        m = m_new
    if l == 0:
        return np.zeros(d), -np.inf
    return acc / l, m + math.log(l)


def rotated_scores(q, r, y):
    """Scores taken in the rotated domain: (R q) . y_t for rotated rows y [N, d]."""
    return np.asarray(y, dtype=np.float64) @ (np.asarray(r, dtype=np.float64) @ np.asarray(q, dtype=np.float64))


def decode_attention(q, k_codes, v_codes, k_arts, v_arts, scale=None, seq_lens=None):
    """Decode attention on the compressed cache, by its plain definition:
    reconstruct K and V per KV head, then ordinary softmax attention per q head
    (contiguous GQA groups: q head g reads KV head g // (Hq/Hkv)).

    q [Hq, d]; k_codes / v_codes: list over KV heads of code arrays [N_h, d];
    k_arts / v_arts: list of calibration artefacts.  Returns (out [Hq, d], lse [Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    hkv = len(k_codes)
    group = hq // hkv
    out = np.zeros_like(q)
    lse = np.zeros(hq)
    for h in range(hkv):
        n = k_codes[h].shape[0] if seq_lens is None else int(seq_lens[h])
        kh = reconstruct(k_codes[h][:n], k_arts[h])
        vh = reconstruct(v_codes[h][:n], v_arts[h])
        for g in range(h * group, (h + 1) * group):
            out[g], lse[g] = attention(q[g], kh, vh, scale)
    return out, lse


# ----------------------------------------------------------------------------------
# Token tiers (joint token x channel allocation)  [RDKV abstract: each token gets a width
# between zero bits and full precision from reverse water-filling, decided once when prefill
# ends; AATC Key points: the distortion separates over tokens and channels]
# ----------------------------------------------------------------------------------
TIERS = (0, 2, 4, 16)


def tier_distortions(sigma2_list, d, max_bits=MAX_BITS):
    """Per-tier vector distortion D(tau) = sum over the given tensors of
    sum_i sigma_i^2 4^-b_i(tau), where b(tau) is the water-filling at tau*d bits;
    D(0) = total variance (evicted), D(16) = 0 (kept raw)."""
    out = []
    for tau in TIERS:
        tot = 0.0
        for s2 in sigma2_list:
            s2 = np.asarray(s2, dtype=np.float64)
            if tau == 0:
                tot += s2.sum()
            elif tau == 16:
                tot += 0.0
            else:
                b = waterfill_bits(s2, tau * d, max_bits)
                tot += float(np.sum(s2 * np.ldexp(1.0, -2 * b)))
        out.append(tot)
    return np.array(out)


def _tiers_at(weights, dist, lam, d):
    costs = weights[:, None] * dist[None, :] + lam * d * np.array(TIERS, dtype=np.float64)[None, :]
    # ties go to the lower tier: argmin returns the first minimum
    return np.array(TIERS)[np.argmin(costs, axis=1)]


def token_tiers(attn_mass, dist, d, avg_bits, return_lambda=False):
    """Tier per token in {0,2,4,16} minimising sum_t a_t^2 D(tau_t) subject to
    sum_t tau_t d <= avg_bits * N * d, via a Lagrange multiplier found by bisection
    (the smallest multiplier, hence the largest total, that meets the budget).
    With return_lambda the multiplier is returned too: (tiers, lambda)."""
    a = np.asarray(attn_mass, dtype=np.float64)
    w = a * a
    n = a.shape[0]
    budget = avg_bits * n * d
    dist = np.asarray(dist, dtype=np.float64)

    def total(lam):
        return float(np.sum(_tiers_at(w, dist, lam, d)) * d)

    lam = 0.0
    if total(0.0) > budget:
        lo, hi = 0.0, 1.0
        while total(hi) > budget:
            hi *= 2.0
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if total(mid) > budget:
                lo = mid
            else:
                hi = mid
        lam = hi
    tiers = _tiers_at(w, dist, lam, d)
    return (tiers, lam) if return_lambda else tiers


def segment_attention(q, segments, scale=None):
    """One softmax over the union of several segments of reconstructed tokens.

    segments: list of (k [n_s, d], v [n_s, d]) already in the original basis
    (coded segments reconstructed with their own artefacts; raw segments as stored).
    Evicted tokens are simply absent."""
    k = np.concatenate([np.asarray(s[0], dtype=np.float64) for s in segments], axis=0)
    v = np.concatenate([np.asarray(s[1], dtype=np.float64) for s in segments], axis=0)
    return attention(q, k, v, scale)

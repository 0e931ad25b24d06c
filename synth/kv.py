"""Seeded generators for correlated, outlier-heavy key/value vectors.

Recipe (per config, layer, KV head and tensor K|V):
  1. Q: a Haar-random orthogonal d x d matrix (QR of a standard normal matrix with
     the signs of R's diagonal moved into Q, Mezzadri 2007).
  2. Lambda = diag(i^-1.5), i = 1..d.
  3. z iid N(0,1), or Student-t with 3 degrees of freedom scaled to unit variance.
  4. x = z Lambda^(1/2) Q^T, so x ~ (0, Q Lambda Q^T).
  5. Two seeded original-basis coordinates are multiplied by 10.
  6. Rounded to the storage dtype (fp32, or bf16 with round-to-nearest-even).

Seeds come from numpy SeedSequence(20260814, spawn_key=(cfg, layer, head, tensor,
purpose, extra)).  Small draws use numpy's PCG64 on the host.  Large draws
(``draw_device``) use torch's generator on the chosen device with the same recipe
and the same Q/Lambda/outliers; they are a different random stream and are only
used where the host draw would be too slow.
"""
import numpy as np

ROOT_SEED = 20260814
K, V = 0, 1
PURPOSE = {"Q": 0, "calib": 1, "context": 2, "query": 3, "outlier": 4, "zipf": 5,
           "append": 6, "device": 7}

__all__ = ["ROOT_SEED", "K", "V", "PURPOSE", "seed_seq", "rng", "haar_orthogonal",
           "spectrum", "outlier_coords", "basis", "draw", "round_bf16", "bf16_bits", "to_dtype",
           "draw_device", "queries", "peaked_queries", "zipf_mass", "torch_dtype"]


def seed_seq(cfg, layer, head, tensor, purpose, extra=0):
    return np.random.SeedSequence(ROOT_SEED, spawn_key=(int(cfg), int(layer), int(head), int(tensor),
                                                        PURPOSE[purpose], int(extra)))


def rng(cfg, layer, head, tensor, purpose, extra=0):
    return np.random.Generator(np.random.PCG64(seed_seq(cfg, layer, head, tensor, purpose, extra)))


def haar_orthogonal(g, d):
    a = g.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def spectrum(d):
    return np.arange(1, d + 1, dtype=np.float64) ** -1.5


def outlier_coords(cfg, layer, head, tensor, d=128):
    g = rng(cfg, layer, head, tensor, "outlier")
    return np.sort(g.choice(d, size=2, replace=False))


def basis(cfg, layer, head, tensor, d=128):
    """(Q, lambda, outlier coordinates) of one (config, layer, head, tensor)."""
    q = haar_orthogonal(rng(cfg, layer, head, tensor, "Q"), d)
    return q, spectrum(d), outlier_coords(cfg, layer, head, tensor, d)


def round_bf16(x):
    """Round float values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x):
    """Raw bf16 bit patterns (uint16) of float values that are exactly representable in bf16."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def to_dtype(x, dtype):
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(np.asarray(x, dtype=np.float32))
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def _marginal(g, n, d, marginal):
    z = g.standard_normal((n, d))
    if marginal == "t3":
        chi2 = (g.standard_normal((n, d, 3)) ** 2).sum(-1)
        z = z / np.sqrt(chi2 / 3.0) / np.sqrt(3.0)
    elif marginal != "gauss":
        raise ValueError(marginal)
    return z


def draw(cfg, layer, head, tensor, purpose, n, d=128, marginal="gauss", dtype="bf16", extra=0):
    """n vectors of one head/tensor as float32 (values exact in ``dtype``); f64 if dtype=='f64'."""
    q, lam, out = basis(cfg, layer, head, tensor, d)
    g = rng(cfg, layer, head, tensor, purpose, extra)
    z = _marginal(g, n, d, marginal)
    x = (z * np.sqrt(lam)[None, :]) @ q.T
    x[:, out] *= 10.0
    return to_dtype(x, dtype)


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f64": torch.float64}[dtype]


def draw_device(cfg, layer, head, tensor, n, d=128, marginal="gauss", dtype="bf16", device="cuda",
                extra=0):
    """Large draw with torch's generator on ``device``; same recipe and basis as ``draw``."""
    import torch
    q, lam, out = basis(cfg, layer, head, tensor, d)
    seed = int(seed_seq(cfg, layer, head, tensor, "device", extra).generate_state(1)[0])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    z = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
    if marginal == "t3":
        c = torch.randn((n, d, 3), generator=gen, device=device, dtype=torch.float32)
        z = z / torch.sqrt((c * c).sum(-1) / 3.0) / np.sqrt(3.0)
    m = torch.from_numpy((np.sqrt(lam)[:, None] * q.T)).to(device=device, dtype=torch.float32)
    x = z @ m
    x[:, torch.as_tensor(out, device=device)] *= 10.0
    return x.to(torch_dtype(dtype))


def queries(cfg, layer, n_q_heads, n_kv_heads, keys, d=128, target_std=2.0):
    """One query per q head: a draw from its KV head's key generator, scaled so that the
    fp64 scores q.k/sqrt(d) over ``keys[h]`` (at most 4096 sampled rows) have std target_std.

    keys: sequence of arrays [n_h, d] (host) per KV head.  Returns float32 [n_q_heads, d].
    """
    group = n_q_heads // n_kv_heads
    out = np.zeros((n_q_heads, d), dtype=np.float64)
    for g in range(n_q_heads):
        h = g // group
        qr = draw(cfg, layer, h, K, "query", 1, d=d, dtype="f64", extra=g)[0]
        kh = np.asarray(keys[h], dtype=np.float64)
        if kh.shape[0] > 4096:
            idx = rng(cfg, layer, h, K, "query", extra=1000 + g).choice(kh.shape[0], 4096, replace=False)
            kh = kh[idx]
        s = kh @ qr / np.sqrt(d)
        sd = s.std()
        out[g] = qr * (target_std / sd if sd > 0 else 1.0)
    return out.astype(np.float32)


def peaked_queries(cfg, layer, n_q_heads, n_kv_heads, keys, d=128, margin=12.0):
    """Near one-hot queries: q head g points along one seeded key k_t of its KV head, scaled so
    that the score q.k_t/sqrt(d) exceeds every other score over ``keys[h]`` by ``margin``
    (e^-12 ~ 6e-6 for the runner-up's weight at the default).  Returns float32 [n_q_heads, d]."""
    group = n_q_heads // n_kv_heads
    out = np.zeros((n_q_heads, d), dtype=np.float64)
    for g in range(n_q_heads):
        h = g // group
        kh = np.asarray(keys[h], dtype=np.float64)
        norms = np.einsum("ij,ij->i", kh, kh)
        # among the 64 longest keys, in a seeded order, the first whose own direction scores it
        # above every other key
        cand = np.argsort(-norms, kind="stable")[:64]
        cand = cand[rng(cfg, layer, h, K, "query", extra=2000 + g).permutation(cand.size)]
        for t in cand:
            s = kh @ (kh[t] / np.sqrt(d))
            gap = s[t] - np.max(np.delete(s, t))
            if gap > 0:
                break
        if not gap > 0:
            raise ValueError("no key dominates its own direction")
        out[g] = kh[t] * (margin / gap)
    return out.astype(np.float32)


def zipf_mass(cfg, layer, head, n, exponent=1.1):
    """Attention mass a_t proportional to r_t^-exponent for a seeded permutation r of 1..n."""
    g = rng(cfg, layer, head, K, "zipf")
    r = g.permutation(n) + 1
    a = r.astype(np.float64) ** -exponent
    return a / a.sum()

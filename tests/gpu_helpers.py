"""Shared helpers for the GPU parity tests: build inputs, run the oracle, compare codes."""
import math

import numpy as np

import oracle as O
import synth


bits16 = synth.bf16_bits


class Case:
    """Synthetic layer: per-head calibration, context K/V and queries, oracle artefacts."""

    def __init__(self, cfg, n_kv, group, n_tokens, batch=1, dtype="bf16", rotation="klt", bpe_k=2.0,
                 bpe_v=None, marginal="gauss", layer=0, n_calib=1024, aware=False, v_rotation=None,
                 n_q_cal=512, quant_k="uniform", quant_v="uniform"):
        self.cfg, self.n_kv, self.group, self.n, self.batch = cfg, n_kv, group, n_tokens, batch
        self.dtype, self.rotation, self.layer = dtype, rotation, layer
        self.v_rotation = rotation if v_rotation is None else v_rotation
        aware = aware or rotation == "nova"          # the non-orthogonal key transform needs queries
        self.bpe_k, self.bpe_v = bpe_k, bpe_k if bpe_v is None else bpe_v
        self.n_q = n_kv * group
        self.cal = {}
        self.x = {}
        for t in (synth.K, synth.V):
            self.cal[t] = [synth.draw(cfg, layer, h, t, "calib", n_calib, dtype=dtype, marginal=marginal)
                           for h in range(n_kv)]
            self.x[t] = np.stack([np.stack([synth.draw(cfg, layer, h, t, "context", n_tokens, dtype=dtype,
                                                       marginal=marginal, extra=b)
                                            for h in range(n_kv)]) for b in range(batch)])  # [b,h,n,d]
        self.q = np.stack([synth.queries(cfg, layer, self.n_q, n_kv, [self.x[synth.K][b, h] for h in range(n_kv)])
                           for b in range(batch)])  # [b, n_q, d]
        # attention-aware keys: calibration queries drawn like the decode queries (their KV
        # head's key generator), n_q_cal per head
        self.q_cal = [synth.draw(cfg, layer, h, synth.K, "query", n_q_cal, dtype="f64", extra=50000) if aware
                      else None for h in range(n_kv)]
        self.quant = {synth.K: quant_k, synth.V: quant_v}
        self.art = {synth.K: [O.calibrate(c, rotation, self.bpe_k, q_cal=qc, quantizer=quant_k)
                              for c, qc in zip(self.cal[synth.K], self.q_cal)],
                    synth.V: [O.calibrate(c, self.v_rotation, self.bpe_v, quantizer=quant_v) for c in self.cal[synth.V]]}
        self.codes = {t: np.stack([np.stack([O.encode_codes(self.x[t][b, h], self.art[t][h])
                                             for h in range(n_kv)]) for b in range(batch)])
                      for t in (synth.K, synth.V)}

    def blobs(self, tensor):
        from compressed_decode_attention_head_amd import api
        bpe = self.bpe_k if tensor == synth.K else self.bpe_v
        out = []
        for h, c in enumerate(self.cal[tensor]):
            xc = c if self.dtype == "f32" else bits16(c)
            qz = self.quant[tensor]
            if tensor == synth.V:
                blob = api.calibrate(xc, self.v_rotation, bpe, quantizer=qz)
            elif self.rotation == "nova":
                blob = api.calibrate(xc, "nova", bpe, query_moment=api.query_moment(self.q_cal[h]), quantizer=qz)
            else:
                blob = api.calibrate(xc, self.rotation, bpe, quantizer=qz)
                if self.q_cal[h] is not None:
                    w = api.query_channel_weights(blob, self.q_cal[h])
                    blob = api.calibrate(xc, self.rotation, bpe, channel_weight=w, quantizer=qz)
            out.append(blob)
        return out

    def torch_x(self, tensor, device="cuda"):
        import torch
        t = torch.from_numpy(np.ascontiguousarray(self.x[tensor], dtype=np.float32))
        if self.dtype == "bf16":
            t = t.to(torch.bfloat16)
        return t.to(device)

    def make_cache(self, capacity=None, device="cuda"):
        from compressed_decode_attention_head_amd import api
        cap = capacity or -(-self.n // 64) * 64
        return api.CompressedKVCache(self.blobs(synth.K), self.blobs(synth.V), self.batch, cap, device=device)

    def queries(self, mode):
        """Queries [batch, n_q, d] float32 at another temperature: a float is the std of the
        scores over the context (the default queries have 2.0); "peaked" points each q head at
        one key, 12 above every other score (near one-hot attention)."""
        keys = [[self.x[synth.K][b, h] for h in range(self.n_kv)] for b in range(self.batch)]
        if mode == "peaked":
            return np.stack([synth.peaked_queries(self.cfg, self.layer, self.n_q, self.n_kv, keys[b])
                             for b in range(self.batch)])
        return np.stack([synth.queries(self.cfg, self.layer, self.n_q, self.n_kv, keys[b], target_std=float(mode))
                         for b in range(self.batch)])

    def oracle_attention(self, seq_lens=None, scale=None, q=None):
        q = self.q if q is None else q
        out = np.zeros((self.batch, self.n_q, 128))
        lse = np.zeros((self.batch, self.n_q))
        for b in range(self.batch):
            n = self.n if seq_lens is None else int(seq_lens[b])
            ks = [self.codes[synth.K][b, h][:n] for h in range(self.n_kv)]
            vs = [self.codes[synth.V][b, h][:n] for h in range(self.n_kv)]
            out[b], lse[b] = O.decode_attention(q[b], ks, vs, self.art[synth.K], self.art[synth.V], scale)
        return out, lse


def excused_mismatch_report(x, art, got, want):
    """Code mismatches; each is excused iff the oracle's y is within 1e-5 max(|e|, |x_t|) of a
    bin edge e.  Returns (n_mismatch, n_unexcused)."""
    bad = np.argwhere(got != want)
    if bad.size == 0:
        return 0, 0
    y = O.rotate(x, art)
    unexcused = 0
    for t, i in bad:
        b = int(art["bits"][i])
        edges = art["o"][i] + (np.arange(1, 2 ** b) - 2 ** (b - 1)) * art["delta"][i]
        k = np.argmin(np.abs(edges - y[t, i]))
        e = edges[k]
        tol = 1e-5 * max(abs(e), float(np.linalg.norm(x[t])))
        if abs(y[t, i] - e) > tol:
            unexcused += 1
    return len(bad), unexcused


def assert_codes_match(x, art, got, want, dtype, what=""):
    """Codes bit-exact up to the bin-edge excuse: every mismatch excused, and at most
    floor(1e-6 x codes) of them in this comparison (so none below a million codes).  Walsh-Hadamard
    coefficients of bf16 rows are exact sums times one rounded constant on both sides, so there
    no mismatch at all is allowed."""
    n_bad, n_unexc = excused_mismatch_report(x, art, got, want)
    assert n_unexc == 0, (what, n_bad, n_unexc)
    assert n_bad <= int(1e-6 * want.size), (what, n_bad, want.size)
    if art.get("rotation") == "wht" and dtype == "bf16":
        assert n_bad == 0, (what, n_bad)
    return n_bad


def unpack_all(words, bits, n, tensor):
    fn = O.unpack_k if tensor == synth.K else O.unpack_v
    return fn(np.asarray(words, dtype=np.uint32), bits, n)


def scale_default():
    return 1.0 / math.sqrt(128)

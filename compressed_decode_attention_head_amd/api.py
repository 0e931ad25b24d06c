"""Python face of libaatc: the same calls as include/aatc.h on numpy arrays and torch tensors.

Every step of the compression path runs inside libaatc (host solver in C++, device steps in
HIP kernels).  This module only validates shapes, allocates with torch and passes pointers.
"""
import ctypes

import numpy as np

from . import _native as N

__all__ = ["calibrate", "calib_view", "validate", "bits_budget", "packed_bytes", "v_tiles",
           "tier_distortions", "token_tiers", "decode_attn_segments", "CompressedKVCache", "AatcError"]

AatcError = N.AatcError


def _np_dtype_code(x):
    if x.dtype == np.float32:
        return N.DTYPE["f32"]
    if x.dtype == np.float64:
        return N.DTYPE["f64"]
    if x.dtype == np.uint16:        # raw bf16 bits
        return N.DTYPE["bf16"]
    raise TypeError("calibration data must be float32, float64 or bf16 bits (uint16)")


def calibrate(x, rotation="klt", bits_per_elem=2.0, max_bits=8, d=128, channel_weight=None, query_moment=None,
              quantizer="uniform"):
    """aatc_calibrate on host rows x [M, d]; returns the artefact blob (uint8 array).
    channel_weight: optional d weights of the rotated channels (query_channel_weights).
    query_moment: the d x d E[q q^T] of calibration queries (query_moment), for rotation "nova".
    quantizer: "uniform" or "lloyd-max"."""
    L = N.lib()
    x = np.ascontiguousarray(x)
    if x.ndim != 2:
        raise ValueError("x must be [n_calib, d]")
    wptr = None
    if channel_weight is not None:
        w = np.ascontiguousarray(channel_weight, dtype=np.float64)
        if w.shape != (d,):
            raise ValueError("channel_weight must have d entries")
        wptr = w.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    mptr = None
    if query_moment is not None:
        mom = np.ascontiguousarray(query_moment, dtype=np.float64)
        if mom.shape != (d, d):
            raise ValueError("query_moment must be d x d")
        mptr = mom.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    p = N.CalibParams(d, N.ROTATION[rotation], float(bits_per_elem), int(max_bits), N.QUANTIZER[quantizer], wptr,
                      mptr)
    nbytes = L.aatc_calib_bytes(d) or N.CALIB_DTYPE.itemsize
    out = np.zeros(nbytes, dtype=np.uint8)
    N.check(L.aatc_calibrate(ctypes.byref(p), x.ctypes.data, _np_dtype_code(x), x.shape[0], x.shape[1],
                             out.ctypes.data, out.nbytes))
    return out


def query_channel_weights(blob, q):
    """aatc_query_channel_weights: attention-aware key weights E[(R q)_i^2] over the host query
    rows q [n, d] (float32, float64 or bf16 bits) for a key blob's rotation."""
    L = N.lib()
    q = np.ascontiguousarray(q)
    if q.ndim != 2:
        raise ValueError("q must be [n, d]")
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    w = np.zeros(q.shape[1], dtype=np.float64)
    N.check(L.aatc_query_channel_weights(blob.ctypes.data, blob.nbytes, q.ctypes.data, _np_dtype_code(q), q.shape[0],
                                         q.shape[1], w.ctypes.data))
    return w


def query_moment(q):
    """aatc_query_moment: E[q q^T] (d x d, fp64) over the host query rows q [n, d] (float32,
    float64 or bf16 bits), the input of the "nova" key transform."""
    L = N.lib()
    q = np.ascontiguousarray(q)
    if q.ndim != 2:
        raise ValueError("q must be [n, d]")
    m = np.zeros((q.shape[1], q.shape[1]), dtype=np.float64)
    N.check(L.aatc_query_moment(q.ctypes.data, _np_dtype_code(q), q.shape[0], q.shape[1], m.ctypes.data))
    return m


def joint_kv_split(k_blobs, v_blobs, total_bits, k_weight=None, scale=0.0):
    """aatc_joint_kv_split: (B_K, B_V) for a layer's per-head K and V blobs (host uint8 arrays),
    optional key weights [n_heads, d] (query_channel_weights) and total bits per (K, V) pair."""
    L = N.lib()
    if len(k_blobs) != len(v_blobs) or not k_blobs:
        raise ValueError("one K and one V blob per head")
    kb = np.ascontiguousarray(np.concatenate([np.asarray(b, dtype=np.uint8) for b in k_blobs]))
    vb = np.ascontiguousarray(np.concatenate([np.asarray(b, dtype=np.uint8) for b in v_blobs]))
    wp = None
    if k_weight is not None:
        w = np.ascontiguousarray(k_weight, dtype=np.float64)
        if w.shape != (len(k_blobs), N.D):
            raise ValueError("k_weight must be [n_heads, d]")
        wp = w.ctypes.data
    bk, bv = ctypes.c_int32(), ctypes.c_int32()
    N.check(L.aatc_joint_kv_split(kb.ctypes.data, vb.ctypes.data, len(k_blobs), wp, float(scale), int(total_bits),
                                  ctypes.byref(bk), ctypes.byref(bv)))
    return bk.value, bv.value


def calib_view(blob):
    """Read-only structured view of a blob (fields as in struct aatc_calib)."""
    return np.frombuffer(np.asarray(blob, dtype=np.uint8).tobytes()[:N.CALIB_DTYPE.itemsize],
                         dtype=N.CALIB_DTYPE)[0]


def validate(blob):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    N.check(N.lib().aatc_calib_validate(blob.ctypes.data, blob.nbytes))


def v_tiles(blob):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    return int(N.lib().aatc_calib_v_tiles(blob.ctypes.data))


def bits_budget(bits_per_elem, d=128):
    return int(N.lib().aatc_bits_budget(float(bits_per_elem), d))


def packed_bytes(total_bits, n_tokens):
    return int(N.lib().aatc_packed_bytes(int(total_bits), int(n_tokens)))


def tier_distortions(sigma2_list, max_bits=8, d=128):
    """aatc_tier_distortions: D(tau) for tiers (0, 2, 4, 16) from rotated variances [n, d]."""
    s2 = np.ascontiguousarray(np.stack([np.asarray(x, dtype=np.float64) for x in sigma2_list]))
    out = np.zeros(4, dtype=np.float64)
    N.check(N.lib().aatc_tier_distortions(s2.ctypes.data, s2.shape[0], d, int(max_bits), out.ctypes.data))
    return out


def token_tiers(attn_mass, dist, avg_bits, d=128):
    """aatc_token_tiers: tier (0, 2, 4 or 16) per token under an average bit budget."""
    a = np.ascontiguousarray(attn_mass, dtype=np.float64)
    dist = np.ascontiguousarray(dist, dtype=np.float64)
    out = np.zeros(a.shape[0], dtype=np.int8)
    N.check(N.lib().aatc_token_tiers(a.ctypes.data, a.shape[0], dist.ctypes.data, d, float(avg_bits),
                                     out.ctypes.data))
    return out


def _segments_struct(segments, batch, n_kv_heads):
    import torch
    arr = (N.Segment * len(segments))()
    keep = []
    for i, sg in enumerate(segments):
        sl = sg.get("seq_lens")
        if sl is not None:
            if sl.dtype != torch.int32 or sl.numel() != batch * n_kv_heads or not sl.is_contiguous():
                raise ValueError("segment seq_lens must be a contiguous int32 [batch, n_kv_heads] tensor")
            arr[i].seq_lens_dev = sl.data_ptr()
        arr[i].max_seq_len = int(sg["max_seq_len"])
        if "cache" in sg:
            arr[i].cache = ctypes.pointer(sg["cache"].struct)
            keep.append(arr[i].cache)
        else:
            k, v = sg["k_raw"], sg["v_raw"]
            if (k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or k.shape != v.shape or k.dim() != 4
                    or not k.is_contiguous() or not v.is_contiguous() or k.shape[:2] != (batch, n_kv_heads)):
                raise ValueError("raw segments are contiguous bf16 [batch, n_kv_heads, capacity, 128] tensors")
            arr[i].k_raw, arr[i].v_raw = k.data_ptr(), v.data_ptr()
            arr[i].raw_capacity = k.shape[2]
    return arr, keep


def decode_attn_segments_workspace_bytes(segments, batch, n_kv_heads, n_q_heads):
    """aatc_decode_attn_segments_workspace_bytes for the same segment list as decode_attn_segments."""
    arr, _keep = _segments_struct(segments, batch, n_kv_heads)
    need = N.lib().aatc_decode_attn_segments_workspace_bytes(arr, len(segments), batch, n_kv_heads, n_q_heads)
    if need == 0:
        raise ValueError("invalid segments: " + N.lib().aatc_last_error().decode())
    return need


def decode_attn_segments(segments, q, batch, n_kv_heads, scale=0.0, workspace=None, out=None, lse=None,
                         stream=None):
    """aatc_decode_attn_segments.  segments: list of dicts, each either
    {"cache": CompressedKVCache, "seq_lens": int32 [batch, n_kv] tensor, "max_seq_len": n} or
    {"k_raw": bf16 [batch, n_kv, cap, 128], "v_raw": same, "seq_lens": ..., "max_seq_len": n}."""
    import torch
    if q.dtype != torch.float32 or not q.is_contiguous() or q.dim() != 3 or q.shape[0] != batch:
        raise ValueError("q must be a contiguous fp32 [batch, n_q_heads, 128] tensor")
    arr, _keep = _segments_struct(segments, batch, n_kv_heads)
    n_q = q.shape[1]
    L = N.lib()
    need = L.aatc_decode_attn_segments_workspace_bytes(arr, len(segments), batch, n_kv_heads, n_q)
    if need == 0:
        raise ValueError("invalid segments: " + L.aatc_last_error().decode())
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((batch, n_q), dtype=torch.float32, device=q.device)
    N.check(L.aatc_decode_attn_segments(arr, len(segments), batch, n_kv_heads, q.data_ptr(), n_q, float(scale),
                                        out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                        _stream_ptr(stream)))
    return out, lse


def decode_attn_dense_workspace_bytes(batch, n_kv_heads, n_q_heads, max_seq_len):
    """aatc_decode_attn_dense_workspace_bytes."""
    need = N.lib().aatc_decode_attn_dense_workspace_bytes(batch, n_kv_heads, n_q_heads, max_seq_len)
    if need == 0:
        raise ValueError("invalid shape: " + N.lib().aatc_last_error().decode())
    return need


def decode_attn_dense(k, v, q, max_seq_len, seq_lens=None, scale=0.0, workspace=None, out=None, lse=None,
                      stream=None):
    """aatc_decode_attn_dense: softmax attention over an uncompressed bf16 cache.
    k, v: contiguous bf16 [batch, n_kv, capacity, 128]; q: contiguous fp32 [batch, n_q, 128];
    seq_lens: contiguous int32 [batch, n_kv] or None (max_seq_len everywhere)."""
    import torch
    if (k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or k.shape != v.shape or k.dim() != 4
            or not k.is_contiguous() or not v.is_contiguous()):
        raise ValueError("k and v must be contiguous bf16 [batch, n_kv_heads, capacity, 128] tensors")
    batch, n_kv, cap = k.shape[0], k.shape[1], k.shape[2]
    if q.dtype != torch.float32 or not q.is_contiguous() or q.dim() != 3 or q.shape[0] != batch:
        raise ValueError("q must be a contiguous fp32 [batch, n_q_heads, 128] tensor")
    sl = 0
    if seq_lens is not None:
        if seq_lens.dtype != torch.int32 or seq_lens.numel() != batch * n_kv or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be a contiguous int32 [batch, n_kv_heads] tensor")
        sl = seq_lens.data_ptr()
    n_q = q.shape[1]
    L = N.lib()
    if workspace is None:
        workspace = torch.empty(decode_attn_dense_workspace_bytes(batch, n_kv, n_q, max_seq_len), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((batch, n_q), dtype=torch.float32, device=q.device)
    N.check(L.aatc_decode_attn_dense(k.data_ptr(), v.data_ptr(), batch, n_kv, cap, sl or None, int(max_seq_len),
                                     q.data_ptr(), n_q, float(scale), out.data_ptr(), lse.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))
    return out, lse


def probe_read(buf, sink=None, stream=None):
    """aatc_probe_read: one streaming read of the device tensor `buf` (measurement helper)."""
    import torch
    if sink is None:
        sink = torch.empty(N.lib().aatc_probe_read_sink_bytes(), dtype=torch.uint8, device=buf.device)
    N.check(N.lib().aatc_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                    _stream_ptr(stream)))
    return sink


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class CompressedKVCache:
    """One layer's compressed K/V cache on the GPU: per-head artefacts + packed tiles.

    k_blobs / v_blobs: one artefact per KV head (from ``calibrate``).  Memory is
    [batch][n_kv_heads][capacity/64 tiles][2B words] per tensor (uint32 as torch.int32).
    """

    def __init__(self, k_blobs, v_blobs, batch, capacity_tokens, device="cuda"):
        import torch
        if capacity_tokens % 64:
            raise ValueError("capacity_tokens must be a multiple of 64")
        if len(k_blobs) != len(v_blobs) or not k_blobs:
            raise ValueError("need one K and one V artefact per KV head")
        for b in list(k_blobs) + list(v_blobs):
            validate(b)
        kb = {int(calib_view(b)["total_bits"]) for b in k_blobs}
        vb = {int(calib_view(b)["total_bits"]) for b in v_blobs}
        if len(kb) != 1 or len(vb) != 1:
            raise ValueError("all heads of a tensor must share the bit budget")
        self.batch, self.n_kv, self.capacity = int(batch), len(k_blobs), int(capacity_tokens)
        self.k_bits, self.v_bits = kb.pop(), vb.pop()
        self.v_tiles = max(v_tiles(b) for b in v_blobs)
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.k_blobs_host = [np.asarray(b, dtype=np.uint8) for b in k_blobs]
        self.v_blobs_host = [np.asarray(b, dtype=np.uint8) for b in v_blobs]
        self.k_calib = torch.from_numpy(np.concatenate(self.k_blobs_host)).to(self.device)
        self.v_calib = torch.from_numpy(np.concatenate(self.v_blobs_host)).to(self.device)
        tiles = self.capacity // 64
        # + 4 words: decode attention copies whole 16-byte units, up to 15 bytes past the end
        self.k_codes = torch.zeros(4 + self.batch * self.n_kv * tiles * 2 * self.k_bits, dtype=torch.int32,
                                   device=self.device)
        self.v_codes = torch.zeros(4 + self.batch * self.n_kv * tiles * 2 * self.v_bits, dtype=torch.int32,
                                   device=self.device)
        kq = {int(calib_view(b)["quantizer"]) for b in k_blobs}
        vq = {int(calib_view(b)["quantizer"]) for b in v_blobs}
        if len(kq) != 1 or len(vq) != 1:
            raise ValueError("all heads of a tensor must share the quantizer")
        self.quantizer = kq.pop() | (vq.pop() << 1)
        self._struct = N.Cache(self.batch, self.n_kv, 128, self.k_bits, self.v_bits, self.v_tiles,
                               self.quantizer, 0, self.capacity, self.k_calib.data_ptr(), self.v_calib.data_ptr(),
                               self.k_codes.data_ptr(), self.v_codes.data_ptr())

    @property
    def struct(self):
        return self._struct

    def codes(self, which):
        """Packed words of one tensor as [batch, n_kv, capacity/64 * 2B] int32 (a view)."""
        c = self.k_codes if which == 0 else self.v_codes
        bits = self.k_bits if which == 0 else self.v_bits
        return c[: self.batch * self.n_kv * (self.capacity // 64) * 2 * bits].view(self.batch, self.n_kv, -1)

    @staticmethod
    def _dt(t):
        import torch
        if t.dtype == torch.float32:
            return N.DTYPE["f32"]
        if t.dtype == torch.bfloat16:
            return N.DTYPE["bf16"]
        raise TypeError("float32 or bfloat16 tensors only")

    def encode(self, which, x, token_offset=0, stream=None):
        """aatc_encode: x [batch, n_kv, n, 128] (any strides, channel stride 1)."""
        if x.dim() != 4 or x.shape[0] != self.batch or x.shape[1] != self.n_kv or x.shape[3] != 128:
            raise ValueError("x must be [batch, n_kv_heads, n, 128]")
        if x.stride(3) != 1:
            raise ValueError("channel stride must be 1")
        if x.device != self.device:
            raise ValueError("x must live on the cache's device")
        st = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
        N.check(N.lib().aatc_encode(ctypes.byref(self._struct), int(which), x.data_ptr(), self._dt(x), st,
                                    int(token_offset), int(x.shape[2]), _stream_ptr(stream)))

    def encode_kv(self, k, v, token_offset=0, stream=None):
        """aatc_encode_kv: K and V rows [batch, n_kv, n, 128] of one dtype, one launch."""
        for x in (k, v):
            if x.dim() != 4 or x.shape[0] != self.batch or x.shape[1] != self.n_kv or x.shape[3] != 128:
                raise ValueError("k and v must be [batch, n_kv_heads, n, 128]")
            if x.stride(3) != 1:
                raise ValueError("channel stride must be 1")
            if x.device != self.device:
                raise ValueError("k and v must live on the cache's device")
        if k.shape != v.shape or k.dtype != v.dtype:
            raise ValueError("k and v must have one shape and dtype")
        sk = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
        sv = (ctypes.c_int64 * 3)(v.stride(0), v.stride(1), v.stride(2))
        N.check(N.lib().aatc_encode_kv(ctypes.byref(self._struct), k.data_ptr(), v.data_ptr(), self._dt(k), sk, sv,
                                       int(token_offset), int(k.shape[2]), _stream_ptr(stream)))

    def decode(self, which, token_offset, n_tokens, out_dtype="f32", stream=None):
        """aatc_decode: reconstruction x_hat [batch, n_kv, n, 128]."""
        import torch
        dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out = torch.empty((self.batch, self.n_kv, int(n_tokens), 128), dtype=dt, device=self.device)
        st = (ctypes.c_int64 * 3)(out.stride(0), out.stride(1), out.stride(2))
        N.check(N.lib().aatc_decode(ctypes.byref(self._struct), int(which), int(token_offset), int(n_tokens),
                                    out.data_ptr(), N.DTYPE[out_dtype], st, _stream_ptr(stream)))
        return out

    def workspace_bytes(self, n_q_heads, max_seq_len):
        return int(N.lib().aatc_decode_attn_workspace_bytes(ctypes.byref(self._struct), int(n_q_heads),
                                                            int(max_seq_len)))

    def new_workspace(self, n_q_heads, max_seq_len):
        """Decode-attention workspace (partial records; its contents need no initialisation)."""
        import torch
        return torch.empty(self.workspace_bytes(n_q_heads, max_seq_len), dtype=torch.uint8, device=self.device)

    def _q_dtype(self, q):
        import torch
        if q.dtype not in (torch.float32, torch.bfloat16) or not q.is_contiguous() or q.dim() != 3 \
                or q.shape[0] != self.batch:
            raise ValueError("q must be a contiguous fp32 or bf16 [batch, n_q_heads, 128] tensor")
        return N.DTYPE["f32"] if q.dtype == torch.float32 else N.DTYPE["bf16"]

    def decode_attn(self, q, max_seq_len, seq_lens=None, scale=0.0, workspace=None, out=None, lse=None,
                    stream=None):
        """aatc_decode_attn: q [batch, n_q_heads, 128] fp32 or bf16 -> (out [batch, n_q_heads, 128] fp32,
        lse [batch, n_q])."""
        import torch
        qdt = self._q_dtype(q)
        n_q = q.shape[1]
        if workspace is None:
            workspace = self.new_workspace(n_q, max_seq_len)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((self.batch, n_q), dtype=torch.float32, device=self.device)
        sl = 0
        if seq_lens is not None:
            if seq_lens.dtype != torch.int32 or seq_lens.device != self.device or seq_lens.numel() != self.batch:
                raise ValueError("seq_lens must be an int32 [batch] tensor on the cache's device")
            sl = seq_lens.data_ptr()
        N.check(N.lib().aatc_decode_attn(ctypes.byref(self._struct), q.data_ptr(), qdt, int(n_q), sl or None,
                                         int(max_seq_len), float(scale), out.data_ptr(), lse.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))
        return out, lse

    def decode_attn_noalloc(self, q, max_seq_len, out, lse=None, seq_lens=None, scale=0.0, stream=None):
        """aatc_decode_attn_noalloc: aatc_decode_attn with the library's static per-GPU workspace;
        out (and lse, if given) are the caller's [batch, n_q_heads, 128] / [batch, n_q] fp32 tensors."""
        import torch
        qdt = self._q_dtype(q)
        if out.shape != q.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous fp32 tensor shaped like q")
        if lse is not None and (lse.shape != q.shape[:2] or lse.dtype != torch.float32 or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous fp32 [batch, n_q_heads] tensor")
        N.check(N.lib().aatc_decode_attn_noalloc(ctypes.byref(self._struct), q.data_ptr(), qdt, int(q.shape[1]),
                                                 self._seq_ptr(seq_lens), int(max_seq_len), float(scale),
                                                 out.data_ptr(), None if lse is None else lse.data_ptr(),
                                                 _stream_ptr(stream)))
        return out, lse

    def _seq_ptr(self, seq_lens):
        import torch
        if seq_lens is None:
            return None
        if seq_lens.dtype != torch.int32 or seq_lens.device != self.device or seq_lens.numel() != self.batch:
            raise ValueError("seq_lens must be an int32 [batch] tensor on the cache's device")
        return seq_lens.data_ptr()

    def decode_attn_partial(self, q, max_seq_len, workspace, seq_lens=None, scale=0.0, stream=None):
        """aatc_decode_attn_partial: the cache pass; partial records go to `workspace`."""
        qdt = self._q_dtype(q)
        N.check(N.lib().aatc_decode_attn_partial(ctypes.byref(self._struct), q.data_ptr(), qdt, int(q.shape[1]),
                                                 self._seq_ptr(seq_lens), int(max_seq_len), float(scale),
                                                 workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))

    def decode_attn_merge(self, n_q_heads, max_seq_len, workspace, out, lse=None, seq_lens=None, stream=None):
        """aatc_decode_attn_merge: partial records in `workspace` -> out [batch, n_q, 128], lse."""
        N.check(N.lib().aatc_decode_attn_merge(ctypes.byref(self._struct), int(n_q_heads), self._seq_ptr(seq_lens),
                                               int(max_seq_len), out.data_ptr(),
                                               lse.data_ptr() if lse is not None else None,
                                               workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))
        return out, lse

"""ctypes view of libaatc.so (include/aatc.h).  Argument marshalling only."""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libaatc.so")

AATC_OK = 0
STATUS = {0: "AATC_OK", 1: "AATC_ERR_INVALID_ARGUMENT", 2: "AATC_ERR_UNSUPPORTED", 3: "AATC_ERR_BUDGET",
          4: "AATC_ERR_NUMERICAL", 5: "AATC_ERR_BAD_ARTEFACT", 6: "AATC_ERR_BUFFER_TOO_SMALL",
          7: "AATC_ERR_HIP"}
DTYPE = {"f32": 0, "bf16": 1, "f64": 2}
ROTATION = {"klt": 0, "wht": 1, "identity": 2, "nova": 3}
D = 128
MAX_FIELDS = 384
LEVELS = 510
QUANTIZER = {"uniform": 0, "lloyd-max": 1}

# numpy mirror of struct aatc_calib (checked against aatc_calib_bytes at load time)
CALIB_DTYPE = np.dtype([
    ("magic", "<u4"), ("version", "<u4"), ("d", "<i4"), ("rotation", "<i4"),
    ("total_bits", "<i4"), ("max_bits", "<i4"), ("n_coded", "<i4"), ("n_fields", "<i4"),
    ("n_fields4", "<i4"), ("n_fields2", "<i4"), ("n_fields1", "<i4"), ("n_calib", "<i4"),
    ("checksum", "<u8"),
    ("R", "<f8", (D * D,)), ("mu", "<f8", (D,)), ("o", "<f8", (D,)), ("sigma2", "<f8", (D,)),
    ("delta", "<f8", (D,)), ("inv_delta", "<f8", (D,)),
    ("R32", "<f4", (D * D,)), ("o32", "<f4", (D,)), ("delta32", "<f4", (D,)),
    ("bits", "u1", (D,)), ("plane_channel", "u1", (D * 8,)), ("plane_bit", "u1", (D * 8,)),
    ("field_channel", "<u2", (MAX_FIELDS,)), ("field_shift", "u1", (MAX_FIELDS,)),
    ("field_width", "u1", (MAX_FIELDS,)), ("field_word", "<u2", (MAX_FIELDS,)),
    ("channel_field", "<i2", (D * 3,)), ("E", "<f8", (D * D,)),
    ("quantizer", "<i4"), ("pad0", "<i4"), ("scale", "<f8", (D,)), ("inv_scale", "<f8", (D,)),
    ("scale32", "<f4", (D,)), ("level", "<f8", (LEVELS,)), ("thresh", "<f8", (LEVELS,)),
    ("level32", "<f4", (LEVELS,)), ("reserved", "u1", (64,)),
], align=True)


class CalibParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("rotation", ctypes.c_int32), ("bits_per_elem", ctypes.c_double),
                ("max_bits", ctypes.c_int32), ("quantizer", ctypes.c_int32),
                ("channel_weight", ctypes.POINTER(ctypes.c_double)),
                ("query_moment", ctypes.POINTER(ctypes.c_double))]


class Cache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("d", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("v_tiles", ctypes.c_int32),
                ("quantizer", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("capacity_tokens", ctypes.c_int64),
                ("k_calib", ctypes.c_void_p), ("v_calib", ctypes.c_void_p),
                ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p)]


class Segment(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(Cache)), ("k_raw", ctypes.c_void_p), ("v_raw", ctypes.c_void_p),
                ("raw_capacity", ctypes.c_int64), ("seq_lens_dev", ctypes.c_void_p),
                ("max_seq_len", ctypes.c_int64)]


class AatcError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status
        self.name = STATUS.get(status, str(status))


_lib = None


def lib():
    """The loaded library; raises if libaatc.so has not been built (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libaatc.so is not built; run compressed_decode_attention_head_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
    L.aatc_status_string.restype = ctypes.c_char_p
    L.aatc_status_string.argtypes = [ctypes.c_int]
    L.aatc_last_error.restype = ctypes.c_char_p
    L.aatc_last_error.argtypes = []
    L.aatc_calib_bytes.restype = sz
    L.aatc_calib_bytes.argtypes = [i32]
    L.aatc_bits_budget.restype = i32
    L.aatc_bits_budget.argtypes = [dbl, i32]
    L.aatc_packed_bytes.restype = sz
    L.aatc_packed_bytes.argtypes = [i32, i64]
    L.aatc_calibrate.restype = ctypes.c_int
    L.aatc_calibrate.argtypes = [ctypes.POINTER(CalibParams), vp, ctypes.c_int, i64, i64, vp, sz]
    L.aatc_query_channel_weights.restype = ctypes.c_int
    L.aatc_query_channel_weights.argtypes = [vp, sz, vp, ctypes.c_int, i64, i64, vp]
    L.aatc_calib_validate.restype = ctypes.c_int
    L.aatc_calib_validate.argtypes = [vp, sz]
    L.aatc_calib_v_tiles.restype = i32
    L.aatc_calib_v_tiles.argtypes = [vp]
    L.aatc_encode.restype = ctypes.c_int
    L.aatc_encode.argtypes = [ctypes.POINTER(Cache), i32, vp, ctypes.c_int, ctypes.POINTER(i64), i64, i64, vp]
    L.aatc_encode_kv.restype = ctypes.c_int
    L.aatc_encode_kv.argtypes = [ctypes.POINTER(Cache), vp, vp, ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                 i64, i64, vp]
    L.aatc_decode.restype = ctypes.c_int
    L.aatc_decode.argtypes = [ctypes.POINTER(Cache), i32, i64, i64, vp, ctypes.c_int, ctypes.POINTER(i64), vp]
    L.aatc_decode_attn_workspace_bytes.restype = sz
    L.aatc_decode_attn_workspace_bytes.argtypes = [ctypes.POINTER(Cache), i32, i64]
    L.aatc_decode_attn.restype = ctypes.c_int
    L.aatc_decode_attn.argtypes = [ctypes.POINTER(Cache), vp, i32, i32, vp, i64, ctypes.c_float, vp, vp, vp, sz, vp]
    L.aatc_decode_attn_partial.restype = ctypes.c_int
    L.aatc_probe_read_sink_bytes.restype = sz
    L.aatc_probe_read_sink_bytes.argtypes = []
    L.aatc_probe_read.restype = ctypes.c_int
    L.aatc_probe_read.argtypes = [vp, sz, vp, vp]
    L.aatc_decode_attn_noalloc.restype = ctypes.c_int
    L.aatc_decode_attn_noalloc.argtypes = [ctypes.POINTER(Cache), vp, i32, i32, vp, i64, ctypes.c_float, vp, vp, vp]
    L.aatc_decode_attn_partial.argtypes = [ctypes.POINTER(Cache), vp, i32, i32, vp, i64, ctypes.c_float, vp, sz, vp]
    L.aatc_decode_attn_merge.restype = ctypes.c_int
    L.aatc_decode_attn_merge.argtypes = [ctypes.POINTER(Cache), i32, vp, i64, vp, vp, vp, sz, vp]
    L.aatc_tier_distortions.restype = ctypes.c_int
    L.aatc_tier_distortions.argtypes = [vp, i32, i32, i32, vp]
    L.aatc_token_tiers.restype = ctypes.c_int
    L.aatc_token_tiers.argtypes = [vp, i64, vp, i32, dbl, vp]
    L.aatc_decode_attn_segments_workspace_bytes.restype = sz
    L.aatc_decode_attn_segments_workspace_bytes.argtypes = [ctypes.POINTER(Segment), i32, i32, i32, i32]
    L.aatc_decode_attn_segments.restype = ctypes.c_int
    L.aatc_decode_attn_segments.argtypes = [ctypes.POINTER(Segment), i32, i32, i32, vp, i32, ctypes.c_float, vp,
                                            vp, vp, sz, vp]
    L.aatc_joint_kv_split.restype = ctypes.c_int
    L.aatc_joint_kv_split.argtypes = [vp, vp, i32, vp, ctypes.c_float, i32, vp, vp]
    L.aatc_query_moment.restype = ctypes.c_int
    L.aatc_query_moment.argtypes = [vp, ctypes.c_int, i64, i64, vp]
    L.aatc_decode_attn_dense_workspace_bytes.restype = sz
    L.aatc_decode_attn_dense_workspace_bytes.argtypes = [i32, i32, i32, i64]
    L.aatc_decode_attn_dense.restype = ctypes.c_int
    L.aatc_decode_attn_dense.argtypes = [vp, vp, i32, i32, i64, vp, i64, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]
    if L.aatc_calib_bytes(D) != CALIB_DTYPE.itemsize:
        raise RuntimeError("aatc_calib layout mismatch: library %d bytes, binding %d bytes"
                           % (L.aatc_calib_bytes(D), CALIB_DTYPE.itemsize))
    _lib = L
    return L


def check(status):
    if status != AATC_OK:
        raise AatcError(status, lib().aatc_last_error().decode())


EXPORTS = ["aatc_status_string", "aatc_last_error", "aatc_calib_bytes", "aatc_bits_budget",
           "aatc_packed_bytes", "aatc_calibrate", "aatc_query_channel_weights", "aatc_calib_validate",
           "aatc_calib_v_tiles",
           "aatc_encode", "aatc_encode_kv", "aatc_decode", "aatc_decode_attn_workspace_bytes", "aatc_decode_attn", "aatc_decode_attn_noalloc",
           "aatc_probe_read_sink_bytes", "aatc_probe_read",
           "aatc_decode_attn_partial", "aatc_decode_attn_merge", "aatc_tier_distortions",
           "aatc_token_tiers", "aatc_decode_attn_segments_workspace_bytes", "aatc_decode_attn_segments",
           "aatc_decode_attn_dense_workspace_bytes", "aatc_decode_attn_dense", "aatc_query_moment",
           "aatc_joint_kv_split"]

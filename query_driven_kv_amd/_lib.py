"""ctypes binding of the C ABI in include/think.h (libthinkkv.so, built in-tree).

Argument marshalling only: every step of the pruning path runs in the HIP
kernels behind the C ABI.  Importing this module fails loudly when the
library has not been built; there is no fallback.
"""
import ctypes
import os

_SO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libthinkkv.so")

THINK_F32, THINK_BF16 = 0, 1
STATUS = {0: "THINK_OK", -1: "THINK_ERR_NULL", -2: "THINK_ERR_SHAPE", -3: "THINK_ERR_KEEP",
          -4: "THINK_ERR_DTYPE", -5: "THINK_ERR_UNSUPPORTED", -6: "THINK_ERR_WORKSPACE",
          -7: "THINK_ERR_HIP", -8: "THINK_ERR_WAIT"}

# every function include/think.h declares
EXPORTS = ("think_abi_version", "think_keep_from_ratio", "think_score_workspace_bytes",
           "think_decode_workspace_bytes", "think_score", "think_score_select", "think_select",
           "think_compact_k",
           "think_decode_attn", "think_decode_attn_static", "think_decode_attn_partial",
           "think_decode_attn_combine",
           "think_append_kv", "think_append_decode_attn", "think_k2_state_bytes",
           "think_prefill_write_kv",
           "think_score_select_k2", "think_score_select_compact",
           "think_score_compact_workspace_bytes", "think_score_compact_single_read",
           "think_score_compact_status", "think_single_read_test_give_up", "think_probe_stream",
           "think_status_string", "think_last_hip_error")


class think_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_capacity", ctypes.c_int32), ("dtype", ctypes.c_int32)]

    def __repr__(self):
        return ("think_dims(B=%d, Hq=%d, Hkv=%d, D=%d, S_cap=%d, dtype=%d)" %
                (self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                 self.seq_capacity, self.dtype))


class ThinkError(RuntimeError):
    def __init__(self, fn, status, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn} returned {STATUS.get(status, status)}: {lib.think_status_string(status).decode()}"
        if status == -7:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


def _load():
    if not os.path.exists(_SO):
        raise ImportError(
            f"{_SO} is not built; build it with `python -m query_driven_kv_amd.build` "
            "(or __graft_entry__.build()). There is no fallback path.")
    l = ctypes.CDLL(_SO)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pd = ctypes.POINTER(think_dims)
    l.think_abi_version.restype = ctypes.c_int
    l.think_keep_from_ratio.argtypes = [i32, ctypes.c_double]
    l.think_keep_from_ratio.restype = i32
    l.think_score_workspace_bytes.argtypes = [pd]
    l.think_score_workspace_bytes.restype = sz
    l.think_decode_workspace_bytes.argtypes = [pd, i32]
    l.think_decode_workspace_bytes.restype = sz
    l.think_score.argtypes = [pd, vp, vp, vp, i32, vp, vp, sz, vp]
    l.think_score_select.argtypes = [pd, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    l.think_select.argtypes = [pd, vp, i32, vp, vp, vp]
    l.think_compact_k.argtypes = [pd, vp, vp, vp, i32, vp, vp]
    l.think_decode_attn.argtypes = [pd, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    l.think_decode_attn_static.argtypes = [pd, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp]
    l.think_decode_attn_partial.argtypes = [pd, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp, sz, vp]
    l.think_decode_attn_combine.argtypes = [pd, vp, i32, vp, vp, sz, vp]
    l.think_append_kv.argtypes = [pd, vp, vp, vp, vp, i32, vp, vp, vp]
    l.think_append_decode_attn.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp,
                                           vp, sz, vp]
    l.think_k2_state_bytes.argtypes = [pd]
    l.think_k2_state_bytes.restype = sz
    l.think_prefill_write_kv.argtypes = [pd, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    l.think_score_select_k2.argtypes = [pd, vp, sz, vp, i32, i32, vp, vp, vp, vp]
    l.think_score_select_compact.argtypes = [pd, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    l.think_score_compact_workspace_bytes.argtypes = [pd, i32]
    l.think_score_compact_workspace_bytes.restype = sz
    l.think_score_compact_single_read.argtypes = [pd, i32]
    l.think_score_compact_single_read.restype = ctypes.c_int
    l.think_score_compact_status.argtypes = [pd, i32, i32, vp, sz, vp]
    l.think_score_compact_status.restype = ctypes.c_int
    l.think_single_read_test_give_up.argtypes = [ctypes.c_int]
    l.think_single_read_test_give_up.restype = ctypes.c_int
    l.think_probe_stream.argtypes = [vp, sz, vp, sz, vp]
    l.think_probe_stream.restype = ctypes.c_int
    l.think_status_string.argtypes = [ctypes.c_int]
    l.think_status_string.restype = ctypes.c_char_p
    l.think_last_hip_error.restype = ctypes.c_int
    for name in ("think_score", "think_score_select", "think_select", "think_compact_k",
                 "think_decode_attn", "think_decode_attn_static",
                 "think_decode_attn_partial", "think_decode_attn_combine", "think_append_kv",
                 "think_append_decode_attn",
                 "think_prefill_write_kv", "think_score_select_k2", "think_score_select_compact"):
        getattr(l, name).restype = ctypes.c_int
    return l


lib = _load()
LIB_PATH = _SO


def check(fn_name, status):
    if status != 0:
        raise ThinkError(fn_name, status, lib.think_last_hip_error() if status == -7 else 0)

"""ctypes binding of libkvq (include/kvq.h), with the same names as the C ABI.

Argument marshalling only: every step of the path runs in the HIP library.
There is no CPU fallback -- if libkvq.so is missing, load() raises.

The C ABI, its layout and the citations of the pages it implements are
documented in include/kvq.h.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_CAPACITY, KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH = range(6)
KVQ_F16, KVQ_BF16 = 0, 1
KVQ_ROTATE_KEYS, KVQ_ROTATE_VALUES = 1, 2
KVQ_DEV_RESIDUAL_FULL, KVQ_DEV_BLOCKS_FULL, KVQ_DEV_BAD_PAGE, KVQ_DEV_BAD_COUNT, KVQ_DEV_TOO_LONG = 1, 2, 4, 8, 16

EXPORTED = ("kvq_layout_bytes", "kvq_workspace_size", "kvq_append", "kvq_append_flush", "kvq_flush_residual",
            "kvq_decode_attention", "kvq_decode_partials", "kvq_decode_combine", "kvq_get_device_error",
            "kvq_status_string", "kvq_decode_attention_multi", "kvq_workspace_size_multi",
            "kvq_decode_attention_noalloc")
KVQ_NOALLOC_WORKSPACE_BYTES = 64 << 20


class kvq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "k_bits", "v_bits", "k_group", "v_group",
        "residual", "res_capacity", "max_blocks", "num_pages", "dtype", "sink", "fp8_blocks", "rotate")]


class kvq_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("record", "blocks", "block_table", "ring", "state", "sink",
                                               "fp8_record", "fp8")]


class kvq_cache(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("k_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("k_sink", ctypes.c_void_p), ("v_sink", ctypes.c_void_p), ("fp8", ctypes.c_void_p)]


class KVQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def library_path_exists() -> bool:
    return os.path.exists(LIBRARY_PATH)


def load():
    """Load libkvq.so (built in-tree). Raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not library_path_exists():
        raise RuntimeError(f"libkvq.so is not built at {LIBRARY_PATH}; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIBRARY_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    cfgp, cachep = ctypes.POINTER(kvq_config), ctypes.POINTER(kvq_cache)
    sig = {
        "kvq_layout_bytes": [cfgp, ctypes.POINTER(kvq_layout)],
        "kvq_workspace_size": [cfgp, I32, ctypes.POINTER(SZ)],
        "kvq_append": [cfgp, cachep, P, P, P, I32, P],
        "kvq_append_flush": [cfgp, cachep, P, P, P, I32, P],
        "kvq_flush_residual": [cfgp, cachep, P],
        "kvq_decode_attention": [cfgp, cachep, P, P, F, I32, P, SZ, P],
        "kvq_decode_partials": [cfgp, cachep, P, F, I32, P, SZ, P],
        "kvq_decode_combine": [cfgp, cachep, P, I32, P, SZ, P],
        "kvq_get_device_error": [cfgp, cachep, P, ctypes.POINTER(I32)],
        "kvq_status_string": [ctypes.c_int],
        "kvq_decode_attention_multi": [cfgp, cachep, P, I32, P, F, I32, P, SZ, P],
        "kvq_workspace_size_multi": [cfgp, I32, I32, ctypes.POINTER(SZ)],
        "kvq_decode_attention_noalloc": [cfgp, cachep, P, P, F, I32, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "kvq_status_string" else ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kvq_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != KVQ_OK:
        raise KVQError(status, where)


# --- thin wrappers with the C names ---------------------------------------------------

def kvq_layout_bytes(cfg: kvq_config) -> kvq_layout:
    out = kvq_layout()
    _check(load().kvq_layout_bytes(ctypes.byref(cfg), ctypes.byref(out)), "kvq_layout_bytes")
    return out


def kvq_workspace_size(cfg: kvq_config, max_seq_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().kvq_workspace_size(ctypes.byref(cfg), int(max_seq_tokens), ctypes.byref(n)),
           "kvq_workspace_size")
    return n.value


def kvq_workspace_size_multi(cfg: kvq_config, max_seq_tokens: int, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().kvq_workspace_size_multi(ctypes.byref(cfg), int(max_seq_tokens), int(T), ctypes.byref(n)),
           "kvq_workspace_size_multi")
    return n.value


def kvq_append(cfg, cache, k_new_ptr, v_new_ptr, n_new_ptr, n_max, stream):
    _check(load().kvq_append(ctypes.byref(cfg), ctypes.byref(cache), k_new_ptr, v_new_ptr,
                             n_new_ptr, int(n_max), stream), "kvq_append")


def kvq_append_flush(cfg, cache, k_new_ptr, v_new_ptr, n_new_ptr, n_max, stream):
    _check(load().kvq_append_flush(ctypes.byref(cfg), ctypes.byref(cache), k_new_ptr, v_new_ptr,
                                   n_new_ptr, int(n_max), stream), "kvq_append_flush")


def kvq_flush_residual(cfg, cache, stream):
    _check(load().kvq_flush_residual(ctypes.byref(cfg), ctypes.byref(cache), stream), "kvq_flush_residual")


def kvq_decode_attention(cfg, cache, q_ptr, out_ptr, softmax_scale, max_seq_tokens, ws_ptr, ws_bytes, stream):
    _check(load().kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(cache), q_ptr, out_ptr,
                                       float(softmax_scale), int(max_seq_tokens), ws_ptr, int(ws_bytes),
                                       stream), "kvq_decode_attention")


def kvq_decode_attention_noalloc(cfg, cache, q_ptr, out_ptr, softmax_scale, max_seq_tokens, stream):
    _check(load().kvq_decode_attention_noalloc(ctypes.byref(cfg), ctypes.byref(cache), q_ptr, out_ptr,
                                               float(softmax_scale), int(max_seq_tokens), stream),
           "kvq_decode_attention_noalloc")


def kvq_decode_attention_multi(cfg, cache, q_ptr, T, out_ptr, softmax_scale, max_seq_tokens, ws_ptr, ws_bytes,
                               stream):
    _check(load().kvq_decode_attention_multi(ctypes.byref(cfg), ctypes.byref(cache), q_ptr, int(T), out_ptr,
                                             float(softmax_scale), int(max_seq_tokens), ws_ptr, int(ws_bytes),
                                             stream), "kvq_decode_attention_multi")


def kvq_decode_partials(cfg, cache, q_ptr, softmax_scale, max_seq_tokens, ws_ptr, ws_bytes, stream):
    _check(load().kvq_decode_partials(ctypes.byref(cfg), ctypes.byref(cache), q_ptr, float(softmax_scale),
                                      int(max_seq_tokens), ws_ptr, int(ws_bytes), stream), "kvq_decode_partials")


def kvq_decode_combine(cfg, cache, out_ptr, max_seq_tokens, ws_ptr, ws_bytes, stream):
    _check(load().kvq_decode_combine(ctypes.byref(cfg), ctypes.byref(cache), out_ptr, int(max_seq_tokens), ws_ptr,
                                     int(ws_bytes), stream), "kvq_decode_combine")


def kvq_get_device_error(cfg, cache, stream) -> int:
    err = ctypes.c_int32(0)
    _check(load().kvq_get_device_error(ctypes.byref(cfg), ctypes.byref(cache), stream, ctypes.byref(err)),
           "kvq_get_device_error")
    return err.value


def kvq_status_string(status: int) -> str:
    return status_string(status)

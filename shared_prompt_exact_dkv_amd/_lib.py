"""ctypes binding of libdkv (include/dkv.h): argument marshalling only.

Every step of the attention runs in libdkv's HIP kernels; torch supplies device
memory and the current stream.  Importing works without the library, but every
call raises if libdkv.so has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdkv.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dkv.h")

DKV_OK, DKV_ERR_INVALID_ARG, DKV_ERR_UNSUPPORTED, DKV_ERR_WORKSPACE, DKV_ERR_HIP = range(5)
DKV_BF16, DKV_FP32, DKV_FP16 = 0, 1, 2
DKV_CALL_CTX_FWD, DKV_CALL_FWD, DKV_CALL_CTX_BWD, DKV_CALL_BWD, DKV_CALL_BWD_SPLIT = range(5)
DKV_ACC_ZERO, DKV_ACC_FINALIZE, DKV_ACC_SPLIT = 1, 2, 4
(DKV_PACK, DKV_UNPACK, DKV_UNPACK_BWD, DKV_FIRST_TOKEN_GATHER,
 DKV_FIRST_TOKEN_SCATTER) = range(5)


class DkvParams(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("ctx_len", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_dev", ctypes.c_void_p),
        ("num_groups", ctypes.c_int32),
        ("ctx_cu_host", ctypes.POINTER(ctypes.c_int32)),
        ("group_seq_cu_host", ctypes.POINTER(ctypes.c_int32)),
        ("kv_head_of_q", ctypes.POINTER(ctypes.c_int32)),
    ]


class DkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("dkv status %d: %s" % (status, msg))
        self.status = status


_lib = None
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_pp = ctypes.POINTER(DkvParams)

_SIGS = {
    "dkv_workspace_size": (_sz, [_pp, ctypes.c_int]),
    "dkv_ctx_fwd": (ctypes.c_int, [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dkv_fwd": (ctypes.c_int, [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dkv_ctx_bwd": (ctypes.c_int, [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   ctypes.c_int, _vp, _sz, _vp]),
    "dkv_bwd": (ctypes.c_int, [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, ctypes.c_int, _vp, _vp, _vp, _sz, _vp]),
    "dkv_bwd_noalloc": (ctypes.c_int, [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp]),
    "dkv_cast_acc": (ctypes.c_int, [_pp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]),
    "dkv_layout_workspace_size": (_sz, [_pp, ctypes.c_int]),
    "dkv_layout": (ctypes.c_int, [_pp, ctypes.c_int, ctypes.c_int64, _vp, _vp, _vp, _sz, _vp]),
    "dkv_timing_enable": (None, [ctypes.c_int]),
    "dkv_timing_reset": (None, []),
    "dkv_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int), ctypes.c_int]),
    "dkv_last_error": (ctypes.c_char_p, []),
    "dkv_version": (ctypes.c_char_p, []),
}


def header_functions() -> list:
    """Names of the functions include/dkv.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dkv_[a-z_]+)\s*\(", txt)))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdkv.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().dkv_last_error().decode()


def check(status: int):
    if status != DKV_OK:
        raise DkvError(status, last_error())


def timing_read() -> dict:
    """{kernel class: (total ms, launches)} since the last reset (waits for events)."""
    n = 16
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    k = lib().dkv_timing_read(names, ms, cnt, n)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(k)}


def _i32(vals):
    if vals is None:
        return None, None
    arr = (ctypes.c_int32 * len(vals))(*[int(c) for c in vals])
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))


def make_params(*, num_seqs, ctx_len, num_heads_q, num_heads_kv, head_dim, window_left=-1,
                softmax_scale=0.0, dtype=DKV_BF16, cu_host=None, cu_dev=0, ctx_cu_host=None,
                group_seq_cu_host=None, kv_head_of_q=None):
    """Build a DkvParams.  Returns (params, keepalive); keep the second alive while the
    params are in use (it owns the host arrays: cu_seqlens, the prompt groups and the
    head map)."""
    arr, ptr = _i32(cu_host)
    carr, cptr = _i32(ctx_cu_host)
    garr, gptr = _i32(group_seq_cu_host)
    harr, hptr = _i32(kv_head_of_q)
    ng = 0
    if ctx_cu_host is not None or group_seq_cu_host is not None:
        if ctx_cu_host is None or group_seq_cu_host is None:
            raise ValueError("ctx_cu_host and group_seq_cu_host go together")
        ng = len(ctx_cu_host) - 1
    p = DkvParams(num_seqs, ctx_len, num_heads_q, num_heads_kv, head_dim, window_left,
                  float(softmax_scale), dtype, ptr, cu_dev, ng, cptr, gptr, hptr)
    return p, (arr, carr, garr, harr)

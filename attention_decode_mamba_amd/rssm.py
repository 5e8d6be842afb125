"""ctypes binding of ``librssm.so`` (include/rssm.h): argument marshalling only.

Every function has the C name and takes the same arguments; device pointers are
Python ints (``tensor.data_ptr()``), streams are raw ``hipStream_t`` handles
(``torch.cuda.current_stream().cuda_stream``) or 0.  Negative return codes raise
:class:`RssmError`.  There is no fallback: if the library is missing, loading it
raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "librssm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "rssm.h")

RSSM_OK = 0
RSSM_E_NULL = -1
RSSM_E_SHAPE = -2
RSSM_E_DTYPE = -3
RSSM_E_ALIGN = -4
RSSM_E_RANGE = -5
RSSM_E_HIP = -6
RSSM_E_DEVICE = -7

RSSM_DEVERR_VERIFY_CAPACITY = 1
RSSM_DEVERR_ACCEPT_RANGE = 2
RSSM_DEVERR_CURSOR = 4
RSSM_DEVERR_TREE = 8

RSSM_KIND_MAMBA2 = 0
RSSM_KIND_GDN = 1
RSSM_KIND_KDA = 2
RSSM_DTYPE_F32 = 0
RSSM_DTYPE_BF16 = 1
RSSM_READ_NONE = 0
RSSM_READ_FP8 = 1
RSSM_READ_MXFP4 = 2

_I32 = ctypes.c_int32
_VP = ctypes.c_void_p


class rssm_config(ctypes.Structure):
    _fields_ = [(n, _I32) for n in ("kind", "batch", "n_heads", "n_qk_heads", "dv", "dk", "L",
                                      "t_max", "capacity", "in_dtype", "read_copy")]


class rssm_state(ctypes.Structure):
    _fields_ = [("s_ckpt", _VP), ("s_read", _VP), ("s_read_scale", _VP), ("ring", _VP),
                ("n_committed", _VP), ("n_ckpt", _VP), ("err", _VP)]


class rssm_buffer_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("s_ckpt", "s_read", "s_read_scale", "ring",
                                                 "n_committed", "n_ckpt", "err")]


class RssmError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {rssm_strerror(code)} ({code})")
        self.code = code


_lib: Optional[ctypes.CDLL] = None

_SIGS = {
    "rssm_check_config": (_I32, [ctypes.POINTER(rssm_config)]),
    "rssm_sizes": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_buffer_sizes)]),
    "rssm_ring_offsets": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(ctypes.c_int64)]),
    "rssm_init_state": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state), _VP, _VP]),
    "rssm_decode_step": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state),
                                _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "rssm_flush": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state), _I32, _VP]),
    "rssm_verify": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state), _I32,
                           _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "rssm_commit": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state), _VP, _I32, _VP]),
    "rssm_decode_step_conventional": (_I32, [ctypes.POINTER(rssm_config), _VP, _VP, _VP, _VP,
                                             _VP, _VP, _VP, _VP]),
    "rssm_verify_tree": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state), _I32, _VP,
                                _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "rssm_verify_fold": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state), _I32, _I32, _VP,
                                _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "rssm_commit_tree": (_I32, [ctypes.POINTER(rssm_config), ctypes.POINTER(rssm_state), _VP, _VP, _VP, _I32,
                                _VP]),
    "rssm_verify_snapshot": (_I32, [ctypes.POINTER(rssm_config), _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP,
                                    _VP, _VP, _VP]),
    "rssm_commit_snapshot": (_I32, [ctypes.POINTER(rssm_config), _VP, _VP, _I32, _VP, _VP]),
    "rssm_get_error": (_I32, [ctypes.POINTER(rssm_state), _VP]),
    "rssm_stream_copy": (_I32, [_VP, _VP, ctypes.c_size_t, _VP]),
    "rssm_strerror": (ctypes.c_char_p, [_I32]),
    "rssm_version": (_I32, []),
}


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m attention_decode_mamba_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_symbols() -> list:
    """Function names declared in include/rssm.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rssm_[a-z_]+)\s*\(", text)))


def _ck(code: int, what: str) -> int:
    if code < 0:
        raise RssmError(code, what)
    return code


def _p(x) -> Optional[int]:
    if x is None:
        return None
    return int(x)


def rssm_strerror(code: int) -> str:
    return lib().rssm_strerror(code).decode()


def rssm_version() -> int:
    return lib().rssm_version()


def rssm_check_config(cfg: rssm_config) -> int:
    return _ck(lib().rssm_check_config(ctypes.byref(cfg)), "rssm_check_config")


def rssm_sizes(cfg: rssm_config) -> rssm_buffer_sizes:
    out = rssm_buffer_sizes()
    _ck(lib().rssm_sizes(ctypes.byref(cfg), ctypes.byref(out)), "rssm_sizes")
    return out


def rssm_ring_offsets(cfg: rssm_config) -> list:
    out = (ctypes.c_int64 * 5)()
    _ck(lib().rssm_ring_offsets(ctypes.byref(cfg), out), "rssm_ring_offsets")
    return list(out)


def rssm_init_state(cfg, st, s0, stream=0) -> int:
    return _ck(lib().rssm_init_state(ctypes.byref(cfg), ctypes.byref(st), _p(s0), _p(stream)),
               "rssm_init_state")


def rssm_decode_step(cfg, st, alpha, beta, v, k, q, y, stream=0) -> int:
    return _ck(lib().rssm_decode_step(ctypes.byref(cfg), ctypes.byref(st), _p(alpha), _p(beta),
                                      _p(v), _p(k), _p(q), _p(y), _p(stream)), "rssm_decode_step")


def rssm_flush(cfg, st, min_records: int, stream=0) -> int:
    return _ck(lib().rssm_flush(ctypes.byref(cfg), ctypes.byref(st), min_records, _p(stream)),
               "rssm_flush")


def rssm_verify(cfg, st, T: int, alpha, beta, v, k, q, o, stream=0) -> int:
    return _ck(lib().rssm_verify(ctypes.byref(cfg), ctypes.byref(st), T, _p(alpha), _p(beta),
                                 _p(v), _p(k), _p(q), _p(o), _p(stream)), "rssm_verify")


def rssm_commit(cfg, st, n_accept, T: int, stream=0) -> int:
    return _ck(lib().rssm_commit(ctypes.byref(cfg), ctypes.byref(st), _p(n_accept), T, _p(stream)),
               "rssm_commit")


def rssm_decode_step_conventional(cfg, s, alpha, beta, v, k, q, y, stream=0) -> int:
    return _ck(lib().rssm_decode_step_conventional(ctypes.byref(cfg), _p(s), _p(alpha), _p(beta),
                                                   _p(v), _p(k), _p(q), _p(y), _p(stream)),
               "rssm_decode_step_conventional")


def rssm_verify_tree(cfg, st, T: int, parent, alpha, beta, v, k, q, o, stream=0) -> int:
    return _ck(lib().rssm_verify_tree(ctypes.byref(cfg), ctypes.byref(st), T, _p(parent), _p(alpha), _p(beta),
                                      _p(v), _p(k), _p(q), _p(o), _p(stream)), "rssm_verify_tree")


def rssm_verify_fold(cfg, st, min_records: int, T: int, parent, alpha, beta, v, k, q, o, stream=0) -> int:
    return _ck(lib().rssm_verify_fold(ctypes.byref(cfg), ctypes.byref(st), min_records, T, _p(parent), _p(alpha),
                                      _p(beta), _p(v), _p(k), _p(q), _p(o), _p(stream)), "rssm_verify_fold")


def rssm_commit_tree(cfg, st, parent, path, n_accept, T: int, stream=0) -> int:
    return _ck(lib().rssm_commit_tree(ctypes.byref(cfg), ctypes.byref(st), _p(parent), _p(path), _p(n_accept), T,
                                      _p(stream)), "rssm_commit_tree")


def rssm_verify_snapshot(cfg, snap, cur, T: int, alpha, beta, v, k, q, o, err, stream=0) -> int:
    return _ck(lib().rssm_verify_snapshot(ctypes.byref(cfg), _p(snap), _p(cur), T, _p(alpha), _p(beta), _p(v),
                                          _p(k), _p(q), _p(o), _p(err), _p(stream)), "rssm_verify_snapshot")


def rssm_commit_snapshot(cfg, cur, n_accept, T: int, err, stream=0) -> int:
    return _ck(lib().rssm_commit_snapshot(ctypes.byref(cfg), _p(cur), _p(n_accept), T, _p(err), _p(stream)),
               "rssm_commit_snapshot")


def rssm_get_error(st, stream=0) -> int:
    return _ck(lib().rssm_get_error(ctypes.byref(st), _p(stream)), "rssm_get_error")


def rssm_stream_copy(src, dst, nbytes: int, stream=0) -> int:
    return _ck(lib().rssm_stream_copy(_p(src), _p(dst), nbytes, _p(stream)), "rssm_stream_copy")

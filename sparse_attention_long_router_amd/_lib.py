"""ctypes binding of libmoga.so (declared in include/moga.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
There is no fallback: if the library is missing, importing this module fails.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoga.so")

MOGA_OP_ROUTE = 0
MOGA_OP_PERMUTE = 1
MOGA_OP_GROUP_ATTENTION = 2
MOGA_OP_UNPERMUTE = 3
MOGA_OP_STGA_ATTENTION = 4
MOGA_OP_BALANCE_STATS = 5
MOGA_OP_ROUTE_BACKWARD = 6
MOGA_OP_ATTENTION_BACKWARD = 7

# every symbol include/moga.h declares, with its ctypes signature
_c = ctypes
_vp, _i32, _i64, _f32, _sz = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_float, _c.c_size_t
SIGNATURES = {
    "moga_route": (_c.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moga_permute": (_c.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _sz, _vp]),
    "moga_group_attention": (_c.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _sz, _vp]),
    "moga_group_attention_unpermute": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _f32,
                                                   _f32, _vp, _vp, _sz, _vp]),
    "moga_permute_vt": (_c.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
    "moga_permute_vt_noalloc": (_c.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp]),
    "moga_group_attention_unpermute_vt": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _f32,
                                                      _f32, _vp, _vp, _sz, _vp]),
    "moga_group_attention_unpermute_vtq": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _f32,
                                                       _f32, _vp, _vp, _sz, _vp]),
    "moga_group_attention_fused": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _f32, _f32,
                                              _vp, _vp, _sz, _vp]),
    "moga_unpermute": (_c.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _f32, _vp, _vp]),
    "moga_stga_attention": (_c.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                       _f32, _f32, _vp, _vp, _sz, _vp]),
    "moga_stga_shot_attention": (_c.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f32, _f32, _f32, _vp, _vp, _sz, _vp]),
    "moga_stga_shot_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moga_balance_stats": (_c.c_int, [_vp, _vp, _i64, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moga_group_attention_train": (_c.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _sz,
                                              _vp]),
    "moga_unpermute_backward": (_c.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moga_group_attention_backward": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                                 _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moga_attention_backward_staged_bytes": (_sz, [_vp, _i32, _i32]),
    "moga_route_backward": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moga_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32]),
    "moga_strerror": (_c.c_char_p, [_i32]),
    "moga_version": (_i32, []),
}


BUILD_HINT = "run `python sparse_attention_long_router_amd/build.py`"
# moga_version() of the sources this binding matches (csrc/api.hip)
EXPECTED_VERSION = 410


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; {BUILD_HINT}")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        try:
            fn = getattr(lib, name)
        except AttributeError:
            raise ImportError(f"{LIB_PATH} lacks {name} (stale build); {BUILD_HINT}") from None
        fn.restype = res
        fn.argtypes = args
    got = int(lib.moga_version())
    if got != EXPECTED_VERSION:
        raise ImportError(f"{LIB_PATH} is version {got}, the binding expects {EXPECTED_VERSION} (stale build); "
                          f"{BUILD_HINT}")
    return lib


LIB = _load()


class MogaError(RuntimeError):
    pass


def check(status: int, what: str):
    if status != 0:
        raise MogaError(f"{what}: {LIB.moga_strerror(status).decode()} (status {status})")


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(op: int, N: int, M: int, H: int = 1, D: int = 64) -> int:
    return int(LIB.moga_workspace_bytes(op, N, M, H, D))


def version() -> int:
    return int(LIB.moga_version())

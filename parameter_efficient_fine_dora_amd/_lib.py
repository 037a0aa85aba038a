"""ctypes view of libdora.so (include/dora.h).  No torch here: loading and the
host-only entry points work without a GPU."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdora.so")

F32, BF16 = 0, 1
FLAG_EXACT_NORM_GRAD = 1 << 0
FLAG_SEPARATE_COMPOSE = 1 << 1
OP_NORM, OP_FORWARD, OP_BACKWARD, OP_MERGE, OP_VERA_GRADS = 0, 1, 2, 3, 4
ERR = {0: "DORA_OK", -1: "DORA_ERR_NULL", -2: "DORA_ERR_SHAPE", -3: "DORA_ERR_DTYPE",
       -4: "DORA_ERR_ALIGN", -5: "DORA_ERR_WORKSPACE", -6: "DORA_ERR_HIP", -7: "DORA_ERR_FLAGS"}
ERR_CODE = {v: k for k, v in ERR.items()}
NOALLOC_SCRATCH_BYTES = 64 << 20   # DORA_NOALLOC_SCRATCH_BYTES


class DoraShape(ctypes.Structure):
    _fields_ = [
        ("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64), ("r", ctypes.c_int64),
        ("tokens", ctypes.c_int64), ("dtype", ctypes.c_int32), ("s", ctypes.c_float),
        ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
    ]


class DoraError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {ERR.get(code, code)} ({strerror(code)})")


_lib = None
_vp, _sz, _i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_SIGS = {
    "dora_workspace_bytes": (_sz, [ctypes.POINTER(DoraShape), _i]),
    "dora_norm": (_i, [ctypes.POINTER(DoraShape), _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dora_forward": (_i, [ctypes.POINTER(DoraShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _vp, _sz, _vp]),
    "dora_forward_noalloc": (_i, [ctypes.POINTER(DoraShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp]),
    "dora_backward": (_i, [ctypes.POINTER(DoraShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dora_merge": (_i, [ctypes.POINTER(DoraShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dora_vera_scale": (_i, [ctypes.POINTER(DoraShape), _vp, _vp, _vp, _vp, _vp]),
    "dora_vera_grads": (_i, [ctypes.POINTER(DoraShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dora_strerror": (ctypes.c_char_p, [_i]),
    "dora_timing_enable": (_i, [_i]),
    "dora_timing_collect": (_i, [ctypes.c_char_p, _sz]),
    "dora_probe_mfma": (_i, [ctypes.c_int64, _i, _vp, _vp]),
    "dora_probe_mfma_flops": (ctypes.c_double, [ctypes.c_int64, _i]),
    "dora_probe_stream": (_i, [_vp, _vp, _vp, ctypes.c_int64, _vp]),
}


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m parameter_efficient_fine_dora_amd.build` "
                "(the DoRA ops run only in the HIP library)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().dora_strerror(int(code)).decode()


def shape(d_out, d_in, r, tokens, dtype, s, flags=0) -> DoraShape:
    return DoraShape(int(d_out), int(d_in), int(r), int(tokens), int(dtype), float(s), int(flags), 0)


def workspace_bytes(sh: DoraShape, op: int) -> int:
    return int(lib().dora_workspace_bytes(ctypes.byref(sh), int(op)))

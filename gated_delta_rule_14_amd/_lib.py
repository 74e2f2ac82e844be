"""ctypes loader for libkda.so (the HIP kernels behind the C ABI in include/kda.h).

The library is built in-tree by gated_delta_rule_14_amd/build.py.  There is
no fallback of any kind: if the shared object is missing, every call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK = 0
KDA_F32, KDA_BF16 = 0, 1

# Every symbol include/kda.h declares, with (restype, argtypes).
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "kda_status_str": (ctypes.c_char_p, [_i]),
    "kda_version": (ctypes.c_char_p, []),
    "kda_chunk_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_chunk_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp,
                           _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_chunk_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp,
                                   _i, _i, _i, _i, _i, _i, _i, _vp]),
    "kda_recurrent_step": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                _i, _i, _i, _i, _i, _vp]),
    "kda_out_gate_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_out_gate": (_i, [_vp, _vp, _f, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_gdn_chunk_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_gdn_chunk_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp,
                               _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_gdn_recurrent_step": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                    _i, _i, _i, _i, _i, _vp]),
    "kda_recurrent_layer_step_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "kda_recurrent_layer_step": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _f, _vp, _vp, _vp,
                                      _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_chunk_layer_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "kda_recurrent_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "kda_recurrent_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_stream_scale": (_i, [_vp, _sz, _f, _i, _vp]),
    "kda_chunk_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_chunk_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_dplr_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp,
                          _i, _i, _i, _i, _i, _i, _vp]),
    "kda_dplr_recurrent_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                     _i, _i, _i, _i, _i, _vp]),
    "kda_dplr_chunk_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_dplr_chunk_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp,
                                _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_chunk_layer_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _f, _vp, _vp, _vp, _vp,
                                 _i, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
}

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg}")
        self.status = status


def lib():
    """The loaded libkda.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libkda.so is not built ({LIB_PATH} missing): run `python -c "
            f"'import __graft_entry__ as g; g.build()'` from the repository root")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    _lib = handle
    return handle


def check(fn_name, status):
    if status != KDA_OK:
        msg = lib().kda_status_str(status).decode()
        raise KdaError(fn_name, status, msg)

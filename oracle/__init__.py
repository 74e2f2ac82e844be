"""fp64 CPU oracle for the Kimi Delta Attention (KDA) operator.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path (the HIP library and
its binding) never does, and this package never imports the product.

Two independent formulations live here:

* ``forward`` / ``out_gate`` -- ctypes front end of ``kdaref.c``: the
  token-by-token recurrence of Eq. 1 of the Kimi Linear tech report
  (section 3), read from the updated state, with the decay
  alpha = exp(g_min * sigmoid(z)) and the RMSNorm x sigmoid-gate epilogue and
  projection of the "KDA Recurrence" problem statement.  fp64 throughout.
* ``chunked.forward`` -- numpy fp64 evaluation of the chunk form of the tech
  report's appendix B (Propositions 1 and 2, Eqs. 16-19), used to pin the
  algebra that the chunkwise GPU path relies on.

Arrays: numpy float64, float32, or uint16 holding bfloat16 bit patterns.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

F64, F32, BF16 = 0, 1, 2


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.kdaref_forward.argtypes = [vp, vp, vp, vp, vp, i, d, vp, i, vp, vp,
                                   i, i, i, i, i, i]
    lib.kdaref_forward.restype = i
    lib.kdaref_out_gate.argtypes = [vp, i, vp, i, d, vp, i, vp,
                                    i, i, i, i, i, i]
    lib.kdaref_out_gate.restype = i
    _lib = lib
    return lib


def _code(a):
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle: unsupported dtype {a.dtype}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def forward(q, k, v, z, beta, g_min, s0=None, want_o=True, nthreads=None):
    """Sequential KDA recurrence in fp64.

    q, k, z: (B, T, H, dk); v: (B, T, H, dv); beta: (B, T, H), all one dtype.
    s0: (B, H, dk, dv) float64/float32 or None (zeros).
    Returns (o, s_final) as float64 arrays; o is None when want_o is False.
    """
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, z, beta)]
    q, k, v, z, beta = arrs
    dt = _code(q)
    for x in arrs:
        if _code(x) != dt:
            raise TypeError("oracle: q, k, v, z, beta must share one dtype")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and z.shape == (B, T, H, dk)
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if s0 is not None:
        s0 = np.ascontiguousarray(s0)
        assert s0.shape == (B, H, dk, dv)
        dts0 = _code(s0)
        if dts0 == BF16:
            raise TypeError("oracle: s0 must be float64 or float32")
    o = np.empty((B, T, H, dv), np.float64) if want_o else None
    s_fin = np.empty((B, H, dk, dv), np.float64)
    rc = _load().kdaref_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), dt, float(g_min),
        _ptr(s0) if s0 is not None else None, dts0 if s0 is not None else F64,
        _ptr(o) if o is not None else None, _ptr(s_fin),
        B, T, H, dk, dv, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kdaref_forward failed with code {rc}")
    return o, s_fin


def out_gate(o, gate, eps, w=None, nthreads=None):
    """RMSNorm over each head's dv values x sigmoid(gate), concat, then y W^T.

    o, gate: (B, T, H, dv); w: (d_model, H*dv) or None.
    Returns float64 (B, T, d_model), or (B, T, H*dv) when w is None.
    """
    o = np.ascontiguousarray(o)
    gate = np.ascontiguousarray(gate)
    B, T, H, dv = o.shape
    assert gate.shape == o.shape
    if w is not None:
        w = np.ascontiguousarray(w)
        d_model = w.shape[0]
        assert w.shape == (d_model, H * dv)
        out = np.empty((B, T, d_model), np.float64)
    else:
        d_model = 0
        out = np.empty((B, T, H * dv), np.float64)
    rc = _load().kdaref_out_gate(
        _ptr(o), _code(o), _ptr(gate), _code(gate), float(eps),
        _ptr(w) if w is not None else None, _code(w) if w is not None else F64,
        _ptr(out), B, T, H, dv, d_model, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kdaref_out_gate failed with code {rc}")
    return out


def layer(q, k, v, z, beta, gate, w, s0, g_min, eps, nthreads=None):
    """The full layer of the "KDA Recurrence" problem: recurrence, then the
    epilogue and projection.  Returns {"outputs", "final_state"} in fp64."""
    o, s = forward(q, k, v, z, beta, g_min, s0, nthreads=nthreads)
    out = out_gate(o, gate, eps, w, nthreads=nthreads)
    return {"outputs": out, "final_state": s}


def bf16_to_f64(a):
    """Exact widening of uint16 bfloat16 bit patterns to float64."""
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(a):
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

"""Python front end of libkda: argument marshalling only.

Every step of the operator runs in the HIP kernels of libkda.so; torch is
used for device memory (outputs, workspaces) and for the current HIP stream.
Names follow the C ABI in include/kda.h:

  chunk_fwd       -> kda_chunk_fwd        chunkwise prefill
  chunk_fwd_noalloc -> kda_chunk_fwd_noalloc  the same without a workspace,
                     on the library's static scratch array (no allocation)
  recurrent_step  -> kda_recurrent_step   one decode token, state in place
  out_gate        -> kda_out_gate         RMSNorm x sigmoid gate (+ projection)
  gdn_chunk_fwd   -> kda_gdn_chunk_fwd       scalar-gate prefill, z (B,T,H)
  gdn_recurrent_step -> kda_gdn_recurrent_step scalar-gate decode, z (B,H)
  recurrent_layer_step -> kda_recurrent_layer_step: one decode token of the
                     whole layer (step + RMSNorm x gate in one launch,
                     then the projection)
  chunk_layer_fwd -> kda_chunk_layer_fwd: the prefill of the whole layer
                     (chunkwise recurrence with RMSNorm x gate in its
                     kernels, then the projection)
  recurrent_bwd   -> kda_recurrent_bwd: gradients of the recurrence with
                     respect to q, k, v, z, beta and s0 (fp32)
  chunk_bwd       -> kda_chunk_bwd: the same gradients by 64-token chunks
                     on MFMA
  dplr_fwd        -> kda_dplr_fwd: the general diagonal-plus-low-rank
                     recurrence S = (Diag(alpha) - a b^T) S + k v^T over a
                     sequence (token-sequential)
  dplr_recurrent_step -> kda_dplr_recurrent_step: one DPLR token, state
                     in place
  dplr_chunk_fwd  -> kda_dplr_chunk_fwd: the DPLR recurrence by 64-token
                     chunks (decayed products per 16-token block pair)
  layer           -> kda_chunk_layer_fwd, returning the
                     {"outputs", "final_state"} dictionary of the
                     "KDA Recurrence" problem (final_state kept in fp32)
"""
import ctypes

import torch

from ._lib import KDA_BF16, KDA_F32, check, lib

CHUNK = 64


def _dt(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"libkda: unsupported dtype {t.dtype} (bf16 or fp32)")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"libkda: {name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"libkda: {name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"libkda: {name} must be contiguous")


def chunk_fwd_workspace_bytes(B, T, H, dk, dv, dtype):
    return int(lib().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, CHUNK,
                                                   KDA_BF16 if dtype == torch.bfloat16 else KDA_F32))


def chunk_fwd(q, k, v, z, beta, g_min, s0=None, *, o=None, s_final=None, workspace=None,
              want_state=True):
    """Chunkwise prefill. q, k, z: (B,T,H,dk); v: (B,T,H,dv); beta: (B,T,H);
    s0: (B,H,dk,dv) fp32 or None.  Returns (o, s_final); s_final is fp32 and
    None when want_state is False.  s_final may be passed as s0 (in place)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if s0 is not None:
        _need(s0, "s0", dev)
        if s0.dtype != torch.float32:
            raise TypeError("libkda: s0 must be float32")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if want_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_state:
        s_final = None
    need = lib().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, CHUNK, _dt(q))
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=dev)
    check("kda_chunk_fwd", lib().kda_chunk_fwd(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(s0), _p(o), _p(s_final),
        B, T, H, dk, dv, CHUNK, _dt(q), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev)))
    return o, s_final


NOALLOC_SCRATCH_BYTES = 192 << 20


def chunk_fwd_noalloc(q, k, v, z, beta, g_min, s0=None, *, o=None, s_final=None, want_state=True):
    """chunk_fwd on the library's static scratch array (kda_chunk_fwd_noalloc):
    no workspace is passed and the library allocates nothing.  Calls on one
    GPU share that array and must not overlap."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if s0 is not None:
        _need(s0, "s0", dev)
        if s0.dtype != torch.float32:
            raise TypeError("libkda: s0 must be float32")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if want_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_state:
        s_final = None
    check("kda_chunk_fwd_noalloc", lib().kda_chunk_fwd_noalloc(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(s0), _p(o), _p(s_final),
        B, T, H, dk, dv, CHUNK, _dt(q), _stream(dev)))
    return o, s_final


def recurrent_step(q, k, v, z, beta, g_min, state, *, o=None):
    """One decode token. q, k, z: (B,H,dk); v: (B,H,dv); beta: (B,H);
    state: (B,H,dk,dv) fp32, updated in place.  Returns o (B,H,dv)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta), ("state", state)):
        _need(t, name, dev)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if state.dtype != torch.float32:
        raise TypeError("libkda: state must be float32")
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    check("kda_recurrent_step", lib().kda_recurrent_step(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(state), _p(o),
        B, H, dk, dv, _dt(q), _stream(dev)))
    return o


def gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, dtype):
    return int(lib().kda_gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, CHUNK,
                                                       KDA_BF16 if dtype == torch.bfloat16 else KDA_F32))


def gdn_chunk_fwd(q, k, v, z, beta, g_min, s0=None, *, o=None, s_final=None, workspace=None, want_state=True):
    """Scalar-gate (Gated DeltaNet) prefill: as chunk_fwd, but z is (B,T,H),
    one decay logit per token and head."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(z.shape) != (B, T, H):
        raise ValueError(f"libkda: scalar-gate z must be (B, T, H) = {(B, T, H)}, got {tuple(z.shape)}")
    if s0 is not None:
        _need(s0, "s0", dev)
        if s0.dtype != torch.float32:
            raise TypeError("libkda: s0 must be float32")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if want_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_state:
        s_final = None
    need = lib().kda_gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, CHUNK, _dt(q))
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=dev)
    check("kda_gdn_chunk_fwd", lib().kda_gdn_chunk_fwd(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(s0), _p(o), _p(s_final),
        B, T, H, dk, dv, CHUNK, _dt(q), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev)))
    return o, s_final


def gdn_recurrent_step(q, k, v, z, beta, g_min, state, *, o=None):
    """Scalar-gate (Gated DeltaNet) decode token: as recurrent_step, but z is
    (B,H)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta), ("state", state)):
        _need(t, name, dev)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(z.shape) != (B, H):
        raise ValueError(f"libkda: scalar-gate z must be (B, H) = {(B, H)}, got {tuple(z.shape)}")
    if state.dtype != torch.float32:
        raise TypeError("libkda: state must be float32")
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    check("kda_gdn_recurrent_step", lib().kda_gdn_recurrent_step(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(state), _p(o),
        B, H, dk, dv, _dt(q), _stream(dev)))
    return o


def out_gate_workspace_bytes(B, T, H, dv, d_model, dtype, with_projection):
    return int(lib().kda_out_gate_workspace_bytes(B, T, H, dv, d_model,
                                                  KDA_BF16 if dtype == torch.bfloat16 else KDA_F32,
                                                  int(bool(with_projection))))


def out_gate(o, gate, eps, w=None, *, y=None, workspace=None):
    """RMSNorm over each head's dv values x sigmoid(gate), heads concatenated;
    projected by w (d_model, H*dv) when given.  o, gate: (B,T,H,dv)."""
    dev = o.device
    _need(o, "o", dev)
    _need(gate, "gate", dev)
    B, T, H, dv = o.shape
    d_model = 0
    if w is not None:
        _need(w, "w", dev)
        d_model = w.shape[0]
        if w.dtype != torch.bfloat16:
            raise TypeError("libkda: projection w must be bfloat16")
    if y is None:
        width = d_model if w is not None else H * dv
        y = torch.empty((B, T, width), dtype=o.dtype, device=dev)
    need = lib().kda_out_gate_workspace_bytes(B, T, H, dv, d_model, _dt(o), int(w is not None))
    if workspace is None and need > 0:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("kda_out_gate", lib().kda_out_gate(
        _p(o), _p(gate), float(eps), _p(w), _p(y), B, T, H, dv, d_model, _dt(o),
        _p(workspace), ws_bytes, _stream(dev)))
    return y


def recurrent_layer_step_workspace_bytes(B, H, dv, d_model, dtype, with_projection):
    return int(lib().kda_recurrent_layer_step_workspace_bytes(
        B, H, dv, d_model, KDA_BF16 if dtype == torch.bfloat16 else KDA_F32, int(bool(with_projection))))


def recurrent_layer_step(q, k, v, z, beta, g_min, state, gate, eps, w=None, *, y=None, o=None,
                         want_o=False, workspace=None):
    """One decode token of the layer. q, k, z: (B,H,dk); v, gate: (B,H,dv);
    beta: (B,H); state: (B,H,dk,dv) fp32, updated in place; w: (d_model, H*dv)
    bf16 or None.  Returns y ((B, d_model) with w, else (B, H*dv)), or
    (y, o) when want_o (o: the raw read-out, (B,H,dv))."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta), ("state", state), ("gate", gate)):
        _need(t, name, dev)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if state.dtype != torch.float32:
        raise TypeError("libkda: state must be float32")
    d_model = 0
    if w is not None:
        _need(w, "w", dev)
        d_model = w.shape[0]
        if w.dtype != torch.bfloat16:
            raise TypeError("libkda: projection w must be bfloat16")
    if y is None:
        y = torch.empty((B, d_model if w is not None else H * dv), dtype=q.dtype, device=dev)
    if want_o and o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    need = lib().kda_recurrent_layer_step_workspace_bytes(B, H, dv, d_model, _dt(q), int(w is not None))
    if workspace is None and need > 0:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("kda_recurrent_layer_step", lib().kda_recurrent_layer_step(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(state), _p(gate), float(eps), _p(w),
        _p(o), _p(y), B, H, dk, dv, d_model, _dt(q), _p(workspace), ws_bytes, _stream(dev)))
    return (y, o) if want_o else y


def chunk_layer_fwd_workspace_bytes(B, T, H, dk, dv, d_model, dtype, with_projection):
    return int(lib().kda_chunk_layer_fwd_workspace_bytes(
        B, T, H, dk, dv, CHUNK, d_model, KDA_BF16 if dtype == torch.bfloat16 else KDA_F32,
        int(bool(with_projection))))


def chunk_layer_fwd(q, k, v, z, beta, g_min, gate, eps, w=None, s0=None, *, y=None, o=None,
                    want_o=False, s_final=None, want_state=True, workspace=None):
    """Prefill of the layer. q, k, z: (B,T,H,dk); v, gate: (B,T,H,dv);
    beta: (B,T,H); s0: (B,H,dk,dv) fp32 or None; w: (d_model, H*dv) bf16 or
    None.  Returns (y, s_final): y is (B,T,d_model) with w, else (B,T,H*dv);
    s_final is fp32, or None when want_state is False.  With want_o, returns
    (y, s_final, o) with o the raw outputs (B,T,H,dv)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta), ("gate", gate)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if s0 is not None:
        _need(s0, "s0", dev)
        if s0.dtype != torch.float32:
            raise TypeError("libkda: s0 must be float32")
    d_model = 0
    if w is not None:
        _need(w, "w", dev)
        d_model = w.shape[0]
        if w.dtype != torch.bfloat16:
            raise TypeError("libkda: projection w must be bfloat16")
    if y is None:
        y = torch.empty((B, T, d_model if w is not None else H * dv), dtype=q.dtype, device=dev)
    if want_o and o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if want_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_state:
        s_final = None
    need = lib().kda_chunk_layer_fwd_workspace_bytes(B, T, H, dk, dv, CHUNK, d_model, _dt(q),
                                                     int(w is not None))
    if workspace is None and need > 0:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("kda_chunk_layer_fwd", lib().kda_chunk_layer_fwd(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(s0), _p(gate), float(eps), _p(w),
        _p(o), _p(y), _p(s_final), B, T, H, dk, dv, CHUNK, d_model, _dt(q), _p(workspace), ws_bytes,
        _stream(dev)))
    return (y, s_final, o) if want_o else (y, s_final)


def recurrent_bwd_workspace_bytes(B, T, H, dk, dv):
    return int(lib().kda_recurrent_bwd_workspace_bytes(B, T, H, dk, dv))


def recurrent_bwd(q, k, v, z, beta, g_min, s0, grad_o, grad_s_final=None, *, want_s0=True, workspace=None):
    """Gradients of the recurrence (the backward of chunk_fwd). Inputs as for
    chunk_fwd; grad_o: (B,T,H,dv) in the token dtype; grad_s_final:
    (B,H,dk,dv) fp32 or None.  Returns a dict of fp32 tensors dq, dk, dv, dz,
    dbeta and ds0 (None when want_s0 is False)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta), ("grad_o", grad_o)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    for name, t in (("s0", s0), ("grad_s_final", grad_s_final)):
        if t is not None:
            _need(t, name, dev)
            if t.dtype != torch.float32:
                raise TypeError(f"libkda: {name} must be float32")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
           "dv": torch.empty((B, T, H, dv), **f32), "dz": torch.empty((B, T, H, dk), **f32),
           "dbeta": torch.empty((B, T, H), **f32),
           "ds0": torch.empty((B, H, dk, dv), **f32) if want_s0 else None}
    need = lib().kda_recurrent_bwd_workspace_bytes(B, T, H, dk, dv)
    if workspace is None and need > 0:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("kda_recurrent_bwd", lib().kda_recurrent_bwd(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(s0), _p(grad_o), _p(grad_s_final),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dz"]), _p(out["dbeta"]), _p(out["ds0"]),
        B, T, H, dk, dv, _dt(q), _p(workspace), ws_bytes, _stream(dev)))
    return out


def chunk_bwd_workspace_bytes(B, T, H, dk, dv, dtype):
    return int(lib().kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, CHUNK,
                                                   KDA_BF16 if dtype == torch.bfloat16 else KDA_F32))


def chunk_bwd(q, k, v, z, beta, g_min, s0, grad_o, grad_s_final=None, *, want_s0=True, workspace=None):
    """Chunkwise gradients (kda_chunk_bwd); arguments and results as
    recurrent_bwd."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta), ("grad_o", grad_o)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    for name, t in (("s0", s0), ("grad_s_final", grad_s_final)):
        if t is not None:
            _need(t, name, dev)
            if t.dtype != torch.float32:
                raise TypeError(f"libkda: {name} must be float32")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
           "dv": torch.empty((B, T, H, dv), **f32), "dz": torch.empty((B, T, H, dk), **f32),
           "dbeta": torch.empty((B, T, H), **f32),
           "ds0": torch.empty((B, H, dk, dv), **f32) if want_s0 else None}
    need = lib().kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, CHUNK, _dt(q))
    if workspace is None and need > 0:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("kda_chunk_bwd", lib().kda_chunk_bwd(
        _p(q), _p(k), _p(v), _p(z), _p(beta), float(g_min), _p(s0), _p(grad_o), _p(grad_s_final),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dz"]), _p(out["dbeta"]), _p(out["ds0"]),
        B, T, H, dk, dv, CHUNK, _dt(q), _p(workspace), ws_bytes, _stream(dev)))
    return out


def dplr_fwd(q, k, v, z, a, b, g_min, s0=None, *, o=None, s_final=None, want_state=True):
    """DPLR recurrence over a sequence. q, k, z, a, b: (B,T,H,dk); v: (B,T,H,dv);
    s0: (B,H,dk,dv) fp32 or None.  Returns (o, s_final), s_final fp32 (None
    when want_state is False)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("a", a), ("b", b)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("k", k), ("z", z), ("a", a), ("b", b)):
        if tuple(t.shape) != (B, T, H, dk):
            raise ValueError(f"libkda: {name} must be {(B, T, H, dk)}, got {tuple(t.shape)}")
    if tuple(v.shape[:3]) != (B, T, H):
        raise ValueError(f"libkda: v must be (B, T, H, dv), got {tuple(v.shape)}")
    if s0 is not None:
        _need(s0, "s0", dev)
        if s0.dtype != torch.float32:
            raise TypeError("libkda: s0 must be float32")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if want_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_state:
        s_final = None
    check("kda_dplr_fwd", lib().kda_dplr_fwd(
        _p(q), _p(k), _p(v), _p(z), _p(a), _p(b), float(g_min), _p(s0), _p(o), _p(s_final),
        B, T, H, dk, dv, _dt(q), _stream(dev)))
    return o, s_final


def dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, dtype):
    return int(lib().kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, CHUNK,
                                                        KDA_BF16 if dtype == torch.bfloat16 else KDA_F32))


def dplr_chunk_fwd(q, k, v, z, a, b, g_min, s0=None, *, o=None, s_final=None, workspace=None,
                   want_state=True):
    """Chunkwise DPLR prefill; arguments and results as dplr_fwd."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("a", a), ("b", b)):
        _need(t, name, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"libkda: {name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("k", k), ("z", z), ("a", a), ("b", b)):
        if tuple(t.shape) != (B, T, H, dk):
            raise ValueError(f"libkda: {name} must be {(B, T, H, dk)}, got {tuple(t.shape)}")
    if tuple(v.shape[:3]) != (B, T, H):
        raise ValueError(f"libkda: v must be (B, T, H, dv), got {tuple(v.shape)}")
    if s0 is not None:
        _need(s0, "s0", dev)
        if s0.dtype != torch.float32:
            raise TypeError("libkda: s0 must be float32")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if want_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_state:
        s_final = None
    need = lib().kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, CHUNK, _dt(q))
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=dev)
    check("kda_dplr_chunk_fwd", lib().kda_dplr_chunk_fwd(
        _p(q), _p(k), _p(v), _p(z), _p(a), _p(b), float(g_min), _p(s0), _p(o), _p(s_final),
        B, T, H, dk, dv, CHUNK, _dt(q), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev)))
    return o, s_final


def dplr_recurrent_step(q, k, v, z, a, b, g_min, state, *, o=None):
    """One DPLR token. q, k, z, a, b: (B,H,dk); v: (B,H,dv); state (B,H,dk,dv)
    fp32, updated in place.  Returns o (B,H,dv)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("a", a), ("b", b), ("state", state)):
        _need(t, name, dev)
    B, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("k", k), ("z", z), ("a", a), ("b", b)):
        if tuple(t.shape) != (B, H, dk):
            raise ValueError(f"libkda: {name} must be {(B, H, dk)}, got {tuple(t.shape)}")
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv):
        raise TypeError("libkda: state must be float32 (B, H, dk, dv)")
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    check("kda_dplr_recurrent_step", lib().kda_dplr_recurrent_step(
        _p(q), _p(k), _p(v), _p(z), _p(a), _p(b), float(g_min), _p(state), _p(o),
        B, H, dk, dv, _dt(q), _stream(dev)))
    return o


def stream_scale(x, s, variant=6):
    """x <- s * x in place (fp32, 16-byte accesses): the read-modify-write
    rate of the GPU's HBM, the ceiling of the decode step (kda_stream_scale)."""
    _need(x, "x", x.device)
    if x.dtype != torch.float32:
        raise TypeError("libkda: stream_scale takes float32")
    check("kda_stream_scale", lib().kda_stream_scale(_p(x), x.numel(), float(s), int(variant), _stream(x.device)))
    return x


def layer(query, key, value, decay_logits, write_strength, output_gate_logits,
          output_projection, initial_state, g_min, eps):
    """The KDA layer of the "KDA Recurrence" problem: recurrence (chunkwise),
    RMSNorm x sigmoid gate, head concat and projection.  Inputs are not
    modified.  Returns {"outputs": (B,T,d_model), "final_state": (B,H,dk,dv) fp32}."""
    s0 = initial_state
    if s0 is not None and s0.dtype != torch.float32:
        s0 = s0.float().contiguous()
    out, s = chunk_layer_fwd(query, key, value, decay_logits, write_strength, g_min, output_gate_logits,
                             eps, output_projection, s0)
    return {"outputs": out, "final_state": s}

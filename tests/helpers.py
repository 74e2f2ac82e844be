"""Shared helpers for the GPU parity tests: relative Frobenius errors and
oracle runs on host copies of the exact bits the GPU consumed."""
import numpy as np

import kda_inputs as ki
import oracle

# Parity bars: fp32 token tensors 1e-5 on outputs and state; bf16 token
# tensors with an fp32 state 2e-2 on outputs and 1e-2 on the final state.
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-2)}


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def host(t):
    return ki.to_host_bits(t)


def f64(t):
    return t.detach().double().cpu().numpy()


def oracle_prefill(x, g_min=ki.G_MIN, heads=None, batches=None):
    """Oracle on the host copy of prefill inputs x (dict of device tensors).
    heads / batches select a subset (sampled outputs); returns (o, s)."""
    sel_b = slice(None) if batches is None else batches
    sel_h = slice(None) if heads is None else heads

    def cut(t, lead_h_axis):
        a = host(t)
        a = a[sel_b]
        idx = [slice(None)] * a.ndim
        idx[lead_h_axis] = sel_h
        return np.ascontiguousarray(a[tuple(idx)])

    q, k, v, z = (cut(x[n], 2) for n in ("q", "k", "v", "z"))
    beta = cut(x["beta"], 2)
    s0 = cut(x["s0"], 1) if x.get("s0") is not None else None
    return oracle.forward(q, k, v, z, beta, g_min, s0)


def block_rel_max(got, ref, block=64):
    """Largest error of one block of `block` tokens of one (batch, head):
    ||got - ref||_F over the block, divided by that head's ||ref||_F scaled
    to the block's share of the sequence, sqrt(block_len / T).  With o laid
    out (B, T, H, d), a defect confined to a few tokens shows up here at
    full size instead of being averaged over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    B, T, H = ref.shape[:3]
    if T == 0:
        return 0.0
    d = (got - ref).reshape(B, T, H, -1)
    r = ref.reshape(B, T, H, -1)
    head = np.sqrt((r * r).sum(axis=(1, 3)))                      # (B, H)
    nb = (T + block - 1) // block
    pad = nb * block - T
    d2 = np.pad((d * d).sum(axis=3), ((0, 0), (0, pad), (0, 0)))   # (B, nb*block, H)
    blk = np.sqrt(d2.reshape(B, nb, block, H).sum(axis=2))         # (B, nb, H)
    lens = np.full(nb, block, np.float64)
    lens[-1] = T - (nb - 1) * block
    scale = head[:, None, :] * np.sqrt(lens / T)[None, :, None]
    return float((blk / np.maximum(scale, 1e-300)).max())

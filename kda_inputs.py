"""Seeded synthetic inputs for the KDA operator.

Shared by the tests, the smoke check and the benchmark: the GPU path and the
oracle always consume the very same bits (the oracle gets a host copy of what
this module produced).  This module holds none of the operator's arithmetic:
it only draws random tensors and prepares them the way the workloads below
describe (L2-normalised keys and queries, sigmoid-squashed write strengths).

Workloads (shapes and value distributions of the pages' setting: 32 heads,
d_k = d_v = 128, 64-token chunks):

  tiny_fp32    B=1, T=256, H=1, d=64, fp32, S0 = 0, no epilogue
  prefill_32k  B=1, T=32768, H=32, d=128, bf16 inputs, S0 ~ N(0, 0.01)
  train_8x8k   B=8, T=8192, H=32, d=128, bf16, S0 = 0, epilogue + projection
               to d_model = 2304 with W ~ N(0, 1/4096) in bf16
  decode_256   B=256 sequences, H=32, d=128, 1024 single-token steps,
               S0 ~ N(0, 0.01) in fp32
  long_1m      B=1, T=1048576, H=32, d=128, bf16, z ~ N(2, 1), S0 = 0,
               RMSNorm x gate epilogue without projection

Generators: q, k ~ N(0,1), L2-normalised over d_k per (b, t, h), q then scaled
by d_k^-1/2; v ~ N(0,1); decay logits z ~ N(z_mean, 1); beta = sigmoid(N(0,1));
for the general DPLR recurrence a = sigmoid(N(0,1)) x a unit row, b a unit row;
output-gate logits ~ N(0,1); N(mu, x) takes x as a variance.  Normal draws are
made in fp32 on the requested device with a torch.Generator seeded per
tensor, then rounded (round-to-nearest-even) to the workload dtype.
"""
import math

import torch

WORKLOADS = {
    "tiny_fp32": dict(B=1, T=256, H=1, dk=64, dv=64, chunk=64, dtype=torch.float32,
                      z_mean=0.0, s0_var=0.0, epilogue=None),
    "prefill_32k": dict(B=1, T=32768, H=32, dk=128, dv=128, chunk=64, dtype=torch.bfloat16,
                        z_mean=0.0, s0_var=0.01, epilogue=None),
    "train_8x8k": dict(B=8, T=8192, H=32, dk=128, dv=128, chunk=64, dtype=torch.bfloat16,
                       z_mean=0.0, s0_var=0.0, epilogue="projection", d_model=2304),
    "decode_256": dict(B=256, H=32, dk=128, dv=128, steps=1024, dtype=torch.bfloat16,
                       z_mean=0.0, s0_var=0.01),
    "long_1m": dict(B=1, T=1048576, H=32, dk=128, dv=128, chunk=64, dtype=torch.bfloat16,
                    z_mean=2.0, s0_var=0.0, epilogue="gate"),
}

G_MIN = -5.0
EPS = 1e-6

# tensor ids, mixed into the per-tensor seed
_Q, _K, _V, _Z, _BETA, _GATE, _S0, _W, _A, _B = range(10)


def _gen(seed, tensor_id, step, device):
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + tensor_id * 7_919 + int(step) * 104_729) % (2 ** 62))
    return g


def _randn(shape, seed, tid, step, device):
    return torch.randn(shape, generator=_gen(seed, tid, step, device), device=device,
                       dtype=torch.float32)


def _unit_rows(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def token_inputs(lead, dk, dv, dtype, seed, device="cpu", z_mean=0.0, step=0):
    """q, k, v, z, beta for token-major shapes lead + (d,), beta of shape lead.

    lead is (B, T, H) for prefill or (B, H) for one decode step.
    """
    lead = tuple(lead)
    q = _unit_rows(_randn(lead + (dk,), seed, _Q, step, device)) * (dk ** -0.5)
    k = _unit_rows(_randn(lead + (dk,), seed, _K, step, device))
    v = _randn(lead + (dv,), seed, _V, step, device)
    z = _randn(lead + (dk,), seed, _Z, step, device) + z_mean
    beta = torch.sigmoid(_randn(lead, seed, _BETA, step, device))
    return {n: t.to(dtype).contiguous() for n, t in
            dict(q=q, k=k, v=v, z=z, beta=beta).items()}


def gate_logits(lead, dv, dtype, seed, device="cpu", step=0):
    return _randn(tuple(lead) + (dv,), seed, _GATE, step, device).to(dtype).contiguous()


def initial_state(B, H, dk, dv, var, seed, device="cpu"):
    """fp32 state; zeros when var == 0."""
    if var == 0.0:
        return torch.zeros((B, H, dk, dv), dtype=torch.float32, device=device)
    return (_randn((B, H, dk, dv), seed, _S0, 0, device) * math.sqrt(var)).contiguous()


def projection(d_model, width, seed, device="cpu", dtype=torch.bfloat16):
    """W of shape (d_model, width) ~ N(0, 1/width)."""
    return (_randn((d_model, width), seed, _W, 0, device) * (width ** -0.5)).to(dtype).contiguous()


def prefill_inputs(B, T, H, dk, dv, dtype, seed, device="cpu", z_mean=0.0, s0_var=0.0,
                   gate=False, d_model=None):
    out = token_inputs((B, T, H), dk, dv, dtype, seed, device, z_mean)
    out["s0"] = initial_state(B, H, dk, dv, s0_var, seed, device)
    if gate:
        out["gate"] = gate_logits((B, T, H), dv, dtype, seed, device)
    if d_model:
        out["w"] = projection(d_model, H * dv, seed, device)
    return out


def workload_inputs(name, seed, device="cpu", **override):
    """Inputs of a named prefill workload (not decode_256)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    ep = cfg.get("epilogue")
    return prefill_inputs(cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"], cfg["dtype"], seed,
                          device, z_mean=cfg["z_mean"], s0_var=cfg["s0_var"],
                          gate=ep is not None, d_model=cfg.get("d_model") if ep == "projection" else None)


def decode_step_inputs(B, H, dk, dv, dtype, seed, step, device="cpu", z_mean=0.0):
    """One decode token per sequence: q, k, z (B, H, dk); v (B, H, dv); beta (B, H)."""
    return token_inputs((B, H), dk, dv, dtype, seed, device, z_mean, step=step + 1)


def dplr_inputs(lead, dk, dv, dtype, seed, device="cpu", z_mean=0.0, step=0):
    """Inputs of the general diagonal-plus-low-rank recurrence: q, k, v, z as
    token_inputs draws them, and two independent low-rank directions drawn
    like KDA's bound ones but from their own streams: a = sigmoid(N(0,1)) x
    a unit row (the scale of beta k), b = a unit row (the scale of k)."""
    lead = tuple(lead)
    out = token_inputs(lead, dk, dv, dtype, seed, device, z_mean, step)
    del out["beta"]
    sa = torch.sigmoid(_randn(lead + (1,), seed, _A, step + 1_000, device))
    a = _unit_rows(_randn(lead + (dk,), seed, _A, step, device)) * sa
    b = _unit_rows(_randn(lead + (dk,), seed, _B, step, device))
    out["a"] = a.to(dtype).contiguous()
    out["b"] = b.to(dtype).contiguous()
    return out


def to_host_bits(t):
    """Host numpy view of a tensor for the oracle: float64/float32 as is,
    bfloat16 as its uint16 bit patterns (widened exactly by the oracle)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()

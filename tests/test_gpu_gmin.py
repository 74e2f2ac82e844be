"""GPU parity across the decay bound g_min ("KDA Recurrence": any g_min < 0).

The chunkwise kernels split each decay product inside a chunk into factors
around 16-row block references, each spanning up to eight tokens of decay;
they run for g_min >= KDA_CHUNK_G_MIN_LIMIT (-8), and the prefill calls take
the token-sequential kernel below it.  These cases cover both sides of the
limit, with decay logits z ~ N(2, 1) (most alpha near e^{g_min}) and with z
saturated (every alpha exactly e^{g_min}, the largest factors the chunkwise
kernels can meet), on every plan: single level, two levels (segments), the
one-pass plan of 256 chains, decode, the layer calls and the scalar gate.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gated_delta_rule_14_amd import kda
from helpers import TOL, block_rel_max, f64, host, oracle_prefill, rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GMINS = [-0.5, -5.0, -8.0, -11.0, -20.0]


def _check(x, tag, g_min, label, heads=None, o=None, s=None):
    if o is None:
        o, s = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, x.get("s0"))
    torch.cuda.synchronize()
    ro, rs = oracle_prefill(x, g_min=g_min, heads=heads)
    if heads is not None:
        o, s = o[:, :, heads], s[:, heads]
    go, gs = f64(o), f64(s)
    eo, es, eb = rel(go, ro), rel(gs, rs), block_rel_max(go, ro)
    print(f"g_min={g_min} {label} {tag}: o {eo:.2e} (worst block {eb:.2e}) state {es:.2e}")
    to, ts = TOL[tag]
    assert eo < to and es < ts and eb < to, (eo, eb, es)


@pytest.mark.parametrize("g_min", GMINS)
@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
@pytest.mark.parametrize("T", [300, 2113])
def test_prefill_g_min(g_min, dtype, tag, T):
    """T = 300: one level; T = 2113 with 2 chains: segments (compose, scan,
    expand) on the chunkwise side of the limit."""
    x = ki.prefill_inputs(1, T, 2, 128, 128, dtype, seed=T + int(-10 * g_min), device=DEV, s0_var=0.01,
                          z_mean=2.0)
    _check(x, tag, g_min, f"T={T}")


@pytest.mark.parametrize("g_min", [-8.0, -8.01, -20.0])
@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
def test_prefill_saturated_decay(g_min, dtype, tag):
    """z = 30: sigmoid(z) = 1 in fp32, so every channel of every token decays
    by exactly e^{g_min}.  At g_min = -8 the chunkwise kernels meet their
    largest factors (2^{8 * 8 * log2 e}); just below the limit the
    token-sequential kernel runs."""
    x = ki.prefill_inputs(1, 2113, 2, 128, 128, dtype, seed=77, device=DEV, s0_var=0.01)
    x["z"] = torch.full_like(x["z"], 30.0)
    _check(x, tag, g_min, "z=30")


@pytest.mark.parametrize("g_min", [-0.5, -8.0, -20.0])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_prefill_g_min_widths(g_min, dk, dv):
    x = ki.prefill_inputs(1, 2100, 2, dk, dv, torch.bfloat16, seed=dk + dv, device=DEV, s0_var=0.01, z_mean=2.0)
    _check(x, "bf16", g_min, f"dk={dk} dv={dv}")


@pytest.mark.parametrize("g_min", GMINS)
def test_one_pass_plan_g_min(g_min):
    """256 chains (B=2, H=128): one expand pass over whole sequences, the plan
    of the 8x8192 training shape; the oracle runs on sampled heads."""
    x = ki.prefill_inputs(2, 640, 128, 128, 128, torch.bfloat16, seed=5, device=DEV, s0_var=0.01, z_mean=2.0)
    _check(x, "bf16", g_min, "256 chains", heads=[0, 63, 127])


@pytest.mark.parametrize("g_min", GMINS)
@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
def test_decode_g_min(g_min, dtype, tag):
    B, H, d, steps = 3, 2, 128, 40
    state = ki.initial_state(B, H, d, d, 0.01, 61, DEV)
    s0 = state.double().cpu().numpy().reshape(B * H, 1, d, d)
    outs, ins = [], {n: [] for n in ("q", "k", "v", "z", "beta")}
    for t in range(steps):
        x = ki.decode_step_inputs(B, H, d, d, dtype, 61, t, DEV, z_mean=2.0)
        o = kda.recurrent_step(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, state)
        outs.append(f64(o).reshape(B * H, d))
        for n in ins:
            a = host(x[n])
            ins[n].append(a.reshape((B * H,) + a.shape[2:]))
    torch.cuda.synchronize()
    st = {n: np.ascontiguousarray(np.stack(v, axis=1)[:, :, None]) for n, v in ins.items()}
    ro, rs = oracle.forward(st["q"], st["k"], st["v"], st["z"], st["beta"], g_min, np.ascontiguousarray(s0))
    go = np.stack(outs, axis=1)                       # (B * H, steps, d)
    eo, es = rel(go, ro[:, :, 0]), rel(f64(state).reshape(B * H, d, d), rs[:, 0])
    print(f"g_min={g_min} decode {tag}: o {eo:.2e} state {es:.2e}")
    to, ts = TOL[tag]
    assert eo < to and es < ts


@pytest.mark.parametrize("g_min", [-5.0, -20.0])
@pytest.mark.parametrize("proj", [False, True])
def test_layer_prefill_g_min(g_min, proj):
    """kda_chunk_layer_fwd on both sides of the limit (segmented plan with the
    epilogue in the prefill's kernels; token-sequential kernel with the
    epilogue on its fp32 read-out), with and without the projection."""
    d_model = 272 if proj else None
    x = ki.prefill_inputs(1, 2113, 2, 128, 128, torch.bfloat16, seed=91, device=DEV, s0_var=0.01, z_mean=2.0,
                          gate=True, d_model=d_model)
    w = x.get("w")
    y, s, o = kda.chunk_layer_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, x["gate"], ki.EPS, w, x["s0"],
                                  want_o=True)
    torch.cuda.synchronize()
    ro, rs = oracle_prefill(x, g_min=g_min)
    ry = oracle.out_gate(ro, host(x["gate"]), ki.EPS, None if w is None else host(w))
    eo, es, ey = rel(f64(o), ro), rel(f64(s), rs), rel(f64(y), ry)
    print(f"g_min={g_min} layer prefill (projection {proj}): o {eo:.2e} y {ey:.2e} state {es:.2e}")
    assert eo < 2e-2 and ey < 2e-2 and es < 1e-2


@pytest.mark.parametrize("g_min", [-5.0, -20.0])
@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
def test_gdn_prefill_g_min(g_min, dtype, tag):
    x = ki.prefill_inputs(1, 700, 2, 128, 128, dtype, seed=93, device=DEV, s0_var=0.01, z_mean=2.0)
    zs = x["z"][..., 0].contiguous()
    o, s = kda.gdn_chunk_fwd(x["q"], x["k"], x["v"], zs, x["beta"], g_min, x["s0"])
    x["z"] = zs[..., None].expand_as(x["z"]).contiguous()
    _check(x, tag, g_min, "scalar gate", o=o, s=s)


def test_sequential_kernel_matches_decode_steps():
    """Below the limit the prefill takes the token-sequential kernel, whose
    token step is the decode step's arithmetic: T prefill tokens agree with T
    successive kda_recurrent_step calls to fp32 rounding."""
    B, T, H, d, g_min = 2, 50, 3, 128, -12.0
    x = ki.prefill_inputs(B, T, H, d, d, torch.float32, seed=95, device=DEV, s0_var=0.01, z_mean=2.0)
    o, s = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, x["s0"])
    st = x["s0"].clone()
    od = [kda.recurrent_step(*(x[n][:, t].contiguous() for n in ("q", "k", "v", "z", "beta")), g_min, st)
          for t in range(T)]
    torch.cuda.synchronize()
    assert rel(f64(torch.stack(od, 1)), f64(o)) < 1e-6
    assert rel(f64(st), f64(s)) < 1e-6

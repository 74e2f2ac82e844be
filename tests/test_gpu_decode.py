"""GPU parity of kda_recurrent_step against the fp64 oracle.

A run of decode steps is the recurrence over a sequence of single tokens,
so the oracle is run once over the stacked per-step inputs.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gated_delta_rule_14_amd import kda
from helpers import TOL, f64, host, rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_steps(B, H, dk, dv, dtype, steps, seed, s0_var=0.01, heads=None, z_mean=0.0):
    """Run `steps` decode steps on the GPU; return GPU outputs / state and the
    oracle's, restricted to the flat (b*H + h) indices in `heads` (selected
    on the device, so that only those heads are copied to the host)."""
    state = ki.initial_state(B, H, dk, dv, s0_var, seed, DEV)
    sel = np.arange(B * H) if heads is None else np.asarray(heads)
    sel_d = torch.as_tensor(sel, device=DEV)
    s0_host = state.reshape(B * H, dk, dv)[sel_d].double().cpu().numpy()
    outs, ins = [], {n: [] for n in ("q", "k", "v", "z", "beta")}
    for t in range(steps):
        d = ki.decode_step_inputs(B, H, dk, dv, dtype, seed, t, DEV, z_mean=z_mean)
        o = kda.recurrent_step(d["q"], d["k"], d["v"], d["z"], d["beta"], ki.G_MIN, state)
        outs.append(o.reshape(B * H, dv)[sel_d].double())
        for n in ins:
            a = d[n]
            ins[n].append(a.reshape((B * H,) + tuple(a.shape[2:]))[sel_d].clone())
    torch.cuda.synchronize()
    # oracle layout: (batch = selected head, T = steps, H = 1, d)
    stack = {n: np.ascontiguousarray(host(torch.stack(v, dim=1))[:, :, None]) for n, v in ins.items()}
    ro, rs = oracle.forward(stack["q"], stack["k"], stack["v"], stack["z"], stack["beta"], ki.G_MIN,
                            np.ascontiguousarray(s0_host[:, None]))
    go = torch.stack(outs, dim=1).cpu().numpy()       # (sel, steps, dv)
    gs = state.reshape(B * H, dk, dv)[sel_d].double().cpu().numpy()
    return go, gs, ro[:, :, 0], rs[:, 0]


@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_small(dtype, tag, dk, dv):
    go, gs, ro, rs = run_steps(3, 2, dk, dv, dtype, steps=24, seed=100 + dk + dv)
    to, ts = TOL[tag]
    eo, es = rel(go, ro), rel(gs, rs)
    print(f"decode {tag} dk={dk} dv={dv}: o {eo:.2e} state {es:.2e}")
    assert eo < to and es < ts


def test_decode_long_memory():
    """z ~ N(-8, 1): alpha close to 1, the state carries information across
    all steps, so an error in the carried state cannot fade away."""
    go, gs, ro, rs = run_steps(2, 2, 128, 128, torch.float32, steps=200, seed=5, z_mean=-8.0)
    eo, es = rel(go, ro), rel(gs, rs)
    print(f"decode long memory: o {eo:.2e} state {es:.2e}")
    assert eo < 1e-5 and es < 1e-5


def test_decode_state_in_place_and_deterministic():
    B, H, d = 8, 4, 128
    d_in = ki.decode_step_inputs(B, H, d, d, torch.bfloat16, 9, 0, DEV)
    s1 = ki.initial_state(B, H, d, d, 0.01, 9, DEV)
    s2 = s1.clone()
    ptr = s1.data_ptr()
    before = {n: t.clone() for n, t in d_in.items()}
    o1 = kda.recurrent_step(d_in["q"], d_in["k"], d_in["v"], d_in["z"], d_in["beta"], ki.G_MIN, s1)
    o2 = kda.recurrent_step(d_in["q"], d_in["k"], d_in["v"], d_in["z"], d_in["beta"], ki.G_MIN, s2)
    torch.cuda.synchronize()
    assert s1.data_ptr() == ptr
    assert torch.equal(s1, s2) and torch.equal(o1, o2)
    for n, t in d_in.items():
        assert torch.equal(t, before[n]), n


@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
def test_decode_heads_dealt_over_workgroups(dtype, tag):
    """1000 heads of d = 128: more heads than one launch has workgroups (two
    per compute unit) and not a multiple of them, so a workgroup takes one or
    more heads in turn, loading the next head's state meanwhile.  Every head
    is checked against the oracle on its own, and every head is bit-equal to
    the same sequences stepped in a call so small that each workgroup takes
    one head."""
    B, H, d = 125, 8, 128
    go, gs, ro, rs = run_steps(B, H, d, d, dtype, steps=6, seed=31)
    to, ts = TOL[tag]
    eo = max(rel(go[i], ro[i]) for i in range(B * H))
    es = max(rel(gs[i], rs[i]) for i in range(B * H))
    print(f"decode {tag} 1000 heads: worst head o {eo:.2e} state {es:.2e}")
    assert eo < to and es < ts

    d_in = ki.decode_step_inputs(B, H, d, d, dtype, 77, 0, DEV)
    s_full = ki.initial_state(B, H, d, d, 0.01, 77, DEV)
    for lo, hi in ((0, 3), (120, 125)):
        s_part = s_full[lo:hi].clone()
        o_part = kda.recurrent_step(*(d_in[n][lo:hi].contiguous() for n in ("q", "k", "v", "z", "beta")),
                                    ki.G_MIN, s_part)
        if lo == 0:
            s_ref = s_full.clone()
            o_full = kda.recurrent_step(d_in["q"], d_in["k"], d_in["v"], d_in["z"], d_in["beta"], ki.G_MIN, s_ref)
        torch.cuda.synchronize()
        assert torch.equal(o_full[lo:hi], o_part) and torch.equal(s_ref[lo:hi], s_part), (lo, hi)


def test_decode_full_size_sampled():
    """B=256 sequences, H=32, d=128, fp32 state, bf16 tokens: the full decode
    workload, all 1024 steps with all 8192 heads launched; 64 heads checked
    over every step, as a whole and step by step."""
    rng = np.random.default_rng(0)
    heads = np.sort(rng.choice(256 * 32, 64, replace=False))
    go, gs, ro, rs = run_steps(256, 32, 128, 128, torch.bfloat16, steps=1024, seed=3, heads=heads)
    eo, es = rel(go, ro), rel(gs, rs)
    # per step and head, against that head's average step
    d = np.sqrt(((go - ro) ** 2).sum(axis=2))
    scale = np.sqrt((ro ** 2).sum(axis=(1, 2)) / ro.shape[1])[:, None]
    ew = float((d / scale).max())
    print(f"decode full size (1024 steps, 64 sampled heads): o {eo:.2e} (worst step {ew:.2e}) state {es:.2e}")
    assert eo < 2e-2 and es < 1e-2 and ew < 2e-2


def run_layer_steps(B, H, dk, dv, dtype, steps, seed, d_model=0, batches=None, s0_var=0.01):
    """`steps` tokens of kda_recurrent_layer_step (recurrence step with the
    RMSNorm x gate epilogue fused, then the projection when d_model > 0).
    Returns the GPU's y (B_sel, steps, width) and the oracle's: the fp64
    recurrence over the stacked tokens of the selected batch rows (all their
    heads), then the oracle epilogue on its fp64 outputs."""
    state = ki.initial_state(B, H, dk, dv, s0_var, seed, DEV)
    s0_host = state.double().cpu().numpy()
    w = ki.projection(d_model, H * dv, seed, DEV) if d_model else None
    bsel = np.arange(B) if batches is None else np.asarray(batches)
    ys, gates, ins = [], [], {n: [] for n in ("q", "k", "v", "z", "beta")}
    for t in range(steps):
        d = ki.decode_step_inputs(B, H, dk, dv, dtype, seed, t, DEV)
        g = ki.gate_logits((B, H), dv, dtype, seed, DEV, step=t + 1)
        y = kda.recurrent_layer_step(d["q"], d["k"], d["v"], d["z"], d["beta"], ki.G_MIN, state, g, ki.EPS, w)
        ys.append(f64(y)[bsel])
        gates.append(host(g)[bsel])
        for n in ins:
            ins[n].append(host(d[n])[bsel])
    torch.cuda.synchronize()
    nb = len(bsel)
    # oracle layout: batch = (selected row, head), T = steps, H = 1
    stack = {}
    for n, v in ins.items():
        a = np.stack(v, axis=2)                        # (nb, H, steps, ...)
        stack[n] = np.ascontiguousarray(a.reshape((nb * H, steps, 1) + a.shape[3:]))
    s0 = np.ascontiguousarray(s0_host[bsel].reshape(nb * H, 1, dk, dv))
    ro, _ = oracle.forward(stack["q"], stack["k"], stack["v"], stack["z"], stack["beta"], ki.G_MIN, s0)
    ro = ro.reshape(nb, H, steps, dv).transpose(0, 2, 1, 3)          # (nb, steps, H, dv)
    gate_h = np.ascontiguousarray(np.stack(gates, axis=1))          # (nb, steps, H, dv)
    ry = oracle.out_gate(np.ascontiguousarray(ro), gate_h, ki.EPS, None if w is None else host(w))
    return np.stack(ys, axis=1), ry


@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_layer_step_small(dtype, tag, dk, dv):
    gy, ry = run_layer_steps(3, 2, dk, dv, dtype, steps=12, seed=200 + dk + dv)
    e = rel(gy, ry)
    print(f"layer step {tag} dk={dk} dv={dv}: y {e:.2e}")
    assert e < TOL[tag][0]


@pytest.mark.parametrize("dv,d_model", [(64, 48), (128, 272)])
def test_layer_step_projection_small(dv, d_model):
    gy, ry = run_layer_steps(5, 3, 128, dv, torch.bfloat16, steps=6, seed=31 + dv, d_model=d_model)
    e = rel(gy, ry)
    print(f"layer step + projection dv={dv} d_model={d_model}: {e:.2e}")
    assert e < 2e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_layer_step_matches_step_then_gate(dtype):
    """The fused call leaves the same state and read-out as kda_recurrent_step
    (bit for bit: same arithmetic), and its y equals kda_out_gate applied to
    that read-out up to the read-out's rounding to the token dtype."""
    B, H, d = 6, 4, 128
    d_in = ki.decode_step_inputs(B, H, d, d, dtype, 17, 0, DEV)
    g = ki.gate_logits((B, H), d, dtype, 17, DEV, step=1)
    s1 = ki.initial_state(B, H, d, d, 0.01, 17, DEV)
    s2 = s1.clone()
    y1, o1 = kda.recurrent_layer_step(d_in["q"], d_in["k"], d_in["v"], d_in["z"], d_in["beta"], ki.G_MIN, s1, g,
                                      ki.EPS, want_o=True)
    o2 = kda.recurrent_step(d_in["q"], d_in["k"], d_in["v"], d_in["z"], d_in["beta"], ki.G_MIN, s2)
    y2 = kda.out_gate(o2.view(B, 1, H, d), g.view(B, 1, H, d), ki.EPS).view(B, H * d)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(o1, o2)
    e = rel(f64(y1), f64(y2))
    print(f"fused vs step-then-gate ({dtype}): {e:.2e}")
    assert e < (1e-6 if dtype == torch.float32 else 1e-2)


def test_layer_step_full_size_sampled():
    """B=256 sequences, H=32, d=128, bf16 tokens, fp32 state, projection to
    d_model = 2304: the decode workload shape through the whole layer for 4
    tokens, every head launched; 3 batch rows checked (all their heads, so
    that the projection's rows are complete)."""
    gy, ry = run_layer_steps(256, 32, 128, 128, torch.bfloat16, steps=4, seed=41, d_model=2304,
                             batches=[0, 117, 255])
    e = rel(gy, ry)
    print(f"layer step full size (4 tokens, 3 rows, projection 4096 -> 2304): {e:.2e}")
    assert e < 2e-2

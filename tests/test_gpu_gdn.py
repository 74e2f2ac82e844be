"""GPU parity of the scalar-gate (Gated DeltaNet) calls, kda_gdn_chunk_fwd
and kda_gdn_recurrent_step, against the fp64 oracle given the same logit in
every key channel (which is what a scalar decay is: Diag(alpha) = alpha I),
and bit-equality with the channel-wise calls on that repeated z."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gated_delta_rule_14_amd import kda
from helpers import TOL, f64, host, oracle_prefill, rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def scalar_gate_inputs(B, T, H, dk, dv, dtype, seed, z_mean=0.0, s0_var=0.01):
    x = ki.prefill_inputs(B, T, H, dk, dv, dtype, seed, DEV, z_mean=z_mean, s0_var=s0_var)
    # one logit per (token, head): the first channel's draw
    x["zs"] = x["z"][..., 0].contiguous()
    x["z"] = x["zs"][..., None].expand(B, T, H, dk).contiguous()
    return x


def check_prefill(x, tag, heads=None, label=""):
    o, s = kda.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["zs"], x["beta"], ki.G_MIN, x["s0"])
    torch.cuda.synchronize()
    ro, rs = oracle_prefill(x, heads=heads)
    go, gs = f64(o), f64(s)
    if heads is not None:
        go, gs = go[:, :, heads], gs[:, heads]
    eo, es = rel(go, ro), rel(gs, rs)
    print(f"gdn prefill {label} {tag}: o {eo:.2e} state {es:.2e}")
    to, ts = TOL[tag]
    assert eo < to and es < ts, (eo, es)
    return o, s


@pytest.mark.parametrize("T", [1, 65, 300])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
def test_gdn_prefill_small(T, dk, dv, dtype, tag):
    check_prefill(scalar_gate_inputs(2, T, 3, dk, dv, dtype, 300 + T + dk), tag, label=f"T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("z_mean", [0.0, -8.0])
@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
def test_gdn_prefill_two_level(z_mean, dtype, tag):
    """Few chains over a long sequence (segments, compose, scan, expand);
    z ~ N(-8, 1) keeps alpha close to 1 so the carried state matters."""
    check_prefill(scalar_gate_inputs(1, 2113, 2, 128, 128, dtype, 77, z_mean=z_mean), tag,
                  label=f"two-level z_mean={z_mean}")


def test_gdn_prefill_equals_channelwise_call():
    """Same kernels: the scalar-gate call gives the channel-wise call's bits
    for z repeated over the channels (32k-token prefill shape, sampled heads
    checked against the oracle too)."""
    x = scalar_gate_inputs(1, 32768, 32, 128, 128, torch.bfloat16, 5)
    o1, s1 = check_prefill(x, "bf16", heads=[3, 30], label="prefill_32k shape")
    o2, s2 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
def test_gdn_decode_steps(dk, dv, dtype, tag):
    """Successive scalar-gate decode tokens against the oracle over the same
    stacked tokens, and bit-equality with kda_recurrent_step on repeated z."""
    B, H, steps = 3, 2, 16
    state = ki.initial_state(B, H, dk, dv, 0.01, 8, DEV)
    ref_state = state.clone()
    s0_host = state.double().cpu().numpy().reshape(B * H, 1, dk, dv)
    outs, ins = [], {n: [] for n in ("q", "k", "v", "z", "beta")}
    for t in range(steps):
        d = ki.decode_step_inputs(B, H, dk, dv, dtype, 8, t, DEV)
        zs = d["z"][..., 0].contiguous()
        zf = zs[..., None].expand(B, H, dk).contiguous()
        o = kda.gdn_recurrent_step(d["q"], d["k"], d["v"], zs, d["beta"], ki.G_MIN, state)
        o2 = kda.recurrent_step(d["q"], d["k"], d["v"], zf, d["beta"], ki.G_MIN, ref_state)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(state, ref_state), t
        outs.append(f64(o).reshape(B * H, dv))
        for n, tt in (("q", d["q"]), ("k", d["k"]), ("v", d["v"]), ("z", zf), ("beta", d["beta"])):
            a = host(tt)
            ins[n].append(a.reshape((B * H,) + a.shape[2:]))
    stack = {n: np.ascontiguousarray(np.stack(v, axis=1)[:, :, None]) for n, v in ins.items()}
    ro, rs = oracle.forward(stack["q"], stack["k"], stack["v"], stack["z"], stack["beta"], ki.G_MIN, s0_host)
    eo = rel(np.stack(outs, axis=1), ro[:, :, 0])
    es = rel(state.double().cpu().numpy().reshape(B * H, dk, dv), rs[:, 0])
    print(f"gdn decode {tag} dk={dk} dv={dv}: o {eo:.2e} state {es:.2e}")
    to, ts = TOL[tag]
    assert eo < to and es < ts


def test_gdn_prefill_one_pass_equals_channelwise_call():
    """256 chains (the one-pass plan: every chain in one workgroup, no
    segments) with a ragged last chunk: the scalar-gate call gives the
    channel-wise call's bits, and sampled heads match the oracle."""
    x = scalar_gate_inputs(8, 300, 32, 128, 128, torch.bfloat16, 41)
    o1, s1 = check_prefill(x, "bf16", heads=[0, 17, 31], label="one pass, 8 x 300 x 32")
    o2, s2 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)

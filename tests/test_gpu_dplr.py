"""GPU parity of the general DPLR recurrence (kda_dplr_fwd and
kda_dplr_recurrent_step) against the fp64 DPLR oracle.

"Diagonal-Plus-Low-Rank Matrices and Kimi Delta Attention", sections 1 and 3:
S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, with a
and b independent.  Section 3's binding (a = beta k, b = k * alpha, write key
beta k) is also checked against libkda's own KDA prefill.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from gated_delta_rule_14_amd import kda
from helpers import TOL, block_rel_max, f64, host, rel
from oracle import dplr as odplr

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("q", "k", "v", "z", "a", "b")


def inputs(B, T, H, dk, dv, dtype, seed, s0_var=0.01, z_mean=0.0):
    x = ki.dplr_inputs((B, T, H), dk, dv, dtype, seed, DEV, z_mean)
    x["s0"] = ki.initial_state(B, H, dk, dv, s0_var, seed, DEV)
    return x


def oracle_of(x, g_min=ki.G_MIN, heads=None):
    sel = slice(None) if heads is None else heads
    arrs = [np.ascontiguousarray(host(x[n])[:, :, sel]) for n in NAMES]
    s0 = np.ascontiguousarray(host(x["s0"])[:, sel])
    return odplr.forward(*arrs, g_min, s0)


def gpu_fwd(x, g_min=ki.G_MIN):
    return kda.dplr_fwd(*(x[n] for n in NAMES), g_min, x["s0"])


@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_dplr_fwd_small(dtype, tag, dk, dv):
    """Two sequences, three heads, a ragged 150 tokens, nonzero S0."""
    x = inputs(2, 150, 3, dk, dv, dtype, seed=40 + dk + dv)
    o, s = gpu_fwd(x)
    torch.cuda.synchronize()
    ro, rs = oracle_of(x)
    to, ts = TOL[tag]
    eo, es = rel(f64(o), ro), rel(f64(s), rs)
    print(f"dplr {tag} dk={dk} dv={dv}: o {eo:.2e} state {es:.2e}")
    assert eo < to and es < ts
    assert block_rel_max(f64(o), ro) < 2 * to


@pytest.mark.parametrize("T", [0, 1, 2, 63])
def test_dplr_fwd_short(T):
    """T = 0 returns S0 untouched as the final state; T = 1, 2, 63 cover the
    prefetch of the next token at the sequence's end."""
    x = inputs(1, T, 2, 128, 128, torch.float32, seed=7 + T)
    o, s = gpu_fwd(x)
    torch.cuda.synchronize()
    ro, rs = oracle_of(x)
    if T == 0:
        assert torch.equal(s, x["s0"])
        return
    assert rel(f64(o), ro) < 1e-5 and rel(f64(s), rs) < 1e-5


def test_dplr_fwd_zero_state_and_no_final_state():
    x = inputs(1, 70, 2, 64, 64, torch.float32, seed=3, s0_var=0.0)
    o1, _ = kda.dplr_fwd(*(x[n] for n in NAMES), ki.G_MIN, None, want_state=False)
    o2, s2 = gpu_fwd(x)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    ro, rs = oracle_of(x)
    assert rel(f64(o1), ro) < 1e-5 and rel(f64(s2), rs) < 1e-5


@pytest.mark.parametrize("g_min", [-0.5, -12.0])
def test_dplr_fwd_decay_range(g_min):
    """The token-sequential kernel has no decay bound: slow and very fast
    forgetting both hold the fp32 bar."""
    x = inputs(1, 200, 2, 128, 128, torch.float32, seed=11)
    o, s = gpu_fwd(x, g_min)
    torch.cuda.synchronize()
    ro, rs = oracle_of(x, g_min)
    eo, es = rel(f64(o), ro), rel(f64(s), rs)
    print(f"dplr g_min={g_min}: o {eo:.2e} state {es:.2e}")
    assert eo < 1e-5 and es < 1e-5


def test_dplr_binding_gives_kda():
    """Section 3: a = beta k, b = k * alpha and the write key beta k turn the
    DPLR recurrence into KDA; libkda's DPLR kernel then agrees with its KDA
    prefill (fp32, the two kernels' own rounding apart)."""
    B, T, H, d = 1, 300, 4, 128
    x = ki.prefill_inputs(B, T, H, d, d, torch.float32, seed=21, device=DEV, s0_var=0.01)
    alpha = torch.exp(ki.G_MIN * torch.sigmoid(x["z"].double()))
    bk = (x["beta"].double()[..., None] * x["k"].double()).float().contiguous()
    b = (x["k"].double() * alpha).float().contiguous()
    o1, s1 = kda.dplr_fwd(x["q"], bk, x["v"], x["z"], bk, b, ki.G_MIN, x["s0"])
    o2, s2 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"])
    torch.cuda.synchronize()
    eo, es = rel(f64(o1), f64(o2)), rel(f64(s1), f64(s2))
    print(f"binding: o {eo:.2e} state {es:.2e}")
    assert eo < 2e-5 and es < 2e-5


def test_dplr_full_size_sampled():
    """The 32-head, 32768-token bf16 prefill shape: every head on the GPU,
    two heads against the oracle (token by token, every 64-token block)."""
    B, T, H, d = 1, 32768, 32, 128
    x = inputs(B, T, H, d, d, torch.bfloat16, seed=5)
    o, s = gpu_fwd(x)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    heads = [0, 31]
    ro, rs = oracle_of(x, heads=heads)
    go, gs = f64(o[:, :, heads]), f64(s[:, heads])
    eo, es, eb = rel(go, ro), rel(gs, rs), block_rel_max(go, ro)
    print(f"dplr full size: o {eo:.2e} state {es:.2e} worst block {eb:.2e}")
    assert eo < 2e-2 and es < 1e-2 and eb < 4e-2


def run_steps(B, H, dk, dv, dtype, steps, seed, heads=None):
    """Decode steps on the GPU, the oracle over the stacked per-step inputs
    of the heads `heads` (flat b * H + h)."""
    state = ki.initial_state(B, H, dk, dv, 0.01, seed, DEV)
    sel = np.arange(B * H) if heads is None else np.asarray(heads)
    sel_d = torch.as_tensor(sel, device=DEV)
    s0 = state.reshape(B * H, dk, dv)[sel_d].double().cpu().numpy()
    outs, ins = [], {n: [] for n in NAMES}
    for t in range(steps):
        d = ki.dplr_inputs((B, H), dk, dv, dtype, seed, DEV, step=t + 1)
        o = kda.dplr_recurrent_step(*(d[n] for n in NAMES), ki.G_MIN, state)
        outs.append(o.reshape(B * H, dv)[sel_d].double())
        for n in NAMES:
            ins[n].append(d[n].reshape((B * H,) + tuple(d[n].shape[2:]))[sel_d].clone())
    torch.cuda.synchronize()
    stack = [np.ascontiguousarray(host(torch.stack(ins[n], dim=1))[:, :, None]) for n in NAMES]
    ro, rs = odplr.forward(*stack, ki.G_MIN, np.ascontiguousarray(s0[:, None]))
    go = torch.stack(outs, dim=1).cpu().numpy()
    gs = state.reshape(B * H, dk, dv)[sel_d].double().cpu().numpy()
    return go, gs, ro[:, :, 0], rs[:, 0]


@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_dplr_step_small(dtype, tag, dk, dv):
    go, gs, ro, rs = run_steps(3, 2, dk, dv, dtype, steps=20, seed=60 + dk + dv)
    to, ts = TOL[tag]
    eo, es = rel(go, ro), rel(gs, rs)
    print(f"dplr step {tag} dk={dk} dv={dv}: o {eo:.2e} state {es:.2e}")
    assert eo < to and es < ts


def test_dplr_step_full_size_sampled():
    """256 sequences x 32 heads (the decode batch), 8 steps, 6 heads checked."""
    heads = [0, 1, 500, 4097, 8190, 8191]
    go, gs, ro, rs = run_steps(256, 32, 128, 128, torch.bfloat16, steps=8, seed=13, heads=heads)
    eo, es = rel(go, ro), rel(gs, rs)
    print(f"dplr step full size: o {eo:.2e} state {es:.2e}")
    assert eo < 2e-2 and es < 1e-2


def test_dplr_steps_equal_prefill():
    """A run of single-token steps and the sequence kernel compute the same
    per-token arithmetic (fp32)."""
    B, T, H, d = 2, 40, 3, 128
    x = inputs(B, T, H, d, d, torch.float32, seed=17)
    o1, s1 = gpu_fwd(x)
    state = x["s0"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.dplr_recurrent_step(*(x[n][:, t].contiguous() for n in NAMES), ki.G_MIN, state))
    torch.cuda.synchronize()
    o2 = torch.stack(outs, dim=1)
    assert rel(f64(o2), f64(o1)) < 1e-6 and rel(f64(state), f64(s1)) < 1e-6


def test_dplr_inputs_untouched_and_deterministic():
    x = inputs(1, 100, 4, 128, 128, torch.bfloat16, seed=19)
    before = {n: t.clone() for n, t in x.items()}
    o1, s1 = gpu_fwd(x)
    o2, s2 = gpu_fwd(x)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    for n, t in x.items():
        assert torch.equal(t, before[n]), n


# ---------------------------------------------------------------- chunkwise
def gpu_chunk(x, g_min=ki.G_MIN, workspace=None):
    return kda.dplr_chunk_fwd(*(x[n] for n in NAMES), g_min, x["s0"], workspace=workspace)


@pytest.mark.parametrize("dtype,tag", [(torch.float32, "f32"), (torch.bfloat16, "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [150, 2100])
def test_dplr_chunk_small(dtype, tag, dk, dv, T):
    """150 tokens: one chain per column tile over three chunks (the last
    ragged); 2100 tokens: 33 chunks, the two-level plan (segments of 16
    chunks, a ragged last segment and chunk)."""
    x = inputs(2, T, 2, dk, dv, dtype, seed=80 + dk + dv + T)
    o, s = gpu_chunk(x)
    torch.cuda.synchronize()
    ro, rs = oracle_of(x)
    to, ts = TOL[tag]
    eo, es, eb = rel(f64(o), ro), rel(f64(s), rs), block_rel_max(f64(o), ro)
    print(f"dplr chunk {tag} dk={dk} dv={dv} T={T}: o {eo:.2e} state {es:.2e} worst block {eb:.2e}")
    assert eo < to and es < ts and eb < 2 * to


@pytest.mark.parametrize("T", [1, 63, 64, 65, 2048])
def test_dplr_chunk_edges(T):
    x = inputs(1, T, 3, 128, 128, torch.float32, seed=90 + T)
    o, s = gpu_chunk(x)
    torch.cuda.synchronize()
    ro, rs = oracle_of(x)
    assert rel(f64(o), ro) < 1e-5 and rel(f64(s), rs) < 1e-5


def test_dplr_chunk_t0_returns_s0():
    x = inputs(1, 0, 2, 64, 64, torch.float32, seed=1)
    o, s = gpu_chunk(x)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(s, x["s0"])


@pytest.mark.parametrize("g_min", [-0.5, -8.0])
def test_dplr_chunk_decay_range(g_min):
    """Up to the chunkwise decay bound (block factors reach 2^92 at -8)."""
    x = inputs(1, 1100, 2, 128, 128, torch.float32, seed=31)
    o, s = gpu_chunk(x, g_min)
    torch.cuda.synchronize()
    ro, rs = oracle_of(x, g_min)
    eo, es, eb = rel(f64(o), ro), rel(f64(s), rs), block_rel_max(f64(o), ro)
    print(f"dplr chunk g_min={g_min}: o {eo:.2e} state {es:.2e} worst block {eb:.2e}")
    assert eo < 1e-5 and es < 1e-5 and eb < 2e-5


def test_dplr_chunk_below_limit_runs_token_kernel():
    """Below the bound the chunkwise call is the token-sequential kernel."""
    x = inputs(1, 300, 2, 128, 128, torch.bfloat16, seed=33)
    o1, s1 = gpu_chunk(x, -9.0)
    o2, s2 = gpu_fwd(x, -9.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_dplr_chunk_long_memory():
    """z ~ N(-6, 1): alpha near 1, the carried state matters over 4096 tokens
    (two-level plan, 4 segments)."""
    x = inputs(1, 4096, 2, 128, 128, torch.float32, seed=35, z_mean=-6.0)
    o, s = gpu_chunk(x)
    torch.cuda.synchronize()
    ro, rs = oracle_of(x)
    eo, es, eb = rel(f64(o), ro), rel(f64(s), rs), block_rel_max(f64(o), ro)
    print(f"dplr chunk long memory: o {eo:.2e} state {es:.2e} worst block {eb:.2e}")
    assert eo < 1e-5 and es < 1e-5 and eb < 2e-5


def test_dplr_chunk_binding_gives_kda():
    """Section 3's binding through the chunkwise DPLR kernels against libkda's
    KDA prefill (bf16 tokens, both chunkwise)."""
    B, T, H, d = 1, 2100, 4, 128
    x = ki.prefill_inputs(B, T, H, d, d, torch.bfloat16, seed=23, device=DEV, s0_var=0.01)
    alpha = torch.exp(ki.G_MIN * torch.sigmoid(x["z"].double()))
    bk = (x["beta"].double()[..., None] * x["k"].double()).to(torch.bfloat16).contiguous()
    b = (x["k"].double() * alpha).to(torch.bfloat16).contiguous()
    o1, s1 = kda.dplr_chunk_fwd(x["q"], bk, x["v"], x["z"], bk, b, ki.G_MIN, x["s0"])
    o2, s2 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"])
    torch.cuda.synchronize()
    eo, es = rel(f64(o1), f64(o2)), rel(f64(s1), f64(s2))
    print(f"chunk binding: o {eo:.2e} state {es:.2e}")
    assert eo < 2e-2 and es < 1e-2


@pytest.mark.parametrize("T", [150, 2100])
def test_dplr_chunk_nan_workspace(T):
    """Every workspace byte the kernels read is written first in the same
    call: a NaN-filled workspace gives the same bits as a fresh one."""
    x = inputs(1, T, 2, 128, 128, torch.bfloat16, seed=37)
    need = kda.dplr_chunk_fwd_workspace_bytes(1, T, 2, 128, 128, torch.bfloat16)
    ws = torch.full((need // 4 + 1,), float("nan"), dtype=torch.float32, device=DEV)
    o1, s1 = gpu_chunk(x, workspace=ws.view(torch.uint8))
    o2, s2 = gpu_chunk(x)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_dplr_chunk_full_size_sampled():
    """The 32-head, 32768-token bf16 prefill through the chunkwise kernels
    (two-level plan, 32 segments): two heads against the oracle."""
    B, T, H, d = 1, 32768, 32, 128
    x = inputs(B, T, H, d, d, torch.bfloat16, seed=5)
    o, s = gpu_chunk(x)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    heads = [0, 31]
    ro, rs = oracle_of(x, heads=heads)
    go, gs = f64(o[:, :, heads]), f64(s[:, heads])
    eo, es, eb = rel(go, ro), rel(gs, rs), block_rel_max(go, ro)
    print(f"dplr chunk full size: o {eo:.2e} state {es:.2e} worst block {eb:.2e}")
    assert eo < 2e-2 and es < 1e-2 and eb < 4e-2


def test_dplr_chunk_deterministic():
    x = inputs(1, 2100, 4, 128, 128, torch.bfloat16, seed=39)
    o1, s1 = gpu_chunk(x)
    o2, s2 = gpu_chunk(x)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)

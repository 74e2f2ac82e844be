"""GPU parity of kda_chunk_bwd (gradients of the recurrence by 64-token chunks)
against the fp64 oracle's gradients (oracle/backward.py, pinned against finite
differences of the forward oracle).

Bars (relative Frobenius error per gradient), fixed before the first run:
  * fp32 tokens (d_v = 64, every product on fp32 MFMA): 1e-5, the fp32 bar of
    the forward and of kda_recurrent_bwd;
  * bf16 tokens: 2e-2, the bf16 bar of the forward's outputs.  The chunk
    recurrences then contract bf16-rounded operands (2^-9 relative) with fp32
    accumulation, as kda_chunk_fwd does, and every gradient inherits that
    rounding through sums of d terms.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from gated_delta_rule_14_amd import kda
from helpers import f64, host, rel
from oracle.backward import backward as oracle_backward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dz", "dbeta", "ds0")
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def grads_in(x, dtype, seed, with_dsf):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    B, T, H, dv = x["v"].shape
    dk = x["q"].shape[-1]
    do = torch.randn((B, T, H, dv), generator=g, device=DEV).to(dtype)
    dsf = torch.randn((B, H, dk, dv), generator=g, device=DEV) if with_dsf else None
    return do, dsf


def check(x, do, dsf, label, g_min=ki.G_MIN, heads=None, batches=None, tol=None):
    s0 = x.get("s0")
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, s0, do, dsf)
    torch.cuda.synchronize()
    bsel = slice(None) if batches is None else batches
    hsel = slice(None) if heads is None else heads

    def cut(t, hax):
        a = host(t)[bsel]
        idx = [slice(None)] * a.ndim
        idx[hax] = hsel
        return np.ascontiguousarray(a[tuple(idx)])

    ref = oracle_backward(cut(x["q"], 2), cut(x["k"], 2), cut(x["v"], 2), cut(x["z"], 2), cut(x["beta"], 2),
                          g_min, None if s0 is None else cut(s0, 1), cut(do, 2), None if dsf is None else cut(dsf, 1))
    errs = {}
    for n in NAMES:
        hax = 1 if n == "ds0" else 2
        gv = f64(got[n])[bsel]
        idx = [slice(None)] * gv.ndim
        idx[hax] = hsel
        errs[n] = rel(gv[tuple(idx)], ref[n])
    print(f"chunk bwd {label}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    bar = TOL[x["q"].dtype] if tol is None else tol
    assert max(errs.values()) < bar, errs
    return got


@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 150, 2, 64, 64), (2, 70, 1, 128, 64), (1, 64, 2, 64, 64),
                                         (1, 1, 1, 128, 64), (1, 300, 1, 128, 64)])
def test_chunk_bwd_f32(B, T, H, dk, dv):
    x = ki.prefill_inputs(B, T, H, dk, dv, torch.float32, seed=T + dk, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, torch.float32, seed=T, with_dsf=True)
    check(x, do, dsf, f"f32 B={B} T={T} H={H} dk={dk} dv={dv}")


@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 150, 2, 128, 128), (2, 70, 1, 64, 128), (1, 65, 2, 128, 64),
                                         (1, 64, 1, 64, 64), (1, 1, 1, 128, 128), (1, 1000, 2, 128, 128)])
def test_chunk_bwd_bf16(B, T, H, dk, dv):
    x = ki.prefill_inputs(B, T, H, dk, dv, torch.bfloat16, seed=T + dk + 1, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, torch.bfloat16, seed=T + 1, with_dsf=True)
    check(x, do, dsf, f"bf16 B={B} T={T} H={H} dk={dk} dv={dv}")


def test_chunk_bwd_no_initial_state_no_final_gradient():
    x = ki.prefill_inputs(1, 130, 2, 128, 64, torch.float32, seed=5, device=DEV)
    x["s0"] = None
    do, _ = grads_in(x, torch.float32, seed=6, with_dsf=False)
    check(x, do, None, "f32 s0 = 0, grad_s_final = 0")


@pytest.mark.parametrize("g_min", [-0.5, -8.0])
def test_chunk_bwd_decay_range(g_min):
    """Up to the chunkwise decay bound, where the block factors reach 2^92."""
    x = ki.prefill_inputs(1, 260, 2, 128, 64, torch.float32, seed=21, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, torch.float32, seed=22, with_dsf=True)
    check(x, do, dsf, f"f32 g_min={g_min}", g_min=g_min)


def test_chunk_bwd_long_memory():
    """z ~ N(-6, 1): alpha near 1, the gradients reach back over 1000 tokens."""
    x = ki.prefill_inputs(1, 1000, 1, 64, 64, torch.float32, seed=23, device=DEV, z_mean=-6.0, s0_var=0.01)
    do, dsf = grads_in(x, torch.float32, seed=24, with_dsf=True)
    check(x, do, dsf, "f32 z ~ N(-6,1), T=1000")


def test_chunk_bwd_token_kernel_cases():
    """fp32 tokens with d_v = 128, and g_min below the chunkwise bound, run the
    token-sequential kernel: the same bits as kda_recurrent_bwd."""
    for dtype, dv, g_min in ((torch.float32, 128, ki.G_MIN), (torch.bfloat16, 128, -9.0)):
        x = ki.prefill_inputs(1, 100, 2, 128, dv, dtype, seed=25, device=DEV, s0_var=0.01)
        do, dsf = grads_in(x, dtype, seed=26, with_dsf=True)
        a = kda.chunk_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, x["s0"], do, dsf)
        b = kda.recurrent_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, x["s0"], do, dsf)
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(a[n], b[n]), (dtype, n)


def test_chunk_bwd_empty_sequence():
    x = ki.prefill_inputs(2, 0, 2, 64, 64, torch.bfloat16, seed=9, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, torch.bfloat16, seed=9, with_dsf=True)
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], do, dsf)
    torch.cuda.synchronize()
    assert torch.equal(got["ds0"], dsf)


def test_chunk_bwd_nan_workspace_and_determinism():
    """Every workspace byte the kernels read is written first in the same call."""
    x = ki.prefill_inputs(1, 200, 2, 128, 128, torch.bfloat16, seed=27, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, torch.bfloat16, seed=28, with_dsf=True)
    need = kda.chunk_bwd_workspace_bytes(1, 200, 2, 128, 128, torch.bfloat16)
    ws = torch.full((need // 4 + 1,), float("nan"), dtype=torch.float32, device=DEV).view(torch.uint8)
    a = kda.chunk_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], do, dsf, workspace=ws)
    b = kda.chunk_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], do, dsf)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_chunk_bwd_train_8x8k_sampled():
    """The training shape (B=8, T=8192, H=32, d=128, bf16) at full size, all
    256 chains launched; the oracle runs four sampled (batch, head) chains."""
    x = ki.workload_inputs("train_8x8k", seed=11, device=DEV)
    do, dsf = grads_in(x, torch.bfloat16, seed=11, with_dsf=True)
    check(x, do, dsf, "train_8x8k (batches 0, 7 x heads 0, 31)", heads=[0, 31], batches=[0, 7])

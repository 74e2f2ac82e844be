"""GPU parity of kda_recurrent_bwd (gradients of the recurrence) against the
fp64 oracle's gradients (oracle/backward.py, itself pinned against finite
differences of the forward oracle).

The kernel computes in fp32 from the exact token values (bf16 inputs are
widened exactly), so both dtypes share the fp32 bar of the forward: relative
Frobenius error below 1e-5 for every gradient.  The errors measured here,
up to 8192 tokens, are 1e-7 to 6e-7: fp32 rounding (2^-24) through sums
of d terms, with no growth along the sequence, because the decay and the
unit-norm keys keep the state's propagation contractive.
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
TOL = 1e-5
NAMES = ("dq", "dk", "dv", "dz", "dbeta", "ds0")


def grads_in(x, dtype, seed, with_dsf):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    B, T, H, dv = x["v"].shape
    dk = x["q"].shape[-1]
    do = torch.randn((B, T, H, dv), generator=g, device=DEV).to(dtype)
    dsf = torch.randn((B, H, dk, dv), generator=g, device=DEV) if with_dsf else None
    return do, dsf


def check(x, do, dsf, label, heads=None, batches=None):
    s0 = x.get("s0")
    got = kda.recurrent_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, s0, do, dsf)
    torch.cuda.synchronize()
    bsel = slice(None) if batches is None else batches
    hsel = slice(None) if heads is None else heads

    def cut(t, hax):
        a = host(t)[bsel]
        idx = [slice(None)] * a.ndim
        idx[hax] = hsel
        return np.ascontiguousarray(a[tuple(idx)])

    ref = oracle_backward(cut(x["q"], 2), cut(x["k"], 2), cut(x["v"], 2), cut(x["z"], 2), cut(x["beta"], 2),
                          ki.G_MIN, None if s0 is None else cut(s0, 1), cut(do, 2),
                          None if dsf is None else cut(dsf, 1))
    errs = {}
    for n in NAMES:
        hax = 1 if n == "ds0" else 2
        gv = f64(got[n])[bsel]
        idx = [slice(None)] * gv.ndim
        idx[hax] = hsel
        errs[n] = rel(gv[tuple(idx)], ref[n])
    print(f"bwd {label}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    assert max(errs.values()) < TOL, errs
    return got


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 150, 2, 64, 64), (2, 70, 1, 128, 128), (1, 65, 2, 128, 64),
                                         (1, 64, 1, 64, 128), (1, 1, 1, 128, 128)])
def test_bwd_small(dtype, B, T, H, dk, dv):
    x = ki.prefill_inputs(B, T, H, dk, dv, dtype, seed=T + dk, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, dtype, seed=T, with_dsf=True)
    check(x, do, dsf, f"{dtype} B={B} T={T} H={H} dk={dk} dv={dv}")


def test_bwd_no_initial_state_no_final_gradient():
    x = ki.prefill_inputs(1, 130, 2, 128, 128, torch.bfloat16, seed=5, device=DEV)
    x["s0"] = None
    do, _ = grads_in(x, torch.bfloat16, seed=6, with_dsf=False)
    check(x, do, None, "s0 = 0, grad_s_final = 0")


def test_bwd_long_memory():
    """Slow decay (z ~ N(2, 1)) over 300 tokens: gradients reach far back."""
    x = ki.prefill_inputs(1, 300, 1, 128, 128, torch.bfloat16, seed=7, device=DEV, z_mean=2.0, s0_var=0.01)
    do, dsf = grads_in(x, torch.bfloat16, seed=8, with_dsf=True)
    check(x, do, dsf, "z ~ N(2,1), T=300")


def test_bwd_empty_sequence_and_determinism():
    x = ki.prefill_inputs(2, 0, 2, 64, 64, torch.float32, seed=9, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, torch.float32, seed=9, with_dsf=True)
    got = kda.recurrent_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], do, dsf)
    torch.cuda.synchronize()
    assert torch.equal(got["ds0"], dsf)
    x = ki.prefill_inputs(1, 200, 2, 128, 128, torch.bfloat16, seed=10, device=DEV, s0_var=0.01)
    do, dsf = grads_in(x, torch.bfloat16, seed=10, with_dsf=True)
    a = kda.recurrent_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], do, dsf)
    b = kda.recurrent_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], do, dsf)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_bwd_train_8x8k_sampled():
    """The training shape (B=8, T=8192, H=32, d=128, bf16) at full size, all
    256 chains launched; the oracle runs one sampled (batch, head) chain."""
    x = ki.workload_inputs("train_8x8k", seed=11, device=DEV)
    do, dsf = grads_in(x, torch.bfloat16, seed=11, with_dsf=True)
    check(x, do, dsf, "train_8x8k (batch 6, head 19)", heads=[19], batches=[6])

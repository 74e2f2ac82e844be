"""kda_chunk_fwd_noalloc, the variant of kda_chunk_fwd for callers that cannot
allocate: called through the C ABI, it must give kda_chunk_fwd's results bit
for bit on two calls in a row, the second one smaller (the static scratch
array keeps the first call's contents), and match the oracle."""
import pytest
import torch

import kda_inputs as ki
from gated_delta_rule_14_amd import kda
from helpers import TOL, f64, oracle_prefill, rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(x):
    args = (x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"])
    o1, s1 = kda.chunk_fwd(*args)
    o2, s2 = kda.chunk_fwd_noalloc(*args)
    torch.cuda.synchronize()
    return o1, s1, o2, s2


@pytest.mark.parametrize("dtype,tag", [(torch.bfloat16, "bf16"), (torch.float32, "f32")])
def test_noalloc_matches_chunk_fwd_twice(dtype, tag):
    # first call: segmented plan (compose, scan, expand with the T' hand-off
    # for bf16; per-chunk products for fp32); second call smaller, ragged
    for B, T, H in ((1, 4157, 3), (2, 700, 2)):
        x = ki.prefill_inputs(B, T, H, 128, 128, dtype, seed=T, device=DEV, s0_var=0.01)
        assert kda.chunk_fwd_workspace_bytes(B, T, H, 128, 128, dtype) <= kda.NOALLOC_SCRATCH_BYTES
        o1, s1, o2, s2 = _both(x)
        assert torch.equal(o1, o2) and torch.equal(s1, s2), (B, T, H)
        ro, rs = oracle_prefill(x)
        eo, es = rel(f64(o2), ro), rel(f64(s2), rs)
        print(f"noalloc {tag} B={B} T={T} H={H}: o {eo:.2e} state {es:.2e}")
        assert eo < TOL[tag][0] and es < TOL[tag][1]


def test_noalloc_full_prefill_shape_then_small():
    """The 32-head 32768-token bf16 prefill (176 MiB of scratch), then a small
    call: both bit-equal to kda_chunk_fwd."""
    x = ki.workload_inputs("prefill_32k", seed=1, device=DEV)
    o1, s1, o2, s2 = _both(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    del x, o1, s1, o2, s2
    x = ki.prefill_inputs(1, 1100, 2, 64, 64, torch.bfloat16, seed=3, device=DEV, s0_var=0.01)
    o1, s1, o2, s2 = _both(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_noalloc_rejects_oversize_without_launching():
    x = ki.prefill_inputs(1, 64, 64, 128, 128, torch.bfloat16, seed=4, device=DEV)
    # 64 heads of 32768 tokens need more than the static array: rejected on
    # the host (the pointers are never used), nothing written
    q = x["q"]
    lib = kda.lib()
    st = lib.kda_chunk_fwd_noalloc(
        kda._p(q), kda._p(q), kda._p(q), kda._p(q), kda._p(q), -5.0, None, kda._p(q), None,
        1, 32768, 64, 128, 128, 64, 1, kda._stream(q.device))
    assert st == 8, st

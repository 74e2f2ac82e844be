"""GPU parity of kda_out_gate (RMSNorm x sigmoid gate, optional projection)
and of the full layer against the fp64 oracle."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gated_delta_rule_14_amd import kda
from helpers import f64, host, rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def synth(B, T, H, dv, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    o = (torch.randn((B, T, H, dv), generator=g, device=DEV) * 0.3).to(dtype)
    gate = torch.randn((B, T, H, dv), generator=g, device=DEV).to(dtype)
    return o, gate


@pytest.mark.parametrize("dtype,tol", [(torch.float32, 1e-5), (torch.bfloat16, 2e-2)])
@pytest.mark.parametrize("dv", [64, 128])
def test_gate_no_projection(dtype, tol, dv):
    o, gate = synth(2, 37, 3, dv, dtype, 1)
    y = kda.out_gate(o, gate, ki.EPS)
    torch.cuda.synchronize()
    ref = oracle.out_gate(host(o), host(gate), ki.EPS)
    e = rel(f64(y), ref)
    print(f"gate dv={dv} {dtype}: {e:.2e}")
    assert y.shape == (2, 37, 3 * dv) and e < tol


@pytest.mark.parametrize("M_T,d_model", [(100, 48), (300, 272)])
def test_gate_projection_small(M_T, d_model):
    o, gate = synth(2, M_T, 4, 64, torch.bfloat16, 2)
    w = ki.projection(d_model, 4 * 64, seed=3, device=DEV)
    y = kda.out_gate(o, gate, ki.EPS, w)
    torch.cuda.synchronize()
    ref = oracle.out_gate(host(o), host(gate), ki.EPS, host(w))
    e = rel(f64(y), ref)
    print(f"gate+projection T={M_T} d_model={d_model}: {e:.2e}")
    assert y.shape == (2, M_T, d_model) and e < 2e-2


def test_layer_small_against_oracle_layer():
    x = ki.prefill_inputs(2, 90, 2, 64, 64, torch.bfloat16, seed=4, device=DEV, s0_var=0.01,
                          gate=True, d_model=96)
    res = kda.layer(x["q"], x["k"], x["v"], x["z"], x["beta"], x["gate"], x["w"], x["s0"], ki.G_MIN, ki.EPS)
    torch.cuda.synchronize()
    h = {n: host(t) for n, t in x.items()}
    ref = oracle.layer(h["q"], h["k"], h["v"], h["z"], h["beta"], h["gate"], h["w"], h["s0"], ki.G_MIN, ki.EPS)
    assert set(res) == {"outputs", "final_state"}
    assert res["outputs"].shape == (2, 90, 96) and res["outputs"].dtype == torch.bfloat16
    assert res["final_state"].shape == (2, 2, 64, 64)
    eo = rel(f64(res["outputs"]), ref["outputs"])
    es = rel(f64(res["final_state"]), ref["final_state"])
    print(f"layer: outputs {eo:.2e} final_state {es:.2e}")
    assert eo < 2e-2 and es < 1e-2


def test_train_8x8k_epilogue_projection_sampled_rows():
    """The training-shape epilogue at full size: (B=8, T=8192, H=32, d_v=128)
    outputs gated and projected to d_model = 2304 with W ~ N(0, 1/4096);
    oracle on 64 sampled (b, t) rows of the full launch."""
    B, T, H, dv, dm = 8, 8192, 32, 128, 2304
    o, gate = synth(B, T, H, dv, torch.bfloat16, 5)
    w = ki.projection(dm, H * dv, seed=5, device=DEV)
    y = kda.out_gate(o, gate, ki.EPS, w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(B * T, 64, replace=False))
    oh = host(o).reshape(B * T, H, dv)[rows][None]
    gh = host(gate).reshape(B * T, H, dv)[rows][None]
    ref = oracle.out_gate(np.ascontiguousarray(oh), np.ascontiguousarray(gh), ki.EPS, host(w))[0]
    e = rel(f64(y).reshape(B * T, dm)[rows], ref)
    print(f"train_8x8k epilogue + projection (64 rows): {e:.2e}")
    assert e < 2e-2


def test_train_8x8k_layer_sampled():
    """The training-shape layer end to end (chunkwise prefill, then the
    gate + projection to d_model = 2304): the oracle runs the recurrence for
    one sampled batch row (all 32 heads, all 8192 tokens) and the epilogue
    and projection on 32 sampled tokens of it."""
    x = ki.workload_inputs("train_8x8k", seed=6, device=DEV)
    res = kda.layer(x["q"], x["k"], x["v"], x["z"], x["beta"], x["gate"], x["w"], x["s0"], ki.G_MIN, ki.EPS)
    torch.cuda.synchronize()
    B, T, H, dv = x["v"].shape
    b = 5
    rng = np.random.default_rng(3)
    ts = np.sort(rng.choice(T, 32, replace=False))
    # oracle recurrence for batch b, all heads (needed for the projected rows), then epilogue on sampled tokens
    cut = {n: np.ascontiguousarray(host(x[n])[b:b + 1]) for n in ("q", "k", "v", "z", "beta")}
    ro, rs = oracle.forward(cut["q"], cut["k"], cut["v"], cut["z"], cut["beta"], ki.G_MIN, None)
    gh = np.ascontiguousarray(host(x["gate"])[b:b + 1, ts])
    ref = oracle.out_gate(np.ascontiguousarray(ro[:, ts]), gh, ki.EPS, host(x["w"]))
    e_out = rel(f64(res["outputs"])[b:b + 1, ts], ref)
    e_s = rel(f64(res["final_state"])[b:b + 1], rs)
    print(f"train_8x8k layer (batch {b}, 32 rows): outputs {e_out:.2e} final_state {e_s:.2e}")
    assert e_out < 2e-2 and e_s < 1e-2


# ------------------------------------------------------------------ projection GEMM
def _gemm_case(B, T, H, dv, dm, seed, rows=None):
    """kda_out_gate with the projection against numpy fp64 on the exact bf16
    gated rows kda_out_gate returns without it: isolates libkda's GEMM (fp32
    accumulation, output rounded to bf16).  rows: sampled row indices of the
    B*T rows (all rows when None).  Returns the relative error and the worst
    row's error against the matrix's average row."""
    o, gate = synth(B, T, H, dv, torch.bfloat16, seed)
    w = ki.projection(dm, H * dv, seed=seed, device=DEV)
    y = kda.out_gate(o, gate, ki.EPS)                  # (B, T, H*dv) bf16, no projection
    out = kda.out_gate(o, gate, ki.EPS, w)             # (B, T, dm)
    torch.cuda.synchronize()
    M = B * T
    yr = f64(y).reshape(M, H * dv)
    got = f64(out).reshape(M, dm)
    if rows is not None:
        yr, got = yr[rows], got[rows]
    ref = yr @ f64(w).T
    e = rel(got, ref)
    d = np.sqrt(((got - ref) ** 2).sum(axis=1))
    ew = float(d.max() / max(np.sqrt((ref ** 2).sum(axis=1)).mean(), 1e-300))
    return e, ew


@pytest.mark.parametrize("B,T,H,dv,dm", [
    (1, 1000, 8, 128, 512),      # 256 x 256 tiles, ragged last M tile
    (1, 1283, 4, 128, 384),      # 128 x 128 tiles (N a multiple of 128 only), ragged M
    (2, 1500, 2, 64, 272),       # 64 x 16 tiles (N = 17 * 16), ragged M
    (1, 256, 32, 128, 2304),     # decode batch: K split in eight, fp32 partials summed in order
    (1, 1024, 32, 128, 2304),    # the largest split-K M
    (1, 1025, 32, 128, 2304),    # the smallest whole-K M with ragged tiles
    (1, 3, 1, 64, 16),           # K = 64 (one stage), tiny M and N
])
def test_projection_gemm_shapes(B, T, H, dv, dm):
    e, ew = _gemm_case(B, T, H, dv, dm, seed=T + dm)
    print(f"projection GEMM M={B * T} K={H * dv} N={dm}: rel {e:.2e} worst row {ew:.2e}")
    assert e < 5e-3 and ew < 1e-2


def test_projection_gemm_full_training_shape():
    """M = 65,536 (8 x 8192), K = 4096, N = 2304: the training-shape
    projection at full size; 2048 rows sampled across all 256 M tiles."""
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(8 * 8192, 2048, replace=False))
    e, ew = _gemm_case(8, 8192, 32, 128, 2304, seed=9, rows=rows)
    print(f"projection GEMM 65536 x 4096 -> 2304 (2048 rows): rel {e:.2e} worst row {ew:.2e}")
    assert e < 5e-3 and ew < 1e-2


def test_projection_gemm_deterministic():
    o, gate = synth(1, 300, 32, 128, torch.bfloat16, 11)
    w = ki.projection(2304, 4096, seed=11, device=DEV)
    a = kda.out_gate(o, gate, ki.EPS, w)
    b = kda.out_gate(o, gate, ki.EPS, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

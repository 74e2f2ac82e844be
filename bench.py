"""Benchmark of the KDA operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode]

One step is one kda_chunk_fwd call over the 32k-token prefill workload
(B=1, T=32768, H=32, d_k=d_v=128, 64-token chunks, bf16 token tensors, fp32
state, S0 ~ N(0, 0.01)): gate, decay scan, intra-chunk products, triangular
solve, W/U, and the chunk-to-chunk state propagation with outputs.  Inputs
are generated on the GPU before timing and stay resident in HBM.

Also measured in the same run:
  * decode: kda_recurrent_step over B=256 sequences, H=32, d=128, fp32 state,
    1024 successive tokens (inputs for all steps pre-generated in HBM);
  * epilogue: RMSNorm x gate + projection of the training-shape workload
    (8 x 8192 tokens, 4096 -> 2304), against the bf16 MFMA peak;
  * cpu_baseline: the fp64 oracle on the host cores over the prefill
    workload (all heads over the full 32k tokens);
  * workloads: kda_chunk_fwd over the other prefill shapes -- the tiny fp32
    case (launch latency), the 8 x 8192 training shape, and the 1M-token
    sequence with the RMSNorm x gate epilogue (kda_chunk_layer_fwd, the
    epilogue inside the prefill kernels, timed beside kda_chunk_fwd +
    kda_out_gate) -- the training-shape layer with its projection
    (kda_chunk_layer_fwd, likewise), and the scalar-gate (Gated DeltaNet)
    prefill at the 32k shape;
  * backward: kda_chunk_bwd (the recurrence's gradients by 64-token chunks)
    on the 8 x 8192 training shape, beside kda_recurrent_bwd (token-sequential);
  * dplr: KDA against the general diagonal-plus-low-rank recurrence at the
    32k shape, and one decode step of each;
  * ceilings: what this GPU reaches -- libkda's streaming read-modify-write
    kernel, an in-place torch scale, a device copy and a large bf16 matmul --
    so that each kernel's rate can be read against them as well as against
    the published peaks.

Counter support: --copy-only runs a 1 GiB device copy for counter
calibration; --pmc-summary turns rocprofv3 FETCH_SIZE / WRITE_SIZE runs into
profiles/prefill_32k_traffic.json, which later runs report as `traffic`
while the kernel sources are unchanged.

Prints one JSON line.
"""
import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import glob
import hashlib

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA

PREFILL_BYTES_PER_TOKEN_HEAD = 4 * 128 * 2 + 2 + 128 * 2      # q, k, z, v in; beta; o out (bf16)
PREFILL_FLOP_PER_TOKEN_HEAD = 163840                           # chunk form, d = 128, C = 64
# The general DPLR chunk form (d = 128, C = 64, full tiles): four decayed C x C
# products 4 * 2Cd, Mbk V 2Cd, W = T R_B and U = T (Mbk V) 2 * 2Cd, then per
# token W S, (Q e^G) S 2 * 2d^2, [Mqk | Mqa][V; Y] 2 * 2C d and the state
# update [K~ | A~]^T [V; Y] 4 d^2.
DPLR_FLOP_PER_TOKEN_HEAD = 4 * 2 * 64 * 128 + 2 * 64 * 128 + 2 * 2 * 64 * 128 + 2 * 2 * 128 * 128 \
    + 2 * 2 * 64 * 128 + 4 * 128 * 128                        # 278,528
DECODE_BYTES_PER_HEAD_STEP = 2 * 128 * 128 * 4 + 4 * 128 * 2 + 2 + 128 * 2
DECODE_FLOP_PER_HEAD_STEP = 114688
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_32k_traffic.json")
CSRC = os.path.join(ROOT, "gated_delta_rule_14_amd", "csrc")


# the sources of the kernels whose counters the traffic record holds (the
# prefill's pipelined kernels and segment scan, the decode step, the gate
# kernel, the projection GEMM) and the device header they include
TRAFFIC_SOURCES = ("seg.hip", "decode.hip", "out_gate.hip", "gemm.hip", "kda_device.hpp")


def kernel_source_hash():
    """Hash of the measured kernels' sources with comments and blank lines
    removed, so that the stored counters stay attached to the code they were
    taken on."""
    import re
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        text = open(os.path.join(CSRC, name), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--decode-steps", type=int, default=1024)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=32)
    p.add_argument("--no-epilogue", action="store_true")
    p.add_argument("--no-workloads", action="store_true", help="skip the tiny, training and 1M-token shapes")
    p.add_argument("--no-long", action="store_true", help="skip the 1M-token shape")
    p.add_argument("--no-ceilings", action="store_true")
    p.add_argument("--no-dplr", action="store_true", help="skip the KDA vs general DPLR comparison")
    p.add_argument("--no-backward", action="store_true", help="skip the 8x8192 backward")
    p.add_argument("--copy-only", action="store_true",
                   help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    p.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs of the prefill and of --copy-only "
                        "into profiles/prefill_32k_traffic.json")
    return p.parse_args()


def bench_prefill(torch, kda, ki, steps, warmup):
    cfg = ki.WORKLOADS["prefill_32k"]
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    dev = torch.device("cuda:0")
    x = ki.workload_inputs("prefill_32k", seed=1, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    s = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(B, T, H, dk, dv, torch.bfloat16), dtype=torch.uint8,
                     device=dev)

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], o=o, s_final=s,
                      workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) * 1e-3 for a, b in ev]
    mean = sum(per) / len(per)
    tok = B * T
    bytes_alg = B * T * H * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * B * H * dk * dv * 4
    flop_alg = B * T * H * PREFILL_FLOP_PER_TOKEN_HEAD
    return dict(wall=wall, mean=mean, tokens=tok, bytes=bytes_alg, flop=flop_alg, B=B, T=T, H=H, dk=dk, dv=dv)


def bench_decode(torch, kda, ki, nsteps):
    cfg = ki.WORKLOADS["decode_256"]
    B, H, dk, dv = cfg["B"], cfg["H"], cfg["dk"], cfg["dv"]
    dev = torch.device("cuda:0")
    state = ki.initial_state(B, H, dk, dv, cfg["s0_var"], seed=3, device=dev)
    steps = [ki.decode_step_inputs(B, H, dk, dv, torch.bfloat16, 3, t, dev) for t in range(nsteps)]
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)
    for d in steps[:4]:
        kda.recurrent_step(d["q"], d["k"], d["v"], d["z"], d["beta"], ki.G_MIN, state, o=o)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for d in steps:
        kda.recurrent_step(d["q"], d["k"], d["v"], d["z"], d["beta"], ki.G_MIN, state, o=o)
    b.record()
    torch.cuda.synchronize()
    total = a.elapsed_time(b) * 1e-3
    per = total / nsteps
    bytes_step = B * H * DECODE_BYTES_PER_HEAD_STEP
    gbs = bytes_step / per / 1e9
    layer = bench_decode_layer(torch, kda, ki, state, steps[:min(nsteps, 256)], B, H, dv)
    return {
        "workload": "decode_256", "B": B, "H": H, "dk": dk, "dv": dv, "steps": nsteps,
        "value": B * nsteps / total, "unit": "tokens/s", "us_per_step": per * 1e6,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode"),
                     "algorithmic_bytes": bytes_step, "kernel": "decode_step_kernel"},
        "layer_step": layer,
    }


def bench_decode_layer(torch, kda, ki, state, steps, B, H, dv, d_model=2304):
    """The whole layer per decode token (recurrence step, RMSNorm x gate,
    projection to d_model): kda_recurrent_layer_step (epilogue fused into the
    step's launch, then the GEMM) against kda_recurrent_step followed by
    kda_out_gate (three launches)."""
    dev = torch.device("cuda:0")
    gates = [ki.gate_logits((B, H), dv, torch.bfloat16, 3, dev, step=t + 1) for t in range(len(steps))]
    w = ki.projection(d_model, H * dv, 3, dev)
    y = torch.empty((B, d_model), dtype=torch.bfloat16, device=dev)
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)
    lws = torch.empty(kda.recurrent_layer_step_workspace_bytes(B, H, dv, d_model, torch.bfloat16, True),
                      dtype=torch.uint8, device=dev)
    gws = torch.empty(kda.out_gate_workspace_bytes(B, 1, H, dv, d_model, torch.bfloat16, True), dtype=torch.uint8,
                      device=dev)

    def fused():
        for d, g in zip(steps, gates):
            kda.recurrent_layer_step(d["q"], d["k"], d["v"], d["z"], d["beta"], ki.G_MIN, state, g, ki.EPS, w, y=y,
                                     workspace=lws)

    def unfused():
        for d, g in zip(steps, gates):
            kda.recurrent_step(d["q"], d["k"], d["v"], d["z"], d["beta"], ki.G_MIN, state, o=o)
            kda.out_gate(o.view(B, 1, H, dv), g.view(B, 1, H, dv), ki.EPS, w, y=y.view(B, 1, d_model),
                         workspace=gws)

    n = len(steps)
    t_f = _time_calls(torch, fused, 1) / n
    t_u = _time_calls(torch, unfused, 1) / n
    return {"d_model": d_model, "steps": n, "us_per_step_fused": round(t_f * 1e6, 1),
            "us_per_step_unfused": round(t_u * 1e6, 1),
            "kernels": "fused: decode_step_kernel with the gate epilogue + split-K proj_gemm_kernel<256,128> "
                       "+ split_sum_kernel; unfused: decode_step_kernel + gate_kernel + the same GEMM"}


def bench_epilogue(torch, kda, ki, steps=5):
    """RMSNorm x gate + projection of the training-shape workload:
    (8, 8192, 32, 128) -> (8, 8192, 2304) bf16; the projection is the only
    MFMA-bound part of the path."""
    cfg = ki.WORKLOADS["train_8x8k"]
    B, T, H, dv, dm = cfg["B"], cfg["T"], cfg["H"], cfg["dv"], cfg["d_model"]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    o = (torch.randn((B, T, H, dv), generator=g, device=dev) * 0.3).to(torch.bfloat16)
    gate = ki.gate_logits((B, T, H), dv, torch.bfloat16, 5, dev)
    w = ki.projection(dm, H * dv, 5, dev)
    y = torch.empty((B, T, dm), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(kda.out_gate_workspace_bytes(B, T, H, dv, dm, torch.bfloat16, True), dtype=torch.uint8,
                     device=dev)
    for _ in range(2):
        kda.out_gate(o, gate, ki.EPS, w, y=y, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        kda.out_gate(o, gate, ki.EPS, w, y=y, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    per = a.elapsed_time(b) * 1e-3 / steps
    flop = 2.0 * B * T * H * dv * dm
    tf = flop / per / 1e12
    # the gate kernel alone (no projection), and a vendor GEMM on the same
    # gated rows for comparison (torch's F.linear: y W^T on hipBLASLt); the
    # comparison is context only, nothing of libkda runs on it
    yg = torch.empty((B, T, H * dv), dtype=torch.bfloat16, device=dev)
    t_gate = _time_calls(torch, lambda: kda.out_gate(o, gate, ki.EPS, y=yg), steps)
    y2 = yg.view(B * T, H * dv)
    t_vendor = _time_calls(torch, lambda: torch.nn.functional.linear(y2, w), steps)
    t_gemm = per - t_gate
    return {"workload": "train_8x8k epilogue", "M": B * T, "K": H * dv, "N": dm, "us_per_call": round(per * 1e6, 1),
            "value": round(B * T / per, 1), "unit": "tokens/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": "gate_kernel + proj_gemm_kernel<256,256> (projection FLOP only)"},
            "gate_us": round(t_gate * 1e6, 1), "gemm_us": round(t_gemm * 1e6, 1),
            "gemm_tflops": round(flop / t_gemm / 1e12, 1), "gemm_frac": round(flop / t_gemm / 1e12 / BF16_PEAK_TFLOPS, 4),
            "vendor_gemm_us_for_comparison": round(t_vendor * 1e6, 1)}


def _time_calls(torch, fn, calls, warmup=1):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(calls):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / calls


def bench_workload(torch, kda, ki, name, seed, calls):
    """One kda_chunk_fwd call over a named prefill workload, or where the
    workload has the RMSNorm x gate epilogue (no projection) one
    kda_chunk_layer_fwd call (raw outputs not kept), timed beside
    kda_chunk_fwd + kda_out_gate; inputs resident in HBM.  Algorithmic bytes:
    the token tensors once each, S0 read when it is given, S_final written;
    the gate workload counts its gate logits read and y written in place of
    o."""
    cfg = ki.WORKLOADS[name]
    B, T, H, dk, dv, dt = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"], cfg["dtype"]
    dev = torch.device("cuda:0")
    x = ki.workload_inputs(name, seed=seed, device=dev)
    s0 = x["s0"] if cfg["s0_var"] > 0 else None
    gate = cfg.get("epilogue") == "gate"
    o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    s = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kda.chunk_fwd_workspace_bytes(B, T, H, dk, dv, dt), 16), dtype=torch.uint8, device=dev)
    y = torch.empty((B, T, H * dv), dtype=dt, device=dev) if gate else None
    lws = None
    if gate:
        need = kda.chunk_layer_fwd_workspace_bytes(B, T, H, dk, dv, 0, dt, False)
        lws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def call():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, s0, o=o, s_final=s, workspace=ws)
        if gate:
            kda.out_gate(o, x["gate"], ki.EPS, y=y)

    def layer_call():
        kda.chunk_layer_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["gate"], ki.EPS, None, s0,
                            y=y, s_final=s, workspace=lws)

    per = _time_calls(torch, layer_call if gate else call, calls)
    esz = 2 if dt == torch.bfloat16 else 4
    per_th = (3 * dk + 2 * dv) * esz + esz + (dv * esz if gate else 0)   # q, k, z, v, o or y (+ gate); beta
    nbytes = B * T * H * per_th + B * H * dk * dv * 4 * (2 if s0 is not None else 1)
    out = {"workload": name, "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
           "dtype": "bf16" if dt == torch.bfloat16 else "f32", "calls": calls,
           "us_per_call": round(per * 1e6, 1), "value": round(B * T / per, 1), "unit": "tokens/s",
           "kernels": "kda_chunk_layer_fwd (epilogue in the prefill kernels)" if gate else "kda_chunk_fwd"}
    if gate:
        out["us_per_call_two_calls"] = round(_time_calls(torch, call, calls) * 1e6, 1)
    if dk == 128 and dv == 128:
        gbs = nbytes / per / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes,
                           "mfma_frac": round(B * T * H * PREFILL_FLOP_PER_TOKEN_HEAD / per / 1e12 /
                                              BF16_PEAK_TFLOPS, 4)}
    del x, o, s, ws, y, lws
    torch.cuda.empty_cache()
    return out


def bench_train_layer(torch, kda, ki, calls=5):
    """The training-shape layer end to end (8 x 8192 tokens, H = 32, d = 128:
    chunkwise prefill, RMSNorm x gate, projection 4096 -> 2304) as one
    kda_chunk_layer_fwd call (raw outputs not kept), beside kda_chunk_fwd +
    kda_out_gate."""
    cfg = ki.WORKLOADS["train_8x8k"]
    B, T, H, dk, dv, dm = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"], cfg["d_model"]
    dev = torch.device("cuda:0")
    x = ki.workload_inputs("train_8x8k", seed=2, device=dev)
    s0 = x["s0"] if cfg["s0_var"] > 0 else None
    y = torch.empty((B, T, dm), dtype=torch.bfloat16, device=dev)
    s = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    lws = torch.empty(max(kda.chunk_layer_fwd_workspace_bytes(B, T, H, dk, dv, dm, torch.bfloat16, True), 16),
                      dtype=torch.uint8, device=dev)
    per = _time_calls(torch, lambda: kda.chunk_layer_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN,
                                                         x["gate"], ki.EPS, x["w"], s0, y=y, s_final=s,
                                                         workspace=lws), calls)
    del lws
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    cws = torch.empty(max(kda.chunk_fwd_workspace_bytes(B, T, H, dk, dv, torch.bfloat16), 16), dtype=torch.uint8,
                      device=dev)
    gws = torch.empty(kda.out_gate_workspace_bytes(B, T, H, dv, dm, torch.bfloat16, True), dtype=torch.uint8,
                      device=dev)

    def two():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, s0, o=o, s_final=s, workspace=cws)
        kda.out_gate(o, x["gate"], ki.EPS, x["w"], y=y, workspace=gws)

    per2 = _time_calls(torch, two, calls)
    del x, y, s, o, cws, gws
    torch.cuda.empty_cache()
    return {"workload": "train_8x8k layer", "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "d_model": dm,
            "dtype": "bf16", "calls": calls, "us_per_call": round(per * 1e6, 1), "value": round(B * T / per, 1),
            "unit": "tokens/s", "us_per_call_two_calls": round(per2 * 1e6, 1),
            "kernels": "kda_chunk_layer_fwd (epilogue in the prefill kernels, then libkda's projection GEMM)"}


def bench_backward(torch, kda, ki, calls=2):
    """The gradients with respect to q, k, v, z, beta and S0 for given
    gradients of o and S_final on the training shape (B=8, T=8192, H=32,
    d=128, bf16 tokens): kda_chunk_bwd (chunkwise, MFMA) and, beside it,
    kda_recurrent_bwd (token-sequential).  Algorithmic bytes per token-head:
    the token inputs and the output gradient (bf16, 5 x 256 + 2) and the fp32
    gradients written (4 x 512 + 4)."""
    cfg = ki.WORKLOADS["train_8x8k"]
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    dev = torch.device("cuda:0")
    x = ki.workload_inputs("train_8x8k", seed=2, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    do = torch.randn((B, T, H, dv), generator=g, device=dev).to(torch.bfloat16)
    dsf = torch.randn((B, H, dk, dv), generator=g, device=dev)
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(B, T, H, dk, dv, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    per = _time_calls(torch, lambda: kda.chunk_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, None,
                                                   do, dsf, workspace=ws), 5)
    ws_bytes = ws.numel()
    del ws
    ws = torch.empty(kda.recurrent_bwd_workspace_bytes(B, T, H, dk, dv), dtype=torch.uint8, device=dev)
    per_seq = _time_calls(torch, lambda: kda.recurrent_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN,
                                                           None, do, dsf, workspace=ws), calls)
    nbytes = B * T * H * (5 * 256 + 2 + 4 * 512 + 4) + 2 * B * H * dk * dv * 4
    gbs = nbytes / per / 1e9
    del x, do, dsf, ws
    torch.cuda.empty_cache()
    return {"workload": "train_8x8k backward", "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "dtype": "bf16",
            "calls": 5, "us_per_call": round(per * 1e6, 1), "value": round(B * T / per, 1), "unit": "tokens/s",
            "kernels": "kda_chunk_bwd (chunk_intra_kernel, chain_kernel storing states, dchain_kernel, "
                       "dintra16_kernel)",
            "workspace_bytes": ws_bytes,
            "token_sequential_us_per_call": round(per_seq * 1e6, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes}}


def bench_gdn_prefill(torch, kda, ki, calls=10):
    """The scalar-gate (Gated DeltaNet) prefill at the 32k shape: z is one
    logit per (token, head), which the pipelined prefill kernels read
    directly (decay factors once per token).  Algorithmic bytes count z at
    2 B per token-head."""
    cfg = ki.WORKLOADS["prefill_32k"]
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    dev = torch.device("cuda:0")
    x = ki.workload_inputs("prefill_32k", seed=1, device=dev)
    zs = x["z"][..., 0].contiguous()
    del x["z"]
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    s = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    per = _time_calls(torch, lambda: kda.gdn_chunk_fwd(x["q"], x["k"], x["v"], zs, x["beta"], ki.G_MIN, x["s0"],
                                                       o=o, s_final=s, workspace=ws), calls)
    nbytes = B * T * H * ((2 * dk + 2 * dv) * 2 + 2 + 2) + 2 * B * H * dk * dv * 4
    gbs = nbytes / per / 1e9
    del x, zs, o, s, ws
    torch.cuda.empty_cache()
    return {"workload": "prefill_32k scalar gate (Gated DeltaNet)", "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
            "dtype": "bf16", "calls": calls, "us_per_call": round(per * 1e6, 1), "value": round(B * T / per, 1),
            "unit": "tokens/s", "kernels": "kda_gdn_chunk_fwd (pipe_first_kernel + scan_x3_kernel + pipe_last_kernel, scalar logit)",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes}}


def bench_dplr(torch, kda, ki, calls=5):
    """KDA against the general DPLR recurrence S = (Diag(alpha) - a b^T) S +
    k v^T with independent a, b, at the 32-head 32k-token bf16 prefill shape
    and the 256 x 32 decode batch: KDA's chunkwise prefill beside the
    chunkwise DPLR kernels (four decayed products per chunk where KDA has
    two, contractions over twice the tokens in the chunk step) and the
    token-sequential DPLR kernel; one decode step of each."""
    cfg = ki.WORKLOADS["prefill_32k"]
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    bf = torch.bfloat16
    dev = torch.device("cuda:0")
    s0 = ki.initial_state(B, H, dk, dv, cfg["s0_var"], seed=6, device=dev)
    o = torch.empty((B, T, H, dv), dtype=bf, device=dev)
    s = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    x = ki.prefill_inputs(B, T, H, dk, dv, bf, seed=6, device=dev)
    ws = torch.empty(max(kda.chunk_fwd_workspace_bytes(B, T, H, dk, dv, bf), 16), dtype=torch.uint8, device=dev)
    kda_s = _time_calls(torch, lambda: kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, s0,
                                                     o=o, s_final=s, workspace=ws), calls)
    del x, ws
    x = ki.dplr_inputs((B, T, H), dk, dv, bf, seed=6, device=dev)
    args = [x[n] for n in ("q", "k", "v", "z", "a", "b")]
    ws = torch.empty(kda.dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, bf), dtype=torch.uint8, device=dev)
    chunk_s = _time_calls(torch, lambda: kda.dplr_chunk_fwd(*args, ki.G_MIN, s0, o=o, s_final=s, workspace=ws),
                          calls)
    ws_bytes = ws.numel()
    del ws
    seq_s = _time_calls(torch, lambda: kda.dplr_fwd(*args, ki.G_MIN, s0, o=o, s_final=s), 2)
    del x, args, o, s, s0
    torch.cuda.empty_cache()

    dcfg = ki.WORKLOADS["decode_256"]
    Bd = dcfg["B"]
    state = ki.initial_state(Bd, H, dk, dv, dcfg["s0_var"], seed=7, device=dev)
    od = torch.empty((Bd, H, dv), dtype=bf, device=dev)
    d = ki.decode_step_inputs(Bd, H, dk, dv, bf, 7, 0, dev)
    kda_step = _time_calls(torch, lambda: kda.recurrent_step(d["q"], d["k"], d["v"], d["z"], d["beta"], ki.G_MIN,
                                                             state, o=od), 50, warmup=5)
    dd = ki.dplr_inputs((Bd, H), dk, dv, bf, seed=7, device=dev, step=1)
    dargs = [dd[n] for n in ("q", "k", "v", "z", "a", "b")]
    dplr_step = _time_calls(torch, lambda: kda.dplr_recurrent_step(*dargs, ki.G_MIN, state, o=od), 50, warmup=5)
    del state, od, d, dd, dargs
    torch.cuda.empty_cache()
    tokens = B * T
    # token tensors once each (bf16): KDA q, k, z, v, beta, o; DPLR q, k, z, a, b, v, o
    kda_bytes = tokens * H * (5 * 256 + 2) + 2 * B * H * dk * dv * 4
    dplr_bytes = tokens * H * 7 * 256 + 2 * B * H * dk * dv * 4
    return {
        "workload": "prefill_32k shape, KDA vs general DPLR", "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
        "dtype": "bf16",
        "kda_chunk_us": round(kda_s * 1e6, 1), "kda_tokens_per_s": round(tokens / kda_s, 1),
        "dplr_chunk_us": round(chunk_s * 1e6, 1), "dplr_chunk_tokens_per_s": round(tokens / chunk_s, 1),
        "dplr_seq_us": round(seq_s * 1e6, 1), "dplr_seq_tokens_per_s": round(tokens / seq_s, 1),
        "dplr_chunk_over_kda_time": round(chunk_s / kda_s, 3),
        "flop_per_token_head": {"kda": PREFILL_FLOP_PER_TOKEN_HEAD, "dplr": DPLR_FLOP_PER_TOKEN_HEAD},
        "algorithmic_bytes": {"kda": kda_bytes, "dplr": dplr_bytes},
        "dplr_chunk_hbm_gbs": round(dplr_bytes / chunk_s / 1e9, 1),
        "dplr_chunk_mfma_frac": round(tokens * H * DPLR_FLOP_PER_TOKEN_HEAD / chunk_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        "dplr_chunk_workspace_bytes": ws_bytes,
        "decode_step_us": {"kda": round(kda_step * 1e6, 1), "dplr": round(dplr_step * 1e6, 1)},
        "kernels": "kda_chunk_fwd (pipe_first_kernel, scan_x3_kernel, pipe_last_kernel); kda_dplr_chunk_fwd (dplr_intra_kernel, "
                   "dplr_chain_kernel x3, seg_scan_kernel); kda_dplr_fwd (dplr_seq_kernel); "
                   "decode_step_kernel vs dplr_step_kernel",
    }


def measured_ceilings(torch, kda):
    """Rates this GPU reaches: libkda's streaming read-modify-write kernel
    (kda_stream_scale: in-place fp32 scale over 512 MiB, the decode state's
    access pattern; every variant, the best kept), the same through torch's
    x.mul_, a 512 MiB device copy, and a bf16 8192^3 matmul."""
    dev = torch.device("cuda:0")
    n = 128 * 1024 * 1024
    x = torch.ones(n, dtype=torch.float32, device=dev)
    best = (0.0, None)
    for var in [u | (nt << 2) | (w << 3) for u in range(4) for nt in (0, 1) for w in (0, 8)]:
        t = _time_calls(torch, lambda: kda.stream_scale(x, 0.999999, var), 10, warmup=3)
        best = max(best, (2 * n * 4 / t / 1e9, var))
    t_rmw = _time_calls(torch, lambda: x.mul_(0.999999), 10, warmup=3)
    d = torch.empty_like(x)
    t_copy = _time_calls(torch, lambda: d.copy_(x), 10, warmup=3)
    del x, d
    m = 8192
    a = torch.randn((m, m), device=dev).to(torch.bfloat16)
    b = torch.randn((m, m), device=dev).to(torch.bfloat16)
    t_mm = _time_calls(torch, lambda: torch.matmul(a, b), 10, warmup=3)
    del a, b
    torch.cuda.empty_cache()
    v = best[1]
    return {"hbm_rmw_hip_gbs": round(best[0], 1),
            "hbm_rmw_hip_variant": {"float4_per_thread": 1 << (v & 3), "nontemporal": bool(v & 4),
                                    "waves_per_cu": (v >> 3) or "one pass"},
            "hbm_rmw_gbs": round(2 * n * 4 / t_rmw / 1e9, 1), "hbm_copy_gbs": round(2 * n * 4 / t_copy / 1e9, 1),
            "mfma_bf16_tflops": round(2 * m ** 3 / t_mm / 1e12, 1),
            "how": "kda_stream_scale (HIP, 16 variants, best kept) and torch x.mul_ in place over 512 MiB fp32, "
                   "torch copy_ (512 MiB), torch.matmul bf16 8192^3; HIP events, mean of 10 after 3 warm-up calls"}


def copy_only(torch):
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": src.numel(), "calls": 3}), flush=True)


def _pmc_per_dispatch(path, counter):
    import csv
    import collections
    acc = collections.defaultdict(float)
    n = collections.Counter()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = r["Kernel_Name"]
        acc[k] += float(r["Counter_Value"])
        n[(k, r["Dispatch_Id"])] += 1
    disp = collections.Counter(k for (k, _) in n)
    return {k: acc[k] / disp[k] for k in acc}


def pmc_summary(fetch_csv, write_csv, cfetch_csv, cwrite_csv):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the prefill kernels,
    scaled by what the same counters read for a 1 GiB device copy."""
    f = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    wr = _pmc_per_dispatch(write_csv, "WRITE_SIZE")
    cf = _pmc_per_dispatch(cfetch_csv, "FETCH_SIZE")
    cw = _pmc_per_dispatch(cwrite_csv, "WRITE_SIZE")
    copy_k = max(cf, key=cf.get)
    true_kib = (1 << 30) / 1024.0
    sf, sw = true_kib / cf[copy_k], true_kib / cw[max(cw, key=cw.get)]
    kernels = {}
    for k in sorted(set(f) | set(wr)):
        if "kda" not in k:
            continue
        kernels[k] = {"fetch_kib": round(f.get(k, 0.0), 1), "write_kib": round(wr.get(k, 0.0), 1),
                      "hbm_bytes": round((f.get(k, 0.0) * sf + wr.get(k, 0.0) * sw) * 1024)}
    out = {"source_hash": kernel_source_hash(), "copy_fetch_scale": round(sf, 4), "copy_write_scale": round(sw, 4),
           "copy_kernel": copy_k, "kernels": kernels,
           "prefill_hbm_bytes_per_call": sum(v["hbm_bytes"] for k, v in kernels.items()
                                             if "pipe_" in k or "seg_kernel" in k or "scan_x3" in k
                                             or "seg_scan" in k or "chunk_intra" in k or "chain_kernel" in k),
           "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -f csv -- python bench.py --no-cpu --steps 2 "
                      "--warmup 1 --decode-steps 8 --no-epilogue --no-workloads --no-ceilings --no-dplr --no-backward; same with "
                      "--copy-only for the "
                      "scale factors"}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))


def measured_traffic(which):
    """HBM bytes per prefill call ("prefill") or per decode step ("decode")
    from the committed counter summary, or None when the kernels have changed
    since the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    if which == "prefill":
        return t.get("prefill_hbm_bytes_per_call")
    for k, v in t.get("kernels", {}).items():
        if "decode_step_kernel" in k:
            return v["hbm_bytes"]
    return None


def cpu_baseline(torch, ki, nheads):
    import numpy as np

    import oracle
    cfg = ki.WORKLOADS["prefill_32k"]
    T, H = cfg["T"], cfg["H"]
    x = ki.workload_inputs("prefill_32k", seed=1, device="cuda:0")
    heads = list(range(nheads))
    h = {n: np.ascontiguousarray(ki.to_host_bits(x[n])[:, :, heads]) for n in ("q", "k", "v", "z", "beta")}
    s0 = np.ascontiguousarray(ki.to_host_bits(x["s0"])[:, heads])
    del x
    share, logical, why = host_cpu_share()
    threads = share
    t0 = time.perf_counter()
    oracle.forward(h["q"], h["k"], h["v"], h["z"], h["beta"], ki.G_MIN, s0, nthreads=threads)
    dt = time.perf_counter() - t0
    # a token is one (b, t) position over all H heads: scale the sample by nheads / H
    return {"value": T * nheads / H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"prefill_32k, {nheads} of {H} heads over all {T} tokens, fp64, {dt:.1f} s "
                      f"on {threads} threads ({dt * threads:.0f} s of CPU time)",
            "host_logical_cpus": logical, "cores_reason": why, "cpu_model": cpu_model()}


def host_cpu_share():
    """Threads the oracle may use: the CPUs this process is allowed to run on
    (its affinity mask), capped by OMP_NUM_THREADS when the host sets it (a
    shared host gives each GPU a share of its cores).  Returns (threads,
    logical CPUs of the host, how the count was reached)."""
    logical = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = logical
    why = f"{allowed} CPUs in this process's affinity mask of {logical} logical CPUs"
    share = allowed
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and 0 < int(omp) < share:
        share = int(omp)
        why += f", capped at the host's per-job share OMP_NUM_THREADS={omp}"
    return share, logical, why


def cpu_model():
    """The host CPU's model string, family/model/stepping and hypervisor, as
    lscpu and /proc/cpuinfo report them."""
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ":" in ln:
                k, v = ln.split(":", 1)
                info[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if "Model name" not in info:
        try:
            with open("/proc/cpuinfo") as f:
                info["Model name"] = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                                          "")
        except OSError:
            pass
    parts = [info.get("Vendor ID", ""), info.get("Model name", ""),
             f"family {info.get('CPU family', '?')} model {info.get('Model', '?')} stepping {info.get('Stepping', '?')}",
             f"{info.get('Socket(s)', '?')} socket(s) x {info.get('Core(s) per socket', '?')} cores x "
             f"{info.get('Thread(s) per core', '?')} threads"]
    if info.get("Hypervisor vendor"):
        parts.append(f"hypervisor {info['Hypervisor vendor']}")
    return ", ".join(p for p in parts if p)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the operator shards over (batch, head) chains with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import kda_inputs as ki
    from gated_delta_rule_14_amd import kda
    from gated_delta_rule_14_amd import _lib

    _lib.lib()
    if args.copy_only:
        copy_only(torch)
        return
    r = bench_prefill(torch, kda, ki, args.steps, args.warmup)
    tok_s = r["tokens"] / r["mean"]
    gbs = r["bytes"] / r["mean"] / 1e9
    line = {
        "metric": "KDA tokens/s (prefill T=32k,H=32,d=128; decode B=256) + % MFMA/HBM roofline",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["mean"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_32k", "B": r["B"], "T": r["T"], "H": r["H"], "dk": r["dk"],
                   "dv": r["dv"], "chunk": 64, "state": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("prefill"),
                     "algorithmic_bytes": r["bytes"],
                     "kernel": "kda_chunk_fwd: pipe_first_kernel (segment 0 expand + compose) + scan_x3_kernel + pipe_last_kernel (light expands + last segment expand)",
                     "mfma_frac": round(r["flop"] / r["mean"] / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_decode:
        line["decode"] = bench_decode(torch, kda, ki, args.decode_steps)
    if not args.no_epilogue:
        line["epilogue"] = bench_epilogue(torch, kda, ki)
    if not args.no_workloads:
        wl = [bench_workload(torch, kda, ki, "tiny_fp32", 0, 20),
              bench_workload(torch, kda, ki, "train_8x8k", 2, 5),
              bench_train_layer(torch, kda, ki)]
        wl.append(bench_gdn_prefill(torch, kda, ki))
        if not args.no_long:
            wl.append(bench_workload(torch, kda, ki, "long_1m", 4, 2))
        line["workloads"] = wl
    if not args.no_backward:
        line["backward"] = bench_backward(torch, kda, ki)
    if not args.no_dplr:
        line["dplr"] = bench_dplr(torch, kda, ki)
    if not args.no_ceilings:
        c = measured_ceilings(torch, kda)
        line["ceilings"] = c
        line["roofline"]["frac_of_measured_copy"] = round(gbs / c["hbm_copy_gbs"], 4)
        if "decode" in line:
            line["decode"]["roofline"]["frac_of_measured_rmw"] = round(
                line["decode"]["roofline"]["achieved"] / c["hbm_rmw_gbs"], 4)
            line["decode"]["roofline"]["frac_of_hip_rmw_ceiling"] = round(
                line["decode"]["roofline"]["achieved"] / c["hbm_rmw_hip_gbs"], 4)
        if "epilogue" in line:
            line["epilogue"]["roofline"]["frac_of_measured_matmul"] = round(
                line["epilogue"]["roofline"]["achieved"] / c["mfma_bf16_tflops"], 4)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(torch, ki, args.cpu_heads)
        line["cpu_baseline"]["gpu_over_oracle"] = round(line["value"] / line["cpu_baseline"]["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

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
  * cpu_baseline: the fp64 oracle on the host cores over a bounded sample of
    the prefill workload (a few heads over the full 32k tokens).

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA

PREFILL_BYTES_PER_TOKEN_HEAD = 4 * 128 * 2 + 2 + 128 * 2      # q, k, z, v in; beta; o out (bf16)
PREFILL_FLOP_PER_TOKEN_HEAD = 163840                           # chunk form, d = 128, C = 64
DECODE_BYTES_PER_HEAD_STEP = 2 * 128 * 128 * 4 + 4 * 128 * 2 + 2 + 128 * 2
DECODE_FLOP_PER_HEAD_STEP = 114688


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--decode-steps", type=int, default=1024)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=32)
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
    return {
        "workload": "decode_256", "B": B, "H": H, "dk": dk, "dv": dv, "steps": nsteps,
        "value": B * nsteps / total, "unit": "tokens/s", "us_per_step": per * 1e6,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }


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
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.forward(h["q"], h["k"], h["v"], h["z"], h["beta"], ki.G_MIN, s0, nthreads=threads)
    dt = time.perf_counter() - t0
    # a token is one (b, t) position over all H heads: scale the sample by nheads / H
    return {"value": T * nheads / H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"prefill_32k, {nheads} of {H} heads over all {T} tokens, fp64, {dt:.1f} s"}


def main():
    args = parse()
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
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "kda_chunk_fwd (intra + inter launches)",
                     "mfma_frac": round(r["flop"] / r["mean"] / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_decode:
        line["decode"] = bench_decode(torch, kda, ki, args.decode_steps)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(torch, ki, args.cpu_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

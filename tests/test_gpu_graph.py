"""libkda calls under HIP graph capture, the way a serving loop replays
them: nothing in the library allocates, synchronises or records memsets, so
a captured call must replay to the same bits as the eager call.  Each graph
is replayed several times with the program's own eager work and
synchronisations in between, and every replay is checked."""
import pytest
import torch

import kda_inputs as ki
from gated_delta_rule_14_amd import kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_decode_layer_step_graph_replays():
    B, H, d, dm = 32, 8, 128, 256
    steps = [ki.decode_step_inputs(B, H, d, d, torch.bfloat16, 51, t, DEV) for t in range(3)]
    gates = [ki.gate_logits((B, H), d, torch.bfloat16, 51, DEV, step=t + 1) for t in range(3)]
    w = ki.projection(dm, H * d, 51, DEV)
    state = ki.initial_state(B, H, d, d, 0.01, 51, DEV)
    ref_state = state.clone()
    y = torch.empty((B, dm), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(kda.recurrent_layer_step_workspace_bytes(B, H, d, dm, torch.bfloat16, True),
                     dtype=torch.uint8, device=DEV)
    # static input slots the graph reads; each replay copies the next token in
    slot = {n: torch.empty_like(t) for n, t in steps[0].items()}
    gslot = torch.empty_like(gates[0])

    def step():
        kda.recurrent_layer_step(slot["q"], slot["k"], slot["v"], slot["z"], slot["beta"], ki.G_MIN, state, gslot,
                                 ki.EPS, w, y=y, o=o, want_o=True, workspace=ws)

    # eager warm-up on a scratch state: creates the GEMM plan outside capture
    scratch = state.clone()
    for n in slot:
        slot[n].copy_(steps[0][n])
    gslot.copy_(gates[0])
    kda.recurrent_layer_step(slot["q"], slot["k"], slot["v"], slot["z"], slot["beta"], ki.G_MIN, scratch, gslot,
                             ki.EPS, w, y=y, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for t in range(3):
        for n in slot:
            slot[n].copy_(steps[t][n])
        gslot.copy_(gates[t])
        g.replay()
        torch.cuda.synchronize()
        got_y, got_o, got_s = y.clone(), o.clone(), state.clone()
        # the eager call on its own state, with eager work of the program between replays
        ry, ro = kda.recurrent_layer_step(steps[t]["q"], steps[t]["k"], steps[t]["v"], steps[t]["z"],
                                          steps[t]["beta"], ki.G_MIN, ref_state, gates[t], ki.EPS, w, want_o=True)
        torch.cuda.synchronize()
        assert torch.equal(got_s, ref_state), f"state after replay {t}"
        assert torch.equal(got_o, ro), f"read-out after replay {t}"
        assert torch.equal(got_y, ry), f"projected output after replay {t}"


def test_chunk_fwd_graph_replays():
    """The bf16 prefill with segments (compose, scan, expand) captured once:
    replays with new inputs copied into the static slots match eager calls."""
    B, T, H, d = 1, 4096, 4, 128
    xs = [ki.prefill_inputs(B, T, H, d, d, torch.bfloat16, 60 + i, DEV, s0_var=0.01) for i in range(3)]
    slot = {n: torch.empty_like(t) for n, t in xs[0].items()}
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=DEV)
    s = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(B, T, H, d, d, torch.bfloat16), dtype=torch.uint8, device=DEV)
    assert ws.numel() > 0     # several segments per chain: the two-level path

    def call():
        kda.chunk_fwd(slot["q"], slot["k"], slot["v"], slot["z"], slot["beta"], ki.G_MIN, slot["s0"], o=o,
                      s_final=s, workspace=ws)

    for n in slot:
        slot[n].copy_(xs[0][n])
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in (1, 2, 0):
        for n in slot:
            slot[n].copy_(xs[i][n])
        g.replay()
        torch.cuda.synchronize()
        got_o, got_s = o.clone(), s.clone()
        x = xs[i]
        ro, rs = kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"])
        torch.cuda.synchronize()
        assert torch.equal(got_o, ro) and torch.equal(got_s, rs), f"replay with inputs {i}"


def test_chunk_layer_fwd_graph_replays():
    """The prefill of the layer with the epilogue fused (segmented plan) and
    the projection, captured once: replays with new inputs copied into the
    static slots match eager calls."""
    B, T, H, d, dm = 1, 4096, 4, 128, 192
    xs = [ki.prefill_inputs(B, T, H, d, d, torch.bfloat16, 70 + i, DEV, s0_var=0.01, gate=True) for i in range(3)]
    w = ki.projection(dm, H * d, 70, DEV)
    slot = {n: torch.empty_like(t) for n, t in xs[0].items()}
    y = torch.empty((B, T, dm), dtype=torch.bfloat16, device=DEV)
    s = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
    ws = torch.empty(kda.chunk_layer_fwd_workspace_bytes(B, T, H, d, d, dm, torch.bfloat16, True),
                     dtype=torch.uint8, device=DEV)

    def call():
        kda.chunk_layer_fwd(slot["q"], slot["k"], slot["v"], slot["z"], slot["beta"], ki.G_MIN, slot["gate"],
                            ki.EPS, w, slot["s0"], y=y, s_final=s, workspace=ws)

    for n in slot:
        slot[n].copy_(xs[0][n])
    call()     # eager: creates the GEMM plan outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in (1, 2, 0):
        for n in slot:
            slot[n].copy_(xs[i][n])
        g.replay()
        torch.cuda.synchronize()
        got_y, got_s = y.clone(), s.clone()
        x = xs[i]
        ry, rs = kda.chunk_layer_fwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["gate"], ki.EPS, w,
                                     x["s0"])
        torch.cuda.synchronize()
        assert torch.equal(got_y, ry) and torch.equal(got_s, rs), f"replay with inputs {i}"


def test_recurrent_bwd_graph_replays():
    """The backward captured once (workspace given): replays with new inputs
    copied into the static slots match eager calls bit for bit."""
    B, T, H, d = 1, 150, 2, 64
    xs = [ki.prefill_inputs(B, T, H, d, d, torch.bfloat16, 80 + i, DEV, s0_var=0.01) for i in range(3)]
    g = torch.Generator(device=DEV)
    g.manual_seed(80)
    dos = [torch.randn((B, T, H, d), generator=g, device=DEV).to(torch.bfloat16) for _ in range(3)]
    slot = {n: torch.empty_like(t) for n, t in xs[0].items()}
    dslot = torch.empty_like(dos[0])
    ws = torch.empty(kda.recurrent_bwd_workspace_bytes(B, T, H, d, d), dtype=torch.uint8, device=DEV)
    out = {}

    def call():
        out.update(kda.recurrent_bwd(slot["q"], slot["k"], slot["v"], slot["z"], slot["beta"], ki.G_MIN,
                                     slot["s0"], dslot, workspace=ws))

    for n in slot:
        slot[n].copy_(xs[0][n])
    dslot.copy_(dos[0])
    call()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call()
    torch.cuda.synchronize()
    for i in (1, 2, 0):
        for n in slot:
            slot[n].copy_(xs[i][n])
        dslot.copy_(dos[i])
        gr.replay()
        torch.cuda.synchronize()
        got = {n: t.clone() for n, t in out.items()}
        x = xs[i]
        ref = kda.recurrent_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], ki.G_MIN, x["s0"], dos[i])
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(got[n], ref[n]), (n, i)

"""Graph capture: every entry point is a sequence of kernel launches on the
caller's stream (no allocation, no memset, no synchronisation inside the
library), so launch-bound steps can be captured once and replayed.  Two
steps are captured with torch's graph API: the forward (chunk states + SMA
with R and lse) and a decode step (decode against the cache, then the
decode-side update of the in-progress memory).  Each graph is replayed
several times, with eager work and synchronisations between the replays and
its outputs overwritten before each, and every replay must equal the eager
step bit for bit."""
import pytest
import torch

import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import same, say

pytestmark = pytest.mark.gpu


def capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    torch.cuda.synchronize()
    return g, outs


def test_forward_step_graph_replays():
    cfg = dict(batch=2, seqlen=2048, nheads=4, ngroups=4, chunk=256, d_state=128, d_head=64, dtype="bf16")
    S = cfg["chunk"]
    d = synth.draw_fwd_torch(**cfg, seed=31)
    other = synth.draw_fwd_torch(**cfg, seed=32)

    def step(x=d):
        dH = dart.dart_chunk_states(x["X"], x["B"], x["A"], S)
        out, R, lse = dart.dart_sma_fwd(x["Q"], x["C"], x["E"], dH, x["Y"], x["gate"], S, want_R=True,
                                        want_lse=True)
        return dH, out, R, lse

    eager = [t.clone() for t in step()]
    g, outs = capture(step)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        step(other)                       # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("dH", "out", "R", "lse"), eager, outs):
            same(x, y, f"forward graph replay {rep}: {name}")
    say("forward step: 3 graph replays equal the eager step")


def test_decode_step_graph_replays():
    b, H, G, Mx, S = 8, 4, 2, 16, 64
    dd = synth.draw_decode_torch(batch=b, nheads=H, ngroups=G, max_chunks=Mx, d_state=128, d_head=64, seed=33)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(34)
    x = torch.randn((b, H, 64), generator=gen, device="cuda").to(torch.bfloat16)
    Bt = (torch.randn((b, G, 128), generator=gen, device="cuda") / 11.3).to(torch.bfloat16)
    a = torch.rand((b, H), generator=gen, device="cuda") * 0.5 + 0.5
    # positions: some rows close a chunk with this token, one is padding
    pos = torch.tensor([5 * S - 1, 3 * S + 7, 63, 2 * S - 1, -1, 7 * S - 1, S, 11 * S + 2], dtype=torch.int32,
                       device="cuda")
    state0 = torch.randn((b, H, 64, 128), generator=gen, device="cuda") * 0.1
    cache0 = dd["cache"].clone()
    nch0 = torch.tensor([4, 3, 0, 1, 2, 6, 1, 11], dtype=torch.int32, device="cuda")
    state, cache, nch = state0.clone(), cache0.clone(), nch0.clone()

    def reset():
        state.copy_(state0)
        cache.copy_(cache0)
        nch.copy_(nch0)

    def step():
        out, R, lse = dart.dart_sma_decode(dd["q"], dd["c"], dd["e"], cache, dd["y"], dd["gate"], n_chunks=nch,
                                           want_R=True, want_lse=True)
        dart.dart_decode_state_update(x, Bt, a, state, pos, cache, S, n_chunks=nch)
        return out, R, lse

    reset()
    eager = [t.clone() for t in step()] + [state.clone(), cache.clone(), nch.clone()]
    reset()
    g, outs = capture(step)
    for rep in range(3):
        reset()
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, e, y in zip(("out", "R", "lse", "state", "cache", "n_chunks"), eager,
                              list(outs) + [state, cache, nch]):
            same(e, y, f"decode graph replay {rep}: {name}")
    say("decode step: 3 graph replays equal the eager step")

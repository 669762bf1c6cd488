"""Whole-output GPU parity on the very-long-context workload (b=1, H=32,
L=65536, S=256: 255 earlier chunks for the last tokens; N=128, P=64, bf16;
seed 0), in the launch the benchmark times: every chunk memory [§3 Eq. 5] and
every out, R and lse [§3 Eq. 8-11] of every head against the fp64 oracle end
to end, eight heads per test so that each test stays short."""
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, MaxErr, f64, same, say, to_oracle_mem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    cfg = synth.workload(synth.VLONG)
    say("full size", cfg["name"], "on the GPU")
    S = cfg["chunk"]
    d = synth.draw_fwd_torch(**cfg, seed=0)
    dH = dart.dart_chunk_states(d["X"], d["B"], d["A"], S)
    out_bench, _, _ = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S)
    out, R, lse = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S,
                                    want_R=True, want_lse=True)
    torch.cuda.synchronize()
    same(out_bench, out, "out of the two forward launches (b, t, h)")
    for t in (dH, out, R, lse):
        assert not torch.isnan(t).any()
    host = {k: v.cpu() for k, v in d.items()}
    host.update(dH=dH.cpu(), out=out.cpu(), R=R.cpu(), lse=lse.cpu())
    del d, dH, out_bench, out, R, lse
    torch.cuda.empty_cache()
    say("  GPU done; outputs on the host")
    return cfg, host


@pytest.mark.parametrize("h0", [0, 8, 16, 24])
def test_vlong_end_to_end(run, h0):
    cfg, h = run
    S, hpg = cfg["chunk"], cfg["nheads"] // cfg["ngroups"]
    acc = {k: MaxErr(k) for k in ("dH", "out", "R", "lse")}
    for hh in range(h0, h0 + 8):
        gi = hh // hpg
        memo = O.chunk_states_head(f64(h["X"][0, :, hh]), f64(h["B"][0, :, gi]), f64(h["A"][0, :, hh]), S)
        acc["dH"].add(to_oracle_mem(f64(h["dH"][0, hh])), memo, hh)
        R, lse = O.sma_head(f64(h["Q"][0, :, gi]), f64(h["C"][0, :, gi]), f64(h["E"][0, :, gi]), memo, S)
        acc["R"].add(f64(h["R"][0, :, hh]), R, hh)
        acc["lse"].add(f64(h["lse"][0, hh]), lse, hh)
        out = O.gated_residual(f64(h["Y"][0, :, hh]), f64(h["gate"][0, :, hh]), R)
        acc["out"].add(f64(h["out"][0, :, hh]), out, hh)
    for a in acc.values():
        a.check(TOL["bf16"])

"""Whole-output GPU parity on the long-context workload (b=2, H=24,
L=16384, S=256, N=128, P=64, bf16; seed 0), in the launches the benchmark
times: every element of every output against the fp64 oracle, one (batch
row, head) at a time so that host memory stays bounded.

* chunk states [§3 Eq. 5] and the forward [§3 Eq. 8-11] end to end
  (X, B, A -> chunk memories -> SMA -> gated residual) at the bf16 bar, and
  R and lse again on the GPU's own chunk memories at the same-input bar;
* the backward [§3 Eq. 5, 8-11 differentiated; App. C Eq. 33-35]: dQ, dC,
  dE, d_dH and dgate from the GPU forward's R and lse and the seed-3 loss
  gradient, then dX, dB, dA from the GPU's d_dH;
* the RMS-normalised score branch [App. B.1 Eq. 25-27] on the GPU's own
  chunk memories (eps = 1e-6, no norm weights), and its backward: dQ, dC,
  dE, d_dH, dgate and the gradients of the RMSNorm weights (at weight 1),
  those of each batch row alone from a call on that row, and the call on
  both rows equal to their sum;
* the SSM branch by the chunked scan [App. A Eq. 15-24] against the step
  recurrence, its chunk memories bit for bit against dart_chunk_states.
"""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, TOL_SAME_INPUT, MaxErr, f64, same, say, to_oracle_mem

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module")
def run():
    """Every GPU call of this module on one draw; results moved to the host."""
    cfg = synth.workload(synth.LONG)
    say("full size", cfg["name"], "on the GPU")
    b, H, L, S, P = cfg["batch"], cfg["nheads"], cfg["seqlen"], cfg["chunk"], cfg["d_head"]
    d = synth.draw_fwd_torch(**cfg, seed=0)
    g = {}
    # forward: the benchmark's launch (R and lse not requested), then again
    # with them; out must not change
    g["dH"] = dart.dart_chunk_states(d["X"], d["B"], d["A"], S)
    out_bench, _, _ = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], g["dH"], d["Y"], d["gate"], S)
    g["out"], g["R"], g["lse"] = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], g["dH"], d["Y"], d["gate"], S,
                                                   want_R=True, want_lse=True)
    torch.cuda.synchronize()
    same(out_bench, g["out"], "out of the two forward launches (b, t, h)")
    del out_bench
    # backward
    g["dout"] = synth.draw_grad_torch((b, L, H, P), "bf16", seed=3)
    g["dQ"], g["dC"], g["dE"], g["ddH"], g["dgate"] = dart.dart_sma_bwd(
        d["Q"], d["C"], d["E"], g["dH"], d["gate"], g["R"], g["lse"], g["dout"], S)
    g["dX"], g["dB"], g["dA"] = dart.dart_chunk_states_bwd(d["X"], d["B"], d["A"], g["ddH"], S)
    # normalised score branch
    dHr, g["r"], score = dart.dart_chunk_states_rms(d["X"], d["B"], d["A"], S, EPS)
    g["out_rms"], g["R_rms"], g["lse_rms"] = dart.dart_sma_fwd_rms(
        d["Q"], d["C"], d["E"], dHr, score, d["Y"], d["gate"], S, EPS, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    same(dHr, g["dH"], "dart_chunk_states_rms memories against dart_chunk_states (b, h, c)")
    # its backward, the benchmark's call, then each batch row alone for the
    # weight gradients (sums over every row and head)
    (g["dQ_rms"], g["dC_rms"], g["dE_rms"], g["ddH_rms"], g["dgate_rms"], g["dwq"], g["dwe"]) = \
        dart.dart_sma_bwd_rms(d["Q"], d["C"], d["E"], dHr, score, d["gate"], g["R_rms"], g["lse_rms"], g["dout"],
                              S, EPS, want_dw=True)
    for bi in range(b):
        row = lambda t: t[bi:bi + 1].contiguous()
        res = dart.dart_sma_bwd_rms(row(d["Q"]), row(d["C"]), row(d["E"]), row(dHr), row(score), row(d["gate"]),
                                    row(g["R_rms"]), row(g["lse_rms"]), row(g["dout"]), S, EPS,
                                    want_dgate=False, want_dw=True)
        g[f"dwq{bi}"], g[f"dwe{bi}"] = res[5], res[6]
        del res
    torch.cuda.synchronize()
    del dHr, score
    # SSM branch
    g["Y_ssm"], dH_ssd, g["H_final"] = dart.dart_ssd_fwd(d["X"], d["B"], d["C"], d["A"], S, want_final=True)
    torch.cuda.synchronize()
    same(dH_ssd, g["dH"], "dart_ssd_fwd memories against dart_chunk_states (b, h, c)")
    del dH_ssd
    for k, v in g.items():
        assert not torch.isnan(v).any(), k
    host = {k: v.cpu() for k, v in d.items()}
    host.update({k: v.cpu() for k, v in g.items()})
    del d, g
    torch.cuda.empty_cache()
    say("  GPU done; outputs on the host")
    return cfg, host


def head_inputs(cfg, h, bi, hh):
    """float64 numpy views of one (batch row, head): X, B, C, Q, E, a, Y, gate."""
    gi = hh // (cfg["nheads"] // cfg["ngroups"])
    return dict(X=f64(h["X"][bi, :, hh]), B=f64(h["B"][bi, :, gi]), C=f64(h["C"][bi, :, gi]),
                Q=f64(h["Q"][bi, :, gi]), E=f64(h["E"][bi, :, gi]), a=f64(h["A"][bi, :, hh]),
                Y=f64(h["Y"][bi, :, hh]), gate=f64(h["gate"][bi, :, hh]))


def heads(cfg):
    return [(bi, hh) for bi in range(cfg["batch"]) for hh in range(cfg["nheads"])]


def test_long_chunk_states_and_forward_end_to_end(run):
    cfg, h = run
    S = cfg["chunk"]
    acc = {k: MaxErr(k) for k in ("dH", "out", "R", "lse")}
    for bi, hh in heads(cfg):
        x = head_inputs(cfg, h, bi, hh)
        memo = O.chunk_states_head(x["X"], x["B"], x["a"], S)
        acc["dH"].add(to_oracle_mem(f64(h["dH"][bi, hh])), memo, (bi, hh))
        R, lse = O.sma_head(x["Q"], x["C"], x["E"], memo, S)
        acc["R"].add(f64(h["R"][bi, :, hh]), R, (bi, hh))
        acc["lse"].add(f64(h["lse"][bi, hh]), lse, (bi, hh))
        acc["out"].add(f64(h["out"][bi, :, hh]), O.gated_residual(x["Y"], x["gate"], R), (bi, hh))
    for a in acc.values():
        a.check(TOL["bf16"])


def test_long_forward_same_input(run):
    """R and lse on the GPU's own (bf16) chunk memories: float32 dot products
    of exact bf16 products and a float32 softmax on both sides' inputs."""
    cfg, h = run
    S = cfg["chunk"]
    acc = {k: MaxErr(k) for k in ("R", "lse")}
    for bi, hh in heads(cfg):
        x = head_inputs(cfg, h, bi, hh)
        R, lse = O.sma_head(x["Q"], x["C"], x["E"], to_oracle_mem(f64(h["dH"][bi, hh])), S)
        acc["R"].add(f64(h["R"][bi, :, hh]), R, (bi, hh))
        acc["lse"].add(f64(h["lse"][bi, hh]), lse, (bi, hh))
    for a in acc.values():
        a.check(TOL_SAME_INPUT["bf16"])


@pytest.mark.parametrize("bi", [0, 1])
def test_long_backward(run, bi):
    """Every gradient of batch row bi: the SMA backward on the GPU's chunk
    memories with the oracle's own lse, then the chunk-state backward from the
    GPU's d_dH (the input that call received)."""
    cfg, h = run
    S = cfg["chunk"]
    acc = {k: MaxErr(k) for k in ("dQ", "dC", "dE", "d_dH", "dgate", "dX", "dB", "dA")}
    for hh in range(cfg["nheads"]):
        x = head_inputs(cfg, h, bi, hh)
        mem = to_oracle_mem(f64(h["dH"][bi, hh]))
        R, lse = O.sma_head(x["Q"], x["C"], x["E"], mem, S)
        _, dR, dg = O.gated_residual_backward(f64(h["dout"][bi, :, hh]), x["gate"], R)
        dQ, dC, dE, ddH = O.sma_head_backward(x["Q"], x["C"], x["E"], mem, S, dR, lse)
        gi = hh // (cfg["nheads"] // cfg["ngroups"])   # G = H here: no group sums
        acc["dQ"].add(f64(h["dQ"][bi, :, gi]), dQ, hh)
        acc["dC"].add(f64(h["dC"][bi, :, gi]), dC, hh)
        acc["dE"].add(f64(h["dE"][bi, :, gi]), dE, hh)
        acc["d_dH"].add(to_oracle_mem(f64(h["ddH"][bi, hh])), ddH, hh)
        acc["dgate"].add(f64(h["dgate"][bi, :, hh]), dg, hh)
        dX, dB, dA = O.chunk_states_head_backward(x["X"], x["B"], x["a"], S,
                                                  to_oracle_mem(f64(h["ddH"][bi, hh])))
        acc["dX"].add(f64(h["dX"][bi, :, hh]), dX, hh)
        acc["dB"].add(f64(h["dB"][bi, :, gi]), dB, hh)
        acc["dA"].add(f64(h["dA"][bi, :, hh]), dA, hh)
    for a in acc.values():
        a.check(TOL["bf16"])


def test_long_normalised_branch(run):
    """r of every chunk memory, and R, lse, out of every token, on the GPU's
    own chunk memories."""
    cfg, h = run
    S = cfg["chunk"]
    acc = {k: MaxErr(k) for k in ("r", "out", "R", "lse")}
    for bi, hh in heads(cfg):
        x = head_inputs(cfg, h, bi, hh)
        mem = to_oracle_mem(f64(h["dH"][bi, hh]))
        acc["r"].add(f64(h["r"][bi, hh]), O.chunk_inv_rms(mem, EPS), (bi, hh))
        R, lse = O.sma_head_rms(x["Q"], x["C"], x["E"], mem, S, EPS)
        acc["R"].add(f64(h["R_rms"][bi, :, hh]), R, (bi, hh))
        acc["lse"].add(f64(h["lse_rms"][bi, hh]), lse, (bi, hh))
        acc["out"].add(f64(h["out_rms"][bi, :, hh]), O.gated_residual(x["Y"], x["gate"], R), (bi, hh))
    acc["r"].check(TOL_SAME_INPUT["bf16"])
    for k in ("out", "R", "lse"):
        acc[k].check(TOL["bf16"])


@pytest.mark.parametrize("bi", [0, 1])
def test_long_normalised_backward(run, bi):
    """Every gradient of the normalised branch for batch row bi, on the
    GPU's chunk memories with the oracle's own R and lse; the weight
    gradients against the GPU call on that row alone."""
    cfg, h = run
    S, N, P = cfg["chunk"], cfg["d_state"], cfg["d_head"]
    acc = {k: MaxErr(k) for k in ("dQ", "dC", "dE", "d_dH", "dgate", "dw_q", "dw_e")}
    dwq, dwe = np.zeros(N), np.zeros(P)
    for hh in range(cfg["nheads"]):
        x = head_inputs(cfg, h, bi, hh)
        mem = to_oracle_mem(f64(h["dH"][bi, hh]))
        R, lse = O.sma_head_rms(x["Q"], x["C"], x["E"], mem, S, EPS)
        _, dR, dg = O.gated_residual_backward(f64(h["dout"][bi, :, hh]), x["gate"], R)
        dQ, dC, dE, ddH, wq, we = O.sma_head_backward_rms(x["Q"], x["C"], x["E"], mem, S, EPS, dR, lse,
                                                          np.ones(N), np.ones(P))
        gi = hh // (cfg["nheads"] // cfg["ngroups"])   # G = H here: no group sums
        acc["dQ"].add(f64(h["dQ_rms"][bi, :, gi]), dQ, hh)
        acc["dC"].add(f64(h["dC_rms"][bi, :, gi]), dC, hh)
        acc["dE"].add(f64(h["dE_rms"][bi, :, gi]), dE, hh)
        acc["d_dH"].add(to_oracle_mem(f64(h["ddH_rms"][bi, hh])), ddH, hh)
        acc["dgate"].add(f64(h["dgate_rms"][bi, :, hh]), dg, hh)
        dwq += wq
        dwe += we
    acc["dw_q"].add(f64(h[f"dwq{bi}"]), dwq)
    acc["dw_e"].add(f64(h[f"dwe{bi}"]), dwe)
    for a in acc.values():
        a.check(TOL["bf16"])


def test_long_normalised_weight_gradients_sum_over_rows(run):
    """The call on both batch rows gives the sum of the per-row calls (up
    to float32 rounding of the fixed-order sums)."""
    cfg, h = run
    for k in ("dwq", "dwe"):
        both, parts = f64(h[k]), f64(h[k + "0"]) + f64(h[k + "1"])
        assert np.abs(both - parts).max() <= 1e-5 * np.abs(parts).max(), k


@pytest.mark.parametrize("bi", [0, 1])
def test_long_ssm_branch(run, bi):
    """Y and the state after the last token of batch row bi against the step
    recurrence H_t = a_t H_{t-1} + B_t^T X_t, Y_t = C_t H_t."""
    cfg, h = run
    acc = {k: MaxErr(k) for k in ("Y", "H_final")}
    for hh in range(cfg["nheads"]):
        x = head_inputs(cfg, h, bi, hh)
        Y, Hl = O.ssm_output_head(x["X"], x["B"], x["C"], x["a"])
        acc["Y"].add(f64(h["Y_ssm"][bi, :, hh]), Y, hh)
        acc["H_final"].add(f64(h["H_final"][bi, hh]).T, Hl, hh)
    for a in acc.values():
        a.check(TOL["bf16"])

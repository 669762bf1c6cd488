"""GPU parity of dart_sma_bwd_rms, the backward of the normalised score branch
[App. B.1 Eq. 25-27 differentiated; App. C Eq. 33-35], against the fp64
oracle's sma_backward_rms (pinned by finite differences of its own forward).

* same-input: chunk memories drawn directly, the score memory from
  dart_chunk_rms of the same memories, R and lse from the GPU forward; every
  gradient (dQ, dC, dE, d_dH, dgate, dw_q, dw_e) is compared entry by entry
  with the oracle given the same memories (its own R and lse);
* end to end: X, B, A -> dart_chunk_states_rms -> dart_sma_fwd_rms ->
  dart_sma_bwd_rms -> dart_chunk_states_bwd against the same chain in the
  oracle (dX, dB, dA too).  For bf16 the chain is also checked on the chunk
  memories as stored, and the fp64 comparison allows, on top of the bf16
  bar, the amount by which the oracle's own gradients move when its memories
  are rounded to bfloat16 (measured in the test: ~2e-2 at logits up to ~90);
* shapes: grouped heads (sums over a group), ragged last chunk, a chunk
  longer than the sequence (no token sees a chunk: every gradient but dgate
  is zero), chunks of one token, odd N and P, scalar and per-channel gates,
  with and without RMSNorm weights, fp32 and bf16 inputs;
* determinism: two calls agree bit for bit.

Tolerances (max-abs-normalised, as elsewhere).  fp32 inputs: 1e-4, float32
arithmetic throughout.  bf16 inputs: the bf16 bar 2e-2.  The normalised
logits have a standard deviation of about sqrt(P) (8 for P = 64), so the
chunk weights are sharp; the score memory the logits are recomputed from is
stored in float16 (relative rounding 2^-11) and the matrix-core forward rounds
RMSNorm(Q_t) to float16 as well, so p = exp(l - lse) carries a relative error
of a few 1e-3 that dl = p (dR . V - D) passes on to every gradient.
"""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, dev, err, host, say, to_oracle_mem

pytestmark = pytest.mark.gpu

EPS = 1e-6


def weights(N, P, seed, on):
    if not on:
        return None, None
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 2.0, N), rng.uniform(0.5, 2.0, P)


def tw(w):
    return None if w is None else torch.from_numpy(np.asarray(w, dtype=np.float32)).cuda()


def gpu_chain(d, cfg, mem_t, score_t, dout, wq, we):
    dt = cfg["dtype"]
    Q, C, E = dev(d["Q"], dt), dev(d["C"], dt), dev(d["E"], dt)
    Y, g = dev(d["Y"], dt), dev(d["gate"], dt)
    _, R, lse = dart.dart_sma_fwd_rms(Q, C, E, mem_t, score_t, Y, g, cfg["chunk"], EPS, want_R=True,
                                      want_lse=True)
    dQ, dC, dE, ddH, dg, dwq, dwe = dart.dart_sma_bwd_rms(Q, C, E, mem_t, score_t, g, R, lse, dev(dout, dt),
                                                          cfg["chunk"], EPS, tw(wq), tw(we), want_dw=True)
    torch.cuda.synchronize()
    got = dict(Q=host(dQ), C=host(dC), E=host(dE), dH=host(ddH), gate=host(dg), wq=host(dwq), we=host(dwe))
    return got, ddH


def oracle_chain(d, cfg, mem_oracle, dout, wq, we):
    N, P = cfg["d_state"], cfg["d_head"]
    gpc = d["gate"].ndim == 4
    R, lse = O.sma_forward_rms(d["Q"], d["C"], d["E"], mem_oracle, cfg["chunk"], EPS, wq, we)
    _, dR, dg = O.gated_residual_backward(dout, d["gate"], R, gpc)
    # a weight that is not given is 1, and its gradient is still reported
    wq1 = np.ones(N) if wq is None else wq
    we1 = np.ones(P) if we is None else we
    dQ, dC, dE, ddH, dwq, dwe = O.sma_backward_rms(d["Q"], d["C"], d["E"], mem_oracle, cfg["chunk"], EPS, dR,
                                                   lse, wq1, we1)
    return dict(Q=dQ, C=dC, E=dE, dH=np.swapaxes(ddH, -1, -2), gate=dg, wq=dwq, we=dwe)


def compare(got, ref, tol, label):
    errs = {k: err(got[k], ref[k]) for k in ref}
    say(f"  {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert not np.isnan(got[k]).any(), k
        assert v <= tol, (k, v)


CASES = [
    # (config, gate per channel, RMSNorm weights)
    (dict(batch=1, nheads=2, ngroups=1, seqlen=300, chunk=64, d_state=16, d_head=16, dtype="f32"), True, True),
    (dict(batch=2, nheads=3, ngroups=3, seqlen=97, chunk=20, d_state=40, d_head=24, dtype="f32"), False, False),
    (dict(batch=1, nheads=4, ngroups=2, seqlen=700, chunk=128, d_state=128, d_head=64, dtype="bf16"), True, True),
    (dict(batch=2, nheads=2, ngroups=2, seqlen=513, chunk=256, d_state=128, d_head=64, dtype="bf16"), False, False),
    (dict(batch=1, nheads=3, ngroups=1, seqlen=150, chunk=1, d_state=128, d_head=64, dtype="bf16"), True, True),
    (dict(batch=1, nheads=2, ngroups=2, seqlen=333, chunk=50, d_state=32, d_head=48, dtype="bf16"), True, False),
    (dict(batch=1, nheads=2, ngroups=2, seqlen=300, chunk=64, d_state=256, d_head=256, dtype="f32"), False, True),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_bwd_rms_same_input(ci):
    cfg, gpc, wts = CASES[ci]
    say("sma_bwd_rms same-input", cfg, "gpc", gpc, "weights", wts)
    dt = cfg["dtype"]
    N, P = cfg["d_state"], cfg["d_head"]
    d = synth.draw_fwd(**cfg, seed=81 + ci, gate_per_channel=gpc)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, N, P, dt, seed=91 + ci)
    dout = synth.draw_grad((cfg["batch"], cfg["seqlen"], cfg["nheads"], P), dt, 101 + ci)
    wq, we = weights(N, P, 111 + ci, wts)
    mem_t = dev(mem, dt)
    _, s = dart.dart_chunk_rms(mem_t, cfg["seqlen"], cfg["chunk"], EPS, tw(wq), tw(we), want_r=False)
    got, _ = gpu_chain(d, cfg, mem_t, s, dout, wq, we)
    ref = oracle_chain(d, cfg, to_oracle_mem(mem), dout, wq, we)
    compare(got, ref, TOL[dt], "same-input")


def test_bwd_rms_chunk_longer_than_sequence():
    cfg = dict(batch=2, nheads=2, ngroups=1, seqlen=50, chunk=64, d_state=24, d_head=8, dtype="f32")
    d = synth.draw_fwd(**cfg, seed=121)
    mem = synth.draw_memories(2, 2, 1, 24, 8, "f32", seed=122)
    dout = synth.draw_grad((2, 50, 2, 8), "f32", 123)
    wq, we = weights(24, 8, 124, True)
    mem_t = dev(mem)
    _, s = dart.dart_chunk_rms(mem_t, 50, 64, EPS, tw(wq), tw(we), want_r=False)
    got, _ = gpu_chain(d, cfg, mem_t, s, dout, wq, we)
    for k in ("Q", "C", "E", "dH", "wq", "we"):
        assert not got[k].any(), k
    ref = oracle_chain(d, cfg, to_oracle_mem(mem), dout, wq, we)
    compare(got, ref, TOL["f32"], "no visible chunk")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bwd_rms_end_to_end(dt):
    cfg = dict(batch=1, nheads=2, ngroups=1, seqlen=600, chunk=128, d_state=128, d_head=64, dtype=dt)
    if dt == "f32":
        cfg.update(d_state=32, d_head=16, chunk=64)
    say("sma_bwd_rms end-to-end", cfg)
    N, P = cfg["d_state"], cfg["d_head"]
    d = synth.draw_fwd(**cfg, seed=131)
    dout = synth.draw_grad((1, cfg["seqlen"], 2, P), dt, 132)
    wq, we = weights(N, P, 133, True)
    X, B, A = dev(d["X"], dt), dev(d["B"], dt), dev(d["A"], "f32")
    dH, _, s = dart.dart_chunk_states_rms(X, B, A, cfg["chunk"], EPS, tw(wq), tw(we), want_r=False)
    got, ddH = gpu_chain(d, cfg, dH, s, dout, wq, we)
    dX, dB, dA = dart.dart_chunk_states_bwd(X, B, A, ddH, cfg["chunk"])
    torch.cuda.synchronize()
    got.update(X=host(dX), B=host(dB), A=host(dA))

    def with_chunk_grads(ref):
        rX, rB, rA = O.chunk_states_backward(d["X"], d["B"], d["A"], cfg["chunk"],
                                             np.swapaxes(ref["dH"], -1, -2))
        ref.update(X=rX, B=rB, A=rA)
        return ref

    memo = O.chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
    ref = with_chunk_grads(oracle_chain(d, cfg, memo, dout, wq, we))
    if dt == "f32":
        compare(got, ref, TOL[dt], "end-to-end")
        return
    # bf16: the chunk memories are stored in bfloat16, and with logits up to
    # ~90 that rounding alone moves the oracle's own gradients by ~2e-2.
    # (a) the chain on the memories as the GPU stored them, at the bf16 bar;
    stored = to_oracle_mem(host(dH))
    compare(got, with_chunk_grads(oracle_chain(d, cfg, stored, dout, wq, we)), TOL[dt], "on stored memories")
    # (b) against the fp64 memories, at the bar plus the oracle's own change
    # when its memories are rounded to bfloat16.
    rounded = torch.from_numpy(memo).to(torch.bfloat16).to(torch.float64).numpy()
    ref_r = with_chunk_grads(oracle_chain(d, cfg, rounded, dout, wq, we))
    sens = max(err(ref_r[k], ref[k]) for k in ref)
    say(f"  oracle change from bf16 memories: {sens:.2e}")
    compare(got, ref, TOL[dt] + sens, "end-to-end")


def test_bwd_rms_deterministic():
    cfg, gpc, wts = CASES[2]
    d = synth.draw_fwd(**cfg, seed=141, gate_per_channel=gpc)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(1, 4, M, 128, 64, "bf16", seed=142)
    dout = synth.draw_grad((1, cfg["seqlen"], 4, 64), "bf16", 143)
    wq, we = weights(128, 64, 144, True)
    mem_t = dev(mem, "bf16")
    _, s = dart.dart_chunk_rms(mem_t, cfg["seqlen"], cfg["chunk"], EPS, tw(wq), tw(we), want_r=False)
    a, _ = gpu_chain(d, cfg, mem_t, s, dout, wq, we)
    b, _ = gpu_chain(d, cfg, mem_t, s, dout, wq, we)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


# bf16, N = 128, P = 64: the matrix-core backward.  Shapes as for the plain
# branch's matrix-core backward: tiles spanning several chunks (S < 128),
# chunk starts inside a 64-token sub-block of the d_dH pass (S % 64 != 0),
# grouped heads, ragged tails, a sequence shorter than one wave's 32 tokens,
# odd b*H*M*L, chunks of 1 and 3 tokens, the evaluation-time size 32, both
# gate forms, with and without RMSNorm weights.
MFMA_CASES = [
    (dict(batch=1, nheads=4, ngroups=2, seqlen=1000, chunk=96), True, True),
    (dict(batch=2, nheads=2, ngroups=2, seqlen=777, chunk=64), False, True),
    (dict(batch=1, nheads=2, ngroups=1, seqlen=1300, chunk=256), True, False),
    (dict(batch=2, nheads=2, ngroups=1, seqlen=20, chunk=8), False, True),
    (dict(batch=1, nheads=3, ngroups=1, seqlen=777, chunk=64), True, True),
    (dict(batch=1, nheads=2, ngroups=1, seqlen=151, chunk=1), True, True),
    (dict(batch=1, nheads=3, ngroups=3, seqlen=403, chunk=3), False, False),
    (dict(batch=2, nheads=2, ngroups=2, seqlen=1061, chunk=32), True, True),
]


def run_path(path, *args):
    prev = dart.set_path(path)
    try:
        return gpu_chain(*args)[0]
    finally:
        dart.set_path(prev)


@pytest.mark.parametrize("ci", range(len(MFMA_CASES)))
def test_mfma_bwd_rms_against_oracle_and_general(ci):
    base, gpc, wts = MFMA_CASES[ci]
    cfg = dict(base, d_state=128, d_head=64, dtype="bf16")
    say("mfma sma_bwd_rms", cfg, "gpc", gpc, "weights", wts)
    d = synth.draw_fwd(**cfg, seed=151 + ci, gate_per_channel=gpc)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, 128, 64, "bf16", seed=161 + ci)
    dout = synth.draw_grad((cfg["batch"], cfg["seqlen"], cfg["nheads"], 64), "bf16", 171 + ci)
    wq, we = weights(128, 64, 181 + ci, wts)
    mem_t = dev(mem, "bf16")
    _, s = dart.dart_chunk_rms(mem_t, cfg["seqlen"], cfg["chunk"], EPS, tw(wq), tw(we), want_r=False)
    got = run_path(dart.DART_PATH_AUTO, d, cfg, mem_t, s, dout, wq, we)
    gen = run_path(dart.DART_PATH_GENERAL, d, cfg, mem_t, s, dout, wq, we)
    ref = oracle_chain(d, cfg, to_oracle_mem(mem), dout, wq, we)
    compare(got, ref, TOL["bf16"], "mfma vs oracle")
    compare(got, gen, TOL["bf16"], "mfma vs general")


def test_mfma_bwd_rms_deterministic():
    base, gpc, wts = MFMA_CASES[0]
    cfg = dict(base, d_state=128, d_head=64, dtype="bf16")
    d = synth.draw_fwd(**cfg, seed=191, gate_per_channel=gpc)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(1, 4, M, 128, 64, "bf16", seed=192)
    dout = synth.draw_grad((1, cfg["seqlen"], 4, 64), "bf16", 193)
    wq, we = weights(128, 64, 194, True)
    mem_t = dev(mem, "bf16")
    _, s = dart.dart_chunk_rms(mem_t, cfg["seqlen"], cfg["chunk"], EPS, tw(wq), tw(we), want_r=False)
    runs = [gpu_chain(d, cfg, mem_t, s, dout, wq, we)[0] for _ in range(3)]
    for r in runs[1:]:
        for k in runs[0]:
            assert np.array_equal(runs[0][k], r[k]), k

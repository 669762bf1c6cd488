"""GPU parity of dart_sma_bwd and dart_chunk_states_bwd against the fp64
oracle's backward [§3 Eq. 5, 8-11 differentiated; App. C Eq. 33-35].

* same-input: chunk memories drawn directly; the GPU backward gets the GPU
  forward's R and lse, the oracle its own; every gradient (dQ, dC, dE, d_dH,
  dgate) is compared entry by entry;
* end to end: X, B, A -> chunk states -> forward -> backward -> chunk-state
  backward on the GPU against the same chain in the oracle (dX, dB, dA too);
* shapes cover grouped heads (summed gradients), a ragged last chunk, a
  chunk longer than the sequence, the scalar gate, and fp32 and bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, TOL_SAME_INPUT, dev, err, host, same, say, to_oracle_mem

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(d, mem, cfg, dout, gate_pc):
    dt = cfg["dtype"]
    Q, C, E = dev(d["Q"], dt), dev(d["C"], dt), dev(d["E"], dt)
    Y, g = dev(d["Y"], dt), dev(d["gate"], dt)
    dH = mem if torch.is_tensor(mem) else dev(mem, dt)
    _, R, lse = dart.dart_sma_fwd(Q, C, E, dH, Y, g, cfg["chunk"], want_R=True, want_lse=True)
    go = dev(dout, dt)
    dQ, dC, dE, ddH, dg = dart.dart_sma_bwd(Q, C, E, dH, g, R, lse, go, cfg["chunk"])
    torch.cuda.synchronize()
    return dict(Q=host(dQ), C=host(dC), E=host(dE), dH=host(ddH), gate=host(dg)), ddH


def run_bwd_path(d, mem, cfg, dout, gate_pc, path):
    prev = dart.set_path(path)
    try:
        got, _ = gpu_fwd_bwd(d, mem, cfg, dout, gate_pc)
    finally:
        dart.set_path(prev)
    return got


def oracle_bwd(d, mem_oracle, cfg, dout, gate_pc):
    R, lse = O.sma_forward(d["Q"], d["C"], d["E"], mem_oracle, cfg["chunk"])
    _, dR, dg = O.gated_residual_backward(dout, d["gate"], R, gate_pc)
    dQ, dC, dE, ddH = O.sma_backward(d["Q"], d["C"], d["E"], mem_oracle, cfg["chunk"], dR, lse)
    return dict(Q=dQ, C=dC, E=dE, dH=np.swapaxes(ddH, -1, -2), gate=dg)


def compare(got, ref, tol, label):
    errs = {k: err(got[k], ref[k]) for k in ref}
    say(f"  {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert not np.isnan(got[k]).any(), k
        assert v <= tol, (k, v)


CASES = [
    # fp32, grouped heads, ragged last chunk
    dict(batch=1, nheads=2, ngroups=1, seqlen=300, chunk=64, d_state=16, d_head=16, dtype="f32"),
    # bf16 at the MFMA shapes, scalar gate in one case
    dict(batch=1, nheads=2, ngroups=2, seqlen=700, chunk=128, d_state=128, d_head=64, dtype="bf16"),
    # odd sizes and a chunk that does not divide L
    dict(batch=2, nheads=3, ngroups=3, seqlen=97, chunk=20, d_state=40, d_head=24, dtype="f32"),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("gate_pc", [True, False])
def test_sma_bwd_same_input(ci, gate_pc):
    cfg = CASES[ci]
    say("sma_bwd same-input", cfg, "gate_pc", gate_pc)
    d = synth.draw_fwd(**cfg, seed=11, gate_per_channel=gate_pc)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, cfg["d_state"], cfg["d_head"],
                              cfg["dtype"], std=1.0, seed=12)
    dout = synth.draw_grad((cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["d_head"]), cfg["dtype"], 13)
    ref = oracle_bwd(d, to_oracle_mem(mem), cfg, dout, gate_pc)
    # general kernels: float32 arithmetic on the exact inputs
    got = run_bwd_path(d, mem, cfg, dout, gate_pc, dart.DART_PATH_GENERAL)
    compare(got, ref, TOL_SAME_INPUT[cfg["dtype"]], "same-input general")
    # default path (the matrix core for bf16, N = 128, P = 64): dR and the
    # weighted MFMA operands are rounded to bf16 once each, ~2^-9 relative
    got = run_bwd_path(d, mem, cfg, dout, gate_pc, dart.DART_PATH_AUTO)
    compare(got, ref, TOL[cfg["dtype"]], "same-input default")


@pytest.mark.parametrize("ci", [0, 1])
def test_backward_end_to_end(ci):
    cfg = CASES[ci]
    say("backward end-to-end", cfg)
    dt = cfg["dtype"]
    d = synth.draw_fwd(**cfg, seed=21)
    dout = synth.draw_grad((cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["d_head"]), dt, 22)
    X, B = dev(d["X"], dt), dev(d["B"], dt)
    A = dev(d["A"], "f32")
    dH = dart.dart_chunk_states(X, B, A, cfg["chunk"])
    got, ddH = gpu_fwd_bwd(d, dH, cfg, dout, True)
    dX, dB, dA = dart.dart_chunk_states_bwd(X, B, A, ddH, cfg["chunk"])
    torch.cuda.synchronize()
    got.update(X=host(dX), B=host(dB), A=host(dA))

    memo = O.chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
    ref = oracle_bwd(d, memo, cfg, dout, True)
    ddH_o = np.swapaxes(ref["dH"], -1, -2)
    rX, rB, rA = O.chunk_states_backward(d["X"], d["B"], d["A"], cfg["chunk"], ddH_o)
    ref.update(X=rX, B=rB, A=rA)
    compare(got, ref, TOL[dt], "end-to-end")


def test_chunk_states_bwd_same_input_and_edges():
    # d_dH given directly: the chunk-state backward alone, fp32, grouped
    # heads, a chunk longer than the sequence and a zero decay
    for cfg in (dict(batch=1, nheads=4, ngroups=2, seqlen=70, chunk=32, d_state=24, d_head=12),
                dict(batch=2, nheads=2, ngroups=2, seqlen=50, chunk=64, d_state=8, d_head=8)):
        say("chunk_states_bwd same-input", cfg)
        d = synth.draw_fwd(**cfg, dtype="f32", seed=31)
        d["A"][0, 5, 0] = 0.0
        S = min(cfg["chunk"], cfg["seqlen"])
        M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
        g = synth.draw_memories(cfg["batch"], cfg["nheads"], M, cfg["d_state"], cfg["d_head"], "f32",
                                seed=32)
        dX, dB, dA = dart.dart_chunk_states_bwd(dev(d["X"]), dev(d["B"]), dev(d["A"]), dev(g),
                                                cfg["chunk"])
        torch.cuda.synchronize()
        rX, rB, rA = O.chunk_states_backward(d["X"], d["B"], d["A"], S, to_oracle_mem(g))
        compare(dict(X=host(dX), B=host(dB), A=host(dA)), dict(X=rX, B=rB, A=rA), TOL["f32"], "cs-bwd")


def test_bwd_deterministic():
    cfg = CASES[1]
    d = synth.draw_fwd(**cfg, seed=41)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, 128, 64, "bf16", seed=42)
    dout = synth.draw_grad((1, cfg["seqlen"], 2, 64), "bf16", 43)
    a, _ = gpu_fwd_bwd(d, mem, cfg, dout, True)
    b, _ = gpu_fwd_bwd(d, mem, cfg, dout, True)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_mfma_bwd_deterministic_many_chunk_groups():
    """The d_dH pass adds its two terms into a zeroed d_dH from separate
    blocks; with two addends per entry the sum must not depend on which
    lands first.  Several chunk groups per head, chunk starts inside a
    64-token sub-block, grouped heads; three runs must agree bit for bit."""
    cfg = dict(batch=2, nheads=4, ngroups=2, seqlen=2500, chunk=96, d_state=128, d_head=64, dtype="bf16")
    d = synth.draw_fwd(**cfg, seed=44)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, 128, 64, "bf16", seed=45)
    dout = synth.draw_grad((cfg["batch"], cfg["seqlen"], cfg["nheads"], 64), "bf16", 46)
    runs = [gpu_fwd_bwd(d, mem, cfg, dout, True)[0] for _ in range(3)]
    for r in runs[1:]:
        for k in runs[0]:
            assert np.array_equal(runs[0][k], r[k]), k


def test_mfma_bwd_repeat_bitwise_full_size():
    """Three backward calls at b2 H24 L16384 agree bit for bit: the d_dH
    pass streams up to 256 token sub-blocks per block through its LDS ring,
    each waited for before it is read."""
    cfg = synth.workload(synth.LONG)
    S = cfg["chunk"]
    d = synth.draw_fwd_torch(**cfg, seed=12)
    dH = dart.dart_chunk_states(d["X"], d["B"], d["A"], S)
    _, R, lse = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S, want_R=True, want_lse=True)
    dout = synth.draw_grad_torch(tuple(d["Y"].shape), "bf16", 13)
    first = dart.dart_sma_bwd(d["Q"], d["C"], d["E"], dH, d["gate"], R, lse, dout, S)
    for _ in range(2):
        again = dart.dart_sma_bwd(d["Q"], d["C"], d["E"], dH, d["gate"], R, lse, dout, S)
        torch.cuda.synchronize()
        for name, x, y in zip(("dQ", "dC", "dE", "d_dH", "dgate"), first, again):
            same(x, y, f"{name} of repeated backward calls")
        del again
    say("backward repeat at full size: bitwise")


# bf16, N = 128, P = 64: the matrix-core backward.  Shapes chosen to exercise
# tiles spanning several chunks (S < 128), chunk starts inside a 64-token
# sub-block of the d_dH pass (S % 64 != 0), grouped heads, a ragged tail,
# one chunk group per block boundary (M > 4) and the scalar gate.
MFMA_CASES = [
    dict(batch=1, nheads=4, ngroups=2, seqlen=1000, chunk=96, d_state=128, d_head=64, dtype="bf16"),
    dict(batch=2, nheads=2, ngroups=2, seqlen=777, chunk=64, d_state=128, d_head=64, dtype="bf16"),
    dict(batch=1, nheads=2, ngroups=1, seqlen=1300, chunk=256, d_state=128, d_head=64, dtype="bf16"),
    dict(batch=1, nheads=3, ngroups=3, seqlen=200, chunk=50, d_state=128, d_head=64, dtype="bf16"),
    # shorter than one wave's 32 tokens (waves 1-3 load and store nothing),
    # scalar gate
    dict(batch=2, nheads=2, ngroups=1, seqlen=20, chunk=8, d_state=128, d_head=64, dtype="bf16"),
    # b*H*M*L and b*H*L odd: the workspace parts after the (p, dl) rows and
    # after the decay weights start on a 256-byte boundary all the same
    dict(batch=1, nheads=3, ngroups=1, seqlen=777, chunk=64, d_state=128, d_head=64, dtype="bf16"),
    # every token its own chunk; chunks of 3; the evaluation-time size 32
    dict(batch=1, nheads=2, ngroups=1, seqlen=151, chunk=1, d_state=128, d_head=64, dtype="bf16"),
    dict(batch=1, nheads=3, ngroups=3, seqlen=403, chunk=3, d_state=128, d_head=64, dtype="bf16"),
    dict(batch=2, nheads=2, ngroups=2, seqlen=1061, chunk=32, d_state=128, d_head=64, dtype="bf16"),
]


@pytest.mark.parametrize("ci", range(len(MFMA_CASES)))
def test_mfma_bwd_against_oracle_and_general(ci):
    cfg = MFMA_CASES[ci]
    gate_pc = ci not in (1, 4, 7)
    say("mfma bwd", cfg, "gate_pc", gate_pc)
    d = synth.draw_fwd(**cfg, seed=51 + ci, gate_per_channel=gate_pc)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, 128, 64, "bf16", std=1.0, seed=61 + ci)
    dout = synth.draw_grad((cfg["batch"], cfg["seqlen"], cfg["nheads"], 64), "bf16", 71 + ci)
    got = run_bwd_path(d, mem, cfg, dout, gate_pc, dart.DART_PATH_AUTO)
    gen = run_bwd_path(d, mem, cfg, dout, gate_pc, dart.DART_PATH_GENERAL)
    ref = oracle_bwd(d, to_oracle_mem(mem), cfg, dout, gate_pc)
    compare(got, ref, TOL["bf16"], "mfma vs oracle")
    compare(got, gen, TOL["bf16"], "mfma vs general")


def test_mfma_bwd_sharp_weights():
    """Logits scaled up so the chunk weights are far from uniform (the
    graded draw gives nearly uniform weights, under which a misrouted chunk
    or a wrong p would hide)."""
    cfg = MFMA_CASES[2]
    d = synth.draw_fwd(**cfg, seed=81, gains={"Q": 8.0 * 11.3})
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(1, 2, M, 128, 64, "bf16", std=1.0, seed=82)
    dout = synth.draw_grad((1, cfg["seqlen"], 2, 64), "bf16", 83)
    got = run_bwd_path(d, mem, cfg, dout, True, dart.DART_PATH_AUTO)
    ref = oracle_bwd(d, to_oracle_mem(mem), cfg, dout, True)
    compare(got, ref, TOL["bf16"], "mfma sharp vs oracle")


@pytest.mark.parametrize("cfg", [
    dict(batch=1, nheads=4, ngroups=2, seqlen=900, chunk=300, d_state=128, d_head=64),  # 2 weight groups
    dict(batch=2, nheads=2, ngroups=2, seqlen=333, chunk=100, d_state=128, d_head=64),
    dict(batch=1, nheads=2, ngroups=1, seqlen=512, chunk=256, d_state=128, d_head=64),
    # chunks of 40 tokens: waves 2 and 3 of every pass hold none
    dict(batch=2, nheads=3, ngroups=3, seqlen=200, chunk=40, d_state=128, d_head=64),
    # b*H*L odd with grouped heads: the per-head dB partials start on a
    # 256-byte boundary of the workspace
    dict(batch=1, nheads=3, ngroups=1, seqlen=777, chunk=64, d_state=128, d_head=64),
    dict(batch=1, nheads=2, ngroups=2, seqlen=95, chunk=1, d_state=128, d_head=64),
    dict(batch=1, nheads=3, ngroups=1, seqlen=301, chunk=3, d_state=128, d_head=64),
    dict(batch=2, nheads=2, ngroups=1, seqlen=1061, chunk=32, d_state=128, d_head=64),
])
def test_chunk_states_bwd_mfma(cfg):
    """dX, dB, dA on the matrix core (d_dH rounded to bf16 as its operand)
    against the oracle and the general kernels."""
    say("chunk_states_bwd mfma", cfg)
    d = synth.draw_fwd(**cfg, dtype="bf16", seed=91)
    d["A"][0, 7, 0] = 0.0
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    gmem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, 128, 64, "f32", seed=92)
    X, B, A, G = dev(d["X"], "bf16"), dev(d["B"], "bf16"), dev(d["A"]), dev(gmem)
    out = {}
    for path in (dart.DART_PATH_AUTO, dart.DART_PATH_GENERAL):
        prev = dart.set_path(path)
        try:
            dX, dB, dA = dart.dart_chunk_states_bwd(X, B, A, G, cfg["chunk"])
        finally:
            dart.set_path(prev)
        torch.cuda.synchronize()
        out[path] = dict(X=host(dX), B=host(dB), A=host(dA))
    rX, rB, rA = O.chunk_states_backward(d["X"], d["B"], d["A"], cfg["chunk"], to_oracle_mem(gmem))
    ref = dict(X=rX, B=rB, A=rA)
    compare(out[dart.DART_PATH_GENERAL], ref, TOL_SAME_INPUT["bf16"], "cs-bwd general")
    compare(out[dart.DART_PATH_AUTO], ref, TOL["bf16"], "cs-bwd mfma")


@pytest.mark.parametrize("gate_pc", [True, False])
def test_mfma_bwd_without_dgate(gate_pc):
    """dgate is optional: without it the matrix-core backward computes the
    same dQ, dC, dE and d_dH, bit for bit (its stores of dgate go nowhere)."""
    cfg = dict(batch=1, nheads=2, ngroups=2, seqlen=650, chunk=128, d_state=128, d_head=64, dtype="bf16")
    say("mfma bwd without dgate", cfg, "gate_pc", gate_pc)
    d = synth.draw_fwd(**cfg, seed=71, gate_per_channel=gate_pc)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, 128, 64, "bf16", std=1.0, seed=72)
    dout = synth.draw_grad((cfg["batch"], cfg["seqlen"], cfg["nheads"], 64), "bf16", 73)
    dt = cfg["dtype"]
    Q, C, E = dev(d["Q"], dt), dev(d["C"], dt), dev(d["E"], dt)
    Y, g, dH = dev(d["Y"], dt), dev(d["gate"], dt), dev(mem, dt)
    _, R, lse = dart.dart_sma_fwd(Q, C, E, dH, Y, g, cfg["chunk"], want_R=True, want_lse=True)
    go = dev(dout, dt)
    with_g = dart.dart_sma_bwd(Q, C, E, dH, g, R, lse, go, cfg["chunk"], want_dgate=True)
    without = dart.dart_sma_bwd(Q, C, E, dH, g, R, lse, go, cfg["chunk"], want_dgate=False)
    torch.cuda.synchronize()
    assert without[4] is None
    for name, a, b in zip(["dQ", "dC", "dE", "d_dH"], with_g[:4], without[:4]):
        assert torch.equal(a, b), name
    ref = oracle_bwd(d, to_oracle_mem(mem), cfg, dout, gate_pc)
    assert err(host(with_g[4]), ref["gate"]) <= TOL["bf16"]

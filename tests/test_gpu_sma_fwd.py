"""GPU parity of dart_sma_fwd against the fp64 oracle [§3 Eq. 8-11].

Two kinds of checks:
  * same-input: the chunk memories are drawn directly (or taken from the
    oracle's own inputs) so the GPU and the oracle consume identical values;
    R and lse are then held to a tight bound and the softmax is exercised with
    sharp logits (the graded distributions give nearly uniform weights, under
    which a routing error would hide);
  * end-to-end: X, B, A -> dart_chunk_states -> dart_sma_fwd against the
    oracle's chunk_states -> sma_forward, at the stated tolerances.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, TOL_SAME_INPUT, dev, err, host, say, to_oracle_mem

pytestmark = pytest.mark.gpu


def run_fwd(d, mem, cfg, gate_pc=True, path=dart.DART_PATH_AUTO, want=True, out_alias=False):
    dt = cfg["dtype"]
    Q, C, E = dev(d["Q"], dt), dev(d["C"], dt), dev(d["E"], dt)
    Y, g = dev(d["Y"], dt), dev(d["gate"], dt)
    dH = mem if torch.is_tensor(mem) else dev(mem, dt)
    b, L, H, P = Y.shape
    out = Y if out_alias else torch.full_like(Y, float("nan"))
    R = torch.full((b, L, H, P), float("nan"), device="cuda") if want else None
    lse = torch.full((b, H, L), float("nan"), device="cuda") if want else None
    prev = dart.set_path(path)
    try:
        dart.dart_sma_fwd(Q, C, E, dH, Y, g, cfg["chunk"], out=out, R=R, lse=lse)
    finally:
        dart.set_path(prev)
    torch.cuda.synchronize()
    return host(out), (host(R) if want else None), (host(lse) if want else None)


def oracle_fwd(d, mem_oracle, cfg, gate_pc=True):
    R, lse = O.sma_forward(d["Q"], d["C"], d["E"], mem_oracle, cfg["chunk"])
    out = O.gated_residual(d["Y"], d["gate"], R, gate_per_channel=gate_pc)
    return out, R, lse


def check(got, ref, tol_out, tol_r, label):
    e_out, e_r, e_l = err(got[0], ref[0]), err(got[1], ref[1]), err(got[2], ref[2])
    say(f"  {label}: out {e_out:.2e}  R {e_r:.2e}  lse {e_l:.2e}")
    assert not np.isnan(got[0]).any() and not np.isnan(got[1]).any() and not np.isnan(got[2]).any()
    assert e_out <= tol_out and e_r <= tol_r and e_l <= tol_r, (e_out, e_r, e_l)


def same_input_case(cfg, gains=None, mem_std=1.0, gate_pc=True, seed=0, path=dart.DART_PATH_AUTO):
    say("sma_fwd same-input", cfg, gains, "mem_std", mem_std, "gate_pc", gate_pc, "path", path)
    d = synth.draw_fwd(**cfg, seed=seed, gate_per_channel=gate_pc, gains=gains)
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    mem = synth.draw_memories(cfg["batch"], cfg["nheads"], M, cfg["d_state"], cfg["d_head"],
                              cfg["dtype"], std=mem_std, seed=seed + 1)
    got = run_fwd(d, mem, cfg, gate_pc, path)
    ref = oracle_fwd(d, to_oracle_mem(mem), cfg, gate_pc)
    check(got, ref, TOL[cfg["dtype"]], TOL_SAME_INPUT[cfg["dtype"]], "same-input")
    return d, mem, got, ref


BF = dict(d_state=128, d_head=64, dtype="bf16", a_lo=1.0, a_hi=16.0)


@pytest.mark.parametrize("qgain", [1.0, math.sqrt(128), 8 * math.sqrt(128)])
def test_mfma_sharpness_sweep(qgain):
    # logit std ~0.1, ~1 and ~8: from near-uniform to near one-hot routing
    cfg = dict(BF, batch=2, nheads=4, ngroups=4, seqlen=2048, chunk=256)
    same_input_case(cfg, gains={"Q": qgain})


@pytest.mark.parametrize("L,S,G,gate_pc", [
    (1000, 256, 1, True),    # ragged tail tile, L % S != 0, one shared group
    (777, 64, 2, False),     # tiles span several chunks, scalar gate
    (333, 16, 4, True),
    (640, 100, 4, True),     # S not a multiple of the token tile
    (700, 300, 2, True),     # S > token tile
    (129, 128, 4, False),    # one token in the second chunk
    (100, 256, 4, True),     # everything in chunk 0
    (20, 8, 2, True),        # waves 1-3 of the tile hold no token, two chunks in view
    (40, 16, 1, False),      # the same with a shared group and the scalar gate
    (5000, 1000, 1, True),
    (301, 1, 2, True),       # every token its own chunk: a tile streams up to 300 memories
    (999, 3, 1, False),      # a tile spans 43 chunks, ragged tail, scalar gate
    (2065, 32, 4, True),     # the evaluation-time chunk size: four chunks per tile, ragged tail
    (4096 + 77, 64, 2, False),
])
def test_mfma_stress_shapes(L, S, G, gate_pc):
    cfg = dict(BF, batch=2, nheads=4, ngroups=G, seqlen=L, chunk=S)
    same_input_case(cfg, gains={"Q": math.sqrt(128)}, gate_pc=gate_pc, seed=L)


@pytest.mark.parametrize("b,H,G,L,S,gate_pc", [
    (1, 3, 3, 128 * 200 + 37, 1024, True),   # 3 of 8 head slots real, ragged tail tile
    (1, 2, 1, 128 * 70 + 5, 64, False),      # long tiles of many small chunks, scalar gate
    (2, 4, 2, 128 * 80, 256, True),          # no padded head slots
])
def test_mfma_several_tiles_per_block(b, H, G, L, S, gate_pc):
    # More (head, tile) items than the chip holds 128-token tiles at once (two
    # per compute unit), with padded head slots, a ragged tail and long tiles
    # of many small chunks; every output is checked.
    cfg = dict(BF, batch=b, nheads=H, ngroups=G, seqlen=L, chunk=S)
    items = (b * H + 7) // 8 * 8 * ((L + 127) // 128)
    assert items > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    same_input_case(cfg, gains={"Q": math.sqrt(128)}, gate_pc=gate_pc, seed=L + S)


@pytest.mark.parametrize("N,P,dtype,L,S", [
    (16, 16, "f32", 1024, 64), (64, 32, "bf16", 500, 32), (7, 5, "f32", 300, 16),
    (256, 256, "f32", 192, 64), (1, 1, "f32", 50, 5), (128, 64, "f32", 700, 256),
])
def test_general_shapes(N, P, dtype, L, S):
    cfg = dict(batch=2, nheads=3, ngroups=3, seqlen=L, chunk=S, d_state=N, d_head=P, dtype=dtype)
    same_input_case(cfg, gains={"Q": math.sqrt(N)}, seed=N + P)


def test_planted_retrieval():
    """Every token of chunk i >= 2 routes to one planted memory by a wide
    margin, so R must equal C_t dH_{c*} (a wrong chunk index or visibility
    rule cannot pass)."""
    cfg = dict(BF, batch=1, nheads=2, ngroups=2, seqlen=1536, chunk=256)
    d = synth.draw_fwd(**cfg, seed=4)
    M = 6
    mem = synth.draw_memories(1, 2, M, 128, 64, "bf16", std=0.01, seed=5)
    # memory 1 gets a large constant block along e's sign pattern, so that
    # q dH_1 e >> q dH_c e for every other c (q, e positive by construction)
    d["Q"] = np.abs(d["Q"]) * np.float32(math.sqrt(128))
    d["E"] = np.abs(d["E"])
    mem[:, :, 1] = synth.round_bf16(np.full_like(mem[:, :, 1], 0.5))
    got = run_fwd(d, mem, cfg)
    ref = oracle_fwd(d, to_oracle_mem(mem), cfg)
    check(got, ref, TOL["bf16"], TOL_SAME_INPUT["bf16"], "planted")
    # and the closed form: tokens of chunks >= 2 read C_t dH_1
    memo = to_oracle_mem(mem)
    for t in (512, 900, 1535):
        want = d["C"][0, t, 0].astype(np.float64) @ memo[0, 0, 1]
        assert err(got[1][0, t, 0], want) <= 1e-3


def test_first_chunk_and_zero_gate():
    cfg = dict(BF, batch=1, nheads=4, ngroups=4, seqlen=1024, chunk=256)
    d = synth.draw_fwd(**cfg, seed=6)
    mem = synth.draw_memories(1, 4, 4, 128, 64, "bf16", seed=7)
    out, R, lse = run_fwd(d, mem, cfg)
    assert (R[:, :256] == 0).all() and np.isneginf(lse[:, :, :256]).all()
    assert np.array_equal(out[:, :256], d["Y"][:, :256].astype(np.float64))
    # g == 0 (the SMA-removal ablation): out == Y_ssm bit for bit
    d["gate"][:] = 0
    out, _, _ = run_fwd(d, mem, cfg)
    assert np.array_equal(out, d["Y"].astype(np.float64))


def test_single_visible_chunk_reads_values():
    # tokens of chunk 1 see only dH_0: R_t = C_t dH_0 whatever the logits
    cfg = dict(BF, batch=1, nheads=2, ngroups=1, seqlen=512, chunk=256)
    d = synth.draw_fwd(**cfg, seed=8, gains={"Q": 30.0})
    mem = synth.draw_memories(1, 2, 2, 128, 64, "bf16", seed=9)
    _, R, _ = run_fwd(d, mem, cfg)
    memo = to_oracle_mem(mem)
    want = np.einsum("tn,hnp->thp", d["C"][0, 256:, 0].astype(np.float64), memo[0, :, 0])
    assert err(R[0, 256:], want) <= 1e-3


def test_out_may_alias_y_and_outputs_are_optional():
    cfg = dict(BF, batch=1, nheads=4, ngroups=4, seqlen=1024, chunk=256)
    d = synth.draw_fwd(**cfg, seed=10)
    mem = synth.draw_memories(1, 4, 4, 128, 64, "bf16", seed=11)
    full = run_fwd(d, mem, cfg)
    bare = run_fwd(d, mem, cfg, want=False)
    aliased = run_fwd(d, mem, cfg, want=False, out_alias=True)
    assert np.array_equal(full[0], bare[0]) and np.array_equal(full[0], aliased[0])


def test_mfma_matches_general_kernel():
    cfg = dict(BF, batch=1, nheads=4, ngroups=2, seqlen=1300, chunk=256)
    d = synth.draw_fwd(**cfg, seed=12, gains={"Q": math.sqrt(128)})
    mem = synth.draw_memories(1, 4, 6, 128, 64, "bf16", seed=13)
    a = run_fwd(d, mem, cfg, path=dart.DART_PATH_AUTO)
    b = run_fwd(d, mem, cfg, path=dart.DART_PATH_GENERAL)
    assert err(a[1], b[1]) <= 1e-4 and err(a[2], b[2]) <= 1e-4 and err(a[0], b[0]) <= 1e-2


def test_deterministic():
    cfg = dict(BF, batch=2, nheads=4, ngroups=4, seqlen=2048, chunk=256)
    d = synth.draw_fwd(**cfg, seed=14)
    mem = synth.draw_memories(2, 4, 8, 128, 64, "bf16", seed=15)
    a, b = run_fwd(d, mem, cfg), run_fwd(d, mem, cfg)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------------------------- end-to-end
def end_to_end(cfg, seed=0):
    say("end-to-end", cfg["name"] if "name" in cfg else cfg)
    d = synth.draw_fwd(**cfg, seed=seed)
    dt = cfg["dtype"]
    dH = dart.dart_chunk_states(dev(d["X"], dt), dev(d["B"], dt), dev(d["A"], "f32"), cfg["chunk"])
    got = run_fwd(d, dH, cfg)
    memo = O.chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
    ref = oracle_fwd(d, memo, cfg)
    tol = TOL[dt]
    check(got, ref, tol, tol, "end-to-end")


def test_end_to_end_tiny_fp32():
    end_to_end(synth.workload(synth.TINY))


def test_end_to_end_block_bf16():
    end_to_end(synth.workload(synth.BLOCK))

"""GPU parity of dart_chunk_states against the fp64 oracle [§3 Eq. 5]."""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, dev, err, host, same, say, to_oracle_mem

pytestmark = pytest.mark.gpu


def run_cs(d, cfg, path=dart.DART_PATH_AUTO):
    dt = cfg["dtype"]
    X, B, A = dev(d["X"], dt), dev(d["B"], dt), dev(d["A"], "f32")
    M = dart.num_chunks(cfg["seqlen"], cfg["chunk"])
    b, H, N, P = cfg["batch"], cfg["nheads"], cfg["d_state"], cfg["d_head"]
    dH = torch.full((b, H, M, P, N), float("nan"), dtype=X.dtype, device="cuda")  # canary
    prev = dart.set_path(path)
    try:
        dart.dart_chunk_states(X, B, A, cfg["chunk"], dH=dH)
    finally:
        dart.set_path(prev)
    torch.cuda.synchronize()
    return host(dH)


def check_full(cfg, seed=0, path=dart.DART_PATH_AUTO, tol=None):
    say("chunk_states", cfg, "path", path)
    d = synth.draw_fwd(**cfg, seed=seed)
    got = run_cs(d, cfg, path)
    assert np.isfinite(got).all(), "unwritten or non-finite chunk memory"
    ref = O.chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
    e = err(to_oracle_mem(got), ref)
    say("  err", e)
    assert e <= (tol or TOL[cfg["dtype"]]), e
    return e


def test_tiny_fp32_config():
    check_full(synth.workload(synth.TINY))


def test_block_bf16_config():
    check_full(synth.workload(synth.BLOCK))


@pytest.mark.parametrize("L,S,G,dtype,N,P", [
    (1000, 256, 1, "bf16", 128, 64),   # L % S != 0, shared groups
    (700, 64, 2, "bf16", 128, 64),
    (333, 16, 3, "bf16", 128, 64),
    (300, 100, 6, "bf16", 128, 64),    # chunk not a multiple of the 64-token LDS block
    (130, 1, 6, "bf16", 128, 64),      # S = 1
    (257, 3, 2, "bf16", 128, 64),      # S = 3, ragged tail
    (1005, 32, 3, "bf16", 128, 64),    # the evaluation-time chunk size, ragged tail
    (600, 300, 2, "bf16", 128, 64),    # S > 256
    (257, 3, 1, "f32", 16, 16),
    (200, 50, 2, "f32", 7, 5),         # odd N, P on the general kernel
    (64, 32, 1, "bf16", 64, 32),
    (96, 48, 1, "f32", 256, 256),
])
def test_stress_shapes(L, S, G, dtype, N, P):
    cfg = dict(batch=2, nheads=6, ngroups=G, seqlen=L, chunk=S, d_state=N, d_head=P,
               dtype=dtype, a_lo=1.0, a_hi=16.0)
    check_full(cfg, seed=L + S)


def test_decay_special_cases():
    # A == 1: dH = B^T X ; A == 0: only the last token of each chunk survives
    cfg = dict(batch=1, nheads=2, ngroups=1, seqlen=600, chunk=256, d_state=128, d_head=64,
               dtype="bf16")
    d = synth.draw_fwd(**cfg, seed=3)
    for fill in (1.0, 0.0):
        d["A"] = np.full_like(d["A"], fill)
        got = to_oracle_mem(run_cs(d, cfg))
        ref = O.chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
        assert err(got, ref) <= TOL["bf16"]


def test_mfma_matches_general_kernel():
    cfg = synth.workload(synth.BLOCK, batch=1, nheads=4, ngroups=2, seqlen=1100)
    d = synth.draw_fwd(**cfg, seed=5)
    fast = run_cs(d, cfg, dart.DART_PATH_AUTO)
    gen = run_cs(d, cfg, dart.DART_PATH_GENERAL)
    # both round the same float32 sums (in different orders) once to bf16
    assert err(fast, gen) <= 1e-2


def test_repeat_launches_bitwise_full_size():
    """Three launches at b1 H32 L65536 agree bit for bit, with S = 256 (4
    sub-blocks of 64 tokens per chunk) and S = 1024 (16): each sub-block of
    the LDS ring is waited for before it is read, whatever the timing of the
    loads still in flight."""
    for S in (256, 1024):
        cfg = synth.workload(synth.VLONG, chunk=S)
        d = synth.draw_fwd_torch(**cfg, seed=11)
        runs = [dart.dart_chunk_states(d["X"], d["B"], d["A"], S) for _ in range(3)]
        torch.cuda.synchronize()
        say("chunk states repeat, S =", S)
        for r in runs[1:]:
            same(runs[0], r, f"dH of repeated launches, S = {S} (b, h, c)")
        del runs, d
        torch.cuda.empty_cache()


def test_deterministic():
    cfg = synth.workload(synth.BLOCK, batch=1, nheads=4, ngroups=4)
    d = synth.draw_fwd(**cfg, seed=9)
    a, b = run_cs(d, cfg), run_cs(d, cfg)
    assert np.array_equal(a, b)

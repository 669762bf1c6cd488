"""GPU parity of dart_sma_decode against the fp64 oracle [§4 "Inference
Cache"; §3 Eq. 8-11], and its consistency with dart_sma_fwd."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, TOL_SAME_INPUT, dev, err, host, say, to_oracle_mem

pytestmark = pytest.mark.gpu


def run_dec(d, dtype, n_chunks=None, gate_pc=True, path=dart.DART_PATH_AUTO):
    q, c, e = dev(d["q"], dtype), dev(d["c"], dtype), dev(d["e"], dtype)
    cache, y, g = dev(d["cache"], dtype), dev(d["y"], dtype), dev(d["gate"], dtype)
    nc = None if n_chunks is None else torch.tensor(n_chunks, dtype=torch.int32, device="cuda")
    b, H, _, P, _ = cache.shape
    out = torch.full_like(y, float("nan"))
    R = torch.full((b, H, P), float("nan"), device="cuda")
    lse = torch.full((b, H), float("nan"), device="cuda")
    prev = dart.set_path(path)
    try:
        dart.dart_sma_decode(q, c, e, cache, y, g, n_chunks=nc, out=out, R=R, lse=lse)
    finally:
        dart.set_path(prev)
    torch.cuda.synchronize()
    return host(out), host(R), host(lse)


def oracle_dec(d, n_chunks, H, G, gate_pc=True):
    R, lse = O.sma_decode(d["q"], d["c"], d["e"], to_oracle_mem(d["cache"]), n_chunks, hpg=H // G)
    return O.gated_residual(d["y"], d["gate"], R, gate_per_channel=gate_pc), R, lse


def check(got, ref, dtype, label):
    e = [err(g, r) for g, r in zip(got, ref)]
    say(f"  {label}: out {e[0]:.2e}  R {e[1]:.2e}  lse {e[2]:.2e}")
    assert e[0] <= TOL[dtype] and e[1] <= TOL_SAME_INPUT[dtype] and e[2] <= TOL_SAME_INPUT[dtype], e


@pytest.mark.parametrize("b,H,G,M,N,P,dtype,gate_pc,qgain", [
    (3, 4, 2, 37, 128, 64, "bf16", True, 1.0),
    (5, 6, 1, 256, 128, 64, "bf16", False, math.sqrt(128)),
    (2, 4, 4, 9, 128, 64, "bf16", True, 8 * math.sqrt(128)),
    (2, 3, 3, 20, 16, 16, "f32", True, 4.0),
    (2, 2, 1, 13, 64, 32, "bf16", True, 8.0),
    (1, 2, 2, 5, 7, 5, "f32", False, 1.0),
])
def test_decode_shapes(b, H, G, M, N, P, dtype, gate_pc, qgain):
    say("decode", b, H, G, M, N, P, dtype, gate_pc, qgain)
    d = synth.draw_decode(b, H, G, M, N, P, dtype, seed=M, gate_per_channel=gate_pc,
                          gains={"q": qgain})
    rng = np.random.default_rng(M)
    n_chunks = [int(x) for x in rng.integers(0, M + 1, b)]
    n_chunks[0] = M
    got = run_dec(d, dtype, n_chunks, gate_pc)
    check(got, oracle_dec(d, n_chunks, H, G, gate_pc), dtype, "decode")
    # n_chunks omitted = every chunk valid
    got = run_dec(d, dtype, None, gate_pc)
    check(got, oracle_dec(d, [M] * b, H, G, gate_pc), dtype, "decode all")


def test_decode_empty_and_single():
    d = synth.draw_decode(3, 4, 4, 8, 128, 64, "bf16", seed=1)
    out, R, lse = run_dec(d, "bf16", [0, 1, 0])
    assert (R[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.array_equal(out[0], d["y"][0].astype(np.float64))
    memo = to_oracle_mem(d["cache"])
    want = np.einsum("hn,hnp->hp", np.repeat(d["c"][1], 1, 0).astype(np.float64), memo[1, :, 0])
    assert err(R[1], want) <= 1e-3


def test_decode_zero_max_chunks():
    d = synth.draw_decode(2, 3, 3, 0, 128, 64, "bf16", seed=2)
    out, R, lse = run_dec(d, "bf16")
    assert (R == 0).all() and np.isneginf(lse).all() and np.array_equal(out, d["y"].astype(np.float64))


def test_decode_matches_forward_row():
    """A token of chunk i decoded against the cache dH_0..dH_{i-1} equals that
    token's row of dart_sma_fwd."""
    cfg = dict(batch=2, nheads=4, ngroups=2, seqlen=2048, chunk=256, d_state=128, d_head=64,
               dtype="bf16")
    d = synth.draw_fwd(**cfg, seed=3, gains={"Q": math.sqrt(128)})
    X, B, A = dev(d["X"], "bf16"), dev(d["B"], "bf16"), dev(d["A"], "f32")
    Q, C, E = dev(d["Q"], "bf16"), dev(d["C"], "bf16"), dev(d["E"], "bf16")
    Y, g = dev(d["Y"], "bf16"), dev(d["gate"], "bf16")
    dH = dart.dart_chunk_states(X, B, A, 256)
    out, R, lse = dart.dart_sma_fwd(Q, C, E, dH, Y, g, 256, want_R=True, want_lse=True)
    for t in (256, 1000, 2047):
        i = t // 256
        nc = torch.full((2,), i, dtype=torch.int32, device="cuda")
        od, Rd, ld = dart.dart_sma_decode(Q[:, t].contiguous(), C[:, t].contiguous(),
                                          E[:, t].contiguous(), dH, Y[:, t].contiguous(),
                                          g[:, t].contiguous(), n_chunks=nc, want_R=True,
                                          want_lse=True)
        torch.cuda.synchronize()
        assert err(host(Rd), host(R[:, t])) <= 1e-4
        assert err(host(ld), host(lse[:, :, t])) <= 1e-4
        assert err(host(od), host(out[:, t])) <= 1e-2


def test_mfma_matches_general_kernel():
    d = synth.draw_decode(4, 4, 2, 70, 128, 64, "bf16", seed=4, gains={"q": 11.0})
    a = run_dec(d, "bf16", [70, 3, 0, 33], path=dart.DART_PATH_AUTO)
    b = run_dec(d, "bf16", [70, 3, 0, 33], path=dart.DART_PATH_GENERAL)
    assert err(a[1], b[1]) <= 1e-4 and err(a[2], b[2]) <= 1e-4


@pytest.mark.parametrize("dt,N,P", [("bf16", 128, 64), ("f32", 16, 16)])
def test_decode_scalar_gate_token_slice(dt, N, P):
    """A scalar gate sliced for one token from a [1][L][H] tensor (here a
    30-byte offset: H = 5, token 3) is accepted, and gives exactly what an
    aligned copy of it gives, plain and normalised branch."""
    b, H, G, Mx, L, tok = 1, 5, 5, 9, 7, 3
    d = synth.draw_decode(batch=b, nheads=H, ngroups=G, max_chunks=Mx, d_state=N, d_head=P, dtype=dt, seed=61,
                          gate_per_channel=False)
    seq = torch.rand((b, L, H), device="cuda").to(torch.bfloat16 if dt == "bf16" else torch.float32)
    gate = seq[:, tok]
    assert gate.is_contiguous() and gate.data_ptr() % 16 != 0
    args = (dev(d["q"], dt), dev(d["c"], dt), dev(d["e"], dt), dev(d["cache"], dt))
    y = dev(d["y"], dt)
    n = torch.tensor([6], dtype=torch.int32, device="cuda")
    a = dart.dart_sma_decode(*args, y, gate, n_chunks=n, want_R=True, want_lse=True)
    c = dart.dart_sma_decode(*args, y, gate.clone(), n_chunks=n, want_R=True, want_lse=True)
    r_cache, _ = dart.dart_chunk_rms(args[3].reshape(b, H, Mx, P, N), Mx, 1, 1e-6, want_score=False)
    an = dart.dart_sma_decode_rms(*args, r_cache, y, gate, 1e-6, n_chunks=n, want_R=True, want_lse=True)
    cn = dart.dart_sma_decode_rms(*args, r_cache, y, gate.clone(), 1e-6, n_chunks=n, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    for x, z in zip(a + an, c + cn):
        assert torch.equal(x, z)

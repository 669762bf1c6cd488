"""dart_sma_decode_noalloc (the decode entry point for callers that cannot
allocate) against dart_sma_decode with a caller workspace, through the C ABI:
the same kernels on the same inputs must give the same out, R and lse bit for
bit, on consecutive calls that share the library's scratch (each smaller than
the one before, so stale partials of a larger call lie beyond what the next
one reads), and both must meet the oracle [§4 "Inference Cache"; §3 Eq.
8-11]."""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, TOL_SAME_INPUT, err, host, say

pytestmark = pytest.mark.gpu


def case(b, H, G, M, N, P, dtype, counts, seed):
    say("noalloc decode", dict(b=b, H=H, G=G, max_chunks=M, N=N, P=P, dtype=dtype, n_chunks=counts))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = synth.draw_decode(b, H, G, M, N, P, dtype, seed=seed, gains={"q": float(np.sqrt(N))})
    t = {k: torch.from_numpy(v).to("cuda").to(dt).contiguous() for k, v in d.items()}
    nc = torch.tensor(counts, dtype=torch.int32, device="cuda")
    args = (t["q"], t["c"], t["e"], t["cache"], t["y"], t["gate"])
    out_a = torch.full_like(t["y"], float("nan"))
    R_a = torch.full((b, H, P), float("nan"), device="cuda")
    lse_a = torch.full((b, H), float("nan"), device="cuda")
    dart.dart_sma_decode_noalloc(*args, n_chunks=nc, out=out_a, R=R_a, lse=lse_a)
    out_b, R_b, lse_b = dart.dart_sma_decode(*args, n_chunks=nc, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(R_a, R_b) and torch.equal(lse_a, lse_b)
    Rr, lr = O.sma_decode(d["q"], d["c"], d["e"], np.swapaxes(d["cache"], -1, -2), counts, hpg=H // G)
    outr = O.gated_residual(d["y"], d["gate"], Rr)
    e_out, e_r, e_l = err(host(out_a), outr), err(host(R_a), Rr), err(host(lse_a), lr)
    say(f"  out {e_out:.2e}  R {e_r:.2e}  lse {e_l:.2e}")
    tol = TOL_SAME_INPUT[dtype]
    assert e_out <= TOL[dtype] and e_r <= tol and e_l <= tol


def test_noalloc_matches_workspace_decode_on_consecutive_calls():
    # matrix-core path: b * H = 192 rows and heads in 10 ranges each, ragged
    # counts (0 and max included), then a smaller problem, then the general
    # path (float32)
    case(8, 24, 24, 48, 128, 64, "bf16", [48, 0, 1, 47, 17, 48, 5, 40], seed=1)
    case(3, 4, 2, 20, 128, 64, "bf16", [20, 0, 7], seed=2)
    case(2, 3, 1, 9, 16, 16, "f32", [9, 4], seed=3)


def test_noalloc_at_the_scratch_limit():
    # b * H = 15360 single-range partials: 4,055,040 bytes of the 4 MiB scratch
    b, H, M = 256, 60, 2
    need = dart.decode_workspace_bytes(b, H, 64, M)
    assert 4 << 20 >= need > (4 << 20) - 256 * 1024
    say("noalloc decode at the limit", dict(b=b, H=H, max_chunks=M, partial_bytes=need))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    bf = torch.bfloat16
    q = (torch.randn((b, H, 128), generator=gen, device="cuda")).to(bf)
    c = (torch.randn((b, H, 128), generator=gen, device="cuda") / 11.3).to(bf)
    e = (torch.randn((b, H, 64), generator=gen, device="cuda") / 8).to(bf)
    cache = torch.randn((b, H, M, 64, 128), generator=gen, device="cuda").to(bf)
    y = torch.randn((b, H, 64), generator=gen, device="cuda").to(bf)
    g = torch.rand((b, H, 64), generator=gen, device="cuda").to(bf)
    a = dart.dart_sma_decode_noalloc(q, c, e, cache, y, g, want_R=True, want_lse=True)
    w = dart.dart_sma_decode(q, c, e, cache, y, g, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    for x, z in zip(a, w):
        assert torch.equal(x, z)
    # spot-check the last (row, head), whose partial sits at the end of the scratch
    bi, hh = b - 1, H - 1
    r, l = O.sma_token(host(q[bi, hh]), host(c[bi, hh]), host(e[bi, hh]),
                       np.swapaxes(host(cache[bi, hh]), -1, -2))
    assert err(host(a[1][bi, hh]), r) <= TOL_SAME_INPUT["bf16"]
    assert abs(float(a[2][bi, hh]) - l) <= TOL_SAME_INPUT["bf16"] * max(1.0, abs(l))

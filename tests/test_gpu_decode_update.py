"""GPU parity of dart_decode_state_update (decode-side cache maintenance)
against the oracle's streaming update [§2 Eq. 2 within a chunk; §3 Eq. 5;
§4 "Inference Cache"], and consistency of streamed decoding with the forward:
decoding token t against the streamed cache gives the forward's R_t."""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, dev, err, host, say, to_oracle_mem

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,N,P,S", [("bf16", 128, 64, 32), ("bf16", 128, 64, 64),
                                      ("f32", 16, 8, 8), ("f32", 12, 5, 7)])
def test_streaming_update_matches_oracle(dt, N, P, S):
    b, H, G = 3, 4, 2
    L = 3 * S + 5
    lags = [0, 2, S + 3]          # row 2 starts late: its first steps are padding
    say("decode update", dt, N, P, S, "lags", lags)
    cfg = dict(batch=b, seqlen=L, nheads=H, ngroups=G, d_state=N, d_head=P, chunk=S)
    d = synth.draw_fwd(**cfg, dtype=dt, seed=5)
    Mx = L // S + 1
    X, Bm, A = dev(d["X"], dt), dev(d["B"], dt), dev(d["A"], "f32")
    state = torch.zeros((b, H, P, N), device="cuda")
    cache = torch.zeros((b, H, Mx, P, N), device="cuda", dtype=X.dtype)
    nch = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    steps = L + max(lags)
    for k in range(steps):
        pos = [k - lg if 0 <= k - lg < L else -1 for lg in lags]
        idx = [max(p, 0) for p in pos]
        x = torch.stack([X[i, idx[i]] for i in range(b)]).contiguous()
        bt = torch.stack([Bm[i, idx[i]] for i in range(b)]).contiguous()
        at = torch.stack([A[i, idx[i]] for i in range(b)]).contiguous()
        dart.dart_decode_state_update(x, bt, at, state, torch.tensor(pos, dtype=torch.int32, device="cuda"),
                                      cache, S, n_chunks=nch)
    torch.cuda.synchronize()
    assert host(nch).tolist() == [L // S] * b
    hs, hc = host(state), host(cache)
    for i in range(b):
        for h in range(H):
            ref_cache, ref_state = O.decode_stream(d["X"][i, :, h], d["B"][i, :, h // (H // G)],
                                                   d["A"][i, :, h], S)
            e1 = err(to_oracle_mem(hc[i, h, : L // S]), ref_cache)
            e2 = err(np.swapaxes(hs[i, h], 0, 1), ref_state)
            assert e1 <= TOL[dt] and e2 <= 1e-5, (i, h, e1, e2)
            assert np.abs(hc[i, h, L // S:]).max() == 0   # never closed: never written
    say("  cache and state match")


def test_streamed_decode_equals_forward():
    """Stream one sequence through the cache update; decoding each of a few
    tokens against the cache as it stood then gives the forward's R_t, lse_t
    computed on the same bf16 cache."""
    dt, N, P, S, H, G = "bf16", 128, 64, 64, 2, 2
    L = 4 * S + 9
    cfg = dict(batch=1, seqlen=L, nheads=H, ngroups=G, d_state=N, d_head=P, chunk=S)
    d = synth.draw_fwd(**cfg, dtype=dt, seed=9)
    Q, C, E = dev(d["Q"], dt), dev(d["C"], dt), dev(d["E"], dt)
    X, Bm, A = dev(d["X"], dt), dev(d["B"], dt), dev(d["A"], "f32")
    Y, g = dev(d["Y"], dt), dev(d["gate"], dt)
    Mx = L // S + 1
    state = torch.zeros((1, H, P, N), device="cuda")
    cache = torch.zeros((1, H, Mx, P, N), device="cuda", dtype=torch.bfloat16)
    nch = torch.zeros((1,), dtype=torch.int32, device="cuda")
    picks = {S - 1, S, 2 * S + 5, 4 * S + 8}
    got = {}
    for t in range(L):
        if t in picks:  # decode token t before its own update: chunks < chunk(t) are visible
            _, R, lse = dart.dart_sma_decode(Q[:, t], C[:, t], E[:, t], cache, Y[:, t], g[:, t],
                                             n_chunks=nch, want_R=True, want_lse=True)
            got[t] = (host(R), host(lse), int(host(nch)[0]))
        dart.dart_decode_state_update(X[:, t].contiguous(), Bm[:, t].contiguous(), A[:, t].contiguous(),
                                      state, torch.tensor([t], dtype=torch.int32, device="cuda"),
                                      cache, S, n_chunks=nch)
    # the forward over the same (streamed, bf16) chunk memories
    M = dart.num_chunks(L, S)
    dH = torch.zeros((1, H, M, P, N), device="cuda", dtype=torch.bfloat16)
    dH[:, :, : L // S] = cache[:, :, : L // S]
    _, Rf, lsef = dart.dart_sma_fwd(Q, C, E, dH, Y, g, S, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    Rf, lsef = host(Rf), host(lsef)
    for t, (R, lse, nb) in got.items():
        assert nb == t // S
        e_r = err(R[0], Rf[0, t])
        e_l = err(lse[0], lsef[0, :, t])
        say(f"  token {t}: n_chunks {nb}  R {e_r:.2e}  lse {e_l:.2e}")
        assert e_r <= 1e-3 and e_l <= 1e-3


def test_update_decode_workload_shape():
    """The decode workload's shape (64 rows, 24 heads, N = 128, P = 64,
    S = 256) in the launch the benchmark times: one token per row in the
    middle of chunk 100 against a random float32 in-progress state, then a
    token that closes the chunk (its memory goes to cache row 100 and the
    state restarts from zero).  Every entry against the oracle's update."""
    cfg = synth.workload(synth.DECODE)
    b, H, G, N, P, S = cfg["batch"], cfg["nheads"], cfg["ngroups"], cfg["d_state"], cfg["d_head"], cfg["chunk"]
    say("decode update, decode workload shape", cfg["name"])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    x = torch.randn((b, H, P), generator=gen, device="cuda").to(torch.bfloat16)
    Bt = (torch.randn((b, G, N), generator=gen, device="cuda") / N ** 0.5).to(torch.bfloat16)
    a = torch.rand((b, H), generator=gen, device="cuda") * 0.5 + 0.5
    state0 = torch.randn((b, H, P, N), generator=gen, device="cuda")
    cache = torch.zeros((b, H, 256, P, N), device="cuda", dtype=torch.bfloat16)
    nch = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    hpg = H // G
    for pos_in_chunk, closes in [(7, False), (S - 1, True)]:
        state = state0.clone()
        pos = torch.full((b,), 256 * 100 + pos_in_chunk, dtype=torch.int32, device="cuda")
        dart.dart_decode_state_update(x, Bt, a, state, pos, cache, S, n_chunks=nch)
        torch.cuda.synchronize()
        xs, bs, av, s0 = host(x), host(Bt), host(a), host(state0)
        # oracle, all (row, head) at once: a_t H + B_t^T x_t, stored (P, N)
        new = av[:, :, None, None] * s0 + np.einsum("bhp,bhn->bhpn", xs, bs[:, np.arange(H) // hpg])
        for bi, h in [(0, 0), (b - 1, H - 1), (17, 5)]:
            ref, closed = O.decode_state_update(s0[bi, h].T, xs[bi, h], bs[bi, h // hpg], av[bi, h],
                                                256 * 100 + pos_in_chunk, S)
            np.testing.assert_allclose(new[bi, h], (closed if closes else ref).T, rtol=1e-12, atol=1e-12)
        if closes:
            e_c = err(host(cache[:, :, 100]), new)
            e_s = float(np.abs(host(state)).max())
            say(f"  closing token: cache row {e_c:.2e}, state after {e_s:.1e}")
            assert e_c <= TOL["bf16"] and e_s == 0.0
            assert (host(nch) == 101).all()
        else:
            e_s = err(host(state), new)
            say(f"  mid-chunk token: state {e_s:.2e}")
            assert e_s <= TOL["f32"]

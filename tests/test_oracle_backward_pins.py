"""Pins for the oracle's backward pass, independent of its formulas.

* Central finite differences of the scalar loss sum(dout * out), with out
  computed by the oracle's forward (chunk states -> SMA -> gated residual),
  against every analytic gradient: dX, dB, dA, dQ, dC, dE, dY, dgate.  Grouped
  projections (G < H) check the sums over heads; a ragged last chunk and a
  zero decay are included.
* Closed forms: a token that sees exactly one chunk has weight 1, so its dQ
  and dE vanish and dC_t = dH_0 dR_t; with every decay equal to 1,
  dX_s = B_s d_dH_c; a chunk's first token has dA = 0.
"""
import numpy as np
import pytest

import oracle as O


def _inputs(rng, b, L, H, G, N, P):
    return dict(
        X=rng.standard_normal((b, L, H, P)),
        B=rng.standard_normal((b, L, G, N)) / np.sqrt(N),
        A=np.exp(-rng.uniform(0.05, 0.8, (b, L, H))),
        Q=rng.standard_normal((b, L, G, N)),
        C=rng.standard_normal((b, L, G, N)),
        E=rng.standard_normal((b, L, G, P)),
        Y=rng.standard_normal((b, L, H, P)),
    )


def _loss(d, S, dout, gpc):
    dH = O.chunk_states(d["X"], d["B"], d["A"], S)
    R, _ = O.sma_forward(d["Q"], d["C"], d["E"], dH, S)
    out = O.gated_residual(d["Y"], d["gate"], R, gpc)
    return float((dout * out).sum())


def _analytic(d, S, dout, gpc):
    dH = O.chunk_states(d["X"], d["B"], d["A"], S)
    R, lse = O.sma_forward(d["Q"], d["C"], d["E"], dH, S)
    dY, dR, dgate = O.gated_residual_backward(dout, d["gate"], R, gpc)
    dQ, dC, dE, ddH = O.sma_backward(d["Q"], d["C"], d["E"], dH, S, dR, lse)
    dX, dB, dA = O.chunk_states_backward(d["X"], d["B"], d["A"], S, ddH)
    return dict(X=dX, B=dB, A=dA, Q=dQ, C=dC, E=dE, Y=dY, gate=dgate)


@pytest.mark.parametrize("gpc,zero_decay", [(True, False), (False, True)])
def test_backward_matches_finite_differences(gpc, zero_decay):
    rng = np.random.default_rng(7)
    b, L, H, G, N, P, S = 1, 11, 2, 1, 3, 2, 4      # chunks of 4, 4, 3 tokens
    d = _inputs(rng, b, L, H, G, N, P)
    d["gate"] = rng.uniform(0.2, 1.0, (b, L, H, P) if gpc else (b, L, H))
    if zero_decay:
        d["A"][0, 6, 1] = 0.0                       # inside chunk 1, head 1
    dout = rng.standard_normal((b, L, H, P))
    grads = _analytic(d, S, dout, gpc)
    eps = 1e-6
    for name in ("X", "B", "A", "Q", "C", "E", "Y", "gate"):
        x = d[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = _loss(d, S, dout, gpc)
            x[idx] = keep - eps
            dn = _loss(d, S, dout, gpc)
            x[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        scale = max(np.abs(num).max(), 1e-3)
        err = np.abs(grads[name] - num).max() / scale
        assert err < 1e-6, (name, err)


def test_single_visible_chunk_closed_form():
    rng = np.random.default_rng(3)
    L, N, P, S = 8, 4, 3, 4                         # tokens 4..7 see chunk 0 only
    Q, C = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    E = rng.standard_normal((L, P))
    dH = rng.standard_normal((2, N, P))
    dR = rng.standard_normal((L, P))
    dQ, dC, dE, ddH = O.sma_head_backward(Q, C, E, dH, S, dR)
    assert np.abs(dQ[4:]).max() < 1e-12 and np.abs(dE[4:]).max() < 1e-12
    np.testing.assert_allclose(dC[4:], dR[4:] @ dH[0].T, rtol=1e-12, atol=1e-12)
    # chunk-0 tokens see nothing: every gradient there is zero
    assert np.abs(dQ[:4]).max() == 0 and np.abs(dC[:4]).max() == 0 and np.abs(dE[:4]).max() == 0
    # the last chunk is never read
    assert np.abs(ddH[1]).max() == 0
    np.testing.assert_allclose(ddH[0], C[4:].T @ dR[4:], rtol=1e-12, atol=1e-12)


def test_chunk_states_backward_unit_decay_and_first_token():
    rng = np.random.default_rng(5)
    L, N, P, S = 10, 3, 2, 4
    X, B = rng.standard_normal((L, P)), rng.standard_normal((L, N))
    G = rng.standard_normal((3, N, P))
    dX, dB, da = O.chunk_states_head_backward(X, B, np.ones(L), S, G)
    for t in range(L):
        c = t // S
        np.testing.assert_allclose(dX[t], B[t] @ G[c], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dB[t], G[c] @ X[t], rtol=1e-12, atol=1e-12)
    # with unit decays, da_k = sum_{s<k in the chunk} B_s G_c X_s^T
    for t in range(L):
        c, s0 = t // S, (t // S) * S
        want = sum(B[s] @ G[c] @ X[s] for s in range(s0, t))
        assert abs(da[t] - want) < 1e-12
    a = np.exp(-rng.uniform(0.1, 1.0, L))
    _, _, da = O.chunk_states_head_backward(X, B, a, S, G)
    assert da[0] == 0 and da[4] == 0 and da[8] == 0


def test_token_backward_matches_finite_differences():
    """The per-token backward against central differences of dR_t . R_t,
    with R_t from the oracle's per-token forward, in every input it takes
    (q, c, e and each visible chunk memory)."""
    rng = np.random.default_rng(17)
    N, P, n = 5, 3, 4
    q, c, e = rng.standard_normal(N), rng.standard_normal(N), rng.standard_normal(P)
    dH = rng.standard_normal((n, N, P))
    g = rng.standard_normal(P)
    dq, dc, de, ddH = O.sma_token_backward(q, c, e, dH, g)
    args = [q, c, e, dH]
    got = [dq, dc, de, ddH]
    eps = 1e-6
    for x, ana in zip(args, got):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = float(g @ O.sma_token(*args)[0])
            x[idx] = keep - eps
            dn = float(g @ O.sma_token(*args)[0])
            x[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        np.testing.assert_allclose(ana, num, rtol=1e-6, atol=1e-8)


def test_token_backward_sums_to_head_backward():
    """Summing the per-token backward over a head's tokens gives the head
    backward (its pinned counterpart): dQ, dC, dE row by row, d_dH summed."""
    rng = np.random.default_rng(18)
    L, S, N, P = 23, 5, 4, 3
    Q, C, E = rng.standard_normal((L, N)), rng.standard_normal((L, N)), rng.standard_normal((L, P))
    M = O.num_chunks(L, S)
    dH = rng.standard_normal((M, N, P))
    dR = rng.standard_normal((L, P))
    hq, hc, he, hdd = O.sma_head_backward(Q, C, E, dH, S, dR)
    tdd = np.zeros_like(hdd)
    for t in range(L):
        i = t // S
        dq, dc, de, dd = O.sma_token_backward(Q[t], C[t], E[t], dH[:i], dR[t])
        np.testing.assert_allclose(dq, hq[t], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dc, hc[t], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(de, he[t], rtol=1e-10, atol=1e-12)
        tdd[:i] += dd
    np.testing.assert_allclose(tdd, hdd, rtol=1e-10, atol=1e-12)

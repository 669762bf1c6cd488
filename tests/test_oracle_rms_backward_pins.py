"""Pins for the oracle's backward of the normalised score branch
[App. B.1 Eq. 25-27, differentiated], independent of its own formulas.

* Central finite differences of the scalar loss sum(dR * R), with R computed
  by the oracle's normalised forward (itself pinned by hand values, the
  reduction to the plain branch and its invariances), against every analytic
  gradient: dQ, dC, dE, d dH, dwq, dwe.  Grouped projections (G < H), a
  ragged last chunk, a nonzero eps and both with and without RMSNorm weights
  are covered; a second case runs the whole chain X, B, A -> chunk states ->
  normalised SMA and checks dX, dB, dA through the plain chunk-state backward.
* RMSNorm's own backward against finite differences, and its invariant: with
  eps = 0 the normalisation does not see the scale of x, so x . dx = 0.
* Invariants of the branch at eps = 0: every query and key enters the logits
  only through its direction, so dQ_t . Q_t = 0 and dE_t . E_t = 0; the value readout is the plain one, so dC equals the plain
  branch's dC when both have the same softmax weights (entries +-1, eps = 0).
* Closed form: a token that sees exactly one chunk has weight 1, so its dQ and
  dE vanish and its dC_t = dH_0 dR_t.
"""
import numpy as np
import pytest

import oracle as O


def _fd(f, x, step=1e-6):
    num = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        keep = x[idx]
        x[idx] = keep + step
        up = f()
        x[idx] = keep - step
        dn = f()
        x[idx] = keep
        num[idx] = (up - dn) / (2 * step)
    return num


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-3)


def test_rms_norm_backward_matches_finite_differences():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 5))
    g = rng.standard_normal((3, 5))
    for eps in (0.0, 0.3):
        num = _fd(lambda: float((g * O.rms_norm(x, eps)).sum()), x)
        assert _rel(O.rms_norm_backward(x, eps, g), num) < 1e-7
    # eps = 0: the output does not depend on |x|, so the gradient is orthogonal to x
    dx = O.rms_norm_backward(x, 0.0, g)
    np.testing.assert_allclose((dx * x).sum(axis=-1), 0.0, atol=1e-12)


@pytest.mark.parametrize("weights,G", [(False, 1), (True, 2)])
def test_backward_matches_finite_differences(weights, G):
    rng = np.random.default_rng(17)
    b, L, H, N, P, S, eps = 1, 11, 2, 3, 4, 4, 1e-2     # chunks of 4, 4, 3 tokens
    Q = rng.standard_normal((b, L, G, N))
    C = rng.standard_normal((b, L, G, N))
    E = rng.standard_normal((b, L, G, P))
    dH = rng.standard_normal((b, H, O.num_chunks(L, S), N, P))
    dR = rng.standard_normal((b, L, H, P))
    wq = rng.uniform(0.5, 1.5, N) if weights else None
    we = rng.uniform(0.5, 1.5, P) if weights else None

    def loss():
        R, _ = O.sma_forward_rms(Q, C, E, dH, S, eps, wq, we)
        return float((dR * R).sum())

    dQ, dC, dE, ddH, dwq, dwe = O.sma_backward_rms(Q, C, E, dH, S, eps, dR, None, wq, we)
    for name, x, got in (("Q", Q, dQ), ("C", C, dC), ("E", E, dE), ("dH", dH, ddH)):
        assert _rel(got, _fd(loss, x)) < 1e-6, name
    if weights:
        assert _rel(dwq, _fd(loss, wq)) < 1e-6
        assert _rel(dwe, _fd(loss, we)) < 1e-6
    else:
        assert not dwq.any() and not dwe.any()


def test_chain_through_chunk_states_matches_finite_differences():
    rng = np.random.default_rng(23)
    b, L, H, G, N, P, S, eps = 1, 10, 2, 1, 3, 2, 4, 1e-3
    X = rng.standard_normal((b, L, H, P))
    B = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    A = np.exp(-rng.uniform(0.05, 0.8, (b, L, H)))
    Q = rng.standard_normal((b, L, G, N))
    C = rng.standard_normal((b, L, G, N))
    E = rng.standard_normal((b, L, G, P))
    dR = rng.standard_normal((b, L, H, P))

    def loss():
        dH = O.chunk_states(X, B, A, S)
        R, _ = O.sma_forward_rms(Q, C, E, dH, S, eps)
        return float((dR * R).sum())

    dH = O.chunk_states(X, B, A, S)
    _, lse = O.sma_forward_rms(Q, C, E, dH, S, eps)
    _, _, _, ddH, _, _ = O.sma_backward_rms(Q, C, E, dH, S, eps, dR, lse)
    dX, dB, dA = O.chunk_states_backward(X, B, A, S, ddH)
    for name, x, got in (("X", X, dX), ("B", B, dB), ("A", A, dA)):
        assert _rel(got, _fd(loss, x)) < 1e-6, name


def test_scale_invariance_at_zero_eps():
    rng = np.random.default_rng(29)
    L, N, P, S = 24, 4, 5, 6
    M = O.num_chunks(L, S)
    Q, C = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    E = rng.standard_normal((L, P))
    dH = rng.standard_normal((M, N, P))
    dR = rng.standard_normal((L, P))
    dQ, dC, dE, ddH, _, _ = O.sma_head_backward_rms(Q, C, E, dH, S, 0.0, dR)
    np.testing.assert_allclose((dQ * Q).sum(axis=1), 0.0, atol=1e-10)
    np.testing.assert_allclose((dE * E).sum(axis=1), 0.0, atol=1e-10)
    assert np.abs(dQ[S:]).max() > 1e-3 and np.abs(dE[S:]).max() > 1e-3


def test_value_readout_matches_plain_branch():
    # entries +-1 and eps = 0: every normalisation is the identity at this
    # point, so the softmax weights and hence dC agree with the plain branch
    rng = np.random.default_rng(31)
    L, N, P, S = 30, 4, 6, 7
    M = O.num_chunks(L, S)
    pm = lambda shape: rng.choice([-1.0, 1.0], size=shape)
    Q, E, dH = pm((L, N)), pm((L, P)), pm((M, N, P))
    C = rng.standard_normal((L, N))
    dR = rng.standard_normal((L, P))
    _, dC0, _, _ = O.sma_head_backward(Q, C, E, dH, S, dR)
    _, dC1, _, _, _, _ = O.sma_head_backward_rms(Q, C, E, dH, S, 0.0, dR)
    np.testing.assert_allclose(dC1, dC0, rtol=1e-12, atol=1e-12)


def test_single_visible_chunk_closed_form():
    rng = np.random.default_rng(37)
    L, N, P, S = 8, 4, 3, 4                          # tokens 4..7 see chunk 0 only
    Q, C = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    E = rng.standard_normal((L, P))
    dH = rng.standard_normal((2, N, P))
    dR = rng.standard_normal((L, P))
    dQ, dC, dE, ddH, _, _ = O.sma_head_backward_rms(Q, C, E, dH, S, 1e-6, dR)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-14)     # p = 1 up to rounding
    np.testing.assert_allclose(dE, 0.0, atol=1e-14)
    np.testing.assert_allclose(dC[4:], dR[4:] @ dH[0].T, rtol=1e-12)
    np.testing.assert_allclose(dC[:4], 0.0)
    np.testing.assert_allclose(ddH[0], C[4:].T @ dR[4:], rtol=1e-12)   # value part only
    np.testing.assert_allclose(ddH[1], 0.0)

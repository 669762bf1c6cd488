"""Pins for the fp64 oracle, independent of the oracle itself.

Each test checks the oracle against something the paper or mathematics fixes:
brute force of the step recurrence, closed forms worked by hand, special
cases that reduce to a library routine, an independent streaming algorithm,
and the numbers the paper prints.  Citations refer to "DART: Decoded Attention
over Recurrent States for Efficient Long-Context Sequence Modeling"
(arXiv 2608.02032).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- chunk states
def test_decay_weights_closed_form():
    # constant decay a: w_s = a^(e-s) [§3 Eq. 5, §2 Eq. 3]
    a = np.full(7, 0.8)
    w = O.decay_weights(a)
    np.testing.assert_allclose(w, 0.8 ** np.arange(6, -1, -1), rtol=1e-15)
    # the writing token's own decay never enters its weight: a_0 is unused
    a2 = a.copy()
    a2[0] = 123.0
    np.testing.assert_array_equal(O.decay_weights(a2), w)
    assert O.decay_weights(np.array([0.3]))[0] == 1.0
    # deep underflow stays a clean zero, never NaN
    w = O.decay_weights(np.full(2000, 1e-3))
    assert np.isfinite(w).all() and w[0] == 0.0 and w[-1] == 1.0


def test_chunk_states_hand_example():
    # N = P = 1, L = 5, S = 2: chunks {0,1}, {2,3}, {4}  [§3 Eq. 5]
    X = np.array([[1.0], [2.0], [3.0], [4.0], [5.0]])
    B = np.ones((5, 1))
    a = np.array([0.5, 0.25, 0.5, 0.125, 0.9])
    dH = O.chunk_states_head(X, B, a, 2)[:, 0, 0]
    # dH0 = a1*B0X0 + B1X1 = 0.25 + 2 ; dH1 = a3*B2X2 + B3X3 = 0.375 + 4 ; dH2 = B4X4
    np.testing.assert_array_equal(dH, [2.25, 4.375, 5.0])
    # boundary states [App. A Eq. 18]: H[1] = a2 a3 H[0] + dH1, H[2] = a4 H[1] + dH2
    Hb = O.boundary_states(dH[:, None, None], a, 2)[:, 0, 0]
    np.testing.assert_allclose(Hb, [2.25, 0.5 * 0.125 * 2.25 + 4.375, 0.9 * 4.515625 + 5.0],
                               rtol=1e-15)


@pytest.mark.parametrize("L,S", [(37, 1), (37, 3), (37, 4), (37, 8), (16, 8), (5, 9)])
def test_chunk_states_brute_force(L, S):
    """The step recurrence [§2 Eq. 2] restarted from zero at each chunk start
    ends at dH_[c] on the chunk's last token; run once from t=0 it equals the
    chunk sums composed with inter-chunk decay [App. A Eq. 17-18]."""
    rng = np.random.default_rng(L * 100 + S)
    N, P = 3, 2
    X, B = rand(rng, L, P), rand(rng, L, N)
    a = rng.uniform(0.2, 1.0, L)
    dH = O.chunk_states_head(X, B, a, S)
    M = O.num_chunks(L, S)
    assert dH.shape == (M, N, P)
    full = O.ssm_recurrence(X, B, a)
    for c in range(M):
        s0, s1 = O.chunk_bounds(c, L, S)
        local = O.ssm_recurrence(X[s0:s1], B[s0:s1], a[s0:s1])
        np.testing.assert_allclose(local[-1], dH[c], rtol=1e-12, atol=1e-12)
    Hb = O.boundary_states(dH, a, S)
    for c in range(M):
        _, s1 = O.chunk_bounds(c, L, S)
        np.testing.assert_allclose(Hb[c], full[s1 - 1], rtol=1e-12, atol=1e-12)


def test_chunk_states_no_decay_is_plain_matmul():
    # A == 1  =>  dH_[c] = B_c^T X_c
    rng = np.random.default_rng(1)
    L, S, N, P = 50, 16, 5, 3
    X, B = rand(rng, L, P), rand(rng, L, N)
    dH = O.chunk_states_head(X, B, np.ones(L), S)
    for c in range(O.num_chunks(L, S)):
        s0, s1 = O.chunk_bounds(c, L, S)
        np.testing.assert_allclose(dH[c], np.matmul(B[s0:s1].T, X[s0:s1]), rtol=1e-13, atol=1e-13)


def test_chunk_states_full_decay_keeps_last_token():
    # A == 0  =>  only the chunk's last token survives: dH_[c] = B_e^T X_e
    rng = np.random.default_rng(2)
    L, S, N, P = 23, 6, 4, 3
    X, B = rand(rng, L, P), rand(rng, L, N)
    dH = O.chunk_states_head(X, B, np.zeros(L), S)
    for c in range(O.num_chunks(L, S)):
        e = O.chunk_bounds(c, L, S)[1] - 1
        np.testing.assert_array_equal(dH[c], np.outer(B[e], X[e]))


def test_chunk_states_unit_chunks():
    # S == 1  =>  dH_t = B_t^T X_t whatever the decay
    rng = np.random.default_rng(3)
    X, B = rand(rng, 9, 2), rand(rng, 9, 4)
    dH = O.chunk_states_head(X, B, rng.uniform(0, 1, 9), 1)
    for t in range(9):
        np.testing.assert_array_equal(dH[t], np.outer(B[t], X[t]))


def test_chunk_states_batched_groups():
    # heads sharing one projection group read the same B  [§3 Fig. 2; App. B.2]
    rng = np.random.default_rng(4)
    b, L, H, G, N, P, S = 2, 20, 4, 1, 3, 2, 8
    X, B, A = rand(rng, b, L, H, P), rand(rng, b, L, G, N), rng.uniform(0.5, 1, (b, L, H))
    dH = O.chunk_states(X, B, A, S)
    for bi in range(b):
        for h in range(H):
            np.testing.assert_array_equal(dH[bi, h], O.chunk_states_head(X[bi, :, h], B[bi, :, 0], A[bi, :, h], S))


# ------------------------------------------------------------------------ SMA
def test_sma_two_chunk_closed_form():
    """Token with two visible chunks, N=2, P=3, values worked by hand
    [§3 Eq. 8-10; App. C Eq. 32].  The 1/sqrt(N) scale, the roles of Q (routing),
    E (key decoding) and C (value readout) are all visible in the result."""
    dH = np.zeros((2, 2, 3))
    dH[0, 0, 0] = 1.0
    dH[1, 1, 1] = 2.0
    q, c, e = np.array([3.0, 1.0]), np.array([1.0, 1.0]), np.array([1.0, 1.0, 0.0])
    # K0 = dH0 e = (1,0), K1 = dH1 e = (0,2);  l0 = 3/sqrt2, l1 = 2/sqrt2
    l0, l1 = 3 / math.sqrt(2), 2 / math.sqrt(2)
    g0 = 1.0 / (1.0 + math.exp(l1 - l0))
    R, lse = O.sma_token(q, c, e, dH)
    np.testing.assert_allclose(R, [g0, 2 * (1 - g0), 0.0], rtol=1e-14, atol=1e-15)
    assert abs(lse - math.log(math.exp(l0) + math.exp(l1))) < 1e-13
    # the same through the per-head routine: token 2 of L=3, S=1 sees chunks 0, 1
    Q = np.stack([np.zeros(2), np.zeros(2), q])
    C = np.stack([np.zeros(2), np.zeros(2), c])
    E = np.stack([np.zeros(3), np.zeros(3), e])
    dH3 = np.concatenate([dH, 100 * np.ones((1, 2, 3))])  # own chunk must stay invisible
    Rh, lh = O.sma_head(Q, C, E, dH3, 1)
    np.testing.assert_allclose(Rh[2], R, rtol=1e-14, atol=1e-15)
    assert abs(lh[2] - lse) < 1e-13


def _random_head(rng, L, S, N, P, qscale=1.0):
    M = O.num_chunks(L, S)
    return (qscale * rand(rng, L, N), rand(rng, L, N), rand(rng, L, P), rand(rng, M, N, P))


def test_sma_first_chunk_empty_and_one_visible_chunk():
    rng = np.random.default_rng(5)
    L, S, N, P = 40, 8, 6, 4
    Q, C, E, dH = _random_head(rng, L, S, N, P)
    R, lse = O.sma_head(Q, C, E, dH, S)
    # chunk 0: empty history => R = 0, lse = -inf  [§3 after Eq. 10; §4 Algorithm 1, finalisation]
    assert (R[:S] == 0).all() and np.isneginf(lse[:S]).all()
    # chunk 1: a single visible chunk => softmax weight 1 => R_t = C_t dH_0, lse = l_{t,0}
    for t in range(S, 2 * S):
        np.testing.assert_allclose(R[t], C[t] @ dH[0], rtol=1e-12, atol=1e-12)
        assert abs(lse[t] - Q[t] @ (dH[0] @ E[t]) / math.sqrt(N)) < 1e-12


@pytest.mark.parametrize("zero", ["Q", "E"])
def test_sma_uniform_weights(zero):
    # Q == 0 or E == 0 => all logits 0 => g = 1/i, R_t = C_t mean_{c<i} dH_c, lse = log i
    rng = np.random.default_rng(6)
    L, S, N, P = 45, 9, 5, 3
    Q, C, E, dH = _random_head(rng, L, S, N, P)
    if zero == "Q":
        Q[:] = 0
    else:
        E[:] = 0
    R, lse = O.sma_head(Q, C, E, dH, S)
    for t in range(S, L):
        i = t // S
        np.testing.assert_allclose(R[t], C[t] @ dH[:i].mean(axis=0), rtol=1e-12, atol=1e-13)
        assert abs(lse[t] - math.log(i)) < 1e-13


def test_sma_planted_retrieval():
    # one chunk dominates the logits by >= 30 => R_t ~= C_t dH_{c*}
    rng = np.random.default_rng(7)
    N, P, n = 8, 4, 6
    dH = 0.01 * rand(rng, n, N, P)
    e = rand(rng, P)
    q = np.zeros(N)
    star = 3
    # make K_{c*} = dH_{c*} e point along q
    dH[star] = np.outer(np.ones(N), e) / (e @ e)  # dH e = 1-vector
    q[:] = 40.0 * math.sqrt(N) / N                 # l_{c*} = 40, others ~ 0
    c = rand(rng, N)
    R, lse = O.sma_token(q, c, e, dH)
    np.testing.assert_allclose(R, c @ dH[star], rtol=1e-9, atol=1e-12)
    assert abs(lse - 40.0) < 1e-6


def test_sma_matches_streaming_online_softmax():
    """App. C Eq. 29-31: the streaming recurrence over chunks, run here one
    chunk at a time, must give the oracle's R and lse."""
    rng = np.random.default_rng(8)
    N, P, n = 7, 5, 13
    q, c, e = rand(rng, N) * 3, rand(rng, N), rand(rng, P) * 3
    dH = rand(rng, n, N, P)
    m, d, o = -math.inf, 0.0, np.zeros(P)
    for j in range(n):
        x = q @ (dH[j] @ e) / math.sqrt(N)
        v = c @ dH[j]
        m_new = max(m, x)
        d = math.exp(m - m_new) * d + math.exp(x - m_new)
        o = math.exp(m - m_new) * o + math.exp(x - m_new) * v
        m = m_new
    R, lse = O.sma_token(q, c, e, dH)
    np.testing.assert_allclose(R, o / d, rtol=1e-12, atol=1e-13)
    assert abs(lse - (m + math.log(d))) < 1e-12


def test_sma_linear_in_read_vector():
    # logits do not depend on C, so R is linear in C
    rng = np.random.default_rng(9)
    L, S, N, P = 30, 6, 4, 3
    Q, C1, E, dH = _random_head(rng, L, S, N, P)
    C2 = rand(rng, L, N)
    R1, _ = O.sma_head(Q, C1, E, dH, S)
    R2, _ = O.sma_head(Q, C2, E, dH, S)
    R3, _ = O.sma_head(Q, 2 * C1 - 3 * C2, E, dH, S)
    np.testing.assert_allclose(R3, 2 * R1 - 3 * R2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("L,S", [(50, 7), (64, 16), (33, 33), (10, 1)])
def test_sma_head_equals_per_token(L, S):
    # the chunk-batched routine equals the per-token definition, ragged tail included
    rng = np.random.default_rng(L + S)
    N, P = 6, 5
    Q, C, E, dH = _random_head(rng, L, S, N, P, qscale=2.0)
    R, lse = O.sma_head(Q, C, E, dH, S)
    for t in range(L):
        r, l = O.sma_token(Q[t], C[t], E[t], dH[: t // S])
        np.testing.assert_allclose(R[t], r, rtol=1e-12, atol=1e-13)
        assert (np.isneginf(l) and np.isneginf(lse[t])) or abs(lse[t] - l) < 1e-12


def test_sma_forward_group_sharing():
    rng = np.random.default_rng(10)
    b, L, H, G, N, P, S = 2, 24, 4, 2, 3, 4, 6
    Q, C, E = rand(rng, b, L, G, N), rand(rng, b, L, G, N), rand(rng, b, L, G, P)
    dH = rand(rng, b, H, O.num_chunks(L, S), N, P)
    R, lse = O.sma_forward(Q, C, E, dH, S)
    assert R.shape == (b, L, H, P) and lse.shape == (b, H, L)
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            r, l = O.sma_head(Q[bi, :, g], C[bi, :, g], E[bi, :, g], dH[bi, h], S)
            np.testing.assert_array_equal(R[bi, :, h], r)
            np.testing.assert_array_equal(lse[bi, h], l)


# ------------------------------------------------------------------- residual
def test_gated_residual_special_cases():
    rng = np.random.default_rng(11)
    Y, R = rand(rng, 5, 3, 4), rand(rng, 5, 3, 4)
    # g == 0: the SMA-removal ablation [§5.3 "SMA Branch"] leaves the SSM output untouched
    np.testing.assert_array_equal(O.gated_residual(Y, np.zeros((5, 3, 4)), R), Y)
    # g == 1, Y == 0: out is the SMA readout itself
    np.testing.assert_array_equal(O.gated_residual(np.zeros_like(Y), np.ones((5, 3, 4)), R), R)
    # scalar gate per token [§3 Eq. 11] == per-channel gate with equal channels
    g = rng.random((5, 3))
    np.testing.assert_array_equal(O.gated_residual(Y, g, R, gate_per_channel=False),
                                  O.gated_residual(Y, np.repeat(g[..., None], 4, -1), R))


# --------------------------------------------------------------------- decode
def test_decode_special_cases_and_consistency():
    rng = np.random.default_rng(12)
    b, H, G, Mx, N, P = 3, 2, 2, 5, 4, 3
    q, c, e = rand(rng, b, G, N), rand(rng, b, G, N), rand(rng, b, G, P)
    cache = rand(rng, b, H, Mx, N, P)
    R, lse = O.sma_decode(q, c, e, cache, [0, 1, 5])
    assert (R[0] == 0).all() and np.isneginf(lse[0]).all()          # n_b = 0
    for h in range(H):
        np.testing.assert_allclose(R[1, h], c[1, h] @ cache[1, h, 0], rtol=1e-12)  # n_b = 1
    # decode of a token of chunk i against the cache dH_0..i-1 equals that
    # token's row of the forward pass  [§4 "Inference Cache"]
    L, S = 25, 5
    Q, C, E, dH = _random_head(rng, L, S, N, P)
    Rf, lf = O.sma_head(Q, C, E, dH, S)
    for t in (S, 2 * S + 3, L - 1):
        i = t // S
        Rd, ld = O.sma_decode(Q[t][None, None], C[t][None, None], E[t][None, None],
                              dH[None, None], [i])
        np.testing.assert_allclose(Rd[0, 0], Rf[t], rtol=1e-12, atol=1e-13)
        assert abs(ld[0, 0] - lf[t]) < 1e-12


# ---------------------------------------------------------- cache accounting
def test_cache_ratio_matches_paper():
    with open(os.path.join(GOLDEN, "cache_ratio.json")) as f:
        g = json.load(f)
    r = O.cache_ratio(g["N"], g["S"])
    assert round(100 * r) == g["ratio_percent"]
    assert round(100 * (1 - r)) == g["saving_percent"]
    # the same from tensor sizes: chunk memories [M][N][P] vs a KV cache [L][2][P]
    L, N, P, S = 65536, g["N"], 64, g["S"]
    chunk_cache = np.zeros((O.num_chunks(L, S), N, P), dtype=np.float16)
    kv_cache = np.zeros((L, 2, P), dtype=np.float16)
    assert chunk_cache.nbytes / kv_cache.nbytes == r


# ---- decode-side cache maintenance --------------------------------------------


def test_decode_stream_reproduces_chunk_states():
    """Streaming the in-progress chunk update token by token closes every
    complete chunk with exactly the Eq. 5 memory, and the state after a
    partial last chunk is that chunk's Eq. 5 memory too (it decays to its
    last present token)."""
    rng = np.random.default_rng(17)
    for L, S in ((40, 8), (37, 8), (16, 16), (5, 8)):
        X, B = rng.standard_normal((L, 3)), rng.standard_normal((L, 4))
        a = np.exp(-rng.uniform(0.0, 1.0, L))
        cache, state = O.decode_stream(X, B, a, S)
        ref = O.chunk_states_head(X, B, a, S)
        assert cache.shape[0] == L // S
        np.testing.assert_allclose(cache, ref[: L // S], rtol=1e-12, atol=1e-12)
        if L % S:
            np.testing.assert_allclose(state, ref[-1], rtol=1e-12, atol=1e-12)
        else:
            assert np.abs(state).max() == 0


def test_decode_state_matches_step_recurrence_from_chunk_start():
    """Within a chunk the state is the Eq. 2 recurrence restarted from zero at
    the chunk's first token."""
    rng = np.random.default_rng(19)
    L, S = 29, 10
    X, B = rng.standard_normal((L, 2)), rng.standard_normal((L, 3))
    a = np.exp(-rng.uniform(0.0, 2.0, L))
    state = np.zeros((3, 2))
    for t in range(L):
        state, closed = O.decode_state_update(state, X[t], B[t], a[t], t, S)
        s0 = (t // S) * S
        want = O.ssm_recurrence(X[s0:t + 1], B[s0:t + 1], a[s0:t + 1])[-1]
        got = closed if closed is not None else state
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)

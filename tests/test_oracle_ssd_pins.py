"""Pins for the oracle's SSM branch output Y_t = C_t H_t [§2 Eq. 2; App. A
Eq. 15] and its chunked scan [App. A Eq. 17-24].

* The chunked scan (chunk contributions, boundary states, intra- and
  inter-chunk terms) equals the step recurrence for chunk sizes that divide
  L, do not divide it, exceed it and equal 1, with and without an initial
  state.
* Closed forms: with every a_t = 1 the output is causal linear attention,
  Y = tril(C B^T) X (numpy); with every a_t = 0 only the token itself is
  read, Y_t = (C_t . B_t) X_t; the structured-attention form of §2 Eq. 4,
  Y = (L_SSD o C B^T) X with L_SSD built entry by entry; an initial state
  alone decays as Y_t = (prod_{k<=t} a_k) C_t H0.
* The chunk contributions returned with Y are the pinned chunk states.
"""
import numpy as np
import pytest

import oracle as O


def _draw(rng, L, N, P, lo=0.3, hi=1.0):
    return (rng.standard_normal((L, P)), rng.standard_normal((L, N)), rng.standard_normal((L, N)),
            rng.uniform(lo, hi, L))


@pytest.mark.parametrize("L,S", [(24, 8), (23, 5), (10, 16), (9, 1), (17, 17)])
@pytest.mark.parametrize("with_h0", [False, True])
def test_chunked_scan_equals_recurrence(L, S, with_h0):
    rng = np.random.default_rng(L * 100 + S)
    N, P = 3, 4
    X, B, C, a = _draw(rng, L, N, P)
    a[L // 2] = 0.0                                  # a full reset inside the sequence
    H0 = rng.standard_normal((N, P)) if with_h0 else None
    Y_rec, H_rec = O.ssm_output_head(X, B, C, a, H0)
    Y_chk, dH, H_chk = O.ssd_chunked_head(X, B, C, a, S, H0)
    np.testing.assert_allclose(Y_chk, Y_rec, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(H_chk, H_rec, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dH, O.chunk_states_head(X, B, a, S), rtol=0, atol=0)


def test_unit_decay_is_causal_linear_attention():
    rng = np.random.default_rng(1)
    L, N, P = 15, 4, 3
    X, B, C, _ = _draw(rng, L, N, P)
    Y, _ = O.ssm_output_head(X, B, C, np.ones(L))
    np.testing.assert_allclose(Y, np.tril(C @ B.T) @ X, rtol=1e-12, atol=1e-12)


def test_zero_decay_reads_only_the_token():
    rng = np.random.default_rng(2)
    L, N, P = 11, 5, 2
    X, B, C, _ = _draw(rng, L, N, P)
    Y, _ = O.ssm_output_head(X, B, C, np.zeros(L))
    np.testing.assert_allclose(Y, (C * B).sum(axis=1)[:, None] * X, rtol=1e-12, atol=1e-12)


def test_structured_attention_form():
    rng = np.random.default_rng(3)
    L, N, P = 9, 3, 2
    X, B, C, a = _draw(rng, L, N, P)
    Lssd = np.zeros((L, L))
    for i in range(L):
        for j in range(i + 1):
            Lssd[i, j] = np.prod(a[j + 1:i + 1])     # empty product = 1 on the diagonal
    Y, _ = O.ssm_output_head(X, B, C, a)
    np.testing.assert_allclose(Y, (Lssd * (C @ B.T)) @ X, rtol=1e-12, atol=1e-12)


def test_initial_state_alone_decays():
    rng = np.random.default_rng(4)
    L, N, P = 7, 3, 2
    _, _, C, a = _draw(rng, L, N, P)
    H0 = rng.standard_normal((N, P))
    Y, Hl = O.ssm_output_head(np.zeros((L, P)), np.zeros((L, N)), C, a, H0)
    np.testing.assert_allclose(Y, np.cumprod(a)[:, None] * (C @ H0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Hl, np.prod(a) * H0, rtol=1e-12)

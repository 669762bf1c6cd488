"""Pins for the oracle's RMS-normalised score branch [App. B.1 Eq. 25-27],
independent of its own formulas.

* Hand-worked RMSNorm and inverse-RMS values (non-square shapes, so a
  reduction over the wrong axis fails), with and without eps and weights.
* Reduction to the plain branch: with eps = 0 and inputs whose RMS is already
  1 (entries +-1), every normalisation is the identity and the branch must
  equal the pinned unnormalised ``sma_head``; with RMSNorm weights it must
  equal the plain branch on the weighted Q and E.
* Invariances of the definition (eps = 0): scaling Q_t or E_t by a positive
  number, or a chunk memory's key rows by positive factors d_n with C scaled
  by 1/d_n, changes neither R nor lse.  The last one fails if r is taken
  along the wrong axis or if the value readout were normalised too.
* Special cases and cross-call consistency: first chunk, one visible chunk,
  and decode of a token equals its forward row.
"""
import math

import numpy as np
import pytest

import oracle as O


def test_rms_norm_hand_values():
    x = np.array([[3.0, 4.0], [1.0, -1.0]])
    # mean of squares 12.5 and 1
    want = np.array([[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], [1.0, -1.0]])
    np.testing.assert_allclose(O.rms_norm(x, 0.0), want, rtol=1e-15)
    np.testing.assert_allclose(O.rms_norm(x, 0.5), x / np.sqrt(np.array([[13.0], [1.5]])), rtol=1e-15)
    w = np.array([2.0, 0.5])
    np.testing.assert_allclose(O.rms_norm(x, 0.0, w), want * w, rtol=1e-15)
    # three channels: the mean is over the last axis only
    y = np.array([1.0, 2.0, 2.0])                     # mean of squares 3
    np.testing.assert_allclose(O.rms_norm(y, 0.0), y / math.sqrt(3.0), rtol=1e-15)


def test_chunk_inv_rms_hand_values():
    # one chunk memory, N = 2 key rows, P = 3 value columns
    dH = np.array([[[1.0, 2.0, 2.0], [0.0, 0.0, 0.0]]])
    r = O.chunk_inv_rms(dH, 1e-6)
    assert r.shape == (1, 2)
    np.testing.assert_allclose(r[0, 0], 1 / math.sqrt(3.0 + 1e-6), rtol=1e-15)
    np.testing.assert_allclose(r[0, 1], 1000.0, rtol=1e-12)   # all-zero row: eps^(-1/2)


def _pm1(rng, shape):
    return rng.choice([-1.0, 1.0], size=shape)


@pytest.mark.parametrize("L,S", [(40, 8), (37, 5)])
def test_unit_rms_inputs_reduce_to_plain_branch(L, S):
    rng = np.random.default_rng(11)
    N, P = 4, 6
    M = O.num_chunks(L, S)
    Q, E, dH = _pm1(rng, (L, N)), _pm1(rng, (L, P)), _pm1(rng, (M, N, P))
    C = rng.standard_normal((L, N))
    R0, lse0 = O.sma_head(Q, C, E, dH, S)
    R1, lse1 = O.sma_head_rms(Q, C, E, dH, S, 0.0)
    np.testing.assert_allclose(R1, R0, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse1), np.isinf(lse0))
    f = np.isfinite(lse0)
    np.testing.assert_allclose(lse1[f], lse0[f], rtol=1e-12)
    # RMSNorm weights multiply the normalised Q and E per channel
    wq, we = rng.uniform(0.5, 2.0, N), rng.uniform(0.5, 2.0, P)
    R0, lse0 = O.sma_head(Q * wq, C, E * we, dH, S)
    R1, lse1 = O.sma_head_rms(Q, C, E, dH, S, 0.0, wq, we)
    np.testing.assert_allclose(R1, R0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse1[f], lse0[f], rtol=1e-12)


def test_score_invariances():
    rng = np.random.default_rng(12)
    L, S, N, P = 48, 8, 5, 3
    M = O.num_chunks(L, S)
    Q, C = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    E, dH = rng.standard_normal((L, P)), rng.standard_normal((M, N, P))
    R0, lse0 = O.sma_head_rms(Q, C, E, dH, S, 0.0)
    f = np.isfinite(lse0)
    # per-token positive scale of Q and E
    a = rng.uniform(0.1, 10.0, (L, 1))
    b = rng.uniform(0.1, 10.0, (L, 1))
    R1, lse1 = O.sma_head_rms(Q * a, C, E * b, dH, S, 0.0)
    np.testing.assert_allclose(R1, R0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse1[f], lse0[f], rtol=1e-10)
    # key rows of every chunk memory scaled by d_n > 0, C by 1 / d_n
    d = rng.uniform(0.2, 5.0, (M, N))
    dH2 = dH * d[:, :, None]
    # C dH is unchanged only when every chunk uses the same d: use one d
    d1 = d[0]
    R2, lse2 = O.sma_head_rms(Q, C / d1, E, dH * d1[None, :, None], S, 0.0)
    np.testing.assert_allclose(R2, R0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse2[f], lse0[f], rtol=1e-10)
    # factors d_{c,n} that differ per chunk still leave every logit, hence
    # lse, unchanged (only the value readouts change)
    _, lse3 = O.sma_head_rms(Q, C, E, dH2, S, 0.0)
    np.testing.assert_allclose(lse3[f], lse0[f], rtol=1e-10)
    # the unnormalised branch is not invariant (the pins above are not vacuous)
    _, lse4 = O.sma_head(Q, C, E, dH2, S)
    assert np.abs(lse4[f] - lse0[f]).max() > 1e-3


def test_special_cases_and_decode_consistency():
    rng = np.random.default_rng(13)
    L, S, N, P = 24, 6, 4, 3
    M = O.num_chunks(L, S)
    Q, C = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    E, dH = rng.standard_normal((L, P)), rng.standard_normal((M, N, P))
    wq, we = rng.uniform(0.5, 2.0, N), rng.uniform(0.5, 2.0, P)
    R, lse = O.sma_head_rms(Q, C, E, dH, S, 1e-5, wq, we)
    assert np.all(R[:S] == 0) and np.all(np.isneginf(lse[:S]))
    np.testing.assert_allclose(R[S:2 * S], C[S:2 * S] @ dH[0], rtol=1e-12)   # one chunk: weight 1
    # decode of every token against the chunks before it equals its row
    for t in (S, 2 * S + 3, L - 1):
        i = t // S
        cache = np.zeros((1, 1, M, N, P))
        cache[0, 0, :i] = dH[:i]
        Rd, ld = O.sma_decode_rms(Q[t][None, None], C[t][None, None], E[t][None, None], cache,
                                  np.array([i]), 1e-5, 1, wq, we)
        np.testing.assert_allclose(Rd[0, 0], R[t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ld[0, 0], lse[t], rtol=1e-12)
    Rd, ld = O.sma_decode_rms(Q[:1][None], C[:1][None], E[:1][None], dH[None, None], np.array([0]), 1e-5)
    assert np.all(Rd == 0) and np.isneginf(ld[0, 0])


def test_batched_forward_group_sharing():
    rng = np.random.default_rng(14)
    b, L, H, G, N, P, S = 2, 20, 4, 2, 3, 2, 5
    M = O.num_chunks(L, S)
    Q, C = rng.standard_normal((b, L, G, N)), rng.standard_normal((b, L, G, N))
    E, dH = rng.standard_normal((b, L, G, P)), rng.standard_normal((b, H, M, N, P))
    R, lse = O.sma_forward_rms(Q, C, E, dH, S, 1e-6)
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            r, l = O.sma_head_rms(Q[bi, :, g], C[bi, :, g], E[bi, :, g], dH[bi, h], S, 1e-6)
            np.testing.assert_array_equal(R[bi, :, h], r)
            np.testing.assert_array_equal(lse[bi, h], l)

"""fp64 CPU oracle for DART chunk state memories and state-memory attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables) and imports nothing from it.

Every function below is the plain definition from the paper
"DART: Decoded Attention over Recurrent States for Efficient Long-Context
Sequence Modeling" (arXiv 2608.02032), evaluated in float64 with numpy.
Citations name the paper's section and equation, e.g. [§3 Eq. 5].

Conventions (the paper's notation, 0-based indices):
  * tokens t = 0..L-1, chunk size S, chunk(t) = t // S (the paper writes the
    1-based c(t) = ceil(t/S)); chunk c holds tokens [cS, min((c+1)S, L)), so
    M = ceil(L/S) chunks, the last one possibly shorter;
  * X (L, P), B (L, N), C (L, N), Q (L, N), E (L, P): one row per token;
  * chunk state memories dH (M, N, P), each the paper's N x P matrix
    (key axis N, value axis P) -- the oracle keeps the paper's orientation;
  * a (L,): the scalar decay a_t of A_t = a_t I_N  [§2 Eq. 2].

Readings where the paper leaves a step open (each is also listed in the
design notes):
  * a token sees chunk c iff c < chunk(t) -- strictly earlier chunks only
    [§3 Eq. 10; §4 Algorithm 1, loop over history chunks j < i];
  * a token with no visible chunk gets R_t = 0 and lse_t = -inf
    [§3 text after Eq. 10; §4 Algorithm 1, finalisation];
  * the gate is given after its activation, either one scalar per token
    (the paper's G_t) or one value per channel, and out = Y_ssm + g * R
    [§3 Eq. 11];
  * a partial last chunk decays to its own last token (e(c) is the last index
    actually in the chunk) [§3 text under Eq. 5].

  * the RMS-normalised score branch [App. B.1 Eq. 25-27] uses one eps for
    both RMSNorms and for r_c, and an optional per-channel RMSNorm weight
    applied after the normalisation;
  * the backward pass takes the loss gradient of ``out`` (or of R) and the
    forward's saved lse, and recovers the chunk weights as p = exp(l - lse)
    [App. C Eq. 33-35]; gradients of projections shared by a group of heads
    are summed over those heads.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``,
``tests/test_oracle_backward_pins.py``, ``tests/test_oracle_rms_pins.py`` and
``tests/test_oracle_ssd_pins.py`` against brute force, closed forms,
special cases, central finite differences (the backward) and the paper's
printed numbers; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "num_chunks",
    "chunk_bounds",
    "decay_weights",
    "chunk_states_head",
    "chunk_states",
    "ssm_recurrence",
    "boundary_states",
    "sma_token",
    "sma_head",
    "sma_forward",
    "gated_residual",
    "sma_decode",
    "cache_ratio",
    "sma_head_backward",
    "sma_token_backward",
    "sma_backward",
    "gated_residual_backward",
    "chunk_states_head_backward",
    "chunk_states_backward",
    "decode_state_update",
    "decode_stream",
    "rms_norm",
    "chunk_inv_rms",
    "sma_token_rms",
    "sma_head_rms",
    "sma_forward_rms",
    "sma_decode_rms",
    "rms_norm_backward",
    "sma_head_backward_rms",
    "sma_backward_rms",
    "ssm_output_head",
    "ssd_chunked_head",
    "ssm_output",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def num_chunks(L: int, S: int) -> int:
    """M = ceil(L / S)  [§4 "Training Complexity"; §4 Algorithm 1, chunking]."""
    return -(-L // S)


def chunk_bounds(c: int, L: int, S: int) -> tuple[int, int]:
    """Token range [s0, s1) of chunk c; e(c) = s1 - 1 is its last index [§3]."""
    return c * S, min((c + 1) * S, L)


def decay_weights(a_chunk) -> np.ndarray:
    """Weights w_s = A_{s+1:e(c)} = prod_{k=s+1}^{e(c)} a_k for the tokens of
    one chunk, in token order  [§3 Eq. 5 and the text under it; §2 Eq. 3].

    The product starts at s+1: the writing token's own decay is not applied,
    and the chunk's last token gets the empty product, 1.  Computed as a
    suffix product (never as a ratio of prefix products, which would divide
    0 by 0 once the prefix underflows)."""
    a = _f64(a_chunk)
    n = a.shape[0]
    w = np.empty(n, dtype=np.float64)
    if n == 0:
        return w
    w[n - 1] = 1.0
    for s in range(n - 2, -1, -1):
        w[s] = w[s + 1] * a[s + 1]
    return w


def chunk_states_head(X, B, a, S: int) -> np.ndarray:
    """Chunk state contributions of one head  [§3 Eq. 5; App. A Eq. 20]:

        dH_[c] = sum_{s in [c]} A_{s+1:e(c)} B_s^T X_s      (N x P)

    X (L, P), B (L, N), a (L,)  ->  dH (M, N, P)."""
    X, B, a = _f64(X), _f64(B), _f64(a)
    L, P = X.shape
    N = B.shape[1]
    M = num_chunks(L, S)
    dH = np.zeros((M, N, P), dtype=np.float64)
    for c in range(M):
        s0, s1 = chunk_bounds(c, L, S)
        w = decay_weights(a[s0:s1])
        # sum_s w_s * outer(B_s, X_s), written as one matrix product
        dH[c] = B[s0:s1].T @ (w[:, None] * X[s0:s1])
    return dH


def chunk_states(X, B, A, S: int) -> np.ndarray:
    """Batched chunk_states_head.  X (b, L, H, P), B (b, L, G, N),
    A (b, L, H)  ->  dH (b, H, M, N, P).  Head h reads projection group
    h // (H // G)  [§3 Fig. 2 caption; App. B.2]."""
    X, B, A = _f64(X), _f64(B), _f64(A)
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    assert H % G == 0
    hpg = H // G
    out = np.zeros((b, H, num_chunks(L, S), N, P), dtype=np.float64)
    for bi in range(b):
        for h in range(H):
            out[bi, h] = chunk_states_head(X[bi, :, h], B[bi, :, h // hpg], A[bi, :, h], S)
    return out


def ssm_recurrence(X, B, a, H0=None) -> np.ndarray:
    """Brute-force Mamba-2 step recurrence  [§2 Eq. 2; App. A Eq. 15]:

        H_t = a_t H_{t-1} + B_t^T X_t,   H_{-1} = H0 (zero by default)

    X (L, P), B (L, N), a (L,)  ->  all states H (L, N, P)."""
    X, B, a = _f64(X), _f64(B), _f64(a)
    L, P = X.shape
    N = B.shape[1]
    Hs = np.zeros((L, N, P), dtype=np.float64)
    h = np.zeros((N, P)) if H0 is None else _f64(H0).copy()
    for t in range(L):
        h = a[t] * h + np.outer(B[t], X[t])
        Hs[t] = h
    return Hs


def boundary_states(dH, a, S: int) -> np.ndarray:
    """Chunk-boundary states from the chunk contributions  [App. A Eq. 17-18]:

        H_[c] = A_{a_c:b_c} H_[c-1] + dH_[c],   H_[-1] = 0

    where A_{a_c:b_c} is the product of the decays of every token of chunk c.
    dH (M, N, P), a (L,)  ->  H_[c] (M, N, P)."""
    dH, a = _f64(dH), _f64(a)
    L = a.shape[0]
    M = dH.shape[0]
    out = np.zeros_like(dH)
    prev = np.zeros(dH.shape[1:])
    for c in range(M):
        s0, s1 = chunk_bounds(c, L, S)
        decay = 1.0
        for k in range(s0, s1):
            decay *= a[k]
        prev = decay * prev + dH[c]
        out[c] = prev
    return out


def sma_token(q, c, e, dH_visible):
    """State-memory attention of one token over its visible chunk memories
    [§3 Eq. 8-10]:

        V_c = C_t dH_c (P),  K_c = dH_c E_t (N),  l_c = Q_t K_c / sqrt(N)
        g = softmax_c(l),    R_t = sum_c g_c V_c

    q, c (N,), e (P,), dH_visible (n, N, P).  Returns (R (P,), lse) with
    lse = log sum_c exp(l_c)  [App. C Eq. 32]; an empty set gives (0, -inf)
    [§3 text after Eq. 10]."""
    q, c, e, dH = _f64(q), _f64(c), _f64(e), _f64(dH_visible)
    N, P = dH.shape[1], dH.shape[2]
    n = dH.shape[0]
    if n == 0:
        return np.zeros(P), -math.inf
    V = np.einsum("n,cnp->cp", c, dH)          # value readout C_t dH_c  [Eq. 6, 8]
    K = np.einsum("cnp,p->cn", dH, e)          # key readout dH_c E_t    [Eq. 6, 8]
    logits = (K @ q) / math.sqrt(N)            # [Eq. 9]
    m = logits.max()
    p = np.exp(logits - m)                     # stable softmax [App. C Eq. 28]
    d = p.sum()
    R = (p[:, None] * V).sum(axis=0) / d       # [Eq. 10]
    return R, m + math.log(d)                  # [App. C Eq. 32]


def sma_head(Q, C, E, dH, S: int):
    """SMA readout of one head for every token  [§3 Eq. 8-10]:
    Q, C (L, N), E (L, P), dH (M, N, P)  ->  R (L, P), lse (L,).

    The tokens of one target chunk i share the visible set {0..i-1}, so the
    same formulas as ``sma_token`` are evaluated for all of them at once with
    matrix products; no term is reordered or dropped."""
    Q, C, E, dH = _f64(Q), _f64(C), _f64(E), _f64(dH)
    L, N = Q.shape
    P = E.shape[1]
    M = num_chunks(L, S)
    R = np.zeros((L, P), dtype=np.float64)
    lse = np.full(L, -math.inf, dtype=np.float64)
    scale = 1.0 / math.sqrt(N)
    for i in range(1, M):
        s0, s1 = chunk_bounds(i, L, S)
        hist = dH[:i]                                       # (i, N, P)
        V = np.einsum("tn,cnp->tcp", C[s0:s1], hist, optimize=True)   # C_t dH_c
        K = np.einsum("cnp,tp->tcn", hist, E[s0:s1], optimize=True)   # dH_c E_t
        logits = np.einsum("tn,tcn->tc", Q[s0:s1], K) * scale
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        d = p.sum(axis=1, keepdims=True)
        R[s0:s1] = np.einsum("tc,tcp->tp", p, V, optimize=True) / d
        lse[s0:s1] = (m + np.log(d))[:, 0]
    return R, lse


def sma_forward(Q, C, E, dH, S: int):
    """Batched sma_head.  Q, C (b, L, G, N), E (b, L, G, P),
    dH (b, H, M, N, P)  ->  R (b, L, H, P), lse (b, H, L)."""
    Q, C, E = _f64(Q), _f64(C), _f64(E)
    b, L, G, N = Q.shape
    H = dH.shape[1]
    P = E.shape[3]
    hpg = H // G
    R = np.zeros((b, L, H, P))
    lse = np.zeros((b, H, L))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            R[bi, :, h], lse[bi, h] = sma_head(Q[bi, :, g], C[bi, :, g], E[bi, :, g], dH[bi, h], S)
    return R, lse


def gated_residual(Y, gate, R, gate_per_channel: bool = True) -> np.ndarray:
    """Gated residual  Y_t = C_t H_t + G_t R_t  [§3 Eq. 11], with the SSM
    branch output C_t H_t given as Y.  ``gate`` is post-activation: shape
    (..., P) when per channel, else (...) and broadcast over P."""
    Y, gate, R = _f64(Y), _f64(gate), _f64(R)
    g = gate if gate_per_channel else gate[..., None]
    return Y + g * R


def sma_decode(q, c, e, cache, n_chunks, hpg: int = 1):
    """Decode: one new token per batch row against its chunk-memory cache
    [§4 "Inference Cache"; §3 Eq. 8-10].  The new token lies after the last
    complete cached chunk, so every cached chunk 0..n_b-1 is visible.

    q, c (b, G, N), e (b, G, P), cache (b, H, Mmax, N, P), n_chunks (b,)
    ->  R (b, H, P), lse (b, H)."""
    q, c, e, cache = _f64(q), _f64(c), _f64(e), _f64(cache)
    b, H = cache.shape[0], cache.shape[1]
    P = cache.shape[4]
    R = np.zeros((b, H, P))
    lse = np.zeros((b, H))
    for bi in range(b):
        nb = int(n_chunks[bi])
        for h in range(H):
            g = h // hpg
            R[bi, h], lse[bi, h] = sma_token(q[bi, g], c[bi, g], e[bi, g], cache[bi, h, :nb])
    return R, lse


def cache_ratio(N: int, S: int) -> float:
    """Chunk-memory cache over the matched token-level KV cache, per head
    [§4 Eq. 14]: (L N P / S) / (2 L P) = N / (2 S)."""
    return N / (2.0 * S)


def decode_state_update(state, x, B_t, a_t, pos: int, S: int):
    """One decode step of the in-progress chunk memory  [§2 Eq. 2 restricted
    to the current chunk; App. A Eq. 20; §4 "Inference Cache"]:

        state <- a_t state + B_t^T x_t          (N x P, zero at a chunk's start)

    The token at absolute position ``pos`` closes its chunk when
    pos % S == S - 1; the closed chunk's memory is then returned and the state
    restarts from zero.  Returns (new_state, closed_memory_or_None)."""
    state, x, B_t = _f64(state), _f64(x), _f64(B_t)
    new = float(a_t) * state + np.outer(B_t, x)
    if pos % S == S - 1:
        return np.zeros_like(new), new
    return new, None


def decode_stream(X, B, a, S: int):
    """Run decode_state_update over a whole sequence of one head:
    X (L, P), B (L, N), a (L,)  ->  (cache of the closed chunks (L // S, N, P),
    in-progress state after the last token (N, P))."""
    X, B, a = _f64(X), _f64(B), _f64(a)
    L, P = X.shape
    N = B.shape[1]
    state = np.zeros((N, P))
    cache = []
    for t in range(L):
        state, closed = decode_state_update(state, X[t], B[t], a[t], t, S)
        if closed is not None:
            cache.append(closed)
    return (np.stack(cache) if cache else np.zeros((0, N, P))), state


# ---------------------------------------------------------------------------
# Backward pass.  The paper trains through the SMA branch with recomputation
# [§4 "Efficient Training"; App. C "Recomputation"]: the forward keeps only R
# and lse, and the backward recovers the chunk weights from recomputed logits
# as p = exp(l - lse)  [App. C Eq. 33-35].  The gradients below are the chain
# rule through the forward definitions, written out term by term.
# ---------------------------------------------------------------------------


def gated_residual_backward(dout, gate, R, gate_per_channel: bool = True):
    """Gradients of out = Y + g * R  [§3 Eq. 11] for a loss gradient dout:
    returns (dY, dR, dgate) with dY = dout, dR = g * dout and dgate = dout * R
    (summed over P for a scalar gate)."""
    dout, gate, R = _f64(dout), _f64(gate), _f64(R)
    g = gate if gate_per_channel else gate[..., None]
    dg = dout * R if gate_per_channel else (dout * R).sum(axis=-1)
    return dout.copy(), g * dout, dg


def sma_head_backward(Q, C, E, dH, S: int, dR, lse=None):
    """Gradients of the SMA readout of one head  [§3 Eq. 8-10]:
    Q, C (L, N), E (L, P), dH (M, N, P), dR (L, P) = dLoss/dR
    ->  dQ (L, N), dC (L, N), dE (L, P), d_dH (M, N, P).

    With l_tc = Q_t dH_c E_t / sqrt(N), p_tc = exp(l_tc - lse_t) the chunk
    weights [App. C Eq. 35], V_tc = C_t dH_c and R_t = sum_c p_tc V_tc:
        dV_tc = p_tc dR_t
        dp_tc = dR_t . V_tc,      dl_tc = p_tc (dp_tc - sum_c' p_tc' dp_tc')
        dC_t  = sum_c dH_c dV_tc
        dQ_t  = sum_c dl_tc dH_c E_t / sqrt(N)
        dE_t  = sum_c dl_tc dH_c^T Q_t / sqrt(N)
        d dH_c = sum_{t: c < chunk(t)} C_t^T dV_tc + dl_tc Q_t^T E_t / sqrt(N)
    (sum_c' p_tc' dp_tc' = dR_t . R_t).  ``lse`` defaults to the forward's."""
    Q, C, E, dH, dR = _f64(Q), _f64(C), _f64(E), _f64(dH), _f64(dR)
    L, N = Q.shape
    P = E.shape[1]
    M = num_chunks(L, S)
    if lse is None:
        _, lse = sma_head(Q, C, E, dH, S)
    lse = _f64(lse)
    scale = 1.0 / math.sqrt(N)
    dQ = np.zeros((L, N))
    dC = np.zeros((L, N))
    dE = np.zeros((L, P))
    ddH = np.zeros((M, N, P))
    for i in range(1, M):
        s0, s1 = chunk_bounds(i, L, S)
        hist = dH[:i]                                                       # (i, N, P)
        V = np.einsum("tn,cnp->tcp", C[s0:s1], hist, optimize=True)          # C_t dH_c
        K = np.einsum("cnp,tp->tcn", hist, E[s0:s1], optimize=True)          # dH_c E_t
        logits = np.einsum("tn,tcn->tc", Q[s0:s1], K) * scale                # [Eq. 9]
        p = np.exp(logits - lse[s0:s1, None])                                # [App. C Eq. 35]
        g = dR[s0:s1]
        dp = np.einsum("tp,tcp->tc", g, V)
        dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        # dC_t = sum_c dH_c dV_tc = sum_c p_tc (dH_c dR_t)
        G = np.einsum("cnp,tp->tcn", hist, g, optimize=True)                 # dH_c dR_t
        dC[s0:s1] = np.einsum("tc,tcn->tn", p, G)
        dQ[s0:s1] = np.einsum("tc,tcn->tn", dl, K) * scale
        W = np.einsum("tn,cnp->tcp", Q[s0:s1], hist, optimize=True)          # Q_t dH_c
        dE[s0:s1] = np.einsum("tc,tcp->tp", dl, W) * scale
        # d dH_c = sum_t (p_tc C_t)^T dR_t + (dl_tc Q_t)^T E_t / sqrt(N)
        pC = p[:, :, None] * C[s0:s1, None, :]                               # (t, c, n)
        dlQ = dl[:, :, None] * Q[s0:s1, None, :]
        ddH[:i] += np.einsum("tcn,tp->cnp", pC, g, optimize=True)
        ddH[:i] += np.einsum("tcn,tp->cnp", dlQ, E[s0:s1], optimize=True) * scale
    return dQ, dC, dE, ddH


def sma_token_backward(q, c, e, dH_visible, dR_t):
    """Gradients of one token's SMA readout R_t  [§3 Eq. 8-10] for a loss
    gradient dR_t (P,) on R_t: q, c (N,), e (P,), dH_visible (n, N, P)
    ->  dq (N,), dc (N,), de (P,), d_dH (n, N, P) (this token's share of
    the gradient of every visible chunk memory).

    Per token, with V_c = C_t dH_c, K_c = dH_c E_t, l_c = Q_t K_c / sqrt(N)
    and g = softmax(l):  dV_c = g_c dR_t;  dl_c = g_c (dR_t . V_c - dR_t . R_t)
    (the softmax Jacobian, R_t = sum_c g_c V_c);  dq = sum_c dl_c K_c / sqrt(N),
    de = sum_c dl_c dH_c^T q / sqrt(N),  dc = sum_c dH_c dV_c,
    d_dH_c = c^T dV_c + dl_c q^T e / sqrt(N).  An empty set gives zeros."""
    q, c, e, dH, g = _f64(q), _f64(c), _f64(e), _f64(dH_visible), _f64(dR_t)
    n, N, P = dH.shape
    if n == 0:
        return np.zeros(N), np.zeros(N), np.zeros(P), np.zeros((0, N, P))
    scale = 1.0 / math.sqrt(N)
    V = np.einsum("n,cnp->cp", c, dH)          # C_t dH_c
    K = np.einsum("cnp,p->cn", dH, e)          # dH_c E_t
    logits = (K @ q) * scale
    w = np.exp(logits - logits.max())
    w /= w.sum()                               # softmax weights g_c
    R = w @ V
    dl = w * (V @ g - R @ g)
    dq = (dl @ K) * scale
    de = np.einsum("c,cnp,n->p", dl, dH, q) * scale
    dc = np.einsum("c,cnp,p->n", w, dH, g)
    d_dH = w[:, None, None] * np.outer(c, g)[None] + dl[:, None, None] * np.outer(q, e)[None] * scale
    return dq, dc, de, d_dH


def sma_backward(Q, C, E, dH, S: int, dR, lse=None):
    """Batched sma_head_backward.  Q, C (b, L, G, N), E (b, L, G, P),
    dH (b, H, M, N, P), dR (b, L, H, P), lse (b, H, L) or None
    ->  dQ, dC (b, L, G, N), dE (b, L, G, P) (each summed over the heads that
    share the group), d_dH (b, H, M, N, P)."""
    Q, C, E, dR = _f64(Q), _f64(C), _f64(E), _f64(dR)
    b, L, G, N = Q.shape
    H = dH.shape[1]
    hpg = H // G
    dQ, dC, dE = np.zeros_like(Q), np.zeros_like(C), np.zeros_like(E)
    ddH = np.zeros(dH.shape)
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            q, c, e, dd = sma_head_backward(Q[bi, :, g], C[bi, :, g], E[bi, :, g], dH[bi, h], S,
                                            dR[bi, :, h], None if lse is None else lse[bi, h])
            dQ[bi, :, g] += q
            dC[bi, :, g] += c
            dE[bi, :, g] += e
            ddH[bi, h] = dd
    return dQ, dC, dE, ddH


def chunk_states_head_backward(X, B, a, S: int, d_dH):
    """Gradients of dH_[c] = sum_{s in [c]} w_s B_s^T X_s, w_s = A_{s+1:e(c)}
    [§3 Eq. 5] for d_dH (M, N, P):  ->  dX (L, P), dB (L, N), da (L,).

        dX_s = w_s B_s d_dH_c,   dB_s = w_s d_dH_c X_s^T,
        dw_s = B_s d_dH_c X_s^T,
        da_k = sum_{s<k in [c]} dw_s dw_s/da_k
             = sum_{s<k} dw_s (prod_{j=s+1}^{k-1} a_j) (prod_{j=k+1}^{e(c)} a_j).
    The products are formed directly, without dividing by a_k (which may
    be 0); a chunk's first token gets da = 0 (its decay is not in the chunk's
    weights)."""
    X, B, a, d_dH = _f64(X), _f64(B), _f64(a), _f64(d_dH)
    L, P = X.shape
    N = B.shape[1]
    M = num_chunks(L, S)
    dX = np.zeros((L, P))
    dB = np.zeros((L, N))
    da = np.zeros(L)
    for c in range(M):
        s0, s1 = chunk_bounds(c, L, S)
        w = decay_weights(a[s0:s1])
        G = d_dH[c]                                   # (N, P)
        BG = B[s0:s1] @ G                             # B_s d_dH_c     (n, P)
        dX[s0:s1] = w[:, None] * BG
        dB[s0:s1] = w[:, None] * (X[s0:s1] @ G.T)     # (d_dH_c X_s^T)^T
        dw = (BG * X[s0:s1]).sum(axis=1)
        n = s1 - s0
        for k in range(1, n):
            # prod_{j=s+1}^{k-1} a_j for s = 0..k-1 (chunk-local indices)
            inner = np.ones(k)
            for s in range(k - 2, -1, -1):
                inner[s] = inner[s + 1] * a[s0 + s + 1]
            da[s0 + k] = (dw[:k] * inner).sum() * w[k]
    return dX, dB, da


def chunk_states_backward(X, B, A, S: int, d_dH):
    """Batched chunk_states_head_backward.  X (b, L, H, P), B (b, L, G, N),
    A (b, L, H), d_dH (b, H, M, N, P)  ->  dX (b, L, H, P), dB (b, L, G, N)
    (summed over the heads of a group), dA (b, L, H)."""
    X, B, A = _f64(X), _f64(B), _f64(A)
    b, L, H, P = X.shape
    G = B.shape[2]
    hpg = H // G
    dX, dB, dA = np.zeros_like(X), np.zeros_like(B), np.zeros_like(A)
    for bi in range(b):
        for h in range(H):
            x, bb, aa = chunk_states_head_backward(X[bi, :, h], B[bi, :, h // hpg], A[bi, :, h], S,
                                                   d_dH[bi, h])
            dX[bi, :, h] = x
            dB[bi, :, h // hpg] += bb
            dA[bi, :, h] = aa
    return dX, dB, dA


# ---------------------------------------------------------------------------
# RMS-normalised score branch  [§3 text after Eq. 10; App. B.1 Eq. 25-27].
# Only the logits change: the query and the key readout vector are
# RMS-normalised per token, and the key readout of chunk c is rescaled along
# the key axis N by the inverse RMS of dH_c taken over the value axis P.  The
# value readout V_c = C_t dH_c is the plain one of §3 Eq. 8.
# Readings: one eps serves the two RMSNorms and r_c; each RMSNorm may carry a
# per-channel weight applied after the normalisation (None = 1).
# ---------------------------------------------------------------------------


def rms_norm(x, eps: float, weight=None):
    """RMSNorm over the last axis  [App. B.1 Eq. 25]:
    x / sqrt(mean(x^2) + eps), then times ``weight`` (per channel) if given."""
    x = _f64(x)
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return y if weight is None else y * _f64(weight)


def chunk_inv_rms(dH, eps: float):
    """r_c of App. B.1 Eq. 26: the inverse RMS of each chunk memory along
    the value axis, r_{c,n} = (mean_p dH_c[n, p]^2 + eps)^(-1/2).
    dH (..., N, P)  ->  r (..., N)."""
    dH = _f64(dH)
    return 1.0 / np.sqrt((dH * dH).mean(axis=-1) + eps)


def sma_token_rms(q, c, e, dH_visible, eps: float, wq=None, we=None):
    """The normalised score branch for one token  [App. B.1 Eq. 25-27]:

        qn = RMSNorm(Q_t), en = RMSNorm(E_t)                      [Eq. 25]
        K_c = r_c * (dH_c en),  l_c = qn . K_c / sqrt(N)           [Eq. 26-27]
        g = softmax_c(l),  V_c = C_t dH_c,  R_t = sum_c g_c V_c    [Eq. 27]

    q, c (N,), e (P,), dH_visible (n, N, P).  Returns (R (P,), lse)."""
    c, dH = _f64(c), _f64(dH_visible)
    N, P = dH.shape[1], dH.shape[2]
    n = dH.shape[0]
    if n == 0:
        return np.zeros(P), -math.inf
    qn = rms_norm(q, eps, wq)
    en = rms_norm(e, eps, we)
    r = chunk_inv_rms(dH, eps)                               # (n, N)  [Eq. 26]
    K = r * np.einsum("cnp,p->cn", dH, en)                   # [Eq. 26]
    logits = (K @ qn) / math.sqrt(N)                         # [Eq. 27]
    V = np.einsum("n,cnp->cp", c, dH)                        # [§3 Eq. 8]
    m = logits.max()
    p = np.exp(logits - m)
    d = p.sum()
    return (p[:, None] * V).sum(axis=0) / d, m + math.log(d)


def sma_head_rms(Q, C, E, dH, S: int, eps: float, wq=None, we=None):
    """sma_token_rms for every token of one head, batched per target chunk
    as in ``sma_head``:  Q, C (L, N), E (L, P), dH (M, N, P)
    ->  R (L, P), lse (L,)."""
    C, dH = _f64(C), _f64(dH)
    L, N = C.shape
    P = dH.shape[2]
    M = num_chunks(L, S)
    Qn = rms_norm(Q, eps, wq)                                # [Eq. 25]
    En = rms_norm(E, eps, we)
    r = chunk_inv_rms(dH, eps)                               # (M, N)  [Eq. 26]
    R = np.zeros((L, P))
    lse = np.full(L, -math.inf)
    scale = 1.0 / math.sqrt(N)
    for i in range(1, M):
        s0, s1 = chunk_bounds(i, L, S)
        hist = dH[:i]
        V = np.einsum("tn,cnp->tcp", C[s0:s1], hist, optimize=True)
        K = r[:i][None] * np.einsum("cnp,tp->tcn", hist, En[s0:s1], optimize=True)
        logits = np.einsum("tn,tcn->tc", Qn[s0:s1], K) * scale
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        d = p.sum(axis=1, keepdims=True)
        R[s0:s1] = np.einsum("tc,tcp->tp", p, V, optimize=True) / d
        lse[s0:s1] = (m + np.log(d))[:, 0]
    return R, lse


def sma_forward_rms(Q, C, E, dH, S: int, eps: float, wq=None, we=None):
    """Batched sma_head_rms (layouts as ``sma_forward``); wq (N,) and we (P,)
    are the RMSNorm weights shared by every head, or None."""
    Q, C, E = _f64(Q), _f64(C), _f64(E)
    b, L, G, N = Q.shape
    H = dH.shape[1]
    P = E.shape[3]
    hpg = H // G
    R = np.zeros((b, L, H, P))
    lse = np.zeros((b, H, L))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            R[bi, :, h], lse[bi, h] = sma_head_rms(Q[bi, :, g], C[bi, :, g], E[bi, :, g], dH[bi, h], S,
                                                   eps, wq, we)
    return R, lse


def rms_norm_backward(x, eps: float, dy_hat):
    """Gradient of z = x / sqrt(mean(x^2) + eps) for a gradient dy_hat on z
    (over the last axis of size D):  with rho = (mean(x^2) + eps)^(-1/2),
    dz_i/dx_j = rho delta_ij - rho^3 x_i x_j / D, so
        dx = rho dy_hat - rho^3 x (x . dy_hat) / D."""
    x, g = _f64(x), _f64(dy_hat)
    D = x.shape[-1]
    rho = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return rho * g - rho ** 3 * x * (x * g).sum(axis=-1, keepdims=True) / D


def sma_head_backward_rms(Q, C, E, dH, S: int, eps: float, dR, lse=None, wq=None, we=None):
    """Gradients of the normalised score branch of one head  [App. B.1
    Eq. 25-27 with §3 Eq. 8-10, differentiated]; training recomputes the
    logits and takes the weights as p = exp(l - lse) [App. C Eq. 33-35].

    Forward (as ``sma_head_rms``): qn = RMSNorm(Q_t) * wq, en = RMSNorm(E_t) * we,
    r_c = inverse RMS of dH_c along P, S_c = diag(r_c) dH_c,
    l_tc = qn S_c en / sqrt(N), V_tc = C_t dH_c, R_t = sum_c softmax(l)_c V_tc.

    Backward for dR = dLoss/dR:
        dl_tc = p_tc (dR_t . V_tc - dR_t . R_t)           (softmax, as the plain branch)
        d qn_t = sum_c dl_tc S_c en_t / sqrt(N)
        d en_t = sum_c dl_tc S_c^T qn_t / sqrt(N)
        dS_c   = sum_t dl_tc qn_t^T en_t / sqrt(N)
        d dH_c = sum_t p_tc C_t^T dR_t                     (value readout)
               + r_c * dS_c - (r_c^3 / P) * dH_c * rowsum_p(dS_c * dH_c)   (through S_c and r_c)
        dC_t   = sum_c p_tc dH_c dR_t
        dQ_t   = RMSNorm backward of Q_t for d qn_t * wq, dwq = sum_t d qn_t * z_q,t
        dE_t   = RMSNorm backward of E_t for d en_t * we, dwe = sum_t d en_t * z_e,t
    with z the RMSNorm outputs before the weights.  Q, C (L, N), E (L, P),
    dH (M, N, P), dR (L, P) -> dQ, dC (L, N), dE (L, P), d_dH (M, N, P),
    dwq (N,), dwe (P,) (zeros where no weight is given).  ``lse`` defaults to
    the forward's."""
    Q, C, E, dH, dR = _f64(Q), _f64(C), _f64(E), _f64(dH), _f64(dR)
    L, N = Q.shape
    P = E.shape[1]
    M = num_chunks(L, S)
    wq_ = np.ones(N) if wq is None else _f64(wq)
    we_ = np.ones(P) if we is None else _f64(we)
    if lse is None:
        _, lse = sma_head_rms(Q, C, E, dH, S, eps, wq, we)
    lse = _f64(lse)
    scale = 1.0 / math.sqrt(N)
    Zq, Ze = rms_norm(Q, eps), rms_norm(E, eps)              # [Eq. 25] before the weights
    Qn, En = Zq * wq_, Ze * we_
    r = chunk_inv_rms(dH, eps)                               # (M, N)  [Eq. 26]
    Sm = r[:, :, None] * dH                                  # S_c = diag(r_c) dH_c
    dQn, dC, dEn = np.zeros((L, N)), np.zeros((L, N)), np.zeros((L, P))
    dS, ddH = np.zeros((M, N, P)), np.zeros((M, N, P))
    for i in range(1, M):
        s0, s1 = chunk_bounds(i, L, S)
        hist, shist = dH[:i], Sm[:i]
        V = np.einsum("tn,cnp->tcp", C[s0:s1], hist, optimize=True)          # C_t dH_c
        K = np.einsum("cnp,tp->tcn", shist, En[s0:s1], optimize=True)        # S_c en_t
        logits = np.einsum("tn,tcn->tc", Qn[s0:s1], K) * scale               # [Eq. 27]
        p = np.exp(logits - lse[s0:s1, None])                                # [App. C Eq. 35]
        g = dR[s0:s1]
        dp = np.einsum("tp,tcp->tc", g, V)
        dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        G = np.einsum("cnp,tp->tcn", hist, g, optimize=True)                 # dH_c dR_t
        dC[s0:s1] = np.einsum("tc,tcn->tn", p, G)
        dQn[s0:s1] = np.einsum("tc,tcn->tn", dl, K) * scale
        W = np.einsum("tn,cnp->tcp", Qn[s0:s1], shist, optimize=True)        # qn_t S_c
        dEn[s0:s1] = np.einsum("tc,tcp->tp", dl, W) * scale
        pC = p[:, :, None] * C[s0:s1, None, :]
        dlQ = dl[:, :, None] * Qn[s0:s1, None, :]
        ddH[:i] += np.einsum("tcn,tp->cnp", pC, g, optimize=True)
        dS[:i] += np.einsum("tcn,tp->cnp", dlQ, En[s0:s1], optimize=True) * scale
    # through S_c = diag(r_c) dH_c and r_c = (mean_p dH_c^2 + eps)^(-1/2)
    ddH += r[:, :, None] * dS - (r ** 3 / P)[:, :, None] * dH * (dS * dH).sum(axis=2, keepdims=True)
    dQ = rms_norm_backward(Q, eps, dQn * wq_)
    dE = rms_norm_backward(E, eps, dEn * we_)
    dwq = (dQn * Zq).sum(axis=0) if wq is not None else np.zeros(N)
    dwe = (dEn * Ze).sum(axis=0) if we is not None else np.zeros(P)
    return dQ, dC, dE, ddH, dwq, dwe


def sma_backward_rms(Q, C, E, dH, S: int, eps: float, dR, lse=None, wq=None, we=None):
    """Batched sma_head_backward_rms (layouts as ``sma_backward``): gradients
    of projections shared by a group are summed over its heads, and dwq, dwe
    over every batch row and head."""
    Q, C, E, dR = _f64(Q), _f64(C), _f64(E), _f64(dR)
    b, L, G, N = Q.shape
    H = dH.shape[1]
    P = E.shape[3]
    hpg = H // G
    dQ, dC, dE = np.zeros_like(Q), np.zeros_like(C), np.zeros_like(E)
    ddH = np.zeros(dH.shape)
    dwq, dwe = np.zeros(N), np.zeros(P)
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            q, c, e, dd, wqg, weg = sma_head_backward_rms(
                Q[bi, :, g], C[bi, :, g], E[bi, :, g], dH[bi, h], S, eps, dR[bi, :, h],
                None if lse is None else lse[bi, h], wq, we)
            dQ[bi, :, g] += q
            dC[bi, :, g] += c
            dE[bi, :, g] += e
            ddH[bi, h] = dd
            dwq += wqg
            dwe += weg
    return dQ, dC, dE, ddH, dwq, dwe


def sma_decode_rms(q, c, e, cache, n_chunks, eps: float, hpg: int = 1, wq=None, we=None):
    """Decode with the normalised score branch (layouts as ``sma_decode``):
    every cached chunk 0..n_b-1 is visible; r_c is the inverse RMS of the
    cached memory [App. B.1 Eq. 26]."""
    q, c, e, cache = _f64(q), _f64(c), _f64(e), _f64(cache)
    b, H = cache.shape[0], cache.shape[1]
    P = cache.shape[4]
    R = np.zeros((b, H, P))
    lse = np.zeros((b, H))
    for bi in range(b):
        nb = int(n_chunks[bi])
        for h in range(H):
            g = h // hpg
            R[bi, h], lse[bi, h] = sma_token_rms(q[bi, g], c[bi, g], e[bi, g], cache[bi, h, :nb], eps,
                                                 wq, we)
    return R, lse


# ---------------------------------------------------------------------------
# SSM branch: the Mamba-2 output Y_t = C_t H_t  [§2 Eq. 2; App. A Eq. 15],
# and its chunked scan [App. A Eq. 17-24].  The step recurrence is the
# definition; the chunked form is the algorithm the GPU path follows and is
# pinned against it.
# ---------------------------------------------------------------------------


def ssm_output_head(X, B, C, a, H0=None):
    """Y_t = C_t H_t along the step recurrence H_t = a_t H_{t-1} + B_t^T X_t
    [§2 Eq. 2; App. A Eq. 15], H_{-1} = H0 (zero by default).
    X (L, P), B, C (L, N), a (L,)  ->  Y (L, P), last state (N, P)."""
    X, C = _f64(X), _f64(C)
    L, P = X.shape
    N = C.shape[1]
    if L == 0:
        return np.zeros((0, P)), (np.zeros((N, P)) if H0 is None else _f64(H0).copy())
    Hs = ssm_recurrence(X, B, a, H0)
    return np.einsum("tn,tnp->tp", C, Hs), Hs[-1].copy()


def ssd_chunked_head(X, B, C, a, S: int, H0=None):
    """The Mamba-2 chunked scan of one head, in the paper's steps:
    chunk contributions dH_[c] [App. A Eq. 20], boundary states
    H_[c] = A_{a_c:b_c} H_[c-1] + dH_[c] with H_[-1] = H0 [Eq. 17-18], and
    Y_t = Y_t^intra + Y_t^inter [Eq. 19] with
        Y_t^intra = sum_{s in chunk, s <= t} C_t A_{s+1:t} B_s^T X_s   [Eq. 21]
        Y_t^inter = C_t A_{a_c:t} H_[c-1]                              [Eq. 22]
    Returns (Y (L, P), dH (M, N, P), last boundary state (N, P))."""
    X, B, C, a = _f64(X), _f64(B), _f64(C), _f64(a)
    L, P = X.shape
    N = B.shape[1]
    M = num_chunks(L, S)
    dH = chunk_states_head(X, B, a, S)
    Y = np.zeros((L, P))
    prev = np.zeros((N, P)) if H0 is None else _f64(H0).copy()
    for c in range(M):
        s0, s1 = chunk_bounds(c, L, S)
        for t in range(s0, s1):
            y = np.zeros(P)
            for s in range(s0, t + 1):
                dec = 1.0
                for k in range(s + 1, t + 1):
                    dec *= a[k]                      # A_{s+1:t}  [Eq. 16]
                y += dec * (C[t] @ B[s]) * X[s]
            dec = 1.0
            for k in range(s0, t + 1):
                dec *= a[k]                          # A_{a_c:t}
            Y[t] = y + dec * (C[t] @ prev)
        full = 1.0
        for k in range(s0, s1):
            full *= a[k]                             # A_{a_c:b_c}
        prev = full * prev + dH[c]                   # [Eq. 18]
    return Y, dH, prev


def ssm_output(X, B, C, A, H0=None):
    """Batched ssm_output_head.  X (b, L, H, P), B, C (b, L, G, N), A (b, L, H),
    H0 (b, H, N, P) or None  ->  Y (b, L, H, P), last states (b, H, N, P)."""
    X, B, C, A = _f64(X), _f64(B), _f64(C), _f64(A)
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    Y = np.zeros((b, L, H, P))
    Hl = np.zeros((b, H, N, P))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            Y[bi, :, h], Hl[bi, h] = ssm_output_head(X[bi, :, h], B[bi, :, g], C[bi, :, g], A[bi, :, h],
                                                     None if H0 is None else H0[bi, h])
    return Y, Hl

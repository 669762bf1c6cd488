"""Seeded random-shape sweep of every entry point against the fp64 oracle.

Each of the 64 cases draws its shape from a fixed seed: half of them at the
matrix-core shape (bf16, N = 128, P = 64), the rest at any N, P <= 256 in
float32 or bf16 (general kernels); H in 1..4 with every divisor for G, b in
{1, 2}, S in {1, 3, 8, 32, 64, 96, 128, 256}, L up to 600 (up to 150 for
S <= 3), either gate form.  Per case, on the GPU's own chunk memories where a
step consumes them:
* chunk states [§3 Eq. 5] end to end;
* the forward [§3 Eq. 8-11]: R and lse at the same-input bar, out at the
  dtype's bar;
* the backward [App. C Eq. 33-35] and the chunk-state backward;
* the normalised branch [App. B.1 Eq. 25-27] with RMSNorm weights, forward
  and backward;
* the SSM branch [App. A Eq. 15-24] against the step recurrence;
* decode [§4 "Inference Cache"] of the last token against the oracle.
Tolerances as in the other modules (max-abs-normalised).  When no token sees
two chunks (L < 2 S) every chunk weight is exactly 1, so the gradients that
flow through the logits (dQ, dE, the RMSNorm weights') are zero: the
oracle's are then rounding noise, and those outputs are held absolutely to
the tolerance times the size of dC (the readout's gradient)."""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, TOL_SAME_INPUT, dev, err, host, say, to_oracle_mem

pytestmark = pytest.mark.gpu

EPS = 1e-6
N_CASES = 64


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    mfma = i % 2 == 0
    if mfma:
        dt, N, P = "bf16", 128, 64
    else:
        dt = str(rng.choice(["f32", "bf16"]))
        N = int(rng.choice([8, 16, 24, 40, 64, 96, 128, 200, 256]))
        P = int(rng.choice([8, 16, 32, 48, 64, 100, 256]))
    H = int(rng.integers(1, 5))
    G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
    b = int(rng.integers(1, 3))
    S = int(rng.choice([1, 3, 8, 32, 64, 96, 128, 256]))
    L = int(rng.integers(1, 151 if S <= 3 else 601))
    gpc = bool(rng.random() < 0.5)
    return dict(batch=b, seqlen=L, nheads=H, ngroups=G, d_state=N, d_head=P, chunk=S, dtype=dt), gpc


def check(name, got, ref, tol, scale=None):
    """err() at the tolerance; with `scale`, a reference that is zero up to
    rounding (max |ref| < 1e-6 scale) is held to tol * scale absolutely."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    assert not np.isnan(got).any(), name
    if scale is not None and np.abs(ref).max(initial=0.0) < 1e-6 * scale:
        e = float(np.abs(got - ref).max(initial=0.0)) / scale
    else:
        e = err(got, ref)
    assert e <= tol, (name, e, tol)
    return e


@pytest.mark.parametrize("ci", range(N_CASES))
def test_random_shape_chain(ci):
    cfg, gpc = draw_case(ci)
    say("random shape", ci, cfg, "gate per channel", gpc)
    dt, S, L = cfg["dtype"], cfg["chunk"], cfg["seqlen"]
    b, H, G, N, P = cfg["batch"], cfg["nheads"], cfg["ngroups"], cfg["d_state"], cfg["d_head"]
    tol, same = TOL[dt], TOL_SAME_INPUT[dt]
    d = synth.draw_fwd(**cfg, seed=2000 + ci, gate_per_channel=gpc)
    dout = synth.draw_grad((b, L, H, P), dt, 3000 + ci)
    rng = np.random.default_rng(4000 + ci)
    wq, we = rng.uniform(0.5, 2.0, N), rng.uniform(0.5, 2.0, P)
    t = {k: dev(v, "f32" if k == "A" else dt) for k, v in d.items()}
    wq_t = torch.from_numpy(wq.astype(np.float32)).cuda()
    we_t = torch.from_numpy(we.astype(np.float32)).cuda()
    errs = {}

    # chunk states, end to end
    dH = dart.dart_chunk_states(t["X"], t["B"], t["A"], S)
    torch.cuda.synchronize()
    mem = to_oracle_mem(host(dH))
    errs["dH"] = check("dH", mem, O.chunk_states(d["X"], d["B"], d["A"], S), tol)

    # forward on the GPU's memories
    out, R, lse = dart.dart_sma_fwd(t["Q"], t["C"], t["E"], dH, t["Y"], t["gate"], S, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    Rr, lr = O.sma_forward(d["Q"], d["C"], d["E"], mem, S)
    errs["R"] = check("R", host(R), Rr, same)
    errs["lse"] = check("lse", host(lse), lr, same)
    errs["out"] = check("out", host(out), O.gated_residual(d["Y"], d["gate"], Rr, gpc), tol)

    # backward from the GPU forward's R and lse; chunk-state backward from the GPU's d_dH
    dQ, dC, dE, ddH, dg = dart.dart_sma_bwd(t["Q"], t["C"], t["E"], dH, t["gate"], R, lse, dev(dout, dt), S)
    dX, dB, dA = dart.dart_chunk_states_bwd(t["X"], t["B"], t["A"], ddH, S)
    torch.cuda.synchronize()
    _, dR, dgr = O.gated_residual_backward(dout, d["gate"], Rr, gpc)
    rQ, rC, rE, rdH = O.sma_backward(d["Q"], d["C"], d["E"], mem, S, dR, lr)
    sc = float(np.abs(rC).max(initial=0.0))
    for k, g_, r_ in (("dQ", dQ, rQ), ("dC", dC, rC), ("dE", dE, rE), ("dgate", dg, dgr)):
        errs[k] = check(k, host(g_), r_, tol, sc if k in ("dQ", "dE") else None)
    errs["d_dH"] = check("d_dH", to_oracle_mem(host(ddH)), rdH, tol)
    rX, rB, rA = O.chunk_states_backward(d["X"], d["B"], d["A"], S, to_oracle_mem(host(ddH)))
    for k, g_, r_ in (("dX", dX, rX), ("dB", dB, rB), ("dA", dA, rA)):
        errs[k] = check(k, host(g_), r_, tol)

    # normalised branch on the GPU's memories, with RMSNorm weights
    _, score = dart.dart_chunk_rms(dH, L, S, EPS, wq_t, we_t, want_r=False)
    out_n, R_n, lse_n = dart.dart_sma_fwd_rms(t["Q"], t["C"], t["E"], dH, score, t["Y"], t["gate"], S, EPS,
                                              want_R=True, want_lse=True)
    g = dart.dart_sma_bwd_rms(t["Q"], t["C"], t["E"], dH, score, t["gate"], R_n, lse_n, dev(dout, dt), S, EPS,
                              wq_t, we_t, want_dw=True)
    torch.cuda.synchronize()
    Rn, ln = O.sma_forward_rms(d["Q"], d["C"], d["E"], mem, S, EPS, wq, we)
    errs["R_rms"] = check("R_rms", host(R_n), Rn, tol)
    errs["lse_rms"] = check("lse_rms", host(lse_n), ln, 1e-3 if dt == "bf16" else 1e-4)
    errs["out_rms"] = check("out_rms", host(out_n), O.gated_residual(d["Y"], d["gate"], Rn, gpc), tol)
    _, dRn, dgn = O.gated_residual_backward(dout, d["gate"], Rn, gpc)
    ref = O.sma_backward_rms(d["Q"], d["C"], d["E"], mem, S, EPS, dRn, ln, wq, we)
    names = ("dQ_rms", "dC_rms", "dE_rms", "d_dH_rms", "dw_q", "dw_e")
    gots = (g[0], g[1], g[2], g[3], g[5], g[6])
    sc = float(np.abs(ref[1]).max(initial=0.0))
    for k, g_, r_ in zip(names, gots, ref):
        got = to_oracle_mem(host(g_)) if k == "d_dH_rms" else host(g_)
        errs[k] = check(k, got, r_, tol, sc if k in ("dQ_rms", "dE_rms", "dw_q", "dw_e") else None)
    errs["dgate_rms"] = check("dgate_rms", host(g[4]), dgn, tol)

    # SSM branch against the step recurrence
    Y_ssm, dH_ssd, _ = dart.dart_ssd_fwd(t["X"], t["B"], t["C"], t["A"], S)
    torch.cuda.synchronize()
    assert torch.equal(dH_ssd, dH)
    Ys, _ = O.ssm_output(d["X"], d["B"], d["C"], d["A"])
    errs["Y_ssm"] = check("Y_ssm", host(Y_ssm), Ys, tol)

    # decode of the last token against the memories before it
    nb = (L - 1) // S
    last = lambda x: x[:, L - 1].clone()  # a fresh, aligned buffer even when the slice is contiguous
    n_t = torch.full((b,), nb, dtype=torch.int32, device="cuda")
    _, Rd, ld = dart.dart_sma_decode(last(t["Q"]), last(t["C"]), last(t["E"]), dH, last(t["Y"]), last(t["gate"]),
                                     n_chunks=n_t, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    Rdr, ldr = O.sma_decode(d["Q"][:, L - 1], d["C"][:, L - 1], d["E"][:, L - 1], mem, [nb] * b, hpg=H // G)
    errs["R_dec"] = check("R_dec", host(Rd), Rdr, same)
    errs["lse_dec"] = check("lse_dec", host(ld), ldr, same)
    say("  " + "  ".join(f"{k} {v:.1e}" for k, v in errs.items()))

"""Whole-output GPU parity on the decode workload (b=64, H=24, one new token
per row against 256 cached chunk memories of 128 x 64 bf16 each; seed 0), in
the launch the benchmark times: out, R and lse of every (row, head) against
the oracle's decode [§4 "Inference Cache"; §3 Eq. 8-11], the cache converted
one batch row at a time so that host memory stays bounded."""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, TOL_SAME_INPUT, MaxErr, f64, say

pytestmark = pytest.mark.gpu


def test_decode_every_row():
    cfg = synth.workload(synth.DECODE)
    say("full size", cfg["name"])
    b, H, G, M = cfg["batch"], cfg["nheads"], cfg["ngroups"], cfg["max_chunks"]
    d = synth.draw_decode_torch(**cfg, seed=0)
    out_bench, _, _ = dart.dart_sma_decode(d["q"], d["c"], d["e"], d["cache"], d["y"], d["gate"])
    out, R, lse = dart.dart_sma_decode(d["q"], d["c"], d["e"], d["cache"], d["y"], d["gate"],
                                       want_R=True, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_bench, out)
    h = {k: v.cpu() for k, v in d.items()}
    h.update(out=out.cpu(), R=R.cpu(), lse=lse.cpu())
    del d, out_bench, out, R, lse
    torch.cuda.empty_cache()
    q, c, e, y, gate = (f64(h[k]) for k in ("q", "c", "e", "y", "gate"))
    acc = {k: MaxErr(k) for k in ("out", "R", "lse")}
    for bi in range(b):
        # the library stores each memory [P][N]; the oracle takes [N][P]
        cache = np.swapaxes(f64(h["cache"][bi:bi + 1]), -1, -2)
        Rr, lr = O.sma_decode(q[bi:bi + 1], c[bi:bi + 1], e[bi:bi + 1], cache, [M], hpg=H // G)
        acc["R"].add(f64(h["R"][bi]), Rr[0], bi)
        acc["lse"].add(f64(h["lse"][bi]), lr[0], bi)
        acc["out"].add(f64(h["out"][bi]), O.gated_residual(y[bi], gate[bi], Rr[0]), bi)
    acc["R"].check(TOL_SAME_INPUT["bf16"])
    acc["lse"].check(TOL_SAME_INPUT["bf16"])
    acc["out"].check(TOL["bf16"])


def test_decode_rms_every_row():
    """The same workload with the normalised score branch [App. B.1 Eq. 25-27]:
    r of every cached memory from dart_chunk_rms, RMSNorm weights drawn in
    [0.5, 2], eps = 1e-6; out, R and lse of every (row, head) against the
    oracle's normalised decode on the cache as stored."""
    cfg = synth.workload(synth.DECODE)
    say("full size, normalised branch", cfg["name"])
    b, H, G, M = cfg["batch"], cfg["nheads"], cfg["ngroups"], cfg["max_chunks"]
    N, P = cfg["d_state"], cfg["d_head"]
    eps = 1e-6
    d = synth.draw_decode_torch(**cfg, seed=0)
    rng = np.random.default_rng(5)
    wq, we = rng.uniform(0.5, 2.0, N), rng.uniform(0.5, 2.0, P)
    wq_t = torch.from_numpy(wq.astype(np.float32)).cuda()
    we_t = torch.from_numpy(we.astype(np.float32)).cuda()
    r_cache, _ = dart.dart_chunk_rms(d["cache"].reshape(b, H, M, P, N), M, 1, eps, want_score=False)
    out, R, lse = dart.dart_sma_decode_rms(d["q"], d["c"], d["e"], d["cache"], r_cache, d["y"], d["gate"], eps,
                                           wq_t, we_t, want_R=True, want_lse=True)
    torch.cuda.synchronize()
    h = {k: v.cpu() for k, v in d.items()}
    h.update(out=out.cpu(), R=R.cpu(), lse=lse.cpu())
    del d, out, R, lse, r_cache
    torch.cuda.empty_cache()
    q, c, e, y, gate = (f64(h[k]) for k in ("q", "c", "e", "y", "gate"))
    acc = {k: MaxErr(k) for k in ("out", "R", "lse")}
    for bi in range(b):
        cache = np.swapaxes(f64(h["cache"][bi:bi + 1]), -1, -2)
        Rr, lr = O.sma_decode_rms(q[bi:bi + 1], c[bi:bi + 1], e[bi:bi + 1], cache, [M], eps, H // G, wq, we)
        acc["R"].add(f64(h["R"][bi]), Rr[0], bi)
        acc["lse"].add(f64(h["lse"][bi]), lr[0], bi)
        acc["out"].add(f64(h["out"][bi]), O.gated_residual(y[bi], gate[bi], Rr[0]), bi)
    # the split query rows round q r_c w_q to float16 per chunk (~1e-5 on R, lse)
    acc["R"].check(TOL_SAME_INPUT["bf16"])
    acc["lse"].check(TOL_SAME_INPUT["bf16"])
    acc["out"].check(TOL["bf16"])

"""GPU parity of dart_ssd_fwd, the SSM branch by the Mamba-2 chunked scan
[§2 Eq. 2; App. A Eq. 15-24], against the oracle's step recurrence
(Y_t = C_t H_t, the definition; the chunked form is pinned to it on the CPU).

Checked: Y, the chunk memories dH (and that they equal dart_chunk_states),
the state after the last token; float32 inputs through the general kernels
at 1e-4, bfloat16 through the matrix-core kernels at 2e-2 (the state entering
each chunk is rounded to bfloat16 once, the decayed scores too); partial last
chunks, an initial state, zero decays inside a chunk, grouped B and C, chunk
sizes 32 to 256 and one the matrix-core output kernel does not take (100).
"""
import numpy as np
import pytest
import torch

import oracle as O
import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import TOL, dev, err, host, say, to_oracle_mem

pytestmark = pytest.mark.gpu


def run(cfg, seed, with_h0, zero_at=()):
    dt = cfg["dtype"]
    d = synth.draw_fwd(**cfg, seed=seed)
    for t in zero_at:
        d["A"][:, t, :] = 0.0
    b, H, N, P = cfg["batch"], cfg["nheads"], cfg["d_state"], cfg["d_head"]
    H0 = np.random.default_rng(seed + 1).standard_normal((b, H, P, N)).astype(np.float32) if with_h0 else None
    Y, dH, Hf = dart.dart_ssd_fwd(dev(d["X"], dt), dev(d["B"], dt), dev(d["C"], dt), dev(d["A"], "f32"), cfg["chunk"],
                                  H0=None if H0 is None else torch.from_numpy(H0).cuda(), want_final=True)
    dH2 = dart.dart_chunk_states(dev(d["X"], dt), dev(d["B"], dt), dev(d["A"], "f32"), cfg["chunk"])
    torch.cuda.synchronize()
    assert torch.equal(dH, dH2), "chunk memories differ from dart_chunk_states"
    Yr, Hl = O.ssm_output(d["X"], d["B"], d["C"], d["A"], None if H0 is None else np.swapaxes(H0, -1, -2))
    dHr = O.chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
    e_y, e_d, e_f = err(host(Y), Yr), err(to_oracle_mem(host(dH)), dHr), err(np.swapaxes(host(Hf), -1, -2), Hl)
    say(f"  Y {e_y:.2e}  dH {e_d:.2e}  H_final {e_f:.2e}")
    tol = TOL[dt]
    assert e_y <= tol and e_d <= tol and e_f <= tol, (e_y, e_d, e_f)


CASES = [
    (dict(batch=2, seqlen=300, nheads=4, ngroups=2, d_state=16, d_head=8, chunk=64, dtype="f32"), True, (70,)),
    (dict(batch=1, seqlen=257, nheads=3, ngroups=3, d_state=24, d_head=40, chunk=100, dtype="f32"), False, ()),
    (dict(batch=2, seqlen=1100, nheads=4, ngroups=2, d_state=128, d_head=64, chunk=256, dtype="bf16"), True, (300,)),
    (dict(batch=1, seqlen=1024, nheads=2, ngroups=1, d_state=128, d_head=64, chunk=256, dtype="bf16"), False, ()),
    (dict(batch=1, seqlen=700, nheads=2, ngroups=2, d_state=128, d_head=64, chunk=64, dtype="bf16"), True, ()),
    (dict(batch=1, seqlen=333, nheads=2, ngroups=2, d_state=128, d_head=64, chunk=32, dtype="bf16"), False, (40, 41)),
    (dict(batch=1, seqlen=450, nheads=2, ngroups=2, d_state=128, d_head=64, chunk=100, dtype="bf16"), True, ()),
    (dict(batch=1, seqlen=600, nheads=2, ngroups=1, d_state=32, d_head=48, chunk=128, dtype="bf16"), True, ()),
    # weak decay (A_t ~ 0.99): terms from every earlier 32-token slice of a
    # chunk and from earlier chunks stay large; zero decays on both sides of
    # slice boundaries (63 | 64, 287 | 288) and inside a slice (200)
    (dict(batch=1, seqlen=1100, nheads=2, ngroups=2, d_state=128, d_head=64, chunk=256, dtype="bf16",
          a_lo=0.01, a_hi=0.05), True, (63, 64, 200, 287, 288)),
    (dict(batch=2, seqlen=1000, nheads=2, ngroups=1, d_state=128, d_head=64, chunk=128, dtype="bf16",
          a_lo=0.01, a_hi=0.05), False, (31, 32, 95, 700)),
    (dict(batch=1, seqlen=2048, nheads=3, ngroups=3, d_state=128, d_head=64, chunk=256, dtype="bf16",
          a_lo=0.01, a_hi=0.05), True, ()),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_ssd_matches_recurrence(ci):
    cfg, with_h0, zeros = CASES[ci]
    say("ssd", cfg, "H0", with_h0, "zero decays at", zeros)
    run(cfg, 50 + ci, with_h0, zeros)

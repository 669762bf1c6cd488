"""Concurrent calls: the library keeps no state between calls beyond the
per-thread error text and kernel-family selection, so calls on different
streams, from different host threads, may overlap on one GPU.  Two inputs
are run each on its own stream (default priority) from its own thread --
chunk states, forward with R and lse, backward -- several times over, and
every result must equal the same call run alone, bit for bit.  (The one
exception the header states, dart_sma_decode_noalloc's per-GPU scratch, is
not exercised here.)"""
import threading

import pytest
import torch

import state_memory_attention_amd as dart
from state_memory_attention_amd import synth

from gpu_helpers import same, say

pytestmark = pytest.mark.gpu

CFG = dict(batch=2, seqlen=3000, nheads=4, ngroups=2, chunk=256, d_state=128, d_head=64, dtype="bf16")


def chain(d, dout):
    S = CFG["chunk"]
    dH = dart.dart_chunk_states(d["X"], d["B"], d["A"], S)
    out, R, lse = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S, want_R=True, want_lse=True)
    grads = dart.dart_sma_bwd(d["Q"], d["C"], d["E"], dH, d["gate"], R, lse, dout, S)
    return (dH, out, R, lse) + tuple(grads)


NAMES = ("dH", "out", "R", "lse", "dQ", "dC", "dE", "d_dH", "dgate")


def test_two_streams_two_threads_match_serial_runs():
    inputs = []
    for seed in (21, 22):
        d = synth.draw_fwd_torch(**CFG, seed=seed)
        dout = synth.draw_grad_torch(tuple(d["Y"].shape), "bf16", seed + 100)
        inputs.append((d, dout))
    alone = [chain(d, dout) for d, dout in inputs]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = [None, None]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                res = [chain(*inputs[i]) for _ in range(3)]
            streams[i].synchronize()
            results[i] = res
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for i in range(2):
        for rep, res in enumerate(results[i]):
            for name, x, y in zip(NAMES, alone[i], res):
                same(x, y, f"input {i}, concurrent run {rep}: {name}")
    say("two streams, two threads, 3 runs each: bitwise equal to the serial runs")

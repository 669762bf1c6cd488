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


def test_ring_kernels_under_memory_contention():
    """The kernels that stream through an LDS ring give the same bits while
    another stream saturates HBM with 1 GiB copies (longer and more varied
    load latencies): chunk states at b1 H32 L65536 with S = 1024 (16 ring
    stages per chunk), and at b2 H24 L16384 the forward (with R and lse), the
    normalised forward and the backward, each against a run on a quiet GPU.
    A guard on run-to-run equality under load, not a detector of every wait
    error: a stage issued two iterations before it is read has almost always
    landed."""
    cfg_v = synth.workload(synth.VLONG, chunk=1024)
    dv = synth.draw_fwd_torch(**cfg_v, seed=41)
    cfg_l = synth.workload(synth.LONG)
    S_l = cfg_l["chunk"]
    dl = synth.draw_fwd_torch(**cfg_l, seed=42)
    dH_l = dart.dart_chunk_states(dl["X"], dl["B"], dl["A"], S_l)
    _, R_l, lse_l = dart.dart_sma_fwd(dl["Q"], dl["C"], dl["E"], dH_l, dl["Y"], dl["gate"], S_l, want_R=True,
                                  want_lse=True)
    dout_l = synth.draw_grad_torch(tuple(dl["Y"].shape), "bf16", 43)

    dHr, _, score = dart.dart_chunk_states_rms(dl["X"], dl["B"], dl["A"], S_l, 1e-6)

    def work():
        cs = dart.dart_chunk_states(dv["X"], dv["B"], dv["A"], 1024)
        fw = dart.dart_sma_fwd(dl["Q"], dl["C"], dl["E"], dH_l, dl["Y"], dl["gate"], S_l, want_R=True,
                               want_lse=True)
        fr = dart.dart_sma_fwd_rms(dl["Q"], dl["C"], dl["E"], dHr, score, dl["Y"], dl["gate"], S_l, 1e-6)[0]
        bw = dart.dart_sma_bwd(dl["Q"], dl["C"], dl["E"], dH_l, dl["gate"], R_l, lse_l, dout_l, S_l)
        return (cs,) + tuple(fw) + (fr,) + tuple(bw)

    quiet = work()
    torch.cuda.synchronize()
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    noise, main = torch.cuda.Stream(), torch.cuda.Stream()
    noise.wait_stream(torch.cuda.current_stream())
    main.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(noise):
        for _ in range(12):
            dst.copy_(src)
    with torch.cuda.stream(main):
        loud = [work() for _ in range(2)]
    torch.cuda.synchronize()
    for rep, res in enumerate(loud):
        for name, x, y in zip(("dH (S = 1024)", "out", "R", "lse", "normalised out", "dQ", "dC", "dE", "d_dH",
                               "dgate"), quiet, res):
            same(x, y, f"under contention, run {rep}: {name}")
    say("ring kernels under memory contention: bitwise equal to the quiet runs")

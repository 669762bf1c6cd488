"""Seeded input generator: determinism, shapes, rounding and distributions."""
import numpy as np
import pytest
import torch

from state_memory_attention_amd import synth


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.round_bf16(x), ref)


def test_draw_fwd_deterministic_and_shaped():
    cfg = synth.workload(synth.TINY)
    a = synth.draw_fwd(**cfg, seed=0)
    b = synth.draw_fwd(**cfg, seed=0)
    c = synth.draw_fwd(**cfg, seed=1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["X"], c["X"])
    L, N, P = cfg["seqlen"], cfg["d_state"], cfg["d_head"]
    assert a["X"].shape == (1, L, 1, P) and a["B"].shape == (1, L, 1, N)
    assert a["E"].shape == (1, L, 1, P) and a["A"].shape == (1, L, 1)
    assert a["gate"].shape == (1, L, 1, P)
    assert ((a["A"] > 0) & (a["A"] <= 1)).all()
    assert ((a["gate"] >= 0) & (a["gate"] < 1)).all()
    assert abs(a["Q"].std() * np.sqrt(N) - 1) < 0.05


def test_draw_fwd_bf16_values_are_bf16():
    cfg = synth.workload(synth.BLOCK, seqlen=512, batch=1, nheads=2, ngroups=1)
    d = synth.draw_fwd(**cfg, seed=0, gate_per_channel=False)
    for k in ("X", "B", "C", "Q", "E", "Y", "gate"):
        np.testing.assert_array_equal(synth.round_bf16(d[k]), d[k])
    assert d["gate"].shape == (1, 512, 2)


def test_draw_decode_shapes():
    cfg = synth.workload(synth.DECODE, batch=2, max_chunks=3)
    d = synth.draw_decode(**cfg, seed=0)
    assert d["cache"].shape == (2, 24, 3, 64, 128)
    assert d["q"].shape == (2, 24, 128) and d["e"].shape == (2, 24, 64)


def test_workloads_by_name():
    names = [w["name"] for w in synth.WORKLOADS]
    assert names == [synth.TINY, synth.BLOCK, synth.LONG, synth.VLONG, synth.DECODE]
    assert len(set(names)) == len(names)
    w = synth.workload(synth.LONG)
    assert (w["batch"], w["nheads"], w["seqlen"], w["chunk"]) == (2, 24, 16384, 256)
    w["chunk"] = 1  # a copy: the table is unchanged
    assert synth.workload(synth.LONG)["chunk"] == 256
    v = synth.workload(synth.LONG, chunk=32, name="long_S32")
    assert (v["name"], v["chunk"], v["seqlen"]) == ("long_S32", 32, 16384)
    with pytest.raises(KeyError):
        synth.workload("no_such_workload")

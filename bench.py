"""Benchmark of the DART hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = dart_chunk_states + dart_sma_fwd over one batch of synthetic input
(the long-context bf16 forward: b=2, H=24, L=16384, S=256, N=128, P=64 by
default), inputs resident in HBM before the timed region.  Prints one JSON
line: whole-job tokens/s, the roofline of the dominant kernel (dart_sma_fwd,
bound by bf16 MFMA) measured with HIP events on the launch stream; beside it
the other forward workloads (b4 H24 L2048 and b1 H32 L65536), the chunk sizes
64 and 32 on the headline shape, two matrix-core ceilings (a plain MFMA loop
and the vendor GEMM), the backward, the normalised and SSM branches, the
decode call's HBM roofline, and the fp64 oracle timed on a bounded sample on
the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "SMA+chunk-state fwd tokens/s at L=16K,N=128,P=64,S=256; % bf16 MFMA peak"
_CSRC = "state_memory_attention_amd/csrc/"
# the source files (kernel file and the device headers it includes) whose
# hash keys a committed counter summary to the code it was taken on
KERNEL_SOURCES = {
    "sma_fwd": [_CSRC + "sma_fwd_mfma.hip", _CSRC + "dev_common.h"],
    "chunk_states": [_CSRC + "chunk_states_mfma.hip", _CSRC + "dev_common.h", _CSRC + "lds_dma.h"],
    "decode": [_CSRC + "sma_decode_mfma.hip", _CSRC + "dev_common.h", _CSRC + "lds_dma.h"],
    "sma_bwd": [_CSRC + "sma_bwd_mfma.hip", _CSRC + "dev_common.h", _CSRC + "lds_dma.h"],
    "chunk_states_bwd": [_CSRC + "sma_bwd_mfma.hip", _CSRC + "dev_common.h", _CSRC + "lds_dma.h"],
    "state_update": [_CSRC + "decode_update.hip", _CSRC + "dev_common.h"],
    "sma_fwd_rms": [_CSRC + "sma_fwd_rms_mfma.hip", _CSRC + "dev_common.h", _CSRC + "lds_dma.h"],
    "chunk_states_rms": [_CSRC + "chunk_states_mfma.hip", _CSRC + "dev_common.h", _CSRC + "lds_dma.h"],
    "ssd": [_CSRC + "ssd.hip", _CSRC + "dev_common.h", _CSRC + "lds_dma.h"],
    "sma_bwd_rms": [_CSRC + "sma_bwd_rms_mfma.hip", _CSRC + "sma_bwd_mfma.hip", _CSRC + "dev_common.h",
                    _CSRC + "lds_dma.h"],
}


def source_hash(rels):
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def fwd_pairs(b, H, L, S):
    """(token, visible chunk) pairs: sum over tokens of chunk(t)."""
    M = -(-L // S)
    full = sum(i * S for i in range(M - 1))
    last = (M - 1) * (L - (M - 1) * S)
    return b * H * (full + last)


def fwd_flops(cfg):
    """Algorithmic flops: 4NP per (token, visible chunk) pair for the two
    products Q dH and C dH, plus 2SNP per chunk memory built (2 N P per token)."""
    b, H, L, S, N, P = (cfg[k] for k in ("batch", "nheads", "seqlen", "chunk", "d_state", "d_head"))
    return 4 * N * P * fwd_pairs(b, H, L, S), 2 * N * P * b * H * L


def tile_pairs(b, H, L, S, tile=128):
    """(token, chunk) products the forward's 128-token tiles compute: every
    token slot of a tile (padded tail slots included) against every chunk
    before the chunk of the tile's last token; the products of chunks a token
    cannot see are computed and masked."""
    n = 0
    for t0 in range(0, L, tile):
        t_last = min(t0 + tile, L) - 1
        n += tile * (t_last // S)
    return b * H * n


def path_bytes(cfg):
    """Compulsory HBM bytes of one step (chunk states + forward): X, B, A
    read and the chunk memories written; Q, C, E, the memories, Y and the gate
    read and out written."""
    b, H, G, L, S, N, P = (cfg[k] for k in ("batch", "nheads", "ngroups", "seqlen", "chunk", "d_state", "d_head"))
    M = -(-L // S)
    tok_h, tok_g, mem = b * L * H * P * 2, b * L * G * N * 2, b * H * M * N * P * 2
    return (tok_h + tok_g + b * L * H * 4 + mem) + (2 * tok_g + b * L * G * P * 2 + mem + 3 * tok_h)


def bwd_flops(cfg):
    """Algorithmic flops of the SMA backward: 12NP per (token, visible chunk)
    pair (the recomputed W and V products 4NP, dQ and dC 4NP, the two d_dH
    contractions 4NP)."""
    b, H, L, S, N, P = (cfg[k] for k in ("batch", "nheads", "seqlen", "chunk", "d_state", "d_head"))
    return 12 * N * P * fwd_pairs(b, H, L, S)


def ssd_bytes(cfg):
    """Compulsory HBM bytes of the SSM branch (bf16): X, B, C, A read, Y and
    the chunk memories written, the state entering every chunk written and
    read back."""
    b, H, G, L, S, N, P = (cfg[k] for k in ("batch", "nheads", "ngroups", "seqlen", "chunk", "d_state", "d_head"))
    M = -(-L // S)
    tok_h, tok_g, mem = b * L * H * P * 2, b * L * G * N * 2, b * H * M * P * N * 2
    return 2 * tok_h + 2 * tok_g + 3 * mem + b * L * H * 4


def time_step(torch, dart, synth, cfg, steps, warmup, sets=1):
    """Events around dart_chunk_states and dart_sma_fwd of every step on the
    launch stream; ``sets`` input draws are used in turn (two keep a working
    set near the last-level cache size from being served from it)."""
    b, H, L, S = cfg["batch"], cfg["nheads"], cfg["seqlen"], cfg["chunk"]
    M = dart.num_chunks(L, S)
    ds = [synth.draw_fwd_torch(**cfg, seed=k) for k in range(sets)]
    dHs = [torch.empty((b, H, M, cfg["d_head"], cfg["d_state"]), dtype=torch.bfloat16, device="cuda")
           for _ in range(sets)]
    outs = [torch.empty_like(d["Y"]) for d in ds]

    def cs(k):
        d = ds[k % sets]
        dart.dart_chunk_states(d["X"], d["B"], d["A"], S, dH=dHs[k % sets])

    def fwd(k):
        d = ds[k % sets]
        dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dHs[k % sets], d["Y"], d["gate"], S, out=outs[k % sets])

    for k in range(warmup):
        cs(k)
        fwd(k)
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record(st)
        cs(k)
        ev[k][1].record(st)
        fwd(k)
        ev[k][2].record(st)
    torch.cuda.synchronize()
    t_cs = sum(e[0].elapsed_time(e[1]) for e in ev) / steps / 1e3
    t_fwd = sum(e[1].elapsed_time(e[2]) for e in ev) / steps / 1e3
    del ds, dHs, outs
    torch.cuda.empty_cache()
    return t_cs, t_fwd


def step_record(cfg, t_cs, t_fwd):
    b, H, L, S = cfg["batch"], cfg["nheads"], cfg["seqlen"], cfg["chunk"]
    f_sma, f_cs = fwd_flops(cfg)
    nbytes = path_bytes(cfg)
    return {"workload": cfg["name"], "tokens_per_s": b * L / (t_cs + t_fwd),
            "us_chunk_states": t_cs * 1e6, "us_sma_fwd": t_fwd * 1e6,
            "sma_fwd_TFLOPs": f_sma / t_fwd / 1e12, "sma_fwd_frac": f_sma / t_fwd / 1e12 / PEAK_BF16_TFLOPS,
            "path_mfma_frac": (f_sma + f_cs) / (t_cs + t_fwd) / 1e12 / PEAK_BF16_TFLOPS,
            "path_bytes": nbytes, "path_GBs": nbytes / (t_cs + t_fwd) / 1e9,
            "path_hbm_frac": nbytes / (t_cs + t_fwd) / 1e9 / PEAK_HBM_GBS}


def time_configs(torch, dart, synth, steps, warmup, skip):
    """The other forward workloads in the same run: the single-layer block
    (b4 H24 L2048, HBM-bound: both fractions reported; two input sets in
    turn, since its 0.3 GB working set is near the 256 MB last-level cache)
    and the very long context (b1 H32 L65536), each with the step's
    tokens/s and the forward's and the path's bf16 MFMA fractions."""
    res = {}
    for name in (synth.BLOCK, synth.LONG, synth.VLONG):
        if name == skip:
            continue
        cfg = synth.workload(name)
        t_cs, t_fwd = time_step(torch, dart, synth, cfg, steps, warmup, sets=2 if name == synth.BLOCK else 1)
        rec = step_record(cfg, t_cs, t_fwd)
        rec["traffic_sma_fwd"] = traffic_record("sma_fwd", cfg["name"])
        res[cfg["name"]] = rec
    return res


def time_chunk_sizes(torch, dart, synth, steps, warmup):
    """The evaluation-time chunk sizes on the long-context shape (b2 H24
    L16384): the same step at S = 64 and S = 32.  Pairs, and so algorithmic
    flops, grow as 1/S; a 128-token tile then spans 2 or 4 chunks and also
    computes (and masks) the products of the chunks its earlier tokens cannot
    see, which ``masked_frac`` counts."""
    res = {}
    for S in (64, 32):
        cfg = synth.workload(synth.LONG, chunk=S, name=f"long_bf16_b2_h24_L16384_S{S}")
        b, H, L = cfg["batch"], cfg["nheads"], cfg["seqlen"]
        t_cs, t_fwd = time_step(torch, dart, synth, cfg, steps, warmup)
        rec = step_record(cfg, t_cs, t_fwd)
        alg, done = fwd_pairs(b, H, L, S), tile_pairs(b, H, L, S)
        rec.update(pairs=alg, computed_pairs=done, masked_frac=1 - alg / done)
        res[f"S{S}"] = rec
    return res


def time_gemm_probe(torch, steps, warmup, fwd_tflops):
    """An independent matrix-core ceiling: the vendor bf16 GEMM behind
    torch.matmul, (8192 x 6144) @ (6144 x 8192) with float32 accumulation
    (8.2e11 flop, about one forward launch), contiguous operands drawn
    N(0, 1), timed with events on the same stream."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    M_, K_, N_ = 8192, 6144, 8192
    a = torch.randn((M_, K_), generator=gen, device="cuda").to(torch.bfloat16)
    bm = torch.randn((K_, N_), generator=gen, device="cuda").to(torch.bfloat16)
    c = torch.empty((M_, N_), dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        torch.matmul(a, bm, out=c)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        torch.matmul(a, bm, out=c)
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    flop = 2 * M_ * K_ * N_
    tflops = flop / t / 1e12
    del a, bm, c
    torch.cuda.empty_cache()
    return {"shape": [M_, K_, N_], "flop_per_call": flop, "us_per_call": t * 1e6, "achieved_TFLOPs": tflops,
            "frac_of_peak": tflops / PEAK_BF16_TFLOPS, "fwd_frac_of_gemm": fwd_tflops / tflops}


def time_backward(torch, dart, synth, cfg, steps=5, warmup=1):
    """The backward of the hot path on the same workload: dart_sma_bwd (the
    three matrix-core passes) from the forward's R and lse and a synthetic
    loss gradient, then dart_chunk_states_bwd; algorithmic flops from
    bwd_flops."""
    b, H, L, S = cfg["batch"], cfg["nheads"], cfg["seqlen"], cfg["chunk"]
    d = synth.draw_fwd_torch(**cfg, seed=0)
    dH = dart.dart_chunk_states(d["X"], d["B"], d["A"], S)
    _, R, lse = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S, want_R=True, want_lse=True)
    dout = synth.draw_grad_torch((b, L, H, cfg["d_head"]), "bf16", seed=3)
    import ctypes

    from state_memory_attention_amd import dart as D
    dims = D.Dims(b, L, H, cfg["ngroups"], cfg["d_state"], cfg["d_head"], S)
    ws = torch.empty(int(D.lib().dart_sma_bwd_workspace_bytes(ctypes.byref(dims))), dtype=torch.uint8,
                     device="cuda")
    ws2 = torch.empty(int(D.lib().dart_chunk_states_bwd_workspace_bytes(ctypes.byref(dims))),
                      dtype=torch.uint8, device="cuda")

    def run():
        g = dart.dart_sma_bwd(d["Q"], d["C"], d["E"], dH, d["gate"], R, lse, dout, S, workspace=ws)
        return g

    for _ in range(warmup):
        g = run()
        dart.dart_chunk_states_bwd(d["X"], d["B"], d["A"], g[3], S, workspace=ws2)
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record(st)
        g = run()
        ev[k][1].record(st)
        dart.dart_chunk_states_bwd(d["X"], d["B"], d["A"], g[3], S, workspace=ws2)
        ev[k][2].record(st)
    torch.cuda.synchronize()
    t_bwd = sum(e[0].elapsed_time(e[1]) for e in ev) / steps / 1e3
    t_csb = sum(e[1].elapsed_time(e[2]) for e in ev) / steps / 1e3
    flops = bwd_flops(cfg)
    res = {"workload": cfg["name"], "kernel": "dart_sma_bwd", "us_per_call": t_bwd * 1e6,
           "flop_per_call": flops, "achieved_TFLOPs": flops / t_bwd / 1e12,
           "peak_TFLOPs": PEAK_BF16_TFLOPS, "frac": flops / t_bwd / 1e12 / PEAK_BF16_TFLOPS,
           "chunk_states_bwd_us": t_csb * 1e6, "grad_dtype": "f32",
           "traffic": {k: traffic_record(k, cfg["name"], "sma_bwd") for k in ("sma_bwd_a", "sma_bwd_bc", "sma_bwd_d")}}
    res["traffic"]["chunk_states_bwd"] = traffic_record("chunk_states_bwd", cfg["name"])
    del d, dH, R, lse, dout, ws, ws2, g
    torch.cuda.empty_cache()
    return res


def time_rms(torch, dart, synth, cfg, steps=10, warmup=2, eps=1e-6):
    """The hot path with the RMS-normalised score branch on the same
    workload: dart_chunk_states_rms (chunk memories plus the float16 score
    memory) and dart_sma_fwd_rms.  Same algorithmic flops as the plain
    forward (4NP per pair; the normalisation is O(L (N + P)) per head).
    Then its backward, dart_sma_bwd_rms (with the RMSNorm weight gradients),
    from the forward's R and lse: 12NP per pair as the plain backward (the
    chain through r_c and the RMSNorms is O(M N P + L (N + P)) per head)."""
    b, H, L, S = cfg["batch"], cfg["nheads"], cfg["seqlen"], cfg["chunk"]
    N, P = cfg["d_state"], cfg["d_head"]
    d = synth.draw_fwd_torch(**cfg, seed=0)
    M = dart.num_chunks(L, S)
    dH = torch.empty((b, H, M, P, N), dtype=torch.bfloat16, device="cuda")
    dHs = torch.empty((b, H, M, P, N), dtype=torch.float16, device="cuda")
    out = torch.empty_like(d["Y"])

    def cs():
        dart.dart_chunk_states_rms(d["X"], d["B"], d["A"], S, eps, dH=dH, dH_score=dHs, want_r=False)

    def fwd():
        dart.dart_sma_fwd_rms(d["Q"], d["C"], d["E"], dH, dHs, d["Y"], d["gate"], S, eps, out=out)

    for _ in range(warmup):
        cs()
        fwd()
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record(st)
        cs()
        ev[k][1].record(st)
        fwd()
        ev[k][2].record(st)
    torch.cuda.synchronize()
    t_cs = sum(e[0].elapsed_time(e[1]) for e in ev) / steps / 1e3
    t_fwd = sum(e[1].elapsed_time(e[2]) for e in ev) / steps / 1e3
    f_sma, _ = fwd_flops(cfg)
    res = {"workload": cfg["name"], "kernel": "dart_sma_fwd_rms", "us_per_call": t_fwd * 1e6,
           "traffic": traffic_record("sma_fwd_rms", cfg["name"]),
           "achieved_TFLOPs": f_sma / t_fwd / 1e12, "peak_TFLOPs": PEAK_BF16_TFLOPS,
           "frac": f_sma / t_fwd / 1e12 / PEAK_BF16_TFLOPS, "chunk_states_rms_us": t_cs * 1e6,
           "tokens_per_s": b * L / (t_cs + t_fwd)}
    # backward: R and lse of the forward and a synthetic dout; no RMSNorm
    # weights, as the score memory above was formed without them (their
    # gradients, at weight 1, are computed all the same)
    _, R, lse = dart.dart_sma_fwd_rms(d["Q"], d["C"], d["E"], dH, dHs, d["Y"], d["gate"], S, eps, out=out,
                                      want_R=True, want_lse=True)
    dout = synth.draw_grad_torch((b, L, H, P), "bf16", seed=3)
    import ctypes

    from state_memory_attention_amd import dart as D
    dims = D.Dims(b, L, H, cfg["ngroups"], N, P, S)
    ws = torch.empty(int(D.lib().dart_sma_bwd_rms_workspace_bytes(ctypes.byref(dims))), dtype=torch.uint8,
                     device="cuda")

    def bwd():
        return dart.dart_sma_bwd_rms(d["Q"], d["C"], d["E"], dH, dHs, d["gate"], R, lse, dout, S, eps,
                                     want_dw=True, workspace=ws)

    for _ in range(warmup):
        g = bwd()
    bsteps = max(steps // 2, 1)
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(bsteps)]
    torch.cuda.synchronize()
    for k in range(bsteps):
        evb[k][0].record(st)
        g = bwd()
        evb[k][1].record(st)
    torch.cuda.synchronize()
    t_bwd = sum(e[0].elapsed_time(e[1]) for e in evb) / bsteps / 1e3
    fb = bwd_flops(cfg)
    res["backward"] = {"kernel": "dart_sma_bwd_rms", "us_per_call": t_bwd * 1e6, "flop_per_call": fb,
                       "achieved_TFLOPs": fb / t_bwd / 1e12, "peak_TFLOPs": PEAK_BF16_TFLOPS,
                       "frac": fb / t_bwd / 1e12 / PEAK_BF16_TFLOPS, "grad_dtype": "f32",
                       "traffic": {k: traffic_record(k, cfg["name"], "sma_bwd_rms")
                                   for k in ("sma_bwd_rms_a", "sma_bwd_rms_bc_q", "sma_bwd_rms_bc_c",
                                             "sma_bwd_rms_d")}}
    del d, dH, dHs, out, R, lse, dout, ws, g
    torch.cuda.empty_cache()
    return res


def time_ssd(torch, dart, synth, cfg, steps=10, warmup=2):
    """The SSM branch by the chunked scan on the same workload: dart_ssd_fwd
    (chunk states, chunk decays, scan over chunks, outputs).  Bound by HBM:
    compulsory bytes = X, B, C, A read, Y and the chunk memories written, the
    state entering every chunk written and read back."""
    import ctypes

    from state_memory_attention_amd import dart as D
    b, H, L, S = cfg["batch"], cfg["nheads"], cfg["seqlen"], cfg["chunk"]
    G, N, P = cfg["ngroups"], cfg["d_state"], cfg["d_head"]
    M = dart.num_chunks(L, S)
    d = synth.draw_fwd_torch(**cfg, seed=0)
    Y = torch.empty_like(d["X"])
    dH = torch.empty((b, H, M, P, N), dtype=torch.bfloat16, device="cuda")
    dims = D.Dims(b, L, H, G, N, P, S)
    ws = torch.empty(int(D.lib().dart_ssd_fwd_workspace_bytes(ctypes.byref(dims), 1)), dtype=torch.uint8,
                     device="cuda")

    def run():
        dart.dart_ssd_fwd(d["X"], d["B"], d["C"], d["A"], S, Y=Y, dH=dH, workspace=ws)

    for _ in range(warmup):
        run()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        run()
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    nbytes = ssd_bytes(cfg)
    res = {"workload": cfg["name"], "kernel": "dart_ssd_fwd", "us_per_call": t * 1e6, "bytes_per_call": nbytes,
           "achieved_GBs": nbytes / t / 1e9, "peak_GBs": PEAK_HBM_GBS, "frac": nbytes / t / 1e9 / PEAK_HBM_GBS,
           "tokens_per_s": b * L / t, "traffic_out_kernel": traffic_record("ssd_out", cfg["name"], "ssd")}
    del d, Y, dH, ws
    torch.cuda.empty_cache()
    return res


def traffic_record(kernel, workload, sources=None):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[sources or kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_info():
    """BLAS library and thread count numpy uses, from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if not libs:
            return {"threads": 1, "backend": "none found"}
        top = max(libs, key=lambda i: i.get("num_threads", 1))
        return {"threads": int(top.get("num_threads", 1)),
                "backend": f"{top.get('internal_api')} {top.get('version')} ({os.path.basename(top.get('filepath', ''))})"}
    except Exception as exc:  # threadpoolctl missing or failing: report that
        return {"threads": 1, "backend": f"unknown ({exc.__class__.__name__})"}


def cpu_baseline(cfg, budget_s=12.0):
    """The fp64 oracle (chunk states + SMA of whole heads, the same recipe,
    seed 0, numpy generator) timed on the host, one head at a time until the
    budget is spent; scaled to tokens/s of the full workload."""
    import numpy as np

    import oracle as O
    from state_memory_attention_amd import synth

    one = dict(cfg, batch=1, nheads=1, ngroups=1)
    heads, t_total = 0, 0.0
    while t_total < budget_s and heads < cfg["batch"] * cfg["nheads"]:
        d = synth.draw_fwd(**one, seed=heads)
        t0 = time.perf_counter()
        dH = O.chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
        R, _ = O.sma_forward(d["Q"], d["C"], d["E"], dH, cfg["chunk"])
        O.gated_residual(d["Y"], d["gate"], R)
        t_total += time.perf_counter() - t0
        heads += 1
    # the full workload is batch * nheads such head-sequences of L tokens each
    value = heads * cfg["seqlen"] / (t_total * cfg["nheads"])
    blas = blas_info()
    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
           if k in os.environ}
    return {"value": value, "unit": "tokens/s", "cores": blas["threads"], "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "host_affinity_cores": len(os.sched_getaffinity(0)),
            "blas": blas["backend"], "thread_env": env,
            "sample": f"{heads} whole head-sequence(s) of the same workload (L={cfg['seqlen']}, "
                      f"S={cfg['chunk']}, N={cfg['d_state']}, P={cfg['d_head']}), chunk states + SMA + "
                      f"gated residual in fp64 numpy, {t_total:.1f} s; scaled by heads/(batch*nheads)"}


def time_decode(torch, dart, synth, steps=20, warmup=3):
    cfg = synth.workload(synth.DECODE)
    d = synth.draw_decode_torch(**cfg, seed=0)
    ws = torch.empty(dart.decode_workspace_bytes(cfg["batch"], cfg["nheads"], cfg["d_head"],
                                                 cfg["max_chunks"]), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["y"])
    args = (d["q"], d["c"], d["e"], d["cache"], d["y"], d["gate"])
    for _ in range(warmup):
        dart.dart_sma_decode(*args, out=out, workspace=ws)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        dart.dart_sma_decode(*args, out=out, workspace=ws)
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    nbytes = d["cache"].numel() * 2 + sum(d[k].numel() * 2 for k in ("q", "c", "e", "y", "gate")) + out.numel() * 2
    gbs = nbytes / t / 1e9
    res = {"workload": cfg["name"], "us_per_call": t * 1e6, "bytes_per_call": nbytes,
           "achieved_GBs": gbs, "peak_GBs": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS,
           "traffic": traffic_record("decode", cfg["name"])}
    res["read_probe"] = time_read_probe(torch, d["cache"], steps, warmup, gbs)
    res["state_update"] = time_state_update(torch, dart, synth, cfg, d["cache"], steps, warmup)
    del d, ws, out
    torch.cuda.empty_cache()
    return res


def time_mfma_probe(torch, dH, Q, steps, warmup, fwd_tflops):
    """What back-to-back v_mfma_f32_32x32x16_bf16 sustain on this device
    (libdart_probe.so: operands in registers, two waves per SIMD on every CU,
    the forward's 32-MFMA burst, no memory traffic), run right after the
    timed forward with operands taken from the workload (chunk memories as A,
    queries as B): the practical ceiling for the forward at the clock the chip
    holds under dense matrix load, beside the 2.5 PF figure."""
    import ctypes

    probe = ctypes.CDLL(os.path.join(ROOT, "state_memory_attention_amd", "probes", "libdart_probe.so"))
    probe.dart_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    ops = torch.cat([dH.reshape(-1)[:4096], Q.reshape(-1)[:4096]]).contiguous()
    blocks, iters = 512, 400
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    stream = ctypes.c_void_p(st.cuda_stream)
    for _ in range(warmup):
        assert probe.dart_probe_mfma(ops.data_ptr(), blocks, iters, sink.data_ptr(), stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        assert probe.dart_probe_mfma(ops.data_ptr(), blocks, iters, sink.data_ptr(), stream) == 0
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    flop = blocks * 4 * iters * 32 * 32 * 32 * 16 * 2
    tflops = flop / t / 1e12
    return {"flop_per_launch": flop, "us_per_call": t * 1e6, "achieved_TFLOPs": tflops,
            "frac_of_peak": tflops / PEAK_BF16_TFLOPS, "fwd_frac_of_probe": fwd_tflops / tflops}


def time_read_probe(torch, buf, steps, warmup, decode_gbs):
    """What a streaming read of the same bytes draws from HBM on this
    device (libdart_probe.so: 16-byte non-temporal loads, eight in flight per
    lane, 8192 blocks): the practical ceiling for a read-bound call, beside the
    8 TB/s figure."""
    import ctypes

    probe = ctypes.CDLL(os.path.join(ROOT, "state_memory_attention_amd", "probes", "libdart_probe.so"))
    probe.dart_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    stream = ctypes.c_void_p(st.cuda_stream)
    nbytes = buf.numel() * buf.element_size()
    for _ in range(warmup):
        assert probe.dart_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        assert probe.dart_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream) == 0
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    gbs = nbytes / t / 1e9
    return {"bytes": nbytes, "us_per_call": t * 1e6, "achieved_GBs": gbs,
            "decode_frac_of_probe": decode_gbs / gbs}


def _state_update_inputs(torch, cfg):
    """One new token per batch row of the decode workload: x (b, H, P) and
    B (b, G, N) in bf16, decay a (b, H), a float32 in-progress state
    (b, H, P, N) and positions in the middle of chunk 100 (S = 256)."""
    b, H, G, N, P = cfg["batch"], cfg["nheads"], cfg["ngroups"], cfg["d_state"], cfg["d_head"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    x = torch.randn((b, H, P), generator=gen, device="cuda").to(torch.bfloat16)
    Bt = (torch.randn((b, G, N), generator=gen, device="cuda") / N ** 0.5).to(torch.bfloat16)
    a = torch.rand((b, H), generator=gen, device="cuda") * 0.5 + 0.5
    state = torch.zeros((b, H, P, N), device="cuda")
    pos = torch.full((b,), 256 * 100 + 7, dtype=torch.int32, device="cuda")
    return x, Bt, a, state, pos


def time_state_update(torch, dart, synth, cfg, cache, steps, warmup):
    """dart_decode_state_update on the decode workload: one token per row
    absorbed into the float32 in-progress chunk memories (b, H, P, N).  The
    positions are mid-chunk, so every call reads and writes the whole state
    and writes no cache row (the per-token steady state; a chunk close writes
    the dtype row instead of the state, fewer bytes)."""
    x, Bt, a, state, pos = _state_update_inputs(torch, cfg)
    nch = torch.zeros((cfg["batch"],), dtype=torch.int32, device="cuda")
    S = 256
    for _ in range(warmup):
        dart.dart_decode_state_update(x, Bt, a, state, pos, cache, S, n_chunks=nch)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        dart.dart_decode_state_update(x, Bt, a, state, pos, cache, S, n_chunks=nch)
    e1.record(st)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    nbytes = 2 * state.numel() * 4 + (x.numel() + Bt.numel()) * 2 + a.numel() * 4
    gbs = nbytes / t / 1e9
    return {"kernel": "dart_decode_state_update", "us_per_call": t * 1e6, "bytes_per_call": nbytes,
            "achieved_GBs": gbs, "peak_GBs": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS,
            "traffic": traffic_record("state_update", cfg["name"])}


COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written


def profile_kernels(launches=3):
    """Program for hardware-counter runs: a plain 1 GiB device copy (whose
    HBM bytes are known), then `launches` calls of each hot-path kernel on
    the full-size workloads, synchronised between phases."""
    import torch

    import state_memory_attention_amd as dart
    from state_memory_attention_amd import synth

    import ctypes

    probe = ctypes.CDLL(os.path.join(ROOT, "state_memory_attention_amd", "probes", "libdart_probe.so"))
    probe.dart_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(launches):
        assert probe.dart_probe_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, stream) == 0
    torch.cuda.synchronize()
    del src, dst
    for name in (synth.LONG, synth.VLONG):
        cfg = synth.workload(name)
        d = synth.draw_fwd_torch(**cfg, seed=0)
        dH = dart.dart_chunk_states(d["X"], d["B"], d["A"], cfg["chunk"])
        for _ in range(launches):
            dart.dart_chunk_states(d["X"], d["B"], d["A"], cfg["chunk"], dH=dH)
        torch.cuda.synchronize()
        out = torch.empty_like(d["Y"])
        for _ in range(launches):
            dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], cfg["chunk"], out=out)
        torch.cuda.synchronize()
        if name == synth.LONG:
            # the matrix-core yardstick on the same operand values (time_mfma_probe)
            probe.dart_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p]
            ops = torch.cat([dH.reshape(-1)[:4096], d["Q"].reshape(-1)[:4096]]).contiguous()
            sink = torch.zeros(512 * 256, dtype=torch.float32, device="cuda")
            for _ in range(launches):
                assert probe.dart_probe_mfma(ops.data_ptr(), 512, 400, sink.data_ptr(), stream) == 0
            torch.cuda.synchronize()
            del ops, sink
            # the vendor GEMM of time_gemm_probe
            gen = torch.Generator(device="cuda")
            gen.manual_seed(5)
            ga = torch.randn((8192, 6144), generator=gen, device="cuda").to(torch.bfloat16)
            gb = torch.randn((6144, 8192), generator=gen, device="cuda").to(torch.bfloat16)
            gc = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
            for _ in range(launches):
                torch.matmul(ga, gb, out=gc)
            torch.cuda.synchronize()
            del ga, gb, gc
        del d, dH, out
        torch.cuda.empty_cache()
    cfg = synth.workload(synth.DECODE)
    d = synth.draw_decode_torch(**cfg, seed=0)
    for _ in range(launches):
        dart.dart_sma_decode(d["q"], d["c"], d["e"], d["cache"], d["y"], d["gate"])
    torch.cuda.synchronize()
    upd = _state_update_inputs(torch, cfg)
    for _ in range(launches):
        dart.dart_decode_state_update(*upd, d["cache"], 256, n_chunks=None)
    torch.cuda.synchronize()
    del d, upd
    torch.cuda.empty_cache()
    # backward of the long-context workload: the forward's R and lse first
    cfg = synth.workload(synth.LONG)
    S = cfg["chunk"]
    d = synth.draw_fwd_torch(**cfg, seed=0)
    dH = dart.dart_chunk_states(d["X"], d["B"], d["A"], S)
    _, R, lse = dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S, want_R=True, want_lse=True)
    dout = synth.draw_grad_torch((cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["d_head"]), "bf16", seed=3)
    torch.cuda.synchronize()
    for _ in range(launches):
        g = dart.dart_sma_bwd(d["Q"], d["C"], d["E"], dH, d["gate"], R, lse, dout, S)
    torch.cuda.synchronize()
    for _ in range(launches):
        dart.dart_chunk_states_bwd(d["X"], d["B"], d["A"], g[3], S)
    torch.cuda.synchronize()
    del g, R, lse, dout
    # the normalised score branch, then the SSM branch, on the same workload
    M = dart.num_chunks(cfg["seqlen"], S)
    dHs = torch.empty((cfg["batch"], cfg["nheads"], M, cfg["d_head"], cfg["d_state"]), dtype=torch.float16,
                      device="cuda")
    for _ in range(launches):
        dart.dart_chunk_states_rms(d["X"], d["B"], d["A"], S, 1e-6, dH=dH, dH_score=dHs, want_r=False)
    torch.cuda.synchronize()
    out = torch.empty_like(d["Y"])
    for _ in range(launches):
        dart.dart_sma_fwd_rms(d["Q"], d["C"], d["E"], dH, dHs, d["Y"], d["gate"], S, 1e-6, out=out)
    torch.cuda.synchronize()
    # its backward (after the plain backward's passes, which come first in
    # dispatch order among the kernels both use)
    _, R, lse = dart.dart_sma_fwd_rms(d["Q"], d["C"], d["E"], dH, dHs, d["Y"], d["gate"], S, 1e-6, out=out,
                                      want_R=True, want_lse=True)
    dout = synth.draw_grad_torch((cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["d_head"]), "bf16", seed=3)
    torch.cuda.synchronize()
    for _ in range(launches):
        g = dart.dart_sma_bwd_rms(d["Q"], d["C"], d["E"], dH, dHs, d["gate"], R, lse, dout, S, 1e-6,
                                  want_dw=True)
    torch.cuda.synchronize()
    del g, R, lse, dout
    for _ in range(launches):
        dart.dart_ssd_fwd(d["X"], d["B"], d["C"], d["A"], S, Y=out, dH=dH)
    torch.cuda.synchronize()
    print("profile-kernels done", flush=True)


def _read_counter_csv(path, counter):
    """Per-dispatch values of one counter from rocprofv3's counter_collection
    CSV: list of (dispatch_id, kernel_name, value) in dispatch order."""
    import csv

    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            did = int(r["Dispatch_Id"])
            name = r["Kernel_Name"]
            rows.setdefault(did, [name, 0.0])
            rows[did][1] += float(r["Counter_Value"])
    return [(k, v[0], v[1]) for k, v in sorted(rows.items())]


def summarize_counters(fetch_csv, write_csv, launches=3):
    """Turn the FETCH_SIZE and WRITE_SIZE runs of ``--profile-kernels`` into
    HBM bytes per launch of each hot kernel, scaled by the calibration copy,
    and write profiles/traffic_<kernel>_<workload>.json."""
    from state_memory_attention_amd import synth

    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")
    assert len(fetch) == len(write), (len(fetch), len(write))
    # the calibration copies: `launches` dispatches of copy16_kernel (1 GiB each way)
    copies = [v for _, n, v in fetch if "copy16_kernel" in n]
    wcopies = [v for _, n, v in write if "copy16_kernel" in n]
    assert len(copies) == launches and len(wcopies) == launches
    f_scale = COPY_BYTES / (sum(copies) / len(copies) * 1024)   # counters are KiB per dispatch
    w_scale = COPY_BYTES / (sum(wcopies) / len(wcopies) * 1024)

    def per_kernel(substr, first, count):
        sel_f = [v for _, n, v in fetch if substr in n][first:first + count]
        sel_w = [v for _, n, v in write if substr in n][first:first + count]
        return (sum(sel_f) / len(sel_f) * 1024 * f_scale, sum(sel_w) / len(sel_w) * 1024 * w_scale)

    out = []
    w_long, w_vlong, w_dec = synth.LONG, synth.VLONG, synth.DECODE
    # (file label, source set, kernel symbol, workload, index of the first
    # counted dispatch of that symbol in the --profile-kernels program)
    plan = [("chunk_states", "chunk_states", "chunk_states_mfma_kernel", w_long, 1),
            ("sma_fwd", "sma_fwd", "sma_fwd_mfma_kernel", w_long, 0),
            ("chunk_states", "chunk_states", "chunk_states_mfma_kernel", w_vlong, 1 + launches + 1),
            ("sma_fwd", "sma_fwd", "sma_fwd_mfma_kernel", w_vlong, launches),
            ("decode", "decode", "sma_decode_partial_lds_kernel", w_dec, 0),
            ("state_update", "state_update", "decode_update_kernel", w_dec, 0),
            ("sma_bwd_a", "sma_bwd", "sma_bwd_a_kernel", w_long, 0),
            ("sma_bwd_bc", "sma_bwd", "sma_bwd_bc_kernel", w_long, 0),
            ("sma_bwd_d", "sma_bwd", "sma_bwd_d_kernel", w_long, 0),
            ("chunk_states_bwd", "chunk_states_bwd", "chunk_states_bwd_mfma_kernel", w_long, 0),
            ("chunk_states_rms", "chunk_states_rms", "chunk_states_mfma_kernel<true,", w_long, 0),
            ("sma_fwd_rms", "sma_fwd_rms", "sma_fwd_rms_mfma_kernel", w_long, 0),
            ("sma_bwd_rms_a", "sma_bwd_rms", "sma_bwd_rms_a_kernel", w_long, 0),
            ("sma_bwd_rms_bc_q", "sma_bwd_rms", "sma_bwd_bc_kernel<1>", w_long, 0),
            ("sma_bwd_rms_bc_c", "sma_bwd_rms", "sma_bwd_bc_kernel<2>", w_long, 0),
            ("sma_bwd_rms_d", "sma_bwd_rms", "sma_bwd_d_kernel", w_long, launches),
            ("ssd_out", "ssd", "ssd_out_mfma_kernel", w_long, 0),
            ("ssd_state_pass", "ssd", "state_pass_kernel", w_long, 0)]
    for label, kernel, sym, workload, first in plan:
        rd, wr = per_kernel(sym, first, launches)
        rec = {"kernel": sym, "workload": workload, "source_sha256_16": source_hash(KERNEL_SOURCES[kernel]),
               "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
               "hbm_bytes_per_launch": rd + wr, "fetch_scale": f_scale, "write_scale": w_scale,
               "calibration": f"plain 16-byte-vector copy (libdart_probe.so) of {COPY_BYTES} bytes: FETCH_SIZE and WRITE_SIZE (KiB) "
                              "scaled so that the copy reads and writes exactly its size"}
        path = os.path.join(ROOT, "profiles", f"traffic_{label}_{workload}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        out.append(rec)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_bf16_b2_h24_L16384",
                    choices=["long_bf16_b2_h24_L16384", "vlong_bf16_b1_h32_L65536"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-rms", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads and the S = 64 / 32 variants")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="run each hot kernel a few times for a hardware-counter pass, then exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn FETCH_SIZE/WRITE_SIZE runs of --profile-kernels into profiles/traffic_*.json")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.profile_kernels:
        profile_kernels()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the library runs the "
              "hot path on a single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import state_memory_attention_amd as dart
    from state_memory_attention_amd import synth

    cfg = synth.workload(args.workload)
    b, H, L, S = cfg["batch"], cfg["nheads"], cfg["seqlen"], cfg["chunk"]
    d = synth.draw_fwd_torch(**cfg, seed=0)
    M = dart.num_chunks(L, S)
    dH = torch.empty((b, H, M, cfg["d_head"], cfg["d_state"]), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(d["Y"])

    def step():
        dart.dart_chunk_states(d["X"], d["B"], d["A"], S, dH=dH)
        dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S, out=out)

    for _ in range(args.warmup):
        step()
    st = torch.cuda.current_stream()  # the library launches on this stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(st)
        dart.dart_chunk_states(d["X"], d["B"], d["A"], S, dH=dH)
        ev[k][1].record(st)
        dart.dart_sma_fwd(d["Q"], d["C"], d["E"], dH, d["Y"], d["gate"], S, out=out)
        ev[k][2].record(st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    t_cs = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps / 1e3
    t_fwd = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps / 1e3

    f_sma, f_cs = fwd_flops(cfg)
    achieved = f_sma / t_fwd / 1e12
    value = b * L * args.steps / elapsed
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded torch generator on the GPU; recipe in state_memory_attention_amd/synth.py)",
        "config": {"workload": cfg["name"], "batch": b, "nheads": H, "ngroups": cfg["ngroups"],
                   "seqlen": L, "chunk": S, "d_state": cfg["d_state"], "d_head": cfg["d_head"]},
        "roofline": {"bound": "mfma", "kernel": "dart_sma_fwd", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_record("sma_fwd", cfg["name"]),
                     "flop_per_launch": f_sma, "us_per_launch": t_fwd * 1e6},
        "kernels_us": {"dart_chunk_states": t_cs * 1e6, "dart_sma_fwd": t_fwd * 1e6},
        "path_mfma_frac": (f_sma + f_cs) / (t_cs + t_fwd) / 1e12 / PEAK_BF16_TFLOPS,
    }
    result["mfma_probe"] = time_mfma_probe(torch, dH, d["Q"], args.steps, args.warmup, achieved)
    del d, dH, out
    torch.cuda.empty_cache()
    result["gemm_probe"] = time_gemm_probe(torch, args.steps, args.warmup, achieved)
    if not args.no_configs:
        result["configs"] = time_configs(torch, dart, synth, args.steps, args.warmup, args.workload)
        result["chunk_sizes"] = time_chunk_sizes(torch, dart, synth, args.steps, args.warmup)
    if not args.no_rms:
        result["rms"] = time_rms(torch, dart, synth, cfg)
    if not args.no_ssd:
        result["ssd"] = time_ssd(torch, dart, synth, cfg)
    if not args.no_backward:
        result["backward"] = time_backward(torch, dart, synth, cfg)
    if not args.no_decode:
        result["decode"] = time_decode(torch, dart, synth)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

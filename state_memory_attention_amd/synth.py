"""Seeded synthetic inputs for the DART hot path.

This module only draws inputs: it holds none of the method's arithmetic, so
both the HIP path's tests and the fp64 oracle can consume what it returns.

Recipe (one generator per call, seeded; draws in this order, each a full
C-order tensor in the library's layout):

    X ~ N(0,1)/sqrt(P)   [b][L][H][P]
    B ~ N(0,1)/sqrt(N)   [b][L][G][N]
    C ~ N(0,1)/sqrt(N)   [b][L][G][N]
    Q ~ N(0,1)/sqrt(N)   [b][L][G][N]
    E ~ N(0,1)/sqrt(P)   [b][L][G][P]
    z ~ N(-2, 0.5)       [b][L][H]        (0.5 is the standard deviation)
    a ~ U[a_lo, a_hi]    [H]              (one draw per head)
    Y ~ N(0,1)           [b][L][H][P]
    g ~ U[0,1]           [b][L][H][P]  (or [b][L][H] for a scalar gate)

and the decay fed to the library is A = exp(-softplus(z) * a), in float32.
For bf16 configurations every tensor except A is rounded to bf16 (round to
nearest even) before anyone sees it, so the oracle and the GPU consume the
same values.  ``gains`` multiplies selected tensors after the draw (used by
stress inputs that sharpen the softmax).

Two backends draw with the same recipe: ``numpy`` (PCG64, host; small and
medium sizes) and ``torch`` (Philox on the given device; full-size runs where
host generation would take minutes).  Their streams differ, each is
deterministic for a given seed.
"""
from __future__ import annotations

import math

import numpy as np

# The five workloads: one tiny fp32 case, three bf16 forward cases and one
# bf16 decode case, each named by its shape.  a_lo/a_hi bound the per-head
# decay rate.
WORKLOADS = [
    dict(name="tiny_fp32_L1024_S64_N16_P16", kind="fwd", batch=1, nheads=1, ngroups=1,
         seqlen=1024, chunk=64, d_state=16, d_head=16, dtype="f32", a_lo=1.0, a_hi=4.0),
    dict(name="block_bf16_b4_h24_L2048", kind="fwd", batch=4, nheads=24, ngroups=24,
         seqlen=2048, chunk=256, d_state=128, d_head=64, dtype="bf16", a_lo=1.0, a_hi=16.0),
    dict(name="long_bf16_b2_h24_L16384", kind="fwd", batch=2, nheads=24, ngroups=24,
         seqlen=16384, chunk=256, d_state=128, d_head=64, dtype="bf16", a_lo=1.0, a_hi=16.0),
    dict(name="vlong_bf16_b1_h32_L65536", kind="fwd", batch=1, nheads=32, ngroups=32,
         seqlen=65536, chunk=256, d_state=128, d_head=64, dtype="bf16", a_lo=1.0, a_hi=16.0),
    dict(name="decode_bf16_b64_h24_M256", kind="decode", batch=64, nheads=24, ngroups=24,
         max_chunks=256, chunk=256, d_state=128, d_head=64, dtype="bf16"),
]
TINY, BLOCK, LONG, VLONG, DECODE = (w["name"] for w in WORKLOADS)


def workload(key: str, /, **changes) -> dict:
    """A copy of the settings of the workload named `key`, with `changes`
    applied (a new `name` among them, for a variant)."""
    for w in WORKLOADS:
        if w["name"] == key:
            return dict(w, **changes)
    raise KeyError(f"no workload named {key!r}")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return
    them as float32.  Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _softplus(z):
    return np.logaddexp(0.0, z)


def fwd_shapes(batch, seqlen, nheads, ngroups, d_state, d_head):
    b, L, H, G, N, P = batch, seqlen, nheads, ngroups, d_state, d_head
    return dict(X=(b, L, H, P), B=(b, L, G, N), C=(b, L, G, N), Q=(b, L, G, N),
                E=(b, L, G, P), z=(b, L, H), a=(H,), Y=(b, L, H, P))


def draw_fwd(batch, seqlen, nheads, ngroups, d_state, d_head, dtype="bf16",
             a_lo=1.0, a_hi=16.0, seed=0, gate_per_channel=True, gains=None, **_):
    """Host (numpy) draw of one forward problem.  Returns a dict of float32
    numpy arrays X, B, C, Q, E, A, Y, gate (bf16-valued when dtype='bf16')."""
    rng = np.random.default_rng(seed)
    sh = fwd_shapes(batch, seqlen, nheads, ngroups, d_state, d_head)
    N, P = d_state, d_head
    out = {}
    out["X"] = rng.standard_normal(sh["X"], dtype=np.float32) / np.float32(math.sqrt(P))
    out["B"] = rng.standard_normal(sh["B"], dtype=np.float32) / np.float32(math.sqrt(N))
    out["C"] = rng.standard_normal(sh["C"], dtype=np.float32) / np.float32(math.sqrt(N))
    out["Q"] = rng.standard_normal(sh["Q"], dtype=np.float32) / np.float32(math.sqrt(N))
    out["E"] = rng.standard_normal(sh["E"], dtype=np.float32) / np.float32(math.sqrt(P))
    z = rng.standard_normal(sh["z"], dtype=np.float32) * np.float32(0.5) - np.float32(2.0)
    a = rng.uniform(a_lo, a_hi, size=sh["a"]).astype(np.float32)
    out["Y"] = rng.standard_normal(sh["Y"], dtype=np.float32)
    gshape = sh["Y"] if gate_per_channel else sh["z"]
    out["gate"] = rng.random(gshape, dtype=np.float32)
    out["A"] = np.exp(-_softplus(z.astype(np.float64)) * a.astype(np.float64)).astype(np.float32)
    for k, v in (gains or {}).items():
        out[k] = (out[k] * np.float32(v)).astype(np.float32)
    if dtype == "bf16":
        for k in ("X", "B", "C", "Q", "E", "Y", "gate"):
            out[k] = round_bf16(out[k])
    return out


def draw_decode(batch, nheads, ngroups, max_chunks, d_state, d_head, dtype="bf16",
                seed=0, gate_per_channel=True, gains=None, **_):
    """Host (numpy) draw of one decode problem, in this order:
    q, c ~ N(0,1)/sqrt(N) [b][G][N];  e ~ N(0,1)/sqrt(P) [b][G][P];
    cache ~ N(0,1) [b][H][Mmax][P][N] (the library's storage layout: each
    chunk memory stored with its N axis innermost);  y ~ N(0,1) [b][H][P];
    gate ~ U[0,1] [b][H][P] (or [b][H])."""
    rng = np.random.default_rng(seed)
    b, H, G, M, N, P = batch, nheads, ngroups, max_chunks, d_state, d_head
    out = {}
    out["q"] = rng.standard_normal((b, G, N), dtype=np.float32) / np.float32(math.sqrt(N))
    out["c"] = rng.standard_normal((b, G, N), dtype=np.float32) / np.float32(math.sqrt(N))
    out["e"] = rng.standard_normal((b, G, P), dtype=np.float32) / np.float32(math.sqrt(P))
    out["cache"] = rng.standard_normal((b, H, M, P, N), dtype=np.float32)
    out["y"] = rng.standard_normal((b, H, P), dtype=np.float32)
    out["gate"] = rng.random((b, H, P) if gate_per_channel else (b, H), dtype=np.float32)
    for k, v in (gains or {}).items():
        out[k] = (out[k] * np.float32(v)).astype(np.float32)
    if dtype == "bf16":
        for k in list(out):
            out[k] = round_bf16(out[k])
    return out


def draw_fwd_torch(batch, seqlen, nheads, ngroups, d_state, d_head, dtype="bf16",
                   a_lo=1.0, a_hi=16.0, seed=0, gate_per_channel=True, device="cuda",
                   gains=None, **_):
    """Same recipe as ``draw_fwd``, drawn with torch's generator on ``device``.
    Returns torch tensors already in the compute dtype (A stays float32)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    sh = fwd_shapes(batch, seqlen, nheads, ngroups, d_state, d_head)
    N, P = d_state, d_head
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    f32 = torch.float32

    def normal(shape, std=1.0, mean=0.0):
        t = torch.randn(shape, generator=gen, device=device, dtype=f32)
        if std != 1.0:
            t.mul_(std)
        if mean != 0.0:
            t.add_(mean)
        return t

    out = {}
    out["X"] = normal(sh["X"], 1.0 / math.sqrt(P))
    out["B"] = normal(sh["B"], 1.0 / math.sqrt(N))
    out["C"] = normal(sh["C"], 1.0 / math.sqrt(N))
    out["Q"] = normal(sh["Q"], 1.0 / math.sqrt(N))
    out["E"] = normal(sh["E"], 1.0 / math.sqrt(P))
    z = normal(sh["z"], 0.5, -2.0)
    a = torch.rand(sh["a"], generator=gen, device=device, dtype=f32) * (a_hi - a_lo) + a_lo
    out["Y"] = normal(sh["Y"])
    gshape = sh["Y"] if gate_per_channel else sh["z"]
    out["gate"] = torch.rand(gshape, generator=gen, device=device, dtype=f32)
    out["A"] = torch.exp(-torch.nn.functional.softplus(z.double()) * a.double()).to(f32)
    for k, v in (gains or {}).items():
        out[k] = out[k] * v
    for k in ("X", "B", "C", "Q", "E", "Y", "gate"):
        out[k] = out[k].to(tdt).contiguous()
    return out


def draw_decode_torch(batch, nheads, ngroups, max_chunks, d_state, d_head, dtype="bf16",
                      seed=0, gate_per_channel=True, device="cuda", **_):
    """Same recipe as ``draw_decode``, drawn with torch's generator on ``device``."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    b, H, G, M, N, P = batch, nheads, ngroups, max_chunks, d_state, d_head
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    f32 = torch.float32
    out = {}
    out["q"] = torch.randn((b, G, N), generator=gen, device=device, dtype=f32) / math.sqrt(N)
    out["c"] = torch.randn((b, G, N), generator=gen, device=device, dtype=f32) / math.sqrt(N)
    out["e"] = torch.randn((b, G, P), generator=gen, device=device, dtype=f32) / math.sqrt(P)
    cache = torch.empty((b, H, M, P, N), device=device, dtype=tdt)
    for bi in range(b):  # one batch row at a time keeps the float32 staging small
        cache[bi] = torch.randn((H, M, P, N), generator=gen, device=device, dtype=f32).to(tdt)
    out["cache"] = cache
    out["y"] = torch.randn((b, H, P), generator=gen, device=device, dtype=f32)
    out["gate"] = torch.rand((b, H, P) if gate_per_channel else (b, H), generator=gen,
                             device=device, dtype=f32)
    for k in ("q", "c", "e", "y", "gate"):
        out[k] = out[k].to(tdt).contiguous()
    return out


def draw_memories(batch, nheads, n_chunks, d_state, d_head, dtype="bf16", std=1.0, seed=0):
    """Host draw of chunk memories for the forward or decode call alone:
    i.i.d. N(0, std^2) in the library's storage layout [b][H][M][P][N]
    (each memory with its N axis innermost), bf16-rounded for bf16."""
    rng = np.random.default_rng(seed)
    m = rng.standard_normal((batch, nheads, n_chunks, d_head, d_state), dtype=np.float32)
    m *= np.float32(std)
    return round_bf16(m) if dtype == "bf16" else m


def draw_grad(shape, dtype="bf16", seed=0) -> np.ndarray:
    """Loss gradient dout ~ N(0, 1) of the given shape (numpy float32,
    bf16-valued when dtype='bf16'), for the backward pass."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(shape, dtype=np.float32)
    return round_bf16(g) if dtype == "bf16" else g


def draw_grad_torch(shape, dtype="bf16", seed=0):
    """GPU draw of a loss gradient of the given shape, N(0, 1)."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    t = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)

"""Shared helpers for the GPU parity tests: the error metric, host/device
conversion, and the oracle evaluated on the exact values the GPU consumed."""
import math
import sys

import numpy as np
import torch

import oracle as O

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max-abs-normalised, fp32 / bf16 inputs
# R and lse of the forward/decode call computed from the same inputs as the
# oracle: float32 dot products of exact bf16 products and a float32 softmax;
# the bound leaves two orders of magnitude over the expected ~1e-5.
TOL_SAME_INPUT = {"f32": 1e-4, "bf16": 1e-3}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def dev(x, dtype="f32"):
    """numpy float32 array -> contiguous GPU tensor (exact for bf16-valued input)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(tdtype(dtype)).contiguous()


def host(t):
    return t.detach().to(torch.float64).cpu().numpy()


def err(gpu, ref):
    """max |gpu - ref| / max |ref| over finite reference entries (absolute
    if the reference is all zero); -inf entries must match exactly."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    ninf = np.isneginf(ref)
    assert np.array_equal(ninf, np.isneginf(gpu)), "-inf positions differ"
    fin = ~ninf
    if not fin.any():
        return 0.0
    assert np.isfinite(gpu[fin]).all(), "non-finite GPU value where the reference is finite"
    scale = np.abs(ref[fin]).max()
    diff = np.abs(gpu[fin] - ref[fin]).max()
    return float(diff / scale) if scale > 0 else float(diff)


def to_oracle_mem(mem_gpu_layout):
    """[..., P, N] storage -> the oracle's [..., N, P] orientation."""
    return np.swapaxes(np.asarray(mem_gpu_layout, dtype=np.float64), -1, -2)


def oracle_head_states(X, B, A, b, h, G, H, S):
    g = h // (H // G)
    return O.chunk_states_head(X[b, :, h], B[b, :, g], A[b, :, h], S)


def f64(t):
    """torch tensor (any device, any dtype, any strides) -> numpy float64."""
    return t.detach().to("cpu").to(torch.float64).numpy()


class MaxErr:
    """The max-abs-normalised error of ``err`` for one output tensor that is
    checked in pieces (one batch row and head at a time, so that host memory
    stays bounded): running max |gpu - ref| and max |ref| over every piece,
    with the same -inf and finiteness rules."""

    def __init__(self, name):
        self.name, self.diff, self.scale, self.worst, self.count = name, 0.0, 0.0, None, 0

    def add(self, gpu, ref, where=None):
        gpu = np.asarray(gpu, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert gpu.shape == ref.shape, (self.name, where, gpu.shape, ref.shape)
        ninf = np.isneginf(ref)
        assert np.array_equal(ninf, np.isneginf(gpu)), f"{self.name}: -inf positions differ at {where}"
        fin = ~ninf
        self.count += int(gpu.size)
        if not fin.any():
            return
        assert np.isfinite(gpu[fin]).all(), f"{self.name}: non-finite GPU value at {where}"
        d = float(np.abs(gpu[fin] - ref[fin]).max())
        if d > self.diff:
            self.diff, self.worst = d, where
        self.scale = max(self.scale, float(np.abs(ref[fin]).max()))

    def err(self):
        return self.diff / self.scale if self.scale > 0 else self.diff

    def check(self, tol):
        e = self.err()
        say(f"  {self.name}: {e:.2e} over {self.count} entries (largest difference at {self.worst})")
        assert e <= tol, (self.name, e, self.worst)
        return e


def same(x, y, what):
    """Bitwise equality of two GPU results; on a mismatch, say how many
    elements differ, where (the first three indices of the differing
    elements, up to twelve of them) and by how much."""
    if torch.equal(x, y):
        return
    diff = x != y
    idx = diff.nonzero()
    n = int(diff.sum())
    where = sorted(set(tuple(r) for r in idx[:, :3].tolist()))[:12]
    md = float((x.float() - y.float()).abs().max())
    raise AssertionError(f"{what}: {n} of {x.numel()} elements differ, first (i0, i1, i2) {where}, "
                         f"max |diff| {md:.3e}")

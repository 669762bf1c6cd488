"""Python binding of the DART C ABI (libdart.so).

Argument marshalling only: shapes and dtypes are read from torch tensors, the
pointers and torch's current HIP stream are handed to the library, and every
step of the computation runs in its HIP kernels.  If libdart.so is missing or
cannot be loaded, every call raises: there is no fallback implementation.

Layouts (see include/dart.h):
    X, Y, out, R  (b, L, H, P)     B, C, Q  (b, L, G, N)     E  (b, L, G, P)
    A             (b, L, H) float32            gate (b, L, H, P) or (b, L, H)
    dH            (b, H, M, P, N)  -- each chunk memory with its N axis innermost
    lse           (b, H, L) float32
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdart.so")

DART_F32, DART_BF16 = 0, 1
DART_PATH_AUTO, DART_PATH_GENERAL = 0, 1
STATUS = {0: "DART_OK", -1: "DART_ERR_NULL", -2: "DART_ERR_SHAPE", -3: "DART_ERR_UNSUPPORTED",
          -4: "DART_ERR_WORKSPACE", -5: "DART_ERR_HIP", -6: "DART_ERR_ALIGN"}

ENTRY_POINTS = ("dart_chunk_states", "dart_sma_fwd", "dart_sma_decode",
                "dart_sma_decode_workspace_bytes", "dart_sma_decode_noalloc", "dart_sma_bwd", "dart_sma_bwd_workspace_bytes",
                "dart_chunk_states_bwd", "dart_chunk_states_bwd_workspace_bytes",
                "dart_decode_state_update",
                "dart_chunk_states_rms", "dart_chunk_rms", "dart_sma_fwd_rms", "dart_sma_decode_rms",
                "dart_decode_state_update_rms", "dart_sma_bwd_rms", "dart_sma_bwd_rms_workspace_bytes",
                "dart_ssd_fwd", "dart_ssd_fwd_workspace_bytes",
                "dart_status_string", "dart_last_error", "dart_abi_version", "dart_set_path")


class DartError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("d_state", ctypes.c_int64), ("d_head", ctypes.c_int64),
                ("chunk", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdart.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m state_memory_attention_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    dp = ctypes.POINTER(Dims)
    L.dart_chunk_states.argtypes = [dp, i32, vp, vp, vp, vp, vp]
    L.dart_chunk_states.restype = i32
    L.dart_sma_fwd.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    L.dart_sma_fwd.restype = i32
    L.dart_sma_decode.argtypes = [dp, i32, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                  ctypes.c_size_t, vp]
    L.dart_sma_decode.restype = i32
    L.dart_sma_decode_workspace_bytes.argtypes = [dp, i64]
    L.dart_sma_decode_workspace_bytes.restype = ctypes.c_size_t
    L.dart_sma_decode_noalloc.argtypes = [dp, i32, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    L.dart_sma_decode_noalloc.restype = i32
    L.dart_sma_bwd.argtypes = [dp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                               vp, ctypes.c_size_t, vp]
    L.dart_sma_bwd.restype = i32
    L.dart_sma_bwd_workspace_bytes.argtypes = [dp]
    L.dart_sma_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.dart_chunk_states_bwd.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.dart_chunk_states_bwd.restype = i32
    L.dart_chunk_states_bwd_workspace_bytes.argtypes = [dp]
    L.dart_chunk_states_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.dart_decode_state_update.argtypes = [dp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dart_decode_state_update.restype = i32
    f32 = ctypes.c_float
    L.dart_chunk_states_rms.argtypes = [dp, i32, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp]
    L.dart_chunk_states_rms.restype = i32
    L.dart_chunk_rms.argtypes = [dp, i32, vp, f32, vp, vp, vp, vp, vp]
    L.dart_chunk_rms.restype = i32
    L.dart_sma_fwd_rms.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp]
    L.dart_sma_fwd_rms.restype = i32
    L.dart_sma_bwd_rms.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp,
                                   vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.dart_sma_bwd_rms.restype = i32
    L.dart_sma_bwd_rms_workspace_bytes.argtypes = [dp]
    L.dart_sma_bwd_rms_workspace_bytes.restype = ctypes.c_size_t
    L.dart_sma_decode_rms.argtypes = [dp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp,
                                      vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.dart_sma_decode_rms.restype = i32
    L.dart_decode_state_update_rms.argtypes = [dp, i32, i64, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dart_decode_state_update_rms.restype = i32
    L.dart_ssd_fwd.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.dart_ssd_fwd.restype = i32
    L.dart_ssd_fwd_workspace_bytes.argtypes = [dp, i32]
    L.dart_ssd_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.dart_status_string.argtypes = [i32]
    L.dart_status_string.restype = ctypes.c_char_p
    L.dart_last_error.argtypes = []
    L.dart_last_error.restype = ctypes.c_char_p
    L.dart_abi_version.argtypes = []
    L.dart_abi_version.restype = i32
    L.dart_set_path.argtypes = [i32]
    L.dart_set_path.restype = i32
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise DartError(status, lib().dart_last_error().decode())


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return DART_F32
    if dtype == torch.bfloat16:
        return DART_BF16
    raise DartError(-3, f"unsupported dtype {dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    if t.device.type != "cuda":
        raise DartError(-1, "tensors must live on the GPU")
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, shape, dtype, device):
    if t is None:
        raise DartError(-1, f"{name} is None")
    if tuple(t.shape) != tuple(shape):
        raise DartError(-2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise DartError(-3, f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise DartError(-2, f"{name} must be contiguous")
    if t.device != device:
        raise DartError(-2, f"{name} is on {t.device}, expected {device}")


def num_chunks(L: int, S: int) -> int:
    return -(-L // S)


def set_path(path: int) -> int:
    """Select the kernels for this thread (DART_PATH_AUTO or DART_PATH_GENERAL)."""
    return lib().dart_set_path(path)


def abi_version() -> int:
    return lib().dart_abi_version()


def dart_chunk_states(X: torch.Tensor, B: torch.Tensor, A: torch.Tensor, chunk: int,
                      dH: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunk state memories dH (b, H, M, P, N) from X (b, L, H, P),
    B (b, L, G, N) and the float32 decays A (b, L, H)."""
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = X.device, X.dtype
    _need(B, "B", (b, L, G, N), dt, dev)
    _need(A, "A", (b, L, H), torch.float32, dev)
    _need(X, "X", (b, L, H, P), dt, dev)
    if dH is None:
        dH = torch.empty((b, H, M, P, N), dtype=dt, device=dev)
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    dims = Dims(b, L, H, G, N, P, chunk)
    _check(lib().dart_chunk_states(ctypes.byref(dims), _code(dt), _ptr(X), _ptr(B), _ptr(A),
                                   _ptr(dH), _stream(X)))
    return dH


def dart_sma_fwd(Q: torch.Tensor, C: torch.Tensor, E: torch.Tensor, dH: torch.Tensor,
                 Y: torch.Tensor, gate: torch.Tensor, chunk: int,
                 out: Optional[torch.Tensor] = None, R: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, want_R: bool = False,
                 want_lse: bool = False):
    """SMA readout and gated residual.  Returns (out, R, lse); R and lse are
    None unless requested (want_R / want_lse) or passed in."""
    b, L, G, N = Q.shape
    H, P = Y.shape[2], Y.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = Q.device, Q.dtype
    _need(C, "C", (b, L, G, N), dt, dev)
    _need(E, "E", (b, L, G, P), dt, dev)
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    _need(Y, "Y", (b, L, H, P), dt, dev)
    gpc = gate.dim() == 4
    _need(gate, "gate", (b, L, H, P) if gpc else (b, L, H), dt, dev)
    if out is None:
        out = torch.empty((b, L, H, P), dtype=dt, device=dev)
    _need(out, "out", (b, L, H, P), dt, dev)
    if R is None and want_R:
        R = torch.empty((b, L, H, P), dtype=torch.float32, device=dev)
    if R is not None:
        _need(R, "R", (b, L, H, P), torch.float32, dev)
    if lse is None and want_lse:
        lse = torch.empty((b, H, L), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (b, H, L), torch.float32, dev)
    dims = Dims(b, L, H, G, N, P, chunk)
    _check(lib().dart_sma_fwd(ctypes.byref(dims), _code(dt), _ptr(Q), _ptr(C), _ptr(E), _ptr(dH),
                              _ptr(Y), _ptr(gate), int(gpc), _ptr(out), _ptr(R), _ptr(lse),
                              _stream(Q)))
    return out, R, lse


def decode_workspace_bytes(batch: int, nheads: int, d_head: int, max_chunks: int,
                           ngroups: int = 1, d_state: int = 1) -> int:
    dims = Dims(batch, 1, nheads, ngroups, d_state, d_head, 1)
    return int(lib().dart_sma_decode_workspace_bytes(ctypes.byref(dims), max_chunks))


def _decode_args(q, c, e, cache, y, gate, n_chunks, out, R, lse, want_R, want_lse):
    """Shape checks and output allocation shared by the decode wrappers."""
    b, G, N = q.shape
    H, Mx, P = cache.shape[1], cache.shape[2], cache.shape[3]
    dev, dt = q.device, q.dtype
    _need(c, "c", (b, G, N), dt, dev)
    _need(e, "e", (b, G, P), dt, dev)
    _need(cache, "cache", (b, H, Mx, P, N), dt, dev)
    _need(y, "y", (b, H, P), dt, dev)
    gpc = gate.dim() == 3
    _need(gate, "gate", (b, H, P) if gpc else (b, H), dt, dev)
    if n_chunks is not None:
        _need(n_chunks, "n_chunks", (b,), torch.int32, dev)
    if out is None:
        out = torch.empty((b, H, P), dtype=dt, device=dev)
    _need(out, "out", (b, H, P), dt, dev)
    if R is None and want_R:
        R = torch.empty((b, H, P), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((b, H), dtype=torch.float32, device=dev)
    return Dims(b, 1, H, G, N, P, 1), Mx, gpc, out, R, lse


def dart_sma_decode_noalloc(q: torch.Tensor, c: torch.Tensor, e: torch.Tensor, cache: torch.Tensor,
                            y: torch.Tensor, gate: torch.Tensor, n_chunks: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, R: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, want_R: bool = False, want_lse: bool = False):
    """dart_sma_decode without a workspace: the library's own per-GPU scratch
    holds the split partials (the C call allocates nothing; pass out, R and
    lse to allocate nothing here either).  Returns (out, R, lse)."""
    dims, Mx, gpc, out, R, lse = _decode_args(q, c, e, cache, y, gate, n_chunks, out, R, lse, want_R, want_lse)
    _check(lib().dart_sma_decode_noalloc(ctypes.byref(dims), _code(q.dtype), Mx, _ptr(q), _ptr(c), _ptr(e),
                                         _ptr(cache), _ptr(n_chunks), _ptr(y), _ptr(gate), int(gpc),
                                         _ptr(out), _ptr(R), _ptr(lse), _stream(q)))
    return out, R, lse


def dart_sma_decode(q: torch.Tensor, c: torch.Tensor, e: torch.Tensor, cache: torch.Tensor,
                    y: torch.Tensor, gate: torch.Tensor, n_chunks: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, R: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    want_R: bool = False, want_lse: bool = False):
    """Decode one new token per batch row against cache (b, H, Mmax, P, N).
    Returns (out, R, lse)."""
    dims, Mx, gpc, out, R, lse = _decode_args(q, c, e, cache, y, gate, n_chunks, out, R, lse, want_R, want_lse)
    dev, dt = q.device, q.dtype
    need = int(lib().dart_sma_decode_workspace_bytes(ctypes.byref(dims), Mx))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib().dart_sma_decode(ctypes.byref(dims), _code(dt), Mx, _ptr(q), _ptr(c), _ptr(e),
                                 _ptr(cache), _ptr(n_chunks), _ptr(y), _ptr(gate), int(gpc),
                                 _ptr(out), _ptr(R), _ptr(lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(q)))
    return out, R, lse


def _workspace(need: int, dev, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    return workspace


def dart_sma_bwd(Q: torch.Tensor, C: torch.Tensor, E: torch.Tensor, dH: torch.Tensor,
                 gate: torch.Tensor, R: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                 chunk: int, want_dgate: bool = True, workspace: Optional[torch.Tensor] = None):
    """Gradients of out = Y + gate * R(Q, C, E, dH) for dout (b, L, H, P),
    from the forward's R and lse.  Returns float32 (dQ, dC, dE, d_dH, dgate);
    dQ, dC, dE are summed over the heads of a group, d_dH has the dH layout
    (b, H, M, P, N), dgate is None unless want_dgate.  The gradient of Y is
    dout itself."""
    b, L, G, N = Q.shape
    H, P = dout.shape[2], dout.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = Q.device, Q.dtype
    f32 = torch.float32
    _need(C, "C", (b, L, G, N), dt, dev)
    _need(E, "E", (b, L, G, P), dt, dev)
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    gpc = gate.dim() == 4
    _need(gate, "gate", (b, L, H, P) if gpc else (b, L, H), dt, dev)
    _need(R, "R", (b, L, H, P), f32, dev)
    _need(lse, "lse", (b, H, L), f32, dev)
    _need(dout, "dout", (b, L, H, P), dt, dev)
    dQ = torch.empty((b, L, G, N), dtype=f32, device=dev)
    dC = torch.empty((b, L, G, N), dtype=f32, device=dev)
    dE = torch.empty((b, L, G, P), dtype=f32, device=dev)
    ddH = torch.empty((b, H, M, P, N), dtype=f32, device=dev)
    dgate = torch.empty(gate.shape, dtype=f32, device=dev) if want_dgate else None
    dims = Dims(b, L, H, G, N, P, chunk)
    need = int(lib().dart_sma_bwd_workspace_bytes(ctypes.byref(dims)))
    workspace = _workspace(need, dev, workspace)
    _check(lib().dart_sma_bwd(ctypes.byref(dims), _code(dt), _ptr(Q), _ptr(C), _ptr(E), _ptr(dH),
                              _ptr(gate), int(gpc), _ptr(R), _ptr(lse), _ptr(dout), _ptr(dQ),
                              _ptr(dC), _ptr(dE), _ptr(ddH), _ptr(dgate), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(Q)))
    return dQ, dC, dE, ddH, dgate


def dart_chunk_states_bwd(X: torch.Tensor, B: torch.Tensor, A: torch.Tensor, ddH: torch.Tensor,
                          chunk: int, workspace: Optional[torch.Tensor] = None):
    """Gradients of dH = chunk_states(X, B, A) for d_dH (b, H, M, P, N)
    float32.  Returns float32 (dX, dB, dA); dB is summed over the heads of a
    group."""
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = X.device, X.dtype
    f32 = torch.float32
    _need(B, "B", (b, L, G, N), dt, dev)
    _need(A, "A", (b, L, H), f32, dev)
    _need(ddH, "d_dH", (b, H, M, P, N), f32, dev)
    dX = torch.empty((b, L, H, P), dtype=f32, device=dev)
    dB = torch.empty((b, L, G, N), dtype=f32, device=dev)
    dA = torch.empty((b, L, H), dtype=f32, device=dev)
    dims = Dims(b, L, H, G, N, P, chunk)
    need = int(lib().dart_chunk_states_bwd_workspace_bytes(ctypes.byref(dims)))
    workspace = _workspace(need, dev, workspace)
    _check(lib().dart_chunk_states_bwd(ctypes.byref(dims), _code(dt), _ptr(X), _ptr(B), _ptr(A),
                                       _ptr(ddH), _ptr(dX), _ptr(dB), _ptr(dA), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(X)))
    return dX, dB, dA


def dart_decode_state_update(x: torch.Tensor, B: torch.Tensor, a: torch.Tensor,
                             state: torch.Tensor, pos: torch.Tensor, cache: torch.Tensor,
                             chunk: int, n_chunks: Optional[torch.Tensor] = None) -> None:
    """Absorb one new token per batch row into the in-progress chunk memory
    state (b, H, P, N) float32; a chunk the token closes is written to cache
    (b, H, Mmax, P, N).  x (b, H, P), B (b, G, N), a (b, H) float32, pos (b,)
    int32 absolute token positions; n_chunks (b,) int32 receives the number of
    complete chunks.  Updates state, cache and n_chunks in place."""
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    Mx = cache.shape[2]
    dev, dt = x.device, x.dtype
    _need(B, "B", (b, G, N), dt, dev)
    _need(a, "a", (b, H), torch.float32, dev)
    _need(state, "state", (b, H, P, N), torch.float32, dev)
    _need(pos, "pos", (b,), torch.int32, dev)
    _need(cache, "cache", (b, H, Mx, P, N), dt, dev)
    if n_chunks is not None:
        _need(n_chunks, "n_chunks", (b,), torch.int32, dev)
    dims = Dims(b, 1, H, G, N, P, chunk)
    _check(lib().dart_decode_state_update(ctypes.byref(dims), _code(dt), Mx, _ptr(x), _ptr(B),
                                          _ptr(a), _ptr(state), _ptr(pos), _ptr(cache),
                                          _ptr(n_chunks), _stream(x)))


# ---------------------------------------------------------------------------
# RMS-normalised score branch
# ---------------------------------------------------------------------------

def score_dtype(dtype: torch.dtype) -> torch.dtype:
    """Storage type of the score memory: float16 for bfloat16 inputs, else float32."""
    return torch.float16 if dtype == torch.bfloat16 else torch.float32


def _weight(w, name, n, dev):
    if w is not None:
        _need(w, name, (n,), torch.float32, dev)
    return w


def dart_chunk_states_rms(X: torch.Tensor, B: torch.Tensor, A: torch.Tensor, chunk: int, eps: float,
                          w_q: Optional[torch.Tensor] = None, w_e: Optional[torch.Tensor] = None,
                          dH: Optional[torch.Tensor] = None, r: Optional[torch.Tensor] = None,
                          dH_score: Optional[torch.Tensor] = None, want_r: bool = True,
                          want_score: bool = True):
    """Chunk memories dH (b, H, M, P, N), their inverse RMS r (b, H, M, N)
    float32 and the score memory (b, H, M, P, N) with the RMSNorm weights
    w_q (N,), w_e (P,) folded in.  Returns (dH, r, dH_score)."""
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = X.device, X.dtype
    _need(X, "X", (b, L, H, P), dt, dev)
    _need(B, "B", (b, L, G, N), dt, dev)
    _need(A, "A", (b, L, H), torch.float32, dev)
    _weight(w_q, "w_q", N, dev)
    _weight(w_e, "w_e", P, dev)
    if dH is None:
        dH = torch.empty((b, H, M, P, N), dtype=dt, device=dev)
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    if r is None and want_r:
        r = torch.empty((b, H, M, N), dtype=torch.float32, device=dev)
    if r is not None:
        _need(r, "r", (b, H, M, N), torch.float32, dev)
    if dH_score is None and want_score:
        dH_score = torch.empty((b, H, M, P, N), dtype=score_dtype(dt), device=dev)
    if dH_score is not None:
        _need(dH_score, "dH_score", (b, H, M, P, N), score_dtype(dt), dev)
    dims = Dims(b, L, H, G, N, P, chunk)
    _check(lib().dart_chunk_states_rms(ctypes.byref(dims), _code(dt), _ptr(X), _ptr(B), _ptr(A),
                                       float(eps), _ptr(w_q), _ptr(w_e), _ptr(dH), _ptr(r),
                                       _ptr(dH_score), _stream(X)))
    return dH, r, dH_score


def dart_chunk_rms(dH: torch.Tensor, chunk_count_L: int, chunk: int, eps: float,
                   w_q: Optional[torch.Tensor] = None, w_e: Optional[torch.Tensor] = None,
                   r: Optional[torch.Tensor] = None, dH_score: Optional[torch.Tensor] = None,
                   want_r: bool = True, want_score: bool = True):
    """r (b, H, M, N) and the score memory of given chunk memories
    dH (b, H, M, P, N), M = ceil(chunk_count_L / chunk).  Returns (r, dH_score)."""
    b, H, M, P, N = dH.shape
    dev, dt = dH.device, dH.dtype
    if num_chunks(chunk_count_L, chunk) != M:
        raise DartError(-2, f"dH holds {M} chunks, L={chunk_count_L}, S={chunk} give "
                            f"{num_chunks(chunk_count_L, chunk)}")
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    _weight(w_q, "w_q", N, dev)
    _weight(w_e, "w_e", P, dev)
    if r is None and want_r:
        r = torch.empty((b, H, M, N), dtype=torch.float32, device=dev)
    if dH_score is None and want_score:
        dH_score = torch.empty((b, H, M, P, N), dtype=score_dtype(dt), device=dev)
    if r is not None:
        _need(r, "r", (b, H, M, N), torch.float32, dev)
    if dH_score is not None:
        _need(dH_score, "dH_score", (b, H, M, P, N), score_dtype(dt), dev)
    dims = Dims(b, chunk_count_L, H, 1, N, P, chunk)
    _check(lib().dart_chunk_rms(ctypes.byref(dims), _code(dt), _ptr(dH), float(eps), _ptr(w_q), _ptr(w_e),
                                _ptr(r), _ptr(dH_score), _stream(dH)))
    return r, dH_score


def dart_sma_fwd_rms(Q: torch.Tensor, C: torch.Tensor, E: torch.Tensor, dH: torch.Tensor,
                     dH_score: torch.Tensor, Y: torch.Tensor, gate: torch.Tensor, chunk: int,
                     eps: float, out: Optional[torch.Tensor] = None, R: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_R: bool = False, want_lse: bool = False):
    """SMA with the normalised score branch and the gated residual.
    Returns (out, R, lse)."""
    b, L, G, N = Q.shape
    H, P = Y.shape[2], Y.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = Q.device, Q.dtype
    _need(C, "C", (b, L, G, N), dt, dev)
    _need(E, "E", (b, L, G, P), dt, dev)
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    _need(dH_score, "dH_score", (b, H, M, P, N), score_dtype(dt), dev)
    _need(Y, "Y", (b, L, H, P), dt, dev)
    gpc = gate.dim() == 4
    _need(gate, "gate", (b, L, H, P) if gpc else (b, L, H), dt, dev)
    if out is None:
        out = torch.empty((b, L, H, P), dtype=dt, device=dev)
    _need(out, "out", (b, L, H, P), dt, dev)
    if R is None and want_R:
        R = torch.empty((b, L, H, P), dtype=torch.float32, device=dev)
    if R is not None:
        _need(R, "R", (b, L, H, P), torch.float32, dev)
    if lse is None and want_lse:
        lse = torch.empty((b, H, L), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (b, H, L), torch.float32, dev)
    dims = Dims(b, L, H, G, N, P, chunk)
    _check(lib().dart_sma_fwd_rms(ctypes.byref(dims), _code(dt), _ptr(Q), _ptr(C), _ptr(E), _ptr(dH),
                                  _ptr(dH_score), _ptr(Y), _ptr(gate), int(gpc), float(eps), _ptr(out),
                                  _ptr(R), _ptr(lse), _stream(Q)))
    return out, R, lse


def dart_sma_bwd_rms(Q: torch.Tensor, C: torch.Tensor, E: torch.Tensor, dH: torch.Tensor,
                     dH_score: torch.Tensor, gate: torch.Tensor, R: torch.Tensor, lse: torch.Tensor,
                     dout: torch.Tensor, chunk: int, eps: float, w_q: Optional[torch.Tensor] = None,
                     w_e: Optional[torch.Tensor] = None, want_dgate: bool = True,
                     want_dw: bool = False, workspace: Optional[torch.Tensor] = None):
    """Gradients of out = Y + gate * R for the normalised score branch, from
    the forward's R and lse and the score memory it consumed.  Returns float32
    (dQ, dC, dE, d_dH, dgate, dw_q, dw_e); dgate is None unless want_dgate,
    dw_q (N,) and dw_e (P,) None unless want_dw (the gradient with respect to
    each RMSNorm weight at its value, 1 where it is not given)."""
    b, L, G, N = Q.shape
    H, P = dout.shape[2], dout.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = Q.device, Q.dtype
    f32 = torch.float32
    _need(C, "C", (b, L, G, N), dt, dev)
    _need(E, "E", (b, L, G, P), dt, dev)
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    _need(dH_score, "dH_score", (b, H, M, P, N), score_dtype(dt), dev)
    gpc = gate.dim() == 4
    _need(gate, "gate", (b, L, H, P) if gpc else (b, L, H), dt, dev)
    _need(R, "R", (b, L, H, P), f32, dev)
    _need(lse, "lse", (b, H, L), f32, dev)
    _need(dout, "dout", (b, L, H, P), dt, dev)
    if w_q is not None:
        _need(w_q, "w_q", (N,), f32, dev)
    if w_e is not None:
        _need(w_e, "w_e", (P,), f32, dev)
    dQ = torch.empty((b, L, G, N), dtype=f32, device=dev)
    dC = torch.empty((b, L, G, N), dtype=f32, device=dev)
    dE = torch.empty((b, L, G, P), dtype=f32, device=dev)
    ddH = torch.empty((b, H, M, P, N), dtype=f32, device=dev)
    dgate = torch.empty(gate.shape, dtype=f32, device=dev) if want_dgate else None
    dwq = torch.empty((N,), dtype=f32, device=dev) if want_dw else None
    dwe = torch.empty((P,), dtype=f32, device=dev) if want_dw else None
    dims = Dims(b, L, H, G, N, P, chunk)
    need = int(lib().dart_sma_bwd_rms_workspace_bytes(ctypes.byref(dims)))
    workspace = _workspace(need, dev, workspace)
    _check(lib().dart_sma_bwd_rms(ctypes.byref(dims), _code(dt), _ptr(Q), _ptr(C), _ptr(E), _ptr(dH),
                                  _ptr(dH_score), _ptr(gate), int(gpc), float(eps), _ptr(w_q), _ptr(w_e),
                                  _ptr(R), _ptr(lse), _ptr(dout), _ptr(dQ), _ptr(dC), _ptr(dE), _ptr(ddH),
                                  _ptr(dgate), _ptr(dwq), _ptr(dwe), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(Q)))
    return dQ, dC, dE, ddH, dgate, dwq, dwe


def dart_sma_decode_rms(q: torch.Tensor, c: torch.Tensor, e: torch.Tensor, cache: torch.Tensor,
                        r_cache: torch.Tensor, y: torch.Tensor, gate: torch.Tensor, eps: float,
                        w_q: Optional[torch.Tensor] = None, w_e: Optional[torch.Tensor] = None,
                        n_chunks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        R: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, want_R: bool = False,
                        want_lse: bool = False):
    """Decode with the normalised score branch: cache (b, H, Mmax, P, N) and
    r_cache (b, H, Mmax, N) float32.  Returns (out, R, lse)."""
    b, G, N = q.shape
    H, Mx, P = cache.shape[1], cache.shape[2], cache.shape[3]
    dev, dt = q.device, q.dtype
    _need(c, "c", (b, G, N), dt, dev)
    _need(e, "e", (b, G, P), dt, dev)
    _need(cache, "cache", (b, H, Mx, P, N), dt, dev)
    _need(r_cache, "r_cache", (b, H, Mx, N), torch.float32, dev)
    _need(y, "y", (b, H, P), dt, dev)
    _weight(w_q, "w_q", N, dev)
    _weight(w_e, "w_e", P, dev)
    gpc = gate.dim() == 3
    _need(gate, "gate", (b, H, P) if gpc else (b, H), dt, dev)
    if n_chunks is not None:
        _need(n_chunks, "n_chunks", (b,), torch.int32, dev)
    if out is None:
        out = torch.empty((b, H, P), dtype=dt, device=dev)
    _need(out, "out", (b, H, P), dt, dev)
    if R is None and want_R:
        R = torch.empty((b, H, P), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((b, H), dtype=torch.float32, device=dev)
    dims = Dims(b, 1, H, G, N, P, 1)
    need = int(lib().dart_sma_decode_workspace_bytes(ctypes.byref(dims), Mx))
    workspace = _workspace(need, dev, workspace)
    _check(lib().dart_sma_decode_rms(ctypes.byref(dims), _code(dt), Mx, _ptr(q), _ptr(c), _ptr(e),
                                     _ptr(cache), _ptr(r_cache), _ptr(n_chunks), _ptr(y), _ptr(gate),
                                     int(gpc), float(eps), _ptr(w_q), _ptr(w_e), _ptr(out), _ptr(R),
                                     _ptr(lse), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(q)))
    return out, R, lse


def dart_decode_state_update_rms(x: torch.Tensor, B: torch.Tensor, a: torch.Tensor,
                                 state: torch.Tensor, pos: torch.Tensor, cache: torch.Tensor,
                                 r_cache: torch.Tensor, chunk: int, eps: float,
                                 n_chunks: Optional[torch.Tensor] = None) -> None:
    """dart_decode_state_update, also writing r_cache (b, H, Mmax, N) float32
    for every chunk the token closes."""
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    Mx = cache.shape[2]
    dev, dt = x.device, x.dtype
    _need(B, "B", (b, G, N), dt, dev)
    _need(a, "a", (b, H), torch.float32, dev)
    _need(state, "state", (b, H, P, N), torch.float32, dev)
    _need(pos, "pos", (b,), torch.int32, dev)
    _need(cache, "cache", (b, H, Mx, P, N), dt, dev)
    _need(r_cache, "r_cache", (b, H, Mx, N), torch.float32, dev)
    if n_chunks is not None:
        _need(n_chunks, "n_chunks", (b,), torch.int32, dev)
    dims = Dims(b, 1, H, G, N, P, chunk)
    _check(lib().dart_decode_state_update_rms(ctypes.byref(dims), _code(dt), Mx, float(eps), _ptr(x),
                                              _ptr(B), _ptr(a), _ptr(state), _ptr(pos), _ptr(cache),
                                              _ptr(r_cache), _ptr(n_chunks), _stream(x)))


# ---------------------------------------------------------------------------
# SSM branch by the chunked scan
# ---------------------------------------------------------------------------

def dart_ssd_fwd(X: torch.Tensor, B: torch.Tensor, C: torch.Tensor, A: torch.Tensor, chunk: int,
                 H0: Optional[torch.Tensor] = None, Y: Optional[torch.Tensor] = None,
                 dH: Optional[torch.Tensor] = None, H_final: Optional[torch.Tensor] = None,
                 want_final: bool = False, workspace: Optional[torch.Tensor] = None):
    """Y_t = C_t H_t of the SSM branch, with the chunk memories dH
    (b, H, M, P, N).  X (b, L, H, P), B, C (b, L, G, N), A (b, L, H) float32,
    H0 (b, H, P, N) float32 or None.  Returns (Y, dH, H_final)."""
    b, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    M = num_chunks(L, chunk)
    dev, dt = X.device, X.dtype
    _need(X, "X", (b, L, H, P), dt, dev)
    _need(B, "B", (b, L, G, N), dt, dev)
    _need(C, "C", (b, L, G, N), dt, dev)
    _need(A, "A", (b, L, H), torch.float32, dev)
    if H0 is not None:
        _need(H0, "H0", (b, H, P, N), torch.float32, dev)
    if Y is None:
        Y = torch.empty((b, L, H, P), dtype=dt, device=dev)
    _need(Y, "Y", (b, L, H, P), dt, dev)
    if dH is None:
        dH = torch.empty((b, H, M, P, N), dtype=dt, device=dev)
    _need(dH, "dH", (b, H, M, P, N), dt, dev)
    if H_final is None and want_final:
        H_final = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    if H_final is not None:
        _need(H_final, "H_final", (b, H, P, N), torch.float32, dev)
    dims = Dims(b, L, H, G, N, P, chunk)
    need = int(lib().dart_ssd_fwd_workspace_bytes(ctypes.byref(dims), _code(dt)))
    workspace = _workspace(need, dev, workspace)
    _check(lib().dart_ssd_fwd(ctypes.byref(dims), _code(dt), _ptr(X), _ptr(B), _ptr(C), _ptr(A), _ptr(H0),
                              _ptr(Y), _ptr(dH), _ptr(H_final), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(X)))
    return Y, dH, H_final

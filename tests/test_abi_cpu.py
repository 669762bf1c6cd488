"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/dart.h, and rejects bad arguments on the host before any
HIP call (so no error path below touches a device)."""
import ctypes
import os
import re
import subprocess
import threading

import pytest

from state_memory_attention_amd import dart as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dart.h")

pytestmark = pytest.mark.skipif(not os.path.exists(D.LIB_PATH), reason="libdart.so not built")

GiB = 1 << 30
# fake, 16-byte aligned, widely spaced device addresses: never dereferenced,
# because every call below fails validation before launching anything
ADDR = [ctypes.c_void_p((k + 1) << 40) for k in range(16)]


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(dart_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = D.lib()
    names = declared_functions()
    assert set(names) == set(D.ENTRY_POINTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", D.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (dart_\w+)", out))
    assert set(names) <= exported


def test_version_and_status_strings():
    assert D.abi_version() == 1
    lib = D.lib()
    for code, name in D.STATUS.items():
        assert lib.dart_status_string(code).decode() == name
    assert lib.dart_status_string(-99).decode() == "DART_ERR_UNKNOWN"


def dims(b=2, L=512, H=4, G=2, N=128, P=64, S=256):
    return D.Dims(b, L, H, G, N, P, S)


def cs(d, dtype=1, X=ADDR[0], B=ADDR[1], A=ADDR[2], dH=ADDR[3]):
    return D.lib().dart_chunk_states(None if d is None else ctypes.byref(d), dtype, X, B, A, dH, None)


def fwd(d, dtype=1, ptrs=None, gpc=1, R=None, lse=None, out=None):
    p = list(ADDR[:7]) if ptrs is None else ptrs
    if out is not None:
        p[6] = out
    return D.lib().dart_sma_fwd(ctypes.byref(d), dtype, p[0], p[1], p[2], p[3], p[4], p[5], gpc,
                                p[6], R, lse, None)


def dec(d, max_chunks=8, ws=ADDR[10], ws_bytes=GiB, dtype=1, n_chunks=None, cache=ADDR[3]):
    return D.lib().dart_sma_decode(ctypes.byref(d), dtype, max_chunks, ADDR[0], ADDR[1], ADDR[2],
                                   cache, n_chunks, ADDR[4], ADDR[5], 1, ADDR[6], None, None,
                                   ws, ws_bytes, None)


def last():
    return D.lib().dart_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("batch", -1, -2), ("seqlen", -5, -2), ("nheads", 0, -2), ("ngroups", 0, -2), ("ngroups", 3, -2),
    ("d_state", 0, -2), ("d_head", -1, -2), ("chunk", 0, -2), ("d_state", 257, -3), ("d_head", 512, -3),
    ("seqlen", 1 << 31, -2),
])
def test_bad_dims(field, value, code):
    d = dims()
    setattr(d, field, value)
    assert cs(d) == code and last() != ""
    assert fwd(d) == code and last() != ""


def test_null_dims_and_bad_dtype():
    assert cs(None) == -1 and "dims" in last()
    assert cs(dims(), dtype=2) == -3
    assert fwd(dims(), dtype=7) == -3


def test_null_and_misaligned_pointers():
    assert cs(dims(), X=None) == -1 and "X" in last()
    assert cs(dims(), A=None) == -1 and "A" in last()
    assert cs(dims(), dH=ctypes.c_void_p((5 << 40) + 8)) == -6 and "dH" in last()
    p = list(ADDR[:7])
    p[5] = None
    assert fwd(dims(), ptrs=p) == -1 and "gate" in last()
    assert fwd(dims(), R=ctypes.c_void_p((9 << 40) + 4)) == -6 and "R" in last()


def test_aliasing_rules():
    d = dims()
    # out overlapping Q is rejected; out == Y_ssm (index 4) is the allowed alias
    assert fwd(d, out=ctypes.c_void_p(ADDR[0].value + 64)) == -2 and "overlaps" in last()
    assert fwd(d, out=ctypes.c_void_p(ADDR[4].value + 64)) == -2
    assert cs(d, dH=ctypes.c_void_p(ADDR[0].value)) == -2


def test_empty_calls_launch_nothing():
    # b = 0 or L = 0 return OK before touching pointers or the device
    assert cs(dims(b=0), X=None) == 0
    assert fwd(dims(L=0)) == 0
    assert dec(dims(b=0)) == 0


def test_decode_validation():
    d = dims()
    assert dec(d, max_chunks=-1) == -2
    need = D.lib().dart_sma_decode_workspace_bytes(ctypes.byref(d), 8)
    assert need > 0
    assert dec(d, ws=None) == -4 and "workspace" in last()
    assert dec(d, ws_bytes=need - 1) == -4
    assert dec(d, cache=None) == -1 and "cache" in last()
    assert dec(d, n_chunks=ctypes.c_void_p((11 << 40) + 2)) == -6


def test_decode_scalar_gate_alignment():
    # a scalar gate ([b][H]) needs only its element's alignment: a 2-byte
    # offset passes the gate check and the call stops at the NULL output
    # (nothing launches); a 1-byte offset, or a per-channel gate off a
    # 16-byte boundary, is refused
    d = dims()

    def call(gate, gpc, out=None):
        return D.lib().dart_sma_decode(ctypes.byref(d), 1, 8, ADDR[0], ADDR[1], ADDR[2], ADDR[3], None, ADDR[4],
                                       gate, gpc, out, None, None, ADDR[10], GiB, None)

    assert call(ctypes.c_void_p(ADDR[5].value + 2), 0) == -1 and "out" in last()
    assert call(ctypes.c_void_p(ADDR[5].value + 1), 0) == -6 and "gate" in last()
    assert call(ctypes.c_void_p(ADDR[5].value + 2), 1) == -6 and "gate" in last()
    assert call(None, 0, ADDR[6]) == -1 and "gate" in last()


def dec_noalloc(d, max_chunks=8, dtype=1, cache=ADDR[3], out=ADDR[6]):
    return D.lib().dart_sma_decode_noalloc(ctypes.byref(d), dtype, max_chunks, ADDR[0], ADDR[1], ADDR[2],
                                           cache, None, ADDR[4], ADDR[5], 1, out, None, None, None)


def test_decode_noalloc_validation():
    """Every failing case returns before any HIP call: bad arguments, and
    split partials larger than the library's scratch."""
    d = dims()
    assert dec_noalloc(d, max_chunks=-1) == -2
    assert dec_noalloc(d, cache=None) == -1 and "cache" in last()
    assert dec_noalloc(d, out=ctypes.c_void_p((12 << 40) + 8)) == -6 and "out" in last()
    assert dec_noalloc(dims(b=0)) == 0
    # b * H = 32768 rows and heads need 32768 * 66 * 4 bytes of partials: over the 4 MiB scratch
    big = dims(b=1024, H=32, G=32)
    need = D.lib().dart_sma_decode_workspace_bytes(ctypes.byref(big), 256)
    assert need > 4 << 20
    assert dec_noalloc(big, max_chunks=256) == -4 and "scratch" in last()
    # the largest problem that fits is checked against the same limit the header states
    text = open(HEADER).read()
    assert "DART_DECODE_SCRATCH_BYTES ((size_t)4 << 20)" in text


def test_decode_workspace_size_function():
    f = D.lib().dart_sma_decode_workspace_bytes
    d = dims(b=64, H=24)
    assert f(None, 256) == 0 and f(ctypes.byref(d), -1) == 0
    sizes = [f(ctypes.byref(d), m) for m in (0, 1, 16, 256)]
    assert all(s >= 64 * 24 * (64 + 2) * 4 for s in sizes)
    assert sizes == sorted(sizes)


def test_error_text_is_thread_local():
    assert cs(None) == -1 and last() != ""
    seen = []
    t = threading.Thread(target=lambda: seen.append(last()))
    t.start()
    t.join()
    assert seen == [""]
    # a successful (empty) call clears this thread's message
    assert cs(dims(b=0)) == 0 and last() == ""


def test_path_selection_round_trips():
    prev = D.set_path(D.DART_PATH_GENERAL)
    assert D.set_path(D.DART_PATH_AUTO) == D.DART_PATH_GENERAL
    D.set_path(prev)


def bwd(d, dtype=1, ws=ADDR[15], ws_bytes=1 << 40, dgate=None, over=None):
    p = list(ADDR[:13])
    for k, v in (over or {}).items():
        p[k] = v
    # Q C E dH gate R lse dout | dQ dC dE d_dH
    return D.lib().dart_sma_bwd(ctypes.byref(d), dtype, p[0], p[1], p[2], p[3], p[4], 1, p[5], p[6],
                                p[7], p[8], p[9], p[10], p[11], dgate, ws, ws_bytes, None)


def csb(d, dtype=1, ws=ADDR[15], ws_bytes=1 << 40, over=None):
    p = list(ADDR[:7])
    for k, v in (over or {}).items():
        p[k] = v
    return D.lib().dart_chunk_states_bwd(ctypes.byref(d), dtype, p[0], p[1], p[2], p[3], p[4], p[5],
                                         p[6], ws, ws_bytes, None)


def test_backward_validation():
    d = dims()
    need = D.lib().dart_sma_bwd_workspace_bytes(ctypes.byref(d))
    b, L, H, G, N, P, S = 2, 512, 4, 2, 128, 64, 256
    M = 2
    # the larger of the two layouts: (p, dl) per (chunk, token) and head, plus
    # per-head partials when heads are grouped; the MFMA path also keeps dR
    # in bfloat16 and the chunk memories transposed (256-byte aligned sections)
    r256 = lambda n: -(-n // 256) * 256
    general = 4 * (2 * b * H * M * L + b * L * H * (2 * N + P))
    mfma = (r256(4 * 2 * b * H * M * L) + r256(2 * b * L * H * P) + r256(4 * b * L * H * (2 * N + P))
            + r256(2 * b * H * M * P * N))
    assert need == max(general, mfma)
    assert bwd(d, ws=None) == -4 and "workspace" in last()
    assert bwd(d, ws_bytes=need - 1) == -4
    assert bwd(d, over={0: None}) == -1 and "Q" in last()
    assert bwd(d, over={5: None}) == -1 and "R" in last()
    assert bwd(d, over={11: None}) == -1 and "d_dH" in last()
    assert bwd(d, over={8: ctypes.c_void_p(ADDR[8].value + 4)}) == -6
    assert bwd(d, dgate=ctypes.c_void_p((14 << 40) + 8)) == -6
    # a gradient overlapping an input
    assert bwd(d, over={8: ctypes.c_void_p(ADDR[0].value)}) == -2 and "overlaps" in last()
    assert bwd(dims(L=0)) == 0 and bwd(dims(b=0)) == 0
    assert bwd(d, dtype=3) == -3
    # ungrouped heads need no per-head partials
    d1 = dims(G=4)
    assert D.lib().dart_sma_bwd_workspace_bytes(ctypes.byref(d1)) == max(
        4 * 2 * b * H * M * L, r256(4 * 2 * b * H * M * L) + r256(2 * b * L * H * P) + r256(2 * b * H * M * P * N))
    assert D.lib().dart_sma_bwd_workspace_bytes(None) == 0


def test_chunk_states_backward_validation():
    d = dims()
    need = D.lib().dart_chunk_states_bwd_workspace_bytes(ctypes.byref(d))
    assert need == 4 * (2 * 2 * 4 * 512 + 2 * 512 * 4 * 128)
    assert csb(d, ws=None) == -4
    assert csb(d, ws_bytes=need - 1) == -4
    assert csb(d, over={3: None}) == -1 and "d_dH" in last()
    assert csb(d, over={6: ctypes.c_void_p(ADDR[6].value + 2)}) == -6
    assert csb(d, over={4: ctypes.c_void_p(ADDR[1].value)}) == -2
    assert csb(dims(b=0)) == 0


def upd(d, max_chunks=4, dtype=1, over=None):
    p = [ADDR[0], ADDR[1], ADDR[2], ADDR[3], ADDR[4], ADDR[5], ADDR[6]]  # x B a state pos cache n
    for k, v in (over or {}).items():
        p[k] = v
    return D.lib().dart_decode_state_update(ctypes.byref(d), dtype, max_chunks, *p, None)


def test_decode_update_validation():
    d = dims()
    assert upd(d, over={3: None}) == -1 and "state" in last()
    assert upd(d, over={4: None}) == -1 and "pos" in last()
    assert upd(d, over={5: None}) == -1 and "cache" in last()
    assert upd(d, over={6: ctypes.c_void_p(ADDR[6].value + 2)}) == -6
    assert upd(d, over={3: ctypes.c_void_p(ADDR[3].value + 4)}) == -6 and "state" in last()
    assert upd(d, over={2: ctypes.c_void_p(ADDR[2].value + 1)}) == -6 and "a" in last()
    assert upd(d, over={0: ctypes.c_void_p(ADDR[0].value + 1)}) == -6 and "x" in last()
    assert upd(d, over={3: ctypes.c_void_p(ADDR[0].value)}) == -2 and "overlaps" in last()
    assert upd(d, max_chunks=-1) == -2
    bad = dims(S=0)
    assert upd(bad) == -2
    assert upd(dims(b=0)) == 0


def cs_rms(d, dtype=1, eps=1e-6, over=None):
    p = [ADDR[0], ADDR[1], ADDR[2], None, None, ADDR[3], ADDR[4], ADDR[5]]  # X B A wq we dH r dHs
    for k, v in (over or {}).items():
        p[k] = v
    return D.lib().dart_chunk_states_rms(ctypes.byref(d), dtype, p[0], p[1], p[2], eps, p[3], p[4],
                                         p[5], p[6], p[7], None)


def fwd_rms(d, dtype=1, eps=1e-6, over=None):
    p = list(ADDR[:8])  # Q C E dH dHs Y gate out
    for k, v in (over or {}).items():
        p[k] = v
    return D.lib().dart_sma_fwd_rms(ctypes.byref(d), dtype, p[0], p[1], p[2], p[3], p[4], p[5], p[6], 1,
                                    eps, p[7], None, None, None)


def dec_rms(d, max_chunks=8, eps=1e-6, over=None, ws_bytes=1 << 40):
    p = list(ADDR[:10])  # q c e cache r_cache y gate out ws wq
    for k, v in (over or {}).items():
        p[k] = v
    return D.lib().dart_sma_decode_rms(ctypes.byref(d), 1, max_chunks, p[0], p[1], p[2], p[3], p[4], None,
                                       p[5], p[6], 1, eps, p[9], None, p[7], None, None, p[8], ws_bytes,
                                       None)


def upd_rms(d, max_chunks=4, eps=1e-6, over=None):
    p = [ADDR[0], ADDR[1], ADDR[2], ADDR[3], ADDR[4], ADDR[5], ADDR[6], None]  # x B a state pos cache r n
    for k, v in (over or {}).items():
        p[k] = v
    return D.lib().dart_decode_state_update_rms(ctypes.byref(d), 1, max_chunks, eps, *p, None)


def test_rms_validation():
    d = dims()
    # chunk states with r and the score memory
    assert cs_rms(d, over={5: None}) == -1 and "dH" in last()
    assert cs_rms(d, eps=-1.0) == -2 and "eps" in last()
    assert cs_rms(d, eps=float("nan")) == -2
    assert cs_rms(d, over={3: ctypes.c_void_p(ADDR[9].value + 2)}) == -6 and "w_q" in last()
    assert cs_rms(d, over={6: ctypes.c_void_p(ADDR[4].value + 4)}) == -6 and "r" in last()
    assert cs_rms(d, over={7: ctypes.c_void_p(ADDR[0].value)}) == -2 and "overlaps" in last()
    assert cs_rms(dims(b=0)) == 0
    # forward: the score memory is required
    assert fwd_rms(d, over={4: None}) == -1 and "dH_score" in last()
    assert fwd_rms(d, over={4: ctypes.c_void_p(ADDR[4].value + 8)}) == -6
    assert fwd_rms(d, over={7: ctypes.c_void_p(ADDR[4].value)}) == -2 and "overlaps" in last()
    assert fwd_rms(d, eps=float("inf")) == -2
    assert fwd_rms(dims(L=0)) == 0
    # decode: r_cache required when chunks are cached
    assert dec_rms(d, over={4: None}) == -1 and "r_cache" in last()
    assert dec_rms(d, over={9: ctypes.c_void_p(ADDR[9].value + 1)}) == -6 and "w_q" in last()
    assert dec_rms(d, ws_bytes=0) == -4
    assert dec_rms(d, over={7: ctypes.c_void_p(ADDR[4].value)}) == -2 and "overlaps" in last()
    # update: r_cache required, 16-byte aligned
    assert upd_rms(d, over={6: None}) == -1 and "r_cache" in last()
    assert upd_rms(d, over={6: ctypes.c_void_p(ADDR[6].value + 4)}) == -6
    assert upd_rms(d, eps=-0.5) == -2
    assert upd_rms(dims(b=0)) == 0


MORE = [ctypes.c_void_p((k + 1) << 40) for k in range(24)]


def bwd_rms(d, dtype=1, eps=1e-6, ws=MORE[23], ws_bytes=1 << 40, over=None):
    p = list(MORE[:20])
    p[12] = p[13] = p[14] = None  # w_q, w_e unweighted; dgate skipped
    for k, v in (over or {}).items():
        p[k] = v
    # Q C E dH dHs gate | R lse dout dQ dC dE | w_q w_e dgate | d_dH dw_q dw_e
    return D.lib().dart_sma_bwd_rms(ctypes.byref(d), dtype, p[0], p[1], p[2], p[3], p[4], p[5], 1, eps,
                                    p[12], p[13], p[6], p[7], p[8], p[9], p[10], p[11], p[15], p[14],
                                    p[16], p[17], ws, ws_bytes, None)


def test_rms_backward_validation():
    d = dims()
    b, L, H, G, N, P, S = 2, 512, 4, 2, 128, 64, 256
    M = 2
    up = lambda n: -(-n // 64) * 64
    split = min(1024, max(1, -(-(b * L * G) // 64)))
    want = 4 * (up(2 * b * H * M * L) + up(b * L * H * N) + up(b * L * H * P) + up(b * L * H * N)
                + up(2 * b * L * G) + up(b * H * M * P * N) + up(b * L * G * N) + up(b * L * G * P)
                + up(split * (N + P)))
    # the matrix-core layout: the plain backward's (with dH transposed), the
    # score memory transposed, RMSNorm factors, dT, weight-gradient rows and
    # column-sum partials (256-byte aligned sections)
    r256 = lambda n: -(-n // 256) * 256

    def mfma_rms(G):
        part = r256(4 * b * L * H * (2 * N + P)) if G != H else 0
        plain = r256(4 * 2 * b * H * M * L) + r256(2 * b * L * H * P) + part + r256(2 * b * H * M * P * N)
        msplit = min(1024, max(1, -(-(b * H * M) // 64)))
        return (r256(plain) + r256(2 * b * H * M * P * N) + r256(4 * 2 * b * L * G) + r256(4 * b * H * M * P * N)
                + r256(4 * b * H * M * N) + r256(4 * b * H * M * P) + r256(4 * msplit * (N + P)))
    need = D.lib().dart_sma_bwd_rms_workspace_bytes(ctypes.byref(d))
    assert need == max(want, mfma_rms(G))
    # ungrouped heads: no per-head dC partials
    G1 = 4
    split1 = min(1024, max(1, -(-(b * L * G1) // 64)))
    want1 = 4 * (up(2 * b * H * M * L) + up(b * L * H * N) + up(b * L * H * P) + up(2 * b * L * G1)
                 + up(b * H * M * P * N) + up(b * L * G1 * N) + up(b * L * G1 * P) + up(split1 * (N + P)))
    assert D.lib().dart_sma_bwd_rms_workspace_bytes(ctypes.byref(dims(G=G1))) == max(want1, mfma_rms(G1))
    assert bwd_rms(d, ws=None) == -4 and "workspace" in last()
    assert bwd_rms(d, ws_bytes=need - 1) == -4
    assert bwd_rms(d, over={4: None}) == -1 and "dH_score" in last()
    assert bwd_rms(d, over={15: None}) == -1 and "d_dH" in last()
    assert bwd_rms(d, eps=-1.0) == -2 and "eps" in last()
    assert bwd_rms(d, eps=float("nan")) == -2
    assert bwd_rms(d, over={12: ctypes.c_void_p(MORE[12].value + 2)}) == -6 and "w_q" in last()
    assert bwd_rms(d, over={16: ctypes.c_void_p(MORE[16].value + 2)}) == -6 and "dw_q" in last()
    assert bwd_rms(d, over={9: ctypes.c_void_p(MORE[9].value + 4)}) == -6 and "dQ" in last()
    # a gradient overlapping an input, and a weight gradient overlapping a weight
    assert bwd_rms(d, over={9: ctypes.c_void_p(MORE[4].value)}) == -2 and "overlaps" in last()
    assert bwd_rms(d, over={12: MORE[12], 16: MORE[12]}) == -2 and "overlaps" in last()
    assert bwd_rms(d, dtype=3) == -3
    assert bwd_rms(dims(L=0)) == 0 and bwd_rms(dims(b=0)) == 0
    assert D.lib().dart_sma_bwd_rms_workspace_bytes(None) == 0
    # 2^31 chunk memories (one block each in the chain kernel): refused on the
    # host (addresses spaced far enough apart for these buffer sizes)
    far = [ctypes.c_void_p((k + 1) << 55) for k in range(24)]
    big = D.Dims(1, 1 << 15, 1 << 16, 1 << 16, 128, 64, 1)
    p = list(far[:20])
    p[12] = p[13] = p[14] = None
    st = D.lib().dart_sma_bwd_rms(ctypes.byref(big), 1, p[0], p[1], p[2], p[3], p[4], p[5], 1, 1e-6, p[12], p[13],
                                  p[6], p[7], p[8], p[9], p[10], p[11], p[15], p[14], p[16], p[17], far[23],
                                  1 << 62, None)
    assert st == -2 and "too large" in last()


def ssd(d, dtype=1, over=None, ws_bytes=1 << 40):
    p = list(ADDR[:10])  # X B C A H0 Y dH Hfin ws
    p[4] = None
    p[7] = None
    for k, v in (over or {}).items():
        p[k] = v
    return D.lib().dart_ssd_fwd(ctypes.byref(d), dtype, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8],
                                ws_bytes, None)


def test_ssd_validation():
    d = dims()
    need = D.lib().dart_ssd_fwd_workspace_bytes(ctypes.byref(d), 1)
    b, L, H, N, P, M = 2, 512, 4, 128, 64, 2
    assert need == -(-(4 * b * H * M) // 256) * 256 + 2 * b * H * M * P * N
    assert D.lib().dart_ssd_fwd_workspace_bytes(ctypes.byref(d), 0) == -(-(4 * b * H * M) // 256) * 256 + 4 * b * H * M * P * N
    assert ssd(d, ws_bytes=need - 1) == -4
    assert ssd(d, over={8: None}) == -4
    assert ssd(d, over={2: None}) == -1 and "C" in last()
    assert ssd(d, over={4: ctypes.c_void_p(ADDR[4].value + 4)}) == -6 and "H0" in last()
    assert ssd(d, over={5: ctypes.c_void_p(ADDR[0].value)}) == -2 and "overlaps" in last()
    assert ssd(dims(L=0)) == 0
    assert ssd(d, dtype=7) == -3

def test_c_program_links_the_in_tree_library():
    """The build step's plain C consumer of include/dart.h
    (tests/c_abi/dart_c_smoke.c) resolves libdart.so to the package's copy
    and needs no Python or torch library; it runs on the GPU in
    tests/test_gpu_c_abi.py."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    binp = os.path.join(root, "tests", "c_abi", "dart_c_smoke.bin")
    if not os.path.exists(binp):
        pytest.skip("the C program is built by state_memory_attention_amd.build (not run here)")
    out = subprocess.run(["ldd", binp], capture_output=True, text=True, timeout=60).stdout
    libs = {line.split()[0]: line for line in out.splitlines() if "=>" in line}
    assert "libdart.so" in libs, out
    assert os.path.realpath(libs["libdart.so"].split("=>")[1].split()[0]) == \
        os.path.realpath(os.path.join(root, "state_memory_attention_amd", "libdart.so"))
    assert "not found" not in out, out
    assert not any("python" in k or "torch" in k for k in libs), out

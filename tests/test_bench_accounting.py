"""The benchmark's work and byte counts (the denominators of every reported
fraction), checked on the host against brute force and the paper's
complexity (§4 "Training Complexity", Eq. 12-13)."""
import itertools

import pytest

import bench

LONG = dict(batch=2, nheads=24, ngroups=24, seqlen=16384, chunk=256, d_state=128, d_head=64)


def brute_pairs(b, H, L, S):
    # token t sees the chunks before its own: chunk(t) = t // S of them
    return b * H * sum(t // S for t in range(L))


@pytest.mark.parametrize("L,S", list(itertools.product([1, 2, 127, 128, 300, 1000, 1024], [1, 3, 64, 100, 256, 2048])))
def test_pairs_equal_brute_force(L, S):
    assert bench.fwd_pairs(2, 3, L, S) == brute_pairs(2, 3, L, S)


def test_pairs_closed_form_and_eq12_scaling():
    # L = M S: S * (0 + 1 + ... + M-1) = L (L - S) / (2 S) per head, i.e. O(L^2 / S)
    for L, S in ((16384, 256), (65536, 256), (4096, 64), (1024, 32)):
        assert bench.fwd_pairs(1, 1, L, S) == L * (L - S) // (2 * S)
    assert bench.fwd_pairs(2, 24, 16384, 256) == 24772608


def test_flops_per_launch_of_the_long_workload():
    f_sma, f_cs = bench.fwd_flops(LONG)
    assert f_sma == 4 * 128 * 64 * 24772608 == 811748818944
    assert f_cs == 2 * 128 * 64 * 2 * 24 * 16384


def test_ratio_to_token_attention_is_n_over_s():
    # Eq. 13: SMA pairs cost 4NP against 4P for a causal token pair (QK^T and
    # PV), over L^2/(2S) chunk pairs against L^2/2 token pairs
    N, P, S, L = 128, 64, 256, 1 << 20
    sma = 4 * N * P * bench.fwd_pairs(1, 1, L, S)
    attn = 4 * P * L * (L + 1) // 2
    assert sma / attn == pytest.approx(N / S, rel=2 * S / L)


@pytest.mark.parametrize("S", [32, 64, 128, 256, 512, 1000])
def test_tile_products_cover_and_mask(S):
    L = 16384
    pairs, computed = bench.fwd_pairs(1, 1, L, S), bench.tile_pairs(1, 1, L, S)
    if S % 128 == 0:
        assert computed == pairs  # a 128-token tile never spans two chunks
    else:
        assert computed > pairs
    if S in (32, 64):
        # a tile spans 128 / S chunks; the tokens of its k-th chunk (k = 0, 1,
        # ...) compute 128/S - 1 - k products they cannot see
        per_tile = S * sum(range(128 // S))
        assert computed - pairs == (L // 128) * per_tile


def test_tile_products_ragged_tail():
    # L = 300, S = 64: tiles [0, 128) and [128, 256) as above (64 masked each),
    # the tail tile [256, 300) pads to 128 slots, all against chunks 0..3
    assert bench.tile_pairs(1, 1, 300, 64) == 128 * 1 + 128 * 3 + 128 * 4
    assert bench.fwd_pairs(1, 1, 300, 64) == 64 * (0 + 1 + 2 + 3) + 44 * 4


def test_path_bytes_of_the_long_workload():
    tok_h = 2 * 16384 * 24 * 64 * 2        # X, E, Y, gate, out
    tok_g = 2 * 16384 * 24 * 128 * 2       # B, Q, C
    a = 2 * 16384 * 24 * 4                 # float32 decays
    mem = 2 * 24 * 64 * 128 * 64 * 2       # chunk memories, written then read
    chunk_states = tok_h + tok_g + a + mem
    forward = 2 * tok_g + tok_h + mem + 3 * tok_h
    assert bench.path_bytes(LONG) == chunk_states + forward == 1211105280


def test_backward_flops_are_three_forward_products():
    # per pair: W and V recomputed (4NP), dQ and dC (4NP), the two d_dH terms (4NP)
    assert bench.bwd_flops(LONG) == 3 * bench.fwd_flops(LONG)[0] == 2435246456832


def test_ssd_bytes_of_the_long_workload():
    x = y = 2 * 16384 * 24 * 64 * 2
    b_in = c_in = 2 * 16384 * 24 * 128 * 2
    a = 2 * 16384 * 24 * 4
    mem = 2 * 24 * 64 * 64 * 128 * 2      # chunk memories out; entering states out and back in
    assert bench.ssd_bytes(LONG) == x + b_in + c_in + a + y + 3 * mem == 758120448

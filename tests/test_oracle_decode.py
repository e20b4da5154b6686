"""Pins of the decode / chunked-prefill oracle (oracle/decode.py), CPU only.

The decode oracle is a separate float64 numpy implementation; it is pinned to the C oracle's
forward (itself pinned in test_oracle.py) through the identity that defines the cached workload:
the new tokens' outputs are the last rows of full causal attention over the whole sequence.  Plus
brute force, closed forms, window edges, ragged lengths, and planted mistakes in a copy of it.
"""
import math
import os

import numpy as np
import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "decode.py")


def seq_case(L, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, L, Hq, D))
    k = rng.standard_normal((1, L, Hkv, D))
    v = rng.standard_normal((1, L, Hkv, D))
    return q, k, v


def decode_from_full(fn, q, k, v, lens, Tq, base, window=0):
    """Run decode_fwd (fn) for the last Tq tokens of each sequence of a batch of full sequences."""
    qn = np.stack([q[b, lens[b]:lens[b] + Tq] for b in range(q.shape[0])])
    return fn(qn, [k[b] for b in range(k.shape[0])], [v[b] for b in range(v.shape[0])], lens, base, window)


@pytest.mark.parametrize("L,Tq,Hq,Hkv,D,base,window", [
    (1, 1, 2, 1, 8, 1e4, 0), (37, 1, 4, 2, 16, 1e4, 0), (50, 7, 6, 2, 8, 1e4, 0),
    (64, 64, 4, 4, 8, 1e4, 0), (90, 5, 8, 2, 32, 5e5, 0), (40, 3, 4, 2, 8, 0.0, 0),
    (80, 6, 4, 1, 16, 1e4, 9), (33, 33, 2, 1, 8, 1e4, 5), (20, 2, 3, 1, 6, 10.0, 1)])
def test_decode_rows_equal_full_causal_rows(L, Tq, Hq, Hkv, D, base, window):
    q, k, v = seq_case(L, Hq, Hkv, D, seed=L * 7 + Tq)
    lens = [L - Tq]
    o, lse = decode_from_full(oracle.decode_fwd, q, k, v, lens, Tq, base, window)
    fo, flse = oracle.fwd(q, k, v, base, window=window)
    assert np.max(np.abs(o[0] - fo[0, L - Tq:])) < 1e-12 * max(1.0, np.max(np.abs(fo)))
    assert np.max(np.abs(lse[0] - flse[0, :, L - Tq:])) < 1e-12


@pytest.mark.parametrize("window", [0, 6])
def test_decode_qk_norm_rows_equal_full_causal_rows(window):
    L, Tq, Hq, Hkv, D = 41, 5, 6, 2, 16
    q, k, v = seq_case(L, Hq, Hkv, D, seed=77)
    qkn = (1.2, 1e-6)
    qn = q[:, L - Tq:]
    o, lse = oracle.decode_fwd(qn, [k[0]], [v[0]], [L - Tq], 1e4, window, qk_norm=qkn)
    fo, flse = oracle.fwd(q, k, v, 1e4, window=window, qk_norm=qkn)
    np.testing.assert_allclose(o[0], fo[0, L - Tq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], flse[0, :, L - Tq:], rtol=0, atol=1e-12)


def test_decode_ragged_batch_each_row_matches_its_own_sequence():
    Tq, Hq, Hkv, D = 3, 4, 2, 16
    lens = [0, 11, 29]
    seqs = [seq_case(n + Tq, Hq, Hkv, D, seed=40 + n) for n in lens]
    qn = np.concatenate([s[0][:, n:n + Tq] for s, n in zip(seqs, lens)])
    o, lse = oracle.decode_fwd(qn, [s[1][0] for s in seqs], [s[2][0] for s in seqs], lens, 1e4)
    for b, (s, n) in enumerate(zip(seqs, lens)):
        fo, flse = oracle.fwd(s[0], s[1], s[2], 1e4)
        np.testing.assert_allclose(o[b], fo[0, n:n + Tq], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], flse[0, :, n:n + Tq], rtol=0, atol=1e-12)


def test_decode_matches_brute_force_tiny():
    q, k, v = seq_case(6, 4, 2, 4, seed=3)
    o, lse = decode_from_full(oracle.decode_fwd, q, k, v, [4], 2, 3.0)
    bo, blse = pins.brute_fwd(q, k, v, 3.0)
    np.testing.assert_allclose(o[0], bo[0, 4:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], blse[0, :, 4:], rtol=0, atol=1e-13)


def test_decode_keys_past_the_new_tokens_are_ignored():
    """The cache may hold more positions than lens + Tq (stale or future tokens): invisible."""
    q, k, v = seq_case(30, 4, 2, 8, seed=5)
    o1, l1 = decode_from_full(oracle.decode_fwd, q[:, :20], k[:, :20], v[:, :20], [17], 3, 1e4)
    k2, v2 = k.copy(), v.copy()
    k2[:, 20:] = 1e3
    v2[:, 20:] = np.nan
    o2, l2 = decode_from_full(oracle.decode_fwd, q, k2, v2, [17], 3, 1e4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_decode_first_token_sees_only_itself():
    q, k, v = seq_case(1, 4, 2, 8, seed=6)
    o, lse = oracle.decode_fwd(q, [k[0]], [v[0]], [0], 1e4)
    np.testing.assert_array_equal(o[0, 0], v[0, 0].repeat(2, axis=0))
    ref = np.sum(q[0, 0] * k[0, 0].repeat(2, axis=0), axis=-1) / math.sqrt(8)   # R_0 = identity
    np.testing.assert_allclose(lse[0, :, 0], ref, rtol=0, atol=1e-14)


def test_decode_rotation_uses_absolute_positions():
    """Shifting every position by the same offset leaves the scores unchanged (relative RoPE):
    a query at p against keys at p - d equals the same pattern at positions 0-based, D = 2."""
    rng = np.random.default_rng(8)
    D, L = 2, 12
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, 1, 1, D))
    # query at position 11 against all 12 keys, versus keys 5..11 moved to positions 0..6 and the
    # query to position 6 with a window of 7: identical visible (relative) pattern
    o1, l1 = oracle.decode_fwd(q, [k], [v], [11], 1.0, window=7)
    o2, l2 = oracle.decode_fwd(q, [k[5:]], [v[5:]], [6], 1.0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_rope_rows_matches_c_oracle_rotation():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 50, 3, 16))
    np.testing.assert_allclose(oracle.rope_rows(x[0], np.arange(50), 5e5)[None], oracle.rope(x, 5e5), rtol=0,
                               atol=1e-13)
    np.testing.assert_allclose(oracle.rope_rows(x[0], np.arange(50), 5e5, half_split=True)[None],
                               oracle.rope(x, 5e5, half_split=True), rtol=0, atol=1e-13)


@pytest.mark.parametrize("window,qkn", [(0, None), (6, None), (0, (1.2, 1e-6))])
def test_half_split_decode_rows_equal_the_c_oracles_half_split_rows(window, qkn):
    """The half-split pairing (i, i + D/2) in decode against the C oracle's full causal half-split
    attention (pinned in test_oracle)."""
    L, Tq, Hq, Hkv, D = 45, 4, 6, 2, 16
    q, k, v = seq_case(L, Hq, Hkv, D, seed=91)
    o, lse = oracle.decode_fwd(q[:, L - Tq:], [k[0]], [v[0]], [L - Tq], 1e4, window, qk_norm=qkn, half_split=True)
    fo, flse = oracle.fwd(q, k, v, 1e4, window=window, qk_norm=qkn, half_split=True)
    np.testing.assert_allclose(o[0], fo[0, L - Tq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], flse[0, :, L - Tq:], rtol=0, atol=1e-12)


# ---- planted mistakes in a copy of oracle/decode.py --------------------------------------------
MUTATIONS = {
    "query_position_not_offset": ("pos = int(lens[b]) + np.arange(Tq)", "pos = np.arange(Tq)"),
    "keys_rotated_by_query_positions": ("kr = rope_rows(k, np.arange(L), base, half_split)",
                                        "kr = rope_rows(k, L - 1 - np.arange(L), base, half_split)"),
    "half_split_halves_swapped": ("a, b = x[..., :D // 2], x[..., D // 2:]", "a, b = x[..., D // 2:], x[..., :D // 2]"),
    "window_off_by_one": ("(pos[:, None] - j[None, :]) < window", "(pos[:, None] - j[None, :]) <= window"),
    "causal_mask_dropped": ("vis = (j[None, :] <= pos[:, None])", "vis = (j[None, :] <= 0 * pos[:, None] + L - 1)"),
    "rotation_sign": ("y[..., 1::2] = a * s + b * c", "y[..., 1::2] = -a * s + b * c"),
    "gqa_mapping": ("g = h // G", "g = h % Hkv"),
    "lse_without_max": ("lse[b, h, :] = (m + np.log(z))[:, 0]", "lse[b, h, :] = np.log(z)[:, 0]"),
}


def mutant(name):
    text = open(SRC).read()
    old, new = MUTATIONS[name]
    assert text.count(old) == 1, name
    ns = {}
    exec(compile(text.replace(old, new), f"mutant_{name}", "exec"), ns)
    return ns["decode_fwd"]


def decode_battery(fn):
    failed = 0
    for L, Tq, Hq, Hkv, D, base, window in [(50, 7, 6, 2, 8, 1e4, 0), (80, 6, 4, 1, 16, 1e4, 9)]:
        q, k, v = seq_case(L, Hq, Hkv, D, seed=L * 7 + Tq)
        o, lse = decode_from_full(fn, q, k, v, [L - Tq], Tq, base, window)
        fo, flse = oracle.fwd(q, k, v, base, window=window)
        if not (np.max(np.abs(o[0] - fo[0, L - Tq:])) < 1e-10 and np.max(np.abs(lse[0] - flse[0, :, L - Tq:])) < 1e-10):
            failed += 1
    # the half-split pairing against the C oracle's
    q, k, v = seq_case(44, 4, 2, 16, seed=44)
    o, lse = fn(q[:, 40:], [k[0]], [v[0]], [40], 1e4, 0, half_split=True)
    fo, flse = oracle.fwd(q, k, v, 1e4, half_split=True)
    if not (np.max(np.abs(o[0] - fo[0, 40:])) < 1e-10 and np.max(np.abs(lse[0] - flse[0, :, 40:])) < 1e-10):
        failed += 1
    return failed


def test_unmutated_decode_passes_battery():
    text = open(SRC).read()
    ns = {}
    exec(compile(text, "copy", "exec"), ns)
    assert decode_battery(ns["decode_fwd"]) == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_decode_mistake_is_caught(name):
    assert decode_battery(mutant(name)) > 0, name

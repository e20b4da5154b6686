"""Pins of the QKV-projection oracle (oracle/qkv.py), CPU only: brute-force sums, the C oracle's
rotation, and composition with the attention oracle (projecting then attending with RoPE off must
equal attending to the raw projections with RoPE on), plus planted mistakes in a copy of it."""
import os

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "qkv.py")


def case(B, T, C, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal(((Hq + 2 * Hkv) * D, C)) / np.sqrt(C)
    return x, w


def test_brute_force_sums_without_rope():
    B, T, C, Hq, Hkv, D = 1, 3, 5, 2, 1, 4
    x, w = case(B, T, C, Hq, Hkv, D, 1)
    q, k, v = oracle.qkv_rope_proj(x, w, Hq, Hkv, 0.0)
    for t in range(T):
        for n in range((Hq + 2 * Hkv) * D):
            s = 0.0
            for c in range(C):
                s += x[0, t, c] * w[n, c]
            head, d = divmod(n, D)
            ref = q[0, t, head, d] if head < Hq else (k[0, t, head - Hq, d] if head < Hq + Hkv else
                                                       v[0, t, head - Hq - Hkv, d])
            assert abs(ref - s) < 1e-13


def test_sampled_positions_equal_the_full_sequence_rows():
    B, T, C, Hq, Hkv, D = 1, 50, 16, 2, 1, 8
    x, w = case(B, T, C, Hq, Hkv, D, 4)
    full = oracle.qkv_rope_proj(x, w, Hq, Hkv, 1e4)
    idx = np.array([0, 7, 31, 49])
    part = oracle.qkv_rope_proj(x[:, idx], w, Hq, Hkv, 1e4, positions=idx)
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a[:, idx], b)


def test_rotation_equals_the_c_oracle_rotation():
    B, T, C, Hq, Hkv, D = 2, 40, 32, 4, 2, 16
    x, w = case(B, T, C, Hq, Hkv, D, 2)
    q, k, v = oracle.qkv_rope_proj(x, w, Hq, Hkv, 5e5)
    q0, k0, v0 = oracle.qkv_rope_proj(x, w, Hq, Hkv, 0.0)
    np.testing.assert_allclose(q, oracle.rope(q0, 5e5), rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, oracle.rope(k0, 5e5), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(v, v0)
    qh, kh, vh = oracle.qkv_rope_proj(x, w, Hq, Hkv, 5e5, half_split=True)
    np.testing.assert_allclose(qh, oracle.rope(q0, 5e5, half_split=True), rtol=0, atol=1e-12)
    np.testing.assert_allclose(kh, oracle.rope(k0, 5e5, half_split=True), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(vh, v0)


@pytest.mark.parametrize("qkn", [None, (1.2, 1e-6)])
def test_projection_then_attention_without_rope_equals_attention_with_rope(qkn):
    B, T, C, Hq, Hkv, D = 1, 30, 24, 6, 2, 8
    x, w = case(B, T, C, Hq, Hkv, D, 3)
    q, k, v = oracle.qkv_rope_proj(x, w, Hq, Hkv, 1e4, qk_norm=qkn)
    q0, k0, _ = oracle.qkv_rope_proj(x, w, Hq, Hkv, 0.0)          # raw projections
    o1, l1 = oracle.fwd(q, k, v, 0.0)
    o2, l2 = oracle.fwd(q0, k0, v, 1e4, qk_norm=qkn)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


MUTATIONS = {
    "weight_read_as_c_by_n": ("y = x @ w.T", "y = x @ w.reshape(w.shape[1], w.shape[0])"),
    "k_before_q": ("q = y[..., :Hq * D].reshape(B, T, Hq, D)", "q = y[..., Hkv * D:(Hq + Hkv) * D].reshape(B, T, Hq, D)"),
    "positions_from_one": ("pos = np.arange(T) if positions is None", "pos = np.arange(1, T + 1) if positions is None"),
    "v_rotated": ("v = y[..., (Hq + Hkv) * D:].reshape(B, T, Hkv, D).copy()",
                  "v = np.stack([rope_rows(y[..., (Hq + Hkv) * D:].reshape(B, T, Hkv, D)[b], np.arange(T), base) for b in range(B)])"),
    "norm_after_k_only": ("q, k = qk_norm_rows(q, *qk_norm), qk_norm_rows(k, *qk_norm)", "k = qk_norm_rows(k, *qk_norm)"),
}


def mutant(name):
    text = open(SRC).read()
    old, new = MUTATIONS[name]
    assert text.count(old) == 1, name
    text = text.replace(old, new).replace("from .decode import", "from oracle.decode import")
    ns = {}
    exec(compile(text, f"mutant_{name}", "exec"), ns)
    return ns["qkv_rope_proj"]


def battery(fn):
    failed = 0
    B, T, C, Hq, Hkv, D = 1, 30, 24, 6, 2, 8
    x, w = case(B, T, C, Hq, Hkv, D, 3)
    for qkn in (None, (1.2, 1e-6)):
        q, k, v = fn(x, w, Hq, Hkv, 1e4, qk_norm=qkn)
        q0, k0, v0 = oracle.qkv_rope_proj(x, w, Hq, Hkv, 0.0)
        o1, _ = oracle.fwd(q, k, v, 0.0)
        o2, _ = oracle.fwd(q0, k0, v0, 1e4, qk_norm=qkn)
        if np.max(np.abs(o1 - o2)) > 1e-10:
            failed += 1
    # the rotation itself (a shift of every position is invisible to attention, not to q' and k')
    q, k, v = fn(x, w, Hq, Hkv, 5e5)
    q0, k0, v0 = oracle.qkv_rope_proj(x, w, Hq, Hkv, 0.0)
    if np.max(np.abs(q - oracle.rope(q0, 5e5))) > 1e-10 or np.max(np.abs(k - oracle.rope(k0, 5e5))) > 1e-10:
        failed += 1
    return failed


def test_unmutated_copy_passes_battery():
    text = open(SRC).read().replace("from .decode import", "from oracle.decode import")
    ns = {}
    exec(compile(text, "copy", "exec"), ns)
    assert battery(ns["qkv_rope_proj"]) == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    assert battery(mutant(name)) > 0

"""Pins for the double-precision oracle (CPU only).

Each test checks the oracle against something other than itself: a brute-force
evaluator written in a different form (complex rotations, no max-subtraction),
torch float64 autograd, central finite differences (the pages' own check, in
double precision: NanoEuler agentlenshq page, "验证与稳定性"; cnblogs page §2.1),
closed forms, invariants and a library routine (SDPA) for the no-RoPE case.
"""
import cmath
import math

import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import inputs


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def case(B, T, Hq, Hkv, D, seed, qk=1.0):
    q = rnd((B, T, Hq, D), seed) * qk
    k = rnd((B, T, Hkv, D), seed + 1) * qk
    v = rnd((B, T, Hkv, D), seed + 2)
    dO = rnd((B, T, Hq, D), seed + 3)
    return q, k, v, dO


def relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------------------
# Brute force: rotations as complex multiplications, softmax as exp/sum without the max
# shift, sums with math.fsum.  Different formulation from the oracle's real 2x2 form.
# --------------------------------------------------------------------------------------
def brute_fwd(q, k, v, base, window=0):
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv

    def rot(row, t):
        out = []
        for p in range(D // 2):
            z = complex(row[2 * p], row[2 * p + 1])
            if base > 0:
                z *= cmath.exp(1j * t * base ** (-2.0 * p / D))
            out.append(z)
        return out

    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qs = [rot(q[b, t, h], t) for t in range(T)]
            ks = [rot(k[b, t, g], t) for t in range(T)]
            for i in range(T):
                keys = [j for j in range(i + 1) if window <= 0 or i - j < window]
                w = []
                for j in keys:
                    s = math.fsum((qs[i][p].conjugate() * ks[j][p]).real for p in range(D // 2))
                    w.append(math.exp(s / math.sqrt(D)))
                z = math.fsum(w)
                lse[b, h, i] = math.log(z)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(wj * v[b, j, g, d] for wj, j in zip(w, keys)) / z
    return o, lse


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 2), (1, 3, 2, 1, 2), (2, 5, 2, 1, 4),
                                   (1, 4, 4, 2, 4), (1, 5, 3, 3, 2)])
@pytest.mark.parametrize("base", [10000.0, 3.0, 0.0])
def test_fwd_matches_brute_force(shape, base):
    q, k, v, _ = case(*shape, seed=7)
    o, lse = oracle.fwd(q, k, v, base)
    ob, lseb = brute_fwd(q, k, v, base)
    assert relerr(o, ob) < 1e-13
    assert np.max(np.abs(lse - lseb)) < 1e-13


def brute_grads_fd(q, k, v, dO, base, h=1e-6):
    """Central differences of the brute-force forward's loss sum(o * dO)."""
    def loss(q_, k_, v_):
        o, _ = brute_fwd(q_, k_, v_, base)
        return math.fsum((o * dO).ravel())

    grads = []
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(arrs[which])
        for idx in np.ndindex(*g.shape):
            x0 = arrs[which][idx]
            arrs[which][idx] = x0 + h
            lp = loss(*arrs)
            arrs[which][idx] = x0 - h
            lm = loss(*arrs)
            arrs[which][idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("shape,base", [((1, 3, 2, 1, 2), 10000.0), ((1, 4, 2, 1, 4), 2.0),
                                        ((1, 4, 4, 2, 2), 0.0)])
def test_bwd_matches_brute_force_finite_differences(shape, base):
    q, k, v, dO = case(*shape, seed=11)
    dq, dk, dv = oracle.bwd(q, k, v, dO, base)
    fq, fk, fv = brute_grads_fd(q, k, v, dO, base)
    for a, n in ((dq, fq), (dk, fk), (dv, fv)):
        assert relerr(a, n) < 1e-7


# --------------------------------------------------------------------------------------
# torch float64 autograd: an independent implementation (complex RoPE via view_as_complex,
# KV heads expanded with repeat_interleave, masked softmax, autograd for the gradients).
# --------------------------------------------------------------------------------------
def torch_attention(q, k, v, base, window=0, qk_norm=None):
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if qk_norm is not None:  # RMS over the head dimension of every (token, head) row, times the gain
        gain, eps = qk_norm
        q = gain * q / torch.sqrt((q * q).mean(dim=-1, keepdim=True) + eps)
        k = gain * k / torch.sqrt((k * k).mean(dim=-1, keepdim=True) + eps)
    if base > 0:
        theta = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
        ang = torch.arange(T, dtype=torch.float64)[:, None] * theta[None, :]
        rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

        def rope(x):
            xc = torch.view_as_complex(x.reshape(*x.shape[:-1], D // 2, 2).contiguous())
            return torch.view_as_real(xc * rot).reshape(x.shape)
        qr, kr = rope(q), rope(k)
    else:
        qr, kr = q, k
    kr = kr.repeat_interleave(Hq // Hkv, dim=2)
    ve = v.repeat_interleave(Hq // Hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", qr, kr) / math.sqrt(D)
    mask = torch.ones(T, T, dtype=torch.bool).triu(1)
    if window > 0:  # keys more than window - 1 positions back are hidden too
        mask |= torch.ones(T, T, dtype=torch.bool).tril(-window)
    s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, ve)
    return o, lse


@pytest.mark.parametrize("shape,base,qk", [((2, 37, 6, 2, 16), 10000.0, 1.0),
                                           ((1, 64, 4, 2, 32), 10000.0, 2.0),
                                           ((1, 33, 4, 4, 8), 0.0, 1.0),
                                           ((1, 50, 8, 2, 64), 5.0e5, 1.0),
                                           ((1, 19, 3, 1, 6), 10.0, 1.0)])
def test_against_torch_float64_autograd(shape, base, qk):
    q, k, v, dO = case(*shape, seed=23, qk=qk)
    o, lse = oracle.fwd(q, k, v, base)
    dq, dk, dv = oracle.bwd(q, k, v, dO, base)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    to, tlse = torch_attention(tq, tk, tv, base)
    (to * torch.tensor(dO)).sum().backward()
    assert relerr(o, to.detach().numpy()) < 1e-12
    assert np.max(np.abs(lse - tlse.detach().numpy())) < 1e-12
    assert relerr(dq, tq.grad.numpy()) < 1e-11
    assert relerr(dk, tk.grad.numpy()) < 1e-11
    assert relerr(dv, tv.grad.numpy()) < 1e-11


def test_no_rope_mha_equals_sdpa():
    """Without RoPE and with Hq = Hkv the path reduces to causal SDPA (library routine)."""
    q, k, v, _ = case(2, 45, 3, 3, 16, seed=31)
    o, _ = oracle.fwd(q, k, v, 0.0)
    t = lambda a: torch.tensor(a).permute(0, 2, 1, 3)  # [B,H,T,D]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    assert relerr(o, ref.permute(0, 2, 1, 3).numpy()) < 1e-13


# --------------------------------------------------------------------------------------
# Central finite differences on the oracle's own forward, in double precision, as the
# pages' gradient check does (pass bar there: max rel err < 1e-2; ours is 1e-6).
# --------------------------------------------------------------------------------------
def fd_check(q, k, v, dO, base, entries=None, h=1e-5, half_split=False):
    dq, dk, dv = oracle.bwd(q, k, v, dO, base, half_split=half_split)
    analytic = [dq, dk, dv]
    worst = 0.0
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        a = analytic[which]
        idxs = list(np.ndindex(*a.shape)) if entries is None else entries[which]
        num = np.zeros(len(idxs))
        ana = np.zeros(len(idxs))
        for n, idx in enumerate(idxs):
            x0 = arrs[which][idx]
            step = h * max(1.0, abs(x0))
            arrs[which][idx] = x0 + step
            lp = float(np.sum(oracle.fwd(*arrs, base, half_split=half_split)[0] * dO))
            arrs[which][idx] = x0 - step
            lm = float(np.sum(oracle.fwd(*arrs, base, half_split=half_split)[0] * dO))
            arrs[which][idx] = x0
            num[n] = (lp - lm) / (2 * step)
            ana[n] = a[idx]
        worst = max(worst, float(np.max(np.abs(ana - num)) / np.max(np.abs(num))))
    return worst


def test_finite_differences_every_entry_tiny():
    q, k, v, dO = case(1, 5, 4, 2, 4, seed=41)
    assert fd_check(q, k, v, dO, 10000.0) < 1e-6


def test_finite_differences_sampled_tiny_cpu_model():
    w = inputs.WORKLOADS["tiny_cpu_model"]
    q, k, v, dO = (t.double().numpy() for t in inputs.make_inputs(w))
    rng = np.random.default_rng(5)
    entries = []
    for a in (q, k, v):
        entries.append([tuple(int(rng.integers(0, s)) for s in a.shape) for _ in range(12)])
    assert fd_check(q, k, v, dO, w.rope_base, entries=entries) < 1e-6


# --------------------------------------------------------------------------------------
# Closed forms and special cases.
# --------------------------------------------------------------------------------------
def test_single_token():
    """T = 1: the only visible key is the query's own; R_0 = I."""
    q, k, v, dO = case(2, 1, 4, 2, 8, seed=51)
    o, lse = oracle.fwd(q, k, v, 10000.0)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0)
    G = 2
    for h in range(4):
        np.testing.assert_array_equal(o[:, 0, h], v[:, 0, h // G])
        ref = np.sum(q[:, 0, h] * k[:, 0, h // G], axis=-1) / math.sqrt(8)
        np.testing.assert_allclose(lse[:, h, 0], ref, rtol=0, atol=1e-14)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[:, 0, 0], dO[:, 0, 0] + dO[:, 0, 1], rtol=0, atol=1e-15)


def test_zero_queries_give_uniform_weights():
    """q = 0 (any RoPE): every visible key has weight 1/(i+1)."""
    _, k, v, dO = case(1, 40, 2, 1, 16, seed=61)
    q = np.zeros((1, 40, 2, 16))
    o, lse = oracle.fwd(q, k, v, 10000.0)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0)
    n = np.arange(1, 41)
    np.testing.assert_allclose(lse[0, 0], np.log(n), rtol=0, atol=1e-14)
    mean = np.cumsum(v[0, :, 0], axis=0) / n[:, None]
    np.testing.assert_allclose(o[0, :, 0], mean, rtol=0, atol=1e-13)
    # dv_j = sum_{i >= j} dO_i / (i + 1), summed over both query heads of the group
    w = dO[0].sum(axis=1) / n[:, None]
    dv_ref = np.cumsum(w[::-1], axis=0)[::-1]
    np.testing.assert_allclose(dv[0, :, 0], dv_ref, rtol=0, atol=1e-13)
    # with q = 0 the scores do not depend on k, so dk = 0 exactly
    assert np.all(dk == 0)


def test_constant_values_have_no_score_gradient():
    """v_j = c for all j: o = c whatever the weights, so dq = dk = 0."""
    q, k, _, dO = case(1, 30, 4, 2, 8, seed=71)
    c = rnd((8,), 72)
    v = np.broadcast_to(c, (1, 30, 2, 8)).copy()
    o, _ = oracle.fwd(q, k, v, 10000.0)
    dq, dk, _ = oracle.bwd(q, k, v, dO, 10000.0)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


def test_d2_rotation_by_t_radians():
    """D = 2: theta_0 = base^0 = 1 for every base, so position t rotates by t radians.

    With q_t = (1, 0) and k_t = (0, 1) the score is sin(i - j) / sqrt(2); a flipped
    rotation sign would give sin(j - i)."""
    T = 9
    q = np.zeros((1, T, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, T, 1, 2)); k[..., 1] = 1.0
    v = rnd((1, T, 1, 2), 81)
    for base in (10000.0, 500000.0, 2.0):
        o, lse = oracle.fwd(q, k, v, base)
        for i in range(T):
            s = np.array([math.sin(i - j) / math.sqrt(2) for j in range(i + 1)])
            w = np.exp(s)
            assert abs(lse[0, 0, i] - math.log(w.sum())) < 1e-14
            np.testing.assert_allclose(o[0, i, 0], (w[:, None] * v[0, : i + 1, 0]).sum(0) / w.sum(),
                                       rtol=0, atol=1e-14)


def test_golden_d2_worked_example():
    """Hand-derivable fixture (tests/golden/rope_d2_worked_example.json)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "rope_d2_worked_example.json")
    with open(path) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64).reshape(1, -1, 1, 2)
    k = np.array(g["k"], dtype=np.float64).reshape(1, -1, 1, 2)
    v = np.array(g["v"], dtype=np.float64).reshape(1, -1, 1, 2)
    o, lse = oracle.fwd(q, k, v, g["rope_base"])
    np.testing.assert_allclose(lse[0, 0], g["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, :, 0], np.array(g["o"]), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------------------
def test_softmax_rows_sum_to_one_and_are_causal():
    """With v = identity rows (T <= D), o row i is the probability row P[i, :]."""
    T = D = 16
    q, k, _, _ = case(1, T, 2, 1, D, seed=91, qk=3.0)
    v = np.eye(T)[None, :, None, :]
    o, _ = oracle.fwd(q, k, v, 10000.0)
    P = o[0, :, 0, :]
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.triu(P, 1) == 0)
    assert np.all(P[np.tril_indices(T)] > 0)


def test_causality_future_perturbation_is_bitwise_invisible():
    B, T, Hq, Hkv, D = 1, 48, 4, 2, 16
    q, k, v, dO = case(B, T, Hq, Hkv, D, seed=101)
    o, lse = oracle.fwd(q, k, v, 10000.0)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0)
    cut = 20
    k2, v2 = k.copy(), v.copy()
    k2[:, cut + 1:] += rnd(k2[:, cut + 1:].shape, 102)
    v2[:, cut + 1:] += rnd(v2[:, cut + 1:].shape, 103)
    o2, lse2 = oracle.fwd(q, k2, v2, 10000.0)
    np.testing.assert_array_equal(o2[:, : cut + 1], o[:, : cut + 1])
    np.testing.assert_array_equal(lse2[:, :, : cut + 1], lse[:, :, : cut + 1])
    # earlier queries / output gradients do not reach later keys' gradients
    q3, dO3 = q.copy(), dO.copy()
    q3[:, :cut] += rnd(q3[:, :cut].shape, 104)
    dO3[:, :cut] += rnd(dO3[:, :cut].shape, 105)
    _, dk3, dv3 = oracle.bwd(q3, k, v, dO3, 10000.0)
    np.testing.assert_allclose(dk3[:, cut:], dk[:, cut:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv3[:, cut:], dv[:, cut:], rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_replicated_kv():
    B, T, Hq, Hkv, D = 2, 33, 6, 2, 8
    G = Hq // Hkv
    q, k, v, dO = case(B, T, Hq, Hkv, D, seed=111)
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    o, lse = oracle.fwd(q, k, v, 10000.0)
    om, lsem = oracle.fwd(q, kr, vr, 10000.0)
    np.testing.assert_array_equal(o, om)
    np.testing.assert_array_equal(lse, lsem)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0)
    dqm, dkm, dvm = oracle.bwd(q, kr, vr, dO, 10000.0)
    np.testing.assert_array_equal(dq, dqm)
    np.testing.assert_allclose(dk, dkm.reshape(B, T, Hkv, G, D).sum(3), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dvm.reshape(B, T, Hkv, G, D).sum(3), rtol=0, atol=1e-13)


def test_thread_count_does_not_change_bits():
    q, k, v, dO = case(1, 70, 4, 2, 16, seed=121)
    a = oracle.fwd(q, k, v, 10000.0, nthreads=1) + oracle.bwd(q, k, v, dO, 10000.0, nthreads=1)
    b = oracle.fwd(q, k, v, 10000.0, nthreads=7) + oracle.bwd(q, k, v, dO, 10000.0, nthreads=7)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_rope_identity_at_zero_norm_and_inverse():
    x = rnd((2, 17, 3, 32), 131)
    y = oracle.rope(x, 10000.0)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])                       # R_0 = I
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-14, atol=0)                      # norm kept
    np.testing.assert_allclose(oracle.rope(y, 10000.0, inverse=True), x, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(oracle.rope(x, 0.0), x)               # base <= 0: off


def test_rope_scores_depend_only_on_relative_position():
    """<R_m a, R_n b> = <R_{m+s} a, R_{n+s} b>: rotate constant rows, compare dot products
    along diagonals, and against the closed form sum_p Re(conj(a_p) b_p e^{i (n-m) theta_p})."""
    T, D, base = 40, 16, 10000.0
    a, b = rnd((D,), 141), rnd((D,), 142)
    A = oracle.rope(np.broadcast_to(a, (1, T, 1, D)).copy(), base)[0, :, 0]
    Bm = oracle.rope(np.broadcast_to(b, (1, T, 1, D)).copy(), base)[0, :, 0]
    S = A @ Bm.T
    ac = a[0::2] + 1j * a[1::2]
    bc = b[0::2] + 1j * b[1::2]
    theta = base ** (-np.arange(0, D, 2) / D)
    for m in range(T):
        for n in range(T):
            ref = np.sum((np.conj(ac) * bc * np.exp(1j * (n - m) * theta)).real)
            assert abs(S[m, n] - ref) < 1e-12


# --------------------------------------------------------------------------------------
# The half-split pairing (element i rotated with element i + D/2).  Scores are dot products
# over the head dimension, so permuting q and k alike changes nothing: the half-split path is
# the interleaved path (pinned above) on inputs whose dimensions are reordered i -> 2i,
# i + D/2 -> 2i + 1, and its gradients are the interleaved ones reordered back.
# --------------------------------------------------------------------------------------
def to_interleaved(x):
    """[..., D] -> the same vector with element i at 2i and element i + D/2 at 2i + 1."""
    D = x.shape[-1]
    y = np.empty_like(x)
    y[..., 0::2], y[..., 1::2] = x[..., :D // 2], x[..., D // 2:]
    return y


def from_interleaved(y):
    return np.concatenate([y[..., 0::2], y[..., 1::2]], axis=-1)


def test_half_split_rope_is_the_interleaved_rotation_of_reordered_dimensions():
    x = rnd((2, 23, 3, 16), 151)
    for inv in (False, True):
        ref = from_interleaved(oracle.rope(to_interleaved(x), 10000.0, inverse=inv))
        np.testing.assert_array_equal(oracle.rope(x, 10000.0, inverse=inv, half_split=True), ref)
    np.testing.assert_array_equal(oracle.rope(x, 0.0, half_split=True), x)


def test_half_split_scores_depend_only_on_relative_position():
    """The closed form of test_rope_scores_depend_only_on_relative_position with the complex
    pairs a_i + i a_{i + D/2}."""
    T, D, base = 33, 16, 500.0
    a, b = rnd((D,), 161), rnd((D,), 162)
    A = oracle.rope(np.broadcast_to(a, (1, T, 1, D)).copy(), base, half_split=True)[0, :, 0]
    Bm = oracle.rope(np.broadcast_to(b, (1, T, 1, D)).copy(), base, half_split=True)[0, :, 0]
    S = A @ Bm.T
    ac = a[:D // 2] + 1j * a[D // 2:]
    bc = b[:D // 2] + 1j * b[D // 2:]
    theta = base ** (-np.arange(0, D, 2) / D)
    for m in range(T):
        for n in range(T):
            ref = np.sum((np.conj(ac) * bc * np.exp(1j * (n - m) * theta)).real)
            assert abs(S[m, n] - ref) < 1e-12


@pytest.mark.parametrize("window,qk", [(0, None), (7, None), (0, (1.2, 1e-6))])
def test_half_split_attention_is_interleaved_attention_of_reordered_q_and_k(window, qk):
    q, k, v, dO = case(2, 29, 6, 2, 16, seed=171)
    o, lse = oracle.fwd(q, k, v, 10000.0, window=window, qk_norm=qk, half_split=True)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0, window=window, qk_norm=qk, half_split=True)
    qi, ki = to_interleaved(q), to_interleaved(k)
    ro, rlse = oracle.fwd(qi, ki, v, 10000.0, window=window, qk_norm=qk)
    rq, rk, rv = oracle.bwd(qi, ki, v, dO, 10000.0, window=window, qk_norm=qk)
    assert relerr(o, ro) < 1e-14 and np.max(np.abs(lse - rlse)) < 1e-13
    assert relerr(dq, from_interleaved(rq)) < 1e-13
    assert relerr(dk, from_interleaved(rk)) < 1e-13
    assert relerr(dv, rv) < 1e-13
    # and the pairing matters: the interleaved path on the same inputs gives other scores
    assert relerr(o, oracle.fwd(q, k, v, 10000.0, window=window, qk_norm=qk)[0]) > 1e-3


def test_half_split_finite_differences_every_entry_tiny():
    q, k, v, dO = case(1, 5, 4, 2, 4, seed=43)
    assert fd_check(q, k, v, dO, 10000.0, half_split=True) < 1e-6


def test_rejects_bad_shapes():
    q, k, v, dO = case(1, 4, 3, 2, 8, seed=1)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, 10000.0)          # Hq % Hkv != 0
    q, k, v, dO = case(1, 4, 2, 1, 5, seed=1)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, 10000.0)          # odd D with RoPE on
    oracle.fwd(q, k, v, 0.0)                  # odd D without RoPE is fine


def test_workloads_follow_the_pages_model_configs():
    """tests/golden/pages_model_configs.json holds the figures the pages print."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_model_configs.json")
    with open(path) as f:
        g = json.load(f)
    cpu, gpu = g["cpu_model"], g["gpu_model"]
    w1 = inputs.WORKLOADS["tiny_cpu_model"]
    w2 = inputs.WORKLOADS["nanoeuler_gpu_layer"]
    assert (w1.Hq, w1.Hkv, w1.Hq * w1.D, w1.T) == (cpu["q_heads"], cpu["kv_heads"], cpu["dim"], cpu["context"])
    assert (w2.Hq, w2.Hkv, w2.Hq * w2.D, w2.T) == (gpu["q_heads"], gpu["kv_heads"], gpu["dim"], gpu["context"])
    assert w2.D == gpu["head_dim"]


def test_bwd_given_exact_o_reproduces_bwd_bitwise():
    """bwd_given_o with the exact o is the plain backward; dv never depends on o."""
    q, k, v, dO = case(2, 41, 6, 2, 16, seed=151)
    o, _ = oracle.fwd(q, k, v, 10000.0)
    a = oracle.bwd(q, k, v, dO, 10000.0)
    b = oracle.bwd_given_o(q, k, v, o, dO, 10000.0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    o2 = o + 1e-3 * rnd(o.shape, 152)
    dq2, dk2, dv2 = oracle.bwd_given_o(q, k, v, o2, dO, 10000.0)
    np.testing.assert_array_equal(dv2, a[2])
    assert relerr(dq2, a[0]) > 1e-6  # Delta does enter dq


def test_bwd_given_o_matches_autograd_with_delta_from_o():
    """Against torch: with Delta from a perturbed o, the backward equals autograd of
    sum(o * dO) plus the extra term -sum_i (Delta~_i - Delta_i) * lse_i (lse's gradient is P)."""
    q, k, v, dO = case(1, 23, 4, 2, 8, seed=161)
    o, _ = oracle.fwd(q, k, v, 100.0)
    o2 = o + 1e-2 * rnd(o.shape, 162)
    dq2, dk2, dv2 = oracle.bwd_given_o(q, k, v, o2, dO, 100.0)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    to, tlse = torch_attention(tq, tk, tv, 100.0)
    extra = torch.tensor(np.einsum("bthd,bthd->bht", dO, o2 - o))  # Delta~ - Delta
    loss = (to * torch.tensor(dO)).sum() - (extra * tlse).sum()
    loss.backward()
    assert relerr(dq2, tq.grad.numpy()) < 1e-11
    assert relerr(dk2, tk.grad.numpy()) < 1e-11
    assert relerr(dv2, tv.grad.numpy()) < 1e-11


# --------------------------------------------------------------------------------------
# Sliding window (query i sees keys i - W + 1 .. i): the nanochat guide's window_pattern,
# where "S" layers see a quarter of the context.
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("shape,window", [((1, 6, 2, 1, 4), 1), ((1, 6, 4, 2, 4), 2), ((2, 7, 2, 2, 2), 3),
                                          ((1, 5, 3, 1, 4), 5)])
def test_window_matches_brute_force(shape, window):
    q, k, v, _ = case(*shape, seed=301)
    o, lse = oracle.fwd(q, k, v, 3.0, window=window)
    bo, blse = brute_fwd(q, k, v, 3.0, window=window)
    assert relerr(o, bo) < 1e-13
    assert np.max(np.abs(lse - blse)) < 1e-13


@pytest.mark.parametrize("shape,base,window", [((2, 37, 6, 2, 16), 10000.0, 8), ((1, 64, 4, 2, 32), 10000.0, 16),
                                               ((1, 33, 4, 4, 8), 0.0, 5), ((1, 19, 3, 1, 6), 10.0, 1)])
def test_window_against_torch_float64_autograd(shape, base, window):
    q, k, v, dO = case(*shape, seed=311)
    o, lse = oracle.fwd(q, k, v, base, window=window)
    dq, dk, dv = oracle.bwd(q, k, v, dO, base, window=window)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    to, tlse = torch_attention(tq, tk, tv, base, window=window)
    (to * torch.tensor(dO)).sum().backward()
    assert relerr(o, to.detach().numpy()) < 1e-12
    assert np.max(np.abs(lse - tlse.detach().numpy())) < 1e-12
    assert relerr(dq, tq.grad.numpy()) < 1e-11
    assert relerr(dk, tk.grad.numpy()) < 1e-11
    assert relerr(dv, tv.grad.numpy()) < 1e-11


def test_window_of_at_least_T_is_the_full_causal_prefix():
    q, k, v, dO = case(1, 21, 4, 2, 8, seed=321)
    full = oracle.fwd(q, k, v, 10000.0) + oracle.bwd(q, k, v, dO, 10000.0)
    for W in (21, 22, 1000):
        got = oracle.fwd(q, k, v, 10000.0, window=W) + oracle.bwd(q, k, v, dO, 10000.0, window=W)
        for a, b in zip(got, full):
            np.testing.assert_array_equal(a, b)


def test_window_one_sees_only_itself():
    """W = 1: o_i = v_i, lse_i = q'_i . k'_i / sqrt(D); P = 1 makes dS = 0, so dq = dk = 0."""
    q, k, v, dO = case(1, 9, 4, 2, 8, seed=331)
    o, lse = oracle.fwd(q, k, v, 10000.0, window=1)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0, window=1)
    qr, kr = oracle.rope(q, 10000.0), oracle.rope(k, 10000.0)
    for h in range(4):
        np.testing.assert_array_equal(o[0, :, h], v[0, :, h // 2])
        ref = np.sum(qr[0, :, h] * kr[0, :, h // 2], axis=-1) / math.sqrt(8)
        np.testing.assert_allclose(lse[0, h], ref, rtol=0, atol=1e-13)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, :, 0], dO[0, :, 0] + dO[0, :, 1], rtol=0, atol=1e-15)


def test_window_zero_queries_average_the_window():
    """q = 0: every visible key has weight 1 / min(i + 1, W)."""
    W, T = 7, 30
    _, k, v, dO = case(1, T, 2, 1, 16, seed=341)
    q = np.zeros((1, T, 2, 16))
    o, lse = oracle.fwd(q, k, v, 10000.0, window=W)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0, window=W)
    n = np.minimum(np.arange(1, T + 1), W)
    np.testing.assert_allclose(lse[0, 0], np.log(n), rtol=0, atol=1e-14)
    mean = np.array([v[0, max(0, i - W + 1):i + 1, 0].mean(axis=0) for i in range(T)])
    np.testing.assert_allclose(o[0, :, 0], mean, rtol=0, atol=1e-13)
    # dv_j = sum over the queries i = j .. j + W - 1 that see key j of dO_i / n_i (both heads)
    w = dO[0].sum(axis=1) / n[:, None]
    dv_ref = np.array([w[j:min(T, j + W)].sum(axis=0) for j in range(T)])
    np.testing.assert_allclose(dv[0, :, 0], dv_ref, rtol=0, atol=1e-13)
    assert np.all(dk == 0)


def test_window_keys_outside_the_window_are_invisible():
    """Perturbing key/value j changes only the queries j .. j + W - 1, bitwise."""
    W, T, j = 6, 25, 9
    q, k, v, dO = case(1, T, 4, 2, 8, seed=351)
    o, lse = oracle.fwd(q, k, v, 10000.0, window=W)
    k2, v2 = k.copy(), v.copy()
    k2[0, j] += 1.0
    v2[0, j] -= 2.0
    o2, lse2 = oracle.fwd(q, k2, v2, 10000.0, window=W)
    outside = [i for i in range(T) if not (j <= i <= j + W - 1)]
    np.testing.assert_array_equal(o[0, outside], o2[0, outside])
    np.testing.assert_array_equal(lse[0, :, outside], lse2[0, :, outside])
    inside = list(range(j, j + W))
    assert np.all(np.any(o[0, inside] != o2[0, inside], axis=(1, 2)))


def test_window_finite_differences_tiny():
    q, k, v, dO = case(1, 7, 4, 2, 4, seed=361)
    W = 3
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0, window=W)
    worst = 0.0
    for which, a in enumerate((dq, dk, dv)):
        arrs = [q.copy(), k.copy(), v.copy()]
        for idx in np.ndindex(*a.shape):
            x0 = arrs[which][idx]
            step = 1e-5 * max(1.0, abs(x0))
            arrs[which][idx] = x0 + step
            lp = float(np.sum(oracle.fwd(*arrs, 10000.0, window=W)[0] * dO))
            arrs[which][idx] = x0 - step
            lm = float(np.sum(oracle.fwd(*arrs, 10000.0, window=W)[0] * dO))
            arrs[which][idx] = x0
            worst = max(worst, abs((lp - lm) / (2 * step) - a[idx]) / np.max(np.abs(a)))
    assert worst < 1e-6


# --------------------------------------------------------------------------------------
# QK norm (nanochat guide, 模型架构速览: q and k normalised and scaled up by 1.2).
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("shape,base,window,qkn", [((2, 37, 6, 2, 16), 10000.0, 0, (1.2, 1e-6)),
                                                   ((1, 33, 4, 4, 8), 0.0, 0, (1.2, 0.0)),
                                                   ((1, 50, 8, 2, 32), 5.0e5, 9, (1.2, 1e-6)),
                                                   ((1, 19, 3, 1, 6), 10.0, 0, (0.7, 0.25))])
def test_qk_norm_against_torch_float64_autograd(shape, base, window, qkn):
    q, k, v, dO = case(*shape, seed=371)
    o, lse = oracle.fwd(q, k, v, base, window=window, qk_norm=qkn)
    dq, dk, dv = oracle.bwd(q, k, v, dO, base, window=window, qk_norm=qkn)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    to, tlse = torch_attention(tq, tk, tv, base, window=window, qk_norm=qkn)
    (to * torch.tensor(dO)).sum().backward()
    assert relerr(o, to.detach().numpy()) < 1e-12
    assert np.max(np.abs(lse - tlse.detach().numpy())) < 1e-12
    assert relerr(dq, tq.grad.numpy()) < 1e-11
    assert relerr(dk, tk.grad.numpy()) < 1e-11
    assert relerr(dv, tv.grad.numpy()) < 1e-11


def test_qk_norm_self_score_closed_form():
    """T = 1 (R_0 = I) and k = q: the only score is |x_hat|^2 / sqrt(D) with |x_hat|^2 =
    gain^2 * D * ms / (ms + eps), ms = mean(x^2) -- independent of the direction of x."""
    rng = np.random.default_rng(381)
    D, gain = 16, 1.2
    for eps in (0.0, 1e-6, 0.5):
        q = rng.standard_normal((1, 1, 2, D)) * rng.uniform(0.1, 3.0)
        k = q[:, :, :1].copy()
        q[:, :, 1] = q[:, :, 0]                 # both query heads equal the key
        v = rng.standard_normal((1, 1, 1, D))
        o, lse = oracle.fwd(q, k, v, 1e4, qk_norm=(gain, eps))
        ms = float(np.mean(q[0, 0, 0] ** 2))
        ref = gain ** 2 * D * ms / (ms + eps) / math.sqrt(D)
        np.testing.assert_allclose(lse[0, :, 0], [ref, ref], rtol=1e-14, atol=0)
        np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])


def test_qk_norm_rescaling_rows_changes_nothing():
    """eps = 0: scaling any q or k row by c > 0 leaves o and lse unchanged, and the gradient with
    respect to that row scales by 1 / c (the loss is invariant along the row)."""
    q, k, v, dO = case(1, 23, 4, 2, 8, seed=391)
    qkn = (1.2, 0.0)
    o, lse = oracle.fwd(q, k, v, 1e4, qk_norm=qkn)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 1e4, qk_norm=qkn)
    c = np.random.default_rng(392).uniform(0.2, 5.0, size=(1, 23, 4, 1))
    ck = np.random.default_rng(393).uniform(0.2, 5.0, size=(1, 23, 2, 1))
    o2, lse2 = oracle.fwd(q * c, k * ck, v, 1e4, qk_norm=qkn)
    dq2, dk2, dv2 = oracle.bwd(q * c, k * ck, v, dO, 1e4, qk_norm=qkn)
    assert relerr(o2, o) < 1e-13 and np.max(np.abs(lse2 - lse)) < 1e-13
    assert relerr(dq2 * c, dq) < 1e-12 and relerr(dk2 * ck, dk) < 1e-12 and relerr(dv2, dv) < 1e-12
    # and the gradient is orthogonal to its row (no component along the scale direction)
    assert np.max(np.abs(np.sum(dq * q, axis=-1))) < 1e-12 * np.max(np.abs(dq)) * np.max(np.abs(q)) * 8
    assert np.max(np.abs(np.sum(dk * k, axis=-1))) < 1e-12 * np.max(np.abs(dk)) * np.max(np.abs(k)) * 8


def test_qk_norm_finite_differences_tiny():
    q, k, v, dO = case(1, 6, 4, 2, 4, seed=401)
    qkn = (1.2, 1e-3)
    dq, dk, dv = oracle.bwd(q, k, v, dO, 10000.0, window=4, qk_norm=qkn)
    worst = 0.0
    for which, a in enumerate((dq, dk, dv)):
        arrs = [q.copy(), k.copy(), v.copy()]
        for idx in np.ndindex(*a.shape):
            x0 = arrs[which][idx]
            step = 1e-5 * max(1.0, abs(x0))
            arrs[which][idx] = x0 + step
            lp = float(np.sum(oracle.fwd(*arrs, 10000.0, window=4, qk_norm=qkn)[0] * dO))
            arrs[which][idx] = x0 - step
            lm = float(np.sum(oracle.fwd(*arrs, 10000.0, window=4, qk_norm=qkn)[0] * dO))
            arrs[which][idx] = x0
            worst = max(worst, abs((lp - lm) / (2 * step) - a[idx]) / np.max(np.abs(a)))
    assert worst < 1e-6


def test_qk_norm_given_o_with_exact_o_is_the_exact_gradient():
    q, k, v, dO = case(1, 30, 6, 2, 16, seed=411)
    qkn = (1.2, 1e-6)
    o, _ = oracle.fwd(q, k, v, 1e4, qk_norm=qkn)
    a = oracle.bwd(q, k, v, dO, 1e4, qk_norm=qkn)
    b = oracle.bwd_given_o(q, k, v, o, dO, 1e4, qk_norm=qkn)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)

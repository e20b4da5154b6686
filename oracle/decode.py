"""Oracle for attention of new tokens against a key/value cache (decode, chunked prefill).

TEST INFRASTRUCTURE ONLY: used by the test suite and the benchmark's CPU-baseline leg, never
by the product package.  Plain float64 numpy, written from the definition; it shares no code
with the HIP library nor with ne_oracle.c.

What it computes.  The pages' model runs decoder-only causal attention with RoPE on q and k and
grouped-query heads ("NanoEuler: 使用 C 和 CUDA 从零开始构建的 GPT-2 规模 LLM", 技术规格,
核心架构与设计); nanochat generates with a KV cache ("nanochat 全栈 LLM 训练实践指南", 项目定位 and
测试体系) and uses sliding windows (模型架构速览, window_pattern).  With a cache, sequence b already
holds L_b = lens[b] tokens and adds Tq: new token t sits at absolute position p = L_b + t, its
query is rotated by p, every key j by its own position j, and it attends to keys
max(0, p - W + 1) .. p (W <= 0: all of 0 .. p).  This is exactly row p of full causal attention
over the L_b + Tq tokens, which the tests use as one pin.

Readings (as in ne_oracle.c): RoPE rotates adjacent pairs (2i, 2i+1) by +p*theta_i,
theta_i = base^(-2i/D), base <= 0 disables it (half_split: the pairs (i, i + D/2) instead, at the
same angles); scale 1/sqrt(D) after RoPE; query head h reads KV
head h // (Hq/Hkv); lse is the natural-log log-sum-exp of the scaled scores.
"""
import numpy as np


def rope_rows(x, positions, base, half_split=False):
    """Rotate x[..., P, H, D] (P positions along axis -3) pairwise by positions * theta_i: pairs
    (2i, 2i+1), or (i, i + D/2) with half_split."""
    x = np.asarray(x, dtype=np.float64)
    if base <= 0.0:
        return x.copy()
    D = x.shape[-1]
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]   # [P, D/2]
    c = np.cos(ang)[:, None, :]                                               # [P, 1, D/2]
    s = np.sin(ang)[:, None, :]
    if half_split:
        a, b = x[..., :D // 2], x[..., D // 2:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = a * c - b * s
    y[..., 1::2] = a * s + b * c
    return y


def qk_norm_rows(x, gain, eps):
    """gain * x / sqrt(mean(x^2) + eps) over the last axis (the QK norm of 模型架构速览)."""
    return gain * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def decode_fwd(q_new, k_seq, v_seq, lens, base, window=0, qk_norm=None, half_split=False):
    """o [B][Tq][Hq][D], lse [B][Hq][Tq] for queries q_new [B][Tq][Hq][D] at positions lens[b] + t.

    k_seq[b], v_seq[b]: the raw (un-rotated) keys and values [L][Hkv][D] of sequence b at positions
    0 .. L - 1, L >= lens[b] + Tq (positions past lens[b] + Tq - 1 are never visible).
    qk_norm (gain, eps): rows of q and k are normalised first (rows of the cache when appended).
    half_split: the rotation pairs (i, i + D/2)."""
    q_new = np.asarray(q_new, dtype=np.float64)
    B, Tq, Hq, D = q_new.shape
    o = np.zeros((B, Tq, Hq, D))
    lse = np.zeros((B, Hq, Tq))
    for b in range(B):
        L = int(lens[b]) + Tq                        # positions 0 .. L - 1 exist for this step
        k = np.asarray(k_seq[b], dtype=np.float64)[:L]
        v = np.asarray(v_seq[b], dtype=np.float64)[:L]
        if k.shape[0] < L or v.shape[0] < L:
            raise ValueError(f"sequence {b} holds {k.shape[0]} positions, {L} needed")
        Hkv = k.shape[1]
        G = Hq // Hkv
        pos = int(lens[b]) + np.arange(Tq)
        qb = q_new[b]
        if qk_norm is not None:
            qb, k = qk_norm_rows(qb, *qk_norm), qk_norm_rows(k, *qk_norm)
        qr = rope_rows(qb, pos, base, half_split)                # [Tq][Hq][D]
        kr = rope_rows(k, np.arange(L), base, half_split)        # [L][Hkv][D]
        j = np.arange(L)
        vis = (j[None, :] <= pos[:, None])
        if window > 0:
            vis &= (pos[:, None] - j[None, :]) < window
        for h in range(Hq):
            g = h // G
            s = qr[:, h, :] @ kr[:, g, :].T / np.sqrt(D)     # [Tq][L]
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            z = p.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (p / z) @ v[:, g, :]
            lse[b, h, :] = (m + np.log(z))[:, 0]
    return o, lse

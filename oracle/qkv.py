"""Oracle for the QKV projection with a RoPE (and optional QK-norm) epilogue.

TEST INFRASTRUCTURE ONLY: used by the test suite, never by the product package.  Plain float64
numpy, written from the definition; it shares no code with the HIP library.

What it computes.  The pages' model projects every token's hidden vector to queries, keys and
values with a matrix product ("NanoEuler: 使用 C 和 CUDA 从零开始构建的 GPT-2 规模 LLM", 内核实现:
the matrix products run through cuBLAS on TF32 tensor cores) and then rotates q and k (RoPE,
技术规格) in a kernel of its own -- a separate pass with its own launch and memory traffic, as the
author concedes in the cnblogs walkthrough ("用 100KB C/CUDA 单文件复刻 GPT-2...", §3.4).  Fusing the
rotation into the product's epilogue writes q' and k' directly.

Readings: x [B][T][C]; the weight is [N][C] with N = (Hq + 2 Hkv) D, rows ordered as the Hq query
heads, then the Hkv key heads, then the Hkv value heads, each D consecutive features (so
y = x W^T, as a linear layer stores its weight); token t of each sequence has position t;
q' = R_t(norm(y_q)), k' = R_t(norm(y_k)), v = y_v, with norm the optional QK norm
(gain * y / sqrt(mean(y^2) + eps) per head) and R_t the rotation of the attention oracle.
"""
import numpy as np

from .decode import qk_norm_rows, rope_rows


def qkv_rope_proj(x, w, Hq, Hkv, base, qk_norm=None, positions=None, half_split=False):
    """Return (q', k', v) as float64 arrays [B][T][H][D]; positions (default 0 .. T-1) are those of
    the T tokens given (a sample of a longer sequence may be checked by passing its positions);
    half_split: the rotation pairs (i, i + D/2) instead of (2i, 2i+1)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, C = x.shape
    N = w.shape[0]
    D = N // (Hq + 2 * Hkv)
    if w.shape[1] != C or D * (Hq + 2 * Hkv) != N:
        raise ValueError(f"weight {w.shape} does not match C={C}, Hq={Hq}, Hkv={Hkv}")
    y = x @ w.T                                           # [B][T][N]
    q = y[..., :Hq * D].reshape(B, T, Hq, D)
    k = y[..., Hq * D:(Hq + Hkv) * D].reshape(B, T, Hkv, D)
    v = y[..., (Hq + Hkv) * D:].reshape(B, T, Hkv, D).copy()
    if qk_norm is not None:
        q, k = qk_norm_rows(q, *qk_norm), qk_norm_rows(k, *qk_norm)
    pos = np.arange(T) if positions is None else np.asarray(positions)
    qr = np.stack([rope_rows(q[b], pos, base, half_split) for b in range(B)])
    kr = np.stack([rope_rows(k[b], pos, base, half_split) for b in range(B)])
    return qr, kr, v

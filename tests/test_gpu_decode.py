"""GPU parity of the key/value-cache entry points (ne_kv_cache_append, ne_rope_attn_decode) against
the decode oracle (oracle/decode.py), needs an MI355X.

Bars as in test_gpu_parity.py (fp16 MFMA operands: 2e-3 of each output's scale; 16-bit outputs add
half an ulp).  The cache holds keys rotated at their positions and values, both rounded to fp16
once, exactly as the training path's operand copies; the oracle rotates the raw inputs in float64.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_parity import DEV, check, f64

pytestmark = pytest.mark.gpu

_NAME = {torch.bfloat16: "bf16", torch.float16: "f16"}


def seqs(B, P, Hq, Hkv, D, seed, dtype):
    """Raw q, k, v of B sequences of P positions (CPU, storage dtype)."""
    return (inputs.gaussian((B, P, Hq, D), seed, 1.0, dtype), inputs.gaussian((B, P, Hkv, D), seed + 1, 1.0, dtype),
            inputs.gaussian((B, P, Hkv, D), seed + 2, 1.0, dtype))


def unpack_cache(half, B, Hkv, Tcap, D):
    """Keys and values [B][Hkv][Tcap][D] from the cache layout of include/ne_rope_attn.h: per group,
    tiles of 32 positions; in a tile the key block (unit u, lane l: key l % 32, dimensions
    16u + 8(l / 32) + e) and then the value block (unit (kk, db), lane l, element j: dimension
    32db + l % 32 of key 16kk + s(8(l / 32) + j), s swapping bits 2 and 3)."""
    t = half.reshape(B, Hkv, Tcap // 32, 64 * D)
    kb = t[..., :32 * D].reshape(B, Hkv, Tcap // 32, D // 16, 2, 32, 8)       # [u][l / 32][l % 32][e]
    keys = kb.transpose(0, 1, 2, 5, 3, 4, 6).reshape(B, Hkv, Tcap, D)
    vb = t[..., 32 * D:].reshape(B, Hkv, Tcap // 32, 2, D // 32, 2, 32, 8)     # [kk][db][l / 32][l % 32][j]
    vb = vb.transpose(0, 1, 2, 3, 5, 7, 4, 6).reshape(B, Hkv, Tcap // 32, 32, D)  # [16kk + 8(l / 32) + j][d]
    pos = np.arange(32)
    swap = (pos & ~15) + 8 * ((pos >> 2) & 1) + 4 * ((pos >> 3) & 1) + (pos & 3)   # its own inverse
    vals = vb[:, :, :, swap, :].reshape(B, Hkv, Tcap, D)
    return keys, vals


def fill_cache(k, v, Tcap, base, chunks):
    """Append positions 0 .. P-1 of every sequence in chunks of the given sizes; returns the cache."""
    B, P, Hkv, D = k.shape
    cache = binding.new_kv_cache(B, Tcap, Hkv, D, k.dtype, DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    p = 0
    for n in chunks:
        n = min(n, P - p)
        if n <= 0:
            break
        lens = torch.full((B,), p, dtype=torch.int32, device=DEV)
        binding.ne_kv_cache_append(cache, lens, kd[:, p:p + n].contiguous(), vd[:, p:p + n].contiguous(), Tcap, base)
        p += n
    assert p == P
    return cache


def run_decode(q_new, cache, lens, Tcap, Hkv, base, window, out_dtype):
    o, lse = binding.ne_rope_attn_decode(q_new.to(DEV), cache, lens, Tcap, Hkv, base, window, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def decode_parity(B, P, Tq, Hq, Hkv, D, lens, window, in_dt, out_dt, Tcap=None, base=1.0e4, chunks=(64,) * 1000,
                  seed=600):
    Tcap = Tcap or (P + 63) // 64 * 64
    q, k, v = seqs(B, P, Hq, Hkv, D, seed, _NAME[in_dt])
    cache = fill_cache(k, v, Tcap, base, chunks)
    q_new = torch.stack([q[b, lens[b]:lens[b] + Tq] for b in range(B)])
    o, lse = run_decode(q_new, cache, lens, Tcap, Hkv, base, window, out_dt)
    ro, rlse = oracle.decode_fwd(f64(q_new), [f64(k[b]) for b in range(B)], [f64(v[b]) for b in range(B)], lens,
                                 base, window)
    check("o", o, ro, in_dt, out_dt)
    check("lse", lse, rlse, in_dt, out_dt)
    return o, lse


@pytest.mark.parametrize("case", [
    # B, P, Tq, Hq, Hkv, D, lens, window, in, out
    (3, 200, 1, 8, 2, 128, [0, 57, 199], 0, torch.bfloat16, torch.float32),
    (2, 300, 5, 12, 4, 64, [10, 295], 0, torch.bfloat16, torch.bfloat16),
    (2, 256, 17, 8, 2, 128, [0, 239], 0, torch.float16, torch.float32),
    (1, 640, 1, 4, 4, 32, [639], 100, torch.bfloat16, torch.float32),
    (2, 512, 9, 6, 2, 128, [100, 500], 64, torch.bfloat16, torch.float32),
    (4, 130, 3, 3, 1, 64, [0, 1, 64, 127], 0, torch.float16, torch.float16),
    (1, 96, 96, 4, 2, 64, [0], 0, torch.bfloat16, torch.float32),
])
def test_decode_parity(case):
    B, P, Tq, Hq, Hkv, D, lens, window, in_dt, out_dt = case
    decode_parity(B, P, Tq, Hq, Hkv, D, lens, window, in_dt, out_dt, chunks=(37, 1, 64, 200, 500, 1000))


@pytest.mark.parametrize("base", [1.0e4, 0.0])
def test_append_writes_rotated_keys_and_transposed_values(base):
    B, P, Hkv, D, Tcap = 2, 150, 2, 64, 192
    _, k, v = seqs(B, P, 2, Hkv, D, 700, "bf16")
    cache = fill_cache(k, v, Tcap, base, (10, 1, 50, 89)).cpu()
    kc, vc = unpack_cache(cache.view(torch.float16).double().numpy(), B, Hkv, Tcap, D)
    ref_k = np.stack([oracle.rope_rows(f64(k[b]), np.arange(P), base) for b in range(B)])   # [B][P][Hkv][D]
    for b in range(B):
        for g in range(Hkv):
            rk = ref_k[b, :, g]
            assert np.all(np.abs(kc[b, g, :P] - rk) <= 2.0 ** -11 * np.abs(rk) + 1e-6)
            np.testing.assert_array_equal(vc[b, g, :P], f64(v[b, :, g]).astype(np.float16).astype(np.float64))
    assert np.all(kc[:, :, P:] == 0) and np.all(vc[:, :, P:] == 0)


def test_decode_token_by_token_loop():
    """Prompt appended at once, then per step: append one token, attend, advance the lengths."""
    B, Hq, Hkv, D, Tcap, prompt, steps = 2, 8, 2, 128, 128, 40, 24
    q, k, v = seqs(B, prompt + steps, Hq, Hkv, D, 710, "bf16")
    cache = binding.new_kv_cache(B, Tcap, Hkv, D, torch.bfloat16, DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    binding.ne_kv_cache_append(cache, lens, kd[:, :prompt].contiguous(), vd[:, :prompt].contiguous(), Tcap, 1e4)
    lens += prompt
    for s in range(steps):
        p = prompt + s
        binding.ne_kv_cache_append(cache, lens, kd[:, p:p + 1].contiguous(), vd[:, p:p + 1].contiguous(), Tcap, 1e4)
        o, lse = binding.ne_rope_attn_decode(qd[:, p:p + 1].contiguous(), cache, lens, Tcap, Hkv, 1e4)
        lens += 1
        torch.cuda.synchronize()
        ro, rlse = oracle.decode_fwd(f64(q[:, p:p + 1]), [f64(k[b]) for b in range(B)],
                                     [f64(v[b]) for b in range(B)], [p] * B, 1e4)
        check("o", o.cpu(), ro, torch.bfloat16, torch.float32)
        check("lse", lse.cpu(), rlse, torch.bfloat16, torch.float32)
    assert lens.cpu().tolist() == [prompt + steps] * B


def test_decode_long_cache_full_context():
    """Cache of 8192 positions (the long-context shape, RoPE base 5e5), one new token."""
    decode_parity(2, 8192, 1, 32, 8, 128, [8191, 4000], 0, torch.bfloat16, torch.float32, Tcap=8192, base=5.0e5,
                  chunks=(1024,) * 8, seed=720)


def test_decode_window_quarter_context():
    decode_parity(2, 2048, 4, 12, 4, 128, [2044, 1500], 512, torch.bfloat16, torch.float32, chunks=(512,) * 4,
                  seed=730)


def test_decode_clamps_out_of_range_lengths():
    B, P, Tq, Hq, Hkv, D, Tcap = 2, 128, 2, 4, 2, 64, 128
    q, k, v = seqs(B, P, Hq, Hkv, D, 740, "bf16")
    cache = fill_cache(k, v, Tcap, 1e4, (128,))
    q_new = q[:, :Tq].contiguous()
    o1, l1 = run_decode(q_new, cache, [10 ** 6, -5], Tcap, Hkv, 1e4, 0, torch.float32)
    o2, l2 = run_decode(q_new, cache, [Tcap - Tq, 0], Tcap, Hkv, 1e4, 0, torch.float32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_is_bitwise_deterministic():
    B, P, Tq, Hq, Hkv, D = 2, 1000, 3, 8, 2, 128
    q, k, v = seqs(B, P, Hq, Hkv, D, 750, "bf16")
    cache = fill_cache(k, v, 1024, 1e4, (1000,))
    q_new = q[:, -Tq:].contiguous()
    a = run_decode(q_new, cache, [P - Tq] * B, 1024, Hkv, 1e4, 0, torch.float32)
    b = run_decode(q_new, cache, [P - Tq] * B, 1024, Hkv, 1e4, 0, torch.float32)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_agrees_with_the_training_forward():
    """Chunked prefill of a whole sequence (lens 0, Tq = T) against ne_rope_attn_fwd on it."""
    B, T, Hq, Hkv, D = 1, 192, 8, 2, 64
    q, k, v = seqs(B, T, Hq, Hkv, D, 760, "bf16")
    cache = fill_cache(k, v, 192, 1e4, (192,))
    o, lse = run_decode(q, cache, [0], 192, Hkv, 1e4, 0, torch.float32)
    fo, flse = binding.ne_rope_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 1e4)
    assert float((o - fo.cpu()).abs().max()) < 2e-3 * float(fo.abs().max())
    assert float((lse - flse.cpu()).abs().max()) < 2e-3 * float(flse.abs().max())
